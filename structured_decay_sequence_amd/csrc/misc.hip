// Decode step, decay-operand builders and the decay-range check.
#include "common.hpp"
#include "kernels.hpp"

namespace lattn {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Single recurrent token (HDLA note, "Key design 3", one step of the general
// recurrence):  state <- D state - A (B^T state) + K V^T,  out = state^T q.
// One workgroup per (batch*head, d_v slice of BV columns); the slice of the
// state is staged in LDS, B^T state is reduced over d_k per column.
struct StepArgs {
  Problem p;
  const void* q;
  const void* k;
  const void* v;
  const float* ld;
  const void* A;
  const void* B;
  float* state;
  void* out;
  int BV;
};

template <typename TI>
__global__ __launch_bounds__(kThreads) void step_kernel(StepArgs a) {
  extern __shared__ float smem[];
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv, r_ab = p.r_ab, r_kv = p.r_kv, BV = a.BV;
  const int nvt = dv / BV;
  const int64_t bh = blockIdx.x / nvt;
  const int c0 = (blockIdx.x % nvt) * BV;
  const int tid = threadIdx.x;
  float* S = smem;              // dk x BV
  float* Wr = S + dk * BV;      // r_ab x BV : (B^T S)
  const TI* qp = static_cast<const TI*>(a.q);
  const TI* kp = static_cast<const TI*>(a.k);
  const TI* vp = static_cast<const TI*>(a.v);
  const TI* Ap = static_cast<const TI*>(a.A);
  const TI* Bp = static_cast<const TI*>(a.B);
  float* st = a.state + static_cast<size_t>(bh) * dk * dv;

  for (int e = tid; e < dk * BV; e += kThreads) S[e] = st[(e / BV) * dv + c0 + e % BV];
  __syncthreads();
  for (int e = tid; e < r_ab * BV; e += kThreads) {
    const int r = e / BV, c = e % BV;
    float s = 0.f;
    for (int i = 0; i < dk; ++i)
      s += Elem<TI>::load(Bp, (static_cast<size_t>(bh) * r_ab + r) * dk + i) * S[i * BV + c];
    Wr[e] = s;
  }
  __syncthreads();
  for (int e = tid; e < dk * BV; e += kThreads) {
    const int i = e / BV, c = e % BV;
    const float l = p.scalar ? a.ld[bh] : a.ld[static_cast<size_t>(bh) * dk + i];
    float s = expf(l) * S[e];
    for (int r = 0; r < r_ab; ++r)
      s -= Elem<TI>::load(Ap, (static_cast<size_t>(bh) * r_ab + r) * dk + i) * Wr[r * BV + c];
    for (int r = 0; r < r_kv; ++r)
      s += Elem<TI>::load(kp, (static_cast<size_t>(bh) * r_kv + r) * dk + i) *
           Elem<TI>::load(vp, (static_cast<size_t>(bh) * r_kv + r) * dv + c0 + c);
    S[e] = s;
  }
  __syncthreads();
  for (int e = tid; e < dk * BV; e += kThreads) st[(e / BV) * dv + c0 + e % BV] = S[e];
  for (int c = tid; c < BV; c += kThreads) {
    float s = 0.f;
    for (int i = 0; i < dk; ++i) s += S[i * BV + c] * Elem<TI>::load(qp, static_cast<size_t>(bh) * dk + i);
    Elem<TI>::store(static_cast<TI*>(a.out), static_cast<size_t>(bh) * dv + c0 + c, s);
  }
}

// ---------------------------------------------------------------------------
// HDLA decay operands (HDLA note, "Key design 2"/"Key design 3"): one wave per
// token.  u = lambda (.) k, c = k^T u, A = [b k, b u], B = [u - b c k, k], V = b v.
struct HdlaArgs {
  Problem p;
  const void* k;
  const void* v;
  const float* ll;
  const float* beta;
  void* A;
  void* B;
  void* V;
};

template <typename TI>
__global__ __launch_bounds__(kThreads) void hdla_params_kernel(HdlaArgs a) {
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv;
  const int lane = threadIdx.x & 63;
  const int64_t tok = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (tok >= p.BH * p.T) return;
  const TI* kp = static_cast<const TI*>(a.k) + static_cast<size_t>(tok) * dk;
  const float* lp = a.ll + static_cast<size_t>(tok) * dk;
  const float b = a.beta[tok];
  float c = 0.f;
  for (int i = lane; i < dk; i += 64) {
    const float kv = Elem<TI>::load(kp, i);
    c += kv * (expf(lp[i]) * kv);
  }
  c = wave_sum(c);
  TI* Ao = static_cast<TI*>(a.A) + static_cast<size_t>(tok) * 2 * dk;
  TI* Bo = static_cast<TI*>(a.B) + static_cast<size_t>(tok) * 2 * dk;
  for (int i = lane; i < dk; i += 64) {
    const float kv = Elem<TI>::load(kp, i);
    const float u = expf(lp[i]) * kv;
    Elem<TI>::store(Ao, i, b * kv);
    Elem<TI>::store(Ao, dk + i, b * u);
    Elem<TI>::store(Bo, i, u - b * c * kv);
    Elem<TI>::store(Bo, dk + i, kv);
  }
  const TI* vp = static_cast<const TI*>(a.v) + static_cast<size_t>(tok) * dv;
  TI* Vo = static_cast<TI*>(a.V) + static_cast<size_t>(tok) * dv;
  for (int i = lane; i < dv; i += 64) Elem<TI>::store(Vo, i, b * Elem<TI>::load(vp, i));
}

// Gated DeltaNet operands (HLA note, "Prerequisites: Gated DeltaNet"):
// A = exp(g) b k, B = k, V = b v.  One wave per token.
struct GdnArgs {
  Problem p;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  void* A;
  void* B;
  void* V;
};

template <typename TI>
__global__ __launch_bounds__(kThreads) void gdn_params_kernel(GdnArgs a) {
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv;
  const int lane = threadIdx.x & 63;
  const int64_t tok = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (tok >= p.BH * p.T) return;
  const float b = a.beta[tok];
  const float coef = expf(a.g[tok]) * b;
  const TI* kp = static_cast<const TI*>(a.k) + static_cast<size_t>(tok) * dk;
  TI* Ao = static_cast<TI*>(a.A) + static_cast<size_t>(tok) * dk;
  TI* Bo = static_cast<TI*>(a.B) + static_cast<size_t>(tok) * dk;
  for (int i = lane; i < dk; i += 64) {
    const float kv = Elem<TI>::load(kp, i);
    Elem<TI>::store(Ao, i, coef * kv);
    Elem<TI>::store(Bo, i, kv);
  }
  const TI* vp = static_cast<const TI*>(a.v) + static_cast<size_t>(tok) * dv;
  TI* Vo = static_cast<TI*>(a.V) + static_cast<size_t>(tok) * dv;
  for (int i = lane; i < dv; i += 64) Elem<TI>::store(Vo, i, b * Elem<TI>::load(vp, i));
}

// ---------------------------------------------------------------------------
// Per chunk: max over tokens and channels of -G (chunk-local inclusive
// cumulative log-decay).  One workgroup per chunk, one thread per channel.
// A NaN anywhere in the chunk makes its entry NaN (fmaxf alone would drop it).
__device__ __forceinline__ float nan_max(float a, float b) {
  return (a != a || b != b) ? __builtin_nanf("") : fmaxf(a, b);
}

__global__ __launch_bounds__(kThreads) void decay_range_kernel(Problem p, const float* ld,
                                                               float* chunk_max) {
  __shared__ float red[kThreads / 64];
  const int64_t job = blockIdx.x;
  const int64_t bh = job / p.N, j = job % p.N;
  const int64_t t0 = j * p.C;
  const int n = static_cast<int>(p.T - t0 < p.C ? p.T - t0 : p.C);
  const int64_t tok0 = bh * p.T + t0;
  const int nchan = p.scalar ? 1 : p.dk;
  float m = 0.f;
  for (int i = threadIdx.x; i < nchan; i += kThreads) {
    float g = 0.f;
    for (int t = 0; t < n; ++t) {
      g += p.scalar ? ld[tok0 + t] : ld[(tok0 + t) * p.dk + i];
      m = nan_max(m, -g);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = nan_max(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < kThreads / 64; ++w) r = nan_max(r, red[w]);
    chunk_max[job] = r;
  }
}

__global__ __launch_bounds__(kThreads) void copy_state_kernel(int64_t n, const float* S0, float* Sfin) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) Sfin[i] = S0 ? S0[i] : 0.f;
}

}  // namespace

hipError_t launch_step(const Problem& p, const void* q, const void* k, const void* v,
                       const float* ld, const void* A, const void* B, float* state, void* out,
                       hipStream_t s) {
  const int BV = (p.dv % 32 == 0) ? 32 : 16;
  StepArgs a{p, q, k, v, ld, A, B, state, out, BV};
  const size_t lds = static_cast<size_t>(p.dk + p.r_ab) * BV * sizeof(float);
  const int64_t blocks = p.BH * (p.dv / BV);
  if (blocks == 0) return hipSuccess;
  if (p.bf16)
    hipLaunchKernelGGL(step_kernel<bf16_raw>, dim3(blocks), dim3(kThreads), lds, s, a);
  else
    hipLaunchKernelGGL(step_kernel<float>, dim3(blocks), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_hdla_params(const Problem& p, const void* k, const void* v,
                              const float* log_lambda, const float* beta, void* A, void* B,
                              void* V_out, hipStream_t s) {
  HdlaArgs a{p, k, v, log_lambda, beta, A, B, V_out};
  const int64_t toks = p.BH * p.T;
  if (toks == 0) return hipSuccess;
  const int64_t blocks = (toks + kThreads / 64 - 1) / (kThreads / 64);
  if (p.bf16)
    hipLaunchKernelGGL(hdla_params_kernel<bf16_raw>, dim3(blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(hdla_params_kernel<float>, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gdn_params(const Problem& p, const void* k, const void* v, const float* g,
                             const float* beta, void* A, void* B, void* V_out, hipStream_t s) {
  GdnArgs a{p, k, v, g, beta, A, B, V_out};
  const int64_t toks = p.BH * p.T;
  if (toks == 0) return hipSuccess;
  const int64_t blocks = (toks + kThreads / 64 - 1) / (kThreads / 64);
  if (p.bf16)
    hipLaunchKernelGGL(gdn_params_kernel<bf16_raw>, dim3(blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(gdn_params_kernel<float>, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decay_range(const Problem& p, const float* ld, float* chunk_max, hipStream_t s) {
  const int64_t blocks = p.BH * p.N;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(decay_range_kernel, dim3(blocks), dim3(kThreads), 0, s, p, ld, chunk_max);
  return hipGetLastError();
}

hipError_t launch_copy_state(const Problem& p, const float* S0, float* Sfin, hipStream_t s) {
  const int64_t n = p.BH * p.dk * p.dv;
  if (n == 0 || Sfin == nullptr) return hipSuccess;
  hipLaunchKernelGGL(copy_state_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                     n, S0, Sfin);
  return hipGetLastError();
}

}  // namespace lattn
