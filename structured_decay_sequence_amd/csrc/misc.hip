// Decode step, decay-operand builders and the decay-range check.
#include "common.hpp"
#include "kernels.hpp"

namespace lattn {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Single recurrent token (HDLA note, "Key design 3", one step of the general
// recurrence):  state <- D state - A (B^T state) + K V^T,  out = state^T q.
// Memory-bound: every state element is read and written once.  One workgroup
// of four waves per (batch*head, 64-column slice of d_v): lane c owns column
// c of the slice, wave w owns rows w, w + 4, w + 8, ... (so every state load
// or store of a wave is one contiguous row piece).  Each thread keeps its
// rows in registers; the two sums over d_k (B^T state and state^T q) are a
// per-thread partial over its rows, then a fixed-order sum of the four
// waves' partials through LDS.  The token's vectors (q, K, A, B, exp(l)) are
// staged in LDS once per workgroup.
constexpr int kStepWaves = 4;
constexpr int kStepCols = 64;

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
};

// RPT is the register bucket of rows per thread; EXACT means d_k == 4 * RPT,
// so no row of the bucket is unused and every row loop runs unguarded.
template <typename TI, int RPT, bool EXACT>
__global__ __launch_bounds__(kStepWaves * 64) void step_kernel(StepArgs a) {
  extern __shared__ float smem[];
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv, r_ab = p.r_ab, r_kv = p.r_kv;
  const int nsl = (dv + kStepCols - 1) / kStepCols;
  const int64_t bh = blockIdx.x / nsl;
  const int c0 = (blockIdx.x % nsl) * kStepCols;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = c0 + lane;
  const bool col = c < dv;
  const int cl = col ? c : dv - 1;        // loads of a column past d_v read a valid one
  const int nm = EXACT ? RPT : dk / kStepWaves;   // rows per thread: d_k is a multiple of 16
  // LDS: q [dk], exp(l) [dk], K [r_kv][dk], A [r_ab][dk], B [r_ab][dk], then the
  // wave partials of B^T state [4][r_ab][64] and of the readout [4][64].
  float* qs = smem;
  float* es = qs + dk;
  float* ks = es + dk;
  float* as = ks + r_kv * dk;
  float* bs = as + r_ab * dk;
  float* wpart = bs + r_ab * dk;
  float* opart = wpart + kStepWaves * r_ab * kStepCols;
  // Every global load is issued before any is waited on, so the step costs one
  // memory round trip: this thread's state rows i = wave + 4m (m < nm) of
  // column c first, then the token's vectors (thread t holds element t; d_k is
  // at most the 256 threads), then V_t for this column.
  float* srow = a.state + bh * dk * dv + static_cast<int64_t>(wave) * dv + cl;
  const int64_t rstride = static_cast<int64_t>(kStepWaves) * dv;
  float S[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) S[m] = m < nm ? srow[m * rstride] : 0.f;
  const int t = threadIdx.x < dk ? threadIdx.x : dk - 1;
  // The loads are unconditional (rank indices clamped, rank-0 A and B read q
  // instead) and the unused values are dropped afterwards, so no branch holds
  // a load back.
  const TI* qp = static_cast<const TI*>(a.q) + bh * dk;
  const TI* kp = static_cast<const TI*>(a.k) + bh * r_kv * dk;
  const int ra = r_ab > 0 ? r_ab : 1;
  const TI* Ap = r_ab > 0 ? static_cast<const TI*>(a.A) + bh * r_ab * dk : qp;
  const TI* Bp = r_ab > 0 ? static_cast<const TI*>(a.B) + bh * r_ab * dk : qp;
  const float qv = Elem<TI>::load(qp, t);
  const float lv = p.scalar ? a.ld[bh] : a.ld[bh * dk + t];
  float kv[4], av[8], bv[8], vv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) kv[r] = Elem<TI>::load(kp, (r < r_kv ? r : r_kv - 1) * dk + t);
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    av[r] = Elem<TI>::load(Ap, (r < ra ? r : ra - 1) * dk + t);
    bv[r] = Elem<TI>::load(Bp, (r < ra ? r : ra - 1) * dk + t);
  }
  const TI* vp = static_cast<const TI*>(a.v) + bh * r_kv * dv + cl;
#pragma unroll
  for (int r = 0; r < 4; ++r) vv[r] = Elem<TI>::load(vp, static_cast<size_t>(r < r_kv ? r : r_kv - 1) * dv);
  if (threadIdx.x < dk) {
    qs[t] = qv;
    es[t] = expf(lv);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r < r_kv) ks[r * dk + t] = kv[r];
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (r < r_ab) {
        as[r * dk + t] = av[r];
        bs[r * dk + t] = bv[r];
      }
  }
  __syncthreads();
  // B^T state: partial over this thread's rows, per decay rank.
  for (int r = 0; r < r_ab; ++r) {
    const float* br = bs + r * dk + wave;
    float w = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m)
      if (m < nm) w += br[kStepWaves * m] * S[m];
    wpart[(wave * r_ab + r) * kStepCols + lane] = w;
  }
  __syncthreads();
  // The update of this thread's rows: decay, the low-rank correction with the
  // summed partials, the write.
#pragma unroll
  for (int m = 0; m < RPT; ++m)
    if (m < nm) S[m] *= es[wave + kStepWaves * m];
  for (int r = 0; r < r_ab; ++r) {
    float w = 0.f;
#pragma unroll
    for (int u = 0; u < kStepWaves; ++u) w += wpart[(u * r_ab + r) * kStepCols + lane];
    const float* ar = as + r * dk + wave;
#pragma unroll
    for (int m = 0; m < RPT; ++m)
      if (m < nm) S[m] -= ar[kStepWaves * m] * w;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r < r_kv) {
      const float* kr = ks + r * dk + wave;
#pragma unroll
      for (int m = 0; m < RPT; ++m)
        if (m < nm) S[m] += kr[kStepWaves * m] * vv[r];
    }
  }
  float o = 0.f;
#pragma unroll
  for (int m = 0; m < RPT; ++m)
    if (m < nm) o += S[m] * qs[wave + kStepWaves * m];
  opart[wave * kStepCols + lane] = o;
  if (col) {
#pragma unroll
    for (int m = 0; m < RPT; ++m)
      if (m < nm) srow[m * rstride] = S[m];
  }
  __syncthreads();
  if (wave == 0 && col) {
    float r = 0.f;
#pragma unroll
    for (int u = 0; u < kStepWaves; ++u) r += opart[u * kStepCols + lane];
    Elem<TI>::store(static_cast<TI*>(a.out), static_cast<size_t>(bh) * dv + c, r);
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

template <typename TI, int RPT>
void launch_step_rows(const Problem& p, const StepArgs& a, size_t lds, int64_t blocks, hipStream_t s) {
  if (p.dk == kStepWaves * RPT)
    hipLaunchKernelGGL((step_kernel<TI, RPT, true>), dim3(blocks), dim3(kStepWaves * 64), lds, s, a);
  else
    hipLaunchKernelGGL((step_kernel<TI, RPT, false>), dim3(blocks), dim3(kStepWaves * 64), lds, s, a);
}

template <typename TI>
hipError_t launch_step_t(const Problem& p, const StepArgs& a, size_t lds, int64_t blocks, hipStream_t s) {
  // Rows per thread: the smallest bucket with 4 * RPT >= d_k.
  if (p.dk <= 16)
    launch_step_rows<TI, 4>(p, a, lds, blocks, s);
  else if (p.dk <= 32)
    launch_step_rows<TI, 8>(p, a, lds, blocks, s);
  else if (p.dk <= 64)
    launch_step_rows<TI, 16>(p, a, lds, blocks, s);
  else if (p.dk <= 128)
    launch_step_rows<TI, 32>(p, a, lds, blocks, s);
  else
    launch_step_rows<TI, 64>(p, a, lds, blocks, s);
  return hipGetLastError();
}

hipError_t launch_step(const Problem& p, const void* q, const void* k, const void* v,
                       const float* ld, const void* A, const void* B, float* state, void* out,
                       hipStream_t s) {
  if (p.r_ab > 8 || p.r_kv > 4 || p.dk > 256) return hipErrorInvalidValue;
  StepArgs a{p, q, k, v, ld, A, B, state, out};
  const size_t lds = (static_cast<size_t>(2 + p.r_kv + 2 * p.r_ab) * p.dk +
                      static_cast<size_t>(kStepWaves) * (p.r_ab + 1) * kStepCols) * sizeof(float);
  const int64_t blocks = p.BH * ((p.dv + kStepCols - 1) / kStepCols);
  if (blocks == 0) return hipSuccess;
  return p.bf16 ? launch_step_t<bf16_raw>(p, a, lds, blocks, s) : launch_step_t<float>(p, a, lds, blocks, s);
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
