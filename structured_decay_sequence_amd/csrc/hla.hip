// Query-conditioned composition of exact chunk transitions (HLA note, "Core
// method" and "Method steps", steps 5 and 7), on the chunk operators in
// row-major fp32 (from the bf16 MFMA prepare where it takes the shape and the
// storage is bf16, else from the general prepare).
//
// With the chunk operator M_j = [[Acal_j, Z_j], [Qbar_j, R_j]] of the base
// path (Acal_j the chunk's exact transition, B_j = Z_j V_j its exact write,
// Qbar_j and R_j V_j the chunk's outputs from an incoming state and from a
// zero state), the output of query i in chunk c is
//   o_i = O_intra,i + Qbar_i S_{i,c-1},
//   S_{i,c-1} = sum_{j<c} w_{i,j} (M_{i,c-1} ... M_{i,j+1}) B_j,
//   M_{i,l} = (1 - w_{i,l}) I + w_{i,l} Acal_l,
// since the history starts from a zero state.  Read backwards over the history
// with all queries of chunk c as the rows of R (C x d_k), starting at
// R = Qbar_c and O = O_intra,c:
//   for j = c-1 .. 0:  O += diag(w_{:,j}) R B_j;   R <- R + diag(w_{:,j}) (R Acal_j - R)
// which is one C x d_k x (d_k + d_v) product per (query chunk, history chunk)
// pair.  A history chunk whose gates are all below the threshold (taken as
// zero) leaves R and O unchanged and is skipped.
#include "common.hpp"
#include "kernels.hpp"
#include "tile_f32.hpp"

namespace lattn {
namespace {

struct HlaSumArgs {
  Problem p;
  const float* M;   // row-major fp32 chunk operators
  const void* v;
  float* AT;        // Acal_j^T   [BH, N, dk, dk]
  float* BT;        // B_j^T      [BH, N, dv, dk]
  float* OI;        // R_j V_j    [BH, N, C, dv]
};

// Per chunk: Acal^T, and [Z ; R] V_j with the top rows stored transposed.
template <typename TI>
__global__ __launch_bounds__(256) void hla_summaries_kernel(HlaSumArgs a) {
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv, C = p.C, r_kv = p.r_kv, nk = p.nk(), ncol = p.mcols();
  const int dkT = dk / 16, MT = p.mrows() / 16, CT = dv / 16;
  const int64_t job = blockIdx.x;
  const int64_t bh = job / p.N, j = job % p.N;
  const int64_t t0 = j * C;
  const int n = static_cast<int>(p.T - t0 < C ? p.T - t0 : C);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const float* Mj = a.M + static_cast<size_t>(job) * p.mrows() * ncol;
  const TI* vp = static_cast<const TI*>(a.v);
  float* AT = a.AT + static_cast<size_t>(job) * dk * dk;
  for (int e = tid; e < dk * dk; e += 256) AT[e] = Mj[static_cast<size_t>(e % dk) * ncol + e / dk];
  for (int tile = wave; tile < MT * CT; tile += 4) {
    const int rt = tile / CT, ct = tile % CT;
    const float* arow = Mj + static_cast<size_t>(rt * 16 + lr) * ncol + dk + 4 * lg;
    f32x4 acc = zero4();
    for (int kb = 0; kb < nk / 16; ++kb) {
      f32x4 b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = kb * 16 + 4 * lg + e;   // write row: token m / r_kv of the chunk
        b[e] = m / r_kv < n ? Elem<TI>::load(vp, (static_cast<size_t>(bh * p.T + t0) * r_kv + m) * dv + ct * 16 + lr)
                            : 0.f;
      }
      acc = mfma16(ld4(arow + kb * 16), b, acc);
    }
    if (rt < dkT) {
      st4(a.BT + (static_cast<size_t>(job) * dv + ct * 16 + lr) * dk + rt * 16 + 4 * lg, acc);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = (rt - dkT) * 16 + 4 * lg + e;
        a.OI[(static_cast<size_t>(job) * C + t) * dv + ct * 16 + lr] = acc[e];
      }
    }
  }
}

struct HlaArgs {
  Problem p;
  const float* M;
  const float* AT;
  const float* BT;
  const float* OI;
  const float* gates;   // [BH, T, N]
  float theta;
  void* out;
};

constexpr int kHlaThreads = 512;   // eight waves
constexpr int kHlaTiles = 8;       // tiles of R and of O per wave: (C/16)(d/16) <= 64

// One workgroup per (batch*head, query chunk c).  R (C x d_k, fp32) lives in
// LDS; wave w owns O tiles w, w+8, ... (in registers for the whole walk) and
// the same R tiles, whose new values are written back after a barrier.
template <typename TI>
__global__ __launch_bounds__(kHlaThreads) void hla_compose_kernel(HlaArgs a) {
  extern __shared__ __align__(16) float Rs[];
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv, C = p.C, ncol = p.mcols();
  const int N = static_cast<int>(p.N);
  const int LDR = dk + 4;
  const int64_t job = blockIdx.x;
  const int64_t bh = job / N;
  const int c = static_cast<int>(job % N);
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const int n = static_cast<int>(p.T - t0 < C ? p.T - t0 : C);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int nrt = C / 16, nctv = dv / 16, nctk = dk / 16;
  const int nO = nrt * nctv, nR = nrt * nctk;
  const float* Mc = a.M + static_cast<size_t>(job) * p.mrows() * ncol;
  const float* gb = a.gates + static_cast<size_t>(bh * p.T + t0) * N;   // row t: gb[t * N + j]
  const float theta = a.theta;

  for (int e = tid; e < C * dk; e += kHlaThreads) {
    const int t = e / dk, i = e % dk;
    Rs[t * LDR + i] = Mc[static_cast<size_t>(dk + t) * ncol + i];   // Qbar_c
  }
  f32x4 O[kHlaTiles], Rn[kHlaTiles];
#pragma unroll
  for (int u = 0; u < kHlaTiles; ++u) {
    O[u] = zero4();
    Rn[u] = zero4();
    const int o = wave + 8 * u;
    if (o < nO) {
      const int rt = o / nctv, ct = o % nctv;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        O[u][e] = a.OI[(static_cast<size_t>(job) * C + rt * 16 + 4 * lg + e) * dv + ct * 16 + lr];
    }
  }
  // gate of chunk j for row t of this chunk (rows past its end: 0)
  auto gate = [&](int t, int j) {
    float w = t < n ? gb[static_cast<size_t>(t) * N + j] : 0.f;
    return w < theta ? 0.f : w;
  };
  __syncthreads();

  for (int j = c - 1; j >= 0; --j) {
    int act = 0;
    for (int t = tid; t < n; t += kHlaThreads) act |= gb[static_cast<size_t>(t) * N + j] >= theta;
    if (!__syncthreads_or(act)) continue;
    const float* ATj = a.AT + static_cast<size_t>(bh * N + j) * dk * dk;
    const float* BTj = a.BT + static_cast<size_t>(bh * N + j) * dv * dk;
#pragma unroll
    for (int u = 0; u < kHlaTiles; ++u) {
      const int o = wave + 8 * u;
      if (o < nO) {
        const int rt = o / nctv, ct = o % nctv;
        const float* arow = Rs + (rt * 16 + lr) * LDR + 4 * lg;
        const float* brow = BTj + static_cast<size_t>(ct * 16 + lr) * dk + 4 * lg;
        f32x4 acc = zero4();
        for (int kb = 0; kb < nctk; ++kb) acc = mfma16(ld4(arow + kb * 16), ld4(brow + kb * 16), acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) O[u][e] += gate(rt * 16 + 4 * lg + e, j) * acc[e];
      }
      const int r = wave + 8 * u;
      if (r < nR) {
        const int rt = r / nctk, ct = r % nctk;
        const float* arow = Rs + (rt * 16 + lr) * LDR + 4 * lg;
        const float* brow = ATj + static_cast<size_t>(ct * 16 + lr) * dk + 4 * lg;
        f32x4 acc = zero4();
        for (int kb = 0; kb < nctk; ++kb) acc = mfma16(ld4(arow + kb * 16), ld4(brow + kb * 16), acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = rt * 16 + 4 * lg + e;
          const float old = Rs[t * LDR + ct * 16 + lr];
          Rn[u][e] = old + gate(t, j) * (acc[e] - old);
        }
      }
    }
    __syncthreads();   // every product has read R
#pragma unroll
    for (int u = 0; u < kHlaTiles; ++u) {
      const int r = wave + 8 * u;
      if (r < nR) {
        const int rt = r / nctk, ct = r % nctk;
#pragma unroll
        for (int e = 0; e < 4; ++e) Rs[(rt * 16 + 4 * lg + e) * LDR + ct * 16 + lr] = Rn[u][e];
      }
    }
    __syncthreads();
  }

  TI* op = static_cast<TI*>(a.out);
#pragma unroll
  for (int u = 0; u < kHlaTiles; ++u) {
    const int o = wave + 8 * u;
    if (o < nO) {
      const int rt = o / nctv, ct = o % nctv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = rt * 16 + 4 * lg + e;
        if (t < n) Elem<TI>::store(op, static_cast<size_t>(bh * p.T + t0 + t) * dv + ct * 16 + lr, O[u][e]);
      }
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

bool hla_supported(const Problem& p) { return p.dk <= 128 && p.dv <= 128; }

HlaPlan hla_plan(const Problem& p) {
  HlaPlan h{};
  const size_t chunks = static_cast<size_t>(p.BH * p.N);
  h.gen_bytes = align256(f32_operators_bytes(p));
  h.at_bytes = align256(chunks * p.dk * p.dk * sizeof(float));
  h.bt_bytes = align256(chunks * p.dv * p.dk * sizeof(float));
  h.oi_bytes = align256(chunks * p.C * p.dv * sizeof(float));
  h.total_bytes = h.gen_bytes + h.at_bytes + h.bt_bytes + h.oi_bytes;
  return h;
}

hipError_t launch_hla(const Problem& p, const void* q, const void* k, const float* ld, const void* A,
                      const void* B, const void* v, const float* gates, float theta, void* out,
                      void* workspace, hipStream_t s) {
  if (p.BH * p.N == 0) return hipSuccess;
  if (!hla_supported(p)) return hipErrorInvalidValue;
  const HlaPlan h = hla_plan(p);
  char* ws = static_cast<char*>(workspace);
  float* AT = reinterpret_cast<float*>(ws + h.gen_bytes);
  float* BT = reinterpret_cast<float*>(ws + h.gen_bytes + h.at_bytes);
  float* OI = reinterpret_cast<float*>(ws + h.gen_bytes + h.at_bytes + h.bt_bytes);
  const float* M = nullptr;   // fp32 chunk operators inside the workspace
  hipError_t e = f32_operators(p, q, k, ld, A, B, workspace, &M, s);
  if (e != hipSuccess) return e;
  HlaSumArgs sa{p, M, v, AT, BT, OI};
  const dim3 grid(static_cast<unsigned>(p.BH * p.N));
  if (p.bf16)
    hipLaunchKernelGGL(hla_summaries_kernel<bf16_raw>, grid, dim3(256), 0, s, sa);
  else
    hipLaunchKernelGGL(hla_summaries_kernel<float>, grid, dim3(256), 0, s, sa);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  HlaArgs ca{p, M, AT, BT, OI, gates, theta, out};
  const size_t lds = static_cast<size_t>(p.C) * (p.dk + 4) * sizeof(float);
  const void* fn = p.bf16 ? reinterpret_cast<const void*>(hla_compose_kernel<bf16_raw>)
                          : reinterpret_cast<const void*>(hla_compose_kernel<float>);
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  if (p.bf16)
    hipLaunchKernelGGL(hla_compose_kernel<bf16_raw>, grid, dim3(kHlaThreads), lds, s, ca);
  else
    hipLaunchKernelGGL(hla_compose_kernel<float>, grid, dim3(kHlaThreads), lds, s, ca);
  return hipGetLastError();
}

}  // namespace lattn
