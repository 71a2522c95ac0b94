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
//
// The gating chunk may be longer than the summary chunk: on the bf16 path a
// gating chunk of L = 64, 128 or 256 tokens is summarised from 1, 2 or 4
// consecutive 64-token chunk operators by fast_gate_summaries (bf16 MFMAs on
// the prepare's fragment-ordered tiles); elsewhere the summary chunk is the
// gating chunk (at most 128 tokens) and hla_summaries_kernel reads the general
// path's fp32 operators.  Either way the composition below sees, per gating
// chunk, Acal^T, B^T, the queries' incoming-state operator QB and their
// zero-state outputs OI.
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
  float* QB;        // Qbar_j     [BH, N, C, dk]
  float* OI;        // R_j V_j    [BH, N, C, dv]
};

// Per chunk: Acal^T, Qbar, and [Z ; R] V_j with the top rows stored transposed.
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
  float* QB = a.QB + static_cast<size_t>(job) * C * dk;
  for (int e = tid; e < C * dk; e += 256) QB[e] = Mj[static_cast<size_t>(dk + e / dk) * ncol + e % dk];
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
  Problem p;        // C is the gating chunk, N the gating chunks per (batch, head)
  const float* QB;
  const float* AT;
  const float* BT;
  const float* OI;
  const float* gates;   // [BH, T, N]
  float theta;
  void* out;
};

constexpr int kHlaTiles = 8;       // tiles of R and of O per wave: (C/16)(d/16) <= 8 NWV

// One workgroup per (batch*head, query chunk c), longest walks first.  R
// (C x d_k, fp32) lives in LDS; wave w owns O tiles w, w+NWV, ... (in registers
// for the whole walk) and the same R tiles, whose new values are written back
// after a barrier.  NWV = 8 waves for chunks up to 128 tokens, 16 for 256.
template <typename TI, int NWV>
__global__ __launch_bounds__(64 * NWV) void hla_compose_kernel(HlaArgs a) {
  constexpr int kHlaThreads = 64 * NWV;
  extern __shared__ __align__(16) float Rs[];
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv, C = p.C;
  const int N = static_cast<int>(p.N);
  const int LDR = dk + 4;
  // Query chunk c walks c history chunks: the workgroups are dispatched
  // longest walk first (c descending), so short walks fill in at the end.
  const int c = N - 1 - static_cast<int>(blockIdx.x / p.BH);
  const int64_t bh = blockIdx.x % p.BH;
  const int64_t job = bh * N + c;
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const int n = static_cast<int>(p.T - t0 < C ? p.T - t0 : C);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int nrt = C / 16, nctv = dv / 16, nctk = dk / 16;
  const int nO = nrt * nctv, nR = nrt * nctk;
  const float* Qc = a.QB + static_cast<size_t>(job) * C * dk;
  const float* gb = a.gates + static_cast<size_t>(bh * p.T + t0) * N;   // row t: gb[t * N + j]
  const float theta = a.theta;

  for (int e = tid; e < C * dk; e += kHlaThreads) {
    const int t = e / dk, i = e % dk;
    Rs[t * LDR + i] = t < n ? Qc[static_cast<size_t>(t) * dk + i] : 0.f;   // Qbar_c
  }
  f32x4 O[kHlaTiles], Rn[kHlaTiles];
#pragma unroll
  for (int u = 0; u < kHlaTiles; ++u) {
    O[u] = zero4();
    Rn[u] = zero4();
    const int o = wave + NWV * u;
    if (o < nO) {
      const int rt = o / nctv, ct = o % nctv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = rt * 16 + 4 * lg + e;
        O[u][e] = t < n ? a.OI[(static_cast<size_t>(job) * C + t) * dv + ct * 16 + lr] : 0.f;
      }
    }
  }
  float* gs = Rs + C * LDR;   // gates of the current history chunk per row (below theta, or past the end: 0)
  __syncthreads();

  // Per history chunk, wave w runs up to 2 kHlaTiles tile products: task 2u is
  // its O tile w + 8u (B_j^T fragments), task 2u + 1 its R tile w + 8u
  // (Acal_j^T fragments).  The next task's fragments are loaded while the
  // current task's MFMAs run.
  auto task = [&](const float* ATj, const float* BTj, int k, int& rt, int& ct, const float*& bp) {
    const int idx = wave + NWV * (k >> 1);
    if ((k & 1) == 0) {
      if (idx >= nO) return false;
      rt = idx / nctv;
      ct = idx % nctv;
      bp = BTj + static_cast<size_t>(ct * 16 + lr) * dk + 4 * lg;
    } else {
      if (idx >= nR) return false;
      rt = idx / nctk;
      ct = idx % nctk;
      bp = ATj + static_cast<size_t>(ct * 16 + lr) * dk + 4 * lg;
    }
    return true;
  };
  for (int j = c - 1; j >= 0; --j) {
    int act = 0;
    for (int t = tid; t < C; t += kHlaThreads) {
      const float w = t < n ? gb[static_cast<size_t>(t) * N + j] : 0.f;
      // Only a gate below the threshold counts as 0; a NaN gate is applied
      // (and propagates), so it keeps the chunk active.
      act |= !(w < theta);
      gs[t] = w < theta ? 0.f : w;
    }
    if (!__syncthreads_or(act)) continue;
    const float* ATj = a.AT + static_cast<size_t>(bh * N + j) * dk * dk;
    const float* BTj = a.BT + static_cast<size_t>(bh * N + j) * dv * dk;
    f32x4 bf[2][8];
    auto fetch = [&](int k, f32x4 (&f)[8]) {
      int rt, ct;
      const float* bp;
      if (!task(ATj, BTj, k, rt, ct, bp)) return;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        if (kb < nctk) f[kb] = ld4(bp + kb * 16);
    };
    fetch(0, bf[0]);
#pragma unroll
    for (int k = 0; k < 2 * kHlaTiles; ++k) {
      if (k + 1 < 2 * kHlaTiles) fetch(k + 1, bf[(k + 1) & 1]);
      int rt, ct;
      const float* bp;
      if (!task(ATj, BTj, k, rt, ct, bp)) continue;
      const float* arow = Rs + (rt * 16 + lr) * LDR + 4 * lg;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        if (kb < nctk) acc = mfma16(ld4(arow + kb * 16), bf[k & 1][kb], acc);
      const int u = k >> 1;
      if ((k & 1) == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) O[u][e] += gs[rt * 16 + 4 * lg + e] * acc[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = rt * 16 + 4 * lg + e;
          const float old = Rs[t * LDR + ct * 16 + lr];
          Rn[u][e] = old + gs[t] * (acc[e] - old);
        }
      }
    }
    __syncthreads();   // every product has read R
#pragma unroll
    for (int u = 0; u < kHlaTiles; ++u) {
      const int r = wave + NWV * u;
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
    const int o = wave + NWV * u;
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

// The same composition on the bf16 path, on bf16 MFMAs (16x16x32, fp32
// accumulate).  Each wave keeps one column tile of O (c_v = w % (d_v/16)) and
// of R (c_k = w % (d_k/16)) and the row tiles w / n_c + (NWV / n_c) u, so the
// B operands of a history chunk (Acal_j^T and B_j^T column tiles, bf16 in
// memory) are loaded once per wave.  R is carried in fp32 by the wave that
// owns each tile; its bf16 copy in LDS (rows padded to d_k + 16) is the A
// operand of the next chunk's products.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 hbf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 hbf16x4;

struct HlaBf16Args {
  Problem p;        // C is the gating chunk, N the gating chunks per (batch, head)
  const float* QB;
  const __bf16* AT;
  const __bf16* BT;
  const float* OI;
  const float* gates;
  float theta;
  void* out;
};

template <int NWV, int DK, int DV>
__global__ __launch_bounds__(64 * NWV) void hla_compose_bf16_kernel(HlaBf16Args a) {
  constexpr int LDR = DK + 16;                 // bf16 per row of the A-operand copy of R
  constexpr int KB = DK / 32;                  // 32-deep K steps
  constexpr int NCV = DV / 16, NCK = DK / 16;  // column tiles of O and of R
  static_assert(NWV % NCV == 0 && NWV % NCK == 0, "whole column tiles per wave");
  extern __shared__ __align__(16) unsigned char smem[];
  const Problem& p = a.p;
  const int C = p.C;
  const int N = static_cast<int>(p.N);
  const int c = N - 1 - static_cast<int>(blockIdx.x / p.BH);   // longest walks first
  const int64_t bh = blockIdx.x % p.BH;
  const int64_t job = bh * N + c;
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const int n = static_cast<int>(p.T - t0 < C ? p.T - t0 : C);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int nrt = C / 16;
  __bf16* Rb = reinterpret_cast<__bf16*>(smem);
  float* gs = reinterpret_cast<float*>(smem + static_cast<size_t>(C) * LDR * 2);
  const int cv = wave % NCV, ck = wave % NCK;
  const int rv0 = wave / NCV, rk0 = wave / NCK;
  constexpr int SV = NWV / NCV, SK = NWV / NCK;   // row-tile strides
  const int nov = (nrt - rv0 + SV - 1) / SV, nok = (nrt - rk0 + SK - 1) / SK;   // tiles this wave owns
  const float* Qc = a.QB + static_cast<size_t>(job) * C * DK;
  const float* Oc = a.OI + static_cast<size_t>(job) * C * DV;
  f32x4 O[kHlaTiles], Rf[kHlaTiles];
#pragma unroll
  for (int u = 0; u < kHlaTiles; ++u) {
    O[u] = zero4();
    Rf[u] = zero4();
    if (u < nov) {
      const int rt = rv0 + SV * u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = rt * 16 + 4 * lg + e;
        O[u][e] = t < n ? Oc[static_cast<size_t>(t) * DV + cv * 16 + lr] : 0.f;
      }
    }
    if (u < nok) {
      const int rt = rk0 + SK * u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = rt * 16 + 4 * lg + e;
        const float r = t < n ? Qc[static_cast<size_t>(t) * DK + ck * 16 + lr] : 0.f;
        Rf[u][e] = r;
        Rb[t * LDR + ck * 16 + lr] = (__bf16)r;
      }
    }
  }
  const float* gb = a.gates + static_cast<size_t>(bh * p.T + t0) * N;
  const float theta = a.theta;
  __syncthreads();
  for (int j = c - 1; j >= 0; --j) {
    int act = 0;
    for (int t = tid; t < C; t += 64 * NWV) {
      const float w = t < n ? gb[static_cast<size_t>(t) * N + j] : 0.f;
      // Only a gate below the threshold counts as 0; a NaN gate is applied
      // (and propagates), so it keeps the chunk active.
      act |= !(w < theta);
      gs[t] = w < theta ? 0.f : w;
    }
    if (!__syncthreads_or(act)) continue;
    const __bf16* BTj = a.BT + (static_cast<size_t>(bh) * N + j) * DV * DK + static_cast<size_t>(cv * 16 + lr) * DK;
    const __bf16* ATj = a.AT + (static_cast<size_t>(bh) * N + j) * DK * DK + static_cast<size_t>(ck * 16 + lr) * DK;
    hbf16x8 bfv[KB], bfk[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      bfv[kb] = *reinterpret_cast<const hbf16x8*>(BTj + kb * 32 + 8 * lg);
      bfk[kb] = *reinterpret_cast<const hbf16x8*>(ATj + kb * 32 + 8 * lg);
    }
    // O += diag(g) R B_j
#pragma unroll
    for (int u = 0; u < kHlaTiles; ++u) {
      if (u < nov) {
        const int rt = rv0 + SV * u;
        const __bf16* arow = Rb + (rt * 16 + lr) * LDR + 8 * lg;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const hbf16x8*>(arow + kb * 32), bfv[kb], acc,
                                                        0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) O[u][e] += gs[rt * 16 + 4 * lg + e] * acc[e];
      }
    }
    // R <- R + diag(g) (R Acal_j - R), in fp32 by the owning wave
#pragma unroll
    for (int u = 0; u < kHlaTiles; ++u) {
      if (u < nok) {
        const int rt = rk0 + SK * u;
        const __bf16* arow = Rb + (rt * 16 + lr) * LDR + 8 * lg;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const hbf16x8*>(arow + kb * 32), bfk[kb], acc,
                                                        0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) Rf[u][e] += gs[rt * 16 + 4 * lg + e] * (acc[e] - Rf[u][e]);
      }
    }
    __syncthreads();   // every product has read the bf16 copy of R
#pragma unroll
    for (int u = 0; u < kHlaTiles; ++u) {
      if (u < nok) {
        const int rt = rk0 + SK * u;
#pragma unroll
        for (int e = 0; e < 4; ++e) Rb[(rt * 16 + 4 * lg + e) * LDR + ck * 16 + lr] = (__bf16)Rf[u][e];
      }
    }
    __syncthreads();
  }
  __bf16* op = static_cast<__bf16*>(a.out);
#pragma unroll
  for (int u = 0; u < kHlaTiles; ++u) {
    if (u < nov) {
      const int rt = rv0 + SV * u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = rt * 16 + 4 * lg + e;
        if (t < n) op[static_cast<size_t>(bh * p.T + t0 + t) * DV + cv * 16 + lr] = (__bf16)O[u][e];
      }
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

// The bf16 path: the 64-token operators of the MFMA prepare, summarised per
// gating chunk of 64, 128 or 256 tokens.
bool hla_fast(const Problem& p) {
  return p.bf16 && (p.dk == 64 || p.dk == 128) && p.r_kv == 1 && p.r_ab >= 0 && p.r_ab <= 2 && p.dv % 64 == 0 &&
         p.dv <= 128 && (p.C == 64 || p.C == 128 || p.C == 256);
}

Problem hla_sub_problem(const Problem& p) {
  Problem q = p;
  q.C = 64;
  q.N = (p.T + 63) / 64;
  return q;
}

bool hla_supported(const Problem& p) {
  return p.dk <= 128 && p.dv <= 128 && (p.C <= 128 || hla_fast(p));
}

HlaPlan hla_plan(const Problem& p) {
  HlaPlan h{};
  const size_t chunks = static_cast<size_t>(p.BH * p.N);   // gating chunks
  h.gen_bytes = align256(hla_fast(p) ? fast_workspace_bytes(hla_sub_problem(p)) : f32_operators_bytes(p));
  h.at_bytes = align256(chunks * p.dk * p.dk * sizeof(float));
  h.bt_bytes = align256(chunks * p.dv * p.dk * sizeof(float));
  h.qb_bytes = align256(chunks * p.C * p.dk * sizeof(float));
  h.oi_bytes = align256(chunks * p.C * p.dv * sizeof(float));
  h.total_bytes = h.gen_bytes + h.at_bytes + h.bt_bytes + h.qb_bytes + h.oi_bytes;
  return h;
}

template <int NWV, int DK, int DV>
hipError_t launch_compose_bf16_t(const Problem& p, const HlaBf16Args& ca, hipStream_t s) {
  const size_t lds = static_cast<size_t>(p.C) * (DK + 16) * 2 + static_cast<size_t>(p.C) * sizeof(float);
  const void* fn = reinterpret_cast<const void*>(hla_compose_bf16_kernel<NWV, DK, DV>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((hla_compose_bf16_kernel<NWV, DK, DV>), dim3(static_cast<unsigned>(p.BH * p.N)), dim3(64 * NWV),
                     lds, s, ca);
  return hipGetLastError();
}

template <int NWV>
hipError_t launch_compose_bf16_w(const Problem& p, const HlaBf16Args& ca, hipStream_t s) {
  if (p.dk == 128 && p.dv == 128) return launch_compose_bf16_t<NWV, 128, 128>(p, ca, s);
  if (p.dk == 128 && p.dv == 64) return launch_compose_bf16_t<NWV, 128, 64>(p, ca, s);
  if (p.dk == 64 && p.dv == 128) return launch_compose_bf16_t<NWV, 64, 128>(p, ca, s);
  if (p.dk == 64 && p.dv == 64) return launch_compose_bf16_t<NWV, 64, 64>(p, ca, s);
  return hipErrorInvalidValue;
}

hipError_t launch_compose_bf16(const Problem& p, const float* QB, const __bf16* AT, const __bf16* BT, const float* OI,
                               const float* gates, float theta, void* out, hipStream_t s) {
  HlaBf16Args ca{p, QB, AT, BT, OI, gates, theta, out};
  // enough waves that each owns at most kHlaTiles row tiles of O and of R
  return p.C > 128 ? launch_compose_bf16_w<16>(p, ca, s) : launch_compose_bf16_w<8>(p, ca, s);
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
  float* QB = reinterpret_cast<float*>(ws + h.gen_bytes + h.at_bytes + h.bt_bytes);
  float* OI = reinterpret_cast<float*>(ws + h.gen_bytes + h.at_bytes + h.bt_bytes + h.qb_bytes);
  hipError_t e;
  if (hla_fast(p)) {
    const Problem ps = hla_sub_problem(p);
    e = fast_prepare(ps, q, k, ld, A, B, workspace, s);
    if (e == hipSuccess) e = fast_gate_summaries(ps, p.C / 64, workspace, v, AT, BT, QB, OI, s);
    if (e != hipSuccess) return e;
    return launch_compose_bf16(p, QB, reinterpret_cast<const __bf16*>(AT), reinterpret_cast<const __bf16*>(BT), OI,
                               gates, theta, out, s);
  } else {
    const float* M = nullptr;   // fp32 chunk operators inside the workspace
    e = f32_operators(p, q, k, ld, A, B, workspace, &M, s);
    if (e == hipSuccess) {
      HlaSumArgs sa{p, M, v, AT, BT, QB, OI};
      const dim3 grid(static_cast<unsigned>(p.BH * p.N));
      if (p.bf16)
        hipLaunchKernelGGL(hla_summaries_kernel<bf16_raw>, grid, dim3(256), 0, s, sa);
      else
        hipLaunchKernelGGL(hla_summaries_kernel<float>, grid, dim3(256), 0, s, sa);
      e = hipGetLastError();
    }
  }
  if (e != hipSuccess) return e;
  HlaArgs ca{p, QB, AT, BT, OI, gates, theta, out};
  const size_t lds = static_cast<size_t>(p.C) * (p.dk + 4 + 1) * sizeof(float);   // R, then the row gates
  const dim3 grid(static_cast<unsigned>(p.BH * p.N));
  const bool wide = p.C > 128;
  const void* fn = wide ? (p.bf16 ? reinterpret_cast<const void*>(hla_compose_kernel<bf16_raw, 16>)
                                  : reinterpret_cast<const void*>(hla_compose_kernel<float, 16>))
                        : (p.bf16 ? reinterpret_cast<const void*>(hla_compose_kernel<bf16_raw, 8>)
                                  : reinterpret_cast<const void*>(hla_compose_kernel<float, 8>));
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  if (wide) {
    if (p.bf16)
      hipLaunchKernelGGL((hla_compose_kernel<bf16_raw, 16>), grid, dim3(1024), lds, s, ca);
    else
      hipLaunchKernelGGL((hla_compose_kernel<float, 16>), grid, dim3(1024), lds, s, ca);
  } else {
    if (p.bf16)
      hipLaunchKernelGGL((hla_compose_kernel<bf16_raw, 8>), grid, dim3(512), lds, s, ca);
    else
      hipLaunchKernelGGL((hla_compose_kernel<float, 8>), grid, dim3(512), lds, s, ca);
  }
  return hipGetLastError();
}

}  // namespace lattn
