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
// accumulate).  The query rows are independent (each carries its own gates),
// so a workgroup takes 64 rows of a gating chunk: a gating chunk of L tokens
// spreads over L / 64 workgroups.  Each
// wave keeps one column tile of O (c_v = w % (d_v/16)) and of R
// (c_k = w % (d_k/16)) and the row tiles w / n_c + (NWV / n_c) u, so the B
// operands of a history chunk (Acal_j^T and B_j^T column tiles, bf16 in
// memory) are loaded once per wave, one history chunk ahead together with its
// gates, while the current chunk's products run.  R is carried in fp32 by the
// wave that owns each tile; its bf16 copy in LDS (rows padded to d_k + 16) is
// the A operand of the next chunk's products.
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

constexpr int kHcRows = 64;   // query rows per workgroup (one gate per lane)
constexpr int kHcWaves = 8;

// A barrier that orders LDS only: the next history chunk's global loads stay
// in flight across it.
__device__ __forceinline__ void hc_lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int DK, int DV>
__global__ __launch_bounds__(64 * kHcWaves) void hla_compose_bf16_kernel(HlaBf16Args a) {
  constexpr int NWV = kHcWaves, CR = kHcRows;
  constexpr int LDR = DK + 16;                 // bf16 per row of the A-operand copy of R
  constexpr int KB = DK / 32;                  // 32-deep K steps
  constexpr int NCV = DV / 16, NCK = DK / 16;  // column tiles of O and of R
  constexpr int NRT = CR / 16;                 // row tiles
  static_assert(NWV % NCV == 0 && NWV % NCK == 0, "whole column tiles per wave");
  constexpr int SV = NWV / NCV, SK = NWV / NCK;   // row-tile strides
  static_assert(NRT % SV == 0 && NRT % SK == 0, "whole row tiles per wave");
  constexpr int TV = NRT / SV, TK = NRT / SK;     // row tiles per wave, of O and of R
  extern __shared__ __align__(16) unsigned char smem[];
  const Problem& p = a.p;
  const int C = p.C;
  const int N = static_cast<int>(p.N);
  const int RS = C / CR;                       // row blocks per gating chunk
  // Blocks go round-robin over the 8 XCDs, so block b takes a head with
  // bh % 8 == b % 8: each XCD's L2 then holds the history operands of its
  // own heads only, which every query chunk and row block of those heads reads.
  const int64_t per = (p.BH + 7) / 8 * 8 * RS;
  const int c = N - 1 - static_cast<int>(blockIdx.x / per);   // longest walks first
  const int64_t rem = blockIdx.x % per, grp = rem / 8;
  const int64_t bh = (grp / RS) * 8 + rem % 8;
  if (bh >= p.BH) return;                      // past the last head (the whole workgroup)
  const int r0 = static_cast<int>(grp % RS) * CR;             // first query row of the block
  const int64_t job = bh * N + c;
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const int64_t left = p.T - t0 - r0;
  if (left <= 0) return;                       // rows past the sequence (the whole workgroup)
  const int n = static_cast<int>(left < CR ? left : CR);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  __bf16* Rb = reinterpret_cast<__bf16*>(smem);
  const int cv = wave % NCV, ck = wave % NCK;
  const int rv0 = wave / NCV, rk0 = wave / NCK;
  const float* Qc = a.QB + (static_cast<size_t>(job) * C + r0) * DK;
  const float* Oc = a.OI + (static_cast<size_t>(job) * C + r0) * DV;
  // Every row of the block lies inside the gating chunk's QB and OI rows, so
  // the loads go out unconditionally, all before the first use; rows past
  // the sequence are zeroed after.
  f32x4 O[TV], Rf[TK];
#pragma unroll
  for (int u = 0; u < TV; ++u) {
    const int rt = rv0 + SV * u;
#pragma unroll
    for (int e = 0; e < 4; ++e) O[u][e] = Oc[static_cast<size_t>(rt * 16 + 4 * lg + e) * DV + cv * 16 + lr];
  }
#pragma unroll
  for (int u = 0; u < TK; ++u) {
    const int rt = rk0 + SK * u;
#pragma unroll
    for (int e = 0; e < 4; ++e) Rf[u][e] = Qc[static_cast<size_t>(rt * 16 + 4 * lg + e) * DK + ck * 16 + lr];
  }
#pragma unroll
  for (int u = 0; u < TV; ++u) {
    const int rt = rv0 + SV * u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (rt * 16 + 4 * lg + e >= n) O[u][e] = 0.f;
  }
#pragma unroll
  for (int u = 0; u < TK; ++u) {
    const int rt = rk0 + SK * u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = rt * 16 + 4 * lg + e;
      if (t >= n) Rf[u][e] = 0.f;
      Rb[t * LDR + ck * 16 + lr] = (__bf16)Rf[u][e];
    }
  }
  const float* gb = a.gates + static_cast<size_t>(bh * p.T + t0 + r0) * N;
  const float theta = a.theta;
  // this wave's B-operand rows of history chunk j, and the gate of row
  // `lane` (every wave loads all 64, so each decides alone whether the chunk
  // is active, and all decide alike)
  const size_t bts = static_cast<size_t>(DV) * DK, ats = static_cast<size_t>(DK) * DK;
  const __bf16* BTb = a.BT + static_cast<size_t>(bh) * N * bts + static_cast<size_t>(cv * 16 + lr) * DK + 8 * lg;
  const __bf16* ATb = a.AT + static_cast<size_t>(bh) * N * ats + static_cast<size_t>(ck * 16 + lr) * DK + 8 * lg;
  hbf16x8 nv[KB], nk[KB];
  float ng = 0.f;
  auto fetch = [&](int j) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      nv[kb] = *reinterpret_cast<const hbf16x8*>(BTb + j * bts + kb * 32);
      nk[kb] = *reinterpret_cast<const hbf16x8*>(ATb + j * ats + kb * 32);
    }
    ng = lane < n ? gb[static_cast<size_t>(lane) * N + j] : 0.f;
  };
  if (c > 0) fetch(c - 1);
  hc_lds_barrier();
  for (int j = c - 1; j >= 0; --j) {
    hbf16x8 bfv[KB], bfk[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      bfv[kb] = nv[kb];
      bfk[kb] = nk[kb];
    }
    const float w = ng;
    if (j > 0) fetch(j - 1);
    // Only a gate below the threshold counts as 0; a NaN gate is applied (and
    // propagates), so it keeps the chunk active.
    if (__ballot(lane < n && !(w < theta)) == 0) continue;
    const float g = w < theta ? 0.f : w;   // rows past the sequence hold 0
    // O += diag(g) R B_j
#pragma unroll
    for (int u = 0; u < TV; ++u) {
      const int rt = rv0 + SV * u;
      const __bf16* arow = Rb + (rt * 16 + lr) * LDR + 8 * lg;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const hbf16x8*>(arow + kb * 32), bfv[kb], acc,
                                                      0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) O[u][e] += __shfl(g, rt * 16 + 4 * lg + e, 64) * acc[e];
    }
    // R <- R + diag(g) (R Acal_j - R), in fp32 by the owning wave
#pragma unroll
    for (int u = 0; u < TK; ++u) {
      const int rt = rk0 + SK * u;
      const __bf16* arow = Rb + (rt * 16 + lr) * LDR + 8 * lg;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const hbf16x8*>(arow + kb * 32), bfk[kb], acc,
                                                      0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) Rf[u][e] += __shfl(g, rt * 16 + 4 * lg + e, 64) * (acc[e] - Rf[u][e]);
    }
    hc_lds_barrier();   // every product has read the bf16 copy of R
#pragma unroll
    for (int u = 0; u < TK; ++u) {
      const int rt = rk0 + SK * u;
#pragma unroll
      for (int e = 0; e < 4; ++e) Rb[(rt * 16 + 4 * lg + e) * LDR + ck * 16 + lr] = (__bf16)Rf[u][e];
    }
    hc_lds_barrier();
  }
  __bf16* op = static_cast<__bf16*>(a.out);
#pragma unroll
  for (int u = 0; u < TV; ++u) {
    const int rt = rv0 + SV * u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = rt * 16 + 4 * lg + e;
      if (t < n) op[static_cast<size_t>(bh * p.T + t0 + r0 + t) * DV + cv * 16 + lr] = (__bf16)O[u][e];
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

template <int DK, int DV>
hipError_t launch_compose_bf16_t(const Problem& p, const HlaBf16Args& ca, hipStream_t s) {
  const size_t lds = static_cast<size_t>(kHcRows) * (DK + 16) * 2;
  const void* fn = reinterpret_cast<const void*>(hla_compose_bf16_kernel<DK, DV>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const int64_t blocks = (p.BH + 7) / 8 * 8 * p.N * (p.C / kHcRows);
  hipLaunchKernelGGL((hla_compose_bf16_kernel<DK, DV>), dim3(static_cast<unsigned>(blocks)), dim3(64 * kHcWaves), lds,
                     s, ca);
  return hipGetLastError();
}

hipError_t launch_compose_bf16(const Problem& p, const float* QB, const __bf16* AT, const __bf16* BT, const float* OI,
                               const float* gates, float theta, void* out, hipStream_t s) {
  HlaBf16Args ca{p, QB, AT, BT, OI, gates, theta, out};
  if (p.C % kHcRows != 0) return hipErrorInvalidValue;   // gating chunks of whole row blocks
  if (p.dk == 128 && p.dv == 128) return launch_compose_bf16_t<128, 128>(p, ca, s);
  if (p.dk == 128 && p.dv == 64) return launch_compose_bf16_t<128, 64>(p, ca, s);
  if (p.dk == 64 && p.dv == 128) return launch_compose_bf16_t<64, 128>(p, ca, s);
  if (p.dk == 64 && p.dv == 64) return launch_compose_bf16_t<64, 64>(p, ca, s);
  return hipErrorInvalidValue;
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
