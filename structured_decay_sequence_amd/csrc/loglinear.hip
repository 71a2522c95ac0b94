// Log-linear lift of the recurrence (Log-Linear note, "Key design" 1-4), on
// the chunk operators in row-major fp32 (from the bf16 MFMA prepare where it
// takes the shape and the storage is bf16, else from the general prepare).
//
// Query t weights key s by lam[t, l(t, s)], l the level of s in the Fenwick
// split of t's prefix: 0 for s = t, else the highest bit where t and s differ
// plus one.  With chunks of C = 2^c tokens aligned at multiples of C, keys in
// the query's own chunk have levels <= c, and a key in an earlier chunk I of
// query chunk J has level c + 1 + m with m the highest differing bit of I and
// J.  For each m the earlier chunks at that level form one aligned block:
// the left half of J's block of 2^(m+1) chunks, present when bit m of J is 1.
// So, with the chunk operator M_J = [[Acal_J, Z_J], [Qbar_J, R_J]]:
//   O_J = (R_J (.) Lam_J) V_J + sum_m diag(lam[:, c+1+m]) Qbar_J S^(m)_J,
// where Lam_J[t, s] = lam[t, l(t, s)] inside the chunk and the level-m state
// S^(m) is the recurrence run over the left half of the block from a zero
// state, then carried through the right half by the transitions alone:
//   left half  S^(m) <- Acal_J S^(m) + Z_J V_J   (zero at the block's start)
//   right half read Qbar_J S^(m), then S^(m) <- Acal_J S^(m).
// That is one chunkwise scan per level (the note's O(log T) scans), run here
// in one kernel with every level's state resident in LDS.
#include "common.hpp"
#include "kernels.hpp"
#include "tile_f32.hpp"

namespace lattn {
namespace {

__device__ __forceinline__ int bit_length(unsigned x) { return x == 0 ? 0 : 32 - __clz(x); }

struct LlIntraArgs {
  Problem p;
  const float* M;
  const void* v;
  const float* lam;   // [BH, T, L]
  int L;
  float* ZVT;         // (Z_j V_j)^T   [BH, N, dv, dk]
  float* OI;          // (R_j (.) Lam_j) V_j   [BH, N, C, dv]
};

// Per chunk: [Z ; R (.) Lam] V_j, the top rows stored transposed.
template <typename TI>
__global__ __launch_bounds__(256) void ll_intra_kernel(LlIntraArgs a) {
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
  for (int tile = wave; tile < MT * CT; tile += 4) {
    const int rt = tile / CT, ct = tile % CT;
    const int t = rt * 16 + lr - dk;   // this lane's A row as a token of the chunk (rows of R)
    const float* arow = Mj + static_cast<size_t>(rt * 16 + lr) * ncol + dk + 4 * lg;
    const float* lrow = a.lam + static_cast<size_t>(bh * p.T + t0 + (t > 0 && t < n ? t : 0)) * a.L;
    f32x4 acc = zero4();
    for (int kb = 0; kb < nk / 16; ++kb) {
      f32x4 x = ld4(arow + kb * 16);
      if (rt >= dkT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = (kb * 16 + 4 * lg + e) / r_kv;   // key token of this column
          // R is zero above the token diagonal; rows past the chunk's end are not stored
          x[e] = (t < n && s <= t) ? x[e] * lrow[bit_length(static_cast<unsigned>(t ^ s))] : 0.f;
        }
      }
      f32x4 b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = kb * 16 + 4 * lg + e;
        b[e] = m / r_kv < n ? Elem<TI>::load(vp, (static_cast<size_t>(bh * p.T + t0) * r_kv + m) * dv + ct * 16 + lr)
                            : 0.f;
      }
      acc = mfma16(x, b, acc);
    }
    if (rt < dkT) {
      st4(a.ZVT + (static_cast<size_t>(job) * dv + ct * 16 + lr) * dk + rt * 16 + 4 * lg, acc);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tt = (rt - dkT) * 16 + 4 * lg + e;
        a.OI[(static_cast<size_t>(job) * C + tt) * dv + ct * 16 + lr] = acc[e];
      }
    }
  }
}

struct LlScanArgs {
  Problem p;
  const float* M;
  const float* ZVT;
  const float* OI;
  const float* lam;
  int L;
  int c;       // log2(C)
  int nlev;    // inter-chunk levels: bit_length(N - 1)
  int nbuf;    // copies of each level state: 2 (read one, write the other by chunk parity) or 1
  void* out;
};

constexpr int kLlBV = 16;     // d_v columns per workgroup
constexpr int kLlQW = 3;      // row tiles per wave: (d_k + C) / 16 <= 12 over four waves
constexpr int kLlKB = 8;      // K slices of the state product: d_k <= 128

// One workgroup (four waves) per (batch*head, 16-column d_v slice); chunks in
// order.  Every level's state S^(m) (d_k x 16, fp32) is kept in LDS as S^T.
// Wave w owns row tiles w, w+4, w+8 of [Acal ; Qbar] and holds their operator
// fragments in registers for all levels of a chunk.  With two copies of each
// state (where they fit in LDS), chunk J reads copy J mod 2 and writes the
// other, so the levels run back to back with one barrier per chunk; with one
// copy, each level waits for every wave's reads before its writes.
template <typename TI>
__global__ __launch_bounds__(256) void ll_scan_kernel(LlScanArgs a) {
  extern __shared__ __align__(16) float ls[];
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv, C = p.C, ncol = p.mcols();
  const int MT = p.mrows() / 16, dkT = dk / 16, KB = dk / 16;
  const int LDS_ = dk + 4;
  const int nvt = dv / kLlBV;
  const int64_t N = p.N;
  const int b = blockIdx.x;
  const int grp = b / (8 * nvt), rem = b % (8 * nvt);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + rem % 8;
  const int c0 = (rem / 8) * kLlBV;
  if (bh >= p.BH) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  for (int e = tid; e < a.nbuf * a.nlev * kLlBV * LDS_; e += 256) ls[e] = 0.f;
  __syncthreads();
  TI* op = static_cast<TI*>(a.out);

  for (int64_t J = 0; J < N; ++J) {
    const int64_t job = bh * N + J;
    const float* MJ = a.M + static_cast<size_t>(job) * p.mrows() * ncol;
    const int64_t t0 = J * C;
    const int n = static_cast<int>(p.T - t0 < C ? p.T - t0 : C);
    f32x4 fa[kLlQW][kLlKB], zv[kLlQW], oacc[kLlQW];
#pragma unroll
    for (int u = 0; u < kLlQW; ++u) {
      const int mt = wave + 4 * u < MT ? wave + 4 * u : MT - 1;
      // only the fragments the products read: tiles in range, K slices below d_k
#pragma unroll
      for (int kb = 0; kb < kLlKB; ++kb)
        fa[u][kb] = kb < KB && wave + 4 * u < MT ? ld4(MJ + static_cast<size_t>(mt * 16 + lr) * ncol + kb * 16 + 4 * lg)
                                                 : zero4();
      zv[u] = zero4();
      oacc[u] = zero4();
      if (wave + 4 * u >= MT) continue;
      if (mt < dkT) {
        zv[u] = ld4(a.ZVT + (static_cast<size_t>(job) * dv + c0 + lr) * dk + mt * 16 + 4 * lg);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          oacc[u][e] = a.OI[(static_cast<size_t>(job) * C + (mt - dkT) * 16 + 4 * lg + e) * dv + c0 + lr];
      }
    }
    for (int m = 0; m < a.nlev; ++m) {
      const bool right = (J >> m) & 1;
      const bool reset = !right && (J & ((2LL << m) - 1)) == 0;
      const bool two = a.nbuf == 2;
      float* S = ls + (m * a.nbuf + (two ? static_cast<int>(J & 1) : 0)) * kLlBV * LDS_;        // read
      float* Sw = two ? ls + (m * 2 + static_cast<int>((J + 1) & 1)) * kLlBV * LDS_ : S;    // written
      f32x4 acc[kLlQW];
#pragma unroll
      for (int u = 0; u < kLlQW; ++u) {
        acc[u] = zero4();
        const int mt = wave + 4 * u;
        // rows of Qbar are read only in the right half
        if (mt < MT && !reset && (right || mt < dkT)) {
#pragma unroll
          for (int kb = 0; kb < kLlKB; ++kb)
            if (kb < KB) acc[u] = mfma16(fa[u][kb], ld4(S + lr * LDS_ + kb * 16 + 4 * lg), acc[u]);
        }
      }
      if (!two) __syncthreads();   // every product has read S^(m)
#pragma unroll
      for (int u = 0; u < kLlQW; ++u) {
        const int mt = wave + 4 * u;
        if (mt >= MT) break;
        if (mt < dkT) {
          f32x4 s = acc[u];
          if (!right) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] += zv[u][e];
          }
          st4(Sw + lr * LDS_ + mt * 16 + 4 * lg, s);
        } else if (right) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = (mt - dkT) * 16 + 4 * lg + e;
            const float w = t < n ? a.lam[static_cast<size_t>(bh * p.T + t0 + t) * a.L + a.c + 1 + m] : 0.f;
            oacc[u][e] += w * acc[u][e];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kLlQW; ++u) {
      const int mt = wave + 4 * u;
      if (mt < MT && mt >= dkT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = (mt - dkT) * 16 + 4 * lg + e;
          if (t < n) Elem<TI>::store(op, static_cast<size_t>(bh * p.T + t0 + t) * dv + c0 + lr, oacc[u][e]);
        }
      }
    }
    __syncthreads();   // the state writes of this chunk before the next chunk's reads
  }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

int loglinear_levels(int64_t T) {
  if (T <= 0) return 0;
  int b = 0;
  for (uint64_t x = static_cast<uint64_t>(T - 1); x; x >>= 1) ++b;
  return 1 + b;
}

static int inter_levels(int64_t N) {
  int b = 0;
  for (uint64_t x = N > 0 ? static_cast<uint64_t>(N - 1) : 0; x; x >>= 1) ++b;
  return b;
}

// LDS of one copy of the level states
size_t loglinear_scan_lds(const Problem& p) {
  return static_cast<size_t>(inter_levels(p.N)) * kLlBV * (p.dk + 4) * sizeof(float);
}
constexpr size_t kLlLdsMax = 150 * 1024;
// copies of each level state the scan keeps: two where they fit
int loglinear_scan_bufs(const Problem& p) { return 2 * loglinear_scan_lds(p) <= kLlLdsMax ? 2 : 1; }

bool loglinear_supported(const Problem& p) {
  return p.dk <= 128 && p.dv <= 128 && p.mrows() <= 16 * 4 * kLlQW && loglinear_scan_lds(p) <= kLlLdsMax;
}

LlPlan loglinear_plan(const Problem& p) {
  LlPlan h{};
  const size_t chunks = static_cast<size_t>(p.BH * p.N);
  h.gen_bytes = align256(f32_operators_bytes(p));
  h.zv_bytes = align256(chunks * p.dv * p.dk * sizeof(float));
  h.oi_bytes = align256(chunks * p.C * p.dv * sizeof(float));
  h.total_bytes = h.gen_bytes + h.zv_bytes + h.oi_bytes;
  return h;
}

hipError_t launch_loglinear(const Problem& p, const void* q, const void* k, const float* ld, const void* A,
                            const void* B, const void* v, const float* lam, void* out, void* workspace,
                            hipStream_t s) {
  if (p.BH * p.N == 0) return hipSuccess;
  if (!loglinear_supported(p)) return hipErrorInvalidValue;
  const LlPlan h = loglinear_plan(p);
  char* ws = static_cast<char*>(workspace);
  float* ZVT = reinterpret_cast<float*>(ws + h.gen_bytes);
  float* OI = reinterpret_cast<float*>(ws + h.gen_bytes + h.zv_bytes);
  const float* M = nullptr;   // fp32 chunk operators inside the workspace
  hipError_t e = f32_operators(p, q, k, ld, A, B, workspace, &M, s);
  if (e != hipSuccess) return e;
  const int L = loglinear_levels(p.T);
  LlIntraArgs ia{p, M, v, lam, L, ZVT, OI};
  const dim3 grid(static_cast<unsigned>(p.BH * p.N));
  if (p.bf16)
    hipLaunchKernelGGL(ll_intra_kernel<bf16_raw>, grid, dim3(256), 0, s, ia);
  else
    hipLaunchKernelGGL(ll_intra_kernel<float>, grid, dim3(256), 0, s, ia);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  int c = 0;
  while ((1 << c) < p.C) ++c;
  const int nbuf = loglinear_scan_bufs(p);
  LlScanArgs sa{p, M, ZVT, OI, lam, L, c, inter_levels(p.N), nbuf, out};
  const size_t lds = loglinear_scan_lds(p) * nbuf;
  const void* fn = p.bf16 ? reinterpret_cast<const void*>(ll_scan_kernel<bf16_raw>)
                          : reinterpret_cast<const void*>(ll_scan_kernel<float>);
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds > 0 ? lds : 16));
  if (e != hipSuccess) return e;
  const int64_t nvt = p.dv / kLlBV;
  const dim3 sgrid(static_cast<unsigned>((p.BH + 7) / 8 * 8 * nvt));
  if (p.bf16)
    hipLaunchKernelGGL(ll_scan_kernel<bf16_raw>, sgrid, dim3(256), lds, s, sa);
  else
    hipLaunchKernelGGL(ll_scan_kernel<float>, sgrid, dim3(256), lds, s, sa);
  return hipGetLastError();
}

}  // namespace lattn
