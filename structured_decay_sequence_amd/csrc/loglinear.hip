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

// ---------------------------------------------------------------------------
// The same lift on the bf16 MFMA prepare's operators (bf16 storage, C = 64,
// d_k = 64), read in their fragment order with no fp32 copy, on bf16 MFMAs
// (16x16x32, fp32 accumulate).  A fragment (row tile mt, K pair kp) is 64
// lanes x 8 bf16: lane (g, i) holds row 16 mt + i at the columns
// 32 kp + 16 h + 4 g + e (h = 0, 1; e = 0..3).  A 16x16 result tile in
// accumulator layout (lane (g, i): rows 4 g + e, column i) of row tiles 2 kp
// and 2 kp + 1 is therefore, side by side, the B operand of K pair kp: a level
// state feeds the next chunk's product with no lane exchange.
//
// One workgroup of eight waves per (batch*head, 16-column d_v slice), chunks
// in order; two waves per SIMD, one of each role:
//  * level waves (w < 4) own the inter-chunk levels m = w, w + 4, ... and
//    carry their states in fp32 registers: in a right half of level m they
//    read the state out (Qbar S, weighted per token by the level's weight)
//    into a partial output of the chunk's 64 tokens, then transport it
//    (S <- Acal S, plus Z V in a left half);
//  * token waves (w >= 4) form the chunk-local output (R (.) Lam) V of the
//    tokens 16 (w - 4) .. + 15, add the level waves' partials one chunk later
//    (after the barrier that publishes them) and store the result.
// The token waves, which hold few registers, also stage the inputs: a chunk's
// operator (32 KB), V slice and level weights are loaded into a ring of PD
// register sets PD chunks ahead, and written to the other half of a
// double-buffered LDS stage at the end of the chunk before their use; the
// partial outputs alternate the same way, so each chunk needs one barrier.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 lbf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lbf16x4;
typedef unsigned int lu32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int lu32x2 __attribute__((ext_vector_type(2)));

constexpr int kFC = 64;     // chunk of the bf16 operators
constexpr int kFLW = 4;     // level waves
constexpr int kFTW = 4;     // token waves: one per 16-token tile of the chunk
constexpr int kFW = kFLW + kFTW;
constexpr int kFLPW = 4;    // inter-chunk levels per level wave (up to 16 levels)
constexpr int kFBV = 16;    // d_v columns per workgroup
constexpr int kFLamIt = 6;  // staged weights per token-wave lane: 64 tokens x (c + 1 + 16) <= 6 x 256
constexpr int kFPD = 2;     // chunks in flight ahead of the one being staged
// Row stride (floats) of the staged level weights [level][token]: 4 mod 64,
// so that the staging writes (levels of a few consecutive tokens across the
// lanes) fall in distinct LDS banks, and rows stay 16-byte aligned.
constexpr int kFWS = kFC + 4;

template <int DK>
struct LlFastCfg {
  static constexpr int MT = (DK + kFC) / 16;         // operator row tiles
  static constexpr int KP = (DK + kFC) / 32;         // operator K pairs
  static constexpr int DT = DK / 16;                 // channel row tiles
  static constexpr int DP = DK / 32;                 // channel K pairs
  static constexpr int TP = kFC / 32;                // token K pairs
  static constexpr int OPB = MT * KP * 1024;         // bytes of one chunk operator
  static constexpr int OPIT = OPB / (16 * 64 * kFTW); // 16-byte operator pieces per token-wave lane
  static constexpr int VB = TP * 1024;               // V slice as B fragments
  static constexpr int PB = kFLW * (kFC / 16) * 1024; // partial outputs of the level waves (fp32 tiles)
  static_assert(OPB % (16 * 64 * kFTW) == 0 && DT % 2 == 0 && kFC * kFBV == 4 * 64 * kFTW,
                "bf16 log-linear tiling");
};

__device__ __forceinline__ lbf16x4 f4_to_b4(const f32x4& v) {
  lbf16x4 r;
  r[0] = (__bf16)v[0];
  r[1] = (__bf16)v[1];
  r[2] = (__bf16)v[2];
  r[3] = (__bf16)v[3];
  return r;
}
__device__ __forceinline__ lbf16x8 cat8(const lbf16x4& x, const lbf16x4& y) {
  lbf16x8 r;
  r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
  r[4] = y[0]; r[5] = y[1]; r[6] = y[2]; r[7] = y[3];
  return r;
}
__device__ __forceinline__ f32x4 mfma_bf16(const lbf16x8& x, const lbf16x8& y, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
}
// Workgroup barrier ordering LDS only (global stores stay in flight).
__device__ __forceinline__ void ll_lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

struct LlFastArgs {
  Problem p;
  const __bf16* M;     // fragment-ordered chunk operators
  const __bf16* v;
  const float* lam;    // [BH, T, L]
  int L;
  int c;               // log2(C)
  int nlev;            // inter-chunk levels
  int LS;              // weights staged per token: min(L, c + 1 + nlev)
  __bf16* out;
};

template <int DK>
__global__ __launch_bounds__(64 * kFW) void ll_fast_kernel(LlFastArgs a) {
  using Cfg = LlFastCfg<DK>;
  constexpr int DT = Cfg::DT, DP = Cfg::DP, TP = Cfg::TP, KP = Cfg::KP;
  constexpr int NTH = 64 * kFTW, NTT = kFC / 16;   // staging threads: the token waves
  extern __shared__ __align__(16) unsigned char smem[];
  const Problem& p = a.p;
  const int nvt = p.dv / kFBV;
  const int b = blockIdx.x;
  // the d_v slices of one (batch, head) share blockIdx % 8, hence an XCD and its L2
  const int grp = b / (8 * nvt), rem = b % (8 * nvt);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + rem % 8;
  const int c0 = (rem / 8) * kFBV;
  if (bh >= p.BH) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t N = p.N, T = p.T;
  const int nlev = a.nlev, LS = a.LS;
  const int nlw = nlev < kFLW ? nlev : kFLW;   // level waves that own a level
  unsigned char* opL = smem;                                   // [2][OPB]
  unsigned char* vL = opL + 2 * Cfg::OPB;                      // [2][VB]
  f32x4* pL = reinterpret_cast<f32x4*>(vL + 2 * Cfg::VB);      // [2][level wave][token tile][lane]
  float* wL = reinterpret_cast<float*>(vL + 2 * Cfg::VB + 2 * Cfg::PB);   // [2][LS][kFWS]

  // ---- staging of one chunk (token waves): global -> registers, then
  // registers -> LDS.  sid: this lane's index among the token waves' lanes.
  const int sid = tid - 64 * kFLW;
  // This lane's level weights: (token, level) pairs sid + NTH i of the chunk's
  // token-major block, fixed for the whole walk (-1: none).
  int wtk[kFLamIt], wlv[kFLamIt];
  // This lane's V piece: token sid / 4, columns 4 (sid % 4) .. + 3; and its
  // place in the B fragments of the token K pairs (token t sits in pair
  // t / 32, half (t / 16) % 2, lane group (t / 4) % 4, element t % 4).
  const int tv = sid >> 2, cv = 4 * (sid & 3);
  const int vpos = (tv >> 5) * 64 * 8 + ((tv >> 2) & 3) * 16 * 8 + ((tv >> 4) & 1) * 4 + (tv & 3) + cv * 8;
  struct Stage {
    lu32x4 op[Cfg::OPIT];
    lu32x2 v;
    float w[kFLamIt];
  };
  auto load_chunk = [&](Stage& st, int64_t J) {
    const int64_t job = bh * N + J;
    const lu32x4* src = reinterpret_cast<const lu32x4*>(a.M + static_cast<size_t>(job) * (Cfg::OPB / 2));
#pragma unroll
    for (int i = 0; i < Cfg::OPIT; ++i) st.op[i] = src[i * NTH + sid];
    const int64_t t0 = J * kFC;
    const int n = static_cast<int>(T - t0 < kFC ? T - t0 : kFC);
    st.v = lu32x2{0u, 0u};
    if (tv < n) st.v = *reinterpret_cast<const lu32x2*>(a.v + static_cast<size_t>(bh * T + t0 + tv) * p.dv + c0 + cv);
#pragma unroll
    for (int i = 0; i < kFLamIt; ++i) {
      const int t = wtk[i] < 0 ? 0 : (wtk[i] < n ? wtk[i] : n - 1);   // padded tokens read the last one
      st.w[i] = a.lam[static_cast<size_t>(bh * T + t0 + t) * a.L + (wtk[i] < 0 ? 0 : wlv[i])];
    }
  };
  auto stage_chunk = [&](const Stage& st, int buf) {
    lu32x4* od = reinterpret_cast<lu32x4*>(opL + buf * Cfg::OPB);
#pragma unroll
    for (int i = 0; i < Cfg::OPIT; ++i) od[i * NTH + sid] = st.op[i];
    __bf16* vd = reinterpret_cast<__bf16*>(vL + buf * Cfg::VB);
    const lbf16x4 vv = __builtin_bit_cast(lbf16x4, st.v);
#pragma unroll
    for (int j = 0; j < 4; ++j) vd[vpos + 8 * j] = vv[j];
    float* wd = wL + buf * LS * kFWS;   // level weights transposed: [level][token]
#pragma unroll
    for (int i = 0; i < kFLamIt; ++i)
      if (wtk[i] >= 0) wd[wlv[i] * kFWS + wtk[i]] = st.w[i];
  };
  Stage ring[kFPD];
  if (wave >= kFLW) {
#pragma unroll
    for (int i = 0; i < kFLamIt; ++i) {
      const int idx = sid + NTH * i;
      const int t = idx / LS;
      wtk[i] = idx < kFC * LS ? t : -1;
      wlv[i] = idx - t * LS;
    }
    load_chunk(ring[0], 0);
    stage_chunk(ring[0], 0);
#pragma unroll
    for (int k = 1; k < kFPD; ++k) load_chunk(ring[k], k < N ? k : N - 1);
  }
  ll_lds_barrier();
  if (wave < kFLW) {
    // ================= level wave
    f32x4 S[kFLPW][DT];
#pragma unroll
    for (int u = 0; u < kFLPW; ++u)
#pragma unroll
      for (int i = 0; i < DT; ++i) S[u][i] = zero4();
    for (int64_t J = 0; J < N; ++J) {
      const int buf = static_cast<int>(J & 1);
      if (wave < nlev) {
        const lbf16x8* opf = reinterpret_cast<const lbf16x8*>(opL + buf * Cfg::OPB);
        const lbf16x8* vb = reinterpret_cast<const lbf16x8*>(vL + buf * Cfg::VB);
        const float* wb = wL + buf * LS * kFWS;
        lbf16x8 vfr[TP];
#pragma unroll
        for (int q = 0; q < TP; ++q) vfr[q] = vb[q * 64 + lane];
        f32x4 zv[DT];
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          zv[i] = zero4();
#pragma unroll
          for (int q = 0; q < TP; ++q) zv[i] = mfma_bf16(opf[(i * KP + DP + q) * 64 + lane], vfr[q], zv[i]);
        }
        lbf16x8 af[DT][DP];
#pragma unroll
        for (int i = 0; i < DT; ++i)
#pragma unroll
          for (int kp = 0; kp < DP; ++kp) af[i][kp] = opf[(i * KP + kp) * 64 + lane];
        // Qbar fragments, if a level of this wave is read out in this chunk
        bool any_right = false;
#pragma unroll
        for (int u = 0; u < kFLPW; ++u) {
          const int m = wave + kFLW * u;
          any_right |= m < nlev && ((J >> m) & 1);
        }
        lbf16x8 qf[NTT][DP];
        f32x4 part[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          part[tt] = zero4();
#pragma unroll
          for (int kp = 0; kp < DP; ++kp)
            qf[tt][kp] = any_right ? opf[((DT + tt) * KP + kp) * 64 + lane] : lbf16x8{};
        }
#pragma unroll
        for (int u = 0; u < kFLPW; ++u) {
          const int m = wave + kFLW * u;
          if (m < nlev) {
            const bool right = (J >> m) & 1;
            const bool reset = !right && (J & ((2LL << m) - 1)) == 0;
            if (reset) {
#pragma unroll
              for (int i = 0; i < DT; ++i) S[u][i] = zv[i];
            } else {
              lbf16x8 sb[DP];
#pragma unroll
              for (int kp = 0; kp < DP; ++kp) sb[kp] = cat8(f4_to_b4(S[u][2 * kp]), f4_to_b4(S[u][2 * kp + 1]));
              if (right) {
                // readout of the state entering this chunk, weighted per token
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                  f32x4 acc = zero4();
#pragma unroll
                  for (int kp = 0; kp < DP; ++kp) acc = mfma_bf16(qf[tt][kp], sb[kp], acc);
                  const f32x4 w = *reinterpret_cast<const f32x4*>(wb + (a.c + 1 + m) * kFWS + 16 * tt + 4 * lg);
#pragma unroll
                  for (int e = 0; e < 4; ++e) part[tt][e] += w[e] * acc[e];
                }
              }
#pragma unroll
              for (int i = 0; i < DT; ++i) {
                f32x4 acc = right ? zero4() : zv[i];
#pragma unroll
                for (int kp = 0; kp < DP; ++kp) acc = mfma_bf16(af[i][kp], sb[kp], acc);
                S[u][i] = acc;
              }
            }
          }
        }
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) pL[((buf * kFLW + wave) * NTT + tt) * 64 + lane] = part[tt];
      }
      ll_lds_barrier();
    }
  } else {
    // ================= token wave: tokens 16 tt .. 16 tt + 15 of every chunk
    const int tt = wave - kFLW;
    const int tq = 16 * tt + lr;   // this lane's row of the R fragments
    // The K pair qd = tt / 2 holds the diagonal tile: its weights go element by
    // element (key s <= tq at level bit_length(tq ^ s), 0 on the diagonal; -1:
    // masked).  For tt >= 2 the pair 0 (keys 0 .. 31) is at level c = 6 for
    // every row: its product is scaled by row afterwards.
    const int qd = tt >> 1;
    int woff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = 32 * qd + 16 * (j >> 2) + 4 * lg + (j & 3);
      const int lev = 32 - __clz(tq ^ s);
      woff[j] = (s <= tq && lev < LS) ? lev * kFWS + tq : -1;
    }
    const bool lower = tt >= 2 && LS > 6;
    f32x4 o_prev = zero4();
    auto finish = [&](int64_t Jp, int pbuf) {
      // chunk Jp's output: its chunk-local part plus the level waves' partials
      f32x4 o = o_prev;
      for (int w = 0; w < nlw; ++w) {
        const f32x4 pp = pL[((pbuf * kFLW + w) * NTT + tt) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] += pp[e];
      }
      const int64_t t0 = Jp * kFC;
      const int n = static_cast<int>(T - t0 < kFC ? T - t0 : kFC);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tt + 4 * lg + e;
        if (t < n) a.out[static_cast<size_t>(bh * T + t0 + t) * p.dv + c0 + lr] = (__bf16)o[e];
      }
    };
    // Chunk J loads chunk J + PD into ring slot J % PD (which held chunk J,
    // staged at the end of chunk J - 1) and stages chunk J + 1 from slot
    // (J + 1) % PD; past the end the loads repeat the last chunk, unread.
    auto step = [&](const int64_t J, Stage& ld_slot, const Stage& st_slot) {
      const int buf = static_cast<int>(J & 1);
      load_chunk(ld_slot, J + kFPD < N ? J + kFPD : N - 1);
      if (J > 0) finish(J - 1, buf ^ 1);
      const lbf16x8* opf = reinterpret_cast<const lbf16x8*>(opL + buf * Cfg::OPB);
      const lbf16x8* vb = reinterpret_cast<const lbf16x8*>(vL + buf * Cfg::VB);
      const float* wb = wL + buf * LS * kFWS;
      lbf16x8 rf = opf[((DT + tt) * KP + DP + qd) * 64 + lane];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float w = woff[j] >= 0 ? wb[woff[j]] : 0.f;
        rf[j] = (__bf16)((float)rf[j] * w);
      }
      f32x4 o = mfma_bf16(rf, vb[qd * 64 + lane], zero4());
      if (lower) {
        const f32x4 acc = mfma_bf16(opf[((DT + tt) * KP + DP) * 64 + lane], vb[lane], zero4());
        const f32x4 w = *reinterpret_cast<const f32x4*>(wb + 6 * kFWS + 16 * tt + 4 * lg);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] += w[e] * acc[e];
      }
      o_prev = o;
      stage_chunk(st_slot, buf ^ 1);
      ll_lds_barrier();
    };
    for (int64_t J = 0; J < N; J += kFPD) {
#pragma unroll
      for (int k = 0; k < kFPD; ++k)
        if (J + k < N) step(J + k, ring[k], ring[(k + 1) % kFPD]);
    }
    finish(N - 1, static_cast<int>((N - 1) & 1));
  }
}

size_t ll_fast_lds(int LS) {
  using Cfg = LlFastCfg<64>;
  return 2 * static_cast<size_t>(Cfg::OPB + Cfg::VB + Cfg::PB) + 2 * static_cast<size_t>(LS) * kFWS * sizeof(float);
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

// The bf16 route: the bf16 MFMA prepare's shapes at d_k = 64, up to 16
// inter-chunk levels (2^16 chunks).
static bool loglinear_fast(const Problem& p) {
  return fast_supported(p) && p.dk == 64 && inter_levels(p.N) <= kFLW * kFLPW;
}

bool loglinear_supported(const Problem& p) {
  if (loglinear_fast(p)) return true;
  return p.dk <= 128 && p.dv <= 128 && p.mrows() <= 16 * 4 * kLlQW && loglinear_scan_lds(p) <= kLlLdsMax;
}

LlPlan loglinear_plan(const Problem& p) {
  LlPlan h{};
  if (loglinear_fast(p)) {
    h.gen_bytes = align256(fast_workspace_bytes(p));
    h.total_bytes = h.gen_bytes;
    return h;
  }
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
  if (loglinear_fast(p)) {
    hipError_t e = fast_prepare(p, q, k, ld, A, B, workspace, s);
    if (e != hipSuccess) return e;
    const int nlev = inter_levels(p.N);
    const int L = loglinear_levels(p.T);
    const int LS = L < 7 + nlev ? L : 7 + nlev;   // weights read per token: c = 6
    LlFastArgs fa{p, static_cast<const __bf16*>(workspace), static_cast<const __bf16*>(v), lam, L, 6, nlev, LS,
                  static_cast<__bf16*>(out)};
    const size_t lds = ll_fast_lds(LS);
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(ll_fast_kernel<64>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const int64_t nvt = p.dv / kFBV;
    const dim3 grid(static_cast<unsigned>((p.BH + 7) / 8 * 8 * nvt));
    hipLaunchKernelGGL(ll_fast_kernel<64>, grid, dim3(64 * kFW), lds, s, fa);
    return hipGetLastError();
  }
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
