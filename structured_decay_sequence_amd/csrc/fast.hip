// bf16 MFMA path (gfx950) for chunk C = 64, write rank r_kv = 1, decay rank
// r_ab in {0, 1, 2}, d_k in {64, 128}: the GLA, Gated DeltaNet and HDLA shapes.
//
// It computes the same chunk operator as the general path (HDLA note, "Key
// design 3": rank-generalized WY form; HLA note, "Affine maps and closure
// under composition"):
//   M_j = [[Acal, Z], [Qbar, R]],   [S_j ; O_j] = M_j [S_{j-1} ; V_j]
// with bf16 MFMA operands and fp32 accumulation; the triangular solve applies
// its 16x16 diagonal inverses in fp32.
//
// prepare kernel: persistent, one workgroup per compute unit walking the
// (batch*head, chunk) jobs; in the solve and the final product one wave owns
// each 16-column tile of the chunk operator's input side (the d_k "W"
// columns, then the 64 "X" columns) and runs on its own columns with no
// barrier.  The operator is stored in MFMA operand
// order: each 16x16 tile is the A-operand fragment of a 16x16x16 MFMA (lane
// l holds row l%16, columns 4*(l/16)..+3), and the tiles of columns 2m and
// 2m+1 are interleaved per lane, so one 16-byte load gives a lane the eight
// K values of a 16x16x32 MFMA over both.
//
// scan kernel: one workgroup per (batch*head, d_v slice); chunks in order, the
// state slice kept in LDS as the bf16 B operand, per chunk one MFMA product.
#include "common.hpp"
#include "kernels.hpp"

namespace lattn {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kC = 64;    // chunk length of this path
constexpr int kNK = 64;   // C * r_kv

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Workgroup barrier that orders LDS only.  The waves of these kernels talk to
// each other through LDS alone, so a barrier need not wait for in-flight
// global loads (the register prefetch of the next chunk stays in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) {
  bf16x4 r;
  r[0] = (__bf16)v[0];
  r[1] = (__bf16)v[1];
  r[2] = (__bf16)v[2];
  r[3] = (__bf16)v[3];
  return r;
}
__device__ __forceinline__ f32x4 to_f32x4(bf16x4 v) {
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}
__device__ __forceinline__ bf16x4 lds4(const __bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ bf16x8 lds8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
// The transposing 64-bit LDS read (16-bit elements) works on groups of 16
// lanes: element e of lane (g, i) is the (i%4)-th value fetched by lane
// (g, 4e + i/4).  Lane (g, j) therefore supplies the address of
// X[4g + j/4][4(j%4) .. 4(j%4)+3] so that lane (g, i) receives X[4g+e][i]:
// a tile's transpose in MFMA operand order.
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Row layout of the prepare kernel's operand arrays, chosen so that both a
// 16-row x 16-byte MFMA fragment read and a transposing tile read run at the
// LDS's full rate (measured on gfx950): d_k = 128 rows are padded to 144
// bf16 (addresses stay additive, so lane offsets fold into immediates);
// d_k = 64 rows are unpadded with their 16-byte pieces XOR-permuted by the
// row index (piece q of row r at q ^ ((r >> 1) & 7)).
template <int DK>
struct XRow {
  static constexpr int LD = DK == 128 ? 144 : DK;   // bf16 per row
};
// Element offset of the 16-byte piece q of row `row`.
template <int DK>
__device__ __forceinline__ int xoff(int row, int q) {
  if (DK == 128) return row * XRow<DK>::LD + 8 * q;
  return row * DK + 8 * (q ^ ((row >> 1) & 7));
}
// MFMA row fragment: rows r0 + lane%16, 16-byte piece q0 + lane/16.
template <int DK>
__device__ __forceinline__ bf16x8 xrow8(const __bf16* X, int r0, int q0, int lane) {
  return lds8(X + xoff<DK>(r0 + (lane & 15), q0 + (lane >> 4)));
}
// Transposing read of the 16x16 tile at rows r0.., columns c0.. (c0 % 16 == 0)
// of a swizzled operand array: lane (g, i) receives X[r0 + 4g + e][c0 + i].
template <int DK>
__device__ __forceinline__ bf16x4 xtr4(const __bf16* X, int r0, int c0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int row = r0 + 4 * g + (j >> 2);
  const __bf16* ptr = X + xoff<DK>(row, (c0 >> 3) + ((j & 3) >> 1)) + 4 * (j & 1);
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(ptr));
  return __builtin_bit_cast(bf16x4, r);
}

// ---------------------------------------------------------------------------
// Prepare kernel.  Persistent: each workgroup walks chunks blockIdx.x,
// blockIdx.x + gridDim.x, ...; the next chunk's raw inputs are loaded into
// registers while the current one is being solved.
//
// Roles inside a chunk (DK/8 or KT waves, whichever is more):
//  * scaling: wave w owns tokens TPWV*w .. TPWV*w + TPWV-1, lane (g, c) owns
//    the 8-channel piece c of token TPWV*w + g, so that every load reads whole
//    rows.  The chunk-local cumulative log-decay is a prefix sum over tokens:
//    inside the wave by lane shuffles, across waves through per-wave totals in
//    LDS.  It is kept in base-2 units so that every decay factor is one exp2.
//  * Gram blocks: the upper-triangular tiles of A~ [B~ ; Q~]^T.  At d_k = 128
//    the diagonal blocks go to the waves that invert them and the rest to the
//    waves with no X column, in contiguous runs; at d_k = 64 all waves share
//    them, then invert.
//  * solve and operator: wave w < KT owns the 16-column input tile w.
// Operand source of the prepare kernel: the decay operands A, B given
// (generic), or formed on the fly from a family's raw parameters.  kGenericBw:
// generic, and the decay-scaled operands also go to memory for the chunked
// backward.
enum PrepMode { kGeneric = 0, kHdla = 1, kGdn = 2, kGenericBw = 3 };

template <int DK, int RAB, bool SCAL, int MODE>
struct PrepCfg {
  static constexpr int NA = kC * RAB;            // decay rows of a chunk (0: diagonal decay only)
  static constexpr int NB = NA / 16;             // 16-row blocks of the solve
  static constexpr int NBA = NB > 0 ? NB : 1;    // array extent
  static constexpr int RB = RAB > 0 ? RAB : 1;   // divisor in code that rank 0 never runs
  static constexpr int KIN = DK + kNK;           // operator input width
  static constexpr int ROUT = DK + kC;           // operator output height
  static constexpr int KT = KIN / 16;
  static constexpr int MT = ROUT / 16;
  static constexpr int NO = DK / 8;              // 16-byte channel pieces per row
  static constexpr int NW = NO > KT ? NO : KT;
  static constexpr int NT = 64 * NW;
  static constexpr int TPWV = 64 / NO;           // tokens per wave in the scaling phase
  static constexpr int LDA = NA + 16;            // padded row of M_A (bf16; 32 mod 64 bytes)
  static constexpr int LDB = 260;                // floats per diagonal block (padded)
  static constexpr int NCS = NB + kC / 16;       // column blocks of the Gram tiles
  static constexpr int NTILE = NB * NCS - NB * (NB - 1) / 2;
  static constexpr int FULL_SLOTS = NTILE / NW;  // tile slots every wave has
  // d_k = 128: the inversion and the X-wave products overlap the Gram tiles
  // (NINV waves invert, NXW waves are X columns, NWORK waves take the
  // off-diagonal tiles).  d_k = 64 has too few waves for that split.
  static constexpr bool OVERLAP = DK == 128;
  static constexpr int NINV = NB * 16 / 64;
  static constexpr int NXW = KT - DK / 16;
  static constexpr int NWORK = NW - NINV - NXW;
  // LDS regions (bytes)
  static constexpr int R_XL = (NA + kC) * XRow<DK>::LD * 2;
  static constexpr int R_XR = (NA + kNK) * XRow<DK>::LD * 2;
  static constexpr int R_LD = NB * LDB * 4;
  static constexpr int R_LP = (NB * (NB - 1) / 2) * 256 * 2;
  // M_A; also holds the per-wave decay totals of the scaling phase
  static constexpr int R_MA = kC * LDA * 2 > NW * DK * 4 ? kC * LDA * 2 : NW * DK * 4;
  static constexpr int R_EG = DK * 4;
  static constexpr int DIB = 260;                // floats per inverse block (padded)
  static constexpr int R_DI = NB * DIB * 4;
  static constexpr bool GEN = MODE == kGeneric || MODE == kGenericBw;   // A, B given
  static constexpr int R_BT = GEN ? 0 : kC * 4;   // beta per token
  // d_k = 64 runs two resident workgroups per compute unit, so one chunk's
  // VALU scaling overlaps the other's MFMA phases.  To fit two in LDS it keeps
  // a compact layout: the diagonal blocks are inverted in place, and M_A is
  // formed after the solve, into the region of L and B~ (dead by then):
  //   [ L below diagonal | diagonal blocks = inverses | B~ ; Q~ | A~ ; K~ | exp(G_C) | beta ]
  //   [ M_A (after the solve) ........................ )
  static constexpr bool COMPACT = DK == 64 && RAB > 0;
  static constexpr int O_LP = COMPACT ? 0 : R_XL + R_XR + R_LD;
  static constexpr int O_LD = COMPACT ? R_LP : R_XL + R_XR;
  static constexpr int O_XL = COMPACT ? R_LP + R_LD : 0;
  static constexpr int O_XR = O_XL + R_XL;
  static constexpr int O_MA = COMPACT ? 0 : O_LP + R_LP;
  static constexpr int O_EG = COMPACT ? O_XR + R_XR : O_MA + R_MA;
  static constexpr int O_DI = COMPACT ? O_LD : O_EG + R_EG;
  static constexpr int O_BT = COMPACT ? O_EG + R_EG : O_DI + R_DI;
  static constexpr int LDS = O_BT + R_BT;
  static_assert(!COMPACT || R_MA <= R_LP + R_LD + NA * XRow<DK>::LD * 2,
                "compact layout: M_A fits the region of L and B~");
  static_assert(!COMPACT || DIB == LDB, "compact layout: inverses overwrite the diagonal blocks");
  static_assert(GEN || (MODE == kHdla && RAB == 2 && !SCAL) || (MODE == kGdn && RAB == 1 && SCAL),
                "fused modes: HDLA is rank 2 per channel, Gated DeltaNet rank 1 scalar");
  static_assert(NO == NW && KT <= NW, "wave roles: one wave per channel piece");
  static_assert(!OVERLAP || (NB % 4 == 0 && NWORK > 0), "overlapped Gram phase: four diagonal blocks per inverting wave");
};

struct FastPrepArgs {
  Problem p;
  const __bf16* q;
  const __bf16* k;
  const float* ld;
  const __bf16* A;
  const __bf16* B;
  const float* beta;   // fused modes: per-token beta [BH, T]
  __bf16* M;   // fragment-ordered chunk operators
  // kGenericBw: per chunk-head, Q~, K~ [C][dk] and A~, B~ [C r_ab][dk] (bf16),
  // L's 16x16 tiles below the diagonal blocks (bf16, row-major tiles, tile
  // (i, j) at i (i - 1) / 2 + j) and the inverses of its unit lower-triangular
  // diagonal blocks (fp32, row-major)
  // and the chunk-local cumulative log-decay G in base 2, [C][dk] (fp32;
  // padding tokens repeat the last token's), with e^{G} at the chunk's last
  // token [dk]
  __bf16 *qt, *kt, *at, *bt, *lt;
  float *di, *gc, *gam;
};

__device__ __forceinline__ bf16x8 scale8(const bf16x8& raw, const float (&f)[8]) {
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (__bf16)((float)raw[e] * f[e]);
  return out;
}

template <int DK, int RAB, bool SCAL, int MODE>
__global__ __launch_bounds__((PrepCfg<DK, RAB, SCAL, MODE>::NT)) void fast_prepare_kernel(FastPrepArgs a) {
  using Cfg = PrepCfg<DK, RAB, SCAL, MODE>;
  constexpr int NA = Cfg::NA, NB = Cfg::NB, NBA = Cfg::NBA, RB = Cfg::RB, LDA = Cfg::LDA, NW = Cfg::NW,
                LDB = Cfg::LDB;
  constexpr int MT = Cfg::MT, KT = Cfg::KT, NCS = Cfg::NCS, NTILE = Cfg::NTILE;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* Xl = reinterpret_cast<__bf16*>(smem + Cfg::O_XL);     // [B~ ; Q~]
  __bf16* Xr = reinterpret_cast<__bf16*>(smem + Cfg::O_XR);     // [A~ ; K~]
  float* Ldg = reinterpret_cast<float*>(smem + Cfg::O_LD);      // diagonal blocks
  __bf16* Lpk = reinterpret_cast<__bf16*>(smem + Cfg::O_LP);    // L below diagonal
  __bf16* MAs = reinterpret_cast<__bf16*>(smem + Cfg::O_MA);
  float* eGC = reinterpret_cast<float*>(smem + Cfg::O_EG);
  float* Dinv = reinterpret_cast<float*>(smem + Cfg::O_DI);
  float* betas = reinterpret_cast<float*>(smem + Cfg::O_BT);

  const Problem& p = a.p;
  const int lane0 = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int64_t total = p.BH * p.N;
  constexpr float kLog2e = 1.4426950408889634f;

  // ---- raw inputs of one chunk for this lane's (token, channel piece).
  constexpr int NO = Cfg::NO, TPWV = Cfg::TPWV;
  f32x4 ldv[2];
  bf16x8 qv, kv, av[RAB > 0 ? RAB : 1], bv[RAB > 0 ? RAB : 1];
  float btv = 0.f;
  auto chunk_n = [&](int64_t jb, int64_t& tok0) {
    const int64_t bh = jb / p.N, jc = jb % p.N;
    const int64_t t0 = jc * kC;
    tok0 = bh * p.T + t0;
    return static_cast<int>(p.T - t0 < kC ? p.T - t0 : kC);
  };
  // Loads are unconditional: a padded token reads the chunk's last row (the
  // values are discarded), so no branch separates the loads from their use.
  // Two parts, issued at different points of the previous chunk so that the
  // load issue does not bunch up behind one barrier.
  auto load_tok = [&](int64_t jb, int ln, int64_t& tok, int& c0) {
    int64_t tok0;
    const int n = chunk_n(jb, tok0);
    const int t = wave * TPWV + ln / NO;
    tok = tok0 + (t < n ? t : n - 1);
    c0 = (ln % NO) * 8;
  };
  auto load_a = [&](int64_t jb, int ln) {
    int64_t tok;
    int c0;
    load_tok(jb, ln, tok, c0);
    if (SCAL) {
      ldv[0][0] = a.ld[tok];
    } else {
      ldv[0] = *reinterpret_cast<const f32x4*>(a.ld + tok * DK + c0);
      ldv[1] = *reinterpret_cast<const f32x4*>(a.ld + tok * DK + c0 + 4);
    }
    qv = *reinterpret_cast<const bf16x8*>(a.q + tok * DK + c0);
    kv = *reinterpret_cast<const bf16x8*>(a.k + tok * DK + c0);
  };
  auto load_b = [&](int64_t jb, int ln) {
    int64_t tok;
    int c0;
    load_tok(jb, ln, tok, c0);
    if (Cfg::GEN) {
#pragma unroll
      for (int r = 0; r < RAB; ++r) {
        av[r] = *reinterpret_cast<const bf16x8*>(a.A + (tok * RAB + r) * DK + c0);
        bv[r] = *reinterpret_cast<const bf16x8*>(a.B + (tok * RAB + r) * DK + c0);
      }
    } else {
      btv = a.beta[tok];
    }
  };

  int64_t job = blockIdx.x;
  if (job >= total) return;
  load_a(job, lane0);
  load_b(job, lane0);
  for (; job < total; job += gridDim.x) {
    // Lane-derived values are recomputed per chunk from an opaque copy of the
    // lane index: hoisted out of this loop they would all stay live at once.
    int lane = lane0;
    asm volatile("" : "+v"(lane));
    const int lr = lane & 15, lg = lane >> 4;
    const int tid = wave * 64 + lane;
    int64_t tok0_cur;
    const int ncur = chunk_n(job, tok0_cur);   // tokens of this chunk (the rest are padding)
    __bf16* Mout = a.M + static_cast<size_t>(job) * (MT * KT * 256);

    // ---- P0/P1: cumulative log-decay (base 2) and the decay-scaled operands
    //      B~ = B exp(G_{t-1}), Q~ = q exp(G_t), A~ = A exp(-G_t), K~ = K exp(-G_t).
    //      Only the last chunk of a sequence can hold padding tokens; the
    //      other chunks run a copy of this phase with the padding masks
    //      compiled out.
    auto scale_phase = [&](auto padded) {
      constexpr bool PADDED = decltype(padded)::value;
      const int tg = lane / NO, pc = lane % NO;
      const int t = wave * TPWV + tg;
      const bool pad = PADDED && t >= ncur;
      constexpr int NL = SCAL ? 1 : 8;
      float* wtot = reinterpret_cast<float*>(MAs);   // per-wave totals (M_A is not live yet)
      float l2[NL], x[NL];
#pragma unroll
      for (int c = 0; c < NL; ++c) {
        const float v = SCAL ? ldv[0][0] : ldv[c / 4][c % 4];
        l2[c] = pad ? 0.f : v * kLog2e;
        x[c] = l2[c];
      }
      // inclusive prefix over this wave's tokens
#pragma unroll
      for (int sh = NO; sh < 64; sh *= 2) {
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          const float y = __shfl_up(x[c], sh, 64);
          if (lane >= sh) x[c] += y;
        }
      }
      if (tg == TPWV - 1) {
#pragma unroll
        for (int c = 0; c < NL; ++c) wtot[wave * DK + pc * 8 + c] = x[c];
      }
      lds_barrier();
      // totals of the earlier waves: token group g sums waves g, g + TPWV, ...
      float part[NL];
#pragma unroll
      for (int c = 0; c < NL; ++c) part[c] = 0.f;
#pragma unroll
      for (int k = 0; k < NW / TPWV; ++k) {
        const int w2 = tg + k * TPWV;
        if (w2 < wave) {
#pragma unroll
          for (int c = 0; c < NL; ++c) part[c] += wtot[w2 * DK + pc * 8 + c];
        }
      }
#pragma unroll
      for (int sh = NO; sh < 64; sh *= 2) {
#pragma unroll
        for (int c = 0; c < NL; ++c) part[c] += __shfl_xor(part[c], sh, 64);
      }
      float g2[NL];
#pragma unroll
      for (int c = 0; c < NL; ++c) g2[c] = part[c] + x[c];
      if constexpr (MODE == kGenericBw) {
        // the chunked backward's copy of G (its epilogues' decay factors;
        // chunk bases wave-uniform, lane offsets 32-bit)
        float* gco = a.gc + static_cast<size_t>(job) * (kC * DK);
        const int lo = t * DK + pc * 8;
        *reinterpret_cast<f32x4*>(gco + lo) = f32x4{g2[0], g2[SCAL ? 0 : 1], g2[SCAL ? 0 : 2], g2[SCAL ? 0 : 3]};
        *reinterpret_cast<f32x4*>(gco + lo + 4) =
            f32x4{g2[SCAL ? 0 : 4], g2[SCAL ? 0 : 5], g2[SCAL ? 0 : 6], g2[SCAL ? 0 : 7]};
      }
      float fp[8], fn[8], fx[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int cc = SCAL ? 0 : c;
        fp[c] = pad ? 0.f : __builtin_amdgcn_exp2f(g2[cc]);
        fn[c] = pad ? 0.f : __builtin_amdgcn_exp2f(-g2[cc]);
        fx[c] = pad ? 0.f : __builtin_amdgcn_exp2f(g2[cc] - l2[cc]);
      }
      if (t == kC - 1) {
        float e8[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          e8[c] = __builtin_amdgcn_exp2f(g2[SCAL ? 0 : c]);
          eGC[pc * 8 + c] = e8[c];
        }
        if constexpr (MODE == kGenericBw) {
          // and of e^{G} at the chunk's last token
          float* gmo = a.gam + static_cast<size_t>(job) * DK + pc * 8;
          *reinterpret_cast<f32x4*>(gmo) = f32x4{e8[0], e8[1], e8[2], e8[3]};
          *reinterpret_cast<f32x4*>(gmo + 4) = f32x4{e8[4], e8[5], e8[6], e8[7]};
        }
      }
      const bf16x8 sq = scale8(qv, fp), sk = scale8(kv, fn);
      *reinterpret_cast<bf16x8*>(Xl + xoff<DK>(NA + t, pc)) = sq;
      *reinterpret_cast<bf16x8*>(Xr + xoff<DK>(NA + t, pc)) = sk;
      if constexpr (MODE == kGenericBw) {
        // the chunked backward's copies: row t of the chunk, channels pc*8 ..
        // (chunk bases wave-uniform, lane offsets 32-bit)
        const size_t cb = static_cast<size_t>(job) * (kC * DK);
        const int lo = t * DK + pc * 8;
        *reinterpret_cast<bf16x8*>(a.qt + cb + lo) = sq;
        *reinterpret_cast<bf16x8*>(a.kt + cb + lo) = sk;
      }
      if (Cfg::GEN) {
#pragma unroll
        for (int r = 0; r < RAB; ++r) {
          const bf16x8 sa = scale8(av[r], fn), sb = scale8(bv[r], fx);
          *reinterpret_cast<bf16x8*>(Xr + xoff<DK>(RAB * t + r, pc)) = sa;
          *reinterpret_cast<bf16x8*>(Xl + xoff<DK>(RAB * t + r, pc)) = sb;
          if constexpr (MODE == kGenericBw) {
            const size_t cb = static_cast<size_t>(job) * (kC * RAB * DK);
            const int lo = (t * RAB + r) * DK + pc * 8;
            *reinterpret_cast<bf16x8*>(a.at + cb + lo) = sa;
            *reinterpret_cast<bf16x8*>(a.bt + cb + lo) = sb;
          }
        }
      } else {
        // Decay operands from the raw parameters.  With lambda = exp(l) and
        // exp(G_{t-1}) lambda = exp(G_t):
        //   HDLA  A = [b k, b u], B = [u - b c k, k], u = lambda k, c = k^T u
        //         A~ = [b k e^{-G_t}, b k e^{-G_{t-1}}],
        //         B~ = [k (e^{G_t} - b c e^{G_{t-1}}), k e^{G_{t-1}}]
        //   GDN   A = e^g b k, B = k:  A~ = b k e^{-G_{t-1}},  B~ = k e^{G_{t-1}}
        // The write K V^T = k (b v)^T keeps k here; b scales the operator's
        // value columns instead (below), so V is the raw v.
        const float b = pad ? 0.f : btv;
        if (pc == 0) betas[t] = b;
        float fnx[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) fnx[c] = b * fn[c] * __builtin_amdgcn_exp2f(l2[SCAL ? 0 : c]);
        if (MODE == kGdn) {
          *reinterpret_cast<bf16x8*>(Xr + xoff<DK>(t, pc)) = scale8(kv, fnx);
          *reinterpret_cast<bf16x8*>(Xl + xoff<DK>(t, pc)) = scale8(kv, fx);
        } else {
          // c = sum_i k_i^2 lambda_i over all channels: this lane's piece, then
          // the pieces of the same token (NO consecutive lanes).
          float cp = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float kc = (float)kv[c];
            cp += kc * kc * __builtin_amdgcn_exp2f(l2[c]);
          }
#pragma unroll
          for (int sh = 1; sh < NO; sh *= 2) cp += __shfl_xor(cp, sh, 64);
          float fb0[8], fa0[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            fb0[c] = fp[c] - b * cp * fx[c];
            fa0[c] = b * fn[c];
          }
          *reinterpret_cast<bf16x8*>(Xr + xoff<DK>(2 * t, pc)) = scale8(kv, fa0);
          *reinterpret_cast<bf16x8*>(Xr + xoff<DK>(2 * t + 1, pc)) = scale8(kv, fnx);
          *reinterpret_cast<bf16x8*>(Xl + xoff<DK>(2 * t, pc)) = scale8(kv, fb0);
          *reinterpret_cast<bf16x8*>(Xl + xoff<DK>(2 * t + 1, pc)) = scale8(kv, fx);
        }
      }
    };
    if (ncur < kC) {
      scale_phase(std::integral_constant<bool, true>{});
    } else {
      scale_phase(std::integral_constant<bool, false>{});
    }
    // The next chunk's inputs travel while this one is solved.
    const int64_t nxt = job + gridDim.x < total ? job + gridDim.x : total - 1;
    if (!Cfg::OVERLAP) load_a(nxt, lane);
    lds_barrier();

    // ---- P2: Gram blocks.  P^T = A~ [B~ ; Q~]^T, tiles (rs, cs) with cs >= rs,
    //      written straight to LDS.
    // A~ fragments of row block rs (the A operand of every tile in that row).
    auto gram_a = [&](int rs, bf16x8 (&af)[DK / 32]) {
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) af[kb] = xrow8<DK>(Xr, rs * 16, kb * 4, lane);
    };
    auto gram_tile = [&](int rs, int cs, const bf16x8 (&af)[DK / 32]) {
      // Which entries survive the token masks is uniform per tile except on
      // the diagonal: L tiles below it keep everything; an M_A tile (tokens tt)
      // keeps everything when its first token is >= the last token of the s
      // rows, nothing when its last token is < their first.
      const int tt = cs - NB;
      const bool zero = cs >= NB && 16 * tt + 15 < (16 * rs) / RB;
      const bool masked = cs < NB ? cs == rs : (!zero && 16 * tt < (16 * rs + 15) / RB);
      f32x4 acc = zero4();
      if (!zero) {
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
          acc = mfma32(af[kb], xrow8<DK>(Xl, cs * 16, kb * 4, lane), acc);
      }
      // lane holds P^T[s = rs*16 + 4lg + e][col = cs*16 + lr]
      if (masked) {
        const int row = cs < NB ? (cs * 16 + lr) / RB : tt * 16 + lr + 1;  // token bound: keep s/RAB < row
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!((rs * 16 + 4 * lg + e) / RB < row)) acc[e] = 0.f;
      }
      if (cs < NB) {
        if (cs == rs) {
          *reinterpret_cast<f32x4*>(Ldg + cs * LDB + lr * 16 + 4 * lg) = acc;
        } else {
          const int blk = cs * (cs - 1) / 2 + rs;
          *reinterpret_cast<bf16x4*>(Lpk + blk * 256 + lr * 16 + 4 * lg) = to_bf16x4(acc);
        }
      } else {
        // columns s = 32b + 16h + 4g + e at 32b + 8g + 4h + e (the K order of the operator product)
        *reinterpret_cast<bf16x4*>(MAs + (tt * 16 + lr) * LDA + (rs >> 1) * 32 + (rs & 1) * 4 + 8 * lg) = to_bf16x4(acc);
      }
    };
    // Tile idx of the row-major list of tiles (rs, cs), cs >= rs + skip.
    auto gram_tile_at = [&](int idx, int skip) {
      int rs = 0;
      while (idx >= NCS - skip - rs) {
        idx -= NCS - skip - rs;
        ++rs;
      }
      bf16x8 af[DK / 32];
      gram_a(rs, af);
      gram_tile(rs, rs + skip + idx, af);
    };

    // ---- P3: inverses of the unit lower-triangular diagonal blocks (I + L_ii),
    //      fp32, kept in fp32 for the diagonal apply below (fp32 MFMAs).
    //      Thread (blk, c) forms column c of block blk by forward substitution.
    auto invert_blocks = [&]() {
      if (tid < NB * 16) {
        const int blk = tid / 16, c = tid % 16;
        const float* Lb = Ldg + blk * LDB;
        float* Db = Dinv + blk * Cfg::DIB;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = (r == c) ? 1.f : 0.f;
#pragma unroll
          for (int m = 0; m < r; ++m) v -= Lb[r * 16 + m] * x[m];
          x[r] = v;
          Db[r * 16 + c] = v;
        }
      }
    };
    // The parts of an X wave's columns that need no solve: L_K = B~ K~^T (its
    // right-hand side, token(row) > chunk-write row) and M_K^T = K~ Q~^T (the
    // base of R, t >= s), from one copy of its K~ rows.
    bf16x4 lk[NBA], mk[kC / 16];
    auto x_products = [&]() {
      const int x = wave - DK / 16;
      bf16x8 kf[DK / 32];
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) kf[kb] = xrow8<DK>(Xr, NA + x * 16, kb * 4, lane);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        f32x4 g = zero4();
        // A tile whose rows all belong to tokens at or before the column
        // block's first token is all masked: skip its product.
        if ((i * 16 + 15) / RB > x * 16) {
#pragma unroll
          for (int kb = 0; kb < DK / 32; ++kb) g = mfma32(xrow8<DK>(Xl, i * 16, kb * 4, lane), kf[kb], g);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!((i * 16 + 4 * lg + e) / RB > x * 16 + lr)) g[e] = 0.f;
        lk[i] = to_bf16x4(g);
        // One tile at a time, converted to bf16 right away: interleaved tiles
        // kept in fp32 to the end only raise register pressure.
        asm volatile("" : "+v"(lk[i]));
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int tt = 0; tt < kC / 16; ++tt) {
        f32x4 g = zero4();
        if (tt >= x) {   // earlier token blocks are all masked
#pragma unroll
          for (int kb = 0; kb < DK / 32; ++kb) g = mfma32(kf[kb], xrow8<DK>(Xl, NA + tt * 16, kb * 4, lane), g);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!(tt * 16 + lr >= x * 16 + 4 * lg + e)) g[e] = 0.f;
        mk[tt] = to_bf16x4(g);
        asm volatile("" : "+v"(mk[tt]));
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    if (Cfg::OVERLAP) {
      // One phase for P2 and P3: the first NINV waves form the diagonal Gram
      // blocks that their own lanes invert (four blocks per wave, so no
      // other wave's result is waited for), the X waves form L_K and M_K, and
      // the remaining waves share the off-diagonal Gram tiles.
      constexpr int NINV = Cfg::NINV, NXW = Cfg::NXW, NWORK = Cfg::NWORK;
      if (wave < NINV) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (wave * 4 + j < NB) {
            bf16x8 af[DK / 32];
            gram_a(wave * 4 + j, af);
            gram_tile(wave * 4 + j, wave * 4 + j, af);
          }
        }
        // the inversion reads entries written by other lanes of this wave
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        invert_blocks();
      } else if (wave >= DK / 16 && wave < KT) {
        x_products();
      } else {
        // A contiguous run of the row-major list of off-diagonal tiles, so
        // that consecutive tiles share their A~ row block (read once per row).
        const int widx = wave < DK / 16 ? wave - NINV : wave - NINV - NXW;
        constexpr int NOFF = NTILE - NB;
        const int lo = widx * NOFF / NWORK, hi = (widx + 1) * NOFF / NWORK;
        int rs = 0, k = lo;
        while (k >= NCS - 1 - rs) {
          k -= NCS - 1 - rs;
          ++rs;
        }
        int cs = rs + 1 + k, ars = -1;
        bf16x8 af[DK / 32];
#pragma unroll 1
        for (int idx = lo; idx < hi; ++idx) {
          if (rs != ars) {
            gram_a(rs, af);
            ars = rs;
          }
          gram_tile(rs, cs, af);
          if (++cs == NCS) {
            ++rs;
            cs = rs + 1;
          }
        }
      }
      lds_barrier();
      // Issued only now, so that these registers are free during the Gram
      // phase; the solve and the operator product still cover their latency.
      load_a(nxt, lane);
      load_b(nxt, lane);
    } else {
      // All waves share the Gram tiles; then the inversion and the X-wave
      // products run side by side.
      if (Cfg::COMPACT) {
        // Only the L tiles (rs <= cs < NB) here; M_A comes after the solve.
        constexpr int NL = NB * (NB + 1) / 2;
#pragma unroll 1
        for (int idx = wave; idx < NL; idx += NW) {
          int rs = 0, k = idx;
          while (k >= NB - rs) {
            k -= NB - rs;
            ++rs;
          }
          bf16x8 af[DK / 32];
          gram_a(rs, af);
          gram_tile(rs, rs + k, af);
        }
      } else {
#pragma unroll
        for (int sl = 0; sl < Cfg::FULL_SLOTS; ++sl) gram_tile_at(wave + sl * NW, 0);
        if (Cfg::FULL_SLOTS * NW + wave < NTILE) gram_tile_at(Cfg::FULL_SLOTS * NW + wave, 0);
      }
      lds_barrier();
      load_b(nxt, lane);
      invert_blocks();
      if (wave >= DK / 16 && wave < KT) x_products();
      lds_barrier();
    }

    if constexpr (MODE == kGenericBw && RAB > 0) {
      // The chunked backward's copies of L's tiles below the diagonal and of
      // the diagonal blocks' inverses, all complete after the barrier above
      // (and kept until the solve has read them).  The waves that own no
      // solve column copy them where there are such waves.
      constexpr int NTI = NB * (NB - 1) / 2, W0 = NW > KT ? KT : 0, NCP = (NW - W0) * 64;
      constexpr int NLP = NTI * 32, NDI = NB * 64;   // 16-byte pieces
      if (wave >= W0) {
        __bf16* lto = a.lt + static_cast<size_t>(job) * (NTI * 256);
        float* dio = a.di + static_cast<size_t>(job) * (NB * 256);
#pragma unroll 1
        for (int it = tid - W0 * 64; it < NLP + NDI; it += NCP) {
          if (it < NLP) {
            *reinterpret_cast<bf16x8*>(lto + it * 8) = *reinterpret_cast<const bf16x8*>(Lpk + it * 8);
          } else {
            const int d = it - NLP, blk = d / 64, r = d % 64;
            *reinterpret_cast<f32x4*>(dio + blk * 256 + r * 4) =
                *reinterpret_cast<const f32x4*>(Dinv + blk * Cfg::DIB + r * 4);
          }
        }
      }
    }

    // ---- P4: blocked forward substitution on wave kt's columns:
    //      WX_i = (I + L_ii)^{-1} (RHS_i - sum_{j<i} L_ij WX_j).
    auto solve = [&](const int kt, bf16x4 (&wx)[NBA]) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        f32x4 acc;
        if (kt < DK / 16) {
          // W columns: B~ itself.
          acc = to_f32x4(xtr4<DK>(Xl, i * 16, kt * 16, lane));
        } else {
          acc = to_f32x4(lk[i]);   // X columns: L_K
        }
        const __bf16* Lrow = Lpk + (i * (i - 1) / 2) * 256 + lr * 16 + 4 * lg;
#pragma unroll
        for (int jb = 0; jb + 1 < i; jb += 2)
          acc = mfma32(cat(lds4(Lrow + jb * 256), lds4(Lrow + (jb + 1) * 256)), cat(wx[jb], wx[jb + 1]), acc);
        if (i % 2 == 1) {
          // Odd leftover block: padded to a 16x16x32 product with a zero half
          // (the whole chain uses one MFMA shape).
          bf16x4 zb;
          zb[0] = zb[1] = zb[2] = zb[3] = (__bf16)0.f;
          acc = mfma32(cat(lds4(Lrow + (i - 1) * 256), zb), cat(wx[i - 1], zb), acc);
        }
        // (I + L_ii)^{-1} acc in fp32: four 16x16x4 MFMAs over a permuted K,
        // product e pairing column 4*lg + e of the inverse (this lane's row
        // lr) with row 4*lg + e of acc (this lane's acc[e]).
        const f32x4 dF = *reinterpret_cast<const f32x4*>(Dinv + i * Cfg::DIB + lr * 16 + 4 * lg);
        f32x4 o = zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) o = __builtin_amdgcn_mfma_f32_16x16x4f32(dF[e], acc[e], o, 0, 0, 0);
        wx[i] = to_bf16x4(f32x4{-o[0], -o[1], -o[2], -o[3]});   // -WX_i
      }
    };
    auto operator_tiles = [&](const int kt, const bf16x4 (&wx)[NBA]) {
      // ---- P5: operator tiles, transposed product: rows = this wave's input
      //      column tile, columns = output rows m (channels, then tokens):
      //      acc = sum_s WX[s][k] Bmat[m][s],  Bmat = [A~^T ; M_A].
      // Fused modes: the value columns (chunk tokens) carry beta of their token.
      f32x4 vsc = f32x4{1.f, 1.f, 1.f, 1.f};
      if (!Cfg::GEN && kt >= DK / 16) vsc = *reinterpret_cast<const f32x4*>(betas + (kt - DK / 16) * 16 + 4 * lg);
      auto store = [&](int mt, const f32x4& v) {
        const f32x4 w = f32x4{v[0] * vsc[0], v[1] * vsc[1], v[2] * vsc[2], v[3] * vsc[3]};
        *reinterpret_cast<bf16x4*>(Mout + ((mt * (KT / 2) + kt / 2) * 64 + lane) * 8 + (kt & 1) * 4) = to_bf16x4(w);
      };
      // Output rows that are channels (Acal, Z): base I or K~^T, scaled by exp(G_C).
#pragma unroll 1
      for (int mt = 0; mt < DK / 16; ++mt) {
        // The product accumulates onto the base: base + sum (-WX) Bmat.
        f32x4 acc = zero4();
        if (kt < DK / 16) {
          if (kt == mt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = (4 * lg + e == lr) ? 1.f : 0.f;
          }
        } else {
          acc = to_f32x4(xtr4<DK>(Xr, NA + kt * 16 - DK, mt * 16, lane));
        }
#pragma unroll
        for (int jb = 0; jb < NB; jb += 2)
          acc = mfma32(cat(wx[jb], wx[jb + 1]),
                       cat(xtr4<DK>(Xr, jb * 16, mt * 16, lane), xtr4<DK>(Xr, jb * 16 + 16, mt * 16, lane)), acc);
        const float sc = eGC[mt * 16 + lr];
        store(mt, f32x4{sc * acc[0], sc * acc[1], sc * acc[2], sc * acc[3]});
      }
      // Output rows that are tokens (Qbar, R): base Q~ or M_K.
#pragma unroll
      for (int tt = 0; tt < kC / 16; ++tt) {
        const __bf16* Brow = MAs + (tt * 16 + lr) * LDA + 8 * lg;
        f32x4 acc;
        if (kt < DK / 16) {
          acc = to_f32x4(lds4(Xl + xoff<DK>(NA + tt * 16 + lr, 2 * kt + (lg >> 1)) + 4 * (lg & 1)));
        } else {
          acc = to_f32x4(mk[tt]);   // M_K^T
        }
#pragma unroll
        for (int jb = 0; jb < NB; jb += 2) acc = mfma32(cat(wx[jb], wx[jb + 1]), lds8(Brow + jb * 16), acc);
        store(DK / 16 + tt, acc);
      }
    };
    if (!Cfg::COMPACT) {
      if (wave < KT) {
        bf16x4 wx[NBA];
        solve(wave, wx);
        operator_tiles(wave, wx);
      }
    } else {
      bf16x4 wx[NBA];
      if (wave < KT) solve(wave, wx);
      // M_A = Q~ A~^T into the region of L, the inverses and B~, which every
      // wave's solve has finished reading after this barrier.  Wave w forms
      // the four token-column tiles of row block w % NB.
      static_assert(!Cfg::COMPACT || NW % NB == 0, "compact M_A phase: whole row blocks per wave");
      lds_barrier();
      bf16x8 af[DK / 32];
      gram_a(wave % NB, af);
#pragma unroll
      for (int idx = wave; idx < NB * (kC / 16); idx += NW) gram_tile(wave % NB, NB + idx / NB, af);
      lds_barrier();
      if (wave < KT) operator_tiles(wave, wx);
    }
    // P5 reads Xl, Xr and M_A, which the next chunk overwrites.
    lds_barrier();
  }
}

// ---------------------------------------------------------------------------
// Scan kernel: per (batch*head, BV-wide d_v slice), chunks in order,
// Y = M_j [S ; V_j] with the operator fragments read straight from HBM.
//
// The right operand X = [S ; V_j] (KIN x BV) lives in LDS as X^T, bf16, with
// its K index permuted inside every 32-wide block so that one 16-byte read
// gives a lane the eight K values of a 16x16x32 MFMA that pairs two stored
// 16x16 operator tiles: position 8*g + 4*h + e of block b holds
// k = 32*b + 16*h + 4*g + e.  Two such buffers alternate between chunks, so
// one barrier per chunk orders the state write against the next product.
// The operator and V of the next PD chunks are held in registers (a ring of
// PD buffers), so HBM latency overlaps PD chunk steps.  Output rows go
// through an LDS staging buffer and leave as 16-byte row stores one chunk
// later.
template <int DK, int BV, int NWV, int PD>
struct ScanCfg {
  static constexpr int KIN = DK + kNK;
  static constexpr int ROUT = DK + kC;
  static constexpr int KT = KIN / 16;
  static constexpr int KP = KT / 2;
  static constexpr int MT = ROUT / 16;
  static constexpr int NT = 64 * NWV;
  static constexpr int MPW = MT / NWV;     // output row tiles per wave
  static constexpr int NTN = BV / 16;      // output column tiles
  // padded row of X^T (bf16): a row stride of 32 mod 64 bytes keeps the
  // 16-row fragment reads free of LDS bank conflicts (measured on gfx950)
  static constexpr int LDX = KIN + 16;
  static constexpr int XBUF = BV * LDX;    // elements of one X^T buffer
  static constexpr int LDO = BV + 8;       // padded row of the output stage
  static constexpr int OBUF = kC * LDO;
  static constexpr int LDS = 2 * (XBUF + OBUF) * 2;
  // the boundary-state instance stages the DK state rows instead of the output rows
  static constexpr int SBUF = DK * LDO;
  static constexpr int LDS_CK = 2 * (XBUF + SBUF) * 2;
  static constexpr int SITEMS = DK * (BV / 8);       // 16-byte state pieces
  static constexpr int SIT = (SITEMS + NT - 1) / NT;
  static constexpr int MSZ = MT * KT * 256;          // operator elements per chunk
  static constexpr int VT = 2;                       // tokens per V piece
  static constexpr int VITEMS = (kC / VT) * (BV / 8); // VT tokens x 8 columns each
  static constexpr int VIT = (VITEMS + NT - 1) / NT;
  static constexpr int OITEMS = kC * (BV / 8);       // 16-byte output pieces
  static constexpr int OIT = (OITEMS + NT - 1) / NT;
  static_assert(MT % NWV == 0 && KT % 2 == 0 && BV % 16 == 0 && PD % 2 == 0, "scan tiling");
};

__device__ __forceinline__ int kperm(int k) {
  return (k & ~31) | ((k & 12) << 1) | ((k & 16) >> 2) | (k & 3);
}

struct FastScanArgs {
  Problem p;
  const __bf16* M;
  const __bf16* v;
  __bf16* out;         // output rows (the forward instance)
  float* Sfin;
  const float* S0;
  __bf16* ckpt;        // [BH, N + 1, dk, dv]: the state entering every chunk, then the final state (the boundary instance)
  // The instance split in nseg sequence segments of L chunks (the last one
  // shorter): every segment after the first runs from a zero state beside its
  // transport (the product of its chunks' state transitions, from I); its
  // outputs and final state are then corrected with the state entering it
  // (see fast_scan).
  int64_t L;
  int nseg;
  __bf16* U;     // [BH, N - L, C, dk]: the later segments' query rows times their transport so far
  float* Smid;   // [BH, dk, dv]: the state leaving segment 0
  float* Sp;     // [nseg - 1][BH, dk, dv]: segment s's zero-start final state (slot s - 1)
  float* Tf;     // [nseg - 1][BH, dk, dk]: segment s's transport (slot s - 1)
};

// CK: what the scan stores.  kScanOut: the output rows (and the final state);
// kScanStates: the state entering every chunk instead of the output rows (the
// backward's boundary scan); kScanBoth: both (the training forward).
enum ScanStore { kScanOut = 0, kScanStates = 1, kScanBoth = 2 };
template <int DK, int BV, int NWV, int PD, int CK, bool SG = false>
__global__ __launch_bounds__(64 * NWV) void fast_scan_kernel(FastScanArgs a) {
  using Cfg = ScanCfg<DK, BV, NWV, PD>;
  constexpr int KP = Cfg::KP, MPW = Cfg::MPW, NTN = Cfg::NTN, LDX = Cfg::LDX, NT = Cfg::NT;
  constexpr int XBUF = Cfg::XBUF, LDO = Cfg::LDO, OBUF = CK == kScanStates ? Cfg::SBUF : Cfg::OBUF, MSZ = Cfg::MSZ;
  constexpr int VITEMS = Cfg::VITEMS, OITEMS = Cfg::OITEMS, OIT = Cfg::OIT;
  static_assert(Cfg::VIT == 1, "one V piece per thread");
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* X0 = reinterpret_cast<__bf16*>(smem);
  __bf16* O0 = X0 + 2 * XBUF;
  const Problem& p = a.p;
  const int dv = p.dv;
  const int nvt = dv / BV;
  // Workgroups per head: the d_v slices; split in segments, segment 0's
  // slices, then each later segment's slices and its transport's d_k slices.
  static_assert(!SG || CK == kScanOut, "segments: the output instance only");
  const int R = SG ? nvt + (a.nseg - 1) * (nvt + DK / BV) : nvt;
  // Blocks of one (batch, head) land on one XCD (dispatch is round-robin over 8).
  const int b = blockIdx.x;
  const int grp = b / (8 * R), rem = b % (8 * R);
  const int role = rem / 8;
  const int64_t bh = static_cast<int64_t>(grp) * 8 + rem % 8;
  const int64_t N = p.N;
  if (bh >= p.BH || N == 0) return;
  // this workgroup's chunks [j0, j1), its slice, and (split) its segment and role
  int64_t j0 = 0, j1 = N;
  int seg = 0, vt = role;
  bool tr = false;   // a transport slice: columns of I, no V
  if constexpr (SG) {
    if (role >= nvt) {
      const int r = role - nvt, per = nvt + DK / BV;
      seg = 1 + r / per;
      tr = r % per >= nvt;
      vt = r % per - (tr ? nvt : 0);
    }
    j0 = seg * a.L;
    j1 = seg == a.nseg - 1 ? N : j0 + a.L;
  }
  const int c0 = vt * BV;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  const __bf16* Mbh = a.M + static_cast<size_t>(bh) * N * MSZ;
  const int moff = wave * MPW * KP * 512 + lane * 8;
  // V piece of this thread: tokens VT*vs .. VT*vs+VT-1, columns 8*vc .. 8*vc+7.
  constexpr int VT = Cfg::VT;
  const int vitem = tid < VITEMS ? tid : VITEMS - 1;
  const int vs = vitem / (BV / 8), vc = vitem % (BV / 8);
  const __bf16* vbh = a.v + static_cast<size_t>(bh) * p.T * dv + c0;
  // output rows: out [BH, T, dv], or (transport) U [BH, N - js, C, dk]; the
  // final state's destination and row stride
  __bf16* obh = a.out + static_cast<size_t>(bh) * p.T * dv + c0;
  int ost = dv, sst = dv;
  int64_t jb = 0;
  float* sfin = a.Sfin;
  if constexpr (SG) {
    if (tr) {
      vbh = a.v + static_cast<size_t>(bh) * p.T * dv;
      obh = a.U + static_cast<size_t>(bh) * (N - a.L) * kC * DK + c0;
      ost = sst = DK;
      jb = a.L;
    }
    // the last segment's final state matters only for the returned one
    const bool keep = seg < a.nseg - 1 || a.Sfin;
    sfin = seg == 0 ? a.Smid
                    : (!keep ? nullptr
                             : (tr ? a.Tf + static_cast<size_t>(seg - 1) * p.BH * DK * DK
                                   : a.Sp + static_cast<size_t>(seg - 1) * p.BH * DK * dv));
  }

  bf16x8 mf[PD][MPW][KP];
  bf16x8 vb[2][VT];   // V ring: two chunks ahead is enough for its few KB
  auto chunk_len = [&](int64_t jj) {
    const int64_t r = p.T - jj * kC;
    return static_cast<int>(r < kC ? r : kC);   // <= 0 past the last chunk
  };
  // tokens this workgroup stores for chunk jj (none outside its chunks)
  auto store_len = [&](int64_t jj) {
    if constexpr (SG) return jj < j1 ? chunk_len(jj) : 0;
    return chunk_len(jj);
  };
  // Loads are unconditional (chunk and token indices are clamped), so no
  // control flow separates a prefetch from the work it overlaps.
  // The boundary-state instance needs only the operator's state rows: a
  // wave skips its output row tiles (a wave-uniform test).
  auto live = [&](int q) { return CK != kScanStates || wave * MPW + q < DK / 16; };
  auto load_m = [&](bf16x8 (&dst)[MPW][KP], int64_t jj) {
    jj = jj < N ? jj : N - 1;
    const __bf16* Mj = Mbh + static_cast<size_t>(jj) * MSZ;
#pragma unroll
    for (int q = 0; q < MPW; ++q)
      if (live(q)) {
#pragma unroll
        for (int kp = 0; kp < KP; ++kp)
          dst[q][kp] = *reinterpret_cast<const bf16x8*>(Mj + moff + (q * KP + kp) * 512);
      }
  };
  auto load_v = [&](bf16x8 (&dst)[VT], int64_t jj) {
    jj = jj < N ? jj : N - 1;
    const __bf16* vj = vbh + static_cast<size_t>(jj) * kC * dv;
    const int last = chunk_len(jj) - 1;
#pragma unroll
    for (int r = 0; r < VT; ++r) {
      const int s = VT * vs + r < last ? VT * vs + r : last;
      dst[r] = *reinterpret_cast<const bf16x8*>(vj + (s * dv + vc * 8));
    }
  };
  // V_jj^T into the V rows of an X^T buffer (VT tokens per write); rows past
  // the chunk's end are zero.
  typedef __attribute__((__vector_size__(VT * sizeof(__bf16)))) __bf16 bf16xVT;
  auto put_v = [&](__bf16* X, const bf16x8 (&src)[VT], int64_t jj) {
    const int n = SG && tr ? 0 : chunk_len(jj);
    if (tid < VITEMS) {
      const int pos = kperm(DK + VT * vs);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16xVT w;
#pragma unroll
        for (int r = 0; r < VT; ++r) w[r] = VT * vs + r < n ? src[r][e] : (__bf16)0.f;
        *reinterpret_cast<bf16xVT*>(X + (vc * 8 + e) * LDX + pos) = w;
      }
    }
  };
  // Output rows of chunk jj from a staging buffer to HBM (none past the end);
  // the boundary-state instance: the state leaving chunk jj (slot jj + 1).
  auto flush_out = [&](const __bf16* O, int64_t jj) {
    if constexpr (CK == kScanStates) {
      if (jj >= N) return;
      __bf16* ck = a.ckpt + static_cast<size_t>(bh * (N + 1) + jj + 1) * DK * dv + c0;
#pragma unroll
      for (int q = 0; q < Cfg::SIT; ++q) {
        const int it = tid + q * NT;
        const int i = it / (BV / 8), cg = it % (BV / 8);
        if (it < Cfg::SITEMS) *reinterpret_cast<bf16x8*>(ck + (i * dv + cg * 8)) = lds8(O + i * LDO + cg * 8);
      }
      return;
    }
    const int n = store_len(jj);
    // (the unsplit instances keep their own expressions: the boundary-state
    // output instance sits at the VGPR limit of its 12 waves)
    __bf16* oj = SG ? obh + static_cast<size_t>(jj - jb) * kC * ost : obh + static_cast<size_t>(jj) * kC * dv;
    const int os = SG ? ost : dv;
#pragma unroll
    for (int q = 0; q < OIT; ++q) {
      const int it = tid + q * NT;
      const int t = it / (BV / 8), cg = it % (BV / 8);
      if (it < OITEMS && t < n) *reinterpret_cast<bf16x8*>(oj + (t * os + cg * 8)) = lds8(O + t * LDO + cg * 8);
    }
  };

#pragma unroll
  for (int u = 0; u < PD; ++u) load_m(mf[u], j0 + u);
  load_v(vb[0], j0);
  load_v(vb[1], j0 + 1);
  for (int it = tid; it < DK * BV; it += NT) {
    const int i = it / BV, c = it % BV;
    // the state entering chunk j0: the initial state, or (segment 1) zero
    // beside the transport's identity columns
    const float s = SG && seg ? (tr && i == c0 + c ? 1.f : 0.f) : (a.S0 ? a.S0[(bh * DK + i) * dv + c0 + c] : 0.f);
    X0[c * LDX + kperm(i)] = (__bf16)s;
    if (CK == kScanStates) a.ckpt[(static_cast<size_t>(bh * (N + 1)) * DK + i) * dv + c0 + c] = (__bf16)s;
  }
  put_v(X0, vb[0], j0);
  // Ring invariant from here on (j0 is even): at chunk jj, vb[(jj + 1) % 2] holds V_{jj+1}.
  load_v(vb[0], j0 + 2);
  lds_barrier();

  // One chunk: product from X buffer u&1; state and V_{jj+1} into the other,
  // outputs into stage u&1; the previous chunk's stage goes out meanwhile.
  // Steps past the last chunk (to finish a group of PD) compute on clamped
  // data and store nothing.
  auto step = [&](const int u, const int64_t jj) {
    const __bf16* Xc = X0 + (u & 1) * XBUF;
    __bf16* Xn = X0 + ((u + 1) & 1) * XBUF;
    __bf16* Oc = O0 + (u & 1) * OBUF;
    f32x4 acc[MPW][NTN];
#pragma unroll
    for (int q = 0; q < MPW; ++q)
#pragma unroll
      for (int nt = 0; nt < NTN; ++nt) acc[q][nt] = zero4();
    // The next use of each operator register is chunk jj + PD: its load is
    // issued as soon as this chunk's MFMAs have read it, spreading the loads
    // over the product instead of bunching them after it.
    const __bf16* Mnext = Mbh + static_cast<size_t>(jj + PD < N ? jj + PD : N - 1) * MSZ;
    // (a wave whose first row tile is an output tile has no live tile)
#pragma unroll
    for (int kp = 0; kp < (live(0) ? KP : 0); ++kp) {
      bf16x8 bv[NTN];
#pragma unroll
      for (int nt = 0; nt < NTN; ++nt) bv[nt] = lds8(Xc + (nt * 16 + lr) * LDX + kp * 32 + 8 * lg);
#pragma unroll
      for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int q = 0; q < MPW; ++q)
          if (live(q)) acc[q][nt] = mfma32(mf[u][q][kp], bv[nt], acc[q][nt]);
#pragma unroll
      for (int q = 0; q < MPW; ++q)
        if (live(q)) mf[u][q][kp] = *reinterpret_cast<const bf16x8*>(Mnext + moff + (q * KP + kp) * 512);
    }
    if (jj > (SG ? j0 : 0)) flush_out(O0 + ((u + 1) & 1) * OBUF, jj - 1);
#pragma unroll
    for (int q = 0; q < MPW; ++q) {
      const int mt = wave * MPW + q;
#pragma unroll
      for (int nt = 0; nt < NTN; ++nt) {
        const int c = nt * 16 + lr;
        if (mt < DK / 16) {
          const bf16x4 h = to_bf16x4(acc[q][nt]);
          *reinterpret_cast<bf16x4*>(Xn + c * LDX + kperm(mt * 16 + 4 * lg)) = h;
          if (CK == kScanStates) {
            // the state rows, rounded as the next product reads them, staged
            // row-major for the 16-byte stores one chunk later
#pragma unroll
            for (int e = 0; e < 4; ++e) Oc[(mt * 16 + 4 * lg + e) * LDO + c] = h[e];
          }
        } else if (CK != kScanStates) {
          const int t = (mt - DK / 16) * 16 + 4 * lg;
#pragma unroll
          for (int e = 0; e < 4; ++e) Oc[(t + e) * LDO + c] = (__bf16)acc[q][nt][e];
        }
      }
    }
    if (CK == kScanBoth && jj == N - 1) {
      // the state leaving the last chunk (slot N), rounded as the next
      // product would read it
      __bf16* ck = a.ckpt + static_cast<size_t>(bh * (N + 1) + N) * DK * dv + c0;
#pragma unroll
      for (int q = 0; q < MPW; ++q) {
        const int mt = wave * MPW + q;
        if (mt < DK / 16) {
#pragma unroll
          for (int nt = 0; nt < NTN; ++nt) {
            const bf16x4 h = to_bf16x4(acc[q][nt]);
#pragma unroll
            for (int e = 0; e < 4; ++e) ck[(mt * 16 + 4 * lg + e) * dv + nt * 16 + lr] = h[e];
          }
        }
      }
    }
    if (SG ? (jj == j1 - 1 && sfin) : (jj == N - 1 && a.Sfin)) {
#pragma unroll
      for (int q = 0; q < MPW; ++q) {
        const int mt = wave * MPW + q;
        if (mt < DK / 16) {
#pragma unroll
          for (int nt = 0; nt < NTN; ++nt) {
            const int i0 = mt * 16 + 4 * lg, c = nt * 16 + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) (SG ? sfin : a.Sfin)[(bh * DK + i0 + e) * (SG ? sst : dv) + c0 + c] = acc[q][nt][e];
          }
        }
      }
    }
    const int un = (u + 1) % 2;
    put_v(Xn, vb[un], jj + 1);
    load_v(vb[un], jj + 3);
    if constexpr (CK == kScanBoth) {
      // the state entering chunk jj (slot jj), from the operand buffer this
      // step's product read (rewritten only after the barrier below): a
      // thread gathers 8 columns of one row, consecutive threads take
      // consecutive rows, so the 2-byte LDS reads of a wave hit distinct banks
      if (jj < N) {
        __bf16* ck = a.ckpt + static_cast<size_t>(bh * (N + 1) + jj) * DK * dv + c0;
#pragma unroll
        for (int q = 0; q < Cfg::SIT; ++q) {
          const int it = tid + q * NT;
          const int i = it % DK, cg = it / DK;
          if (it < Cfg::SITEMS) {
            bf16x8 w;
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = Xc[(cg * 8 + e) * LDX + kperm(i)];
            *reinterpret_cast<bf16x8*>(ck + (i * dv + cg * 8)) = w;
          }
        }
      }
    }
    lds_barrier();
  };

  for (int64_t j = SG ? j0 : 0; j < (SG ? j1 : N); j += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) step(u, j + u);
  }
  // The last chunk's outputs, unless a step past the end already sent them.
  if constexpr (SG) {
    if ((j1 - j0) % PD == 0) flush_out(O0 + ((j1 - 1 - j0) & 1) * OBUF, j1 - 1);
  } else {
    if (N % PD == 0) flush_out(O0 + ((N - 1) & 1) * OBUF, N - 1);
  }
}

// ---------------------------------------------------------------------------
// Gating-chunk summaries for the query-conditioned composition (HLA note,
// "Method steps", steps 2 and 5): for a gating chunk of G consecutive 64-token
// chunks, the exact affine pair of the whole gating chunk and, for each of its
// queries, the operator on the incoming state and the output from a zero
// state.  It is the scan's product run over the G chunks from the state
// [I | 0], with d_k "transport" columns (value rows zero) next to the d_v
// "write" columns (value rows V):
//   [P' ; Qp] = M_x [P ; 0],      [W' ; Ow] = M_x [W ; V_x],
// so after the G steps P = Acal_J and W = B_J, and the bottom rows of step x
// are its queries' rows: Qp = Qbar_x P (the incoming-state operator) and
// Ow = Qbar_x W + R_x V_x (the outputs from a zero state).  Operators come
// straight from the prepare's fragment-ordered bf16 tiles; the state between
// steps is rounded to bf16 (the MFMA operand), fp32 accumulate.  Stored per
// gating chunk: AT = Acal_J^T [dk][dk] and BT = B_J^T [dv][dk] in bf16 (the B
// operands of the composition's bf16 products), QB [L][dk] and OI [L][dv] in
// fp32.  One workgroup per (batch*head, gating chunk,
// 64-column slice of the d_k + d_v columns), one wave per 16-row tile of M_x.
struct FastGateArgs {
  Problem p;        // the 64-token problem: N = ceil(T / 64)
  int G;            // 64-token chunks per gating chunk
  int64_t NL;       // gating chunks per (batch, head)
  const __bf16* M;  // fragment-ordered chunk operators
  const __bf16* v;  // V [BH, T, dv]
  __bf16* AT;
  __bf16* BT;
  float* QB;
  float* OI;
};

template <int DK>
struct GateCfg {
  static constexpr int KIN = DK + kNK;
  static constexpr int MT = (DK + kC) / 16;
  static constexpr int KP = KIN / 32;
  static constexpr int NT = 64 * MT;
  static constexpr int LDX = KIN + 16;      // padded X^T row (bf16), as in the scan
  static constexpr int XBUF = 64 * LDX;
  static constexpr int LDS = 2 * XBUF * 2;
};

template <int DK>
__global__ __launch_bounds__(GateCfg<DK>::NT) void fast_gate_kernel(FastGateArgs a) {
  using Cfg = GateCfg<DK>;
  constexpr int KP = Cfg::KP, LDX = Cfg::LDX, XBUF = Cfg::XBUF, NT = Cfg::NT, DKT = DK / 16;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* X0 = reinterpret_cast<__bf16*>(smem);
  const Problem& p = a.p;
  const int dv = p.dv, G = a.G;
  const int NS = (DK + dv) / 64;
  const int s = static_cast<int>(blockIdx.x % NS);
  const int64_t job = blockIdx.x / NS;            // (batch*head, gating chunk)
  const int64_t bh = job / a.NL, J = job % a.NL;
  const int L = G * kC;
  const bool tr = s * 64 < DK;                    // transport columns (else write columns)
  const int col0 = tr ? s * 64 : s * 64 - DK;     // first column of the slice in P or W
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t j0 = J * G;
  const int nsub = static_cast<int>(p.N - j0 < G ? p.N - j0 : G);
  const size_t MSZ = static_cast<size_t>(Cfg::MT) * (Cfg::KIN / 16) * 256;
  const __bf16* Mbh = a.M + static_cast<size_t>(bh) * p.N * MSZ;
  // Initial X^T in both buffers: state [I | 0] of this slice, value rows zero.
  for (int it = tid; it < 2 * XBUF; it += NT) X0[it] = (__bf16)0.f;
  __syncthreads();
  if (tr && tid < 64) {
    const int c = tid;   // local column; state row col0 + c holds 1
    X0[c * LDX + kperm(col0 + c)] = (__bf16)1.f;
  }
  // V rows of chunk jj (write slices only) into buffer X, rows past the chunk's end zero.
  auto put_v = [&](__bf16* X, int64_t jj) {
    if (tr) return;
    const int64_t t0 = jj * kC;
    const int n = static_cast<int>(p.T - t0 < kC ? p.T - t0 : kC);
    if (tid < kC * 8) {
      const int t = tid / 8, cg = tid % 8;   // token t, columns 8 cg .. 8 cg + 7 of the slice
      bf16x8 w;
      if (t < n) {
        w = *reinterpret_cast<const bf16x8*>(a.v + (static_cast<size_t>(bh) * p.T + t0 + t) * dv + col0 + 8 * cg);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (__bf16)0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) X[(8 * cg + e) * LDX + kperm(DK + t)] = w[e];
    }
  };
  put_v(X0, j0);
  __syncthreads();
  const int mt = wave;
  for (int x = 0; x < nsub; ++x) {
    const __bf16* Xc = X0 + (x & 1) * XBUF;
    __bf16* Xn = X0 + ((x + 1) & 1) * XBUF;
    const __bf16* Mj = Mbh + static_cast<size_t>(j0 + x) * MSZ;
    bf16x8 mf[KP];
#pragma unroll
    for (int kp = 0; kp < KP; ++kp) mf[kp] = *reinterpret_cast<const bf16x8*>(Mj + ((mt * KP + kp) * 64 + lane) * 8);
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
#pragma unroll
    for (int kp = 0; kp < KP; ++kp) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = mfma32(mf[kp], lds8(Xc + (nt * 16 + lr) * LDX + kp * 32 + 8 * lg), acc[nt]);
    }
    const bool last = x + 1 == nsub;
    if (mt < DKT) {
      // new state rows mt*16 + 4 lg + e of columns c
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int c = nt * 16 + lr;
        if (!last) *reinterpret_cast<bf16x4*>(Xn + c * LDX + kperm(mt * 16 + 4 * lg)) = to_bf16x4(acc[nt]);
        else if (tr) *reinterpret_cast<bf16x4*>(a.AT + (static_cast<size_t>(job) * DK + col0 + c) * DK + mt * 16 + 4 * lg) = to_bf16x4(acc[nt]);
        else *reinterpret_cast<bf16x4*>(a.BT + (static_cast<size_t>(job) * dv + col0 + c) * DK + mt * 16 + 4 * lg) = to_bf16x4(acc[nt]);
      }
    } else {
      // query rows: token x*64 + (mt - DKT)*16 + 4 lg + e of the gating chunk
      float* dst = tr ? a.QB + static_cast<size_t>(job) * L * DK : a.OI + static_cast<size_t>(job) * L * dv;
      const int ld = tr ? DK : dv;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[static_cast<size_t>(x * kC + (mt - DKT) * 16 + 4 * lg + e) * ld + col0 + nt * 16 + lr] = acc[nt][e];
    }
    if (!last) put_v(Xn, j0 + x + 1);
    __syncthreads();
  }
}

template <int DK, int RAB, bool SCAL, int MODE>
hipError_t launch_prep(const Problem& p, const void* q, const void* k, const float* ld,
                       const void* A, const void* B, const float* beta, void* M, hipStream_t s,
                       const PrepBwOut* bw = nullptr) {
  using Cfg = PrepCfg<DK, RAB, SCAL, MODE>;
  FastPrepArgs a{p, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), ld,
                 static_cast<const __bf16*>(A), static_cast<const __bf16*>(B), beta, static_cast<__bf16*>(M),
                 nullptr, nullptr, nullptr, nullptr};
  if (MODE == kGenericBw) {
    if (!bw) return hipErrorInvalidValue;
    a.qt = static_cast<__bf16*>(bw->qt);
    a.kt = static_cast<__bf16*>(bw->kt);
    a.at = static_cast<__bf16*>(bw->at);
    a.bt = static_cast<__bf16*>(bw->bt);
    a.lt = static_cast<__bf16*>(bw->lt);
    a.di = static_cast<float*>(bw->di);
    a.gc = static_cast<float*>(bw->gc);
    a.gam = static_cast<float*>(bw->gam);
  }
  const void* fn = reinterpret_cast<const void*>(fast_prepare_kernel<DK, RAB, SCAL, MODE>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // As many persistent workgroups as can be resident at once (one per compute
  // unit, two with the compact d_k = 64 layout), each walking a strided set of
  // chunks.
  int per_cu = 1;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, Cfg::NT, Cfg::LDS);
  if (e != hipSuccess) return e;
  per_cu = per_cu < 1 ? 1 : (per_cu > 2 ? 2 : per_cu);
  const int64_t jobs = p.BH * p.N;
  const int64_t slots = static_cast<int64_t>(cus) * per_cu;
  const int64_t grid = jobs < slots ? jobs : slots;
  hipLaunchKernelGGL((fast_prepare_kernel<DK, RAB, SCAL, MODE>), dim3(grid), dim3(Cfg::NT), Cfg::LDS, s, a);
  return hipGetLastError();
}

template <int DK, int RAB>
hipError_t launch_prep(const Problem& p, const void* q, const void* k, const float* ld,
                       const void* A, const void* B, void* M, hipStream_t s) {
  return p.scalar ? launch_prep<DK, RAB, true, kGeneric>(p, q, k, ld, A, B, nullptr, M, s)
                  : launch_prep<DK, RAB, false, kGeneric>(p, q, k, ld, A, B, nullptr, M, s);
}

// ---------------------------------------------------------------------------
// The split scan's correction.  The state entering segment s >= 1 is
//   S_1 = Smid,  S_{s+1} = Sp_s + Tf_s S_s
// (fp32, a fixed-order sum; fast_segchain_kernel forms S_s for s >= 2, one
// workgroup per head).  Every output row of segment s then gains U_j S_s
// (bf16 MFMAs with fp32 accumulation, the sum rounded once), and the final
// state is Sp_last + Tf_last S_last (fp32).  fast_segfix_kernel: one
// four-wave workgroup per kSegFixG consecutive chunks after segment 0 (wave
// w: the chunk's 16-token row block w), staging S_s once per segment it
// meets; with a final state, first one workgroup per head for it (its serial
// sums then overlap the chunks' workgroups instead of trailing them).
constexpr int kSegFixG = 8;
struct SegFixArgs {
  Problem p;
  int64_t L;
  int nseg;
  const __bf16* U;
  const float *Smid, *Sp, *Tf;
  float* Sst;   // [nseg - 2][BH, dk, dv]: the state entering segment s >= 2 (slot s - 2)
  __bf16* out;
  float* Sfin;
};

// the state entering segment s >= 1 of head bh
template <int DK>
__device__ __forceinline__ const float* seg_start(const SegFixArgs& a, int s, int64_t bh) {
  const size_t st = static_cast<size_t>(DK) * a.p.dv;
  return s == 1 ? a.Smid + bh * st : a.Sst + (static_cast<size_t>(s - 2) * a.p.BH + bh) * st;
}

// out = Sp + Tf S over [DK][dv] (fp32, a fixed-order sum over k), 256 threads
template <int DK>
__device__ void seg_step(const float* Sp, const float* Tf, const float* S, float* out, int dv, int tid) {
  for (int it = tid; it < DK * dv; it += 256) {
    const int i = it / dv, c = it % dv;
    float s = Sp[it];
    for (int k = 0; k < DK; ++k) s += Tf[i * DK + k] * S[k * dv + c];
    out[it] = s;
  }
}

// Each step of the chain: Tf_s and S_s staged in LDS, a thread forming 4 x 4
// blocks of S_{s+1} (d_v <= 128; the sum over k in a fixed order).
template <int DK>
__global__ __launch_bounds__(256) void fast_segchain_kernel(SegFixArgs a) {
  __shared__ __align__(16) float Ts[DK * DK];
  __shared__ __align__(16) float Ss[DK * 128];
  const int64_t bh = blockIdx.x;
  const int dv = a.p.dv, tid = threadIdx.x;
  const size_t st = static_cast<size_t>(DK) * dv, tt = static_cast<size_t>(DK) * DK;
  const int nb = dv / 4;   // 4-column blocks of a row block
  for (int s = 1; s + 1 < a.nseg; ++s) {
    const size_t slot = static_cast<size_t>(s - 1) * a.p.BH + bh;
    const float* S = seg_start<DK>(a, s, bh);
    for (int it = tid; it < DK * DK; it += 256) Ts[it] = a.Tf[slot * tt + it];
    for (int it = tid; it < DK * dv; it += 256) Ss[it] = S[it];
    __syncthreads();
    for (int blk = tid; blk < (DK / 4) * nb; blk += 256) {
      const int i0 = (blk / nb) * 4, cb = (blk % nb) * 4;
      float acc[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = a.Sp[slot * st + (i0 + r) * dv + cb + c];
      for (int k = 0; k < DK; ++k) {
        const f32x4 sv = *reinterpret_cast<const f32x4*>(Ss + k * dv + cb);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float t = Ts[(i0 + r) * DK + k];
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[r][c] += t * sv[c];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) a.Sst[slot * st + (i0 + r) * dv + cb + c] = acc[r][c];
    }
    __syncthreads();   // the next step stages this one's rows (other threads')
  }
}

template <int DK>
__global__ __launch_bounds__(256) void fast_segfix_kernel(SegFixArgs a) {
  const Problem& p = a.p;
  const int dv = p.dv;
  const int64_t N1 = p.N - a.L, NG = (N1 + kSegFixG - 1) / kSegFixG, nf = a.Sfin ? p.BH : 0;
  const int64_t b = static_cast<int64_t>(blockIdx.x) - nf;
  const int tid = threadIdx.x;
  if (b < 0) {
    const int64_t bh = b + nf;
    const int last = a.nseg - 1;
    const size_t slot = static_cast<size_t>(last - 1) * p.BH + bh;
    seg_step<DK>(a.Sp + slot * DK * dv, a.Tf + slot * DK * DK, seg_start<DK>(a, last, bh), a.Sfin + bh * DK * dv,
                 dv, tid);
    return;
  }
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int LDT = DK + 8;   // S_s^T row (bf16): value column c, K = d_k contiguous
  __bf16* St = reinterpret_cast<__bf16*>(smem);
  float* ob = reinterpret_cast<float*>(smem + static_cast<size_t>(dv) * LDT * 2);   // [C][dv + 4]
  const int LDO = dv + 4;
  const int64_t bh = b / NG, g0 = (b % NG) * kSegFixG;
  const int lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int64_t g1 = g0 + kSegFixG < N1 ? g0 + kSegFixG : N1;
  // The next chunk's U rows and output rows are loaded while this chunk's
  // are formed and stored.  A thread's output pieces: items tid + 256 q of
  // the chunk's (token, 8 columns) pieces (d_v <= 128: at most 4).
  constexpr int OQ = kC * 128 / 8 / 256;
  bf16x8 af[DK / 32], ov[OQ];
  auto load = [&](int64_t jl) {
    // A operand: row 16 w + lr of U_j (padding rows hold whatever the scan
    // left there; a product row depends on its own A row only, and is not
    // stored)
    const __bf16* Ur = a.U + ((bh * N1 + jl) * kC + 16 * w + lr) * DK + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) af[ks] = *reinterpret_cast<const bf16x8*>(Ur + 32 * ks);
    const int64_t j = a.L + jl;
    const int n = static_cast<int>(p.T - j * kC < kC ? p.T - j * kC : kC);
    const __bf16* oj = a.out + (bh * p.T + j * kC) * dv;
#pragma unroll
    for (int q = 0; q < OQ; ++q) {
      const int it = tid + 256 * q, t = it / (dv / 8), c8 = (it % (dv / 8)) * 8;
      if (t < n) ov[q] = *reinterpret_cast<const bf16x8*>(oj + t * dv + c8);
    }
  };
  load(g0);
  int cur = 0;   // the segment whose entering state St holds
  for (int64_t jl = g0; jl < g1; ++jl) {
    const int64_t j = a.L + jl;
    const int n = static_cast<int>(p.T - j * kC < kC ? p.T - j * kC : kC);
    const int sg = static_cast<int>(j / a.L);
    if (sg != cur) {
      __syncthreads();   // every wave is done with the previous segment's state
      const float* Ss = seg_start<DK>(a, sg, bh);
      for (int it = tid; it < DK * dv; it += 256) {
        const int i = it / dv, c = it % dv;
        St[c * LDT + i] = (__bf16)Ss[it];
      }
      cur = sg;
    }
    __syncthreads();   // St staged; the previous chunk's rows are out of ob
    for (int ct = 0; ct < dv / 16; ++ct) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
        acc = mfma32(af[ks], lds8(St + (16 * ct + lr) * LDT + 32 * ks + 8 * lg), acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) ob[(16 * w + 4 * lg + e) * LDO + 16 * ct + lr] = acc[e];
    }
    bf16x8 oc[OQ];
#pragma unroll
    for (int q = 0; q < OQ; ++q) oc[q] = ov[q];
    if (jl + 1 < g1) load(jl + 1);
    __syncthreads();
    __bf16* oj = a.out + (bh * p.T + j * kC) * dv;
#pragma unroll
    for (int q = 0; q < OQ; ++q) {
      const int it = tid + 256 * q, t = it / (dv / 8), c8 = (it % (dv / 8)) * 8;
      if (t < n) {
        bf16x8 o = oc[q];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (__bf16)((float)o[e] + ob[t * LDO + c8 + e]);
        *reinterpret_cast<bf16x8*>(oj + t * dv + c8) = o;
      }
    }
  }
}

template <int DK, int BV, int NWV, int PD, int CK = kScanOut>
hipError_t launch_scan(const Problem& p, const void* M, const void* v, void* out, float* Sfin,
                       const float* S0, void* ckpt, hipStream_t s) {
  using Cfg = ScanCfg<DK, BV, NWV, PD>;
  FastScanArgs a{p, static_cast<const __bf16*>(M), static_cast<const __bf16*>(v),
                 static_cast<__bf16*>(out), Sfin, S0, static_cast<__bf16*>(ckpt)};
  const int nvt = p.dv / BV;
  const int64_t groups = (p.BH + 7) / 8;
  const void* fn = reinterpret_cast<const void*>(fast_scan_kernel<DK, BV, NWV, PD, CK>);
  constexpr int lds = CK == kScanStates ? Cfg::LDS_CK : Cfg::LDS;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fast_scan_kernel<DK, BV, NWV, PD, CK>), dim3(groups * 8 * nvt), dim3(Cfg::NT), lds, s, a);
  return hipGetLastError();
}

// Workspace of the split scan after the chunk operators: U, Smid, Sp, Tf, Sst.
struct SegLayout {
  int64_t L;
  int nseg;
  size_t u, smid, sp, tf, sst, total;
};
size_t seg_align(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
SegLayout seg_layout(const Problem& p, int nseg) {
  SegLayout l{};
  l.nseg = nseg;
  // segments of L chunks, L even (the scan's ring of two), the last one shorter
  l.L = ((p.N + nseg - 1) / nseg + 1) & ~static_cast<int64_t>(1);
  const size_t st = static_cast<size_t>(p.BH) * p.dk * p.dv * 4;
  l.u = 0;
  l.smid = seg_align(static_cast<size_t>(p.BH) * (p.N - l.L) * kC * p.dk * 2);
  l.sp = l.smid + seg_align(st);
  l.tf = l.sp + seg_align((nseg - 1) * st);
  l.sst = l.tf + seg_align(static_cast<size_t>(nseg - 1) * p.BH * p.dk * p.dk * 4);
  l.total = l.sst + seg_align((nseg > 2 ? nseg - 2 : 0) * st);
  return l;
}

template <int DK, int BV, int NWV, int PD>
hipError_t launch_scan_seg(const Problem& p, int nseg, const void* M, const void* v, void* out, float* Sfin,
                           const float* S0, char* scratch, hipStream_t s) {
  using Cfg = ScanCfg<DK, BV, NWV, PD>;
  const SegLayout l = seg_layout(p, nseg);
  FastScanArgs a{p, static_cast<const __bf16*>(M), static_cast<const __bf16*>(v), static_cast<__bf16*>(out), Sfin, S0,
                 nullptr};
  a.L = l.L;
  a.nseg = nseg;
  a.U = reinterpret_cast<__bf16*>(scratch + l.u);
  a.Smid = reinterpret_cast<float*>(scratch + l.smid);
  a.Sp = reinterpret_cast<float*>(scratch + l.sp);
  a.Tf = reinterpret_cast<float*>(scratch + l.tf);
  const int nvt = p.dv / BV, R = nvt + (nseg - 1) * (nvt + DK / BV);
  const int64_t groups = (p.BH + 7) / 8;
  const void* fn = reinterpret_cast<const void*>(fast_scan_kernel<DK, BV, NWV, PD, kScanOut, true>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fast_scan_kernel<DK, BV, NWV, PD, kScanOut, true>), dim3(groups * 8 * R), dim3(Cfg::NT),
                     Cfg::LDS, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  SegFixArgs f{p, l.L, nseg, a.U, a.Smid, a.Sp, a.Tf, reinterpret_cast<float*>(scratch + l.sst),
               static_cast<__bf16*>(out), Sfin};
  if (nseg > 2) {
    hipLaunchKernelGGL(fast_segchain_kernel<DK>, dim3(static_cast<unsigned>(p.BH)), dim3(256), 0, s, f);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t blocks = p.BH * ((p.N - l.L + kSegFixG - 1) / kSegFixG) + (Sfin ? p.BH : 0);
  const size_t lds = static_cast<size_t>(p.dv) * (DK + 8) * 2 + static_cast<size_t>(kC) * (p.dv + 4) * 4;
  hipLaunchKernelGGL(fast_segfix_kernel<DK>, dim3(blocks), dim3(256), lds, s, f);
  return hipGetLastError();
}

}  // namespace

bool fast_supported(const Problem& p) {
  return p.bf16 && p.C == kC && p.r_kv == 1 && (p.r_ab >= 0 && p.r_ab <= 2) &&
         (p.dk == 64 || p.dk == 128) && (p.dv % 64 == 0);
}

// The forward scan splits the sequence in segments (fast_scan) where at
// d_k = 64 its 16-column d_v slices leave the chip's 256 compute units short
// of work: the split scan takes 64-column slices (every slice reads the whole
// chunk operator, so wide slices keep that traffic down), and its workgroups,
// one per compute unit, must all be resident (d_v <= 128).  As many segments
// as that allows, up to three, each of at least 32 chunks.
int fast_scan_segments(const Problem& p) {
  constexpr int64_t kCUs = 256;
  if (!fast_supported(p) || p.dk != 64 || p.dv > 128 || p.BH * (p.dv / 16) >= kCUs) return 1;
  const int64_t nvt = p.dv / 64;
  for (int n = 3; n >= 2; --n)
    if (p.BH * (nvt + (n - 1) * (nvt + 1)) <= kCUs && p.N >= 32 * n) return n;
  return 1;
}

size_t fast_forward_bytes(const Problem& p) {
  const size_t ops = fast_workspace_bytes(p);
  const int n = fast_scan_segments(p);
  return n > 1 ? seg_align(ops) + seg_layout(p, n).total : ops;
}

size_t fast_workspace_bytes(const Problem& p) {
  const size_t tiles = static_cast<size_t>((p.dk + kC) / 16) * ((p.dk + kNK) / 16);
  return static_cast<size_t>(p.BH * p.N) * tiles * 512;
}

hipError_t fast_prepare_bw(const Problem& p, const void* q, const void* k, const float* ld, const void* A,
                           const void* B, void* workspace, const PrepBwOut& out, hipStream_t s) {
  if (p.BH * p.N == 0) return hipSuccess;
  if (!fast_supported(p)) return hipErrorInvalidValue;
#define LATTN_PBW(DK_, RAB_)                                                                                      \
  if (p.dk == DK_ && p.r_ab == RAB_)                                                                             \
    return p.scalar ? launch_prep<DK_, RAB_, true, kGenericBw>(p, q, k, ld, A, B, nullptr, workspace, s, &out)   \
                    : launch_prep<DK_, RAB_, false, kGenericBw>(p, q, k, ld, A, B, nullptr, workspace, s, &out);
  LATTN_PBW(128, 2) LATTN_PBW(128, 1) LATTN_PBW(128, 0) LATTN_PBW(64, 2) LATTN_PBW(64, 1) LATTN_PBW(64, 0)
#undef LATTN_PBW
  return hipErrorInvalidValue;
}

hipError_t fast_prepare(const Problem& p, const void* q, const void* k, const float* ld,
                        const void* A, const void* B, void* workspace, hipStream_t s) {
  if (p.BH * p.N == 0) return hipSuccess;
  if (p.dk == 128 && p.r_ab == 2) return launch_prep<128, 2>(p, q, k, ld, A, B, workspace, s);
  if (p.dk == 128 && p.r_ab == 1) return launch_prep<128, 1>(p, q, k, ld, A, B, workspace, s);
  if (p.dk == 64 && p.r_ab == 2) return launch_prep<64, 2>(p, q, k, ld, A, B, workspace, s);
  if (p.dk == 64 && p.r_ab == 1) return launch_prep<64, 1>(p, q, k, ld, A, B, workspace, s);
  if (p.dk == 128 && p.r_ab == 0) return launch_prep<128, 0>(p, q, k, ld, A, B, workspace, s);
  if (p.dk == 64 && p.r_ab == 0) return launch_prep<64, 0>(p, q, k, ld, A, B, workspace, s);
  return hipErrorInvalidValue;
}

hipError_t fast_prepare_fused(const Problem& p, int family, const void* q, const void* k, const float* ld,
                              const float* beta, void* workspace, hipStream_t s) {
  if (p.BH * p.N == 0) return hipSuccess;
  if (family == kHdla && p.r_ab == 2 && !p.scalar) {
    if (p.dk == 128) return launch_prep<128, 2, false, kHdla>(p, q, k, ld, nullptr, nullptr, beta, workspace, s);
    if (p.dk == 64) return launch_prep<64, 2, false, kHdla>(p, q, k, ld, nullptr, nullptr, beta, workspace, s);
  }
  if (family == kGdn && p.r_ab == 1 && p.scalar) {
    if (p.dk == 128) return launch_prep<128, 1, true, kGdn>(p, q, k, ld, nullptr, nullptr, beta, workspace, s);
    if (p.dk == 64) return launch_prep<64, 1, true, kGdn>(p, q, k, ld, nullptr, nullptr, beta, workspace, s);
  }
  return hipErrorInvalidValue;
}

hipError_t fast_scan(const Problem& p, const void* workspace, const void* v, void* out, float* Sfin,
                     const float* S0, hipStream_t s, void* ckpt) {
  if (p.BH == 0) return hipSuccess;
  if (ckpt && !out) {
    // the boundary-state instance: states instead of output rows
    if (p.dk == 128 && p.BH * (p.dv / 64) >= 256)
      return launch_scan<128, 64, 12, 2, kScanStates>(p, workspace, v, nullptr, Sfin, S0, ckpt, s);
    if (p.dk == 128) return launch_scan<128, 32, 4, 2, kScanStates>(p, workspace, v, nullptr, Sfin, S0, ckpt, s);
    if (p.dk == 64) return launch_scan<64, 16, 4, 4, kScanStates>(p, workspace, v, nullptr, Sfin, S0, ckpt, s);
    return hipErrorInvalidValue;
  }
  if (ckpt) {
    // output rows and the boundary states
    if (p.dk == 128 && p.BH * (p.dv / 64) >= 256)
      return launch_scan<128, 64, 12, 2, kScanBoth>(p, workspace, v, out, Sfin, S0, ckpt, s);
    if (p.dk == 128) return launch_scan<128, 32, 4, 2, kScanBoth>(p, workspace, v, out, Sfin, S0, ckpt, s);
    if (p.dk == 64) return launch_scan<64, 16, 4, 4, kScanBoth>(p, workspace, v, out, Sfin, S0, ckpt, s);
    return hipErrorInvalidValue;
  }
  // Split in sequence segments (d_k = 64, few heads): the scratch after the
  // chunk operators, as fast_forward_bytes counts it.
  if (const int nseg = fast_scan_segments(p); nseg > 1)
    return launch_scan_seg<64, 64, 8, 2>(p, nseg, workspace, v, out, Sfin, S0,
                                         static_cast<char*>(const_cast<void*>(workspace)) +
                                             seg_align(fast_workspace_bytes(p)),
                                         s);
  // Wider d_v slices share each operator load among more columns; narrower
  // ones are used when that leaves too few workgroups to fill the chip.
  if (p.dk == 128 && p.BH * (p.dv / 64) >= 256)
    return launch_scan<128, 64, 12, 2>(p, workspace, v, out, Sfin, S0, ckpt, s);
  if (p.dk == 128) return launch_scan<128, 32, 4, 2>(p, workspace, v, out, Sfin, S0, ckpt, s);
  if (p.dk == 64) return launch_scan<64, 16, 4, 4>(p, workspace, v, out, Sfin, S0, ckpt, s);
  return hipErrorInvalidValue;
}

hipError_t fast_gate_summaries(const Problem& p, int G, const void* workspace, const void* v, void* AT, void* BT,
                               float* QB, float* OI, hipStream_t s) {
  if (p.BH * p.N == 0) return hipSuccess;
  if (G < 1 || G > 4 || p.dv % 64 != 0 || p.r_kv != 1) return hipErrorInvalidValue;
  const int64_t NL = (p.N + G - 1) / G;
  FastGateArgs a{p, G, NL, static_cast<const __bf16*>(workspace), static_cast<const __bf16*>(v),
                 static_cast<__bf16*>(AT), static_cast<__bf16*>(BT), QB, OI};
  const int64_t blocks = p.BH * NL * ((p.dk + p.dv) / 64);
  if (p.dk == 128) {
    const void* fn = reinterpret_cast<const void*>(fast_gate_kernel<128>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, GateCfg<128>::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fast_gate_kernel<128>, dim3(blocks), dim3(GateCfg<128>::NT), GateCfg<128>::LDS, s, a);
  } else if (p.dk == 64) {
    hipLaunchKernelGGL(fast_gate_kernel<64>, dim3(blocks), dim3(GateCfg<64>::NT), GateCfg<64>::LDS, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lattn
