// bf16 MFMA path (gfx950) for chunk C = 64, write rank r_kv = 1, decay rank
// r_ab in {1, 2}, d_k in {64, 128}: the Gated DeltaNet and HDLA shapes.
//
// It computes the same chunk operator as the general path (HDLA note, "Key
// design 3": rank-generalized WY form; HLA note, "Affine maps and closure
// under composition"):
//   M_j = [[Acal, Z], [Qbar, R]],   [S_j ; O_j] = M_j [S_{j-1} ; V_j]
// with bf16 MFMA operands and fp32 accumulation; the triangular solve applies
// its 16x16 diagonal inverses in fp32.
//
// prepare kernel: one workgroup per (batch*head, chunk), NW = (d_k + 64) / 32
// waves.  Wave w owns two 16-column tiles of the chunk operator's input side
// (the d_k "W" columns, then the 64 "X" columns); the solve and the final
// product run per wave on its own columns with no barrier.  The operator is
// stored transposed-by-construction: each 16x16 tile is written as the A-operand
// fragment of a 16x16x16 MFMA (64 lanes x 4 bf16 = 512 bytes, lane order),
// which is exactly how the scan kernel reads it.
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

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
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
// Four values of one column, rows r, r+ld, r+2ld, r+3ld.
__device__ __forceinline__ bf16x4 lds_col4(const __bf16* p, int ld) {
  bf16x4 r;
  r[0] = p[0]; r[1] = p[ld]; r[2] = p[2 * ld]; r[3] = p[3 * ld];
  return r;
}

// ---------------------------------------------------------------------------
// Prepare kernel.
template <int DK, int RAB>
struct PrepCfg {
  static constexpr int NA = kC * RAB;            // decay rows of a chunk
  static constexpr int NB = NA / 16;             // 16-row blocks of the solve
  static constexpr int KIN = DK + kNK;           // operator input width
  static constexpr int ROUT = DK + kC;           // operator output height
  static constexpr int KT = KIN / 16;
  static constexpr int MT = ROUT / 16;
  static constexpr int NW = KIN / 32;            // two input tiles per wave
  static constexpr int NT = 64 * NW;
  static constexpr int WW = DK / 32;             // waves owning W columns
  static constexpr int LD = DK + 8;              // padded row of Xl / Xr (bf16)
  static constexpr int LDA = NA + 8;             // padded row of At^T and M_A (bf16)
  // LDS regions (bytes)
  static constexpr int XL_ROWS = NA + kC;
  static constexpr int XR_ROWS = NA + kNK;
  // A~^T overwrites the B~ rows of Xl once those are dead; when it does not fit
  // there it gets a region of its own (R5), so the Q~ rows stay readable.
  static constexpr bool AT_OVER_B = DK * LDA <= NA * LD;
  static constexpr int R1 = XL_ROWS * LD * 2;
  static constexpr int R2 = XR_ROWS * LD * 2;
  static constexpr int LDIAG = NB * 256 * 4;
  static constexpr int LPACK = (NB * (NB - 1) / 2) * 256 * 2;
  static constexpr int MA = kC * LDA * 2;
  static constexpr int R3_OUT = LDIAG + LPACK + MA;
  static constexpr int R3_G = kC * DK * 4;
  static constexpr int R3 = R3_OUT > R3_G ? R3_OUT : R3_G;
  static constexpr int R4 = DK * 4;
  static constexpr int R5 = AT_OVER_B ? 0 : DK * LDA * 2;
  static constexpr int LDS = R1 + R2 + R3 + R4 + R5;
};

struct FastPrepArgs {
  Problem p;
  const __bf16* q;
  const __bf16* k;
  const float* ld;
  const __bf16* A;
  const __bf16* B;
  __bf16* M;   // fragment-ordered chunk operators
};

template <int DK, int RAB>
__global__ __launch_bounds__((PrepCfg<DK, RAB>::NT)) void fast_prepare_kernel(FastPrepArgs a) {
  using Cfg = PrepCfg<DK, RAB>;
  constexpr int NA = Cfg::NA, NB = Cfg::NB, LD = Cfg::LD, LDA = Cfg::LDA, NW = Cfg::NW;
  constexpr int MT = Cfg::MT, KT = Cfg::KT, WW = Cfg::WW;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* Xl = reinterpret_cast<__bf16*>(smem);                      // [B~ ; Q~]   rows x LD
  __bf16* AT = Cfg::AT_OVER_B ? Xl                                   // A~^T        DK x LDA (after GEMM1)
                              : reinterpret_cast<__bf16*>(smem + Cfg::R1 + Cfg::R2 + Cfg::R3 + Cfg::R4);
  __bf16* Xr = reinterpret_cast<__bf16*>(smem + Cfg::R1);            // [A~ ; K~]   rows x LD
  float* G = reinterpret_cast<float*>(smem + Cfg::R1 + Cfg::R2);     // C x DK (or C) cumulative log-decay
  float* Ldg = G;                                                    // NB x 16 x 16 fp32 diagonal blocks
  __bf16* Lpk = reinterpret_cast<__bf16*>(smem + Cfg::R1 + Cfg::R2 + Cfg::LDIAG);  // -L blocks below the diagonal
  __bf16* MAs = reinterpret_cast<__bf16*>(smem + Cfg::R1 + Cfg::R2 + Cfg::LDIAG + Cfg::LPACK);  // M_A  C x LDA
  float* eGC = reinterpret_cast<float*>(smem + Cfg::R1 + Cfg::R2 + Cfg::R3);                   // exp(G_C) per channel

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t job = blockIdx.x;
  const int64_t bh = job / p.N;
  const int64_t j = job % p.N;
  const int64_t t0 = j * kC;
  const int n = static_cast<int>(p.T - t0 < kC ? p.T - t0 : kC);
  const int64_t tok0 = bh * p.T + t0;
  const bool scalar = p.scalar != 0;

  // ---- P0: chunk-local inclusive cumulative log-decay (padded tokens add 0).
  if (!scalar) {
    for (int i = tid; i < DK; i += Cfg::NT) {
      float g = 0.f;
#pragma unroll 8
      for (int t = 0; t < kC; ++t) {
        const float l = t < n ? a.ld[(tok0 + t) * DK + i] : 0.f;
        g += l;
        G[t * DK + i] = g;
      }
      eGC[i] = __expf(g);
    }
  } else if (wave == 0) {
    float g = lane < n ? a.ld[tok0 + lane] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(g, off, 64);
      if (lane >= off) g += o;
    }
    G[lane] = g;
    const float gc = __shfl(g, 63, 64);
    for (int i = lane; i < DK; i += 64) eGC[i] = __expf(gc);
  }
  __syncthreads();

  // ---- P1: decay-scaled bf16 operands.  Xl = [B~ ; Q~], Xr = [A~ ; K~].
  {
    constexpr int CG = DK / 8;
    constexpr int ITEMS = (Cfg::XL_ROWS + Cfg::XR_ROWS) * CG;
    for (int it = tid; it < ITEMS; it += Cfg::NT) {
      const int row = it / CG, cg = it % CG;
      const __bf16* src;
      int t, gt, sign;        // token, cumulative-decay row to use (-1: none), exponent sign
      __bf16* dst;
      if (row < NA) {                         // B~ = B (.) exp(G_{t-1})
        t = row / RAB;
        src = a.B + ((tok0 + t) * RAB + (row % RAB)) * DK;
        gt = t - 1; sign = 1; dst = Xl + row * LD;
      } else if (row < NA + kC) {             // Q~ = q (.) exp(G_t)
        t = row - NA;
        src = a.q + (tok0 + t) * DK;
        gt = t; sign = 1; dst = Xl + row * LD;
      } else if (row < 2 * NA + kC) {         // A~ = A (.) exp(-G_t)
        const int r = row - NA - kC;
        t = r / RAB;
        src = a.A + ((tok0 + t) * RAB + (r % RAB)) * DK;
        gt = t; sign = -1; dst = Xr + r * LD;
      } else {                                // K~ = K (.) exp(-G_t)
        const int r = row - 2 * NA - kC;
        t = r;
        src = a.k + (tok0 + t) * DK;
        gt = t; sign = -1; dst = Xr + (NA + r) * LD;
      }
      bf16x8 out;
      if (t < n) {
        const bf16x8 raw = *reinterpret_cast<const bf16x8*>(src + cg * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float g = 0.f;
          if (gt >= 0) g = scalar ? G[gt] : G[gt * DK + cg * 8 + e];
          out[e] = (__bf16)((float)raw[e] * __expf(sign > 0 ? g : -g));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = (__bf16)0.f;
      }
      *reinterpret_cast<bf16x8*>(dst + cg * 8) = out;
    }
  }
  __syncthreads();

  const bool wrole = wave < WW;          // owns W columns (channels) or X columns (chunk write rows)
  const int kt0 = 2 * wave;              // first of the wave's two input tiles

  // ---- P2: Gram blocks.  (a) P^T = A~ [B~ ; Q~]^T, tiles (rs, cs), cs >= rs,
  //      split over all waves and written straight to LDS region 3.
  {
    constexpr int CS = NB + kC / 16;
    for (int tile = wave; tile < NB * CS; tile += NW) {
      const int rs = tile / CS, cs = tile % CS;
      if (cs < rs) continue;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const bf16x8 av = lds8(Xr + (rs * 16 + lr) * LD + kb * 32 + 8 * lg);
        const bf16x8 bv = lds8(Xl + (cs * 16 + lr) * LD + kb * 32 + 8 * lg);
        acc = mfma32(av, bv, acc);
      }
      // lane holds P^T[s = rs*16 + 4lg + e][col = cs*16 + lr]
      if (cs < NB) {
        const int sp = cs * 16 + lr;           // row of L (B~ index)
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = rs * 16 + 4 * lg + e;  // column of L (A~ index)
          v[e] = (sp / RAB > s / RAB) ? acc[e] : 0.f;
        }
        if (cs == rs) {
          *reinterpret_cast<f32x4*>(Ldg + cs * 256 + lr * 16 + 4 * lg) = v;
        } else {
          const int blk = cs * (cs - 1) / 2 + rs;
          f32x4 nv = f32x4{-v[0], -v[1], -v[2], -v[3]};
          *reinterpret_cast<bf16x4*>(Lpk + blk * 256 + lr * 16 + 4 * lg) = to_bf16x4(nv);
        }
      } else {
        const int t = (cs - NB) * 16 + lr;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = rs * 16 + 4 * lg + e;
          v[e] = (t >= s / RAB) ? acc[e] : 0.f;
        }
        *reinterpret_cast<bf16x4*>(MAs + t * LDA + rs * 16 + 4 * lg) = to_bf16x4(v);
      }
    }
  }
  __syncthreads();

  // ---- P3: fp32 inverses of the unit lower-triangular diagonal blocks
  //      (I + L_ii), in place.
  {
    float x[16];
    const bool active = tid < NB * 16;
    const int blk = tid / 16, c = tid % 16;
    if (active) {
      const float* Lb = Ldg + blk * 256;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = (r == c) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) v -= Lb[r * 16 + m] * x[m];
        x[r] = v;
      }
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Ldg[blk * 256 + r * 16 + c] = x[r];
    }
  }
  __syncthreads();

  // ---- P4: blocked forward substitution on this wave's columns:
  //      WX_i = (I + L_ii)^{-1} (RHS_i - sum_{j<i} L_ij WX_j).
  bf16x4 wx[NB][2];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    f32x4 acc[2];
    if (wrole) {
      // W columns: B~ itself (4 rows of one channel column per lane).
#pragma unroll
      for (int u = 0; u < 2; ++u)
        acc[u] = to_f32x4(lds_col4(Xl + (i * 16 + 4 * lg) * LD + (kt0 + u) * 16 + lr, LD));
    } else {
      // X columns: L_K = B~ K~^T on this block of rows, token(row) > chunk-write row.
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int x = kt0 + u - DK / 16;
        f32x4 g = zero4();
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          const bf16x8 av = lds8(Xl + (i * 16 + lr) * LD + kb * 32 + 8 * lg);
          const bf16x8 bv = lds8(Xr + (NA + x * 16 + lr) * LD + kb * 32 + 8 * lg);
          g = mfma32(av, bv, g);
        }
        const int sx = x * 16 + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sp = i * 16 + 4 * lg + e;
          if (!(sp / RAB > sx)) g[e] = 0.f;
        }
        acc[u] = g;
      }
    }
    const __bf16* Lrow = Lpk + (i * (i - 1) / 2) * 256 + lr * 16 + 4 * lg;
#pragma unroll
    for (int jb = 0; jb + 1 < i; jb += 2) {
      const bf16x8 av = cat(lds4(Lrow + jb * 256), lds4(Lrow + (jb + 1) * 256));
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[u] = mfma32(av, cat(wx[jb][u], wx[jb + 1][u]), acc[u]);
    }
    if (i % 2 == 1) {
      const bf16x4 av = lds4(Lrow + (i - 1) * 256);
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[u] = mfma16(av, wx[i - 1][u], acc[u]);
    }
    const float* Dv = Ldg + i * 256 + lr * 16 + 4 * lg;
    float dv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) dv[e] = Dv[e];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 o = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) o = mfma_f32(dv[e], acc[u][e], o);
      wx[i][u] = to_bf16x4(o);
    }
  }

  // ---- A~^T (B~ rows of Xl are dead once every wave has finished its solve).
  __syncthreads();
  for (int it = tid; it < DK * (NA / 4); it += Cfg::NT) {
    const int i = it % DK, s4 = it / DK;
    const bf16x4 v = lds_col4(Xr + (s4 * 4) * LD + i, LD);
    *reinterpret_cast<bf16x4*>(AT + i * LDA + s4 * 4) = v;
  }
  __syncthreads();

  // ---- P5: operator tiles, transposed product: rows = this wave's input
  //      columns, columns = output rows m (channels, then tokens):
  //      acc = sum_s WX[s][k] Bmat[m][s],  Bmat = [A~^T ; M_A].
  __bf16* Mout = a.M + static_cast<size_t>(job) * (MT * KT * 256);
  // Output rows that are channels (Acal, Z): base I or K~^T, scaled by exp(G_C).
#pragma unroll 1
  for (int mt = 0; mt < DK / 16; ++mt) {
    const __bf16* Brow = AT + (mt * 16 + lr) * LDA;
    f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
    for (int jb = 0; jb < NB; jb += 2) {
      const bf16x8 bv = cat(lds4(Brow + jb * 16 + 4 * lg), lds4(Brow + (jb + 1) * 16 + 4 * lg));
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[u] = mfma32(cat(wx[jb][u], wx[jb + 1][u]), bv, acc[u]);
    }
    const int m = mt * 16 + lr;
    const float sc = eGC[m];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kt = kt0 + u;
      f32x4 base;
      if (wrole) {
#pragma unroll
        for (int e = 0; e < 4; ++e) base[e] = (kt * 16 + 4 * lg + e == m) ? 1.f : 0.f;
      } else {
        base = to_f32x4(lds_col4(Xr + (NA + kt * 16 - DK + 4 * lg) * LD + m, LD));
      }
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = sc * (base[e] - acc[u][e]);
      *reinterpret_cast<bf16x4*>(Mout + (mt * KT + kt) * 256 + lane * 4) = to_bf16x4(v);
    }
  }
  // Output rows that are tokens (Qbar, R): base Q~ or M_K.
#pragma unroll
  for (int tt = 0; tt < kC / 16; ++tt) {
    const int mt = DK / 16 + tt;
    const __bf16* Brow = MAs + (tt * 16 + lr) * LDA;
    f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
    for (int jb = 0; jb < NB; jb += 2) {
      const bf16x8 bv = cat(lds4(Brow + jb * 16 + 4 * lg), lds4(Brow + (jb + 1) * 16 + 4 * lg));
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[u] = mfma32(cat(wx[jb][u], wx[jb + 1][u]), bv, acc[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kt = kt0 + u;
      f32x4 base;
      if (wrole) {
        base = to_f32x4(lds4(Xl + (NA + tt * 16 + lr) * LD + kt * 16 + 4 * lg));
      } else {
        // M_K^T = K~ Q~^T on (chunk-write rows of this tile) x (tokens of tt), t >= s.
        const int x = kt - DK / 16;
        f32x4 g = zero4();
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          const bf16x8 av = lds8(Xr + (NA + x * 16 + lr) * LD + kb * 32 + 8 * lg);
          const bf16x8 bv = lds8(Xl + (NA + tt * 16 + lr) * LD + kb * 32 + 8 * lg);
          g = mfma32(av, bv, g);
        }
        const int t = tt * 16 + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sx = x * 16 + 4 * lg + e;
          if (!(t >= sx)) g[e] = 0.f;
        }
        base = g;
      }
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = base[e] - acc[u][e];
      *reinterpret_cast<bf16x4*>(Mout + (mt * KT + kt) * 256 + lane * 4) = to_bf16x4(v);
    }
  }
}

// ---------------------------------------------------------------------------
// Scan kernel: per (batch*head, BV-wide d_v slice), chunks in order,
// Y = M_j [S ; V_j] with the operator fragments read straight from HBM.
template <int DK, int BV>
struct ScanCfg {
  static constexpr int KIN = DK + kNK;
  static constexpr int ROUT = DK + kC;
  static constexpr int KT = KIN / 16;
  static constexpr int MT = ROUT / 16;
  static constexpr int NWV = 4;
  static constexpr int MPW = MT / NWV;     // output tiles (rows) per wave
  static constexpr int NTN = BV / 16;      // output tiles (columns)
  static constexpr int LDX = KIN + 8;      // padded row of X^T (bf16)
  static constexpr int LDS = BV * LDX * 2;
};

struct FastScanArgs {
  Problem p;
  const __bf16* M;
  const __bf16* v;
  __bf16* out;
  float* Sfin;
  const float* S0;
};

template <int DK, int BV>
__global__ __launch_bounds__(256) void fast_scan_kernel(FastScanArgs a) {
  using Cfg = ScanCfg<DK, BV>;
  constexpr int KT = Cfg::KT, MT = Cfg::MT, MPW = Cfg::MPW, NTN = Cfg::NTN, LDX = Cfg::LDX;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* Xt = reinterpret_cast<__bf16*>(smem);   // [BV][KIN]: columns 0..DK state^T, DK.. V_j^T
  const Problem& p = a.p;
  const int dv = p.dv;
  const int nvt = dv / BV;
  // Blocks of one (batch, head) land on one XCD (dispatch is round-robin over 8).
  const int b = blockIdx.x;
  const int grp = b / (8 * nvt), rem = b % (8 * nvt);
  const int vt = rem / 8;
  const int64_t bh = static_cast<int64_t>(grp) * 8 + rem % 8;
  if (bh >= p.BH) return;
  const int c0 = vt * BV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  for (int it = tid; it < DK * BV; it += 256) {
    const int i = it / BV, c = it % BV;
    const float s = a.S0 ? a.S0[(bh * DK + i) * dv + c0 + c] : 0.f;
    Xt[c * LDX + i] = (__bf16)s;
  }

  const __bf16* Mbh = a.M + static_cast<size_t>(bh) * p.N * (MT * KT * 256);
  bf16x4 mf[MPW][KT];
  auto load_m = [&](int64_t jj) {
    const __bf16* Mj = Mbh + static_cast<size_t>(jj) * (MT * KT * 256);
#pragma unroll
    for (int q = 0; q < MPW; ++q)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        mf[q][kt] = *reinterpret_cast<const bf16x4*>(Mj + ((wave * MPW + q) * KT + kt) * 256 + lane * 4);
  };
  if (p.N > 0) load_m(0);

  for (int64_t j = 0; j < p.N; ++j) {
    const int64_t t0 = j * kC;
    const int n = static_cast<int>(p.T - t0 < kC ? p.T - t0 : kC);
    const int64_t tok0 = bh * p.T + t0;
    // V_j^T into columns DK.. of X^T.
    for (int it = tid; it < kNK * (BV / 8); it += 256) {
      const int s = it / (BV / 8), cg = it % (BV / 8);
      bf16x8 raw;
      if (s < n) {
        raw = *reinterpret_cast<const bf16x8*>(a.v + (tok0 + s) * dv + c0 + cg * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) raw[e] = (__bf16)0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) Xt[(cg * 8 + e) * LDX + DK + s] = raw[e];
    }
    __syncthreads();
    f32x4 acc[MPW][NTN];
#pragma unroll
    for (int q = 0; q < MPW; ++q)
#pragma unroll
      for (int nt = 0; nt < NTN; ++nt) acc[q][nt] = zero4();
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int nt = 0; nt < NTN; ++nt) {
        const bf16x4 bv = lds4(Xt + (nt * 16 + lr) * LDX + kt * 16 + 4 * lg);
#pragma unroll
        for (int q = 0; q < MPW; ++q) acc[q][nt] = mfma16(mf[q][kt], bv, acc[q][nt]);
      }
    }
    if (j + 1 < p.N) load_m(j + 1);
    __syncthreads();
    const bool last = (j + 1 == p.N);
#pragma unroll
    for (int q = 0; q < MPW; ++q) {
      const int mt = wave * MPW + q;
#pragma unroll
      for (int nt = 0; nt < NTN; ++nt) {
        const int c = nt * 16 + lr;
        if (mt < DK / 16) {
          const int i0 = mt * 16 + 4 * lg;
          *reinterpret_cast<bf16x4*>(Xt + c * LDX + i0) = to_bf16x4(acc[q][nt]);
          if (last && a.Sfin) {
#pragma unroll
            for (int e = 0; e < 4; ++e) a.Sfin[(bh * DK + i0 + e) * dv + c0 + c] = acc[q][nt][e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = (mt - DK / 16) * 16 + 4 * lg + e;
            if (t < n) a.out[(tok0 + t) * dv + c0 + c] = (__bf16)acc[q][nt][e];
          }
        }
      }
    }
  }
}

template <int DK, int RAB>
hipError_t launch_prep(const Problem& p, const void* q, const void* k, const float* ld,
                       const void* A, const void* B, void* M, hipStream_t s) {
  using Cfg = PrepCfg<DK, RAB>;
  FastPrepArgs a{p, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), ld,
                 static_cast<const __bf16*>(A), static_cast<const __bf16*>(B), static_cast<__bf16*>(M)};
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fast_prepare_kernel<DK, RAB>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fast_prepare_kernel<DK, RAB>), dim3(p.BH * p.N), dim3(Cfg::NT), Cfg::LDS, s, a);
  return hipGetLastError();
}

template <int DK, int BV>
hipError_t launch_scan(const Problem& p, const void* M, const void* v, void* out, float* Sfin,
                       const float* S0, hipStream_t s) {
  using Cfg = ScanCfg<DK, BV>;
  FastScanArgs a{p, static_cast<const __bf16*>(M), static_cast<const __bf16*>(v),
                 static_cast<__bf16*>(out), Sfin, S0};
  const int nvt = p.dv / BV;
  const int64_t groups = (p.BH + 7) / 8;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fast_scan_kernel<DK, BV>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fast_scan_kernel<DK, BV>), dim3(groups * 8 * nvt), dim3(256), Cfg::LDS, s, a);
  return hipGetLastError();
}

}  // namespace

bool fast_supported(const Problem& p) {
  return p.bf16 && p.C == kC && p.r_kv == 1 && (p.r_ab == 1 || p.r_ab == 2) &&
         (p.dk == 64 || p.dk == 128) && (p.dv % 64 == 0);
}

size_t fast_workspace_bytes(const Problem& p) {
  const size_t tiles = static_cast<size_t>((p.dk + kC) / 16) * ((p.dk + kNK) / 16);
  return static_cast<size_t>(p.BH * p.N) * tiles * 512;
}

hipError_t fast_prepare(const Problem& p, const void* q, const void* k, const float* ld,
                        const void* A, const void* B, void* workspace, hipStream_t s) {
  if (p.BH * p.N == 0) return hipSuccess;
  if (p.dk == 128 && p.r_ab == 2) return launch_prep<128, 2>(p, q, k, ld, A, B, workspace, s);
  if (p.dk == 128 && p.r_ab == 1) return launch_prep<128, 1>(p, q, k, ld, A, B, workspace, s);
  if (p.dk == 64 && p.r_ab == 2) return launch_prep<64, 2>(p, q, k, ld, A, B, workspace, s);
  if (p.dk == 64 && p.r_ab == 1) return launch_prep<64, 1>(p, q, k, ld, A, B, workspace, s);
  return hipErrorInvalidValue;
}

hipError_t fast_scan(const Problem& p, const void* workspace, const void* v, void* out, float* Sfin,
                     const float* S0, hipStream_t s) {
  if (p.BH == 0) return hipSuccess;
  if (p.dk == 128) return launch_scan<128, 64>(p, workspace, v, out, Sfin, S0, s);
  if (p.dk == 64) return launch_scan<64, 16>(p, workspace, v, out, Sfin, S0, s);
  return hipErrorInvalidValue;
}

}  // namespace lattn
