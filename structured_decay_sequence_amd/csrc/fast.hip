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
// prepare kernel: one workgroup per (batch*head, chunk), one wave per
// 16-column tile of the chunk operator's input side (the d_k "W" columns,
// then the 64 "X" columns); the solve and the final product run per wave on
// its own columns with no barrier.  The operator is stored in MFMA operand
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
  static constexpr int NW = KT;                  // one wave per 16-column input tile
  static constexpr int NT = 64 * NW;
  static constexpr int TPW = 1;
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
  constexpr int NA = Cfg::NA, NB = Cfg::NB, LD = Cfg::LD, LDA = Cfg::LDA, NW = Cfg::NW, NT = Cfg::NT;
  constexpr int MT = Cfg::MT, KT = Cfg::KT, TPW = Cfg::TPW;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* Xl = reinterpret_cast<__bf16*>(smem);                      // [B~ ; Q~]   rows x LD
  __bf16* Xr = reinterpret_cast<__bf16*>(smem + Cfg::R1);            // [A~ ; K~]   rows x LD
  float* G = reinterpret_cast<float*>(smem + Cfg::R1 + Cfg::R2);     // C x DK (or C) cumulative log-decay
  float* Ldg = G;                                                    // NB x 16 x 16 fp32 diagonal blocks
  __bf16* Lpk = reinterpret_cast<__bf16*>(smem + Cfg::R1 + Cfg::R2 + Cfg::LDIAG);  // -L blocks below the diagonal
  __bf16* MAs = reinterpret_cast<__bf16*>(smem + Cfg::R1 + Cfg::R2 + Cfg::LDIAG + Cfg::LPACK);  // M_A  C x LDA
  float* eGC = reinterpret_cast<float*>(smem + Cfg::R1 + Cfg::R2 + Cfg::R3);                   // exp(G_C) per channel
  __bf16* AT = Cfg::AT_OVER_B ? Xl                                   // A~^T        DK x LDA (after the solve)
                              : reinterpret_cast<__bf16*>(smem + Cfg::R1 + Cfg::R2 + Cfg::R3 + Cfg::R4);

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const bool scalar = p.scalar != 0;
  const int64_t total = p.BH * p.N;

  // Raw inputs are staged in registers: q, K and the log-decay one chunk ahead
  // (prefetch), the decay operands A, B at the top of each chunk (fetch_ab).
  constexpr int CG = DK / 8;                                       // 8-channel groups per row
  constexpr int QK_ITEMS = (kC + kNK) * CG;                        // q rows, then K rows
  constexpr int QK_IT = (QK_ITEMS + NT - 1) / NT;
  constexpr int AB_ITEMS = 2 * NA * CG;                            // B rows, then A rows
  constexpr int AB_IT = (AB_ITEMS + NT - 1) / NT;
  constexpr int LITEMS = kC * DK / 4;                              // log-decay float4s (per channel)
  constexpr int LIT = (LITEMS + NT - 1) / NT;
  bf16x8 qkbuf[QK_IT];
  bf16x8 abbuf[AB_IT];
  f32x4 lbuf[LIT];
  float lscal = 0.f;

  auto chunk_n = [&](int64_t jb, int64_t& tok0) {
    const int64_t bh = jb / p.N, jc = jb % p.N;
    const int64_t t0 = jc * kC;
    tok0 = bh * p.T + t0;
    return static_cast<int>(p.T - t0 < kC ? p.T - t0 : kC);
  };
  // Loads are unconditional (an invalid item reads the chunk's first row, which
  // always exists) so that no branch waits on them; the consumer zeroes the
  // items of padded tokens.
  auto prefetch = [&](int64_t jb) {
    int64_t tok0;
    const int n = chunk_n(jb, tok0);
#pragma unroll
    for (int q = 0; q < QK_IT; ++q) {
      const int it = tid + q * NT;
      const int row = it / CG, cg = it % CG;
      const int t = row < kC ? row : row - kC;
      const bool ok = it < QK_ITEMS && t < n;
      const __bf16* src = (row < kC ? a.q : a.k) + (tok0 + (ok ? t : 0)) * DK + (ok ? cg : 0) * 8;
      qkbuf[q] = *reinterpret_cast<const bf16x8*>(src);
    }
    if (!scalar) {
#pragma unroll
      for (int q = 0; q < LIT; ++q) {
        const int e4 = tid + q * NT;
        const bool ok = e4 < LITEMS && (e4 * 4) / DK < n;
        lbuf[q] = *reinterpret_cast<const f32x4*>(a.ld + tok0 * DK + (ok ? e4 * 4 : 0));
      }
    } else {
      lscal = a.ld[tok0 + (tid < n ? tid : 0)];
    }
  };
  auto fetch_ab = [&](int64_t jb) {
    int64_t tok0;
    const int n = chunk_n(jb, tok0);
#pragma unroll
    for (int q = 0; q < AB_IT; ++q) {
      const int it = tid + q * NT;
      const int row = it / CG, cg = it % CG;
      const int r = row < NA ? row : row - NA;
      const int t = r / RAB;
      const bool ok = it < AB_ITEMS && t < n;
      const __bf16* src = (row < NA ? a.B : a.A) +
                          ((tok0 + (ok ? t : 0)) * RAB + (ok ? r % RAB : 0)) * DK + (ok ? cg : 0) * 8;
      abbuf[q] = *reinterpret_cast<const bf16x8*>(src);
    }
  };

  // One workgroup per chunk: every load of the chunk is issued up front.
  const int64_t job = blockIdx.x;
  if (job >= total) return;
  prefetch(job);
  {
  int64_t tok0_cur;
  const int ncur = chunk_n(job, tok0_cur);   // tokens of this chunk (the rest are padding)
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  // Wave w owns input tiles kt0 .. kt0 + ntw - 1; a tile below DK/16 is a "W"
  // tile (channel columns), the others are "X" tiles (chunk-write rows).
  const int ntw = TPW;
  const int kt0 = TPW * wave;
  fetch_ab(job);
  // ---- P0: chunk-local inclusive cumulative log-decay (padded tokens add 0).
  if (!scalar) {
#pragma unroll
    for (int q = 0; q < LIT; ++q) {
      const int e4 = tid + q * NT;
      if (e4 < LITEMS) *reinterpret_cast<f32x4*>(G + e4 * 4) = (e4 * 4) / DK < ncur ? lbuf[q] : zero4();
    }
    lds_barrier();
    for (int i = tid; i < DK; i += NT) {
      float g = 0.f;
#pragma unroll
      for (int t0 = 0; t0 < kC; t0 += 16) {
        float v[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) v[t] = G[(t0 + t) * DK + i];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          g += v[t];
          G[(t0 + t) * DK + i] = g;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      eGC[i] = __expf(g);
    }
  } else {
    if (wave == 0) {
      float g = lane < ncur ? lscal : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(g, off, 64);
        if (lane >= off) g += o;
      }
      G[lane] = g;
      const float gc = __shfl(g, 63, 64);
      for (int i = lane; i < DK; i += 64) eGC[i] = __expf(gc);
    }
  }
  lds_barrier();

  // ---- P1: decay-scaled bf16 operands.  Xl = [B~ ; Q~], Xr = [A~ ; K~].
  //      B~ = B (.) exp(G_{t-1}), Q~ = q (.) exp(G_t), A~ = A (.) exp(-G_t), K~ = K (.) exp(-G_t).
  auto scale_store = [&](const bf16x8& raw, int gt, float sign, int cg, __bf16* dst, bool valid) {
    float g[8];
    if (gt < 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = 0.f;
    } else if (scalar) {
      const float gs = G[gt];
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = gs;
    } else {
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(G + gt * DK + cg * 8);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(G + gt * DK + cg * 8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g[e] = g0[e];
        g[e + 4] = g1[e];
      }
    }
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)(valid ? (float)raw[e] * __expf(sign * g[e]) : 0.f);
    *reinterpret_cast<bf16x8*>(dst + cg * 8) = out;
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int q = 0; q < QK_IT; ++q) {
    const int it = tid + q * NT;
    if (it < QK_ITEMS) {
      const int row = it / CG, cg = it % CG;
      if (row < kC) scale_store(qkbuf[q], row, 1.f, cg, Xl + (NA + row) * LD, row < ncur);
      else scale_store(qkbuf[q], row - kC, -1.f, cg, Xr + (NA + row - kC) * LD, row - kC < ncur);
    }
  }
#pragma unroll
  for (int q = 0; q < AB_IT; ++q) {
    const int it = tid + q * NT;
    if (it < AB_ITEMS) {
      const int row = it / CG, cg = it % CG;
      if (row < NA) scale_store(abbuf[q], row / RAB - 1, 1.f, cg, Xl + row * LD, row / RAB < ncur);
      else scale_store(abbuf[q], (row - NA) / RAB, -1.f, cg, Xr + (row - NA) * LD, (row - NA) / RAB < ncur);
    }
  }
  lds_barrier();

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
  lds_barrier();

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
        __builtin_amdgcn_sched_barrier(0);  // one row of loads in flight at a time
      }
    }
    lds_barrier();
    if (active) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Ldg[blk * 256 + r * 16 + c] = x[r];
    }
  }
  lds_barrier();

  // ---- P4: blocked forward substitution on this wave's columns:
  //      WX_i = (I + L_ii)^{-1} (RHS_i - sum_{j<i} L_ij WX_j).
  bf16x4 wx[NB][TPW];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    f32x4 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int kt = kt0 + u;
      if (u >= ntw) {
        acc[u] = zero4();
      } else if (kt < DK / 16) {
        // W columns: B~ itself (4 rows of one channel column per lane).
        acc[u] = to_f32x4(lds_col4(Xl + (i * 16 + 4 * lg) * LD + kt * 16 + lr, LD));
      } else {
        // X columns: L_K = B~ K~^T on this block of rows, token(row) > chunk-write row.
        const int x = kt - DK / 16;
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
      for (int u = 0; u < TPW; ++u) acc[u] = mfma32(av, cat(wx[jb][u], wx[jb + 1][u]), acc[u]);
    }
    if (i % 2 == 1) {
      // Odd leftover block: padded to a 16x16x32 product with a zero half.  The
      // K=16 instruction is kept out of this chain: interleaved with the K=32
      // products it gave run-to-run differences in the last blocks.
      bf16x4 zb;
      zb[0] = zb[1] = zb[2] = zb[3] = (__bf16)0.f;
      const bf16x8 av = cat(lds4(Lrow + (i - 1) * 256), zb);
#pragma unroll
      for (int u = 0; u < TPW; ++u) acc[u] = mfma32(av, cat(wx[i - 1][u], zb), acc[u]);
    }
    const float* Dv = Ldg + i * 256 + lr * 16 + 4 * lg;
    float dv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) dv[e] = Dv[e];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      f32x4 o = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) o = mfma_f32(dv[e], acc[u][e], o);
      wx[i][u] = to_bf16x4(o);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- A~^T (B~ rows of Xl are dead once every wave has finished its solve).
  lds_barrier();
  for (int it = tid; it < DK * (NA / 4); it += Cfg::NT) {
    const int i = it % DK, s4 = it / DK;
    const bf16x4 v = lds_col4(Xr + (s4 * 4) * LD + i, LD);
    *reinterpret_cast<bf16x4*>(AT + i * LDA + s4 * 4) = v;
  }
  lds_barrier();

  // ---- P5: operator tiles, transposed product: rows = this wave's input
  //      columns, columns = output rows m (channels, then tokens):
  //      acc = sum_s WX[s][k] Bmat[m][s],  Bmat = [A~^T ; M_A].
  __bf16* Mout = a.M + static_cast<size_t>(job) * (MT * KT * 256);
  // Output rows that are channels (Acal, Z): base I or K~^T, scaled by exp(G_C).
#pragma unroll 1
  for (int mt = 0; mt < DK / 16; ++mt) {
    const __bf16* Brow = AT + (mt * 16 + lr) * LDA;
    f32x4 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = zero4();
#pragma unroll
    for (int jb = 0; jb < NB; jb += 2) {
      const bf16x8 bv = cat(lds4(Brow + jb * 16 + 4 * lg), lds4(Brow + (jb + 1) * 16 + 4 * lg));
#pragma unroll
      for (int u = 0; u < TPW; ++u) acc[u] = mfma32(cat(wx[jb][u], wx[jb + 1][u]), bv, acc[u]);
    }
    const int m = mt * 16 + lr;
    const float sc = eGC[m];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int kt = kt0 + u;
      if (u >= ntw) continue;
      f32x4 base;
      if (kt < DK / 16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) base[e] = (kt * 16 + 4 * lg + e == m) ? 1.f : 0.f;
      } else {
        base = to_f32x4(lds_col4(Xr + (NA + kt * 16 - DK + 4 * lg) * LD + m, LD));
      }
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = sc * (base[e] - acc[u][e]);
      *reinterpret_cast<bf16x4*>(Mout + ((mt * (KT / 2) + kt / 2) * 64 + lane) * 8 + (kt & 1) * 4) =
          to_bf16x4(v);
    }
  }
  // Output rows that are tokens (Qbar, R): base Q~ or M_K.
#pragma unroll
  for (int tt = 0; tt < kC / 16; ++tt) {
    const int mt = DK / 16 + tt;
    const __bf16* Brow = MAs + (tt * 16 + lr) * LDA;
    f32x4 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = zero4();
#pragma unroll
    for (int jb = 0; jb < NB; jb += 2) {
      const bf16x8 bv = cat(lds4(Brow + jb * 16 + 4 * lg), lds4(Brow + (jb + 1) * 16 + 4 * lg));
#pragma unroll
      for (int u = 0; u < TPW; ++u) acc[u] = mfma32(cat(wx[jb][u], wx[jb + 1][u]), bv, acc[u]);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int kt = kt0 + u;
      if (u >= ntw) continue;
      f32x4 base;
      if (kt < DK / 16) {
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
      *reinterpret_cast<bf16x4*>(Mout + ((mt * (KT / 2) + kt / 2) * 64 + lane) * 8 + (kt & 1) * 4) =
          to_bf16x4(v);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

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
  static constexpr int LDX = KIN + 8;      // padded row of X^T (bf16)
  static constexpr int XBUF = BV * LDX;    // elements of one X^T buffer
  static constexpr int LDO = BV + 8;       // padded row of the output stage
  static constexpr int OBUF = kC * LDO;
  static constexpr int LDS = 2 * (XBUF + OBUF) * 2;
  static constexpr int MSZ = MT * KT * 256;          // operator elements per chunk
  static constexpr int VITEMS = (kC / 4) * (BV / 8); // 4 tokens x 8 columns each
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
  __bf16* out;
  float* Sfin;
  const float* S0;
};

template <int DK, int BV, int NWV, int PD>
__global__ __launch_bounds__(64 * NWV) void fast_scan_kernel(FastScanArgs a) {
  using Cfg = ScanCfg<DK, BV, NWV, PD>;
  constexpr int KP = Cfg::KP, MPW = Cfg::MPW, NTN = Cfg::NTN, LDX = Cfg::LDX, NT = Cfg::NT;
  constexpr int XBUF = Cfg::XBUF, LDO = Cfg::LDO, OBUF = Cfg::OBUF, MSZ = Cfg::MSZ;
  constexpr int VITEMS = Cfg::VITEMS, OITEMS = Cfg::OITEMS, OIT = Cfg::OIT;
  static_assert(Cfg::VIT == 1, "one V piece per thread");
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* X0 = reinterpret_cast<__bf16*>(smem);
  __bf16* O0 = X0 + 2 * XBUF;
  const Problem& p = a.p;
  const int dv = p.dv;
  const int nvt = dv / BV;
  // Blocks of one (batch, head) land on one XCD (dispatch is round-robin over 8).
  const int b = blockIdx.x;
  const int grp = b / (8 * nvt), rem = b % (8 * nvt);
  const int vt = rem / 8;
  const int64_t bh = static_cast<int64_t>(grp) * 8 + rem % 8;
  const int64_t N = p.N;
  if (bh >= p.BH || N == 0) return;
  const int c0 = vt * BV;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  const __bf16* Mbh = a.M + static_cast<size_t>(bh) * N * MSZ;
  const int moff = wave * MPW * KP * 512 + lane * 8;
  // V piece of this thread: tokens 4*vs .. 4*vs+3, columns 8*vc .. 8*vc+7.
  const int vitem = tid < VITEMS ? tid : VITEMS - 1;
  const int vs = vitem / (BV / 8), vc = vitem % (BV / 8);
  const __bf16* vbh = a.v + static_cast<size_t>(bh) * p.T * dv + c0;
  __bf16* obh = a.out + static_cast<size_t>(bh) * p.T * dv + c0;

  bf16x8 mf[PD][MPW][KP];
  bf16x8 vb[PD][4];
  auto chunk_len = [&](int64_t jj) {
    const int64_t r = p.T - jj * kC;
    return static_cast<int>(r < kC ? r : kC);   // <= 0 past the last chunk
  };
  // Loads are unconditional (chunk and token indices are clamped), so no
  // control flow separates a prefetch from the work it overlaps.
  auto load_m = [&](bf16x8 (&dst)[MPW][KP], int64_t jj) {
    jj = jj < N ? jj : N - 1;
    const __bf16* Mj = Mbh + static_cast<size_t>(jj) * MSZ;
#pragma unroll
    for (int q = 0; q < MPW; ++q)
#pragma unroll
      for (int kp = 0; kp < KP; ++kp)
        dst[q][kp] = *reinterpret_cast<const bf16x8*>(Mj + moff + (q * KP + kp) * 512);
  };
  auto load_v = [&](bf16x8 (&dst)[4], int64_t jj) {
    jj = jj < N ? jj : N - 1;
    const __bf16* vj = vbh + static_cast<size_t>(jj) * kC * dv;
    const int last = chunk_len(jj) - 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = 4 * vs + r < last ? 4 * vs + r : last;
      dst[r] = *reinterpret_cast<const bf16x8*>(vj + (s * dv + vc * 8));
    }
  };
  // V_jj^T into the V rows of an X^T buffer (four tokens per 8-byte write);
  // rows past the chunk's end are zero.
  auto put_v = [&](__bf16* X, const bf16x8 (&src)[4], int64_t jj) {
    const int n = chunk_len(jj);
    if (tid < VITEMS) {
      const int pos = kperm(DK + 4 * vs);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = 4 * vs + r < n ? src[r][e] : (__bf16)0.f;
        *reinterpret_cast<bf16x4*>(X + (vc * 8 + e) * LDX + pos) = w;
      }
    }
  };
  // Output rows of chunk jj from a staging buffer to HBM (none past the end).
  auto flush_out = [&](const __bf16* O, int64_t jj) {
    const int n = chunk_len(jj);
    __bf16* oj = obh + static_cast<size_t>(jj) * kC * dv;
#pragma unroll
    for (int q = 0; q < OIT; ++q) {
      const int it = tid + q * NT;
      const int t = it / (BV / 8), cg = it % (BV / 8);
      if (it < OITEMS && t < n) *reinterpret_cast<bf16x8*>(oj + (t * dv + cg * 8)) = lds8(O + t * LDO + cg * 8);
    }
  };

#pragma unroll
  for (int u = 0; u < PD; ++u) {
    load_m(mf[u], u);
    load_v(vb[u], u);
  }
  for (int it = tid; it < DK * BV; it += NT) {
    const int i = it / BV, c = it % BV;
    const float s = a.S0 ? a.S0[(bh * DK + i) * dv + c0 + c] : 0.f;
    X0[c * LDX + kperm(i)] = (__bf16)s;
  }
  put_v(X0, vb[0], 0);
  // Ring invariant from here on: at chunk jj, vb[(jj + 1) % PD] holds V_{jj+1}.
  load_v(vb[0], PD);
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
#pragma unroll
    for (int kp = 0; kp < KP; ++kp) {
      bf16x8 bv[NTN];
#pragma unroll
      for (int nt = 0; nt < NTN; ++nt) bv[nt] = lds8(Xc + (nt * 16 + lr) * LDX + kp * 32 + 8 * lg);
#pragma unroll
      for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int q = 0; q < MPW; ++q) acc[q][nt] = mfma32(mf[u][q][kp], bv[nt], acc[q][nt]);
    }
    load_m(mf[u], jj + PD);
    if (jj > 0) flush_out(O0 + ((u + 1) & 1) * OBUF, jj - 1);
#pragma unroll
    for (int q = 0; q < MPW; ++q) {
      const int mt = wave * MPW + q;
#pragma unroll
      for (int nt = 0; nt < NTN; ++nt) {
        const int c = nt * 16 + lr;
        if (mt < DK / 16) {
          *reinterpret_cast<bf16x4*>(Xn + c * LDX + kperm(mt * 16 + 4 * lg)) = to_bf16x4(acc[q][nt]);
        } else {
          const int t = (mt - DK / 16) * 16 + 4 * lg;
#pragma unroll
          for (int e = 0; e < 4; ++e) Oc[(t + e) * LDO + c] = (__bf16)acc[q][nt][e];
        }
      }
    }
    if (jj == N - 1 && a.Sfin) {
#pragma unroll
      for (int q = 0; q < MPW; ++q) {
        const int mt = wave * MPW + q;
        if (mt < DK / 16) {
#pragma unroll
          for (int nt = 0; nt < NTN; ++nt) {
            const int i0 = mt * 16 + 4 * lg, c = nt * 16 + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) a.Sfin[(bh * DK + i0 + e) * dv + c0 + c] = acc[q][nt][e];
          }
        }
      }
    }
    const int un = (u + 1) % PD;
    put_v(Xn, vb[un], jj + 1);
    load_v(vb[un], jj + 1 + PD);
    lds_barrier();
  };

  for (int64_t j = 0; j < N; j += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) step(u, j + u);
  }
  // The last chunk's outputs, unless a step past the end already sent them.
  if (N % PD == 0) flush_out(O0 + ((N - 1) & 1) * OBUF, N - 1);
}

template <int DK, int RAB>
hipError_t launch_prep(const Problem& p, const void* q, const void* k, const float* ld,
                       const void* A, const void* B, void* M, hipStream_t s) {
  using Cfg = PrepCfg<DK, RAB>;
  FastPrepArgs a{p, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), ld,
                 static_cast<const __bf16*>(A), static_cast<const __bf16*>(B), static_cast<__bf16*>(M)};
  const void* fn = reinterpret_cast<const void*>(fast_prepare_kernel<DK, RAB>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fast_prepare_kernel<DK, RAB>), dim3(p.BH * p.N), dim3(Cfg::NT), Cfg::LDS, s, a);
  return hipGetLastError();
}

template <int DK, int BV, int NWV, int PD>
hipError_t launch_scan(const Problem& p, const void* M, const void* v, void* out, float* Sfin,
                       const float* S0, hipStream_t s) {
  using Cfg = ScanCfg<DK, BV, NWV, PD>;
  FastScanArgs a{p, static_cast<const __bf16*>(M), static_cast<const __bf16*>(v),
                 static_cast<__bf16*>(out), Sfin, S0};
  const int nvt = p.dv / BV;
  const int64_t groups = (p.BH + 7) / 8;
  const void* fn = reinterpret_cast<const void*>(fast_scan_kernel<DK, BV, NWV, PD>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fast_scan_kernel<DK, BV, NWV, PD>), dim3(groups * 8 * nvt), dim3(Cfg::NT), Cfg::LDS,
                     s, a);
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
  // Wider d_v slices share each operator load among more columns; narrower
  // ones are used when that leaves too few workgroups to fill the chip.
  if (p.dk == 128 && p.BH * (p.dv / 64) >= 256) return launch_scan<128, 64, 12, 2>(p, workspace, v, out, Sfin, S0, s);
  if (p.dk == 128) return launch_scan<128, 32, 4, 2>(p, workspace, v, out, Sfin, S0, s);
  if (p.dk == 64) return launch_scan<64, 16, 4, 4>(p, workspace, v, out, Sfin, S0, s);
  return hipErrorInvalidValue;
}

}  // namespace lattn
