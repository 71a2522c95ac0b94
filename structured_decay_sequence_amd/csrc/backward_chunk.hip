// Chunked backward on bf16 MFMAs: bf16 storage, C = 64, r_kv = 1, r_ab <= 2,
// d_k and d_v in {64, 128}.  Every chunk's gradients come from matrix
// products over the chunk (the pages print no backward; this is the chain rule
// of the chunk form of the HDLA note's "Key design 3" recurrence).
//
// Inside a chunk (tokens t = 0 .. C-1, G_t the chunk-local cumulative
// log-decay, S_in the state entering, dS_end the cotangent of the state
// leaving), with the decay-scaled operands of the forward
//   Qt = q e^{G_t},  Kt = k e^{-G_t},  At = A e^{-G_t},  Bt = B e^{G_{t-1}},
// and Gamma = e^{G_{C-1}}:
//   forward rank rows  Y = B_t S_{t-1}:   (I + L) Y = Bt S_in + M_<(Bt Kt^T) V,
//                       L = M_<(Bt At^T)  (strictly earlier tokens);
//   adjoint rank rows  X = A_t dS_t:      (I + L^T) X = At Gamma dS_end + M_>=(At Qt^T) dO;
//   gradients of the scaled operands (M_rel: keep key token s rel query token t)
//     dQt = dO S_in^T     + M_<=(dO V^T) Kt  - M_<=(dO Y^T) At
//     dKt = V (Gamma dS)^T + M_>=(V dO^T) Qt - M_>(V X^T) Bt
//     dV  = Kt Gamma dS   + M_>=(Kt Qt^T) dO - M_>(Kt Bt^T) X
//     dAt = -[Y (Gamma dS)^T + M_>=(Y dO^T) Qt - M_>(Y X^T) Bt]
//     dBt = -[X S_in^T    + M_<(X V^T) Kt    - M_<(X Y^T) At]
//   and the raw ones dq = dQt e^{G_t}, dk = dKt e^{-G_t}, dA = dAt e^{-G_t},
//   dB = dBt e^{G_{t-1}}.  The log-decay enters only through those scalings and
//   Gamma, so its gradient is (channel-wise, chunk-local reverse sum)
//     dlog_decay_u = sum_{t >= u} [q dq - k dk - sum_r A dA + sum_r B_{t+1} dB_{t+1}]_t
//                    + rowdot(dS_end, S_end) on the chunk's last token.
// S_in and dS_end come from the chunk-boundary scans.
//
// Kernels, each over all chunks, in order (the scaled operands, G (base 2),
// Gamma, the blocks of L and the inverses of its unit diagonal blocks come
// from the forward's prepare kernel, which forms them anyway): the grouped
// products out = A W0 + sum_i s_i mask_i(A B_i^T) C_i of the forward
// right-hand side and of the adjoint one, each group going on to its solve
// (Y by forward and X by backward substitution, one wave per 16 value
// columns); the grouped products of dK with dA (and dV, whose operands that
// group stages anyway), and of dQ with dB.  A product group
// stages its chunk's B-side operands in LDS row-major, straight from where
// they live (the prepare's arrays, the V and dO rows of the sequence, the
// bf16 boundary states and cotangents); operands needed transposed are read
// with the transposing LDS read.  The gradient groups' epilogues also form
// the log-decay gradient.
// Every contraction uses one K order: K values 32 ks + 16 h + 4 g + e sit at
// element 4 h + e of lane group g, so that a score tile pair in accumulator
// layout is directly the A operand of the product that follows.
#include "common.hpp"
#include "kernels.hpp"

namespace lattn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 cb8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 cb4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float cf4;
typedef short ci16x4 __attribute__((ext_vector_type(4)));

constexpr int kCC = 64;   // chunk length of this path

__device__ __forceinline__ cf4 cz4() { return cf4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ cf4 mfma_b(const cb8& x, const cb8& y, const cf4& acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
}
__device__ __forceinline__ cb4 to_b4(const cf4& v) {
  cb4 r;
  r[0] = (__bf16)v[0];
  r[1] = (__bf16)v[1];
  r[2] = (__bf16)v[2];
  r[3] = (__bf16)v[3];
  return r;
}
__device__ __forceinline__ cb8 cat8(const cb4& x, const cb4& y) {
  cb8 r;
  r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
  r[4] = y[0]; r[5] = y[1]; r[6] = y[2]; r[7] = y[3];
  return r;
}
__device__ __forceinline__ cb4 zb4() {
  cb4 r;
  r[0] = r[1] = r[2] = r[3] = (__bf16)0.f;
  return r;
}
// The fragment of a K-contiguous row in the shared K order: the K values
// 32 ks + 4 g + (0..3) and 32 ks + 16 + 4 g + (0..3) for lane group g.
__device__ __forceinline__ cb8 rowfrag(const __bf16* row, int ks, int lane) {
  const int g = lane >> 4;
  return cat8(*reinterpret_cast<const cb4*>(row + 32 * ks + 4 * g),
              *reinterpret_cast<const cb4*>(row + 32 * ks + 16 + 4 * g));
}
// Transposing LDS read of a row-major bf16 array (ld elements per row): lane
// (g, i) receives X[r0 + 4 g + e][c0 + i], e = 0..3.  The 64-bit transposing
// read works on groups of 16 lanes, element e of lane (g, i) being the
// (i % 4)-th value fetched by lane (g, 4 e + i / 4); so lane (g, j) fetches
// X[r0 + 4 g + j / 4][c0 + 4 (j % 4) .. + 3].
__device__ __forceinline__ cb4 ltr4(const __bf16* X, int ld, int r0, int c0, int lane) {
  const int g = lane >> 4, jl = lane & 15;
  const __bf16* ptr = X + (r0 + 4 * g + (jl >> 2)) * ld + c0 + 4 * (jl & 3);
  const ci16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) ci16x4*)(ptr));
  return __builtin_bit_cast(cb4, r);
}

// Per-chunk buffers of the chunked backward.
struct BcBufs {
  float* gc;                 // [C][dk] cumulative log-decay, base 2
  float* gam;                // [dk] e^{G} at the chunk's last token
  __bf16 *qt, *kt;           // [C][dk]
  __bf16 *at, *bt;           // [NA][dk]
  __bf16* lt;                // [NB (NB - 1) / 2][16][16] L below the diagonal blocks (bf16 tiles)
  float* di;                 // [NB][16][16] the inverses of the diagonal blocks I + L_ii (fp32)
  __bf16 *y, *x;             // [NA][dv]
  float* gk;                 // [C][dk] the decay gradient's terms of the dK group
  float* ends;               // [dk] rowdot(dS_end, S_end), from the dK group's staging
};

size_t bc_align(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// The decay-scaled operands Q~, K~, A~, B~ laid out from base (nullptr: only
// count).  Returns the bytes used.
size_t bc_ops_layout(const Problem& p, char* base, PrepBwOut* o) {
  const size_t J = static_cast<size_t>(p.BH * p.N);
  const size_t cdk = static_cast<size_t>(kCC) * p.dk, adk = static_cast<size_t>(kCC) * p.r_ab * p.dk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = base ? base + off : nullptr;
    off += bc_align(bytes);
    return r;
  };
  const size_t nb = static_cast<size_t>(kCC) * p.r_ab / 16;
  PrepBwOut t{};
  t.qt = take(J * cdk * 2);
  t.kt = take(J * cdk * 2);
  t.at = take(J * adk * 2);
  t.bt = take(J * adk * 2);
  t.lt = take(J * (nb * (nb > 0 ? nb - 1 : 0) / 2) * 256 * 2);
  t.di = take(J * nb * 256 * 4);
  t.gc = take(J * cdk * 4);
  t.gam = take(J * p.dk * 4);
  if (o) *o = t;
  return off;
}

// Lays the buffers out in ws (nullptr: only count); with ops given, the
// scaled operands live there instead of in ws.  Returns the bytes used.
size_t bc_layout(const Problem& p, char* ws, BcBufs* b, const PrepBwOut* ops = nullptr) {
  const size_t J = static_cast<size_t>(p.BH * p.N);
  const size_t NA = static_cast<size_t>(kCC) * p.r_ab;
  const size_t cdk = static_cast<size_t>(kCC) * p.dk, ndv = NA * p.dv;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = ws ? ws + off : nullptr;
    off += bc_align(bytes);
    return r;
  };
  BcBufs t{};
  PrepBwOut o{};
  if (ops) {
    o = *ops;
  } else {
    off += bc_ops_layout(p, ws ? ws + off : nullptr, &o);
  }
  t.qt = static_cast<__bf16*>(o.qt);
  t.kt = static_cast<__bf16*>(o.kt);
  t.at = static_cast<__bf16*>(o.at);
  t.bt = static_cast<__bf16*>(o.bt);
  t.lt = static_cast<__bf16*>(o.lt);
  t.di = static_cast<float*>(o.di);
  t.gc = static_cast<float*>(o.gc);
  t.gam = static_cast<float*>(o.gam);
  t.y = reinterpret_cast<__bf16*>(take(J * ndv * 2));
  t.x = reinterpret_cast<__bf16*>(take(J * ndv * 2));
  t.gk = reinterpret_cast<float*>(take(J * cdk * 4));
  t.ends = reinterpret_cast<float*>(take(J * p.dk * 4));
  if (b) *b = t;
  return off;
}

// ---------------------------------------------------------------------------
// Grouped products out = A W0 + sum_i s_i mask_i(A B_i^T) C_i over one chunk.
// A group is one or two kinds whose products read the same B-side operands
// (W0, B1, C1, B2, C2): one workgroup per chunk stages them in LDS once, then
// each wave forms 16 rows of one kind's output, its A rows read from memory.
// The pairs: (dK, dA) and (dQ, dB), since those read the same operands; at
// r_ab > 0 dV (which needs the adjoint solve's X) runs as a third role of
// the (dK, dA) group, whose staging holds all of its operands (BcDvInDk),
// and the right-hand sides of the two solves run alone, each group going on
// to its solve.
enum BcKind { kRhsY = 0, kRhsX = 1, kDq = 2, kDk = 3, kDv = 4, kDa = 5, kDb = 6 };
enum BcMask { kLE = 0, kLT = 1, kGE = 2, kGT = 3 };   // keep key token s rel query token t
// Where a chunk's operand lives: a per-chunk bf16 array of the prep or the
// solve; the sequence's own rows t0 .. t0 + C - 1 (bf16 [T][cols], zero past
// the sequence); the bf16 boundary states (N + 1 per head: the caller names
// the slot); the bf16 boundary cotangents, scaled by Gamma per row.
enum BcSrcKind { kSrcChunk = 0, kSrcSeq = 1, kSrcState = 2, kSrcCotG = 3 };
struct BcSrc {
  const void* ptr;
  int kind;
};

template <int KIND, int DK, int DV, int RAB>
struct BcKindCfg {
  static constexpr int NA = kCC * RAB;
  static constexpr bool ROWS_A = KIND == kRhsY || KIND == kRhsX || KIND == kDa || KIND == kDb;
  static constexpr int M = ROWS_A ? NA : kCC;                                  // rows of A
  static constexpr int RA = ROWS_A ? RAB : 1;                                  // rows per token of A
  // value-column outputs (A rows over d_k)
  static constexpr bool VOUT = KIND == kRhsY || KIND == kRhsX || KIND == kDv;
  static constexpr int KA = VOUT ? DK : DV;
  static constexpr int NOUT = VOUT ? DV : DK;
  static constexpr int MSK1 = (KIND == kRhsY || KIND == kDb) ? kLT : (KIND == kDq ? kLE : kGE);
  static constexpr bool HASW0 = true, T1 = true;
  static constexpr bool TERM2 = (KIND >= kDq && KIND <= kDb) && RAB > 0;
  static constexpr int MSK2 = KIND == kDq ? kLE : (KIND == kDb ? kLT : kGT);
  static constexpr float SIGN = (KIND == kDa || KIND == kDb) ? -1.f : 1.f;
  // W0 as it lives in memory: its transpose (S_in or Gamma dS_end for dQ, dK,
  // dA, dB), read by rows; or W0 itself (dV and the right-hand sides), read
  // with the transposing LDS read
  static constexpr bool W0T = KIND == kDq || KIND == kDk || KIND == kDa || KIND == kDb;
  // where the shared operands live (see BcSrcKind)
  static constexpr int SW0 = (KIND == kRhsY || KIND == kDq || KIND == kDb) ? kSrcState : kSrcCotG;
  static constexpr int SB1 = (KIND == kDq || KIND == kDb || KIND == kDk || KIND == kDa) ? kSrcSeq : kSrcChunk;
  static constexpr int SC1 = (KIND == kRhsY || KIND == kRhsX || KIND == kDv) ? kSrcSeq : kSrcChunk;
};

// LDS layout of a kind's staged operands (bf16 elements).  Rows read by
// 8-byte pieces (W0^T, B1, B2) are padded by 8 elements, rows read with the
// transposing read (W0, C1, C2) by 16: both keep those reads free of LDS bank
// conflicts.
template <int KIND, int DK, int DV, int RAB>
struct BcStage {
  using K = BcKindCfg<KIND, DK, DV, RAB>;
  static constexpr int NA = K::NA, KA = K::KA, NOUT = K::NOUT;
  static constexpr int W0R = K::HASW0 ? (K::W0T ? NOUT : KA) : 0, W0C = K::W0T ? KA : NOUT;
  static constexpr int LW0 = W0C + (K::W0T ? 8 : 16), LB = KA + 8, LC = NOUT + 16;
  static constexpr int OW = 0, OB1 = OW + W0R * LW0, OC1 = OB1 + (K::T1 ? kCC * LB : 0);
  static constexpr int OB2 = OC1 + (K::T1 ? kCC * LC : 0), OC2 = OB2 + (K::TERM2 ? NA * LB : 0);
  static constexpr int TOTAL = OC2 + (K::TERM2 ? NA * LC : 0);
};


// Where a kind's product reads its B-side operands in LDS (offsets and row
// strides, bf16 elements): by default its own staging layout; a kind that
// runs inside another kind's group reads that group's staging instead.
template <int KIND, int DK, int DV, int RAB>
struct BcOwnPlace {
  using L = BcStage<KIND, DK, DV, RAB>;
  static constexpr int OW = L::OW, LW0 = L::LW0, OB1 = L::OB1, LB1 = L::LB, OC1 = L::OC1, LC1 = L::LC,
                       OB2 = L::OB2, LB2 = L::LB, OC2 = L::OC2, LC2 = L::LC;
};
// dV (K~ Gamma dS_end + M_>=(K~ Q~^T) dO - M_>(K~ B~^T) X) inside the (dK, dA)
// group, whose staging holds the same operands in other roles: Gamma dS_end
// rows as its W0 (read transposed here), Q~ as its C1, dO as its B1, B~ as
// its C2 and X as its B2.
template <int DK, int DV, int RAB>
struct BcDvInDk {
  using L = BcStage<kDk, DK, DV, RAB>;
  static constexpr int OW = L::OW, LW0 = L::LW0, OB1 = L::OC1, LB1 = L::LC, OC1 = L::OB1, LC1 = L::LB,
                       OB2 = L::OC2, LB2 = L::LC, OC2 = L::OB2, LC2 = L::LB;
};

struct BcGroupArgs {
  Problem p;
  BcSrc Aa, Ab;                 // A rows of the two kinds (Ab unused for one kind)
  BcSrc W0, B1, C1, B2, C2;     // the shared B-side operands
  BcBufs w;
  void* outa;                   // the solved rank rows Y or X (bf16, [NA][d_v]), or the first kind's gradient (fp32)
  void* outb;                   // the second kind's gradient
  void* outc;                   // the (dK, dA) group: dV (fp32), formed by its third role
  const __bf16 *xr, *rr;        // dK / dQ groups: raw k or q, and raw A or B (the decay gradient's terms)
  const __bf16* ckpt;           // dK group: the boundary states (the state leaving the chunk, for the chunk-end term)
  float* dld;                   // dQ group: the log-decay gradient
};

template <int MASK>
__device__ __forceinline__ bool bc_keep(int t, int s) {
  return MASK == kLE ? s <= t : (MASK == kLT ? s < t : (MASK == kGE ? s >= t : s > t));
}
// true when no (t, s) of the token ranges survives
template <int MASK>
__device__ __forceinline__ bool bc_empty(int ta0, int ta1, int tb0, int tb1) {
  return MASK == kLE ? tb0 > ta1 : (MASK == kLT ? tb0 >= ta1 : (MASK == kGE ? tb1 < ta0 : tb1 <= ta0));
}

// The A fragments of R consecutive 16-row blocks (rb0 ..) of kind KIND for chunk job.
template <int KIND, int DK, int DV, int RAB, int R>
__device__ __forceinline__ void bc_afrag(const Problem& p, int64_t job, int rb0, const BcSrc& As,
                                         cb8 (&af)[R][BcKindCfg<KIND, DK, DV, RAB>::KA / 32], int lane) {
  using K = BcKindCfg<KIND, DK, DV, RAB>;
  const int lr = lane & 15;
  const int64_t bh = job / p.N, t0 = (job % p.N) * kCC;
  const int n = static_cast<int>(p.T - t0 < kCC ? p.T - t0 : kCC);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = 16 * (rb0 + r) + lr;
    const __bf16* arow;
    if (As.kind == kSrcSeq) {
      const int rr = row < n ? row : n - 1;   // a padding row's output is not written
      arow = static_cast<const __bf16*>(As.ptr) + (bh * p.T + t0 + rr) * K::KA;
    } else {
      arow = static_cast<const __bf16*>(As.ptr) + (job * K::M + row) * K::KA;
    }
#pragma unroll
    for (int ks = 0; ks < K::KA / 32; ++ks) af[r][ks] = rowfrag(arow, ks, lane);
  }
}

// R consecutive 16-row blocks (rb0 ..) of kind KIND's product for chunk job,
// B side in LDS: acc[r] (accumulator layout: lane holds rows 4 lg + e of
// block rb0 + r, column 16 ot + lr).  Every B-side fragment read from LDS
// serves the R blocks, so waves of two blocks halve those reads.  PL: where
// the operands sit in LDS (BcOwnPlace, or another group's staging).
template <int KIND, int DK, int DV, int RAB, int R, class PL = BcOwnPlace<KIND, DK, DV, RAB>>
__device__ __forceinline__ void bc_prod(const Problem& p, int64_t job, int rb0,
                                        const cb8 (&af)[R][BcKindCfg<KIND, DK, DV, RAB>::KA / 32], const __bf16* lds,
                                        cf4 (&acc)[R][BcKindCfg<KIND, DK, DV, RAB>::NOUT / 16], int lane) {
  using K = BcKindCfg<KIND, DK, DV, RAB>;
  constexpr int KS = K::KA / 32, OT = K::NOUT / 16, NA = K::NA;
  const int lr = lane & 15, lg = lane >> 4;
  const int r0 = 16 * rb0;
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) {
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][ot] = cz4();
    if constexpr (K::HASW0) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        cb8 bw;
        if constexpr (K::W0T)
          bw = rowfrag(lds + PL::OW + (16 * ot + lr) * PL::LW0, ks, lane);
        else
          bw = cat8(ltr4(lds + PL::OW, PL::LW0, 32 * ks, 16 * ot, lane),
                    ltr4(lds + PL::OW, PL::LW0, 32 * ks + 16, 16 * ot, lane));
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][ot] = mfma_b(af[r][ks], bw, acc[r][ot]);
      }
    }
  }
  // token range of the R blocks' rows, and each lane's row token per block
  const int ta0 = r0 / K::RA, ta1 = (r0 + 16 * R - 1) / K::RA;
  int trow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) trow[r] = (r0 + 16 * r + lr) / K::RA;
  // one score term: NB columns (RB rows of B per token), mask, sign
  auto term = [&](int oB, int oC, auto nb_, auto rb_, auto mask_, float sg, auto lb_, auto lc_) {
    constexpr int NBc = decltype(nb_)::value, RB = decltype(rb_)::value, MASK = decltype(mask_)::value;
    constexpr int LBt = decltype(lb_)::value, LCt = decltype(lc_)::value;
#pragma unroll 1
    for (int c0 = 0; c0 < NBc; c0 += 32) {
      if (bc_empty<MASK>(ta0, ta1, c0 / RB, (c0 + 31) / RB)) continue;
      cf4 s2[R][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < R; ++r) s2[r][h] = cz4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const cb8 bfr = rowfrag(lds + oB + (c0 + 16 * h + lr) * LBt, ks, lane);
#pragma unroll
          for (int r = 0; r < R; ++r) s2[r][h] = mfma_b(bfr, af[r][ks], s2[r][h]);
        }
        // lane: score(row r0 + 16 r + lr, column c0 + 16 h + 4 lg + e)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s2[r][h][e] = bc_keep<MASK>(trow[r], (c0 + 16 * h + 4 * lg + e) / RB) ? sg * s2[r][h][e] : 0.f;
      }
      cb8 sf[R];
#pragma unroll
      for (int r = 0; r < R; ++r) sf[r] = cat8(to_b4(s2[r][0]), to_b4(s2[r][1]));
#pragma unroll
      for (int ot = 0; ot < OT; ++ot) {
        const cb8 cf = cat8(ltr4(lds + oC, LCt, c0, 16 * ot, lane), ltr4(lds + oC, LCt, c0 + 16, 16 * ot, lane));
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][ot] = mfma_b(sf[r], cf, acc[r][ot]);
      }
    }
  };
  using I1 = std::integral_constant<int, 1>;
  if constexpr (K::T1)
    term(PL::OB1, PL::OC1, std::integral_constant<int, kCC>{}, I1{}, std::integral_constant<int, K::MSK1>{}, 1.f,
         std::integral_constant<int, PL::LB1>{}, std::integral_constant<int, PL::LC1>{});
  if constexpr (K::TERM2)
    term(PL::OB2, PL::OC2, std::integral_constant<int, NA>{}, std::integral_constant<int, (RAB > 0 ? RAB : 1)>{},
         std::integral_constant<int, K::MSK2>{}, -1.f, std::integral_constant<int, PL::LB2>{},
         std::integral_constant<int, PL::LC2>{});
}

// A gradient kind's rows from the LDS copy of the products (ep: M rows of
// NOUT + 4 floats) to memory, four columns per thread: scaled back from the
// decay-scaled operands (e^{+-G} per token and channel) and signed.
template <int KIND, int DK, int DV, int RAB, int NT>
__device__ __forceinline__ void bc_out(const Problem& p, int64_t job, const float* ep, float* out, int tid) {
  using K = BcKindCfg<KIND, DK, DV, RAB>;
  static_assert(KIND == kDv, "the other gradients leave through bc_epi");
  constexpr int C4 = K::NOUT / 4, LE = K::NOUT + 4, ITEMS = K::M * C4;
  const int64_t bh = job / p.N, t0 = (job % p.N) * kCC;
  const int n = static_cast<int>(p.T - t0 < kCC ? p.T - t0 : kCC);
  const int64_t tok0 = bh * p.T + t0;
#pragma unroll 4
  for (int it = tid; it < ITEMS; it += NT) {
    const int t = it / C4, c = (it - t * C4) * 4;
    if (t >= n) continue;
    *reinterpret_cast<cf4*>(out + (tok0 + t) * K::NOUT + c) = *reinterpret_cast<const cf4*>(ep + t * LE + c);
  }
}

// One operand's staging: ROWS x COLS bf16 from source kind SRC, in pieces of
// eight elements, IT per thread (NT threads).  slot: the chunk's index in a
// per-chunk source (for the boundary states, the caller's slot).
template <int SRC, int ROWS, int COLS, int NT>
struct BcStg {
  static constexpr int P = ROWS * COLS / 8, IT = (P + NT - 1) / NT, PR = COLS / 8;
  cb8 x[IT];
  float gs[SRC == kSrcCotG ? IT : 1];
  int n_ = 0;
  __device__ __forceinline__ void load(const void* ptr, const float* gam, int64_t slot, int n, int64_t tok0, int tid) {
    n_ = n;
    const __bf16* src = static_cast<const __bf16*>(ptr);
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int i0 = tid + k * NT, i = i0 < P ? i0 : P - 1;   // the last piece again, not stored
      const int r = i / PR, c8 = (i - r * PR) * 8;
      if constexpr (SRC == kSrcSeq) {
        // rows past the sequence read its last row and are zeroed at the store
        const int rr = r < n ? r : n - 1;
        x[k] = *reinterpret_cast<const cb8*>(src + (tok0 + rr) * COLS + c8);
      } else {
        x[k] = *reinterpret_cast<const cb8*>(src + (slot * ROWS + r) * COLS + c8);
        if constexpr (SRC == kSrcCotG) gs[k] = gam[r];
      }
    }
  }
  __device__ __forceinline__ void store(__bf16* lds, int ld, int tid) {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int i = tid + k * NT;
      if (i < P) {
        const int r = i / PR, c8 = (i - r * PR) * 8;
        cb8 v = x[k];
        if constexpr (SRC == kSrcCotG) {
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = (__bf16)(gs[k] * (float)x[k][u]);
        } else if constexpr (SRC == kSrcSeq) {
          if (r >= n_) {
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = (__bf16)0.f;
          }
        }
        *reinterpret_cast<cb8*>(lds + r * ld + c8) = v;
      }
    }
  }
};

// Epilogue of the (dK, dA) and (dQ, dB) groups (or dK, dQ alone at rank 0):
// the products, still in LDS (ep: the first kind's kCC rows, then the rank
// rows), become the raw operands' gradients, and the decay gradient's
// per-(token, channel) terms are formed beside them.  An item is (token t,
// four channels); one exp2 of the token's cumulative log-decay serves all of
// its outputs (P = the products before their sign):
//   dK group: f = 2^{-G_t}: dK_t = f Pk_t, dA_{t,r} = -f Pa_{t,r},
//             term_t = -f (k_t Pk_t - sum_r A_{t,r} Pa_{t,r})       -> gk
//   dQ group: f = 2^{G_t}:  dq_t = f Pq_t, dB_{t+1,r} = -f Pb_{t+1,r} (inside
//             the chunk; dB_{0,r} = -Pb_{0,r}),
//             term_t = f (q_t Pq_t - sum_r B_{t+1,r} Pb_{t+1,r}) + gk_t -> LDS
// The dQ group, which runs second, then forms the log-decay gradient: per
// channel the reverse sum over the chunk's tokens of term_t, on top of the
// chunk-end term rowdot(dS_end, S_end) (ends).  The global loads (G, raw k or
// q, raw A or B, gk) are issued by load() before the products go through LDS,
// so their latency overlaps that copy.
template <bool KG, int DK, int RAB, int NT>
struct BcEpi {
  static constexpr int C4 = DK / 4, LE = DK + 4, RA = RAB > 0 ? RAB : 1;
  static constexpr int ITEMS = kCC * C4, IT = (ITEMS + NT - 1) / NT;
  static constexpr int LT = DK + 4;   // row of the terms in LDS (floats)
  // reverse sums: SEG segments of the chunk's tokens per channel
  static constexpr int SEG = NT / DK >= 8 ? 8 : (NT / DK >= 4 ? 4 : (NT / DK >= 2 ? 2 : 1));
  static constexpr int TPS = kCC / SEG;
  // LDS the dQ group needs beyond the products (bytes)
  static constexpr int EXTRA = KG ? 0 : (kCC * LT + SEG * DK) * 4;
  cf4 g[IT], gkv[KG ? 1 : IT];
  cb4 xv[IT], rv[IT][RA];
  int n;
  int64_t tok0;
  __device__ __forceinline__ void load(const Problem& p, int64_t job, const BcBufs& w, const __bf16* xr,
                                       const __bf16* rr, int tid) {
    const int64_t bh = job / p.N, t0 = (job % p.N) * kCC;
    n = static_cast<int>(p.T - t0 < kCC ? p.T - t0 : kCC);
    tok0 = bh * p.T + t0;
    const float* gc = w.gc + job * kCC * DK;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int i0 = tid + k * NT, it = i0 < ITEMS ? i0 : ITEMS - 1;
      const int t = it / C4, c = (it - t * C4) * 4;
      const int tt = t < n ? t : n - 1;   // padding tokens read a live row, not kept
      g[k] = *reinterpret_cast<const cf4*>(gc + t * DK + c);
      xv[k] = *reinterpret_cast<const cb4*>(xr + (tok0 + tt) * DK + c);
      if constexpr (!KG) gkv[k] = *reinterpret_cast<const cf4*>(w.gk + (job * kCC + tt) * DK + c);
      if constexpr (RAB > 0) {
        const int tr = KG ? tt : (tt + 1 < n ? tt + 1 : tt);
#pragma unroll
        for (int r = 0; r < RAB; ++r) rv[k][r] = *reinterpret_cast<const cb4*>(rr + ((tok0 + tr) * RAB + r) * DK + c);
      }
    }
  }
  // terms: the dQ group's LDS area for the per-(token, channel) terms
  __device__ __forceinline__ void finish(int64_t job, const float* ep, const BcBufs& w, float* outa, float* outb,
                                         float* terms, int tid) {
    const float* epb = ep + kCC * LE;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int it = tid + k * NT;
      const int t = it / C4, c = (it - t * C4) * 4;
      if (it >= ITEMS) continue;
      if (t >= n) {
        if constexpr (!KG) *reinterpret_cast<cf4*>(terms + t * LT + c) = cf4{0.f, 0.f, 0.f, 0.f};
        continue;
      }
      cf4 f;
#pragma unroll
      for (int u = 0; u < 4; ++u) f[u] = __builtin_amdgcn_exp2f(KG ? -g[k][u] : g[k][u]);
      const cf4 pa = *reinterpret_cast<const cf4*>(ep + t * LE + c);
      cf4 o, v;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        o[u] = pa[u] * f[u];
        v[u] = (float)xv[k][u] * pa[u];
      }
      *reinterpret_cast<cf4*>(outa + (tok0 + t) * DK + c) = o;
      if constexpr (RAB > 0) {
        const int tr = KG ? t : t + 1;   // token of the rank rows
        if (tr < n) {
#pragma unroll
          for (int r = 0; r < RAB; ++r) {
            const cf4 pb = *reinterpret_cast<const cf4*>(epb + (tr * RAB + r) * LE + c);
            cf4 ob;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              v[u] -= (float)rv[k][r][u] * pb[u];
              ob[u] = -pb[u] * f[u];
            }
            *reinterpret_cast<cf4*>(outb + ((tok0 + tr) * RAB + r) * DK + c) = ob;
          }
        }
        if (!KG && t == 0) {
#pragma unroll
          for (int r = 0; r < RAB; ++r) {
            const cf4 pb = *reinterpret_cast<const cf4*>(epb + r * LE + c);
            *reinterpret_cast<cf4*>(outb + (tok0 * RAB + r) * DK + c) = cf4{-pb[0], -pb[1], -pb[2], -pb[3]};
          }
        }
      }
      if constexpr (KG) {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] *= -f[u];
        *reinterpret_cast<cf4*>(w.gk + (job * kCC + t) * DK + c) = v;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = v[u] * f[u] + gkv[k][u];
        *reinterpret_cast<cf4*>(terms + t * LT + c) = v;
      }
    }
  }
  // dQ group, after finish() and a barrier: the log-decay gradient.  Thread
  // (segment sg, channel c) sums its TPS tokens; then, on top of the later
  // segments and the chunk-end term, writes the reverse running sum.  Scalar
  // decay: the per-(token, channel) sums go back to LDS and are added over
  // the channels per token.
  __device__ __forceinline__ void reverse(const Problem& p, int64_t job, const BcBufs& w, float* terms, float* dld,
                                          int tid) {
    static_assert(!KG, "the dQ group forms the log-decay gradient");
    float* segt = terms + kCC * LT;
    const int c = tid % DK, sg = tid / DK;
    const bool act = tid < SEG * DK;
    if (act) {
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < TPS; ++u) sum += terms[(sg * TPS + u) * LT + c];
      segt[sg * DK + c] = sum;
    }
    __syncthreads();
    if (act) {
      float acc = w.ends[job * DK + c];
#pragma unroll
      for (int s2 = SEG - 1; s2 > 0; --s2)
        if (s2 > sg) acc += segt[s2 * DK + c];
#pragma unroll
      for (int u = TPS - 1; u >= 0; --u) {
        const int t = sg * TPS + u;
        acc += terms[t * LT + c];
        if (p.scalar)
          terms[t * LT + c] = acc;
        else if (t < n)
          dld[(tok0 + t) * DK + c] = acc;
      }
    }
    if (p.scalar) {
      // 8 threads per token, each over every eighth channel
      __syncthreads();
      for (int idx = tid; idx < kCC * 8; idx += NT) {
        const int t = idx / 8, part = idx % 8;
        float sum = 0.f;
#pragma unroll
        for (int c2 = part; c2 < DK; c2 += 8) sum += terms[t * LT + c2];
#pragma unroll
        for (int sh = 1; sh < 8; sh *= 2) sum += __shfl_xor(sum, sh, 64);
        if (part == 0 && t < n) dld[tok0 + t] = sum;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Solve, inside the right-hand side's own group.  Once the products are done
// the group's waves put the right-hand side's tiles (bf16, rounded as the
// substitution's own products round the solved blocks), the blocks of L and
// the inverses of its diagonal blocks in the LDS the staging used, then each
// wave solves 16 columns of values.
//  * The blocks of L = M_<(Bt At^T) (rank rows; tokens row / r_ab) come from
//    the prepare, which formed them for the forward's own solve: the 16x16
//    bf16 tiles below the diagonal and the fp32 inverses D_i of the diagonal
//    blocks I + L_ii.  Their loads are issued after the staging's, and held
//    in registers through the products; the X group stores them transposed.
//  * Y: forward substitution Y_i = D_i (R_i - sum_{j<i} L_ij Y_j); X: backward
//    substitution X_i = D_i^T (R_i - sum_{j>i} L_ji^T X_j).  The products pair
//    two 16-row blocks into one 16x16x32 MFMA (a lone block padded with
//    zeros), the solved blocks fed back from registers as the B operand; the
//    diagonal inverses apply in fp32.
template <int DK, int DV, int RAB>
struct BcSolveCfg {
  static constexpr int NA = kCC * RAB, NB = NA / 16, NTI = NB * (NB > 0 ? NB - 1 : 0) / 2;
  static constexpr int NCT = DV / 16;
  // LDS (bytes): L's tiles (bf16), the diagonal blocks' inverses (fp32), the
  // right-hand side in tile order [NB][NCT][64 lanes][4] (bf16)
  static constexpr int OL = 0, ODI = OL + NTI * 512, ORH = ODI + NB * 1024, LDS = ORH + NA * DV * 2;
  // 16-byte pieces of the tiles and of the inverses
  static constexpr int NLP = NTI * 32, NDP = NB * 64;
};

template <int DK, int DV, int RAB, int NT>
struct BcSolveStg {
  using Cf = BcSolveCfg<DK, DV, RAB>;
  static constexpr int NIT = (Cf::NLP + Cf::NDP + NT - 1) / NT > 0 ? (Cf::NLP + Cf::NDP + NT - 1) / NT : 1;
  cb8 pc[NIT];
  __device__ __forceinline__ void load(const BcBufs& w, int64_t job, int tid) {
    const cb8* gl = reinterpret_cast<const cb8*>(w.lt + job * Cf::NTI * 256);
    const cb8* gd = reinterpret_cast<const cb8*>(w.di + job * Cf::NB * 256);
#pragma unroll
    for (int q = 0; q < NIT; ++q) {
      const int it = tid + q * NT;
      if (it < Cf::NLP) pc[q] = gl[it];
      else if (it < Cf::NLP + Cf::NDP) pc[q] = gd[it - Cf::NLP];
    }
  }
  // the pieces as loaded (Y), or every tile transposed (X)
  template <bool TR>
  __device__ __forceinline__ void store(unsigned char* sm, int tid) const {
    __bf16* Lb = reinterpret_cast<__bf16*>(sm + Cf::OL);
    float* Di = reinterpret_cast<float*>(sm + Cf::ODI);
#pragma unroll
    for (int q = 0; q < NIT; ++q) {
      const int it = tid + q * NT;
      if (it < Cf::NLP) {
        if constexpr (TR) {
          // tile it / 32, row (it % 32) / 2, columns 8 (it % 2) .. + 7
          const int b0 = (it >> 5) * 256, r = (it >> 1) & 15, c0 = (it & 1) * 8;
#pragma unroll
          for (int u = 0; u < 8; ++u) Lb[b0 + (c0 + u) * 16 + r] = pc[q][u];
        } else {
          *reinterpret_cast<cb8*>(Lb + it * 8) = pc[q];
        }
      } else if (it < Cf::NLP + Cf::NDP) {
        const int i2 = it - Cf::NLP;
        if constexpr (TR) {
          // block i2 / 64, row (i2 % 64) / 4, columns 4 (i2 % 4) .. + 3
          const cf4 f = __builtin_bit_cast(cf4, pc[q]);
          const int b0 = (i2 >> 6) * 256, r = (i2 >> 2) & 15, c0 = (i2 & 3) * 4;
#pragma unroll
          for (int u = 0; u < 4; ++u) Di[b0 + (c0 + u) * 16 + r] = f[u];
        } else {
          *reinterpret_cast<cb8*>(Di + i2 * 4) = pc[q];
        }
      }
    }
  }
};

// The substitution over the LDS above: wave wv solves the value column tiles
// wv, wv + NW, .. and writes them to out ([NA][d_v], bf16).
template <int DK, int DV, int RAB, bool ISX, int NW>
__device__ __forceinline__ void bc_substitute(const unsigned char* sm, __bf16* out, int wave, int lane) {
  using Cf = BcSolveCfg<DK, DV, RAB>;
  constexpr int NB = Cf::NB, NCT = Cf::NCT;
  const __bf16* Lt = reinterpret_cast<const __bf16*>(sm + Cf::OL);
  const float* Dg = reinterpret_cast<const float*>(sm + Cf::ODI);
  const __bf16* R = reinterpret_cast<const __bf16*>(sm + Cf::ORH);
  const int lr = lane & 15, lg = lane >> 4;
  auto ltile = [&](int blk) { return *reinterpret_cast<const cb4*>(Lt + blk * 256 + lr * 16 + 4 * lg); };
  for (int ct = wave; ct < NCT; ct += NW) {
    cb4 nb[NB];   // -solution blocks in bf16, the B operand of later blocks
    auto rhs = [&](int i) {
      const cb4 r = *reinterpret_cast<const cb4*>(R + ((i * NCT + ct) * 64 + lane) * 4);
      return cf4{(float)r[0], (float)r[1], (float)r[2], (float)r[3]};
    };
    auto finish = [&](int i, cf4 acc) {
      const cf4 dF = *reinterpret_cast<const cf4*>(Dg + i * 256 + lr * 16 + 4 * lg);
      cf4 o = cz4();
#pragma unroll
      for (int e = 0; e < 4; ++e) o = __builtin_amdgcn_mfma_f32_16x16x4f32(dF[e], acc[e], o, 0, 0, 0);
      nb[i] = to_b4(cf4{-o[0], -o[1], -o[2], -o[3]});
      // lane holds rows 16 i + 4 lg + e, column 16 ct + lr
#pragma unroll
      for (int e = 0; e < 4; ++e) out[(16 * i + 4 * lg + e) * DV + 16 * ct + lr] = (__bf16)o[e];
    };
    if constexpr (!ISX) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        cf4 acc = rhs(i);
        const int base = i * (i - 1) / 2;   // tiles (i, 0 .. i-1)
#pragma unroll
        for (int jb = 0; jb + 1 < i; jb += 2)
          acc = mfma_b(cat8(ltile(base + jb), ltile(base + jb + 1)), cat8(nb[jb], nb[jb + 1]), acc);
        if (i % 2 == 1) acc = mfma_b(cat8(ltile(base + i - 1), zb4()), cat8(nb[i - 1], zb4()), acc);
        finish(i, acc);
      }
    } else {
#pragma unroll
      for (int i = NB - 1; i >= 0; --i) {
        cf4 acc = rhs(i);
        // tiles (L_ji)^T for j = i+1 .. NB-1, stored at index j (j - 1) / 2 + i
        int jb = i + 1;
#pragma unroll
        for (; jb + 1 < NB; jb += 2)
          acc = mfma_b(cat8(ltile(jb * (jb - 1) / 2 + i), ltile((jb + 1) * jb / 2 + i)), cat8(nb[jb], nb[jb + 1]), acc);
        if (jb < NB) acc = mfma_b(cat8(ltile(jb * (jb - 1) / 2 + i), zb4()), cat8(nb[jb], zb4()), acc);
        finish(i, acc);
      }
    }
  }
}

template <int KA_, int KB_>
struct BcGroupWaves {
  // 16-row blocks per wave of the second kind: the rank-row gradients (dA,
  // dB) take two, so that with the first kind's one per wave every SIMD
  // holds three blocks, and their B-side reads serve two blocks.
  static constexpr int RB = (KB_ == kDa || KB_ == kDb) ? 2 : 1;
  // At r_ab > 0 the (dK, dA) group also forms dV, whose operands it stages
  // anyway (BcDvInDk): one wave per 16-token block (WC of them).
  template <int RAB>
  static constexpr bool fuse_dv() { return KA_ == kDk && RAB > 0; }
  template <int RAB>
  static constexpr int wc() { return fuse_dv<RAB>() ? kCC / 16 : 0; }
  template <int DK, int DV, int RAB>
  static constexpr int count() {
    return BcKindCfg<KA_, DK, DV, RAB>::M / 16 +
           (KB_ >= 0 ? BcKindCfg<(KB_ >= 0 ? KB_ : KA_), DK, DV, RAB>::M / (16 * RB) : 0) + wc<RAB>();
  }
  // output rows of the group (both kinds)
  template <int DK, int DV, int RAB>
  static constexpr int rows() {
    return BcKindCfg<KA_, DK, DV, RAB>::M + (KB_ >= 0 ? BcKindCfg<(KB_ >= 0 ? KB_ : KA_), DK, DV, RAB>::M : 0);
  }
};

template <int KA_, int KB_, int DK, int DV, int RAB, int NW>
__device__ __forceinline__ void bwc_group_body(const BcGroupArgs& a, const int64_t job) {
  using K = BcKindCfg<KA_, DK, DV, RAB>;
  using L = BcStage<KA_, DK, DV, RAB>;
  constexpr int WA = K::M / 16, KS = K::KA / 32, OT = K::NOUT / 16;
  // the right-hand side groups, which go on to solve (bc_substitute)
  constexpr bool RHS = KA_ == kRhsY || KA_ == kRhsX;
  static_assert(!RHS || KB_ < 0, "a right-hand side group holds one kind");
  using LB_ = BcStage<(KB_ >= 0 ? KB_ : KA_), DK, DV, RAB>;
  static_assert(LB_::OW == L::OW && LB_::OB1 == L::OB1 && LB_::OC1 == L::OC1 && LB_::OB2 == L::OB2 &&
                    LB_::OC2 == L::OC2 && LB_::LW0 == L::LW0 && LB_::LB == L::LB && LB_::LC == L::LC,
                "the two kinds of a group read one staging layout");
  extern __shared__ __align__(16) unsigned char smem_[];
  __bf16* lds = reinterpret_cast<__bf16*>(smem_);
  const Problem& p = a.p;
  const int64_t bh = job / p.N, jc = job % p.N;
  const int n = static_cast<int>(p.T - jc * kCC < kCC ? p.T - jc * kCC : kCC);
  const int64_t tok0 = bh * p.T + jc * kCC;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool isa = wave < WA;
  constexpr int RB = BcGroupWaves<KA_, KB_>::RB;
  constexpr int KB2 = KB_ >= 0 ? KB_ : KA_;
  // the fused dV waves come last
  constexpr bool FDV = BcGroupWaves<KA_, KB_>::template fuse_dv<RAB>();
  constexpr int WC = BcGroupWaves<KA_, KB_>::template wc<RAB>();
  using KC = BcKindCfg<kDv, DK, DV, RAB>;
  constexpr int KSC = KC::KA / 32, OTC = KC::NOUT / 16;
  const bool isc = FDV && wave >= NW - WC;
  // first 16-row block of this wave within its kind
  const int rb = isa ? wave : (isc ? wave - (NW - WC) : (wave - WA) * RB);
  // this wave's A rows first, so that their loads overlap the staging's
  cb8 af[RB][KS];
  cb8 afc[1][KSC];
  if (isa) {
    bc_afrag<KA_, DK, DV, RAB, 1>(p, job, rb, a.Aa, reinterpret_cast<cb8(&)[1][KS]>(af), lane);
  } else if (isc) {
    if constexpr (FDV) bc_afrag<kDv, DK, DV, RAB, 1>(p, job, rb, BcSrc{a.w.kt, kSrcChunk}, afc, lane);
  } else if constexpr (KB_ >= 0) {
    bc_afrag<KB_, DK, DV, RAB, RB>(p, job, rb, a.Ab, af, lane);
  }
  // Staging: every load of every operand is issued before any LDS write, so
  // their latencies overlap.
  BcStg<K::SW0, L::W0R, L::W0C, 64 * NW> s0;
  BcStg<K::SB1, kCC, K::KA, 64 * NW> s1;
  BcStg<K::SC1, kCC, K::NOUT, 64 * NW> s2;
  BcStg<kSrcChunk, (K::TERM2 ? K::NA : 16), K::KA, 64 * NW> s3;
  BcStg<kSrcChunk, (K::TERM2 ? K::NA : 16), K::NOUT, 64 * NW> s4;
  // the boundary states have N + 1 slots per head: the state entering chunk
  // jc is slot jc, the one leaving it slot jc + 1
  if constexpr (K::HASW0) s0.load(a.W0.ptr, a.w.gam + job * DK, K::SW0 == kSrcState ? job + bh : job, n, tok0, tid);
  // dK group: the state leaving the chunk, for the chunk-end term of the decay gradient
  BcStg<kSrcState, L::W0R, L::W0C, 64 * NW> se;
  if constexpr (KA_ == kDk) se.load(a.ckpt, nullptr, job + bh + 1, n, tok0, tid);
  if constexpr (K::T1) {
    s1.load(a.B1.ptr, nullptr, job, n, tok0, tid);
    s2.load(a.C1.ptr, nullptr, job, n, tok0, tid);
  }
  if constexpr (K::TERM2) {
    s3.load(a.B2.ptr, nullptr, job, n, tok0, tid);
    s4.load(a.C2.ptr, nullptr, job, n, tok0, tid);
  }
  // the solve's blocks of L and diagonal inverses, held through the products
  BcSolveStg<DK, DV, RAB, 64 * NW> ss;
  if constexpr (RHS) ss.load(a.w, job, tid);
  if constexpr (K::HASW0) s0.store(lds + L::OW, L::LW0, tid);
  if constexpr (K::T1) {
    s1.store(lds + L::OB1, L::LB, tid);
    s2.store(lds + L::OC1, L::LC, tid);
  }
  if constexpr (K::TERM2) {
    s3.store(lds + L::OB2, L::LB, tid);
    s4.store(lds + L::OC2, L::LC, tid);
  }
  if constexpr (KA_ == kDk) {
    // rowdot(dS_end, S_end) per state channel: the raw dS_end pieces staged
    // as W0 (before their Gamma scaling) against S_end, summed over the
    // PR threads of a row
    static_assert(L::W0R == DK && L::W0C == DV && K::SW0 == kSrcCotG, "dK group: W0 is dS_end [d_k][d_v]");
    constexpr int PR = DV / 8, P = DK * DV / 8;
#pragma unroll
    for (int k = 0; k < decltype(s0)::IT; ++k) {
      const int i = tid + k * 64 * NW;
      float d = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) d += (float)s0.x[k][u] * (float)se.x[k][u];
#pragma unroll
      for (int sh = 1; sh < PR; sh *= 2) d += __shfl_xor(d, sh, 64);
      if (i < P && i % PR == 0) a.w.ends[job * DK + i / PR] = d;
    }
  }
  __syncthreads();
  cf4 acc[RB][OT];
  cf4 accc[1][OTC];
  // rows of padding tokens only: no gradient to write (the right-hand sides
  // are formed for them too, as zeros, since the solves read every row)
  const int ra = isa || isc ? 1 : BcKindCfg<KB2, DK, DV, RAB>::RA;
  const bool live = RHS || 16 * rb / (isa ? K::RA : ra) < n;
  if (live) {
    if (isa) {
      bc_prod<KA_, DK, DV, RAB, 1>(p, job, rb, reinterpret_cast<const cb8(&)[1][KS]>(af), lds,
                                   reinterpret_cast<cf4(&)[1][OT]>(acc), lane);
    } else if (isc) {
      // dV from this group's staged operands (BcDvInDk)
      if constexpr (FDV) bc_prod<kDv, DK, DV, RAB, 1, BcDvInDk<DK, DV, RAB>>(p, job, rb, afc, lds, accc, lane);
    } else if constexpr (KB_ >= 0) {
      bc_prod<KB_, DK, DV, RAB, RB>(p, job, rb, af, lds, acc, lane);
    }
  }
  if constexpr (RHS) {
    // the right-hand side's tiles, L's blocks and the diagonal inverses into
    // the staging space, then the substitution, one value column tile a wave
    using SC = BcSolveCfg<DK, DV, RAB>;
    static_assert(K::M == SC::NA && K::NOUT == DV && OT == SC::NCT && NW == SC::NB, "solve tiling");
    __syncthreads();   // every wave is done with the staged operands
    __bf16* rt = reinterpret_cast<__bf16*>(smem_ + SC::ORH);
#pragma unroll
    for (int ot = 0; ot < OT; ++ot) *reinterpret_cast<cb4*>(rt + ((rb * OT + ot) * 64 + lane) * 4) = to_b4(acc[0][ot]);
    ss.template store<KA_ == kRhsX>(smem_, tid);
    __syncthreads();
    bc_substitute<DK, DV, RAB, KA_ == kRhsX, NW>(smem_, static_cast<__bf16*>(a.outa) + job * SC::NA * DV, wave, lane);
  } else {
    // The gradients leave through LDS as whole rows: every wave's 16-row
    // blocks of NOUT columns into the (now free) staging space (the first
    // kind's rows, then the second's), then 16-byte stores.
    constexpr int LE = K::NOUT + 4;
    constexpr bool GRAD = KA_ == kDk || KA_ == kDq;   // the fused epilogue (else dV)
    float* ep = reinterpret_cast<float*>(smem_);
    BcEpi<KA_ == kDk, DK, RAB, 64 * NW> epi;
    if constexpr (GRAD) epi.load(p, job, a.w, a.xr, a.rr, tid);
    __syncthreads();   // every wave is done with the staged operands
    // the fused dV rows (d_v + 4 floats each) after both kinds' rows
    float* epc = ep + BcGroupWaves<KA_, KB_>::template rows<DK, DV, RAB>() * LE;
    if (live) {
      const int lr = lane & 15, lg = lane >> 4;
      if (isc) {
        if constexpr (FDV) {
#pragma unroll
          for (int ot = 0; ot < OTC; ++ot)
#pragma unroll
            for (int e = 0; e < 4; ++e) epc[(rb * 16 + 4 * lg + e) * (DV + 4) + 16 * ot + lr] = accc[0][ot][e];
        }
      } else {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          if (isa && r > 0) break;
          const int blk = isa ? rb : WA + rb + r;
#pragma unroll
          for (int ot = 0; ot < OT; ++ot)
#pragma unroll
            for (int e = 0; e < 4; ++e) ep[(blk * 16 + 4 * lg + e) * LE + 16 * ot + lr] = acc[r][ot][e];
        }
      }
    }
    __syncthreads();
    if constexpr (FDV) bc_out<kDv, DK, DV, RAB, 64 * NW>(p, job, epc, static_cast<float*>(a.outc), tid);
    if constexpr (GRAD) {
      static_assert(K::M == kCC && LE == DK + 4, "fused epilogue: token rows, then rank rows, of width d_k");
      float* terms = ep + BcGroupWaves<KA_, KB_>::template rows<DK, DV, RAB>() * LE;   // dQ group: beyond the products
      epi.finish(job, ep, a.w, static_cast<float*>(a.outa), static_cast<float*>(a.outb), terms, tid);
      if constexpr (KA_ == kDq) {
        __syncthreads();
        epi.reverse(p, job, a.w, terms, a.dld, tid);
      }
    } else {
      static_assert(KB_ < 0, "dV runs alone");
      bc_out<KA_, DK, DV, RAB, 64 * NW>(p, job, ep, static_cast<float*>(a.outa), tid);
    }
  }
}

template <int KA_, int KB_, int DK, int DV, int RAB, int NW>
__global__ __launch_bounds__(64 * NW) void bwc_group_kernel(BcGroupArgs a) {
  bwc_group_body<KA_, KB_, DK, DV, RAB, NW>(a, blockIdx.x);
}

// The two right-hand side groups (each with its solve) in one launch: blocks
// b and b + 8, which dispatch places on one XCD, take the Y and the X group
// of one chunk, so that the blocks of L they both read meet in one L2.
template <int DK, int DV, int RAB, int NW>
__global__ __launch_bounds__(64 * NW) void bwc_rhs_pair_kernel(BcGroupArgs ay, BcGroupArgs ax) {
  const int64_t b = blockIdx.x, job = (b >> 4) * 8 + (b & 7);
  if (job >= ay.p.BH * ay.p.N) return;
  if ((b >> 3) & 1)
    bwc_group_body<kRhsX, -1, DK, DV, RAB, NW>(ax, job);
  else
    bwc_group_body<kRhsY, -1, DK, DV, RAB, NW>(ay, job);
}

// ---------------------------------------------------------------------------
// Reverse boundary scan on bf16 MFMAs: the cotangents of the chunk boundary
// states, dS_{j-1} = Acal_j^T dS_j + Qbar_j^T dO_j, from j = N - 1 down, over
// the bf16 MFMA prepare's fragment-ordered operators.  The product needs the
// transpose of the operator's left column block [Acal ; Qbar]: per chunk its
// 16x16 tiles are staged in LDS row-major (from the fragments, which hold
// them row by row) and read with the transposing LDS read.  One workgroup of
// four waves per (batch*head, BV value columns); the cotangent stays in LDS
// as the bf16 B operand, its columns' K index permuted as the forward scan's
// (position 32 b + 8 g + 4 h + e holds row 32 b + 16 h + 4 g + e); the next
// chunk's tiles and dO rows are loaded during the product and staged in the
// other half of a double buffer.
template <int DK, int BV>
struct RsCfg {
  static constexpr int MT = (DK + kCC) / 16;   // operator row (and column) tiles
  static constexpr int KPALL = MT / 2;          // fragment pairs per row tile in memory
  static constexpr int DKT = DK / 16, DP = DK / 32;
  static constexpr int NF = MT * DP;            // fragments staged per chunk
  static constexpr int FPW = NF / 4;
  static constexpr int RPW = DKT / 4;           // output row tiles per wave
  static constexpr int CTN = BV / 16;
  static constexpr int LDX = DK + kCC + 16;     // padded row of X^T
  static constexpr int TBUF = MT * DKT * 256;   // staged tiles (bf16 elements)
  static constexpr int XBUF = BV * LDX;
  static constexpr int MSZ = MT * MT * 256;     // operator elements per chunk
  static constexpr int DITEMS = (kCC / 2) * (BV / 8);   // dO pieces: 2 tokens x 8 columns
  static constexpr int LDS = 2 * (TBUF + XBUF) * 2;
  static_assert(NF % 4 == 0 && DKT % 4 == 0 && DITEMS <= 256, "reverse scan tiling");
};

struct RsArgs {
  Problem p;
  const __bf16* M;
  const __bf16* dout;
  const float* dfinal;
  __bf16* gend;  // [BH, N, dk, dv]: the cotangent of the state leaving each chunk, bf16 (as the scan's products read it)
  float* dS0;    // [BH, dk, dv]
};

__device__ __forceinline__ int rs_kperm(int m) { return (m & ~31) + 8 * ((m >> 2) & 3) + 4 * ((m >> 4) & 1) + (m & 3); }

template <int DK, int BV>
__global__ __launch_bounds__(256) void bw_rscan_kernel(RsArgs a) {
  using Cf = RsCfg<DK, BV>;
  constexpr int FPW = Cf::FPW, RPW = Cf::RPW, CTN = Cf::CTN, LDX = Cf::LDX, DKT = Cf::DKT, DP = Cf::DP;
  extern __shared__ __align__(16) unsigned char smem_[];
  __bf16* Tb = reinterpret_cast<__bf16*>(smem_);
  __bf16* Xb = Tb + 2 * Cf::TBUF;
  const Problem& p = a.p;
  const int dv = p.dv, nvt = dv / BV;
  const int b = blockIdx.x;
  // the value slices of one (batch, head) share blockIdx % 8, hence an XCD and its L2
  const int grp = b / (8 * nvt), rem = b % (8 * nvt);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + rem % 8;
  const int64_t N = p.N;
  if (bh >= p.BH || N == 0) return;
  const int c0 = (rem / 8) * BV;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const __bf16* Mbh = a.M + static_cast<size_t>(bh) * N * Cf::MSZ;
  __bf16* gbh = a.gend + static_cast<size_t>(bh) * N * DK * dv;

  cb8 fr[FPW];
  cb8 dpc[2];
  const int ditem = tid < Cf::DITEMS ? tid : Cf::DITEMS - 1;
  const int dvs = ditem / (BV / 8), dvc = ditem % (BV / 8);   // tokens 2 dvs, 2 dvs + 1; columns 8 dvc ..
  auto chunk_len = [&](int64_t jj) {
    const int64_t r = p.T - jj * kCC;
    return static_cast<int>(r < kCC ? r : kCC);
  };
  auto load_ops = [&](int64_t jj) {
    const __bf16* Mj = Mbh + static_cast<size_t>(jj) * Cf::MSZ;
#pragma unroll
    for (int u = 0; u < FPW; ++u) {
      const int f = wave * FPW + u, mt = f / DP, pp = f % DP;
      fr[u] = *reinterpret_cast<const cb8*>(Mj + ((mt * Cf::KPALL + pp) * 64 + lane) * 8);
    }
  };
  // fragment (mt, pair pp): lane (g, i) holds row i, columns 4 g .. 4 g + 3 of
  // tiles (mt, 2 pp) and (mt, 2 pp + 1)
  auto put_ops = [&](__bf16* T) {
#pragma unroll
    for (int u = 0; u < FPW; ++u) {
      const int f = wave * FPW + u, mt = f / DP, pp = f % DP;
      cb4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = fr[u][e];
        hi[e] = fr[u][4 + e];
      }
      *reinterpret_cast<cb4*>(T + (mt * DKT + 2 * pp) * 256 + lr * 16 + 4 * lg) = lo;
      *reinterpret_cast<cb4*>(T + (mt * DKT + 2 * pp + 1) * 256 + lr * 16 + 4 * lg) = hi;
    }
  };
  auto load_do = [&](int64_t jj) {
    const int n = chunk_len(jj);
    const __bf16* src = a.dout + (static_cast<size_t>(bh) * p.T + jj * kCC) * dv + c0 + 8 * dvc;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int t = 2 * dvs + r;
      if (t < n) {
        dpc[r] = *reinterpret_cast<const cb8*>(src + static_cast<size_t>(t) * dv);
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) dpc[r][u] = (__bf16)0.f;
      }
    }
  };
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 cb2;
  auto put_do = [&](__bf16* X) {
    if (tid < Cf::DITEMS) {
      const int pos = rs_kperm(DK + 2 * dvs);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cb2 w2;
        w2[0] = dpc[0][e];
        w2[1] = dpc[1][e];
        *reinterpret_cast<cb2*>(X + (8 * dvc + e) * LDX + pos) = w2;
      }
    }
  };

  // the cotangent leaving the last chunk: dfinal (or zero)
  for (int it = tid; it < DK * BV; it += 256) {
    const int i = it / BV, c = it % BV;
    const __bf16 g = (__bf16)(a.dfinal ? a.dfinal[(bh * DK + i) * dv + c0 + c] : 0.f);
    gbh[(static_cast<size_t>(N - 1) * DK + i) * dv + c0 + c] = g;
    Xb[c * LDX + rs_kperm(i)] = g;
  }
  load_ops(N - 1);
  put_ops(Tb);
  load_do(N - 1);
  put_do(Xb);
  __syncthreads();
  for (int64_t st = 0; st < N; ++st) {
    const int64_t j = N - 1 - st;
    const int cur = static_cast<int>(st & 1);
    const __bf16* T = Tb + cur * Cf::TBUF;
    const __bf16* X = Xb + cur * Cf::XBUF;
    __bf16* Tn = Tb + (cur ^ 1) * Cf::TBUF;
    __bf16* Xn = Xb + (cur ^ 1) * Cf::XBUF;
    const int64_t jn = j > 0 ? j - 1 : 0;   // the first chunk reloads itself, unused
    load_ops(jn);
    load_do(jn);
    cf4 acc[RPW][CTN];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
      for (int ct = 0; ct < CTN; ++ct) acc[rr][ct] = cz4();
#pragma unroll
    for (int pp = 0; pp < Cf::MT / 2; ++pp) {
      cb8 bx[CTN];
#pragma unroll
      for (int ct = 0; ct < CTN; ++ct) bx[ct] = *reinterpret_cast<const cb8*>(X + (16 * ct + lr) * LDX + 32 * pp + 8 * lg);
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const int kt = wave + 4 * rr;
        const cb8 af = cat8(ltr4(T + (2 * pp * DKT + kt) * 256, 16, 0, 0, lane),
                            ltr4(T + ((2 * pp + 1) * DKT + kt) * 256, 16, 0, 0, lane));
#pragma unroll
        for (int ct = 0; ct < CTN; ++ct) acc[rr][ct] = mfma_b(af, bx[ct], acc[rr][ct]);
      }
    }
    // lane holds rows 16 kt + 4 lg + e (state channels), column 16 ct + lr;
    // the cotangents leaving chunks in bf16 (as the next product reads them),
    // dS0 in fp32
    __bf16* dst = gbh + static_cast<size_t>(j > 0 ? j - 1 : 0) * DK * dv;
    float* d0 = a.dS0 + static_cast<size_t>(bh) * DK * dv;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int kt = wave + 4 * rr;
#pragma unroll
      for (int ct = 0; ct < CTN; ++ct) {
        const int c = 16 * ct + lr;
        const cb4 h = to_b4(acc[rr][ct]);
        if (j > 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[(16 * kt + 4 * lg + e) * dv + c0 + c] = h[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) d0[(16 * kt + 4 * lg + e) * dv + c0 + c] = acc[rr][ct][e];
        }
        *reinterpret_cast<cb4*>(Xn + c * LDX + rs_kperm(16 * kt + 4 * lg)) = h;
      }
    }
    put_ops(Tn);
    put_do(Xn);
    __syncthreads();
  }
}

template <int DK, int BV>
hipError_t launch_rscan_t(const Problem& p, const void* M, const void* dout, const float* dfinal, void* gend,
                          float* dS0, hipStream_t s) {
  using Cf = RsCfg<DK, BV>;
  const void* fn = reinterpret_cast<const void*>(bw_rscan_kernel<DK, BV>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Cf::LDS);
  if (e != hipSuccess) return e;
  const int64_t groups = (p.BH + 7) / 8;
  hipLaunchKernelGGL((bw_rscan_kernel<DK, BV>), dim3(static_cast<unsigned>(groups * 8 * (p.dv / BV))), dim3(256),
                     Cf::LDS, s, RsArgs{p, static_cast<const __bf16*>(M), static_cast<const __bf16*>(dout), dfinal, static_cast<__bf16*>(gend), dS0});
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
template <int DK, int DV, int RAB>
hipError_t launch_bc_t(const Problem& p, const BcBufs& w, const void* q, const void* k, const void* v,
                       const float* ld, const void* A, const void* B, const void* dout, const void* ckpt,
                       const void* gend, float* dq, float* dK, float* dV, float* dld, float* dA,
                       float* dB, hipStream_t s) {
  const int64_t J = p.BH * p.N;
  const unsigned jobs = static_cast<unsigned>(J);
  auto bf = [](const void* x) { return static_cast<const __bf16*>(x); };
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const BcSrc none{nullptr, kSrcChunk};
  auto chunk = [](const void* x) { return BcSrc{x, kSrcChunk}; };
  const BcSrc Vs{v, kSrcSeq}, Os{dout, kSrcSeq}, Sin{ckpt, kSrcState}, GdS{gend, kSrcCotG};
  // one group launch: kinds KA_ (and KB_, sharing the B-side operands)
  // the LDS of a group of kinds KA_ (and KB_, sharing the B-side operands)
  auto group_lds = [&](auto ka_, auto kb_) -> size_t {
    constexpr int KA_ = decltype(ka_)::value, KB_ = decltype(kb_)::value;
    constexpr int NW = BcGroupWaves<KA_, KB_>::template count<DK, DV, RAB>();
    using L = BcStage<KA_, DK, DV, RAB>;
    const size_t stage_b = static_cast<size_t>(L::TOTAL) * 2;
    // the products' copy, and the dQ group's decay-gradient terms beyond it
    const size_t ep_b = static_cast<size_t>(BcGroupWaves<KA_, KB_>::template rows<DK, DV, RAB>()) * (L::NOUT + 4) *
                            sizeof(float) +
                        (KA_ == kDq ? BcEpi<false, DK, RAB, 64 * NW>::EXTRA : 0) +
                        static_cast<size_t>(BcGroupWaves<KA_, KB_>::template wc<RAB>()) * 16 * (DV + 4) * sizeof(float);
    const size_t solve_b = KA_ == kRhsY || KA_ == kRhsX ? static_cast<size_t>(BcSolveCfg<DK, DV, RAB>::LDS) : 0;
    size_t lds = stage_b > ep_b ? stage_b : ep_b;
    return solve_b > lds ? solve_b : lds;
  };
  auto args = [&](BcSrc Aa, BcSrc Ab, BcSrc W0, BcSrc B1, BcSrc C1, BcSrc B2, BcSrc C2, void* outa, void* outb,
                  const void* xr = nullptr, const void* rr = nullptr, void* outc = nullptr) {
    return BcGroupArgs{p, Aa, Ab, W0, B1, C1, B2, C2, w, outa, outb, outc, bf(xr), bf(rr), bf(ckpt), dld};
  };
  // one group launch: kinds KA_ (and KB_), one workgroup per chunk
  auto group = [&](auto ka_, auto kb_, const BcGroupArgs& ga) -> hipError_t {
    constexpr int KA_ = decltype(ka_)::value, KB_ = decltype(kb_)::value;
    constexpr int NW = BcGroupWaves<KA_, KB_>::template count<DK, DV, RAB>();
    const void* fn = reinterpret_cast<const void*>(bwc_group_kernel<KA_, KB_, DK, DV, RAB, NW>);
    const size_t lds = group_lds(ka_, kb_);
    hipError_t e2 = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e2 != hipSuccess) return e2;
    hipLaunchKernelGGL((bwc_group_kernel<KA_, KB_, DK, DV, RAB, NW>), dim3(jobs), dim3(64 * NW), lds, s, ga);
    return hipGetLastError();
  };
  using KN = std::integral_constant<int, -1>;
  if constexpr (RAB > 0) {
    // the forward and the adjoint rank rows: right-hand side, then solve,
    // the two groups of a chunk side by side
    {
      using KY = std::integral_constant<int, kRhsY>;
      using KX = std::integral_constant<int, kRhsX>;
      constexpr int NW = BcGroupWaves<kRhsY, -1>::template count<DK, DV, RAB>();
      static_assert(NW == BcGroupWaves<kRhsX, -1>::template count<DK, DV, RAB>(), "one block size for both");
      const size_t ly = group_lds(KY{}, KN{}), lx = group_lds(KX{}, KN{}), lds = ly > lx ? ly : lx;
      const void* fn = reinterpret_cast<const void*>(bwc_rhs_pair_kernel<DK, DV, RAB, NW>);
      if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds))) != hipSuccess)
        return e;
      hipLaunchKernelGGL((bwc_rhs_pair_kernel<DK, DV, RAB, NW>), dim3((jobs + 7) / 8 * 16), dim3(64 * NW), lds, s,
                         args(chunk(w.bt), none, Sin, chunk(w.kt), Vs, none, none, w.y, nullptr),
                         args(chunk(w.at), none, GdS, chunk(w.qt), Os, none, none, w.x, nullptr));
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // (with dV, whose operands this group stages)
    if ((e = group(std::integral_constant<int, kDk>{}, std::integral_constant<int, kDa>{},
                   args(Vs, chunk(w.y), GdS, Os, chunk(w.qt), chunk(w.x), chunk(w.bt), dK, dA, k, A, dV))) !=
        hipSuccess)
      return e;
    if ((e = group(std::integral_constant<int, kDq>{}, std::integral_constant<int, kDb>{},
                   args(Os, chunk(w.x), Sin, Vs, chunk(w.kt), chunk(w.y), chunk(w.at), dq, dB, q, B))) != hipSuccess)
      return e;
  } else {
    if ((e = group(std::integral_constant<int, kDk>{}, KN{},
                   args(Vs, none, GdS, Os, chunk(w.qt), none, none, dK, nullptr, k, nullptr))) != hipSuccess)
      return e;
    if ((e = group(std::integral_constant<int, kDq>{}, KN{},
                   args(Os, none, Sin, Vs, chunk(w.kt), none, none, dq, nullptr, q, nullptr))) != hipSuccess)
      return e;
  }
  if constexpr (RAB == 0) {
    if ((e = group(std::integral_constant<int, kDv>{}, KN{},
                   args(chunk(w.kt), none, GdS, chunk(w.qt), Os, none, none, dV, nullptr))) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

}  // namespace

bool backward_chunked(const Problem& p) {
  return p.bf16 && p.C == kCC && p.r_kv == 1 && p.r_ab >= 0 && p.r_ab <= 2 && (p.dk == 64 || p.dk == 128) &&
         (p.dv == 64 || p.dv == 128);
}

size_t backward_chunked_bytes(const Problem& p, bool own_ops) {
  const PrepBwOut none{};
  return bc_layout(p, nullptr, nullptr, own_ops ? nullptr : &none);
}

PrepBwOut backward_chunked_prep_out(const Problem& p, void* ws) {
  BcBufs w;
  bc_layout(p, static_cast<char*>(ws), &w);
  return PrepBwOut{w.qt, w.kt, w.at, w.bt, w.lt, w.di, w.gc, w.gam};
}

size_t backward_chunked_ops_bytes(const Problem& p) { return bc_ops_layout(p, nullptr, nullptr); }

PrepBwOut backward_chunked_ops_at(const Problem& p, void* base) {
  PrepBwOut o{};
  bc_ops_layout(p, static_cast<char*>(base), &o);
  return o;
}

hipError_t launch_backward_rscan(const Problem& p, const void* M, const void* dout, const float* dfinal, void* gend,
                                 float* dS0, hipStream_t s) {
  if (p.BH * p.N == 0) return hipSuccess;
  if (!backward_chunked(p)) return hipErrorInvalidValue;
  // 64 value columns per workgroup where that still gives >= 256 workgroups
  const bool wide = p.BH * (p.dv / 64) >= 256;
  if (p.dk == 128) return wide ? launch_rscan_t<128, 64>(p, M, dout, dfinal, gend, dS0, s)
                               : launch_rscan_t<128, 32>(p, M, dout, dfinal, gend, dS0, s);
  if (p.dk == 64) return wide ? launch_rscan_t<64, 64>(p, M, dout, dfinal, gend, dS0, s)
                              : launch_rscan_t<64, 32>(p, M, dout, dfinal, gend, dS0, s);
  return hipErrorInvalidValue;
}

hipError_t launch_backward_chunked(const Problem& p, const void* q, const void* k, const void* v, const float* ld,
                                   const void* A, const void* B, const void* dout, const void* ckpt,
                                   const void* gend, float* dq, float* dK, float* dV, float* dld,
                                   float* dA, float* dB, void* ws, hipStream_t s, const PrepBwOut* ops) {
  if (p.BH * p.N == 0) return hipSuccess;
  if (!backward_chunked(p)) return hipErrorInvalidValue;
  BcBufs w;
  bc_layout(p, static_cast<char*>(ws), &w, ops);
#define LATTN_BC(DK_, DV_, RAB_)                                                                                  \
  if (p.dk == DK_ && p.dv == DV_ && p.r_ab == RAB_)                                                              \
    return launch_bc_t<DK_, DV_, RAB_>(p, w, q, k, v, ld, A, B, dout, ckpt, gend, dq, dK, dV, dld, dA, dB, s);
  LATTN_BC(128, 128, 2) LATTN_BC(128, 128, 1) LATTN_BC(128, 128, 0)
  LATTN_BC(64, 64, 2) LATTN_BC(64, 64, 1) LATTN_BC(64, 64, 0)
  LATTN_BC(128, 64, 2) LATTN_BC(128, 64, 1) LATTN_BC(128, 64, 0)
  LATTN_BC(64, 128, 2) LATTN_BC(64, 128, 1) LATTN_BC(64, 128, 0)
#undef LATTN_BC
  return hipErrorInvalidValue;
}

}  // namespace lattn
