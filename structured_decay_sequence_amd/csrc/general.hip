// General chunk-wise path: any shape the ABI accepts, fp32 arithmetic throughout.
//
// Per chunk (HDLA note, "Key design 3": rank-generalized WY form; HLA note,
// "Affine maps and closure under composition"), with G the chunk-local
// inclusive cumulative log-decay and rows stacked token-major, rank-minor:
//   Bt = B (.) exp(G_{t-1}),  At = A (.) exp(-G_t),  Kt = K (.) exp(-G_t),  Qt = q (.) exp(G_t)
//   L  = Bt At^T, LK = Bt Kt^T        (token(row) >  token(col))
//   MA = Qt At^T, MK = Qt Kt^T        (token(row) >= token(col))
//   [W X] = (I + L)^{-1} [Bt LK]      (unit lower-triangular solve)
//   Acal = diag(exp(G_C)) (I - At^T W),   Z = diag(exp(G_C)) (Kt^T - At^T X)
//   Qbar = Qt - MA W,                     R = MK - MA X
// and the chunk operator M_j = [[Acal, Z], [Qbar, R]] advances the state and
// produces the chunk's outputs in one product:
//   [S_j ; O_j] = M_j [S_{j-1} ; V_j].
// The prepare kernel forms M_j for every chunk in parallel; the scan kernel
// walks the chunks of one (batch, head, d_v slice) in order.
//
// Every product is a wave-level 16x16 tile on the fp32 matrix cores
// (tile_f32.hpp), so the path keeps fp32 operands and fp32 accumulation.
//
// The prepare kernel's operands live in a per-workgroup slot of the
// workspace (row-major fp32); M_j is stored row-major fp32.
#include "common.hpp"
#include "kernels.hpp"
#include "tile_f32.hpp"


namespace lattn {
namespace {

constexpr int kThreads = 256;        // scan and summaries: four waves
constexpr int kWaves = kThreads / 64;
constexpr int kPrepThreads = 512;    // prepare: eight waves (two per SIMD at 256 VGPRs)
constexpr int kPrepWaves = kPrepThreads / 64;

// Offsets (floats) of the prepare kernel's per-slot arrays, all row-major.
struct SlotLayout {
  size_t G, Bt, At, AtT, Kt, KtT, Qt, L, LK, MA, MK, total;
  __host__ __device__ explicit SlotLayout(const Problem& p) {
    const size_t C = p.C, dk = p.dk, na = p.na(), nk = p.nk();
    size_t o = 0;
    G = o;   o += C * dk;     // chunk-local inclusive cumulative log-decay
    Bt = o;  o += na * dk;    // B (.) exp(G_{t-1})
    At = o;  o += na * dk;    // A (.) exp(-G_t)
    AtT = o; o += dk * na;    // At transposed
    Kt = o;  o += nk * dk;    // K (.) exp(-G_t)
    KtT = o; o += dk * nk;    // Kt transposed
    Qt = o;  o += C * dk;     // q (.) exp(G_t)
    L = o;   o += na * na;    // Bt At^T, token(row) > token(col); lower 16x16 blocks only
    LK = o;  o += na * nk;    // Bt Kt^T, token(row) > token(col)
    MA = o;  o += C * na;     // Qt At^T, token(row) >= token(col)
    MK = o;  o += C * nk;     // Qt Kt^T, token(row) >= token(col)
    total = (o + 63) & ~static_cast<size_t>(63);
  }
};

constexpr int kMaxNB = 32;   // 16-row blocks of the solve: chunk * r_ab <= 512
constexpr int kDIB = 260;    // floats per stored 16x16 inverse (padded)

struct PrepArgs {
  Problem p;
  const void* q;
  const void* k;
  const float* ld;
  const void* A;
  const void* B;
  float* M;
  float* scratch;
  size_t slot_floats;
};

// NBMAX: 16-row solve blocks covered (chunk * r_ab <= 16 * NBMAX); NCT: column
// tiles a wave solves at once (NCT * NBMAX tiles per lane stay in registers).
template <typename TI, int NBMAX, int NCT>
__global__ __launch_bounds__(kPrepThreads) void general_prepare_kernel(PrepArgs a) {
  __shared__ __align__(16) float Dinv[kMaxNB * kDIB];   // (I + L_ii)^{-1}, fp32
  __shared__ float eGC[256];                             // exp(G_C) per channel
  const Problem& p = a.p;
  const int dk = p.dk, C = p.C, r_ab = p.r_ab, r_kv = p.r_kv;
  const int na = p.na(), nk = p.nk(), ncol = p.mcols();
  const int nbA = na / 16, dkT = dk / 16;
  const int MT = p.mrows() / 16, KTc = ncol / 16;
  const int RT = (na + C) / 16, CTg = (na + nk) / 16;   // tile rows / columns of the Gram matrix
  const int SR = (RT + 3) / 4, SC = (CTg + 3) / 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const SlotLayout S(p);
  float* slot = a.scratch + static_cast<size_t>(blockIdx.x) * a.slot_floats;
  float* G = slot + S.G;
  float* Bt = slot + S.Bt;
  float* At = slot + S.At;
  float* AtT = slot + S.AtT;
  float* Kt = slot + S.Kt;
  float* KtT = slot + S.KtT;
  float* Qt = slot + S.Qt;
  float* L = slot + S.L;
  float* LK = slot + S.LK;
  float* MA = slot + S.MA;
  float* MK = slot + S.MK;
  const TI* q = static_cast<const TI*>(a.q);
  const TI* kp = static_cast<const TI*>(a.k);
  const TI* Ap = static_cast<const TI*>(a.A);
  const TI* Bp = static_cast<const TI*>(a.B);
  const int64_t total = p.BH * p.N;

  for (int64_t job = blockIdx.x; job < total; job += gridDim.x) {
    const int64_t bh = job / p.N;
    const int64_t j = job % p.N;
    const int64_t t0 = j * C;
    const int n = static_cast<int>(p.T - t0 < C ? p.T - t0 : C);
    const int64_t tok0 = bh * p.T + t0;

    // 1. chunk-local inclusive cumulative log-decay; padded tokens decay by 0.
    for (int i = tid; i < dk; i += kPrepThreads) {
      float g = 0.f;
      // unrolled so that the loads of 16 tokens are in flight together
#pragma unroll 16
      for (int t = 0; t < C; ++t) {
        float l = 0.f;
        if (t < n) l = p.scalar ? a.ld[tok0 + t] : a.ld[(tok0 + t) * dk + i];
        g += l;
        G[t * dk + i] = g;
      }
      eGC[i] = expf(g);
    }
    __syncthreads();

    // 2. decay-scaled operands (zero rows for padded tokens), with the
    //    transposed copies that the operator product reads as row operands.
#pragma unroll 4
    for (int e = tid; e < na * dk; e += kPrepThreads) {
      const int s = e / dk, i = e % dk, t = s / r_ab;
      float bv = 0.f, av = 0.f;
      if (t < n) {
        const size_t idx = (static_cast<size_t>(tok0 + t) * r_ab + (s % r_ab)) * dk + i;
        bv = Elem<TI>::load(Bp, idx) * (t > 0 ? expf(G[(t - 1) * dk + i]) : 1.f);
        av = Elem<TI>::load(Ap, idx) * expf(-G[t * dk + i]);
      }
      Bt[e] = bv;
      At[e] = av;
      AtT[static_cast<size_t>(i) * na + s] = av;
    }
#pragma unroll 4
    for (int e = tid; e < nk * dk; e += kPrepThreads) {
      const int s = e / dk, i = e % dk, t = s / r_kv;
      float kv = 0.f;
      if (t < n)
        kv = Elem<TI>::load(kp, (static_cast<size_t>(tok0 + t) * r_kv + (s % r_kv)) * dk + i) * expf(-G[t * dk + i]);
      Kt[e] = kv;
      KtT[static_cast<size_t>(i) * nk + s] = kv;
    }
#pragma unroll 4
    for (int e = tid; e < C * dk; e += kPrepThreads) {
      const int t = e / dk, i = e % dk;
      float qv = 0.f;
      if (q != nullptr && t < n) qv = Elem<TI>::load(q, static_cast<size_t>(tok0 + t) * dk + i) * expf(G[e]);
      Qt[e] = qv;
    }
    __syncthreads();

    // 3. masked Gram tiles of [Bt ; Qt] [At ; Kt]^T: L (lower blocks, diagonal
    //    included), L_K, M_A, M_K.  Each wave takes 4x4 groups of 16x16 tiles,
    //    so every operand fragment it loads feeds four products.
    for (int st = wave; st < SR * SC; st += kPrepWaves) {
      const int rt0 = 4 * (st / SC), ct0 = 4 * (st % SC);
      // a group wholly above the diagonal of L is never read
      if (rt0 + 3 < nbA && ct0 + 3 < nbA && ct0 > rt0 + 3) continue;
      const float* lp[4];
      const float* rp[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rt = rt0 + u < RT ? rt0 + u : RT - 1, ctl = ct0 + u < CTg ? ct0 + u : CTg - 1;
        const int row = rt * 16 + lr, col = ctl * 16 + lr;
        lp[u] = (row < na ? Bt + static_cast<size_t>(row) * dk : Qt + static_cast<size_t>(row - na) * dk) + 4 * lg;
        rp[u] = (col < na ? At + static_cast<size_t>(col) * dk : Kt + static_cast<size_t>(col - na) * dk) + 4 * lg;
      }
      f32x4 acc[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = zero4();
#pragma unroll 4
      for (int kk = 0; kk < dk; kk += 16) {
        f32x4 fa[4], fb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          fa[u] = ld4(lp[u] + kk);
          fb[u] = ld4(rp[u] + kk);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] = mfma16(fa[u], fb[v], acc[u][v]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int rt = rt0 + u, ctl = ct0 + v;
          if (rt >= RT || ctl >= CTg) continue;
          const bool drow = rt < nbA, dcol = ctl < nbA;   // decay rows / decay columns
          if (drow && dcol && ctl > rt) continue;         // upper blocks of L: never read
          // Token of a row or column: decay rows and columns carry r_ab per
          // token, write columns r_kv, query rows one.  L and L_K keep
          // token(row) > token(col); M_A and M_K keep token(row) >= token(col).
          const int rdiv = drow ? r_ab : 1, cdiv = dcol ? r_ab : r_kv;
          const int r0 = drow ? rt * 16 : rt * 16 - na;
          const int c = (dcol ? ctl * 16 : ctl * 16 - na) + lr;
          const int ctok = c / cdiv;
          float* dst;
          int ldd;
          if (drow) {
            dst = dcol ? L : LK;
            ldd = dcol ? na : nk;
          } else {
            dst = dcol ? MA : MK;
            ldd = dcol ? na : nk;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = r0 + 4 * lg + e, rtok = r / rdiv;
            const bool keep = drow ? rtok > ctok : rtok >= ctok;
            dst[static_cast<size_t>(r) * ldd + c] = keep ? acc[u][v][e] : 0.f;
          }
        }
      }
    }
    __syncthreads();

    // 4. inverses of the unit lower-triangular diagonal blocks (I + L_ii), fp32:
    //    thread (blk, c) forms column c by forward substitution.
    for (int it = tid; it < na; it += kPrepThreads) {
      const int blk = it / 16, c = it % 16;
      const float* Lb = L + static_cast<size_t>(blk * 16) * na + blk * 16;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = (r == c) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) v -= Lb[static_cast<size_t>(r) * na + m] * x[m];
        x[r] = v;
        Dinv[blk * kDIB + r * 16 + c] = v;
      }
    }
    __syncthreads();

    // 5. blocked forward substitution, per wave NCT 16-column tiles of
    //    [Bt | LK] at a time:  WX_i = (I + L_ii)^{-1} (RHS_i - sum_{j<i} L_ij WX_j),
    //    with the WX tiles kept in registers (accumulator layout, which is the
    //    right-operand layout of the next product) and each L fragment feeding
    //    all NCT tiles.
    // 6. then, from the same registers, the chunk operator's columns:
    //    rows of channels  base - At^T WX, base I | Kt^T, scaled by exp(G_C);
    //    rows of tokens    base - M_A WX,  base Qt | M_K.
    float* Mo = a.M + static_cast<size_t>(job) * p.mrows() * ncol;
    for (int ct0 = NCT * wave; ct0 < KTc; ct0 += NCT * kPrepWaves) {
      f32x4 wx[NCT][NBMAX];
#pragma unroll
      for (int i = 0; i < NBMAX; ++i) {
#pragma unroll
        for (int h = 0; h < NCT; ++h) wx[h][i] = zero4();
      }
#pragma unroll
      for (int i = 0; i < NBMAX; ++i) {
        if (i < nbA) {
          f32x4 sm[NCT];
#pragma unroll
          for (int h = 0; h < NCT; ++h) sm[h] = zero4();
          const float* lrow = L + static_cast<size_t>(i * 16 + lr) * na + 4 * lg;
#pragma unroll
          for (int jb = 0; jb < i; ++jb) {
            const f32x4 la = ld4(lrow + jb * 16);
#pragma unroll
            for (int h = 0; h < NCT; ++h) sm[h] = mfma16(la, wx[h][jb], sm[h]);
          }
          const f32x4 dA = ld4(Dinv + i * kDIB + lr * 16 + 4 * lg);
#pragma unroll
          for (int h = 0; h < NCT; ++h) {
            const int ct = ct0 + h < KTc ? ct0 + h : ct0;   // a missing last tile repeats the first
            f32x4 r4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = i * 16 + 4 * lg + e;
              const float rhs = ct < dkT ? Bt[static_cast<size_t>(r) * dk + ct * 16 + lr]
                                         : LK[static_cast<size_t>(r) * nk + (ct - dkT) * 16 + lr];
              r4[e] = rhs - sm[h][e];
            }
            wx[h][i] = mfma16(dA, r4, zero4());
          }
        }
      }
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc[NCT];
#pragma unroll
        for (int h = 0; h < NCT; ++h) acc[h] = zero4();
        const float* arow = (mt < dkT ? AtT + static_cast<size_t>(mt * 16 + lr) * na
                                      : MA + static_cast<size_t>((mt - dkT) * 16 + lr) * na) + 4 * lg;
        // No guard on kb, so that all the loads can be issued ahead: slices
        // past chunk * r_ab read a valid fragment and meet a zero WX tile.
        if (nbA > 0) {
#pragma unroll
          for (int kb = 0; kb < NBMAX; ++kb) {
            const f32x4 fa = ld4(arow + (kb < nbA ? kb : 0) * 16);
#pragma unroll
            for (int h = 0; h < NCT; ++h) acc[h] = mfma16(fa, wx[h][kb], acc[h]);
          }
        }
#pragma unroll
        for (int h = 0; h < NCT; ++h) {
          if (ct0 + h >= KTc) break;
          const int c = (ct0 + h) * 16 + lr;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = mt * 16 + 4 * lg + e;
            float v;
            if (mt < dkT) {
              const float base = c < dk ? (r == c ? 1.f : 0.f) : KtT[static_cast<size_t>(r) * nk + (c - dk)];
              v = eGC[r] * (base - acc[h][e]);
            } else {
              const int t = r - dk;
              const float base = c < dk ? Qt[static_cast<size_t>(t) * dk + c] : MK[static_cast<size_t>(t) * nk + (c - dk)];
              v = base - acc[h][e];
            }
            Mo[static_cast<size_t>(r) * ncol + c] = v;
          }
        }
      }
    }
    __syncthreads();
  }
}

struct ScanArgs {
  Problem p;
  const float* M;
  const void* v;
  void* out;
  float* Sfin;
  const float* S0;
};

constexpr int kBV = 16;   // d_v columns per scan workgroup
constexpr int kVMAX = 4;  // V values per thread prefetched into registers

// Scan: one workgroup per (batch*head, 16-column d_v slice); chunks in order.
// Per chunk one product Y = M_j X with X = [S ; V_j] kept in LDS as X^T
// (column-major in k, so each lane's 4 permuted K values are one 16-byte
// read), double-buffered so that one barrier per chunk orders the state
// write against the next product.  Wave w takes output row tiles w, w + nw,
// ... (QW of them).  The operator is read from HBM in batches of KB K slices
// held in registers; the next batch (the next chunk's first, at the end of a
// chunk) is issued as soon as the current one has been multiplied, since the
// operator does not depend on the state.  V of the next chunk is loaded into
// registers before the product and written to LDS after it.
template <typename TI, int QW, int KB>
__global__ __launch_bounds__(768) void general_scan_kernel(ScanArgs a) {
  extern __shared__ __align__(16) float xs[];
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv, C = p.C, r_kv = p.r_kv, nk = p.nk(), ncol = p.mcols();
  const int MT = p.mrows() / 16, KTc = ncol / 16, dkT = dk / 16;
  const int LDX = ncol + 4;
  const int nvt = dv / kBV;
  const int nthr = blockDim.x, nw = nthr / 64;
  const int64_t N = p.N;
  // Slices of one (batch, head) get block ids that land on one XCD
  // (consecutive ids go round-robin over the 8 XCDs), so they share its L2.
  const int b = blockIdx.x;
  const int grp = b / (8 * nvt), rem = b % (8 * nvt);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + rem % 8;
  const int c0 = (rem / 8) * kBV;
  if (bh >= p.BH) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const TI* vp = static_cast<const TI*>(a.v);
  TI* op = static_cast<TI*>(a.out);
  float* X0 = xs;
  float* X1 = xs + kBV * LDX;

  // V_jj: item e is (write row s = e / kBV, column e % kBV); zero past the chunk's end.
  auto v_at = [&](int64_t jj, int e) {
    const int64_t t0 = jj * C;
    const int n = static_cast<int>(p.T - t0 < C ? p.T - t0 : C);
    const int s = e / kBV, c = e % kBV, t = s / r_kv;
    return t < n ? Elem<TI>::load(vp, (static_cast<size_t>(bh * p.T + t0 + t) * r_kv + (s % r_kv)) * dv + c0 + c) : 0.f;
  };
  float vr[kVMAX];
  auto load_v = [&](int64_t jj) {
#pragma unroll
    for (int q = 0; q < kVMAX; ++q) {
      const int e = tid + q * nthr;
      vr[q] = e < nk * kBV ? v_at(jj, e) : 0.f;
    }
  };
  auto store_v = [&](float* X, int64_t jj) {
#pragma unroll
    for (int q = 0; q < kVMAX; ++q) {
      const int e = tid + q * nthr;
      if (e < nk * kBV) X[(e % kBV) * LDX + dk + e / kBV] = vr[q];
    }
    // shapes with more values than the register copy holds
    for (int e = tid + kVMAX * nthr; e < nk * kBV; e += nthr) X[(e % kBV) * LDX + dk + e / kBV] = v_at(jj, e);
  };
  // Operator fragments of K slices kb0 .. kb0 + KB - 1 of chunk jj; only the
  // (row tile, slice) pairs the products use are loaded.
  f32x4 fa[QW][KB];
  auto load_batch = [&](int64_t jj, int kb0) {
    jj = jj < N ? jj : N - 1;
    const float* Mj = a.M + static_cast<size_t>(bh * N + jj) * p.mrows() * ncol + 4 * lg;
#pragma unroll
    for (int u = 0; u < QW; ++u) {
      const int mt = wave + nw * u;
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const int kb = kb0 + i;
        fa[u][i] = mt < MT && kb < KTc ? ld4(Mj + static_cast<size_t>(mt * 16 + lr) * ncol + kb * 16) : zero4();
      }
    }
  };
  for (int e = tid; e < dk * kBV; e += nthr) {
    const int i = e / kBV, c = e % kBV;
    X0[c * LDX + i] = a.S0 ? a.S0[(bh * dk + i) * dv + c0 + c] : 0.f;
  }
  if (N > 0) {
    load_v(0);
    store_v(X0, 0);
    load_batch(0, 0);
  }
  __syncthreads();

  for (int64_t jj = 0; jj < N; ++jj) {
    const float* X = (jj & 1) ? X1 : X0;
    float* Xn = (jj & 1) ? X0 : X1;
    const int64_t t0 = jj * C;
    const int n = static_cast<int>(p.T - t0 < C ? p.T - t0 : C);
    if (jj + 1 < N) load_v(jj + 1);
    f32x4 acc[QW];
#pragma unroll
    for (int u = 0; u < QW; ++u) acc[u] = zero4();
    const float* xcol = X + lr * LDX + 4 * lg;
    for (int kb0 = 0; kb0 < KTc; kb0 += KB) {
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        if (kb0 + i < KTc) {
          const f32x4 bx = ld4(xcol + (kb0 + i) * 16);
#pragma unroll
          for (int u = 0; u < QW; ++u)
            if (wave + nw * u < MT) acc[u] = mfma16(fa[u][i], bx, acc[u]);
        }
      }
      if (kb0 + KB < KTc) {
        load_batch(jj, kb0 + KB);
      } else {
        load_batch(jj + 1, 0);
      }
    }
    const bool last = jj == N - 1;
#pragma unroll
    for (int u = 0; u < QW; ++u) {
      const int mt = wave + nw * u;
      if (mt >= MT) break;
      if (mt < dkT) {
        // state rows 4lg.. of column lr: one 16-byte write of X^T
        st4(Xn + lr * LDX + mt * 16 + 4 * lg, acc[u]);
        if (last && a.Sfin) {
#pragma unroll
          for (int e = 0; e < 4; ++e) a.Sfin[(bh * dk + mt * 16 + 4 * lg + e) * dv + c0 + lr] = acc[u][e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = (mt - dkT) * 16 + 4 * lg + e;
          if (t < n) Elem<TI>::store(op, static_cast<size_t>(bh * p.T + t0 + t) * dv + c0 + lr, acc[u][e]);
        }
      }
    }
    if (jj + 1 < N) store_v(Xn, jj + 1);
    __syncthreads();
  }
  if (N == 0 && a.Sfin) {
    for (int e = tid; e < dk * kBV; e += nthr) {
      const int i = e / kBV, c = e % kBV;
      a.Sfin[(bh * dk + i) * dv + c0 + c] = X0[c * LDX + i];
    }
  }
}

struct SumArgs {
  Problem p;
  const float* M;
  const void* v;
  float* sumA;
  float* sumB;
};

// sum_A[j] = Acal_j, sum_B[j] = Z_j V_j; one workgroup per chunk.
template <typename TI>
__global__ __launch_bounds__(kThreads) void general_summaries_kernel(SumArgs a) {
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv, C = p.C, r_kv = p.r_kv, nk = p.nk(), ncol = p.mcols();
  const int64_t job = blockIdx.x;
  const int64_t bh = job / p.N, j = job % p.N;
  const int64_t t0 = j * C;
  const int n = static_cast<int>(p.T - t0 < C ? p.T - t0 : C);
  const int64_t tok0 = bh * p.T + t0;
  const float* Mj = a.M + static_cast<size_t>(job) * p.mrows() * ncol;
  const TI* vp = static_cast<const TI*>(a.v);
  for (int e = threadIdx.x; e < dk * dk; e += kThreads) {
    const int i = e / dk, c = e % dk;
    a.sumA[static_cast<size_t>(job) * dk * dk + e] = Mj[static_cast<size_t>(i) * ncol + c];
  }
  for (int e = threadIdx.x; e < dk * dv; e += kThreads) {
    const int i = e / dv, c = e % dv;
    float s = 0.f;
    for (int m = 0; m < nk; ++m) {
      const int t = m / r_kv;
      if (t < n)
        s += Mj[static_cast<size_t>(i) * ncol + dk + m] *
             Elem<TI>::load(vp, (static_cast<size_t>(tok0 + t) * r_kv + (m % r_kv)) * dv + c);
    }
    a.sumB[static_cast<size_t>(job) * dk * dv + e] = s;
  }
}

}  // namespace

GeneralPlan general_plan(const Problem& p) {
  GeneralPlan g{};
  g.slot_floats = SlotLayout(p).total;
  // One resident prepare workgroup per compute unit, each with its own slot.
  const int64_t jobs = p.BH * p.N;
  g.slots = static_cast<int>(jobs < 256 ? (jobs > 0 ? jobs : 1) : 256);
  g.m_bytes = static_cast<size_t>(jobs) * p.mrows() * p.mcols() * sizeof(float);
  g.m_bytes = (g.m_bytes + 255) & ~static_cast<size_t>(255);
  g.total_bytes = g.m_bytes + static_cast<size_t>(g.slots) * g.slot_floats * sizeof(float);
  return g;
}

template <typename TI, int NBMAX, int NCT>
void launch_prepare(const GeneralPlan& g, const PrepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((general_prepare_kernel<TI, NBMAX, NCT>), dim3(g.slots), dim3(kPrepThreads), 0, s, a);
}

template <typename TI>
void launch_prepare(const GeneralPlan& g, const PrepArgs& a, hipStream_t s) {
  // The solve keeps NCT x NBMAX tiles per lane in registers: the smallest
  // instantiation that covers chunk * r_ab.
  const int nb = a.p.na() / 16;
  if (nb <= 8) {
    launch_prepare<TI, 8, 2>(g, a, s);
  } else if (nb <= 16) {
    launch_prepare<TI, 16, 1>(g, a, s);
  } else {
    launch_prepare<TI, kMaxNB, 1>(g, a, s);
  }
}

hipError_t general_prepare(const Problem& p, const void* q, const void* k, const float* ld,
                           const void* A, const void* B, void* workspace, hipStream_t s) {
  const GeneralPlan g = general_plan(p);
  PrepArgs a{p, q, k, ld, A, B, static_cast<float*>(workspace),
             reinterpret_cast<float*>(static_cast<char*>(workspace) + g.m_bytes), g.slot_floats};
  if (p.BH * p.N == 0) return hipSuccess;
  if (p.na() > 16 * kMaxNB) return hipErrorInvalidValue;
  if (p.bf16)
    launch_prepare<bf16_raw>(g, a, s);
  else
    launch_prepare<float>(g, a, s);
  return hipGetLastError();
}

template <typename TI, int QW, int KB>
hipError_t launch_scan(const Problem& p, const ScanArgs& a, size_t lds, int64_t blocks, hipStream_t s) {
  // Dynamic LDS above 64 KiB must be opted into per kernel.
  const void* fn = reinterpret_cast<const void*>(general_scan_kernel<TI, QW, KB>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  // One wave per QW output row tiles: (d_k + C) / 16 <= 24 tiles, at most 12 waves.
  const int mt = p.mrows() / 16;
  const int nw = (mt + QW - 1) / QW;
  hipLaunchKernelGGL((general_scan_kernel<TI, QW, KB>), dim3(blocks), dim3(64 * nw), lds, s, a);
  return hipGetLastError();
}

template <typename TI>
hipError_t launch_scan(const Problem& p, const ScanArgs& a, size_t lds, int64_t blocks, hipStream_t s) {
  // Up to 12 row tiles: one per wave, a whole chunk's operator per load batch
  // (K slices <= 32: two batches); more: two per wave, half-size batches.
  return p.mrows() / 16 <= 12 ? launch_scan<TI, 1, 16>(p, a, lds, blocks, s) : launch_scan<TI, 2, 8>(p, a, lds, blocks, s);
}

hipError_t general_scan(const Problem& p, const void* workspace, const void* v, void* out,
                        float* Sfin, const float* S0, hipStream_t s) {
  ScanArgs a{p, static_cast<const float*>(workspace), v, out, Sfin, S0};
  const size_t lds = static_cast<size_t>(2 * kBV) * (p.mcols() + 4) * sizeof(float);
  const int64_t nvt = p.dv / kBV;
  const int64_t blocks = (p.BH + 7) / 8 * 8 * nvt;
  if (p.BH == 0) return hipSuccess;
  return p.bf16 ? launch_scan<bf16_raw>(p, a, lds, blocks, s) : launch_scan<float>(p, a, lds, blocks, s);
}

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;

// The bf16 path's chunk operators expanded to row-major fp32 ((d_k + C) x
// (d_k + C) per chunk-head).  The bf16 path stores every pair of 16x16 tiles
// (mt, 2kp), (mt, 2kp + 1) as 64 lanes x 8 values: lane l holds row l % 16,
// columns 4(l / 16) .. +3 of the first tile, then the same of the second.
// One thread per lane piece.
__global__ __launch_bounds__(256) void operator_bf16_to_f32_kernel(const __bf16* Mb, float* Mf, int MT, int KT,
                                                                   int64_t pieces) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= pieces) return;
  const int lane = static_cast<int>(i % 64);
  const int64_t pr = i / 64;   // (chunk-head, mt, kp)
  const int KP = KT / 2;
  const int kp = static_cast<int>(pr % KP);
  const int mt = static_cast<int>((pr / KP) % MT);
  const int64_t job = pr / (static_cast<int64_t>(KP) * MT);
  const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(Mb + i * 8);
  const int ncol = KT * 16;
  float* row = Mf + (static_cast<size_t>(job) * MT * 16 + mt * 16 + (lane & 15)) * ncol + 4 * (lane >> 4);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x4 w = f32x4{(float)v[4 * h], (float)v[4 * h + 1], (float)v[4 * h + 2], (float)v[4 * h + 3]};
    st4(row + (2 * kp + h) * 16, w);
  }
}

}  // namespace

size_t f32_operators_bytes(const Problem& p) {
  if (p.bf16 && fast_supported(p)) {
    const size_t fb = (fast_workspace_bytes(p) + 255) & ~static_cast<size_t>(255);
    return fb + static_cast<size_t>(p.BH * p.N) * p.mrows() * p.mcols() * sizeof(float);
  }
  return general_plan(p).total_bytes;
}

hipError_t f32_operators(const Problem& p, const void* q, const void* k, const float* ld, const void* A,
                         const void* B, void* workspace, const float** M, hipStream_t s) {
  if (p.bf16 && fast_supported(p)) {
    const size_t fb = (fast_workspace_bytes(p) + 255) & ~static_cast<size_t>(255);
    float* Mf = reinterpret_cast<float*>(static_cast<char*>(workspace) + fb);
    *M = Mf;
    hipError_t e = fast_prepare(p, q, k, ld, A, B, workspace, s);
    if (e != hipSuccess) return e;
    const int MT = p.mrows() / 16, KT = p.mcols() / 16;
    const int64_t pieces = p.BH * p.N * MT * (KT / 2) * 64;
    hipLaunchKernelGGL(operator_bf16_to_f32_kernel, dim3(static_cast<unsigned>((pieces + 255) / 256)), dim3(256), 0,
                       s, static_cast<const __bf16*>(workspace), Mf, MT, KT, pieces);
    return hipGetLastError();
  }
  *M = static_cast<const float*>(workspace);   // the general prepare stores them at the front
  return general_prepare(p, q, k, ld, A, B, workspace, s);
}

hipError_t general_summaries(const Problem& p, const void* workspace, const void* v, float* sumA,
                             float* sumB, hipStream_t s) {
  SumArgs a{p, static_cast<const float*>(workspace), v, sumA, sumB};
  const int64_t blocks = p.BH * p.N;
  if (blocks == 0) return hipSuccess;
  if (p.bf16)
    hipLaunchKernelGGL(general_summaries_kernel<bf16_raw>, dim3(blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(general_summaries_kernel<float>, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace lattn
