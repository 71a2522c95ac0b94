// Backward pass of the recurrence (the chain rule of the HDLA note's "Key
// design 3" token recurrence, in reverse; the pages print no backward
// formulas):
//   forward   P_t = D_t - A_t B_t^T,  S_t = P_t S_{t-1} + K_t V_t^T,  o_t = S_t^T q_t
//   backward  G <- dS_T;  for t = T-1 .. 0:
//               G += q_t do_t^T;  dq_t = S_t do_t;  dK_t = G V_t;  dV_t = G^T K_t
//               with dP_t = G S_{t-1}^T:  dA_t = -dP_t B_t,  dB_t = -dP_t^T A_t,
//               dlog_decay_t = diag(dP_t) (.) exp(log_decay_t)
//               G <- P_t^T G
//             dS_init = G
// Everything is expressed with matrix-vector products over the state, so dP_t
// (d_k x d_k) is never formed: dA_t = -G (S_{t-1}^T B_t), dB_t = -S_{t-1} (G^T A_t),
// and diag(dP_t) is the row-wise dot of G and S_{t-1}.
//
// Chunk-parallel schedule.  The forward's chunk operators
// M_j = [[Acal_j, Z_j], [Qbar_j, R_j]] (row-major fp32, from the prepare kernels)
// give every chunk boundary without a token walk:
//   states      S_j     = Acal_j S_{j-1} + Z_j V_j             (j = 0 .. N-1)
//   cotangents  dS_{j-1} = Acal_j^T dS_j + Qbar_j^T dO_j        (j = N-1 .. 0)
// one scan each (bw_bound_kernel, fp32 FMAs, one workgroup per (batch, head,
// 32 value columns); the d_v columns of the state are independent).  With the
// state entering chunk j and the cotangent leaving it known, the token-level
// walks of all chunks are independent: backward_kernel takes (batch, head,
// chunk) jobs.  Per job, one 512-thread workgroup (a 32 x 16 grid; thread
// (tr, tc) holds rows tr, tr+32, .. and columns tc, tc+16, .. of S_t, S_{t-1}
// and G in registers) recomputes the chunk's states into its workspace buffer
// (each thread reads back only the values it wrote, stored contiguously per
// thread) and walks the chunk's tokens in reverse.  Sums over columns are
// shuffles inside a row group of 16 lanes; sums over rows are shuffles inside
// the wave, then an LDS exchange between the eight waves (each sum formed
// once, then read back by the threads of its column).
#include "common.hpp"
#include "kernels.hpp"

namespace lattn {
namespace {

constexpr int kBwThreads = 512;
constexpr int kNTR = 32, kNTC = 16;      // thread grid: row groups x column groups
constexpr int kRB = 4, kCB = 8;          // rows / columns per thread: d_k, d_v <= 128
constexpr int kRabMax = 4, kRkvMax = 2;  // rank limits of this kernel
constexpr int kQMax = 2 * kRabMax + kRkvMax;   // LDS stride: column sums per token
constexpr int kWv = kBwThreads / 64;
constexpr int kTokGroup = 8;             // tokens whose operands are staged in LDS at once

// Workgroup barrier that orders LDS only.  The waves exchange data through
// LDS alone (the chunk's recomputed states in global memory are read back by
// the thread that wrote them), so a barrier need not wait for the global
// loads in flight (the next step's state) or for the gradient stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One DPP lane move inside rows of 16 lanes (no LDS traffic): lane i reads
// the lane that the control word names.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Sum over a row of 16 lanes, left in every lane of the row: swap neighbours
// (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), mirror each half row
// (the other quad of the half), mirror the row (the other half).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  return v;
}

// Sum over the four rows of 16 lanes of a wave, left in every lane: swap odd
// and even rows (permlane16 swap), then the two halves (permlane32 swap).
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// floats of one staged token's operands for ranks (RAB, RKV)
constexpr int tok_ops(int rab, int rkv) { return 128 * (3 + 2 * (rab > 0 ? rab : 1) + rkv) + 128 * rkv; }

struct BwArgs {
  Problem p;
  const void* q;
  const void* K;
  const void* V;
  const float* ld;
  const void* A;
  const void* B;
  const void* dout;
  const float* dfinal;
  const float* S0;
  float* dq;
  float* dK;
  float* dV;
  float* dld;
  float* dA;
  float* dB;
  float* dS0;
  const float* ckpt;   // [BH, N, dk, dv]: the state entering each chunk
  const float* gend;   // [BH, N, dk, dv]: the cotangent of the state leaving each chunk
  float* bufs;         // per workgroup: C + 1 states of one chunk
};

// Chunk-boundary scans over the row-major fp32 chunk operators M_j
// ((dk + C) x (dk + C r_kv)).  Forward (REV false): X <- Acal_j X + Z_j V_j,
// storing the X entering chunk j.  Reverse: X <- Acal_j^T X + Qbar_j^T dO_j
// from j = N-1 down, storing the X leaving chunk j.  Padding tokens of a
// ragged last chunk are left out of the sums.
constexpr int kBdThreads = 256, kBdBN = 32;   // 32 row blocks of 4 x 8 column blocks of 4
struct BdArgs {
  Problem p;
  const float* M;
  const void* Y;      // V [BH, T, r_kv, dv] or dO [BH, T, dv]
  const float* init;  // [BH, dk, dv] or null (zero)
  float* out;         // [BH, N, dk, dv]
  float* fin;         // [BH, dk, dv] or null: the value after the last step (final state, or dS_init)
};

template <typename TI, bool REV>
__global__ __launch_bounds__(kBdThreads) void bw_bound_kernel(BdArgs a) {
  typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f4;
  constexpr int BN = kBdBN;
  __shared__ __align__(16) float xs[(128 + 256) * BN];   // state rows, then the chunk's input rows
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv, C = p.C, ncol = p.mcols(), yw = REV ? 1 : p.r_kv;
  const int64_t T = p.T, N = p.N;
  const int nsplit = (dv + BN - 1) / BN;
  const int64_t bh = blockIdx.x / nsplit;
  const int n0 = static_cast<int>(blockIdx.x % nsplit) * BN;
  const int tid = threadIdx.x, ni = tid % (BN / 4), ri = tid / (BN / 4);
  const bool rowok = 4 * ri < dk;   // d_k is a multiple of 16
  const TI* yp = static_cast<const TI*>(a.Y);
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int n = n0 + 4 * ni + c;
      acc[r][c] = (a.init && rowok && n < dv) ? a.init[(bh * dk + 4 * ri + r) * dv + n] : 0.f;
    }
  for (int64_t st = 0; st < N; ++st) {
    const int64_t j = REV ? N - 1 - st : st;
    const int64_t t0 = j * C;
    const int n = static_cast<int>(T - t0 < C ? T - t0 : C);
    const int nin = n * yw;
    float* o = a.out + static_cast<size_t>(bh * N + j) * dk * dv;
    if (rowok) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int col = n0 + 4 * ni + c;
          if (col < dv) o[static_cast<size_t>(4 * ri + r) * dv + col] = acc[r][c];
        }
    }
    lds_barrier();   // the previous step's reads of xs are done
    if (rowok) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<f4*>(&xs[(4 * ri + r) * BN + 4 * ni]) = f4{acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
    }
    const int64_t y0 = (bh * T + t0) * yw;
    for (int e = tid; e < nin * BN; e += kBdThreads) {
      const int m = e / BN, c = e % BN;
      xs[(dk + m) * BN + c] = n0 + c < dv ? Elem<TI>::load(yp, static_cast<size_t>(y0 + m) * dv + n0 + c) : 0.f;
    }
    lds_barrier();
    if (rowok) {
      const float* Mj = a.M + static_cast<size_t>(bh * N + j) * p.mrows() * ncol;
      const int KE = dk + nin;
      float nx[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) nx[r][c] = 0.f;
      if (!REV) {
        // (Acal_j | Z_j) row i, column m: Mj[i * ncol + m]
        int m = 0;
        for (; m + 4 <= KE; m += 4) {
          f4 w[4], x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = *reinterpret_cast<const f4*>(Mj + static_cast<size_t>(4 * ri + r) * ncol + m);
#pragma unroll
          for (int k = 0; k < 4; ++k) x[k] = *reinterpret_cast<const f4*>(&xs[(m + k) * BN + 4 * ni]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
              for (int c = 0; c < 4; ++c) nx[r][c] += w[r][k] * x[k][c];
        }
        for (; m < KE; ++m) {
          const f4 x = *reinterpret_cast<const f4*>(&xs[m * BN + 4 * ni]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float w = Mj[static_cast<size_t>(4 * ri + r) * ncol + m];
#pragma unroll
            for (int c = 0; c < 4; ++c) nx[r][c] += w * x[c];
          }
        }
      } else {
        // (Acal_j^T | Qbar_j^T) row i, column m: Mj[m * ncol + i]
#pragma unroll 4
        for (int m = 0; m < KE; ++m) {
          const f4 w = *reinterpret_cast<const f4*>(Mj + static_cast<size_t>(m) * ncol + 4 * ri);
          const f4 x = *reinterpret_cast<const f4*>(&xs[m * BN + 4 * ni]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) nx[r][c] += w[r] * x[c];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = nx[r][c];
    }
  }
  if (a.fin && rowok) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = n0 + 4 * ni + c;
        if (col < dv) a.fin[(bh * dk + 4 * ri + r) * dv + col] = acc[r][c];
      }
  }
}

// RAB, RKV: the ranks the per-thread operand arrays are sized for (r_ab <= RAB,
// r_kv <= RKV); kQ column sums per token: A^T G, B^T S_{t-1}, K^T G.
template <typename TI, int RAB, int RKV>
__global__ __launch_bounds__(kBwThreads) void backward_kernel(BwArgs a) {
  constexpr int kRab = RAB > 0 ? RAB : 1, kRkv = RKV;
  constexpr int kQ = 2 * kRab + kRkv;
  // per-wave row sums [parity][wave][quantity][column], double-buffered by token
  // parity, then the scalar-decay per-row terms [parity][row]
  extern __shared__ __align__(16) float lds[];
  auto red = [&](int par, int w, int q, int n) -> float& { return lds[((par * kWv + w) * kQMax + q) * 128 + n]; };
  float* dsum0 = lds + 2 * kWv * kQMax * 128;
  auto dsum = [&](int par, int i) -> float& { return dsum0[par * 128 + i]; };
  float* fin0 = dsum0 + 2 * 128;   // column sums [parity][quantity][column]
  auto colfin = [&](int par, int q, int n) -> float& { return fin0[(par * kQMax + q) * 128 + n]; };
  // operands of a group of up to kTokGroup tokens, staged by all threads with
  // coalesced loads: per token exp(log_decay), A, B, K, q (rows), V, dout (columns)
  constexpr int oLam = 0, oA = 128, oB = oA + 128 * kRab, oK = oB + 128 * kRab, oQ = oK + 128 * kRkv,
                oV = oQ + 128, oDo = oV + 128 * kRkv, kOps = oDo + 128;
  float* tokb = fin0 + 2 * kQMax * 128;
  auto tk = [&](int u, int off) -> float& { return tokb[u * kOps + off]; };
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv, C = p.C, r_ab = p.r_ab, r_kv = p.r_kv;
  const int64_t T = p.T, N = p.N;
  int64_t bh = 0;   // the job's (batch, head), set per job
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tr = tid / kNTC, tc = tid % kNTC;
  const TI* qp = static_cast<const TI*>(a.q);
  const TI* Kp = static_cast<const TI*>(a.K);
  const TI* Vp = static_cast<const TI*>(a.V);
  const TI* Ap = static_cast<const TI*>(a.A);
  const TI* Bp = static_cast<const TI*>(a.B);
  const TI* dop = static_cast<const TI*>(a.dout);
  const int nst = kRB * kCB;                                       // register slots per state
  const size_t sstride = static_cast<size_t>(nst) * kBwThreads;   // floats per stored state
  float* buf = a.bufs + static_cast<size_t>(blockIdx.x) * (C + 1) * sstride;   // C + 1 states of one chunk
  auto rowi = [&](int r) { return tr + kNTR * r; };
  auto coln = [&](int c) { return tc + kNTC * c; };
  auto rok = [&](int r) { return tr + kNTR * r < dk; };
  auto cok = [&](int c) { return tc + kNTC * c < dv; };
  // storage of one state: the 32 register slots of thread tid contiguous at
  // tid * 32 (16-byte pieces with immediate offsets from one address)
  typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f4;
  auto st_state = [&](float* base, const float (&S)[kRB][kCB]) {
    f4* d = reinterpret_cast<f4*>(base + static_cast<size_t>(tid) * nst);
#pragma unroll
    for (int r = 0; r < kRB; ++r)
#pragma unroll
      for (int c = 0; c < kCB; c += 4) d[(r * kCB + c) / 4] = f4{S[r][c], S[r][c + 1], S[r][c + 2], S[r][c + 3]};
  };
  auto ld_state = [&](const float* base, float (&S)[kRB][kCB]) {
    const f4* d = reinterpret_cast<const f4*>(base + static_cast<size_t>(tid) * nst);
#pragma unroll
    for (int r = 0; r < kRB; ++r)
#pragma unroll
      for (int c = 0; c < kCB; c += 4) {
        const f4 v = d[(r * kCB + c) / 4];
        S[r][c] = v[0];
        S[r][c + 1] = v[1];
        S[r][c + 2] = v[2];
        S[r][c + 3] = v[3];
      }
  };
  // sum over the 16 column groups of a row group (lanes differing in bits 0..3)
  static_assert(kNTC == 16, "row sums are DPP moves inside rows of 16 lanes");
  auto rowsum = [&](float v) { return row16_sum(v); };
  // Stage tokens t0 .. t0 + cnt - 1 (cnt <= kTokGroup); callers put a barrier
  // before (the previous group has been read) and after.
  auto stage = [&](int64_t t0, int cnt) {
    const int64_t tok0 = bh * T + t0;
    for (int e = tid; e < cnt * dk; e += kBwThreads) {
      const int u = e / dk, i = e % dk;
      tk(u, oLam + i) = expf(p.scalar ? a.ld[tok0 + u] : a.ld[(tok0 + u) * dk + i]);
      tk(u, oQ + i) = Elem<TI>::load(qp, static_cast<size_t>(tok0 + u) * dk + i);
    }
    for (int e = tid; e < cnt * r_ab * dk; e += kBwThreads) {
      const int u = e / (r_ab * dk), x = (e / dk) % r_ab, i = e % dk;
      tk(u, oA + 128 * x + i) = Elem<TI>::load(Ap, static_cast<size_t>(tok0) * r_ab * dk + e);
      tk(u, oB + 128 * x + i) = Elem<TI>::load(Bp, static_cast<size_t>(tok0) * r_ab * dk + e);
    }
    for (int e = tid; e < cnt * r_kv * dk; e += kBwThreads) {
      const int u = e / (r_kv * dk), x = (e / dk) % r_kv, i = e % dk;
      tk(u, oK + 128 * x + i) = Elem<TI>::load(Kp, static_cast<size_t>(tok0) * r_kv * dk + e);
    }
    for (int e = tid; e < cnt * r_kv * dv; e += kBwThreads) {
      const int u = e / (r_kv * dv), x = (e / dv) % r_kv, n = e % dv;
      tk(u, oV + 128 * x + n) = Elem<TI>::load(Vp, static_cast<size_t>(tok0) * r_kv * dv + e);
    }
    for (int e = tid; e < cnt * dv; e += kBwThreads) {
      const int u = e / dv, n = e % dv;
      tk(u, oDo + n) = Elem<TI>::load(dop, static_cast<size_t>(tok0 + u) * dv + n);
    }
  };
  // Per-token operands of this thread's rows and columns, from staged slot u.
  float lam[kRB], Av[kRab][kRB], Bv[kRab][kRB], Kv[kRkv][kRB], Vv[kRkv][kCB];
  auto load_tok = [&](int u) {
#pragma unroll
    for (int r = 0; r < kRB; ++r) {
      const int i = rok(r) ? rowi(r) : 0;
      lam[r] = tk(u, oLam + i);
#pragma unroll
      for (int x = 0; x < kRab; ++x) {
        const bool ok = x < r_ab && rok(r);
        Av[x][r] = ok ? tk(u, oA + 128 * x + i) : 0.f;
        Bv[x][r] = ok ? tk(u, oB + 128 * x + i) : 0.f;
      }
#pragma unroll
      for (int x = 0; x < kRkv; ++x) Kv[x][r] = (x < r_kv && rok(r)) ? tk(u, oK + 128 * x + i) : 0.f;
    }
#pragma unroll
    for (int c = 0; c < kCB; ++c) {
      const int n = cok(c) ? coln(c) : 0;
#pragma unroll
      for (int x = 0; x < kRkv; ++x) Vv[x][c] = (x < r_kv && cok(c)) ? tk(u, oV + 128 * x + n) : 0.f;
    }
  };
  // Sums over rows of this thread's columns, for nq quantities whose per-thread
  // partials are in part[q][c]: inside the wave (lane bits 4, 5), then across
  // the waves through LDS: each column sum is formed once from the eight wave
  // partials and read back by the threads of that column.  Two barriers.
  auto colsum = [&](float (&part)[kQ][kCB], int nq, int par) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if (q >= nq) break;
#pragma unroll
      for (int c = 0; c < kCB; ++c) {
        const float v = rows4_sum(part[q][c]);
        if ((lane >> 4) == 0 && cok(c)) red(par, wave, q, coln(c)) = v;
      }
    }
    lds_barrier();
    for (int e = tid; e < nq * dv; e += kBwThreads) {
      const int q = e / dv, n = e % dv;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWv; ++w) v += red(par, w, q, n);
      colfin(par, q, n) = v;
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if (q >= nq) break;
#pragma unroll
      for (int c = 0; c < kCB; ++c) part[q][c] = cok(c) ? colfin(par, q, coln(c)) : 0.f;
    }
  };
  // One forward token: S <- D S - A (B^T S) + K V^T.
  auto fwd_step = [&](float (&S)[kRB][kCB], int par) {
    float part[kQ][kCB];
#pragma unroll
    for (int x = 0; x < kRab; ++x)
#pragma unroll
      for (int c = 0; c < kCB; ++c) {
        float v = 0.f;
#pragma unroll
        for (int r = 0; r < kRB; ++r) v += Bv[x][r] * S[r][c];
        part[x][c] = v;
      }
    colsum(part, r_ab, par);
#pragma unroll
    for (int r = 0; r < kRB; ++r)
#pragma unroll
      for (int c = 0; c < kCB; ++c) {
        float v = lam[r] * S[r][c];
#pragma unroll
        for (int x = 0; x < kRab; ++x) v -= Av[x][r] * part[x][c];
#pragma unroll
        for (int x = 0; x < kRkv; ++x) v += Kv[x][r] * Vv[x][c];
        S[r][c] = v;
      }
  };

  float S[kRB][kCB], Sp[kRB][kCB], Sn[kRB][kCB], G[kRB][kCB];
  int par = 0;
  for (int64_t job = blockIdx.x; job < p.BH * N; job += gridDim.x) {
    bh = job / N;
    const int64_t j = job % N;
    const int64_t t0 = j * C, t1 = (j + 1) * C < T ? (j + 1) * C : T;
    // the state entering the chunk and the cotangent of the state leaving it
    const float* sb = a.ckpt + static_cast<size_t>(job) * dk * dv;
    const float* gb = a.gend + static_cast<size_t>(job) * dk * dv;
#pragma unroll
    for (int r = 0; r < kRB; ++r)
#pragma unroll
      for (int c = 0; c < kCB; ++c) {
        const bool ok = rok(r) && cok(c);
        S[r][c] = ok ? sb[rowi(r) * dv + coln(c)] : 0.f;
        G[r][c] = ok ? gb[rowi(r) * dv + coln(c)] : 0.f;
      }
    st_state(buf, S);
    for (int64_t tg = t0; tg < t1; tg += kTokGroup) {
      const int cnt = static_cast<int>(t1 - tg < kTokGroup ? t1 - tg : kTokGroup);
      lds_barrier();
      stage(tg, cnt);
      lds_barrier();
      for (int u = 0; u < cnt; ++u) {
        load_tok(u);
        fwd_step(S, par);
        par ^= 1;
        st_state(buf + (tg + u - t0 + 1) * sstride, S);
      }
    }
    __syncthreads();   // once per chunk: the recomputed states are in memory
    // S holds S_{t1-1}; groups of tokens from the end of the chunk
    for (int64_t th = t1; th > t0;) {
      const int64_t tl = th - kTokGroup > t0 ? th - kTokGroup : t0;
      const int cnt = static_cast<int>(th - tl);
      lds_barrier();
      stage(tl, cnt);
      lds_barrier();
      th = tl;
      for (int u = cnt - 1; u >= 0; --u) {
      const int64_t t = tl + u;
      const int64_t tok = bh * T + t;
      load_tok(u);
      // S_{t-1}: loaded during the previous step (the first token of a chunk's
      // walk loads it here)
      if (t == t1 - 1) {
        ld_state(buf + (t - t0) * sstride, Sn);
      }
#pragma unroll
      for (int r = 0; r < kRB; ++r)
#pragma unroll
        for (int c = 0; c < kCB; ++c) Sp[r][c] = Sn[r][c];
      if (t > t0) ld_state(buf + (t - 1 - t0) * sstride, Sn);   // S_{t-2}, for the next step
      float qv[kRB], dov[kCB];
#pragma unroll
      for (int r = 0; r < kRB; ++r) qv[r] = rok(r) ? tk(u, oQ + rowi(r)) : 0.f;
#pragma unroll
      for (int c = 0; c < kCB; ++c) dov[c] = cok(c) ? tk(u, oDo + coln(c)) : 0.f;
      // G += q do^T
#pragma unroll
      for (int r = 0; r < kRB; ++r)
#pragma unroll
        for (int c = 0; c < kCB; ++c) G[r][c] += qv[r] * dov[c];
      // row sums: dq = S_t do, dlog_decay terms = rowdot(G, S_{t-1})
#pragma unroll
      for (int r = 0; r < kRB; ++r) {
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int c = 0; c < kCB; ++c) {
          s1 += S[r][c] * dov[c];
          s2 += G[r][c] * Sp[r][c];
        }
        s1 = rowsum(s1);
        s2 = rowsum(s2) * lam[r];
        if (tc == 0 && rok(r)) {
          a.dq[static_cast<size_t>(tok) * dk + rowi(r)] = s1;
          if (!p.scalar) a.dld[static_cast<size_t>(tok) * dk + rowi(r)] = s2;
          else dsum(par, rowi(r)) = s2;
        }
      }
      // column sums: z = A^T G, w = B^T S_{t-1}, dV = K^T G
      float part[kQ][kCB];
#pragma unroll
      for (int c = 0; c < kCB; ++c) {
#pragma unroll
        for (int x = 0; x < kRab; ++x) {
          float z = 0.f, w = 0.f;
#pragma unroll
          for (int r = 0; r < kRB; ++r) {
            z += Av[x][r] * G[r][c];
            w += Bv[x][r] * Sp[r][c];
          }
          part[x][c] = z;
          part[kRab + x][c] = w;
        }
#pragma unroll
        for (int x = 0; x < kRkv; ++x) {
          float d = 0.f;
#pragma unroll
          for (int r = 0; r < kRB; ++r) d += Kv[x][r] * G[r][c];
          part[2 * kRab + x][c] = d;
        }
      }
      colsum(part, kQ, par);
      if (p.scalar && tid == 0) {
        float s = 0.f;
        for (int i = 0; i < dk; ++i) s += dsum(par, i);
        a.dld[tok] = s;
      }
      if (tr == 0) {
#pragma unroll
        for (int c = 0; c < kCB; ++c)
#pragma unroll
          for (int x = 0; x < kRkv; ++x)
            if (x < r_kv && cok(c)) a.dV[(static_cast<size_t>(tok) * r_kv + x) * dv + coln(c)] = part[2 * kRab + x][c];
      }
      // row sums: dK = G V, dA = -G w, dB = -S_{t-1} z
#pragma unroll
      for (int r = 0; r < kRB; ++r) {
#pragma unroll
        for (int x = 0; x < kRkv; ++x) {
          float s = 0.f;
#pragma unroll
          for (int c = 0; c < kCB; ++c) s += G[r][c] * Vv[x][c];
          s = rowsum(s);
          if (tc == 0 && x < r_kv && rok(r)) a.dK[(static_cast<size_t>(tok) * r_kv + x) * dk + rowi(r)] = s;
        }
#pragma unroll
        for (int x = 0; x < kRab; ++x) {
          float sa = 0.f, sb = 0.f;
#pragma unroll
          for (int c = 0; c < kCB; ++c) {
            sa += G[r][c] * part[kRab + x][c];
            sb += Sp[r][c] * part[x][c];
          }
          sa = rowsum(sa);
          sb = rowsum(sb);
          if (tc == 0 && x < r_ab && rok(r)) {
            a.dA[(static_cast<size_t>(tok) * r_ab + x) * dk + rowi(r)] = -sa;
            a.dB[(static_cast<size_t>(tok) * r_ab + x) * dk + rowi(r)] = -sb;
          }
        }
      }
      // G <- P_t^T G = D G - B (A^T G)
#pragma unroll
      for (int r = 0; r < kRB; ++r)
#pragma unroll
        for (int c = 0; c < kCB; ++c) {
          float v = lam[r] * G[r][c];
#pragma unroll
          for (int x = 0; x < kRab; ++x) v -= Bv[x][r] * part[x][c];
          G[r][c] = v;
        }
#pragma unroll
      for (int r = 0; r < kRB; ++r)
#pragma unroll
        for (int c = 0; c < kCB; ++c) S[r][c] = Sp[r][c];
      par ^= 1;
      }
    }
    if (j == 0) {
#pragma unroll
      for (int r = 0; r < kRB; ++r)
#pragma unroll
        for (int c = 0; c < kCB; ++c)
          if (rok(r) && cok(c)) a.dS0[(bh * dk + rowi(r)) * dv + coln(c)] = G[r][c];
    }
  }
}

}  // namespace

bool backward_supported(const Problem& p) {
  return p.dk <= kNTR * kRB && p.dv <= kNTC * kCB && p.r_ab <= kRabMax && p.r_kv <= kRkvMax;
}

namespace {

constexpr size_t kBwAlign = 256;
size_t bw_align(size_t x) { return (x + kBwAlign - 1) & ~(kBwAlign - 1); }

// Workgroups of the token walk: one resident per compute unit, each with its
// own buffer of C + 1 states.
int64_t bw_walk_groups(const Problem& p) {
  const int64_t jobs = p.BH * p.N;
  return jobs < 256 ? jobs : 256;
}

// Workspace: the chunk operators (and what their prepare needs), the states
// entering the chunks, the cotangents leaving them, then either the token
// walks' buffers or (chunked route) the chunked kernels' buffers.
struct BwLayout {
  size_t ops, ckpt, gend, bufs, chunk, total;
};
BwLayout bw_layout(const Problem& p) {
  BwLayout l{};
  const size_t state = static_cast<size_t>(p.dk) * p.dv;
  l.ops = 0;
  if (backward_chunked(p)) {
    // bf16 boundary states (N + 1 per head) and cotangents (N per head)
    l.ckpt = bw_align(fast_workspace_bytes(p));
    l.gend = l.ckpt + bw_align(static_cast<size_t>(p.BH * (p.N + 1)) * state * 2);
    l.chunk = l.gend + bw_align(static_cast<size_t>(p.BH * p.N) * state * 2);
    l.total = l.chunk + backward_chunked_bytes(p);
  } else {
    const size_t states = static_cast<size_t>(p.BH * p.N) * state * sizeof(float);
    l.ckpt = bw_align(f32_operators_bytes(p));
    l.gend = l.ckpt + bw_align(states);
    l.bufs = l.gend + bw_align(states);
    const size_t st = static_cast<size_t>(kRB) * kCB * kBwThreads;   // floats per stored walk state
    l.total = l.bufs + static_cast<size_t>(bw_walk_groups(p)) * (p.C + 1) * st * sizeof(float);
  }
  return l;
}

// The training pair's saved buffer: the chunk operators, the boundary states
// (bf16, N + 1 per head), then the scaled operands; the saved-state backward's
// workspace: the boundary cotangents, then the chunked kernels' buffers
// without the scaled operands.
struct SavedLayout {
  size_t ckpt, scaled, total, chunk, ws_total;
};
SavedLayout saved_layout(const Problem& p) {
  SavedLayout l{};
  if (!backward_chunked(p)) return l;
  const size_t state = static_cast<size_t>(p.dk) * p.dv;
  l.ckpt = bw_align(fast_workspace_bytes(p));
  l.scaled = l.ckpt + bw_align(static_cast<size_t>(p.BH * (p.N + 1)) * state * 2);
  l.total = l.scaled + backward_chunked_ops_bytes(p);
  l.chunk = bw_align(static_cast<size_t>(p.BH * p.N) * state * 2);
  l.ws_total = l.chunk + backward_chunked_bytes(p, false);
  return l;
}

}  // namespace

size_t backward_workspace_bytes(const Problem& p) { return bw_layout(p).total; }
size_t backward_saved_bytes(const Problem& p) { return saved_layout(p).total; }
size_t backward_saved_workspace_bytes(const Problem& p) { return saved_layout(p).ws_total; }

hipError_t launch_forward_train(const Problem& p, const void* q, const void* k, const void* v, const float* ld,
                                const void* A, const void* B, void* out, float* Sfin, const float* S0, void* saved,
                                hipStream_t s) {
  if (!backward_chunked(p)) return hipErrorInvalidValue;
  const SavedLayout l = saved_layout(p);
  char* sv = static_cast<char*>(saved);
  // the backward instance of the prepare: the same operators, and the scaled
  // operands kept beside them; the scan's instance that also keeps the state
  // entering every chunk
  hipError_t e = fast_prepare_bw(p, q, k, ld, A, B, sv, backward_chunked_ops_at(p, sv + l.scaled), s);
  if (e != hipSuccess) return e;
  return fast_scan(p, sv, v, out, Sfin, S0, s, sv + l.ckpt);
}

hipError_t launch_backward_saved(const Problem& p, const void* q, const void* k, const void* v, const float* ld,
                                 const void* A, const void* B, const void* dout, const float* dfinal,
                                 const void* saved, float* dq, float* dK, float* dV, float* dld,
                                 float* dA, float* dB, float* dS0, void* workspace, hipStream_t s) {
  if (p.BH == 0) return hipSuccess;
  if (!backward_chunked(p)) return hipErrorInvalidValue;
  const SavedLayout l = saved_layout(p);
  char* ws = static_cast<char*>(workspace);
  const char* sv = static_cast<const char*>(saved);
  const PrepBwOut ops = backward_chunked_ops_at(p, const_cast<char*>(sv) + l.scaled);
  // the cotangents leaving the chunks first, into the front of the workspace
  hipError_t e = launch_backward_rscan(p, sv, dout, dfinal, ws, dS0, s);
  if (e != hipSuccess) return e;
  return launch_backward_chunked(p, q, k, v, ld, A, B, dout, sv + l.ckpt, ws, dq, dK, dV, dld, dA, dB, ws + l.chunk,
                                 s, &ops);
}

namespace {

template <typename TI, int RAB, int RKV>
hipError_t launch_bw_t(const Problem& p, const BwArgs& a, size_t lds_base, hipStream_t s) {
  const size_t lds = lds_base + static_cast<size_t>(kTokGroup) * tok_ops(RAB, RKV) * sizeof(float);
  const void* fn = reinterpret_cast<const void*>(backward_kernel<TI, RAB, RKV>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((backward_kernel<TI, RAB, RKV>), dim3(static_cast<unsigned>(bw_walk_groups(p))),
                     dim3(kBwThreads), lds, s, a);
  return hipGetLastError();
}

// The smallest instantiation whose operand arrays cover the ranks.
template <int RAB>
hipError_t launch_bw(const Problem& p, const BwArgs& a, size_t lds, hipStream_t s) {
  if (p.bf16)
    return p.r_kv <= 1 ? launch_bw_t<bf16_raw, RAB, 1>(p, a, lds, s) : launch_bw_t<bf16_raw, RAB, 2>(p, a, lds, s);
  return p.r_kv <= 1 ? launch_bw_t<float, RAB, 1>(p, a, lds, s) : launch_bw_t<float, RAB, 2>(p, a, lds, s);
}

// sfin, dS0: where the final state and the initial state's cotangent go (or
// null); fwd false: the cotangent scan only.
template <typename TI>
hipError_t launch_boundary_scans(const Problem& p, const float* M, const void* v, const void* dout, const float* S0,
                         const float* dfinal, float* ckpt, float* gend, float* sfin, float* dS0, hipStream_t s,
                         bool fwd = true) {
  const unsigned grid = static_cast<unsigned>(p.BH * ((p.dv + kBdBN - 1) / kBdBN));
  hipError_t e;
  if (fwd) {
    hipLaunchKernelGGL((bw_bound_kernel<TI, false>), dim3(grid), dim3(kBdThreads), 0, s,
                       BdArgs{p, M, v, S0, ckpt, sfin});
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((bw_bound_kernel<TI, true>), dim3(grid), dim3(kBdThreads), 0, s,
                     BdArgs{p, M, dout, dfinal, gend, dS0});
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const Problem& p, const void* q, const void* k, const void* v, const float* ld,
                           const void* A, const void* B, const void* dout, const float* dfinal, const float* S0,
                           float* dq, float* dK, float* dV, float* dld, float* dA, float* dB, float* dS0,
                           void* workspace, hipStream_t s) {
  if (p.BH == 0) return hipSuccess;
  if (!backward_supported(p)) return hipErrorInvalidValue;
  const BwLayout l = bw_layout(p);
  char* ws = static_cast<char*>(workspace);
  if (backward_chunked(p)) {
    // Both boundary scans on bf16 MFMAs over the bf16 MFMA prepare's
    // operators: the states entering the chunks and the final state (the
    // forward scan), then the cotangents leaving the chunks; both in bf16.
    // the prepare also leaves the decay-scaled operands for the chunked kernels
    hipError_t e = fast_prepare_bw(p, q, k, ld, A, B, ws + l.ops, backward_chunked_prep_out(p, ws + l.chunk), s);
    if (e != hipSuccess) return e;
    e = fast_scan(p, ws + l.ops, v, nullptr, nullptr, S0, s, ws + l.ckpt);
    if (e != hipSuccess) return e;
    e = launch_backward_rscan(p, ws + l.ops, dout, dfinal, ws + l.gend, dS0, s);
    if (e != hipSuccess) return e;
    return launch_backward_chunked(p, q, k, v, ld, A, B, dout, ws + l.ckpt, ws + l.gend, dq, dK, dV, dld, dA, dB,
                                   ws + l.chunk, s);
  }
  float* ckpt = reinterpret_cast<float*>(ws + l.ckpt);
  float* gend = reinterpret_cast<float*>(ws + l.gend);
  const float* M = nullptr;
  hipError_t e = f32_operators(p, q, k, ld, A, B, ws + l.ops, &M, s);
  if (e != hipSuccess) return e;
  e = p.bf16 ? launch_boundary_scans<bf16_raw>(p, M, v, dout, S0, dfinal, ckpt, gend, nullptr, nullptr, s)
             : launch_boundary_scans<float>(p, M, v, dout, S0, dfinal, ckpt, gend, nullptr, nullptr, s);
  if (e != hipSuccess) return e;
  BwArgs a{p, q, k, v, ld, A, B, dout, dfinal, S0, dq, dK, dV, dld, dA, dB, dS0, ckpt, gend,
           reinterpret_cast<float*>(ws + l.bufs)};
  const size_t lds = (static_cast<size_t>(2) * kWv * kQMax * 128 + 2 * 128 + 2 * kQMax * 128) * sizeof(float);
  if (p.r_ab == 0) return launch_bw<0>(p, a, lds, s);
  if (p.r_ab == 1) return launch_bw<1>(p, a, lds, s);
  if (p.r_ab == 2) return launch_bw<2>(p, a, lds, s);
  return launch_bw<4>(p, a, lds, s);
}

}  // namespace lattn
