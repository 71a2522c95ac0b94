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
#include "common.hpp"
#include "kernels.hpp"

namespace lattn {
namespace {

constexpr int kThreads = 256;

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

template <typename TI>
__global__ __launch_bounds__(kThreads) void general_prepare_kernel(PrepArgs a) {
  const Problem& p = a.p;
  const int dk = p.dk, C = p.C, r_ab = p.r_ab, r_kv = p.r_kv;
  const int na = p.na(), nk = p.nk(), ncol = p.mcols();
  const int tid = threadIdx.x;
  float* G = a.scratch + static_cast<size_t>(blockIdx.x) * a.slot_floats;
  float* Bt = G + static_cast<size_t>(C) * dk;
  float* At = Bt + static_cast<size_t>(na) * dk;
  float* Kt = At + static_cast<size_t>(na) * dk;
  float* Qt = Kt + static_cast<size_t>(nk) * dk;
  float* L = Qt + static_cast<size_t>(C) * dk;
  float* LK = L + static_cast<size_t>(na) * na;
  float* MA = LK + static_cast<size_t>(na) * nk;
  float* MK = MA + static_cast<size_t>(C) * na;
  float* WX = MK + static_cast<size_t>(C) * nk;
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
    for (int i = tid; i < dk; i += kThreads) {
      float g = 0.f;
      for (int t = 0; t < C; ++t) {
        float l = 0.f;
        if (t < n) l = p.scalar ? a.ld[tok0 + t] : a.ld[(tok0 + t) * dk + i];
        g += l;
        G[t * dk + i] = g;
      }
    }
    __syncthreads();

    // 2. decay-scaled operands (zero rows for padded tokens).
    for (int e = tid; e < na * dk; e += kThreads) {
      const int s = e / dk, i = e % dk, t = s / r_ab;
      float bv = 0.f, av = 0.f;
      if (t < n) {
        const size_t idx = (static_cast<size_t>(tok0 + t) * r_ab + (s % r_ab)) * dk + i;
        bv = Elem<TI>::load(Bp, idx);
        av = Elem<TI>::load(Ap, idx);
      }
      const float gex = t > 0 ? G[(t - 1) * dk + i] : 0.f;
      Bt[e] = bv * expf(gex);
      At[e] = av * expf(-G[t * dk + i]);
    }
    for (int e = tid; e < nk * dk; e += kThreads) {
      const int s = e / dk, i = e % dk, t = s / r_kv;
      float kv = 0.f;
      if (t < n) kv = Elem<TI>::load(kp, (static_cast<size_t>(tok0 + t) * r_kv + (s % r_kv)) * dk + i);
      Kt[e] = kv * expf(-G[t * dk + i]);
    }
    for (int e = tid; e < C * dk; e += kThreads) {
      const int t = e / dk, i = e % dk;
      float qv = 0.f;
      if (q != nullptr && t < n) qv = Elem<TI>::load(q, static_cast<size_t>(tok0 + t) * dk + i);
      Qt[e] = qv * expf(G[e]);
    }
    __syncthreads();

    // 3. masked Gram blocks.
    for (int e = tid; e < na * na; e += kThreads) {
      const int r = e / na, c = e % na;
      float s = 0.f;
      if (r / r_ab > c / r_ab)
        for (int i = 0; i < dk; ++i) s += Bt[r * dk + i] * At[c * dk + i];
      L[e] = s;
    }
    for (int e = tid; e < na * nk; e += kThreads) {
      const int r = e / nk, c = e % nk;
      float s = 0.f;
      if (r / r_ab > c / r_kv)
        for (int i = 0; i < dk; ++i) s += Bt[r * dk + i] * Kt[c * dk + i];
      LK[e] = s;
    }
    for (int e = tid; e < C * na; e += kThreads) {
      const int t = e / na, c = e % na;
      float s = 0.f;
      if (t >= c / r_ab)
        for (int i = 0; i < dk; ++i) s += Qt[t * dk + i] * At[c * dk + i];
      MA[e] = s;
    }
    for (int e = tid; e < C * nk; e += kThreads) {
      const int t = e / nk, c = e % nk;
      float s = 0.f;
      if (t >= c / r_kv)
        for (int i = 0; i < dk; ++i) s += Qt[t * dk + i] * Kt[c * dk + i];
      MK[e] = s;
    }
    __syncthreads();

    // 4. forward substitution, one token (r_ab rows) at a time: rows of one token
    //    do not couple (L is zero inside a token's block).
    for (int t = 0; t < C; ++t) {
      for (int e = tid; e < r_ab * ncol; e += kThreads) {
        const int row = t * r_ab + e / ncol, c = e % ncol;
        float v = c < dk ? Bt[row * dk + c] : LK[row * nk + (c - dk)];
        for (int b = 0; b < t * r_ab; ++b) v -= L[row * na + b] * WX[b * ncol + c];
        WX[row * ncol + c] = v;
      }
      __syncthreads();
    }

    // 5. chunk operator M_j.
    float* Mo = a.M + static_cast<size_t>(job) * p.mrows() * ncol;
    for (int e = tid; e < dk * ncol; e += kThreads) {
      const int i = e / ncol, c = e % ncol;
      float s = 0.f;
      for (int b = 0; b < na; ++b) s += At[b * dk + i] * WX[b * ncol + c];
      const float base = c < dk ? (i == c ? 1.f : 0.f) : Kt[(c - dk) * dk + i];
      Mo[e] = expf(G[(C - 1) * dk + i]) * (base - s);
    }
    for (int e = tid; e < C * ncol; e += kThreads) {
      const int t = e / ncol, c = e % ncol;
      float s = 0.f;
      for (int b = 0; b < na; ++b) s += MA[t * na + b] * WX[b * ncol + c];
      const float base = c < dk ? Qt[t * dk + c] : MK[t * nk + (c - dk)];
      Mo[static_cast<size_t>(dk + t) * ncol + c] = base - s;
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
  int BV;
};

// One workgroup per (batch*head, d_v slice of BV columns); chunks in order.
template <typename TI>
__global__ __launch_bounds__(kThreads) void general_scan_kernel(ScanArgs a) {
  extern __shared__ float smem[];
  const Problem& p = a.p;
  const int dk = p.dk, dv = p.dv, C = p.C, r_kv = p.r_kv, nk = p.nk(), ncol = p.mcols();
  const int BV = a.BV;
  const int nvt = dv / BV;
  const int64_t bh = blockIdx.x / nvt;
  const int c0 = (blockIdx.x % nvt) * BV;
  const int tid = threadIdx.x;
  float* S = smem;                       // dk x BV
  float* Vj = S + dk * BV;               // nk x BV
  float* Y = Vj + nk * BV;               // (dk + C) x BV
  const TI* vp = static_cast<const TI*>(a.v);
  TI* op = static_cast<TI*>(a.out);

  for (int e = tid; e < dk * BV; e += kThreads) {
    const int i = e / BV, c = e % BV;
    S[e] = a.S0 ? a.S0[(bh * dk + i) * dv + c0 + c] : 0.f;
  }
  __syncthreads();
  for (int64_t j = 0; j < p.N; ++j) {
    const int64_t t0 = j * C;
    const int n = static_cast<int>(p.T - t0 < C ? p.T - t0 : C);
    const int64_t tok0 = bh * p.T + t0;
    for (int e = tid; e < nk * BV; e += kThreads) {
      const int s = e / BV, c = e % BV, t = s / r_kv;
      Vj[e] = t < n ? Elem<TI>::load(vp, (static_cast<size_t>(tok0 + t) * r_kv + (s % r_kv)) * dv + c0 + c) : 0.f;
    }
    __syncthreads();
    const float* Mj = a.M + static_cast<size_t>(bh * p.N + j) * p.mrows() * ncol;
    for (int e = tid; e < (dk + C) * BV; e += kThreads) {
      const int r = e / BV, c = e % BV;
      const float* mr = Mj + static_cast<size_t>(r) * ncol;
      float s = 0.f;
      for (int m = 0; m < dk; ++m) s += mr[m] * S[m * BV + c];
      for (int m = 0; m < nk; ++m) s += mr[dk + m] * Vj[m * BV + c];
      Y[e] = s;
    }
    __syncthreads();
    for (int e = tid; e < n * BV; e += kThreads) {
      const int t = e / BV, c = e % BV;
      Elem<TI>::store(op, static_cast<size_t>(tok0 + t) * dv + c0 + c, Y[(dk + t) * BV + c]);
    }
    for (int e = tid; e < dk * BV; e += kThreads) S[e] = Y[e];
    __syncthreads();
  }
  if (a.Sfin) {
    for (int e = tid; e < dk * BV; e += kThreads) {
      const int i = e / BV, c = e % BV;
      a.Sfin[(bh * dk + i) * dv + c0 + c] = S[e];
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
  const size_t na = p.na(), nk = p.nk(), C = p.C, dk = p.dk;
  g.slot_floats = C * dk + 2 * na * dk + nk * dk + C * dk + na * na + na * nk + C * na + C * nk +
                  na * (dk + nk);
  g.slot_floats = (g.slot_floats + 63) & ~static_cast<size_t>(63);
  const int64_t jobs = p.BH * p.N;
  g.slots = static_cast<int>(jobs < 1024 ? (jobs > 0 ? jobs : 1) : 1024);
  g.m_bytes = static_cast<size_t>(jobs) * p.mrows() * p.mcols() * sizeof(float);
  g.m_bytes = (g.m_bytes + 255) & ~static_cast<size_t>(255);
  g.total_bytes = g.m_bytes + static_cast<size_t>(g.slots) * g.slot_floats * sizeof(float);
  return g;
}

hipError_t general_prepare(const Problem& p, const void* q, const void* k, const float* ld,
                           const void* A, const void* B, void* workspace, hipStream_t s) {
  const GeneralPlan g = general_plan(p);
  PrepArgs a{p, q, k, ld, A, B, static_cast<float*>(workspace),
             reinterpret_cast<float*>(static_cast<char*>(workspace) + g.m_bytes), g.slot_floats};
  if (p.BH * p.N == 0) return hipSuccess;
  if (p.bf16)
    hipLaunchKernelGGL(general_prepare_kernel<bf16_raw>, dim3(g.slots), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(general_prepare_kernel<float>, dim3(g.slots), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t general_scan(const Problem& p, const void* workspace, const void* v, void* out,
                        float* Sfin, const float* S0, hipStream_t s) {
  const int BV = (p.dv % 32 == 0) ? 32 : 16;
  ScanArgs a{p, static_cast<const float*>(workspace), v, out, Sfin, S0, BV};
  const size_t lds = static_cast<size_t>(p.dk + p.nk() + p.dk + p.C) * BV * sizeof(float);
  const int64_t blocks = p.BH * (p.dv / BV);
  if (blocks == 0) return hipSuccess;
  // Dynamic LDS above 64 KiB must be opted into per kernel.
  if (p.bf16) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(general_scan_kernel<bf16_raw>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    hipLaunchKernelGGL(general_scan_kernel<bf16_raw>, dim3(blocks), dim3(kThreads), lds, s, a);
  } else {
    hipFuncSetAttribute(reinterpret_cast<const void*>(general_scan_kernel<float>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    hipLaunchKernelGGL(general_scan_kernel<float>, dim3(blocks), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
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
