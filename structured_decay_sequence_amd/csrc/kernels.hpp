// Launch interface between the C ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lattn {

// One chunk-wise problem, with every size the kernels need.
struct Problem {
  int64_t BH;      // batch * heads
  int64_t T;       // tokens per (batch, head)
  int dk, dv;
  int r_ab, r_kv;
  int C;           // chunk length
  int64_t N;       // chunks per (batch, head) = ceil(T / C)
  int scalar;      // 1: log_decay is [BH, T]; 0: [BH, T, dk]
  int bf16;        // 1: q, K, V, A, B, out are bf16; 0: fp32
  __host__ __device__ int na() const { return C * r_ab; }
  __host__ __device__ int nk() const { return C * r_kv; }
  // Chunk operator M_j = [[Acal, Z], [Qbar, R]] is (dk + C) x (dk + nk).
  __host__ __device__ int mrows() const { return dk + C; }
  __host__ __device__ int mcols() const { return dk + C * r_kv; }
};

// Workspace plan of the general (fp32-internal) path.
struct GeneralPlan {
  int slots;              // number of per-workgroup scratch slots of the prepare kernel
  size_t slot_floats;     // floats per slot
  size_t m_bytes;         // bytes of the chunk-operator buffer
  size_t total_bytes;
};

GeneralPlan general_plan(const Problem& p);

// General path: every shape the ABI accepts, fp32 internally.
hipError_t general_prepare(const Problem& p, const void* q, const void* k, const float* ld,
                           const void* A, const void* B, void* workspace, hipStream_t s);
hipError_t general_scan(const Problem& p, const void* workspace, const void* v, void* out,
                        float* Sfin, const float* S0, hipStream_t s);
hipError_t general_summaries(const Problem& p, const void* workspace, const void* v, float* sumA,
                             float* sumB, hipStream_t s);

// bf16 MFMA path: bf16 storage, C = 64, r_kv = 1, r_ab in {0, 1, 2}, d_k in {64, 128},
// d_v a multiple of 64.  The workspace holds the fragment-ordered chunk operators.
// fast_scan: with ckpt given, the state entering every chunk and the final
// state, [BH, N + 1, dk, dv], go there in bf16 (the values the scan's own
// products read) and no output rows are written (out is ignored).
bool fast_supported(const Problem& p);
// fast_workspace_bytes: the chunk operators.  fast_forward_bytes: the
// forward's workspace, the operators and (where fast_scan_segments(p) is 2:
// d_k = 64 with few heads) the split scan's scratch after them, which
// fast_scan then takes from its workspace argument (output instance only).
size_t fast_workspace_bytes(const Problem& p);
size_t fast_forward_bytes(const Problem& p);
int fast_scan_segments(const Problem& p);
hipError_t fast_prepare(const Problem& p, const void* q, const void* k, const float* ld,
                        const void* A, const void* B, void* workspace, hipStream_t s);
hipError_t fast_scan(const Problem& p, const void* workspace, const void* v, void* out, float* Sfin,
                     const float* S0, hipStream_t s, void* ckpt = nullptr);
// fast_prepare, which also writes the decay-scaled operands it forms, per
// chunk-head: Q~ = q e^{G_t}, K~ = k e^{-G_t} [C][dk], A~ = A e^{-G_t},
// B~ = B e^{G_{t-1}} [C r_ab][dk] (bf16, zero on padding tokens), and
// (r_ab > 0) the blocks of L = B~ A~^T (rows and columns token-major,
// rank-minor; entries with token(row) > token(col)): its 16x16 tiles below
// the diagonal blocks, bf16 row-major, tile (i, j) at i (i - 1) / 2 + j, and
// the inverses of I + L_ii, fp32 row-major [C r_ab / 16][16][16]; the
// chunk-local cumulative log-decay G in base 2, fp32 [C][dk] (padding tokens
// repeat the last token's), and e^{G} at the chunk's last token [dk] (the
// chunked backward's inputs).
struct PrepBwOut {
  void *qt, *kt, *at, *bt, *lt, *di, *gc, *gam;
};
hipError_t fast_prepare_bw(const Problem& p, const void* q, const void* k, const float* ld, const void* A,
                           const void* B, void* workspace, const PrepBwOut& out, hipStream_t s);
// Gating-chunk summaries for the query-conditioned composition, from the bf16
// prepare's operators of the 64-token problem p: per gating chunk of G
// consecutive chunks (G <= 4), Acal^T [dk][dk] and B^T [dv][dk] in bf16, the
// queries' incoming-state operator QB [64 G][dk] and zero-state outputs OI
// [64 G][dv] in fp32.  v is V [BH, T, dv] (r_kv = 1, d_v a multiple of 64).
hipError_t fast_gate_summaries(const Problem& p, int G, const void* workspace, const void* v, void* AT, void* BT,
                               float* QB, float* OI, hipStream_t s);
// Fused-parameter prepare (family 1: HDLA from log-lambda and beta, rank 2,
// per-channel decay; family 2: Gated DeltaNet from g and beta, rank 1,
// scalar decay).  The operator's value columns carry beta, so the scan reads
// the raw v.
hipError_t fast_prepare_fused(const Problem& p, int family, const void* q, const void* k, const float* ld,
                              const float* beta, void* workspace, hipStream_t s);

// Chunk operators as row-major fp32 (the general path's layout), for the kernels
// that read them (HLA composition, log-linear lift): from the bf16 MFMA prepare
// (expanded to fp32) where it takes the shape and the storage is bf16, else from
// the general prepare.  *M receives their address inside the workspace.
size_t f32_operators_bytes(const Problem& p);
hipError_t f32_operators(const Problem& p, const void* q, const void* k, const float* ld, const void* A,
                         const void* B, void* workspace, const float** M, hipStream_t s);

// Query-conditioned composition (HLA): d_k, d_v <= 128; p.C is the gating
// chunk.  Workspace: the chunk operators (bf16 64-token ones, or the general
// path's fp32 ones), then per gating chunk Acal^T, B^T, the queries'
// incoming-state operator and zero-state outputs (fp32).
struct HlaPlan {
  size_t gen_bytes, at_bytes, bt_bytes, qb_bytes, oi_bytes, total_bytes;
};
// Gating chunks of 64, 128 or 256 tokens on the bf16 path (from the 64-token
// MFMA operators), else a gating chunk equal to the summary chunk (<= 128).
bool hla_fast(const Problem& p);
bool hla_supported(const Problem& p);
HlaPlan hla_plan(const Problem& p);
hipError_t launch_hla(const Problem& p, const void* q, const void* k, const float* ld, const void* A,
                      const void* B, const void* v, const float* gates, float theta, void* out,
                      void* workspace, hipStream_t s);

// Log-linear lift on the general path's chunk operators: d_k, d_v <= 128,
// d_k + C <= 192, every inter-chunk level's state resident in LDS.  Workspace:
// the general path's, then (Z V)^T and the weighted chunk-local outputs.
struct LlPlan {
  size_t gen_bytes, zv_bytes, oi_bytes, total_bytes;
};
int loglinear_levels(int64_t T);
bool loglinear_supported(const Problem& p);
LlPlan loglinear_plan(const Problem& p);
hipError_t launch_loglinear(const Problem& p, const void* q, const void* k, const float* ld, const void* A,
                            const void* B, const void* v, const float* lam, void* out, void* workspace,
                            hipStream_t s);

// Chunked backward on bf16 MFMAs (bf16 storage, C = 64, r_kv = 1, r_ab <= 2,
// d_k, d_v in {64, 128}), from the chunk-boundary states ckpt (bf16 [BH, N + 1,
// dk, dv], fast_scan's boundary instance) and cotangents gend (bf16 [BH, N, dk,
// dv]); writes every gradient but dS0 (which the reverse boundary scan gives).
// ws: backward_chunked_bytes(p, ops == nullptr) bytes (own_ops false: without
// the scaled operands, which then come from elsewhere).
bool backward_chunked(const Problem& p);
size_t backward_chunked_bytes(const Problem& p, bool own_ops = true);
// Where, inside ws, fast_prepare_bw is to put the scaled operands.
PrepBwOut backward_chunked_prep_out(const Problem& p, void* ws);
// The scaled operands on their own, laid out from base: their bytes, and where
// each goes.
size_t backward_chunked_ops_bytes(const Problem& p);
PrepBwOut backward_chunked_ops_at(const Problem& p, void* base);
// The cotangent boundary scan of that route on bf16 MFMAs, over the bf16 MFMA
// prepare's operators M: gend[j] (the cotangent leaving chunk j, bf16) for
// every chunk, and dS0 (fp32).
hipError_t launch_backward_rscan(const Problem& p, const void* M, const void* dout, const float* dfinal, void* gend,
                                 float* dS0, hipStream_t s);
hipError_t launch_backward_chunked(const Problem& p, const void* q, const void* k, const void* v, const float* ld,
                                   const void* A, const void* B, const void* dout, const void* ckpt,
                                   const void* gend, float* dq, float* dK, float* dV, float* dld, float* dA,
                                   float* dB, void* ws, hipStream_t s, const PrepBwOut* ops = nullptr);

// Backward pass, token-serial with chunk checkpoints: d_k, d_v <= 128,
// r_ab <= 4, r_kv <= 2; gradients in fp32.
bool backward_supported(const Problem& p);
size_t backward_workspace_bytes(const Problem& p);
hipError_t launch_backward(const Problem& p, const void* q, const void* k, const void* v, const float* ld,
                           const void* A, const void* B, const void* dout, const float* dfinal, const float* S0,
                           float* dq, float* dK, float* dV, float* dld, float* dA, float* dB, float* dS0,
                           void* workspace, hipStream_t s);
// The training pair on the chunked route (backward_chunked(p)): a forward that
// also keeps, in a caller-owned buffer of backward_saved_bytes(p) bytes, the
// chunk operators and the decay-scaled operands its prepare forms and the
// state entering every chunk; and a backward that reads them there instead of
// forming them again (workspace: backward_saved_workspace_bytes(p)).  Both
// sizes are 0 off that route.
size_t backward_saved_bytes(const Problem& p);
size_t backward_saved_workspace_bytes(const Problem& p);
hipError_t launch_forward_train(const Problem& p, const void* q, const void* k, const void* v, const float* ld,
                                const void* A, const void* B, void* out, float* Sfin, const float* S0, void* saved,
                                hipStream_t s);
hipError_t launch_backward_saved(const Problem& p, const void* q, const void* k, const void* v, const float* ld,
                                 const void* A, const void* B, const void* dout, const float* dfinal,
                                 const void* saved, float* dq, float* dK, float* dV, float* dld,
                                 float* dA, float* dB, float* dS0, void* workspace, hipStream_t s);

hipError_t launch_step(const Problem& p, const void* q, const void* k, const void* v,
                       const float* ld, const void* A, const void* B, float* state, void* out,
                       hipStream_t s);
hipError_t launch_hdla_params(const Problem& p, const void* k, const void* v,
                              const float* log_lambda, const float* beta, void* A, void* B,
                              void* V_out, hipStream_t s);
hipError_t launch_gdn_params(const Problem& p, const void* k, const void* v, const float* g,
                             const float* beta, void* A, void* B, void* V_out, hipStream_t s);
hipError_t launch_decay_range(const Problem& p, const float* ld, float* chunk_max, hipStream_t s);
hipError_t launch_copy_state(const Problem& p, const float* S0, float* Sfin, hipStream_t s);

}  // namespace lattn
