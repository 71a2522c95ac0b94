/*
 * lattn.h -- C ABI of the MI355X (gfx950) chunk-wise forward of the generalized
 * linear-attention recurrence
 *
 *     S_t = (D_t - A_t B_t^T) S_{t-1} + K_t V_t^T,        o_t = S_t^T q_t
 *
 * (HDLA note, "Key design 3": decay of rank r_ab written as diagonal minus
 * low rank, write of rank r_kv; HDLA note, "Overall framework": chunks of C
 * tokens, chunk-state checkpoints, then per-chunk outputs).  D_t is diagonal,
 * D_t = diag(exp(log_decay_t)).  The three named decays map onto it as:
 *   GLA     r_ab = 0                 D_t = Diag(lambda_t)
 *   GDN     r_ab = 1 (scalar decay)  D_t = exp(g_t) I, A_t = exp(g_t) beta_t k_t, B_t = k_t
 *   HDLA    r_ab = 2                 D_t = Diag(lambda_t), A_t = [b k, b u], B_t = [u - b c k, k]
 *                                    (u = lambda (.) k, c = k^T u)
 * lattn_hdla_params / lattn_gdn_params build those operands on the device.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer to contiguous row-major memory,
 *   aligned to 16 bytes.  The caller owns all memory, including the
 *   workspace; the library allocates nothing, keeps no pointer after a call
 *   returns and holds no global mutable state, so calls are reentrant.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the legacy default
 *   stream) and is asynchronous: outputs are valid once the stream is
 *   synchronized.  No entry point synchronizes the host except
 *   lattn_check_decay_range.
 * - Results are deterministic: the kernels use no atomics and no
 *   order-dependent reductions.
 * - Arguments are validated on the host before anything is launched; a
 *   failure returns a negative lattn_status and lattn_last_error() gives a
 *   thread-local message.  NaN/Inf inputs are not checked and propagate.
 * - Element types: q, K, V, A, B and out share dims->dtype (fp32 or bf16);
 *   log_decay and every state tensor are fp32.  Internal accumulation is
 *   fp32 for both dtypes.
 * - No 1/sqrt(d_k) scale is applied: o_t uses the state after token t's
 *   update, as written above; a caller wanting a scaled readout pre-scales q.
 */
#ifndef LATTN_H_
#define LATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LATTN_OK = 0,
  LATTN_EINVAL = -1,        /* bad pointer, shape or rank                          */
  LATTN_EUNSUPPORTED = -2,  /* valid request outside what the kernels implement    */
  LATTN_EWORKSPACE = -3,    /* workspace missing or smaller than required         */
  LATTN_EHIP = -4,          /* a HIP runtime call or kernel launch failed         */
  LATTN_EDECAY_RANGE = -5   /* cumulative log-decay in one chunk exceeds the limit */
} lattn_status;

typedef enum { LATTN_FP32 = 0, LATTN_BF16 = 1 } lattn_dtype;

typedef enum {
  LATTN_DECAY_PER_CHANNEL = 0, /* log_decay [B,H,T,d_k]                 */
  LATTN_DECAY_SCALAR = 1       /* log_decay [B,H,T], broadcast over d_k */
} lattn_decay_mode;

typedef struct {
  int64_t batch;     /* B >= 1                                   */
  int64_t heads;     /* H >= 1                                   */
  int64_t seqlen;    /* T >= 0 (T = 0 is a no-op that copies the initial state) */
  int32_t d_k;       /* 16 <= d_k <= 256, multiple of 16         */
  int32_t d_v;       /* 16 <= d_v <= 256, multiple of 16         */
  lattn_dtype dtype;
  lattn_decay_mode decay_mode;
} lattn_dims;

/* Largest cumulative |log-decay| one chunk may accumulate (exp(80) ~ 5.5e34
 * stays inside fp32); lattn_check_decay_range tests inputs against it. */
#define LATTN_MAX_CHUNK_LOG_DECAY 80.0f

/*
 * lattn_chunk_fwd -- chunk-wise forward over a whole sequence (HDLA note,
 * "Key design 3": rank-generalized chunk-wise algorithm; HLA note, "Affine
 * maps and closure under composition": each chunk's exact affine summary).
 *
 *   q          [B,H,T,d_k]                 dtype
 *   k          K_t   [B,H,T,r_kv,d_k]      dtype
 *   v          V_t   [B,H,T,r_kv,d_v]      dtype
 *   log_decay  [B,H,T,d_k] or [B,H,T]      fp32 (per dims->decay_mode)
 *   A, B       [B,H,T,r_ab,d_k]            dtype; both NULL iff r_ab == 0
 *   r_ab       0..8;  r_kv 1..4
 *   chunk      C in {16, 32, 64, 128}; T need not be a multiple of C (the
 *              last chunk is shorter); C*r_ab <= 512 and C*r_kv <= 256
 *   out        [B,H,T,d_v]                 dtype (written)
 *   final_state    [B,H,d_k,d_v] fp32 (written); NULL = not returned
 *   initial_state  [B,H,d_k,d_v] fp32 (read);    NULL = zero state
 *   workspace  device scratch of at least lattn_chunk_fwd_workspace_size()
 *              bytes, owned by the caller, contents ignored on entry
 * Returns LATTN_OK or a negative lattn_status.
 */
int lattn_chunk_fwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                    const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
                    int chunk, void* out, float* final_state, const float* initial_state,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace lattn_chunk_fwd needs for these arguments (0 on invalid
 * arguments; host-only, launches nothing). */
size_t lattn_chunk_fwd_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk);

/* Size of the library's static per-GPU scratch used by lattn_chunk_fwd_noalloc. */
#define LATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * lattn_chunk_fwd_noalloc -- lattn_chunk_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments and results as lattn_chunk_fwd, minus
 * the workspace: the chunk operators go to a static device array of
 * LATTN_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
 * the process ends (its address is looked up once per device, on the first
 * call with that device current).  The call allocates nothing and calls no
 * allocating routine.
 *   - A problem whose lattn_chunk_fwd_workspace_size() exceeds
 *     LATTN_NOALLOC_SCRATCH_BYTES is rejected with LATTN_EWORKSPACE before
 *     any launch (use lattn_chunk_fwd with a caller-owned workspace).
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents (the kernels overwrite what they read, so nothing needs
 *     clearing).  Calls that overlap in time on one GPU (different streams or
 *     host threads without ordering) race on it; order them on one stream.
 */
int lattn_chunk_fwd_noalloc(const lattn_dims* dims, const void* q, const void* k, const void* v,
                            const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
                            int chunk, void* out, float* final_state, const float* initial_state,
                            hipStream_t stream);

/* Host-only validation of lattn_chunk_fwd's arguments (the same checks the
 * call performs before launching).  Pointers are only tested for NULL and
 * 16-byte alignment, never dereferenced. */
int lattn_chunk_fwd_check(const lattn_dims* dims, const void* q, const void* k, const void* v,
                          const float* log_decay, const void* A, const void* B, int r_ab,
                          int r_kv, int chunk, const void* out, const void* workspace,
                          size_t workspace_bytes);

/*
 * The two stages lattn_chunk_fwd runs, callable one by one (same arguments,
 * same workspace; calling both in order on one stream is lattn_chunk_fwd):
 *
 * lattn_chunk_prepare -- for every chunk in parallel, the exact chunk operator
 *   built from q, K, A, B and the log-decay (HDLA note, "Key design 3": the
 *   rank-generalized WY form; HLA note, "Affine maps and closure under
 *   composition"), written into the workspace.  v is not read.
 * lattn_chunk_scan -- walks the chunks of each (batch, head) in order,
 *   carrying the d_k x d_v state: per chunk one product gives the next state
 *   and the chunk's outputs (HDLA note, "Overall framework": serial chunk-state
 *   checkpoints, then chunk outputs).  Reads v and the workspace written by
 *   lattn_chunk_prepare with the same dims, ranks and chunk.  On the bf16 path
 *   at d_k = 64 with few heads it splits each sequence into up to three
 *   segments walked side by side: each later segment from a zero state beside
 *   the product of its chunks' transitions (the composition of the chunks'
 *   affine maps, HLA note, "Affine maps and closure under composition"), then
 *   its outputs and final state corrected with the state entering it; that
 *   part of the workspace is scratch for the call.
 */
int lattn_chunk_prepare(const lattn_dims* dims, const void* q, const void* k,
                        const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
                        int chunk, void* workspace, size_t workspace_bytes, hipStream_t stream);

int lattn_chunk_scan(const lattn_dims* dims, const void* v, int r_ab, int r_kv, int chunk,
                     void* out, float* final_state, const float* initial_state, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * lattn_chunk_summaries -- the exact affine pair of every chunk (HLA note,
 * "Affine maps and closure under composition"): after chunk j,
 * S_j = sum_A[j] S_{j-1} + sum_B[j].  Inputs as lattn_chunk_fwd (q unused).
 *   sum_A [B,H,N,d_k,d_k] fp32, sum_B [B,H,N,d_k,d_v] fp32, N = ceil(T/C).
 * Needs lattn_chunk_summaries_workspace_size() bytes of workspace.
 */
int lattn_chunk_summaries(const lattn_dims* dims, const void* k, const void* v,
                          const float* log_decay, const void* A, const void* B, int r_ab,
                          int r_kv, int chunk, float* sum_A, float* sum_B, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace lattn_chunk_summaries needs (0 on invalid arguments). */
size_t lattn_chunk_summaries_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk);

/*
 * lattn_hla_fwd -- query-conditioned composition of the exact chunk transitions
 * (HLA note, "Core method" and "Method steps", steps 2, 5 and 7).  For query
 * token i in chunk c = i / chunk, from a zero state, every earlier chunk j in
 * time order is applied with the query's gate w = gates[i, j]:
 *   S <- ((1 - w) I + w A_j) S + w B_j      (A_j, B_j: the chunk's exact pair),
 * a gate below theta counting as 0 (no renormalisation); then the tokens of
 * chunk c up to and including i advance S by the recurrence of
 * lattn_chunk_fwd, and out[i] = S^T q_i (no 1/sqrt(d_k) scale).  All gates 1
 * give lattn_chunk_fwd's output; all gates 0 give each chunk's output from a
 * zero state.
 * Inputs as lattn_chunk_fwd, plus
 *   gates [B,H,T,N] fp32, N = ceil(T / chunk); entries j >= i / chunk unused.
 * out [B,H,T,d_v] in dims->dtype.  No state in or out (the history of every
 * query starts from zero).  d_k and d_v must be <= 128 (LATTN_EUNSUPPORTED).
 * Arithmetic is fp32 for both storage dtypes.
 * Needs lattn_hla_fwd_workspace_size() bytes of caller-owned workspace (the
 * chunk operators and, per chunk, A_j^T, B_j^T and its zero-state outputs).
 * Validation, ownership and stream ordering as lattn_chunk_fwd; NaN gates
 * propagate.
 */
int lattn_hla_fwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                  const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
                  int chunk, const float* gates, float theta, void* out, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace lattn_hla_fwd needs (0 on invalid arguments). */
size_t lattn_hla_fwd_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk);

/*
 * lattn_loglinear_fwd -- log-linear lift of the recurrence (Log-Linear note,
 * "Key design" 1-3).  The prefix of position t (counted from 0) is split
 * Fenwick-style: the token itself at level 0, then from the right one bucket
 * per set bit 2^(l-1) of t at level l, so key s < t sits at level
 * l(t, s) = (highest bit where t and s differ) + 1.  Every key is weighted by
 * the query's weight for its level, with the recurrence's transport
 * Phi(t, s) = P_t ... P_{s+1}, P = D - A B^T, between them:
 *   out[t] = sum_{s <= t} lambda[t, l(t, s)] (Phi(t, s) K_s V_s^T)^T q_t.
 * lambda all 1 gives lattn_chunk_fwd's output.
 * Inputs as lattn_chunk_fwd (zero initial state), plus
 *   lambda [B,H,T,L] fp32, L = lattn_loglinear_levels(T).
 * out [B,H,T,d_v] in dims->dtype; no final state (each level keeps its own).
 * Needs d_k, d_v <= 128 and d_k + chunk <= 192 (LATTN_EUNSUPPORTED); the
 * per-level states of one (batch, head) slice live in LDS, which bounds the
 * number of chunks at 2^17 for d_k = 128.  Arithmetic: for bf16 storage with
 * d_k = 64, chunk 64, r_kv = 1, r_ab <= 2, d_v a multiple of 64 and at most
 * 2^16 chunks, bf16 MFMA operands (the chunk operators and the level states
 * rounded to bf16) with fp32 accumulation and fp32 level states; otherwise
 * fp32 (bf16 storage at other shapes: operators rounded to bf16 where the bf16
 * MFMA prepare forms them, as for lattn_chunk_fwd).
 * Needs lattn_loglinear_fwd_workspace_size() bytes of caller-owned workspace.
 * Validation, ownership and stream ordering as lattn_chunk_fwd.
 */
int lattn_loglinear_fwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                        const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
                        int chunk, const float* lambda, void* out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace lattn_loglinear_fwd needs (0 on invalid arguments). */
size_t lattn_loglinear_fwd_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk);

/* Levels L of a sequence of seqlen tokens: 1 + bit length of (seqlen - 1); 0 for seqlen 0. */
int lattn_loglinear_levels(int64_t seqlen);

/*
 * lattn_chunk_bwd -- backward pass of lattn_chunk_fwd: the gradients of
 *   L = sum_t <dout_t, out_t> + <dfinal, final_state>
 * with respect to every input, by the chain rule of the recurrence (the HDLA
 * note, "Key design 3", trains through it; the pages give no backward
 * formulas).  The state entering and the cotangent leaving every chunk come
 * from two chunk-level scans over the forward's chunk operators; then every
 * chunk's gradients are formed independently, all chunks in parallel:
 *  - bf16 storage, chunk 64, r_kv = 1, r_ab <= 2, d_k and d_v in {64, 128}:
 *    matrix products through the forward's decay-scaled WY factors (a forward
 *    and an adjoint unit-lower solve per chunk) on bf16 MFMAs with fp32
 *    accumulation; operands and the chunk-boundary states and cotangents are
 *    rounded to bf16 as in the bf16 forward;
 *  - every other shape: each chunk's tokens walked in reverse in fp32.
 * As for lattn_chunk_fwd, every chunk's cumulative -log-decay must stay within
 * LATTN_MAX_CHUNK_LOG_DECAY (lattn_check_decay_range).
 * Inputs as lattn_chunk_fwd (initial_state NULL = zero), plus
 *   dout [B,H,T,d_v] in dims->dtype;  dfinal [B,H,d_k,d_v] fp32 or NULL (zero).
 * Outputs, fp32, each in its input's layout: dq [B,H,T,d_k]; dk [B,H,T,r_kv,d_k];
 *   dv [B,H,T,r_kv,d_v]; dlog_decay [B,H,T,d_k] or [B,H,T]; dA, dB [B,H,T,r_ab,d_k]
 *   (NULL iff r_ab == 0); dinitial_state [B,H,d_k,d_v].
 * Needs d_k, d_v <= 128, r_ab <= 4, r_kv <= 2 (LATTN_EUNSUPPORTED), and
 * lattn_chunk_bwd_workspace_size() bytes of caller-owned workspace.
 * Validation, ownership and stream ordering as lattn_chunk_fwd.
 */
int lattn_chunk_bwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                    const float* log_decay, const void* A, const void* B, int r_ab, int r_kv, int chunk,
                    const void* dout, const float* dfinal, const float* initial_state, float* dq, float* dk,
                    float* dv, float* dlog_decay, float* dA, float* dB, float* dinitial_state, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace lattn_chunk_bwd needs (0 on invalid arguments). */
size_t lattn_chunk_bwd_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk);

/*
 * lattn_chunk_fwd_train / lattn_chunk_bwd_saved -- the training pair: the
 * forward of lattn_chunk_fwd, which also keeps in `saved` what the chunked
 * backward would otherwise form again from the inputs (the chunk operators
 * M_j, the decay-scaled operands q e^{G}, k e^{-G}, A e^{-G}, B e^{G_{t-1}} and
 * the state entering every chunk; the HDLA note, "Key design 3", trains
 * through the chunk-wise form), and the backward of lattn_chunk_bwd reading
 * them there.
 * Only on the chunked backward's route: bf16 storage, chunk 64, r_kv = 1,
 * r_ab <= 2, d_k and d_v in {64, 128} (LATTN_EUNSUPPORTED elsewhere; there
 * lattn_chunk_fwd_train_saved_size returns 0, and a caller uses
 * lattn_chunk_fwd and lattn_chunk_bwd).
 * lattn_chunk_fwd_train: arguments and results as lattn_chunk_fwd (out and
 *   final_state computed by the same kernels, so equal to its results, except
 *   at the shapes where lattn_chunk_fwd splits its state scan into sequence
 *   segments, d_k = 64 with few heads, which rounds differently), plus
 *   saved: caller-owned device memory of lattn_chunk_fwd_train_saved_size()
 *   bytes, fully written; no other workspace is needed.
 * lattn_chunk_bwd_saved: arguments and results as lattn_chunk_bwd (equal to
 *   its results), but no initial_state (the saved states carry it), plus
 *   saved as the forward with the same inputs left it (read only; the caller
 *   keeps it unchanged in between), and
 *   lattn_chunk_bwd_saved_workspace_size() bytes of caller-owned workspace.
 * The buffer's content is this library's private layout; it is valid for
 * the one set of inputs (q, k, log_decay, A, B and the shapes) it was made
 * from.  Validation, ownership and stream ordering as lattn_chunk_fwd.
 */
int lattn_chunk_fwd_train(const lattn_dims* dims, const void* q, const void* k, const void* v,
                          const float* log_decay, const void* A, const void* B, int r_ab, int r_kv, int chunk,
                          void* out, float* final_state, const float* initial_state, void* saved,
                          size_t saved_bytes, hipStream_t stream);
int lattn_chunk_bwd_saved(const lattn_dims* dims, const void* q, const void* k, const void* v,
                          const float* log_decay, const void* A, const void* B, int r_ab, int r_kv, int chunk,
                          const void* dout, const float* dfinal, const void* saved, size_t saved_bytes, float* dq, float* dk, float* dv, float* dlog_decay, float* dA,
                          float* dB, float* dinitial_state, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);
/* Bytes of `saved` and of the saved-state backward's workspace (0 off the
 * route or on invalid arguments). */
size_t lattn_chunk_fwd_train_saved_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk);
size_t lattn_chunk_bwd_saved_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk);

/*
 * lattn_step -- one recurrent token for decoding (HLA note, "Reproduction":
 * a prefill algorithm and a dynamic decoding algorithm; the recurrence of
 * HDLA note, "Key design 3", applied once):
 *   state <- (D - A B^T) state + K V^T,   out = state^T q.
 * dims->seqlen must be 1.  q [B,H,d_k]; k [B,H,r_kv,d_k]; v [B,H,r_kv,d_v];
 * log_decay [B,H,d_k] or [B,H]; A, B [B,H,r_ab,d_k] (NULL iff r_ab == 0);
 * state [B,H,d_k,d_v] fp32 read and written in place; out [B,H,d_v] dtype.
 */
int lattn_step(const lattn_dims* dims, const void* q, const void* k, const void* v,
               const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
               float* state, void* out, hipStream_t stream);

/*
 * lattn_hdla_params -- HDLA's decay written as diagonal minus rank 2 (HDLA
 * note, "Key design 2" and "Key design 3"), on the device:
 *   u = exp(log_lambda) (.) k,  c = k^T u,
 *   A = [beta k, beta u],  B = [u - beta c k, k],  V_out = beta v.
 * k [B,H,T,d_k] dtype; v [B,H,T,d_v] dtype; log_lambda [B,H,T,d_k] fp32;
 * beta [B,H,T] fp32.  Outputs (dtype): A, B [B,H,T,2,d_k]; V_out [B,H,T,1,d_v].
 * The generic call then takes K = k, log_decay = log_lambda, r_ab = 2, r_kv = 1.
 * dims->decay_mode must be LATTN_DECAY_PER_CHANNEL.
 */
int lattn_hdla_params(const lattn_dims* dims, const void* k, const void* v,
                      const float* log_lambda, const float* beta, void* A, void* B, void* V_out,
                      hipStream_t stream);

/*
 * lattn_gdn_params -- Gated DeltaNet's decay exp(g)(I - beta k k^T) written as
 * exp(g) I - (exp(g) beta k) k^T (HLA note, "Prerequisites: Gated DeltaNet"):
 *   A = exp(g) beta k,  B = k,  V_out = beta v.
 * k [B,H,T,d_k]; v [B,H,T,d_v] dtype; g, beta [B,H,T] fp32.
 * Outputs (dtype): A, B [B,H,T,1,d_k]; V_out [B,H,T,1,d_v].  The generic call
 * then takes K = k, log_decay = g (scalar mode), r_ab = 1, r_kv = 1.
 */
int lattn_gdn_params(const lattn_dims* dims, const void* k, const void* v, const float* g,
                     const float* beta, void* A, void* B, void* V_out, hipStream_t stream);

/*
 * lattn_hdla_chunk_fwd -- the whole HDLA forward from its raw parameters, with
 * the decay operands formed inside the chunk kernel instead of materialized
 * (HDLA note, "Key design 2": the Householder congruence of a sigmoid-gated
 * diagonal; "Key design 3": its diagonal-minus-rank-2 form and the chunk-wise
 * algorithm).  Computes exactly what lattn_hdla_params followed by
 * lattn_chunk_fwd (r_ab = 2, r_kv = 1, K = k, log_decay = log_lambda)
 * computes, up to rounding: the decay operands and beta v are never rounded
 * to the storage dtype.
 *   q, k [B,H,T,d_k] dtype; v [B,H,T,d_v] dtype; log_lambda [B,H,T,d_k] fp32;
 *   beta [B,H,T] fp32; out [B,H,T,d_v] dtype; final_state, initial_state as
 *   lattn_chunk_fwd.  dims->decay_mode must be LATTN_DECAY_PER_CHANNEL.
 * Workspace: lattn_hdla_chunk_fwd_workspace_size() bytes.  Errors as
 * lattn_chunk_fwd.
 */
int lattn_hdla_chunk_fwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                         const float* log_lambda, const float* beta, int chunk, void* out,
                         float* final_state, const float* initial_state, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);
size_t lattn_hdla_chunk_fwd_workspace_size(const lattn_dims* dims, int chunk);

/*
 * lattn_gdn_chunk_fwd -- the whole Gated DeltaNet forward from its raw
 * parameters (HLA note, "Prerequisites: Gated DeltaNet": decay
 * exp(g)(I - beta k k^T), write beta k v^T), decay operands formed inside the
 * chunk kernel.  Same result as lattn_gdn_params followed by lattn_chunk_fwd
 * (r_ab = 1, r_kv = 1, K = k, log_decay = g), up to rounding.
 *   q, k [B,H,T,d_k] dtype; v [B,H,T,d_v] dtype; g, beta [B,H,T] fp32.
 *   dims->decay_mode must be LATTN_DECAY_SCALAR.
 */
int lattn_gdn_chunk_fwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, int chunk, void* out,
                        float* final_state, const float* initial_state, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);
size_t lattn_gdn_chunk_fwd_workspace_size(const lattn_dims* dims, int chunk);

/*
 * lattn_decay_range -- per chunk, the largest -G over the chunk's tokens and
 * channels, where G is the chunk-local inclusive cumulative log-decay.  The
 * chunk-wise form scales operands by exp(-G); the result must stay below
 * LATTN_MAX_CHUNK_LOG_DECAY.  chunk_max [B,H,N] fp32 (written); an entry is
 * NaN when the chunk's log-decay holds a NaN.  Asynchronous.
 */
int lattn_decay_range(const lattn_dims* dims, const float* log_decay, int chunk,
                      float* chunk_max, hipStream_t stream);

/* Synchronous convenience check built on lattn_decay_range: returns LATTN_OK
 * or LATTN_EDECAY_RANGE (a chunk beyond the limit, or a NaN log-decay).
 * `scratch` is caller-owned device memory of B*H*ceil(T/C) floats that
 * receives the per-chunk maxima: the library allocates nothing, so the
 * buffer the check reduces on the host comes from the caller. */
int lattn_check_decay_range(const lattn_dims* dims, const float* log_decay, int chunk,
                            float* scratch, hipStream_t stream);

/* Name of the kernel pair lattn_chunk_fwd runs for these arguments (host-only;
 * "" on invalid arguments): "general_fp32" (fp32 arithmetic, every shape) or
 * "mfma_bf16" (bf16 MFMA with fp32 accumulation). */
const char* lattn_chunk_fwd_kernels(const lattn_dims* dims, int r_ab, int r_kv, int chunk);

/* Static description of a status code. */
const char* lattn_status_str(int status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* lattn_last_error(void);

/* Library version string. */
const char* lattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LATTN_H_ */
