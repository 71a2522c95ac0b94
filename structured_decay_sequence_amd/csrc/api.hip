// C ABI of liblattn: host-side validation, workspace planning and dispatch.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/lattn.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return LATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const lattn_dims* d) {
  if (d == nullptr) return fail(LATTN_EINVAL, "dims is NULL");
  if (d->batch < 1 || d->heads < 1 || d->seqlen < 0)
    return fail(LATTN_EINVAL, "batch (%lld) and heads (%lld) must be >= 1, seqlen (%lld) >= 0",
                (long long)d->batch, (long long)d->heads, (long long)d->seqlen);
  if (d->d_k < 16 || d->d_k > 256 || d->d_k % 16 != 0)
    return fail(LATTN_EINVAL, "d_k = %d must be a multiple of 16 in [16, 256]", d->d_k);
  if (d->d_v < 16 || d->d_v > 256 || d->d_v % 16 != 0)
    return fail(LATTN_EINVAL, "d_v = %d must be a multiple of 16 in [16, 256]", d->d_v);
  if (d->dtype != LATTN_FP32 && d->dtype != LATTN_BF16)
    return fail(LATTN_EINVAL, "dtype = %d is neither LATTN_FP32 nor LATTN_BF16", (int)d->dtype);
  if (d->decay_mode != LATTN_DECAY_PER_CHANNEL && d->decay_mode != LATTN_DECAY_SCALAR)
    return fail(LATTN_EINVAL, "decay_mode = %d is not a lattn_decay_mode", (int)d->decay_mode);
  return LATTN_OK;
}

int check_ranks(int r_ab, int r_kv) {
  if (r_ab < 0 || r_ab > 8) return fail(LATTN_EINVAL, "r_ab = %d must be in [0, 8]", r_ab);
  if (r_kv < 1 || r_kv > 4) return fail(LATTN_EINVAL, "r_kv = %d must be in [1, 4]", r_kv);
  return LATTN_OK;
}

int check_chunk(int chunk, int r_ab, int r_kv) {
  if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128)
    return fail(LATTN_EINVAL, "chunk = %d must be one of 16, 32, 64, 128", chunk);
  if (chunk * r_ab > 512)
    return fail(LATTN_EUNSUPPORTED, "chunk * r_ab = %d exceeds 512", chunk * r_ab);
  if (chunk * r_kv > 256)
    return fail(LATTN_EUNSUPPORTED, "chunk * r_kv = %d exceeds 256", chunk * r_kv);
  return LATTN_OK;
}

int check_ptr(const void* p, const char* name, bool required) {
  if (p == nullptr) {
    if (required) return fail(LATTN_EINVAL, "%s is NULL", name);
    return LATTN_OK;
  }
  if (!aligned16(p)) return fail(LATTN_EINVAL, "%s is not 16-byte aligned", name);
  return LATTN_OK;
}

lattn::Problem make_problem(const lattn_dims* d, int r_ab, int r_kv, int chunk) {
  lattn::Problem p{};
  p.BH = d->batch * d->heads;
  p.T = d->seqlen;
  p.dk = d->d_k;
  p.dv = d->d_v;
  p.r_ab = r_ab;
  p.r_kv = r_kv;
  p.C = chunk;
  p.N = chunk > 0 ? (d->seqlen + chunk - 1) / chunk : 0;
  p.scalar = d->decay_mode == LATTN_DECAY_SCALAR ? 1 : 0;
  p.bf16 = d->dtype == LATTN_BF16 ? 1 : 0;
  return p;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
  return LATTN_OK;
}

#define LATTN_TRY(expr)        \
  do {                         \
    const int _rc = (expr);    \
    if (_rc != LATTN_OK) return _rc; \
  } while (0)

int check_operands(const lattn_dims* dims, const void* k, const void* v, const float* log_decay,
                   const void* A, const void* B, int r_ab, int r_kv, int chunk) {
  LATTN_TRY(check_dims(dims));
  LATTN_TRY(check_ranks(r_ab, r_kv));
  LATTN_TRY(check_chunk(chunk, r_ab, r_kv));
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(k, "k", need));
  LATTN_TRY(check_ptr(v, "v", need));
  LATTN_TRY(check_ptr(log_decay, "log_decay", need));
  if (r_ab == 0) {
    if (A != nullptr || B != nullptr) return fail(LATTN_EINVAL, "A and B must be NULL when r_ab == 0");
  } else {
    LATTN_TRY(check_ptr(A, "A", need));
    LATTN_TRY(check_ptr(B, "B", need));
  }
  return LATTN_OK;
}

hipError_t run_prepare(const lattn::Problem& p, const void* q, const void* k, const float* ld,
                       const void* A, const void* B, void* ws, hipStream_t s) {
  if (lattn::fast_supported(p)) return lattn::fast_prepare(p, q, k, ld, A, B, ws, s);
  return lattn::general_prepare(p, q, k, ld, A, B, ws, s);
}

hipError_t run_scan(const lattn::Problem& p, void* ws, const void* v, void* out, float* Sfin,
                    const float* S0, hipStream_t s) {
  if (lattn::fast_supported(p)) return lattn::fast_scan(p, ws, v, out, Sfin, S0, s);
  return lattn::general_scan(p, ws, v, out, Sfin, S0, s);
}

// Static scratch of lattn_chunk_fwd_noalloc: each GPU holds its own copy of
// this array, at its own address, for the life of the process.  In host code
// the name stands for a host-side shadow, not device memory, so host code
// only ever uses the device address looked up below.
__device__ __align__(256) unsigned char scratch[LATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current GPU's scratch, looked up once per device with
// that device current.
int noalloc_scratch(void** ptr) {
  int dev = -1;
  LATTN_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(LATTN_EHIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    LATTN_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (p == nullptr) return fail(LATTN_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return LATTN_OK;
}

// The fused family forwards (HDLA, Gated DeltaNet from their raw parameters).
// On the MFMA path the decay operands are formed inside the prepare kernel;
// elsewhere the parameter kernel materializes A, B and beta v in the front of
// the workspace and the generic path runs on them.
struct FusedPlan {
  lattn::Problem p;
  bool fast;
  size_t a_bytes, v_bytes, gen_offset, total;
};

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

FusedPlan fused_plan(const lattn_dims* d, int family, int chunk) {
  FusedPlan f{};
  const int r_ab = family == 1 ? 2 : 1;
  f.p = make_problem(d, r_ab, 1, chunk);
  f.fast = lattn::fast_supported(f.p);
  if (f.fast) {
    f.total = lattn::fast_forward_bytes(f.p);
    return f;
  }
  const size_t e = f.p.bf16 ? 2 : 4;
  const size_t tok = static_cast<size_t>(f.p.BH * f.p.T);
  f.a_bytes = round256(tok * r_ab * f.p.dk * e);
  f.v_bytes = round256(tok * f.p.dv * e);
  f.gen_offset = 2 * f.a_bytes + f.v_bytes;
  f.total = f.gen_offset + lattn::general_plan(f.p).total_bytes;
  return f;
}

int check_fused(int family, const lattn_dims* dims, int chunk) {
  LATTN_TRY(check_dims(dims));
  const int r_ab = family == 1 ? 2 : 1;
  LATTN_TRY(check_chunk(chunk, r_ab, 1));
  if (family == 1 && dims->decay_mode != LATTN_DECAY_PER_CHANNEL)
    return fail(LATTN_EINVAL, "the HDLA forward needs LATTN_DECAY_PER_CHANNEL");
  if (family == 2 && dims->decay_mode != LATTN_DECAY_SCALAR)
    return fail(LATTN_EINVAL, "the Gated DeltaNet forward needs LATTN_DECAY_SCALAR");
  return LATTN_OK;
}

int fused_fwd(int family, const lattn_dims* dims, const void* q, const void* k, const void* v,
              const float* ld, const float* beta, int chunk, void* out, float* final_state,
              const float* initial_state, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  LATTN_TRY(check_fused(family, dims, chunk));
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(q, "q", need));
  LATTN_TRY(check_ptr(k, "k", need));
  LATTN_TRY(check_ptr(v, "v", need));
  LATTN_TRY(check_ptr(ld, family == 1 ? "log_lambda" : "g", need));
  LATTN_TRY(check_ptr(beta, "beta", need));
  LATTN_TRY(check_ptr(out, "out", need));
  LATTN_TRY(check_ptr(final_state, "final_state", false));
  LATTN_TRY(check_ptr(initial_state, "initial_state", false));
  const FusedPlan f = fused_plan(dims, family, chunk);
  if (f.p.T == 0) return hip_status(lattn::launch_copy_state(f.p, initial_state, final_state, stream), "copy state");
  if (workspace == nullptr || workspace_bytes < f.total)
    return fail(LATTN_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, f.total);
  LATTN_TRY(check_ptr(workspace, "workspace", true));
  if (f.fast) {
    LATTN_TRY(hip_status(lattn::fast_prepare_fused(f.p, family, q, k, ld, beta, workspace, stream), "prepare launch"));
    LATTN_TRY(hip_status(lattn::fast_scan(f.p, workspace, v, out, final_state, initial_state, stream), "scan launch"));
    return ok();
  }
  char* ws = static_cast<char*>(workspace);
  void* A = ws;
  void* B = ws + f.a_bytes;
  void* V = ws + 2 * f.a_bytes;
  void* gws = ws + f.gen_offset;
  const lattn::Problem pp = make_problem(dims, family == 1 ? 2 : 1, 1, 1);
  if (family == 1)
    LATTN_TRY(hip_status(lattn::launch_hdla_params(pp, k, v, ld, beta, A, B, V, stream), "hdla params launch"));
  else
    LATTN_TRY(hip_status(lattn::launch_gdn_params(pp, k, v, ld, beta, A, B, V, stream), "gdn params launch"));
  LATTN_TRY(hip_status(run_prepare(f.p, q, k, ld, A, B, gws, stream), "prepare launch"));
  LATTN_TRY(hip_status(run_scan(f.p, gws, V, out, final_state, initial_state, stream), "scan launch"));
  return ok();
}

// The gating chunk of lattn_hla_fwd may also be 256 tokens (the HLA note's
// length) where the bf16 path composes it from 64-token operators.
int check_hla_chunk(const lattn_dims* dims, int r_ab, int r_kv, int chunk) {
  if (chunk != 256) return check_chunk(chunk, r_ab, r_kv);
  LATTN_TRY(check_chunk(64, r_ab, r_kv));
  if (!lattn::hla_fast(make_problem(dims, r_ab, r_kv, chunk)))
    return fail(LATTN_EUNSUPPORTED, "a 256-token gating chunk needs bf16 storage, d_k 64 or 128, r_kv 1, r_ab <= 2 "
                "and d_v a multiple of 64 up to 128");
  return LATTN_OK;
}

// The pointer checks both backward entry points share.
int check_bwd_args(const lattn_dims* dims, const void* q, const void* k, const void* v, const float* log_decay,
                   const void* A, const void* B, int r_ab, int r_kv, int chunk, const void* dout,
                   const float* dfinal, const float* initial_state, const float* dq, const float* dk,
                   const float* dv, const float* dlog_decay, const float* dA, const float* dB,
                   const float* dinitial_state) {
  LATTN_TRY(check_operands(dims, k, v, log_decay, A, B, r_ab, r_kv, chunk));
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(q, "q", need));
  LATTN_TRY(check_ptr(dout, "dout", need));
  LATTN_TRY(check_ptr(dfinal, "dfinal", false));
  LATTN_TRY(check_ptr(initial_state, "initial_state", false));
  LATTN_TRY(check_ptr(dq, "dq", need));
  LATTN_TRY(check_ptr(dk, "dk", need));
  LATTN_TRY(check_ptr(dv, "dv", need));
  LATTN_TRY(check_ptr(dlog_decay, "dlog_decay", need));
  LATTN_TRY(check_ptr(dinitial_state, "dinitial_state", true));
  if (r_ab == 0) {
    if (dA != nullptr || dB != nullptr) return fail(LATTN_EINVAL, "dA and dB must be NULL when r_ab == 0");
  } else {
    LATTN_TRY(check_ptr(dA, "dA", need));
    LATTN_TRY(check_ptr(dB, "dB", need));
  }
  return LATTN_OK;
}

// The training pair's route: the chunked backward's shapes.
int check_train_route(const lattn::Problem& p, const char* who) {
  if (!lattn::backward_chunked(p))
    return fail(LATTN_EUNSUPPORTED, "%s needs bf16 storage, chunk 64, r_kv 1, r_ab <= 2 and d_k, d_v in {64, 128} "
                "(got d_k %d, d_v %d, r_ab %d, r_kv %d, chunk %d); use lattn_chunk_fwd and lattn_chunk_bwd", who,
                p.dk, p.dv, p.r_ab, p.r_kv, p.C);
  return LATTN_OK;
}

}  // namespace

extern "C" {

int lattn_hdla_chunk_fwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                         const float* log_lambda, const float* beta, int chunk, void* out,
                         float* final_state, const float* initial_state, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return fused_fwd(1, dims, q, k, v, log_lambda, beta, chunk, out, final_state, initial_state, workspace,
                   workspace_bytes, stream);
}

size_t lattn_hdla_chunk_fwd_workspace_size(const lattn_dims* dims, int chunk) {
  if (check_fused(1, dims, chunk) != LATTN_OK) return 0;
  return fused_plan(dims, 1, chunk).total;
}

int lattn_gdn_chunk_fwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, int chunk, void* out,
                        float* final_state, const float* initial_state, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  return fused_fwd(2, dims, q, k, v, g, beta, chunk, out, final_state, initial_state, workspace,
                   workspace_bytes, stream);
}

size_t lattn_gdn_chunk_fwd_workspace_size(const lattn_dims* dims, int chunk) {
  if (check_fused(2, dims, chunk) != LATTN_OK) return 0;
  return fused_plan(dims, 2, chunk).total;
}


const char* lattn_version(void) { return "lattn 0.1 (gfx950)"; }

const char* lattn_status_str(int status) {
  switch (status) {
    case LATTN_OK: return "LATTN_OK";
    case LATTN_EINVAL: return "LATTN_EINVAL: invalid argument";
    case LATTN_EUNSUPPORTED: return "LATTN_EUNSUPPORTED: valid but unsupported configuration";
    case LATTN_EWORKSPACE: return "LATTN_EWORKSPACE: workspace missing or too small";
    case LATTN_EHIP: return "LATTN_EHIP: HIP runtime error";
    case LATTN_EDECAY_RANGE: return "LATTN_EDECAY_RANGE: chunk cumulative log-decay out of range";
    default: return "unknown lattn status";
  }
}

const char* lattn_last_error(void) { return g_last_error.c_str(); }

const char* lattn_chunk_fwd_kernels(const lattn_dims* dims, int r_ab, int r_kv, int chunk) {
  if (check_dims(dims) != LATTN_OK || check_ranks(r_ab, r_kv) != LATTN_OK ||
      check_chunk(chunk, r_ab, r_kv) != LATTN_OK)
    return "";
  return lattn::fast_supported(make_problem(dims, r_ab, r_kv, chunk)) ? "mfma_bf16" : "general_fp32";
}

size_t lattn_chunk_fwd_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk) {
  if (check_dims(dims) != LATTN_OK || check_ranks(r_ab, r_kv) != LATTN_OK ||
      check_chunk(chunk, r_ab, r_kv) != LATTN_OK)
    return 0;
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, chunk);
  return lattn::fast_supported(p) ? lattn::fast_forward_bytes(p) : lattn::general_plan(p).total_bytes;
}

size_t lattn_chunk_summaries_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk) {
  if (check_dims(dims) != LATTN_OK || check_ranks(r_ab, r_kv) != LATTN_OK ||
      check_chunk(chunk, r_ab, r_kv) != LATTN_OK)
    return 0;
  return lattn::general_plan(make_problem(dims, r_ab, r_kv, chunk)).total_bytes;
}

size_t lattn_hla_fwd_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk) {
  if (check_dims(dims) != LATTN_OK || check_ranks(r_ab, r_kv) != LATTN_OK ||
      check_hla_chunk(dims, r_ab, r_kv, chunk) != LATTN_OK)
    return 0;
  return lattn::hla_plan(make_problem(dims, r_ab, r_kv, chunk)).total_bytes;
}

int lattn_hla_fwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                  const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
                  int chunk, const float* gates, float theta, void* out, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  LATTN_TRY(check_dims(dims));
  LATTN_TRY(check_hla_chunk(dims, r_ab, r_kv, chunk));
  LATTN_TRY(check_operands(dims, k, v, log_decay, A, B, r_ab, r_kv, chunk == 256 ? 64 : chunk));
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(q, "q", need));
  LATTN_TRY(check_ptr(gates, "gates", need));
  LATTN_TRY(check_ptr(out, "out", need));
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, chunk);
  if (!lattn::hla_supported(p))
    return fail(LATTN_EUNSUPPORTED, "lattn_hla_fwd needs d_k, d_v <= 128 (got %d, %d)", p.dk, p.dv);
  if (!need) return ok();
  const size_t ws = lattn::hla_plan(p).total_bytes;
  if (workspace == nullptr || workspace_bytes < ws)
    return fail(LATTN_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, ws);
  LATTN_TRY(check_ptr(workspace, "workspace", true));
  LATTN_TRY(hip_status(lattn::launch_hla(p, q, k, log_decay, A, B, v, gates, theta, out, workspace, stream),
                       "hla launch"));
  return ok();
}

size_t lattn_loglinear_fwd_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk) {
  if (check_dims(dims) != LATTN_OK || check_ranks(r_ab, r_kv) != LATTN_OK ||
      check_chunk(chunk, r_ab, r_kv) != LATTN_OK)
    return 0;
  return lattn::loglinear_plan(make_problem(dims, r_ab, r_kv, chunk)).total_bytes;
}

int lattn_loglinear_levels(int64_t seqlen) { return lattn::loglinear_levels(seqlen); }

int lattn_loglinear_fwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                        const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
                        int chunk, const float* lambda, void* out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  LATTN_TRY(check_operands(dims, k, v, log_decay, A, B, r_ab, r_kv, chunk));
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(q, "q", need));
  LATTN_TRY(check_ptr(lambda, "lambda", need));
  LATTN_TRY(check_ptr(out, "out", need));
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, chunk);
  if (!lattn::loglinear_supported(p))
    return fail(LATTN_EUNSUPPORTED, "lattn_loglinear_fwd needs d_k, d_v <= 128, d_k + chunk <= 192 and at most "
                "2^17 chunks at d_k = 128 (got d_k %d, d_v %d, chunk %d, %lld chunks)", p.dk, p.dv, p.C,
                (long long)p.N);
  if (!need) return ok();
  const size_t ws = lattn::loglinear_plan(p).total_bytes;
  if (workspace == nullptr || workspace_bytes < ws)
    return fail(LATTN_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, ws);
  LATTN_TRY(check_ptr(workspace, "workspace", true));
  LATTN_TRY(hip_status(lattn::launch_loglinear(p, q, k, log_decay, A, B, v, lambda, out, workspace, stream),
                       "log-linear launch"));
  return ok();
}

size_t lattn_chunk_bwd_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk) {
  if (check_dims(dims) != LATTN_OK || check_ranks(r_ab, r_kv) != LATTN_OK ||
      check_chunk(chunk, r_ab, r_kv) != LATTN_OK)
    return 0;
  return lattn::backward_workspace_bytes(make_problem(dims, r_ab, r_kv, chunk));
}

int lattn_chunk_bwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                    const float* log_decay, const void* A, const void* B, int r_ab, int r_kv, int chunk,
                    const void* dout, const float* dfinal, const float* initial_state, float* dq, float* dk,
                    float* dv, float* dlog_decay, float* dA, float* dB, float* dinitial_state, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  LATTN_TRY(check_bwd_args(dims, q, k, v, log_decay, A, B, r_ab, r_kv, chunk, dout, dfinal, initial_state, dq, dk,
                           dv, dlog_decay, dA, dB, dinitial_state));
  const bool need = dims->seqlen > 0;
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, chunk);
  if (!lattn::backward_supported(p))
    return fail(LATTN_EUNSUPPORTED, "lattn_chunk_bwd needs d_k, d_v <= 128, r_ab <= 4, r_kv <= 2 "
                "(got d_k %d, d_v %d, r_ab %d, r_kv %d)", p.dk, p.dv, r_ab, r_kv);
  if (!need) return hip_status(lattn::launch_copy_state(p, dfinal, dinitial_state, stream), "copy state");
  const size_t ws = lattn::backward_workspace_bytes(p);
  if (workspace == nullptr || workspace_bytes < ws)
    return fail(LATTN_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, ws);
  LATTN_TRY(check_ptr(workspace, "workspace", true));
  LATTN_TRY(hip_status(lattn::launch_backward(p, q, k, v, log_decay, A, B, dout, dfinal, initial_state, dq, dk, dv,
                                              dlog_decay, dA, dB, dinitial_state, workspace, stream),
                       "backward launch"));
  return ok();
}

size_t lattn_chunk_fwd_train_saved_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk) {
  if (check_dims(dims) != LATTN_OK || check_ranks(r_ab, r_kv) != LATTN_OK ||
      check_chunk(chunk, r_ab, r_kv) != LATTN_OK)
    return 0;
  return lattn::backward_saved_bytes(make_problem(dims, r_ab, r_kv, chunk));
}

size_t lattn_chunk_bwd_saved_workspace_size(const lattn_dims* dims, int r_ab, int r_kv, int chunk) {
  if (check_dims(dims) != LATTN_OK || check_ranks(r_ab, r_kv) != LATTN_OK ||
      check_chunk(chunk, r_ab, r_kv) != LATTN_OK)
    return 0;
  return lattn::backward_saved_workspace_bytes(make_problem(dims, r_ab, r_kv, chunk));
}

int lattn_chunk_fwd_train(const lattn_dims* dims, const void* q, const void* k, const void* v,
                          const float* log_decay, const void* A, const void* B, int r_ab, int r_kv, int chunk,
                          void* out, float* final_state, const float* initial_state, void* saved,
                          size_t saved_bytes, hipStream_t stream) {
  LATTN_TRY(check_operands(dims, k, v, log_decay, A, B, r_ab, r_kv, chunk));
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(q, "q", need));
  LATTN_TRY(check_ptr(out, "out", need));
  LATTN_TRY(check_ptr(final_state, "final_state", false));
  LATTN_TRY(check_ptr(initial_state, "initial_state", false));
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, chunk);
  LATTN_TRY(check_train_route(p, "lattn_chunk_fwd_train"));
  if (p.T == 0) return hip_status(lattn::launch_copy_state(p, initial_state, final_state, stream), "copy state");
  const size_t need_b = lattn::backward_saved_bytes(p);
  if (saved == nullptr || saved_bytes < need_b)
    return fail(LATTN_EWORKSPACE, "saved has %zu bytes, %zu needed", saved_bytes, need_b);
  LATTN_TRY(check_ptr(saved, "saved", true));
  LATTN_TRY(hip_status(lattn::launch_forward_train(p, q, k, v, log_decay, A, B, out, final_state, initial_state,
                                                   saved, stream),
                       "training forward launch"));
  return ok();
}

int lattn_chunk_bwd_saved(const lattn_dims* dims, const void* q, const void* k, const void* v,
                          const float* log_decay, const void* A, const void* B, int r_ab, int r_kv, int chunk,
                          const void* dout, const float* dfinal, const void* saved, size_t saved_bytes, float* dq, float* dk, float* dv, float* dlog_decay, float* dA,
                          float* dB, float* dinitial_state, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  LATTN_TRY(check_bwd_args(dims, q, k, v, log_decay, A, B, r_ab, r_kv, chunk, dout, dfinal, nullptr, dq, dk, dv,
                           dlog_decay, dA, dB, dinitial_state));
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, chunk);
  LATTN_TRY(check_train_route(p, "lattn_chunk_bwd_saved"));
  if (p.T == 0) return hip_status(lattn::launch_copy_state(p, dfinal, dinitial_state, stream), "copy state");
  const size_t need_b = lattn::backward_saved_bytes(p);
  if (saved == nullptr || saved_bytes < need_b)
    return fail(LATTN_EWORKSPACE, "saved has %zu bytes, %zu needed", saved_bytes, need_b);
  LATTN_TRY(check_ptr(saved, "saved", true));
  const size_t ws = lattn::backward_saved_workspace_bytes(p);
  if (workspace == nullptr || workspace_bytes < ws)
    return fail(LATTN_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, ws);
  LATTN_TRY(check_ptr(workspace, "workspace", true));
  LATTN_TRY(hip_status(lattn::launch_backward_saved(p, q, k, v, log_decay, A, B, dout, dfinal, saved,
                                                    dq, dk, dv, dlog_decay, dA, dB, dinitial_state, workspace,
                                                    stream),
                       "saved-state backward launch"));
  return ok();
}

int lattn_chunk_fwd_check(const lattn_dims* dims, const void* q, const void* k, const void* v,
                          const float* log_decay, const void* A, const void* B, int r_ab,
                          int r_kv, int chunk, const void* out, const void* workspace,
                          size_t workspace_bytes) {
  LATTN_TRY(check_operands(dims, k, v, log_decay, A, B, r_ab, r_kv, chunk));
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(q, "q", need));
  LATTN_TRY(check_ptr(out, "out", need));
  if (need) {
    const size_t ws = lattn_chunk_fwd_workspace_size(dims, r_ab, r_kv, chunk);
    if (ws > 0 && workspace == nullptr) return fail(LATTN_EWORKSPACE, "workspace is NULL (%zu bytes needed)", ws);
    if (workspace_bytes < ws)
      return fail(LATTN_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, ws);
    LATTN_TRY(check_ptr(workspace, "workspace", ws > 0));
  }
  return ok();
}

int lattn_chunk_fwd(const lattn_dims* dims, const void* q, const void* k, const void* v,
                    const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
                    int chunk, void* out, float* final_state, const float* initial_state,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  LATTN_TRY(lattn_chunk_fwd_check(dims, q, k, v, log_decay, A, B, r_ab, r_kv, chunk, out,
                                  workspace, workspace_bytes));
  LATTN_TRY(check_ptr(final_state, "final_state", false));
  LATTN_TRY(check_ptr(initial_state, "initial_state", false));
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, chunk);
  if (p.T == 0) return hip_status(lattn::launch_copy_state(p, initial_state, final_state, stream), "copy state");
  LATTN_TRY(hip_status(run_prepare(p, q, k, log_decay, A, B, workspace, stream), "prepare launch"));
  LATTN_TRY(hip_status(run_scan(p, workspace, v, out, final_state, initial_state, stream), "scan launch"));
  return ok();
}

int lattn_chunk_fwd_noalloc(const lattn_dims* dims, const void* q, const void* k, const void* v,
                            const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
                            int chunk, void* out, float* final_state, const float* initial_state,
                            hipStream_t stream) {
  // Validation and the size check come first: a rejected call touches no device.
  LATTN_TRY(check_operands(dims, k, v, log_decay, A, B, r_ab, r_kv, chunk));
  const bool nonempty = dims->seqlen > 0;
  LATTN_TRY(check_ptr(q, "q", nonempty));
  LATTN_TRY(check_ptr(out, "out", nonempty));
  const size_t need = lattn_chunk_fwd_workspace_size(dims, r_ab, r_kv, chunk);
  LATTN_TRY(check_ptr(final_state, "final_state", false));
  LATTN_TRY(check_ptr(initial_state, "initial_state", false));
  if (need > LATTN_NOALLOC_SCRATCH_BYTES)
    return fail(LATTN_EWORKSPACE, "lattn_chunk_fwd_noalloc: this problem needs %zu bytes of scratch, the static "
                "scratch holds %zu; call lattn_chunk_fwd with a caller-owned workspace", need,
                (size_t)LATTN_NOALLOC_SCRATCH_BYTES);
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, chunk);
  if (p.T == 0) return hip_status(lattn::launch_copy_state(p, initial_state, final_state, stream), "copy state");
  void* ws = nullptr;
  LATTN_TRY(noalloc_scratch(&ws));
  LATTN_TRY(hip_status(run_prepare(p, q, k, log_decay, A, B, ws, stream), "prepare launch"));
  LATTN_TRY(hip_status(run_scan(p, ws, v, out, final_state, initial_state, stream), "scan launch"));
  return ok();
}

int lattn_chunk_prepare(const lattn_dims* dims, const void* q, const void* k,
                        const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
                        int chunk, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  LATTN_TRY(lattn_chunk_fwd_check(dims, q, k, k, log_decay, A, B, r_ab, r_kv, chunk, q, workspace,
                                  workspace_bytes));
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, chunk);
  if (p.T == 0) return ok();
  LATTN_TRY(hip_status(run_prepare(p, q, k, log_decay, A, B, workspace, stream), "prepare launch"));
  return ok();
}

int lattn_chunk_scan(const lattn_dims* dims, const void* v, int r_ab, int r_kv, int chunk,
                     void* out, float* final_state, const float* initial_state, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  LATTN_TRY(check_dims(dims));
  LATTN_TRY(check_ranks(r_ab, r_kv));
  LATTN_TRY(check_chunk(chunk, r_ab, r_kv));
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(v, "v", need));
  LATTN_TRY(check_ptr(out, "out", need));
  LATTN_TRY(check_ptr(final_state, "final_state", false));
  LATTN_TRY(check_ptr(initial_state, "initial_state", false));
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, chunk);
  if (p.T == 0) return hip_status(lattn::launch_copy_state(p, initial_state, final_state, stream), "copy state");
  const size_t ws = lattn_chunk_fwd_workspace_size(dims, r_ab, r_kv, chunk);
  if (workspace == nullptr || workspace_bytes < ws)
    return fail(LATTN_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, ws);
  LATTN_TRY(check_ptr(workspace, "workspace", true));
  LATTN_TRY(hip_status(run_scan(p, workspace, v, out, final_state, initial_state, stream), "scan launch"));
  return ok();
}

int lattn_chunk_summaries(const lattn_dims* dims, const void* k, const void* v,
                          const float* log_decay, const void* A, const void* B, int r_ab,
                          int r_kv, int chunk, float* sum_A, float* sum_B, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  LATTN_TRY(check_operands(dims, k, v, log_decay, A, B, r_ab, r_kv, chunk));
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(sum_A, "sum_A", need));
  LATTN_TRY(check_ptr(sum_B, "sum_B", need));
  if (!need) return ok();
  const size_t ws = lattn_chunk_summaries_workspace_size(dims, r_ab, r_kv, chunk);
  if (workspace == nullptr || workspace_bytes < ws)
    return fail(LATTN_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, ws);
  LATTN_TRY(check_ptr(workspace, "workspace", true));
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, chunk);
  LATTN_TRY(hip_status(lattn::general_prepare(p, nullptr, k, log_decay, A, B, workspace, stream), "prepare launch"));
  LATTN_TRY(hip_status(lattn::general_summaries(p, workspace, v, sum_A, sum_B, stream), "summaries launch"));
  return ok();
}

int lattn_step(const lattn_dims* dims, const void* q, const void* k, const void* v,
               const float* log_decay, const void* A, const void* B, int r_ab, int r_kv,
               float* state, void* out, hipStream_t stream) {
  LATTN_TRY(check_dims(dims));
  if (dims->seqlen != 1) return fail(LATTN_EINVAL, "lattn_step needs seqlen == 1 (got %lld)", (long long)dims->seqlen);
  LATTN_TRY(check_ranks(r_ab, r_kv));
  LATTN_TRY(check_ptr(q, "q", true));
  LATTN_TRY(check_ptr(k, "k", true));
  LATTN_TRY(check_ptr(v, "v", true));
  LATTN_TRY(check_ptr(log_decay, "log_decay", true));
  LATTN_TRY(check_ptr(state, "state", true));
  LATTN_TRY(check_ptr(out, "out", true));
  if (r_ab == 0) {
    if (A != nullptr || B != nullptr) return fail(LATTN_EINVAL, "A and B must be NULL when r_ab == 0");
  } else {
    LATTN_TRY(check_ptr(A, "A", true));
    LATTN_TRY(check_ptr(B, "B", true));
  }
  const lattn::Problem p = make_problem(dims, r_ab, r_kv, 1);
  LATTN_TRY(hip_status(lattn::launch_step(p, q, k, v, log_decay, A, B, state, out, stream), "step launch"));
  return ok();
}

int lattn_hdla_params(const lattn_dims* dims, const void* k, const void* v,
                      const float* log_lambda, const float* beta, void* A, void* B, void* V_out,
                      hipStream_t stream) {
  LATTN_TRY(check_dims(dims));
  if (dims->decay_mode != LATTN_DECAY_PER_CHANNEL)
    return fail(LATTN_EINVAL, "lattn_hdla_params needs LATTN_DECAY_PER_CHANNEL");
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(k, "k", need));
  LATTN_TRY(check_ptr(v, "v", need));
  LATTN_TRY(check_ptr(log_lambda, "log_lambda", need));
  LATTN_TRY(check_ptr(beta, "beta", need));
  LATTN_TRY(check_ptr(A, "A", need));
  LATTN_TRY(check_ptr(B, "B", need));
  LATTN_TRY(check_ptr(V_out, "V_out", need));
  const lattn::Problem p = make_problem(dims, 2, 1, 1);
  LATTN_TRY(hip_status(lattn::launch_hdla_params(p, k, v, log_lambda, beta, A, B, V_out, stream), "hdla params launch"));
  return ok();
}

int lattn_gdn_params(const lattn_dims* dims, const void* k, const void* v, const float* g,
                     const float* beta, void* A, void* B, void* V_out, hipStream_t stream) {
  LATTN_TRY(check_dims(dims));
  if (dims->decay_mode != LATTN_DECAY_SCALAR)
    return fail(LATTN_EINVAL, "lattn_gdn_params needs LATTN_DECAY_SCALAR");
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(k, "k", need));
  LATTN_TRY(check_ptr(v, "v", need));
  LATTN_TRY(check_ptr(g, "g", need));
  LATTN_TRY(check_ptr(beta, "beta", need));
  LATTN_TRY(check_ptr(A, "A", need));
  LATTN_TRY(check_ptr(B, "B", need));
  LATTN_TRY(check_ptr(V_out, "V_out", need));
  const lattn::Problem p = make_problem(dims, 1, 1, 1);
  LATTN_TRY(hip_status(lattn::launch_gdn_params(p, k, v, g, beta, A, B, V_out, stream), "gdn params launch"));
  return ok();
}

int lattn_decay_range(const lattn_dims* dims, const float* log_decay, int chunk, float* chunk_max,
                      hipStream_t stream) {
  LATTN_TRY(check_dims(dims));
  LATTN_TRY(check_chunk(chunk, 0, 1));
  const bool need = dims->seqlen > 0;
  LATTN_TRY(check_ptr(log_decay, "log_decay", need));
  LATTN_TRY(check_ptr(chunk_max, "chunk_max", need));
  const lattn::Problem p = make_problem(dims, 0, 1, chunk);
  LATTN_TRY(hip_status(lattn::launch_decay_range(p, log_decay, chunk_max, stream), "decay range launch"));
  return ok();
}

int lattn_check_decay_range(const lattn_dims* dims, const float* log_decay, int chunk,
                            float* scratch, hipStream_t stream) {
  LATTN_TRY(lattn_decay_range(dims, log_decay, chunk, scratch, stream));
  const lattn::Problem p = make_problem(dims, 0, 1, chunk);
  const size_t n = static_cast<size_t>(p.BH * p.N);
  if (n == 0) return ok();
  std::vector<float> host(n);
  LATTN_TRY(hip_status(hipMemcpyAsync(host.data(), scratch, n * sizeof(float), hipMemcpyDeviceToHost, stream), "copy chunk maxima"));
  LATTN_TRY(hip_status(hipStreamSynchronize(stream), "synchronize"));
  // A NaN entry (a NaN log-decay in that chunk) fails the check as well.
  float m = 0.f;
  bool nan_seen = false;
  for (float x : host) {
    if (x != x) nan_seen = true;
    else if (x > m) m = x;
  }
  if (nan_seen) return fail(LATTN_EDECAY_RANGE, "log_decay holds NaN");
  if (!(m <= LATTN_MAX_CHUNK_LOG_DECAY))
    return fail(LATTN_EDECAY_RANGE, "chunk cumulative -log-decay reaches %g (limit %g)", (double)m,
                (double)LATTN_MAX_CHUNK_LOG_DECAY);
  return ok();
}

}  // extern "C"
