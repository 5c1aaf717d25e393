// C ABI of libuno: argument validation, workspace sizing and kernel launch.
// The operations and their contracts are documented in include/uno.h.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "../../include/uno.h"
#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return UNO_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(UNO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

uno::SamplingArgs to_args(const uno_sampling_params& sp) {
  uno::SamplingArgs a;
  a.temperature = sp.temperature;
  a.top_p = sp.top_p;
  a.top_k = sp.top_k;
  a.seed = sp.seed;
  return a;
}

// Shared checks of the verifier and the draft sampler.
int check_sampling(const uno_sampling_params& sp, int S, int b, int V, const char* fn) {
  if (S < 0) return fail(UNO_ERR_INVALID_ARG, "%s: S = %d < 0", fn, S);
  if (b < 1 || b > 64) return fail(UNO_ERR_INVALID_ARG, "%s: block size b = %d outside [1, 64]", fn, b);
  if (V < 1) return fail(UNO_ERR_INVALID_ARG, "%s: vocabulary V = %d < 1", fn, V);
  if ((long long)S * b > 0x7fffffffLL)
    return fail(UNO_ERR_INVALID_ARG, "%s: S * b = %lld slots exceeds 2^31 - 1", fn, (long long)S * b);
  if (isnan(sp.temperature)) return fail(UNO_ERR_INVALID_ARG, "%s: temperature is NaN", fn);
  if (!(sp.top_p > 0.0)) return fail(UNO_ERR_INVALID_ARG, "%s: top_p must be > 0 (got %g)", fn, sp.top_p);
  return UNO_OK;
}

}  // namespace

extern "C" {

const char* uno_status_string(int status) {
  switch (status) {
    case UNO_OK: return "UNO_OK";
    case UNO_ERR_INVALID_ARG: return "UNO_ERR_INVALID_ARG";
    case UNO_ERR_UNSUPPORTED: return "UNO_ERR_UNSUPPORTED";
    case UNO_ERR_WORKSPACE: return "UNO_ERR_WORKSPACE";
    case UNO_ERR_HIP: return "UNO_ERR_HIP";
    default: return "UNO_ERR_UNKNOWN";
  }
}

const char* uno_last_error(void) { return g_last_error; }

int uno_abi_version(void) { return 100; }

int uno_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (bytes == 0) return ok();
  if (!workspace) return fail(UNO_ERR_INVALID_ARG, "uno_workspace_init: null workspace");
  if (bytes % 4 != 0) return fail(UNO_ERR_INVALID_ARG, "uno_workspace_init: size %zu is not a multiple of 4", bytes);
  return hip_status(uno::launch_zero(workspace, bytes, static_cast<hipStream_t>(stream)),
                    "uno_workspace_init launch");
}

size_t uno_verify_block_workspace(int S, int b, int V) {
  (void)V;
  if (S <= 0 || b <= 0) return 256;
  return uno::verify_workspace_bytes(S, b);
}

}  // extern "C"

namespace {

// Argument checks and marshalling shared by both verify entry points.
int verify_prepare(const char* fn, const void* p_logits, const void* q_logits, int dtype,
                   const int32_t* draft_tokens, const int64_t* seq_ids, const int64_t* pos_offsets,
                   int S, int b, int V, const uno_sampling_params& sp, int32_t* out_tokens,
                   int32_t* accept_len, int32_t* resampled, uint8_t* slot_accept, float* diag,
                   uno::VerifyArgs* a) {
  int st = check_sampling(sp, S, b, V, fn);
  if (st != UNO_OK) return st;
  if (dtype != UNO_DTYPE_F32 && dtype != UNO_DTYPE_BF16)
    return fail(UNO_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  if (S == 0) return UNO_OK;
  if (!p_logits || !q_logits || !draft_tokens || !seq_ids || !pos_offsets || !out_tokens ||
      !accept_len || !resampled)
    return fail(UNO_ERR_INVALID_ARG, "%s: a required pointer is null", fn);
  a->p = p_logits;
  a->q = q_logits;
  a->bf16 = dtype == UNO_DTYPE_BF16;
  a->draft = draft_tokens;
  a->seq_ids = seq_ids;
  a->pos = pos_offsets;
  a->S = S;
  a->b = b;
  a->V = V;
  a->sp = to_args(sp);
  a->out_tokens = out_tokens;
  a->accept_len = accept_len;
  a->resampled = resampled;
  a->slot_accept = slot_accept;
  a->diag = diag;
  a->ws = nullptr;
  return UNO_OK;
}

}  // namespace

extern "C" {

int uno_verify_block(const void* p_logits, const void* q_logits, int dtype,
                     const int32_t* draft_tokens, const int64_t* seq_ids,
                     const int64_t* pos_offsets, int S, int b, int V,
                     uno_sampling_params sp, int32_t* out_tokens, int32_t* accept_len,
                     int32_t* resampled, uint8_t* slot_accept, float* diag,
                     void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "uno_verify_block";
  uno::VerifyArgs a;
  int st = verify_prepare(fn, p_logits, q_logits, dtype, draft_tokens, seq_ids, pos_offsets, S, b, V, sp,
                          out_tokens, accept_len, resampled, slot_accept, diag, &a);
  if (st != UNO_OK || S == 0) return st == UNO_OK ? ok() : st;
  const size_t need = uno_verify_block_workspace(S, b, V);
  if (!workspace || ws_bytes < need)
    return fail(UNO_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, need);
  a.ws = workspace;
  return hip_status(uno::launch_verify(a, static_cast<hipStream_t>(stream)), "uno_verify_block launch");
}

int uno_verify_block_noalloc(const void* p_logits, const void* q_logits, int dtype,
                             const int32_t* draft_tokens, const int64_t* seq_ids,
                             const int64_t* pos_offsets, int S, int b, int V,
                             uno_sampling_params sp, int32_t* out_tokens, int32_t* accept_len,
                             int32_t* resampled, uint8_t* slot_accept, float* diag, void* stream) {
  const char* fn = "uno_verify_block_noalloc";
  uno::VerifyArgs a;
  int st = verify_prepare(fn, p_logits, q_logits, dtype, draft_tokens, seq_ids, pos_offsets, S, b, V, sp,
                          out_tokens, accept_len, resampled, slot_accept, diag, &a);
  if (st != UNO_OK || S == 0) return st == UNO_OK ? ok() : st;
  const size_t need = uno::verify_workspace_bytes(S, b);
  if (need > uno::verify_scratch_bytes())
    return fail(UNO_ERR_UNSUPPORTED,
                "%s: S = %d sequences of b = %d slots need %zu bytes of scratch and the library's "
                "array holds %zu (S <= 65536 with S * b <= 131072 always fits); call "
                "uno_verify_block with a workspace instead", fn, S, b, need, uno::verify_scratch_bytes());
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = uno::verify_scratch(&a.ws, hs);
  if (e != hipSuccess) return hip_status(e, "uno_verify_block_noalloc scratch set-up");
  return hip_status(uno::launch_verify(a, hs), "uno_verify_block_noalloc launch");
}

int uno_draft_sample(const void* q_logits, int dtype, const int64_t* seq_ids,
                     const int64_t* pos_offsets, int S, int b, int V,
                     uno_sampling_params sp, int32_t* draft_tokens, int32_t* flags,
                     void* stream) {
  const char* fn = "uno_draft_sample";
  int st = check_sampling(sp, S, b, V, fn);
  if (st != UNO_OK) return st;
  if (dtype != UNO_DTYPE_F32 && dtype != UNO_DTYPE_BF16)
    return fail(UNO_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  if (S == 0) return ok();
  if (!q_logits || !seq_ids || !pos_offsets || !draft_tokens)
    return fail(UNO_ERR_INVALID_ARG, "%s: a required pointer is null", fn);
  uno::DraftArgs a;
  a.q = q_logits;
  a.bf16 = dtype == UNO_DTYPE_BF16;
  a.seq_ids = seq_ids;
  a.pos = pos_offsets;
  a.S = S;
  a.b = b;
  a.V = V;
  a.sp = to_args(sp);
  a.draft = draft_tokens;
  a.flags = flags;
  return hip_status(uno::launch_draft(a, static_cast<hipStream_t>(stream)), "uno_draft_sample launch");
}

size_t uno_tv_loss_workspace(int R, int V) {
  (void)V;
  return uno::tv_workspace_bytes(R);
}

int uno_tv_loss_fwd_bwd(const void* teacher_logits, const void* student_logits, int dtype,
                        const uint8_t* response_mask, int R, int V, float temperature,
                        float* loss, float* tv_rows, void* grad_student,
                        void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "uno_tv_loss_fwd_bwd";
  if (R < 0) return fail(UNO_ERR_INVALID_ARG, "%s: R = %d < 0", fn, R);
  if (V < 1) return fail(UNO_ERR_INVALID_ARG, "%s: vocabulary V = %d < 1", fn, V);
  if (!(temperature > 0.0f) || isinf(temperature))
    return fail(UNO_ERR_INVALID_ARG, "%s: temperature must be finite and > 0 (got %g)", fn, double(temperature));
  if (dtype != UNO_DTYPE_F32 && dtype != UNO_DTYPE_BF16)
    return fail(UNO_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  if (!loss) return fail(UNO_ERR_INVALID_ARG, "%s: loss is null", fn);
  if (R > 0 && (!teacher_logits || !student_logits || !response_mask))
    return fail(UNO_ERR_INVALID_ARG, "%s: a required pointer is null", fn);
  const size_t need = uno_tv_loss_workspace(R, V);
  if (!workspace || ws_bytes < need)
    return fail(UNO_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, need);
  const int vmax = uno::tv_max_vocab(dtype == UNO_DTYPE_BF16);
  if (vmax <= 0) return fail(UNO_ERR_HIP, "%s: occupancy query failed", fn);
  if (V > vmax)
    return fail(UNO_ERR_UNSUPPORTED, "%s: V = %d exceeds the %d logits one row team holds on this device",
                fn, V, vmax);
  uno::TvArgs a;
  a.teacher = teacher_logits;
  a.student = student_logits;
  a.bf16 = dtype == UNO_DTYPE_BF16;
  a.mask = response_mask;
  a.R = R;
  a.V = V;
  a.temperature = temperature;
  a.loss = loss;
  a.tv_rows = tv_rows;
  a.grad = grad_student;
  a.ws = workspace;
  return hip_status(uno::launch_tv(a, static_cast<hipStream_t>(stream)), "uno_tv_loss_fwd_bwd launch");
}

size_t uno_gated_lora_linear_workspace(int M, int N, int K, int r) {
  if (M <= 0 || N <= 0 || K <= 0 || r < 0) return 256;
  return uno::gemm_workspace_bytes(M, N, K, r);
}

int uno_gated_lora_linear(const void* X, const void* W, const void* A, const void* B,
                          const uint8_t* row_mask, float scale, void* Y, int M, int N, int K, int r,
                          void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "uno_gated_lora_linear";
  if (M < 0 || N < 0 || K < 1 || r < 0)
    return fail(UNO_ERR_INVALID_ARG, "%s: sizes M = %d, N = %d, K = %d, r = %d out of range", fn, M, N, K, r);
  if (!isfinite(scale)) return fail(UNO_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  if (M == 0 || N == 0) return ok();
  if (!X || !W || !Y) return fail(UNO_ERR_INVALID_ARG, "%s: X, W and Y must not be null", fn);
  if (r > 0 && (!A || !B || !row_mask))
    return fail(UNO_ERR_INVALID_ARG, "%s: A, B and row_mask must not be null when r > 0", fn);
  if (K % 8 != 0 || r % 8 != 0)
    return fail(UNO_ERR_UNSUPPORTED, "%s: K = %d and r = %d must be multiples of 8", fn, K, r);
  const void* ptrs[4] = {X, W, A, B};
  for (int i = 0; i < 4; ++i)
    if (ptrs[i] && reinterpret_cast<uintptr_t>(ptrs[i]) % 16 != 0)
      return fail(UNO_ERR_UNSUPPORTED, "%s: operand %d is not 16-byte aligned", fn, i);
  const long long lim = 0x7fffffffLL;
  if ((long long)M * K * 2 > lim || (long long)N * K * 2 > lim || (long long)M * N > lim ||
      (long long)N * r * 2 > lim || (long long)M * r * 2 > lim)
    return fail(UNO_ERR_UNSUPPORTED, "%s: an operand exceeds 2 GiB", fn);
  const size_t need = uno_gated_lora_linear_workspace(M, N, K, r);
  if (r > 0 && (!workspace || ws_bytes < need))
    return fail(UNO_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, need);
  uno::GemmArgs a;
  a.X = X;
  a.W = W;
  a.A = A;
  a.B = B;
  a.row_mask = row_mask;
  a.scale = scale;
  a.Y = Y;
  a.M = M;
  a.N = N;
  a.K = K;
  a.r = r;
  a.ws = workspace;
  return hip_status(uno::launch_gemm(a, static_cast<hipStream_t>(stream)), "uno_gated_lora_linear launch");
}

size_t uno_gated_lora_linear_bwd_workspace(int M, int N, int K, int r) {
  if (M <= 0 || N <= 0 || K <= 0 || r <= 0) return 256;
  return uno::gemm_bwd_workspace_bytes(M, N, K, r);
}

int uno_gated_lora_linear_bwd(const void* dY, const void* X, const void* W, const void* W_t, const void* A,
                              const void* B, const uint8_t* row_mask, float scale, void* dX, void* dA, void* dB,
                              int M, int N, int K, int r, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "uno_gated_lora_linear_bwd";
  if (M < 0 || N < 1 || K < 1 || r < 1)
    return fail(UNO_ERR_INVALID_ARG, "%s: sizes M = %d, N = %d, K = %d, r = %d out of range", fn, M, N, K, r);
  if (!isfinite(scale)) return fail(UNO_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  if (M == 0) return ok();
  if (!dY || !X || !W || !A || !B || !row_mask || !dA || !dB)
    return fail(UNO_ERR_INVALID_ARG, "%s: only dX may be null", fn);
  if (M % 8 != 0 || N % 8 != 0 || K % 8 != 0 || r % 8 != 0)
    return fail(UNO_ERR_UNSUPPORTED, "%s: M = %d, N = %d, K = %d and r = %d must be multiples of 8", fn, M, N,
                K, r);
  const void* ptrs[9] = {dY, X, W, A, B, dX, dA, dB, W_t};
  for (int i = 0; i < 9; ++i)
    if (ptrs[i] && reinterpret_cast<uintptr_t>(ptrs[i]) % 16 != 0)
      return fail(UNO_ERR_UNSUPPORTED, "%s: operand %d is not 16-byte aligned", fn, i);
  const long long lim = 0x7fffffffLL;
  if ((long long)M * K * 2 > lim || (long long)N * K * 2 > lim || (long long)M * N * 2 > lim ||
      (long long)N * r * 2 > lim || (long long)M * r * 2 > lim || (long long)K * r * 2 > lim)
    return fail(UNO_ERR_UNSUPPORTED, "%s: an operand exceeds 2 GiB", fn);
  const size_t need = uno_gated_lora_linear_bwd_workspace(M, N, K, r);
  if (!workspace || ws_bytes < need)
    return fail(UNO_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, need);
  uno::GemmBwdArgs a;
  a.dY = dY;
  a.X = X;
  a.W = W;
  a.Wt = W_t;
  a.A = A;
  a.B = B;
  a.row_mask = row_mask;
  a.scale = scale;
  a.dX = dX;
  a.dA = dA;
  a.dB = dB;
  a.M = M;
  a.N = N;
  a.K = K;
  a.r = r;
  a.ws = workspace;
  return hip_status(uno::launch_gemm_bwd(a, static_cast<hipStream_t>(stream)), "uno_gated_lora_linear_bwd launch");
}

}  // extern "C"

namespace {

// The model description and its checks, shared by the forward and step entry points.
int model_desc(const uno_model* m, int M, const char* fn, uno::ModelDesc* md) {
  if (!m) return fail(UNO_ERR_INVALID_ARG, "%s: model is null", fn);
  if (!m->embed || !m->lm_head || (m->layers > 0 && !m->weights))
    return fail(UNO_ERR_INVALID_ARG, "%s: a model weight pointer is null", fn);
  if (m->rank > 0 && m->layers > 0 && (!m->lora_a || !m->lora_b))
    return fail(UNO_ERR_INVALID_ARG, "%s: rank %d given without adapter pointers", fn, m->rank);
  for (int i = 0; i < 7 * m->layers; ++i) {
    if (!m->weights[i]) return fail(UNO_ERR_INVALID_ARG, "%s: weight %d is null", fn, i);
    if (m->rank > 0 && (!m->lora_a[i] || !m->lora_b[i]))
      return fail(UNO_ERR_INVALID_ARG, "%s: adapter factor %d is null", fn, i);
  }
  md->hidden = m->hidden;
  md->kv_width = m->kv_width;
  md->head_dim = m->head_dim;
  md->ffn = m->ffn;
  md->vocab = m->vocab;
  md->layers = m->layers;
  md->rank = m->rank;
  md->lora_scale = m->lora_scale;
  md->embed = m->embed;
  md->lm_head = m->lm_head;
  md->w = m->weights;
  md->lora_a = m->lora_a;
  md->lora_b = m->lora_b;
  const size_t lim = size_t(1) << 32;
  if (size_t(m->vocab) * m->hidden * 2 >= lim || size_t(m->ffn) * m->hidden * 2 >= lim)
    return fail(UNO_ERR_UNSUPPORTED, "%s: a weight matrix of 4 GiB or more", fn);
  const int c = uno::model_check(*md, M);
  if (c == 1)
    return fail(UNO_ERR_UNSUPPORTED,
                "%s: unsupported model shape (hidden %d, kv_width %d, head_dim %d, ffn %d, rank %d): hidden and "
                "ffn must be multiples of 128, rank of 32, head_dim of 8 and divide hidden and kv_width, and the "
                "kv heads divide the query heads", fn, m->hidden, m->kv_width, m->head_dim, m->ffn, m->rank);
  if (c == 2) return fail(UNO_ERR_UNSUPPORTED, "%s: %d rows; a forward takes 1 to 64", fn, M);
  return UNO_OK;
}

}  // namespace

extern "C" {

size_t uno_forward_workspace(const uno_model* model, int M) {
  uno::ModelDesc md;
  if (model_desc(model, M, "uno_forward_workspace", &md) != UNO_OK) return 0;
  return uno::forward_workspace_bytes(md, M);
}

int uno_forward(const uno_model* model, const int32_t* tokens, const uint8_t* row_mask, int M, int loops,
                float* logits, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "uno_forward";
  uno::ModelDesc md;
  int st = model_desc(model, M, fn, &md);
  if (st != UNO_OK) return st;
  if (loops < 1) return fail(UNO_ERR_INVALID_ARG, "%s: loops = %d < 1", fn, loops);
  if (!tokens || !logits) return fail(UNO_ERR_INVALID_ARG, "%s: a required pointer is null", fn);
  const size_t need = uno::forward_workspace_bytes(md, M);
  if (!workspace || ws_bytes < need)
    return fail(UNO_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, need);
  return hip_status(uno::launch_forward(md, tokens, row_mask, M, loops, logits, workspace,
                                        static_cast<hipStream_t>(stream)), "uno_forward launch");
}

size_t uno_decode_step_workspace(const uno_model* model, int S, int b) {
  uno::ModelDesc md;
  if (S < 1 || b < 1 || S * b > 64) return 0;
  if (model_desc(model, S * b, "uno_decode_step_workspace", &md) != UNO_OK) return 0;
  return uno::step_workspace_bytes(md, S, b);
}

int uno_decode_step(const uno_model* model, int S, int b, int draft_loops, int verify_loops,
                    uno_sampling_params sp, const int32_t* seed_tokens, const int64_t* seq_ids,
                    const int64_t* pos_offsets, int32_t* out_tokens, int32_t* accept_len, int32_t* resampled,
                    int32_t* draft_tokens, float* draft_logits, float* verify_logits,
                    void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "uno_decode_step";
  int st = check_sampling(sp, S, b, 1, fn);
  if (st != UNO_OK) return st;
  if (S < 1 || (long long)S * b > 64)
    return fail(UNO_ERR_UNSUPPORTED, "%s: S = %d blocks of b = %d rows; a step takes 1 to 64 rows", fn, S, b);
  uno::ModelDesc md;
  if ((st = model_desc(model, S * b, fn, &md)) != UNO_OK) return st;
  if (draft_loops < 1 || verify_loops < 1)
    return fail(UNO_ERR_INVALID_ARG, "%s: loops must be >= 1 (draft %d, verify %d)", fn, draft_loops, verify_loops);
  if (!seed_tokens || !seq_ids || !pos_offsets || !out_tokens)
    return fail(UNO_ERR_INVALID_ARG, "%s: a required pointer is null", fn);
  const size_t need = uno::step_workspace_bytes(md, S, b);
  if (!workspace || ws_bytes < need)
    return fail(UNO_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, need);
  uno::StepArgs a{};
  a.S = S;
  a.b = b;
  a.draft_loops = draft_loops;
  a.verify_loops = verify_loops;
  a.sp = to_args(sp);
  a.seed_tokens = seed_tokens;
  a.seq_ids = seq_ids;
  a.pos = pos_offsets;
  a.out_tokens = out_tokens;
  a.accept_len = accept_len;
  a.resampled = resampled;
  a.drafts = draft_tokens;
  a.draft_logits = draft_logits;
  a.verify_logits = verify_logits;
  a.ws = workspace;
  return hip_status(uno::launch_decode_step(md, a, static_cast<hipStream_t>(stream)), "uno_decode_step launch");
}

size_t uno_ar_step_workspace(const uno_model* model, int S) {
  uno::ModelDesc md;
  if (model_desc(model, S, "uno_ar_step_workspace", &md) != UNO_OK) return 0;
  return uno::ar_step_workspace_bytes(md, S);
}

int uno_ar_step(const uno_model* model, int S, int loops, uno_sampling_params sp, const int32_t* tokens,
                const int64_t* seq_ids, const int64_t* pos_offsets, int32_t* out_tokens, float* logits,
                void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "uno_ar_step";
  int st = check_sampling(sp, S, 1, 1, fn);
  if (st != UNO_OK) return st;
  uno::ModelDesc md;
  if ((st = model_desc(model, S, fn, &md)) != UNO_OK) return st;
  if (loops < 1) return fail(UNO_ERR_INVALID_ARG, "%s: loops = %d < 1", fn, loops);
  if (!tokens || !seq_ids || !pos_offsets || !out_tokens)
    return fail(UNO_ERR_INVALID_ARG, "%s: a required pointer is null", fn);
  const size_t need = uno::ar_step_workspace_bytes(md, S);
  if (!workspace || ws_bytes < need)
    return fail(UNO_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, need);
  uno::StepArgs a{};
  a.S = S;
  a.b = 1;
  a.draft_loops = loops;
  a.verify_loops = loops;
  a.sp = to_args(sp);
  a.seed_tokens = tokens;
  a.seq_ids = seq_ids;
  a.pos = pos_offsets;
  a.out_tokens = out_tokens;
  a.verify_logits = logits;
  a.ws = workspace;
  return hip_status(uno::launch_ar_step(md, a, static_cast<hipStream_t>(stream)), "uno_ar_step launch");
}
}  // extern "C"
