/*
 * uno.h -- C ABI of the MI355X (gfx950) hot path of Uno (Psi-Spec) block
 * draft-and-verify decoding.
 *
 * Sources of the operations (page titles as headed on the pages):
 *  - "LoopUno: Turning Agentic Looped LLMs into Diffusion LLMs in One Hour",
 *    section "How it works": a block of positions is drafted in one forward with
 *    a LoRA that is switched on only for noise positions; the unmodified model
 *    verifies them and the longest correct prefix is kept; the first position is
 *    always the exact autoregressive token. Training is self-distillation with a
 *    total-variation loss, and lossless acceptance equals 1 - TV.
 *  - Same page, "Setup / Recipe": gated LoRA r = 128, alpha = 2048 on all seven
 *    projections, noise rows only.
 *  - "Uno Qwen3-8B" model card: the adapter is applied only to draft-noise rows;
 *    seed, prefill, verification and AR rows use the frozen weights. Its
 *    "Evaluation protocol" table fixes T = 1.0, top-p 0.95, top-k 50, block 16.
 *
 * Conventions shared by every call:
 *  - Every tensor pointer is DEVICE memory owned by the caller. The library never
 *    frees caller memory and keeps no per-call state between calls other than the
 *    caller-provided workspace (and, for uno_verify_block_noalloc only, one static
 *    scratch array per GPU inside the library).
 *  - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    default stream) and runs asynchronously; results are valid after the caller
 *    synchronises the stream.
 *  - Argument errors are detected on the host before anything is launched; the
 *    call then returns a non-zero uno_status and uno_last_error() holds a
 *    message. A launch failure returns UNO_ERR_HIP. Nothing is thrown across the
 *    ABI.
 *  - Rows are contiguous (row-major, no padding). 16-byte aligned rows take the
 *    vectorised path; other alignments are handled by a scalar path.
 *  - Calls on different streams with different workspaces may run concurrently.
 */
#ifndef UNO_H
#define UNO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  UNO_OK = 0,
  UNO_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, out-of-range parameter */
  UNO_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement            */
  UNO_ERR_WORKSPACE = 3,     /* workspace missing or smaller than *_workspace() says   */
  UNO_ERR_HIP = 4            /* a HIP runtime call failed (message in uno_last_error)  */
} uno_status;

typedef enum { UNO_DTYPE_F32 = 0, UNO_DTYPE_BF16 = 1 } uno_dtype;

/* Sampling settings ("Uno Qwen3-8B" model card, "Evaluation protocol" table).
 *   temperature <= 0  -> greedy (one-hot at the argmax, lowest id on ties)
 *   top_k <= 0 or >= V -> top-k off; otherwise tie-inclusive: keep v iff z_v is
 *                        >= the k-th largest logit counted with multiplicity
 *   top_p >= 1        -> top-p off; otherwise tie-grouped: keep v iff the mass of
 *                        strictly more probable tokens is < top_p (0 < top_p)
 *   seed              -> Philox-4x64-10 key word 0 (key word 1 is the sequence id)
 * temperature and top_p are doubles because the filtered-set arithmetic runs in
 * fp64: the top-p comparison uses exactly the value the caller passes. */
typedef struct {
  double temperature;
  double top_p;
  int32_t top_k;
  uint64_t seed;
} uno_sampling_params;

/* Bits of the per-slot flag word written to diag[..., 3] (as a float). */
#define UNO_FLAG_TIE_ACCEPT 1      /* |u_acc - p~(d)/q~(d)| < 1e-6                          */
#define UNO_FLAG_TIE_TOPP_P 2      /* a base-row top-p group boundary within 1e-6 of top_p  */
#define UNO_FLAG_TIE_TOPP_Q 4      /* a draft-row top-p group boundary within 1e-6 of top_p */
#define UNO_FLAG_TIE_ICDF 8        /* the inverse-CDF draw lies within 1e-6*Z of a boundary */
#define UNO_FLAG_Q_ZERO 16         /* draft token outside supp(q~): rejected                */
#define UNO_FLAG_RES_ZERO 32       /* residual mass zero after a rejection: drew from p~    */
#define UNO_FLAG_OVERFLOW 64       /* reserved: no call sets it (overflowing rows take the  */
                                   /* full-row path, with the same results)                  */

/* Human-readable name of a status code (static storage). */
const char* uno_status_string(int status);
/* Detail of the last error returned on this thread (static per-thread storage). */
const char* uno_last_error(void);
/* ABI version of this library (major * 100 + minor). */
int uno_abi_version(void);

/* Fill `bytes` of device memory with zeros on `stream` (a fill kernel, safe to
 * record in a HIP graph). Every workspace must be zeroed once before its first
 * use; each call leaves it valid for the next call (it may carry state from one
 * call to the next), so the caller never writes to it afterwards. */
int uno_workspace_init(void* workspace, size_t bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Lossless block verification ("LoopUno", "How it works").
 *
 * For each sequence s and slot i of a block of b positions, p = filter(p_logits
 * [s,i]) and q = filter(q_logits[s,i]) (temperature, then tie-inclusive top-k,
 * then tie-grouped top-p on the renormalised top-k set, then renormalise).
 *   slot 0      : the AR token, inverse CDF of p~ at u_res (q and draft ignored).
 *   slot i >= 1 : accept draft d iff u_acc < p~(d)/q~(d); otherwise the slot's
 *                 token is drawn from normalise(max(0, p~ - q~)) at u_res.
 * accept_len[s] = first rejected slot (b if none, always >= 1). out_tokens[s,:]
 * holds the kept tokens, then (if accept_len < b) the resampled token, then -1.
 * Uniforms: Philox-4x64-10, key = (seed, seq_ids[s]), counter =
 * (pos_offsets[s] + i, 0, 0, 0); word 0 -> u_acc, word 1 -> u_res, each as
 * (w >> 40) * 2^-24. Filtered-set arithmetic runs in fp64; the top-k selection
 * compares the input values exactly.
 *
 *   p_logits, q_logits : [S, b, V] of `dtype` (bf16 or fp32), contiguous
 *   draft_tokens       : int32 [S, b]; slot 0 ignored
 *   seq_ids, pos_offsets : int64 [S]
 *   out_tokens         : int32 [S, b]  (out)
 *   accept_len         : int32 [S]     (out) the tokens-per-forward numerator
 *   resampled          : int32 [S]     (out) resampled token, -1 if all b kept
 *   slot_accept        : uint8 [S, b]  (out, optional) raw per-slot decisions
 *   diag               : float [S, b, 4] (out, optional) u_acc, p~(d)/q~(d), u_res,
 *                        flag bits (UNO_FLAG_*)
 *   workspace          : >= uno_verify_block_workspace(S, b, V) bytes, zeroed once
 * Limits: 1 <= b <= 64, 1 <= V < 2^31, S >= 0 (S == 0 launches nothing).
 * Every setting is handled: top-k up to 128 (or any top-k when V <= 256) takes
 * a single pass over the logits; top-k off, larger top-k, and rows whose
 * candidate list or tie-inclusive top-k set outgrows the single pass take a
 * multi-pass full-row path (same results, slower). UNO_FLAG_OVERFLOW is no
 * longer produced.
 * ------------------------------------------------------------------------- */
size_t uno_verify_block_workspace(int S, int b, int V);
int uno_verify_block(const void* p_logits, const void* q_logits, int dtype,
                     const int32_t* draft_tokens, const int64_t* seq_ids,
                     const int64_t* pos_offsets, int S, int b, int V,
                     uno_sampling_params sp, int32_t* out_tokens, int32_t* accept_len,
                     int32_t* resampled, uint8_t* slot_accept, float* diag,
                     void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * uno_verify_block for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, results and kernels as uno_verify_block, without the workspace: the
 * per-sequence tickets and slot records live in a static device array inside the
 * library (1310720 bytes per GPU, held until the process ends). The call makes no
 * hipMalloc, hipFree or other allocating call; the first call on a device looks
 * up that GPU's copy of the array and clears it with a fill kernel on `stream`.
 * Every verify kernel leaves the part it used zero again.
 * Limit: the tickets and records, round_up(4 S, 256) + 8 S b bytes (what
 * uno_verify_block_workspace returns), must fit the 1310720-byte array: any call
 * with S <= 65536 sequences and S * b <= 131072 slots does. Larger calls return
 * UNO_ERR_UNSUPPORTED (nothing launched) and must use uno_verify_block.
 * All calls on one GPU share its array: calls that overlap in time on that GPU
 * (on different streams, or from different threads) race and give wrong results.
 * Serialise them, or give each its own workspace through uno_verify_block.
 * ------------------------------------------------------------------------- */
int uno_verify_block_noalloc(const void* p_logits, const void* q_logits, int dtype,
                             const int32_t* draft_tokens, const int64_t* seq_ids,
                             const int64_t* pos_offsets, int S, int b, int V,
                             uno_sampling_params sp, int32_t* out_tokens, int32_t* accept_len,
                             int32_t* resampled, uint8_t* slot_accept, float* diag, void* stream);

/* ---------------------------------------------------------------------------
 * Draft sampler: d[s,i] ~ filter(q_logits[s,i]) for every slot, by inverse CDF
 * at Philox stream 1 (counter = (pos_offsets[s] + i, 1, 0, 0), word 0). This is
 * the draft half of a Psi-Spec step ("LoopUno", "How it works": the block is
 * drafted in one forward); its uniforms are independent of the verifier's.
 *   q_logits : [S, b, V] of `dtype`; draft_tokens : int32 [S, b] (out)
 *   flags    : int32 [S, b] (out, optional) UNO_FLAG_TIE_TOPP_Q / _TIE_ICDF
 * Same limits as uno_verify_block; needs no workspace.
 * ------------------------------------------------------------------------- */
int uno_draft_sample(const void* q_logits, int dtype, const int64_t* seq_ids,
                     const int64_t* pos_offsets, int S, int b, int V,
                     uno_sampling_params sp, int32_t* draft_tokens, int32_t* flags,
                     void* stream);

/* ---------------------------------------------------------------------------
 * TV self-distillation loss, forward and backward ("LoopUno", "How it works" ->
 * "Training is self-distillation").
 *   p = softmax(teacher/T), q = softmax(student/T) over the full vocabulary,
 *   TV_r = 1/2 sum_v |p_v - q_v|, loss = sum_r mask_r TV_r / sum_r mask_r (0 if
 *   no row is masked in), grad[r,j] = mask_r q_j (g_j - sum_v q_v g_v) /
 *   (T * sum mask), g_v = 1/2 sign(q_v - p_v). The teacher gets no gradient.
 *   teacher_logits, student_logits : [R, V] of `dtype`
 *   response_mask : uint8 [R]
 *   loss          : float [1] (out)
 *   tv_rows       : float [R] (out, optional; 0 on masked-out rows)
 *   grad_student  : [R, V] of `dtype` (out, optional; NULL = forward only)
 *   workspace     : >= uno_tv_loss_workspace(R, V) bytes, zeroed once
 * Limits: R >= 0, 1 <= V < 2^31, temperature > 0.
 * ------------------------------------------------------------------------- */
size_t uno_tv_loss_workspace(int R, int V);
int uno_tv_loss_fwd_bwd(const void* teacher_logits, const void* student_logits, int dtype,
                        const uint8_t* response_mask, int R, int V, float temperature,
                        float* loss, float* tv_rows, void* grad_student,
                        void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Row-gated LoRA linear ("Uno Qwen3-8B" model card; "LoopUno", "Setup / Recipe"):
 *   Y[m,n] = sum_k X[m,k] W[n,k] + scale * row_mask[m] * sum_j T[m,j] B[n,j],
 *   T = X A^T (rank r), all bf16 in, fp32 accumulation, bf16 out (round to
 *   nearest even). T is rounded to bf16 after scaling and gating.
 *   X : bf16 [M, K]; W : bf16 [N, K] (nn.Linear layout); A : bf16 [r, K]
 *   (lora_A); B : bf16 [N, r] (lora_B); row_mask : uint8 [M] (1 = noise row,
 *   adapter on); Y : bf16 [M, N] (out, must not alias inputs)
 *   workspace : >= uno_gated_lora_linear_workspace(M, N, K, r) bytes
 * Limits: M, N, K >= 1, r >= 0 (r == 0: plain linear); K and r multiples of 8
 * and all row starts 16-byte aligned (UNO_ERR_UNSUPPORTED otherwise).
 * ------------------------------------------------------------------------- */
size_t uno_gated_lora_linear_workspace(int M, int N, int K, int r);
int uno_gated_lora_linear(const void* X, const void* W, const void* A, const void* B,
                          const uint8_t* row_mask, float scale, void* Y,
                          int M, int N, int K, int r,
                          void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Backward of the row-gated LoRA linear ("LoopUno", "How it works" -> "Training
 * is self-distillation" and "Setup / Recipe": the adapter, switched on for the
 * noise rows only, is what training updates; the base weight W stays frozen).
 * For an upstream gradient dY of Y = X W^T + s diag(m) (X A^T) B^T:
 *   U  = bf16(s diag(m) dY B)            [M, r]
 *   dX = dY W + U A                      [M, K]
 *   dA = U^T X                           [r, K]
 *   dB = s (diag(m) dY)^T (X A^T)        [N, r]
 * bf16 in, fp32 accumulation, bf16 out; X A^T is rounded to bf16 before it meets
 * dY, as U is before it meets A and X.
 *   dY : bf16 [M, N]; X, W, A, B, row_mask, scale : as for the forward
 *   W_t : bf16 [K, N] = W^T, optional. The base weight is frozen, so a caller
 *   can transpose it once and pass it on every step; with NULL, W is transposed
 *   into the workspace on every call.
 *   dX : bf16 [M, K] (out, optional: NULL skips it); dA : bf16 [r, K] (out);
 *   dB : bf16 [N, r] (out); outputs must not alias inputs or each other
 *   workspace : >= uno_gated_lora_linear_bwd_workspace(M, N, K, r) bytes (it
 *   holds transposed copies of W, X, dY and the rank-r factors, and counters of
 *   the reduction slices that each call leaves zero: zero it once with
 *   uno_workspace_init before its first use)
 * Limits: M, N, K, r >= 1; M, N, K and r multiples of 8 and all row starts
 * 16-byte aligned (UNO_ERR_UNSUPPORTED otherwise).
 * ------------------------------------------------------------------------- */
size_t uno_gated_lora_linear_bwd_workspace(int M, int N, int K, int r);
int uno_gated_lora_linear_bwd(const void* dY, const void* X, const void* W, const void* W_t,
                              const void* A, const void* B, const uint8_t* row_mask, float scale,
                              void* dX, void* dA, void* dB, int M, int N, int K, int r,
                              void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The Uno decode step on a synthetic decoder stack ("LoopUno", "How it works":
 * each step drafts a block of positions in one forward with the adapter on for
 * the noise positions only, then the unmodified model verifies them and keeps the
 * longest correct prefix, the first position always being the exact AR token;
 * "Setup / Recipe": gated LoRA on all seven projections, and the looped model runs
 * its layers twice per token, "Limits and next steps": drafting with one loop
 * instead of two; "Uno Qwen3-8B" model card, "Evaluation protocol": the noise
 * mode is random_uniform).
 *
 * The stack: h = embed[token]; per layer (all `loops` times, weights shared):
 *   x = rmsnorm(h); q = G_q(x); k = G_k(x); v = G_v(x);
 *   a = attention over a one-token context (each row attends to itself only, so
 *       query head j returns the value of its kv head, j / (query heads / kv heads));
 *   h = h + G_o(a); x = rmsnorm(h); h = h + G_down(silu(G_gate(x)) * G_up(x));
 * then logits = rmsnorm(h) lm_head^T in fp32. G is the row-gated LoRA linear
 * (uno_gated_lora_linear) with the step's row mask; rmsnorm has unit gain and
 * eps 1e-6; activations are stored in bf16, norms, residual adds and SiLU are
 * computed in fp32. The model's attention is a stand-in: a real model's attention
 * over the context is not part of this library.
 * ------------------------------------------------------------------------- */
typedef struct {
  int hidden;        /* H, a multiple of 128                                        */
  int kv_width;      /* width of k and v (kv heads x head_dim)                      */
  int head_dim;      /* a multiple of 8 dividing H and kv_width; the kv heads must  */
                     /* divide the H / head_dim query heads                         */
  int ffn;           /* F, a multiple of 128                                        */
  int vocab;         /* V                                                            */
  int layers;        /* L                                                            */
  int rank;          /* r of the gated adapter, a multiple of 32 (0: no adapter)    */
  float lora_scale;  /* s = alpha / r                                                */
  const void* embed;    /* bf16 [V, H]                                               */
  const void* lm_head;  /* bf16 [V, H]                                               */
  /* HOST arrays of 7 L DEVICE pointers, layer-major, in the order q, k, v, o, gate,
   * up, down. weights: nn.Linear layout [out, in] (q, o [H, H]; k, v [kv_width, H];
   * gate, up [F, H]; down [H, F]); lora_a: [r, in]; lora_b: [out, r] (both may be
   * NULL when rank == 0). The arrays are read during the call only. */
  const void* const* weights;
  const void* const* lora_a;
  const void* const* lora_b;
} uno_model;

/* One forward of M rows (1 <= M <= 64): tokens int32 [M] (device), row_mask uint8
 * [M] (device; 1 = adapter on; NULL = frozen weights on every row), the layer stack
 * run `loops` >= 1 times, logits fp32 [M, V] (out). Every product takes the
 * weight-streaming path of uno_gated_lora_linear. Workspace: >= the size
 * uno_forward_workspace returns (0 for an invalid model), zeroed once.
 * UNO_ERR_UNSUPPORTED for shapes outside the limits above. */
size_t uno_forward_workspace(const uno_model* model, int M);
int uno_forward(const uno_model* model, const int32_t* tokens, const uint8_t* row_mask, int M, int loops,
                float* logits, void* workspace, size_t ws_bytes, void* stream);

/* One Uno decode step of S sequences with blocks of b rows (S * b <= 64):
 *  1. block rows [seed_tokens[s], n_1 .. n_{b-1}]: noise token n_i is
 *     ((w >> 40) * V) >> 24 for Philox-4x64-10 word 0 at key (sp.seed, seq_ids[s]),
 *     counter (pos_offsets[s] + i, 2, 0, 0) (random_uniform noise);
 *  2. draft forward of the S * b rows, `draft_loops` loops, adapter on rows 1..b-1;
 *  3. draft tokens d ~ q~ of those logits (uno_draft_sample);
 *  4. verify forward of the rows [seed_tokens[s], d_1 .. d_{b-1}] with the frozen
 *     weights, `verify_loops` loops;
 *  5. uno_verify_block with p = the verify logits, q = the draft logits.
 * out_tokens int32 [S, b], accept_len int32 [S] and resampled int32 [S] as for
 * uno_verify_block (accept_len and resampled may be NULL). Optional outputs:
 * draft_tokens int32 [S, b], draft_logits and verify_logits fp32 [S * b, V] (the
 * step then writes its logits there instead of the workspace). The workspace
 * (>= uno_decode_step_workspace, zeroed once) begins with counter areas that each
 * call leaves zero, so one workspace serves calls of any shape. Every kernel runs
 * on `stream`, and the call makes no allocation and no synchronisation, so it can
 * be recorded into a HIP graph. Limits: 1 <= b <= 64, S * b <= 64, loops >= 1. */
size_t uno_decode_step_workspace(const uno_model* model, int S, int b);
int uno_decode_step(const uno_model* model, int S, int b, int draft_loops, int verify_loops,
                    uno_sampling_params sp, const int32_t* seed_tokens, const int64_t* seq_ids,
                    const int64_t* pos_offsets, int32_t* out_tokens, int32_t* accept_len, int32_t* resampled,
                    int32_t* draft_tokens, float* draft_logits, float* verify_logits,
                    void* workspace, size_t ws_bytes, void* stream);

/* One autoregressive step of S sequences (1 <= S <= 64): a frozen forward of the
 * rows tokens[s] (`loops` loops), then the AR token out_tokens[s] = the inverse CDF
 * of the filtered distribution at u_res of (sp.seed, seq_ids[s]; pos_offsets[s], 0,
 * 0, 0): the same draw as slot 0 of uno_verify_block, so it equals out_tokens[s, 0]
 * of a decode step with the same seed token, sequence id and position.
 * logits fp32 [S, V] (optional out). Workspace: >= uno_ar_step_workspace, zeroed
 * once. */
size_t uno_ar_step_workspace(const uno_model* model, int S);
int uno_ar_step(const uno_model* model, int S, int loops, uno_sampling_params sp, const int32_t* tokens,
                const int64_t* seq_ids, const int64_t* pos_offsets, int32_t* out_tokens, float* logits,
                void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UNO_H */
