// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace uno {

struct SamplingArgs {
  double temperature;
  double top_p;
  int top_k;
  uint64_t seed;
};

struct VerifyArgs {
  const void* p;
  const void* q;
  bool bf16;
  const int32_t* draft;
  const int64_t* seq_ids;
  const int64_t* pos;
  int S, b, V;
  SamplingArgs sp;
  int32_t* out_tokens;
  int32_t* accept_len;
  int32_t* resampled;
  uint8_t* slot_accept;
  float* diag;
  void* ws;
};

struct DraftArgs {
  const void* q;
  bool bf16;
  const int64_t* seq_ids;
  const int64_t* pos;
  int S, b, V;
  SamplingArgs sp;
  int32_t* draft;
  int32_t* flags;
};

struct TvArgs {
  const void* teacher;
  const void* student;
  bool bf16;
  const uint8_t* mask;
  int R, V;
  float temperature;
  float* loss;
  float* tv_rows;
  void* grad;
  void* ws;
};

struct GemmArgs {
  const void* X;
  const void* W;
  const void* A;
  const void* B;
  const uint8_t* row_mask;
  float scale;
  void* Y;
  int M, N, K, r;
  void* ws;
  unsigned* tickets = nullptr;   // slice tickets kept apart from ws (else the first 64 KB of ws)
  bool y_f32 = false;            // Y is fp32 (small-M path only)
  // Grouped products (small-M path only): W, A and B stack `groups` products that
  // share X; group g owns columns [gstart[g-1], gstart[g]) of Y and rows
  // [g r, (g + 1) r) of A, and B stacks the groups' B rows like W. gstart values
  // are multiples of 32. The workspace is sized for rank groups * r.
  int groups = 1;
  int gstart[2] = {0, 0};
  // X gathered by heads (small-M path only): with x_group > 0, X row m is read from
  // rows x_stride elements apart, and its 128-column block h (a head of width 128)
  // from source block h / x_group: X = the heads of a one-token attention output
  // expanded from their shared kv heads. K must be a multiple of 128.
  int x_stride = 0;
  int x_group = 0;
};

size_t verify_workspace_bytes(int S, int b);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);
// The verifier's library-owned scratch (a static device array): its size, and its
// device address on the current device, cleared on `stream` at the first request.
size_t verify_scratch_bytes();
hipError_t verify_scratch(void** out, hipStream_t stream);
hipError_t launch_draft(const DraftArgs& a, hipStream_t stream);
size_t tv_workspace_bytes(int R);
int tv_max_vocab(bool bf16);          // largest V one row team covers on this device
hipError_t launch_tv(const TvArgs& a, hipStream_t stream);
size_t gemm_workspace_bytes(int M, int N, int K, int r);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
// Whether launch_gemm takes these arguments' X gathered by heads (x_group > 0).
bool gemm_gathers_x(const GemmArgs& a);

struct GemmBwdArgs {
  const void* dY;
  const void* X;
  const void* W;
  const void* Wt;  // W^T [K, N] or null (then W is transposed into the workspace)
  const void* A;
  const void* B;
  const uint8_t* row_mask;
  float scale;
  void* dX;        // may be null
  void* dA;
  void* dB;
  int M, N, K, r;
  void* ws;
};
size_t gemm_bwd_workspace_bytes(int M, int N, int K, int r);
hipError_t launch_gemm_bwd(const GemmBwdArgs& a, hipStream_t stream);
hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t stream);

// Synthetic decoder stack of the decode step (csrc/model.hip).
struct ModelDesc {
  int hidden, kv_width, head_dim, ffn, vocab, layers, rank;
  float lora_scale;
  const void* embed;             // bf16 [vocab, hidden]
  const void* lm_head;           // bf16 [vocab, hidden]
  const void* const* w;          // host array [layers * 7]: q, k, v, o, gate, up, down
  const void* const* lora_a;     // host array [layers * 7] (rank > 0)
  const void* const* lora_b;
};

struct StepArgs {
  int S, b, draft_loops, verify_loops;
  SamplingArgs sp;
  const int32_t* seed_tokens;    // [S]
  const int64_t* seq_ids;        // [S]
  const int64_t* pos;            // [S]
  int32_t* out_tokens;           // [S, b]
  int32_t* accept_len;           // [S] (optional)
  int32_t* resampled;            // [S] (optional)
  int32_t* drafts;               // [S, b] (optional)
  float* draft_logits;           // [S * b, vocab] (optional)
  float* verify_logits;          // [S * b, vocab] (optional)
  void* ws;
};

// 0 = valid; 1 = the model's shapes are not supported; 2 = M outside [1, 64].
int model_check(const ModelDesc& md, int M);
size_t forward_workspace_bytes(const ModelDesc& md, int M);
hipError_t launch_forward(const ModelDesc& md, const int32_t* tokens, const uint8_t* mask, int M, int loops,
                          float* logits, void* ws, hipStream_t stream);
size_t step_workspace_bytes(const ModelDesc& md, int S, int b);
hipError_t launch_decode_step(const ModelDesc& md, const StepArgs& a, hipStream_t stream);
size_t ar_step_workspace_bytes(const ModelDesc& md, int S);
hipError_t launch_ar_step(const ModelDesc& md, const StepArgs& a, hipStream_t stream);

}  // namespace uno
