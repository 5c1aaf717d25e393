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

}  // namespace uno
