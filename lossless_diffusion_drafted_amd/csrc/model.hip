// The Uno decode step on a synthetic decoder stack ("LoopUno", "How it works":
// each step drafts a block of positions in one forward with the adapter switched
// on for the noise positions only, then the unmodified model verifies them and
// keeps the longest correct prefix; the first position is always the exact AR
// token. "Setup / Recipe": the gated adapter sits on all seven projections; the
// looped model runs its 22 layers twice per token. "Uno Qwen3-8B" model card,
// "Evaluation protocol": noise tokens are drawn uniformly from the vocabulary).
//
// One step of S sequences and block b:
//   1. block rows [seed, noise_1 .. noise_{b-1}] per sequence; noise tokens are
//      uniform over the vocabulary from Philox stream 2 (counter = position + i);
//   2. draft forward over those S*b rows, adapter on the noise rows only;
//   3. draft sampler: d_i ~ q~_i (Philox stream 1);
//   4. verify forward over [seed, d_1 .. d_{b-1}] with the frozen weights;
//   5. lossless verification (p from step 4, q from step 2).
// Layer of the stack (weights shared by every loop of a looped model):
//   x = rmsnorm(h); q, k, v = gated(x); a = attention over a one-token context
//   (each row sees only itself, so every query head returns its kv head's v);
//   h += gated_o(a); x = rmsnorm(h); h += gated_down(silu(gated_gate(x)) *
//   gated_up(x)). Then logits = rmsnorm(h) . lm_head^T in fp32.
// Activations are stored in bf16 between kernels; norms, the residual add and
// SiLU run in fp32. RMSNorm has unit gain and eps = 1e-6.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace uno {
namespace {

constexpr int MT = 256;          // threads of the row kernels
constexpr float kNormEps = 1e-6f;

__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < MT / 64; ++i) t += sh[i];
  __syncthreads();
  return t;
}

__device__ __forceinline__ void unpack8(const uint4& u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_lo(w[e]);
    f[2 * e + 1] = bf16_hi(w[e]);
  }
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = uint32_t(f32_to_bf16(f[2 * e])) | (uint32_t(f32_to_bf16(f[2 * e + 1])) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// h[m] = E[tokens[m]] (or h[m] + y[m] when y is given, rounded to bf16), then
// x[m] = bf16(h[m] / sqrt(mean(h[m]^2) + eps)). One workgroup per row; H % 8 == 0.
__global__ __launch_bounds__(MT) void norm_kernel(const int32_t* tokens, const uint16_t* embed, int V,
                                                  uint16_t* h, const uint16_t* y, uint16_t* x, int H) {
  __shared__ float sh[MT / 64];
  const int m = blockIdx.x;
  uint16_t* hr = h + size_t(m) * H;
  const uint16_t* src = hr;
  if (tokens) {
    int tok = tokens[m];
    tok = tok < 0 ? 0 : (tok >= V ? V - 1 : tok);
    src = embed + size_t(tok) * H;
  }
  const int nc = H / 8;
  float ss = 0.0f;
  for (int c = threadIdx.x; c < nc; c += MT) {
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(src + c * 8), f);
    if (y) {
      float g[8];
      unpack8(*reinterpret_cast<const uint4*>(y + size_t(m) * H + c * 8), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = bf16_to_f32(f32_to_bf16(f[e] + g[e]));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
    *reinterpret_cast<uint4*>(hr + c * 8) = pack8(f);
  }
  const float inv = 1.0f / sqrtf(block_sum(ss, sh) / float(H) + kNormEps);
  for (int c = threadIdx.x; c < nc; c += MT) {
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(hr + c * 8), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] *= inv;
    *reinterpret_cast<uint4*>(x + size_t(m) * H + c * 8) = pack8(f);
  }
}

// a[m, j] = v[m, kv_head(j) * hd + j % hd]: attention over a one-token context
// returns each query head its kv head's value row (v rows vstride apart).
// 16-byte copies (hd % 8 == 0).
__global__ __launch_bounds__(MT) void expand_kernel(const uint16_t* v, int vstride, uint16_t* a, int M, int H,
                                                    int KVW, int hd) {
  const int nc = H / 8;
  const int group = (H / hd) / (KVW / hd);
  for (size_t e = size_t(blockIdx.x) * MT + threadIdx.x; e < size_t(M) * nc; e += size_t(gridDim.x) * MT) {
    const int m = int(e / nc), c = int(e % nc);
    const int j = c * 8, head = j / hd;
    const int src = (head / group) * hd + j % hd;
    *reinterpret_cast<uint4*>(a + size_t(m) * H + j) =
        *reinterpret_cast<const uint4*>(v + size_t(m) * vstride + src);
  }
}

// out[m, :] = bf16(silu(g[m, :]) * u[m, :]) over F columns, silu(g) = g / (1 +
// exp(-g)) in fp32; g and u rows ld elements apart.
__global__ __launch_bounds__(MT) void silu_mul_kernel(const uint16_t* g, const uint16_t* u, int ld, uint16_t* out,
                                                      int M, int F) {
  const int nc = F / 8;
  for (size_t c = size_t(blockIdx.x) * MT + threadIdx.x; c < size_t(M) * nc; c += size_t(gridDim.x) * MT) {
    const size_t m = c / nc, j = (c % nc) * 8;
    float gf[8], uf[8], o[8];
    unpack8(*reinterpret_cast<const uint4*>(g + m * ld + j), gf);
    unpack8(*reinterpret_cast<const uint4*>(u + m * ld + j), uf);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = gf[e] / (1.0f + expf(-gf[e])) * uf[e];
    *reinterpret_cast<uint4*>(out + m * F + j) = pack8(o);
  }
}

// Block rows of a step: row (s, 0) is the seed token; rows (s, i >= 1) are noise
// tokens ((w >> 40) * V) >> 24 of Philox word 0 at (seed, seq_id; pos + i, 2, 0, 0)
// (draft == null), or the draft tokens (draft given: the verify forward's rows).
// mask (optional) marks the noise rows.
__global__ void block_rows_kernel(const int32_t* seed_tok, const int32_t* draft, const int64_t* seq_ids,
                                  const int64_t* pos, int S, int b, int V, uint64_t seed, int32_t* tokens,
                                  uint8_t* mask) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= S * b) return;
  const int s = g / b, i = g - s * b;
  int tok;
  if (i == 0) {
    tok = seed_tok[s];
  } else if (draft) {
    tok = draft[g];
  } else {
    const Philox4 ph = philox4x64_10(uint64_t(pos[s] + i), 2ull, 0ull, 0ull, seed, uint64_t(seq_ids[s]));
    tok = int(((ph.w[0] >> 40) * uint64_t(V)) >> 24);
  }
  tokens[g] = tok;
  if (mask) mask[g] = i > 0 ? 1 : 0;
}

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// Step workspace: [GEMM tickets 64 KB][verify tickets and records 64 KB][rest].
// The first two areas hold only self-clearing counters and records, so they stay
// valid across calls of any shape.
constexpr size_t kStepTickets = 65536;
constexpr size_t kStepVerify = 65536;
constexpr size_t kStepHead = kStepTickets + kStepVerify;

struct FwdBufs {
  uint16_t *h, *x, *q, *k, *v, *a, *o, *g, *u, *mm, *d;
  uint16_t *qkv, *gu;   // outputs of the grouped q | k | v and gate | up products
  void* gemm;           // T and slice tiles of the gated products
};

size_t gemm_scratch(const ModelDesc& md, int M) {
  const int H = md.hidden, F = md.ffn, KVW = md.kv_width;
  // {K, N, rank}: the seven projections, the grouped q | k | v and gate | up
  // products (stacked ranks), the LM head
  const int shapes[10][3] = {{H, H, 1},     {H, KVW, 1},       {H, KVW, 1}, {H, H, 1},
                             {H, F, 1},     {H, F, 1},         {F, H, 1},   {H, H + 2 * KVW, 3},
                             {H, 2 * F, 2}, {H, md.vocab, 0}};
  size_t n = 0;
  for (int i = 0; i < 10; ++i) {
    const size_t b = gemm_workspace_bytes(M, shapes[i][1], shapes[i][0], md.rank * shapes[i][2]);
    if (b > n) n = b;
  }
  return n;                 // includes the 64 KB ticket area, which the step keeps apart
}

FwdBufs carve(const ModelDesc& md, int M, char* p) {
  const size_t H = md.hidden, F = md.ffn, KVW = md.kv_width, m = M;
  FwdBufs f;
  auto take = [&](size_t elems) {
    uint16_t* q = reinterpret_cast<uint16_t*>(p);
    p += al256(elems * 2);
    return q;
  };
  f.h = take(m * H);
  f.x = take(m * H);
  f.q = take(m * H);
  f.k = take(m * KVW);
  f.v = take(m * KVW);
  f.a = take(m * H);
  f.o = take(m * H);
  f.g = take(m * F);
  f.u = take(m * F);
  f.mm = take(m * F);
  f.d = take(m * H);
  f.qkv = take(m * (H + 2 * KVW));
  f.gu = take(m * 2 * F);
  f.gemm = p;
  return f;
}

size_t fwd_bytes(const ModelDesc& md, int M) {
  const size_t H = md.hidden, F = md.ffn, KVW = md.kv_width, m = M;
  return al256(m * H * 2) * 6 + al256(m * KVW * 2) * 2 + al256(m * F * 2) * 3 + al256(m * (H + 2 * KVW) * 2) +
         al256(m * 2 * F * 2) + gemm_scratch(md, M);
}

// Projection `proj` of a layer, or with n > 1 the n projections proj .. proj + n -
// 1 as one grouped product (their weights, and adapter factors, stacked in memory;
// `cols` gives each one's output width).
GemmArgs gated_args(const ModelDesc& md, int layer, int proj, const uint16_t* x, uint16_t* y, int M, int K,
                    const int* cols, int n, const uint8_t* mask, unsigned* tickets, void* scratch) {
  GemmArgs g{};
  g.X = x;
  g.W = md.w[layer * 7 + proj];
  const bool lora = md.rank > 0 && mask != nullptr;
  g.A = lora ? md.lora_a[layer * 7 + proj] : nullptr;
  g.B = lora ? md.lora_b[layer * 7 + proj] : nullptr;
  g.r = lora ? md.rank : 0;
  g.row_mask = lora ? mask : nullptr;
  g.scale = md.lora_scale;
  g.Y = y;
  g.M = M;
  g.K = K;
  g.N = 0;
  for (int i = 0; i < n; ++i) {
    if (i > 0) g.gstart[i - 1] = g.N;
    g.N += cols[i];
  }
  g.groups = n;
  g.ws = scratch;
  g.tickets = tickets;
  return g;
}

hipError_t gated(const ModelDesc& md, int layer, int proj, const uint16_t* x, uint16_t* y, int M, int K,
                 const int* cols, int n, const uint8_t* mask, unsigned* tickets, void* scratch, hipStream_t st) {
  return launch_gemm(gated_args(md, layer, proj, x, y, M, K, cols, n, mask, tickets, scratch), st);
}

// Whether projections proj .. proj + n - 1 of a layer can run as one grouped
// product: each one's weight (and adapter factors) directly after the previous
// one's in memory, and every output width a multiple of 32.
bool stacked(const ModelDesc& md, int layer, int proj, const int* cols, int n, int K, bool lora) {
  auto next_to = [](const void* a, const void* b, size_t bytes) {
    return static_cast<const char*>(a) + bytes == static_cast<const char*>(b);
  };
  for (int i = 0; i < n; ++i)
    if (cols[i] % 32 != 0) return false;
  for (int i = 1; i < n; ++i) {
    const int j = layer * 7 + proj + i;
    if (!next_to(md.w[j - 1], md.w[j], size_t(cols[i - 1]) * K * 2)) return false;
    if (lora && (!next_to(md.lora_a[j - 1], md.lora_a[j], size_t(md.rank) * K * 2) ||
                 !next_to(md.lora_b[j - 1], md.lora_b[j], size_t(cols[i - 1]) * md.rank * 2)))
      return false;
  }
  return true;
}

// The forward of M rows through the stack (`loops` times) and the LM head.
hipError_t forward(const ModelDesc& md, const int32_t* tokens, const uint8_t* mask, int M, int loops,
                   float* logits, unsigned* tickets, char* area, hipStream_t st) {
  const int H = md.hidden, F = md.ffn, KVW = md.kv_width;
  const FwdBufs f = carve(md, M, area);
  hipLaunchKernelGGL(norm_kernel, dim3(M), dim3(MT), 0, st, tokens, static_cast<const uint16_t*>(md.embed),
                     md.vocab, f.h, nullptr, f.x, H);
  hipError_t e = hipGetLastError();
  const int eg = int((size_t(M) * H / 8 + MT - 1) / MT);
  const int fg = int((size_t(M) * F / 8 + MT - 1) / MT);
  const bool lora = md.rank > 0 && mask != nullptr;
  const int qkv_cols[3] = {H, KVW, KVW}, gu_cols[2] = {F, F}, hcol[1] = {H}, kcol[1] = {KVW}, fcol[1] = {F};
  for (int it = 0; it < loops && e == hipSuccess; ++it) {
    for (int l = 0; l < md.layers && e == hipSuccess; ++l) {
      // q | k | v and gate | up run as grouped products when stacked in memory: one
      // launch (and one LoRA-down) instead of three or two, each short launch's
      // fixed cost paid once.
      const uint16_t* v = f.v;
      int vstride = KVW;
      if (stacked(md, l, 0, qkv_cols, 3, H, lora)) {
        if ((e = gated(md, l, 0, f.x, f.qkv, M, H, qkv_cols, 3, mask, tickets, f.gemm, st)) != hipSuccess) break;
        v = f.qkv + H + KVW;
        vstride = H + 2 * KVW;
      } else {
        if ((e = gated(md, l, 0, f.x, f.q, M, H, hcol, 1, mask, tickets, f.gemm, st)) != hipSuccess) break;
        if ((e = gated(md, l, 1, f.x, f.k, M, H, kcol, 1, mask, tickets, f.gemm, st)) != hipSuccess) break;
        if ((e = gated(md, l, 2, f.x, f.v, M, H, kcol, 1, mask, tickets, f.gemm, st)) != hipSuccess) break;
      }
      // The o-projection's input: each query head's attention output is its kv
      // head's value row. With 128-wide heads the small-M product reads those
      // blocks from v itself; otherwise they are copied out first.
      GemmArgs og = gated_args(md, l, 3, v, f.o, M, H, hcol, 1, mask, tickets, f.gemm);
      og.x_stride = vstride;
      og.x_group = md.head_dim == 128 ? H / KVW : 0;
      if (og.x_group == 0 || !gemm_gathers_x(og)) {
        hipLaunchKernelGGL(expand_kernel, dim3(eg < 4096 ? eg : 4096), dim3(MT), 0, st, v, vstride, f.a, M, H, KVW,
                           md.head_dim);
        og.X = f.a;
        og.x_stride = og.x_group = 0;
      }
      if ((e = launch_gemm(og, st)) != hipSuccess) break;
      hipLaunchKernelGGL(norm_kernel, dim3(M), dim3(MT), 0, st, nullptr, nullptr, 0, f.h, f.o, f.x, H);
      if (stacked(md, l, 4, gu_cols, 2, H, lora)) {
        if ((e = gated(md, l, 4, f.x, f.gu, M, H, gu_cols, 2, mask, tickets, f.gemm, st)) != hipSuccess) break;
        hipLaunchKernelGGL(silu_mul_kernel, dim3(fg < 4096 ? fg : 4096), dim3(MT), 0, st, f.gu, f.gu + F, 2 * F,
                           f.mm, M, F);
      } else {
        if ((e = gated(md, l, 4, f.x, f.g, M, H, fcol, 1, mask, tickets, f.gemm, st)) != hipSuccess) break;
        if ((e = gated(md, l, 5, f.x, f.u, M, H, fcol, 1, mask, tickets, f.gemm, st)) != hipSuccess) break;
        hipLaunchKernelGGL(silu_mul_kernel, dim3(fg < 4096 ? fg : 4096), dim3(MT), 0, st, f.g, f.u, F, f.mm, M,
                           F);
      }
      if ((e = gated(md, l, 6, f.mm, f.d, M, F, hcol, 1, mask, tickets, f.gemm, st)) != hipSuccess) break;
      hipLaunchKernelGGL(norm_kernel, dim3(M), dim3(MT), 0, st, nullptr, nullptr, 0, f.h, f.d, f.x, H);
      e = hipGetLastError();
    }
  }
  if (e != hipSuccess) return e;
  GemmArgs g{};
  g.X = f.x;
  g.W = md.lm_head;
  g.Y = logits;
  g.y_f32 = true;
  g.M = M;
  g.N = md.vocab;
  g.K = H;
  g.r = 0;
  g.scale = 1.0f;
  g.ws = f.gemm;
  g.tickets = tickets;
  return launch_gemm(g, st);
}

}  // namespace

int model_check(const ModelDesc& md, int M) {
  if (md.hidden <= 0 || md.kv_width <= 0 || md.head_dim <= 0 || md.ffn <= 0 || md.vocab <= 0 || md.layers < 0)
    return 1;
  if (md.hidden % md.head_dim || md.kv_width % md.head_dim || md.head_dim % 8) return 1;
  if ((md.hidden / md.head_dim) % (md.kv_width / md.head_dim)) return 1;
  // every product of the step takes the weight-streaming path, which reads 128-wide groups
  if (md.hidden % 128 || md.ffn % 128 || md.rank % 32 || md.rank < 0) return 1;
  if (M < 1 || M > 64) return 2;
  return 0;
}

size_t forward_workspace_bytes(const ModelDesc& md, int M) {
  return kStepHead + fwd_bytes(md, M) + al256(size_t(M) * 4);
}

hipError_t launch_forward(const ModelDesc& md, const int32_t* tokens, const uint8_t* mask, int M, int loops,
                          float* logits, void* ws, hipStream_t st) {
  char* c = static_cast<char*>(ws);
  return forward(md, tokens, mask, M, loops, logits, reinterpret_cast<unsigned*>(c), c + kStepHead, st);
}

size_t step_workspace_bytes(const ModelDesc& md, int S, int b) {
  const size_t M = size_t(S) * b;
  // forward area, then tokens [M] x 2, mask [M], drafts [M], draft / verify logits [M, V] fp32
  return kStepHead + fwd_bytes(md, int(M)) + al256(M * 4) * 3 + al256(M) + al256(M * size_t(md.vocab) * 4) * 2 +
         al256(size_t(S) * 4) * 2;
}

hipError_t launch_decode_step(const ModelDesc& md, const StepArgs& a, hipStream_t st) {
  const int S = a.S, b = a.b, M = S * b;
  char* c = static_cast<char*>(a.ws);
  unsigned* tickets = reinterpret_cast<unsigned*>(c);
  void* vws = c + kStepTickets;
  char* fwd = c + kStepHead;
  char* p = fwd + fwd_bytes(md, M);
  auto take = [&](size_t bytes) {
    char* q = p;
    p += al256(bytes);
    return q;
  };
  int32_t* tok_d = reinterpret_cast<int32_t*>(take(size_t(M) * 4));
  int32_t* tok_v = reinterpret_cast<int32_t*>(take(size_t(M) * 4));
  int32_t* drafts = reinterpret_cast<int32_t*>(take(size_t(M) * 4));
  uint8_t* mask = reinterpret_cast<uint8_t*>(take(size_t(M)));
  float* zd = reinterpret_cast<float*>(take(size_t(M) * md.vocab * 4));
  float* zv = reinterpret_cast<float*>(take(size_t(M) * md.vocab * 4));
  int32_t* acc_scratch = reinterpret_cast<int32_t*>(take(size_t(S) * 4));
  int32_t* res_scratch = reinterpret_cast<int32_t*>(take(size_t(S) * 4));
  if (a.draft_logits) zd = a.draft_logits;
  if (a.verify_logits) zv = a.verify_logits;
  if (a.drafts) drafts = a.drafts;

  const int bg = (M + 255) / 256;
  hipLaunchKernelGGL(block_rows_kernel, dim3(bg), dim3(256), 0, st, a.seed_tokens, nullptr, a.seq_ids, a.pos, S,
                     b, md.vocab, a.sp.seed, tok_d, mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = forward(md, tok_d, mask, M, a.draft_loops, zd, tickets, fwd, st)) != hipSuccess) return e;
  DraftArgs da{};
  da.q = zd;
  da.bf16 = false;
  da.seq_ids = a.seq_ids;
  da.pos = a.pos;
  da.S = S;
  da.b = b;
  da.V = md.vocab;
  da.sp = a.sp;
  da.draft = drafts;
  da.flags = nullptr;
  if ((e = launch_draft(da, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(block_rows_kernel, dim3(bg), dim3(256), 0, st, a.seed_tokens, drafts, a.seq_ids, a.pos, S, b,
                     md.vocab, a.sp.seed, tok_v, nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = forward(md, tok_v, nullptr, M, a.verify_loops, zv, tickets, fwd, st)) != hipSuccess) return e;
  VerifyArgs va{};
  va.p = zv;
  va.q = zd;
  va.bf16 = false;
  va.draft = drafts;
  va.seq_ids = a.seq_ids;
  va.pos = a.pos;
  va.S = S;
  va.b = b;
  va.V = md.vocab;
  va.sp = a.sp;
  va.out_tokens = a.out_tokens;
  va.accept_len = a.accept_len ? a.accept_len : acc_scratch;
  va.resampled = a.resampled ? a.resampled : res_scratch;
  va.slot_accept = nullptr;
  va.diag = nullptr;
  va.ws = vws;
  return launch_verify(va, st);
}

size_t ar_step_workspace_bytes(const ModelDesc& md, int S) {
  return kStepHead + fwd_bytes(md, S) + al256(size_t(S) * md.vocab * 4) + al256(size_t(S) * 4) * 2;
}

hipError_t launch_ar_step(const ModelDesc& md, const StepArgs& a, hipStream_t st) {
  const int S = a.S;
  char* c = static_cast<char*>(a.ws);
  unsigned* tickets = reinterpret_cast<unsigned*>(c);
  void* vws = c + kStepTickets;
  char* fwd = c + kStepHead;
  char* p = fwd + fwd_bytes(md, S);
  float* z = reinterpret_cast<float*>(p);
  p += al256(size_t(S) * md.vocab * 4);
  int32_t* acc_scratch = reinterpret_cast<int32_t*>(p);
  int32_t* res_scratch = acc_scratch + al256(size_t(S) * 4) / 4;
  if (a.verify_logits) z = a.verify_logits;
  hipError_t e = forward(md, a.seed_tokens, nullptr, S, a.verify_loops, z, tickets, fwd, st);
  if (e != hipSuccess) return e;
  // The AR token is the verifier's slot 0: the inverse CDF of p~ at u_res of
  // (seed, seq_id; pos, 0, 0, 0), the same draw that gives slot 0 of a block.
  VerifyArgs va{};
  va.p = z;
  va.q = z;
  va.bf16 = false;
  va.draft = a.seed_tokens;            // slot 0's draft is never read
  va.seq_ids = a.seq_ids;
  va.pos = a.pos;
  va.S = S;
  va.b = 1;
  va.V = md.vocab;
  va.sp = a.sp;
  va.out_tokens = a.out_tokens;
  va.accept_len = acc_scratch;
  va.resampled = res_scratch;
  va.ws = vws;
  return launch_verify(va, st);
}

}  // namespace uno
