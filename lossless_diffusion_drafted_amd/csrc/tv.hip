// Total-variation self-distillation loss with its student gradient, fused into
// one pass over the logits ("LoopUno: Turning Agentic Looped LLMs into
// Diffusion LLMs in One Hour", "How it works" -> "Training is self-distillation":
// the student is pushed towards the frozen teacher by minimising TV on the
// response tokens, and 1 - TV is the acceptance rate of lossless verification).
//
// Per response row r (p = softmax(teacher/T), q = softmax(student/T), full vocab):
//   TV_r = 1/2 sum_v |p_v - q_v|,   G_r = 1/2 sum_v q_v sign(q_v - p_v),
//   grad[r, j] = q_j (1/2 sign(q_j - p_j) - G_r) / (T N),   N = #response rows,
//   loss = sum_r TV_r / N.
// Rows outside the response mask get TV 0 and a zero gradient.
//
// Design (HBM-bound: read both rows once, write the gradient once).
// * A row is split over a team of G workgroups that stay resident for the whole
//   launch (cooperative launch). Each thread keeps its slice of both rows in
//   registers as fp32 exp values, so nothing is read twice: per element the
//   three passes cost about 25 VALU lane-ops, with 6 of them for exponentials.
// * Pass 1: per-thread max and sum of exp2((x - m) log2(e)/T); workgroup
//   partials go to the team through device-coherent records, then a team
//   barrier. Pass 2: p, q from the stored exps, sum |q - p| and sum q sign(q - p);
//   the registers now hold (sign, q). Second barrier. Pass 3: the gradient,
//   rounded to bf16 by the hardware conversion, written with streaming stores.
// * Team exchanges are tagged record words in the workspace: each member stores
//   its partials with a tag (call epoch, barrier number) and polls the other
//   members' words until their tags match, so no wait drains the gradient
//   stores in flight. Polls are bounded; one that runs out sets an abort flag
//   that every poller checks, so every wait ends (the loss is then NaN).

#include "../../include/uno.h"
#include "common.h"
#include "kernels.h"

#include <mutex>

namespace uno {
namespace {

// One 1024-thread workgroup per CU; at V = 151936 a team is 4 workgroups. Measured
// against 512-thread workgroups (two per CU, teams of 8): 5.24 against 5.76 ms on the
// 32768 x 151936 self-distillation workload (fewer members per team exchange).
constexpr int TT = 1024;                // threads per workgroup
constexpr int TWAVES = TT / kWave;
constexpr int EPT = 40;                 // elements of each row per thread
constexpr int CHUNK = TT * EPT;         // elements of each row per workgroup
constexpr int kMaxWg = 4096;            // resident workgroups the workspace can serve
constexpr unsigned kSpinLimit = 1u << 21;
constexpr float kLog2e = 1.4426950408889634f;

struct TvPlan {
  int G;          // workgroups per row team
  int nteams;
  int xcd;        // 1: team members share an XCD (grid is a multiple of 8 G)
};

// Workspace: [header | team records (16 words of 64 bits per workgroup) | per-row
// TV (double)]. A record word holds an fp32 value in its low half and a tag in
// its high half: (call epoch << 16) | exchange number.
struct TvHeader {
  unsigned done;
  unsigned abort;
  unsigned nresp;
  unsigned epoch;      // calls completed (mod 2^16 in tags)
};
constexpr int kRecWords = 16;
constexpr size_t kRecOff = 256;
constexpr size_t kRowOff = kRecOff + size_t(kMaxWg) * kRecWords * 8;

struct TvLds {
  float wred[TWAVES][4];
  float rec[64][4];
  int ok;
  int last;
};

// Two floats as a bf16 pair (round to nearest even), a in the low half: one
// v_cvt_pk_bf16_f32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename E> struct TvElem;
template <> struct TvElem<uint16_t> {
  static constexpr int VN = 8;
  __device__ static void unpack(const uint4& v, float (&x)[8]) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
  __device__ static float scalar(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static uint4 pack(const float (&g)[8]) {
    return make_uint4(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                      pack_bf16x2(g[6], g[7]));
  }
  __device__ static void store_scalar(uint16_t* p, float g) { *p = __builtin_bit_cast(uint16_t, (__bf16)g); }
};
template <> struct TvElem<float> {
  static constexpr int VN = 4;
  __device__ static void unpack(const uint4& v, float (&x)[4]) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
  __device__ static float scalar(const float* p) { return *p; }
  __device__ static uint4 pack(const float (&g)[4]) {
    return make_uint4(__float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]),
                      __float_as_uint(g[3]));
  }
  __device__ static void store_scalar(float* p, float g) { *p = g; }
};

// Element j of this thread's slice sits at row offset c0 + (j / VN * TT + tid) * VN + j % VN.
// The buffer view starts at the slice (the range check covers only the per-lane
// offset), so lanes past the row end read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const void* row, int V, int c0, int esize) {
  return make_row_rsrc(static_cast<const char*>(row) + size_t(c0) * esize, uint32_t(size_t(V - c0) * esize));
}

template <typename E>
__device__ __forceinline__ void issue_slice(const E* row, int V, int c0, uint4 (&raw)[EPT / TvElem<E>::VN]) {
  const __amdgpu_buffer_rsrc_t rs = slice_rsrc(row, V, c0, int(sizeof(E)));
#pragma unroll
  for (int u = 0; u < EPT / TvElem<E>::VN; ++u)
    raw[u] = buffer_load16(rs, uint32_t((u * TT + int(threadIdx.x)) * 16), 0u);
}

template <typename E>
__device__ __forceinline__ void unpack_slice(const uint4 (&raw)[EPT / TvElem<E>::VN], float (&x)[EPT]) {
  constexpr int VN = TvElem<E>::VN;
#pragma unroll
  for (int u = 0; u < EPT / VN; ++u) {
    float v[VN];
    TvElem<E>::unpack(raw[u], v);
#pragma unroll
    for (int j = 0; j < VN; ++j) x[u * VN + j] = v[j];
  }
}

// Rows that are not 16-byte aligned: element loads (correct, not fast).
template <typename E>
__device__ __forceinline__ void load_slice_scalar(const E* row, int V, int c0, float (&x)[EPT]) {
  constexpr int VN = TvElem<E>::VN;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < EPT / VN; ++u) {
#pragma unroll
    for (int j = 0; j < VN; ++j) {
      const int e = c0 + (u * TT + tid) * VN + j;
      x[u * VN + j] = e < V ? TvElem<E>::scalar(row + e) : 0.0f;
    }
  }
}

// Both slices of a row; on the vector path every load is issued before any is
// waited on.
template <typename E, bool VEC>
__device__ __forceinline__ void load_slices(const E* trow, const E* srow, int V, int c0, float (&xt)[EPT],
                                            float (&xs)[EPT]) {
  if constexpr (VEC) {
    uint4 rt[EPT / TvElem<E>::VN], rs[EPT / TvElem<E>::VN];
    issue_slice<E>(trow, V, c0, rt);
    issue_slice<E>(srow, V, c0, rs);
    unpack_slice<E>(rt, xt);
    unpack_slice<E>(rs, xs);
  } else {
    load_slice_scalar<E>(trow, V, c0, xt);
    load_slice_scalar<E>(srow, V, c0, xs);
  }
}

// Gradient of this thread's slice from the stored (sign, q): g = q (s h + g0),
// computed and written one 16-byte vector at a time. With zero = true the slice
// is cleared instead (rows outside the response mask).
template <typename E, bool VEC>
__device__ __forceinline__ void store_grad(E* row, int V, int c0, const float (&sg)[EPT], const float (&q)[EPT],
                                           float h, float g0, bool zero) {
  using EL = TvElem<E>;
  constexpr int VN = EL::VN;
  const int tid = threadIdx.x;
  if constexpr (VEC) {
    const __amdgpu_buffer_rsrc_t rs = slice_rsrc(row, V, c0, int(sizeof(E)));
#pragma unroll
    for (int u = 0; u < EPT / VN; ++u) {
      float v[VN];
#pragma unroll
      for (int j = 0; j < VN; ++j) v[j] = zero ? 0.0f : q[u * VN + j] * fmaf(sg[u * VN + j], h, g0);
      const uint4 w = EL::pack(v);
      const u32x4_t wv = {w.x, w.y, w.z, w.w};
      // Out-of-range stores are dropped by the buffer range check.
      __builtin_amdgcn_raw_buffer_store_b128(wv, rs, uint32_t((u * TT + tid) * 16), 0u, kBufNonTemporal);
    }
  } else {
#pragma unroll
    for (int u = 0; u < EPT / VN; ++u) {
#pragma unroll
      for (int j = 0; j < VN; ++j) {
        const int e = c0 + (u * TT + tid) * VN + j;
        const float g = zero ? 0.0f : q[u * VN + j] * fmaf(sg[u * VN + j], h, g0);
        if (e < V) EL::store_scalar(row + e, g);
      }
    }
  }
}

// Team exchange without a counter: each member publishes its n partials as
// tagged words (64-bit device-coherent stores, no wait), and every member polls
// the team's words until all carry the current tag. Nothing older than the
// record (gradient stores) has to retire first. Polls are bounded:
// a poll that runs out raises the abort flag, which every poller checks, so every
// wait ends.
__device__ __forceinline__ void publish(unsigned long long* rec, const float* v, int n, unsigned tag) {
  for (int k = 0; k < n; ++k)
    __hip_atomic_store(&rec[k], ((unsigned long long)tag << 32) | __float_as_uint(v[k]), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ bool gather(const unsigned long long* team_rec, int G, int slot, int n, unsigned tag,
                       unsigned* abort_flag, TvLds& sh) {
  const int tid = threadIdx.x;
  if (tid < G * n) {
    const int j = tid / n, k = tid - j * n;
    const unsigned long long* w = &team_rec[j * kRecWords + slot * 4 + k];
    unsigned spins = 0;
    unsigned long long v = 0ull;
    bool ok = true;
    while (true) {
      v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (unsigned(v >> 32) == tag) break;
      if ((++spins & 63u) == 0u) {
        if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) { ok = false; break; }
        if (spins > kSpinLimit) {
          __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = false;
          break;
        }
      }
      __builtin_amdgcn_s_sleep(1);
    }
    sh.rec[j][k] = __uint_as_float(unsigned(v));
    if (!ok) sh.ok = 0;
  }
  __syncthreads();
  return sh.ok != 0;
}

// Response-mask byte of row r, read through the scalar data cache (a wave-uniform
// load counted apart from vector memory). A vector load here would wait for every
// older vector memory operation, the previous row's gradient stores included,
// before the row's own loads could issue. The aligned word holding the byte lies in
// the same page as the byte.
__device__ __forceinline__ bool row_in_mask(const uint8_t* mask, int r) {
  typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
  const uintptr_t p = reinterpret_cast<uintptr_t>(mask) + uintptr_t(r);
  const uint32_t w = *reinterpret_cast<const_u32_ptr>(p & ~uintptr_t(3));
  return ((w >> ((p & 3u) * 8u)) & 0xffu) != 0u;
}

// Sum / maximum over the 16 lanes of each row (lanes 0-15 hold the result).
__device__ __forceinline__ float lanes16_sum(float v) {
  v = lanes8_sum(v);
  return v + dpp_move<kDppMirror>(v);
}
__device__ __forceinline__ float lanes16_max(float v) {
  v = lanes8_max(v);
  return fmaxf(v, dpp_move<kDppMirror>(v));
}

// Completion, after the workgroup's last row: the last workgroup to finish
// reduces the loss over the rows in a fixed order, resets the header and advances
// the call epoch. Every thread of the (1024-thread) workgroup calls it; `last` is a
// shared int of the caller.
__device__ void tv_complete(const TvArgs& a, char* ws, unsigned nresp, int& last) {
  constexpr int NT = 1024, NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  TvHeader* hdr = reinterpret_cast<TvHeader*>(ws);
  double* row_tv = reinterpret_cast<double*>(ws + kRowOff);
  if (tid == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    const unsigned old = __hip_atomic_fetch_add(&hdr->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == gridDim.x - 1 ? 1 : 0;
  }
  __syncthreads();
  if (!last) return;
  double acc = 0.0;
  for (int r = tid; r < a.R; r += NT)
    if (a.mask[r]) acc += __hip_atomic_load(&row_tv[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  acc = wave_sum(acc);
  __shared__ double wsum[NW];
  if (lane == 0) wsum[wid] = acc;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int w = 0; w < NW; ++w) tot += wsum[w];
    const bool aborted = __hip_atomic_load(&hdr->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    *a.loss = aborted ? __builtin_nanf("") : (nresp ? float(tot / double(nresp)) : 0.0f);
    __hip_atomic_store(&hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&hdr->abort, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = int(hdr->epoch + 1u);
  }
  __syncthreads();
  // Tags carry the epoch mod 2^16: when it wraps, clear every record so that no
  // word left from 2^16 calls ago can match a tag of the coming calls.
  if ((unsigned(last) & 0xffffu) == 0u) {
    unsigned long long* recs = reinterpret_cast<unsigned long long*>(ws + kRecOff);
    for (int i = tid; i < kMaxWg * kRecWords; i += NT) recs[i] = 0ull;
  }
  if (tid == 0) __hip_atomic_store(&hdr->epoch, unsigned(last), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename E, bool VEC>
__global__ __launch_bounds__(TT) __attribute__((amdgpu_waves_per_eu(4, 4))) void tv_kernel(TvArgs a, TvPlan pl) {
  __shared__ TvLds sh;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int G = pl.G;
  int team, member;
  if (pl.xcd) {
    const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
    team = x * (pl.nteams >> 3) + i / G;
    member = i % G;
  } else {
    team = blockIdx.x / G;
    member = blockIdx.x % G;
  }
  char* ws = static_cast<char*>(a.ws);
  TvHeader* hdr = reinterpret_cast<TvHeader*>(ws);
  unsigned long long* team_rec =
      reinterpret_cast<unsigned long long*>(ws + kRecOff + size_t(team) * G * kRecWords * 8);
  unsigned long long* my_rec = team_rec + member * kRecWords;
  const unsigned epoch_tag =
      (__hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xffffu) << 16;
  if (tid == 0) sh.ok = 1;
  double* row_tv = reinterpret_cast<double*>(ws + kRowOff);

  const int V = a.V;
  const int c0 = member * CHUNK;
  const float c = float(double(kLog2e) / double(a.temperature));
  const unsigned nresp = hdr->nresp;
  const float inv_tn = nresp ? float(1.0 / (double(a.temperature) * double(nresp))) : 0.0f;
  const E* tbase = static_cast<const E*>(a.teacher);
  const E* sbase = static_cast<const E*>(a.student);
  E* gbase = static_cast<E*>(a.grad);
  unsigned nbar = 0;
  bool ok = true;

  for (int r = team; ok && r < a.R; r += pl.nteams) {
    E* grow = gbase ? gbase + size_t(r) * V : nullptr;
    if (!row_in_mask(a.mask, r)) {
      if (grow) {
        float z[EPT];
#pragma unroll
        for (int j = 0; j < EPT; ++j) z[j] = 0.0f;
        store_grad<E, VEC>(grow, V, c0, z, z, 0.0f, 0.0f, true);
      }
      if (member == 0 && tid == 0 && a.tv_rows) a.tv_rows[r] = 0.0f;
      continue;
    }
    float et[EPT], es[EPT];
    load_slices<E, VEC>(tbase + size_t(r) * V, sbase + size_t(r) * V, V, c0, et, es);
    if (c0 + CHUNK > V) {                       // last slice of the row: mask the tail
      constexpr int VN = TvElem<E>::VN;
      const int lim = V - c0 - tid * VN;        // element j is in the row iff (j/VN)*TT*VN + j%VN < lim
      if constexpr (VEC) {
        // V is a multiple of VN here: each 16-byte vector is wholly in or out.
#pragma unroll
        for (int u = 0; u < EPT / VN; ++u) {
          if (u * TT * VN >= lim) {
#pragma unroll
            for (int j = 0; j < VN; ++j) { et[u * VN + j] = -INFINITY; es[u * VN + j] = -INFINITY; }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          if ((j / VN) * TT * VN + (j % VN) >= lim) { et[j] = -INFINITY; es[j] = -INFINITY; }
        }
      }
    }
    // ---- pass 1: thread max, exps relative to it, thread sums ----
    float mt = -INFINITY, ms = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPT; ++j) { mt = fmaxf(mt, et[j]); ms = fmaxf(ms, es[j]); }
    if (mt == -INFINITY) mt = 0.0f;             // thread holds no element of the row
    if (ms == -INFINITY) ms = 0.0f;
    const float bt = -mt * c, bs = -ms * c;
    float zt = 0.0f, zs = 0.0f;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      et[j] = __builtin_amdgcn_exp2f(fmaf(et[j], c, bt));
      es[j] = __builtin_amdgcn_exp2f(fmaf(es[j], c, bs));
      zt += et[j];
      zs += es[j];
    }
    // Wave partials (DPP reductions), then the workgroup partial over the sixteen
    // waves in lanes 0-15 of wave 0, then the team.
    {
      const float wmt = wave_max_dpp(zt > 0.0f ? mt : -INFINITY);
      const float wms = wave_max_dpp(zs > 0.0f ? ms : -INFINITY);
      const float st = zt > 0.0f ? zt * __builtin_amdgcn_exp2f((mt - wmt) * c) : 0.0f;
      const float ss = zs > 0.0f ? zs * __builtin_amdgcn_exp2f((ms - wms) * c) : 0.0f;
      const float wzt = wave_sum_dpp(st), wzs = wave_sum_dpp(ss);
      if (lane == 0) { sh.wred[wid][0] = wmt; sh.wred[wid][1] = wzt; sh.wred[wid][2] = wms; sh.wred[wid][3] = wzs; }
      __syncthreads();
      if (wid == 0) {
        const bool in = lane < TWAVES;
        const float m0 = in ? sh.wred[lane][0] : -INFINITY, z0 = in ? sh.wred[lane][1] : 0.0f;
        const float m1 = in ? sh.wred[lane][2] : -INFINITY, z1 = in ? sh.wred[lane][3] : 0.0f;
        const float Mt = lanes16_max(z0 > 0.0f ? m0 : -INFINITY);
        const float Ms = lanes16_max(z1 > 0.0f ? m1 : -INFINITY);
        const float Zt = lanes16_sum(z0 > 0.0f ? z0 * __builtin_amdgcn_exp2f((m0 - Mt) * c) : 0.0f);
        const float Zs = lanes16_sum(z1 > 0.0f ? z1 * __builtin_amdgcn_exp2f((m1 - Ms) * c) : 0.0f);
        if (lane == 0) {
          const float v[4] = {Mt, Zt, Ms, Zs};
          publish(my_rec, v, 4, epoch_tag | ((nbar + 1) & 0xffffu));
        }
      }
    }
    ++nbar;
    if (!gather(team_rec, G, 0, 4, epoch_tag | (nbar & 0xffffu), &hdr->abort, sh)) { ok = false; break; }
    // Team normalisers, computed by every wave from the gathered records (member
    // j in lane j; G <= 64): maxima, then the sums of the rescaled partials.
    float Mt, Ms, lzt, lzs;
    {
      const bool in = lane < G;
      const float m0 = in ? sh.rec[lane][0] : -INFINITY, z0 = in ? sh.rec[lane][1] : 0.0f;
      const float m1 = in ? sh.rec[lane][2] : -INFINITY, z1 = in ? sh.rec[lane][3] : 0.0f;
      Mt = wave_max_dpp(z0 > 0.0f ? m0 : -INFINITY);
      Ms = wave_max_dpp(z1 > 0.0f ? m1 : -INFINITY);
      const float Zt = wave_sum_dpp(z0 > 0.0f ? z0 * __builtin_amdgcn_exp2f((m0 - Mt) * c) : 0.0f);
      const float Zs = wave_sum_dpp(z1 > 0.0f ? z1 * __builtin_amdgcn_exp2f((m1 - Ms) * c) : 0.0f);
      lzt = __builtin_amdgcn_logf(Zt);
      lzs = __builtin_amdgcn_logf(Zs);
    }
    // p = et * at, q = es * as: exp2 of the thread-max offset minus log2 Z.
    const float at = __builtin_amdgcn_exp2f((mt - Mt) * c - lzt);
    const float as = __builtin_amdgcn_exp2f((ms - Ms) * c - lzs);
    // ---- pass 2: |q - p| and q sign(q - p); keep (sign, q) ----
    float tvs = 0.0f, gs = 0.0f;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      // Rounded products, not contracted into the subtraction, so that equal
      // rows give d == 0 exactly.
#pragma clang fp contract(off)
      const float p = et[j] * at, q = es[j] * as;
      const float d = q - p;
      // sign(d): +-1 for |d| >= 2^-126, 0 for d == 0
      const float s = __builtin_amdgcn_fmed3f(d * 0x1p126f, -1.0f, 1.0f);
      tvs = fmaf(d, s, tvs);
      gs = fmaf(q, s, gs);
      et[j] = s;
      es[j] = q;
    }
    __syncthreads();                           // sh.rec / sh.wred reuse
    {
      const float wt = wave_sum_dpp(tvs), wg = wave_sum_dpp(gs);
      if (lane == 0) { sh.wred[wid][0] = wt; sh.wred[wid][1] = wg; }
      __syncthreads();
      if (wid == 0) {
        const bool in = lane < TWAVES;
        const float T = lanes16_sum(in ? sh.wred[lane][0] : 0.0f);
        const float Gs = lanes16_sum(in ? sh.wred[lane][1] : 0.0f);
        if (lane == 0) {
          const float v[2] = {T, Gs};
          publish(my_rec + 4, v, 2, epoch_tag | ((nbar + 1) & 0xffffu));
        }
      }
    }
    ++nbar;
    if (!gather(team_rec, G, 1, 2, epoch_tag | (nbar & 0xffffu), &hdr->abort, sh)) { ok = false; break; }
    double tv = 0.0, gsum = 0.0;
    for (int j = 0; j < G; ++j) { tv += double(sh.rec[j][0]); gsum += double(sh.rec[j][1]); }
    tv *= 0.5;
    gsum *= 0.5;
    if (member == 0 && tid == 0) {
      if (a.tv_rows) a.tv_rows[r] = float(tv);
      __hip_atomic_store(&row_tv[r], tv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // ---- pass 3: gradient ----
    if (grow) {
      const float h = 0.5f * inv_tn, g0 = float(-gsum * double(inv_tn));
      store_grad<E, VEC>(grow, V, c0, et, es, h, g0, false);
    }
    __syncthreads();                           // sh.rec reuse by the next row
  }

  tv_complete(a, ws, nresp, sh.last);
}

// ---------------------------------------------------------------------------
// Pipelined form for bf16 rows with 16-byte alignment (the training workload).
//
// The form above runs each row as load -> pass 1 -> exchange -> pass 2 ->
// exchange -> pass 3, so HBM idles while the CU computes and exchanges, and
// the VALU idles while the row loads. Here the two overlap:
// * Fifteen data waves hold 32 logits of each row per thread (30720 per
//   workgroup). The next response row streams into LDS by DMA (buffer loads that
//   write LDS, 120 KB) while the current row is computed from registers.
// * Wave 15 runs the team exchanges: it combines the data waves' partials,
//   publishes them, and polls the team. It issues no loads of row data, so a
//   poll never waits behind the stream.
// * Pass 1 of the next row runs while the current row's second exchange is in
//   flight, and pass 3 of the current row while the next row's first exchange is.
//   Pass 2 keeps copysign(q, q - p) per element as bf16, two to a register, and a
//   bit mask of the elements with q == p != 0 (sign 0).
// * Barriers here do not fence memory (s_barrier after the LDS counter drains):
//   a workgroup-scope fence would also wait for the DMA in flight.
// * Records: 2 sets per exchange kind, by row parity, so a member can publish
//   the next row's partials before a slower member has read this row's.
constexpr int PT = 1024;
constexpr int PW = PT / kWave;          // 16 waves
constexpr int PDW = PW - 1;             // data waves; wave PDW runs the exchanges
constexpr int PDT = PDW * kWave;        // 960 data threads
constexpr int PVEC = 4;                 // 16-byte vectors of each row per data thread
constexpr int PEPT = PVEC * 8;          // 32 logits of each row per data thread
constexpr int PCHUNK = PDT * PEPT;      // 30720 logits of each row per workgroup

struct PipeLds {
  float wred1[PDW][4];    // pass-1 partials of the data waves
  float wred2[PDW][2];    // pass-2 partials
  float norm[4];          // team max and log2 normaliser of both rows
  float g0;               // gradient offset of the current row
  // Set to 0 by the control wave when an exchange failed, each read only in the
  // barrier interval after the one it is written before: ok_x2 is written before
  // the barrier that publishes g0, ok_x1 before the one that publishes norm.
  int ok_x1;
  int ok_x2;
  int last;
};

__device__ __forceinline__ void pbar() {
  asm volatile("" ::: "memory");
  wait_lgkmcnt0();                         // this wave's LDS writes are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// First response row at or after r in the team's sequence r, r + nt, ... (R if none).
__device__ __forceinline__ int next_resp(const uint8_t* mask, int r, int nt, int R) {
  while (r < R && !row_in_mask(mask, r)) r += nt;
  return r;
}

// Control wave: lane j < G polls member j's n record words from word w0 on,
// two 64-bit words per 16-byte device-coherent load, until all carry `tag`. The
// values land in v[0..n-1] of lane j. Returns false (wave-uniform) when a poll ran
// out or another workgroup raised the abort flag.
__device__ bool ctl_poll(const unsigned long long* team_rec, int G, int w0, int n, unsigned tag,
                         unsigned* abort_flag, float (&v)[4]) {
  const int lane = threadIdx.x & (kWave - 1);
  bool ok = true;
  if (lane < G) {
    const __amdgpu_buffer_rsrc_t rs = make_row_rsrc(team_rec, uint32_t(G * kRecWords * 8));
    const uint32_t off = uint32_t((lane * kRecWords + w0) * 8);
    unsigned spins = 0;
    while (true) {
      const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0u, kBufDeviceCoherent);
      u32x4_t b = a;
      if (n > 2) b = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0u, kBufDeviceCoherent);
      bool hit = a.y == tag && a.w == tag;
      if (n > 2) hit = hit && b.y == tag && b.w == tag;
      if (hit) {
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.z);
        v[2] = __uint_as_float(b.x); v[3] = __uint_as_float(b.z);
        break;
      }
      if ((++spins & 63u) == 0u) {
        if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) { ok = false; break; }
        if (spins > kSpinLimit) {
          __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = false;
          break;
        }
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return __builtin_amdgcn_ballot_w64(!ok) == 0ull;
}

// Data wave: start the DMA of both slices of row r into this wave's LDS area.
__device__ __forceinline__ void pipe_issue(uint4 (*pf)[kWave], const uint16_t* trow, const uint16_t* srow, int V,
                                           int c0, int d) {
  const __amdgpu_buffer_rsrc_t rt = slice_rsrc(trow, V, c0, 2), rs = slice_rsrc(srow, V, c0, 2);
  // This wave's reads of the previous row out of the area must be done first.
  wait_lgkmcnt0();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int u = 0; u < PVEC; ++u) {
    const uint32_t off = uint32_t((u * PDT + d) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, (lds_ptr_t)&pf[u][0], 16, off, 0, 0, kBufNonTemporal);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)&pf[PVEC + u][0], 16, off, 0, 0, kBufNonTemporal);
  }
}

// Data wave: pass 1 of a row whose slices are in this wave's LDS area. The area
// is copied to registers first (the read waits for this wave's DMA), and the DMA
// of the row after (trow2, srow2; none if null) starts at once, so that it has the
// whole of the next row's work to land in. Then thread maxima, the exps relative
// to them, and the wave's (max, sum) pairs into wred1. Vectors past the row end
// count as -inf.
__device__ __forceinline__ void pipe_pass1(uint4 (*pf)[kWave], int V, int c0, int d, float c, float (&et)[PEPT],
                                           float (&es)[PEPT], float& mt, float& ms, PipeLds& sh,
                                           const uint16_t* trow2, const uint16_t* srow2) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  // The compiler does not order these reads after the DMA issued in the previous
  // row (across the loop), so the wait is explicit. It also waits for the
  // gradient stores issued since, which were issued a pass earlier.
  wait_vmcnt<0>();
  asm volatile("" ::: "memory");
  uint4 raw[2 * PVEC];
#pragma unroll
  for (int u = 0; u < 2 * PVEC; ++u) raw[u] = pf[u][lane];
  if (trow2) pipe_issue(pf, trow2, srow2, V, c0, d);   // waits for the reads above first
  const int lim = V - c0 - d * 8;               // vector u is in the row iff u * PDT * 8 < lim
  mt = -INFINITY;
  ms = -INFINITY;
#pragma unroll
  for (int u = 0; u < PVEC; ++u) {
    if (u * PDT * 8 < lim) {
      float x[8], y[8];
      TvElem<uint16_t>::unpack(raw[u], x);
      TvElem<uint16_t>::unpack(raw[PVEC + u], y);
#pragma unroll
      for (int j = 0; j < 8; ++j) { mt = fmaxf(mt, x[j]); ms = fmaxf(ms, y[j]); }
    }
  }
  if (mt == -INFINITY) mt = 0.0f;               // thread holds no element of the row
  if (ms == -INFINITY) ms = 0.0f;
  const float bt = -mt * c, bs = -ms * c;
  float zt = 0.0f, zs = 0.0f;
#pragma unroll
  for (int u = 0; u < 2 * PVEC; ++u) {
    const int v = u >> 1;
    const bool in = v * PDT * 8 < lim, stu = u & 1;
    float x[8];
    TvElem<uint16_t>::unpack(raw[stu ? PVEC + v : v], x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = in ? __builtin_amdgcn_exp2f(fmaf(x[j], c, stu ? bs : bt)) : 0.0f;
      if (stu) { es[v * 8 + j] = e; zs += e; } else { et[v * 8 + j] = e; zt += e; }
    }
  }
  const float wmt = wave_max_dpp(zt > 0.0f ? mt : -INFINITY);
  const float wms = wave_max_dpp(zs > 0.0f ? ms : -INFINITY);
  const float st = zt > 0.0f ? zt * __builtin_amdgcn_exp2f((mt - wmt) * c) : 0.0f;
  const float ss = zs > 0.0f ? zs * __builtin_amdgcn_exp2f((ms - wms) * c) : 0.0f;
  const float wzt = wave_sum_dpp(st), wzs = wave_sum_dpp(ss);
  if (lane == 0) { sh.wred1[wid][0] = wmt; sh.wred1[wid][1] = wzt; sh.wred1[wid][2] = wms; sh.wred1[wid][3] = wzs; }
}

// Control wave: the workgroup's pass-1 partial from the data waves' pairs,
// published as X1 of response row i (record words 4 (i & 1) ...).
__device__ __forceinline__ void ctl_publish1(const PipeLds& sh, float c, unsigned long long* my_rec, unsigned tag,
                                             int i) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool in = lane < PDW;
  const float m0 = in ? sh.wred1[lane][0] : -INFINITY, z0 = in ? sh.wred1[lane][1] : 0.0f;
  const float m1 = in ? sh.wred1[lane][2] : -INFINITY, z1 = in ? sh.wred1[lane][3] : 0.0f;
  const float Mt = lanes16_max(z0 > 0.0f ? m0 : -INFINITY);
  const float Ms = lanes16_max(z1 > 0.0f ? m1 : -INFINITY);
  const float Zt = lanes16_sum(z0 > 0.0f ? z0 * __builtin_amdgcn_exp2f((m0 - Mt) * c) : 0.0f);
  const float Zs = lanes16_sum(z1 > 0.0f ? z1 * __builtin_amdgcn_exp2f((m1 - Ms) * c) : 0.0f);
  if (lane == 0) {
    const float v[4] = {Mt, Zt, Ms, Zs};
    publish(my_rec + 4 * (i & 1), v, 4, tag);
  }
}

// Control wave: X2 of response row i (record words 8 + 2 (i & 1), + 1).
__device__ __forceinline__ void ctl_publish2(const PipeLds& sh, unsigned long long* my_rec, unsigned tag, int i) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool in = lane < PDW;
  const float T = lanes16_sum(in ? sh.wred2[lane][0] : 0.0f);
  const float Gs = lanes16_sum(in ? sh.wred2[lane][1] : 0.0f);
  if (lane == 0) {
    const float v[2] = {T, Gs};
    publish(my_rec + 8 + 2 * (i & 1), v, 2, tag);
  }
}

__global__ __launch_bounds__(PT) __attribute__((amdgpu_waves_per_eu(4, 4))) void tv_pipe_kernel(TvArgs a,
                                                                                                 TvPlan pl) {
  __shared__ uint4 pf_all[PDW][2 * PVEC][kWave];   // row DMA areas, one per data wave
  __shared__ PipeLds sh;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const bool ctl = wid == PDW;
  int d = tid;                                     // data thread index (data waves)
  const int G = pl.G;
  int team, member;
  if (pl.xcd) {
    const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
    team = x * (pl.nteams >> 3) + i / G;
    member = i % G;
  } else {
    team = blockIdx.x / G;
    member = blockIdx.x % G;
  }
  char* ws = static_cast<char*>(a.ws);
  TvHeader* hdr = reinterpret_cast<TvHeader*>(ws);
  unsigned long long* team_rec =
      reinterpret_cast<unsigned long long*>(ws + kRecOff + size_t(team) * G * kRecWords * 8);
  unsigned long long* my_rec = team_rec + member * kRecWords;
  const unsigned epoch_tag =
      (__hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xffffu) << 16;
  double* row_tv = reinterpret_cast<double*>(ws + kRowOff);
  uint4 (*pf)[kWave] = pf_all[ctl ? 0 : wid];
  if (tid == 0) { sh.ok_x1 = 1; sh.ok_x2 = 1; }

  const int V = a.V, R = a.R, nt = pl.nteams;
  const int c0 = member * PCHUNK;
  const float c = float(double(kLog2e) / double(a.temperature));
  const unsigned nresp = hdr->nresp;
  const float inv_tn = nresp ? float(1.0 / (double(a.temperature) * double(nresp))) : 0.0f;
  const float h = 0.5f * inv_tn;
  const uint16_t* tbase = static_cast<const uint16_t*>(a.teacher);
  const uint16_t* sbase = static_cast<const uint16_t*>(a.student);
  uint16_t* gbase = static_cast<uint16_t*>(a.grad);

  // Rows [r0, r1) of the team's sequence are outside the response mask: zero
  // gradient slices (data waves) and zero TV (member 0).
  auto zero_rows = [&](int r0, int r1) {
    for (int r = r0; r < r1; r += nt) {
      if (gbase && !ctl) {
        const __amdgpu_buffer_rsrc_t rs = slice_rsrc(gbase + size_t(r) * V, V, c0, 2);
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < PVEC; ++u)
          __builtin_amdgcn_raw_buffer_store_b128(z, rs, uint32_t((u * PDT + d) * 16), 0u, kBufNonTemporal);
      }
      if (member == 0 && tid == 0 && a.tv_rows) a.tv_rows[r] = 0.0f;
    }
  };

  // The data waves and the control wave run separate loops (so that the data
  // waves' 96 registers of row state are not live across the control code) with
  // the same sequence of barriers: per response row cur (next response row nxt),
  //   B2  norm(cur) ready     -> data: pass 2 of cur          ctl: -
  //   B3  pass-2 partials     -> data: pass 1 of nxt, DMA     ctl: publish X2(cur)
  //   B4  pass-1 partials     -> data: -                      ctl: publish X1(nxt), poll X2(cur)
  //   B5  g0(cur) ready       -> data: pass 3 of cur          ctl: poll X1(nxt)
  // Both sides walk the same row sequence and leave at the same barrier.
  int cur = next_resp(a.mask, team, nt, R);
  int nxt = cur < R ? next_resp(a.mask, cur + nt, nt, R) : R;
  if (ctl) {
    // Team normalisers of response row i from its polled X1 records (member j in
    // lane j; G <= 64), into sh.norm.
    auto norm_x1 = [&](int i) {
      float v[4];
      const bool ok = ctl_poll(team_rec, G, 4 * (i & 1), 4, epoch_tag | ((2u * unsigned(i) + 1u) & 0xffffu),
                               &hdr->abort, v);
      const bool in = lane < G;
      const float m0 = in ? v[0] : -INFINITY, z0 = in ? v[1] : 0.0f;
      const float m1 = in ? v[2] : -INFINITY, z1 = in ? v[3] : 0.0f;
      const float Mt = wave_max_dpp(z0 > 0.0f ? m0 : -INFINITY);
      const float Ms = wave_max_dpp(z1 > 0.0f ? m1 : -INFINITY);
      const float Zt = wave_sum_dpp(z0 > 0.0f ? z0 * __builtin_amdgcn_exp2f((m0 - Mt) * c) : 0.0f);
      const float Zs = wave_sum_dpp(z1 > 0.0f ? z1 * __builtin_amdgcn_exp2f((m1 - Ms) * c) : 0.0f);
      if (lane == 0) {
        sh.norm[0] = Mt; sh.norm[1] = Ms;
        sh.norm[2] = __builtin_amdgcn_logf(Zt); sh.norm[3] = __builtin_amdgcn_logf(Zs);
        if (!ok) sh.ok_x1 = 0;
      }
    };
    if (cur < R) {
      pbar();                                      // pass-1 partials of the first row
      ctl_publish1(sh, c, my_rec, epoch_tag | 1u, 0);
      norm_x1(0);
    }
    for (int i = 0; cur < R; ++i) {
      pbar();                                      // B2
      if (!sh.ok_x1) break;
      const int nxt2 = nxt < R ? next_resp(a.mask, nxt + nt, nt, R) : R;
      pbar();                                      // B3
      ctl_publish2(sh, my_rec, epoch_tag | ((2u * unsigned(i) + 2u) & 0xffffu), i);
      pbar();                                      // B4
      if (nxt < R) ctl_publish1(sh, c, my_rec, epoch_tag | ((2u * unsigned(i) + 3u) & 0xffffu), i + 1);
      {
        float v[4];
        const bool ok = ctl_poll(team_rec, G, 8 + 2 * (i & 1), 2, epoch_tag | ((2u * unsigned(i) + 2u) & 0xffffu),
                                 &hdr->abort, v);
        // TV and the sign sum of row cur: member partials summed in member order.
        double tv = 0.0, gsum = 0.0;
        for (int j = 0; j < G; ++j) { tv += double(readlane_f(v[0], j)); gsum += double(readlane_f(v[1], j)); }
        tv *= 0.5;
        gsum *= 0.5;
        if (lane == 0) {
          sh.g0 = float(-gsum * double(inv_tn));
          if (!ok) sh.ok_x2 = 0;
          if (member == 0) {
            if (a.tv_rows) a.tv_rows[cur] = float(tv);
            __hip_atomic_store(&row_tv[cur], tv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      pbar();                                      // B5
      if (!sh.ok_x2) break;
      if (nxt < R) norm_x1(i + 1);
      cur = nxt;
      nxt = nxt2;
    }
  } else {
    float et[PEPT], es[PEPT];
    uint32_t w[PEPT / 2];                          // pass-2 words of row cur, bf16 pairs
    uint32_t zmask = 0u;
    float mt = 0.0f, ms = 0.0f;
    zero_rows(team, cur);
    if (cur < R) {
      pipe_issue(pf, tbase + size_t(cur) * V, sbase + size_t(cur) * V, V, c0, d);
      pipe_pass1(pf, V, c0, d, c, et, es, mt, ms, sh, nxt < R ? tbase + size_t(nxt) * V : nullptr,
                 sbase + size_t(nxt < R ? nxt : 0) * V);
      pbar();                                      // pass-1 partials of the first row
    }
    while (cur < R) {
      pbar();                                      // B2
      if (!sh.ok_x1) break;
      // Addresses are recomputed from d in each row rather than hoisted out of the
      // loop, where they would hold registers through it.
      asm volatile("" : "+v"(d));
      const int nxt2 = nxt < R ? next_resp(a.mask, nxt + nt, nt, R) : R;
      // ---- pass 2 of row cur: |q - p| and q sign(q - p); keep copysign(q, q - p) ----
      // The kept words are rounded to bf16 pairs (to nearest, relative error <=
      // 2^-9, the exponent range of fp32): they only feed the bf16 gradient.
      // Elements with q == p != 0 have sign 0: zmask gets a 1 for them (element j at
      // bit 31 - j), and they stay out of the sign sum.
      zmask = 0u;
      {
        const float at = __builtin_amdgcn_exp2f((mt - sh.norm[0]) * c - sh.norm[2]);
        const float as = __builtin_amdgcn_exp2f((ms - sh.norm[1]) * c - sh.norm[3]);
        float tvs = 0.0f, gs = 0.0f;
#pragma unroll
        for (int j = 0; j < PEPT; j += 2) {
          float wv[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            // Rounded products, not contracted into the subtraction, so that equal
            // rows give d == 0 exactly.
#pragma clang fp contract(off)
            const float p = et[j + k] * at, q = es[j + k] * as;
            const float dd = q - p;
            const bool z = (dd == 0.0f) & (q != 0.0f);
            tvs += fabsf(dd);
            wv[k] = copysignf(q, dd);
            gs += z ? 0.0f : wv[k];
            zmask = (zmask << 1) + (z ? 1u : 0u);
            asm volatile("" : "+v"(zmask));        // shift each bit in now, not 32 masks later
          }
          w[j / 2] = pack_bf16x2(wv[0], wv[1]);
          // Pack here: left to itself the compiler sinks the conversion into pass 3
          // and keeps 32 fp32 words live through pass 1 of the next row.
          asm volatile("" : "+v"(w[j / 2]));
        }
        const float wt = wave_sum_dpp(tvs), wg = wave_sum_dpp(gs);
        if (lane == 0) { sh.wred2[wid][0] = wt; sh.wred2[wid][1] = wg; }
      }
      pbar();                                      // B3
      if (nxt < R) {
        // ---- pass 1 of row nxt (its DMA was issued a row ago); DMA of row nxt2 ----
        pipe_pass1(pf, V, c0, d, c, et, es, mt, ms, sh, nxt2 < R ? tbase + size_t(nxt2) * V : nullptr,
                   sbase + size_t(nxt2 < R ? nxt2 : 0) * V);
      }
      pbar();                                      // B4
      pbar();                                      // B5
      if (!sh.ok_x2) break;
      // ---- pass 3 of row cur: g = q (s h + g0) = w h + |w| g0, w = copysign(q, q - p) ----
      if (gbase) {
        const float g0 = sh.g0;
        const __amdgpu_buffer_rsrc_t rs = slice_rsrc(gbase + size_t(cur) * V, V, c0, 2);
        const bool anyz = __builtin_amdgcn_ballot_w64(zmask != 0u) != 0ull;
#pragma unroll
        for (int u = 0; u < PVEC; ++u) {
          float g[8];
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const uint32_t pk = w[(u * 8 + j) / 2];
            const float x0 = bf16_lo(pk), x1 = bf16_hi(pk);
            g[j] = fmaf(x0, h, fabsf(x0) * g0);
            g[j + 1] = fmaf(x1, h, fabsf(x1) * g0);
            if (anyz) {                            // sign 0: g = q g0
              if ((zmask >> (31 - (u * 8 + j))) & 1u) g[j] = fabsf(x0) * g0;
              if ((zmask >> (30 - (u * 8 + j))) & 1u) g[j + 1] = fabsf(x1) * g0;
            }
          }
          const uint4 pk = TvElem<uint16_t>::pack(g);
          const u32x4_t wv = {pk.x, pk.y, pk.z, pk.w};
          __builtin_amdgcn_raw_buffer_store_b128(wv, rs, uint32_t((u * PDT + d) * 16), 0u, kBufNonTemporal);
        }
      }
      zero_rows(cur + nt, nxt);
      cur = nxt;
      nxt = nxt2;
    }
  }
  // No DMA may still be writing this workgroup's LDS when it ends (an abort can
  // leave one in flight).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  tv_complete(a, ws, nresp, sh.last);
}

// Counts the response rows and sets the loss to 0 (the main kernel overwrites it
// when there is at least one response row).
__global__ __launch_bounds__(1024) void tv_count_kernel(const uint8_t* mask, int R, void* ws, float* loss) {
  unsigned n = 0;
  for (int r = threadIdx.x; r < R; r += 1024) n += mask[r] != 0;
  n = wave_sum(n);
  __shared__ unsigned part[1024 / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = 0;
    for (int w = 0; w < 1024 / kWave; ++w) t += part[w];
    static_cast<TvHeader*>(ws)->nresp = t;
    *loss = 0.0f;
  }
}

template <typename E, bool VEC>
const void* tv_kernel_ptr() {
  return reinterpret_cast<const void*>(&tv_kernel<E, VEC>);
}

// Resident workgroups of one instantiation on the current device (cached).
int resident_wgs(const void* fn, int slot) {
  static std::mutex mu;
  static int cache[64][5];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev][slot] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, TT, 0) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    const int n = per_cu * cus;
    cache[dev][slot] = n < kMaxWg ? n : kMaxWg;
  }
  return cache[dev][slot];
}

template <typename E, bool VEC>
hipError_t launch_tv_t(const TvArgs& a, int slot, hipStream_t stream) {
  const void* fn = tv_kernel_ptr<E, VEC>();
  const int res = resident_wgs(fn, slot);
  const int G = (a.V + CHUNK - 1) / CHUNK;
  if (res <= 0) return hipErrorInvalidDevice;
  if (G > res || G > 64) return hipErrorInvalidConfiguration;
  TvPlan pl;
  pl.G = G;
  int nteams = res / G;
  if (nteams > a.R) nteams = a.R;
  pl.xcd = 0;
  if (nteams >= 8) {
    nteams &= ~7;
    pl.xcd = 1;
  }
  pl.nteams = nteams;
  TvArgs args = a;
  void* params[] = {&args, &pl};
  return hipLaunchCooperativeKernel(fn, dim3(nteams * G), dim3(TT), params, 0, stream);
}

// The pipelined kernel (bf16, aligned rows). Teams of G = ceil(V / 30720) members.
// A team's members share an XCD when that costs no teams (8 XCDs each holding a
// whole number of teams); otherwise they spread over XCDs. The exchanges are off
// the critical path here, so resident CUs count for more: measured at V = 151936
// (G = 5), 51 spread teams took 4.80 ms against 4.90 ms for 48 XCD-local ones.
hipError_t launch_tv_pipe(const TvArgs& a, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&tv_pipe_kernel);
  const int res = resident_wgs(fn, 4);
  const int G = (a.V + PCHUNK - 1) / PCHUNK;
  if (res <= 0) return hipErrorInvalidDevice;
  if (G > res || G > 64) return hipErrorInvalidConfiguration;
  TvPlan pl;
  pl.G = G;
  int nteams = res / G;
  const int nteams_xcd = ((res / 8) / G) * 8;
  pl.xcd = 0;
  if (nteams_xcd >= 8 && nteams_xcd >= nteams && nteams_xcd <= a.R) {
    nteams = nteams_xcd;
    pl.xcd = 1;
  }
  if (nteams > a.R) nteams = a.R;
  pl.nteams = nteams;
  TvArgs args = a;
  void* params[] = {&args, &pl};
  return hipLaunchCooperativeKernel(fn, dim3(nteams * G), dim3(PT), params, 0, stream);
}

template <typename E>
bool tv_rows_aligned(const void* p, int V) {
  return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && ((size_t(V) * sizeof(E)) % 16 == 0);
}

}  // namespace

size_t tv_workspace_bytes(int R) { return kRowOff + size_t(R > 0 ? R : 0) * 8; }

// bf16 rows go to the pipelined kernel when aligned, else to the register form;
// the smaller of the two limits applies to both.
int tv_max_vocab(bool bf16) {
  if (bf16) {
    int res = resident_wgs(reinterpret_cast<const void*>(&tv_pipe_kernel), 4);
    if (res > 64) res = 64;
    int res2 = resident_wgs(tv_kernel_ptr<uint16_t, false>(), 1);
    if (res2 > 64) res2 = 64;
    const long long a = (long long)res * PCHUNK, b = (long long)res2 * CHUNK;
    return int(a < b ? a : b);
  }
  int res = resident_wgs(tv_kernel_ptr<float, true>(), 2);
  if (res > 64) res = 64;
  return res * CHUNK;
}

hipError_t launch_tv(const TvArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(tv_count_kernel, dim3(1), dim3(1024), 0, stream, a.mask, a.R, a.ws, a.loss);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.R == 0) return e;
  if (a.bf16) {
    const bool vec = tv_rows_aligned<uint16_t>(a.teacher, a.V) && tv_rows_aligned<uint16_t>(a.student, a.V) &&
                     (!a.grad || tv_rows_aligned<uint16_t>(a.grad, a.V));
    return vec ? launch_tv_pipe(a, stream) : launch_tv_t<uint16_t, false>(a, 1, stream);
  }
  const bool vec = tv_rows_aligned<float>(a.teacher, a.V) && tv_rows_aligned<float>(a.student, a.V) &&
                   (!a.grad || tv_rows_aligned<float>(a.grad, a.V));
  return vec ? launch_tv_t<float, true>(a, 2, stream) : launch_tv_t<float, false>(a, 3, stream);
}

}  // namespace uno
