// Lossless block verifier and draft sampler for gfx950.
//
// Operation ("LoopUno: Turning Agentic Looped LLMs into Diffusion LLMs in One
// Hour", section "How it works"; sampling settings from the "Uno Qwen3-8B" model
// card, "Evaluation protocol"): per (sequence, slot) filter the base logits p and
// draft logits q (temperature -> tie-inclusive top-k -> tie-grouped top-p ->
// renormalise), take the AR token at slot 0, accept draft d at slot i >= 1 iff
// u_acc < p~(d)/q~(d), draw a rejected slot from normalise(max(0, p~ - q~)), and
// keep the longest accepted prefix of each block.
//
// Design (one workgroup of 256 threads per slot):
//  * The vocabulary row is streamed once from HBM with 16-byte loads, eight in
//    flight per thread, double-buffered in registers.
//  * A lower bound of the k-th largest logit is taken from the first tile: each
//    wave finds the ceil(k/4)-th largest of its 64 lane maxima; the minimum over
//    the 4 waves has at least k row elements at or above it. Every element at
//    or above the bound is pushed to an LDS candidate list (a few hundred per
//    row for k = 50).
//  * The exact k-th largest value is found by an MSB-first radix select over the
//    candidates' order-preserving keys, restricted to the bits where candidates
//    differ; every candidate >= it forms the tie-inclusive top-k set.
//  * Softmax, top-p and the renormalised distribution are computed in fp64 on
//    that set, one entry per thread. The accept test and both inverse CDFs use
//    the same fp64 values.
//  * Slot records go to the workspace; the last workgroup of a sequence to
//    finish (atomic ticket after a device-scope release fence) runs the prefix
//    scan and resets the ticket for the next call.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace uno {
namespace {

constexpr int VT = 256;               // threads per workgroup
constexpr int VW = VT / kWave;        // waves per workgroup
constexpr int UNR = 8;                // 16-byte loads per thread per tile
constexpr int CAND_CAP = kVerifyCandCap;
constexpr int SEL_CAP = 256;          // largest filtered support on this path (== VT)
constexpr int KMAX_FAST = kVerifyKMaxFast;
constexpr double NEAR_TIE = 1e-6;

constexpr int FLAG_TIE_ACCEPT = 1, FLAG_TIE_TOPP_P = 2, FLAG_TIE_TOPP_Q = 4,
              FLAG_TIE_ICDF = 8, FLAG_Q_ZERO = 16, FLAG_RES_ZERO = 32, FLAG_OVERFLOW = 64;

enum { ROW_OK = 0, ROW_OVERFLOW = 1 };

struct Dist {            // filtered distribution: ascending ids, fp64 probabilities
  int n;
  int ids[SEL_CAP];
  double prob[SEL_CAP];
};

struct Shared {
  float cval[CAND_CAP];
  int cidx[CAND_CAP];
  unsigned hist[256];
  float sval[SEL_CAP];
  int sidx[SEL_CAP];
  double sw[SEL_CAP];
  double cum[SEL_CAP];
  unsigned char skeep[SEL_CAP];
  Dist dp, dq;
  double red_d[VW];
  float red_f[VW];
  unsigned red_u[VW];
  int red_i[VW];
  int cnt, scnt, ires, itie;
  unsigned ures[2];
  double dres[2];
};

struct FilterParams {
  double T;
  double top_p;
  int k_eff;        // tie-inclusive top-k size (V when top-k is off)
  bool greedy;
  bool topp_on;
};

// --- block-wide reductions (all 256 threads call; result broadcast) ---------
__device__ __forceinline__ double block_sum_d(double v, Shared& sh) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.red_d[threadIdx.x / kWave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < VW; ++i) t += sh.red_d[i];
  return t;
}
__device__ __forceinline__ float block_min_f(float v, Shared& sh) {
  v = wave_min(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.red_f[threadIdx.x / kWave] = v;
  __syncthreads();
  float t = sh.red_f[0];
#pragma unroll
  for (int i = 1; i < VW; ++i) t = fminf(t, sh.red_f[i]);
  return t;
}
__device__ __forceinline__ unsigned block_max_u(unsigned v, Shared& sh) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.red_u[threadIdx.x / kWave] = v;
  __syncthreads();
  unsigned t = sh.red_u[0];
#pragma unroll
  for (int i = 1; i < VW; ++i) t = max(t, sh.red_u[i]);
  return t;
}
__device__ __forceinline__ unsigned block_min_u(unsigned v, Shared& sh) {
  v = wave_min(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.red_u[threadIdx.x / kWave] = v;
  __syncthreads();
  unsigned t = sh.red_u[0];
#pragma unroll
  for (int i = 1; i < VW; ++i) t = min(t, sh.red_u[i]);
  return t;
}
__device__ __forceinline__ unsigned block_or_u(unsigned v, Shared& sh) {
  v = wave_or(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.red_u[threadIdx.x / kWave] = v;
  __syncthreads();
  unsigned t = 0;
#pragma unroll
  for (int i = 0; i < VW; ++i) t |= sh.red_u[i];
  return t;
}
__device__ __forceinline__ int block_max_i(int v, Shared& sh) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.red_i[threadIdx.x / kWave] = v;
  __syncthreads();
  int t = sh.red_i[0];
#pragma unroll
  for (int i = 1; i < VW; ++i) t = max(t, sh.red_i[i]);
  return t;
}
__device__ __forceinline__ int block_min_i(int v, Shared& sh) {
  v = wave_min(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.red_i[threadIdx.x / kWave] = v;
  __syncthreads();
  int t = sh.red_i[0];
#pragma unroll
  for (int i = 1; i < VW; ++i) t = min(t, sh.red_i[i]);
  return t;
}

// --- element formats ----------------------------------------------------------
template <typename E> struct Elem;
template <> struct Elem<uint16_t> {        // bf16 bit patterns
  static constexpr int VN = 8;
  __device__ static void unpack(const uint4& r, float* x) {
    x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x); x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
    x[4] = bf16_lo(r.z); x[5] = bf16_hi(r.z); x[6] = bf16_lo(r.w); x[7] = bf16_hi(r.w);
  }
  __device__ static uint4 load_partial(const uint16_t* row, int e0, int V) {
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int e = e0 + 2 * h;
      const uint32_t lo = e < V ? uint32_t(row[e]) : 0xFF80u;          // -inf pad
      const uint32_t hi = e + 1 < V ? uint32_t(row[e + 1]) : 0xFF80u;
      w[h] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
  __device__ static float load1(const uint16_t* row, int e) { return bf16_to_f32(row[e]); }
};
template <> struct Elem<float> {
  static constexpr int VN = 4;
  __device__ static void unpack(const uint4& r, float* x) {
    x[0] = __uint_as_float(r.x); x[1] = __uint_as_float(r.y);
    x[2] = __uint_as_float(r.z); x[3] = __uint_as_float(r.w);
  }
  __device__ static uint4 load_partial(const float* row, int e0, int V) {
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) w[h] = (e0 + h < V) ? __float_as_uint(row[e0 + h]) : 0xFF800000u;
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
  __device__ static float load1(const float* row, int e) { return row[e]; }
};

// --- one row: stream, candidates, exact tie-inclusive top-k, fp64 filter -------
template <typename E, bool VEC>
__device__ __forceinline__ int filter_row(const E* __restrict__ row, int V, const FilterParams& fp,
                          Shared& sh, Dist& out, double& topp_gap) {
  using EL = Elem<E>;
  constexpr int VN = EL::VN;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int nfull = V / VN;                       // whole 16-byte chunks
  const int nchunks = (V + VN - 1) / VN;          // incl. a partial last chunk
  constexpr int PER_TILE = VT * UNR;
  const int ntiles = (nchunks + PER_TILE - 1) / PER_TILE;
  topp_gap = INFINITY;

  // Vector path: one range-checked buffer load per chunk (bytes past the row read
  // as zero and are masked to -inf by index in the last tile). Scalar path for
  // rows that are not 16-byte aligned.
  const int full_tiles = VEC ? nfull / PER_TILE : 0;
  const __amdgpu_buffer_rsrc_t rsrc = make_row_rsrc(row, uint32_t(V) * uint32_t(sizeof(E)));
  auto load_tile = [&](uint4 (&r)[UNR], int t) {
    if (VEC) {
      const uint32_t voff = uint32_t(tid) * 16u;
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        r[u] = buffer_load16(rsrc, voff, uint32_t(t * PER_TILE + u * VT) * 16u);
    } else {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = t * PER_TILE + u * VT + tid;
        if (c < nchunks) {
          r[u] = EL::load_partial(row, c * VN, V);
        } else {
          r[u] = VN == 8 ? make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u)
                         : make_uint4(0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u);
        }
      }
    }
  };
  auto process_tile = [&](const uint4 (&r)[UNR], int t, float thr) {
    const bool tail = t >= full_tiles;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float x[VN];
      EL::unpack(r[u], x);
      const int e0 = (t * PER_TILE + u * VT + tid) * VN;
      if (tail) {
#pragma unroll
        for (int j = 0; j < VN; ++j) x[j] = (e0 + j < V) ? x[j] : -INFINITY;
      }
      float mx = x[0];
#pragma unroll
      for (int j = 1; j < VN; ++j) mx = fmaxf(mx, x[j]);
      if (mx >= thr) {
#pragma unroll
        for (int j = 0; j < VN; ++j) {
          if (x[j] >= thr && e0 + j < V) {
            const int p = atomicAdd(&sh.cnt, 1);
            if (p < CAND_CAP) { sh.cval[p] = x[j]; sh.cidx[p] = e0 + j; }
          }
        }
      }
    }
  };

  if (tid == 0) sh.cnt = 0;
  uint4 A[UNR], B[UNR];
  // Both buffers are always loaded (tiles past the row read as zero on the vector
  // path), so the number of loads in flight is the same on every path and each
  // wait covers exactly the tile about to be processed.
  load_tile(A, 0);
  if (VEC || ntiles > 1) load_tile(B, 1);

  // Lower bound of the k-th largest value from the first tile's lane maxima.
  float thr = -INFINITY;
  if (fp.k_eff <= KMAX_FAST) {
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float x[VN];
      EL::unpack(A[u], x);
      const int e0 = (u * VT + tid) * VN;
#pragma unroll
      for (int j = 0; j < VN; ++j) m = (e0 + j < V) ? fmaxf(m, x[j]) : m;
    }
    const int c = (fp.k_eff + VW - 1) / VW;     // <= 64
    int cnt_ge = 0;
#pragma unroll
    for (int j = 0; j < kWave; ++j) {
      const float mj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), j));
      cnt_ge += (mj >= m) ? 1 : 0;
    }
    const float tw = wave_max(cnt_ge >= c ? m : -INFINITY);
    if (lane == 0) sh.red_f[wid] = tw;
    __syncthreads();
    thr = sh.red_f[0];
#pragma unroll
    for (int i = 1; i < VW; ++i) thr = fminf(thr, sh.red_f[i]);
  } else {
    __syncthreads();
  }

  if (VEC) {
    for (int t = 0; t < ntiles; t += 2) {
      process_tile(A, t, thr);
      load_tile(A, t + 2);
      if (t + 1 < ntiles) process_tile(B, t + 1, thr);
      load_tile(B, t + 3);
    }
  } else {
    process_tile(A, 0, thr);
    for (int t = 1; t < ntiles; t += 2) {
      if (t + 1 < ntiles) load_tile(A, t + 1);
      process_tile(B, t, thr);
      if (t + 1 < ntiles) {
        if (t + 2 < ntiles) load_tile(B, t + 2);
        process_tile(A, t + 1, thr);
      }
    }
  }
  __syncthreads();
  const int C = sh.cnt;
  __syncthreads();                 // every thread has read the count before any reuse
  if (C > CAND_CAP) return ROW_OVERFLOW;

  // Key range of the candidates.
  unsigned kmax = 0u, kmin = 0xffffffffu;
  for (int i = tid; i < C; i += VT) {
    const unsigned k = float_key(sh.cval[i]);
    kmax = max(kmax, k);
    kmin = min(kmin, k);
  }
  kmax = block_max_u(kmax, sh);
  kmin = block_min_u(kmin, sh);
  unsigned diff = 0u;
  for (int i = tid; i < C; i += VT) diff |= float_key(sh.cval[i]) ^ kmax;
  diff = block_or_u(diff, sh);

  // k_eff-th largest key by MSB-first radix select over the differing bits.
  unsigned kstar = kmax;
  if (diff != 0u && fp.k_eff < C) {
    const int hb = 31 - __clz(diff);
    const int lb = __ffs(diff) - 1;
    unsigned pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);
    unsigned prefix = kmax & pmask;
    unsigned remaining = unsigned(fp.k_eff);
    int hi = hb;
    while (true) {
      const int lo = max(hi - 7, lb);
      const int width = hi - lo + 1;
      const unsigned dmask = (1u << width) - 1u;
      for (int i = tid; i < 256; i += VT) sh.hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < C; i += VT) {
        const unsigned k = float_key(sh.cval[i]);
        if ((k & pmask) == prefix) atomicAdd(&sh.hist[(k >> lo) & dmask], 1u);
      }
      __syncthreads();
      if (wid == 0) {
        // lane l owns digits 255-4l .. 252-4l (highest digits first)
        unsigned h[4];
        unsigned s = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { h[q] = sh.hist[255 - 4 * lane - q]; s += h[q]; }
        const unsigned incl = wave_inclusive_scan(s);
        unsigned acc = incl - s;
        if (acc < remaining && remaining <= incl) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (acc + h[q] >= remaining) {
              sh.ures[0] = unsigned(255 - 4 * lane - q);
              sh.ures[1] = acc;
              break;
            }
            acc += h[q];
          }
        }
      }
      __syncthreads();
      const unsigned d = sh.ures[0];
      remaining -= sh.ures[1];
      prefix |= d << lo;
      pmask |= dmask << lo;
      if (lo == lb) break;
      hi = lo - 1;
    }
    const unsigned lowmask = lb == 0 ? 0u : ((1u << lb) - 1u);
    kstar = prefix | (kmax & lowmask);
  } else if (diff != 0u) {
    kstar = kmin;                  // every candidate is in the top-k set
  }

  // Tie-inclusive top-k set.
  if (tid == 0) sh.scnt = 0;
  __syncthreads();
  for (int i = tid; i < C; i += VT) {
    if (float_key(sh.cval[i]) >= kstar) {
      const int p = atomicAdd(&sh.scnt, 1);
      if (p < SEL_CAP) { sh.sval[p] = sh.cval[i]; sh.sidx[p] = sh.cidx[i]; }
    }
  }
  __syncthreads();
  const int n = sh.scnt;
  __syncthreads();
  if (n > SEL_CAP) return ROW_OVERFLOW;
  const float zmax = key_float(kmax);

  if (fp.greedy) {
    // One-hot at the argmax, lowest id on ties (the set holds exactly the ties).
    const int id = block_min_i(tid < n ? sh.sidx[tid] : 0x7fffffff, sh);
    if (tid == 0) { out.n = 1; out.ids[0] = id; out.prob[0] = 1.0; }
    __syncthreads();
    return ROW_OK;
  }

  const int j = tid;
  const bool valid = j < n;
  const float zj = valid ? sh.sval[j] : -INFINITY;
  const int idj = valid ? sh.sidx[j] : 0x7fffffff;
  double w = 0.0;
  if (valid) {
    w = exp((double(zj) - double(zmax)) / fp.T);
    sh.sw[j] = w;
  }
  __syncthreads();
  bool keep = valid;
  if (fp.topp_on) {
    const double ztop = block_sum_d(w, sh);
    double above = 0.0;
    if (valid) {
      for (int i = 0; i < n; ++i) above += (sh.sval[i] > zj) ? sh.sw[i] : 0.0;
    }
    const double mass = above / ztop;
    float gapf = INFINITY;
    if (valid) {
      keep = (zj == zmax) || (mass < fp.top_p);
      // the top group is kept unconditionally, so only lower groups decide
      if (zj != zmax) gapf = float(fabs(mass - fp.top_p));
    }
    topp_gap = double(block_min_f(gapf, sh));
  }
  const double wsum = block_sum_d(keep ? w : 0.0, sh);
  if (valid) sh.skeep[j] = keep ? 1 : 0;
  __syncthreads();
  if (keep) {
    int pos = 0;
    for (int i = 0; i < n; ++i) pos += (sh.skeep[i] && sh.sidx[i] < idj) ? 1 : 0;
    out.ids[pos] = idj;
    out.prob[pos] = w / wsum;
  }
  int nk = 0;
  {
    const unsigned long long bal = __ballot(keep);
    nk = __popcll(bal);
    __syncthreads();
    if (lane == 0) sh.red_i[wid] = nk;
    __syncthreads();
    nk = 0;
#pragma unroll
    for (int i = 0; i < VW; ++i) nk += sh.red_i[i];
  }
  if (tid == 0) out.n = nk;
  __syncthreads();
  return ROW_OK;
}

// Inverse CDF over n <= 256 weights (thread j holds w_j, ids ascending): the first
// j with u*Z < C_j, where C is the inclusive prefix sum and Z = C_{n-1}; falls
// back to the last positive weight. Sets *tie when u*Z lies within 1e-6*Z of a
// decision boundary.
__device__ __forceinline__ int block_icdf(double w, int n, double u, Shared& sh, bool* tie) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const double v = tid < n ? w : 0.0;
  const double inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane == kWave - 1) sh.red_d[wid] = inc;
  __syncthreads();
  double off = 0.0;
  for (int i = 0; i < wid; ++i) off += sh.red_d[i];
  const double c = off + inc;
  if (tid < n) sh.cum[tid] = c;
  if (tid == 0) { sh.ires = -1; sh.itie = 0; }
  __syncthreads();
  const double Z = sh.cum[n - 1];
  const double t = u * Z;
  if (tid < n) {
    const double cprev = tid > 0 ? sh.cum[tid - 1] : 0.0;
    if (c > t && (tid == 0 || cprev <= t)) {
      double gap = INFINITY;
      if (tid < n - 1) gap = fmin(gap, fabs(t - c));
      if (tid > 0) gap = fmin(gap, fabs(t - cprev));
      sh.ires = tid;
      sh.itie = gap < NEAR_TIE * Z ? 1 : 0;
    }
  }
  const int lastpos = block_max_i((tid < n && w > 0.0) ? tid : -1, sh);
  int jj = sh.ires;
  *tie = sh.itie != 0;
  if (jj < 0) jj = lastpos;
  __syncthreads();
  return jj;
}

__device__ __forceinline__ double lookup_prob(const Dist& d, int tok) {
  int lo = 0, hi = d.n;                 // binary search over ascending ids
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (d.ids[mid] < tok) lo = mid + 1; else hi = mid;
  }
  return (lo < d.n && d.ids[lo] == tok) ? d.prob[lo] : 0.0;
}

__device__ __forceinline__ FilterParams make_filter_params(const SamplingArgs& sp, int V) {
  FilterParams fp;
  fp.T = sp.temperature;
  fp.greedy = !(sp.temperature > 0.0);
  fp.top_p = sp.top_p;
  fp.topp_on = !fp.greedy && sp.top_p < 1.0;
  fp.k_eff = fp.greedy ? 1 : ((sp.top_k > 0 && sp.top_k < V) ? sp.top_k : V);
  return fp;
}

// --- kernels -------------------------------------------------------------------
template <typename E, bool VEC>
__global__ __launch_bounds__(VT) void verify_kernel(VerifyArgs a) {
  __shared__ Shared sh;
  const int g = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int b = a.b, V = a.V;
  const int s = g / b, i = g - s * b;
  const int tid = threadIdx.x;
  const FilterParams fp = make_filter_params(a.sp, V);
  const Philox4 ph = philox4x64_10(uint64_t(a.pos[s] + i), 0ull, 0ull, 0ull, a.sp.seed,
                                   uint64_t(a.seq_ids[s]));
  const double u_acc = word_to_uniform(ph.w[0]);
  const double u_res = word_to_uniform(ph.w[1]);
  const size_t off = size_t(g) * size_t(V);

  int flags = 0, tok = -1, acc = 0;
  double ratio = 1.0, gp = INFINITY, gq = INFINITY;
  const int st_p = filter_row<E, VEC>(static_cast<const E*>(a.p) + off, V, fp, sh, sh.dp, gp);
  if (gp < NEAR_TIE) flags |= FLAG_TIE_TOPP_P;
  if (i == 0) {
    acc = 1;
    if (st_p == ROW_OK) {
      bool tie = false;
      const int j = block_icdf(tid < sh.dp.n ? sh.dp.prob[tid] : 0.0, sh.dp.n, u_res, sh, &tie);
      tok = sh.dp.ids[j];
      if (tie) flags |= FLAG_TIE_ICDF;
    } else {
      flags |= FLAG_OVERFLOW;
    }
  } else {
    const int st_q = filter_row<E, VEC>(static_cast<const E*>(a.q) + off, V, fp, sh, sh.dq, gq);
    if (gq < NEAR_TIE) flags |= FLAG_TIE_TOPP_Q;
    if (st_p == ROW_OK && st_q == ROW_OK) {
      const int d = a.draft[g];
      if (tid == 0) { sh.dres[0] = 0.0; sh.dres[1] = 0.0; }
      __syncthreads();
      if (tid < sh.dp.n && sh.dp.ids[tid] == d) sh.dres[0] = sh.dp.prob[tid];
      if (tid < sh.dq.n && sh.dq.ids[tid] == d) sh.dres[1] = sh.dq.prob[tid];
      __syncthreads();
      const double pd = sh.dres[0], qd = sh.dres[1];
      if (qd == 0.0) {
        acc = 0;
        ratio = 0.0;
        flags |= FLAG_Q_ZERO;
      } else {
        ratio = pd / qd;
        acc = u_acc < ratio ? 1 : 0;
        if (fabs(u_acc - ratio) < NEAR_TIE) flags |= FLAG_TIE_ACCEPT;
      }
      if (acc) {
        tok = d;
      } else {
        double r = 0.0;
        if (tid < sh.dp.n) r = fmax(0.0, sh.dp.prob[tid] - lookup_prob(sh.dq, sh.dp.ids[tid]));
        const double rsum = block_sum_d(r, sh);
        if (rsum == 0.0) {
          flags |= FLAG_RES_ZERO;
          r = tid < sh.dp.n ? sh.dp.prob[tid] : 0.0;
        }
        bool tie = false;
        const int j = block_icdf(r, sh.dp.n, u_res, sh, &tie);
        tok = sh.dp.ids[j];
        if (tie) flags |= FLAG_TIE_ICDF;
      }
    } else {
      flags |= FLAG_OVERFLOW;
    }
  }

  // Slot record, then the per-sequence ticket.
  unsigned* counters = static_cast<unsigned*>(a.ws);
  unsigned long long* rec = reinterpret_cast<unsigned long long*>(
      static_cast<char*>(a.ws) + ((size_t(a.S) * 4 + 255) / 256) * 256);
  if (tid == 0) {
    if (a.slot_accept) a.slot_accept[g] = uint8_t(acc);
    if (a.diag) {
      a.diag[size_t(g) * 4 + 0] = float(u_acc);
      a.diag[size_t(g) * 4 + 1] = float(ratio);
      a.diag[size_t(g) * 4 + 2] = float(u_res);
      a.diag[size_t(g) * 4 + 3] = float(flags);
    }
    rec[g] = (unsigned long long)(unsigned)tok | ((unsigned long long)(unsigned)acc << 32);
    __threadfence();
    const unsigned old = atomicAdd(&counters[s], 1u);
    sh.ires = old == unsigned(b - 1) ? 1 : 0;
  }
  __syncthreads();
  if (sh.ires && tid < kWave) {
    __threadfence();
    unsigned long long r = 0x100000000ull | 0xffffffffull;   // (tok -1, acc 1)
    if (tid < b) r = __hip_atomic_load(&rec[size_t(s) * b + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int rtok = int(unsigned(r & 0xffffffffull));
    const int racc = int(r >> 32);
    const unsigned long long rej = __ballot(tid >= 1 && tid < b && racc == 0);
    const int nacc = rej ? (__ffsll((long long)rej) - 1) : b;
    if (tid < b) a.out_tokens[size_t(s) * b + tid] = tid <= nacc ? rtok : -1;
    const int rs = __shfl(rtok, nacc < b ? nacc : 0, kWave);
    if (tid == 0) {
      a.accept_len[s] = nacc;
      a.resampled[s] = nacc < b ? rs : -1;
      __hip_atomic_store(&counters[s], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <typename E, bool VEC>
__global__ __launch_bounds__(VT) void draft_kernel(DraftArgs a) {
  __shared__ Shared sh;
  const int g = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int b = a.b, V = a.V;
  const int s = g / b, i = g - s * b;
  const int tid = threadIdx.x;
  const FilterParams fp = make_filter_params(a.sp, V);
  const Philox4 ph = philox4x64_10(uint64_t(a.pos[s] + i), 1ull, 0ull, 0ull, a.sp.seed,
                                   uint64_t(a.seq_ids[s]));
  const double u = word_to_uniform(ph.w[0]);
  double gq = INFINITY;
  int flags = 0, tok = -1;
  const int st = filter_row<E, VEC>(static_cast<const E*>(a.q) + size_t(g) * V, V, fp, sh, sh.dq, gq);
  if (gq < NEAR_TIE) flags |= FLAG_TIE_TOPP_Q;
  if (st == ROW_OK) {
    bool tie = false;
    const int j = block_icdf(tid < sh.dq.n ? sh.dq.prob[tid] : 0.0, sh.dq.n, u, sh, &tie);
    tok = sh.dq.ids[j];
    if (tie) flags |= FLAG_TIE_ICDF;
  } else {
    flags |= FLAG_OVERFLOW;
  }
  if (tid == 0) {
    a.draft[g] = tok;
    if (a.flags) a.flags[g] = flags;
  }
}

__global__ void zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += size_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

template <typename E>
bool rows_aligned(const void* base, int V) {
  return (reinterpret_cast<uintptr_t>(base) % 16 == 0) && ((size_t(V) * sizeof(E)) % 16 == 0);
}

}  // namespace

size_t verify_workspace_bytes(int S, int b) {
  return ((size_t(S) * 4 + 255) / 256) * 256 + size_t(S) * size_t(b) * 8;
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
  const int grid = a.S * a.b;
  if (grid == 0) return hipSuccess;
  if (a.bf16) {
    const bool vec = rows_aligned<uint16_t>(a.p, a.V) && rows_aligned<uint16_t>(a.q, a.V);
    if (vec) hipLaunchKernelGGL((verify_kernel<uint16_t, true>), dim3(grid), dim3(VT), 0, stream, a);
    else hipLaunchKernelGGL((verify_kernel<uint16_t, false>), dim3(grid), dim3(VT), 0, stream, a);
  } else {
    const bool vec = rows_aligned<float>(a.p, a.V) && rows_aligned<float>(a.q, a.V);
    if (vec) hipLaunchKernelGGL((verify_kernel<float, true>), dim3(grid), dim3(VT), 0, stream, a);
    else hipLaunchKernelGGL((verify_kernel<float, false>), dim3(grid), dim3(VT), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_draft(const DraftArgs& a, hipStream_t stream) {
  const int grid = a.S * a.b;
  if (grid == 0) return hipSuccess;
  if (a.bf16) {
    if (rows_aligned<uint16_t>(a.q, a.V))
      hipLaunchKernelGGL((draft_kernel<uint16_t, true>), dim3(grid), dim3(VT), 0, stream, a);
    else
      hipLaunchKernelGGL((draft_kernel<uint16_t, false>), dim3(grid), dim3(VT), 0, stream, a);
  } else {
    if (rows_aligned<float>(a.q, a.V))
      hipLaunchKernelGGL((draft_kernel<float, true>), dim3(grid), dim3(VT), 0, stream, a);
    else
      hipLaunchKernelGGL((draft_kernel<float, false>), dim3(grid), dim3(VT), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  const size_t n = bytes / 4;
  if (n) {
    const size_t blocks = (n + 255) / 256;
    const int grid = int(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint32_t*>(ptr), n);
  }
  return hipGetLastError();
}

}  // namespace uno
