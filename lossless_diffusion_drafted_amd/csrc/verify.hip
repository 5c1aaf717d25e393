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
//  * The slot's p and q rows are streamed once from HBM, interleaved tile by tile
//    (16-byte buffer loads, eight per thread per tile, one tile in flight while the
//    other is scanned), into one LDS candidate list per row.
//  * A lower bound of each row's k-th largest logit comes from its first tile and
//    is raised as the scan proceeds: each wave takes the ceil(k/4)-th largest of
//    its 64 running lane maxima, so the minimum over the 4 waves has at least k
//    row elements at or above it. For bf16 rows with a positive bound, eight
//    elements are pre-checked with three packed 16-bit max instructions.
//  * After the stream, wave 0 selects and filters the p row while wave 1 does the
//    q row, with no barriers: an MSB-first radix select over the candidates'
//    order-preserving keys (only the bits where they differ) gives the exact
//    k-th largest value; every candidate at or above it forms the tie-inclusive
//    top-k set; softmax, top-p and the renormalised distribution are fp64 on it.
//  * Wave 0 then runs the accept test and the inverse CDF in fp64, writes the
//    slot record with a device-coherent store, and takes a per-sequence ticket;
//    the last workgroup of a sequence runs the prefix scan and resets the ticket.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace uno {
namespace {

constexpr int VT = 256;               // threads per workgroup
constexpr int VW = VT / kWave;        // waves per workgroup
constexpr int UNR = 8;                // 16-byte loads per thread per tile
constexpr int CAND_CAP = 1024;        // candidates kept per row
constexpr int WAVE_SEL_MAX = 512;     // candidates one wave selects from (8 per lane)
constexpr int SEL_CAP = 256;          // largest filtered support on this path
constexpr int KMAX_FAST = kVerifyKMaxFast;
constexpr double NEAR_TIE = 1e-6;
constexpr int PER_TILE = VT * UNR;    // 16-byte chunks per tile

constexpr int FLAG_TIE_ACCEPT = 1, FLAG_TIE_TOPP_P = 2, FLAG_TIE_TOPP_Q = 4,
              FLAG_TIE_ICDF = 8, FLAG_Q_ZERO = 16, FLAG_RES_ZERO = 32, FLAG_OVERFLOW = 64;

enum { ROW_OK = 0, ROW_OVERFLOW = 1 };

typedef short short2_t __attribute__((ext_vector_type(2)));

struct Dist {            // filtered distribution: ascending ids, fp64 probabilities
  int n;
  double gap;            // min |mass above a non-top group - top_p| (inf if top-p off)
  int ids[SEL_CAP];
  double prob[SEL_CAP];
};

struct RowLds {          // per-row state of the selection
  float cval[CAND_CAP];
  int cidx[CAND_CAP];
  alignas(16) float sval[SEL_CAP];
  alignas(16) int sidx[SEL_CAP];
  double sw[SEL_CAP];
  unsigned hist[256];
  float wthr[VW];        // per-wave published lower bounds
  int cnt;               // candidates pushed (may exceed CAND_CAP: overflow)
  int n;                 // size of the tie-inclusive top-k set
  unsigned kmax;         // largest candidate key
  int status;
};

struct Shared {
  RowLds row[2];         // 0: base row p, 1: draft row q
  Dist dist[2];
  alignas(16) float lanebuf[VW][kWave];
  unsigned red_u[VW][3];
  unsigned ures[2];
};

struct FilterParams {
  double T;
  double top_p;
  int k_eff;        // tie-inclusive top-k size (V when top-k is off)
  bool greedy;
  bool topp_on;
};

__device__ __forceinline__ FilterParams make_filter_params(const SamplingArgs& sp, int V) {
  FilterParams fp;
  fp.T = sp.temperature;
  fp.greedy = !(sp.temperature > 0.0);
  fp.top_p = sp.top_p;
  fp.topp_on = !fp.greedy && sp.top_p < 1.0;
  fp.k_eff = fp.greedy ? 1 : ((sp.top_k > 0 && sp.top_k < V) ? sp.top_k : V);
  return fp;
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int ballot_rank(unsigned long long mask) {
  return int(__builtin_amdgcn_mbcnt_hi(unsigned(mask >> 32), __builtin_amdgcn_mbcnt_lo(unsigned(mask), 0u)));
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
  __device__ static uint4 neg_inf() { return make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u); }
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
  __device__ static uint4 neg_inf() { return make_uint4(0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u); }
};

// One row, viewed as 16-byte chunks. The vector path issues one range-checked
// buffer load per chunk: bytes past the row read as zero (no fault) and are
// masked to -inf by index in the last tile, so every tile issues the same number
// of loads and the compiler can wait chunk by chunk. Rows that are not 16-byte
// aligned take a scalar path.
template <typename E, bool VEC>
struct RowView {
  using EL = Elem<E>;
  static constexpr int VN = EL::VN;
  const E* row;
  int V, nfull, nchunks, ntiles, full_tiles;
  __amdgpu_buffer_rsrc_t rsrc;

  __device__ __forceinline__ RowView(const E* r, int V_) : row(r), V(V_) {
    nfull = V / VN;
    nchunks = (V + VN - 1) / VN;
    ntiles = (nchunks + PER_TILE - 1) / PER_TILE;
    full_tiles = VEC ? nfull / PER_TILE : 0;
    rsrc = make_row_rsrc(row, uint32_t(V) * uint32_t(sizeof(E)));
  }

  __device__ __forceinline__ void load_tile(uint4 (&r)[UNR], int t) const {
    const int tid = threadIdx.x;
    if (VEC) {
      const uint32_t voff = uint32_t(tid) * 16u;
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        r[u] = buffer_load16(rsrc, voff, uint32_t(t * PER_TILE + u * VT) * 16u);
    } else {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = t * PER_TILE + u * VT + tid;
        r[u] = c < nchunks ? EL::load_partial(row, c * VN, V) : EL::neg_inf();
      }
    }
  }
};

// Scan state of one row during the stream.
struct RowScan {
  float thr;        // current lower bound of the k-th largest value
  float lmax;       // running maximum of this lane's elements (float path)
  int lmax16;       // running maximum as a signed 16-bit bf16 pattern (packed path)
};

// c-th largest of the wave's 64 lane values (LDS broadcast reads; a wave's LDS
// operations complete in order, so no barrier is needed).
__device__ __forceinline__ float wave_cth_largest(float m, int c, Shared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  sh.lanebuf[wid][lane] = m;
  const float4* lb = reinterpret_cast<const float4*>(sh.lanebuf[wid]);
  int cnt_ge = 0;
#pragma unroll
  for (int j = 0; j < kWave / 4; ++j) {
    const float4 v = lb[j];
    cnt_ge += (v.x >= m) + (v.y >= m) + (v.z >= m) + (v.w >= m);
  }
  return wave_max(cnt_ge >= c ? m : -INFINITY);
}

template <typename E, bool VEC>
__device__ __forceinline__ void process_tile(const RowView<E, VEC>& rv, RowLds& R, const uint4 (&r)[UNR],
                                             int t, RowScan& sc) {
  using EL = Elem<E>;
  constexpr int VN = EL::VN;
  const int tid = threadIdx.x;
  const int V = rv.V;
  const float thr = sc.thr;
  const bool tail = t >= rv.full_tiles;
  // bf16 with a positive bound: signed 16-bit order equals value order for every
  // element that can reach the bound, so a packed max pre-checks 8 elements.
  const bool packed = VN == 8 && !tail && thr > 0.0f;
  const int thr16 = int(__float_as_uint(thr) >> 16);
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int e0 = (t * PER_TILE + u * VT + tid) * VN;
    bool maybe;
    if (packed) {
      const short2_t m01 = __builtin_elementwise_max(__builtin_bit_cast(short2_t, r[u].x),
                                                     __builtin_bit_cast(short2_t, r[u].y));
      const short2_t m23 = __builtin_elementwise_max(__builtin_bit_cast(short2_t, r[u].z),
                                                     __builtin_bit_cast(short2_t, r[u].w));
      const short2_t m = __builtin_elementwise_max(m01, m23);
      const int mx = max(int(m.x), int(m.y));
      sc.lmax16 = max(sc.lmax16, mx);
      maybe = mx >= thr16;
    } else {
      float x[VN];
      EL::unpack(r[u], x);
      if (tail) {
#pragma unroll
        for (int j = 0; j < VN; ++j) x[j] = (e0 + j < V) ? x[j] : -INFINITY;
      }
      float mx = x[0];
#pragma unroll
      for (int j = 1; j < VN; ++j) mx = fmaxf(mx, x[j]);
      sc.lmax = fmaxf(sc.lmax, mx);
      maybe = mx >= thr;
    }
    if (maybe) {
      float x[VN];
      EL::unpack(r[u], x);
#pragma unroll
      for (int j = 0; j < VN; ++j) {
        if (x[j] >= thr && e0 + j < V) {
          const int p = atomicAdd(&R.cnt, 1);
          if (p < CAND_CAP) { R.cval[p] = x[j]; R.cidx[p] = e0 + j; }
        }
      }
    }
  }
}

// Running lane maximum as a float (both paths contribute real element values).
__device__ __forceinline__ float scan_lane_max(const RowScan& sc) {
  const float p = sc.lmax16 > -32768 ? bf16_to_f32(uint16_t(sc.lmax16 & 0xffff)) : -INFINITY;
  return fmaxf(sc.lmax, p);
}

// Publish this wave's bound for row R and return the current minimum over waves.
__device__ __forceinline__ float refresh_bound(RowLds& R, const RowScan& sc, int c, Shared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const float tw = wave_cth_largest(scan_lane_max(sc), c, sh);
  if (lane == 0) R.wthr[wid] = tw;
  float t = R.wthr[0];
#pragma unroll
  for (int i = 1; i < VW; ++i) t = fminf(t, R.wthr[i]);
  return fmaxf(t, sc.thr);
}

// First-tile lane maxima -> initial bound (published; caller synchronises).
template <typename E, bool VEC>
__device__ __forceinline__ void init_bound(const RowView<E, VEC>& rv, RowLds& R, const uint4 (&r)[UNR],
                                           int c, RowScan& sc, Shared& sh) {
  using EL = Elem<E>;
  constexpr int VN = EL::VN;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    float x[VN];
    EL::unpack(r[u], x);
    const int e0 = (u * VT + tid) * VN;
#pragma unroll
    for (int j = 0; j < VN; ++j) sc.lmax = (e0 + j < rv.V) ? fmaxf(sc.lmax, x[j]) : sc.lmax;
  }
  const float tw = wave_cth_largest(sc.lmax, c, sh);
  if (lane == 0) R.wthr[wid] = tw;
}

__device__ __forceinline__ float read_bound(const RowLds& R) {
  float t = R.wthr[0];
#pragma unroll
  for (int i = 1; i < VW; ++i) t = fminf(t, R.wthr[i]);
  return t;
}

__device__ __forceinline__ void reset_row(RowLds& R) {
  if (threadIdx.x == 0) { R.cnt = 0; R.status = ROW_OK; R.n = 0; }
}

// Stream one row (scalar path, or a row without a partner) with double buffering
// inside the row. Caller has reset R (the barrier inside orders that); ends with
// a barrier.
template <typename E, bool VEC>
__device__ __forceinline__ void stream_one(const RowView<E, VEC>& rv, const FilterParams& fp, RowLds& R,
                                           Shared& sh) {
  const bool bounded = fp.k_eff <= KMAX_FAST;
  const int c = (fp.k_eff + VW - 1) / VW;
  uint4 A[UNR], B[UNR];
  rv.load_tile(A, 0);
  if (VEC || rv.ntiles > 1) rv.load_tile(B, 1);
  RowScan sc{-INFINITY, -INFINITY, -32768};
  if (bounded) init_bound(rv, R, A, c, sc, sh);
  __syncthreads();
  if (bounded) sc.thr = read_bound(R);
  if (VEC) {
    for (int t = 0; t < rv.ntiles; t += 2) {
      process_tile(rv, R, A, t, sc);
      rv.load_tile(A, t + 2);
      if (t + 1 < rv.ntiles) process_tile(rv, R, B, t + 1, sc);
      rv.load_tile(B, t + 3);
      if (bounded && (t == 0 || t == 2 || t == 6)) sc.thr = refresh_bound(R, sc, c, sh);
    }
  } else {
    process_tile(rv, R, A, 0, sc);
    for (int t = 1; t < rv.ntiles; t += 2) {
      if (t + 1 < rv.ntiles) rv.load_tile(A, t + 1);
      process_tile(rv, R, B, t, sc);
      if (t + 1 < rv.ntiles) {
        if (t + 2 < rv.ntiles) rv.load_tile(B, t + 2);
        process_tile(rv, R, A, t + 1, sc);
      }
    }
  }
  __syncthreads();
}

// Stream two rows of the same length interleaved tile by tile (vector path).
// Caller has reset both rows; ends with a barrier.
template <typename E>
__device__ __forceinline__ void stream_two(const RowView<E, true>& pv, const RowView<E, true>& qv,
                                           const FilterParams& fp, RowLds& Rp, RowLds& Rq, Shared& sh) {
  const bool bounded = fp.k_eff <= KMAX_FAST;
  const int c = (fp.k_eff + VW - 1) / VW;
  uint4 A[UNR], B[UNR];
  pv.load_tile(A, 0);
  qv.load_tile(B, 0);
  RowScan sp{-INFINITY, -INFINITY, -32768}, sq{-INFINITY, -INFINITY, -32768};
  if (bounded) {
    init_bound(pv, Rp, A, c, sp, sh);
    init_bound(qv, Rq, B, c, sq, sh);
  }
  __syncthreads();
  if (bounded) {
    sp.thr = read_bound(Rp);
    sq.thr = read_bound(Rq);
  }
  for (int t = 0; t < pv.ntiles; ++t) {
    process_tile(pv, Rp, A, t, sp);
    pv.load_tile(A, t + 1);
    process_tile(qv, Rq, B, t, sq);
    qv.load_tile(B, t + 1);
    if (bounded && (t == 1 || t == 3 || t == 7)) {
      sp.thr = refresh_bound(Rp, sp, c, sh);
      sq.thr = refresh_bound(Rq, sq, c, sh);
    }
  }
  __syncthreads();
}

// --- selection: exact tie-inclusive top-k set of a row's candidates ------------

// By one wave (C <= 512 candidates, 8 per lane), without barriers.
__device__ __forceinline__ void wave_select(RowLds& R, const FilterParams& fp) {
  const int lane = threadIdx.x & (kWave - 1);
  const int C = R.cnt;
  constexpr int M = WAVE_SEL_MAX / kWave;
  unsigned key[M];
  unsigned kmax = 0u, kand = 0xffffffffu, kor = 0u;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int i = m * kWave + lane;
    key[m] = 0u;
    if (i < C) {
      key[m] = float_key(R.cval[i]);
      kmax = max(kmax, key[m]);
      kand &= key[m];
      kor |= key[m];
    }
  }
  kmax = wave_max(kmax);
  kor = wave_or(kor);
  kand = ~wave_or(~kand);
  const unsigned diff = kor ^ kand;
  unsigned kstar = kmax;
  if (fp.k_eff >= C) {
    kstar = 0u;                               // every candidate is in the top-k set
  } else if (diff != 0u) {
    const int hb = 31 - __clz(diff);
    const int lb = __ffs(diff) - 1;
    unsigned pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);
    unsigned prefix = kand & pmask;
    unsigned remaining = unsigned(fp.k_eff);
    int hi = hb;
    while (true) {
      const int lo = max(hi - 7, lb);
      const unsigned dmask = (1u << (hi - lo + 1)) - 1u;
#pragma unroll
      for (int q = 0; q < 4; ++q) R.hist[4 * lane + q] = 0u;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (m * kWave + lane < C && (key[m] & pmask) == prefix) atomicAdd(&R.hist[(key[m] >> lo) & dmask], 1u);
      }
      // lane l owns digits 255-4l .. 252-4l (highest digits first)
      unsigned h[4];
      unsigned s = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { h[q] = R.hist[255 - 4 * lane - q]; s += h[q]; }
      const unsigned incl = wave_inclusive_scan(s);
      unsigned acc = incl - s;
      const bool mine = acc < remaining && remaining <= incl;
      unsigned d = 0u, above = 0u;
      if (mine) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (acc + h[q] >= remaining) { d = unsigned(255 - 4 * lane - q); above = acc; break; }
          acc += h[q];
        }
      }
      const int src = __ffsll((long long)__ballot(mine)) - 1;
      d = unsigned(readlane_i(int(d), src));
      above = unsigned(readlane_i(int(above), src));
      remaining -= above;
      prefix |= d << lo;
      pmask |= dmask << lo;
      if (lo == lb) break;
      hi = lo - 1;
    }
    const unsigned lowmask = lb == 0 ? 0u : ((1u << lb) - 1u);
    kstar = prefix | (kand & lowmask);
  }
  // Compact the set (ballot ranks) into sval/sidx.
  int base = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int i = m * kWave + lane;
    const bool sel = i < C && key[m] >= kstar;
    const unsigned long long bal = __ballot(sel);
    const int pos = base + ballot_rank(bal);
    if (sel && pos < SEL_CAP) {
      R.sval[pos] = key_float(key[m]);
      R.sidx[pos] = R.cidx[i];
    }
    base += __popcll(bal);
  }
  if (lane == 0) {
    R.n = base;
    R.kmax = kmax;
    R.status = base > SEL_CAP ? ROW_OVERFLOW : ROW_OK;
  }
}

// By the whole workgroup (512 < C <= 1024 candidates). Every thread calls it.
__device__ __forceinline__ void block_select(RowLds& R, const FilterParams& fp, Shared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int C = R.cnt;
  unsigned kmax = 0u, kand = 0xffffffffu, kor = 0u;
  for (int i = tid; i < C; i += VT) {
    const unsigned k = float_key(R.cval[i]);
    kmax = max(kmax, k);
    kand &= k;
    kor |= k;
  }
  kmax = wave_max(kmax);
  kor = wave_or(kor);
  kand = ~wave_or(~kand);
  __syncthreads();
  if (lane == 0) { sh.red_u[wid][0] = kmax; sh.red_u[wid][1] = kand; sh.red_u[wid][2] = kor; }
  __syncthreads();
  kmax = 0u; kand = 0xffffffffu; kor = 0u;
#pragma unroll
  for (int i = 0; i < VW; ++i) { kmax = max(kmax, sh.red_u[i][0]); kand &= sh.red_u[i][1]; kor |= sh.red_u[i][2]; }
  const unsigned diff = kor ^ kand;
  unsigned kstar = kmax;
  if (fp.k_eff >= C) {
    kstar = 0u;
  } else if (diff != 0u) {
    const int hb = 31 - __clz(diff);
    const int lb = __ffs(diff) - 1;
    unsigned pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);
    unsigned prefix = kand & pmask;
    unsigned remaining = unsigned(fp.k_eff);
    int hi = hb;
    while (true) {
      const int lo = max(hi - 7, lb);
      const unsigned dmask = (1u << (hi - lo + 1)) - 1u;
      for (int i = tid; i < 256; i += VT) R.hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < C; i += VT) {
        const unsigned k = float_key(R.cval[i]);
        if ((k & pmask) == prefix) atomicAdd(&R.hist[(k >> lo) & dmask], 1u);
      }
      __syncthreads();
      if (wid == 0) {
        unsigned h[4];
        unsigned s = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { h[q] = R.hist[255 - 4 * lane - q]; s += h[q]; }
        const unsigned incl = wave_inclusive_scan(s);
        unsigned acc = incl - s;
        if (acc < remaining && remaining <= incl) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (acc + h[q] >= remaining) { sh.ures[0] = unsigned(255 - 4 * lane - q); sh.ures[1] = acc; break; }
            acc += h[q];
          }
        }
      }
      __syncthreads();
      const unsigned d = sh.ures[0];
      remaining -= sh.ures[1];
      prefix |= d << lo;
      pmask |= dmask << lo;
      __syncthreads();
      if (lo == lb) break;
      hi = lo - 1;
    }
    const unsigned lowmask = lb == 0 ? 0u : ((1u << lb) - 1u);
    kstar = prefix | (kand & lowmask);
  }
  if (tid == 0) R.n = 0;
  __syncthreads();
  for (int i = tid; i < C; i += VT) {
    const unsigned k = float_key(R.cval[i]);
    if (k >= kstar) {
      const int p = atomicAdd(&R.n, 1);
      if (p < SEL_CAP) { R.sval[p] = key_float(k); R.sidx[p] = R.cidx[i]; }
    }
  }
  __syncthreads();
  if (tid == 0) {
    R.kmax = kmax;
    R.status = R.n > SEL_CAP ? ROW_OVERFLOW : ROW_OK;
  }
  __syncthreads();
}

// --- fp64 filter of the selected set (one wave, M entries per lane) ------------
// Entry j = m*64 + lane. Pairwise sums run through LDS broadcast reads.
template <int M>
__device__ __forceinline__ void wave_filter_m(const FilterParams& fp, RowLds& R, Dist& out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = R.n;
  const float zmax = key_float(R.kmax);
  float zj[M];
  int idj[M];
  double w[M];
  bool keep[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int j = m * kWave + lane;
    const bool valid = j < n;
    zj[m] = valid ? R.sval[j] : -INFINITY;
    idj[m] = valid ? R.sidx[j] : 0x7fffffff;
    keep[m] = valid;
  }
  if (fp.greedy) {
    // One-hot at the argmax, lowest id on ties (the set holds exactly the ties).
    int mn = idj[0];
#pragma unroll
    for (int m = 1; m < M; ++m) mn = min(mn, idj[m]);
    const int id = wave_min(mn);
    if (lane == 0) { out.n = 1; out.gap = INFINITY; out.ids[0] = id; out.prob[0] = 1.0; }
    return;
  }
  double wl = 0.0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    w[m] = keep[m] ? exp((double(zj[m]) - double(zmax)) / fp.T) : 0.0;
    R.sw[m * kWave + lane] = w[m];
    if (!keep[m]) R.sval[m * kWave + lane] = -INFINITY;
    wl += w[m];
  }
  const int n4 = (n + 3) & ~3;            // padded entries have z = -inf, w = 0
  double gap = INFINITY;
  if (fp.topp_on) {
    const double ztop = wave_sum(wl);
    double above[M];
#pragma unroll
    for (int m = 0; m < M; ++m) above[m] = 0.0;
    for (int i = 0; i < n4; i += 4) {
      const float4 zv = *reinterpret_cast<const float4*>(&R.sval[i]);
      const double w0 = R.sw[i], w1 = R.sw[i + 1], w2 = R.sw[i + 2], w3 = R.sw[i + 3];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        above[m] += (zv.x > zj[m] ? w0 : 0.0) + (zv.y > zj[m] ? w1 : 0.0);
        above[m] += (zv.z > zj[m] ? w2 : 0.0) + (zv.w > zj[m] ? w3 : 0.0);
      }
    }
    double gl = INFINITY;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (keep[m]) {
        const double mass = above[m] / ztop;
        // the top group is kept unconditionally, so only lower groups decide
        if (zj[m] != zmax) gl = fmin(gl, fabs(mass - fp.top_p));
        keep[m] = (zj[m] == zmax) || (mass < fp.top_p);
      }
    }
    gap = wave_min(gl);
  }
  double wk = 0.0;
  int nk = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    wk += keep[m] ? w[m] : 0.0;
    nk += __popcll(__ballot(keep[m]));
    R.sidx[m * kWave + lane] = keep[m] ? idj[m] : 0x7fffffff;   // dropped -> last
  }
  const double wsum = wave_sum(wk);
  // position of each kept entry in ascending-id order
  int pos[M];
#pragma unroll
  for (int m = 0; m < M; ++m) pos[m] = 0;
  for (int i = 0; i < n4; i += 4) {
    const int4 v = *reinterpret_cast<const int4*>(&R.sidx[i]);
#pragma unroll
    for (int m = 0; m < M; ++m) pos[m] += (v.x < idj[m]) + (v.y < idj[m]) + (v.z < idj[m]) + (v.w < idj[m]);
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (keep[m]) {
      out.ids[pos[m]] = idj[m];
      out.prob[pos[m]] = w[m] / wsum;
    }
  }
  if (lane == 0) { out.n = nk; out.gap = gap; }
}

__device__ __forceinline__ void wave_filter(const FilterParams& fp, RowLds& R, Dist& out) {
  if (R.n <= kWave) wave_filter_m<1>(fp, R, out);
  else wave_filter_m<SEL_CAP / kWave>(fp, R, out);
}

// --- inverse CDF (one wave) ------------------------------------------------------
// First j with u*Z < C_j, C the inclusive prefix sum of the weights over ascending
// ids and Z = C_{n-1} (the smallest such j over the wave); falls back to the last
// positive weight. *tie is set when u*Z lies within 1e-6*Z of a decision
// boundary. Blocked layout: lane l holds entries M*l .. M*l+M-1 (n <= 64*M).
// Every lane returns the index.
template <int M>
__device__ __forceinline__ int wave_icdf(const double (&w)[M], int n, double u, bool* tie) {
  const int lane = threadIdx.x & (kWave - 1);
  double c[M];
  double run = 0.0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    run += (M * lane + m < n) ? w[m] : 0.0;
    c[m] = run;
  }
  const double incl = wave_inclusive_scan(run);
  const double up = __shfl_up(incl, 1, kWave);
  const double off = lane > 0 ? up : 0.0;          // exclusive prefix of this lane
  const double Z = readlane_d(incl, kWave - 1);
  const double t = u * Z;
  int hit = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int m = M - 1; m >= 0; --m) {
    const int j = M * lane + m;
    if (j < n && off + c[m] > t) hit = j;
    if (j < n && w[m] > 0.0 && lastpos < 0) lastpos = j;
  }
  int jj = wave_min(hit);
  if (jj == 0x7fffffff) jj = max(wave_max(lastpos), 0);
  // distance of u*Z to the chosen entry's two boundaries
  double gap = INFINITY;
  const int owner = jj / M, mm = jj % M;
  if (lane == owner) {
    double lo = off, hi = off;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (m == mm) hi = off + c[m];
      if (m + 1 == mm) lo = off + c[m];
    }
    if (jj < n - 1) gap = fabs(t - hi);
    if (jj > 0) gap = fmin(gap, fabs(t - lo));
  }
  *tie = readlane_d(gap, owner) < NEAR_TIE * Z;
  return jj;
}

// Inverse CDF of a filtered distribution (ids ascending) at u, by one wave.
__device__ __forceinline__ int sample_dist(const Dist& dd, double u, bool* tie) {
  const int lane = threadIdx.x & (kWave - 1);
  if (dd.n <= kWave) {
    double w[1] = {lane < dd.n ? dd.prob[lane] : 0.0};
    return dd.ids[wave_icdf<1>(w, dd.n, u, tie)];
  }
  constexpr int M = SEL_CAP / kWave;
  double w[M];
#pragma unroll
  for (int m = 0; m < M; ++m) w[m] = (M * lane + m < dd.n) ? dd.prob[M * lane + m] : 0.0;
  return dd.ids[wave_icdf<M>(w, dd.n, u, tie)];
}

__device__ __forceinline__ double lookup_prob(const Dist& d, int tok) {
  int lo = 0, hi = d.n;                 // binary search over ascending ids
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (d.ids[mid] < tok) lo = mid + 1; else hi = mid;
  }
  return (lo < d.n && d.ids[lo] == tok) ? d.prob[lo] : 0.0;
}

struct SlotResult {
  int tok, acc, flags;
  double ratio;
};

// Accept / resample of one draft slot from the filtered p~ (dp) and q~ (dq), by
// one wave. M entries of dp per lane in blocked layout.
template <int M>
__device__ __forceinline__ SlotResult decide_m(const Dist& dp, const Dist& dq, int d, double u_acc, double u_res) {
  const int lane = threadIdx.x & (kWave - 1);
  const int np = dp.n, nq = dq.n;
  SlotResult r;
  r.flags = 0;
  double pd = 0.0, qd = 0.0;
  for (int j = lane; j < np; j += kWave) pd = dp.ids[j] == d ? dp.prob[j] : pd;
  for (int j = lane; j < nq; j += kWave) qd = dq.ids[j] == d ? dq.prob[j] : qd;
  pd = wave_max(pd);
  qd = wave_max(qd);
  if (qd == 0.0) {
    r.acc = 0;
    r.ratio = 0.0;
    r.flags |= FLAG_Q_ZERO;
  } else {
    r.ratio = pd / qd;
    r.acc = u_acc < r.ratio ? 1 : 0;
    if (fabs(u_acc - r.ratio) < NEAR_TIE) r.flags |= FLAG_TIE_ACCEPT;
  }
  if (r.acc) {
    r.tok = d;
    return r;
  }
  double pp[M], res[M];
  double rl = 0.0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int j = M * lane + m;
    pp[m] = j < np ? dp.prob[j] : 0.0;
    const double qv = j < np ? lookup_prob(dq, dp.ids[j]) : 0.0;
    res[m] = j < np ? fmax(0.0, pp[m] - qv) : 0.0;
    rl += res[m];
  }
  if (wave_sum(rl) == 0.0) {
    r.flags |= FLAG_RES_ZERO;
#pragma unroll
    for (int m = 0; m < M; ++m) res[m] = pp[m];
  }
  bool tie = false;
  const int j = wave_icdf<M>(res, np, u_res, &tie);
  r.tok = dp.ids[j];
  if (tie) r.flags |= FLAG_TIE_ICDF;
  return r;
}

// --- kernels -------------------------------------------------------------------
template <typename E, bool VEC>
__global__ __launch_bounds__(VT) void verify_kernel(VerifyArgs a) {
  __shared__ Shared sh;
  const int g = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int b = a.b, V = a.V;
  const int s = g / b, i = g - s * b;
  const int tid = threadIdx.x, wid = tid / kWave;
  const FilterParams fp = make_filter_params(a.sp, V);
  const size_t off = size_t(g) * size_t(V);
  const bool has_q = i > 0;
  RowLds& Rp = sh.row[0];
  RowLds& Rq = sh.row[1];

  const RowView<E, VEC> pv(static_cast<const E*>(a.p) + off, V);
  const RowView<E, VEC> qv(static_cast<const E*>(a.q) + off, V);
  reset_row(Rp);
  reset_row(Rq);
  bool done = false;
  if constexpr (VEC) {
    if (has_q) {
      stream_two<E>(pv, qv, fp, Rp, Rq, sh);
      done = true;
    }
  }
  if (!done) {
    stream_one(pv, fp, Rp, sh);
    if (has_q) stream_one(qv, fp, Rq, sh);
  }

  // Selection: one wave per row when both candidate lists are small enough.
  const int cp = Rp.cnt, cq = has_q ? Rq.cnt : 0;
  __syncthreads();                  // every thread has read the counts
  if (tid == 0) {
    if (cp > CAND_CAP) Rp.status = ROW_OVERFLOW;
    if (cq > CAND_CAP) Rq.status = ROW_OVERFLOW;
  }
  __syncthreads();
  if (cp <= WAVE_SEL_MAX && cq <= WAVE_SEL_MAX) {
    if (wid == 0) wave_select(Rp, fp);
    if (wid == 1 && has_q) wave_select(Rq, fp);
  } else {
    if (Rp.status == ROW_OK) block_select(Rp, fp, sh);
    if (has_q && Rq.status == ROW_OK) block_select(Rq, fp, sh);
  }
  __syncthreads();
  if (wid == 0 && Rp.status == ROW_OK) wave_filter(fp, Rp, sh.dist[0]);
  if (wid == 1 && has_q && Rq.status == ROW_OK) wave_filter(fp, Rq, sh.dist[1]);
  __syncthreads();

  if (wid != 0) return;             // wave 0 finishes the slot alone

  const Philox4 ph = philox4x64_10(uint64_t(a.pos[s] + i), 0ull, 0ull, 0ull, a.sp.seed,
                                   uint64_t(a.seq_ids[s]));
  const double u_acc = word_to_uniform(ph.w[0]);
  const double u_res = word_to_uniform(ph.w[1]);
  const Dist& dp = sh.dist[0];
  const Dist& dq = sh.dist[1];
  SlotResult res;
  res.tok = -1;
  res.acc = 0;
  res.flags = 0;
  res.ratio = 1.0;
  const bool ok_p = Rp.status == ROW_OK;
  const bool ok_q = !has_q || Rq.status == ROW_OK;
  if (!ok_p || !ok_q) {
    res.acc = has_q ? 0 : 1;
    res.flags |= FLAG_OVERFLOW;
  } else if (!has_q) {
    res.acc = 1;
    bool tie = false;
    res.tok = sample_dist(dp, u_res, &tie);
    if (tie) res.flags |= FLAG_TIE_ICDF;
  } else {
    const int d = a.draft[g];
    res = dp.n <= kWave ? decide_m<1>(dp, dq, d, u_acc, u_res)
                        : decide_m<SEL_CAP / kWave>(dp, dq, d, u_acc, u_res);
    if (dq.gap < NEAR_TIE) res.flags |= FLAG_TIE_TOPP_Q;
  }
  if (ok_p && dp.gap < NEAR_TIE) res.flags |= FLAG_TIE_TOPP_P;

  // Slot record, then the per-sequence ticket.
  unsigned* counters = static_cast<unsigned*>(a.ws);
  unsigned long long* rec = reinterpret_cast<unsigned long long*>(
      static_cast<char*>(a.ws) + ((size_t(a.S) * 4 + 255) / 256) * 256);
  int last = 0;
  if (tid == 0) {
    if (a.slot_accept) a.slot_accept[g] = uint8_t(res.acc);
    if (a.diag) {
      a.diag[size_t(g) * 4 + 0] = float(u_acc);
      a.diag[size_t(g) * 4 + 1] = float(res.ratio);
      a.diag[size_t(g) * 4 + 2] = float(u_res);
      a.diag[size_t(g) * 4 + 3] = float(res.flags);
    }
    // The record is written with a device-coherent (write-through) store and the
    // wait below retires it before the ticket increment; the last workgroup reads
    // records with device-coherent loads. This avoids a full L2 write-back fence.
    __hip_atomic_store(&rec[g],
                       (unsigned long long)(unsigned)res.tok | ((unsigned long long)(unsigned)res.acc << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    const unsigned old = __hip_atomic_fetch_add(&counters[s], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == unsigned(b - 1) ? 1 : 0;
  }
  last = readlane_i(last, 0);
  if (last) {
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
  const int tid = threadIdx.x, wid = tid / kWave;
  const FilterParams fp = make_filter_params(a.sp, V);
  RowLds& R = sh.row[1];
  const RowView<E, VEC> qv(static_cast<const E*>(a.q) + size_t(g) * V, V);
  reset_row(R);
  stream_one(qv, fp, R, sh);
  const int c = R.cnt;
  __syncthreads();
  if (c > CAND_CAP && tid == 0) R.status = ROW_OVERFLOW;
  __syncthreads();
  if (c <= WAVE_SEL_MAX) {
    if (wid == 0) wave_select(R, fp);
  } else if (R.status == ROW_OK) {
    block_select(R, fp, sh);
  }
  __syncthreads();
  if (wid != 0) return;
  int flags = 0, tok = -1;
  if (R.status == ROW_OK) {
    wave_filter(fp, R, sh.dist[1]);
    const Philox4 ph = philox4x64_10(uint64_t(a.pos[s] + i), 1ull, 0ull, 0ull, a.sp.seed,
                                     uint64_t(a.seq_ids[s]));
    bool tie = false;
    tok = sample_dist(sh.dist[1], word_to_uniform(ph.w[0]), &tie);
    if (tie) flags |= FLAG_TIE_ICDF;
    if (sh.dist[1].gap < NEAR_TIE) flags |= FLAG_TIE_TOPP_Q;
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
