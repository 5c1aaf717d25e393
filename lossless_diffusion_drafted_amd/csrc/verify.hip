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
//    other is scanned). Waves lower their issue priority as they progress, so the
//    workgroups sharing a CU end their streams together.
//  * A lower bound of each row's k-th largest logit comes from its first tile and
//    is raised after each of the next tiles: each wave takes the ceil(k/4)-th
//    largest of its 64 running lane maxima (a radix select, one ballot per key
//    bit), so the minimum over the 4 waves has at least k row elements at or above
//    it. For bf16 rows with a positive bound, eight elements are pre-checked with
//    three packed 16-bit max instructions.
//  * A 16-byte chunk that may reach the bound is stored whole in its wave's LDS
//    list (ballot-ranked slots, no atomic), or in a spill area shared by the row's
//    waves once that list is full. After the stream the chunks are expanded against
//    the final bound into the row's candidate list.
//  * After the stream, wave 0 selects and filters the p row while wave 1 does the
//    q row, with no barriers: an MSB-first radix select over the candidates'
//    order-preserving keys (only the bits where they differ) gives the exact
//    k-th largest value; every candidate at or above it forms the tie-inclusive
//    top-k set; softmax, top-p and the renormalised distribution are fp64 on it.
//  * Wave 0 then runs the accept test and the inverse CDF in fp64, writes the
//    slot record with a device-coherent store, and takes a per-sequence ticket;
//    the last workgroup of a sequence runs the prefix scan and resets the ticket.

#include <math.h>

#include <mutex>

#include "common.h"
#include "kernels.h"

namespace uno {
namespace {

constexpr int VT = 256;               // threads per workgroup
constexpr int VW = VT / kWave;        // waves per workgroup
constexpr int UNR = 8;                // 16-byte loads per thread per tile
constexpr int CAND_CAP = 1024;        // candidates kept per row
constexpr int WAVE_CHUNKS = 128;      // 16-byte chunks each wave may flag in its own list
constexpr int SPILL_CHUNKS = 153;     // shared by the waves whose own list is full
constexpr int CHUNK_CAP = VT / 64 * WAVE_CHUNKS + SPILL_CHUNKS;   // chunks a row may flag
constexpr int WAVE_SEL_MAX = 512;     // candidates one wave selects from (8 per lane)
constexpr int SEL_CAP = 256;          // largest filtered support on this path
constexpr int KMAX_FAST = 256;          // largest top-k the stream bound is built for
constexpr double NEAR_TIE = 1e-6;
constexpr int PER_TILE = VT * UNR;    // 16-byte chunks per tile

constexpr int FLAG_TIE_ACCEPT = 1, FLAG_TIE_TOPP_P = 2, FLAG_TIE_TOPP_Q = 4,
              FLAG_TIE_ICDF = 8, FLAG_Q_ZERO = 16, FLAG_RES_ZERO = 32;

enum { ROW_OK = 0, ROW_OVERFLOW = 1 };

typedef short short2_t __attribute__((ext_vector_type(2)));

struct Dist {            // filtered distribution: ascending ids, fp64 probabilities
  int n;
  double gap;            // min |mass above a non-top group - top_p| (inf if top-p off)
  int ids[SEL_CAP];
  double prob[SEL_CAP];
};

struct RowLds {          // per-row state of the selection
  union {
    // During the stream: the flagged chunks (raw 16 bytes and the element index
    // of their first entry); wave w's own list at [w * WAVE_CHUNKS, ...), the
    // shared spill area after the four lists.
    struct {
      uint4 cdata[CHUNK_CAP];
      int cpos[CHUNK_CAP];
    };
    // After the stream: the candidate list and the selection's work arrays.
    struct {
      float cval[CAND_CAP];
      int cidx[CAND_CAP];
      alignas(16) float sval[SEL_CAP];
      alignas(16) int sidx[SEL_CAP];
      double sw[SEL_CAP];
      unsigned hist[256];
    };
  };
  float wthr[VW];        // per-wave published lower bounds
  int wchunk[VW];        // chunks in each wave's own list
  int nspill;            // chunks sent to the spill area (may exceed SPILL_CHUNKS: overflow)
  int cnt;               // candidates kept; > CAND_CAP marks an overflow
  int n;                 // size of the tie-inclusive top-k set
  unsigned kmax;         // largest candidate key
  int status;
};

struct Shared {
  RowLds row[2];         // 0: base row p, 1: draft row q
  Dist dist[2];
  unsigned red_u[VW][3];
  unsigned ures[2];
  double u[2];           // the slot's u_acc, u_res (drawn by wave 2 during the selection)
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
  static constexpr int KEY_BITS = 16;      // significant bits of an element's order key
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
  static constexpr int KEY_BITS = 32;
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
  int nchunk;       // chunks in this wave's own list (wave-uniform)
};

// The c-th largest of the wave's 64 lane values: an MSB-first radix select over
// the top `bits` bits of the order keys, one ballot per bit (no LDS). Exact for
// bf16 values with bits = 16 and for any float with bits = 32. NaN lanes count
// as -inf.
__device__ __forceinline__ float wave_cth_largest(float m, int c, int bits) {
  const int drop = 32 - bits;
  const uint32_t key = float_key(m == m ? m : -INFINITY) >> drop;
  uint32_t prefix = 0u, decided = 0u;
  int need = c;
  for (int b = bits - 1; b >= 0; --b) {
    const uint32_t bit = 1u << b;
    const bool one = ((key ^ prefix) & decided) == 0u && (key & bit) != 0u;
    const int n1 = __popcll(__ballot(one));
    if (n1 >= need) prefix |= bit;
    else need -= n1;
    decided |= bit;
  }
  // Below zero the dropped key bits are ones (the key of a negative float is
  // its complement), so they are restored as ones.
  const uint32_t low = ((prefix >> (bits - 1)) & 1u) ? 0u : ((1u << drop) - 1u);
  return key_float((prefix << drop) | low);
}

template <typename E, bool VEC>
__device__ __forceinline__ void process_tile(const RowView<E, VEC>& rv, RowLds& R, const uint4 (&r)[UNR],
                                             int t, RowScan& sc) {
  using EL = Elem<E>;
  constexpr int VN = EL::VN;
  const int tid = threadIdx.x, wid = tid / kWave;
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
    // A chunk that may hold an element at or above the bound is kept whole; its
    // elements are tested against the final bound once the row is read. Slots
    // come from the ballot ranks in the wave's own list (a wave-uniform count, no
    // atomic), or, once that list is full, from the shared spill area.
    const unsigned long long bal = __ballot(maybe);
    if (bal) {
      const int n = __popcll(bal), rank = ballot_rank(bal);
      int pos;
      if (sc.nchunk + n <= WAVE_CHUNKS) {
        pos = wid * WAVE_CHUNKS + sc.nchunk + rank;
        sc.nchunk += n;
      } else {
        int base = 0;
        if ((tid & (kWave - 1)) == 0) base = atomicAdd(&R.nspill, n);
        const int sp = readlane_i(base, 0) + rank;
        pos = sp < SPILL_CHUNKS ? VW * WAVE_CHUNKS + sp : CHUNK_CAP;
      }
      if (maybe && pos < CHUNK_CAP) {
        R.cdata[pos] = r[u];
        R.cpos[pos] = e0;
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
__device__ __forceinline__ float refresh_bound(RowLds& R, const RowScan& sc, int c, int bits) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const float tw = wave_cth_largest(scan_lane_max(sc), c, bits);
  if (lane == 0) R.wthr[wid] = tw;
  float t = R.wthr[0];
#pragma unroll
  for (int i = 1; i < VW; ++i) t = fminf(t, R.wthr[i]);
  return fmaxf(t, sc.thr);
}

// First-tile lane maxima -> initial bound (published; caller synchronises).
template <typename E, bool VEC>
__device__ __forceinline__ void init_bound(const RowView<E, VEC>& rv, RowLds& R, const uint4 (&r)[UNR],
                                           int c, RowScan& sc) {
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
  const float tw = wave_cth_largest(sc.lmax, c, EL::KEY_BITS);
  if (lane == 0) R.wthr[wid] = tw;
}

__device__ __forceinline__ float read_bound(const RowLds& R) {
  float t = R.wthr[0];
#pragma unroll
  for (int i = 1; i < VW; ++i) t = fminf(t, R.wthr[i]);
  return t;
}

__device__ __forceinline__ void reset_row(RowLds& R) {
  if (threadIdx.x == 0) { R.nspill = 0; R.cnt = 0; R.status = ROW_OK; R.n = 0; }
}

// This wave's lane-maximum bound after the whole row and its chunk count
// (published; caller synchronises). The bound is -inf when the stream runs
// unbounded.
__device__ __forceinline__ void publish_row_end(RowLds& R, const RowScan& sc, bool bounded, int c, int bits) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const float tw = bounded ? wave_cth_largest(scan_lane_max(sc), c, bits) : -INFINITY;
  if (lane == 0) {
    R.wthr[wid] = tw;
    R.wchunk[wid] = sc.nchunk;
  }
}

// Chunks this thread holds of the row's list: entry m * VT + threadIdx.x.
constexpr int CHUNKS_PER_THREAD = (CHUNK_CAP + VT - 1) / VT;
struct HeldChunks {
  uint4 d[CHUNKS_PER_THREAD];
  int pos[CHUNKS_PER_THREAD];
  int n;                // valid entries of the list
  bool overflow;
};

// Entry e of the row's list in the order: wave 0's list, ..., wave 3's, spill.
__device__ __forceinline__ void take_chunks(const RowLds& R, HeldChunks& h) {
  int start[VW + 1], off[VW + 1];
  int total = 0;
#pragma unroll
  for (int w = 0; w < VW; ++w) {
    start[w] = total;
    off[w] = w * WAVE_CHUNKS;
    total += R.wchunk[w];
  }
  const int ns = R.nspill;
  start[VW] = total;
  off[VW] = VW * WAVE_CHUNKS;
  h.overflow = ns > SPILL_CHUNKS;
  total += min(ns, SPILL_CHUNKS);
  h.n = total;
#pragma unroll
  for (int m = 0; m < CHUNKS_PER_THREAD; ++m) {
    const int e = m * VT + int(threadIdx.x);
    if (e < total) {
      int seg = 0;
#pragma unroll
      for (int w = 1; w <= VW; ++w) seg = e >= start[w] ? w : seg;
      int src = e - start[0] + off[0];
#pragma unroll
      for (int w = 1; w <= VW; ++w) src = seg == w ? e - start[w] + off[w] : src;
      h.d[m] = R.cdata[src];
      h.pos[m] = R.cpos[src];
    }
  }
}

// The held chunks' elements at or above `thr` become the row's candidate list
// (cval/cidx, count in cnt). An overflowed chunk list makes cnt exceed CAND_CAP,
// which sends the row to the full-row path.
template <typename E>
__device__ __forceinline__ void expand_chunks(RowLds& R, const HeldChunks& h, float thr, int V) {
  using EL = Elem<E>;
  constexpr int VN = EL::VN;
  int cnt = 0;
#pragma unroll
  for (int m = 0; m < CHUNKS_PER_THREAD; ++m) {
    if (m * VT + int(threadIdx.x) < h.n) {
      float x[VN];
      EL::unpack(h.d[m], x);
#pragma unroll
      for (int j = 0; j < VN; ++j) cnt += (x[j] >= thr && h.pos[m] + j < V) ? 1 : 0;
    }
  }
  int p = cnt ? atomicAdd(&R.cnt, cnt) : 0;
#pragma unroll
  for (int m = 0; m < CHUNKS_PER_THREAD; ++m) {
    if (m * VT + int(threadIdx.x) < h.n) {
      float x[VN];
      EL::unpack(h.d[m], x);
#pragma unroll
      for (int j = 0; j < VN; ++j) {
        if (x[j] >= thr && h.pos[m] + j < V) {
          if (p < CAND_CAP) { R.cval[p] = x[j]; R.cidx[p] = h.pos[m] + j; }
          ++p;
        }
      }
    }
  }
  if (threadIdx.x == 0 && h.overflow) atomicAdd(&R.cnt, CAND_CAP + 1);
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
  RowScan sc{-INFINITY, -INFINITY, -32768, 0};
  constexpr int KB = Elem<E>::KEY_BITS;
  if (bounded) init_bound(rv, R, A, c, sc);
  __syncthreads();
  if (bounded) sc.thr = read_bound(R);
  if (VEC) {
    // The bound rises fastest early on, when each tile adds many lane maxima:
    // it is refreshed after each of the first eight tiles.
    for (int t = 0; t < rv.ntiles; t += 2) {
      process_tile(rv, R, A, t, sc);
      rv.load_tile(A, t + 2);
      if (bounded && t < 8) sc.thr = refresh_bound(R, sc, c, KB);
      if (t + 1 < rv.ntiles) process_tile(rv, R, B, t + 1, sc);
      rv.load_tile(B, t + 3);
      if (bounded && t < 8) sc.thr = refresh_bound(R, sc, c, KB);
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
  publish_row_end(R, sc, bounded, c, KB);
  HeldChunks h;
  __syncthreads();                    // every chunk flagged; bounds and counts published
  take_chunks(R, h);
  __syncthreads();                    // the list read before its arrays are reused
  expand_chunks<E>(R, h, bounded ? read_bound(R) : -INFINITY, rv.V);
  __syncthreads();
}

// Issue priority of this wave (0..3). Waves further along a row step down so
// that the workgroups sharing a CU finish their streams together instead of in
// start order.
__device__ __forceinline__ void set_wave_prio(int p) {
  switch (p) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
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
  RowScan sp{-INFINITY, -INFINITY, -32768, 0}, sq{-INFINITY, -INFINITY, -32768, 0};
  constexpr int KB = Elem<E>::KEY_BITS;
  if (bounded) {
    init_bound(pv, Rp, A, c, sp);
    init_bound(qv, Rq, B, c, sq);
  }
  __syncthreads();
  if (bounded) {
    sp.thr = read_bound(Rp);
    sq.thr = read_bound(Rq);
  }
  int prio = -1;
  for (int t = 0; t < pv.ntiles; ++t) {
    const int want = 3 - (t * 4) / pv.ntiles;
    if (want != prio) { set_wave_prio(want); prio = want; }
    process_tile(pv, Rp, A, t, sp);
    pv.load_tile(A, t + 1);
    process_tile(qv, Rq, B, t, sq);
    qv.load_tile(B, t + 1);
    // The bound rises fastest early on, when each tile adds many lane maxima:
    // refreshing it after each of the first 8 tiles keeps fewer candidates.
    if (bounded && t < 8) {
      sp.thr = refresh_bound(Rp, sp, c, KB);
      sq.thr = refresh_bound(Rq, sq, c, KB);
    }
  }
  set_wave_prio(0);
  publish_row_end(Rp, sp, bounded, c, KB);
  publish_row_end(Rq, sq, bounded, c, KB);
  __syncthreads();                    // every chunk flagged; bounds and counts published
  {
    HeldChunks h;
    take_chunks(Rp, h);
    __syncthreads();                  // p's list read before its arrays are reused
    expand_chunks<E>(Rp, h, bounded ? read_bound(Rp) : -INFINITY, pv.V);
  }
  {
    HeldChunks h;
    take_chunks(Rq, h);
    __syncthreads();                  // the same for q
    expand_chunks<E>(Rq, h, bounded ? read_bound(Rq) : -INFINITY, qv.V);
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
// ================================================================================
// Full-row path: used when the settings make the filtered support large (top-k
// off or k > KMAX_SINGLE_PASS over more than SEL_CAP logits) and as the fallback
// of a slot whose single-pass selection overflows. The workgroup streams the whole
// row several times (from L2 after the first pass) and never holds the support:
//  * pass 1: row maximum (lowest id at it) and the top digit histogram of the
//    order-preserving keys; further count passes give the exact tie-inclusive
//    k-th largest key (MSB-first radix select, 8 bits per pass);
//  * mass passes: the tie-grouped top-p cutoff by the same MSB-first search on
//    histograms of softmax mass (the mass strictly above a bucket decides whether
//    it is kept; the bucket where the running mass reaches top_p is refined).
//    Masses are summed as 2^-40 fixed-point integers, so the order of the LDS
//    atomics cannot change the result;
//  * the decision needs p~(d) and q~(d) (one element each) and, on a rejection or
//    at slot 0, one sum pass and one ordered scan pass over the residual or p~
//    (inverse CDF in ascending id order, fp64 block scans).
// ================================================================================
constexpr int KMAX_SINGLE_PASS = 128;      // larger top-k goes to the full-row path
constexpr double FIXED_ONE = 1099511627776.0;   // 2^40

struct FullLds {
  unsigned long long hm[256];   // fixed-point mass per digit
  unsigned hc[256];             // element count per digit
  double dred[VW];
  float fred[VW];
  int ired[VW];
  unsigned uv[4];
  unsigned long long qv[4];
  double dv[4];
  int tok;
};

struct RowSum {
  float m;            // row maximum
  int argmax;         // lowest id at the maximum
  unsigned tau;       // kept iff the element's key >= tau (row key space)
  double Zt;          // kept mass, sum over kept of exp((z - m) / T) (fixed point rounded)
  double gap;         // top-p near-tie gap (infinity if none)
  float c2hi, c2lo;   // log2(e) / T split in two floats
};

template <typename E> struct KeyBits { static constexpr int value = 32; };
template <> struct KeyBits<uint16_t> { static constexpr int value = 16; };

// Order-preserving key in the row's key space (bf16 rows need only the top 16 bits).
template <typename E>
__device__ __forceinline__ unsigned row_key(float x) {
  return float_key(x) >> (32 - KeyBits<E>::value);
}

// exp((z - m) / T) in fp32 with the scaling done in two parts (the fp32 rounding
// of log2(e)/T would otherwise scale every exponent).
__device__ __forceinline__ float mass32(float z, const RowSum& rs) {
  const float d = z - rs.m;
  return __builtin_amdgcn_exp2f(fmaf(d, rs.c2hi, d * rs.c2lo));
}

__device__ __forceinline__ unsigned long long to_fixed(float w) {
  return (unsigned long long)(double(w) * FIXED_ONE + 0.5);
}

// One 16-byte chunk of a row (values past the row read as zeros on the vector
// path and as -inf on the scalar path; callers mask by index).
template <typename E, bool VEC>
__device__ __forceinline__ uint4 load_chunk(const RowView<E, VEC>& rv, int c) {
  if constexpr (VEC) return buffer_load16(rv.rsrc, uint32_t(c) * 16u, 0u);
  else return c < rv.nchunks ? Elem<E>::load_partial(rv.row, c * Elem<E>::VN, rv.V) : Elem<E>::neg_inf();
}

// Calls f(c, xp, xq) once per 16-byte chunk c of the rows (every thread; chunks
// ascend across the workgroup in groups of VT; values past the row are -inf).
// FULL_UNR chunks per row are in flight. f returns true to stop early (uniform
// across the workgroup).
constexpr int FULL_UNR = 4;
template <typename E, bool VEC, typename F>
__device__ __forceinline__ void stream_rows(const RowView<E, VEC>& pv, const RowView<E, VEC>& qv, bool two, F f) {
  using EL = Elem<E>;
  constexpr int VN = EL::VN;
  const int ngroups = (pv.nchunks + VT - 1) / VT;
  for (int g0 = 0; g0 < ngroups; g0 += FULL_UNR) {
    uint4 rp[FULL_UNR], rq[FULL_UNR];
#pragma unroll
    for (int u = 0; u < FULL_UNR; ++u) {
      const int c = (g0 + u) * VT + int(threadIdx.x);
      rp[u] = load_chunk(pv, c);
      if (two) rq[u] = load_chunk(qv, c);
    }
#pragma unroll
    for (int u = 0; u < FULL_UNR; ++u) {
      if (g0 + u >= ngroups) break;
      const int c = (g0 + u) * VT + int(threadIdx.x);
      float xp[VN], xq[VN];
      EL::unpack(rp[u], xp);
      if (two) EL::unpack(rq[u], xq);
#pragma unroll
      for (int j = 0; j < VN; ++j) {
        if (c * VN + j >= pv.V) { xp[j] = -INFINITY; xq[j] = -INFINITY; }
        if (!two) xq[j] = -INFINITY;
      }
      if (f(c, xp, xq)) return;
    }
  }
}

__device__ __forceinline__ double block_sum_d(double v, FullLds& fs) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) fs.dred[wid] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < VW; ++w) t += fs.dred[w];
  return t;
}

// Row summary (all threads return the same value).
template <typename E, bool VEC>
__device__ __forceinline__ RowSum summarize_row(const RowView<E, VEC>& rv, const FilterParams& fp, FullLds& fs) {
  constexpr int KB = KeyBits<E>::value;
  constexpr int LEVELS = KB / 8;
  constexpr int VN = Elem<E>::VN;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int V = rv.V;
  const bool kon = fp.k_eff < V;
  RowSum rs;
  const double c2 = 1.4426950408889634 / fp.T;
  rs.c2hi = float(c2);
  rs.c2lo = float(c2 - double(rs.c2hi));
  rs.gap = INFINITY;

  // pass 1: maximum, lowest id at it, top-digit counts
  fs.hc[tid] = 0u;
  __syncthreads();
  float lm = -INFINITY;
  int li = 0x7fffffff;
  stream_rows(rv, rv, false, [&](int c, const float (&x)[VN], const float (&)[VN]) {
#pragma unroll
    for (int j = 0; j < VN; ++j) {
      const int e = c * VN + j;
      if (e < V) {
        if (x[j] > lm || (x[j] == lm && e < li)) { lm = x[j]; li = e; }
        if (kon) atomicAdd(&fs.hc[row_key<E>(x[j]) >> (KB - 8)], 1u);
      }
    }
    return false;
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(lm, o, kWave);
    const int oi = __shfl_xor(li, o, kWave);
    if (om > lm || (om == lm && oi < li)) { lm = om; li = oi; }
  }
  if (lane == 0) { fs.fred[wid] = lm; fs.ired[wid] = li; }
  __syncthreads();
  lm = fs.fred[0];
  li = fs.ired[0];
#pragma unroll
  for (int w = 1; w < VW; ++w)
    if (fs.fred[w] > lm || (fs.fred[w] == lm && fs.ired[w] < li)) { lm = fs.fred[w]; li = fs.ired[w]; }
  rs.m = lm;
  rs.argmax = li;
  if (fp.greedy) {
    rs.tau = row_key<E>(lm);
    rs.Zt = FIXED_ONE;
    return rs;
  }

  // exact tie-inclusive k-th largest key
  unsigned kth = 0u;
  if (kon) {
    unsigned prefix = 0u, remaining = unsigned(fp.k_eff);
    for (int level = 0; level < LEVELS; ++level) {
      const int shift = KB - 8 * (level + 1);
      if (level > 0) {
        __syncthreads();
        fs.hc[tid] = 0u;
        __syncthreads();
        const unsigned pre = prefix >> (shift + 8);
        stream_rows(rv, rv, false, [&](int c, const float (&x)[VN], const float (&)[VN]) {
#pragma unroll
          for (int j = 0; j < VN; ++j) {
            const unsigned key = row_key<E>(x[j]);
            if (c * VN + j < V && (key >> (shift + 8)) == pre) atomicAdd(&fs.hc[(key >> shift) & 255u], 1u);
          }
          return false;
        });
      }
      __syncthreads();
      if (tid == 0) {
        unsigned cum = 0u, digit = 0u;
        for (int d = 255; d >= 0; --d) {
          if (cum + fs.hc[d] >= remaining) { digit = unsigned(d); break; }
          cum += fs.hc[d];
        }
        fs.uv[0] = prefix | (digit << shift);
        fs.uv[1] = remaining - cum;
      }
      __syncthreads();
      prefix = fs.uv[0];
      remaining = fs.uv[1];
    }
    kth = prefix;
  }

  // mass passes: total mass of the top-k set, then the top-p cutoff
  unsigned prefix = 0u;
  unsigned long long above = 0ull, zk = 0ull, hcut = 0ull;
  unsigned n_above = 0u, nk = 0u, ncut = 0u;
  const int mlevels = fp.topp_on ? LEVELS : 1;
  for (int level = 0; level < mlevels; ++level) {
    const int shift = KB - 8 * (level + 1);
    __syncthreads();
    fs.hm[tid] = 0ull;
    fs.hc[tid] = 0u;
    __syncthreads();
    const unsigned pre = level == 0 ? 0u : prefix >> (shift + 8);
    stream_rows(rv, rv, false, [&](int c, const float (&x)[VN], const float (&)[VN]) {
#pragma unroll
      for (int j = 0; j < VN; ++j) {
        const unsigned key = row_key<E>(x[j]);
        if (c * VN + j < V && key >= kth && (level == 0 || (key >> (shift + 8)) == pre)) {
          const unsigned dgt = (key >> shift) & 255u;
          atomicAdd(&fs.hm[dgt], to_fixed(mass32(x[j], rs)));
          atomicAdd(&fs.hc[dgt], 1u);
        }
      }
      return false;
    });
    __syncthreads();
    if (tid == 0) {
      if (level == 0) {
        unsigned long long t = 0ull;
        unsigned n = 0u;
        for (int d = 0; d < 256; ++d) { t += fs.hm[d]; n += fs.hc[d]; }
        fs.qv[0] = t;
        fs.uv[0] = n;
      }
      if (fp.topp_on) {
        const double thr = fp.top_p * double(level == 0 ? fs.qv[0] : zk);
        unsigned long long run = above;
        unsigned nrun = n_above;
        int cand = -1;
        unsigned long long a_c = 0ull;
        unsigned n_c = 0u;
        for (int d = 255; d >= 0; --d) {
          if (fs.hc[d] > 0u) {
            if (double(run) < thr) { cand = d; a_c = run; n_c = nrun; }
            else break;
          }
          run += fs.hm[d];
          nrun += fs.hc[d];
        }
        if (cand < 0) cand = 0;                  // unreachable: the top bucket always qualifies
        fs.uv[1] = prefix | (unsigned(cand) << shift);
        fs.qv[1] = a_c;
        fs.uv[2] = n_c;
        fs.qv[2] = fs.hm[cand];
        fs.uv[3] = fs.hc[cand];
      }
    }
    __syncthreads();
    if (level == 0) { zk = fs.qv[0]; nk = fs.uv[0]; }
    if (fp.topp_on) {
      prefix = fs.uv[1];
      above = fs.qv[1];
      n_above = fs.uv[2];
      hcut = fs.qv[2];
      ncut = fs.uv[3];
    }
  }
  if (fp.topp_on) {
    rs.tau = prefix;
    rs.Zt = double(above + hcut);
    const double Zk = double(zk);
    if (above > 0ull) rs.gap = fabs(double(above) / Zk - fp.top_p);
    if (n_above + ncut < nk) rs.gap = fmin(rs.gap, fabs(double(above + hcut) / Zk - fp.top_p));
  } else {
    rs.tau = kth;
    rs.Zt = double(zk);
  }
  return rs;
}

// Filtered probability of one element from its logit (fp64 weight).
template <typename E>
__device__ __forceinline__ double full_prob(const RowSum& rs, const FilterParams& fp, float z, int id) {
  if (fp.greedy) return id == rs.argmax ? 1.0 : 0.0;
  if (!(row_key<E>(z) >= rs.tau) || !(z > -INFINITY)) return 0.0;
  return exp((double(z) - double(rs.m)) / fp.T) * FIXED_ONE / rs.Zt;
}

// Per-element weight in the scan passes (fp32 mass, consistent with Zt).
template <typename E>
__device__ __forceinline__ double full_weight(const RowSum& rs, const FilterParams& fp, float z, int id) {
  if (fp.greedy) return id == rs.argmax ? 1.0 : 0.0;
  if (!(row_key<E>(z) >= rs.tau) || !(z > -INFINITY)) return 0.0;
  return double(to_fixed(mass32(z, rs))) / rs.Zt;
}

template <typename E, bool VEC>
__device__ __forceinline__ float load_elem(const RowView<E, VEC>& rv, int e) {
  if constexpr (sizeof(E) == 2) return bf16_to_f32(rv.row[e]);
  else return rv.row[e];
}

// Weight of element e of the residual (mode 1: max(0, p~ - q~)) or of p~ / q~ alone
// (mode 0: the first row's filtered distribution).
template <typename E>
__device__ __forceinline__ double scan_weight(int mode, const RowSum& r1, const RowSum& r2, const FilterParams& fp,
                                              float x1, float x2, int e) {
  const double a = full_weight<E>(r1, fp, x1, e);
  if (mode == 0) return a;
  return fmax(0.0, a - full_weight<E>(r2, fp, x2, e));
}

// Inverse CDF over ascending ids: the first e whose running weight sum exceeds
// u * W (W = total weight). Sets *tie when u*W lies within 1e-6*W of a boundary
// next to the drawn element, and *wsum to W.
template <typename E, bool VEC>
__device__ __forceinline__ int full_icdf(const RowView<E, VEC>& v1, const RowView<E, VEC>& v2, int mode, const RowSum& r1,
                         const RowSum& r2, const FilterParams& fp, double u, FullLds& fs, bool* tie, double* wsum) {
  constexpr int VN = Elem<E>::VN;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const bool two = mode == 1;
  // total weight, positive-weight count and the last positive id
  double lw = 0.0;
  int lastpos = -1;
  stream_rows(v1, v2, two, [&](int c, const float (&x1)[VN], const float (&x2)[VN]) {
#pragma unroll
    for (int j = 0; j < VN; ++j) {
      const int e = c * VN + j;
      if (e < v1.V) {
        const double w = scan_weight<E>(mode, r1, r2, fp, x1[j], x2[j], e);
        lw += w;
        if (w > 0.0) lastpos = e;
      }
    }
    return false;
  });
  const double W = block_sum_d(lw, fs);
  lastpos = wave_max(lastpos);
  __syncthreads();
  if (lane == 0) fs.ired[wid] = lastpos;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < VW; ++w) lastpos = max(lastpos, fs.ired[w]);
  *wsum = W;
  const double t = u * W;
  if (tid == 0) { fs.tok = -1; fs.dv[0] = 0.0; fs.dv[1] = 0.0; }
  __syncthreads();
  double run = 0.0;                            // sum of all earlier sub-tiles (same in every thread)
  stream_rows(v1, v2, two, [&](int c, const float (&x1)[VN], const float (&x2)[VN]) {
    double w[VN];
    double ls = 0.0;
#pragma unroll
    for (int j = 0; j < VN; ++j) {
      const int e = c * VN + j;
      w[j] = e < v1.V ? scan_weight<E>(mode, r1, r2, fp, x1[j], x2[j], e) : 0.0;
      ls += w[j];
    }
    // block inclusive scan of the chunk sums; the crossing chunk is the lowest
    // thread whose inclusive bound exceeds t (unique even under rounding)
    const double incl = wave_inclusive_scan(ls);
    __syncthreads();
    if (lane == kWave - 1) fs.dred[wid] = incl;
    if (tid == 0) fs.ired[0] = 0x7fffffff;
    __syncthreads();
    double woff = 0.0, tot = 0.0;
#pragma unroll
    for (int q = 0; q < VW; ++q) {
      if (q < wid) woff += fs.dred[q];
      tot += fs.dred[q];
    }
    const double bound = run + woff + incl;
    const double up = __shfl_up(bound, 1, kWave);
    const double prev = lane > 0 ? up : run + woff;
    if (bound > t) atomicMin(&fs.ired[0], tid);
    __syncthreads();
    if (tid == fs.ired[0]) {
      double cum = prev;
      int pick = -1, lastp = -1;
      double lo = prev, hi = prev;
#pragma unroll
      for (int j = 0; j < VN; ++j) {
        const double nxt = cum + w[j];
        if (w[j] > 0.0) {
          lastp = j;
          if (pick < 0 && nxt > t) { pick = j; lo = cum; hi = nxt; }
        }
        cum = nxt;
      }
      if (pick < 0) { pick = lastp < 0 ? 0 : lastp; lo = prev; hi = bound; }
      fs.tok = c * VN + pick;
      fs.dv[0] = lo;
      fs.dv[1] = hi;
    }
    __syncthreads();
    run += tot;
    return fs.tok >= 0;
  });
  __syncthreads();
  int tok = fs.tok;
  bool tnear = false;
  if (tok < 0) {
    tok = max(lastpos, 0);                     // rounding left u*W at the very end
  } else {
    const double lo = fs.dv[0], hi = fs.dv[1];
    if (lo > 0.0 && fabs(t - lo) < NEAR_TIE * W) tnear = true;
    if (tok != lastpos && fabs(hi - t) < NEAR_TIE * W) tnear = true;
  }
  *tie = tnear;
  return tok;
}

// One slot by the full-row path (all threads of the workgroup). For a draft-only
// call pass has_q = false with the draft row as `pv` and the draw in u_res.
template <typename E, bool VEC>
__device__ __forceinline__ SlotResult full_slot(const RowView<E, VEC>& pv, const RowView<E, VEC>& qv, bool has_q,
                                const FilterParams& fp, int d, double u_acc, double u_res, FullLds& fs,
                                int* topp_flags) {
  SlotResult res;
  res.flags = 0;
  res.ratio = 1.0;
  const RowSum rp = summarize_row(pv, fp, fs);
  *topp_flags = rp.gap < NEAR_TIE ? FLAG_TIE_TOPP_P : 0;
  bool tie = false;
  double W = 0.0;
  if (!has_q) {
    res.acc = 1;
    res.tok = full_icdf(pv, pv, 0, rp, rp, fp, u_res, fs, &tie, &W);
    if (tie) res.flags |= FLAG_TIE_ICDF;
    return res;
  }
  const RowSum rq = summarize_row(qv, fp, fs);
  if (rq.gap < NEAR_TIE) *topp_flags |= FLAG_TIE_TOPP_Q;
  const bool din = d >= 0 && d < pv.V;
  const double pd = din ? full_prob<E>(rp, fp, load_elem(pv, d), d) : 0.0;
  const double qd = din ? full_prob<E>(rq, fp, load_elem(qv, d), d) : 0.0;
  if (qd == 0.0) {
    res.acc = 0;
    res.ratio = 0.0;
    res.flags |= FLAG_Q_ZERO;
  } else {
    res.ratio = pd / qd;
    res.acc = u_acc < res.ratio ? 1 : 0;
    if (fabs(u_acc - res.ratio) < NEAR_TIE) res.flags |= FLAG_TIE_ACCEPT;
  }
  if (res.acc) {
    res.tok = d;
    return res;
  }
  res.tok = full_icdf(pv, qv, 1, rp, rq, fp, u_res, fs, &tie, &W);
  if (W == 0.0) {                               // zero residual: draw from p~
    res.flags |= FLAG_RES_ZERO;
    res.tok = full_icdf(pv, pv, 0, rp, rp, fp, u_res, fs, &tie, &W);
  }
  if (tie) res.flags |= FLAG_TIE_ICDF;
  return res;
}

template <typename E, bool VEC>
// Four workgroups per CU keep every slot of a 64 x 16 block resident at once.
__global__ __launch_bounds__(VT) __attribute__((amdgpu_waves_per_eu(4))) void verify_kernel(VerifyArgs a) {
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
  // Settings whose filtered support can be large go straight to the full-row
  // path; otherwise the single-pass path runs and falls back to the full-row path
  // for a slot whose candidate list or top-k set overflows.
  bool use_full = fp.k_eff > KMAX_SINGLE_PASS && V > SEL_CAP;
  bool drawn = false;                 // sh.u holds the slot's uniforms
  if (!use_full) {
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
      drawn = true;
      if (wid == 0) wave_select(Rp, fp);
      if (wid == 1 && has_q) wave_select(Rq, fp);
      if (wid == 2) {
        // The slot's uniforms, drawn by an otherwise idle wave off the critical path.
        const Philox4 ph = philox4x64_10(uint64_t(a.pos[s] + i), 0ull, 0ull, 0ull, a.sp.seed,
                                         uint64_t(a.seq_ids[s]));
        if ((tid & (kWave - 1)) == 0) {
          sh.u[0] = word_to_uniform(ph.w[0]);
          sh.u[1] = word_to_uniform(ph.w[1]);
        }
      }
    } else {
      if (Rp.status == ROW_OK) block_select(Rp, fp, sh);
      if (has_q && Rq.status == ROW_OK) block_select(Rq, fp, sh);
    }
    __syncthreads();
    if (wid == 0 && Rp.status == ROW_OK) wave_filter(fp, Rp, sh.dist[0]);
    if (wid == 1 && has_q && Rq.status == ROW_OK) wave_filter(fp, Rq, sh.dist[1]);
    __syncthreads();
    use_full = Rp.status != ROW_OK || (has_q && Rq.status != ROW_OK);
  }

  double u_acc, u_res;
  if (drawn) {
    u_acc = sh.u[0];
    u_res = sh.u[1];
  } else {
    const Philox4 ph = philox4x64_10(uint64_t(a.pos[s] + i), 0ull, 0ull, 0ull, a.sp.seed,
                                     uint64_t(a.seq_ids[s]));
    u_acc = word_to_uniform(ph.w[0]);
    u_res = word_to_uniform(ph.w[1]);
  }
  SlotResult res;
  if (use_full) {
    __shared__ FullLds fsh;
    int topp = 0;
    res = full_slot(pv, qv, has_q, fp, has_q ? a.draft[g] : -1, u_acc, u_res, fsh, &topp);
    res.flags |= topp;
    if (wid != 0) return;
  } else {
    if (wid != 0) return;             // wave 0 finishes the slot alone
    const Dist& dp = sh.dist[0];
    const Dist& dq = sh.dist[1];
    if (!has_q) {
      res.acc = 1;
      res.flags = 0;
      res.ratio = 1.0;
      bool tie = false;
      res.tok = sample_dist(dp, u_res, &tie);
      if (tie) res.flags |= FLAG_TIE_ICDF;
    } else {
      const int d = a.draft[g];
      res = dp.n <= kWave ? decide_m<1>(dp, dq, d, u_acc, u_res)
                          : decide_m<SEL_CAP / kWave>(dp, dq, d, u_acc, u_res);
      if (dq.gap < NEAR_TIE) res.flags |= FLAG_TIE_TOPP_Q;
    }
    if (dp.gap < NEAR_TIE) res.flags |= FLAG_TIE_TOPP_P;
  }

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
    if (tid < b) {
      // Records are cleared once read, so the whole workspace is zero again at
      // the end of the call (a later call may lay it out differently).
      r = __hip_atomic_load(&rec[size_t(s) * b + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&rec[size_t(s) * b + tid], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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
  const Philox4 ph = philox4x64_10(uint64_t(a.pos[s] + i), 1ull, 0ull, 0ull, a.sp.seed,
                                   uint64_t(a.seq_ids[s]));
  const double u = word_to_uniform(ph.w[0]);
  bool use_full = fp.k_eff > KMAX_SINGLE_PASS && V > SEL_CAP;
  if (!use_full) {
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
    use_full = R.status != ROW_OK;
  }
  int flags = 0, tok = -1;
  if (use_full) {
    // the draft row's filtered distribution, drawn like an AR slot
    __shared__ FullLds fsh;
    int topp = 0;
    const SlotResult r = full_slot(qv, qv, false, fp, -1, 0.0, u, fsh, &topp);
    tok = r.tok;
    flags = (r.flags & FLAG_TIE_ICDF) | ((topp & FLAG_TIE_TOPP_P) ? FLAG_TIE_TOPP_Q : 0);
    if (wid != 0) return;
  } else {
    if (wid != 0) return;
    wave_filter(fp, R, sh.dist[1]);
    bool tie = false;
    tok = sample_dist(sh.dist[1], u, &tie);
    if (tie) flags |= FLAG_TIE_ICDF;
    if (sh.dist[1].gap < NEAR_TIE) flags |= FLAG_TIE_TOPP_Q;
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


// ---------------------------------------------------------------------------
// Library-owned scratch of the verifier, for callers that cannot allocate
// (uno_verify_block_noalloc). It holds the per-sequence tickets and slot records
// that a caller workspace holds otherwise, laid out the same way. Each GPU has its
// own copy of the array; host code reaches it only through the device address
// hipGetSymbolAddress returns for the current device, never through its name.
namespace {
constexpr size_t kVerifyScratchBytes = 1310720;   // 256 KiB of tickets + 1 MiB of slot records
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kVerifyScratchBytes];
}  // namespace

size_t verify_scratch_bytes() { return kVerifyScratchBytes; }

hipError_t verify_scratch(void** out, hipStream_t stream) {
  static std::mutex mu;
  static void* ptrs[kScratchDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // Device globals start zeroed; clear the array once more on the first caller's
    // stream so that its first call is ordered after a clear it can see. Every
    // verify call leaves the part it used zero again.
    e = launch_zero(p, kVerifyScratchBytes, stream);
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace uno
