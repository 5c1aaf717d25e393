// Row-gated LoRA linear on gfx950 matrix cores ("Uno Qwen3-8B" model card and
// "LoopUno", "Setup / Recipe": a LoRA adapter whose update is switched on only
// for the rows of the block being denoised; seed/verify rows see the frozen
// weights).
//
//   Y = X W^T + s * diag(mask) (X A^T) B^T,   X [M,K], W [N,K], A [r,K], B [N,r].
//
// Two phases:
//  1. LoRA-down T = bf16(s * X A^T): a skinny GEMM (N = r), one workgroup per
//     32 x 32 tile of T over the whole reduction (fixed sum order).
//  2. The main GEMM over the extended reduction [X | T] [W | B]^T: the delta is
//     r more reduction steps after the K steps, in the same accumulators. The row
//     mask is applied when T's tiles are staged into LDS: rows with mask 0 are
//     loaded out of range, so the buffer unit writes zeros. Those rows add exact
//     zeros and equal the plain X W^T bit for bit.
//
// Main loop: an NS-stage ring of LDS tiles filled by buffer loads that write LDS
// directly (no staging registers), one counted vmcnt wait and one barrier per
// reduction tile. LDS rows are XOR-swizzled in 16-byte chunks so the 16-byte
// fragment reads of 16 consecutive rows hit distinct banks. Each wave owns a
// (BM/WM) x (BN/WN) block of 32 x 32 v_mfma_f32_32x32x16_bf16 tiles. The output
// is staged through LDS and written with 16-byte stores.

#include "../../include/uno.h"
#include "common.h"
#include "kernels.h"

namespace uno {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset past any range: reads 0

template <int BM_, int BN_, int BK_, int WM_, int WN_, int NS_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, NS = NS_;
  static constexpr int NW = WM * WN;
  static constexpr int THREADS = NW * kWave;
  static constexpr int CPR = BK / 8;                 // 16-byte chunks per LDS row
  static constexpr int RS = 16 / CPR;                // rows per 256-byte bank window
  static constexpr int WTM = BM / WM, WTN = BN / WN; // wave tile
  static constexpr int MI = WTM / 32, NJ = WTN / 32; // 32 x 32 blocks per wave
  // LDS-direct loads per thread per tile; a wave instruction fills 64 slots. When
  // the slots do not divide over the workgroup, the surplus wave instructions load
  // out of range into a dummy 1 KB block, so every wave issues the same count.
  static constexpr int A_WI = BM * CPR / kWave, B_WI = BN * CPR / kWave;   // wave instructions
  static constexpr int A_INSTR = (A_WI + NW - 1) / NW;
  static constexpr int B_INSTR = (B_WI + NW - 1) / NW;
  static constexpr int L = A_INSTR + B_INSTR;
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int STAGE_BYTES = (BM + BN) * BK * 2;
  static constexpr int OUT_PITCH = BN + 8;           // bf16 per row of the output staging tile
  static constexpr int RING_BYTES = NS * STAGE_BYTES;
  static constexpr int DUMMY_OFF = RING_BYTES;       // 1 KB sink for surplus wave loads
  static constexpr int OUT_BYTES = BM * OUT_PITCH * 2;
  static constexpr int LDS_BYTES = (RING_BYTES + 1024) > OUT_BYTES ? (RING_BYTES + 1024) : OUT_BYTES;
  static_assert(BM * CPR % kWave == 0 && BN * CPR % kWave == 0, "tiles fill whole wave loads");
  static_assert((NS - 2) * L <= 63, "vmcnt holds at most 63 outstanding loads");
  static_assert(CPR <= 16 && 16 % CPR == 0, "row chunking");
};

// Both double-buffered with long reduction tiles: fewer barriers per MFMA did more
// than deeper prefetch. Measured on 1024 rows: 5 stages of 32 with the fragment
// reads pipelined under the MFMAs were 6% slower on 4096 -> 12288; 64-wide tiles
// in 2 or 3 stages were 3-5% slower on 4096 -> 4096.
using CfgWide = Cfg<256, 192, 64, 4, 2, 2>;    // 8 waves of 64 x 96
using CfgSquare = Cfg<128, 128, 128, 2, 4, 2>; // 8 waves of 64 x 32

struct Seg {
  const uint16_t* a;   // [M, k] row-major (X or T)
  const uint16_t* b;   // [N, k] row-major (W, A or B)
  int k;               // reduction length (multiple of 8)
};

struct GemmParams {
  Seg seg[2];
  int nseg;
  int M, N;
  const uint8_t* mask1;    // row mask applied to segment 1's A rows (may be null)
  uint16_t* y;             // bf16 [M, N]
};

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int m0 = blockIdx.y * C::BM, n0 = blockIdx.x * C::BN;
  const int k0len = p.seg[0].k, k1len = p.nseg > 1 ? p.seg[1].k : 0;
  const int n0tiles = (k0len + C::BK - 1) / C::BK;
  const int ntiles = n0tiles + (k1len + C::BK - 1) / C::BK;

  // Per-thread load plan, fixed for the whole reduction. Slot q of a tile (16
  // bytes) holds row q / CPR, chunk (q % CPR) ^ swz(row). For each load: the byte
  // offset of its chunk at k = 0 in each segment, the chunk's k offset, and
  // whether the row takes part (in range; for segment 1's A rows also unmasked).
  uint32_t a_off0[C::A_INSTR], a_off1[C::A_INSTR], b_off0[C::B_INSTR], b_off1[C::B_INSTR];
  int a_kc[C::A_INSTR], b_kc[C::B_INSTR];
  unsigned a_ok0 = 0, a_ok1 = 0, b_ok = 0;
#pragma unroll
  for (int i = 0; i < C::A_INSTR; ++i) {
    const int q = (i * C::NW + wave) * kWave + lane;
    const int row = q / C::CPR;
    a_kc[i] = ((q % C::CPR) ^ ((row / C::RS) % C::CPR)) * 8;
    const int gr = m0 + row;
    const bool real = i * C::NW + wave < C::A_WI && gr < p.M;
    if (real) a_ok0 |= 1u << i;
    if (real && (p.mask1 == nullptr || p.mask1[gr] != 0)) a_ok1 |= 1u << i;
    a_off0[i] = uint32_t((size_t(gr) * k0len + a_kc[i]) * 2);
    a_off1[i] = uint32_t((size_t(gr) * k1len + a_kc[i]) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::B_INSTR; ++i) {
    const int q = (i * C::NW + wave) * kWave + lane;
    const int row = q / C::CPR;
    b_kc[i] = ((q % C::CPR) ^ ((row / C::RS) % C::CPR)) * 8;
    const int gr = n0 + row;
    if (i * C::NW + wave < C::B_WI && gr < p.N) b_ok |= 1u << i;
    b_off0[i] = uint32_t((size_t(gr) * k0len + b_kc[i]) * 2);
    b_off1[i] = uint32_t((size_t(gr) * k1len + b_kc[i]) * 2);
  }
  // The mask bytes above were read with ordinary loads: retire them so the
  // vmcnt arithmetic of the ring counts only the tile loads.
  wait_vmcnt<0>();

  const __amdgpu_buffer_rsrc_t ra0 = make_row_rsrc(p.seg[0].a, uint32_t(size_t(p.M) * k0len * 2));
  const __amdgpu_buffer_rsrc_t rb0 = make_row_rsrc(p.seg[0].b, uint32_t(size_t(p.N) * k0len * 2));
  const __amdgpu_buffer_rsrc_t ra1 = make_row_rsrc(p.nseg > 1 ? p.seg[1].a : p.seg[0].a,
                                                   uint32_t(size_t(p.M) * k1len * 2));
  const __amdgpu_buffer_rsrc_t rb1 = make_row_rsrc(p.nseg > 1 ? p.seg[1].b : p.seg[0].b,
                                                   uint32_t(size_t(p.N) * k1len * 2));

  // Issue the loads of reduction tile t into ring stage st. Tiles past the end
  // load out of range (zeros), so every step issues exactly L loads.
  auto issue = [&](int t, int st) {
    const bool s0 = t < n0tiles;                       // uniform
    const int kt = s0 ? t * C::BK : (t - n0tiles) * C::BK;
    const int krem = t >= ntiles ? 0 : (s0 ? k0len : k1len) - kt;   // columns left in the segment
    const unsigned aok = s0 ? a_ok0 : a_ok1;
    const uint32_t kb = uint32_t(kt * 2);
    char* base = smem + st * C::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < C::A_INSTR; ++i) {
      const bool ok = ((aok >> i) & 1u) && a_kc[i] < krem;
      const uint32_t off = ok ? (s0 ? a_off0[i] : a_off1[i]) + kb : kOutOfRange;
      char* dst = i * C::NW + wave < C::A_WI ? base + (i * C::NW + wave) * 1024 : smem + C::DUMMY_OFF;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s0 ? ra0 : ra1, (lds_ptr_t)dst, 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::B_INSTR; ++i) {
      const bool ok = ((b_ok >> i) & 1u) && b_kc[i] < krem;
      const uint32_t off = ok ? (s0 ? b_off0[i] : b_off1[i]) + kb : kOutOfRange;
      char* dst = i * C::NW + wave < C::B_WI ? base + C::A_BYTES + (i * C::NW + wave) * 1024
                                             : smem + C::DUMMY_OFF;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s0 ? rb0 : rb1, (lds_ptr_t)dst, 16, off, 0, 0, 0);
    }
  };

  f32x16_t acc[C::MI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Fragment reads: lane l takes row (l % 32) of a 32-row block and the 16-byte
  // chunk 2 ks + l / 32 (k = 16 ks + 8 (l / 32) .. +7).
  const int fr = lane & 31, fh = lane >> 5;
  const int fswz = (fr / C::RS) % C::CPR;            // block bases are multiples of 32
  const int arow = (wm * C::WTM + fr) * C::CPR * 16, brow = (wn * C::WTN + fr) * C::CPR * 16;
  auto compute = [&](int st) {
    const char* As = smem + st * C::STAGE_BYTES + arow;
    const char* Bs = smem + st * C::STAGE_BYTES + C::A_BYTES + brow;
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks) {
      const int ch = ((2 * ks + fh) ^ fswz) * 16;
      bf16x8_t af[C::MI], bfr[C::NJ];
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + i * 32 * C::CPR * 16 + ch);
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + j * 32 * C::CPR * 16 + ch);
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

#pragma unroll
  for (int s = 0; s < C::NS - 1; ++s) issue(s, s);
  // Unrolled by NS so every ring stage index is a constant.
  for (int t0 = 0; t0 < ntiles; t0 += C::NS) {
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      const int t = t0 + s;
      if (t >= ntiles) break;
      // Tile t's loads are done once at most the NS-2 later tiles' are in
      // flight; the barrier then publishes every wave's part and retires the
      // reads of the stage about to be refilled.
      wait_vmcnt<(C::NS - 2) * C::L>();
      __builtin_amdgcn_s_barrier();
      issue(t + C::NS - 1, (s + C::NS - 1) % C::NS);
      compute(s);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  // bf16 tile through LDS, then 16-byte row stores. Accumulator v of a 32 x 32
  // block sits at row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
  uint16_t* out = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int col = wn * C::WTN + j * 32 + fr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * C::WTM + i * 32 + 8 * (v >> 2) + 4 * fh + (v & 3);
        out[row * C::OUT_PITCH + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][v]);
      }
    }
  __syncthreads();
  const bool vec = (p.N % 8) == 0 && (reinterpret_cast<uintptr_t>(p.y) % 16) == 0;
  constexpr int CH = C::BN / 8;
  for (int c = tid; c < C::BM * CH; c += C::THREADS) {
    const int row = c / CH, cc = c % CH;
    const int gr = m0 + row, gc = n0 + cc * 8;
    if (gr >= p.M || gc >= p.N) continue;
    const uint16_t* src = out + row * C::OUT_PITCH + cc * 8;
    uint16_t* dst = p.y + size_t(gr) * p.N + gc;
    if (vec) {
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    } else {
      for (int e = 0; e < 8 && gc + e < p.N; ++e) dst[e] = src[e];
    }
  }
}

// LoRA-down T = bf16(scale * X A^T), X [M, K], A [r, K], T [M, r].
// One workgroup per 32 x 32 tile of T, over the whole reduction, so no
// workgroup waits for another and the sum order is fixed. Wave w of the 8 takes
// a contiguous 1/8 of K in chunks of 64: its lanes load a chunk of the 32 X rows
// and the 32 A rows with row-contiguous 16-byte loads (8 lanes per 128-byte row
// segment), write it to the wave's own LDS tiles and read it back as MFMA
// fragments, while the next three chunks' loads are in flight (the loop is
// latency-bound otherwise). LDS operations of one
// wave execute in order, so the wave needs no barrier. The wave partials are
// summed in LDS in wave order, scaled and rounded.
constexpr int LD_WAVES = 8, LD_KC = 64, LD_PITCH = LD_KC + 8;   // pitch: bf16 per LDS row

__global__ __launch_bounds__(LD_WAVES * 64) void lora_down_kernel(const uint16_t* X, const uint16_t* A, int M,
                                                                  int K, int r, float scale, uint16_t* T,
                                                                  const uint8_t* row_mask) {
  constexpr int TILE = 32 * LD_PITCH;                 // bf16 per operand tile
  constexpr int STAGE_BYTES = LD_WAVES * 2 * TILE * 2;
  constexpr int RED_BYTES = LD_WAVES * 16 * 64 * 4;
  __shared__ __attribute__((aligned(16))) char smem[STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES];
  // Tiles of the same 32 X rows go to consecutive ids on one XCD (workgroups
  // are dealt to the 8 XCDs round robin), so each XCD's L2 fetches those rows once.
  const int ttc = (r + 31) / 32;
  const int tid_x = xcd_contiguous_id(int(blockIdx.x), int(gridDim.x));
  const int tm = tid_x / ttc, tc = tid_x % ttc;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem) + wave * 2 * TILE;
  uint16_t* as = xs + TILE;
  const __amdgpu_buffer_rsrc_t rx = make_row_rsrc(X, uint32_t(size_t(M) * K * 2));
  const __amdgpu_buffer_rsrc_t ra = make_row_rsrc(A, uint32_t(size_t(r) * K * 2));
  // Loads: lane l covers rows l / 8 + 8 j (j < 4) at k offset 8 (l % 8).
  const int lr = lane >> 3, lk = (lane & 7) * 8;
  const int kw = (K + LD_WAVES * LD_KC - 1) / (LD_WAVES * LD_KC) * LD_KC;
  const int kb = wave * kw, ke = min(K, kb + kw);
  constexpr int NB = 4;                               // chunks in flight
  u32x4_t xv[NB][4], av[NB][4];
  auto load = [&](int k, u32x4_t (&xb)[4], u32x4_t (&ab)[4]) {
    const bool in = k + lk < ke;                     // ke is a multiple of 8
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int xrow = tm * 32 + lr + 8 * j, arow = tc * 32 + lr + 8 * j;
      xb[j] = __builtin_amdgcn_raw_buffer_load_b128(
          rx, (in && xrow < M) ? uint32_t((size_t(xrow) * K + k + lk) * 2) : kOutOfRange, 0u, 0);
      ab[j] = __builtin_amdgcn_raw_buffer_load_b128(
          ra, (in && arow < r) ? uint32_t((size_t(arow) * K + k + lk) * 2) : kOutOfRange, 0u, 0);
    }
  };
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  // Fragments: lane l reads row l % 32, k = 16 ks + 8 (l / 32) .. +7.
  const int fo = (lane & 31) * LD_PITCH + (lane >> 5) * 8;
#pragma unroll
  for (int b = 0; b < NB - 1; ++b) load(kb + b * LD_KC, xv[b], av[b]);
  // Chunks past the range load zeros (out of range) and add nothing.
  for (int k0 = kb; k0 < ke; k0 += NB * LD_KC) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int k = k0 + b * LD_KC;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<u32x4_t*>(xs + (lr + 8 * j) * LD_PITCH + lk) = xv[b][j];
        *reinterpret_cast<u32x4_t*>(as + (lr + 8 * j) * LD_PITCH + lk) = av[b][j];
      }
      load(k + (NB - 1) * LD_KC, xv[(b + NB - 1) % NB], av[(b + NB - 1) % NB]);
#pragma unroll
      for (int ks = 0; ks < LD_KC / 16; ++ks) {
        const bf16x8_t xf = *reinterpret_cast<const bf16x8_t*>(xs + fo + ks * 16);
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(as + fo + ks * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, af, acc, 0, 0, 0);
      }
    }
  }
  __syncthreads();                                    // the stage tiles become the reduction buffer
  float* red = reinterpret_cast<float*>(smem);        // [wave][v][lane]
#pragma unroll
  for (int v = 0; v < 16; ++v) red[(wave * 16 + v) * 64 + lane] = acc[v];
  __syncthreads();
  // Accumulator v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
  for (int i = threadIdx.x; i < 16 * 64; i += LD_WAVES * 64) {
    const int v = i >> 6, l = i & 63;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < LD_WAVES; ++w) sum += red[(w * 16 + v) * 64 + l];
    const int row = tm * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3), col = tc * 32 + (l & 31);
    if (row < M && col < r) {
      const float y = (row_mask && row_mask[row] == 0) ? 0.0f : scale * sum;   // masked rows: exact zeros
      T[size_t(row) * r + col] = __builtin_bit_cast(uint16_t, (__bf16)y);
    }
  }
}

// Transpose of a bf16 matrix: dst [C, R] = src [R, C]^T, with source rows whose
// mask byte is 0 written as zeros and, when scale != 1, every value scaled and
// rounded to nearest even. 64 x 64 tiles through LDS; 16-byte loads and stores
// when R and C are multiples of 8 (and the buffers 16-byte aligned), element
// accesses otherwise.
constexpr int TP = 64, TP_PITCH = TP + 8;

__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* src, int R, int C, uint16_t* dst,
                                                         const uint8_t* row_mask, float scale, int vec) {
  __shared__ uint16_t t[TP][TP_PITCH];
  const int r0 = blockIdx.y * TP, c0 = blockIdx.x * TP;
  const int tid = threadIdx.x, lr = tid >> 3, lc = (tid & 7) * 8;
  auto cvt = [&](uint16_t h, bool keep) -> uint16_t {
    if (!keep) return 0;
    if (scale == 1.0f) return h;
    return __builtin_bit_cast(uint16_t, (__bf16)(scale * __uint_as_float(uint32_t(h) << 16)));
  };
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = lr + 32 * i, gr = r0 + rr;
    const bool keep = gr < R && (row_mask == nullptr || row_mask[gr] != 0);
    uint16_t v[8];
    if (vec && gr < R && c0 + lc < C) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + size_t(gr) * C + c0 + lc);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[2 * e] = uint16_t(ww[e] & 0xffff); v[2 * e + 1] = uint16_t(ww[e] >> 16); }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (gr < R && c0 + lc + e < C) ? src[size_t(gr) * C + c0 + lc + e] : 0;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) t[rr][lc + e] = cvt(v[e], keep);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int oc = lr + 32 * i, go = c0 + oc;       // output row = source column
    if (go >= C) continue;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t[lc + e][oc];
    if (vec && r0 + lc < R) {
      uint4 w;
      w.x = uint32_t(v[0]) | (uint32_t(v[1]) << 16);
      w.y = uint32_t(v[2]) | (uint32_t(v[3]) << 16);
      w.z = uint32_t(v[4]) | (uint32_t(v[5]) << 16);
      w.w = uint32_t(v[6]) | (uint32_t(v[7]) << 16);
      *reinterpret_cast<uint4*>(dst + size_t(go) * R + r0 + lc) = w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (r0 + lc + e < R) dst[size_t(go) * R + r0 + lc + e] = v[e];
    }
  }
}

void launch_transpose(const uint16_t* src, int R, int C, uint16_t* dst, const uint8_t* row_mask, float scale,
                      hipStream_t stream) {
  const int vec = (R % 8 == 0 && C % 8 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(dst) % 16 == 0) ? 1 : 0;
  dim3 grid((C + TP - 1) / TP, (R + TP - 1) / TP);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, stream, src, R, C, dst, row_mask, scale, vec);
}

void launch_lora_down(const uint16_t* X, const uint16_t* A, int M, int K, int r, float scale, uint16_t* T,
                      const uint8_t* row_mask, hipStream_t stream) {
  const unsigned tiles = unsigned((M + 31) / 32) * unsigned((r + 31) / 32);
  hipLaunchKernelGGL(lora_down_kernel, dim3(tiles), dim3(LD_WAVES * 64), 0, stream, X, A, M, K, r, scale, T,
                     row_mask);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

template <class C>
void launch_cfg(const GemmParams& g, hipStream_t stream) {
  dim3 grid((g.N + C::BN - 1) / C::BN, (g.M + C::BM - 1) / C::BM, 1);
  hipLaunchKernelGGL(gemm_kernel<C>, grid, dim3(C::THREADS), 0, stream, g);
}

// Wide tiles when they fill the machine in whole waves of workgroups (or many
// of them), square tiles otherwise.
bool use_wide(int M, int N) {
  using W = CfgWide;
  const long tiles = long((M + W::BM - 1) / W::BM) * ((N + W::BN - 1) / W::BN);
  return tiles % 256 == 0 || tiles >= 1024;
}

void launch_main(const GemmParams& g, hipStream_t stream) {
  if (g.M == 0 || g.N == 0) return;
  if (use_wide(g.M, g.N))
    launch_cfg<CfgWide>(g, stream);
  else
    launch_cfg<CfgSquare>(g, stream);
}

}  // namespace

size_t gemm_workspace_bytes(int M, int N, int K, int r) {
  (void)N;
  (void)K;
  if (r <= 0 || M <= 0) return 256;
  return align256(size_t(M) * r * 2);             // T
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const uint16_t* tmat = nullptr;
  if (a.r > 0) {
    // workspace: T bf16 [M, r]
    uint16_t* t = static_cast<uint16_t*>(a.ws);
    launch_lora_down(static_cast<const uint16_t*>(a.X), static_cast<const uint16_t*>(a.A), a.M, a.K, a.r, a.scale,
                     t, nullptr, stream);
    tmat = t;
  }
  GemmParams g{};
  g.seg[0] = Seg{static_cast<const uint16_t*>(a.X), static_cast<const uint16_t*>(a.W), a.K};
  g.nseg = 1;
  if (a.r > 0) {
    g.seg[1] = Seg{tmat, static_cast<const uint16_t*>(a.B), a.r};
    g.nseg = 2;
    g.mask1 = a.row_mask;
  }
  g.M = a.M;
  g.N = a.N;
  g.y = static_cast<uint16_t*>(a.Y);
  launch_main(g, stream);
  return hipGetLastError();
}

// --- backward -------------------------------------------------------------------
// With U = s diag(m) dY B:  dX = dY W + U A,  dA = U^T X,  dB = s (diag(m) dY)^T (X A^T).
// Every product runs on the same MFMA kernel, whose operands are K-contiguous on
// both sides ([M, k] and [N, k]); the operands that are not (W, A, B, X, U, dY,
// T for the contractions over N and over M) are first transposed into the
// workspace, with the row mask and the scale applied by the transposes where the
// formula puts them.
namespace {
struct BwdWs {
  uint16_t *t, *bt, *u, *wt, *at, *ut, *xt, *dyt, *tt;
};
BwdWs bwd_ws(void* ws, int M, int N, int K, int r) {
  char* c = static_cast<char*>(ws);
  BwdWs w;
  auto take = [&](size_t elems) {
    uint16_t* p = reinterpret_cast<uint16_t*>(c);
    c += align256(elems * 2);
    return p;
  };
  w.t = take(size_t(M) * r);
  w.bt = take(size_t(r) * N);
  w.u = take(size_t(M) * r);
  w.wt = take(size_t(K) * N);
  w.at = take(size_t(K) * r);
  w.ut = take(size_t(r) * M);
  w.xt = take(size_t(K) * M);
  w.dyt = take(size_t(N) * M);
  w.tt = take(size_t(r) * M);
  return w;
}
}  // namespace

size_t gemm_bwd_workspace_bytes(int M, int N, int K, int r) {
  if (M <= 0 || N <= 0 || K <= 0 || r <= 0) return 256;
  const size_t m = M, n = N, k = K, rr = r;
  return align256(m * rr * 2) * 3 + align256(rr * n * 2) + align256(k * n * 2) + align256(k * rr * 2) +
         align256(rr * m * 2) + align256(k * m * 2) + align256(n * m * 2);
}

hipError_t launch_gemm_bwd(const GemmBwdArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  const int M = a.M, N = a.N, K = a.K, r = a.r;
  const BwdWs w = bwd_ws(a.ws, M, N, K, r);
  const uint16_t* X = static_cast<const uint16_t*>(a.X);
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  const uint16_t* dY = static_cast<const uint16_t*>(a.dY);
  // T = X A^T (unscaled, every row); U = bf16(s diag(m) dY B) through B^T
  launch_lora_down(X, A, M, K, r, 1.0f, w.t, nullptr, stream);
  launch_transpose(B, N, r, w.bt, nullptr, 1.0f, stream);
  launch_lora_down(dY, w.bt, M, N, r, a.scale, w.u, a.row_mask, stream);
  // dX = [dY | U] [W^T | A^T]^T
  if (a.dX) {
    const uint16_t* wt = static_cast<const uint16_t*>(a.Wt);
    if (!wt) {
      launch_transpose(W, N, K, w.wt, nullptr, 1.0f, stream);
      wt = w.wt;
    }
    launch_transpose(A, r, K, w.at, nullptr, 1.0f, stream);
    GemmParams g{};
    g.seg[0] = Seg{dY, wt, N};
    g.seg[1] = Seg{w.u, w.at, r};
    g.nseg = 2;
    g.M = M;
    g.N = K;
    g.y = static_cast<uint16_t*>(a.dX);
    launch_main(g, stream);
  }
  // dA = U^T X: rows of U^T against rows of X^T, reduction over M
  launch_transpose(w.u, M, r, w.ut, nullptr, 1.0f, stream);
  launch_transpose(X, M, K, w.xt, nullptr, 1.0f, stream);
  {
    GemmParams g{};
    g.seg[0] = Seg{w.ut, w.xt, M};
    g.nseg = 1;
    g.M = r;
    g.N = K;
    g.y = static_cast<uint16_t*>(a.dA);
    launch_main(g, stream);
  }
  // dB = (diag(m) dY)^T (s T): masked rows of dY and the scale go in with the transposes
  launch_transpose(dY, M, N, w.dyt, a.row_mask, 1.0f, stream);
  launch_transpose(w.t, M, r, w.tt, nullptr, a.scale, stream);
  {
    GemmParams g{};
    g.seg[0] = Seg{w.dyt, w.tt, M};
    g.nseg = 1;
    g.M = N;
    g.N = r;
    g.y = static_cast<uint16_t*>(a.dB);
    launch_main(g, stream);
  }
  return hipGetLastError();
}

}  // namespace uno
