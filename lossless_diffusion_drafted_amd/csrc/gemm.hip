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

#include <algorithm>
#include <climits>
#include "common.h"
#include "kernels.h"

namespace uno {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset past any range: reads 0

template <int BM_, int BN_, int BK_, int WM_, int WN_, int NS_, int KG_ = 1>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, NS = NS_;
  static constexpr int KG = KG_;                     // k groups: each takes 1/KG of every reduction tile
  static constexpr int NW = WM * WN * KG;
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
  static_assert(KG == 1 || (KG == 2 && (BK / 16) % 2 == 0), "k groups split the 16-wide steps evenly");
  static_assert(KG == 1 || WM * WN * MI * NJ * 16 * kWave * 4 <= RING_BYTES, "k-group exchange fits the ring");
};

// Both double-buffered with long reduction tiles: fewer barriers per MFMA did more
// than deeper prefetch. Measured on 1024 rows: 5 stages of 32 with the fragment
// reads pipelined under the MFMAs were 6% slower on 4096 -> 12288; 64-wide tiles
// in 2 or 3 stages were 3-5% slower on 4096 -> 4096.
using CfgWide = Cfg<256, 192, 64, 4, 2, 2>;    // 8 waves of 64 x 96
using CfgSquare = Cfg<128, 128, 128, 2, 4, 2>; // 8 waves of 64 x 32
using CfgHalf = Cfg<64, 128, 128, 2, 4, 2>;    // 8 waves of 32 x 32: short products on few tiles
using CfgRow = Cfg<64, 128, 128, 2, 4, 3>;     // the same in a three-stage ring: 17-64 rows, split reduction
using CfgRow96 = Cfg<64, 96, 128, 2, 3, 3>;    // 6 waves of 32 x 32: the same on 96-wide column tiles
using CfgSquareKG = Cfg<128, 128, 128, 2, 2, 2, 2>;   // two k groups of 4 waves of 64 x 64
using CfgSq160 = Cfg<128, 160, 128, 4, 1, 2, 2>;   // two k groups of 4 waves of 32 x 160
using CfgBig = Cfg<256, 256, 64, 4, 2, 2>;    // 8 waves of 64 x 128: products of 4096 rows and more

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
  // Split reduction (the SK form only): slice blockIdx.z of gridDim.z takes
  // reduction tiles [z kper, (z + 1) kper) of the extended reduction; slices store
  // fp32 tiles in `part` and the last of a tile to finish (a ticket) adds them in
  // slice order. Segment 1 may hold several groups' delta rows side by side (row
  // stride t_stride): output columns from nb1 on use its second block of k1len,
  // from nb2 on its third.
  int kper;
  float* part;             // [tiles, slices, BM * BN] fp32
  unsigned* ticket;        // [tiles], zero on entry and on exit
  int t_stride, nb1, nb2;
  // Segment 0's A rows gathered by heads (the SK form, BK = 128): with x_group > 0
  // the rows are x_stride apart and reduction tile t reads source tile t / x_group.
  int x_stride, x_group;
};

// One product on a 2-D grid (tiles_a == 0), or two independent products sharing
// one launch on a 1-D grid: workgroups [0, tiles_a) take pa's tiles, the rest pb's
// (small products that would each leave most CUs idle).
// floor(t / d) = (t * gather_mul(d)) >> 20 for t * d < 2^20: with m = ceil(2^20 /
// d) = (2^20 + e) / d, 0 <= e < d, the error term t * e / (d 2^20) stays below 1 / d.
__device__ inline unsigned gather_mul(int d) { return d > 0 ? ((1u << 20) + unsigned(d) - 1) / unsigned(d) : 0u; }

template <class C, bool SK = false>
__global__ __launch_bounds__(C::THREADS) void gemm_kernel(GemmParams pa, GemmParams pb, int tiles_a) {
  static_assert(!SK || C::KG == 1, "split reduction with one k group");
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave / (C::WM * C::WN), wr = wave % (C::WM * C::WN);
  const int wm = wr / C::WN, wn = wr % C::WN;
  const bool second = tiles_a > 0 && int(blockIdx.x) >= tiles_a;
  const GemmParams& p = second ? pb : pa;
  int tile_m = blockIdx.y, tile_n = blockIdx.x;
  if (tiles_a > 0) {
    const int local = second ? int(blockIdx.x) - tiles_a : int(blockIdx.x);
    const int ntx = (p.N + C::BN - 1) / C::BN;
    tile_m = local / ntx;
    tile_n = local % ntx;
  }
  const int m0 = tile_m * C::BM, n0 = tile_n * C::BN;
  const int k0len = p.seg[0].k, k1len = p.nseg > 1 ? p.seg[1].k : 0;
  const int n0tiles = (k0len + C::BK - 1) / C::BK;
  const int ntiles = n0tiles + (k1len + C::BK - 1) / C::BK;
  // The reduction tiles this workgroup takes: all, or its slice's.
  const int t_begin = SK ? int(blockIdx.z) * p.kper : 0;
  const int t_stop = SK ? min(ntiles, t_begin + p.kper) : ntiles;
  // Segment 1's row stride and this column tile's block of it.
  const int t_stride = SK && p.t_stride ? p.t_stride : k1len;
  const int t_col = SK ? ((n0 >= p.nb1) + (n0 >= p.nb2)) * k1len : 0;
  const int x_group = SK ? p.x_group : 0;
  const int x_stride = x_group > 0 ? p.x_stride : k0len;
  const unsigned x_mul = gather_mul(x_group);
  static_assert(!SK || C::BK == 128, "the gather maps whole 128-wide reduction tiles");

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
    a_off0[i] = uint32_t((size_t(gr) * x_stride + a_kc[i]) * 2);
    a_off1[i] = uint32_t((size_t(gr) * t_stride + t_col + a_kc[i]) * 2);
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

  const __amdgpu_buffer_rsrc_t ra0 = make_row_rsrc(p.seg[0].a, uint32_t(size_t(p.M) * x_stride * 2));
  const __amdgpu_buffer_rsrc_t rb0 = make_row_rsrc(p.seg[0].b, uint32_t(size_t(p.N) * k0len * 2));
  const __amdgpu_buffer_rsrc_t ra1 = make_row_rsrc(p.nseg > 1 ? p.seg[1].a : p.seg[0].a,
                                                   uint32_t(size_t(p.M) * t_stride * 2));
  const __amdgpu_buffer_rsrc_t rb1 = make_row_rsrc(p.nseg > 1 ? p.seg[1].b : p.seg[0].b,
                                                   uint32_t(size_t(p.N) * k1len * 2));

  // Issue the loads of reduction tile t into ring stage st. Tiles past the end
  // load out of range (zeros), so every step issues exactly L loads.
  auto issue = [&](int t, int st) {
    if constexpr (!SK) {
      const bool s0 = t < n0tiles;                       // uniform
      const int kt = s0 ? t * C::BK : (t - n0tiles) * C::BK;
      const int krem = t >= t_stop ? 0 : (s0 ? k0len : k1len) - kt;   // columns left in the segment
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
    } else {
      // Each segment in a branch of its own (the segment is uniform): selecting
      // between the two segments' offset arrays per load would put them in
      // scratch memory here.
      char* base = smem + st * C::STAGE_BYTES;
      const bool s0 = t < n0tiles;
      const int kt = (s0 ? t : t - n0tiles) * C::BK;
      const int krem = t >= t_stop ? 0 : (s0 ? k0len : k1len) - kt;   // columns left in the segment
      const uint32_t kb = uint32_t(kt * 2);
      if (s0) {
        // gathered rows: X's tile t is tile t / x_group of the source
        const uint32_t akb = x_group > 0 ? ((unsigned(t) * x_mul) >> 20) * (C::BK * 2) : kb;
#pragma unroll
        for (int i = 0; i < C::A_INSTR; ++i) {
          const bool ok = ((a_ok0 >> i) & 1u) && a_kc[i] < krem;
          const uint32_t off = ok ? a_off0[i] + akb : kOutOfRange;
          char* dst = i * C::NW + wave < C::A_WI ? base + (i * C::NW + wave) * 1024 : smem + C::DUMMY_OFF;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra0, (lds_ptr_t)dst, 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::B_INSTR; ++i) {
          const bool ok = ((b_ok >> i) & 1u) && b_kc[i] < krem;
          const uint32_t off = ok ? b_off0[i] + kb : kOutOfRange;
          char* dst = i * C::NW + wave < C::B_WI ? base + C::A_BYTES + (i * C::NW + wave) * 1024
                                                 : smem + C::DUMMY_OFF;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb0, (lds_ptr_t)dst, 16, off, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < C::A_INSTR; ++i) {
          const bool ok = ((a_ok1 >> i) & 1u) && a_kc[i] < krem;
          const uint32_t off = ok ? a_off1[i] + kb : kOutOfRange;
          char* dst = i * C::NW + wave < C::A_WI ? base + (i * C::NW + wave) * 1024 : smem + C::DUMMY_OFF;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra1, (lds_ptr_t)dst, 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::B_INSTR; ++i) {
          const bool ok = ((b_ok >> i) & 1u) && b_kc[i] < krem;
          const uint32_t off = ok ? b_off1[i] + kb : kOutOfRange;
          char* dst = i * C::NW + wave < C::B_WI ? base + C::A_BYTES + (i * C::NW + wave) * 1024
                                                 : smem + C::DUMMY_OFF;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb1, (lds_ptr_t)dst, 16, off, 0, 0, 0);
        }
      }
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
  // The fragments of step ks + 1 are read while step ks is multiplied (two
  // register sets), so an MFMA does not wait for the LDS read issued just before it.
  auto compute = [&](int st) {
    const char* As = smem + st * C::STAGE_BYTES + arow;
    const char* Bs = smem + st * C::STAGE_BYTES + C::A_BYTES + brow;
    bf16x8_t af[2][C::MI], bfr[2][C::NJ];
    auto read = [&](int ks, int b) {
      const int ch = ((2 * ks + fh) ^ fswz) * 16;
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
        af[b][i] = *reinterpret_cast<const bf16x8_t*>(As + i * 32 * C::CPR * 16 + ch);
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
        bfr[b][j] = *reinterpret_cast<const bf16x8_t*>(Bs + j * 32 * C::CPR * 16 + ch);
    };
    constexpr int KSG = C::BK / 16 / C::KG;            // steps per k group
    const int ks0 = kg * KSG;
    read(ks0, 0);
#pragma unroll
    for (int kk = 0; kk < KSG; ++kk) {
      const int b = kk & 1;
      if (kk + 1 < KSG) read(ks0 + kk + 1, b ^ 1);
      // (The scheduler would otherwise sink the reads back below the MFMAs.)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][i], bfr[b][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

#pragma unroll
  for (int s = 0; s < C::NS - 1; ++s) issue(t_begin + s, s);
  // Unrolled by NS so every ring stage index is a constant.
  for (int t0 = t_begin; t0 < t_stop; t0 += C::NS) {
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      const int t = t0 + s;
      if (t >= t_stop) break;
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

  if constexpr (SK) {
    // Split reduction: every slice stores its fp32 tile (accumulator order
    // [wave][i][j][v][lane], device-coherent stores) and takes the tile's ticket;
    // the last to finish adds all slices in slice order and writes the output.
    __shared__ int s_last;
    const int ks = int(gridDim.z);
    if (ks > 1) {
      const int tile = tile_m * int(gridDim.x) + tile_n;
      constexpr int TILE = C::BM * C::BN;
      const __amdgpu_buffer_rsrc_t rs =
          make_row_rsrc(p.part + (size_t(tile) * ks + blockIdx.z) * TILE, uint32_t(TILE * 4));
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(acc[i][j][v]), rs,
                uint32_t(((((wave * C::MI + i) * C::NJ + j) * 16 + v) * kWave + lane) * 4), 0u, kBufDeviceCoherent);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        const unsigned old = __hip_atomic_fetch_add(&p.ticket[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == unsigned(ks - 1) ? 1 : 0;
      }
      __syncthreads();
      if (!s_last) return;
      const __amdgpu_buffer_rsrc_t rp = make_row_rsrc(p.part + size_t(tile) * ks * TILE, uint32_t(ks * TILE * 4));
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {
          const uint32_t off = uint32_t((((wave * C::MI + i) * C::NJ + j) * 16 * kWave + lane) * 4);
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
          for (int q = 0; q < ks; ++q) {
            float x[16];
#pragma unroll
            for (int v = 0; v < 16; ++v)
              x[v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                  rp, off + uint32_t((q * TILE + v * kWave) * 4), 0u, kBufDeviceCoherent));
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] += x[v];
          }
        }
      if (tid == 0) __hip_atomic_store(&p.ticket[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  if constexpr (C::KG == 2) {
    // The second k group's sums meet the first's in LDS (fp32, [wave][i][j][v][lane]).
    float* xch = reinterpret_cast<float*>(smem) + wr * (C::MI * C::NJ * 16 * kWave);
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) xch[((i * C::NJ + j) * 16 + v) * kWave + lane] = acc[i][j][v];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] += xch[((i * C::NJ + j) * 16 + v) * kWave + lane];
    }
    __syncthreads();
  }

  // bf16 tile through LDS, then 16-byte row stores. Accumulator v of a 32 x 32
  // block sits at row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
  uint16_t* out = reinterpret_cast<uint16_t*>(smem);
  if (kg == 0) {
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
// One workgroup per 32 x 32 tile of T and slice of the reduction. Wave w of the 8
// takes a contiguous 1/8 of its slice in chunks of 64: its lanes load a chunk of
// the 32 X rows and the 32 A rows with row-contiguous 16-byte loads (8 lanes per
// 128-byte row segment), write it to the wave's own LDS tiles and read it back as
// MFMA fragments, while the next three chunks' loads are in flight (the loop is
// latency-bound otherwise). LDS operations of one wave execute in order, so the
// wave needs no barrier. The wave partials are summed in LDS in wave order.
//   With one slice the workgroup scales, rounds and stores its tile. With KS
// slices (a job whose reduction is KS times another's in the same launch, so that
// its workgroups take as long) each slice stores its fp32 tile with
// device-coherent stores and takes a ticket; the last slice of the tile to
// finish adds the KS tiles in slice order (the sum order is fixed), stores T and
// clears the ticket.
//   Xt, when given, receives X^T [K, M] (rows with mask 0 zeroed when a row mask
// is given) from the chunks already in LDS: each of the tile's column-tile
// workgroups writes a quarter of each chunk's 64 k-rows, 64 contiguous bytes per
// k-row, so X is not read again for it.
constexpr int LD_WAVES = 8, LD_KC = 64, LD_PITCH = LD_KC + 8;   // pitch: bf16 per LDS row
constexpr int LD_MAX_SLICES = 8;

// One LoRA-down product of a launch (a launch may carry two: the backward's T and U).
// Tt, when given, also receives the transposed tile, bf16(tscale * T) [r, M].
struct LdJob {
  const uint16_t* X;
  const uint16_t* A;
  int M, K, r;
  float scale;
  uint16_t* T;
  const uint8_t* row_mask;
  uint16_t* Tt;
  float tscale;
  int tiles;             // 32 x 32 tiles of T
  int ks;                // reduction slices per tile (1..LD_MAX_SLICES)
  float* part;           // [tiles, ks, 32 * 32] fp32 slice tiles (ks > 1)
  unsigned* ticket;      // [tiles], zero on entry and on exit (ks > 1)
  uint16_t* Xt;          // X^T [K, M] or null
};
struct LdJobs {
  LdJob j[2];
  int n;
};

// NB: chunks in flight per wave. NB = 4 at one workgroup per CU; NB = 2 keeps the
// registers within two workgroups per CU, for launches of more workgroups than CUs.
template <int NB>
__global__ __launch_bounds__(LD_WAVES * 64, NB == 2 ? 2 : 1) void lora_down_kernel(LdJobs jobs) {
  constexpr int TILE = 32 * LD_PITCH;                 // bf16 per operand tile
  constexpr int STAGE_BYTES = LD_WAVES * 2 * TILE * 2;
  constexpr int RED_BYTES = LD_WAVES * 16 * 64 * 4;
  __shared__ __attribute__((aligned(16))) char smem[STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES];
  __shared__ int s_last;
  // Workgroups of the same 32 X rows and slice go to consecutive ids on one XCD
  // (workgroups are dealt to the 8 XCDs round robin), so each XCD's L2 fetches
  // those rows once.
  int tid_x = xcd_contiguous_id(int(blockIdx.x), int(gridDim.x));
  const int jb = (jobs.n > 1 && tid_x >= jobs.j[0].tiles * jobs.j[0].ks) ? 1 : 0;
  const LdJob& jo = jobs.j[jb];
  if (jb) tid_x -= jobs.j[0].tiles * jobs.j[0].ks;
  const uint16_t* X = jo.X;
  const uint16_t* A = jo.A;
  const int M = jo.M, K = jo.K, r = jo.r, ks = jo.ks;
  const float scale = jo.scale;
  uint16_t* T = jo.T;
  const uint8_t* row_mask = jo.row_mask;
  const int ttc = (r + 31) / 32;
  const int tc = tid_x % ttc, sl = (tid_x / ttc) % ks, tm = tid_x / (ttc * ks);
  const int tile = tm * ttc + tc;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem) + wave * 2 * TILE;
  uint16_t* as = xs + TILE;
  const __amdgpu_buffer_rsrc_t rx = make_row_rsrc(X, uint32_t(size_t(M) * K * 2));
  const __amdgpu_buffer_rsrc_t ra = make_row_rsrc(A, uint32_t(size_t(r) * K * 2));
  // Loads: lane l covers rows l / 8 + 8 j (j < 4) at k offset 8 (l % 8).
  const int lr = lane >> 3, lk = (lane & 7) * 8;
  const int klen = (K + ks * LD_KC - 1) / (ks * LD_KC) * LD_KC;        // slice length
  const int k0 = sl * klen, k1 = min(K, k0 + klen);
  const int kw = (klen + LD_WAVES * LD_KC - 1) / (LD_WAVES * LD_KC) * LD_KC;
  const int kb = k0 + wave * kw, ke = min(k1, kb + kw);
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
  // The transposed copy: in each chunk, pass p (k-rows 16 p .. 16 p + 15) belongs
  // to column tile p % ttc. Lane l takes k-row 16 p + l / 4 and the 8 X rows
  // 8 (l % 4) .. + 7 of the tile: one 16-byte store.
  const bool xt_on = jo.Xt != nullptr && tc < 4;
  const int xt_row = 8 * (lane & 3);
  uint32_t xt_keep = 0xffu;                           // per lane: which of its 8 rows survive the mask
  if (xt_on) {
    xt_keep = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = tm * 32 + xt_row + e;
      if (row < M && (row_mask == nullptr || row_mask[row] != 0)) xt_keep |= 1u << e;
    }
  }
  // The mask bytes above were read with ordinary loads: retire them so the
  // chunk loads are the only loads counted below.
  wait_vmcnt<0>();
  auto write_xt = [&](int k) {
    for (int p = tc; p < 4; p += ttc) {
      const int kr = 16 * p + (lane >> 2);
      if (k + kr >= ke) continue;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = ((xt_keep >> (2 * e)) & 1u) ? xs[(xt_row + 2 * e) * LD_PITCH + kr] : 0u;
        const uint32_t hi = ((xt_keep >> (2 * e + 1)) & 1u) ? xs[(xt_row + 2 * e + 1) * LD_PITCH + kr] : 0u;
        w[e] = lo | (hi << 16);
      }
      const int row0 = tm * 32 + xt_row;
      uint16_t* dst = jo.Xt + size_t(k + kr) * M + row0;
      if (row0 + 8 <= M && (M % 8) == 0) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        for (int e = 0; e < 8 && row0 + e < M; ++e) dst[e] = uint16_t(w[e / 2] >> (16 * (e & 1)));
      }
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
  for (int k0c = kb; k0c < ke; k0c += NB * LD_KC) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int k = k0c + b * LD_KC;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<u32x4_t*>(xs + (lr + 8 * j) * LD_PITCH + lk) = xv[b][j];
        *reinterpret_cast<u32x4_t*>(as + (lr + 8 * j) * LD_PITCH + lk) = av[b][j];
      }
      load(k + (NB - 1) * LD_KC, xv[(b + NB - 1) % NB], av[(b + NB - 1) % NB]);
#pragma unroll
      for (int kk = 0; kk < LD_KC / 16; ++kk) {
        const bf16x8_t xf = *reinterpret_cast<const bf16x8_t*>(xs + fo + kk * 16);
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(as + fo + kk * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, af, acc, 0, 0, 0);
      }
      if (xt_on && k < ke) write_xt(k);
    }
  }
  __syncthreads();                                    // the stage tiles become the reduction buffer
  float* red = reinterpret_cast<float*>(smem);        // [wave][v][lane]
#pragma unroll
  for (int v = 0; v < 16; ++v) red[(wave * 16 + v) * 64 + lane] = acc[v];
  __syncthreads();
  // Accumulator v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
  auto store_t = [&](int v, int l, float sum) {
    const int row = tm * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3), col = tc * 32 + (l & 31);
    if (row < M && col < r) {
      const float y = (row_mask && row_mask[row] == 0) ? 0.0f : scale * sum;   // masked rows: exact zeros
      const __bf16 yb = (__bf16)y;
      T[size_t(row) * r + col] = __builtin_bit_cast(uint16_t, yb);
      if (jo.Tt) {
        const float yt = jo.tscale == 1.0f ? float(yb) : jo.tscale * float(yb);
        jo.Tt[size_t(col) * M + row] = __builtin_bit_cast(uint16_t, (__bf16)yt);
      }
    }
  };
  if (ks == 1) {
    for (int i = threadIdx.x; i < 16 * 64; i += LD_WAVES * 64) {
      const int v = i >> 6, l = i & 63;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < LD_WAVES; ++w) sum += red[(w * 16 + v) * 64 + l];
      store_t(v, l, sum);
    }
    return;
  }
  // Slice tile in accumulator order [v][lane], device-coherent stores.
  float* part = jo.part + (size_t(tile) * ks + sl) * 1024;
  for (int i = threadIdx.x; i < 16 * 64; i += LD_WAVES * 64) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < LD_WAVES; ++w) sum += red[w * 1024 + i];
    __hip_atomic_store(&part[i], sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Every lane's device-coherent stores are complete before the ticket is taken.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(&jo.ticket[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == unsigned(ks - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  // The slice tiles with device-coherent loads, all issued before the first is
  // summed, then added in slice order.
  const __amdgpu_buffer_rsrc_t rp = make_row_rsrc(jo.part + size_t(tile) * ks * 1024, uint32_t(ks * 1024 * 4));
  for (int i = threadIdx.x; i < 16 * 64; i += LD_WAVES * 64) {
    float v[LD_MAX_SLICES];
#pragma unroll
    for (int q = 0; q < LD_MAX_SLICES; ++q)
      v[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
          rp, q < ks ? uint32_t((q * 1024 + i) * 4) : kOutOfRange, 0u, kBufDeviceCoherent));
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < LD_MAX_SLICES; ++q)
      if (q < ks) sum += v[q];
    store_t(i >> 6, i & 63, sum);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&jo.ticket[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Small-M path. With M <= 64 rows (a decode step's block rows) the tiled kernel
// leaves most CUs idle, and the product is bound by reading W once from HBM.
// Each workgroup owns 32 output columns and one of KS slices of the reduction;
// its four waves split the slice into contiguous runs of 128-wide groups. A wave
// multiplies its 32 W rows (two 16-column blocks) against every X row with
// v_mfma_f32_16x16x32_bf16, M padded to 16-row blocks, in the instruction's own
// operand layout: for the c-th 32-wide step of a group, lane group g (lanes 16 g ..
// 16 g + 15) holds k = 32 c + 8 g .. + 7, so each load instruction reads 64
// contiguous bytes of each of 16 rows and a group reads 256-byte runs of every row.
// (Measured: a layout with 64 contiguous bytes per lane instead, spread over four
// instructions, streamed W 1.3 to 1.6 times slower.) The next group's loads are in
// flight while a group is multiplied; deeper prefetch measured slower (fewer waves
// fit). The delta segment [T | B] (r more reduction steps, T already scaled and
// gated) is taken 32 wide by the tile's last wave.
//   The four wave partials meet in LDS in wave order. With KS > 1 each slice
// stores its fp32 tile with device-coherent stores and takes a ticket (relaxed:
// the stores are complete and coherent before it; an acquire-release ticket, which
// writes back and invalidates L2, measured up to 3 times slower); the last slice
// of a column tile to finish adds the KS tiles in slice order (so the sum order is
// fixed), writes the output and resets the ticket.
struct SkinnyParams {
  const uint16_t* x;      // [M, K]
  const uint16_t* w;      // [N, K]
  const uint16_t* t;      // [M, t_stride] delta rows (scaled and gated), or null when r == 0
  const uint16_t* b;      // [N, r]
  int M, N, K, r, KS;
  // Grouped products: T holds the groups' delta rows side by side (row stride
  // t_stride); columns from nb1 on use T's second block of r, from nb2 on its
  // third (INT_MAX: one group).
  int t_stride, nb1, nb2;
  // X gathered by heads (x_group > 0): X row m at x_stride elements apart, its
  // 128-wide group g read from source group g / x_group.
  int x_stride, x_group;
  float scale;            // epilogue: y = mask[m] ? scale * acc : 0 (mask may be null)
  const uint8_t* mask;
  uint16_t* y;            // [M, N] bf16
  float* yf;              // [M, N] fp32 instead of y when given
  float* part;            // [KS, M, N] fp32 slice tiles (KS > 1)
  unsigned* ticket;       // [ceil(N / 32)], zero on entry and on exit
};

constexpr int SK_COLS = 32;        // output columns per workgroup
constexpr int SK_GROUP = 128;      // reduction elements per group
constexpr int SK_MAX_SLICES = 8;   // K slices of one product at most

template <int MB>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyParams p) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  constexpr int NB = SK_COLS / 16;
  constexpr int ROWS = MB * 16;
  __shared__ float red[4][ROWS][SK_COLS + 1];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int n0 = tile * SK_COLS;
  const int G = p.K / SK_GROUP;
  const int nw = p.KS * 4, wi = ks * 4 + wave;
  const int g0 = int((long long)G * wi / nw), g1 = int((long long)G * (wi + 1) / nw);
  const int fr = lane & 15, fg = lane >> 4;

  const int xs = p.x_group > 0 ? p.x_stride : p.K;        // X row stride
  const unsigned x_mul = gather_mul(p.x_group);
  const __amdgpu_buffer_rsrc_t rx = make_row_rsrc(p.x, uint32_t(size_t(p.M) * xs * 2));
  const __amdgpu_buffer_rsrc_t rw = make_row_rsrc(p.w, uint32_t(size_t(p.N) * p.K * 2));
  uint32_t xo[MB], wo[NB];
  bool xin[MB], win[NB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = i * 16 + fr;
    xin[i] = m < p.M;
    xo[i] = uint32_t((size_t(m) * xs + fg * 8) * 2);
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int n = n0 + j * 16 + fr;
    win[j] = n < p.N;
    wo[j] = uint32_t((size_t(n) * p.K + fg * 8) * 2);
  }

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4_t xa[MB][4], wa[NB][4], xb[MB][4], wb[NB][4];
  // Group g's loads; past the wave's last group they read out of range (zeros), so
  // every call issues the same loads and the waits are counted at compile time.
  auto load = [&](int g, u32x4_t (&xv)[MB][4], u32x4_t (&wv)[NB][4]) {
    const uint32_t kb = uint32_t(g) * SK_GROUP * 2;
    const uint32_t xkb = p.x_group > 0 ? ((unsigned(g) * x_mul) >> 20) * (SK_GROUP * 2) : kb;
    const bool live = g < g1;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        wv[j][c] = __builtin_amdgcn_raw_buffer_load_b128(rw, (live && win[j]) ? wo[j] + kb + c * 64 : kOutOfRange,
                                                         0u, kBufNonTemporal);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        xv[i][c] = __builtin_amdgcn_raw_buffer_load_b128(rx, (live && xin[i]) ? xo[i] + xkb + c * 64 : kOutOfRange,
                                                         0u, 0);
  };
  auto mma = [&](const u32x4_t (&xv)[MB][4], const u32x4_t (&wv)[NB][4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv[i][c]),
                                                              __builtin_bit_cast(bf16x8_t, wv[j][c]),
                                                              acc[i][j], 0, 0, 0);
  };
  // Two register sets, so every index is a constant: the next group's loads are in
  // flight while the current group is multiplied.
  // The scheduling barriers keep each group's loads ahead of the previous group's
  // MFMAs; without them the compiler sank the loads below the MFMAs and waited for
  // nearly all of them at the top of the loop, leaving one group in flight.
  load(g0, xa, wa);
  for (int g = g0; g < g1; g += 2) {
    load(g + 1, xb, wb);
    __builtin_amdgcn_sched_barrier(0);
    mma(xa, wa);
    __builtin_amdgcn_sched_barrier(0);
    load(g + 2, xa, wa);
    __builtin_amdgcn_sched_barrier(0);
    if (g + 1 < g1) mma(xb, wb);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Delta segment: r more reduction steps, 32 wide, on the tile's last wave.
  if (p.r > 0 && wi == nw - 1) {
    const __amdgpu_buffer_rsrc_t rt = make_row_rsrc(p.t, uint32_t(size_t(p.M) * p.t_stride * 2));
    const __amdgpu_buffer_rsrc_t rb = make_row_rsrc(p.b, uint32_t(size_t(p.N) * p.r * 2));
    const int toff = ((n0 >= p.nb1) + (n0 >= p.nb2)) * p.r;   // this tile's group block of T
    for (int s0 = 0; s0 < p.r; s0 += 32) {
      u32x4_t tv[MB], bv[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int m = i * 16 + fr;
        tv[i] = __builtin_amdgcn_raw_buffer_load_b128(
            rt, m < p.M ? uint32_t((size_t(m) * p.t_stride + toff + s0 + fg * 8) * 2) : kOutOfRange, 0u, 0);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = n0 + j * 16 + fr;
        bv[j] = __builtin_amdgcn_raw_buffer_load_b128(
            rb, n < p.N ? uint32_t((size_t(n) * p.r + s0 + fg * 8) * 2) : kOutOfRange, 0u, 0);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, tv[i]),
                                                              __builtin_bit_cast(bf16x8_t, bv[j]),
                                                              acc[i][j], 0, 0, 0);
    }
  }

  // Accumulator v of lane l of a 16 x 16 block is row 4 (l / 16) + v, column l % 16.
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][i * 16 + 4 * fg + v][j * 16 + fr] = acc[i][j][v];
  __syncthreads();

  // the row mask of the epilogue, read once per row
  __shared__ float rowscale[ROWS];
  const int rows = p.M < ROWS ? p.M : ROWS;
  if (tid < rows) rowscale[tid] = (p.mask && p.mask[tid] == 0) ? 0.0f : p.scale;
  __syncthreads();
  auto store = [&](int m, int n, float s) {
    const float y = rowscale[m] * s;
    if (p.yf)
      p.yf[size_t(m) * p.N + n] = y;
    else
      p.y[size_t(m) * p.N + n] = __builtin_bit_cast(uint16_t, (__bf16)y);
  };
  if (p.KS == 1) {
    for (int e = tid; e < rows * SK_COLS; e += 256) {
      const int m = e / SK_COLS, c = e % SK_COLS, n = n0 + c;
      if (n >= p.N) continue;
      store(m, n, red[0][m][c] + red[1][m][c] + red[2][m][c] + red[3][m][c]);
    }
    return;
  }
  float* part = p.part + size_t(ks) * p.M * p.N;
  for (int e = tid; e < rows * SK_COLS; e += 256) {
    const int m = e / SK_COLS, c = e % SK_COLS, n = n0 + c;
    if (n >= p.N) continue;
    const float s = red[0][m][c] + red[1][m][c] + red[2][m][c] + red[3][m][c];
    __hip_atomic_store(&part[size_t(m) * p.N + n], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Every lane's device-coherent stores are complete before the ticket is taken.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(&p.ticket[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == unsigned(p.KS - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  // The slice tiles are read with device-coherent loads (the SC1 policy, what an
  // agent-scope atomic load uses), all of a batch's loads issued before the first
  // is summed: one memory round trip per batch, not one per load.
  const __amdgpu_buffer_rsrc_t rp = make_row_rsrc(p.part, uint32_t(size_t(p.KS) * p.M * p.N * 4));
  constexpr int EB = 4;                                  // elements per thread per batch
  for (int e0 = tid; e0 < rows * SK_COLS; e0 += 256 * EB) {
    float v[EB][SK_MAX_SLICES];
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      const int e = e0 + u * 256, m = e / SK_COLS, n = n0 + e % SK_COLS;
      const bool ok = e < rows * SK_COLS && n < p.N;
#pragma unroll
      for (int q = 0; q < SK_MAX_SLICES; ++q)
        v[u][q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
            rp, (ok && q < p.KS) ? uint32_t(((size_t(q) * p.M + m) * p.N + n) * 4) : kOutOfRange, 0u,
            kBufDeviceCoherent));
    }
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      const int e = e0 + u * 256, m = e / SK_COLS, n = n0 + e % SK_COLS;
      if (e >= rows * SK_COLS || n >= p.N) continue;
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < SK_MAX_SLICES; ++q)
        if (q < p.KS) s += v[u][q];
      store(m, n, s);
    }
  }
  if (tid == 0) __hip_atomic_store(&p.ticket[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Small-M path, streaming form, for wide products (an LM head) at 17-64 rows.
// The product above keeps one 128-wide group of loads in flight per wave, and at
// 64 rows each wave also streams its own copy of X through registers: from HBM
// (weights no cache holds, as in a decode step) the LM head at 64 rows ran at
// 2.6 TB/s. Here the four waves of a workgroup own four adjacent 32-column blocks
// (128 columns) over the whole reduction and share X:
// * X: each 128-wide group's X rows go to LDS once per workgroup, by buffer loads
//   that write LDS, in the MFMA operand order (the load for row block i and
//   32-wide step c writes 1 KB that lane l later reads as its own 16 bytes), so the
//   fragment reads are conflict-free. PD stages.
// * W: each wave loads its own 32 rows of the group into registers, a ring of PD
//   groups (PD - 1 in flight while one is multiplied): 8 KB per wave per group,
//   about 100 KB per CU in flight.
// * One barrier per group: the wait for group g's loads (in order, so W and X),
//   then the barrier, publishes the X stage and retires every wave's reads of the
//   stage refilled next.
// * Each workgroup covers the whole reduction of its columns (products with at
//   least 256 column tiles), so no partials cross waves or workgroups.
constexpr int SK2_COLS = 128;      // output columns per workgroup (32 per wave)

template <int MB, int PD>
__global__ __launch_bounds__(256) void skinny2_kernel(SkinnyParams p) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  constexpr int NB = 2;                                 // 16-column blocks per wave
  constexpr int XL = MB * 4;                            // X load instructions per group (1 KB each)
  constexpr int XW = XL / 4;                            // ... per wave
  constexpr int LPG = XW + NB * 4;                      // loads per wave per group
  constexpr int STAGE = XL * 1024;                      // bytes of one X stage
  __shared__ __attribute__((aligned(1024))) char xs[PD * STAGE];
  __shared__ float rowscale[MB * 16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * SK2_COLS + wave * 32;
  const int g0 = 0, g1 = p.K / SK_GROUP;                // the whole reduction
  const int fr = lane & 15, fg = lane >> 4;

  const __amdgpu_buffer_rsrc_t rx = make_row_rsrc(p.x, uint32_t(size_t(p.M) * p.K * 2));
  const __amdgpu_buffer_rsrc_t rw = make_row_rsrc(p.w, uint32_t(size_t(p.N) * p.K * 2));
  // X load q = wave + 4 e (row block q / 4, step q % 4); lane l reads row
  // 16 (q / 4) + l % 16 at k = 32 (q % 4) + 8 (l / 16).
  uint32_t xo[XW];
  bool xin[XW];
#pragma unroll
  for (int e = 0; e < XW; ++e) {
    const int q = wave + 4 * e, m = (q >> 2) * 16 + fr;
    xin[e] = m < p.M;
    xo[e] = uint32_t((size_t(m) * p.K + (q & 3) * 32 + fg * 8) * 2);
  }
  uint32_t wo[NB];
  bool win[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int n = n0 + j * 16 + fr;
    win[j] = n < p.N;
    wo[j] = uint32_t((size_t(n) * p.K + fg * 8) * 2);
  }

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4_t wr[PD][NB][4];
  // Group g's loads into X stage st and W set st; past the slice they read out of
  // range (zeros), so every step issues LPG loads and the waits are static.
  auto issue = [&](int g, int st, u32x4_t (&wv)[NB][4]) {
    const bool live = g < g1;
    const uint32_t kb = uint32_t(g) * SK_GROUP * 2;
#pragma unroll
    for (int e = 0; e < XW; ++e) {
      // The offset goes through a variable: written inline in the call, it kept the
      // host compiler from emitting the kernel's launch stub.
      const uint32_t off = (live && xin[e]) ? xo[e] + kb : kOutOfRange;
      char* dst = xs + st * STAGE + (wave + 4 * e) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)dst, 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        wv[j][c] = __builtin_amdgcn_raw_buffer_load_b128(rw, (live && win[j]) ? wo[j] + kb + c * 64 : kOutOfRange,
                                                         0u, kBufNonTemporal);
  };
  auto mma = [&](int st, const u32x4_t (&wv)[NB][4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const u32x4_t xf = *reinterpret_cast<const u32x4_t*>(xs + st * STAGE + (i * 4 + c) * 1024 + lane * 16);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xf),
                                                              __builtin_bit_cast(bf16x8_t, wv[j][c]),
                                                              acc[i][j], 0, 0, 0);
      }
  };

#pragma unroll
  for (int s = 0; s < PD - 1; ++s) issue(g0 + s, s, wr[s]);
  // Unrolled by PD so that every stage and register set index is a constant.
  for (int gb = g0; gb < g1; gb += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int g = gb + s;
      if (g >= g1) break;
      wait_vmcnt<(PD - 2) * LPG>();                   // group g's X and W have landed
      __builtin_amdgcn_s_barrier();                   // X stage of g complete; stage (g - 1) free
      issue(g + PD - 1, (s + PD - 1) % PD, wr[(s + PD - 1) % PD]);
      mma(s, wr[s]);
    }
  }
  wait_vmcnt<0>();

  // Delta segment [T | B]: r more reduction steps, 32 wide.
  if (p.r > 0) {
    const __amdgpu_buffer_rsrc_t rt = make_row_rsrc(p.t, uint32_t(size_t(p.M) * p.t_stride * 2));
    const __amdgpu_buffer_rsrc_t rb = make_row_rsrc(p.b, uint32_t(size_t(p.N) * p.r * 2));
    const int toff = ((n0 >= p.nb1) + (n0 >= p.nb2)) * p.r;   // this wave's group block of T
    for (int s0 = 0; s0 < p.r; s0 += 32) {
      u32x4_t tv[MB], bv[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int m = i * 16 + fr;
        tv[i] = __builtin_amdgcn_raw_buffer_load_b128(
            rt, m < p.M ? uint32_t((size_t(m) * p.t_stride + toff + s0 + fg * 8) * 2) : kOutOfRange, 0u, 0);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = n0 + j * 16 + fr;
        bv[j] = __builtin_amdgcn_raw_buffer_load_b128(
            rb, n < p.N ? uint32_t((size_t(n) * p.r + s0 + fg * 8) * 2) : kOutOfRange, 0u, 0);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, tv[i]),
                                                              __builtin_bit_cast(bf16x8_t, bv[j]),
                                                              acc[i][j], 0, 0, 0);
    }
  }

  // the row mask of the epilogue, read once per row
  const int rows = p.M < MB * 16 ? p.M : MB * 16;
  if (tid < rows) rowscale[tid] = (p.mask && p.mask[tid] == 0) ? 0.0f : p.scale;
  __syncthreads();
  auto store = [&](int m, int n, float v) {
    const float y = rowscale[m] * v;
    if (p.yf)
      p.yf[size_t(m) * p.N + n] = y;
    else
      p.y[size_t(m) * p.N + n] = __builtin_bit_cast(uint16_t, (__bf16)y);
  };
  // Accumulator v of lane l of a 16 x 16 block is row 4 (l / 16) + v, column l % 16.
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = i * 16 + 4 * fg + v, n = n0 + j * 16 + fr;
        if (m < p.M && n < p.N) store(m, n, acc[i][j][v]);
      }
}


// Which small-M form a product takes. Measured from HBM (each call a different
// weight), the streaming form won only where its workgroups each cover the whole
// reduction (products with at least 256 column tiles of 128, such as an LM
// head) and M > 16: the LM head 4096 -> 151936 at 64 rows took 366 against
// 483 us. Elsewhere its short slices and the last slice's sum over 128-column
// partial tiles cost more than they save (q 4096 -> 4096 at 64 rows: 22.6 against
// 19.9 us), and at M <= 16 it was slower throughout (LM head at 4 rows: 290
// against 259 us).
bool use_skinny2(int M, int N, int K) { return M > 16 && (N + SK2_COLS - 1) / SK2_COLS >= 256; }

void launch_skinny2(const SkinnyParams& p, hipStream_t stream) {
  const dim3 grid((p.N + SK2_COLS - 1) / SK2_COLS);
  if (p.M <= 32)
    skinny2_kernel<2, 4><<<grid, dim3(256), 0, stream>>>(p);
  else
    skinny2_kernel<4, 4><<<grid, dim3(256), 0, stream>>>(p);
}

// K slices of a small-M product: about one workgroup per CU (measured best
// against 2, 4 and 8 per CU), each wave at least one 128-wide group. Then the
// count whose workgroups spread most evenly over the 256 CUs: time goes as
// ceil(tiles ks / 256) / ks, the most workgroups one CU runs times each one's
// share of the reduction. Fewer slices are taken when that is lower (80 column
// tiles: 3 slices, 240 workgroups, not 4 and 320); more only when it is lower by
// 5% and each wave keeps at least 2.5 groups (640 tiles: 2 slices, not 1;
// 192 tiles stay at 2, as 4 slices of 2 groups a wave measured slower).
int skinny_slices(int N, int K) {
  const int tiles = (N + SK_COLS - 1) / SK_COLS;
  const int G = K / SK_GROUP;
  int cap = G / 4 > 1 ? G / 4 : 1;
  if (cap > SK_MAX_SLICES) cap = SK_MAX_SLICES;
  int ks = (256 + tiles - 1) / tiles;
  if (ks > cap) ks = cap;
  int best = ks;
  long bn = (long(tiles) * ks + 255) / 256, bd = ks;   // the cost bn / bd of the best so far
  for (int k = 1; k <= cap; ++k) {
    if (k > ks && 2 * G < 5 * 4 * k) break;
    const long n = (long(tiles) * k + 255) / 256;
    if (k < ks ? n * bd < bn * k : 20 * n * bd < 19 * bn * k) {
      best = k;
      bn = n;
      bd = k;
    }
  }
  return best;
}

bool skinny_ok(int M, int N, int K, int r, const void* x, const void* w, const void* a, const void* b) {
  const bool al = reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(w) % 16 == 0 &&
                  (r == 0 || (reinterpret_cast<uintptr_t>(a) % 16 == 0 && reinterpret_cast<uintptr_t>(b) % 16 == 0));
  // every operand must fit one buffer resource's 32-bit byte range
  const bool fits = size_t(N) * K * 2 < (size_t(1) << 32) && size_t(M) * K * 2 < (size_t(1) << 32);
  return M >= 1 && M <= 64 && K % SK_GROUP == 0 && r % 32 == 0 && al && fits;
}

void launch_skinny(const SkinnyParams& p, hipStream_t stream) {
  const dim3 grid((p.N + SK_COLS - 1) / SK_COLS, p.KS);
  if (p.M <= 16)
    hipLaunchKernelGGL(skinny_kernel<1>, grid, dim3(256), 0, stream, p);
  else if (p.M <= 32)
    hipLaunchKernelGGL(skinny_kernel<2>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(skinny_kernel<4>, grid, dim3(256), 0, stream, p);
}

// Transpose of a bf16 matrix: dst [C, R] = src [R, C]^T, with source rows whose
// mask byte is 0 written as zeros and, when scale != 1, every value scaled and
// rounded to nearest even. 64 x 64 tiles through LDS; 16-byte loads and stores
// when R and C are multiples of 8 (and the buffers 16-byte aligned), element
// accesses otherwise.
constexpr int TP = 64, TP_PITCH = TP + 8;

// Several transposes in one launch: workgroup b takes tile b - first of the job
// whose tiles [first, first + tiles) hold b (one launch instead of one per
// transpose, each of which paid a launch and a memory round trip).
struct TpJob {
  const uint16_t* src;
  uint16_t* dst;
  const uint8_t* row_mask;
  float scale;
  int R, C, vec, tiles_x, first;
};
struct TpJobs {
  TpJob j[5];
  int n;
};

__global__ __launch_bounds__(256) void transpose_kernel(TpJobs jobs) {
  __shared__ uint16_t t[TP][TP_PITCH];
  int jb = 0;
  while (jb + 1 < jobs.n && int(blockIdx.x) >= jobs.j[jb + 1].first) ++jb;
  const TpJob& jo = jobs.j[jb];
  const uint16_t* src = jo.src;
  uint16_t* dst = jo.dst;
  const uint8_t* row_mask = jo.row_mask;
  const float scale = jo.scale;
  const int R = jo.R, C = jo.C, vec = jo.vec;
  const int tb = int(blockIdx.x) - jo.first;
  const int r0 = (tb / jo.tiles_x) * TP, c0 = (tb % jo.tiles_x) * TP;
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

// Up to five transposes dst [C, R] = src [R, C]^T in one launch (see transpose_kernel).
struct Transposes {
  TpJobs jobs{};
  int tiles = 0;
  void add(const uint16_t* src, int R, int C, uint16_t* dst, const uint8_t* row_mask, float scale) {
    TpJob& j = jobs.j[jobs.n++];
    j.src = src;
    j.dst = dst;
    j.row_mask = row_mask;
    j.scale = scale;
    j.R = R;
    j.C = C;
    j.vec = (R % 8 == 0 && C % 8 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
             reinterpret_cast<uintptr_t>(dst) % 16 == 0) ? 1 : 0;
    j.tiles_x = (C + TP - 1) / TP;
    j.first = tiles;
    tiles += j.tiles_x * ((R + TP - 1) / TP);
  }
  void launch(hipStream_t stream) const {
    if (tiles > 0) hipLaunchKernelGGL(transpose_kernel, dim3(tiles), dim3(256), 0, stream, jobs);
  }
};

void launch_transpose(const uint16_t* src, int R, int C, uint16_t* dst, const uint8_t* row_mask, float scale,
                      hipStream_t stream) {
  Transposes t;
  t.add(src, R, C, dst, row_mask, scale);
  t.launch(stream);
}

LdJob lora_down_job(const uint16_t* X, const uint16_t* A, int M, int K, int r, float scale, uint16_t* T,
                    const uint8_t* row_mask, uint16_t* Tt = nullptr, float tscale = 1.0f, uint16_t* Xt = nullptr) {
  LdJob j{X, A, M, K, r, scale, T, row_mask, Tt, tscale, ((M + 31) / 32) * ((r + 31) / 32), 1, nullptr, nullptr, Xt};
  return j;
}

// Reduction slices for two jobs of one launch: the longer reduction is cut into
// about as many slices as it is times the shorter, so that the workgroups of both
// take about as long.
void balance_slices(LdJob& a, LdJob& b) {
  const int kmin = a.K < b.K ? a.K : b.K;
  if (kmin <= 0) return;
  a.ks = std::min(LD_MAX_SLICES, std::max(1, (a.K + kmin / 2) / kmin));
  b.ks = std::min(LD_MAX_SLICES, std::max(1, (b.K + kmin / 2) / kmin));
}

void launch_lora_downs(const LdJob* jobs, int n, hipStream_t stream) {
  LdJobs js{};
  int tiles = 0;
  for (int i = 0; i < n; ++i) {
    js.j[i] = jobs[i];
    tiles += jobs[i].tiles * jobs[i].ks;
  }
  js.n = n;
  // (Measured on the backward's 512-workgroup launches: two workgroups per CU
  // with two chunks in flight per wave took the MLP-shape backward from 159.6 to
  // 154 us and the down-projection shape from 142 to 134 us.)
  if (tiles > 256)
    hipLaunchKernelGGL(lora_down_kernel<2>, dim3(tiles), dim3(LD_WAVES * 64), 0, stream, js);
  else if (tiles > 0)
    hipLaunchKernelGGL(lora_down_kernel<4>, dim3(tiles), dim3(LD_WAVES * 64), 0, stream, js);
}

void launch_lora_down(const uint16_t* X, const uint16_t* A, int M, int K, int r, float scale, uint16_t* T,
                      const uint8_t* row_mask, int ks, float* part, unsigned* tickets, hipStream_t stream) {
  LdJob j = lora_down_job(X, A, M, K, r, scale, T, row_mask);
  if (ks > 1) {
    j.ks = ks;
    j.part = part;
    j.ticket = tickets;
  }
  launch_lora_downs(&j, 1, stream);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

template <class C>
void launch_cfg(const GemmParams& g, hipStream_t stream) {
  dim3 grid((g.N + C::BN - 1) / C::BN, (g.M + C::BM - 1) / C::BM, 1);
  hipLaunchKernelGGL(gemm_kernel<C>, grid, dim3(C::THREADS), 0, stream, g, g, 0);
}

template <class C>
void launch_pair_cfg(const GemmParams& a, const GemmParams& b, hipStream_t stream) {
  const int ta = ((a.N + C::BN - 1) / C::BN) * ((a.M + C::BM - 1) / C::BM);
  const int tb = ((b.N + C::BN - 1) / C::BN) * ((b.M + C::BM - 1) / C::BM);
  if (ta == 0 || tb == 0) {
    if (ta > 0) launch_cfg<C>(a, stream);
    if (tb > 0) launch_cfg<C>(b, stream);
    return;
  }
  hipLaunchKernelGGL(gemm_kernel<C>, dim3(ta + tb), dim3(C::THREADS), 0, stream, a, b, ta);
}

// Two independent products in one launch: square tiles, or half-height tiles
// when square ones would leave half the CUs idle (the backward's dA and dB at
// 1024 rows: 128 square tiles).
void launch_pair(const GemmParams& a, const GemmParams& b, hipStream_t stream) {
  using C = CfgSquare;
  const long tiles = long((a.N + C::BN - 1) / C::BN) * ((a.M + C::BM - 1) / C::BM) +
                     long((b.N + C::BN - 1) / C::BN) * ((b.M + C::BM - 1) / C::BM);
  if (tiles <= 128)
    launch_pair_cfg<CfgHalf>(a, b, stream);
  else
    launch_pair_cfg<C>(a, b, stream);
}

// Wide tiles when they fill the machine in whole waves of workgroups (or many
// of them), square tiles otherwise.
bool use_wide(int M, int N) {
  using W = CfgWide;
  const long tiles = long((M + W::BM - 1) / W::BM) * ((N + W::BN - 1) / W::BN);
  return tiles % 256 == 0 || tiles >= 1024;
}

// Square tiles run as two k groups of 4 waves of 64 x 64 (fewer LDS bytes per
// MFMA than 8 waves of 64 x 32): measured 48.1 -> 47.9 us at 4096 x 4096 and
// 145.6 -> 143.8 us for the MLP-shape backward, whose dX runs here.
// Products whose square tiles fill less than half the CUs (the looped stack's
// 2560-wide projections at 512 rows: 80 tiles) split the reduction into up to 8
// slices so about 256 workgroups run, each at least three reduction tiles long;
// the last slice of a tile adds the fp32 slice tiles in slice order.
struct SplitPlan {
  int ks;
  size_t part_bytes;
};
SplitPlan split_plan(int M, int N, int k0, int k1) {
  using C = CfgSquare;
  const int tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  const int kt = (k0 + C::BK - 1) / C::BK + (k1 + C::BK - 1) / C::BK;
  SplitPlan s{1, 0};
  if (use_wide(M, N) || tiles >= 128 || tiles > 16384) return s;
  int ks = 256 / tiles;
  if (ks > 8) ks = 8;
  if (ks > kt / 3) ks = kt / 3;
  if (ks < 2) return s;
  const int kper = (kt + ks - 1) / ks;
  s.ks = (kt + kper - 1) / kper;
  s.part_bytes = align256(size_t(tiles) * s.ks * C::BM * C::BN * 4);
  return s;
}

// Share of the CU slots the launch's rounds of workgroups fill (one workgroup per CU).
double round_fill(long tiles) { return double(tiles) / (256.0 * double((tiles + 255) / 256)); }

// 128 x 160 tiles where their rounds fill the CUs clearly better than square ones:
// the looped stack's gate and up (512 rows, 2560 -> 10240) are 320 square tiles, a
// quarter of the CUs taking a second, or 256 tiles of 160 columns in one round.
// Measured there: the seven projections 305 -> 270 us. The same tiles as 5 waves of
// 128 x 32 (one SIMD holding two of them), as 4 waves of 32 x 160, or with 64-wide
// reduction tiles in three stages: 272-274 us.
bool use_sq160(int M, int N) {
  const long rows = (M + 127) / 128;
  return round_fill(rows * ((N + 159) / 160)) > round_fill(rows * ((N + 127) / 128)) + 0.1;
}

// 256 x 256 tiles when they fill whole rounds of the CUs: each W tile is read by
// half as many row tiles as with 128-row tiles, which counts once the weights come
// from HBM. Measured on the seven projections of a 4096-hidden layer at 4096 rows:
// 1896 -> 1641 us per layer (q and o 175 -> 139 us, down 468 -> 382, gate and up
// 398 -> 375 back to back; after a cache flush q 217 -> 156, down 540 -> 423).
// 256 x 128 tiles there: 1734 us.
bool use_big(int M, int N) {
  const long t = long((M + CfgBig::BM - 1) / CfgBig::BM) * ((N + CfgBig::BN - 1) / CfgBig::BN);
  return t >= 256 && t % 256 == 0;
}

void launch_main(const GemmParams& g, hipStream_t stream, float* part = nullptr, unsigned* tickets = nullptr) {
  if (g.M == 0 || g.N == 0) return;
  if (use_big(g.M, g.N)) {
    launch_cfg<CfgBig>(g, stream);
    return;
  }
  if (use_wide(g.M, g.N)) {
    launch_cfg<CfgWide>(g, stream);
    return;
  }
  const SplitPlan sp = split_plan(g.M, g.N, g.seg[0].k, g.nseg > 1 ? g.seg[1].k : 0);
  if (sp.ks > 1 && part && tickets) {
    using C = CfgSquare;
    GemmParams gs = g;
    const int kt = (g.seg[0].k + C::BK - 1) / C::BK + (g.nseg > 1 ? (g.seg[1].k + C::BK - 1) / C::BK : 0);
    gs.kper = (kt + sp.ks - 1) / sp.ks;
    gs.part = part;
    gs.ticket = tickets;
    gs.nb1 = gs.nb2 = INT_MAX;
    const dim3 grid((g.N + C::BN - 1) / C::BN, (g.M + C::BM - 1) / C::BM, sp.ks);
    hipLaunchKernelGGL((gemm_kernel<C, true>), grid, dim3(C::THREADS), 0, stream, gs, gs, 0);
    return;
  }
  if (use_sq160(g.M, g.N)) {
    launch_cfg<CfgSq160>(g, stream);
    return;
  }
  launch_cfg<CfgSquareKG>(g, stream);
}

// Forward workspace: [tickets (64 KB, only ever tickets, so they stay zero between
// calls of any shape)] [T bf16 [M, r]] [small-M slice tiles fp32 [KS, M, max(N, r)]].
constexpr size_t kTicketBytes = 65536;
constexpr int kMaxTickets = int(kTicketBytes / 4);

int small_slices(int M, int N, int K) { return use_skinny2(M, N, K) ? 1 : skinny_slices(N, K); }

void launch_small(const SkinnyParams& p, hipStream_t stream) {
  if (use_skinny2(p.M, p.N, p.K))
    launch_skinny2(p, stream);
  else
    launch_skinny(p, stream);
}

// Reduction slices of the forward's LoRA-down on the tiled path: two when the
// tiles alone would leave CUs idle and their tickets fit the ticket area, four
// when they fill a quarter of the CUs at most and the reduction is long.
// (Measured at the Qwen shapes, 128 tiles: two slices 1.8 us faster per call than
// one; three and four, which take a second round of workgroups, 4-6 us slower.
// At the looped stack's 512 rows and rank 64, 32 tiles: the seven projections in
// 315.8 us with two slices, 305.1 with four, 304.3 with eight.)
int fwd_lora_slices(int M, int K, int r) {
  const int tiles = ((M + 31) / 32) * ((r + 31) / 32);
  if (tiles <= 64 && K >= 2048) return 4;
  return (tiles <= 128 && K >= 1024) ? 2 : 1;
}

// Small-M products at 17-64 rows that are not wide enough for the streaming form
// run on 64-row tiles (the tiled kernel's loads: 256-byte runs of W rows through
// LDS, not the small-M kernel's 64-byte operand-order loads) with the reduction
// in about 256 / tiles slices (at most 8) of at least two reduction tiles. The
// slice count depends on K alone, so the workspace size does not depend on the
// rank; the delta tiles join the last slice's range.
template <class C>
int tiled_small_slices(int M, int N, int K) {
  const int tiles = ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
  const int kt = (K + C::BK - 1) / C::BK;
  int ks = 256 / tiles;                              // one round of workgroups
  if (ks > 8) ks = 8;
  if (ks > kt / 2) ks = kt / 2;
  return ks < 1 ? 1 : ks;
}

// Workgroups per CU-slot of the launch on C's tiles (1: every CU busy in every round).
template <class C>
double tiled_small_fill(int M, int N, int K) {
  const long w = long((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM) * tiled_small_slices<C>(M, N, K);
  return double(w) / (256.0 * double((w + 255) / 256));
}

// Whether C's column tiles fit the groups: each group boundary on a tile boundary.
template <class C>
bool groups_align(const GemmArgs& a) {
  for (int g = 0; g + 1 < a.groups; ++g)
    if (a.gstart[g] % C::BN != 0) return false;   // a column tile reads one group's delta rows
  return (a.N + C::BN - 1) / C::BN <= kMaxTickets;
}

// Column tiles of 128, or of 96 where those fill the CUs better (gate | up at
// 24576 columns: 256 tiles of 96 against 192 of 128, 75% of the CUs). 0: neither
// fits the groups.
int row_tile_bn(const GemmArgs& a) {
  const bool ok128 = groups_align<CfgRow>(a), ok96 = groups_align<CfgRow96>(a);
  if (ok96 && (!ok128 || tiled_small_fill<CfgRow96>(a.M, a.N, a.K) > tiled_small_fill<CfgRow>(a.M, a.N, a.K) + 0.05))
    return 96;
  return ok128 ? 128 : 0;
}

// Where it won (measured per product, weights from HBM): at 33-64 rows every
// decode-step product (4096 -> 12288 at 64 rows 62.4 -> 38.5 us, 12288 -> 4096
// 60.4 -> 43.6, 4096 -> 4096 18.7 -> 15.0); at 17-32 rows the large ones (4096 ->
// 12288 at 32 rows 44.7 -> 35.6 us) and the looped stack's step as a whole (12.8
// -> 10.4 ms), but not the smallest (4096 -> 1024 at 32 rows 16.7 -> 18.9 us).
bool tiled_small_ok(const GemmArgs& a) {
  if (a.M <= 16 || a.M > 64 || a.y_f32 || use_skinny2(a.M, a.N, a.K)) return false;
  if (a.M <= 32 && size_t(a.N) * a.K < (size_t(6) << 20)) return false;
  return row_tile_bn(a) != 0;
}

template <class C>
size_t tiled_small_part_bytes_c(int M, int N, int K) {
  const int ks = tiled_small_slices<C>(M, N, K);
  if (ks <= 1) return 0;
  return align256(size_t((N + C::BN - 1) / C::BN) * ks * C::BM * C::BN * 4);
}

// Either tile width's slice tiles (the groups, which pick it, are not known here).
size_t tiled_small_part_bytes(int M, int N, int K, int r) {
  if (M <= 16 || M > 64 || use_skinny2(M, N, K)) return 0;
  return std::max(tiled_small_part_bytes_c<CfgRow>(M, N, K), tiled_small_part_bytes_c<CfgRow96>(M, N, K));
}

template <class C>
void launch_tiled_small_c(GemmParams g, float* part, unsigned* tickets, hipStream_t stream) {
  const int k0t = (g.seg[0].k + C::BK - 1) / C::BK;
  const int kt = k0t + (g.nseg > 1 ? (g.seg[1].k + C::BK - 1) / C::BK : 0);
  const int ks = tiled_small_slices<C>(g.M, g.N, g.seg[0].k);
  g.kper = (k0t + ks - 1) / ks;
  if (ks * g.kper < kt) g.kper = (kt + ks - 1) / ks;   // the last slice takes the delta tiles too
  g.part = part;
  g.ticket = tickets;
  const dim3 grid((g.N + C::BN - 1) / C::BN, (g.M + C::BM - 1) / C::BM, ks);
  hipLaunchKernelGGL((gemm_kernel<C, true>), grid, dim3(C::THREADS), 0, stream, g, g, 0);
}

void launch_tiled_small(const GemmParams& g, int bn, float* part, unsigned* tickets, hipStream_t stream) {
  if (bn == 96)
    launch_tiled_small_c<CfgRow96>(g, part, tickets, stream);
  else
    launch_tiled_small_c<CfgRow>(g, part, tickets, stream);
}

size_t skinny_part_bytes(int M, int N, int K, int r) {
  int ks = small_slices(M, N, K), ks_r = r > 0 ? small_slices(M, r, K) : 1;
  size_t big = 0;
  if (ks > 1) big = size_t(ks) * M * N * 4;
  if (ks_r > 1 && size_t(ks_r) * M * r * 4 > big) big = size_t(ks_r) * M * r * 4;
  const size_t ts = tiled_small_part_bytes(M, N, K, r);
  if (ts > big) big = ts;
  return align256(big);
}

}  // namespace

size_t gemm_workspace_bytes(int M, int N, int K, int r) {
  if (M <= 0 || N <= 0) return 256;
  size_t n = kTicketBytes + (r > 0 ? align256(size_t(M) * r * 2) : 0);
  // One region serves whichever path runs: the small-M slice tiles or the
  // LoRA-down's slice tiles.
  const size_t sk = (M <= 64 && K % SK_GROUP == 0 && r % 32 == 0) ? skinny_part_bytes(M, N, K, r) : 0;
  size_t ld = r > 0 ? align256(size_t((M + 31) / 32) * ((r + 31) / 32) * LD_MAX_SLICES * 1024 * 4) : 0;
  const size_t sp = split_plan(M, N, K, r).part_bytes;   // the main product's slice tiles (after the LoRA-down)
  if (sp > ld) ld = sp;
  return n + (sk > ld ? sk : ld);
}

bool gemm_gathers_x(const GemmArgs& a) {
  // the gathered X exists on the small-M path's one-pass kernels only
  const int rt = a.r * a.groups;
  const bool small = skinny_ok(a.M, a.N, a.K, a.r, a.X, a.W, a.A, a.B) &&
                     (a.N + SK_COLS - 1) / SK_COLS <= kMaxTickets && (rt + SK_COLS - 1) / SK_COLS <= kMaxTickets;
  return a.x_group > 0 && small && !use_skinny2(a.M, a.N, a.K) && !use_skinny2(a.M, rt, a.K) &&
         (a.K / SK_GROUP) % a.x_group == 0 && size_t(a.K / SK_GROUP) * a.x_group < (size_t(1) << 20) &&
         a.x_stride >= a.K / a.x_group &&
         size_t(a.M) * a.x_stride * 2 < (size_t(1) << 32);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  char* ws = static_cast<char*>(a.ws);
  unsigned* tickets = a.tickets;
  if (tickets == nullptr) {
    tickets = reinterpret_cast<unsigned*>(ws);
    ws += kTicketBytes;
  }
  uint16_t* tws = reinterpret_cast<uint16_t*>(ws);
  const int rt = a.r * a.groups;                  // columns of T
  float* part = reinterpret_cast<float*>(ws + (a.r > 0 ? align256(size_t(a.M) * rt * 2) : 0));
  const bool small = skinny_ok(a.M, a.N, a.K, a.r, a.X, a.W, a.A, a.B) &&
                     (a.N + SK_COLS - 1) / SK_COLS <= kMaxTickets && (rt + SK_COLS - 1) / SK_COLS <= kMaxTickets;
  if (a.y_f32 && !small) return hipErrorInvalidValue;   // fp32 output exists on the small-M path only
  if (a.groups < 1 || a.groups > 3 || (a.groups > 1 && !small)) return hipErrorInvalidValue;
  if (a.x_group < 0 || (a.x_group > 0 && !gemm_gathers_x(a))) return hipErrorInvalidValue;
  if (small) {
    SkinnyParams p{};
    p.M = a.M;
    p.K = a.K;
    p.x_stride = a.x_stride;
    p.x_group = a.x_group;
    p.part = part;
    p.ticket = tickets;
    p.x = static_cast<const uint16_t*>(a.X);
    p.t_stride = rt;
    p.nb1 = a.groups > 1 ? a.gstart[0] : INT_MAX;
    p.nb2 = a.groups > 2 ? a.gstart[1] : INT_MAX;
    if (a.r > 0 && a.x_group == 0 && a.M > 32) {
      // T = bf16(s * diag(mask) X A^T) at 33-64 rows by the tiled LoRA-down, the
      // reduction in up to 8 slices (the groups' A blocks stacked: T holds their
      // delta rows side by side). Measured on the Qwen-shaped Uno step (64 rows):
      // 11.26 -> 11.02 ms; at 32 rows (the looped stack) the small-M kernel's form
      // below stays ahead (9.66 against 9.70 ms).
      const int ks = a.K / 512 < 1 ? 1 : (a.K / 512 > LD_MAX_SLICES ? LD_MAX_SLICES : a.K / 512);
      launch_lora_down(static_cast<const uint16_t*>(a.X), static_cast<const uint16_t*>(a.A), a.M, a.K, rt, a.scale,
                       tws, a.row_mask, ks, part, tickets, stream);
    } else if (a.r > 0) {
      // The same product with A in place of W, on the small-M kernel.
      p.w = static_cast<const uint16_t*>(a.A);
      p.N = rt;
      p.r = 0;
      p.KS = small_slices(a.M, rt, a.K);
      p.scale = a.scale;
      p.mask = a.row_mask;
      p.y = tws;
      launch_small(p, stream);
    }
    if (tiled_small_ok(a)) {
      GemmParams g{};
      g.seg[0] = Seg{static_cast<const uint16_t*>(a.X), static_cast<const uint16_t*>(a.W), a.K};
      g.nseg = 1;
      if (a.r > 0) {
        g.seg[1] = Seg{tws, static_cast<const uint16_t*>(a.B), a.r};   // scaled and gated already
        g.nseg = 2;
      }
      g.M = a.M;
      g.N = a.N;
      g.y = static_cast<uint16_t*>(a.Y);
      g.t_stride = rt;
      g.nb1 = a.groups > 1 ? a.gstart[0] : INT_MAX;
      g.nb2 = a.groups > 2 ? a.gstart[1] : INT_MAX;
      g.x_stride = a.x_stride;
      g.x_group = a.x_group;
      launch_tiled_small(g, row_tile_bn(a), part, tickets, stream);
      return hipGetLastError();
    }
    p.w = static_cast<const uint16_t*>(a.W);
    p.N = a.N;
    p.r = a.r;
    p.t = a.r > 0 ? tws : nullptr;
    p.b = static_cast<const uint16_t*>(a.B);
    p.KS = small_slices(a.M, a.N, a.K);
    p.scale = 1.0f;
    p.mask = nullptr;
    p.y = a.y_f32 ? nullptr : static_cast<uint16_t*>(a.Y);
    p.yf = a.y_f32 ? static_cast<float*>(a.Y) : nullptr;
    launch_small(p, stream);
    return hipGetLastError();
  }
  const uint16_t* tmat = nullptr;
  if (a.r > 0) {
    launch_lora_down(static_cast<const uint16_t*>(a.X), static_cast<const uint16_t*>(a.A), a.M, a.K, a.r, a.scale,
                     tws, nullptr, fwd_lora_slices(a.M, a.K, a.r), part, tickets, stream);
    tmat = tws;
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
  launch_main(g, stream, part, tickets);
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
// Backward workspace: [tickets (64 KB, zero between calls, first so that they keep
// their place across shapes)] [T] [B^T] [U] [W^T] [A^T] [U^T] [X^T] [dY^T] [T^T]
// [LoRA-down slice tiles].
struct BwdWs {
  unsigned* tickets;
  uint16_t *t, *bt, *u, *wt, *at, *ut, *xt, *dyt, *tt;
  float* part;
};
// The backward's two LoRA-downs, T = X A^T and U = s diag(m) dY B, with their
// slices balanced; the slice tiles' size in bytes.
void bwd_lora_jobs(int M, int N, int K, int r, LdJob& jt, LdJob& ju) {
  jt = lora_down_job(nullptr, nullptr, M, K, r, 1.0f, nullptr, nullptr);
  ju = lora_down_job(nullptr, nullptr, M, N, r, 1.0f, nullptr, nullptr);
  if (size_t(jt.tiles) + ju.tiles <= kTicketBytes / 4) balance_slices(jt, ju);
}
size_t bwd_part_bytes(int M, int N, int K, int r) {
  LdJob jt, ju;
  bwd_lora_jobs(M, N, K, r, jt, ju);
  size_t n = 0;
  if (jt.ks > 1) n += size_t(jt.tiles) * jt.ks * 1024 * 4;
  if (ju.ks > 1) n += size_t(ju.tiles) * ju.ks * 1024 * 4;
  const size_t dx = split_plan(M, K, N, r).part_bytes;     // dX's slice tiles, after the LoRA-down
  return align256(n > dx ? n : dx);
}
BwdWs bwd_ws(void* ws, int M, int N, int K, int r) {
  char* c = static_cast<char*>(ws);
  BwdWs w;
  w.tickets = reinterpret_cast<unsigned*>(c);
  c += kTicketBytes;
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
  w.part = reinterpret_cast<float*>(c);
  return w;
}
}  // namespace

size_t gemm_bwd_workspace_bytes(int M, int N, int K, int r) {
  if (M <= 0 || N <= 0 || K <= 0 || r <= 0) return 256;
  const size_t m = M, n = N, k = K, rr = r;
  return kTicketBytes + align256(m * rr * 2) * 3 + align256(rr * n * 2) + align256(k * n * 2) +
         align256(k * rr * 2) + align256(rr * m * 2) + align256(k * m * 2) + align256(n * m * 2) +
         bwd_part_bytes(M, N, K, r);
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
  const uint16_t* wt = static_cast<const uint16_t*>(a.Wt);
  // 1. The weight transposes, one launch: B^T for U; A^T (and W^T when not given)
  //    for dX.
  {
    Transposes t;
    t.add(B, N, r, w.bt, nullptr, 1.0f);
    if (a.dX) {
      t.add(A, r, K, w.at, nullptr, 1.0f);
      if (!wt) t.add(W, N, K, w.wt, nullptr, 1.0f);
    }
    t.launch(stream);
    if (a.dX && !wt) wt = w.wt;
  }
  // 2. T = X A^T (unscaled, every row) and U = bf16(s diag(m) dY B), one launch,
  //    the longer reduction in slices; their epilogues also write (s T)^T and U^T
  //    for dB and dA, and their chunks X^T for dA and (diag(m) dY)^T for dB
  //    (masked rows zeroed).
  {
    LdJob jobs[2];
    bwd_lora_jobs(M, N, K, r, jobs[0], jobs[1]);
    const int ks_t = jobs[0].ks, ks_u = jobs[1].ks;
    jobs[0] = lora_down_job(X, A, M, K, r, 1.0f, w.t, nullptr, w.tt, a.scale, w.xt);
    jobs[1] = lora_down_job(dY, w.bt, M, N, r, a.scale, w.u, a.row_mask, w.ut, 1.0f, w.dyt);
    jobs[0].ks = ks_t;
    jobs[1].ks = ks_u;
    float* part = w.part;
    for (int i = 0; i < 2; ++i) {
      jobs[i].ticket = w.tickets + (i == 0 ? 0 : jobs[0].tiles);
      if (jobs[i].ks > 1) {
        jobs[i].part = part;
        part += size_t(jobs[i].tiles) * jobs[i].ks * 1024;
      }
    }
    launch_lora_downs(jobs, 2, stream);
  }
  // 3. dX = [dY | U] [W^T | A^T]^T
  if (a.dX) {
    GemmParams g{};
    g.seg[0] = Seg{dY, wt, N};
    g.seg[1] = Seg{w.u, w.at, r};
    g.nseg = 2;
    g.M = M;
    g.N = K;
    g.y = static_cast<uint16_t*>(a.dX);
    launch_main(g, stream, w.part, w.tickets);   // the LoRA-down's slices are done with both
  }
  // 4. dA = U^T X (rows of U^T against rows of X^T, reduction over M) and dB =
  //    (diag(m) dY)^T (s T), one launch.
  {
    GemmParams ga{};
    ga.seg[0] = Seg{w.ut, w.xt, M};
    ga.nseg = 1;
    ga.M = r;
    ga.N = K;
    ga.y = static_cast<uint16_t*>(a.dA);
    GemmParams gb{};
    gb.seg[0] = Seg{w.dyt, w.tt, M};
    gb.nseg = 1;
    gb.M = N;
    gb.N = r;
    gb.y = static_cast<uint16_t*>(a.dB);
    launch_pair(ga, gb, stream);
  }
  return hipGetLastError();
}

}  // namespace uno
