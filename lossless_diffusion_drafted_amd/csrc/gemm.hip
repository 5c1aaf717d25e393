// Row-gated LoRA linear on gfx950 matrix cores ("Uno Qwen3-8B" model card and
// "LoopUno", "Setup / Recipe": a LoRA adapter whose update is switched on only
// for the rows of the block being denoised; seed/verify rows see the frozen
// weights).
//
//   Y = X W^T + s * diag(mask) (X A^T) B^T,   X [M,K], W [N,K], A [r,K], B [N,r].
//
// Two phases:
//  1. LoRA-down T = bf16(s * X A^T): a skinny GEMM (N = r), split over K across
//     workgroups; the last slice of each tile sums the fp32 partials in slice
//     order (deterministic), scales and rounds.
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

using CfgWide = Cfg<256, 192, 32, 4, 2, 4>;   // 8 waves of 64 x 96
using CfgSquare = Cfg<128, 128, 64, 2, 4, 2>; // 8 waves of 64 x 32

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
// Workgroup (x, y, z): rows 32y .. 32y+31, columns 128x .. 128x+127 (wave w takes
// 32 of them) over reduction slice z. Lanes load their MFMA fragments straight
// from global memory (16 bytes per operand per step), LD_U steps per batch with
// the next batch in flight. Each slice writes its fp32 partial with
// device-coherent stores; the last slice of a tile (per-tile ticket) reads all
// partials with device-coherent 16-byte loads, sums them in slice order, scales,
// rounds to bf16 and resets the ticket. The result does not depend on the order
// in which slices finish.
constexpr int LD_ROWS = 32, LD_COLS = 128, LD_U = 8, LD_MAX_SPLITS = 16;
constexpr int kCoherent = 16;            // buffer cache policy: device scope (sc1)

__device__ __forceinline__ void ld_batch(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t ra, uint32_t xb,
                                         uint32_t ab, bool xrow, bool arow, int k, int ke, int fh,
                                         bf16x8_t (&xf)[LD_U], bf16x8_t (&af)[LD_U]) {
#pragma unroll
  for (int u = 0; u < LD_U; ++u) {
    const int kk = k + 16 * u;
    const bool in = kk + fh < ke;
    xf[u] = __builtin_bit_cast(bf16x8_t,
                               __builtin_amdgcn_raw_buffer_load_b128(rx, (xrow && in) ? xb + kk * 2 : kOutOfRange, 0u, 0));
    af[u] = __builtin_bit_cast(bf16x8_t,
                               __builtin_amdgcn_raw_buffer_load_b128(ra, (arow && in) ? ab + kk * 2 : kOutOfRange, 0u, 0));
  }
}

__global__ __launch_bounds__(256) void lora_down_kernel(const uint16_t* X, const uint16_t* A, int M, int K, int r,
                                                        int kslice, float scale, float* part, unsigned* tickets,
                                                        uint16_t* T) {
  __shared__ int last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = blockIdx.y * LD_ROWS, cb = blockIdx.x * LD_COLS, c0 = cb + wave * 32;
  const int splits = gridDim.z, z = blockIdx.z;
  const int kb = z * kslice, ke = min(K, kb + kslice);
  const int fr = lane & 31, fh = (lane >> 5) * 8;
  const __amdgpu_buffer_rsrc_t rx = make_row_rsrc(X, uint32_t(size_t(M) * K * 2));
  const __amdgpu_buffer_rsrc_t ra = make_row_rsrc(A, uint32_t(size_t(r) * K * 2));
  const bool xrow = m0 + fr < M, arow = c0 + fr < r;
  const uint32_t xb = uint32_t((size_t(m0 + fr) * K + fh) * 2);
  const uint32_t ab = uint32_t((size_t(c0 + fr) * K + fh) * 2);
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  bf16x8_t x0[LD_U], a0[LD_U], x1[LD_U], a1[LD_U];
  ld_batch(rx, ra, xb, ab, xrow, arow, kb, ke, fh, x0, a0);
  for (int k = kb; k < ke; k += 32 * LD_U) {
    ld_batch(rx, ra, xb, ab, xrow, arow, k + 16 * LD_U, ke, fh, x1, a1);
#pragma unroll
    for (int u = 0; u < LD_U; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0[u], a0[u], acc, 0, 0, 0);
    ld_batch(rx, ra, xb, ab, xrow, arow, k + 32 * LD_U, ke, fh, x0, a0);
#pragma unroll
    for (int u = 0; u < LD_U; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x1[u], a1[u], acc, 0, 0, 0);
  }
  // Partial of this slice, as [split][M][rpad] (rpad = r rounded up to 128, so the
  // reduction reads whole 16-byte groups). Accumulator v sits at row
  // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
  const int rpad = gridDim.x * LD_COLS;
  const size_t plane = size_t(M) * rpad;
  const __amdgpu_buffer_rsrc_t rp = make_row_rsrc(part, uint32_t(size_t(splits) * plane * 4));
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = m0 + 8 * (v >> 2) + (fh >> 1) + (v & 3);
    const uint32_t off = row < M ? uint32_t((z * plane + size_t(row) * rpad + c0 + fr) * 4) : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[v]), rp, off, 0u, kCoherent);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unsigned* ticket = tickets + blockIdx.y * gridDim.x + blockIdx.x;
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == unsigned(splits - 1);
  __syncthreads();
  if (!last) return;
  // 32 x 128 tile = 1024 groups of 4 columns; 4 groups per thread, every split's
  // loads issued before any is summed.
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int gi = threadIdx.x + g * 256;
    const int row = m0 + gi / (LD_COLS / 4), col = cb + (gi % (LD_COLS / 4)) * 4;
    u32x4_t v[LD_MAX_SPLITS];
#pragma unroll
    for (int zz = 0; zz < LD_MAX_SPLITS; ++zz) {
      const uint32_t off = (zz < splits && row < M) ? uint32_t((zz * plane + size_t(row) * rpad + col) * 4) : kOutOfRange;
      v[zz] = __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0u, kCoherent);
    }
    float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int zz = 0; zz < LD_MAX_SPLITS; ++zz) {
      if (zz < splits) {
        sum[0] += __uint_as_float(v[zz].x);
        sum[1] += __uint_as_float(v[zz].y);
        sum[2] += __uint_as_float(v[zz].z);
        sum[3] += __uint_as_float(v[zz].w);
      }
    }
    if (row < M) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < r) T[size_t(row) * r + col + e] = __builtin_bit_cast(uint16_t, (__bf16)(scale * sum[e]));
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Plan {
  int tx, ty, splits, kslice;
};

// LoRA-down grid: about 256 workgroups, reduction slices of at least 128.
Plan lora_plan(int M, int K, int r) {
  Plan pl;
  pl.tx = (r + LD_COLS - 1) / LD_COLS;
  pl.ty = (M + LD_ROWS - 1) / LD_ROWS;
  int splits = 256 / (pl.tx * pl.ty);
  const int max_splits = (K + 127) / 128;
  if (splits > max_splits) splits = max_splits;
  if (splits > LD_MAX_SPLITS) splits = LD_MAX_SPLITS;
  if (splits < 1) splits = 1;
  pl.kslice = ((K + splits - 1) / splits + 15) / 16 * 16;
  pl.splits = (K + pl.kslice - 1) / pl.kslice;
  return pl;
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

}  // namespace

size_t gemm_workspace_bytes(int M, int N, int K, int r) {
  (void)N;
  if (r <= 0 || M <= 0) return 256;
  const Plan pl = lora_plan(M, K, r);
  return align256(size_t(pl.tx) * pl.ty * 4) + align256(size_t(pl.splits) * M * pl.tx * LD_COLS * 4) +
         align256(size_t(M) * r * 2);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const uint16_t* tmat = nullptr;
  if (a.r > 0) {
    // workspace: [tickets (left at zero by every call) | fp32 partials | T bf16 [M, r]]
    const Plan pl = lora_plan(a.M, a.K, a.r);
    char* ws = static_cast<char*>(a.ws);
    unsigned* tickets = reinterpret_cast<unsigned*>(ws);
    const size_t off_part = align256(size_t(pl.tx) * pl.ty * 4);
    float* part = reinterpret_cast<float*>(ws + off_part);
    uint16_t* t = reinterpret_cast<uint16_t*>(ws + off_part + align256(size_t(pl.splits) * a.M * pl.tx * LD_COLS * 4));
    hipLaunchKernelGGL(lora_down_kernel, dim3(pl.tx, pl.ty, pl.splits), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.X), static_cast<const uint16_t*>(a.A), a.M, a.K, a.r,
                       pl.kslice, a.scale, part, tickets, t);
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
  if (use_wide(a.M, a.N))
    launch_cfg<CfgWide>(g, stream);
  else
    launch_cfg<CfgSquare>(g, stream);
  return hipGetLastError();
}

}  // namespace uno
