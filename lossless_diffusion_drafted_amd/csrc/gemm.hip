// Row-gated LoRA linear on gfx950 matrix cores ("Uno Qwen3-8B" model card and
// "LoopUno", "Setup / Recipe": a LoRA adapter whose update is switched on only
// for the rows of the block being denoised; seed/verify rows see the frozen
// weights).
//
//   Y = X W^T + s * diag(mask) (X A^T) B^T,   X [M,K], W [N,K], A [r,K], B [N,r].
//
// Two launches:
//  1. LoRA-down T' = bf16(s * mask[m] * X A^T): a skinny GEMM (N = r), split
//     over K into fp32 partials, then reduced in a fixed order, scaled, gated and
//     rounded to bf16 (deterministic).
//  2. The main GEMM over the extended reduction [X | T'] [W | B]^T: the gated
//     delta is just r more reduction steps after the K steps. Rows with mask 0
//     have T' = 0, so they add exact zeros and equal the plain X W^T bit for bit.
// Tiles: 128 x 128 x 64 per 256-thread workgroup, each wave 64 x 64 as 2 x 2
// blocks of v_mfma_f32_32x32x16_bf16; operands staged through double-buffered
// LDS with a 144-byte row pitch (conflict-free 16-byte fragment reads).

#include "../../include/uno.h"
#include "common.h"
#include "kernels.h"

namespace uno {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int GT = 256;                 // threads per workgroup (4 waves, 2 x 2)
constexpr int PITCH = BK + 8;           // bf16 per LDS row: 144 bytes
constexpr int TILE_ELEMS = BM * PITCH;  // one operand tile in LDS (BM == BN)
constexpr int LOADS = BM * BK / 8 / GT; // 16-byte chunks per thread per operand tile

struct Seg {
  const uint16_t* a;   // [rows_a, k] row-major (X or T')
  const uint16_t* b;   // [rows_b, k] row-major (W, A or B)
  int k;               // reduction length of this segment (multiple of 8)
};

struct GemmParams {
  Seg seg[2];
  int nseg;
  int M, N;
  int ktiles0;         // reduction tiles of segment 0 handled by one split
  int mode;            // 0: bf16 Y [M, N]; 1: fp32 partials P[split][M][N]
  uint16_t* y;
  float* part;
};

__device__ __forceinline__ uint4 load_chunk(__amdgpu_buffer_rsrc_t rs, uint32_t off, bool ok) {
  // Offsets past the range read zero; an invalid chunk is sent out of range.
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off : 0xffffffffu, 0u, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// One operand tile: rows r0..r0+127 of a [rows, k] matrix, columns k0..k0+63;
// columns at or past `kk` (k, or 0 for a tile past the end) read zero.
__device__ __forceinline__ void load_tile(const uint16_t* base, int rows, int k, int r0, int k0, int kk,
                                          uint4 (&reg)[LOADS]) {
  const __amdgpu_buffer_rsrc_t rs = make_row_rsrc(base, uint32_t(size_t(rows) * size_t(k) * 2u));
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int c = int(threadIdx.x) + i * GT;
    const int row = c >> 3, col = (c & 7) * 8;
    const bool ok = (r0 + row < rows) && (k0 + col < kk);
    reg[i] = load_chunk(rs, uint32_t((size_t(r0 + row) * size_t(k) + size_t(k0 + col)) * 2u), ok);
  }
}

__device__ __forceinline__ void store_tile(uint16_t* lds, const uint4 (&reg)[LOADS]) {
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int c = int(threadIdx.x) + i * GT;
    const int row = c >> 3, col = (c & 7) * 8;
    *reinterpret_cast<uint4*>(lds + row * PITCH + col) = reg[i];
  }
}

__global__ __launch_bounds__(GT) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][TILE_ELEMS];   // [buffer][A|B]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int split = blockIdx.z;

  // Reduction tiles of this workgroup: a range of segment 0, then (single split
  // only) every tile of segment 1.
  const int kt_all0 = (p.seg[0].k + BK - 1) / BK;
  const int t_begin = split * p.ktiles0;
  const int t_end0 = min(kt_all0, t_begin + p.ktiles0);
  const int n0tiles = max(0, t_end0 - t_begin);
  const int n1tiles = p.nseg > 1 ? (p.seg[1].k + BK - 1) / BK : 0;
  const int ntiles = n0tiles + n1tiles;

  // Tiles at or past the end are fetched with out-of-range offsets (zeros, no
  // memory traffic), so every step issues the same loads without branches.
  auto fetch = [&](int t, uint4 (&ra)[LOADS], uint4 (&rb)[LOADS]) {
    const Seg& sg = t < n0tiles ? p.seg[0] : p.seg[p.nseg - 1];
    const int k0 = t < n0tiles ? (t_begin + t) * BK : (t - n0tiles) * BK;
    const int kk = t < ntiles ? sg.k : 0;
    load_tile(sg.a, p.M, sg.k, m0, k0, kk, ra);
    load_tile(sg.b, p.N, sg.k, n0, k0, kk, rb);
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Fragment addresses: lane l holds row (l % 32) and k = 8 (l / 32) .. +7 of
  // each 32 x 16 slice.
  const int frow = lane & 31, fk = (lane >> 5) * 8;
  auto compute = [&](const uint16_t* As, const uint16_t* Bs) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 64 + i * 32 + frow) * PITCH + ks * 16 + fk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * 64 + j * 32 + frow) * PITCH + ks * 16 + fk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  // Two register stages: the loads of tile t+2 are in flight while tile t is
  // multiplied out of LDS and tile t+1 waits in registers.
  uint4 ra0[LOADS], rb0[LOADS], ra1[LOADS], rb1[LOADS];
  fetch(0, ra0, rb0);
  fetch(1, ra1, rb1);
  store_tile(lds[0][0], ra0);
  store_tile(lds[0][1], rb0);
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    fetch(t + 2, ra0, rb0);
    compute(lds[0][0], lds[0][1]);
    store_tile(lds[1][0], ra1);
    store_tile(lds[1][1], rb1);
    __syncthreads();
    if (t + 1 < ntiles) {
      fetch(t + 3, ra1, rb1);
      compute(lds[1][0], lds[1][1]);
      store_tile(lds[0][0], ra0);
      store_tile(lds[0][1], rb0);
      __syncthreads();
    }
  }

  // Epilogue. Accumulator v of a 32 x 32 block sits at row 8 (v / 4) + 4 (l / 32)
  // + v % 4 and column l % 32.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < p.M && col < p.N) {
          if (p.mode == 0)
            p.y[size_t(row) * p.N + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][v]);
          else
            p.part[(size_t(split) * p.M + row) * p.N + col] = acc[i][j][v];
        }
      }
    }
  }
}

// T'[m, j] = bf16(scale * mask[m] * sum_z part[z][m][j]), z in increasing order.
__global__ __launch_bounds__(256) void lora_reduce_kernel(const float* part, int splits, int M, int r,
                                                          const uint8_t* mask, float scale, uint16_t* t) {
  const size_t n = size_t(M) * r;
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += size_t(gridDim.x) * 256) {
    float s = 0.0f;
    for (int z = 0; z < splits; ++z) s += part[size_t(z) * n + i];
    const int m = int(i / size_t(r));
    const float v = mask[m] ? scale * s : 0.0f;
    t[i] = __builtin_bit_cast(uint16_t, (__bf16)v);
  }
}

struct Plan {
  int splits, ktiles_per_split;
};

// Split the LoRA-down reduction so that about 256 workgroups run.
Plan lora_plan(int M, int K, int r) {
  const int tiles = ((M + BM - 1) / BM) * ((r + BN - 1) / BN);
  const int kt = (K + BK - 1) / BK;
  int splits = 256 / (tiles > 0 ? tiles : 1);
  const int max_splits = (kt + 3) / 4;           // at least 4 reduction tiles per split
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  const int per = (kt + splits - 1) / splits;
  Plan pl;
  pl.ktiles_per_split = per;
  pl.splits = (kt + per - 1) / per;
  return pl;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t gemm_workspace_bytes(int M, int N, int K, int r) {
  (void)N;
  if (r <= 0 || M <= 0) return 256;
  const Plan pl = lora_plan(M, K, r);
  return align256(size_t(pl.splits) * M * r * 4) + align256(size_t(M) * r * 2);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const uint16_t* tprime = nullptr;
  if (a.r > 0) {
    const Plan pl = lora_plan(a.M, a.K, a.r);
    float* part = static_cast<float*>(a.ws);
    uint16_t* t = reinterpret_cast<uint16_t*>(static_cast<char*>(a.ws) +
                                              align256(size_t(pl.splits) * a.M * a.r * 4));
    GemmParams d{};
    d.seg[0] = Seg{static_cast<const uint16_t*>(a.X), static_cast<const uint16_t*>(a.A), a.K};
    d.nseg = 1;
    d.M = a.M;
    d.N = a.r;
    d.ktiles0 = pl.ktiles_per_split;
    d.mode = 1;
    d.part = part;
    dim3 grid((a.r + BN - 1) / BN, (a.M + BM - 1) / BM, pl.splits);
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(GT), 0, stream, d);
    const size_t n = size_t(a.M) * a.r;
    const int rb = int((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
    hipLaunchKernelGGL(lora_reduce_kernel, dim3(rb), dim3(256), 0, stream, part, pl.splits, a.M, a.r,
                       a.row_mask, a.scale, t);
    tprime = t;
  }
  GemmParams g{};
  g.seg[0] = Seg{static_cast<const uint16_t*>(a.X), static_cast<const uint16_t*>(a.W), a.K};
  g.nseg = 1;
  if (a.r > 0) {
    g.seg[1] = Seg{tprime, static_cast<const uint16_t*>(a.B), a.r};
    g.nseg = 2;
  }
  g.M = a.M;
  g.N = a.N;
  g.ktiles0 = (a.K + BK - 1) / BK;
  g.mode = 0;
  g.y = static_cast<uint16_t*>(a.Y);
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM, 1);
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(GT), 0, stream, g);
  return hipGetLastError();
}

}  // namespace uno
