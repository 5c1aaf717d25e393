// Device helpers shared by the Uno HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uno {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element access. bf16 values widen to fp32 exactly by a 16-bit shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest even (finite values; NaN keeps a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Order-preserving unsigned key of a float. -0 takes the key of +0 so that equal
// values share a key (ties are decided on values, not on bit patterns).
__device__ __forceinline__ uint32_t float_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// 16-byte streaming load with the non-temporal hint (read-once data).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt lgkmcnt(0) (LDS, scalar memory) with the other counters left alone.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Raw buffer loads: a range-checked view of one row. Reads past num_records
// return zero instead of faulting, so every lane issues exactly one load per chunk
// and the compiler can count outstanding loads across a pipelined loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);   // gfx9-family dword3
}
// voff: per-lane byte offset; soff: wave-uniform byte offset (kept in an SGPR).
// The load carries the non-temporal cache policy: streamed data is read once,
// and on gfx950 this raises sustained read bandwidth (measured 6.0 -> 6.9 TB/s
// on a 600 MB row stream).
constexpr int kBufNonTemporal = 2;
// SC1 cache policy: the load is coherent across the device's L2s (what an
// agent-scope atomic load uses).
constexpr int kBufDeviceCoherent = 16;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kBufNonTemporal);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// Wave64 reductions (every lane gets the result). Row steps move values with DPP
// (no LDS): XOR 1 and XOR 2 inside each quad, then the mirror within each
// half-row and within the row; applied in that order to a commutative operation
// they leave the row's result in every lane of the row. The four row results are
// then read from lanes 0, 16, 32 and 48 and combined in that order, the same in
// every lane.
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_move(T v) {
  if constexpr (sizeof(T) == 8) {
    const long long b = __builtin_bit_cast(long long, v);
    const unsigned lo = unsigned(dpp_i<CTRL>(int(b & 0xffffffffll)));
    const unsigned hi = unsigned(dpp_i<CTRL>(int(b >> 32)));
    return __builtin_bit_cast(T, (long long)(((unsigned long long)hi << 32) | lo));
  } else {
    return __builtin_bit_cast(T, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
  }
}
template <typename T>
__device__ __forceinline__ T lane_read(T v, int l) {
  if constexpr (sizeof(T) == 8) {
    const long long b = __builtin_bit_cast(long long, v);
    const unsigned lo = unsigned(__builtin_amdgcn_readlane(int(b & 0xffffffffll), l));
    const unsigned hi = unsigned(__builtin_amdgcn_readlane(int(b >> 32), l));
    return __builtin_bit_cast(T, (long long)(((unsigned long long)hi << 32) | lo));
  } else {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  }
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp_move<kDppQuadXor1>(v));
  v = op(v, dpp_move<kDppQuadXor2>(v));
  v = op(v, dpp_move<kDppHalfMirror>(v));
  v = op(v, dpp_move<kDppMirror>(v));
  return op(op(lane_read(v, 0), lane_read(v, 16)), op(lane_read(v, 32), lane_read(v, 48)));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return wave_reduce(v, [](T a, T b) { return a + b; });
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
  return wave_reduce(v, [](T a, T b) { return b > a ? b : a; });
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
  return wave_reduce(v, [](T a, T b) { return b < a ? b : a; });
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return a | b; });
}
// Value of lane `l` (wave-uniform l) broadcast to every lane.
__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const long long b = __double_as_longlong(v);
  const unsigned lo = unsigned(__builtin_amdgcn_readlane(int(b & 0xffffffffll), l));
  const unsigned hi = unsigned(__builtin_amdgcn_readlane(int(b >> 32), l));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Sum / maximum over the 8 lanes of each half-row (lanes 0-7 hold the result
// for lanes 0-7).
__device__ __forceinline__ float lanes8_sum(float v) {
  v += dpp_move<kDppQuadXor1>(v);
  v += dpp_move<kDppQuadXor2>(v);
  return v + dpp_move<kDppHalfMirror>(v);
}
__device__ __forceinline__ float lanes8_max(float v) {
  v = fmaxf(v, dpp_move<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_move<kDppQuadXor2>(v));
  return fmaxf(v, dpp_move<kDppHalfMirror>(v));
}
// Wave64 sum / maximum without LDS: row reductions by DPP, then the four row
// results read from lanes 0, 16, 32, 48 (the same order in every lane).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = lanes8_sum(v);
  v += dpp_move<kDppMirror>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = lanes8_max(v);
  v = fmaxf(v, dpp_move<kDppMirror>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

// Inclusive prefix sum over lanes 0..63: the prefix within each row of 16 lanes by
// DPP row shifts of 1, 2, 4 and 8 (lanes shifted in from outside the row add 0),
// then the totals of the rows before, read from lanes 15, 31 and 47.
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
  v = v + dpp_move<kRowShr1>(v);
  v = v + dpp_move<kRowShr2>(v);
  v = v + dpp_move<kRowShr4>(v);
  v = v + dpp_move<kRowShr8>(v);
  const T s0 = lane_read(v, 15), s1 = lane_read(v, 31), s2 = lane_read(v, 47);
  const int row = int(threadIdx.x & (kWave - 1)) >> 4;
  T off = T(0);
  if (row >= 1) off = s0;
  if (row >= 2) off = off + s1;
  if (row >= 3) off = off + s2;
  return row == 0 ? v : v + off;
}

// ---------------------------------------------------------------------------
// Philox-4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11): two 64x64->128 multiplies per round, Weyl key schedule.
struct Philox4 { uint64_t w[4]; };

__device__ __forceinline__ Philox4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                                 uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += W0; k1 += W1;
  }
  Philox4 out;
  out.w[0] = c0; out.w[1] = c1; out.w[2] = c2; out.w[3] = c3;
  return out;
}

// Top 24 bits of a word as a uniform in [0, 1), exact in fp32 and fp64.
__device__ __forceinline__ double word_to_uniform(uint64_t w) {
  return double(w >> 40) * (1.0 / 16777216.0);
}

// Map a launch's workgroup id so that each of the 8 XCDs (which receive
// workgroups round-robin) works on one contiguous range of logical ids.
__device__ __forceinline__ int xcd_contiguous_id(int wg, int n) {
  if ((n & 7) != 0) return wg;
  return (wg & 7) * (n >> 3) + (wg >> 3);
}

}  // namespace uno
