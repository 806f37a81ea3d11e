// Device primitives for the gfx950 sampling kernels: wave64 reductions and
// scans, the Philox4x64-10 generator, float32 order keys.
//
// Reductions use xor-butterflies, so every lane of a wave ends with the same
// bits, and cross-wave combinations run in a fixed order through LDS: all
// results are deterministic run to run (no floating-point atomics).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dss {

constexpr int kWave = 64;
constexpr int kBlock = 1024;
constexpr int kWaves = kBlock / kWave;

// ---------------------------------------------------------------------------
// wave64 collectives
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) v = min(v, (uint32_t)__shfl_xor(v, m, kWave));
  return v;
}

// Inclusive prefix sum across the 64 lanes (Hillis-Steele).  Floating-point
// rounding can make neighbouring prefixes non-monotone; callers that locate a
// token guard against that explicitly.
__device__ __forceinline__ double wave_incl_scan(double v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    double y = __shfl_up(v, d, kWave);
    if (lane >= d) v += y;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 64x64->128-bit multiplies by fixed odd constants, a word permutation and a
// xor with the round key; the key is bumped by two Weyl constants between
// rounds.
// ---------------------------------------------------------------------------

struct Philox4x64 {
  uint64_t w[4];
};

__device__ __forceinline__ Philox4x64 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                                    uint64_t c3, uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull;
  constexpr uint64_t kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull;
  constexpr uint64_t kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t lo0 = kM0 * c0, hi0 = __umul64hi(kM0, c0);
    const uint64_t lo1 = kM1 * c2, hi1 = __umul64hi(kM1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  Philox4x64 out;
  out.w[0] = c0;
  out.w[1] = c1;
  out.w[2] = c2;
  out.w[3] = c3;
  return out;
}

// Draw r of the stream (seed, offset, sid): key (seed, 0), counter
// (offset, sid, r / 4, 0), word r % 4, top 53 bits as a uniform in [0, 1).
__device__ __forceinline__ double draw_uniform(uint64_t seed, uint64_t offset, uint64_t sid,
                                               uint32_t r) {
  const Philox4x64 b = philox4x64_10(offset, sid, (uint64_t)(r >> 2), 0ull, seed, 0ull);
  return (double)(b.w[r & 3] >> 11) * 0x1p-53;
}

// ---------------------------------------------------------------------------
// float32 order keys
// ---------------------------------------------------------------------------

// For x >= 0 the raw bits order like the values (the F4 note, §③).
__device__ __forceinline__ uint32_t bits_of(float x) { return __float_as_uint(x); }

// Monotone key for any non-NaN float: negative values have their bits
// inverted, non-negative ones get the sign bit set (the F4 note, §⑧ warns
// that raw bits of negative floats order backwards); -0.0 maps to +0.0.
__device__ __forceinline__ uint32_t signed_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

}  // namespace dss
