// Device primitives for the gfx950 sampling kernels: wave64 reductions and
// scans, the Philox4x64-10 generator, float32 order keys.
//
// Wave reductions and scans run on DPP lane shifts with a fixed association
// order, so every lane of a wave ends with the same bits, and cross-wave
// combinations run in a fixed order through LDS: all results are
// deterministic run to run (no floating-point atomics).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dss {

constexpr int kWave = 64;
constexpr int kBlock = 1024;
constexpr int kWaves = kBlock / kWave;

// ---------------------------------------------------------------------------
// wave64 collectives on DPP (data-parallel primitives of GFX9)
// ---------------------------------------------------------------------------
//
// An inclusive scan over the 64 lanes is four row shifts inside each row of
// 16 lanes (row_shr:1,2,4,8) followed by two row broadcasts (row_bcast:15 into
// rows 1 and 3, row_bcast:31 into rows 2 and 3); a reduction is the scan's
// last lane read back as a scalar.  All lanes of a wave therefore agree
// bit for bit, and the association order is fixed.  No LDS traffic.

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

namespace dpp {
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kWaveShr1 = 0x138;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// lanes whose DPP source is out of range or masked off receive `fill`
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t mov(uint32_t v, uint32_t fill) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double mov(double v, double fill) {
  const uint64_t b = (uint64_t)__double_as_longlong(v), f = (uint64_t)__double_as_longlong(fill);
  const uint32_t lo = mov<CTRL, ROWS>((uint32_t)b, (uint32_t)f);
  const uint32_t hi = mov<CTRL, ROWS>((uint32_t)(b >> 32), (uint32_t)(f >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
}  // namespace dpp

struct OpSum {
  template <class T> __device__ __forceinline__ T operator()(T a, T b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); }
};
struct OpMin {
  __device__ __forceinline__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); }
};

template <class T, class Op>
__device__ __forceinline__ T wave_incl_scan(T v, T identity, Op op) {
  v = op(v, dpp::mov<dpp::kRowShr1, 0xF>(v, identity));
  v = op(v, dpp::mov<dpp::kRowShr2, 0xF>(v, identity));
  v = op(v, dpp::mov<dpp::kRowShr4, 0xF>(v, identity));
  v = op(v, dpp::mov<dpp::kRowShr8, 0xF>(v, identity));
  v = op(v, dpp::mov<dpp::kRowBcast15, 0xA>(v, identity));
  v = op(v, dpp::mov<dpp::kRowBcast31, 0xC>(v, identity));
  return v;
}

__device__ __forceinline__ uint32_t lane63(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}
__device__ __forceinline__ double lane63(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, kWave - 1);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), kWave - 1);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum across the 64 lanes.  Floating-point rounding can make
// neighbouring prefixes non-monotone; callers that locate a token guard
// against that explicitly.
__device__ __forceinline__ double wave_incl_scan(double v) { return wave_incl_scan(v, 0.0, OpSum()); }
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) { return wave_incl_scan(v, 0u, OpSum()); }

// Exclusive prefix: the inclusive prefix of the previous lane (0 in lane 0).
__device__ __forceinline__ double wave_excl_from_incl(double incl) {
  return dpp::mov<dpp::kWaveShr1, 0xF>(incl, 0.0);
}

// Value of lane `l` (wave-uniform) in every lane.
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ int lane_value(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ uint64_t lane_value(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double lane_value(double v, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double wave_sum(double v) { return lane63(wave_incl_scan(v)); }
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) { return lane63(wave_incl_scan(v)); }
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  return lane63(wave_incl_scan(v, 0u, OpMax()));
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  return lane63(wave_incl_scan(v, 0xFFFFFFFFu, OpMin()));
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
  // a select chain rather than b.w[r & 3]: a dynamic index would put the
  // block in scratch memory, and any scratch slows every wave's launch
  const uint32_t j = r & 3u;
  const uint64_t w = j == 0u ? b.w[0] : j == 1u ? b.w[1] : j == 2u ? b.w[2] : b.w[3];
  return (double)(w >> 11) * 0x1p-53;
}

// ---------------------------------------------------------------------------
// global-memory views of plain pointers
// ---------------------------------------------------------------------------
//
// A pointer held in a parameter struct is generic (flat) to the compiler
// unless it can prove otherwise, and flat loads count against the LDS wait
// counter as well as the vector-memory one: every LDS wait would then also
// wait for outstanding HBM reads.  These casts make the accesses
// global-memory instructions.
template <class T>
using gptr = T __attribute__((address_space(1)))*;
template <class T>
__device__ __forceinline__ gptr<T> as_global(T* p) {
  return (gptr<T>)p;
}

// One value through a vector load (global_load), never a scalar load: its
// wait sits at the first use of the value, not at a work-group barrier.
template <typename T>
__device__ __forceinline__ T vload(const T* p) {
  return __hip_atomic_load(as_global(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte global load (HIP's float4 cannot be copied out of another
// address space, the native vector type can)
__device__ __forceinline__ float4 load_f4(gptr<const float4> p) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f x = *(gptr<const v4f>)p;
  return make_float4(x.x, x.y, x.z, x.w);
}

// The same load marked non-temporal (read once, not kept in the caches):
// for the one read of a row, which no later pass of the kernel reads again.
__device__ __forceinline__ float4 load_f4_nt(gptr<const float4> p) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f x = __builtin_nontemporal_load((gptr<const v4f>)p);
  return make_float4(x.x, x.y, x.z, x.w);
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

// float32 value of a signed-order key (the inverse of signed_key; -0.0 comes
// back as +0.0)
__device__ __forceinline__ float from_signed_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

}  // namespace dss
