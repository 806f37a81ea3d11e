// Device helpers shared by the split-row kernels (split_kernels.hip and
// pipe_kernels.hip): order keys, padded LDS histograms and their one-wave
// searches, exact ranks, fixed-point masses, and the one-wave dual-pivot
// loop of the FlashInfer blog ("Sorting-Free GPU Kernels for LLM Sampling",
// section 双枢轴拒绝采样) over a row's top-k set.
#pragma once

#include "stream_device.h"

namespace dss {
namespace {

constexpr int kHistBins = 2048;
constexpr int kMassBins = 256;    // top-p start search: one mass bin per 8 histogram bins
constexpr int kMassShift = 3;

template <bool KEYS>
__device__ __forceinline__ uint32_t key_of(float x) {
  return KEYS ? signed_key(x) : bits_of(x);
}

// Histograms are stored in chunks of NB/64 bins (the bins one lane sums in
// a search), each chunk padded by four words so that the 64 lanes' 16-byte
// reads of their chunks fall in distinct LDS banks.
template <int NB>
struct Padded {
  static constexpr int kChunk = NB / kWave;
  static constexpr int kStride = kChunk + 4;
  static constexpr int kWords = kWave * kStride;
  static __device__ __forceinline__ uint32_t at(uint32_t b) { return b + 4u * (b / kChunk); }
};
using H1 = Padded<kHistBins>;

__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20) & 0xFu;  // HW_REG_XCC_ID
}

// wave index as a scalar, so branches on it are scalar branches
__device__ __forceinline__ int uwave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ int first_lane(uint64_t m) { return __ffsll((long long)m) - 1; }
__device__ __forceinline__ int last_lane(uint64_t m) { return 63 - __clzll((long long)m); }

// position of this lane among the lanes set in m that are below it
__device__ __forceinline__ uint32_t rank_in(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <bool KEYS>
__device__ __forceinline__ uint32_t max4_key(const float4& x) {
  return max(max(key_of<KEYS>(x.x), key_of<KEYS>(x.y)), max(key_of<KEYS>(x.z), key_of<KEYS>(x.w)));
}

template <int NB>
__device__ __forceinline__ void clear_hist(uint32_t* h, int t, int nt) {
  uint4* h4 = reinterpret_cast<uint4*>(h);
  for (int q = t; q < Padded<NB>::kWords / 4; q += nt) h4[q] = make_uint4(0u, 0u, 0u, 0u);
}

// ---------------------------------------------------------------------------
// work-group helpers (every thread of the work-group must call; fixed
// association order, so results are deterministic)
// ---------------------------------------------------------------------------

// Exclusive prefix of v over the work-group in thread order, and the total.
// `red` must not be reused by another scan before every thread has returned
// from this one.  Waves with `active` false (wave-uniform) contribute zeros
// without computing anything.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t& total, uint32_t* red,
                                                    bool active = true) {
  const int lane = lane_id(), w = uwave();
  uint32_t incl = 0u;
  if (active) incl = wave_incl_scan(v);
  if (lane == kWave - 1) red[w] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) {
    const uint32_t t = red[q];
    base += q < w ? t : 0u;
    tot += t;
  }
  total = tot;
  return active ? base + incl - v : 0u;
}

// Largest bin b of the padded histogram hist (NB bins) whose suffix count
// sum_{b' >= b} hist[b'] reaches need, the count strictly above b, and the
// total (bin 0 and total - hist[0] if the total falls short).  One wave:
// lane l sums the l-th chunk of bins from the top, a scan over the lanes
// finds the chunk, a scan over that chunk's bins finds the bin.
template <int NB>
__device__ void wave_find(const uint32_t* hist, uint32_t need, uint32_t& bin, uint32_t& above,
                          uint32_t& total, uint32_t* in_bin = nullptr) {
  using H = Padded<NB>;
  static_assert(H::kChunk % 4 == 0 && H::kChunk <= kWave, "chunk of whole 16-byte reads");
  const int lane = lane_id();
  const int chunk = kWave - 1 - lane;  // lane 0 holds the top chunk
  uint32_t s = 0u;
#pragma unroll
  for (int q = 0; q < H::kChunk; q += 4) {
    const uint4 h = *reinterpret_cast<const uint4*>(hist + chunk * H::kStride + q);
    s += h.x + h.y + h.z + h.w;
  }
  const uint32_t incl = wave_incl_scan(s);
  total = lane63(incl);
  const uint64_t m = __ballot(incl >= need);
  if (m == 0ull) {
    bin = 0u;
    above = total - hist[0];
    if (in_bin) *in_bin = hist[0];
    return;
  }
  const int L = first_lane(m);
  const uint32_t excl_l = lane_value(incl - s, L);
  const int c = kWave - 1 - L;
  const uint32_t h = lane < H::kChunk ? hist[c * H::kStride + H::kChunk - 1 - lane] : 0u;
  const uint32_t incl2 = excl_l + wave_incl_scan(h);
  const int L2 = first_lane(__ballot(lane < H::kChunk && incl2 >= need));
  bin = (uint32_t)(c * H::kChunk + H::kChunk - 1 - L2);
  above = lane_value(incl2 - h, L2);
  if (in_bin) *in_bin = lane_value(h, L2);  // the found bin's own count
}

// ---------------------------------------------------------------------------
// The k-th largest value among the entries of bnd[0..n) whose bits lie in
// [base, base + 2^sh), need of them counting from the top (1 <= need <= the
// number in range).  One wave, no barriers: while more than 64 entries are
// in range, a 2048-way histogram of the next bit field narrows the range
// (the F4 note's threshold search on the bit pattern, §③); then every lane
// takes one entry and counts the entries >= its own (an exact rank).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_kth(const uint64_t* bnd, uint32_t n, uint32_t base, uint32_t sh,
                             uint32_t need, uint32_t* hist, uint32_t* sel) {
  const int lane = lane_id();
  while (true) {
    // entries in range, and (if at most 64) their bits in sel[]
    uint32_t cnt = 0u;
    for (uint32_t c0 = 0; c0 < n; c0 += kWave) {
      const uint32_t c = c0 + lane;
      uint32_t x = (uint32_t)bnd[min(c, n - 1u)];  // unconditional read, n >= 1 here
      asm volatile("" : "+v"(x));
      const bool in = c < n && x - base < (1u << sh) && x >= base;
      const uint64_t m = __ballot(in);
      const uint32_t p = cnt + rank_in(m);
      if (in && p < (uint32_t)kWave) sel[p] = x;
      cnt += (uint32_t)__popcll(m);
    }
    if (cnt <= (uint32_t)kWave || sh == 0u) {
      if (sh == 0u) return base;  // one bit pattern left: every entry in range equals it
      // lane j holds the j-th entry in range; each lane counts the entries
      // >= its own, the other lanes' values read as scalars
      const uint32_t x = lane < (int)cnt ? sel[lane] : 0u;
      uint32_t ge = 0u;
      for (uint32_t j = 0; j < cnt; ++j) ge += (uint32_t)(lane_value(x, (int)j) >= x);
      const uint32_t cand = (lane < (int)cnt && ge >= need) ? x : 0u;
      return wave_max(cand);
    }
    const uint32_t sh2 = sh > 11u ? sh - 11u : 0u;
    clear_hist<kHistBins>(hist, lane, kWave);
    for (uint32_t c = lane; c < n; c += kWave) {
      const uint32_t x = (uint32_t)bnd[c];
      if (x >= base && x - base < (1u << sh)) atomicAdd(&hist[H1::at((x - base) >> sh2)], 1u);
    }
    uint32_t bin, above, total;
    wave_find<kHistBins>(hist, need, bin, above, total);
    base += bin << sh2;
    sh = sh2;
    need -= above;
  }
}

// ---------------------------------------------------------------------------
// The dual-pivot loop on one wave (no barriers).  cand[0..m) holds every
// value of the row above `low` and nothing at or below it, each > 0; their
// mass is the kept mass Z_k, and the top-p bound is pfrac * Z_k.  Lane l
// owns the entries l, l + 64, l + 128, ... (NR of them in registers as
// float64, or E = ceil(m / 64) read from LDS when NR = 0), so every LDS read
// of the entries is one conflict-free row.  The inverse-transform draw
// (blog, 逆变换采样) runs over lane 0's entries, then lane 1's, and so on: a
// fixed order of the candidates, which is all the method needs.  Guards as
// in the streaming engine (blog, 实现细节): only entries with nonzero mass
// are chosen, the first hit wins, and if rounding puts the target at or past
// every running sum the last entry is taken.
//
// Every pivot is one of the entries, so it is >= tau_k and fewer than k
// values exceed it: the top-k half of f(t) always holds here, and f(t) of
// top-k-then-top-p reduces to "the mass above t is below p * Z_k" (or no
// value is above t).
// ---------------------------------------------------------------------------
// x (float32 bits b, x >= 0, finite, at most the value with exponent field
// eg) in units of 2^(eg - 145), rounded down: mant >> (eg - e + 5) for a
// normal x, which is below 2^19, so 4096 of them sum below 2^31.  The
// integer sums are exact and independent of the order of the additions.
__device__ __forceinline__ uint32_t fixed_mass(uint32_t b, uint32_t eg) {
  const uint32_t e = b >> 23;
  const uint32_t mant = (b & 0x7FFFFFu) | 0x800000u;
  return e == 0u ? 0u : mant >> min(eg - e + 5u, 31u);
}

// A starting pivot for the dual-pivot loop above tau_k: the largest key L
// below one of the mass bins such that the top-k mass above L provably
// reaches pfrac * Z_k, so that f(L) is false and no value at or below L can
// be kept (the blog's proof then holds from L).  The mass histogram holds
// lower bounds of the above-bin masses (fixed_mass, unit 2^(eg - 145)); Z_k
// is bounded above by those sums plus one unit per entry plus zb, the mass
// of the boundary entries kept; the test carries a 1e-9 relative margin,
// far above every rounding error of the float64 sums here and in the loop.
// Returns 0 when no bin qualifies.  One wave.
// What wave 0 keeps of the mass histogram for the loop: per lane, the
// suffix mass above its bins (excl) and down to each of them (excl + r[j]),
// lower bounds in float64 with a relative error below 1e-12; slack bounds
// what the rounding down of every entry's mass can have lost.
struct MassView {
  double excl, r[4];
  double slack;
  uint32_t tstar, sh, mb1;  // bin geometry, and the mass bin of the boundary bin
  bool on;
};

template <class Smem>
__device__ __forceinline__ uint32_t top_p_start(const Smem& sm, uint32_t n_above, double zb,
                                                uint32_t eg, float pfrac, double zref,
                                                uint32_t tstar, uint32_t sh, uint32_t bin1,
                                                MassView& mv) {
  constexpr int kPer = kMassBins / kWave;  // bins per lane, the top ones in lane 0
  static_assert(kPer == 4, "one 16-byte read per lane");
  const int lane = lane_id();
  const int c = kWave - 1 - lane;
  // this lane's bins from the top down, and their running sums
  const uint4 mb = *reinterpret_cast<const uint4*>(sm.mh + c * kPer);
  const double unit = __longlong_as_double((long long)((unsigned long long)(eg + 1023u - 145u) << 52));
  mv.r[0] = (double)mb.w * unit;
  mv.r[1] = mv.r[0] + (double)mb.z * unit;
  mv.r[2] = mv.r[1] + (double)mb.y * unit;
  mv.r[3] = mv.r[2] + (double)mb.x * unit;
  const double incl = wave_incl_scan(mv.r[3]);
  mv.excl = wave_excl_from_incl(incl);
  mv.slack = (double)n_above * unit;
  mv.tstar = tstar;
  mv.sh = sh;
  mv.mb1 = bin1 >> kMassShift;
  mv.on = true;
  // an upper bound of the mass top-p compares with: Z_k, or (joint order,
  // zref >= 0) the row's mass
  const double zhi = zref >= 0.0 ? zref * (1.0 + 1e-12) : lane63(incl) * (1.0 + 1e-12) + mv.slack + zb;
  const double target = (double)pfrac * zhi * (1.0 + 1e-9);
  // suffix mass down to each of this lane's bins; the first (highest) bin
  // whose suffix provably reaches the target
  auto ok = [&](double r) {
    const double sfx = mv.excl + r;
    return sfx > 0.0 && sfx * (1.0 - 1e-12) >= target;
  };
  const int j = ok(mv.r[0]) ? 0 : ok(mv.r[1]) ? 1 : ok(mv.r[2]) ? 2 : ok(mv.r[3]) ? 3 : 4;
  const uint64_t m = __ballot(j < 4);
  if (m == 0ull) return 0u;
  const int l1 = first_lane(m);
  const uint32_t b = (uint32_t)(kMassBins - 1 - (kPer * l1 + lane_value(j, l1)));
  const uint32_t edge = tstar + ((b << kMassShift) << sh);
  return edge > 0u ? edge - 1u : 0u;
}

template <int OP, int NR, class Smem>
__device__ int wave_loop(const Smem& sm, int m, float low, float start, float high,
                         float pfrac, double zrow, uint64_t seed, uint64_t offset, uint64_t sid,
                         const MassView& mv, int& rounds) {
  constexpr bool REG = NR > 0;
  const int lane = lane_id();
  const int E = (m + kWave - 1) / kWave;  // entries of the busiest lane (<= 64)
  const uint64_t* cand = sm.u.b.cand;
  if (m <= 0) {  // no value above low (callers never pass this)
    rounds = 0;
    return -1;
  }
  // x of entry c, 0 past the end (never above a pivot).  The read is
  // clamped and its bits masked rather than selected, so that the compiler
  // keeps it unconditional: all reads go out together under one wait.
  auto ld = [&](int c) -> double {
    const uint32_t b = (uint32_t)cand[min(c, m - 1)];
    return (double)__uint_as_float(b & (c < m ? 0xFFFFFFFFu : 0u));
  };
  double xr[REG ? NR : 1];
  if (REG) {
#pragma unroll
    for (int j = 0; j < NR; ++j) xr[j] = ld(lane + kWave * j);
  }
  // f(x) for each of this lane's entries
  auto each = [&](auto&& f) {
    if constexpr (REG) {
#pragma unroll
      for (int j = 0; j < NR; ++j) f(xr[j]);
    } else {
      for (int j = 0; j < E; ++j) f(ld(lane + kWave * j));
    }
  };

  // Z_k: the mass above low (every entry); the loop starts at `start`
  // (>= low), which leaves every value that top-p can keep above it
  const double lk = (double)low;
  double lo = (double)start;
  double zk = 0.0, part = 0.0;  // this lane's mass above low, above lo
  each([&](double x) {
    zk += x > lk ? x : 0.0;
    part += x > lo ? x : 0.0;
  });
  // top-p against Z_k, or against the row's mass Z under the joint order
  const double pz = (double)pfrac * (OP == kOpTopKTopPJoint ? zrow : wave_sum(zk));
  double incl = wave_incl_scan(part);  // prefix over lanes of the mass above lo
  double S = lane63(incl);
  int rnd = 0;
  while (true) {
    const double u = rnd < stream::kPreDraws ? sm.draws[rnd]
                                             : draw_uniform(seed, offset, sid, (uint32_t)rnd);
    ++rnd;
    const double T = u * S;
    const double excl = wave_excl_from_incl(incl);
    const uint64_t nz = __ballot(part > 0.0);
    if (nz == 0ull) {
      rounds = rnd;
      return -1;
    }
    const uint64_t hit = __ballot(part > 0.0 && incl > T);
    const int owner = hit ? first_lane(hit) : last_lane(nz);
    // The owner's entries, its j-th in lane j, and their running sums from
    // the owner's exclusive prefix: the first past T, else the last entry
    // above low.
    const int c = owner + kWave * lane;
    const bool mine = lane < E && c < m;
    const uint64_t oe = cand[mine ? c : m - 1];
    const double ox = (double)__uint_as_float((uint32_t)oe);
    const double xm = (mine && ox > lo) ? ox : 0.0;
    const double run = lane_value(excl, owner) + wave_incl_scan(xm);
    const uint64_t nz2 = __ballot(xm > 0.0);
    const uint64_t h2 = hit ? __ballot(xm > 0.0 && run > T) : 0ull;
    // part > 0 guarantees the owner an entry; the clamp keeps reads in bounds regardless
    const int pl = h2 ? first_lane(h2) : nz2 ? last_lane(nz2) : 0;
    const uint64_t ent = lane_value(oe, pl);
    if (OP == kOpTopK) {
      rounds = rnd;
      return (int)(ent >> 32);
    }
    // When pivot1 lies in a mass bin above the boundary bin's, the mass of
    // the bins from its own up bounds the mass above it from above; if that
    // bound is already below p * Z_k, f(pivot1) holds and the exact sums
    // would accept too, so the draw is accepted without them.
    if ((OP == kOpTopKTopP || OP == kOpTopKTopPJoint) && mv.on) {
      const uint32_t mb = (((uint32_t)ent - mv.tstar) >> mv.sh) >> kMassShift;  // wave-uniform
      if (mb > mv.mb1 && mb < (uint32_t)kMassBins) {
        const uint32_t d = (uint32_t)kMassBins - 1u - mb;
        const uint32_t jj = d & 3u;
        const double r = jj == 0u ? mv.r[0] : jj == 1u ? mv.r[1] : jj == 2u ? mv.r[2] : mv.r[3];
        const double sfx = lane_value(mv.excl + r, (int)(d >> 2));
        if ((sfx * (1.0 + 1e-12) + mv.slack) * (1.0 + 1e-9) < pz) {
          rounds = rnd;
          return (int)(ent >> 32);
        }
      }
    }
    const float pivot1 = __uint_as_float((uint32_t)ent);
    const float pivot2 = (float)(((double)pivot1 + (double)high) * 0.5);
    const double p1 = (double)pivot1, p2 = (double)pivot2;
    double m0 = 0.0, m1 = 0.0;
    each([&](double x) {
      m0 += x > p1 ? x : 0.0;
      m1 += x > p2 ? x : 0.0;
    });
    const double i0 = wave_incl_scan(m0), i1 = wave_incl_scan(m1);
    const double M0 = lane63(i0), M1 = lane63(i1);
    if (M0 < pz || M0 == 0.0) {  // f(pivot1) = 1: accept
      rounds = rnd;
      return (int)(ent >> 32);
    }
    if (M1 < pz || M1 == 0.0) {  // f(pivot2) = 1: the kept set lies in (pivot1, pivot2]
      lo = p1;
      high = pivot2;
      S = M0;
      part = m0;
      incl = i0;
    } else {
      lo = p2;
      S = M1;
      part = m1;
      incl = i1;
    }
    if (rnd >= stream::kMaxRounds) {
      rounds = rnd;
      return -1;
    }
  }
}

}  // namespace
}  // namespace dss
