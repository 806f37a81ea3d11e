// Device code of the streaming engine (one 1024-thread work-group per row,
// every pass over global memory), shared by the streaming kernels and by the
// split-row kernels, which fall back to it when a row's candidates cannot be
// bounded.  See stream_kernels.hip for the design notes.
#pragma once
#include "dss_device.h"
#include "dss_internal.h"

namespace dss {
namespace stream {

constexpr int kTile = 2048;
constexpr int kTileChunks = kTile / (kWave * 4);  // 8 float4 per lane
constexpr int kMaxTiles = (1 << 20) / kTile;      // vocab <= 2^20
constexpr int kPreDraws = 4 * kWave;              // draws precomputed per output
constexpr int kMaxRounds = 4096;                  // safety bound, never reached

struct RowRef {
  gptr<const float> x;
  int V;
  bool vec;
};

// N groups of four, group u at idx_of(u) (a multiple of 4; past the row end
// reads as 0), every load issued before the first value is used.  The
// choice between 16-byte and one-value loads is made once for the batch on
// r.vec, which every lane shares: made per group and per lane, the two kinds
// of load land in the same registers from two arms and the compiler waits
// for each load before the next one is issued.
//
// ZERO = false leaves the groups past the row end unspecified (the caller
// masks them), so that no instruction waits for the loads here: a caller can
// issue the next batch before it uses this one.
template <int N, bool ZERO = true, class I>
__device__ __forceinline__ void load4_batch(const RowRef& r, I&& idx_of, float (&v)[N][4]) {
  if (r.vec) {
    // V % 4 == 0: a group is whole or lies wholly past the row end.  All
    // loads first (from an address inside the row), the zeros after: a
    // select next to each load would make the compiler wait for it there.
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int64_t idx = idx_of(u);
      const float4 q = load_f4((gptr<const float4>)(r.x + (idx < r.V ? idx : 0)));
      v[u][0] = q.x;
      v[u][1] = q.y;
      v[u][2] = q.z;
      v[u][3] = q.w;
    }
    if (ZERO) {
#pragma unroll
      for (int u = 0; u < N; ++u) {
        const bool in = idx_of(u) < r.V;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[u][e] = in ? v[u][e] : 0.0f;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int64_t idx = idx_of(u);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[u][e] = (idx + e < r.V) ? r.x[idx + e] : 0.0f;
    }
  }
}

// Calls body(idx, v, valid) for every group of four values v = x[idx ..
// idx+3] of the row, thread t taking the groups t, t + kBlock, ...  Each
// thread keeps kBatch 16-byte loads in flight (all issued before the first is
// used), so a pass over a row is bound by bandwidth rather than by one load
// latency per group.  Lanes past the last group get valid = false together
// with a copy of the last group (same idx), so a body stays branch-free:
// reductions must ignore invalid groups, stores may repeat the last group's.
// Values past the row end inside the last group read as 0.
constexpr int kBatch = 8;
// Values x[idx .. idx+3]; positions past the row end read as 0 (for rows
// without 16-byte loads; batches of 16-byte loads go through load4_batch or
// the branch on r.vec below).
__device__ __forceinline__ void load4(const RowRef& r, int64_t idx, float (&v)[4]) {
  if (r.vec && idx + 3 < r.V) {
    const float4 q = load_f4((gptr<const float4>)(r.x + idx));
    v[0] = q.x;
    v[1] = q.y;
    v[2] = q.z;
    v[3] = q.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (idx + e < r.V) ? r.x[idx + e] : 0.0f;
  }
}

template <class F>
__device__ __forceinline__ void for_each4(const RowRef& r, F&& body) {
  const int nvec = (r.V + 3) / 4;
  for (int f0 = threadIdx.x; f0 < nvec; f0 += kBlock * kBatch) {
    float v[kBatch][4];
    if (r.vec) {
      // V % 4 == 0 and a 16-byte aligned row: every clamped group is whole
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float4 q = load_f4((gptr<const float4>)(r.x + 4ll * min(f0 + u * kBlock, nvec - 1)));
        v[u][0] = q.x;
        v[u][1] = q.y;
        v[u][2] = q.z;
        v[u][3] = q.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) load4(r, 4ll * min(f0 + u * kBlock, nvec - 1), v[u]);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int f = f0 + u * kBlock;
      body(4ll * min(f, nvec - 1), v[u], f < nvec);
    }
  }
}

// ---------------------------------------------------------------------------
// block-wide reduction of a small record; every thread gets the same result
// ---------------------------------------------------------------------------

struct Red {
  double d0, d1;
  uint32_t s0, s1, mn, mx;
};

struct RedSmem {
  double d[kWaves][2];
  uint32_t u[kWaves][4];
};

__device__ inline Red block_reduce(Red v, RedSmem& sm) {
  v.d0 = wave_sum(v.d0);
  v.d1 = wave_sum(v.d1);
  v.s0 = wave_sum(v.s0);
  v.s1 = wave_sum(v.s1);
  v.mn = wave_min(v.mn);
  v.mx = wave_max(v.mx);
  if (lane_id() == 0) {
    const int w = wave_id();
    sm.d[w][0] = v.d0;
    sm.d[w][1] = v.d1;
    sm.u[w][0] = v.s0;
    sm.u[w][1] = v.s1;
    sm.u[w][2] = v.mn;
    sm.u[w][3] = v.mx;
  }
  __syncthreads();
  Red out{0.0, 0.0, 0u, 0u, 0xFFFFFFFFu, 0u};
  for (int w = 0; w < kWaves; ++w) {  // fixed order: deterministic
    out.d0 += sm.d[w][0];
    out.d1 += sm.d[w][1];
    out.s0 += sm.u[w][0];
    out.s1 += sm.u[w][1];
    out.mn = min(out.mn, sm.u[w][2]);
    out.mx = max(out.mx, sm.u[w][3]);
  }
  __syncthreads();
  return out;
}

__device__ __forceinline__ Red red_zero() { return Red{0.0, 0.0, 0u, 0u, 0xFFFFFFFFu, 0u}; }

// ---------------------------------------------------------------------------
// threshold search on order keys (F4 note §②-③, §⑤)
// ---------------------------------------------------------------------------
//
// Finds the largest key t with crit(t), where crit is count(key >= t) >= k
// (MASS = false) or mass(key >= t) >= pz (MASS = true).  Invariant: crit(lo)
// holds and crit(hi) fails.  Each pass evaluates crit at two pivots (1/3 and
// 2/3 of [lo, hi)) and records the smallest key >= lo and the largest key
// < hi; those two are themselves a satisfying and (plus one) a failing point,
// and when they coincide only one distinct value is left: it is the answer.
// KEYS selects signed-order keys (logits) instead of raw bits (x >= 0).
template <bool MASS, bool KEYS>
__device__ uint32_t threshold_search(const RowRef& r, uint32_t lo, uint32_t hi, uint32_t k,
                                     double pz, RedSmem& sm) {
  while (hi - lo > 1u) {
    const uint32_t d = hi - lo;
    const uint32_t p1 = lo + max(1u, d / 3u);
    const uint32_t p2 = lo + max(1u, (d / 3u) * 2u);
    Red acc = red_zero();
    for_each4(r, [&](int64_t idx, const float (&v)[4], bool valid) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // key 0 stands for "no value": it is below every pivot (p1, p2 >= 1)
        // and leaves the trackers' results unchanged but for the early exit
        const bool in = valid && idx + e < r.V;
        const uint32_t key = in ? (KEYS ? signed_key(v[e]) : bits_of(v[e])) : 0u;
        const bool a1 = key >= p1, a2 = key >= p2;
        acc.s0 += a1 ? 1u : 0u;
        acc.s1 += a2 ? 1u : 0u;
        if (MASS) {
          acc.d0 += a1 ? (double)v[e] : 0.0;
          acc.d1 += a2 ? (double)v[e] : 0.0;
        }
        acc.mn = min(acc.mn, key >= lo ? key : 0xFFFFFFFFu);
        acc.mx = max(acc.mx, key < hi ? key : 0u);
      }
    });
    const Red t = block_reduce(acc, sm);
    if (t.mn > t.mx) break;  // no value in [lo, hi): cannot happen; keep lo
    if (t.mn == t.mx) return t.mn;
    uint32_t nlo = t.mn, nhi = t.mx + 1u;
    const bool ok1 = MASS ? (t.d0 >= pz) : (t.s0 >= k);
    const bool ok2 = MASS ? (t.d1 >= pz) : (t.s1 >= k);
    if (ok2) {
      nlo = max(nlo, p2);
    } else if (ok1) {
      nlo = max(nlo, p1);
      nhi = min(nhi, p2);
    } else {
      nhi = min(nhi, p1);
    }
    lo = nlo;
    hi = nhi;
  }
  return lo;
}

// mass and count of {bits >= tau} (x >= 0)
__device__ inline Red mass_at_least(const RowRef& r, uint32_t tau, RedSmem& sm) {
  Red acc = red_zero();
  for_each4(r, [&](int64_t idx, const float (&v)[4], bool valid) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool t = valid && idx + e < r.V && bits_of(v[e]) >= tau;
      acc.d0 += t ? (double)v[e] : 0.0;
      acc.s0 += t ? 1u : 0u;
    }
  });
  return block_reduce(acc, sm);
}

__device__ __forceinline__ float clamp01(float v) { return fminf(fmaxf(v, 0.0f), 1.0f); }

// ---------------------------------------------------------------------------
// sampling
// ---------------------------------------------------------------------------

struct SampleSmem {
  double tm[3][kMaxTiles];  // per-tile mass above: current low, pivot a, pivot b
  double draws[kPreDraws];
  RedSmem red;
  double bc_d[2];
  double extra_u;
  int bc_tok;
};

// Sum of tm[0..n) in exactly the order the tile search of locate() uses, so
// that S(low) computed here is the last prefix that search sees.  One wave.
__device__ inline double tile_scan_total(const double* tm, int n) {
  double carry = 0.0;
  for (int base = 0; base < n; base += kWave) {
    const int t = base + lane_id();
    const double m = t < n ? tm[t] : 0.0;
    const double incl = wave_incl_scan(m) + carry;
    carry = lane63(incl);
  }
  return carry;
}

// Inverse-transform draw over the candidates {x > low} (blog, 逆变换采样;
// explainer, "不带过滤时"): the first index j, in index order, whose
// inclusive candidate prefix exceeds T.  Tiles first (tm = mass above low per
// tile), then the one tile.  Guards (blog, 实现细节: a parallel prefix sum of
// non-negative values need not be monotone): only candidates with nonzero
// mass can be selected; the first hit in index order wins; if rounding puts T
// at or past the scanned total, the last candidate is taken.  Wave 0 works,
// the result is broadcast; every thread must call this.
__device__ inline int locate(const RowRef& r, const double* tm, int n_tiles, double T, float low,
                      SampleSmem& sm) {
  if (wave_id() == 0) {
    const int lane = lane_id();
    double carry = 0.0, excl_hit = 0.0, excl_last = 0.0;
    int tile = -1, last_nz = -1;
    for (int base = 0; base < n_tiles; base += kWave) {
      const int t = base + lane;
      const double m = t < n_tiles ? tm[t] : 0.0;
      const double incl = wave_incl_scan(m) + carry;
      const double excl = incl - m;
      const uint64_t hit = __ballot(m > 0.0 && incl > T);
      const uint64_t nz = __ballot(m > 0.0);
      if (nz) {
        const int l = 63 - __clzll((long long)nz);
        last_nz = base + l;
        excl_last = lane_value(excl, l);
      }
      if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        tile = base + l;
        excl_hit = lane_value(excl, l);
        break;
      }
      carry = lane63(incl);
    }
    double Tl = T - excl_hit;
    if (tile < 0) {
      tile = last_nz;
      Tl = T - excl_last;
    }
    int found = -1;
    if (tile >= 0) {
      const int64_t tbase = (int64_t)tile * kTile;
      double run_carry = 0.0;
      int last_cand = -1;
      float vt[kTileChunks][4];  // the whole tile in flight at once
      load4_batch<kTileChunks>(r, [&](int q) { return tbase + q * (kWave * 4) + lane * 4; }, vt);
#pragma unroll
      for (int q = 0; q < kTileChunks; ++q) {
        const int64_t idx = tbase + q * (kWave * 4) + lane * 4;
        const float (&v)[4] = vt[q];
        double s = 0.0;
        bool cand[4];
        int my_last = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cand[e] = (idx + e < r.V) && (v[e] > low);
          s += cand[e] ? (double)v[e] : 0.0;
          my_last = cand[e] ? (int)(idx + e) : my_last;
        }
        const double incl = wave_incl_scan(s);
        const double excl = wave_excl_from_incl(incl);
        double run = run_carry + excl;
        int hit_e = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          run += cand[e] ? (double)v[e] : 0.0;
          hit_e = (hit_e < 0 && cand[e] && run > Tl) ? e : hit_e;
        }
        const uint64_t hm = __ballot(hit_e >= 0);
        if (hm) {
          const int l = __ffsll((long long)hm) - 1;
          const int e = lane_value(hit_e, l);
          found = (int)(tbase + q * (kWave * 4) + l * 4 + e);
          break;
        }
        const uint64_t cm = __ballot(my_last >= 0);
        if (cm) last_cand = lane_value(my_last, 63 - __clzll((long long)cm));
        run_carry += lane63(incl);
      }
      if (found < 0) found = last_cand;
    }
    if (lane == 0) sm.bc_tok = found;
  }
  __syncthreads();
  const int tok = sm.bc_tok;
  __syncthreads();
  return tok;
}

// One (mass, count) pass at pivots a <= b: per-tile masses above each pivot
// into tma / tmb, per-lane counts of values above each pivot.
__device__ inline void pivot_pass(const RowRef& r, int n_tiles, float a, float b, double* tma,
                           double* tmb, uint32_t& ca, uint32_t& cb) {
  const int lane = lane_id();
  for (int t = wave_id(); t < n_tiles; t += kWaves) {
    const int64_t base = (int64_t)t * kTile;
    double sa = 0.0, sb = 0.0;
    float vt[kTileChunks][4];
    load4_batch<kTileChunks>(r, [&](int q) { return base + q * (kWave * 4) + lane * 4; }, vt);
#pragma unroll
    for (int q = 0; q < kTileChunks; ++q) {
      const float (&v)[4] = vt[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // padding past the row end reads as 0, never above a pivot >= 0
        const bool ga = v[e] > a, gb = v[e] > b;
        sa += ga ? (double)v[e] : 0.0;
        ca += ga ? 1u : 0u;
        sb += gb ? (double)v[e] : 0.0;
        cb += gb ? 1u : 0u;
      }
    }
    sa = wave_sum(sa);
    sb = wave_sum(sb);
    if (lane == 0) {
      tma[t] = sa;
      tmb[t] = sb;
    }
  }
}

// f(t) of the blog's dual-pivot section: 1 iff threshold t already
// satisfies the filter.  Top-k counts the values above t, top-p compares
// their mass with p * Z_C (Z_C = the row's mass for top-p and for the joint
// order, the top-k set's for top-k-then-top-p), min-p compares t with
// min_p * max; "count == 0" makes f(max) = 1 also for p = 0.
template <int OP>
__device__ __forceinline__ bool predicate(float t, double mass_above, uint32_t count_above,
                                          int k, double pz, double minp_thr) {
  if (OP == kOpNone) return true;
  if (OP == kOpMinP) return (double)t >= minp_thr;
  const bool ok_k = (OP == kOpTopP) ? true : (count_above < (uint32_t)k);
  if (OP == kOpTopK) return ok_k;
  const bool ok_p = (mass_above < pz) || count_above == 0u;
  return ok_k && ok_p;
}

__device__ __forceinline__ void write_sample(const SampleParams& P, int i, int tok, int rounds) {
  as_global(P.samples)[i] = tok;
  if (P.valid) as_global(P.valid)[i] = tok >= 0 ? 1 : 0;
  if (P.rounds) as_global(P.rounds)[i] = rounds;
}


// Min-p sampling of output i in two reads of the row (every thread of the
// work-group calls): per-tile maxima and the row maximum M, then the kept
// mass {x >= min_p * M} (the product exact in float64) of every tile whose
// maximum reaches the threshold (the others hold nothing kept and are not
// read again), one draw and the walk of one tile in index order.  This is
// the blog's loop started just below the threshold, where the first draw
// is accepted (rounds = 1); the pages' loop from low = 0 stays with
// sample_row.
__device__ __forceinline__ void sample_row_minp(const SampleParams& P, int i, SampleSmem& sm) {
  const int lane = lane_id();
  const int wave = wave_id();
  const int row = P.indices ? as_global(P.indices)[i] : i;
  const float mp = P.min_p_arr ? as_global(P.min_p_arr)[i] : P.min_p;
  if (!(row >= 0 && row < P.rows) || isnan(mp)) {  // block-uniform
    if (threadIdx.x == 0) write_sample(P, i, -1, 0);
    return;
  }
  const uint64_t seed = P.seed_arr ? as_global(P.seed_arr)[i] : P.seed;
  const uint64_t offset = P.offset_arr ? as_global(P.offset_arr)[i] : P.offset;
  const uint64_t sid = P.seed_arr ? 0ull : (uint64_t)i;
  const RowRef r{as_global(P.probs + (int64_t)row * P.vocab), P.vocab, P.vec_ok != 0};
  const int n_tiles = (P.vocab + kTile - 1) / kTile;

  // pass 0: the maximum of every tile (bits; a sign bit, inf or NaN shows as
  // a pattern >= 0x7F800000) into tm[1], the row's maximum
  uint32_t mbits = 0u;
  for (int t = wave; t < n_tiles; t += kWaves) {
    const int64_t base = (int64_t)t * kTile;
    float vt[kTileChunks][4];
    load4_batch<kTileChunks>(r, [&](int q) { return base + q * (kWave * 4) + lane * 4; }, vt);
    uint32_t tb = 0u;
#pragma unroll
    for (int q = 0; q < kTileChunks; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) tb = max(tb, bits_of(vt[q][e]));
    tb = wave_max(tb);
    mbits = max(mbits, tb);
    if (lane == 0) sm.tm[1][t] = tb < 0x7F800000u ? (double)__uint_as_float(tb) : 0.0;
  }
  Red red0 = red_zero();
  red0.mx = mbits;
  const uint32_t maxbits = block_reduce(red0, sm.red).mx;  // (its barriers publish tm[1])
  // sign bit, inf or NaN anywhere, or nothing positive: invalid row
  if (maxbits >= 0x7F800000u || maxbits == 0u) {
    if (threadIdx.x == 0) write_sample(P, i, -1, 0);
    return;
  }
  const double thr = (double)clamp01(mp) * (double)__uint_as_float(maxbits);
  // pass 1: kept mass per tile, read only where the tile's maximum reaches thr
  for (int t = wave; t < n_tiles; t += kWaves) {
    double s = 0.0;
    if (sm.tm[1][t] >= thr) {  // wave-uniform
      const int64_t base = (int64_t)t * kTile;
      float vt[kTileChunks][4];
      load4_batch<kTileChunks>(r, [&](int q) { return base + q * (kWave * 4) + lane * 4; }, vt);
#pragma unroll
      for (int q = 0; q < kTileChunks; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) s += (double)vt[q][e] >= thr ? (double)vt[q][e] : 0.0;
      s = wave_sum(s);
    }
    if (lane == 0) sm.tm[0][t] = s;
  }
  __syncthreads();
  if (wave == 0) {
    const double z = tile_scan_total(sm.tm[0], n_tiles);
    if (lane == 0) sm.bc_d[0] = z * draw_uniform(seed, offset, sid, 0u);
  }
  __syncthreads();
  const double T = sm.bc_d[0];
  __syncthreads();
  // {x >= thr} = {x > low}: low is the float32 just below the smallest
  // float32 >= thr (for thr = 0 the zeros, which carry no mass, are left out)
  float f = (float)thr;
  if ((double)f < thr) f = __uint_as_float(__float_as_uint(f) + 1u);
  const float low = f > 0.0f ? __uint_as_float(__float_as_uint(f) - 1u) : 0.0f;
  const int tok = locate(r, sm.tm[0], n_tiles, T, low, sm);
  if (threadIdx.x == 0) write_sample(P, i, tok, tok >= 0 ? 1 : 0);
}

// Sample output i with the streaming engine; every thread of the
// work-group must call this (it contains barriers).
template <int OP>
__device__ __forceinline__ void sample_row(const SampleParams& P, int i, SampleSmem& sm) {
  const int lane = lane_id();
  const int wave = wave_id();

  const int row = P.indices ? as_global(P.indices)[i] : i;
  const int k = P.top_k_arr ? as_global(P.top_k_arr)[i] : P.top_k;
  const float pp = P.top_p_arr ? as_global(P.top_p_arr)[i] : P.top_p;
  const float mp = P.min_p_arr ? as_global(P.min_p_arr)[i] : P.min_p;
  bool ok = row >= 0 && row < P.rows;
  if (OP == kOpTopK || OP == kOpTopKTopP || OP == kOpTopKTopPJoint) ok = ok && k > 0;
  if (OP == kOpTopP || OP == kOpTopKTopP || OP == kOpTopKTopPJoint) ok = ok && !isnan(pp);
  if (OP == kOpMinP) ok = ok && !isnan(mp);
  if (!ok) {  // block-uniform
    if (threadIdx.x == 0) write_sample(P, i, -1, 0);
    return;
  }
  const uint64_t seed = P.seed_arr ? as_global(P.seed_arr)[i] : P.seed;
  const uint64_t offset = P.offset_arr ? as_global(P.offset_arr)[i] : P.offset;
  const uint64_t sid = P.seed_arr ? 0ull : (uint64_t)i;
  if (wave == 0) {
    if (OP == kOpNone) {
      if (lane == 0) sm.draws[0] = draw_uniform(seed, offset, sid, 0u);
    } else {
      const Philox4x64 b = philox4x64_10(offset, sid, (uint64_t)lane, 0ull, seed, 0ull);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.draws[4 * lane + e] = (double)(b.w[e] >> 11) * 0x1p-53;
    }
  }

  const RowRef r{as_global(P.probs + (int64_t)row * P.vocab), P.vocab, P.vec_ok != 0};
  const int n_tiles = (P.vocab + kTile - 1) / kTile;

  // pass 0: tile masses (mass above low = 0), max bits, validity
  uint32_t mbits = 0u;
  for (int t = wave; t < n_tiles; t += kWaves) {
    const int64_t base = (int64_t)t * kTile;
    double s = 0.0;
    float vt[kTileChunks][4];
    load4_batch<kTileChunks>(r, [&](int q) { return base + q * (kWave * 4) + lane * 4; }, vt);
#pragma unroll
    for (int q = 0; q < kTileChunks; ++q) {
      const float (&v)[4] = vt[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mbits = max(mbits, bits_of(v[e]));
        s += (double)v[e];
      }
    }
    s = wave_sum(s);
    if (lane == 0) sm.tm[0][t] = s;
  }
  Red red0 = red_zero();
  red0.mx = mbits;
  const uint32_t maxbits = block_reduce(red0, sm.red).mx;
  if (wave == 0) {
    const double z = tile_scan_total(sm.tm[0], n_tiles);
    if (lane == 0) sm.bc_d[0] = z;
  }
  __syncthreads();
  const double Z = sm.bc_d[0];
  __syncthreads();
  // sign bit, inf or NaN anywhere, or nothing positive: invalid row
  if (maxbits >= 0x7F800000u || !(Z > 0.0)) {
    if (threadIdx.x == 0) write_sample(P, i, -1, 0);
    return;
  }
  const float M = __uint_as_float(maxbits);

  double zc = Z;
  if (OP == kOpTopKTopP && k < P.vocab) {
    const uint32_t tau_k = threshold_search<false, false>(r, 0u, maxbits + 1u, (uint32_t)k, 0.0, sm.red);
    zc = mass_at_least(r, tau_k, sm.red).d0;
  }
  // (the joint order compares with the row's own mass: zc stays Z)
  const double pz = (OP == kOpTopP || OP == kOpTopKTopP || OP == kOpTopKTopPJoint)
                        ? (double)clamp01(pp) * zc
                        : 0.0;
  const double minp_thr = (OP == kOpMinP) ? (double)clamp01(mp) * (double)M : 0.0;

  float low = 0.0f, high = M;
  double S = Z;
  int cur = 0, rnd = 0, token = -1;
  while (true) {
    double u;
    if (rnd < kPreDraws) {
      u = sm.draws[rnd];
    } else {
      if (threadIdx.x == 0) sm.extra_u = draw_uniform(seed, offset, sid, (uint32_t)rnd);
      __syncthreads();
      u = sm.extra_u;
      __syncthreads();
    }
    ++rnd;
    token = locate(r, sm.tm[cur], n_tiles, u * S, low, sm);
    if (OP == kOpNone || token < 0) break;
    const float pivot1 = r.x[token];
    const float pivot2 = (float)(((double)pivot1 + (double)high) * 0.5);
    const int ia = (cur + 1) % 3, ib = (cur + 2) % 3;
    uint32_t ca = 0u, cb = 0u;
    pivot_pass(r, n_tiles, pivot1, pivot2, sm.tm[ia], sm.tm[ib], ca, cb);
    Red cr = red_zero();
    cr.s0 = ca;
    cr.s1 = cb;
    cr = block_reduce(cr, sm.red);
    if (wave == 0) {
      const double ma = tile_scan_total(sm.tm[ia], n_tiles);
      const double mb = tile_scan_total(sm.tm[ib], n_tiles);
      if (lane == 0) {
        sm.bc_d[0] = ma;
        sm.bc_d[1] = mb;
      }
    }
    __syncthreads();
    const double Ma = sm.bc_d[0], Mb = sm.bc_d[1];
    __syncthreads();
    if (predicate<OP>(pivot1, Ma, cr.s0, k, pz, minp_thr)) break;  // accept
    if (P.single_pivot) {  // single pivot: only the rejected value moves low
      low = pivot1;
      S = Ma;
      cur = ia;
    } else if (predicate<OP>(pivot2, Mb, cr.s1, k, pz, minp_thr)) {
      low = pivot1;
      high = pivot2;
      S = Ma;
      cur = ia;
    } else {
      low = pivot2;
      S = Mb;
      cur = ib;
    }
    if (rnd >= kMaxRounds) {
      token = -1;
      break;
    }
  }
  if (threadIdx.x == 0) write_sample(P, i, token, token >= 0 ? rnd : 0);
}

// ---------------------------------------------------------------------------
// renormalisation and logit masking
// ---------------------------------------------------------------------------

// (vec: V % 4 == 0 and 16-byte aligned rows, so every group is whole; the
// stores are global-memory instructions, not flat ones)
__device__ __forceinline__ void store4(gptr<float> out, int V, bool vec, int64_t idx,
                                       const float (&o)[4]) {
  if (vec) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    v4f q;
    q.x = o[0];
    q.y = o[1];
    q.z = o[2];
    q.w = o[3];
    *(gptr<v4f>)(out + idx) = q;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (idx + e < V) out[idx + e] = o[e];
  }
}

// Renormalise (top-k, top-p) or mask (top-k logits) one row with the
// streaming engine; every thread of the work-group must call this.
template <int KIND>
__device__ __forceinline__ void renorm_row(const RenormParams& P, int row, RedSmem& red) {
  const int V = P.vocab;
  const RowRef r{as_global(P.in + (int64_t)row * V), V, P.vec_ok != 0};
  const gptr<float> out = as_global(P.out + (int64_t)row * V);
  const int nvec = (V + 3) / 4;
  const int k = P.top_k_arr ? P.top_k_arr[row] : P.top_k;
  const float pp = P.top_p_arr ? P.top_p_arr[row] : P.top_p;

  // pass 0: max key, total mass, NaN (logits) / sign-inf-NaN (probs) check
  Red acc = red_zero();
  for_each4(r, [&](int64_t idx, const float (&v)[4], bool valid) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = valid && idx + e < V;
      if (KIND == kMaskLogits) {
        acc.mx = max(acc.mx, in ? signed_key(v[e]) : 0u);
        acc.s0 += (in && (bits_of(v[e]) & 0x7FFFFFFFu) > 0x7F800000u) ? 1u : 0u;
      } else {
        acc.mx = max(acc.mx, in ? bits_of(v[e]) : 0u);
        acc.d0 += in ? (double)v[e] : 0.0;
      }
    }
  });
  const Red s0 = block_reduce(acc, red);
  bool ok;
  if (KIND == kMaskLogits) {
    ok = s0.s0 == 0u && k > 0;
  } else {
    ok = s0.mx < 0x7F800000u && s0.d0 > 0.0;
    if (KIND == kRenormTopK) ok = ok && k > 0;
    if (KIND == kRenormTopP) ok = ok && !isnan(pp);
  }
  if (!ok) {
    const float qnan = __uint_as_float(0x7FC00000u);
    const float o[4] = {qnan, qnan, qnan, qnan};
    for (int f = threadIdx.x; f < nvec; f += kBlock) store4(out, V, P.vec_ok != 0, 4ll * f, o);
    if (P.row_status && threadIdx.x == 0) P.row_status[row] = 1;
    return;
  }

  uint32_t tau;
  if (KIND == kRenormTopK) {
    tau = (k >= V) ? 0u : threshold_search<false, false>(r, 0u, s0.mx + 1u, (uint32_t)k, 0.0, red);
  } else if (KIND == kRenormTopP) {
    const float pc = clamp01(pp);
    if (pc >= 1.0f) {
      tau = 0u;  // every positive value is kept; zeros renormalise to zero anyway
    } else if (pc <= 0.0f) {
      tau = s0.mx;  // only the maximum and its ties
    } else {
      tau = threshold_search<true, false>(r, 0u, s0.mx + 1u, 0u, (double)pc * s0.d0, red);
    }
  } else {
    tau = (k >= V) ? 0u : threshold_search<false, true>(r, 0u, s0.mx + 1u, (uint32_t)k, 0.0, red);
  }

  if (KIND == kMaskLogits) {
    const float ninf = __uint_as_float(0xFF800000u);
    // invalid groups are copies of the last one: never stored (the op may
    // run in place, where a repeated store could write a value twice renormalised)
    for_each4(r, [&](int64_t idx, const float (&v)[4], bool valid) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = signed_key(v[e]) >= tau ? v[e] : ninf;
      if (valid) store4(out, V, P.vec_ok != 0, idx, o);
    });
  } else {
    const double zk = mass_at_least(r, tau, red).d0;
    const double inv = 1.0 / zk;
    for_each4(r, [&](int64_t idx, const float (&v)[4], bool valid) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = bits_of(v[e]) >= tau ? (float)((double)v[e] * inv) : 0.0f;
      if (valid) store4(out, V, P.vec_ok != 0, idx, o);
    });
  }
  if (P.row_status && threadIdx.x == 0) P.row_status[row] = 0;
}

// One wave: the largest bin b of md[0, NB) whose mass from the top,
// M(b) = sum_{b' >= b} md[b'], reaches `need` (need = pfrac * total when
// pfrac >= 0) and is positive; `above` = M(b + 1).  If rounding leaves every
// M(b) below need, the lowest bin with mass is taken (everything kept).
// Lane l sums the chunk of NB / 64 bins that is l-th from the top; a scan
// over lanes finds the chunk and a scan over that chunk's bins the bin.
template <int NB>
__device__ __forceinline__ void mass_find(const double* md, double need, double pfrac, uint32_t& bin,
                          double& above, double& total) {
  constexpr int C = NB / kWave;
  const int lane = lane_id();
  const int c = kWave - 1 - lane;
  double s = 0.0;
#pragma unroll
  for (int q = C - 1; q >= 0; --q) {
    if ((q & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // four reads in flight at a time
    s += md[c * C + q];
  }
  const double incl = wave_incl_scan(s);
  const double excl = wave_excl_from_incl(incl);
  total = lane63(incl);
  if (pfrac >= 0.0) need = pfrac * total;
  uint64_t hit = __ballot(incl >= need && incl > 0.0);
  int L = hit ? (__ffsll((long long)hit) - 1) : (63 - __clzll((long long)(__ballot(s > 0.0) | 1ull)));
  const bool fallback = hit == 0ull;
  const int cc = kWave - 1 - L;
  const double ex = lane_value(excl, L);
  const double m = lane < C ? md[cc * C + C - 1 - lane] : 0.0;
  const double incl2 = wave_incl_scan(m) + ex;
  const double sh = wave_excl_from_incl(incl2);
  const double excl2 = lane == 0 ? ex : sh;
  uint64_t hit2 = fallback ? 0ull : __ballot(lane < C && incl2 >= need && incl2 > 0.0);
  if (hit2 == 0ull) hit2 = 1ull << (63 - __clzll((long long)(__ballot(lane < C && m > 0.0) | 1ull)));
  const int Q = __ffsll((long long)hit2) - 1;
  bin = (uint32_t)(cc * C + C - 1 - Q);
  above = lane_value(excl2, Q);
}

// ---- exact top-k / top-k-then-top-p sampling, one work-group per output ---
//
// The split engine's in-kernel fallback for rows it cannot bound (k above its
// cap, flat rows, huge tie groups).  Instead of the rejection loop from
// low = 0 (one pass per round, many rounds on rows whose kept set reaches
// deep into a long tail) it finds the kept set exactly, as the resident
// engine does, with passes over the row: tau_k by count histograms of bits
// [30:21], [20:10] and [9:0] (the F4 note's threshold search on the bit
// pattern, 1023 pivots per pass), the top-p cut inside {x >= tau_k} by the
// same three levels on exact significand sums, then one inverse-transform
// draw over {x >= tau} (blog, 逆变换采样): tile masses, then one tile.
// About eight passes whatever the row.

struct RadixSmem {
  uint64_t hh[2048];   // one level's histogram (counts, or significand sums)
  double md[2048];     // the level as counts or masses
  SampleSmem s;        // tile masses and the locate() scratch
  uint32_t res[4];
  double resd[4];
};

__device__ __forceinline__ uint32_t radix_sig(uint32_t key) {
  return (key & 0x7FFFFFu) | (key >= 0x800000u ? 0x800000u : 0u);
}

// One pass: the values with pattern >= cut and pattern >> hs == prefix, by
// bin (pattern >> ls) & (NB - 1): counts, or 24-bit significand sums (each
// bin one quarter-binade or part of one, so exact integers); folded into md
// as counts or masses (exponent e; e < 0: level 1, bin b holds exponent
// b >> 2).  Every thread calls.
template <bool COUNT, int NB>
__device__ __forceinline__ void radix_pass(const RowRef& r, uint32_t cut, int hs, uint32_t prefix,
                                           int ls, int e, RadixSmem& sm) {
  // 2048 / NB copies of every bin (lane parity picks one with two copies),
  // so that lanes piling into one bin mostly hit different words
  constexpr uint32_t C = 2048 / NB;
  const uint32_t cp = (uint32_t)lane_id() & (C - 1u);
  for (int b = threadIdx.x; b < 2048; b += kBlock) sm.hh[b] = 0ull;
  __syncthreads();
  for_each4(r, [&](int64_t idx, const float (&v)[4], bool valid) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t key = bits_of(v[q]);
      if (valid && idx + q < r.V && key >= cut && (key >> hs) == prefix)
        atomicAdd(&sm.hh[((key >> ls) & (uint32_t)(NB - 1)) * C + cp],
                  COUNT ? 1ull : (unsigned long long)radix_sig(key));
    }
  });
  __syncthreads();
  for (int b = threadIdx.x; b < NB; b += kBlock) {
    uint64_t x = 0ull;
#pragma unroll
    for (uint32_t c = 0; c < C; ++c) x += sm.hh[b * C + c];
    const uint32_t ex = e < 0 ? (uint32_t)b >> 2 : (uint32_t)e;
    sm.md[b] = COUNT ? (double)x : ldexp((double)x, (int)max(ex, 1u) - 150);
  }
  __syncthreads();
}

// tau = the largest pattern t with F(t) >= need, F(t) the count (COUNT) or
// mass of the values >= max(t, cut); pfrac >= 0 sets need = pfrac * F(cut).
// kept = F(tau).  A count search from cut = 0 also checks the row: a value
// with the sign bit set is left out of the level-1 total, an inf or NaN
// falls in the top four bins; either sets `bad` and ends the search.  Every
// thread calls.
template <bool COUNT>
__device__ __forceinline__ void radix_search(const RowRef& r, uint32_t cut, double need_in,
                                             double pfrac, RadixSmem& sm, uint32_t& tau,
                                             double& kept, bool& bad) {
  const int lane = lane_id(), wave = wave_id();
  radix_pass<COUNT, 1024>(r, cut, 31, 0u, 21, -1, sm);
  if (wave == 0) {
    uint32_t b;
    double above, total;
    mass_find<1024>(sm.md, need_in, pfrac, b, above, total);
    if (lane == 0) {
      sm.res[0] = b;
      sm.res[3] = (COUNT && cut == 0u &&
                   (total < (double)r.V || sm.md[1020] + sm.md[1021] + sm.md[1022] + sm.md[1023] > 0.0))
                      ? 1u : 0u;
      sm.resd[0] = above;
      sm.resd[1] = total;
      sm.resd[2] = pfrac >= 0.0 ? pfrac * total : need_in;
    }
  }
  __syncthreads();
  const uint32_t b1 = sm.res[0];
  const double above1 = sm.resd[0], ftot = sm.resd[1], need = sm.resd[2];
  bad = sm.res[3] != 0u;
  __syncthreads();
  if (bad) return;
  if (!COUNT && pfrac >= 1.0) {  // every value >= cut
    tau = cut;
    kept = ftot;
    return;
  }
  const int e1 = (int)(b1 >> 2);
  radix_pass<COUNT, 2048>(r, cut, 21, b1, 10, e1, sm);
  if (wave == 0) {
    uint32_t b;
    double above, total;
    mass_find<2048>(sm.md, need - above1, -1.0, b, above, total);
    if (lane == 0) {
      sm.res[1] = b;
      sm.resd[0] = above;
    }
  }
  __syncthreads();
  const uint32_t pre2 = (b1 << 11) | sm.res[1];
  const double above2 = sm.resd[0];
  __syncthreads();
  radix_pass<COUNT, 1024>(r, cut, 10, pre2, 0, e1, sm);
  if (wave == 0) {
    uint32_t b;
    double above, total;
    mass_find<1024>(sm.md, need - above1 - above2, -1.0, b, above, total);
    if (lane == 0) {
      sm.res[2] = b;
      sm.resd[0] = above;
      sm.resd[1] = sm.md[b];
    }
  }
  __syncthreads();
  tau = (pre2 << 10) | sm.res[2];
  kept = above1 + above2 + (sm.resd[0] + sm.resd[1]);
  __syncthreads();
}

// Output i by the exact passes above (OP: top-k; top-k-then-top-p, whose
// top-p target is p * Z_k; or the joint order, whose top-p cut is taken on
// the whole row and the kept set is {x >= max(tau_k, tau_p)}); rounds = 1.
// Every thread calls.
template <int OP>
__device__ __forceinline__ void sample_row_exact(const SampleParams& P, int i, RadixSmem& sm) {
  static_assert(OP == kOpTopK || OP == kOpTopKTopP || OP == kOpTopKTopPJoint,
                "the top-k filters only");
  constexpr bool kP = OP == kOpTopKTopP || OP == kOpTopKTopPJoint;
  const int lane = lane_id(), wave = wave_id();
  const int row = P.indices ? as_global(P.indices)[i] : i;
  const int k = P.top_k_arr ? as_global(P.top_k_arr)[i] : P.top_k;
  const float pp = kP ? (P.top_p_arr ? as_global(P.top_p_arr)[i] : P.top_p) : 0.0f;
  if (!(row >= 0 && row < P.rows) || k <= 0 || isnan(pp)) {  // block-uniform
    if (threadIdx.x == 0) write_sample(P, i, -1, 0);
    return;
  }
  const uint64_t seed = P.seed_arr ? as_global(P.seed_arr)[i] : P.seed;
  const uint64_t offset = P.offset_arr ? as_global(P.offset_arr)[i] : P.offset;
  const uint64_t sid = P.seed_arr ? 0ull : (uint64_t)i;
  const RowRef r{as_global(P.probs + (int64_t)row * P.vocab), P.vocab, P.vec_ok != 0};
  const int n_tiles = (P.vocab + kTile - 1) / kTile;

  // tau_k (the count search also rejects a row with a sign bit, inf or
  // NaN; a row with nothing positive ends with an empty draw below)
  uint32_t tk;
  double cnt;
  bool bad;
  radix_search<true>(r, 0u, (double)k, -1.0, sm, tk, cnt, bad);
  if (bad) {
    if (threadIdx.x == 0) write_sample(P, i, -1, 0);
    return;
  }
  uint32_t tau = max(tk, 1u);  // zeros carry no mass
  if (kP) {
    // top-k first: the cut inside {x >= tau_k}; joint: on the whole row
    uint32_t tp;
    double zk;
    radix_search<false>(r, OP == kOpTopKTopP ? tau : 1u, 0.0, (double)clamp01(pp), sm, tp, zk, bad);
    tau = max(tp, tau);
  }
  // one draw over {x >= tau} = {x > low}
  const float low = __uint_as_float(tau - 1u);
  uint32_t ca = 0u, cb = 0u;
  pivot_pass(r, n_tiles, low, low, sm.s.tm[0], sm.s.tm[1], ca, cb);
  __syncthreads();
  if (wave == 0) {
    const double z = tile_scan_total(sm.s.tm[0], n_tiles);
    if (lane == 0) sm.s.bc_d[0] = z * draw_uniform(seed, offset, sid, 0u);
  }
  __syncthreads();
  const double T = sm.s.bc_d[0];
  __syncthreads();
  const int tok = locate(r, sm.s.tm[0], n_tiles, T, low, sm.s);
  if (threadIdx.x == 0) write_sample(P, i, tok, tok >= 0 ? 1 : 0);
}

// ---- top-k selection (explainer, 选择 top-k 值本身) ----------------------

// A row with no top-k set (a NaN in it): NaN values, index -1, status 1.
__device__ __forceinline__ void select_invalid(const SelectParams& Q, int row) {
  const gptr<float> vo = as_global(Q.values + (int64_t)row * Q.k);
  const gptr<int32_t> io = as_global(Q.indices + (int64_t)row * Q.k);
  for (int j = threadIdx.x; j < Q.k; j += kBlock) {
    vo[j] = __uint_as_float(0x7FC00000u);
    io[j] = -1;
  }
  if (Q.row_status && threadIdx.x == 0) Q.row_status[row] = 1;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Compare-exchange of the entries at positions i < j: ascending (i takes the
// smaller) when `up`, else descending.
__device__ __forceinline__ void cmp_swap(uint64_t& a, uint64_t& b, bool up) {
  const uint64_t lo = a < b ? a : b, hi = a < b ? b : a;
  a = up ? lo : hi;
  b = up ? hi : lo;
}

// One step of a bitonic network on the 256 entries one wave holds, entry
// base + 64 r + lane in x[r]: the pairs `stride` apart, ascending inside a
// block of `size` entries whose `size` bit is set, descending otherwise.
__device__ __forceinline__ void chunk_step(uint64_t (&x)[4], uint32_t base, uint32_t size,
                                           uint32_t stride, uint32_t lane) {
  if (stride == 128u) {
    cmp_swap(x[0], x[2], ((base + lane) & size) != 0u);
    cmp_swap(x[1], x[3], ((base + 64u + lane) & size) != 0u);
  } else if (stride == 64u) {
    cmp_swap(x[0], x[1], ((base + lane) & size) != 0u);
    cmp_swap(x[2], x[3], ((base + 128u + lane) & size) != 0u);
  } else {
    const bool lower = (lane & stride) == 0u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint64_t y = shfl_xor_u64(x[r], (int)stride);
      const bool up = ((base + 64u * r + lane) & size) != 0u;
      x[r] = (lower == up) ? (x[r] < y ? x[r] : y) : (x[r] < y ? y : x[r]);
    }
  }
}

// Sorts ent[0, P) into descending order: P a power of two <= kSelectMax,
// the first n <= P entries given, the rest taken as 0 (below every real
// entry).  A bitonic network in which every wave keeps a chunk of 256
// entries in registers and runs all strides below 256 with lane shuffles;
// only the strides of 256 and more go through LDS, one barrier each (18
// barriers for 4096 entries instead of 78).  With CONV the entries arrive
// as key | index << 32 and are sorted as key << 32 | ~index: descending
// keys, equal keys by ascending index.  Every thread of the work-group
// calls it; it ends with a barrier.
template <bool CONV>
__device__ __forceinline__ void sort_desc(uint64_t* ent, uint32_t n, uint32_t P) {
  const uint32_t tid = threadIdx.x, lane = (uint32_t)lane_id();
  const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane((int)(tid >> 6)) * 256u;
  const bool act = base < P;  // wave-uniform
  uint64_t x[4];
  if (act) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t p = base + 64u * r + lane;
      const uint64_t e = p < n ? ent[p] : 0ull;
      x[r] = (CONV && p < n) ? ((e << 32) | (uint64_t)(~(uint32_t)(e >> 32))) : e;
    }
    const uint32_t top = P < 256u ? P : 256u;
    for (uint32_t size = 2u; size <= top; size <<= 1)
      for (uint32_t stride = size >> 1; stride > 0u; stride >>= 1)
        chunk_step(x, base, size, stride, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t p = base + 64u * r + lane;
      if (p < P) ent[p] = x[r];
    }
  }
  for (uint32_t size = 512u; size <= P; size <<= 1) {
    __syncthreads();
    for (uint32_t stride = size >> 1; stride >= 256u; stride >>= 1) {
      for (uint32_t t = tid; t < P / 2u; t += kBlock) {
        const uint32_t i = 2u * t - (t & (stride - 1u)), j = i + stride;
        const uint64_t a = ent[i], b = ent[j];
        const bool up = (i & size) != 0u;
        if (up ? (a > b) : (a < b)) {
          ent[i] = b;
          ent[j] = a;
        }
      }
      __syncthreads();
    }
    if (act) {  // P >= 512 here: every active wave's chunk lies inside [0, P)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = ent[base + 64u * r + lane];
      for (uint32_t stride = 128u; stride > 0u; stride >>= 1) chunk_step(x, base, size, stride, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) ent[base + 64u * r + lane] = x[r];
    }
  }
  __syncthreads();
}

// The row's first k sorted entries (key << 32 | ~index): indices, and the
// values, decoded from their signed-order keys; a zero key is read back from
// the row, since -0.0 and +0.0 share it.  Status 0.
__device__ __forceinline__ void select_write(const SelectParams& Q, int row, const uint64_t* ent) {
  const int k = Q.k;
  const gptr<const float> x = as_global(Q.in + (int64_t)row * Q.vocab);
  const gptr<float> vo = as_global(Q.values + (int64_t)row * k);
  const gptr<int32_t> io = as_global(Q.indices + (int64_t)row * k);
  for (int j = threadIdx.x; j < k; j += kBlock) {
    const uint32_t ix = ~(uint32_t)ent[j];
    const uint32_t key = (uint32_t)(ent[j] >> 32);
    // (always a position of the row; the test keeps any read inside it)
    const bool in = ix < (uint32_t)Q.vocab;
    float val = __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
    if (in && key == 0x80000000u) val = x[ix];
    vo[j] = in ? val : __uint_as_float(0x7FC00000u);
    io[j] = in ? (int32_t)ix : -1;
  }
  if (Q.row_status && threadIdx.x == 0) Q.row_status[row] = 0;
}

// Top-k selection (explainer, 选择 top-k 值本身: values and indices rather
// than a sample), one work-group per row: tau = the k-th largest signed-order
// key by the F4 threshold search; one pass counts, per 2048-value tile, the
// values above tau and those equal to it, which fixes where the ties still
// needed end (in index order); a second pass gathers exactly k entries
// (key << 32 | ~index) into LDS; sort_desc puts them in descending key
// order, equal keys by ascending index; the row's values and indices are
// written.  A NaN makes the row invalid (NaN values, index -1, status 1).
struct SelectSmem {
  RedSmem red;
  uint64_t ent[kSelectMax];
  uint32_t ties[kMaxTiles];
  uint32_t n;
  uint32_t cut_tile;
  uint32_t cut_need;
};

__device__ __forceinline__ void select_row(const SelectParams& Q, int row, SelectSmem& sm) {
  const int V = Q.vocab, k = Q.k;
  const int lane = lane_id(), wave = wave_id();
  const RowRef r{as_global(Q.in + (int64_t)row * V), V, Q.vec_ok != 0};
  Red acc = red_zero();
  for_each4(r, [&](int64_t idx, const float (&v)[4], bool valid) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = valid && idx + e < V;
      acc.mx = max(acc.mx, in ? signed_key(v[e]) : 0u);
      acc.s0 += (in && isnan(v[e])) ? 1u : 0u;
    }
  });
  const Red s0 = block_reduce(acc, sm.red);
  if (s0.s0 != 0u) {
    select_invalid(Q, row);
    return;
  }
  // the k-th largest key (k <= V); keys of real values are >= 1
  const uint32_t tau = threshold_search<false, true>(r, 0u, s0.mx + 1u, (uint32_t)k, 0.0, sm.red);

  // per tile: values equal to tau; above tau over the row
  const int n_tiles = (V + kTile - 1) / kTile;
  uint32_t gt = 0u;
  for (int t = wave; t < n_tiles; t += kWaves) {
    const int64_t base = (int64_t)t * kTile;
    uint32_t eq = 0u;
    // a quarter of a tile per batch (the selection kernels keep much else live)
    for (int h = 0; h < kTileChunks; h += kTileChunks / 4) {
      float vt[kTileChunks / 4][4];
      load4_batch<kTileChunks / 4>(r, [&](int q) { return base + (h + q) * (kWave * 4) + lane * 4; },
                                   vt);
#pragma unroll
      for (int q = 0; q < kTileChunks / 4; ++q) {
        const float (&v)[4] = vt[q];
        const int64_t idx = base + (h + q) * (kWave * 4) + lane * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = idx + e < V ? signed_key(v[e]) : 0u;
          eq += key == tau ? 1u : 0u;
          gt += key > tau ? 1u : 0u;
        }
      }
    }
    eq = wave_sum(eq);
    if (lane == 0) sm.ties[t] = eq;
  }
  Red cg = red_zero();
  cg.s0 = gt;
  const uint32_t above = block_reduce(cg, sm.red).s0;  // (its barriers also publish ties[])
  if (wave == 0) {
    // the tile where the ties still needed (k - above, in index order) end
    const uint32_t need = (uint32_t)k - above;
    uint32_t carry = 0u;
    bool found = false;
    for (int base = 0; base < n_tiles && !found; base += kWave) {
      const int t = base + lane;
      const uint32_t c = t < n_tiles ? sm.ties[t] : 0u;
      const uint32_t incl = wave_incl_scan(c) + carry;
      const uint64_t hit = __ballot(t < n_tiles && incl >= need && c > 0u);
      if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        if (lane == 0) {
          sm.cut_tile = (uint32_t)(base + l);
          sm.cut_need = need - (lane_value(incl, l) - lane_value(c, l));
        }
        found = true;
      }
      carry = lane63(incl);
    }
    if (!found && lane == 0) {  // need == 0 cannot happen (count(key >= tau) >= k > above)
      sm.cut_tile = 0u;
      sm.cut_need = 0u;
    }
    if (lane == 0) sm.n = 0u;
  }
  __syncthreads();
  const uint32_t cut = sm.cut_tile, cneed = sm.cut_need;

  // gather: every value above tau; the ties of tiles before the cut; the
  // first cneed ties (index order) of the cut tile
  for (int t = wave; t < n_tiles; t += kWaves) {
    const int64_t base = (int64_t)t * kTile;
    uint32_t tie_carry = 0u;
    for (int h = 0; h < kTileChunks; h += kTileChunks / 4) {
    float vt[kTileChunks / 4][4];
    load4_batch<kTileChunks / 4>(r, [&](int q) { return base + (h + q) * (kWave * 4) + lane * 4; },
                                 vt);
#pragma unroll
    for (int q = 0; q < kTileChunks / 4; ++q) {
      const float (&v)[4] = vt[q];
      const int64_t idx = base + (h + q) * (kWave * 4) + lane * 4;
      uint32_t key[4];
      uint32_t my_ties = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[e] = idx + e < V ? signed_key(v[e]) : 0u;
        my_ties += key[e] == tau ? 1u : 0u;
      }
      const uint32_t tincl = wave_incl_scan(my_ties);
      uint32_t trank = tie_carry + tincl - my_ties;  // ties before this lane's first value
      bool take[4];
      uint32_t cnt = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool tie = key[e] == tau;
        take[e] = key[e] > tau || (tie && ((uint32_t)t < cut || ((uint32_t)t == cut && trank < cneed)));
        trank += tie ? 1u : 0u;
        cnt += take[e] ? 1u : 0u;
      }
      tie_carry += lane63(tincl);
      const uint32_t cincl = wave_incl_scan(cnt);
      uint32_t pos = 0u;
      if (lane == kWave - 1 && cincl > 0u) pos = atomicAdd(&sm.n, cincl);
      pos = __shfl(pos, kWave - 1) + cincl - cnt;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (take[e] && pos < (uint32_t)kSelectMax)
          sm.ent[pos] = ((uint64_t)key[e] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(idx + e));
        pos += take[e] ? 1u : 0u;
      }
    }
    }
  }
  __syncthreads();
  uint32_t P = 1u;
  while (P < (uint32_t)k) P <<= 1;
  sort_desc<false>(sm.ent, (uint32_t)k, P);
  select_write(Q, row, sm.ent);
}

// Probabilities of one row from logits with a temperature (explainer,
// 采样流水线究竟在计算什么), one work-group, three passes over the row: the
// maximum m (and NaN / +inf), S = the sum of exp((z - m) * (1 / T)), then
// out = float32(exp((z - m) * (1 / T)) / S), all in float64.  A NaN or +inf
// logit, no finite logit, or T not a finite positive number NaN-fill the
// row; returns whether it was valid.  Every thread calls.
__device__ __forceinline__ bool softmax_row(const float* in, float* out_row, int V, float T, bool vec,
                                   RedSmem& red) {
  const RowRef r{as_global(in), V, vec};
  const gptr<float> out = as_global(out_row);
  Red acc = red_zero();
  for_each4(r, [&](int64_t idx, const float (&v)[4], bool valid) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = valid && idx + e < V;
      acc.mx = max(acc.mx, ok ? signed_key(v[e]) : 0u);
      acc.s0 += (ok && (isnan(v[e]) || v[e] == __builtin_inff())) ? 1u : 0u;
    }
  });
  const Red s0 = block_reduce(acc, red);
  const float zmax = from_signed_key(s0.mx);
  const int nvec = (V + 3) / 4;
  if (s0.s0 != 0u || !(T > 0.0f) || T == __builtin_inff() || zmax == -__builtin_inff()) {
    const float qnan = __uint_as_float(0x7FC00000u);
    const float o[4] = {qnan, qnan, qnan, qnan};
    for (int f = threadIdx.x; f < nvec; f += kBlock) store4(out, V, vec, 4ll * f, o);
    return false;
  }
  const double m = (double)zmax, it = 1.0 / (double)T;
  Red sum = red_zero();
  for_each4(r, [&](int64_t idx, const float (&v)[4], bool valid) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sum.d0 += (valid && idx + e < V) ? exp(((double)v[e] - m) * it) : 0.0;
  });
  const double S = block_reduce(sum, red).d0;
  for_each4(r, [&](int64_t idx, const float (&v)[4], bool valid) {
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (float)(exp(((double)v[e] - m) * it) / S);
    if (valid) store4(out, V, vec, idx, o);
  });
  return true;
}

}  // namespace stream
}  // namespace dss
