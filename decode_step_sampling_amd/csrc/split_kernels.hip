// Split-row engine for top-k and top-k-then-top-p sampling.
//
// The dual-pivot rejection loop of the FlashInfer blog ("Sorting-Free GPU
// Kernels for LLM Sampling", section 双枢轴拒绝采样) only ever draws from the
// values above the current `low`, and its correctness proof (section
// 拒绝采样器正确性的理论证明) holds from any starting pivot below every kept
// value.  This engine therefore:
//
//  1. splits each row into W slices, one 1024-thread work-group per slice,
//     and reads every slice from HBM exactly once into registers (16-byte
//     loads);
//  2. each slice finds a local bound t_s whose upper set holds at least k of
//     its values, from a 2048-bin LDS histogram of the float32 bit patterns
//     (bits >> 20: 1/8-binade bins) of the values within 8 binades of the
//     slice maximum (all values if that is not enough), and publishes those
//     few values with their indices.  The union over slices contains every
//     value >= t* = max_s t_s of the row, and at least k of them;
//  3. the last slice work-group of the row to finish (a relaxed arrival
//     counter) gathers the candidates, finds the k-th largest tau_k with three
//     histogram passes over the bit fields (the F4 note's threshold search on
//     the float32 bit pattern, §③, done 2048 ways per pass instead of 2 or 3)
//     and runs the dual-pivot loop on the candidates from just below tau_k,
//     where f(low) = 0 still holds.  That tail runs on four waves, one per
//     SIMD, so its serial steps are not shared four ways.
//
// All W work-groups of a row are placed on one XCD (work-groups are dispatched
// to the eight XCDs round-robin, so block b runs on XCD b % 8), which lets the
// hand-off use the XCD's shared L2 with relaxed atomics instead of
// device-wide acquire/release fences (measured at several microseconds each
// on gfx950).  Every published header carries the row's generation number and
// the writer's XCC id; the finishing work-group checks both and falls back to
// the streaming engine (stream_device.h) if anything looks foreign, if a
// slice overflowed its candidate buffer, or if k is too large to bound.
#include "stream_device.h"

namespace dss {
namespace {

constexpr int kHistBins = 2048;
constexpr int kSliceCandMax = 4096;
constexpr int kWaveCap = 512;  // per-wave append buffer during the read
constexpr int kRowCandMax = 8192;
constexpr int kSplitKCap = 1536;
constexpr int kMaxSlices = 16;
constexpr int kHdrWords = 8;
constexpr int kTailWaves = 4;
constexpr int kTailThreads = kTailWaves * kWave;

struct SplitParams {
  int W;           // slices per output
  int L;           // slice length in values (multiple of 4)
  int out0;        // first output handled by this launch
  int n_out;       // outputs handled by this launch
  uint32_t* ctr;   // [kChunk] arrival counters (zero between calls)
  uint32_t* gen;   // [kChunk] generation numbers
  uint32_t* hdr;   // [n_out][W][kHdrWords]
  uint64_t* cand;  // [n_out][W][kSliceCandMax]: bits | (index << 32)
};

struct SplitSmem {
  union {
    struct {
      uint32_t bits[kWaves][kWaveCap];
      uint32_t idx[kWaves][kWaveCap];
    } pw;                         // per-wave appends during the read
    stream::SampleSmem stream;    // streaming fallback
  } a;
  struct {
    uint32_t bits[kRowCandMax];
    uint32_t idx[kRowCandMax];
  } c;                            // candidates, compacted
  uint32_t hist[kHistBins];
  double draws[stream::kPreDraws];
  double red_d[kWaves][2];
  uint32_t red_u[kWaves][4];
  uint32_t wcnt[kWaves];
  uint32_t hdr[kMaxSlices][kHdrWords];
  uint32_t off[kMaxSlices + 1];
  uint32_t gen;
  int flag;
  int hit_lane[kWaves];
  int tok;
  uint32_t res[4];
  double extra_u;
};

__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20) & 0xFu;  // HW_REG_XCC_ID
}

// wave index as a scalar, so branches on it are scalar branches
__device__ __forceinline__ int uwave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// work-group helpers over the first NW waves (every participating thread
// must call; fixed association order, so results are deterministic)
// ---------------------------------------------------------------------------

template <int NW>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t& total, SplitSmem& sm) {
  const int lane = lane_id(), w = uwave();
  const uint32_t incl = wave_incl_scan(v);
  if (lane == kWave - 1) sm.red_u[w][0] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    const uint32_t t = sm.red_u[q][0];
    base += q < w ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

template <int NW>
__device__ double block_excl_scan(double v, SplitSmem& sm) {
  const int lane = lane_id(), w = uwave();
  const double incl = wave_incl_scan(v);
  const double excl = wave_excl_from_incl(incl);
  if (lane == kWave - 1) sm.red_d[w][0] = incl;
  __syncthreads();
  double base = 0.0;
#pragma unroll
  for (int q = 0; q < NW; ++q) base += q < w ? sm.red_d[q][0] : 0.0;
  __syncthreads();
  return base + excl;
}

struct Pair {
  double m0, m1;
  uint32_t c0, c1;
};

template <int NW>
__device__ Pair block_sum(Pair v, SplitSmem& sm) {
  v.m0 = wave_sum(v.m0);
  v.m1 = wave_sum(v.m1);
  v.c0 = wave_sum(v.c0);
  v.c1 = wave_sum(v.c1);
  if (lane_id() == 0) {
    const int w = uwave();
    sm.red_d[w][0] = v.m0;
    sm.red_d[w][1] = v.m1;
    sm.red_u[w][0] = v.c0;
    sm.red_u[w][1] = v.c1;
  }
  __syncthreads();
  Pair out{0.0, 0.0, 0u, 0u};
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    out.m0 += sm.red_d[q][0];
    out.m1 += sm.red_d[q][1];
    out.c0 += sm.red_u[q][0];
    out.c1 += sm.red_u[q][1];
  }
  __syncthreads();
  return out;
}

template <int NW>
__device__ uint32_t block_max(uint32_t v, SplitSmem& sm) {
  v = wave_max(v);
  if (lane_id() == 0) sm.red_u[uwave()][0] = v;
  __syncthreads();
  uint32_t out = 0;
#pragma unroll
  for (int q = 0; q < NW; ++q) out = max(out, sm.red_u[q][0]);
  __syncthreads();
  return out;
}

// Largest bin b of hist[0..nb) whose suffix count sum_{b' >= b} hist[b']
// reaches need; returns b, the count strictly above b, and the total.  If
// the total is below need, returns bin 0.  Thread t owns the bins
// nb-1-t*BPT down to nb-(t+1)*BPT.
template <int NW>
__device__ void suffix_find(const uint32_t* hist, int nb, uint32_t need, uint32_t& bin,
                            uint32_t& above, uint32_t& total, SplitSmem& sm) {
  constexpr int T = NW * kWave;
  const int bpt = (nb + T - 1) / T;
  const int t = threadIdx.x;
  const int top = nb - 1 - t * bpt;
  uint32_t mine = 0u;
  for (int q = 0; q < bpt; ++q) {
    const int b = top - q;
    if (b >= 0) mine += hist[b];
  }
  const uint32_t excl = block_excl_scan<NW>(mine, total, sm);
  if (t == 0) {
    sm.res[0] = 0u;
    sm.res[1] = total - hist[0];
  }
  __syncthreads();
  if (excl < need && excl + mine >= need) {
    uint32_t run = excl;
    for (int q = 0; q < bpt; ++q) {
      const int b = top - q;
      const uint32_t h = b >= 0 ? hist[b] : 0u;
      if (run + h >= need) {
        sm.res[0] = (uint32_t)b;
        sm.res[1] = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
  bin = sm.res[0];
  above = sm.res[1];
  __syncthreads();
}

// k-th largest bit pattern among bits[0..n) (1 <= k <= n; non-negative
// floats, so bit 31 is clear): three histogram passes over bit fields
// [30:20], [19:9] and [8:0], each keeping only the values that match the
// bits fixed so far.
template <int NW>
__device__ uint32_t kth_largest(const uint32_t* bits, int n, uint32_t k, SplitSmem& sm) {
  constexpr int T = NW * kWave;
  uint32_t prefix = 0u, pmask = 0u;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = pass == 0 ? 20 : pass == 1 ? 9 : 0;
    const int nb = pass == 2 ? 512 : 2048;
    for (int q = threadIdx.x; q < nb; q += T) sm.hist[q] = 0u;
    __syncthreads();
    for (int c = threadIdx.x; c < n; c += T) {
      const uint32_t x = bits[c];
      if ((x & pmask) == prefix) atomicAdd(&sm.hist[(x >> sh) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    uint32_t bin, above, total;
    suffix_find<NW>(sm.hist, nb, k, bin, above, total, sm);
    k -= above;
    prefix |= bin << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
  }
  return prefix;
}

template <int OP>
__device__ __forceinline__ bool split_predicate(double mass_above, uint32_t count_above, int k,
                                                double pz) {
  const bool ok_k = count_above < (uint32_t)k;
  if (OP == kOpTopK) return ok_k;
  return ok_k && ((mass_above < pz) || count_above == 0u);
}

// The rejection loop on the candidates sm.c.bits/idx[0..n) (every value
// above `low` of the row is among them), run by the first NW waves.  Thread
// t owns the contiguous entries [t*E, t*E + E); the inverse-transform draw
// runs over the entries in that order.  Returns the token (row index) or -1.
template <int OP, int NW>
__device__ int candidate_loop(SplitSmem& sm, int n, float low, float high, int k, double pz,
                              uint64_t seed, uint64_t offset, uint64_t sid, int& rounds) {
  constexpr int T = NW * kWave;
  const int E = (n + T - 1) / T;
  const int c0 = min(n, (int)threadIdx.x * E), c1 = min(n, c0 + E);
  const uint32_t* cb = sm.c.bits;
  const int lane = lane_id(), w = uwave();

  Pair acc{0.0, 0.0, 0u, 0u};
  for (int c = c0; c < c1; ++c) {
    const float x = __uint_as_float(cb[c]);
    if (x > low) acc.m0 += (double)x;
  }
  double S = block_sum<NW>(acc, sm).m0;  // S(low)

  int rnd = 0;
  while (true) {
    double u;
    if (rnd < stream::kPreDraws) {
      u = sm.draws[rnd];
    } else {
      if (threadIdx.x == 0) sm.extra_u = draw_uniform(seed, offset, sid, (uint32_t)rnd);
      __syncthreads();
      u = sm.extra_u;
      __syncthreads();
    }
    ++rnd;
    const double T_ = u * S;
    // locate: the first candidate, in entry order, whose running sum exceeds
    // T_; guards as in the streaming engine (first hit wins; if rounding puts
    // T_ past every sum, the last candidate is taken)
    double part = 0.0;
    for (int c = c0; c < c1; ++c) {
      const float x = __uint_as_float(cb[c]);
      if (x > low) part += (double)x;
    }
    const double excl = block_excl_scan<NW>(part, sm);
    const uint64_t hm = __ballot(part > 0.0 && excl + part > T_);
    const uint64_t nz = __ballot(part > 0.0);
    if (lane == 0) {
      sm.hit_lane[w] = hm ? (__ffsll((long long)hm) - 1) : -1;
      sm.red_u[w][2] = nz ? (uint32_t)(64 - __clzll((long long)nz)) : 0u;
    }
    __syncthreads();
    int win = -1, last = -1;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      if (win < 0 && sm.hit_lane[q] >= 0) win = q * kWave + sm.hit_lane[q];
      if (sm.red_u[q][2] > 0u) last = q * kWave + (int)sm.red_u[q][2] - 1;
    }
    const int owner = win >= 0 ? win : last;
    if ((int)threadIdx.x == owner) {
      int tok = -1, last_c = -1;
      double run = excl;
      for (int c = c0; c < c1; ++c) {
        const float x = __uint_as_float(cb[c]);
        if (x > low) {
          run += (double)x;
          last_c = c;
          if (win >= 0 && run > T_) {
            tok = c;
            break;
          }
        }
      }
      sm.tok = tok >= 0 ? tok : last_c;
    }
    if (owner < 0 && threadIdx.x == 0) sm.tok = -1;
    __syncthreads();
    const int e = sm.tok;
    __syncthreads();
    if (e < 0) {
      rounds = rnd;
      return -1;
    }
    const float pivot1 = __uint_as_float(cb[e]);
    const int token = (int)sm.c.idx[e];
    const float pivot2 = (float)(((double)pivot1 + (double)high) * 0.5);
    Pair pv{0.0, 0.0, 0u, 0u};
    for (int c = c0; c < c1; ++c) {
      const float x = __uint_as_float(cb[c]);
      if (x > pivot1) {
        pv.m0 += (double)x;
        pv.c0 += 1u;
      }
      if (x > pivot2) {
        pv.m1 += (double)x;
        pv.c1 += 1u;
      }
    }
    pv = block_sum<NW>(pv, sm);
    if (split_predicate<OP>(pv.m0, pv.c0, k, pz)) {
      rounds = rnd;
      return token;
    }
    if (split_predicate<OP>(pv.m1, pv.c1, k, pz)) {
      low = pivot1;
      high = pivot2;
      S = pv.m0;
    } else {
      low = pivot2;
      S = pv.m1;
    }
    if (rnd >= stream::kMaxRounds) {
      rounds = rnd;
      return -1;
    }
  }
}

enum SplitMode : int { kDone = 0, kFallback = 1 };

// Everything but the streaming fallback; returns kFallback when the output
// must be sampled by the streaming engine instead (one call site, below).
template <int OP, int NV>
__device__ __forceinline__ int split_sample(const SampleParams& P, const SplitParams& S,
                                           SplitSmem& sm, int& out_i) {
  const int W = S.W;
  const int b = blockIdx.x, xcd = b & 7, local = b >> 3;
  const int li = (local / W) * 8 + xcd;  // the W slices of an output share b % 8
  const int s = local % W;
  if (li >= S.n_out) return kDone;
  const int i = S.out0 + li;
  out_i = i;
  const int tid = threadIdx.x, lane = lane_id(), wave = uwave();

  const int row = P.indices ? P.indices[i] : i;
  const int k = P.top_k_arr ? P.top_k_arr[i] : P.top_k;
  const float pp = (OP == kOpTopKTopP) ? (P.top_p_arr ? P.top_p_arr[i] : P.top_p) : 0.0f;
  const bool ok = row >= 0 && row < P.rows && k > 0 && (OP != kOpTopKTopP || !isnan(pp));
  if (!ok || k > kSplitKCap) {
    // no hand-off for this output: slice 0 answers alone
    if (s != 0) return kDone;
    if (!ok) {
      if (tid == 0) stream::write_sample(P, i, -1, 0);
      return kDone;
    }
    return kFallback;
  }
  const uint64_t seed = P.seed_arr ? P.seed_arr[i] : P.seed;
  const uint64_t offset = P.offset_arr ? P.offset_arr[i] : P.offset;
  const uint64_t sid = P.seed_arr ? 0ull : (uint64_t)i;

  // ---- phase A: one HBM read of the slice into registers --------------------
  const int V = P.vocab;
  const int s0 = s * S.L;
  const int s1 = min(s0 + S.L, V);
  const int nvec = (s1 - s0) / 4;
  const uint32_t n_s = (uint32_t)(s1 - s0);
  // The slice's bound must not exceed its own k-th largest value; a slice
  // shorter than k has none, and its bound is 0 (all of it is a candidate).
  // The row's k-th largest is at least every slice's, so the maximum of the
  // bounds keeps every value of the row's top k.
  const uint32_t need = (uint32_t)k;
  const float4* src = reinterpret_cast<const float4*>(P.probs + (int64_t)row * V + s0);
  // Loads are issued unconditionally (a lane past the end re-reads the last
  // vector and ignores it) so that they sit in one basic block and every
  // later use waits only for its own vector, not for the whole slice.
  float4 v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = src[min(tid + j * kBlock, nvec - 1)];
  // while the slice is in flight: the row's arrival generation (kept in a
  // register until the header is written), the first 256 draws of the
  // stream, and a cleared histogram
  uint32_t gen = 0u;
  if (W > 1 && tid == 0)
    gen = __hip_atomic_load(&S.gen[li], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (wave == 0) {
    const Philox4x64 ph = philox4x64_10(offset, sid, (uint64_t)lane, 0ull, seed, 0ull);
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.draws[4 * lane + e] = (double)(ph.w[e] >> 11) * 0x1p-53;
  }
  for (int q = tid; q < kHistBins; q += kBlock) sm.hist[q] = 0u;
  __syncthreads();  // histogram cleared (does not wait for the loads)

  // Provisional bound from the first vector of every thread (the first
  // 4096 values of the slice): the edge of the bin holding the r-th largest
  // sample value, r sized for about 1.5 * need + 64 values over the slice.
  {
    const uint32_t q[4] = {bits_of(v[0].x), bits_of(v[0].y), bits_of(v[0].z), bits_of(v[0].w)};
    if (tid < nvec) {
#pragma unroll
      for (int e = 0; e < 4; ++e) atomicAdd(&sm.hist[min(q[e] >> 20, (uint32_t)(kHistBins - 1))], 1u);
    }
  }
  __syncthreads();
  const uint32_t nsamp = 4u * (uint32_t)min(nvec, kBlock);
  const uint32_t r = min(nsamp, max(1u, (uint32_t)(((1.5 * min(need, n_s) + 64.0) * nsamp) / n_s) + 1u));
  uint32_t bin, above, total;
  suffix_find<kWaves>(sm.hist, kHistBins, r, bin, above, total, sm);
  const uint32_t t_prov = n_s <= need ? 0u : bin << 20;

  // As each vector lands: slice maximum, and every value >= t_prov appended
  // to this wave's LDS buffer in (vector, element, lane) order.
  uint32_t mb = 0u;
  uint32_t wcnt = 0u;  // wave-uniform
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int f = tid + j * kBlock;
    const bool in = f < nvec;
    const uint32_t q[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mb = max(mb, in ? q[e] : 0u);
      const bool sel = in && q[e] >= t_prov;
      const uint64_t m = __ballot(sel);
      if (m) {
        if (sel) {
          const uint32_t p =
              wcnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (p < (uint32_t)kWaveCap) {
            sm.a.pw.bits[wave][p] = q[e];
            sm.a.pw.idx[wave][p] = (uint32_t)(s0 + 4 * f + e);
          }
        }
        wcnt += (uint32_t)__popcll(m);
      }
    }
  }
  if (lane == 0) sm.wcnt[wave] = wcnt;
  if (tid == 0) sm.gen = gen;
  const uint32_t slice_max = block_max<kWaves>(mb, sm);  // also publishes wcnt[]
  const bool bad = slice_max >= 0x7F800000u;             // sign bit, inf or NaN somewhere
  uint32_t tot = 0u, wbase = 0u;
  bool wave_ovf = false;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) {
    const uint32_t c = sm.wcnt[q];
    wbase += q < wave ? c : 0u;
    tot += c;
    wave_ovf |= c > (uint32_t)kWaveCap;
  }
  const bool fast = !wave_ovf && (tot >= need || t_prov == 0u) && tot <= (uint32_t)kSliceCandMax;

  // local bound t_s and the published list: the appended values (fast path),
  // else a full histogram of the slice and a compaction from registers
  uint32_t t_bits, cnt;
  if (fast) {
    t_bits = t_prov;
    cnt = tot;
  } else {
    for (int q = tid; q < kHistBins; q += kBlock) sm.hist[q] = 0u;
    __syncthreads();
    // the slice is re-read (from L2) rather than kept in registers: this
    // path is taken only by flat rows, and freeing v[] keeps the common
    // path free of spills
    for (int f = tid; f < nvec; f += kBlock) {
      const float4 x = src[f];
      const uint32_t q[4] = {bits_of(x.x), bits_of(x.y), bits_of(x.z), bits_of(x.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) atomicAdd(&sm.hist[min(q[e] >> 20, (uint32_t)(kHistBins - 1))], 1u);
    }
    __syncthreads();
    suffix_find<kWaves>(sm.hist, kHistBins, need, bin, above, total, sm);
    t_bits = bin << 20;
    uint32_t mine = 0u;
    for (int f = tid; f < nvec; f += kBlock) {
      const float4 x = src[f];
      mine += (uint32_t)(bits_of(x.x) >= t_bits) + (uint32_t)(bits_of(x.y) >= t_bits) +
              (uint32_t)(bits_of(x.z) >= t_bits) + (uint32_t)(bits_of(x.w) >= t_bits);
    }
    uint32_t pos = block_excl_scan<kWaves>(mine, cnt, sm);
    if (cnt <= (uint32_t)kSliceCandMax && !bad) {  // compaction into sm.c, thread-major
      for (int f = tid; f < nvec; f += kBlock) {
        const float4 x = src[f];
        const uint32_t q[4] = {bits_of(x.x), bits_of(x.y), bits_of(x.z), bits_of(x.w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (q[e] >= t_bits) {
            sm.c.bits[pos] = q[e];
            sm.c.idx[pos] = (uint32_t)(s0 + 4 * f + e);
            ++pos;
          }
        }
      }
    }
  }
  const bool overflow = cnt > (uint32_t)kSliceCandMax;
  const bool publish = !bad && !overflow;

  uint32_t gmax;
  int n;
  if (W == 1) {
    // the whole row is in this work-group: candidates into sm.c
    if (fast && publish) {
      const uint32_t c = min(sm.wcnt[wave], (uint32_t)kWaveCap);
      for (uint32_t p = lane; p < c; p += kWave) {
        sm.c.bits[wbase + p] = sm.a.pw.bits[wave][p];
        sm.c.idx[wbase + p] = sm.a.pw.idx[wave][p];
      }
    }
    __syncthreads();
    if (bad || slice_max == 0u) {
      if (tid == 0) stream::write_sample(P, i, -1, 0);
      return kDone;
    }
    if (overflow) return kFallback;
    gmax = slice_max;
    n = (int)cnt;
    if (wave >= kTailWaves) return kDone;
  } else {
    uint64_t* dst = S.cand + ((int64_t)li * W + s) * kSliceCandMax;
    if (publish) {
      if (fast) {
        const uint32_t c = min(sm.wcnt[wave], (uint32_t)kWaveCap);
        for (uint32_t p = lane; p < c; p += kWave)
          dst[wbase + p] = (uint64_t)sm.a.pw.bits[wave][p] | ((uint64_t)sm.a.pw.idx[wave][p] << 32);
      } else {
        __syncthreads();  // compaction into sm.c complete
        for (uint32_t c = tid; c < cnt; c += kBlock)
          dst[c] = (uint64_t)sm.c.bits[c] | ((uint64_t)sm.c.idx[c] << 32);
      }
    }
    if (tid == 0) {
      uint32_t* h = S.hdr + ((int64_t)li * W + s) * kHdrWords;
      h[0] = t_bits;
      h[1] = publish ? cnt : 0xFFFFFFFFu;
      h[2] = slice_max;
      h[3] = sm.gen;
      h[4] = xcc_id();
    }
    // hand-off: this work-group's stores reach the XCD's L2 before it arrives
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(&S.ctr[li], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      sm.flag = (old == (uint32_t)(W - 1));
    }
    __syncthreads();
    if (!sm.flag) return kDone;

    // ---- phase B: the last slice work-group of the row ----------------------
    const uint32_t me = xcc_id();
    if (tid == 0) {
      __hip_atomic_store(&S.ctr[li], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&S.gen[li], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid < W * kHdrWords) {
      sm.hdr[tid / kHdrWords][tid % kHdrWords] =
          __hip_atomic_load(S.hdr + (int64_t)li * W * kHdrWords + tid, __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    bool foreign = false, ovf = false;
    uint32_t tstar = 0u, ntot = 0u;
    gmax = 0u;
    for (int q = 0; q < W; ++q) {
      foreign |= sm.hdr[q][3] != sm.gen || sm.hdr[q][4] != me;
      ovf |= sm.hdr[q][1] == 0xFFFFFFFFu;
      gmax = max(gmax, sm.hdr[q][2]);
      tstar = max(tstar, sm.hdr[q][0]);
      if (sm.hdr[q][1] != 0xFFFFFFFFu) ntot += sm.hdr[q][1];
    }
    if (!foreign && (gmax >= 0x7F800000u || gmax == 0u)) {
      if (tid == 0) stream::write_sample(P, i, -1, 0);
      return kDone;
    }
    if (foreign || ovf || ntot > (uint32_t)kRowCandMax) return kFallback;

    // gather: every thread issues its (up to 8) loads before using any, then
    // keeps the entries >= t*; order (thread, slot), which is fixed
    if (tid == 0) {
      uint32_t acc = 0u;
      for (int q = 0; q < W; ++q) {
        sm.off[q] = acc;
        acc += sm.hdr[q][1];
      }
      for (int q = W; q <= kMaxSlices; ++q) sm.off[q] = acc;
    }
    __syncthreads();
    constexpr int kPer = kRowCandMax / kBlock;
    uint64_t ent[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const uint32_t g = (uint32_t)(tid + q * kBlock);
      ent[q] = 0ull;
      if (g < ntot) {
        int sl = 0;  // slice holding entry g: sm.off is non-decreasing
#pragma unroll
        for (int step = kMaxSlices / 2; step >= 1; step >>= 1)
          if (sl + step < W && sm.off[sl + step] <= g) sl += step;
        ent[q] = __hip_atomic_load(S.cand + ((int64_t)li * W + sl) * kSliceCandMax + (g - sm.off[sl]),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    uint32_t keep = 0u;
#pragma unroll
    for (int q = 0; q < kPer; ++q)
      keep += (uint32_t)(tid + q * kBlock < (int)ntot && (uint32_t)ent[q] >= tstar);
    uint32_t nstar;
    uint32_t wpos = block_excl_scan<kWaves>(keep, nstar, sm);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if (tid + q * kBlock < (int)ntot && (uint32_t)ent[q] >= tstar) {
        sm.c.bits[wpos] = (uint32_t)ent[q];
        sm.c.idx[wpos] = (uint32_t)(ent[q] >> 32);
        ++wpos;
      }
    }
    __syncthreads();
    if (tstar > 0u && nstar < (uint32_t)k) return kFallback;  // guard: not reached
    n = (int)nstar;
    if (wave >= kTailWaves) return kDone;
  }

  // ---- tail (four waves): k-th largest, top-k mass, dual-pivot loop --------
  // The candidates are every value >= t* of the row, at least k of them (or
  // the whole row).  tau_k is found exactly; the loop then starts just below
  // it, where f(low) = 0 because at least k values exceed low.
  const uint32_t tau_k =
      ((uint32_t)k <= (uint32_t)n) ? kth_largest<kTailWaves>(sm.c.bits, n, (uint32_t)k, sm) : 0u;
  double pz = 0.0;
  if (OP == kOpTopKTopP) {
    Pair z{0.0, 0.0, 0u, 0u};
    for (int c = tid; c < n; c += kTailThreads)
      if (sm.c.bits[c] >= tau_k) z.m0 += (double)__uint_as_float(sm.c.bits[c]);
    z = block_sum<kTailWaves>(z, sm);
    pz = (double)stream::clamp01(pp) * z.m0;
  }
  const float low = tau_k > 0u ? __uint_as_float(tau_k - 1u) : 0.0f;
  int rounds = 0;
  const int e = candidate_loop<OP, kTailWaves>(sm, n, low, __uint_as_float(gmax), k, pz, seed,
                                               offset, sid, rounds);
  if (tid == 0) stream::write_sample(P, i, e, e >= 0 ? rounds : 0);
  return kDone;
}

template <int OP, int NV>
__global__ __launch_bounds__(kBlock) void split_sample_kernel(SampleParams P, SplitParams S) {
  __shared__ SplitSmem sm;
  int i = 0;
  const int mode = split_sample<OP, NV>(P, S, sm, i);
  if (mode == kFallback) stream::sample_row<OP>(P, i, sm.a.stream);
}

template <int OP, int NV>
void launch_one(const SampleParams& p, const SplitParams& sp, hipStream_t s) {
  const int groups = (sp.n_out + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * sp.W)), block(kBlock);
  hipLaunchKernelGGL((split_sample_kernel<OP, NV>), grid, block, 0, s, p, sp);
}

template <int OP>
void launch_nv(int nv, const SampleParams& p, const SplitParams& sp, hipStream_t s) {
  switch (nv) {
    case 2: launch_one<OP, 2>(p, sp, s); break;
    case 4: launch_one<OP, 4>(p, sp, s); break;
    case 6: launch_one<OP, 6>(p, sp, s); break;
    case 8: launch_one<OP, 8>(p, sp, s); break;
    case 10: launch_one<OP, 10>(p, sp, s); break;
    default: launch_one<OP, 12>(p, sp, s); break;
  }
}

constexpr int kChunk = 2048;     // outputs per launch (bounds the workspace)
constexpr int kMaxSliceLen = 12 * 4 * kBlock;

// The arrival counters and generation numbers sit at fixed offsets for the
// largest chunk, so calls of any shape can share one workspace: counters are
// zero between calls, generations only ever grow.
constexpr size_t kCtlBytes = 2 * (size_t)kChunk * 4;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

SplitPlan plan_split(int op, int rows, int vocab, int num_outputs, uint32_t flags, int vec_ok) {
  SplitPlan plan{0, 0, 0, 0, 0};
  (void)rows;
  if (op != kOpTopK && op != kOpTopKTopP) return plan;
  if (flags & (DSS_FLAG_STREAMING | DSS_FLAG_FROM_ZERO)) return plan;
  if (!vec_ok || vocab < 1024 || num_outputs <= 0) return plan;
  const int wmin = (vocab + kMaxSliceLen - 1) / kMaxSliceLen;
  const int wt = (256 + num_outputs - 1) / num_outputs;
  int W = max(wmin, min(wt, kMaxSlices));
  if (W > kMaxSlices) return plan;
  int L = 0;
  for (;; --W) {  // largest W <= chosen one whose slices are all non-empty
    L = ((vocab + 4 * W - 1) / (4 * W)) * 4;
    if (W == 1 || (int64_t)(W - 1) * L < vocab) break;
  }
  int nv = (L / 4 + kBlock - 1) / kBlock;
  nv = nv <= 2 ? 2 : nv <= 4 ? 4 : nv <= 6 ? 6 : nv <= 8 ? 8 : nv <= 10 ? 10 : 12;
  const int ch = min(num_outputs, kChunk);
  plan.W = W;
  plan.L = L;
  plan.nv = nv;
  plan.chunk = ch;
  plan.workspace = W == 1 ? 0
                          : kCtlBytes + align256((size_t)ch * W * kHdrWords * 4) +
                                (size_t)ch * W * kSliceCandMax * 8;
  return plan;
}

hipError_t launch_split_sample(int op, const SampleParams& p, const SplitPlan& plan,
                               void* workspace, hipStream_t s) {
  char* ws = static_cast<char*>(workspace);
  const size_t ch = (size_t)plan.chunk;
  SplitParams sp;
  sp.W = plan.W;
  sp.L = plan.L;
  sp.ctr = reinterpret_cast<uint32_t*>(ws);
  sp.gen = sp.ctr + kChunk;
  sp.hdr = reinterpret_cast<uint32_t*>(ws + kCtlBytes);
  sp.cand = reinterpret_cast<uint64_t*>(ws + kCtlBytes + align256(ch * plan.W * kHdrWords * 4));
  for (int out0 = 0; out0 < p.num_outputs; out0 += plan.chunk) {
    sp.out0 = out0;
    sp.n_out = min(plan.chunk, p.num_outputs - out0);
    if (op == kOpTopK) {
      launch_nv<kOpTopK>(plan.nv, p, sp, s);
    } else {
      launch_nv<kOpTopKTopP>(plan.nv, p, sp, s);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dss
