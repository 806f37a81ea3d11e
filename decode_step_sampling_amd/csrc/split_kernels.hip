// Split-row engine for top-k and top-k-then-top-p sampling.
//
// The dual-pivot rejection loop of the FlashInfer blog ("Sorting-Free GPU
// Kernels for LLM Sampling", section 双枢轴拒绝采样) only ever draws from the
// values above the current `low`, and its correctness proof (section
// 拒绝采样器正确性的理论证明) holds from any starting pivot below every kept
// value.  This engine therefore:
//
//  1. splits each row into W slices, one 1024-thread work-group per slice.
//     Waves 1..15 read the slice from HBM exactly once into registers
//     (16-byte loads, all issued up front); wave 0 clears the histogram and
//     computes the row's first 256 Philox draws while the slice is in
//     flight;
//  2. from the first landed vector of every reading thread (3840 values) the
//     slice takes a provisional bound: the edge of a 1/8-binade bin of the
//     float32 bit patterns (bits >> 20) above which about 1.5 k + 64 of the
//     slice's values should lie.  As each vector lands the reading waves
//     append the values at or above that bound, with their indices, to
//     per-wave LDS lists.  If the lists hold at least k values the bound
//     stands (it is then at most the slice's k-th largest value); otherwise
//     the slice is histogrammed in full and the exact 1/8-binade bound of
//     its k-th largest value is used.  Each slice publishes its bound and
//     its list.  The union over slices contains every value >= t* = max_s t_s
//     of the row, and at least k of them;
//  3. the last slice work-group of the row to finish (a relaxed arrival
//     counter) gathers the candidates into registers, finds the k-th largest
//     tau_k with three histogram passes over the bit fields [30:20], [19:9]
//     and [8:0] (the F4 note's threshold search on the float32 bit pattern,
//     §③, done 2048 ways per pass instead of 2 or 3), compacts the values
//     >= tau_k with their mass Z_k, and one wave runs the dual-pivot loop on
//     them from just below tau_k, where f(low) = 0 still holds.
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

constexpr int kLoadWaves = kWaves - 1;             // waves 1..15 read the slice
constexpr int kLoadThreads = kLoadWaves * kWave;   // 960
constexpr int kHistBins = 2048;
constexpr int kFineBins = 512;
constexpr int kSliceCandMax = 4096;
constexpr int kWaveCap = 448;  // per-wave append list during the read
constexpr int kRowCandMax = 8192;
constexpr int kPer = kRowCandMax / kBlock;  // gathered entries per thread
constexpr int kSplitKCap = 1536;
constexpr int kMaxSlices = 16;
constexpr int kHdrWords = 8;
constexpr uint32_t kNoList = 0xFFFFFFFFu;  // header count of a slice that published nothing

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
using H3 = Padded<kFineBins>;

struct SplitSmem {
  union {
    struct {
      uint32_t bits[kWaves][kWaveCap + kWave];  // per-wave appends during the read,
      uint32_t idx[kWaves][kWaveCap + kWave];   // then one dummy slot per lane
    } pw;
    uint64_t bnd[kRowCandMax];      // candidates in the bin of the k-th largest
    stream::SampleSmem stream;      // streaming fallback
  } a;
  uint64_t cand[kRowCandMax];       // candidates (bits | index << 32)
  alignas(16) uint32_t hist[H1::kWords];
  double draws[stream::kPreDraws];
  double red_d[kWaves];
  uint32_t red_u[kWaves];
  uint32_t wcnt[kWaves];
  uint32_t wmax[kWaves];
  uint32_t off[kMaxSlices + 1];
  uint32_t res[4];
  uint32_t fres[4];
  uint32_t tprov;  // provisional bound | 1 once set (0 until then)
  int flag;
};
static_assert(sizeof(SplitSmem) <= 160 * 1024, "LDS budget of one gfx950 work-group");
static_assert(kMaxSlices <= kWaves, "per-slice counts reuse the per-wave count slots");

__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20) & 0xFu;  // HW_REG_XCC_ID
}

// wave index as a scalar, so branches on it are scalar branches
__device__ __forceinline__ int uwave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ int first_lane(uint64_t m) { return __ffsll((long long)m) - 1; }
__device__ __forceinline__ int last_lane(uint64_t m) { return 63 - __clzll((long long)m); }

template <int NB>
__device__ __forceinline__ void clear_hist(uint32_t* h, int t, int nt) {
  uint4* h4 = reinterpret_cast<uint4*>(h);
  for (int q = t; q < Padded<NB>::kWords / 4; q += nt) h4[q] = make_uint4(0u, 0u, 0u, 0u);
}

// ---------------------------------------------------------------------------
// work-group helpers (every thread of the work-group must call; fixed
// association order, so results are deterministic)
// ---------------------------------------------------------------------------

__device__ uint32_t block_excl_scan(uint32_t v, uint32_t& total, SplitSmem& sm) {
  const int lane = lane_id(), w = uwave();
  const uint32_t incl = wave_incl_scan(v);
  if (lane == kWave - 1) sm.red_u[w] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) {
    const uint32_t t = sm.red_u[q];
    base += q < w ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

// Largest bin b of the padded histogram hist (NB bins) whose suffix count
// sum_{b' >= b} hist[b'] reaches need, the count strictly above b, and the
// total (bin 0 and total - hist[0] if the total falls short).  One wave:
// lane l sums the l-th chunk of bins from the top, a scan over the lanes
// finds the chunk, a scan over that chunk's bins finds the bin.
template <int NB>
__device__ void wave_find(const uint32_t* hist, uint32_t need, uint32_t& bin, uint32_t& above,
                          uint32_t& total) {
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
}

// The same, answered by wave 0 and handed to every thread.  The histogram
// must be complete (a barrier before the call); consecutive calls must be
// separated by a barrier.
template <int NB>
__device__ void block_find(const uint32_t* hist, uint32_t need, uint32_t& bin, uint32_t& above,
                           uint32_t& total, SplitSmem& sm) {
  if (uwave() == 0) {
    wave_find<NB>(hist, need, bin, above, total);
    if (lane_id() == 0) {
      sm.fres[0] = bin;
      sm.fres[1] = above;
      sm.fres[2] = total;
    }
  }
  __syncthreads();
  bin = sm.fres[0];
  above = sm.fres[1];
  total = sm.fres[2];
}

template <int OP>
__device__ __forceinline__ bool split_predicate(double mass_above, uint32_t count_above, int k,
                                                double pz) {
  const bool ok_k = count_above < (uint32_t)k;
  if (OP == kOpTopK) return ok_k;
  return ok_k && ((mass_above < pz) || count_above == 0u);
}

// ---------------------------------------------------------------------------
// The dual-pivot loop on one wave (no barriers).  cand[0..m) holds every
// value of the row above `low` (and nothing at or below it); their mass is
// the kept mass Z_k, and the top-p bound is pfrac * Z_k.  Lane l owns the contiguous entries [l*E, l*E + E), held in NR
// registers (NR >= E; NR = 0: read from LDS), and the inverse-transform draw runs over
// the entries in that order (blog, 逆变换采样).  Guards as in the streaming
// engine (blog, 实现细节): only entries with nonzero mass are chosen, the
// first hit wins, and if rounding puts the target at or past every running
// sum the last entry is taken.
// ---------------------------------------------------------------------------
template <int OP, int NR>
__device__ int wave_loop(const SplitSmem& sm, int m, float low, float high, int k, float pfrac,
                         uint64_t seed, uint64_t offset, uint64_t sid, int& rounds) {
  constexpr bool REG = NR > 0;
  const int lane = lane_id();
  const int E = (m + kWave - 1) / kWave;
  const int c0 = min(m, lane * E), c1 = min(m, c0 + E);
  const uint64_t* cand = sm.cand;
  float xr[REG ? NR : 1];
  if (REG) {
#pragma unroll
    for (int j = 0; j < NR; ++j) xr[j] = c0 + j < c1 ? __uint_as_float((uint32_t)cand[c0 + j]) : 0.0f;
  }
  // x of this lane's j-th entry (0.0 past the end: never above a pivot)
  auto X = [&](int j) -> float {
    if (REG) return xr[j];
    return c0 + j < c1 ? __uint_as_float((uint32_t)cand[c0 + j]) : 0.0f;
  };
  const int n = REG ? NR : E;  // entries past c1 read as 0.0

  double part = 0.0;  // mass above low of this lane's entries
#pragma unroll
  for (int j = 0; j < n; ++j) {
    const float x = X(j);
    if (x > low) part += (double)x;
  }
  double S = wave_sum(part);  // mass above low: the kept mass Z_k at the start
  const double pz = (double)pfrac * S;
  int rnd = 0;
  while (true) {
    const double u = rnd < stream::kPreDraws ? sm.draws[rnd]
                                             : draw_uniform(seed, offset, sid, (uint32_t)rnd);
    ++rnd;
    const double T = u * S;
    const double incl = wave_incl_scan(part);
    const double excl = wave_excl_from_incl(incl);
    const uint64_t hit = __ballot(part > 0.0 && incl > T);
    const uint64_t nz = __ballot(part > 0.0);
    if (nz == 0ull) {
      rounds = rnd;
      return -1;
    }
    const int owner = hit ? first_lane(hit) : last_lane(nz);
    // the owner's entries, one per lane (a serial walk if a lane owns more
    // than 64): first running sum past T, else the last entry above low
    int e = -1;
    const int o0 = min(m, owner * E), o1 = min(m, o0 + E);
    const double base = lane_value(excl, owner);
    if (o1 - o0 <= kWave) {
      const int c = o0 + lane;
      const float x = c < o1 ? __uint_as_float((uint32_t)cand[c]) : 0.0f;
      const double xm = x > low ? (double)x : 0.0;
      const double run = base + wave_incl_scan(xm);
      const uint64_t h2 = __ballot(hit != 0ull && xm > 0.0 && run > T);
      const uint64_t n2 = __ballot(xm > 0.0);
      e = o0 + (h2 ? first_lane(h2) : last_lane(n2));
    } else {
      double run = base;
      for (int c = o0; c < o1; ++c) {
        const float x = __uint_as_float((uint32_t)cand[c]);
        if (x > low) {
          run += (double)x;
          e = c;
          if (hit != 0ull && run > T) break;
        }
      }
    }
    e = min(max(e, 0), m - 1);  // part > 0 guarantees an entry; keep the read in bounds regardless
    const uint64_t ent = cand[e];
    const float pivot1 = __uint_as_float((uint32_t)ent);
    const int token = (int)(ent >> 32);
    if (OP == kOpTopK) {
      // every entry is >= tau_k, so fewer than k values exceed pivot1
      rounds = rnd;
      return token;
    }
    const float pivot2 = (float)(((double)pivot1 + (double)high) * 0.5);
    double m0 = 0.0, m1 = 0.0;
    uint32_t n0 = 0u, n1 = 0u;
#pragma unroll
    for (int j = 0; j < n; ++j) {
      const float x = X(j);
      if (x > pivot1) {
        m0 += (double)x;
        ++n0;
      }
      if (x > pivot2) {
        m1 += (double)x;
        ++n1;
      }
    }
    const double M0 = wave_sum(m0), M1 = wave_sum(m1);
    const uint32_t N0 = wave_sum(n0), N1 = wave_sum(n1);
    if (split_predicate<OP>(M0, N0, k, pz)) {
      rounds = rnd;
      return token;
    }
    if (split_predicate<OP>(M1, N1, k, pz)) {
      low = pivot1;
      high = pivot2;
      S = M0;
      part = m0;
    } else {
      low = pivot2;
      S = M1;
      part = m1;
    }
    if (rnd >= stream::kMaxRounds) {
      rounds = rnd;
      return -1;
    }
  }
}

enum SplitMode : int { kDone = 0, kFallback = 1 };

// Bounded wait for the provisional bound of wave 1.  Every wave gets out:
// after the spin limit the bound 0 is used, which appends the whole slice,
// overflows the lists and sends the slice down the full-histogram path.
__device__ __forceinline__ uint32_t wait_tprov(SplitSmem& sm) {
  for (int spin = 0; spin < (1 << 16); ++spin) {
    const uint32_t t = __hip_atomic_load(&sm.tprov, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (t & 1u) return t & ~1u;
    __builtin_amdgcn_s_sleep(1);
  }
  return 0u;
}

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

  const int row = P.indices ? as_global(P.indices)[i] : i;
  const int k = P.top_k_arr ? as_global(P.top_k_arr)[i] : P.top_k;
  const float pp =
      (OP == kOpTopKTopP) ? (P.top_p_arr ? as_global(P.top_p_arr)[i] : P.top_p) : 0.0f;
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
  const uint64_t seed = P.seed_arr ? as_global(P.seed_arr)[i] : P.seed;
  const uint64_t offset = P.offset_arr ? as_global(P.offset_arr)[i] : P.offset;
  const uint64_t sid = P.seed_arr ? 0ull : (uint64_t)i;
  if (tid == 0) sm.tprov = 0u;
  __syncthreads();  // before any load: costs little, orders the clear before the polls

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
  const gptr<const float4> src =
      as_global(reinterpret_cast<const float4*>(P.probs + (int64_t)row * V + s0));
  const bool reader = wave > 0;
  const int rt = tid - kWave;  // reader thread index
  // Loads are issued unconditionally (a lane past the end re-reads the last
  // vector and ignores it) so that they sit in one basic block and every
  // later use waits only for its own vector, not for the whole slice.
  float4 v[NV];
  if (reader) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = load_f4(src + min(rt + j * kLoadThreads, nvec - 1));
  }
  uint32_t gen = 0u;
  if (reader) {
    // Wave 1's loads go out first and land first: its values are the sample
    // for the provisional bound, the edge of the 1/8-binade bin (bits >> 20)
    // above which about 1.5 * need + 64 of the slice's values should lie.
    uint32_t t_prov;
    if (wave == 1) {
      clear_hist<kHistBins>(sm.hist, lane, kWave);
      uint32_t nsamp = 0u;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        if (rt + j * kLoadThreads < nvec) {
          const uint32_t q[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            atomicAdd(&sm.hist[H1::at(min(q[e] >> 20, (uint32_t)(kHistBins - 1)))], 1u);
        }
        nsamp += 4u * (uint32_t)__popcll(__ballot(rt + j * kLoadThreads < nvec));
      }
      const uint32_t r =
          min(nsamp, max(1u, (uint32_t)(((1.5 * min(need, n_s) + 64.0) * nsamp) / n_s) + 1u));
      uint32_t bin, above, total;
      wave_find<kHistBins>(sm.hist, r, bin, above, total);
      t_prov = n_s <= need ? 0u : bin << 20;
      if (lane == 0) __hip_atomic_store(&sm.tprov, t_prov | 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      t_prov = wait_tprov(sm);
    }

    // As each vector lands: the slice maximum (lanes past the end hold a
    // copy of a real vector, so they may join in), and every value >= t_prov
    // appended to this wave's list in (vector, element, lane) order.  Lanes
    // with nothing to append write a dummy slot of their own, so the store
    // needs no branch.  A list that could overflow with the next vector
    // stops; its count is set past the cap, which sends the slice down the
    // full-histogram path.
    uint32_t mb = 0u;
    uint32_t wcnt = 0u;  // wave-uniform
    uint32_t* lbits = sm.a.pw.bits[wave];
    uint32_t* lidx = sm.a.pw.idx[wave];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (wcnt > (uint32_t)(kWaveCap - 4 * kWave)) {
        wcnt = kWaveCap + 1;
        break;
      }
      const int f = rt + j * kLoadThreads;
      const bool in = f < nvec;
      // exec is full here, so the compare masks need no further masking
      const uint64_t in_m = __builtin_amdgcn_uicmp((uint32_t)f, (uint32_t)nvec, 36);  // <
      const uint32_t q[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
      mb = max(max(mb, q[0]), q[1]);
      mb = max(max(mb, q[2]), q[3]);
      const uint32_t idx0 = (uint32_t)(s0 + 4 * f);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t m = __builtin_amdgcn_uicmp(q[e], t_prov, 35) & in_m;  // >=
        const bool sel = in && q[e] >= t_prov;
        const uint32_t p = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const uint32_t slot = sel ? wcnt + p : (uint32_t)(kWaveCap + lane);
        lbits[slot] = q[e];
        lidx[slot] = idx0 + (uint32_t)e;
        wcnt += (uint32_t)__popcll(m);
      }
    }
    mb = wave_max(mb);
    if (lane == 0) {
      sm.wcnt[wave] = wcnt;
      sm.wmax[wave] = mb;
      if (wave == 1) sm.res[0] = t_prov;
    }
  } else {
    // wave 0: the row's arrival generation and the first 256 draws of the
    // output's stream, while the slice lands
    if (W > 1 && lane == 0)
      gen = __hip_atomic_load(as_global(S.gen + li), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const Philox4x64 ph = philox4x64_10(offset, sid, (uint64_t)lane, 0ull, seed, 0ull);
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.draws[4 * lane + e] = (double)(ph.w[e] >> 11) * 0x1p-53;
    if (lane == 0) {
      sm.wcnt[0] = 0u;
      sm.wmax[0] = 0u;
    }
  }
  __syncthreads();
  const uint32_t t_prov = sm.res[0];
  uint32_t tot = 0u, wbase = 0u, slice_max = 0u;
  bool wave_ovf = false;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) {
    const uint32_t c = sm.wcnt[q];
    wbase += q < wave ? c : 0u;
    tot += c;
    wave_ovf |= c > (uint32_t)kWaveCap;
    slice_max = max(slice_max, sm.wmax[q]);
  }
  const bool fast = !wave_ovf && (tot >= need || t_prov == 0u) && tot <= (uint32_t)kSliceCandMax;

  // The slice's bound t_bits and its list: the appended values (fast path),
  // else a full histogram of the slice and a compaction into sm.cand.  The
  // full path reads the slice again (it is in L2 now) into fresh registers,
  // every reading thread's vectors in flight at once, rather than keeping
  // v[] alive: only flat rows and rare short samples take it, and freeing
  // v[] keeps the common path free of spills.
  uint32_t t_bits, cnt;
  if (fast) {
    t_bits = t_prov;
    cnt = tot;
  } else {
    float4 w[NV];
    if (reader) {
#pragma unroll
      for (int j = 0; j < NV; ++j) w[j] = load_f4(src + min(rt + j * kLoadThreads, nvec - 1));
    }
    clear_hist<kHistBins>(sm.hist, tid, kBlock);
    __syncthreads();
    uint32_t mx = 0u;
    if (reader) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        if (rt + j * kLoadThreads < nvec) {
          const uint32_t q[4] = {bits_of(w[j].x), bits_of(w[j].y), bits_of(w[j].z), bits_of(w[j].w)};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            mx = max(mx, q[e]);
            atomicAdd(&sm.hist[H1::at(min(q[e] >> 20, (uint32_t)(kHistBins - 1)))], 1u);
          }
        }
      }
    }
    mx = wave_max(mx);
    __syncthreads();  // histogram complete; wmax free
    if (lane == 0) sm.wmax[wave] = mx;
    uint32_t bin, above, total;
    block_find<kHistBins>(sm.hist, need, bin, above, total, sm);  // its barrier publishes wmax[]
    t_bits = bin << 20;
    uint32_t mine = 0u;
    if (reader) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        if (rt + j * kLoadThreads < nvec) {
          mine += (uint32_t)(bits_of(w[j].x) >= t_bits) + (uint32_t)(bits_of(w[j].y) >= t_bits) +
                  (uint32_t)(bits_of(w[j].z) >= t_bits) + (uint32_t)(bits_of(w[j].w) >= t_bits);
        }
      }
    }
    uint32_t pos = block_excl_scan(mine, cnt, sm);
    slice_max = 0u;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) slice_max = max(slice_max, sm.wmax[q]);
    if (reader && cnt <= (uint32_t)kSliceCandMax && slice_max < 0x7F800000u) {
      // thread-major order
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int f = rt + j * kLoadThreads;
        if (f < nvec) {
          const uint32_t q[4] = {bits_of(w[j].x), bits_of(w[j].y), bits_of(w[j].z), bits_of(w[j].w)};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (q[e] >= t_bits) {
              sm.cand[pos] = (uint64_t)q[e] | ((uint64_t)(uint32_t)(s0 + 4 * f + e) << 32);
              ++pos;
            }
          }
        }
      }
    }
  }
  const bool bad = slice_max >= 0x7F800000u;  // a sign bit, an inf or a NaN somewhere
  const bool overflow = cnt > (uint32_t)kSliceCandMax;
  const bool publish = !bad && !overflow;

  uint32_t gmax, tstar;
  uint64_t ent[kPer];  // thread t's candidates
  uint32_t live = 0u;  // bit q: ent[q] is a candidate >= t*
  if (W == 1) {
    // the whole row is in this work-group: candidates via sm.cand
    if (fast && publish && wave > 0) {
      const uint32_t c = sm.wcnt[wave];
      for (uint32_t p = lane; p < c; p += kWave)
        sm.cand[wbase + p] = (uint64_t)sm.a.pw.bits[wave][p] | ((uint64_t)sm.a.pw.idx[wave][p] << 32);
    }
    __syncthreads();
    if (bad || slice_max == 0u) {
      if (tid == 0) stream::write_sample(P, i, -1, 0);
      return kDone;
    }
    if (overflow) return kFallback;
    gmax = slice_max;
    tstar = t_bits;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const uint32_t g = (uint32_t)(tid + q * kBlock);
      ent[q] = g < cnt ? sm.cand[g] : 0ull;
      if (g < cnt) live |= 1u << q;
    }
    __syncthreads();  // sm.cand is read (it is rewritten below)
    clear_hist<kHistBins>(sm.hist, tid, kBlock);
    __syncthreads();
  } else {
    const gptr<uint64_t> dst = as_global(S.cand + ((int64_t)li * W + s) * kSliceCandMax);
    if (publish) {
      if (fast) {
        if (wave > 0) {
          const uint32_t c = sm.wcnt[wave];
          for (uint32_t p = lane; p < c; p += kWave)
            dst[wbase + p] = (uint64_t)sm.a.pw.bits[wave][p] | ((uint64_t)sm.a.pw.idx[wave][p] << 32);
        }
      } else {
        __syncthreads();  // compaction into sm.cand complete
        for (uint32_t c = tid; c < cnt; c += kBlock) dst[c] = sm.cand[c];
      }
    }
    if (tid == 0) {
      const gptr<uint32_t> h = as_global(S.hdr + ((int64_t)li * W + s) * kHdrWords);
      h[0] = t_bits;
      h[1] = publish ? cnt : kNoList;
      h[2] = slice_max;
      h[3] = gen;
      h[4] = xcc_id();
    }
    // hand-off: this work-group's stores reach the XCD's L2 before it arrives
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(as_global(S.ctr + li), 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      sm.flag = (old == (uint32_t)(W - 1));
    }
    __syncthreads();
    if (!sm.flag) return kDone;

    // ---- phase B: the last slice work-group of the row ----------------------
    // Every thread loads its slots of the slices' lists at once, without
    // waiting for the counts: slot G = t + 1024 q is position G % win of
    // slice G / win, win = 8192 / W.  Meanwhile wave 0 reads the W headers
    // (lane q: slice q) and sums them up, and every thread clears the
    // histogram.  A slot is a candidate if its position is below its
    // slice's count; a slice whose list is longer than its window sends the
    // row to an exact gather.
    const uint32_t win = (uint32_t)(kRowCandMax / W);  // <= kSliceCandMax for W >= 2
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const uint32_t G = (uint32_t)(tid + q * kBlock);
      const uint32_t sl = G / win;  // == W for the last slots when W does not divide 8192
      ent[q] = 0ull;
      if (sl < (uint32_t)W)
        ent[q] = __hip_atomic_load(
            as_global(S.cand + ((int64_t)li * W + sl) * kSliceCandMax + (G - sl * win)),
            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (wave == 0) {
      const uint32_t me = xcc_id();
      const uint32_t mygen = (uint32_t)__builtin_amdgcn_readfirstlane((int)gen);
      if (lane == 0) {
        __hip_atomic_store(as_global(S.ctr + li), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(as_global(S.gen + li), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const bool mine = lane < W;
      uint32_t ht = 0u, hc = 0u, hm = 0u, hg = mygen, hx = me;
      if (mine) {
        const gptr<uint32_t> h = as_global(S.hdr + ((int64_t)li * W + lane) * kHdrWords);
        ht = __hip_atomic_load(h + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hc = __hip_atomic_load(h + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hm = __hip_atomic_load(h + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hg = __hip_atomic_load(h + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hx = __hip_atomic_load(h + 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const bool foreign = __ballot(mine && (hg != mygen || hx != me)) != 0ull;
      const bool ovf = __ballot(mine && hc > (uint32_t)kSliceCandMax) != 0ull;  // kNoList too
      const bool spill = __ballot(mine && hc <= (uint32_t)kSliceCandMax && hc > win) != 0ull;
      const uint32_t cc = (mine && hc <= (uint32_t)kSliceCandMax) ? hc : 0u;
      const uint32_t incl = wave_incl_scan(cc);
      const uint32_t all = lane63(incl);
      const uint32_t gm = wave_max(hm);
      const uint32_t ts = wave_max(ht);
      if (lane <= kMaxSlices) sm.off[lane] = lane < W ? incl - cc : all;
      if (lane < kMaxSlices) sm.wcnt[lane] = cc;  // per-slice counts (0 past W)
      if (lane == 0) {
        uint32_t status = 0u;  // 0: go on, 1: invalid row, 2: fall back, 3: exact gather
        if (foreign) status = 2u;
        else if (gm >= 0x7F800000u || gm == 0u) status = 1u;
        else if (ovf || all > (uint32_t)kRowCandMax) status = 2u;
        else if (spill) status = 3u;
        sm.res[0] = ts;
        sm.res[1] = all;
        sm.res[2] = gm;
        sm.res[3] = status;
      }
    }
    clear_hist<kHistBins>(sm.hist, tid, kBlock);
    __syncthreads();
    const uint32_t status = sm.res[3];
    if (status == 1u) {
      if (tid == 0) stream::write_sample(P, i, -1, 0);
      return kDone;
    }
    if (status == 2u) return kFallback;
    tstar = sm.res[0];
    gmax = sm.res[2];
    if (status == 0u) {
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const uint32_t G = (uint32_t)(tid + q * kBlock);
        const uint32_t sl = G / win;
        if (sl < (uint32_t)W && G - sl * win < sm.wcnt[sl]) live |= 1u << q;
      }
    } else {
      // exact gather: entry g of the row's concatenated lists is position
      // g - off[sl] of slice sl, the last slice with off[sl] <= g (the
      // offsets in scalar registers; every load issued before any is used)
      const uint32_t ntot = sm.res[1];
      uint32_t off[kMaxSlices];
#pragma unroll
      for (int q = 0; q < kMaxSlices; ++q)
        off[q] = (uint32_t)__builtin_amdgcn_readfirstlane((int)sm.off[q]);
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const uint32_t g = (uint32_t)(tid + q * kBlock);
        int sl = 0;
        uint32_t base = 0u;
#pragma unroll
        for (int t = 1; t < kMaxSlices; ++t) {
          if (t < W && off[t] <= g) {
            sl = t;
            base = off[t];
          }
        }
        ent[q] = 0ull;
        if (g < ntot) {
          ent[q] = __hip_atomic_load(
              as_global(S.cand + ((int64_t)li * W + sl) * kSliceCandMax + (g - base)),
              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          live |= 1u << q;
        }
      }
    }
  }
  // candidates below t* take no part (bits of valid values have bit 31
  // clear, so bits >> 20 is a bin of the 2048)
#pragma unroll
  for (int q = 0; q < kPer; ++q)
    if ((uint32_t)ent[q] < tstar) live &= ~(1u << q);

  // ---- tau_k, first pass: a histogram of bits [30:20] ------------------------
  // Most candidates sit in the few bins just above t*: the four bins from
  // t*'s are counted in 8-bit register fields and added once per wave, the
  // rest go straight to LDS.
  const uint32_t b0 = tstar >> 20;
  uint32_t packed = 0u;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    if (live & (1u << q)) {
      const uint32_t bq = ((uint32_t)ent[q] >> 20) & (kHistBins - 1);
      const uint32_t d = bq - b0;
      if (d < 4u) packed += 1u << (8u * d);
      else atomicAdd(&sm.hist[H1::at(bq)], 1u);
    }
  }
  {
    const uint32_t even = wave_sum(packed & 0x00FF00FFu);         // fields 0 and 2
    const uint32_t odd = wave_sum((packed >> 8) & 0x00FF00FFu);   // fields 1 and 3
    if (lane == 0) {
      const uint32_t c4[4] = {even & 0xFFFFu, odd & 0xFFFFu, even >> 16, odd >> 16};
#pragma unroll
      for (int d = 0; d < 4; ++d)
        if (c4[d] != 0u && b0 + d < (uint32_t)kHistBins) atomicAdd(&sm.hist[H1::at(b0 + d)], c4[d]);
    }
  }
  __syncthreads();
  uint32_t bin1, above1, nstar;
  block_find<kHistBins>(sm.hist, (uint32_t)k, bin1, above1, nstar, sm);
  if (nstar < (uint32_t)k && tstar > 0u) return kFallback;  // guard: fewer than k at or above t*
  const bool all_kept = nstar < (uint32_t)k;  // t* = 0 and k above the row's nonzero count

  // ---- the candidates above bin1 into sm.cand, those in bin1 into a side
  // list (both in (thread, slot) order, one packed scan) -----------------------
  uint32_t na = 0u, nb = 0u, ma = 0u, mb2 = 0u;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    if (live & (1u << q)) {
      const uint32_t x = (uint32_t)ent[q];
      const uint32_t bq = (x >> 20) & (kHistBins - 1);
      if (all_kept ? x > 0u : bq > bin1) {
        ma |= 1u << q;
        ++na;
      } else if (!all_kept && bq == bin1) {
        mb2 |= 1u << q;
        ++nb;
      }
    }
  }
  const uint32_t pk = na | (nb << 16);  // each field stays below 2^14
  const uint32_t pincl = wave_incl_scan(pk);
  if (lane == kWave - 1) sm.red_u[wave] = pincl;
  __syncthreads();
  uint32_t pbase = 0u, ptot = 0u;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) {
    const uint32_t t = sm.red_u[q];
    pbase += q < wave ? t : 0u;
    ptot += t;
  }
  uint32_t pa = (pbase + pincl - pk) & 0xFFFFu, pb = (pbase + pincl - pk) >> 16;
  uint64_t* bnd = sm.a.bnd;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    if (ma & (1u << q)) sm.cand[pa++] = ent[q];
    if (mb2 & (1u << q)) bnd[pb++] = ent[q];
  }
  __syncthreads();
  if (wave != 0) return kDone;

  // ---- wave 0 from here on: tau_k inside bin1, the top-k list, the loop -----
  uint32_t m = ptot & 0xFFFFu;
  uint32_t tau_k = 0u;
  if (!all_kept) {
    const uint32_t nbt = ptot >> 16;
    const uint32_t need2 = (uint32_t)k - above1;  // 1 <= need2 <= nbt
    // bits [19:9] then [8:0] of the boundary entries, in sm.hist (one wave:
    // its LDS operations are ordered, no barrier needed)
    uint32_t bin2, above2, t2, bin3, above3, t3;
    clear_hist<kHistBins>(sm.hist, lane, kWave);
    for (uint32_t c = lane; c < nbt; c += kWave)
      atomicAdd(&sm.hist[H1::at(((uint32_t)bnd[c] >> 9) & (kHistBins - 1))], 1u);
    wave_find<kHistBins>(sm.hist, need2, bin2, above2, t2);
    const uint32_t hi = (bin1 << 11) | bin2;
    clear_hist<kFineBins>(sm.hist, lane, kWave);
    for (uint32_t c = lane; c < nbt; c += kWave) {
      const uint32_t x = (uint32_t)bnd[c];
      if ((x >> 9) == hi) atomicAdd(&sm.hist[H3::at(x & (kFineBins - 1))], 1u);
    }
    wave_find<kFineBins>(sm.hist, need2 - above2, bin3, above3, t3);
    tau_k = (hi << 9) | bin3;
    // the boundary entries >= tau_k follow the others, in list order
    for (uint32_t c0 = 0; c0 < nbt; c0 += kWave) {
      const uint32_t c = c0 + lane;
      const uint64_t en = c < nbt ? bnd[c] : 0ull;
      const bool take = c < nbt && (uint32_t)en >= tau_k && (uint32_t)en > 0u;
      const uint64_t tm = __builtin_amdgcn_ballot_w64(take);
      const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(tm >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)tm, 0u));
      if (take) sm.cand[m + pos] = en;
      m += (uint32_t)__popcll(tm);
    }
  }

  // ---- the dual-pivot loop on wave 0 ----------------------------------------
  const float pfrac = OP == kOpTopKTopP ? stream::clamp01(pp) : 0.0f;
  const float low = tau_k > 0u ? __uint_as_float(tau_k - 1u) : 0.0f;
  int rounds = 0;
  const float high = __uint_as_float(gmax);
  int e;
  if (m <= 4 * kWave) {
    e = wave_loop<OP, 4>(sm, (int)m, low, high, k, pfrac, seed, offset, sid, rounds);
  } else if (m <= 8 * kWave) {
    e = wave_loop<OP, 8>(sm, (int)m, low, high, k, pfrac, seed, offset, sid, rounds);
  } else if (m <= 16 * kWave) {
    e = wave_loop<OP, 16>(sm, (int)m, low, high, k, pfrac, seed, offset, sid, rounds);
  } else {  // (32 entries per lane in registers would spill the kernel)
    e = wave_loop<OP, 0>(sm, (int)m, low, high, k, pfrac, seed, offset, sid, rounds);
  }
  if (lane == 0) stream::write_sample(P, i, e, e >= 0 ? rounds : 0);
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
    default: launch_one<OP, 10>(p, sp, s); break;
  }
}

constexpr int kChunk = 2048;     // outputs per launch (bounds the workspace)
constexpr int kMaxNv = 10;  // vectors per reading thread (12 spills the kernel)
constexpr int kMaxSliceLen = kMaxNv * 4 * kLoadThreads;

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
  int nv = (L / 4 + kLoadThreads - 1) / kLoadThreads;
  nv = nv <= 2 ? 2 : nv <= 4 ? 4 : nv <= 6 ? 6 : nv <= 8 ? 8 : 10;
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
