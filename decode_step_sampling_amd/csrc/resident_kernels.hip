// Resident-slice engine: plain, top-p, min-p, top-k and top-k-then-top-p
// sampling, top-p renormalisation.
//
// Top-p needs the row's total mass before any value can be classified, so a
// slice cannot bound its candidates alone the way the split engine does for
// top-k.  Here the W work-groups of a row keep their slices in registers for
// the whole kernel and meet at row barriers (a counter in the XCD's L2 and a
// bounded spin), so the row is read from HBM exactly once:
//
//  1. As each 16-byte vector lands, its values go into an LDS mass histogram
//     on the top ten bits of the float32 pattern (F4 note §③: for x >= 0 the
//     bits order like the values).  Every bin holds one binade quarter, so
//     the bin's mass is an exact integer sum of 24-bit significands times one
//     power of two: sums are exact and their order does not matter.
//  2. The slices add their histograms into the row's (global atomics, integer
//     adds), meet, and every work-group finds the same bin where the mass
//     from the top crosses p * Z (the F4 note's threshold search on the bit
//     pattern, section ⑤, with 1023 pivots per pass instead of two).  Two
//     more levels (the next eleven bits, then the last ten) pin the exact
//     threshold tau = the largest pattern t with mass(bits >= t) >= p * Z.
//  3. Renormalisation writes x / Z_kept or 0 straight from the registers.
//     Sampling publishes the kept mass of every wave's values; the wave whose
//     range holds u * Z_kept walks its values (blog, 逆变换采样: the first
//     value whose inclusive prefix exceeds the target).  This is the
//     dual-pivot loop of the blog's 双枢轴拒绝采样 section started at
//     low = the largest value below tau: every draw is then a value >= tau,
//     which f accepts, so it ends after one round.
//
// Plain sampling uses tau = the smallest positive pattern and min-p the
// smallest float >= min_p * max (blog, min-p section), both known without a
// histogram.  Top-k runs the same three levels on counts (tau_k = the k-th
// largest pattern, ties kept) and top-k-then-top-p then the mass levels on
// the values >= tau_k only, so the top-p target is p * Z_k; with a scalar k
// up to 8192 both thresholds come from one search whose histograms carry
// (count, mass) pairs (res_search_kp).  Every wave owns a contiguous range
// of its slice, so the walk visits values in index order: the draw is the
// inverse transform of the kept set.
//
// Work-group b runs on XCD b % 8, so the W work-groups of output li are the
// blocks with equal b % 8 (as in the split engine), and the row's counters
// live in that XCD's L2.  Every launch holds at most as many work-groups as
// the device keeps resident at once, so no work-group waits on one that
// cannot start; a spin that still runs out of time marks the output invalid
// instead of hanging.  It also marks the slot's arrival counter broken (its
// top bit, set by a compare-and-swap that fails if the barrier completes
// meanwhile): every later arrival at that counter, in this launch or any
// later one, fails at once, so a dirty slot is never counted as clean.  The
// mark stays until the caller zeroes the workspace (dss_workspace_status
// reports it).
#include "stream_device.h"

// Phase clock stamps of the resident sampling kernel, as in split_kernels.hip
// (compiled in only with -DDSS_PHASE_STAMPS; dss_debug_set_stamps_resident).
#ifdef DSS_PHASE_STAMPS
__device__ unsigned long long* g_dss_stamps_res;
extern "C" __attribute__((visibility("default"))) int dss_debug_set_stamps_resident(void* p) {
  return hipMemcpyToSymbol(HIP_SYMBOL(g_dss_stamps_res), &p, sizeof(p)) == hipSuccess ? 0 : -4;
}
#define DSS_RSTAMP(n)                                                              \
  do {                                                                             \
    if (threadIdx.x == 0 && g_dss_stamps_res)                                      \
      g_dss_stamps_res[blockIdx.x * 32 + (n)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define DSS_RSTAMP(n) \
  do {                \
  } while (0)
#endif

namespace dss {
namespace {

constexpr int kRMaxW = 16;
// The resident kernel's own op id for top-k then top-p by the one search on
// (count, mass) pairs; calls with a scalar k up to kResidentSegKeys take it.
constexpr int kOpResPairs = 16;
constexpr int kRMaxNv = 12;  // 16-byte loads per thread (48 values; more run out of registers)
constexpr int kRWideNv = 16;  // plain, top-p and min-p sampling: 64 values per thread
constexpr int kRB1 = 1024;   // level 1: bits [30:21]
constexpr int kRB2 = 2048;   // level 2: bits [20:10]
constexpr int kRB3 = 1024;   // level 3: bits [9:0]
constexpr int kRHistWords = 8192;  // LDS histogram words: bins x copies
constexpr uint32_t kBroken = 0x80000000u;    // arrival-counter mark of a barrier given up

// Per-output control block in the workspace, zero between calls.
struct RowSlot {
  uint32_t ctl[64];  // 0 barrier arrivals, 1 XCC ids (bit mask), 2 maximum pattern, 3 bad value
  uint64_t h1[kRB1];  // mass histograms (integer significand sums) of the three levels
  uint64_t h2[kRB2];
  uint64_t h3[kRB3];
  uint64_t k1[kRB1];  // count histograms of the three levels (top-k)
  uint64_t k2[kRB2];
  uint64_t k3[kRB3];
  double chunk[kRMaxW * kWaves];  // kept mass of every (slice, wave) range
};
constexpr int kRLevelWords = kRB1 + kRB2 + kRB3;  // one set of three histograms

struct ResidentParams {
  int W;      // slices per output (a power of two)
  int L;      // slice length in values (multiple of 4)
  int out0;   // first output of this launch
  int n_out;  // outputs of this launch
  RowSlot* slots;
  uint32_t* lists;  // [n_out * W][kResidentSegKeys] boundary-bin keys per work-group
  uint64_t spin;    // ticks of the 100 MHz constant clock a row barrier waits at most
};

enum ResKind : int { kResSample = 0, kResRenorm = 1 };

struct ResSmem {
  alignas(16) uint64_t hh[kRHistWords];  // histogram copies (lanes spread over copies)
  uint64_t sink[kWave];                  // per-lane target of adds outside a histogram
  double md[kRB2];                       // bin masses of the level being searched
  uint32_t wmax[kWaves];
  uint32_t wbad[kWaves];
  uint32_t wsc[kWaves];           // per-wave totals of a block scan
  uint32_t off[kRMaxW + 1];       // list offsets of the slices
  uint32_t res[4];
  double resd[4];
  double wsd[kWaves];  // per-wave sums of a bin search
  double wsd2[kWaves];
  double fab, ftot, fab2;  // a bin search's result: sums above the bin, total
  uint32_t fbin;
  uint32_t lcnt;  // keys this work-group has put into its list segment
  uint32_t bcnt;  // keys of one bin gathered from the list into bkeys
  double udraw;   // the output's uniform draw
  uint32_t bkeys[kWave];
  int flag;
  // top-k then top-p in one search: masses of the level being searched, and
  // those of levels one and two kept for the top-p cut
  double mm[kRB2];
  double m1[kRB1];
  double m2[kRB2];
};
static_assert(sizeof(ResSmem) <= 136 * 1024, "LDS of the resident kernel");

__device__ __forceinline__ int r_uwave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ uint32_t r_xcc_id() {
  return __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20) & 0xFu;  // HW_REG_XCC_ID
}

// threadIdx.x, opaque to the compiler: per-thread LDS addresses derived from
// it are then formed where they are used instead of being kept in registers
// through the whole kernel.
__device__ __forceinline__ int fresh_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// A work-group-uniform value held in scalar registers.
__device__ __forceinline__ uint32_t r_uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ double r_uniform(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ int r_first_lane(uint64_t m) { return __ffsll((long long)m) - 1; }
__device__ __forceinline__ int r_last_lane(uint64_t m) { return 63 - __clzll((long long)m); }

// 24-bit significand of a non-negative float32 pattern (hidden bit for
// normal numbers); value = sig * 2^(max(exponent, 1) - 150)
__device__ __forceinline__ uint32_t sig_of(uint32_t key) {
  return (key & 0x7FFFFFu) | (key >= 0x800000u ? 0x800000u : 0u);
}
__device__ __forceinline__ double bin_mass(uint64_t s, uint32_t exponent) {
  return ldexp((double)s, (int)max(exponent, 1u) - 150);
}

__device__ __forceinline__ uint32_t max4(const float4& x) {
  return max(max(bits_of(x.x), bits_of(x.y)), max(bits_of(x.z), bits_of(x.w)));
}

// Arrive at the row barrier and wait until `target` arrivals are counted.
// Every thread must call; each thread's earlier global stores and atomics are
// complete (vmcnt 0) before thread 0 arrives.  False if the counter is
// broken, or if the wait runs past `spin` ticks: the waiter then breaks the
// counter itself, with a compare-and-swap on the count it last saw, so that
// either the barrier completed first (the swap fails and the new count
// passes) or every work-group that arrives later fails too.  Arrivals only
// raise the count, so a barrier that was reached can no longer be broken.
__device__ __forceinline__ bool row_barrier(gptr<uint32_t> ctr, uint32_t target, uint64_t spin,
                                            ResSmem& sm) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0 && spin == 0ull) {
    // a limit of zero (a test setting) gives up on arrival: the counter is
    // marked broken without being counted
    __hip_atomic_fetch_or(ctr, kBroken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.flag = 0;
  } else if (threadIdx.x == 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    uint32_t c = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    int ok = 0;
    while (true) {
      if (c & kBroken) break;
      if (c >= target) {
        ok = 1;
        break;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 >= spin) {
        uint32_t seen = c;
        __hip_atomic_compare_exchange_strong(ctr, &seen, c | kBroken, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (seen == c) break;  // broken by this work-group
        c = seen;              // the count moved: examine it again
        continue;
      }
      __builtin_amdgcn_s_sleep(1);
      c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    sm.flag = ok;
  }
  __syncthreads();
  return sm.flag != 0;
}

// Leave the row after the last read of its slot.  The work-group that
// leaves last (all W have passed `passed` barriers and then left) clears what
// the row used (hist_words words of the histograms from word hist_first of
// h1 on) and finally the arrival counter, so the slot is zero for the next
// launch.  Every thread must call.
__device__ __forceinline__ void row_leave(gptr<RowSlot> slot, uint32_t passed, int W, int hist_words, ResSmem& sm,
                                          int hist_first = 0) {
  __syncthreads();
  const gptr<uint32_t> ctr = (gptr<uint32_t>)slot->ctl;
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.flag = old == passed * (uint32_t)W + (uint32_t)W - 1u;
  }
  __syncthreads();
  if (!sm.flag) return;
  const int t = threadIdx.x;
  const gptr<uint64_t> h = (gptr<uint64_t>)slot->h1 + hist_first;  // h1 .. k3 are contiguous
  for (int q = t; q < hist_words; q += kBlock) h[q] = 0ull;
  if (t < kRMaxW * kWaves) ((gptr<double>)slot->chunk)[t] = 0.0;
  if (t >= 1 && t < 64) ctr[t] = 0u;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (t == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum the LDS histogram copies of every bin and add the non-zero sums into
// the row's global histogram g (NB bins, kRHistWords / NB copies per bin).
template <int NB, bool OPAQUE = false>
__device__ __forceinline__ void publish_hist(const ResSmem& sm, gptr<uint64_t> g) {
  constexpr int C = kRHistWords / NB;
  for (int b = OPAQUE ? fresh_tid() : (int)threadIdx.x; b < NB; b += kBlock) {
    uint64_t s = 0ull;
#pragma unroll
    for (int c = 0; c < C; ++c) s += sm.hh[b * C + c];
    if (s != 0ull) __hip_atomic_fetch_add(g + b, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// (OPAQUE: the thread index through fresh_tid, for the kernels that would
// otherwise keep the derived addresses in registers throughout)
template <bool OPAQUE = false>
__device__ __forceinline__ void clear_lds_hist(ResSmem& sm) {
  uint4* h4 = reinterpret_cast<uint4*>(sm.hh);
  for (int q = OPAQUE ? fresh_tid() : (int)threadIdx.x; q < kRHistWords / 2; q += kBlock)
    h4[q] = make_uint4(0u, 0u, 0u, 0u);
}

// Adds into the LDS histogram copies (C words per bin, copy lane % C) that
// merge a thread's consecutive values landing in one bin into a single add:
// rows with huge tie groups or a narrow value range send most of their values
// to a few bins, where the adds of a work-group would otherwise queue on a few
// LDS words.  Integer adds, so the merged sums are the same.  Values outside
// the histogram (`on` false) form runs of their own that go to the lane's
// sink word, so each value costs one compare-and-select and the only branch
// is around the add that ends a run (per-value branches on the exec mask
// would keep the work-group's one scalar unit busy instead).
constexpr uint32_t kNoBin = 0xFFFFFFFFu;
template <int C>
struct HistRun {
  uint32_t bin = kNoBin;
  unsigned long long acc = 0ull;
  __device__ __forceinline__ void flush(ResSmem& sm) {
    const uint32_t lane = (uint32_t)lane_id();
    uint64_t* const w =
        bin != kNoBin ? &sm.hh[bin * (uint32_t)C + (lane & (uint32_t)(C - 1))] : &sm.sink[lane];
    atomicAdd(reinterpret_cast<unsigned long long*>(w), acc);
  }
  __device__ __forceinline__ void put(ResSmem& sm, bool on, uint32_t b, unsigned long long add) {
    const uint32_t bb = on ? b : kNoBin;
    const bool chg = bb != bin;
    if (chg) flush(sm);
    acc = (chg ? 0ull : acc) + add;
    bin = bb;
  }
};

// The bin of sm.md (NB bins) where the mass from the top first reaches
// `need` (pfrac >= 0: need = pfrac * total): the first bin from the top whose
// inclusive suffix sum is >= need and > 0, or, when rounding or need > total
// leaves no such bin, the lowest non-zero bin (bin NB - 1 if all are zero).
// `above` is the sum of the bins above it (TWO: `above2` the same sum over
// sm.mm).  All sixteen waves take part: each sums NB / 16 bins (one or two
// per lane), one wave scan over the wave sums finds the crossing wave, and
// that wave finds the bin.  Every thread calls and gets the result.
template <int NB, bool TWO = false>
__device__ __forceinline__ void res_find(ResSmem& sm, double need, double pfrac, uint32_t& bin,
                                         double& above, double& total, double* above2 = nullptr) {
  constexpr int PW = NB / kWaves, PL = PW / kWave;  // bins per wave, per lane
  static_assert(PL == 1 || PL == 2, "one or two bins per lane");
  const int lane = lane_id(), w = r_uwave();
  double m[PL], n[PL];
  double s = 0.0, s2 = 0.0;
#pragma unroll
  for (int q = 0; q < PL; ++q) {
    const int b = NB - 1 - (w * PW + lane * PL + q);
    m[q] = sm.md[b];
    s += m[q];
    if (TWO) {
      n[q] = sm.mm[b];
      s2 += n[q];
    }
  }
  const double incl = wave_incl_scan(s);
  const double incl2 = TWO ? wave_incl_scan(s2) : 0.0;
  if (lane == kWave - 1) {
    sm.wsd[w] = incl;
    if (TWO) sm.wsd2[w] = incl2;
  }
  __syncthreads();
  const double t = lane < kWaves ? sm.wsd[lane] : 0.0;
  const double tincl = wave_incl_scan(t);
  const double tincl2 = TWO ? wave_incl_scan(lane < kWaves ? sm.wsd2[lane] : 0.0) : 0.0;
  const double tot = lane63(tincl);
  if (pfrac >= 0.0) need = pfrac * tot;
  const uint64_t hit = __ballot(lane < kWaves && tincl >= need && tincl > 0.0);
  const bool fb = hit == 0ull;
  const int wc = fb ? r_last_lane(__ballot(lane < kWaves && t > 0.0) | 1ull) : r_first_lane(hit);
  if (w == wc) {
    const double exw = wc == 0 ? 0.0 : lane_value(tincl, wc - 1);
    const double in2 = incl + exw;
    uint64_t h2 = fb ? 0ull : __ballot(in2 >= need && in2 > 0.0);
    const bool lfb = h2 == 0ull;
    if (lfb) h2 = 1ull << r_last_lane(__ballot(s > 0.0) | 1ull);
    const int L = r_first_lane(h2);
    const double ex2 = L == 0 ? exw : lane_value(in2, L - 1);
    double ex3 = 0.0;
    if (TWO) {
      const double exw2 = wc == 0 ? 0.0 : lane_value(tincl2, wc - 1);
      const double in3 = incl2 + exw2;
      ex3 = L == 0 ? exw2 : lane_value(in3, L - 1);
    }
    if (lane == L) {
      int q = 0;
      double ab = ex2, ab2 = ex3;
      if (PL == 2) {
        const bool c0 = !lfb && ex2 + m[0] >= need && ex2 + m[0] > 0.0;
        if (!c0 && (lfb ? m[PL - 1] > 0.0 : true)) {
          q = 1;
          ab = ex2 + m[0];
          if (TWO) ab2 = ex3 + n[0];
        }
      }
      sm.fbin = (uint32_t)(NB - 1 - (w * PW + L * PL + q));
      sm.fab = ab;
      sm.ftot = tot;
      if (TWO) sm.fab2 = ab2;
    }
  }
  __syncthreads();
  bin = r_uniform(sm.fbin);
  above = r_uniform(sm.fab);
  total = r_uniform(sm.ftot);
  if (TWO) *above2 = r_uniform(sm.fab2);
}

// The same search by one wave (stream::mass_find; the other waves wait at
// the barrier): cheaper where the search is not on the critical path of
// many waves' work, as in top-p alone.
template <int NB>
__device__ __forceinline__ void res_find_w0(ResSmem& sm, double need, double pfrac, uint32_t& bin,
                                            double& above, double& total) {
  if (r_uwave() == 0) {
    uint32_t b;
    double a, t;
    stream::mass_find<NB>(sm.md, need, pfrac, b, a, t);
    if (lane_id() == 0) {
      sm.fbin = b;
      sm.fab = a;
      sm.ftot = t;
    }
  }
  __syncthreads();
  bin = r_uniform(sm.fbin);
  above = r_uniform(sm.fab);
  total = r_uniform(sm.ftot);
}

// Load the row's histogram g (NB bins) as masses into sm.md; `exponent` < 0:
// level 1, bin b holds exponent b >> 2.
template <int NB>
__device__ __forceinline__ void load_masses(gptr<uint64_t> g, int exponent, ResSmem& sm) {
  for (int b = threadIdx.x; b < NB; b += kBlock) {
    const uint64_t s = __hip_atomic_load(g + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.md[b] = bin_mass(s, exponent < 0 ? (uint32_t)b >> 2 : (uint32_t)exponent);
  }
}

// The slice is loaded so that wave w owns the contiguous vector range
// [w * 64 * NV, (w + 1) * 64 * NV): its load j covers vectors
// w * 64 * NV + 64 j + lane (64 consecutive 16-byte vectors, one coalesced
// 1 KB read per instruction).  Thread position of load j: vbase + 64 j with
// vbase = w * 64 * NV + lane.  Index order inside the slice is therefore
// (wave, load, lane, element).

// An empty asm that "changes" one vector together with a loop's running
// value: the vector's arithmetic cannot start before the previous
// iteration's result exists (scheduling barriers do not hold back pure
// arithmetic), which keeps loops over the loads from converting every value
// at once and running out of registers.
template <class T>
__device__ __forceinline__ void fence_vec(float4& x, T& chain) {
  asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w), "+v"(chain));
}

// Kept mass (patterns >= tau) of this wave's values: per lane a sequential
// sum, over the lanes a wave scan.  Lane-uniform.
template <int NV>
__device__ __forceinline__ double wave_mass(float4 (&v)[NV], int vbase, int nvec, uint32_t tau) {
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    fence_vec(v[j], acc);  // one load at a time (register pressure)
    const bool in = vbase + j * kWave < nvec;
    const float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += (in && bits_of(x[e]) >= tau) ? (double)x[e] : 0.0;
  }
  return lane63(wave_incl_scan(acc));
}

// The (load j, lane l) group of four values the owner wave's walk stopped
// at; j = -1 if the wave holds no kept mass.  Wave-uniform.
struct WalkPick {
  int j;
  int l;
};

// Inverse transform over the wave's kept values in index order (load j,
// lane, element).  The lane sums of every load go to LDS at j * 64 + lane
// (index order); lane l then takes the NV consecutive entries
// [l * NV, (l + 1) * NV), so one wave scan of the lanes' totals finds the
// lane whose entries cross T, and that lane walks its entries.  Sets pk to
// the crossing entry's (load, lane) and returns the target left inside that
// entry (or a target past its mass when rounding leaves no crossing, so
// that its last kept value is taken).  lds: NV * 64 doubles used by this
// wave alone.
template <int NV>
__device__ __forceinline__ double wave_walk(float4 (&v)[NV], int vbase, int nvec, uint32_t tau,
                                            double T, double* lds, WalkPick& pk) {
  const int lane = lane_id();
  double chain = 0.0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    fence_vec(v[j], chain);  // one load at a time (register pressure)
    const bool in = vbase + j * kWave < nvec;
    const float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) s += (in && bits_of(x[e]) >= tau) ? (double)x[e] : 0.0;
    lds[j * kWave + lane] = s;
    chain = s;
  }
  __builtin_amdgcn_wave_barrier();
  double q[NV];
  double t = 0.0;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    q[k] = lds[lane * NV + k];
    t += q[k];
  }
  const double incl = wave_incl_scan(t);
  const uint64_t hit = __ballot(t > 0.0 && incl > T);
  const uint64_t nz = __ballot(t > 0.0);
  pk = WalkPick{-1, -1};
  if (nz == 0ull) return 0.0;
  const int L = hit ? r_first_lane(hit) : r_last_lane(nz);
  // lane L: its entries in order
  int ent = -1;
  double tl = 0.0;
  if (lane == L) {
    double run = incl - t;
    int lastk = -1;
    double mlast = 0.0;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const double before = run;
      run += q[k];
      const bool pos = q[k] > 0.0;
      lastk = pos ? k : lastk;
      mlast = pos ? q[k] : mlast;
      if (hit && ent < 0 && pos && run > T) {
        ent = k;
        tl = T - before;
      }
    }
    if (ent < 0) {
      ent = lastk;
      tl = 2.0 * mlast;
    }
    ent += L * NV;
  }
  const int e = __builtin_amdgcn_readlane(ent, L);
  pk = WalkPick{e / kWave, e % kWave};
  return lane_value(tl, L);
}

// The value the walk picked, decided by lane pk.l: the first kept value of
// its load pk.j whose prefix (from 0 inside the group) exceeds T, or its
// last kept one when none does (rounding, or the no-crossing target).  Returns the value's position in the slice in lane pk.l, -1
// elsewhere.  (Every load is examined and only load pk.j's result kept:
// selecting the vector by a run-time index would move v to scratch memory.)
template <int NV>
__device__ __forceinline__ int pick_value(float4 (&v)[NV], int vbase, uint32_t tau, double T,
                                          const WalkPick& pk) {
  if (pk.j < 0 || lane_id() != pk.l) return -1;
  int e_out = -1;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    fence_vec(v[j], e_out);
    const float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
    double acc = 0.0;
    int pick = -1, lastk = -1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool k = bits_of(x[e]) >= tau && x[e] > 0.0f;
      lastk = k ? e : lastk;
      acc += k ? (double)x[e] : 0.0;
      pick = (k && pick < 0 && acc > T) ? e : pick;
    }
    const int e = pick >= 0 ? pick : lastk;
    e_out = j == pk.j ? e : e_out;
  }
  return e_out < 0 ? -1 : 4 * (vbase + pk.j * kWave) + e_out;
}

typedef float r_v4f __attribute__((ext_vector_type(4)));

// An empty asm that "changes" the slice's registers: values the compiler
// derived from them earlier are not kept live past this point for reuse
// (with the slice itself live, such reuse runs the kernel out of registers).
template <int NV>
__device__ __forceinline__ void fence_values(float4 (&v)[NV]) {
#pragma unroll
  for (int j = 0; j < NV; ++j) asm volatile("" : "+v"(v[j].x), "+v"(v[j].y), "+v"(v[j].z), "+v"(v[j].w));
}

// Exclusive prefix of v over the work-group in thread order, and the total.
// Every thread must call.
__device__ __forceinline__ uint32_t res_block_scan(uint32_t v, uint32_t& total, ResSmem& sm) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == kWave - 1) sm.wsc[w] = incl;
  __syncthreads();
  uint32_t base = 0u, tot = 0u;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) {
    const uint32_t t = sm.wsc[q];
    base += q < w ? t : 0u;
    tot += t;
  }
  total = tot;
  __syncthreads();
  return base + incl - v;
}

// Fold the LDS histogram copies of NB bins into masses md (exponent e).
template <int NB>
__device__ __forceinline__ void fold_masses(ResSmem& sm, uint32_t exponent) {
  constexpr int C = kRHistWords / NB;
  for (int b = threadIdx.x; b < NB; b += kBlock) {
    uint64_t s = 0ull;
#pragma unroll
    for (int c = 0; c < C; ++c) s += sm.hh[b * C + c];
    sm.md[b] = bin_mass(s, exponent);
  }
}

// An invalid output: sample -1 (sampling), or the slice NaN-filled and the
// row's status set by slice 0 (renormalisation).
template <int KIND, int NV>
__device__ __forceinline__ void res_invalid(const SampleParams& P, const RenormParams& RP, int i,
                                            int row, int s, int vbase, int nvec, gptr<r_v4f> dst) {
  const int tid = threadIdx.x;
  if (KIND == kResSample) {
    if (s == 0 && tid == 0) stream::write_sample(P, i, -1, 0);
  } else {
    const float qnan = __uint_as_float(0x7FC00000u);
    r_v4f o;
    o.x = o.y = o.z = o.w = qnan;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (vbase + j * kWave < nvec) dst[vbase + j * kWave] = o;
    if (s == 0 && tid == 0 && RP.row_status) as_global(RP.row_status)[row] = 1;
  }
}

// Load a row histogram g (NB bins) into sm.md: counts as they are, or
// significand sums as masses (`exponent` < 0: level 1, bin b holds exponent
// b >> 2).
template <bool COUNT, int NB>
__device__ __forceinline__ void load_level(gptr<uint64_t> g, int exponent, ResSmem& sm) {
  for (int b = threadIdx.x; b < NB; b += kBlock) {
    const uint64_t x = __hip_atomic_load(g + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.md[b] = COUNT ? (double)x : bin_mass(x, exponent < 0 ? (uint32_t)b >> 2 : (uint32_t)exponent);
  }
}

// Fold the LDS histogram copies of NB bins into sm.md (counts, or masses of
// exponent e).
template <bool COUNT, int NB>
__device__ __forceinline__ void fold_level(ResSmem& sm, uint32_t exponent) {
  constexpr int C = kRHistWords / NB;
  for (int b = threadIdx.x; b < NB; b += kBlock) {
    uint64_t x = 0ull;
#pragma unroll
    for (int c = 0; c < C; ++c) x += sm.hh[b * C + c];
    sm.md[b] = COUNT ? (double)x : bin_mass(x, exponent);
  }
}

// One histogram entry of a value pattern: 1 (counts) or its significand.
template <bool COUNT>
__device__ __forceinline__ unsigned long long level_add(uint32_t key) {
  return COUNT ? 1ull : (unsigned long long)sig_of(key);
}

// Exact threshold on the resident slices, for top-k (COUNT: the F4 note's
// search on counts, section ⑤ with 1023 pivots per pass) and for top-p
// inside a top-k set (masses): tau = the largest pattern t with F(t) >= need,
// F(t) the count or the mass of the values x >= max(t, cut); pfrac >= 0 sets
// need = pfrac * F(cut).  kept = F(tau).  Levels: bits [30:21] as a row
// histogram, then inside the crossing bin bits [20:10] and [9:0], either as
// two more row histograms or, when that bin holds at most kResidentSegKeys
// values, from a key list that every work-group resolves alone.  Every
// thread calls; false if a row barrier timed out.
template <bool COUNT, int NV>
__device__ __forceinline__ bool res_search(float4 (&v)[NV], int vbase, int nvec, uint32_t cut,
                                           double need_in, double pfrac, gptr<uint64_t> g1,
                                           gptr<uint64_t> g2, gptr<uint64_t> g3,
                                           gptr<uint32_t> ctl, gptr<uint32_t> seg_base, int li,
                                           int s, int W, uint64_t spin, uint32_t& passed,
                                           ResSmem& sm, uint32_t& tau, double& kept) {
  const int tid = threadIdx.x, lane = lane_id(), wave = r_uwave();
#ifdef DSS_PHASE_STAMPS
  const uint32_t passed0 = passed;
#endif
  clear_lds_hist(sm);
  __syncthreads();
  {
    HistRun<8> run;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      fence_vec(v[j], run.acc);  // one load at a time (register pressure)
      const bool in = vbase + j * kWave < nvec;
      const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        run.put(sm, in && k4[e] >= cut, min(k4[e] >> 21, (uint32_t)(kRB1 - 1)), level_add<COUNT>(k4[e]));
    }
    run.flush(sm);
  }
  __syncthreads();
  publish_hist<kRB1>(sm, g1);
  __syncthreads();
  clear_lds_hist(sm);
  DSS_RSTAMP((COUNT ? 4 : 10) + 2 * (int)passed - 2 * (int)passed0);
  if (!row_barrier(ctl, (passed + 1u) * (uint32_t)W, spin, sm)) return false;
  DSS_RSTAMP((COUNT ? 5 : 11) + 2 * (int)passed - 2 * (int)passed0);
  ++passed;
  load_level<COUNT, kRB1>(g1, -1, sm);
  __syncthreads();
  uint32_t b1;
  double above1, ftot;
  res_find<kRB1>(sm, need_in, pfrac, b1, above1, ftot);
  const double need = pfrac >= 0.0 ? pfrac * ftot : need_in;
  const uint32_t e1 = b1 >> 2;
  if (!COUNT && pfrac >= 1.0) {  // every value >= cut
    tau = cut;
    kept = ftot;
    return true;
  }
  // values of the row in bin b1: the count itself, or at most the
  // significand sum / 2^23 (normal numbers)
  const bool use_list = COUNT ? sm.md[b1] <= (double)kResidentSegKeys
                              : e1 >= 1u && ldexp(sm.md[b1], 127 - (int)e1) <= (double)kResidentSegKeys;
  uint32_t pre2, b3;
  double above2, above3, m3;
  if (use_list) {
    uint32_t cnt = 0u;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const bool in = vbase + j * kWave < nvec;
      const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) cnt += (in && (k4[e] >> 21) == b1 && k4[e] >= cut) ? 1u : 0u;
    }
    uint32_t mine;
    uint32_t pos = res_block_scan(cnt, mine, sm);
    const gptr<uint32_t> seg = seg_base + (size_t)(li * W + s) * kResidentSegKeys;
    if (cnt != 0u) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const bool in = vbase + j * kWave < nvec;
        const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (in && (k4[e] >> 21) == b1 && k4[e] >= cut) seg[pos++] = k4[e];
      }
    }
    if (tid == 0) __hip_atomic_store(ctl + 8 + s, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    DSS_RSTAMP((COUNT ? 4 : 10) + 2 * (int)passed - 2 * (int)passed0);
    if (!row_barrier(ctl, (passed + 1u) * (uint32_t)W, spin, sm)) return false;
    DSS_RSTAMP((COUNT ? 5 : 11) + 2 * (int)passed - 2 * (int)passed0);
    ++passed;
    if (wave == 0) {
      const uint32_t c = lane < W ? __hip_atomic_load(ctl + 8 + lane, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                                  : 0u;
      const uint32_t incl = wave_incl_scan(c);
      if (lane <= kRMaxW) sm.off[lane] = incl - c;
    }
    __syncthreads();
    const uint32_t n = sm.off[W];
    constexpr int kPer = kResidentSegKeys / kBlock;
    constexpr uint32_t kNone = 0xFFFFFFFFu;  // above every non-negative pattern
    uint32_t kk[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const uint32_t g = (uint32_t)tid + (uint32_t)(q * kBlock);
      int sl = 0;
      for (int t = 1; t < W; ++t) sl = g >= sm.off[t] ? t : sl;
      const uint32_t at = min(g - sm.off[sl], (uint32_t)(kResidentSegKeys - 1));
      const uint32_t k = __hip_atomic_load(seg_base + (size_t)(li * W + sl) * kResidentSegKeys + at,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      kk[q] = g < n ? k : kNone;
    }
    // level 2 in LDS: bits [20:10], copy lane % 4
    {
      HistRun<4> run;
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        run.put(sm, kk[q] != kNone, (kk[q] >> 10) & (uint32_t)(kRB2 - 1), level_add<COUNT>(kk[q]));
      run.flush(sm);
    }
    __syncthreads();
    fold_level<COUNT, kRB2>(sm, e1);
    __syncthreads();
    clear_lds_hist(sm);
    {
      uint32_t b2;
      double total;
      res_find<kRB2>(sm, need - above1, -1.0, b2, above2, total);
      pre2 = (b1 << 11) | b2;
    }
    // level 3 in LDS: bits [9:0] of the keys with bits [30:10] == pre2
    {
      HistRun<8> run;
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        run.put(sm, kk[q] != kNone && (kk[q] >> 10) == pre2, kk[q] & (uint32_t)(kRB3 - 1),
                level_add<COUNT>(kk[q]));
      run.flush(sm);
    }
    __syncthreads();
    fold_level<COUNT, kRB3>(sm, e1);
    __syncthreads();
  } else {
    // level 2: values in bin b1, by bits [20:10], copy lane % 4
    {
      HistRun<4> run;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        fence_vec(v[j], run.acc);  // one load at a time (register pressure)
        const bool in = vbase + j * kWave < nvec;
        const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          run.put(sm, in && (k4[e] >> 21) == b1 && k4[e] >= cut, (k4[e] >> 10) & (uint32_t)(kRB2 - 1),
                  level_add<COUNT>(k4[e]));
      }
      run.flush(sm);
    }
    __syncthreads();
    publish_hist<kRB2>(sm, g2);
    __syncthreads();
    clear_lds_hist(sm);
    DSS_RSTAMP((COUNT ? 4 : 10) + 2 * (int)passed - 2 * (int)passed0);
    if (!row_barrier(ctl, (passed + 1u) * (uint32_t)W, spin, sm)) return false;
    DSS_RSTAMP((COUNT ? 5 : 11) + 2 * (int)passed - 2 * (int)passed0);
    ++passed;
    load_level<COUNT, kRB2>(g2, (int)e1, sm);
    __syncthreads();
    {
      uint32_t b2;
      double total;
      res_find<kRB2>(sm, need - above1, -1.0, b2, above2, total);
      pre2 = (b1 << 11) | b2;
    }
    // level 3: values with bits [30:10] == pre2, by bits [9:0], copy lane % 8
    {
      HistRun<8> run;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        fence_vec(v[j], run.acc);  // one load at a time (register pressure)
        const bool in = vbase + j * kWave < nvec;
        const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          run.put(sm, in && (k4[e] >> 10) == pre2 && k4[e] >= cut, k4[e] & (uint32_t)(kRB3 - 1),
                  level_add<COUNT>(k4[e]));
      }
      run.flush(sm);
    }
    __syncthreads();
    publish_hist<kRB3>(sm, g3);
    DSS_RSTAMP((COUNT ? 4 : 10) + 2 * (int)passed - 2 * (int)passed0);
    if (!row_barrier(ctl, (passed + 1u) * (uint32_t)W, spin, sm)) return false;
    DSS_RSTAMP((COUNT ? 5 : 11) + 2 * (int)passed - 2 * (int)passed0);
    ++passed;
    load_level<COUNT, kRB3>(g3, (int)e1, sm);
    __syncthreads();
  }
  {
    double total;
    res_find<kRB3>(sm, need - above1 - above2, -1.0, b3, above3, total);
    m3 = sm.md[b3];
  }
  __syncthreads();
  tau = (pre2 << 10) | b3;
  kept = above1 + above2 + (above3 + m3);
  return true;
}

// ---- top-k then top-p in one search ------------------------------------------
//
// Every level histogram carries (count, significand sum) pairs packed in one
// 64-bit word (count << 44 | sum: a row of fewer than 2^20 values cannot
// carry out of either field), so the count search that pins tau_k also
// yields the exact masses of every bin it visits.  Z_k is then known with
// tau_k, and the top-p cut p * Z_k (which lies at or above tau_k) is found
// from the same histograms: on the count search's own path (bins above the
// path bin whole, the path bin with its part >= tau_k, lower bins nothing),
// or, where it leaves that path, inside a bin that lies wholly above the
// top-k boundary bin.  Fewer than k values lie above that boundary, and the
// last round of the count search also puts them into a key list, so the
// cut is finished in LDS without another row barrier.  Whether the cut
// stays on the path at a level is a comparison of the mass above the path
// bin with p * Z_k; the bin searches run only where it leaves.  Three row
// barriers for both thresholds (the first one also level 1's, filled as the
// slice lands) instead of up to seven.
constexpr int kPairShift = 44;
constexpr uint64_t kSigMask = (1ull << kPairShift) - 1ull;
constexpr int kListPer = kResidentSegKeys / kBlock;  // list keys per thread after a gather

__device__ __forceinline__ unsigned long long pair_of(uint32_t key) {
  return (1ull << kPairShift) | (unsigned long long)sig_of(key);
}
// The same for a key inside a level-1 bin, whose values share one exponent:
// hb is the bin's hidden bit (0x800000, or 0 for the subnormal bins).
__device__ __forceinline__ unsigned long long pair_in(uint32_t key, uint32_t hb) {
  return (1ull << kPairShift) | (unsigned long long)((key & 0x7FFFFFu) | hb);
}

// The level masses kept for the top-p cut, chosen at compile time (a fixed
// LDS offset rather than a pointer held in registers): 0 none / sm.mm,
// 1 sm.m1, 2 sm.m2.
template <int A>
__device__ __forceinline__ double* level_array(ResSmem& sm) {
  return A == 1 ? sm.m1 : A == 2 ? sm.m2 : sm.mm;
}


// Row histogram g (NB bins of pairs) into sm.md (counts) and sm.mm (masses,
// exponent < 0: level 1, bin b holds exponent b >> 2); masses also into
// level_array<SAVE> (SAVE != 0).
template <int NB, int SAVE>
__device__ __forceinline__ void load_pairs(gptr<uint64_t> g, int exponent, ResSmem& sm) {
  for (int b = fresh_tid(); b < NB; b += kBlock) {
    const uint64_t x = __hip_atomic_load(g + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const double m = bin_mass(x & kSigMask, exponent < 0 ? (uint32_t)b >> 2 : (uint32_t)exponent);
    sm.md[b] = (double)(x >> kPairShift);
    sm.mm[b] = m;
    if (SAVE != 0) level_array<SAVE>(sm)[b] = m;
  }
}

// The same from the LDS copies; MASS: masses into sm.md only.
template <int NB, bool MASS, int SAVE>
__device__ __forceinline__ void fold_pairs(ResSmem& sm, uint32_t exponent) {
  constexpr int C = kRHistWords / NB;
  for (int b = fresh_tid(); b < NB; b += kBlock) {
    uint64_t x = 0ull;
#pragma unroll
    for (int c = 0; c < C; ++c) x += sm.hh[b * C + c];
    const double m = bin_mass(x & kSigMask, exponent);
    if (MASS) {
      sm.md[b] = m;
    } else {
      sm.md[b] = (double)(x >> kPairShift);
      sm.mm[b] = m;
      if (SAVE != 0) level_array<SAVE>(sm)[b] = m;
    }
  }
}

// sm.md = a level's masses as far as they are kept: bins above bk whole,
// bin bk `kept`, lower bins nothing.
template <int NB, int SRC>
__device__ __forceinline__ void kept_masses(uint32_t bk, double kept, ResSmem& sm) {
  for (int b = fresh_tid(); b < NB; b += kBlock)
    sm.md[b] = (uint32_t)b > bk ? level_array<SRC>(sm)[b] : (uint32_t)b == bk ? kept : 0.0;
}

// Puts `key` into this work-group's list segment when `take` (in any order):
// the lanes that take reserve their slots with one LDS add per wave.
__device__ __forceinline__ void list_put(bool take, uint32_t key, gptr<uint32_t> seg, ResSmem& sm) {
  const uint64_t m = __ballot(take);
  if (m != 0ull) {
    const int f = r_first_lane(m);
    uint32_t base = 0u;
    if (lane_id() == f) base = atomicAdd(&sm.lcnt, (uint32_t)__popcll(m));
    base = __builtin_amdgcn_readlane(base, f);
    const uint32_t pos =
        base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (take && pos < (uint32_t)kResidentSegKeys) seg[pos] = key;
  }
}

// Every work-group's list segment of the output into kk (kListPer keys per
// thread, kNoBin past the end).  Every thread calls.
__device__ __forceinline__ void read_list(uint32_t (&kk)[kListPer], gptr<uint32_t> ctl,
                                          gptr<uint32_t> seg_base, int li, int W, ResSmem& sm) {
  const int tid = threadIdx.x, lane = lane_id(), wave = r_uwave();
  if (wave == 0) {
    const uint32_t c = lane < W ? min(__hip_atomic_load(ctl + 8 + lane, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT),
                                      (uint32_t)kResidentSegKeys)
                                : 0u;
    const uint32_t incl = wave_incl_scan(c);
    if (lane <= kRMaxW) sm.off[lane] = incl - c;
  }
  __syncthreads();
  const uint32_t n = sm.off[W];
#pragma unroll
  for (int q = 0; q < kListPer; ++q) {
    const uint32_t g = (uint32_t)tid + (uint32_t)(q * kBlock);
    int sl = 0;
    for (int t = 1; t < W; ++t) sl = g >= sm.off[t] ? t : sl;
    const uint32_t at = min(g - sm.off[sl], (uint32_t)(kResidentSegKeys - 1));
    const uint32_t k = __hip_atomic_load(seg_base + (size_t)(li * W + sl) * kResidentSegKeys + at,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    kk[q] = g < n ? k : kNoBin;
  }
}

// One level over the list in LDS: the keys with key >> pshift == prefix, by
// bits [20:10] (NB = 2048) or [9:0] (NB = 1024), into sm.md / sm.mm (MASS:
// masses into sm.md).  Every thread calls.
template <int NB, bool MASS, int SAVE>
__device__ __forceinline__ void list_level(const uint32_t (&kk)[kListPer], uint32_t pshift,
                                           uint32_t prefix, uint32_t exponent, ResSmem& sm) {
  constexpr int C = kRHistWords / NB;
  constexpr uint32_t bshift = NB == kRB2 ? 10u : 0u;
  clear_lds_hist<true>(sm);
  __syncthreads();
  {
    HistRun<C> run;
#pragma unroll
    for (int q = 0; q < kListPer; ++q)
      run.put(sm, kk[q] != kNoBin && (kk[q] >> pshift) == prefix, (kk[q] >> bshift) & (uint32_t)(NB - 1),
              pair_of(kk[q]));
    run.flush(sm);
  }
  __syncthreads();
  fold_pairs<NB, MASS, SAVE>(sm, exponent);
  __syncthreads();
}

// The largest list key x with key >> pshift == prefix whose suffix mass
// (the mass of those keys >= x) is >= need, and that mass, found by one wave
// when the bin holds at most 64 of the list's keys (the keys share one
// exponent, so every such sum is exact); when none reaches need (rounding)
// the bin's smallest key.  False, with nothing found, when the bin holds no
// key or more than 64.  Every thread calls.
__device__ __forceinline__ bool bin_brute(const uint32_t (&kk)[kListPer], uint32_t pshift,
                                          uint32_t prefix, double need, ResSmem& sm, uint32_t& tau,
                                          double& mass) {
  const int lane = lane_id(), wave = r_uwave();
  if (threadIdx.x == 0) sm.bcnt = 0u;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kListPer; ++q) {
    const bool take = kk[q] != kNoBin && (kk[q] >> pshift) == prefix;
    const uint64_t m = __ballot(take);
    if (m != 0ull) {
      const int f = r_first_lane(m);
      uint32_t base = 0u;
      if (lane == f) base = atomicAdd(&sm.bcnt, (uint32_t)__popcll(m));
      base = __builtin_amdgcn_readlane(base, f);
      const uint32_t pos =
          base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (take && pos < (uint32_t)kWave) sm.bkeys[pos] = kk[q];
    }
  }
  __syncthreads();
  const uint32_t n = r_uniform(sm.bcnt);
  if (n == 0u || n > (uint32_t)kWave) return false;
  if (wave == 0) {
    const uint32_t x = (uint32_t)lane < n ? sm.bkeys[lane] : 0u;
    const double vx = (uint32_t)lane < n ? (double)__uint_as_float(x) : 0.0;
    double M = 0.0;
    for (uint32_t u = 0; u < n; ++u) {
      const uint32_t y = __builtin_amdgcn_readlane(x, (int)u);
      const double vy = lane_value(vx, (int)u);
      M += y >= x ? vy : 0.0;
    }
    const bool in = (uint32_t)lane < n;
    const bool cand = in && M >= need;
    const uint64_t hit = __ballot(cand);
    // the largest candidate, or the smallest key
    const uint32_t pickx = hit ? wave_max(cand ? x : 0u) : ~wave_max(in ? ~x : 0u);
    const int at = r_first_lane(__ballot(in && x == pickx));
    const double pm = lane_value(M, at);
    if (lane == 0) {
      sm.fbin = pickx;
      sm.fab = pm;
    }
  }
  __syncthreads();
  tau = r_uniform(sm.fbin);
  mass = r_uniform(sm.fab);
  __syncthreads();
  return true;
}

// tau = the top-p threshold inside the top-k set: with tau_k the k-th
// largest pattern (ties kept) and Z_k the mass of {x >= tau_k}, the largest
// pattern t with mass(x >= t) >= p * Z_k (p >= 1: tau_k itself); kept = the
// mass of {x >= tau}.  Same results as the count search followed by the
// mass search with cut = max(tau_k, 1).  Needs k <= kResidentSegKeys and the
// level-1 pairs of every slice in g1 (published before the first row
// barrier, with sm.lcnt zero).  Every thread calls; false if a row barrier
// timed out.
template <int NV>
__device__ __forceinline__ bool res_search_kp(float4 (&v)[NV], int vbase, int nvec, int k, float pc,
                                              gptr<uint64_t> g1, gptr<uint64_t> g2, gptr<uint64_t> g3,
                                              gptr<uint32_t> ctl, gptr<uint32_t> seg_base, int li,
                                              int s, int W, uint64_t spin, uint32_t& passed,
                                              ResSmem& sm, uint32_t& tau, double& kept) {
  const int tid = threadIdx.x;
  const gptr<uint32_t> seg = seg_base + (size_t)(li * W + s) * kResidentSegKeys;
  // level 1 (every value by bits [30:21]) went into g1 as the slice landed
  load_pairs<kRB1, 1>(g1, -1, sm);
  __syncthreads();
  uint32_t b1, b2, b3;
  double cab1, cab2, cab3, mab1, mab2, mab3, tot;
  res_find<kRB1, true>(sm, (double)k, -1.0, b1, cab1, tot, &mab1);
  const uint32_t e1 = b1 >> 2;
  const uint32_t hb1 = e1 >= 1u ? 0x800000u : 0u;  // hidden bit of bin b1's values
  // bin b1 and everything above it fit one list: gather them all now
  const bool use_list = cab1 + sm.md[b1] <= (double)kResidentSegKeys;
  uint32_t pre2;
  if (use_list) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const bool in = vbase + j * kWave < nvec;
      const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) list_put(in && (k4[e] >> 21) >= b1, k4[e], seg, sm);
    }
    __syncthreads();
    if (tid == 0) __hip_atomic_store(ctl + 8 + s, sm.lcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    DSS_RSTAMP(6);
    if (!row_barrier(ctl, (passed + 1u) * (uint32_t)W, spin, sm)) return false;
    DSS_RSTAMP(7);
    ++passed;
    uint32_t kk[kListPer];
    read_list(kk, ctl, seg_base, li, W, sm);
    list_level<kRB2, false, 2>(kk, 21u, b1, e1, sm);
    res_find<kRB2, true>(sm, (double)k - cab1, -1.0, b2, cab2, tot, &mab2);
    pre2 = (b1 << 11) | b2;
    list_level<kRB3, false, 0>(kk, 10u, pre2, e1, sm);
  } else {
    // level 2: values in bin b1 by bits [20:10]
    {
      HistRun<4> run;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        fence_vec(v[j], run.acc);  // one load at a time (register pressure)
        const bool in = vbase + j * kWave < nvec;
        const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          run.put(sm, in && (k4[e] >> 21) == b1, (k4[e] >> 10) & (uint32_t)(kRB2 - 1), pair_in(k4[e], hb1));
      }
      run.flush(sm);
    }
    __syncthreads();
    publish_hist<kRB2, true>(sm, g2);
    __syncthreads();
    clear_lds_hist<true>(sm);
    DSS_RSTAMP(6);
    if (!row_barrier(ctl, (passed + 1u) * (uint32_t)W, spin, sm)) return false;
    DSS_RSTAMP(7);
    ++passed;
    load_pairs<kRB2, 2>(g2, (int)e1, sm);
    __syncthreads();
    res_find<kRB2, true>(sm, (double)k - cab1, -1.0, b2, cab2, tot, &mab2);
    pre2 = (b1 << 11) | b2;
    // level 3: values with bits [30:10] == pre2 by bits [9:0]; the values
    // above that bin (fewer than k) into the list
    {
      HistRun<8> run;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        fence_vec(v[j], run.acc);  // one load at a time (register pressure)
        const bool in = vbase + j * kWave < nvec;
        const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          run.put(sm, in && (k4[e] >> 10) == pre2, k4[e] & (uint32_t)(kRB3 - 1), pair_in(k4[e], hb1));
        // one vote per vector: listed values are few
        if (__ballot(in && (max(max(k4[0], k4[1]), max(k4[2], k4[3])) >> 10) > pre2) != 0ull) {
#pragma unroll
          for (int e = 0; e < 4; ++e) list_put(in && (k4[e] >> 10) > pre2, k4[e], seg, sm);
        }
      }
      run.flush(sm);
    }
    __syncthreads();
    publish_hist<kRB3, true>(sm, g3);
    if (tid == 0) __hip_atomic_store(ctl + 8 + s, sm.lcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    DSS_RSTAMP(8);
    if (!row_barrier(ctl, (passed + 1u) * (uint32_t)W, spin, sm)) return false;
    DSS_RSTAMP(9);
    ++passed;
    load_pairs<kRB3, 0>(g3, (int)e1, sm);
    __syncthreads();
  }
  res_find<kRB3, true>(sm, (double)k - cab1 - cab2, -1.0, b3, cab3, tot, &mab3);
  const uint32_t tk = max((pre2 << 10) | b3, 1u);  // zeros carry no mass
  const double m3 = mab3 + sm.mm[b3];              // kept part of bin pre2
  const double zk = mab1 + (mab2 + m3);
  if (pc >= 1.0f) {
    __syncthreads();
    tau = tk;
    kept = zk;
    return true;
  }
  // ---- the top-p cut p * Z_k, from the top ----------------------------------
  const double need = (double)pc * zk;
  double ap1, ap2, ap3, t;
  uint32_t p1, p2, p3;
  // on the path at a level when the mass above the path bin stays below the
  // target (a comparison; the bin search runs only otherwise)
  if (mab1 < need) {
    p1 = b1;
    ap1 = mab1;
  } else {
    kept_masses<kRB1, 1>(b1, mab2 + m3, sm);
    __syncthreads();
    res_find<kRB1>(sm, need, -1.0, p1, ap1, t);
  }
  if (p1 == b1) {
    if (ap1 + mab2 < need) {
      p2 = b2;
      ap2 = mab2;
    } else {
      kept_masses<kRB2, 2>(b2, m3, sm);
      __syncthreads();
      res_find<kRB2>(sm, need - ap1, -1.0, p2, ap2, t);
    }
    if (p2 == b2) {
      kept_masses<kRB3, 0>(b3, sm.mm[b3], sm);
      __syncthreads();
    } else {  // inside L2 bin p2 > b2: every value there is in the list
      uint32_t kk[kListPer];
      read_list(kk, ctl, seg_base, li, W, sm);
      uint32_t x;
      double mx;
      if (bin_brute(kk, 10u, (b1 << 11) | p2, need - ap1 - ap2, sm, x, mx)) {
        tau = max(x, tk);
        kept = ap1 + ap2 + mx;
        return true;
      }
      list_level<kRB3, true, 0>(kk, 10u, (b1 << 11) | p2, e1, sm);
    }
  } else {  // inside L1 bin p1 > b1: every value there is in the list
    uint32_t kk[kListPer];
    read_list(kk, ctl, seg_base, li, W, sm);
    uint32_t x;
    double mx;
    if (bin_brute(kk, 21u, p1, need - ap1, sm, x, mx)) {
      tau = max(x, tk);
      kept = ap1 + mx;
      return true;
    }
    list_level<kRB2, true, 0>(kk, 21u, p1, p1 >> 2, sm);
    res_find<kRB2>(sm, need - ap1, -1.0, p2, ap2, t);
    list_level<kRB3, true, 0>(kk, 10u, (p1 << 11) | p2, p1 >> 2, sm);
  }
  res_find<kRB3>(sm, need - ap1 - ap2, -1.0, p3, ap3, t);
  tau = max((((p1 << 11) | p2) << 10) | p3, tk);
  kept = ap1 + ap2 + (ap3 + sm.md[p3]);
  __syncthreads();
  return true;
}

template <int KIND, int OP, int NV>
__global__ __launch_bounds__(kBlock) void resident_kernel(SampleParams P, RenormParams RP,
                                                          ResidentParams R) {
  __shared__ ResSmem sm;
  DSS_RSTAMP(0);
  constexpr bool kTopP = OP == kOpTopP;  // top-p alone: level-1 masses while the slice lands
  constexpr bool kPairs = OP == kOpResPairs;  // top-k then top-p, one search on pairs
  constexpr bool kTopK = OP == kOpTopK || OP == kOpTopKTopP || kPairs;
  // histogram words the row's last work-group clears (masses, then counts;
  // the pair search uses the count set only)
  constexpr int kHistWords = kPairs ? kRLevelWords : kTopK ? 2 * kRLevelWords : kTopP ? kRLevelWords : 0;
  constexpr int kHistFirst = kPairs ? kRLevelWords : 0;
  const int W = R.W;
  const int b = blockIdx.x, xcd = b & 7, local = b >> 3;
  const int li = (local / W) * 8 + xcd;  // the W slices of an output share b % 8
  const int s = local % W;
  if (li >= R.n_out) return;
  const int i = R.out0 + li;
  const int tid = threadIdx.x, lane = lane_id(), wave = r_uwave();

  const int rows = KIND == kResSample ? P.rows : RP.rows;
  const int V = KIND == kResSample ? P.vocab : RP.vocab;
  const int row = KIND == kResSample ? (P.indices ? as_global(P.indices)[i] : i) : i;
  const bool row_ok = row >= 0 && row < rows;
  const float* base = KIND == kResSample ? P.probs : RP.in;

  // ---- one HBM read of the slice into registers ------------------------------
  const int s0 = s * R.L;
  const int s1 = min(s0 + R.L, V);
  const int nvec = (s1 - s0) / 4;
  const gptr<const float4> src =
      as_global(reinterpret_cast<const float4*>(base + (int64_t)(row_ok ? row : 0) * V + s0));
  constexpr int kInFlight = NV < 5 ? NV : 5;
  float4 v[NV];
  const int vbase = wave * (kWave * NV) + lane;  // this thread's vector of load 0
  auto issue = [&](int j) __attribute__((always_inline)) {
    v[j] = load_f4_nt(src + min(vbase + j * kWave, nvec - 1));
  };
#pragma unroll
  for (int j = 0; j < kInFlight; ++j) issue(j);

  // parameters (read before any store, so they are scalar loads)
  float prm = 0.0f;
  if (KIND == kResRenorm) prm = RP.top_p_arr ? as_global(RP.top_p_arr)[i] : RP.top_p;
  else if (OP == kOpTopP || OP == kOpTopKTopP || kPairs)
    prm = P.top_p_arr ? as_global(P.top_p_arr)[i] : P.top_p;
  else if (OP == kOpMinP) prm = P.min_p_arr ? as_global(P.min_p_arr)[i] : P.min_p;
  const int kk = kTopK ? (P.top_k_arr ? as_global(P.top_k_arr)[i] : P.top_k) : 1;
  const uint64_t seed = KIND != kResSample ? 0ull : P.seed_arr ? as_global(P.seed_arr)[i] : P.seed;
  const uint64_t offset =
      KIND != kResSample ? 0ull : P.offset_arr ? as_global(P.offset_arr)[i] : P.offset;
  const uint64_t sid = (KIND == kResSample && P.seed_arr) ? 0ull : (uint64_t)i;
  const float pc = stream::clamp01(prm);
  // the output's draw, while the slice is in flight (only thread 0 uses it)
  // (kept in LDS until the draw rather than in registers through the searches)
  if (KIND == kResSample && wave == 0) {
    const double u = draw_uniform(seed, offset, sid, 0u);
    if (lane == 0) sm.udraw = u;
  }

  const gptr<r_v4f> dst = KIND == kResRenorm
                              ? (gptr<r_v4f>)as_global(RP.out + (int64_t)row * V + s0)
                              : (gptr<r_v4f>)nullptr;

  if (!row_ok || isnan(prm) || kk <= 0) {  // the same decision in every slice of the output
    res_invalid<KIND, NV>(P, RP, i, row, s, vbase, nvec, dst);
    return;
  }

  if (kTopP || kPairs) clear_lds_hist<kPairs>(sm);
  __syncthreads();

  // as each vector lands: its maximum pattern, and (top-p) its values'
  // significands added into bin bits[30:21] of the LDS histogram, copy
  // lane % 8, so that lanes hitting one bin mostly hit different words
  // (top-k then top-p by pairs: the values' (count, significand) pairs)
  uint32_t mx = 0u;
  HistRun<8> lrun;
  auto next = [&](int j) __attribute__((always_inline)) {
    if (j + kInFlight < NV) {
      __builtin_amdgcn_sched_barrier(0);
      issue(j + kInFlight);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const bool in = vbase + j * kWave < nvec;
    const uint32_t m = max4(v[j]);
    mx = max(mx, in ? m : 0u);
    if (kTopP && in) {
      const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        atomicAdd(&sm.hh[min(k4[e] >> 21, (uint32_t)(kRB1 - 1)) * 8u + (uint32_t)(lane & 7)],
                  (unsigned long long)sig_of(k4[e]));
    }
    if (kPairs) {
      const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) lrun.put(sm, in, min(k4[e] >> 21, (uint32_t)(kRB1 - 1)), pair_of(k4[e]));
    }
    next(j);
  }
  if (kPairs) lrun.flush(sm);
  mx = wave_max(mx);
  if (lane == 0) sm.wmax[wave] = mx;
  __syncthreads();

  const gptr<RowSlot> slot = as_global(R.slots + li);
  const gptr<uint32_t> ctl = (gptr<uint32_t>)slot->ctl;
  if (tid == 0) {
    uint32_t smax = 0u;
    for (int w = 0; w < kWaves; ++w) smax = max(smax, sm.wmax[w]);
    // a sign bit, an inf or a NaN shows as a pattern >= 0x7F800000
    __hip_atomic_fetch_max(ctl + 2, smax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(ctl + 1, 1u << r_xcc_id(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // plain sampling: tau is the smallest positive pattern, known now, so the
  // kept masses go out with the first arrival
  uint32_t tau = 1u;
  // publish the kept mass of this wave's range (chunk s * 16 + wave)
  auto publish_chunks = [&]() __attribute__((always_inline)) {
    fence_values<NV>(v);
    const double m = wave_mass<NV>(v, vbase, nvec, tau);
    if (lane == 0) ((gptr<double>)slot->chunk)[s * kWaves + wave] = m;
  };
  if (OP == kOpNone && KIND == kResSample) publish_chunks();
  if (kTopP) publish_hist<kRB1>(sm, (gptr<uint64_t>)slot->h1);
  if (kPairs) publish_hist<kRB1, true>(sm, (gptr<uint64_t>)slot->k1);

  uint32_t passed = 0u;
  // a wait that timed out: the output is reported invalid (every slice of
  // it times out too, its counters never reach the target)
  if (kTopP || kPairs) {
    __syncthreads();
    clear_lds_hist<kPairs>(sm);
    if (tid == 0) sm.lcnt = 0u;
  }
  DSS_RSTAMP(1);
  if (!row_barrier(ctl, (uint32_t)W, R.spin, sm)) return res_invalid<KIND, NV>(P, RP, i, row, 0, vbase, nvec, dst);
  DSS_RSTAMP(2);
  passed = 1u;
  const uint32_t gmax = __hip_atomic_load(ctl + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t xm = __hip_atomic_load(ctl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool bad = gmax >= 0x7F800000u || gmax == 0u || __popc(xm) != 1;

  double zkept = 0.0;
  if (bad) {
    res_invalid<KIND, NV>(P, RP, i, row, s, vbase, nvec, dst);
    row_leave(slot, passed, W, kHistWords, sm, kHistFirst);
    return;
  }

  if (kTopP) {
    // ---- threshold search, three levels --------------------------------------
    load_masses<kRB1>((gptr<uint64_t>)slot->h1, -1, sm);
    __syncthreads();
    uint32_t b1;
    double above1, ztot;
    res_find_w0<kRB1>(sm, 0.0, (double)pc, b1, above1, ztot);
    const double need = (double)pc * ztot;
    const uint32_t e1 = b1 >> 2;
    // the row's values in bin b1 number at most its significand sum / 2^23
    // (normal numbers): a small bin goes out as a key list instead of two
    // more rounds of row histograms
    const bool use_list = e1 >= 1u && ldexp(sm.md[b1], 127 - (int)e1) <= (double)kResidentSegKeys;
    if (pc >= 1.0f) {
      tau = 1u;  // every positive value
      zkept = ztot;
    } else if (use_list) {
      // this slice's keys in bin b1, in thread order, to its segment
      uint32_t cnt = 0u;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const bool in = vbase + j * kWave < nvec;
        const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) cnt += (in && (k4[e] >> 21) == b1) ? 1u : 0u;
      }
      uint32_t mine;
      uint32_t pos = res_block_scan(cnt, mine, sm);
      const gptr<uint32_t> seg = as_global(R.lists + (size_t)(li * W + s) * kResidentSegKeys);
      if (cnt != 0u) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const bool in = vbase + j * kWave < nvec;
          const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (in && (k4[e] >> 21) == b1) seg[pos++] = k4[e];
        }
      }
      if (tid == 0) __hip_atomic_store(ctl + 8 + s, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!row_barrier(ctl, 2u * (uint32_t)W, R.spin, sm)) return res_invalid<KIND, NV>(P, RP, i, row, 0, vbase, nvec, dst);
      passed = 2u;
      // every work-group: all of the row's keys in bin b1 (at most kResidentSegKeys)
      if (wave == 0) {
        const uint32_t c = lane < W ? __hip_atomic_load(ctl + 8 + lane, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT)
                                    : 0u;
        const uint32_t incl = wave_incl_scan(c);
        if (lane <= kRMaxW) sm.off[lane] = incl - c;
      }
      __syncthreads();
      const uint32_t n = sm.off[W];
      constexpr int kPer = kResidentSegKeys / kBlock;
      uint32_t kk[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const uint32_t g = (uint32_t)tid + (uint32_t)(q * kBlock);
        int sl = 0;
        for (int t = 1; t < W; ++t) sl = g >= sm.off[t] ? t : sl;
        const uint32_t at = min(g - sm.off[sl], (uint32_t)(kResidentSegKeys - 1));
        const uint32_t k = __hip_atomic_load(R.lists + (size_t)(li * W + sl) * kResidentSegKeys + at,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        kk[q] = g < n ? k : 0u;
      }
      // level 2 in LDS: bits [20:10], copy lane % 4
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        if (kk[q] != 0u)
          atomicAdd(&sm.hh[((kk[q] >> 10) & (uint32_t)(kRB2 - 1)) * 4u + (uint32_t)(lane & 3)],
                    (unsigned long long)sig_of(kk[q]));
      __syncthreads();
      fold_masses<kRB2>(sm, e1);
      __syncthreads();
      clear_lds_hist(sm);
      uint32_t b2;
      double above2, total2;
      res_find_w0<kRB2>(sm, need - above1, -1.0, b2, above2, total2);
      const uint32_t pre2 = (b1 << 11) | b2;
      // level 3 in LDS: bits [9:0] of the keys with bits [30:10] == pre2
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        if (kk[q] != 0u && (kk[q] >> 10) == pre2)
          atomicAdd(&sm.hh[(kk[q] & (uint32_t)(kRB3 - 1)) * 8u + (uint32_t)(lane & 7)],
                    (unsigned long long)sig_of(kk[q]));
      __syncthreads();
      fold_masses<kRB3>(sm, e1);
      __syncthreads();
      {
        uint32_t b3;
        double above, total;
        res_find_w0<kRB3>(sm, need - above1 - above2, -1.0, b3, above, total);
        tau = (pre2 << 10) | b3;
        zkept = above1 + above2 + (above + sm.md[b3]);
      }
    } else {
      // level 2: values in bin b1, by bits [20:10], copy lane % 4
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const bool in = vbase + j * kWave < nvec;
        const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (in && (k4[e] >> 21) == b1)
            atomicAdd(&sm.hh[((k4[e] >> 10) & (uint32_t)(kRB2 - 1)) * 4u + (uint32_t)(lane & 3)],
                      (unsigned long long)sig_of(k4[e]));
      }
      __syncthreads();
      publish_hist<kRB2>(sm, (gptr<uint64_t>)slot->h2);
      __syncthreads();
      clear_lds_hist(sm);
      if (!row_barrier(ctl, 2u * (uint32_t)W, R.spin, sm)) return res_invalid<KIND, NV>(P, RP, i, row, 0, vbase, nvec, dst);
      passed = 2u;
      load_masses<kRB2>((gptr<uint64_t>)slot->h2, (int)(b1 >> 2), sm);
      __syncthreads();
      uint32_t b2;
      double above2, total2;
      res_find_w0<kRB2>(sm, need - above1, -1.0, b2, above2, total2);
      const uint32_t pre2 = (b1 << 11) | b2;
      // level 3: values with bits [30:10] == pre2, by bits [9:0], copy lane % 8
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const bool in = vbase + j * kWave < nvec;
        const uint32_t k4[4] = {bits_of(v[j].x), bits_of(v[j].y), bits_of(v[j].z), bits_of(v[j].w)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (in && (k4[e] >> 10) == pre2)
            atomicAdd(&sm.hh[(k4[e] & (uint32_t)(kRB3 - 1)) * 8u + (uint32_t)(lane & 7)],
                      (unsigned long long)sig_of(k4[e]));
      }
      __syncthreads();
      publish_hist<kRB3>(sm, (gptr<uint64_t>)slot->h3);
      if (!row_barrier(ctl, 3u * (uint32_t)W, R.spin, sm)) return res_invalid<KIND, NV>(P, RP, i, row, 0, vbase, nvec, dst);
      passed = 3u;
      load_masses<kRB3>((gptr<uint64_t>)slot->h3, (int)(b1 >> 2), sm);
      __syncthreads();
      {
        uint32_t b3;
        double above, total;
        res_find_w0<kRB3>(sm, need - above1 - above2, -1.0, b3, above, total);
        tau = (pre2 << 10) | b3;
        zkept = above1 + above2 + (above + sm.md[b3]);
      }
    }
  } else if (OP == kOpMinP) {
    // the smallest float32 >= min_p * max (an exact double product)
    const double thr = (double)pc * (double)__uint_as_float(gmax);
    float f = (float)thr;
    if ((double)f < thr) f = __uint_as_float(bits_of(f) + 1u);
    tau = max(bits_of(f), 1u);
  } else if (kPairs) {
    // both thresholds from one search on (count, mass) pairs (k at most
    // kResidentSegKeys, checked by the launcher)
    if (!res_search_kp<NV>(v, vbase, nvec, kk, pc, (gptr<uint64_t>)slot->k1, (gptr<uint64_t>)slot->k2,
                           (gptr<uint64_t>)slot->k3, ctl, as_global(R.lists), li, s, W, R.spin, passed,
                           sm, tau, zkept))
      return res_invalid<KIND, NV>(P, RP, i, row, 0, vbase, nvec, dst);
  } else if (kTopK) {
    // tau_k = the k-th largest pattern (ties kept), by counts; then, for
    // top-k-then-top-p, the top-p threshold inside {x >= tau_k} by masses
    uint32_t tk;
    double cnt;
    if (!res_search<true, NV>(v, vbase, nvec, 0u, (double)kk, -1.0, (gptr<uint64_t>)slot->k1,
                              (gptr<uint64_t>)slot->k2, (gptr<uint64_t>)slot->k3, ctl,
                              as_global(R.lists), li, s, W, R.spin, passed, sm, tk, cnt))
      return res_invalid<KIND, NV>(P, RP, i, row, 0, vbase, nvec, dst);
    tau = max(tk, 1u);  // zeros carry no mass
    if (OP == kOpTopKTopP) {
      uint32_t tp;
      double zk;
      if (!res_search<false, NV>(v, vbase, nvec, tau, 0.0, (double)pc, (gptr<uint64_t>)slot->h1,
                                 (gptr<uint64_t>)slot->h2, (gptr<uint64_t>)slot->h3, ctl,
                                 as_global(R.lists), li, s, W, R.spin, passed, sm, tp, zk))
        return res_invalid<KIND, NV>(P, RP, i, row, 0, vbase, nvec, dst);
      tau = max(tp, tau);
    }
  }

  if (KIND == kResRenorm) {
    const double inv = 1.0 / zkept;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      r_v4f o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = bits_of(x[e]) >= tau ? (float)((double)x[e] * inv) : 0.0f;
      if (vbase + j * kWave < nvec) dst[vbase + j * kWave] = o;
    }
    if (s == 0 && tid == 0 && RP.row_status) as_global(RP.row_status)[row] = 0;
    row_leave(slot, passed, W, kRLevelWords, sm);
    return;
  }

  // ---- sampling: kept mass per (slice, wave), one draw, the owner walks -----
  if (OP != kOpNone) {
    publish_chunks();
    DSS_RSTAMP(16);
    if (!row_barrier(ctl, (passed + 1u) * (uint32_t)W, R.spin, sm))
      return res_invalid<KIND, NV>(P, RP, i, row, 0, vbase, nvec, dst);
    DSS_RSTAMP(17);
    ++passed;
  }
  // every work-group, wave 0: the chunk holding u * (total kept mass);
  // lane l holds chunks [4l, 4l + 4) (slice-major, index order)
  if (wave == 0) {
    const int nch = W * kWaves;
    double cmq[4];
    double ls = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = 4 * lane + q;
      cmq[q] = c < nch ? __hip_atomic_load((gptr<double>)slot->chunk + c, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)
                       : 0.0;
      ls += cmq[q];
    }
    const double incl = wave_incl_scan(ls);
    const double T = sm.udraw * lane63(incl);
    const uint64_t hit = __ballot(ls > 0.0 && incl > T);
    const bool fallback = hit == 0ull;
    const int L = fallback ? r_last_lane(__ballot(ls > 0.0) | 1ull) : r_first_lane(hit);
    if (lane == L) {
      double acc = incl - ls;
      int pick = -1, lastc = -1;
      double ex_pick = 0.0, mlast = 0.0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double before = acc;
        acc += cmq[q];
        if (cmq[q] > 0.0) {
          lastc = q;
          mlast = cmq[q];
          if (pick < 0 && !fallback && acc > T) {
            pick = q;
            ex_pick = before;
          }
        }
      }
      const int q = pick >= 0 ? pick : lastc;
      sm.res[3] = q < 0 ? 0xFFFFFFFFu : (uint32_t)(4 * L + q);
      // no prefix beyond T (rounding): a target past the chunk's mass makes
      // the owner wave take its last kept value
      sm.resd[3] = pick >= 0 ? T - ex_pick : 2.0 * mlast;
    }
  }
  __syncthreads();
  const uint32_t c = sm.res[3];
  if (c == 0xFFFFFFFFu) {  // cannot happen for a valid row (its maximum is kept)
    if (s == 0 && tid == 0) stream::write_sample(P, i, -1, 0);
  } else if ((int)c / kWaves == s && (int)c % kWaves == wave) {
    // the owner wave; the slot is left afterwards, off this path
    const double Tl = sm.resd[3];
    fence_values<NV>(v);
    WalkPick pk;
    const double Te = wave_walk<NV>(v, vbase, nvec, tau, Tl, sm.md, pk);
    fence_values<NV>(v);
    const int pos = pick_value<NV>(v, vbase, tau, Te, pk);
    if (pk.j < 0) {
      if (lane == 0) stream::write_sample(P, i, -1, 0);
    } else if (lane == pk.l) {
      stream::write_sample(P, i, pos >= 0 ? s0 + pos : -1, pos >= 0 ? 1 : 0);
    }
  }
  DSS_RSTAMP(18);
  row_leave(slot, passed, W, kHistWords, sm, kHistFirst);
}

// ---------------------------------------------------------------------------
// Probabilities from logits with a temperature (explainer, 采样流水线究竟在
// 计算什么: p_i = exp(z_i / T) / sum_j exp(z_j / T)).  The W work-groups of a
// row keep its slices in registers: the row's maximum m at the first
// barrier, the sum S of exp((z_i - m) / T) at the second, then every slice
// writes float32(exp((z_i - m) / T) / S).  Differences, scaling, exponentials
// and sums are float64 (the maximum is subtracted for range only); a NaN or
// +inf logit, no finite logit, or T not a finite positive number make the
// row invalid (NaN-filled, status 1).
// ---------------------------------------------------------------------------


template <int NV>
__global__ __launch_bounds__(kBlock) void softmax_kernel(SoftmaxParams Q, ResidentParams R) {
  __shared__ ResSmem sm;
  const int W = R.W;
  const int b = blockIdx.x, xcd = b & 7, local = b >> 3;
  const int li = (local / W) * 8 + xcd;
  const int s = local % W;
  if (li >= R.n_out) return;
  const int row = R.out0 + li;
  const int tid = threadIdx.x, lane = lane_id(), wave = r_uwave();
  const int V = Q.vocab;
  const int s0 = s * R.L;
  const int s1 = min(s0 + R.L, V);
  const int nvec = (s1 - s0) / 4;
  const gptr<const float4> src =
      as_global(reinterpret_cast<const float4*>(Q.in + (int64_t)row * V + s0));
  constexpr int kInFlight = NV < 5 ? NV : 5;
  const int vbase = wave * (kWave * NV) + lane;
  float4 v[NV];
  auto issue = [&](int j) __attribute__((always_inline)) {
    v[j] = load_f4_nt(src + min(vbase + j * kWave, nvec - 1));
  };
#pragma unroll
  for (int j = 0; j < kInFlight; ++j) issue(j);
  const float T = Q.temp_arr ? as_global(Q.temp_arr)[row] : Q.temp;
  const gptr<r_v4f> dst = (gptr<r_v4f>)as_global(Q.out + (int64_t)row * V + s0);

  // as the slice lands: its largest signed-order key, and NaN / +inf
  uint32_t mk = 0u;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const bool in = vbase + j * kWave < nvec;
    const float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mk = max(mk, in ? signed_key(x[e]) : 0u);
      bad = bad || (in && (isnan(x[e]) || x[e] == __builtin_inff()));
    }
    if (j + kInFlight < NV) {
      __builtin_amdgcn_sched_barrier(0);
      issue(j + kInFlight);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  mk = wave_max(mk);
  const bool wb = __ballot(bad) != 0ull;
  if (lane == 0) {
    sm.wmax[wave] = mk;
    sm.wbad[wave] = wb ? 1u : 0u;
  }
  __syncthreads();
  const gptr<RowSlot> slot = as_global(R.slots + li);
  const gptr<uint32_t> ctl = (gptr<uint32_t>)slot->ctl;
  if (tid == 0) {
    uint32_t smax = 0u, sbad = 0u;
    for (int w = 0; w < kWaves; ++w) {
      smax = max(smax, sm.wmax[w]);
      sbad |= sm.wbad[w];
    }
    __hip_atomic_fetch_max(ctl + 2, smax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (sbad) __hip_atomic_fetch_or(ctl + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(ctl + 1, 1u << r_xcc_id(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  auto invalid = [&]() __attribute__((always_inline)) {
    r_v4f o;
    o.x = o.y = o.z = o.w = __uint_as_float(0x7FC00000u);
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (vbase + j * kWave < nvec) dst[vbase + j * kWave] = o;
    if (s == 0 && tid == 0 && Q.row_status) as_global(Q.row_status)[row] = 1;
  };
  if (!row_barrier(ctl, (uint32_t)W, R.spin, sm)) return invalid();
  const uint32_t gk = __hip_atomic_load(ctl + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t gb = __hip_atomic_load(ctl + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t xm = __hip_atomic_load(ctl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float zmax = from_signed_key(gk);
  if (gb != 0u || __popc(xm) != 1 || !(T > 0.0f) || T == __builtin_inff() ||
      zmax == -__builtin_inff()) {
    invalid();
    row_leave(slot, 1u, W, 0, sm);
    return;
  }
  const double m = (double)zmax, it = 1.0 / (double)T;

  // the slice's sum of exponentials, in a fixed order
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    fence_vec(v[j], acc);
    const bool in = vbase + j * kWave < nvec;
    const float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += in ? exp(((double)x[e] - m) * it) : 0.0;
  }
  acc = wave_sum(acc);
  if (lane == 0) sm.md[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    double z = 0.0;
    for (int w = 0; w < kWaves; ++w) z += sm.md[w];
    __hip_atomic_store((gptr<double>)slot->chunk + s, z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!row_barrier(ctl, 2u * (uint32_t)W, R.spin, sm)) return invalid();
  if (wave == 0) {
    const double z = lane < W ? __hip_atomic_load((gptr<double>)slot->chunk + lane, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT)
                              : 0.0;
    const double tot = lane63(wave_incl_scan(z));
    if (lane == 0) sm.resd[0] = tot;
  }
  __syncthreads();
  const double S = sm.resd[0];
  double chain = 0.0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    fence_vec(v[j], chain);
    const float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
    r_v4f o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (float)(exp(((double)x[e] - m) * it) / S);
    if (vbase + j * kWave < nvec) dst[vbase + j * kWave] = o;
    chain = (double)o[0];
  }
  if (s == 0 && tid == 0 && Q.row_status) as_global(Q.row_status)[row] = 0;
  row_leave(slot, 2u, W, 0, sm);
}

}  // namespace
}  // namespace dss

namespace dss {
namespace {

static_assert(sizeof(RowSlot) == kResidentSlotBytes, "workspace layout of the resident engine");
static_assert(sizeof(RowSlot) % 16 == 0, "slots cleared in 16-byte words");


template <int KIND, int OP, int NV>
hipError_t launch_res_one(const SampleParams& p, const RenormParams& rp, const SplitPlan& plan,
                          void* workspace, hipStream_t s, const LaunchEvents& ev) {
  // work-groups the device keeps resident at once, asked once per process
  static int cap = -1;
  if (cap < 0) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(resident_kernel<KIND, OP, NV>), kBlock, 0);
    if (e != hipSuccess) return e;
    cap = cus * per_cu;
  }
  ResidentParams R;
  R.W = plan.W;
  R.L = plan.L;
  R.slots = reinterpret_cast<RowSlot*>(static_cast<char*>(workspace) + kCtlRegionBytes);
  R.spin = spin_limit_ticks();
  R.lists = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + kCtlRegionBytes +
                                        (size_t)kResidentSlots * kResidentSlotBytes);
  // outputs per launch: whole groups of eight (one per XCD), all resident
  const int per = min(plan.chunk, (cap / (8 * plan.W)) * 8);
  const int total = KIND == kResSample ? p.num_outputs : rp.rows;
  if (per <= 0) return hipErrorInvalidConfiguration;
  for (int out0 = 0; out0 < total; out0 += per) {
    R.out0 = out0;
    R.n_out = min(per, total - out0);
    const bool first = out0 == 0, last = out0 + per >= total;
    const dim3 grid((unsigned)(((R.n_out + 7) / 8) * 8 * plan.W)), block(kBlock);
    launch_kernel(resident_kernel<KIND, OP, NV>, grid, block, s, ev, first, last, p, rp, R);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int KIND, int OP>
hipError_t launch_res_nv(const SampleParams& p, const RenormParams& rp, const SplitPlan& plan,
                         void* ws, hipStream_t s, const LaunchEvents& ev) {
  // the top-k searches keep more live state: their plans stop at eight loads
  constexpr bool kTopKOp = OP == kOpTopK || OP == kOpTopKTopP || OP == kOpResPairs;
  switch (plan.nv) {
    case 1: return launch_res_one<KIND, OP, 1>(p, rp, plan, ws, s, ev);
    case 2: return launch_res_one<KIND, OP, 2>(p, rp, plan, ws, s, ev);
    case 4: return launch_res_one<KIND, OP, 4>(p, rp, plan, ws, s, ev);
    case 8: return launch_res_one<KIND, OP, 8>(p, rp, plan, ws, s, ev);
    case 10:
      if constexpr (kTopKOp) return hipErrorInvalidValue;
      else return launch_res_one<KIND, OP, 10>(p, rp, plan, ws, s, ev);
    case 12:
      if constexpr (kTopKOp) return hipErrorInvalidValue;
      else return launch_res_one<KIND, OP, 12>(p, rp, plan, ws, s, ev);
    case 16:  // plain, top-p, min-p and pair-search sampling only (plan_resident's wide plans)
      if constexpr (KIND == kResSample &&
                    (OP == kOpNone || OP == kOpMinP || OP == kOpTopP || OP == kOpResPairs))
        return launch_res_one<KIND, OP, 16>(p, rp, plan, ws, s, ev);
      else return hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

SplitPlan plan_resident(int op, int vocab, int num_outputs, uint32_t flags, int vec_ok,
                        bool sample, bool pairs) {
  SplitPlan plan{0, 0, 0, 0, 0, 0};
  if (op != kOpNone && op != kOpTopP && op != kOpMinP && op != kOpTopK && op != kOpTopKTopP)
    return plan;
  if (flags & (DSS_FLAG_STREAMING | DSS_FLAG_FROM_ZERO | DSS_FLAG_SINGLE_PIVOT)) return plan;
  if (!vec_ok || vocab < 1024 || num_outputs <= 0) return plan;
  // values a slice holds: 48 per thread, 32 for the top-k searches
  const bool topk = op == kOpTopK || op == kOpTopKTopP;
  const int kMaxSlice = (topk ? 8 : kRMaxNv) * 4 * kBlock;
  int wmin = (vocab + kMaxSlice - 1) / kMaxSlice;
  // (the pair search may hold 64 values per thread, so rows up to sixteen
  // such slices stay resident)
  constexpr int kWideSlice = kRWideNv * 4 * kBlock;
  if ((pairs ? (vocab + kWideSlice - 1) / kWideSlice : wmin) > kRMaxW) return plan;
  // plain, top-p and min-p sampling, and top-k then top-p by the pair
  // search, keep few other values live and may hold 64 values per thread:
  // half the slices, so twice the outputs per launch when a batch needs more
  // than one launch
  const bool wide = sample && (op == kOpNone || op == kOpMinP || op == kOpTopP || pairs);
  if (wide) wmin = (vocab + kRWideNv * 4 * kBlock - 1) / (kRWideNv * 4 * kBlock);
  const int wt = (kResidentSlots + num_outputs - 1) / num_outputs;
  // W: a power of two, at least wmin, about 256 work-groups in all, no empty slice
  int W = 1;
  while (W < wmin || (W * 2 <= kRMaxW && W * 2 <= wt)) W *= 2;
  int L = 0;
  for (;; W /= 2) {
    L = ((vocab + 4 * W - 1) / (4 * W)) * 4;
    if (W == 1 || (int64_t)(W - 1) * L < vocab) break;
  }
  if (W < wmin) return plan;
  int nv = (L / 4 + kBlock - 1) / kBlock;
  nv = nv <= 2 ? nv : nv <= 4 ? 4 : nv <= 8 ? 8 : nv <= 10 ? 10 : nv <= 12 ? 12 : kRWideNv;
  if (topk && nv > 8) {  // the pair search holds 64 values per thread, the others at most 32
    if (!wide) return plan;
    nv = kRWideNv;
  }
  plan.W = W;
  plan.L = L;
  plan.nv = nv;
  plan.chunk = min(num_outputs, kResidentSlots / W);
  plan.handoff = kFixedRegionBytes;
  plan.workspace = kFixedRegionBytes;
  return plan;
}

namespace {
// Zero every slot whose arrival counter carries the broken mark (a row
// barrier given up in an earlier launch), for a workspace that no caller can
// zero.  One work-group per slot; the kernels that use the slots come later
// on the same stream, so no work-group of theirs can see a half-cleared slot.
__global__ __launch_bounds__(256) void repair_kernel(RowSlot* slots) {
  const gptr<RowSlot> slot = as_global(slots + blockIdx.x);
  const uint32_t c = __hip_atomic_load((gptr<uint32_t>)slot->ctl, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  if (!(c & kBroken)) return;
  uint4* w = reinterpret_cast<uint4*>(slots + blockIdx.x);
  for (int q = threadIdx.x; q < (int)(sizeof(RowSlot) / 16); q += 256)
    w[q] = make_uint4(0u, 0u, 0u, 0u);
}
}  // namespace

hipError_t launch_resident_repair(void* workspace, hipStream_t s) {
  RowSlot* slots = reinterpret_cast<RowSlot*>(static_cast<char*>(workspace) + kCtlRegionBytes);
  hipLaunchKernelGGL(repair_kernel, dim3(kResidentSlots), dim3(256), 0, s, slots);
  return hipGetLastError();
}

hipError_t launch_resident_sample(int op, const SampleParams& p, const SplitPlan& plan,
                                  void* workspace, hipStream_t s, const LaunchEvents& ev) {
  const RenormParams rp{};
  hipError_t e;
  if (op == kOpNone) e = launch_res_nv<kResSample, kOpNone>(p, rp, plan, workspace, s, ev);
  else if (op == kOpTopP) e = launch_res_nv<kResSample, kOpTopP>(p, rp, plan, workspace, s, ev);
  else if (op == kOpTopK) e = launch_res_nv<kResSample, kOpTopK>(p, rp, plan, workspace, s, ev);
  else if (resident_pairs(op, p.top_k_arr, p.top_k, p.vocab))
    e = launch_res_nv<kResSample, kOpResPairs>(p, rp, plan, workspace, s, ev);
  else if (op == kOpTopKTopP) e = launch_res_nv<kResSample, kOpTopKTopP>(p, rp, plan, workspace, s, ev);
  else e = launch_res_nv<kResSample, kOpMinP>(p, rp, plan, workspace, s, ev);
  // a device that cannot hold one group of work-groups at once: streaming engine
  if (e == hipErrorInvalidConfiguration) e = launch_stream_sample(op, p, s, ev);
  return e;
}

SplitPlan plan_softmax(int rows, int vocab, uint32_t flags, int vec_ok) {
  // the same slicing as the resident sampling kernels (a plain op id)
  if (flags & DSS_FLAG_STREAMING) return SplitPlan{0, 0, 0, 0, 0, 0};
  return plan_resident(kOpNone, vocab, rows, 0u, vec_ok);
}

namespace {
template <int NV>
hipError_t launch_softmax_nv(const SoftmaxParams& q, const SplitPlan& plan, void* workspace,
                             hipStream_t s, const LaunchEvents& ev) {
  static int cap = -1;
  if (cap < 0) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(softmax_kernel<NV>), kBlock, 0);
    if (e != hipSuccess) return e;
    cap = cus * per_cu;
  }
  ResidentParams R;
  R.W = plan.W;
  R.L = plan.L;
  R.slots = reinterpret_cast<RowSlot*>(static_cast<char*>(workspace) + kCtlRegionBytes);
  R.spin = spin_limit_ticks();
  R.lists = nullptr;
  const int per = min(plan.chunk, (cap / (8 * plan.W)) * 8);
  if (per <= 0) return hipErrorInvalidConfiguration;
  for (int out0 = 0; out0 < q.rows; out0 += per) {
    R.out0 = out0;
    R.n_out = min(per, q.rows - out0);
    const bool first = out0 == 0, last = out0 + per >= q.rows;
    const dim3 grid((unsigned)(((R.n_out + 7) / 8) * 8 * plan.W)), block(kBlock);
    launch_kernel(softmax_kernel<NV>, grid, block, s, ev, first, last, q, R);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
}  // namespace

hipError_t launch_softmax(const SoftmaxParams& q, const SplitPlan& plan, void* workspace,
                          hipStream_t s, const LaunchEvents& ev) {
  hipError_t e = hipErrorInvalidConfiguration;
  if (plan.W > 0) {
    switch (plan.nv) {
      case 1: e = launch_softmax_nv<1>(q, plan, workspace, s, ev); break;
      case 2: e = launch_softmax_nv<2>(q, plan, workspace, s, ev); break;
      case 4: e = launch_softmax_nv<4>(q, plan, workspace, s, ev); break;
      case 8: e = launch_softmax_nv<8>(q, plan, workspace, s, ev); break;
      case 10: e = launch_softmax_nv<10>(q, plan, workspace, s, ev); break;
      default: e = launch_softmax_nv<12>(q, plan, workspace, s, ev); break;
    }
  }
  if (e == hipErrorInvalidConfiguration) e = launch_stream_softmax(q, s, ev);
  return e;
}

hipError_t launch_resident_renorm(const RenormParams& rp, const SplitPlan& plan, void* workspace,
                                  hipStream_t s, const LaunchEvents& ev) {
  const SampleParams p{};
  hipError_t e = launch_res_nv<kResRenorm, kOpTopP>(p, rp, plan, workspace, s, ev);
  if (e == hipErrorInvalidConfiguration) e = launch_stream_renorm(kRenormTopP, rp, s, ev);
  return e;
}

}  // namespace dss
