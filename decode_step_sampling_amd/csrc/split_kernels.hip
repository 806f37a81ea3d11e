// Split-row engine for top-k and top-k-then-top-p sampling.
//
// The dual-pivot rejection loop of the FlashInfer blog ("Sorting-Free GPU
// Kernels for LLM Sampling", section 双枢轴拒绝采样) only ever draws from the
// values above the current `low`, and its correctness proof (section
// 拒绝采样器正确性的理论证明) holds from any starting pivot below every kept
// value.  The engine therefore reads each row from HBM exactly once and runs
// the loop on the row's top-k set only:
//
//  1. Each row is cut into W slices, one 1024-thread work-group per slice;
//     every thread issues all of its 16-byte loads of the slice at once.  As
//     each vector lands the thread takes its maximum (on the float32 bit
//     pattern, which orders non-negative values like the values, F4 note §③)
//     and counts it in a 2048-bin LDS histogram of the top eleven bits.
//  2. The slice bound b is the lower edge of the histogram bin holding the
//     k-th largest vector maximum.  At least k vectors, hence at least k
//     values, are >= b, so b never exceeds the slice's k-th largest value and
//     therefore never exceeds the row's: every value of the row's top-k set
//     lies at or above the bound of its slice.  No estimate is involved.
//  3. Vectors holding a value >= b are staged in LDS (one block scan), their
//     elements >= b are extracted (a second scan) and published as
//     (bits | index << 32) entries.
//  4. The last work-group of the row to arrive (a relaxed arrival counter)
//     loads every slice's entries, keeps those >= t* = max_s b_s (the row's
//     top-k set lies above t*, and at least k entries do), finds the k-th
//     largest tau_k with a histogram on a key relative to t* followed by an
//     exact rank inside the boundary bin, and one wave runs the dual-pivot
//     loop on the values >= tau_k, starting just below tau_k, where f(low) = 0
//     still holds.
//
// All W work-groups of a row are placed on one XCD (work-groups are dispatched
// to the eight XCDs round-robin, so block b runs on XCD b % 8), which lets the
// hand-off use the XCD's shared L2 with relaxed atomics instead of
// device-wide acquire/release fences.  Every published header carries the
// row's generation number and the writer's XCC id; the finishing work-group
// checks both and falls back to the streaming engine (stream_device.h) if
// anything looks foreign, or if a list overflows its capacity (flat rows).
#include "split_device.h"

// Phase clock stamps of the split sampling kernel (compiled in only with
// -DDSS_PHASE_STAMPS, for the measurement build libdss_stamps.so): thread 0
// of every work-group writes the 100 MHz constant clock at the phase
// boundaries marked DSS_STAMP(n) into stamps[block * 32 + n]; the buffer is
// set by dss_debug_set_stamps (that build only).
#ifdef DSS_PHASE_STAMPS
__device__ unsigned long long* g_dss_stamps;
extern "C" __attribute__((visibility("default"))) int dss_debug_set_stamps(void* p) {
  return hipMemcpyToSymbol(HIP_SYMBOL(g_dss_stamps), &p, sizeof(p)) == hipSuccess ? 0 : -4;
}
#define DSS_STAMP(n)                                                          \
  do {                                                                        \
    if (threadIdx.x == 0 && g_dss_stamps)                                     \
      g_dss_stamps[blockIdx.x * 32 + (n)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define DSS_STAMP(n) \
  do {               \
  } while (0)
#endif

namespace dss {
namespace {

constexpr int kStageMax = 3072;   // vectors a slice stages in LDS
constexpr int kRegion = kStageMax / 16;  // staging region of one wave (provisional bound)
constexpr int kListMax = kSplitListEntries;  // entries a slice publishes
constexpr int kRowCandMax = 8192; // entries of all slices of a row (the merge's LDS copy)
constexpr int kKeptMax = 4096;    // entries of the top-k set (ties included)
constexpr int kBndMax = 4096;     // entries in the boundary bin
constexpr int kSplitKCap = 2048;
static_assert(kSplitKCap == kSplitKCapHost, "the host routes on the same cap");
static_assert(kSplitScalarKW == kRowCandMax / 2, "half of a row's merge capacity");
constexpr int kMaxSlices = 16;    // a power of two
constexpr int kHdrWords = kSplitHdrWords;
constexpr int kLoadBatch = 8;     // list loads a merge thread keeps in flight
constexpr int kDepth = 5;         // slice loads a thread keeps in flight
constexpr uint32_t kNoList = 0xFFFFFFFFu;  // header count of a slice that published nothing

struct SplitParams {
  int W;           // slices per output (a power of two)
  int wlog;        // log2(W)
  int L;           // slice length in values (multiple of 4)
  int out0;        // first output handled by this launch
  int n_out;       // outputs handled by this launch
  uint32_t* ctr;   // [kChunk] arrival counters (zero between calls)
  uint32_t* gen;   // [kChunk] generation numbers
  uint32_t* hdr;   // [n_out][W][kHdrWords]
  uint64_t* list;  // [n_out][W][kListMax]: key | (index << 32)
  uint32_t* r_tau;    // renorm / mask: [n_out] tau_k as an order key
  double* r_z;        // renorm: [n_out] kept mass Z_k
  uint8_t* r_status;  // renorm / mask: [n_out] 0 ok, 1 invalid row, 2 written already
  // Finishing work-groups (sampling with per-output k over more than one
  // wave of work-groups): the slices of an output with k above the
  // candidate cap publish their histograms and leave; one work-group per
  // output, placed after every slice in the grid, waits for them and merges.
  int fin;         // 1: the grid ends with finishing work-groups
  int nsb;         // work-groups of slices (the finishing ones start here)
  uint64_t spin;   // ticks of the 100 MHz constant clock a finisher waits at most
  int test_foreign;  // 1: every hand-off is treated as foreign (a test setting)
};

// What the split engine computes: a sample; tau_k (and Z_k) for a top-k
// renormalisation or a top-k logit mask, written by a second kernel; the
// top-k values and indices themselves (selection: the top-k set, already in
// LDS, sorted by key and index); or a sample from logits, the softmax fused
// in (kKindLogits: the slices rank logits by their signed-order keys and
// publish their maxima; the finishing work-group turns its candidates into
// the softmax's weights exp((z - m) / T) before the rest runs as for
// kKindSample).
enum SplitKind : int { kKindSample = 0, kKindRenorm = 1, kKindMask = 2, kKindSelect = 3,
                       kKindLogits = 4 };

struct LkSmem {                  // the large-k merge (inside SplitSmem's union)
  stream::SampleSmem s;          // tile masses and the locate() scratch
  double md[kHistBins];          // the row's bin masses
  unsigned long long hm[kHistBins];  // significand sums of one selection level
  uint32_t tst[stream::kMaxTiles];  // per tile: where its gathered keys start,
  uint32_t tcn[stream::kMaxTiles];  // and how many there are
  uint32_t nlist;                // keys gathered
  uint32_t res[8];
  double resd[4];
};

// Order key of a value: the float32 bits for probabilities (non-negative,
// F4 note §③), the signed-order key for logits (F4 note §⑧).
struct SplitSmem {
  uint64_t full[kRowCandMax + kWave];  // every slice's entries, in (slice, position) order;
                                       // the last kWave slots take branch-free dummy writes
  union {
    struct {
      float4 vec[kStageMax + kWave];     // staged vectors (+ per-lane dummy slots)
      uint32_t vidx[kStageMax + kWave];  // their vector index inside the slice
    } a;
    struct {
      uint64_t cand[kKeptMax + kWave];  // the top-k set, in candidate order (+ dummies)
      uint64_t bnd[kBndMax + kWave];    // entries in the boundary bin (+ dummies)
    } b;
    stream::SampleSmem stream;   // streaming fallback
    stream::SelectSmem sel;      // streaming fallback of a selection
    stream::RadixSmem radix;     // exact fallback of top-k sampling
    struct {                     // large k, a slice: count and significand sum of
      unsigned long long cm[2][kHistBins];  // each bin of bits [30:20] packed in one
    } lk;                                   // word; two copies (lane parity)
    LkSmem lm;                   // large k, the merge
  } u;
  alignas(16) uint32_t hist[H1::kWords];
  // fixed-point masses of the top-k entries above the boundary bin, per
  // group of eight histogram bins (+ per-lane dummy slots)
  alignas(16) uint32_t mh[kMassBins + kWave];
  double draws[stream::kPreDraws];
  double etab[64];                // logits: 2^(j / 64), j = 0 .. 63 (table_exp)
  uint32_t red[4][kWaves];        // per-wave partials of the block scans
  uint32_t wmax[kWaves];
  uint32_t wnan[kWaves];
  uint32_t off[kMaxSlices + 1];
  uint32_t sel[kWave];
  uint32_t res[8];
  uint32_t fres[4];
  uint32_t tp;                    // provisional slice bound
  double wz[kWaves];              // joint order: per-wave totals of the slice
  double zs;                      // joint order: the slice's total, then the row's
  uint32_t wcnt[kWaves];          // vectors each wave staged (0xFFFFFFFF: overflow)
  int flag;
};
static_assert(sizeof(SplitSmem) <= 160 * 1024, "LDS budget of one gfx950 work-group");

enum SplitMode : int { kDone = 0, kFallback = 1, kLargeKMerge = 2 };

// exp(x) in float64 for x <= 0 (0 below -745, and for -inf): x = n ln2/64 + r
// with n = round(64 x / ln2) (the constant ln2/64 split in two so that n
// times its first part is exact), |r| <= ln2/128, exp(r) by its Taylor
// polynomial to degree 5 (truncation below 4e-17), times tab[n mod 64] =
// 2^((n mod 64) / 64), scaled by 2^floor(n / 64).  Within about 2 ulp.
__device__ __forceinline__ double table_exp(double x, const double* tab) {
  if (!(x > -745.0)) return 0.0;
  const double n = __builtin_rint(x * 0x1.71547652b82fep+6);  // 64 / ln2
  const int ni = (int)n;
  double r = __builtin_fma(-n, 0x1.62e42fefa0000p-7, x);
  r = __builtin_fma(-n, 0x1.cf79abc9e3b3ap-46, r);
  double p = __builtin_fma(r, 1.0 / 120.0, 1.0 / 24.0);
  p = __builtin_fma(p, r, 1.0 / 6.0);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  return __builtin_ldexp(p * tab[ni & 63], ni >> 6);
}

// Everything but the streaming fallback; returns kFallback when the output
// must be sampled by the streaming engine instead (one call site, below).
// Reports output i (chunk-local li) invalid; every thread calls it.
template <int KIND>
__device__ __forceinline__ void split_invalid(const SampleParams& P, const SplitParams& S,
                                              const SelectParams& Q, int i, int li) {
  if (KIND == kKindSelect) {
    stream::select_invalid(Q, i);
    return;
  }
  if (threadIdx.x != 0) return;
  if (KIND == kKindSample || KIND == kKindLogits) stream::write_sample(P, i, -1, 0);
  else as_global(S.r_status)[li] = 1;
}

// ---- large k (above the candidate cap) -----------------------------------
// Every slice counts its values and sums their 24-bit significands per bin
// of bits [30:20] (one eighth of a binade: a bin's mass is an exact integer
// times one power of two) and publishes the two histograms through the
// hand-off area instead of a candidate list.  The last work-group of the row
// adds them up and finds the bin b_k holding the k-th largest value (counts
// from the top) and the bins the top-p cut can fall in; one pass over the
// row gathers the keys of those bins, and two more histogram levels over
// the gathered keys (bits [19:9], then [8:0]) give tau_k, Z_k and the top-p
// cut exactly (the threshold search of the F4 note, §③, with 2047 pivots per
// level); one more pass gives the kept mass of every tile for the draw
// (blog, 逆变换采样).  Rows whose boundary bins hold more values than the
// gather keeps go to the exact passes of the streaming engine.
constexpr uint32_t kLargeList = 0xFFFFFFFEu;  // header count of a slice that published histograms
constexpr int kFinMinBlocks = 256;  // one work-group per compute unit on the whole chip
constexpr uint32_t kLkGather = 16384;         // keys the merge gathers (LDS)
// A slice's bin word: the count above this bit, the significand sum below
// (a slice holds at most 10 vectors per thread, a copy half of them, each
// significand below 2^24: sums below 2^44, counts below 2^20).
constexpr int kLkCountShift = 44;
static_assert(10 * 4 * kBlock / 2 <= (1 << 20) && 64 - kLkCountShift >= 20, "packed bin words");


// Inside the keys x of bin `bin` (x >> 20 == bin) with x >= cut: the largest
// key t such that the values >= t number (COUNT) or weigh (mass in units of
// the bin's power of two) at least `need`; need is at most what the bin
// holds there.  Two levels, bits [19:9] then [8:0]; every thread calls.
// The mass levels search suffix sums from the top, kept in md in plain
// bin order.
template <bool COUNT>
__device__ uint32_t lk_select(const uint32_t* keys, uint32_t n, uint32_t bin, uint32_t cut,
                              double need, uint32_t* hist, LkSmem& lm, double* wz) {
  const int tid = threadIdx.x, lane = lane_id(), wave = uwave();
  uint32_t s0 = 0u, s1 = 0u;
  for (int lev = 0; lev < 2; ++lev) {
    const uint32_t nb = lev == 0 ? 2048u : 512u;
    const uint32_t hsh = lev == 0 ? 20u : 9u;  // the bits above this level's field
    const uint32_t hval = lev == 0 ? bin : ((bin << 11) | s0);
    const uint32_t fsh = lev == 0 ? 9u : 0u;   // the field's shift
    for (uint32_t q = (uint32_t)tid; q < (uint32_t)kHistBins; q += kBlock) {
      if (COUNT) hist[H1::at(q)] = 0u;
      else lm.hm[q] = 0ull;
    }
    __syncthreads();
    for (uint32_t c = (uint32_t)tid; c < n; c += kBlock) {
      const uint32_t x = keys[c];
      if ((x >> hsh) != hval || x < cut) continue;
      const uint32_t q = (x >> fsh) & (nb - 1u);
      if (COUNT) atomicAdd(&hist[H1::at(q)], 1u);
      else atomicAdd(&lm.hm[q], (unsigned long long)stream::radix_sig(x));
    }
    __syncthreads();
    if (!COUNT) {
      // suffix sums from the top (thread t: sub-bins 2047 - 2t, 2046 - 2t),
      // integers below 2^53 and so exact in float64 whatever the order
      const uint32_t bh = (uint32_t)(kHistBins - 1 - 2 * tid), bl = bh - 1u;
      const double vh = (double)lm.hm[bh], vl = (double)lm.hm[bl];
      const double vin = wave_incl_scan(vh + vl);
      if (lane == kWave - 1) wz[wave] = vin;
      __syncthreads();
      double vw = 0.0;
      for (int w2 = 0; w2 < wave; ++w2) vw += wz[w2];
      const double top = vw + wave_excl_from_incl(vin) + vh;
      lm.md[bh] = top;
      lm.md[bl] = top + vl;
      __syncthreads();
    }
    // the largest sub-bin whose suffix (from the top) reaches need
    if (wave == 0) {
      uint32_t found;
      double above;
      if (COUNT) {
        uint32_t ac, tot;
        wave_find<kHistBins>(hist, (uint32_t)need, found, ac, tot);
        above = (double)ac;
      } else {
        // (with a positive suffix; if none reaches need, the lowest sub-bin
        // holding mass: the largest whose suffix is still the whole total)
        const double m0 = lm.md[(uint32_t)lane * 32u];
        const uint64_t m1 = __ballot(m0 >= need && m0 > 0.0);
        const double tgt = m1 != 0ull ? need : lm.md[0];
        const uint64_t mm = m1 != 0ull ? m1 : __ballot(m0 >= tgt);
        const uint32_t L = (uint32_t)last_lane(mm | 1ull);
        const double mb = lane < 32 ? lm.md[L * 32u + (uint32_t)lane] : 0.0;
        const uint64_t m2 = __ballot(lane < 32 && mb >= tgt && (m1 == 0ull || mb > 0.0));
        found = L * 32u + (uint32_t)last_lane(m2 | 1ull);
        above = found + 1u < (uint32_t)kHistBins ? lm.md[found + 1u] : 0.0;
      }
      if (lane == 0) {
        lm.res[7] = found;
        lm.resd[3] = above;
      }
    }
    __syncthreads();
    if (lev == 0) s0 = lm.res[7];
    else s1 = lm.res[7];
    need -= lm.resd[3];
    __syncthreads();
  }
  return (bin << 20) | (s0 << 9) | s1;
}

// The merge's part.  Every thread calls; returns kFallback when the gather
// would overflow.
template <int OP>
__device__ __forceinline__ int large_k_merge(const SampleParams& P, const SplitParams& S,
                                             SplitSmem& sm, int i) {
  const int W = S.W, li = i - S.out0;
  const int row = P.indices ? as_global(P.indices)[i] : i;
  const int k = P.top_k_arr ? as_global(P.top_k_arr)[i] : P.top_k;
  const float pp = OP == kOpTopK ? 0.0f : P.top_p_arr ? as_global(P.top_p_arr)[i] : P.top_p;
  const uint64_t seed = P.seed_arr ? as_global(P.seed_arr)[i] : P.seed;
  const uint64_t offset = P.offset_arr ? as_global(P.offset_arr)[i] : P.offset;
  const uint64_t sid = P.seed_arr ? 0ull : (uint64_t)i;
  const uint64_t* hbase = S.list + (int64_t)li * W * kListMax;
  constexpr bool kJoint = OP == kOpTopKTopPJoint;
  constexpr bool kTopPPart = OP == kOpTopKTopP || kJoint;
  const int tid = threadIdx.x, lane = lane_id(), wave = uwave();
  LkSmem& lm = sm.u.lm;
  uint32_t* keys = reinterpret_cast<uint32_t*>(sm.full);
  static_assert(sizeof(sm.full) >= (kLkGather + kWave) * 4, "gathered keys (+ dummies) fit full[]");
  // The row's histograms, thread t holding bins 2047 - 2t and 2046 - 2t:
  // the exact integer masses into hm, then (one block scan from the top)
  // suffix counts C[b] (values in bins >= b, C[2048] = 0, in full[]) and
  // suffix masses M[b] (float64, fixed association, in md), so that every
  // decision below is a lookup or a two-step ballot search.
  uint32_t* sc = keys;  // [kHistBins + 1], free until the row pass
  {
    const uint32_t bh = (uint32_t)(kHistBins - 1 - 2 * tid), bl = bh - 1u;
    unsigned long long mh = 0ull, ml = 0ull;
    uint32_t ch = 0u, cl = 0u;
    for (int q = 0; q < W; ++q) {
      const gptr<const uint64_t> h = as_global(hbase + (size_t)q * kListMax);
      const gptr<const uint32_t> hc = (gptr<const uint32_t>)(h + kHistBins);
      mh += __hip_atomic_load(h + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ml += __hip_atomic_load(h + bl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ch += __hip_atomic_load(hc + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      cl += __hip_atomic_load(hc + bl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    lm.hm[bh] = mh;
    lm.hm[bl] = ml;
    const double dh = ldexp((double)mh, (int)max(bh >> 3, 1u) - 150);
    const double dl = ldexp((double)ml, (int)max(bl >> 3, 1u) - 150);
    const uint32_t cp = ch + cl;
    const double dp = dh + dl;
    const uint32_t cin = wave_incl_scan(cp);
    const double din = wave_incl_scan(dp);
    if (lane == kWave - 1) {
      sm.wcnt[wave] = cin;
      sm.wz[wave] = din;
    }
    __syncthreads();
    uint32_t cw = 0u;
    double dw = 0.0;
    for (int w2 = 0; w2 < wave; ++w2) {
      cw += sm.wcnt[w2];
      dw += sm.wz[w2];
    }
    const uint32_t cex = cw + cin - cp;
    const double mtop = (dw + wave_excl_from_incl(din)) + dh;
    sc[bh] = cex + ch;
    sc[bl] = cex + cp;
    lm.md[bh] = mtop;
    lm.md[bl] = mtop + dl;
    if (tid == 0) {
      sc[kHistBins] = 0u;
      lm.nlist = 0u;
    }
  }
  __syncthreads();
  const float pc = stream::clamp01(pp);
  // M[b], with M[2048] = 0
  auto msuf = [&](uint32_t b) { return b < (uint32_t)kHistBins ? lm.md[b] : 0.0; };
  // the largest bin b >= lo whose suffix mass reaches need (and is positive);
  // without one, the lowest bin holding mass.  One wave.
  auto mfind = [&](double need, uint32_t lo) -> uint32_t {
    const uint32_t c0 = max((uint32_t)lane * 32u, lo);
    const double m0 = c0 < (uint32_t)kHistBins ? lm.md[c0] : 0.0;
    const uint64_t m1 = __ballot((uint32_t)lane * 32u + 31u >= lo && m0 >= need && m0 > 0.0);
    if (m1 != 0ull) {
      const uint32_t L = (uint32_t)last_lane(m1);
      const uint32_t b = L * 32u + (uint32_t)lane;
      const double mb = lane < 32 ? lm.md[b] : 0.0;
      const uint64_t m2 = __ballot(lane < 32 && b >= lo && mb >= need && mb > 0.0);
      return L * 32u + (uint32_t)last_lane(m2);
    }
    // lowest bin with mass: bin 0 if it holds some, else the lowest
    // non-empty bin above it (every value there is positive)
    if (lm.hm[0] > 0ull) return 0u;
    const uint32_t need_c = sc[1];
    const uint64_t n1 = __ballot(sc[(uint32_t)lane * 32u] >= need_c);
    const uint32_t L = (uint32_t)last_lane(n1);
    const uint64_t n2 = __ballot(lane < 32 && sc[L * 32u + (uint32_t)lane] >= need_c);
    return max(L * 32u + (uint32_t)last_lane(n2), 1u);
  };
  if (wave == 0) {
    const uint32_t total = sc[0];
    const bool all = total < (uint32_t)k;  // every value kept by top-k
    // b_k: the largest bin whose suffix count reaches k
    uint32_t bk = 0u;
    if (!all) {
      const uint64_t m1 = __ballot(sc[(uint32_t)lane * 32u] >= (uint32_t)k);
      const uint32_t L = (uint32_t)last_lane(m1);
      const uint64_t m2 = __ballot(lane < 32 && sc[L * 32u + (uint32_t)lane] >= (uint32_t)k);
      bk = L * 32u + (uint32_t)last_lane(m2);
    }
    const uint32_t above = sc[bk + 1u];
    // masses above b_k (the top-k set's certain part), of b_k (exact), of the row
    const double mab = msuf(bk + 1u), mtot = msuf(0u);
    const double mbk = ldexp((double)lm.hm[bk], (int)max(bk >> 3, 1u) - 150);
    // the bins the top-p cut can fall in, [plo, phi]
    uint32_t plo = bk, phi = bk;
    if (kTopPPart) {
      if (kJoint || all) {
        plo = phi = mfind((double)pc * mtot, 0u);
      } else {
        // the top-k set's mass Z_k lies in [mab, mab + mbk]; a target the
        // bins above b_k reach falls above b_k, any other in b_k
        const double tlo = (double)pc * mab, thi = (double)pc * (mab + mbk);
        phi = tlo <= mab && mab > 0.0 ? max(mfind(tlo, bk + 1u), bk) : bk;
        plo = thi <= mab && mab > 0.0 ? max(mfind(thi, bk + 1u), bk) : bk;
      }
    }
    // keys to gather: bin b_k (unless every value is kept) and [plo, phi]
    const uint32_t n = (sc[plo] - sc[phi + 1u]) +
                       (!all && (bk < plo || bk > phi) ? sc[bk] - sc[bk + 1u] : 0u);
    if (lane == 0) {
      lm.res[0] = bk;
      lm.res[1] = above;
      lm.res[2] = all ? 1u : 0u;
      lm.res[3] = plo;
      lm.res[4] = phi;
      lm.res[5] = n;
      lm.resd[0] = mab;
      lm.resd[1] = mtot;
    }
  }
  __syncthreads();
  const uint32_t bk = lm.res[0], above = lm.res[1], plo = lm.res[3], phi = lm.res[4];
  const bool all = lm.res[2] != 0u;
  if (lm.res[5] > kLkGather) return kFallback;  // block-uniform
  // One pass over the row, a wave per tile of 2048 values (eight 16-byte
  // loads per lane).  The keys of the gathered bins go to keys[], each tile's in
  // one block (lane order); the values above every gathered bin are kept
  // whatever tau turns out to be (tau lies in a gathered bin), so their mass
  // per tile is summed now (values below the gathered bins are below tau
  // and never kept).
  const stream::RowRef r{as_global(P.probs + (int64_t)row * P.vocab), P.vocab, P.vec_ok != 0};
  const int n_tiles = (P.vocab + stream::kTile - 1) / stream::kTile;
  const uint32_t gtop = all ? phi : max(phi, bk);     // the highest gathered bin
  const uint32_t cert = ((gtop + 1u) << 20) - 1u;     // keys above: kept
  // gathered: keys in [lo1, lo1 + w1) (bins plo..phi) or [lo2, lo2 + w2) (bin b_k)
  const uint32_t lo1 = plo << 20, w1 = (phi - plo + 1u) << 20;
  const uint32_t lo2 = bk << 20, w2 = all ? 0u : 1u << 20;
  constexpr int kC = stream::kTileChunks;
  auto tile_load = [&](int t, float (&vt)[kC][4]) {
    const int64_t tb = (int64_t)t * stream::kTile;
    stream::load4_batch<kC, false>(r, [&](int q) { return tb + q * (kWave * 4) + lane * 4; }, vt);
  };
  auto tile_take = [&](int t, const float (&vt)[kC][4]) {
    // value e of load q is inside the row when q * 256 + e < lim
    const int lim = min(P.vocab - t * stream::kTile, stream::kTile) - lane * 4;
    double cs = 0.0;
    uint32_t cnt = 0u, gm = 0u;  // bit 4q + e: value e of load q is gathered
#pragma unroll
    for (int q = 0; q < kC; ++q) {
      float gs = 0.0f;  // a group's kept values in float32, then added in float64
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = bits_of(vt[q][e]);
        const bool in = q * (kWave * 4) + e < lim;
        const bool g = in && (x - lo1 < w1 || x - lo2 < w2);
        gs += (in && x > cert) ? vt[q][e] : 0.0f;
        gm |= g ? 1u << (4 * q + e) : 0u;
        cnt += g ? 1u : 0u;
      }
      cs += (double)gs;
    }
    cs = wave_sum(cs);
    const uint32_t incl = wave_incl_scan(cnt);
    const uint32_t tot = lane63(incl);
    uint32_t base = 0u;
    if (lane == kWave - 1 && tot > 0u) base = atomicAdd(&lm.nlist, tot);
    base = lane_value(base, kWave - 1);
    // every value stored, the others into this lane's dummy slot past the
    // keys (the gathered ones number exactly n <= kLkGather, counted by the
    // histograms, so their positions stay below kLkGather)
    uint32_t pos = base + incl - cnt;
#pragma unroll
    for (int q = 0; q < kC; ++q) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool g = (gm >> (4 * q + e)) & 1u;
        keys[min(g ? pos : kLkGather + (uint32_t)lane, kLkGather + (uint32_t)lane)] =
            bits_of(vt[q][e]);
        pos += g ? 1u : 0u;
      }
    }
    if (lane == 0) {
      lm.s.tm[1][t] = cs;
      lm.tst[t] = base;
      lm.tcn[t] = tot;
    }
  };
  for (int t = wave; t < n_tiles; t += kWaves) {  // wave-uniform
    float vt[kC][4];
    tile_load(t, vt);
    tile_take(t, vt);
  }
  __syncthreads();
  const uint32_t n = min(lm.nlist, kLkGather);
  // tau_k: the (k - above)-th largest key of bin b_k
  const uint32_t tk = all ? 0u : lk_select<true>(keys, n, bk, 0u, (double)((uint32_t)k - above),
                                                 sm.hist, lm, sm.wz);
  // Z_k: the bins above b_k, then b_k's values >= tau_k (exact integer
  // significand sums, below 2^53, so their float64 sum is exact)
  double sk = 0.0;
  for (uint32_t c = (uint32_t)tid; c < n; c += kBlock) {
    const uint32_t x = keys[c];
    sk += (!all && (x >> 20) == bk && x >= tk) ? (double)stream::radix_sig(x) : 0.0;
  }
  sk = wave_sum(sk);
  if (lane == 0) sm.wz[wave] = sk;
  __syncthreads();
  if (tid == 0) {
    double z = 0.0;
    for (int w = 0; w < kWaves; ++w) z += sm.wz[w];
    lm.resd[2] = all ? lm.resd[1] : lm.resd[0] + ldexp(z, (int)max(bk >> 3, 1u) - 150);
  }
  __syncthreads();
  const double zk = lm.resd[2];
  uint32_t tau = max(tk, 1u);  // zeros carry no mass
  if (kTopPPart) {
    // the cut: the smallest prefix (descending) whose mass reaches p * Z
    // (Z_k, or the row's mass for the joint order).  Its bin: the bins
    // above b_k count fully, b_k with its values >= tau_k (top-k first)
    const double target = (double)pc * (kJoint ? lm.resd[1] : zk);
    if (wave == 0) {
      // (top-k first: the bins above b_k count fully, b_k with its values
      // >= tau_k, so a target beyond the bins above b_k falls in b_k)
      uint32_t bp;
      double ab;
      const double mab = lm.resd[0];
      if (!kJoint && !all) {
        bp = target <= mab && mab > 0.0 ? max(mfind(target, bk + 1u), bk) : bk;
      } else {
        bp = mfind(target, 0u);
      }
      ab = bp == bk && !kJoint && !all ? mab : msuf(bp + 1u);
      if (lane == 0) {
        lm.res[6] = bp;
        lm.resd[3] = ab;
      }
    }
    __syncthreads();
    const uint32_t bp = lm.res[6];
    const double ab = lm.resd[3];
    // inside bin b_p (gathered: b_p lies in [plo, phi] or is b_k), by mass
    // in units of the bin's power of two
    const double unit = ldexp(1.0, (int)max(bp >> 3, 1u) - 150);
    const double need = max((target - ab) / unit, 0.0);
    const uint32_t tp = (bp >= plo && bp <= phi) || (!all && bp == bk)
                            ? lk_select<false>(keys, n, bp, (!kJoint && bp == bk) ? tk : 0u, need,
                                               sm.hist, lm, sm.wz)
                            : tk;
    tau = max(tau, tp);
  }
  // the kept mass of every tile: the part above the gathered bins, plus the
  // tile's gathered values >= tau (lane order inside the tile's block, fixed
  // association), then one draw (rounds = 1: the blog's loop started just
  // below tau, where every draw is accepted)
  const float low = __uint_as_float(tau - 1u);
  for (int t = wave; t < n_tiles; t += kWaves) {
    const uint32_t t0 = lm.tst[t], tn = lm.tcn[t];
    double us = 0.0;
    for (uint32_t j = (uint32_t)lane; j < tn; j += kWave) {
      const uint32_t x = keys[min(t0 + j, kLkGather - 1u)];
      us += x >= tau ? (double)__uint_as_float(x) : 0.0;
    }
    us = wave_sum(us);
    if (lane == 0) lm.s.tm[0][t] = lm.s.tm[1][t] + us;
  }
  __syncthreads();
  if (wave == 0) {
    const double z = stream::tile_scan_total(lm.s.tm[0], n_tiles);
    if (lane == 0) lm.s.bc_d[0] = z * draw_uniform(seed, offset, sid, 0u);
  }
  __syncthreads();
  const double T = lm.s.bc_d[0];
  __syncthreads();
  const int tok = stream::locate(r, lm.s.tm[0], n_tiles, T, low, lm.s);
  if (threadIdx.x == 0) stream::write_sample(P, i, tok, tok >= 0 ? 1 : 0);
  return kDone;
}

// A finishing work-group (see SplitParams::fin).  Every work-group of the
// slices comes before it in the grid and the dispatcher starts work-groups
// in grid order, so the slices it waits for are running or done and the
// wait ends; it is bounded all the same (S.spin), and a finisher that gives
// up samples the output with the exact streaming passes instead.  Either
// way it takes the output's W arrivals off the counter and advances the
// generation, so the counter is back at zero once every slice has arrived
// (before the next launch on the stream starts).
template <int OP>
__device__ __forceinline__ int large_k_finish(const SampleParams& P, const SplitParams& S,
                                              SplitSmem& sm, int& out_i) {
  constexpr bool kTopPPart = OP == kOpTopKTopP || OP == kOpTopKTopPJoint;
  const int W = S.W;
  const int b = (int)blockIdx.x - S.nsb, xcd = b & 7, li = (b >> 3) * 8 + xcd;
  if (li >= S.n_out) return kDone;
  const int i = S.out0 + li;
  out_i = i;
  const int lane = lane_id(), wave = uwave();
  const int row = P.indices ? as_global(P.indices)[i] : i;
  const bool row_ok = row >= 0 && row < P.rows;
  const int k = as_global(P.top_k_arr)[i];
  const float pp = kTopPPart ? (P.top_p_arr ? as_global(P.top_p_arr)[i] : P.top_p) : 0.0f;
  // the slices' own test: any other output was answered by its slices
  if (!(k > kSplitKCap && row_ok && !(kTopPPart && isnan(pp)))) return kDone;
  const gptr<uint32_t> ctr = as_global(S.ctr + li);
  if (threadIdx.x == 0) {
    int ok = 0;
    if (S.spin != 0ull) {  // (a limit of zero, a test setting, gives up at once)
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (true) {
        const uint32_t c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int32_t)c >= W) {
          ok = 1;
          break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 >= S.spin) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    sm.flag = ok;
  }
  __syncthreads();
  const bool arrived = sm.flag != 0;
  if (wave == 0) {
    // the headers (each written before its slice arrived)
    const gptr<uint32_t> h = as_global(S.hdr + ((int64_t)li * W + (lane & (W - 1))) * kHdrWords);
    const bool mine = arrived && lane < W;
    const uint32_t hc = mine ? __hip_atomic_load(h + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    const uint32_t hg = mine ? __hip_atomic_load(h + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    const uint32_t hx = mine ? __hip_atomic_load(h + 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    const uint32_t hb = mine ? __hip_atomic_load(h + 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    const uint32_t mygen = __hip_atomic_load(as_global(S.gen + li), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool foreign =
        __ballot(mine && (hg != mygen || hx != xcc_id() || hc != kLargeList)) != 0ull ||
        S.test_foreign != 0;
    const bool anybad = __ballot(mine && hb != 0u) != 0ull;
    if (lane == 0) {
      __hip_atomic_fetch_sub(ctr, (uint32_t)W, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(as_global(S.gen + li), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.res[0] = !arrived || foreign ? 2u : anybad ? 1u : 0u;
    }
  }
  __syncthreads();
  const uint32_t st = sm.res[0];
  __syncthreads();
  if (st == 1u) {
    if (threadIdx.x == 0) stream::write_sample(P, i, -1, 0);
    return kDone;
  }
  return st == 0u ? kLargeKMerge : kFallback;
}

template <int KIND, int OP, int NV>
__device__ __forceinline__ int split_sample(const SampleParams& P, const SplitParams& S,
                                           const SelectParams& Q, SplitSmem& sm, int& out_i) {
  // sampling from logits (softmax fused)
  constexpr bool kLogits = KIND == kKindLogits;
  constexpr bool kSampling = KIND == kKindSample || kLogits;
  // logits, and any values to select from: signed-order keys
  constexpr bool KEYS = KIND == kKindMask || KIND == kKindSelect || kLogits;
  // top-k-then-top-p sampling keeps a mass histogram for the loop's start
  constexpr bool kJoint = OP == kOpTopKTopPJoint;
  static_assert(!(kLogits && kJoint), "the joint order needs every probability's mass");
  constexpr bool kTopPPart = OP == kOpTopKTopP || kJoint;
  constexpr bool kMass = kSampling && kTopPPart;
  static_assert(kMassBins + kWave <= kBlock, "one clearing store per thread");
  constexpr uint32_t kSh = KEYS ? 21u : 20u;  // top eleven bits of a key
  const int W = S.W;
  const int b = blockIdx.x, xcd = b & 7, local = b >> 3;
  const int li = (local / W) * 8 + xcd;  // the W slices of an output share b % 8
  // The dispatcher hands an XCD's work-groups to its shader engines in turn
  // and waits, in order, for a compute unit of the engine whose turn it is.
  // Without the rotation slice s of every output would land on engine s % 4,
  // and the long-running last arrivers (often the same slice index) would
  // fill one engine while the others idle and every later work-group waits.
  const int s = (local % W + local / W) % W;
  if (li >= S.n_out) return kDone;
  const int i = S.out0 + li;
  out_i = i;
  const int tid = threadIdx.x, lane = lane_id(), wave = uwave();

  const int row = P.indices ? as_global(P.indices)[i] : i;
  const bool row_ok = row >= 0 && row < P.rows;

  // ---- phase A: one HBM read of the slice into registers --------------------
  // The loads go out before anything else is read (they depend on the row
  // only).  They are unconditional (a thread past the end re-reads the last
  // vector and ignores it) so that they sit in one basic block and every
  // later use waits only for its own vector, not for the whole slice.
  const int V = P.vocab;
  const int s0 = s * S.L;
  const int s1 = min(s0 + S.L, V);
  const int nvec = (s1 - s0) / 4;
  const gptr<const float4> src = as_global(
      reinterpret_cast<const float4*>(P.probs + (int64_t)(row_ok ? row : 0) * V + s0));
  // Only kInFlight loads per thread go out now; each later one leaves as an
  // earlier vector is processed.  A wave stalls while the CU cannot accept
  // another load, so issuing all of them at once would leave every wave
  // stuck at its last load until most of the slice had landed.
  constexpr int kInFlight = NV < kDepth ? NV : kDepth;
  float4 v[NV];
  // (a row that a second kernel reads again, renormalisation and masking,
  // stays cacheable; every other kind reads it once: non-temporal)
  constexpr bool kOnce = KIND == kKindSample || KIND == kKindSelect || kLogits;
  auto issue = [&](int j) {
    const gptr<const float4> a = src + min(tid + j * kBlock, nvec - 1);
    v[j] = kOnce ? load_f4_nt(a) : load_f4(a);
  };

  // The output's parameters go out first, as vector loads from always-valid
  // addresses (the probabilities stand in for an absent array): a scalar
  // load would be waited for by the first work-group barrier (its counter
  // also covers LDS traffic), and under the slice reads its answer takes
  // microseconds, during which no further slice load could leave.  A vector
  // load is waited for only where its value is used, and loads return in
  // order, so these arrive before the first slice vector does.
  const int k_raw = vload(P.top_k_arr ? P.top_k_arr + i : reinterpret_cast<const int*>(P.probs));
  const float pp_raw =
      vload(P.top_p_arr ? P.top_p_arr + i : reinterpret_cast<const float*>(P.probs));
  const uint64_t seed_raw =
      vload(P.seed_arr ? P.seed_arr + i : reinterpret_cast<const uint64_t*>(P.probs));
  const uint64_t off_raw =
      vload(P.offset_arr ? P.offset_arr + i : reinterpret_cast<const uint64_t*>(P.probs));
  const float t_raw = kLogits ? vload(P.temp_arr ? P.temp_arr + (row_ok ? row : 0)
                                                 : reinterpret_cast<const float*>(P.probs))
                              : 1.0f;
#pragma unroll
  for (int j = 0; j < kInFlight; ++j) issue(j);
  const int k = P.top_k_arr ? k_raw : P.top_k;
  const float pp = kTopPPart ? (P.top_p_arr ? pp_raw : P.top_p) : 0.0f;
  const uint64_t seed = !kSampling ? 0ull : P.seed_arr ? seed_raw : P.seed;
  const uint64_t offset = !kSampling ? 0ull : P.offset_arr ? off_raw : P.offset;
  // logits: the temperature, and its inverse as the oracle of the softmax
  // takes it (t = (z - m) * (1 / T) in float64)
  const float temp = kLogits ? (P.temp_arr ? t_raw : P.temp) : 1.0f;
  const double itemp = kLogits ? 1.0 / (double)temp : 1.0;

  // ---- large k: histograms instead of candidate lists (see large_k_merge).
  // Decided as soon as the parameters arrive, before the landing loop, so
  // that this path and the candidate path never hold their registers at once.
  constexpr bool kLargeK = KIND == kKindSample &&
                           (OP == kOpTopK || OP == kOpTopKTopP || OP == kOpTopKTopPJoint);
  if (kLargeK && W > 1 && k > kSplitKCap && row_ok && !(kTopPPart && isnan(pp))) {
    auto& lk = sm.u.lk;
    for (int q = tid; q < kHistBins; q += kBlock) lk.cm[0][q] = lk.cm[1][q] = 0ull;
    uint32_t gen = 0u;
    if (wave == 0 && lane == 0)
      gen = __hip_atomic_load(as_global(S.gen + li), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int cp = lane & 1;
    uint32_t mx = 0u;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (j + kInFlight < NV) {
        __builtin_amdgcn_sched_barrier(0);
        issue(j + kInFlight);
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool in = tid + j * kBlock < nvec;
      // one vector at a time (the compiler would otherwise work ahead on
      // all of them and run out of registers)
      float4 x = v[j];
      asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
      const uint32_t k4[4] = {bits_of(x.x), bits_of(x.y), bits_of(x.z), bits_of(x.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!in) continue;
        mx = max(mx, k4[e]);
        const uint32_t b = min(k4[e] >> 20, (uint32_t)(kHistBins - 1));
        atomicAdd(&lk.cm[cp][b], (1ull << kLkCountShift) | stream::radix_sig(k4[e]));
      }
    }
    mx = wave_max(mx);
    if (lane == 0) sm.wmax[wave] = mx;
    __syncthreads();
    const gptr<uint64_t> dst = as_global(S.list + ((int64_t)li * W + s) * kListMax);
    for (int q = tid; q < kHistBins; q += kBlock) {
      const unsigned long long a = lk.cm[0][q], c = lk.cm[1][q];
      constexpr unsigned long long kM = (1ull << kLkCountShift) - 1ull;
      dst[q] = (a & kM) + (c & kM);
      ((gptr<uint32_t>)(dst + kHistBins))[q] = (uint32_t)((a >> kLkCountShift) + (c >> kLkCountShift));
    }
    if (tid == 0) {
      uint32_t smax = 0u;
      for (int w = 0; w < kWaves; ++w) smax = max(smax, sm.wmax[w]);
      const gptr<uint32_t> h = as_global(S.hdr + ((int64_t)li * W + s) * kHdrWords);
      h[0] = 0u;
      h[1] = kLargeList;
      h[2] = smax;
      h[3] = gen;
      h[4] = xcc_id();
      h[5] = smax >= 0x7F800000u ? 1u : 0u;  // a sign bit, an inf or a NaN
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (S.fin) {  // the output's finishing work-group merges
      if (tid == 0)
        __hip_atomic_fetch_add(as_global(S.ctr + li), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return kDone;
    }
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(as_global(S.ctr + li), 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      sm.flag = (old == (uint32_t)(W - 1));
    }
    __syncthreads();
    if (!sm.flag) return kDone;
    // the last slice: the headers (all written before their arrivals)
    if (wave == 0) {
      const gptr<uint32_t> h = as_global(S.hdr + ((int64_t)li * W + (lane & (W - 1))) * kHdrWords);
      const uint32_t hc = __hip_atomic_load(h + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t hg = __hip_atomic_load(h + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t hx = __hip_atomic_load(h + 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t hb = __hip_atomic_load(h + 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool mine = lane < W;
      const uint32_t mygen = (uint32_t)__builtin_amdgcn_readfirstlane((int)gen);
      const bool foreign =
          __ballot(mine && (hg != mygen || hx != xcc_id() || hc != kLargeList)) != 0ull ||
          S.test_foreign != 0;
      const bool anybad = __ballot(mine && hb != 0u) != 0ull;
      if (lane == 0) {
        __hip_atomic_store(as_global(S.ctr + li), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(as_global(S.gen + li), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.res[0] = foreign ? 2u : anybad ? 1u : 0u;
      }
    }
    __syncthreads();
    if (sm.res[0] == 1u) {
      split_invalid<KIND>(P, S, Q, i, li);
      return kDone;
    }
    if (sm.res[0] == 2u) return kFallback;
    return kLargeKMerge;
  }

  // while the slice is in flight: clear the histogram; wave 0 reads the
  // row's generation (used only when the slice publishes).  Nothing here
  // waits for a global load: the barrier below would otherwise hold back
  // every later load of the slice.  The draws of the output's stream are
  // computed by the work-group that runs the loop, while its list reads are
  // in flight (fill_draws).
  clear_hist<kHistBins>(sm.hist, tid, kBlock);
  const uint64_t sid = P.seed_arr ? 0ull : (uint64_t)i;
  uint32_t gen = 0u;
  if (wave == 0 && W > 1 && lane == 0)
    gen = __hip_atomic_load(as_global(S.gen + li), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the first 256 draws of the output's stream into sm.draws (one wave)
  auto fill_draws = [&]() {
    const Philox4x64 ph = philox4x64_10(offset, sid, (uint64_t)lane, 0ull, seed, 0ull);
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.draws[4 * lane + e] = (double)(ph.w[e] >> 11) * 0x1p-53;
  };
  __syncthreads();
  DSS_STAMP(1);

  // As each vector lands: its maximum (float32 bits) counted in the
  // histogram of bits [30:20] (bin 2047 also takes the patterns with the sign
  // bit set), and its staging key, the maximum + 1, or 0 for a thread past
  // the end.  A lane past the end counts into a padding word of the
  // histogram that no search reads.
  //
  // The first J0 slots of every thread (about 30% of the slice) are a
  // sample: once they are counted, wave 0 takes from the histogram a
  // provisional bound tp, the edge of the bin holding the r-th largest
  // sample maximum, r well above the sample's expected share of k.  From then
  // on every vector with a value >= tp is staged in LDS as it lands, in its
  // wave's region at a position taken from ballots, so that the staging
  // stores fall inside the landing window.  After the last vector, if
  // tp <= bnd and no region overflowed, the staged vectors include every
  // vector with a value >= bnd; otherwise the slice stages again from its
  // registers with bnd itself (the general path).
  constexpr int J0 = NV >= 4 ? (3 * NV + 5) / 10 : 0;
  const uint32_t pad = (uint32_t)lane * H1::kStride + H1::kChunk;
  uint32_t key[NV];
  uint32_t mx = 0u;
  bool nan_seen = false;  // logits: a NaN invalidates the row
  double zsum = 0.0;      // joint order: this thread's values, summed in a fixed order
  auto count = [&](int j) {
    const bool in = tid + j * kBlock < nvec;
    if constexpr (kJoint)
      zsum += in ? ((double)v[j].x + (double)v[j].y) + ((double)v[j].z + (double)v[j].w) : 0.0;
    const uint32_t m = max4_key<KEYS>(v[j]);
    key[j] = in ? m + 1u : 0u;
    mx = max(mx, in ? m : 0u);
    atomicAdd(&sm.hist[in ? H1::at(min(m >> kSh, (uint32_t)(kHistBins - 1))) : pad], 1u);
    if (KEYS)
      nan_seen = nan_seen || (in && (isnan(v[j].x) || isnan(v[j].y) || isnan(v[j].z) || isnan(v[j].w)));
  };
  uint32_t tp = 0xFFFFFFFFu;
  uint32_t wp = 0u;  // vectors this wave has staged (wave-uniform)
  bool wovf = false;
  auto stage = [&](int j) {
    const bool hit = key[j] > tp;
    const uint64_t hm = __ballot(hit);
    const uint32_t c = (uint32_t)__popcll(hm);
    if (wp + c <= (uint32_t)kRegion) {
      if (hit) {
        const uint32_t slot = (uint32_t)(wave * kRegion) + wp + rank_in(hm);
        sm.u.a.vec[slot] = v[j];
        sm.u.a.vidx[slot] = (uint32_t)(tid + j * kBlock);
      }
    } else {
      wovf = true;
    }
    wp += c;
  };
  auto next = [&](int j) {  // the load that takes slot j's place in flight
    if (j + kInFlight < NV) {
      __builtin_amdgcn_sched_barrier(0);
      issue(j + kInFlight);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
#pragma unroll
  for (int j = 0; j < J0; ++j) {
    count(j);
    next(j);
  }
  if (J0 > 0) {
    __syncthreads();
    if (wave == 0) {
      const float fk = (float)k * ((float)J0 / (float)NV);
      const uint32_t r = (uint32_t)(fk + 3.0f * __builtin_sqrtf(fk) + 2.0f);
      uint32_t bin, above, total;
      wave_find<kHistBins>(sm.hist, r, bin, above, total);
      if (lane == 0) sm.tp = total < r ? 0u : bin << kSh;
    }
    __syncthreads();
    DSS_STAMP(2);
    tp = sm.tp;
#pragma unroll
    for (int j = 0; j < J0; ++j) stage(j);
  }
#pragma unroll
  for (int j = J0; j < NV; ++j) {
    count(j);
    next(j);
    if (J0 > 0) stage(j);
  }
  mx = wave_max(mx);
  if (lane == 0) {
    sm.wmax[wave] = mx;
    sm.wcnt[wave] = wovf ? 0xFFFFFFFFu : wp;
  }
  if constexpr (kJoint) {
    const double wz = wave_sum(zsum);
    if (lane == 0) sm.wz[wave] = wz;
  }
  if (KEYS) {
    const bool wn = __ballot(nan_seen) != 0ull;
    if (lane == 0) sm.wnan[wave] = wn ? 1u : 0u;
  }
  DSS_STAMP(3);
  // the parameters' checks, once the slice has landed (every slice of the
  // output decides alike)
  const bool ok = row_ok && k > 0 && (!kTopPPart || !isnan(pp)) &&
                  (!kLogits || (temp > 0.0f && temp != __builtin_inff()));
  if (!ok || k > kSplitKCap) {
    // no hand-off for this output: slice 0 answers alone
    if (s != 0) return kDone;
    if (!ok) {
      split_invalid<KIND>(P, S, Q, i, li);
      return kDone;
    }
    return kFallback;
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t bin, above, total, nbin;
    wave_find<kHistBins>(sm.hist, (uint32_t)k, bin, above, total, &nbin);
    const uint32_t smax = wave_max(lane < kWaves ? sm.wmax[lane] : 0u);
    const bool anynan = KEYS && __ballot(lane < kWaves && sm.wnan[lane] != 0u) != 0ull;
    const uint32_t bnd = total < (uint32_t)k ? 0u : bin << kSh;  // fewer than k vectors: all of it
    const bool ovf = __ballot(lane < kWaves && sm.wcnt[lane] == 0xFFFFFFFFu) != 0ull;
    if (lane == 0) {
      sm.res[0] = bnd;
      sm.res[1] = smax;
      sm.res[2] = anynan ? 1u : 0u;
      sm.res[3] = (J0 > 0 && tp <= bnd && !ovf) ? 1u : 0u;
      sm.res[4] = bin;
      sm.res[5] = above;
      sm.res[6] = nbin;
      // refine the bound (below) when its bin holds far more vectors than needed
      sm.res[7] = (bnd > 0u && bin < (uint32_t)(kHistBins - 1) &&
                   above + nbin > max(2u * (uint32_t)k, (uint32_t)k + 1024u)) ? 1u : 0u;
      if (kJoint) {
        double z = 0.0;
        for (int w = 0; w < kWaves; ++w) z += sm.wz[w];
        sm.zs = z;
      }
    }
  }
  __syncthreads();
  // A bin holding far more vectors than the bound needs (flat rows, whose
  // values share a few bins): histograms of the next bits of the vector
  // maxima inside that bin (eleven, then the rest) narrow the bound the same
  // certified way, so the slice publishes about k entries instead of most of
  // the slice.  Each level counts into the same LDS histogram.
  if (sm.res[7] != 0u) {  // block-uniform
    uint32_t pre = sm.res[4], ab = sm.res[5], nb = sm.res[6];
    uint32_t hsh = kSh;  // bits below the prefix
    const uint32_t limit = max(2u * (uint32_t)k, (uint32_t)k + 1024u);
#pragma unroll 1
    for (int lev = 0; lev < 2 && ab + nb > limit && hsh > 0u; ++lev) {  // block-uniform
      const uint32_t sh2 = hsh > 11u ? hsh - 11u : 0u;
      const uint32_t mask = (1u << (hsh - sh2)) - 1u;
      __syncthreads();
      clear_hist<kHistBins>(sm.hist, tid, kBlock);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const uint32_t m = key[j] - 1u;
        const bool hit = key[j] != 0u && (m >> hsh) == pre;
        atomicAdd(&sm.hist[hit ? H1::at((m >> sh2) & mask) : pad], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t bin2, above2, total2, nbin2;
        wave_find<kHistBins>(sm.hist, (uint32_t)k - ab, bin2, above2, total2, &nbin2);
        if (lane == 0) {
          const uint32_t p2 = (pre << (hsh - sh2)) | bin2;
          const uint32_t b = p2 << sh2;
          sm.res[0] = b;
          sm.res[3] = (sm.res[3] != 0u && tp <= b) ? 1u : 0u;
          sm.res[4] = p2;
          sm.res[5] = ab + above2;
          sm.res[6] = nbin2;
        }
      }
      __syncthreads();
      pre = sm.res[4];
      ab = sm.res[5];
      nb = sm.res[6];
      hsh = sh2;
    }
  }
  DSS_STAMP(4);
  const uint32_t bnd = sm.res[0];
  const uint32_t smax = sm.res[1];
  // probabilities: a sign bit, an inf or a NaN somewhere; logits: a NaN
  // (and, sampling from logits, a +inf)
  const bool bad = KEYS ? (sm.res[2] != 0u || (kLogits && smax == 0xFF800000u))
                        : smax >= 0x7F800000u;
  const bool fast = sm.res[3] != 0u;

  // The general path: the vectors with a value >= bnd (key > bnd), staged
  // in thread order, branch-free (stores to per-lane dummy slots).
  uint32_t nstage = 0u;
  bool stage_ok = !bad;
  if (!fast) {
    uint32_t nv_hit = 0u;
#pragma unroll
    for (int j = 0; j < NV; ++j) nv_hit += key[j] > bnd ? 1u : 0u;
    uint32_t pos = block_excl_scan(nv_hit, nstage, sm.red[0]);
    stage_ok = !bad && nstage <= (uint32_t)kStageMax;
    if (stage_ok) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const bool hit = key[j] > bnd;
        const uint32_t slot = hit ? pos : (uint32_t)(kStageMax + lane);
        sm.u.a.vec[slot] = v[j];
        sm.u.a.vidx[slot] = (uint32_t)(tid + j * kBlock);
        pos += hit ? 1u : 0u;
      }
    }
    __syncthreads();
  }

  // The staged vectors' positive elements >= bnd as (key | index << 32) into
  // full[] (the row's list when W == 1, a staging copy otherwise), in
  // (thread, slot, element) order.  Slot q of a thread is the q-th vector of
  // its wave's region (provisional bound) or staged vector tid + q * 1024.
  const uint32_t bthr = max(bnd, 1u);
  constexpr int kSt = kStageMax / kBlock;
  static_assert(kSt == kRegion / kWave, "three staging slots per thread either way");
  uint32_t xb[kSt][4];
  uint32_t sidx[kSt];
  uint32_t ne = 0u;
#pragma unroll
  for (int q = 0; q < kSt; ++q) {
    const uint32_t first = fast ? (uint32_t)(q * kWave) : (uint32_t)(q * kBlock);
    const uint32_t n = fast ? wp : nstage;
    xb[q][0] = xb[q][1] = xb[q][2] = xb[q][3] = 0u;
    sidx[q] = 0u;
    if (!stage_ok || first >= n) continue;  // wave-uniform
    const uint32_t g = fast ? (uint32_t)(lane + q * kWave) : (uint32_t)(tid + q * kBlock);
    const bool live = g < n;
    const uint32_t slot = !live ? (uint32_t)(kStageMax + lane)
                          : fast ? (uint32_t)(wave * kRegion) + g
                                 : g;
    const float4 x = sm.u.a.vec[slot];
    sidx[q] = sm.u.a.vidx[slot];
    xb[q][0] = live ? key_of<KEYS>(x.x) : 0u;
    xb[q][1] = live ? key_of<KEYS>(x.y) : 0u;
    xb[q][2] = live ? key_of<KEYS>(x.z) : 0u;
    xb[q][3] = live ? key_of<KEYS>(x.w) : 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) ne += xb[q][e] >= bthr ? 1u : 0u;
  }
  uint32_t nlist;
  uint32_t epos = block_excl_scan(ne, nlist, sm.red[1]);
  const bool publish = stage_ok && nlist <= (uint32_t)kListMax;
  if (publish) {
#pragma unroll
    for (int q = 0; q < kSt; ++q) {
      const uint32_t first = fast ? (uint32_t)(q * kWave) : (uint32_t)(q * kBlock);
      if (first >= (fast ? wp : nstage)) continue;  // wave-uniform
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool take = xb[q][e] >= bthr;
        const uint32_t slot = take ? epos : (uint32_t)(kRowCandMax + lane);
        sm.full[slot] = (uint64_t)xb[q][e] | ((uint64_t)(uint32_t)(s0 + 4 * sidx[q] + e) << 32);
        epos += take ? 1u : 0u;
      }
    }
  }
  __syncthreads();
  DSS_STAMP(6);

  uint32_t tstar, gmax, ntot;
  if (W == 1) {
    // the whole row is in this work-group: full[] holds its list
    // (logits: no finite value, the -inf key or below, is an invalid row)
    if (bad || smax == 0u || (kLogits && smax <= 0x007FFFFFu)) {
      split_invalid<KIND>(P, S, Q, i, li);
      return kDone;
    }
    if (!publish) return kFallback;
    clear_hist<kHistBins>(sm.hist, tid, kBlock);
    if (kMass && tid < kMassBins + kWave) sm.mh[tid] = 0u;
    if (kSampling && wave == 1) fill_draws();
    if (kLogits && wave == 2) sm.etab[lane] = exp2((double)lane * (1.0 / 64.0));
    __syncthreads();  // histogram clears, draws, table
    tstar = bnd;
    gmax = smax;
    ntot = nlist;
  } else {
    const gptr<uint64_t> dst = as_global(S.list + ((int64_t)li * W + s) * kListMax);
    if (publish) {
      for (uint32_t g = tid; g < nlist; g += kBlock) dst[g] = sm.full[g];
    }
    if (tid == 0) {
      const gptr<uint32_t> h = as_global(S.hdr + ((int64_t)li * W + s) * kHdrWords);
      h[0] = bnd;
      h[1] = publish ? nlist : kNoList;
      h[2] = smax;
      h[3] = gen;
      h[4] = xcc_id();
      h[5] = bad ? 1u : 0u;
      if (kJoint) {
        const uint64_t zb = (uint64_t)__double_as_longlong(sm.zs);
        h[6] = (uint32_t)zb;
        h[7] = (uint32_t)(zb >> 32);
      }
    }
    // hand-off: this work-group's stores reach the XCD's L2 before it arrives
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    DSS_STAMP(7);
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(as_global(S.ctr + li), 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      sm.flag = (old == (uint32_t)(W - 1));
    }
    __syncthreads();
    DSS_STAMP(8);
    if (!sm.flag) return kDone;

    // ---- phase B: the last slice work-group of the row ----------------------
    // Wave 0 reads the W headers (lane q: slice q).  At the same time every
    // thread loads, speculatively, a batch of positions of one slice's list:
    // the threads form W groups of 1024 / W, group q reading slice q, as far
    // as about twice this work-group's own count (lists of one row have
    // similar lengths); the headers then say which positions are real.
    const int gsz = kBlock >> S.wlog;
    const int sl = tid >> (10 - S.wlog);
    const int lt = tid & (gsz - 1);
    const gptr<uint64_t> lst = as_global(S.list + ((int64_t)li * W + sl) * kListMax);
    // positions [0, spec) of every list are loaded now (spec <= one batch).
    // Wave 0's header reads go out first (a wave's loads return in order),
    // then every thread's list reads.  All reads are unconditional, at
    // clamped addresses, so that they leave back to back and no wait for
    // one of them sits inside a branch; what they return is masked later.
    const uint32_t spec = min((uint32_t)(kLoadBatch * gsz), 2u * (publish ? nlist : 0u) + 128u);
    const bool mine = wave == 0 && lane < W;
    uint32_t ht = 0u, hc = 0u, hm = 0u, hg = 0u, hx = 0u, hb = 0u, hz0 = 0u, hz1 = 0u;
    if (wave == 0) {
      const gptr<uint32_t> h =
          as_global(S.hdr + ((int64_t)li * W + (lane & (W - 1))) * kHdrWords);
      ht = __hip_atomic_load(h + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      hc = __hip_atomic_load(h + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      hm = __hip_atomic_load(h + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      hg = __hip_atomic_load(h + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      hx = __hip_atomic_load(h + 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      hb = __hip_atomic_load(h + 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (kJoint) {
        hz0 = __hip_atomic_load(h + 6, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hz1 = __hip_atomic_load(h + 7, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    uint64_t e8[kLoadBatch];
#pragma unroll
    for (int q = 0; q < kLoadBatch; ++q)
      e8[q] = __hip_atomic_load(lst + min((uint32_t)(lt + q * gsz), spec - 1u), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
    // while those reads are in flight, one wave computes the output's draws
    if (kSampling && wave == 1) fill_draws();
    if (kLogits && wave == 2) sm.etab[lane] = exp2((double)lane * (1.0 / 64.0));
    if (wave == 0) {
      const uint32_t me = xcc_id();
      const uint32_t mygen = (uint32_t)__builtin_amdgcn_readfirstlane((int)gen);
      if (lane == 0) {
        __hip_atomic_store(as_global(S.ctr + li), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(as_global(S.gen + li), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const bool anybad = __ballot(mine && hb != 0u) != 0ull;
      const bool foreign = __ballot(mine && (hg != mygen || hx != me)) != 0ull || S.test_foreign != 0;
      const bool ovf = __ballot(mine && hc > (uint32_t)kListMax) != 0ull;  // kNoList too
      const uint32_t cc = (mine && hc <= (uint32_t)kListMax) ? hc : 0u;
      const uint32_t incl = wave_incl_scan(cc);
      const uint32_t all = lane63(incl);
      const uint32_t gm = wave_max(hm);
      const uint32_t ts = wave_max(ht);
      const uint32_t nmax = wave_max(cc);
      if (lane <= kMaxSlices) sm.off[lane] = lane < W ? incl - cc : all;
      if (kJoint) {  // the row's mass: the slices' totals in slice order
        const double z =
            mine ? __longlong_as_double((long long)(((uint64_t)hz1 << 32) | hz0)) : 0.0;
        const double zr = lane63(wave_incl_scan(z));
        if (lane == 0) sm.zs = zr;
      }
      if (lane == 0) {
        uint32_t status = 0u;  // 0: go on, 1: invalid row, 2: fall back
        if (foreign) status = 2u;
        else if (anybad || (!KEYS && gm == 0u) || (kLogits && gm <= 0x007FFFFFu)) status = 1u;
        else if (ovf || all > (uint32_t)kRowCandMax) status = 2u;
        sm.res[2] = ts;
        sm.res[3] = all;
        sm.res[4] = gm;
        sm.res[5] = status;
        sm.res[6] = nmax;
      }
    }
    clear_hist<kHistBins>(sm.hist, tid, kBlock);
    if (kMass && tid < kMassBins + kWave) sm.mh[tid] = 0u;
    __syncthreads();
    DSS_STAMP(9);
    const uint32_t status = sm.res[5];
    if (status == 1u) {
      split_invalid<KIND>(P, S, Q, i, li);
      return kDone;
    }
    if (status == 2u) return kFallback;
    tstar = sm.res[2];
    ntot = sm.res[3];
    gmax = sm.res[4];
    const uint32_t nmax = sm.res[6];

    // the real positions into full[], in (slice, position) order; positions
    // past the speculative batch (rare) in further batches
    const uint32_t n_sl = sm.off[sl + 1] - sm.off[sl];
    const uint32_t o_sl = sm.off[sl];
#pragma unroll
    for (int q = 0; q < kLoadBatch; ++q) {
      if ((uint32_t)(q * gsz) >= min(spec, nmax)) continue;  // wave-uniform
      const uint32_t pos = (uint32_t)(lt + q * gsz);
      sm.full[pos < n_sl && pos < spec ? o_sl + pos : (uint32_t)(kRowCandMax + lane)] = e8[q];
    }
    uint64_t* out = sm.full + o_sl;
    for (uint32_t p0 = 0; nmax > spec && p0 < nmax; p0 += (uint32_t)(kLoadBatch * gsz)) {
#pragma unroll
      for (int q = 0; q < kLoadBatch; ++q) {
        const uint32_t pos = p0 + (uint32_t)(lt + q * gsz);
        e8[q] = (pos < n_sl && pos >= spec)
                    ? __hip_atomic_load(lst + pos, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                    : 0ull;
      }
#pragma unroll
      for (int q = 0; q < kLoadBatch; ++q) {
        const uint32_t pos = p0 + (uint32_t)(lt + q * gsz);
        if (pos < n_sl && pos >= spec) out[pos] = e8[q];
      }
    }
    __syncthreads();
    DSS_STAMP(10);
  }

  // From here on every thread holds entries, slot q of thread t being entry
  // t + 1024 q, all in registers.  Slots are visited in pairs behind
  // one wave-uniform test, and everything inside is branch-free.
  constexpr int kMw = 16, kMt = kMw * kWave, kSlots = kRowCandMax / kMt, kGrp = 2;
  const bool worker = wave < kMw;
  // logits: from here on entries carry the softmax's weights w = float32(
  // exp((z - m) / T)), m the row's largest logit, so w is 1 at the maximum
  // and a non-decreasing function of the logit key.  Top-k, top-p and the
  // draw compare values only with each other and with fractions of their
  // sums, so the normaliser S = sum_j w_j would cancel: it is never formed.
  // The bound t* becomes w(t*): an entry >= t* has w >= w(t*) (keys below
  // the -inf key are no logits: bound 0).
  const uint32_t tkey = tstar;
  const double lmax = kLogits ? (double)from_signed_key(gmax) : 0.0;
  auto prob_bits = [&](uint32_t key) -> uint32_t {
    const float w = (float)table_exp(((double)from_signed_key(key) - lmax) * itemp, sm.etab);
    return bits_of(w);
  };
  if constexpr (kLogits) {
    tstar = tkey <= 0x007FFFFFu ? 0u : prob_bits(tkey);
    gmax = prob_bits(gmax);
  }
  const uint32_t range = gmax - tstar;
  const uint32_t sh = range < (uint32_t)kHistBins ? 0u : 21u - (uint32_t)__clz((int)range);
  uint64_t en[kSlots];
  uint32_t kq[kSlots];  // (bits - t*) >> sh for an entry >= t*, 0xFFFFFFFF for none
  if (worker) {
#pragma unroll
    for (int q0 = 0; q0 < kSlots; q0 += kGrp) {
      if ((uint32_t)(q0 * kMt) >= ntot) continue;  // wave-uniform
#pragma unroll
      for (int q = q0; q < q0 + kGrp; ++q) {
        const uint32_t g = (uint32_t)(tid + q * kMt);
        en[q] = sm.full[g < ntot ? g : (uint32_t)(kRowCandMax + lane)];
        uint32_t x = (uint32_t)en[q];
        bool in = g < ntot && x >= tstar;
        if constexpr (kLogits) {
          // an entry at or above t* (keys), as its weight; zero ones carry no mass
          in = g < ntot && x >= tkey;
          x = in ? prob_bits(x) : 0u;
          en[q] = (en[q] & 0xFFFFFFFF00000000ull) | x;
          in = in && x >= tstar && x > 0u;
        }
        kq[q] = in ? (x - tstar) >> sh : 0xFFFFFFFFu;
      }
    }
  }

  // ---- tau_k: a histogram of the entries >= t* on the key (bits - t*) >> sh,
  // sh chosen so that the keys up to the row maximum fit 2048 bins ----------
  if (worker) {
#pragma unroll
    for (int q0 = 0; q0 < kSlots; q0 += kGrp) {
      if ((uint32_t)(q0 * kMt) >= ntot) continue;
#pragma unroll
      for (int q = q0; q < q0 + kGrp; ++q)
        atomicAdd(&sm.hist[kq[q] != 0xFFFFFFFFu ? H1::at(kq[q]) : pad], 1u);
    }
  }
  __syncthreads();
  DSS_STAMP(11);
  if (wave == 0) {
    uint32_t bin, above, total;
    wave_find<kHistBins>(sm.hist, (uint32_t)k, bin, above, total);
    if (lane == 0) {
      sm.fres[0] = bin;
      sm.fres[1] = above;
      sm.fres[2] = total;
    }
  }
  __syncthreads();
  DSS_STAMP(12);
  const uint32_t bin1 = sm.fres[0], above1 = sm.fres[1], nstar = sm.fres[2];
  if (nstar < (uint32_t)k && tstar > 0u) return kFallback;  // guard: fewer than k at or above t*
  const bool all_kept = nstar < (uint32_t)k;  // t* = 0 and k above the row's entry count
  // logits: values below t* can round to p(t*) itself, so tau_k must lie
  // strictly above p(t*); the boundary bin above the lowest one ensures it
  if (kLogits && !all_kept && tstar > 0u && bin1 == 0u) return kFallback;

  // ---- the entries above bin1 into cand, those in bin1 into bnd (both in
  // (slot, thread) order, one packed scan) --------------------------------------
  // above: kept for sure (every positive entry when all are kept); in bin1:
  // the boundary.  Entries are positive, so "above" is key > bin1 or, when
  // all are kept, key != none.
  const uint32_t hi_cut = all_kept ? 0xFFFFFFFEu : bin1;  // key > hi_cut and != none: above
  uint32_t na = 0u, nb = 0u;
  if (worker) {
#pragma unroll
    for (int q0 = 0; q0 < kSlots; q0 += kGrp) {
      if ((uint32_t)(q0 * kMt) >= ntot) continue;
#pragma unroll
      for (int q = q0; q < q0 + kGrp; ++q) {
        const bool some = kq[q] != 0xFFFFFFFFu;
        na += (some && (all_kept || kq[q] > hi_cut)) ? 1u : 0u;
        nb += (some && !all_kept && kq[q] == bin1) ? 1u : 0u;
      }
    }
  }
  uint32_t ptot;
  const uint32_t pk = block_excl_scan(na | (nb << 16), ptot, sm.red[2], worker);  // fields < 2^14
  const uint32_t n_above = ptot & 0xFFFFu, n_bnd = ptot >> 16;
  // the top-k set (above-bin entries and the boundary entries >= tau_k) must
  // fit cand[]; decided here, while every wave is still present
  if (n_above + n_bnd > (uint32_t)kKeptMax || n_bnd > (uint32_t)kBndMax) return kFallback;
  uint32_t pa = pk & 0xFFFFu, pb = pk >> 16;
  if (worker) {
#pragma unroll
    for (int q0 = 0; q0 < kSlots; q0 += kGrp) {
      if ((uint32_t)(q0 * kMt) >= ntot) continue;
#pragma unroll
      for (int q = q0; q < q0 + kGrp; ++q) {
        const bool some = kq[q] != 0xFFFFFFFFu;
        const bool ta = some && (all_kept || kq[q] > hi_cut);
        const bool tb = some && !all_kept && kq[q] == bin1;
        // one store per entry: into cand, into bnd, or a dummy slot
        uint64_t* const dst = ta   ? sm.u.b.cand + pa
                              : tb ? sm.u.b.bnd + pb
                                   : sm.u.b.cand + (kKeptMax + lane);
        *dst = en[q];
        if (kMass) {
          // (masked rather than selected, so that no branch forms around it)
          const uint32_t mb = ta ? kq[q] >> kMassShift : (uint32_t)(kMassBins + lane);
          atomicAdd(&sm.mh[mb], fixed_mass((uint32_t)en[q], gmax >> 23) & (ta ? ~0u : 0u));
        }
        pa += ta ? 1u : 0u;
        pb += tb ? 1u : 0u;
      }
    }
  }
  __syncthreads();
  DSS_STAMP(13);
  if (KIND != kKindSelect && wave != 0) return kDone;

  // ---- wave 0 from here on: tau_k inside bin1, the top-k list, the loop -----
  // (a selection keeps every wave for the sort)
  uint32_t m = n_above;
  uint32_t tau_k = 0u;
  double zb = 0.0;  // mass of the boundary entries kept (per lane, then summed)
  if (wave == 0 && !all_kept) {
    tau_k = wave_kth(sm.u.b.bnd, n_bnd, tstar + (bin1 << sh), sh, (uint32_t)k - above1, sm.hist,
                     sm.sel);
    // the boundary entries >= tau_k follow the others, in list order
    for (uint32_t c0 = 0; c0 < n_bnd; c0 += kWave) {
      const uint32_t c = c0 + lane;
      const uint64_t en = c < n_bnd ? sm.u.b.bnd[c] : 0ull;
      const bool take = c < n_bnd && (uint32_t)en >= tau_k && (uint32_t)en > 0u;
      const uint64_t tm = __ballot(take);
      const uint32_t p = m + rank_in(tm);
      if (take) sm.u.b.cand[p] = en;  // p < n_above + n_bnd <= kKeptMax
      m += (uint32_t)__popcll(tm);
      zb += take ? (double)__uint_as_float((uint32_t)en) : 0.0;
    }
  }

  DSS_STAMP(14);
  if constexpr (KIND == kKindSelect) {
    // cand[0, m) holds every entry >= tau_k (m >= k, more where tau_k is
    // tied); sorted by descending key, equal keys by ascending index, its
    // first k entries are the output
    if (wave == 0 && lane == 0) sm.res[7] = m;
    __syncthreads();
    const uint32_t ms = sm.res[7];
    uint32_t P2 = 1u;
    while (P2 < ms) P2 <<= 1;
    stream::sort_desc<true>(sm.u.b.cand, ms, P2);
    stream::select_write(Q, i, sm.u.b.cand);
    return kDone;
  }
  if (!kSampling) {
    // renormalisation / masking: tau_k, and the kept mass Z_k in a fixed order
    double zs = 0.0;
    if (KIND == kKindRenorm) {
      for (uint32_t c = lane; c < m; c += kWave)
        zs += (double)__uint_as_float((uint32_t)sm.u.b.cand[c]);
      zs = wave_sum(zs);
    }
    if (lane == 0) {
      as_global(S.r_tau)[li] = tau_k;
      as_global(S.r_z)[li] = zs;
      as_global(S.r_status)[li] = 0;
    }
    return kDone;
  }

  // ---- the dual-pivot loop on wave 0 ----------------------------------------
  const float pfrac = kTopPPart ? stream::clamp01(pp) : 0.0f;
  const uint32_t lowk = tau_k > 0u ? tau_k - 1u : 0u;
  uint32_t startk = lowk;
  MassView mv;
  mv.on = false;
  if (kMass) {
    const uint32_t L =
        top_p_start(sm, n_above, wave_sum(zb), gmax >> 23, pfrac, kJoint ? sm.zs : -1.0, tstar,
                    sh, bin1, mv);
    startk = max(startk, L);
  }
  DSS_STAMP(15);
  const float low = __uint_as_float(lowk), start = __uint_as_float(startk);
  int rounds = 0;
  const float high = __uint_as_float(gmax);
  const double zrow = kJoint ? sm.zs : 0.0;
  int e;
  if (m <= 4 * kWave) {
    e = wave_loop<OP, 4>(sm, (int)m, low, start, high, pfrac, zrow, seed, offset, sid, mv, rounds);
  } else if (m <= 8 * kWave) {
    e = wave_loop<OP, 8>(sm, (int)m, low, start, high, pfrac, zrow, seed, offset, sid, mv, rounds);
  } else if (m <= 16 * kWave) {
    e = wave_loop<OP, 16>(sm, (int)m, low, start, high, pfrac, zrow, seed, offset, sid, mv, rounds);
  } else {  // (32 float64 entries per lane in registers would spill the kernel)
    e = wave_loop<OP, 0>(sm, (int)m, low, start, high, pfrac, zrow, seed, offset, sid, mv, rounds);
  }
  DSS_STAMP(16);
  if (lane == 0) stream::write_sample(P, i, e, e >= 0 ? rounds : 0);
  return kDone;
}

template <int KIND, int OP, int NV>
__global__ __launch_bounds__(kBlock) void split_kernel(SampleParams P, SplitParams S,
                                                       RenormParams RP, SelectParams Q) {
  __shared__ SplitSmem sm;
  int i = 0;
  int mode = kDone;
  bool finisher = false;
  if constexpr (KIND == kKindSample &&
                (OP == kOpTopK || OP == kOpTopKTopP || OP == kOpTopKTopPJoint)) {
    if (S.fin && (int)blockIdx.x >= S.nsb) {
      mode = large_k_finish<OP>(P, S, sm, i);
      finisher = true;
    }
  }
  if (!finisher) {
    DSS_STAMP(0);
    mode = split_sample<KIND, OP, NV>(P, S, Q, sm, i);
  }
  if constexpr (KIND == kKindSample &&
                (OP == kOpTopK || OP == kOpTopKTopP || OP == kOpTopKTopPJoint)) {
    if (mode == kLargeKMerge) mode = large_k_merge<OP>(P, S, sm, i);
  }
  if (mode == kFallback) {
    if constexpr (KIND == kKindLogits) {
      // the output's row as probabilities into its part of prob_buf (the
      // one-work-group softmax), then the exact sampler on them
      const int row = P.indices ? as_global(P.indices)[i] : i;
      if (!(row >= 0 && row < P.rows)) {
        if (threadIdx.x == 0) stream::write_sample(P, i, -1, 0);
        return;
      }
      const float T = P.temp_arr ? as_global(P.temp_arr)[row] : P.temp;
      stream::softmax_row(P.probs + (int64_t)row * P.vocab, P.prob_buf + (int64_t)i * P.vocab,
                          P.vocab, T, P.vec_ok != 0, sm.u.stream.red);
      __syncthreads();
      SampleParams Q2 = P;
      Q2.probs = P.prob_buf;
      Q2.indices = nullptr;
      Q2.rows = P.num_outputs;
      Q2.vec_ok = P.vocab % 4 == 0;
      stream::sample_row_exact<OP>(Q2, i, sm.u.radix);
    } else if constexpr (KIND == kKindSample &&
                  (OP == kOpTopK || OP == kOpTopKTopP || OP == kOpTopKTopPJoint)) {
      stream::sample_row_exact<OP>(P, i, sm.u.radix);
    } else if constexpr (KIND == kKindSample) {
      stream::sample_row<OP>(P, i, sm.u.stream);
    } else if constexpr (KIND == kKindSelect) {
      stream::select_row(Q, i, sm.u.sel);
    } else {
      // the whole row by the streaming engine, output written here
      stream::renorm_row<KIND == kKindRenorm ? kRenormTopK : kMaskLogits>(RP, i, sm.u.stream.red);
      if (threadIdx.x == 0) as_global(S.r_status)[i - S.out0] = 2;
    }
  }
}

// The write pass of a split renormalisation / mask: work-group c of output
// li covers vectors [c * kBlock * kWB, (c + 1) * kBlock * kWB) of its row,
// kWB 16-byte loads in flight per thread.  out = x / Z_k (renorm) or x (mask)
// where key(x) >= tau_k, else 0 or -inf; invalid rows are NaN-filled.
constexpr int kWB = 8;
template <int KIND>
__global__ __launch_bounds__(kBlock) void split_write_kernel(RenormParams P, SplitParams S,
                                                             int nchunk) {
  constexpr bool KEYS = KIND == kKindMask;
  const int li = blockIdx.x / nchunk, c = blockIdx.x - li * nchunk;
  const int row = S.out0 + li;
  const uint32_t st = as_global(S.r_status)[li];
  if (st == 2u) return;
  const int V = P.vocab, nvec = V / 4;
  typedef float v4f __attribute__((ext_vector_type(4)));
  const gptr<const v4f> src = (gptr<const v4f>)as_global(P.in + (int64_t)row * V);
  const gptr<v4f> dst = (gptr<v4f>)as_global(P.out + (int64_t)row * V);
  const int f0 = c * kBlock * kWB + threadIdx.x;
  v4f x[kWB];
#pragma unroll
  for (int u = 0; u < kWB; ++u) x[u] = src[min(f0 + u * kBlock, nvec - 1)];
  const uint32_t tau = as_global(S.r_tau)[li];
  const double inv = KIND == kKindRenorm ? 1.0 / as_global(S.r_z)[li] : 0.0;
  const float qnan = __uint_as_float(0x7FC00000u), ninf = __uint_as_float(0xFF800000u);
#pragma unroll
  for (int u = 0; u < kWB; ++u) {
    v4f o;
    for (int e = 0; e < 4; ++e) {
      const float v = x[u][e];
      const bool keep = key_of<KEYS>(v) >= tau;
      o[e] = st == 1u ? qnan
             : KEYS   ? (keep ? v : ninf)
                      : (keep ? (float)((double)v * inv) : 0.0f);
    }
    if (f0 + u * kBlock < nvec) dst[f0 + u * kBlock] = o;
  }
  if (c == 0 && threadIdx.x == 0 && P.row_status) as_global(P.row_status)[row] = st == 1u ? 1 : 0;
}

template <int KIND, int OP, int NV>
void launch_one(const SampleParams& p, const SplitParams& sp, const RenormParams& rp,
                const SelectParams& q, hipStream_t s, const LaunchEvents& ev, bool first,
                bool last) {
  const int groups = (sp.n_out + 7) / 8;
  SplitParams S = sp;
  S.nsb = groups * 8 * sp.W;
  // finishing work-groups: only where an output's k is read per output (it
  // may exceed the cap) and the slices alone take more than one work-group
  // per compute unit, so that a merge holding a compute unit would keep
  // slices waiting
  constexpr bool kTopKOps = KIND == kKindSample &&
                            (OP == kOpTopK || OP == kOpTopKTopP || OP == kOpTopKTopPJoint);
  S.fin = kTopKOps && p.top_k_arr != nullptr && sp.W > 1 && S.nsb > kFinMinBlocks ? 1 : 0;
  S.spin = spin_limit_ticks();
  S.test_foreign = handoff_test_mode();
  const dim3 grid((unsigned)(S.nsb + (S.fin ? groups * 8 : 0))), block(kBlock);
  launch_kernel(split_kernel<KIND, OP, NV>, grid, block, s, ev, first, last, p, S, rp, q);
}

template <int KIND, int OP>
void launch_nv(int nv, const SampleParams& p, const SplitParams& sp, const RenormParams& rp,
               hipStream_t s, const LaunchEvents& ev, bool first, bool last,
               const SelectParams& q = SelectParams{}) {
  switch (nv) {
    case 1: launch_one<KIND, OP, 1>(p, sp, rp, q, s, ev, first, last); break;
    case 2: launch_one<KIND, OP, 2>(p, sp, rp, q, s, ev, first, last); break;
    case 3: launch_one<KIND, OP, 3>(p, sp, rp, q, s, ev, first, last); break;
    case 4: launch_one<KIND, OP, 4>(p, sp, rp, q, s, ev, first, last); break;
    case 6: launch_one<KIND, OP, 6>(p, sp, rp, q, s, ev, first, last); break;
    case 8: launch_one<KIND, OP, 8>(p, sp, rp, q, s, ev, first, last); break;
    default: launch_one<KIND, OP, 10>(p, sp, rp, q, s, ev, first, last); break;
  }
}

constexpr int kChunk = kSplitChunk;  // outputs per launch (bounds the workspace)
constexpr int kMaxNv = 10;  // vectors per thread
constexpr int kMaxSliceLen = kMaxNv * 4 * kBlock;

// The arrival counters and generation numbers sit at fixed offsets for the
// largest chunk, so calls of any shape can share one workspace: counters are
// zero between calls, generations only ever grow.
constexpr size_t kCtlBytes = 2 * (size_t)kChunk * 4;
static_assert(kCtlBytes == kCtlRegionBytes, "workspace layout shared with the resident engine");

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

SplitPlan plan_split(int op, int rows, int vocab, int num_outputs, uint32_t flags, int vec_ok) {
  SplitPlan plan{0, 0, 0, 0, 0, 0};
  (void)rows;
  if (op != kOpTopK && op != kOpTopKTopP && op != kOpTopKTopPJoint) return plan;
  if (flags & (DSS_FLAG_STREAMING | DSS_FLAG_FROM_ZERO | DSS_FLAG_SINGLE_PIVOT)) return plan;
  if (!vec_ok || vocab < 1024 || num_outputs <= 0) return plan;
  const int wmin = (vocab + kMaxSliceLen - 1) / kMaxSliceLen;
  const int wt = (256 + num_outputs - 1) / num_outputs;
  if (wmin > kMaxSlices) return plan;
  // W: a power of two, at least wmin, about 256 work-groups in all, at most
  // kMaxSlices, and no empty slice (or the measurement hook's choice)
  int W = 1;
  while (W < wmin || (W * 2 <= kMaxSlices && W * 2 <= wt)) W *= 2;
  if (forced_split_slices() > 0) W = max(forced_split_slices(), wmin);
  int L = 0;
  for (;; W /= 2) {
    L = ((vocab + 4 * W - 1) / (4 * W)) * 4;
    if (W == 1 || (int64_t)(W - 1) * L < vocab) break;
  }
  if (W < wmin) return plan;
  int nv = (L / 4 + kBlock - 1) / kBlock;
  nv = nv <= 4 ? nv : nv <= 6 ? 6 : nv <= 8 ? 8 : 10;
  const int ch = min(num_outputs, kChunk);
  plan.W = W;
  plan.L = L;
  plan.nv = nv;
  plan.chunk = ch;
  plan.handoff = W == 1 ? 0
                        : align256(kFixedRegionBytes + align256((size_t)ch * W * kHdrWords * 4) +
                                   (size_t)ch * W * kListMax * 8);
  plan.workspace = plan.handoff;
  return plan;
}

namespace {
// the hand-off region of a plan, then (renorm / mask) the per-output results.
// The results never overlap the control words (arrival counters, generation
// numbers at fixed offsets), which every op sharing a workspace relies on,
// even when the plan itself needs no hand-off (W == 1).
size_t result_bytes(size_t ch) { return align256(ch * 4) + align256(ch * 8) + align256(ch); }
size_t results_offset(const SplitPlan& plan) { return max(plan.handoff, align256(kFixedRegionBytes)); }

SplitParams split_params(const SplitPlan& plan, void* workspace) {
  char* ws = static_cast<char*>(workspace);
  const size_t ch = (size_t)plan.chunk;
  SplitParams sp;
  sp.fin = 0;
  sp.nsb = 0;
  sp.spin = 0ull;
  sp.test_foreign = 0;
  sp.W = plan.W;
  sp.wlog = 0;
  while ((1 << sp.wlog) < plan.W) ++sp.wlog;
  sp.L = plan.L;
  sp.ctr = reinterpret_cast<uint32_t*>(ws);
  sp.gen = sp.ctr + kChunk;
  sp.hdr = reinterpret_cast<uint32_t*>(ws + kFixedRegionBytes);
  sp.list = reinterpret_cast<uint64_t*>(ws + kFixedRegionBytes + align256(ch * plan.W * kHdrWords * 4));
  char* res = ws + results_offset(plan);
  sp.r_tau = reinterpret_cast<uint32_t*>(res);
  sp.r_z = reinterpret_cast<double*>(res + align256(ch * 4));
  sp.r_status = reinterpret_cast<uint8_t*>(res + align256(ch * 4) + align256(ch * 8));
  return sp;
}
}  // namespace

SplitPlan plan_split_renorm(int kind, int rows, int vocab, uint32_t flags, int vec_ok) {
  SplitPlan plan{0, 0, 0, 0, 0, 0};
  if (kind != kRenormTopK && kind != kMaskLogits) return plan;
  plan = plan_split(kOpTopK, rows, vocab, rows, flags, vec_ok);
  if (plan.W > 0) plan.workspace = results_offset(plan) + result_bytes((size_t)plan.chunk);
  return plan;
}

hipError_t launch_split_sample(int op, const SampleParams& p, const SplitPlan& plan,
                               void* workspace, hipStream_t s, const LaunchEvents& ev) {
  SplitParams sp = split_params(plan, workspace);
  const RenormParams rp{};
  for (int out0 = 0; out0 < p.num_outputs; out0 += plan.chunk) {
    sp.out0 = out0;
    sp.n_out = min(plan.chunk, p.num_outputs - out0);
    const bool first = out0 == 0, last = out0 + plan.chunk >= p.num_outputs;
    if (op == kOpTopK) {
      launch_nv<kKindSample, kOpTopK>(plan.nv, p, sp, rp, s, ev, first, last);
    } else if (op == kOpTopKTopPJoint) {
      launch_nv<kKindSample, kOpTopKTopPJoint>(plan.nv, p, sp, rp, s, ev, first, last);
    } else {
      launch_nv<kKindSample, kOpTopKTopP>(plan.nv, p, sp, rp, s, ev, first, last);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_split_logits(int op, const SampleParams& p, const SplitPlan& plan,
                               void* workspace, hipStream_t s, const LaunchEvents& ev) {
  if (op != kOpTopKTopP || !p.prob_buf) return hipErrorInvalidValue;
  SplitParams sp = split_params(plan, workspace);
  const RenormParams rp{};
  for (int out0 = 0; out0 < p.num_outputs; out0 += plan.chunk) {
    sp.out0 = out0;
    sp.n_out = min(plan.chunk, p.num_outputs - out0);
    const bool first = out0 == 0, last = out0 + plan.chunk >= p.num_outputs;
    launch_nv<kKindLogits, kOpTopKTopP>(plan.nv, p, sp, rp, s, ev, first, last);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_split_renorm(int kind, const RenormParams& rp, const SplitPlan& plan,
                               void* workspace, hipStream_t s, const LaunchEvents& ev) {
  // the results must lie inside the workspace the plan sized
  if (results_offset(plan) + result_bytes((size_t)plan.chunk) > plan.workspace)
    return hipErrorInvalidValue;
  SplitParams sp = split_params(plan, workspace);
  SampleParams p{};
  p.probs = rp.in;
  p.rows = rp.rows;
  p.vocab = rp.vocab;
  p.num_outputs = rp.rows;
  p.top_k_arr = rp.top_k_arr;
  p.top_k = rp.top_k;
  p.vec_ok = 1;
  const int nvec = rp.vocab / 4;
  const int nchunk = (nvec + kBlock * kWB - 1) / (kBlock * kWB);
  for (int out0 = 0; out0 < p.num_outputs; out0 += plan.chunk) {
    sp.out0 = out0;
    sp.n_out = min(plan.chunk, p.num_outputs - out0);
    const bool first = out0 == 0, last = out0 + plan.chunk >= p.num_outputs;
    const dim3 wgrid((unsigned)(sp.n_out * nchunk)), block(kBlock);
    if (kind == kRenormTopK) {
      launch_nv<kKindRenorm, kOpTopK>(plan.nv, p, sp, rp, s, ev, first, false);
      launch_kernel(split_write_kernel<kKindRenorm>, wgrid, block, s, ev, false, last, rp, sp, nchunk);
    } else {
      launch_nv<kKindMask, kOpTopK>(plan.nv, p, sp, rp, s, ev, first, false);
      launch_kernel(split_write_kernel<kKindMask>, wgrid, block, s, ev, false, last, rp, sp, nchunk);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

SplitPlan plan_split_select(int rows, int vocab, int k, uint32_t flags, int vec_ok) {
  SplitPlan plan{0, 0, 0, 0, 0, 0};
  if (k < 1 || k > kSplitKCap) return plan;
  return plan_split(kOpTopK, rows, vocab, rows, flags & DSS_FLAG_STREAMING, vec_ok);
}

hipError_t launch_split_select(const SelectParams& q, const SplitPlan& plan, void* workspace,
                               hipStream_t s, const LaunchEvents& ev) {
  SplitParams sp = split_params(plan, workspace);
  const RenormParams rp{};
  SampleParams p{};
  p.probs = q.in;
  p.rows = q.rows;
  p.vocab = q.vocab;
  p.num_outputs = q.rows;
  p.top_k = q.k;
  p.vec_ok = 1;
  for (int out0 = 0; out0 < p.num_outputs; out0 += plan.chunk) {
    sp.out0 = out0;
    sp.n_out = min(plan.chunk, p.num_outputs - out0);
    const bool first = out0 == 0, last = out0 + plan.chunk >= p.num_outputs;
    launch_nv<kKindSelect, kOpTopK>(plan.nv, p, sp, rp, s, ev, first, last, q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dss
