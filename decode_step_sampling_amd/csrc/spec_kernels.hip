// Chain speculative verification.
//
// The FlashInfer blog ("Sorting-Free GPU Kernels for LLM Sampling", section
// 社区采用和其他应用) points out that the rejection sampling behind its
// sampler also verifies speculative drafts (chain speculative sampling); the
// pages give no algorithm, so the standard one is implemented (Leviathan,
// Kalman & Matias 2023; Chen et al. 2023): draft token d_j is accepted iff
// u_j * q_j(d_j) < p_j(d_j); at the first rejection j* one token is drawn
// from the residual max(0, p_j* - q_j*) (from p_j* if that residual is zero
// everywhere); with every draft accepted, a bonus token is drawn from p_n.
// The draw is the inverse transform of the blog's 逆变换采样 section: the
// first index, in index order, whose inclusive prefix exceeds u * Z.
//
// Work: per row n pairs of single values for the acceptance chain, then one
// read of the one or two rows the final draw needs.  Each row is cut into W
// slices, one 1024-thread work-group per slice, all W on one XCD (block b
// runs on XCD b % 8).  Every work-group evaluates the acceptance chain
// itself (one lane per draft; the same decision everywhere), reads its slice
// once, and publishes the residual mass of each wave's contiguous range
// ("chunk").  The last work-group to arrive (a relaxed counter in the XCD's
// L2) adds the W * 16 chunk masses in order, draws u * Z, finds the chunk
// and walks it: one wave re-reads that chunk (about 1/16 of a slice).
// Headers carry the row's generation number and the writer's XCC id; if
// anything looks foreign the last work-group recomputes every chunk mass
// itself, so a broken placement costs time, never a wrong token.
#include "dss_device.h"
#include "dss_internal.h"

namespace dss {
namespace {

constexpr int kSpecHdr = 4;       // header words: generation, XCC id, bad value seen, 0
constexpr int kSpecNv = 10;       // 16-byte vectors per lane in a chunk walk
constexpr uint32_t kBadBits = 0x7F800000u;

struct SpecSmem {
  double cm[kSpecMaxW * kWaves];  // chunk masses of the row, slice-major
  double un;                      // the final draw u_n
  double tl;                      // target inside the chosen chunk
  uint32_t wbad[kWaves];
  int jstar;                      // first rejected position (n: none)
  int invalid;
  int flag;
  int cstar;                      // chosen chunk
  int tok;
};

__device__ __forceinline__ int s_uwave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ uint32_t s_xcc_id() {
  return __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20) & 0xFu;  // HW_REG_XCC_ID
}

// Residual weight of one value pair: max(0, p - q) with the difference taken
// in float64, or p itself when there is no draft row.
template <bool RES>
__device__ __forceinline__ double weight(float p, float q) {
  if (!RES) return (double)p;
  const double d = (double)p - (double)q;
  return d > 0.0 ? d : 0.0;
}

__device__ __forceinline__ bool bad4(const float4& x) {
  return max(max(__float_as_uint(x.x), __float_as_uint(x.y)),
             max(__float_as_uint(x.z), __float_as_uint(x.w))) >= kBadBits;
}

// The mass of this wave's chunk of a slice: vectors [c0, c1) of the rows
// P, Q (vector indices of the row), read coalesced (lane + 64 t), summed per
// lane in t order and then over the wave in a fixed tree.  Sets `bad` when
// any value read has its sign bit set or is NaN / inf.  Lane-uniform.
template <bool RES>
__device__ __forceinline__ double chunk_mass(gptr<const float4> P, gptr<const float4> Q, int c0,
                                             int c1, bool& bad) {
  const int lane = lane_id();
  double acc = 0.0;
  bool b = false;
  constexpr int U = 5;  // vectors per lane in flight (twice that with a draft row)
  for (int t0 = c0; t0 < c1; t0 += U * kWave) {
    float4 x[U], y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(t0 + u * kWave + lane, c1 - 1);
      x[u] = load_f4(P + t);
      y[u] = RES ? load_f4(Q + t) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = t0 + u * kWave + lane < c1;
      b = b || (in && (bad4(x[u]) || (RES && bad4(y[u]))));
      const double w = ((weight<RES>(x[u].x, y[u].x) + weight<RES>(x[u].y, y[u].y)) +
                        weight<RES>(x[u].z, y[u].z)) + weight<RES>(x[u].w, y[u].w);
      acc += in ? w : 0.0;
    }
  }
  bad = __ballot(b) != 0ull;
  return wave_sum(acc);
}

// Every chunk mass of the row computed by this work-group alone (slice
// after slice), into sm.cm; returns whether a bad value was seen.
template <bool RES>
__device__ __forceinline__ bool local_masses(gptr<const float4> P, gptr<const float4> Q, int W,
                                             int Lv, int CH, int nvec, SpecSmem& sm) {
  const int wave = s_uwave(), lane = lane_id();
  bool bad = false;
  for (int s = 0; s < W; ++s) {
    const int v0 = s * Lv, v1 = min(v0 + Lv, nvec);
    const int c0 = min(v0 + wave * CH, v1), c1 = min(c0 + CH, v1);
    bool b = false;
    const double m = c0 < c1 ? chunk_mass<RES>(P, Q, c0, c1, b) : 0.0;
    bad = bad || b;
    if (lane == 0) sm.cm[s * kWaves + wave] = m;
  }
  if (lane == 0) sm.wbad[wave] = bad ? 1u : 0u;
  __syncthreads();
  bool any = false;
  for (int w = 0; w < kWaves; ++w) any = any || sm.wbad[w] != 0u;
  __syncthreads();
  return any;
}

// One wave: the first value of vectors [c0, c1) (index order) whose
// inclusive prefix exceeds tl; lane l takes the contiguous vectors
// [c0 + l * m, c0 + (l + 1) * m), m = ceil((c1 - c0) / 64) <= kSpecNv.  A
// first pass sums each lane's vectors (five loads of each row in flight), a
// wave scan finds the lane, and that lane re-reads its vectors (now in
// cache) to find the value.  A target past the chunk's walked mass
// (rounding) takes its last positive value.  Returns the position in the
// row (4 * vector + element), or -1 if the chunk holds no positive weight.
template <bool RES>
__device__ __forceinline__ int chunk_walk(gptr<const float4> P, gptr<const float4> Q, int c0,
                                          int c1, double tl) {
  const int lane = lane_id();
  const int m = (c1 - c0 + kWave - 1) / kWave;
  const int a0 = c0 + lane * m;
  const int a1 = min(a0 + m, c1);  // this lane's vectors [a0, a1)
  constexpr int U = 5;
  static_assert(kSpecNv % U == 0, "whole batches");
  double ls = 0.0;
  int lastpos = -1;
#pragma unroll
  for (int t0 = 0; t0 < kSpecNv; t0 += U) {
    if (t0 >= m) break;  // wave-uniform
    float4 x[U], y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = min(a0 + t0 + u, c1 - 1);
      x[u] = load_f4(P + v);
      y[u] = RES ? load_f4(Q + v) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = a0 + t0 + u < a1;
      const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
      const float ys[4] = {y[u].x, y[u].y, y[u].z, y[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double w = in ? weight<RES>(xs[e], ys[e]) : 0.0;
        ls += w;
        lastpos = w > 0.0 ? 4 * (a0 + t0 + u) + e : lastpos;
      }
    }
  }
  const double incl = wave_incl_scan(ls);
  const uint64_t hit = __ballot(ls > 0.0 && incl > tl);
  const uint64_t any = __ballot(ls > 0.0);
  if (any == 0ull) return -1;
  const bool past = hit == 0ull;
  const int L = past ? 63 - __clzll((long long)any) : __ffsll((long long)hit) - 1;
  int pos = -1;
  if (lane == L) {
    if (past) {
      pos = lastpos;
    } else {
      double acc = incl - ls;
      for (int v = a0; v < a1 && pos < 0; ++v) {
        const float4 x = load_f4(P + v);
        const float4 y = RES ? load_f4(Q + v) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const float xs[4] = {x.x, x.y, x.z, x.w};
        const float ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double w = weight<RES>(xs[e], ys[e]);
          acc += w;
          if (pos < 0 && w > 0.0 && acc > tl) pos = 4 * v + e;
        }
      }
      if (pos < 0) pos = lastpos;  // rounding inside the lane
    }
  }
  return __builtin_amdgcn_readlane(pos, L);
}

__device__ __forceinline__ void spec_invalid(const SpecParams& S, int r) {
  const int n = S.n;
  for (int j = threadIdx.x; j <= n; j += kBlock) as_global(S.tokens)[(int64_t)r * (n + 1) + j] = -1;
  if (threadIdx.x == 0) {
    as_global(S.accepted)[r] = 0;
    if (S.valid) as_global(S.valid)[r] = 0;
  }
}

// Row r's result: the accepted drafts, the drawn token, then -1.
__device__ __forceinline__ void spec_write(const SpecParams& S, int r, int jstar, int tok) {
  const int n = S.n;
  const gptr<int32_t> out = as_global(S.tokens) + (int64_t)r * (n + 1);
  for (int j = threadIdx.x; j <= n; j += kBlock)
    out[j] = j < jstar ? as_global(S.ids)[(int64_t)r * n + j] : j == jstar ? tok : -1;
  if (threadIdx.x == 0) {
    as_global(S.accepted)[r] = jstar;
    if (S.valid) as_global(S.valid)[r] = 1;
  }
}

// The last work-group of a row (or the only one): the draw from the chunk
// masses in sm.cm, the walk, the outputs.
template <bool RES>
__device__ __forceinline__ void spec_finish(const SpecParams& S, const SpecPlan& Pl, int r,
                                            gptr<const float4> P, gptr<const float4> Q,
                                            int nvec, SpecSmem& sm) {
  const int wave = s_uwave(), lane = lane_id();
  const int W = Pl.W;
  const int nch = W * kWaves;  // <= 256: four chunks per lane
  if (wave == 0) {
    double cmq[4];
    double ls = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = 4 * lane + q;
      cmq[q] = c < nch ? sm.cm[c] : 0.0;
      ls += cmq[q];
    }
    const double incl = wave_incl_scan(ls);
    const double Z = lane63(incl);
    const double T = sm.un * Z;
    const uint64_t hit = __ballot(ls > 0.0 && incl > T);
    const bool none = Z <= 0.0;
    const bool past = hit == 0ull;
    const int L = past ? 63 - __clzll((long long)(__ballot(ls > 0.0) | 1ull))
                       : __ffsll((long long)hit) - 1;
    if (lane == L) {
      double acc = incl - ls;
      int pick = -1, lastc = -1;
      double ex = 0.0, mlast = 0.0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double before = acc;
        acc += cmq[q];
        if (cmq[q] > 0.0) {
          lastc = q;
          mlast = cmq[q];
          if (pick < 0 && !past && acc > T) {
            pick = q;
            ex = before;
          }
        }
      }
      const int q = pick >= 0 ? pick : lastc;
      sm.cstar = (none || q < 0) ? -1 : 4 * L + q;
      sm.tl = pick >= 0 ? T - ex : 2.0 * mlast;
    }
  }
  __syncthreads();
  const int c = sm.cstar;
  if (c < 0) {  // no positive weight left (handled by the caller for RES)
    if (wave == 0 && lane == 0) sm.tok = -1;
  } else if (wave == 0) {
    const int s = c / kWaves, w = c % kWaves;
    const int v0 = s * Pl.Lv, v1 = min(v0 + Pl.Lv, nvec);
    const int c0 = min(v0 + w * Pl.CH, v1), c1 = min(c0 + Pl.CH, v1);
    const int pos = chunk_walk<RES>(P, Q, c0, c1, sm.tl);
    if (lane == 0) sm.tok = pos;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kBlock) void spec_kernel(SpecParams S, SpecPlan Pl, int out0,
                                                      int n_out) {
  __shared__ SpecSmem sm;
  const int W = Pl.W;
  const int b = blockIdx.x, xcd = b & 7, local = b >> 3;
  const int li = (local / W) * 8 + xcd;  // the W slices of a row share b % 8
  const int s = local % W;
  if (li >= n_out) return;
  const int r = out0 + li;
  const int tid = threadIdx.x, lane = lane_id(), wave = s_uwave();
  const int n = S.n, V = S.vocab;
  const int nvec = V / 4;

  // ---- the acceptance chain: lane j tests draft j (wave 0) ------------------
  const uint64_t seed = S.seed_arr ? as_global(S.seed_arr)[r] : S.seed;
  const uint64_t offset = S.offset_arr ? as_global(S.offset_arr)[r] : S.offset;
  const uint64_t sid = S.seed_arr ? 0ull : (uint64_t)r;
  uint32_t gen = 0u;
  if (wave == 0) {
    if (W > 1 && lane == 0)
      gen = __hip_atomic_load(as_global(Pl.gen + li), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool stop = false, broken = false;
    if (lane < n) {
      const int d = as_global(S.ids)[(int64_t)r * n + lane];
      if (d < 0 || d >= V) {
        stop = broken = true;
      } else {
        const float pj = as_global(S.p)[((int64_t)r * (n + 1) + lane) * V + d];
        const float qj = as_global(S.q)[((int64_t)r * n + lane) * V + d];
        if (__float_as_uint(pj) >= kBadBits || __float_as_uint(qj) >= kBadBits) {
          stop = broken = true;
        } else {
          // u * q < p decided exactly: prod = fl(u * q), err its rounding error
          const double u = draw_uniform(seed, offset, sid, (uint32_t)lane);
          const double prod = u * (double)qj;
          const double err = __builtin_fma(u, (double)qj, -prod);
          const bool accept = prod < (double)pj || (prod == (double)pj && err < 0.0);
          stop = !accept;
        }
      }
    }
    const uint64_t sm_ = __ballot(stop);
    const int jstar = sm_ ? __ffsll((long long)sm_) - 1 : n;
    const bool inval = sm_ && (__ballot(broken) >> jstar & 1ull);
    if (lane == 0) {
      sm.jstar = jstar;
      sm.invalid = inval ? 1 : 0;
      sm.un = draw_uniform(seed, offset, sid, (uint32_t)n);
    }
  }
  __syncthreads();
  const int jstar = sm.jstar;
  if (sm.invalid) {  // the same decision in every slice of the row
    if (s == 0) spec_invalid(S, r);
    return;
  }
  const bool res = jstar < n;
  const gptr<const float4> P =
      (gptr<const float4>)as_global(S.p + ((int64_t)r * (n + 1) + jstar) * V);
  const gptr<const float4> Q =
      (gptr<const float4>)as_global(S.q + ((int64_t)r * n + (res ? jstar : 0)) * V);

  // ---- this slice's chunk masses --------------------------------------------
  const int v0 = s * Pl.Lv, v1 = min(v0 + Pl.Lv, nvec);
  const int c0 = min(v0 + wave * Pl.CH, v1), c1 = min(c0 + Pl.CH, v1);
  bool bad = false;
  double m = 0.0;
  if (c0 < c1) m = res ? chunk_mass<true>(P, Q, c0, c1, bad) : chunk_mass<false>(P, Q, c0, c1, bad);
  if (lane == 0) sm.wbad[wave] = bad ? 1u : 0u;

  bool foreign = false;
  if (W == 1) {
    if (lane == 0) sm.cm[wave] = m;
    __syncthreads();
  } else {
    const int64_t slot = (int64_t)li * W + s;
    if (lane == 0) as_global(Pl.masses)[slot * kWaves + wave] = m;
    __syncthreads();
    if (tid == 0) {
      uint32_t anyb = 0u;
      for (int w = 0; w < kWaves; ++w) anyb |= sm.wbad[w];
      const gptr<uint32_t> h = as_global(Pl.hdr + slot * kSpecHdr);
      h[0] = gen;
      h[1] = s_xcc_id();
      h[2] = anyb;
    }
    // hand-off: this work-group's stores reach the XCD's L2 before it arrives
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(as_global(Pl.ctr + li), 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      sm.flag = old == (uint32_t)(W - 1);
    }
    __syncthreads();
    if (!sm.flag) return;

    // ---- the last work-group of the row -------------------------------------
    if (wave == 0) {
      uint32_t hg = 0u, hx = 0u, hb = 0u;
      if (lane < W) {
        const gptr<uint32_t> h = as_global(Pl.hdr + ((int64_t)li * W + lane) * kSpecHdr);
        hg = __hip_atomic_load(h + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hx = __hip_atomic_load(h + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hb = __hip_atomic_load(h + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const uint32_t mygen = (uint32_t)__builtin_amdgcn_readfirstlane((int)gen);
      const bool fr = __ballot(lane < W && (hg != mygen || hx != s_xcc_id())) != 0ull;
      const bool anyb = __ballot(lane < W && hb != 0u) != 0ull;
      if (lane == 0) {
        __hip_atomic_store(as_global(Pl.ctr + li), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(as_global(Pl.gen + li), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.flag = fr ? 1 : 0;
        sm.wbad[0] = anyb ? 1u : 0u;
      }
    }
    for (int c = tid; c < W * kWaves; c += kBlock)
      sm.cm[c] = __hip_atomic_load(as_global(Pl.masses) + (int64_t)li * W * kWaves + c,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    foreign = sm.flag != 0;
    bad = sm.wbad[0] != 0u;
    __syncthreads();
  }
  if (W == 1) {
    uint32_t anyb = 0u;
    for (int w = 0; w < kWaves; ++w) anyb |= sm.wbad[w];
    bad = anyb != 0u;
    __syncthreads();
  }
  if (foreign)  // recompute every chunk here (same order, same sums)
    bad = res ? local_masses<true>(P, Q, W, Pl.Lv, Pl.CH, nvec, sm)
              : local_masses<false>(P, Q, W, Pl.Lv, Pl.CH, nvec, sm);
  if (bad) {
    spec_invalid(S, r);
    return;
  }
  int tok;
  if (res) {
    spec_finish<true>(S, Pl, r, P, Q, nvec, sm);
    tok = sm.tok;
    if (sm.cstar < 0) {
      // the residual is zero everywhere: draw from p_j* itself
      __syncthreads();
      local_masses<false>(P, Q, W, Pl.Lv, Pl.CH, nvec, sm);
      spec_finish<false>(S, Pl, r, P, Q, nvec, sm);
      tok = sm.tok;
    }
  } else {
    spec_finish<false>(S, Pl, r, P, Q, nvec, sm);
    tok = sm.tok;
  }
  if (tok < 0) {
    spec_invalid(S, r);
    return;
  }
  spec_write(S, r, jstar, tok);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

SpecPlan plan_spec(int rows, int vocab, int n, int vec_ok) {
  SpecPlan pl{};
  if (!vec_ok || vocab % 4 != 0 || rows <= 0 || n < 0 || n > kSpecMaxN) return pl;
  const int nvec = vocab / 4;
  // W: a power of two, at least enough slices that a chunk fits one wave's
  // walk (64 * kSpecNv vectors), about 256 work-groups in all
  const int cap = kWaves * kWave * kSpecNv;  // vectors of one slice at most
  const int wmin = (nvec + cap - 1) / cap;
  if (wmin > kSpecMaxW) return pl;
  const int wt = (256 + rows - 1) / rows;
  int W = 1;
  while (W < wmin || (W * 2 <= kSpecMaxW && W * 2 <= wt)) W *= 2;
  while (W > 1 && (int64_t)(W - 1) * ((nvec + W - 1) / W) >= nvec) W /= 2;  // no empty slice
  if (W < wmin) return pl;
  pl.W = W;
  pl.Lv = (nvec + W - 1) / W;
  pl.CH = (pl.Lv + kWaves - 1) / kWaves;
  pl.per_launch = min(rows, kSpecRowsPerLaunch);
  const size_t ch = (size_t)pl.per_launch;
  pl.workspace = W == 1 ? 0
                        : align256(kFixedRegionBytes + align256(ch * W * kSpecHdr * 4) +
                                   ch * W * kWaves * 8);
  return pl;
}

hipError_t launch_spec(const SpecParams& sp, const SpecPlan& plan, void* workspace,
                       hipStream_t s, const LaunchEvents& ev) {
  SpecPlan pl = plan;
  char* ws = static_cast<char*>(workspace);
  if (pl.W > 1) {
    // counters and generations at the fixed control words every op shares
    // (zero between calls / only growing); headers and masses after the
    // fixed region, written before they are read
    pl.ctr = reinterpret_cast<uint32_t*>(ws);
    pl.gen = pl.ctr + kSpecRowsPerLaunch;
    pl.hdr = reinterpret_cast<uint32_t*>(ws + kFixedRegionBytes);
    pl.masses = reinterpret_cast<double*>(
        ws + kFixedRegionBytes + align256((size_t)plan.per_launch * pl.W * kSpecHdr * 4));
  }
  for (int out0 = 0; out0 < sp.rows; out0 += plan.per_launch) {
    const int n_out = min(plan.per_launch, sp.rows - out0);
    const int groups = (n_out + 7) / 8;
    const bool first = out0 == 0, last = out0 + plan.per_launch >= sp.rows;
    launch_kernel(spec_kernel, dim3((unsigned)(groups * 8 * pl.W)), dim3(kBlock), s, ev, first,
                  last, sp, pl, out0, n_out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dss
