// Streaming engine: one 1024-thread work-group per output (sampling) or per
// row (renorm, logit masking).  Every pass reads the row from global memory,
// so it works for any vocabulary size up to DSS_MAX_VOCAB and any filter
// parameters.  It follows the pages' schedule literally:
//
//  * sampling: the dual-pivot rejection loop of the FlashInfer blog
//    ("Sorting-Free GPU Kernels for LLM Sampling", section 双枢轴拒绝采样),
//    low = 0, high = max, one inverse-transform draw (section 逆变换采样) and
//    one (mass, count) pass at both pivots per round, all inside one kernel;
//  * renorm / masking: the threshold search on the float32 bit pattern of the
//    F4 note ("F4 讲解：不排序的 top-k / top-p", §②-③), with two pivots per
//    pass at 1/3 and 2/3 of the interval and the min/max trackers of §⑤ that
//    stop the search as soon as one distinct value is left.
//
// Row layout during the rejection loop: the row is cut into tiles of 2048
// values; wave w of the work-group handles tiles w, w + 16, ..., reading each
// tile with eight coalesced 16-byte loads per lane.  Every pivot pass leaves
// the mass above each pivot per tile in LDS, so the next round's
// inverse-transform draw scans the tile masses (one wave) and then one tile.
#include "stream_device.h"

namespace dss {
namespace {

using namespace stream;

template <int OP>
__global__ __launch_bounds__(kBlock) void stream_sample_kernel(SampleParams P) {
  __shared__ SampleSmem sm;
  sample_row<OP>(P, blockIdx.x, sm);
}

template <int KIND>
__global__ __launch_bounds__(kBlock) void stream_renorm_kernel(RenormParams P) {
  __shared__ RedSmem red;
  renorm_row<KIND>(P, blockIdx.x, red);
}

// Top-k selection (explainer, 选择 top-k 值本身: values and indices rather
// than a sample), one work-group per row: tau = the k-th largest signed-order
// key by the F4 threshold search; one pass counts, per 2048-value tile, the
// values above tau and those equal to it, which fixes where the ties still
// needed end (in index order); a second pass gathers exactly k entries
// (key << 32 | ~index) into LDS; a bitonic sort puts them in descending key
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

__global__ __launch_bounds__(kBlock) void stream_select_kernel(SelectParams Q) {
  __shared__ SelectSmem sm;
  const int row = blockIdx.x, V = Q.vocab, k = Q.k;
  const int lane = lane_id(), wave = wave_id(), tid = threadIdx.x;
  const RowRef r{as_global(Q.in + (int64_t)row * V), V, Q.vec_ok != 0};
  const gptr<float> vo = as_global(Q.values + (int64_t)row * k);
  const gptr<int32_t> io = as_global(Q.indices + (int64_t)row * k);
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
    for (int j = tid; j < k; j += kBlock) {
      vo[j] = __uint_as_float(0x7FC00000u);
      io[j] = -1;
    }
    if (Q.row_status && tid == 0) Q.row_status[row] = 1;
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
#pragma unroll
    for (int q = 0; q < kTileChunks; ++q) {
      float v[4];
      const int64_t idx = base + q * (kWave * 4) + lane * 4;
      load4(r, idx, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = idx + e < V ? signed_key(v[e]) : 0u;
        eq += key == tau ? 1u : 0u;
        gt += key > tau ? 1u : 0u;
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
#pragma unroll
    for (int q = 0; q < kTileChunks; ++q) {
      float v[4];
      const int64_t idx = base + q * (kWave * 4) + lane * 4;
      load4(r, idx, v);
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
  __syncthreads();
  // pad to a power of two with zeros (below every real entry), then sort
  uint32_t P = 1u;
  while (P < (uint32_t)k) P <<= 1;
  for (uint32_t j = (uint32_t)k + tid; j < P; j += kBlock) sm.ent[j] = 0ull;
  __syncthreads();
  for (uint32_t size = 2u; size <= P; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0u; stride >>= 1) {
      for (uint32_t t = tid; t < P / 2u; t += kBlock) {
        const uint32_t i = 2u * t - (t & (stride - 1u));
        const uint32_t j = i + stride;
        const uint64_t a = sm.ent[i], b = sm.ent[j];
        const bool up = (i & size) != 0u;  // this block ascending (the final block descends)
        if (up ? (a > b) : (a < b)) {
          sm.ent[i] = b;
          sm.ent[j] = a;
        }
      }
      __syncthreads();
    }
  }
  // the values themselves are read back by index (the key folds -0.0 into +0.0)
  for (int j = tid; j < k; j += kBlock) {
    const int32_t ix = (int32_t)(0xFFFFFFFFu - (uint32_t)sm.ent[j]);
    vo[j] = r.x[ix];
    io[j] = ix;
  }
  if (Q.row_status && tid == 0) Q.row_status[row] = 0;
}

// Probabilities from logits, one work-group per row, three passes: the
// maximum (and NaN / +inf), the sum of exp((z - m) / T), the write; the same
// arithmetic as the resident kernel (explainer, 采样流水线究竟在计算什么).
__global__ __launch_bounds__(kBlock) void stream_softmax_kernel(SoftmaxParams Q) {
  __shared__ RedSmem red;
  const int row = blockIdx.x, V = Q.vocab;
  const RowRef r{as_global(Q.in + (int64_t)row * V), V, Q.vec_ok != 0};
  const gptr<float> out = as_global(Q.out + (int64_t)row * V);
  const float T = Q.temp_arr ? Q.temp_arr[row] : Q.temp;
  Red acc = red_zero();
  for_each4(r, [&](int64_t idx, const float (&v)[4], bool valid) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = valid && idx + e < V;
      acc.mx = max(acc.mx, in ? signed_key(v[e]) : 0u);
      acc.s0 += (in && (isnan(v[e]) || v[e] == __builtin_inff())) ? 1u : 0u;
    }
  });
  const Red s0 = block_reduce(acc, red);
  const uint32_t k = s0.mx;
  const float zmax = __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
  const int nvec = (V + 3) / 4;
  if (s0.s0 != 0u || !(T > 0.0f) || T == __builtin_inff() || zmax == -__builtin_inff()) {
    const float qnan = __uint_as_float(0x7FC00000u);
    const float o[4] = {qnan, qnan, qnan, qnan};
    for (int f = threadIdx.x; f < nvec; f += kBlock) store4(out, V, Q.vec_ok != 0, 4ll * f, o);
    if (Q.row_status && threadIdx.x == 0) Q.row_status[row] = 1;
    return;
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
    if (valid) store4(out, V, Q.vec_ok != 0, idx, o);
  });
  if (Q.row_status && threadIdx.x == 0) Q.row_status[row] = 0;
}

}  // namespace

hipError_t launch_stream_sample(int op, const SampleParams& p, hipStream_t s, const LaunchEvents& ev) {
  const dim3 grid((unsigned)p.num_outputs), block(kBlock);
  switch (op) {
    case kOpNone: launch_kernel(stream_sample_kernel<kOpNone>, grid, block, s, ev, true, true, p); break;
    case kOpTopK: launch_kernel(stream_sample_kernel<kOpTopK>, grid, block, s, ev, true, true, p); break;
    case kOpTopP: launch_kernel(stream_sample_kernel<kOpTopP>, grid, block, s, ev, true, true, p); break;
    case kOpMinP: launch_kernel(stream_sample_kernel<kOpMinP>, grid, block, s, ev, true, true, p); break;
    case kOpTopKTopP:
      launch_kernel(stream_sample_kernel<kOpTopKTopP>, grid, block, s, ev, true, true, p);
      break;
    case kOpTopKTopPJoint:
      launch_kernel(stream_sample_kernel<kOpTopKTopPJoint>, grid, block, s, ev, true, true, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stream_renorm(int kind, const RenormParams& p, hipStream_t s,
                                const LaunchEvents& ev) {
  const dim3 grid((unsigned)p.rows), block(kBlock);
  switch (kind) {
    case kRenormTopK: launch_kernel(stream_renorm_kernel<kRenormTopK>, grid, block, s, ev, true, true, p); break;
    case kRenormTopP: launch_kernel(stream_renorm_kernel<kRenormTopP>, grid, block, s, ev, true, true, p); break;
    case kMaskLogits: launch_kernel(stream_renorm_kernel<kMaskLogits>, grid, block, s, ev, true, true, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dss

namespace dss {
namespace {

// Plain streaming read for the bench's achievable-read reference: every
// work-group reads its contiguous share of n float4 once, five 16-byte loads
// in flight per thread, and folds the maximum bit pattern into *out
// (order-independent).  Nothing else happens to the
// data, so its time is the read rate the GPU reaches at this size.  (One
// atomic per work-group: per-wave atomics on one address serialise.)
constexpr int kReadDepth = 5;  // loads in flight per thread

// NV vectors per thread (NV * 1024 >= the work-group's share): the first
// kReadDepth loads leave at once, each later one as an earlier vector is
// consumed, which keeps the CU's load queue full without stalling the waves.
template <int NV>
__global__ __launch_bounds__(kBlock) void stream_read_kernel(const float4* x, int64_t n4,
                                                             int64_t chunk, uint32_t* out) {
  const int64_t b0 = (int64_t)blockIdx.x * chunk;
  const int64_t b1 = b0 + chunk < n4 ? b0 + chunk : n4;
  const gptr<const float4> src = as_global(x) + b0;
  const int len = (int)(b1 - b0);
  constexpr int D = NV < kReadDepth ? NV : kReadDepth;
  float4 v[NV];
  auto issue = [&](int j) { v[j] = load_f4(src + min((int)threadIdx.x + j * kBlock, len - 1)); };
#pragma unroll
  for (int j = 0; j < D; ++j) issue(j);
  uint32_t mx = 0u;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const uint32_t m = max(max(__float_as_uint(v[j].x), __float_as_uint(v[j].y)),
                           max(__float_as_uint(v[j].z), __float_as_uint(v[j].w)));
    mx = ((int)threadIdx.x + j * kBlock < len) ? max(mx, m) : mx;
    if (j + D < NV) {
      __builtin_amdgcn_sched_barrier(0);
      issue(j + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __shared__ uint32_t wm[kWaves];
  mx = wave_max(mx);
  if ((threadIdx.x & (kWave - 1)) == 0) wm[threadIdx.x / kWave] = mx;
  __syncthreads();
  if (threadIdx.x < kWave) {
    const uint32_t m = wave_max(threadIdx.x < kWaves ? wm[threadIdx.x] : 0u);
    if (threadIdx.x == 0)
      __hip_atomic_fetch_max(as_global(out), m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t s, const LaunchEvents& ev) {
  launch_kernel(stream_select_kernel, dim3((unsigned)p.rows), dim3(kBlock), s, ev, true, true, p);
  return hipGetLastError();
}

hipError_t launch_stream_softmax(const SoftmaxParams& p, hipStream_t s, const LaunchEvents& ev) {
  launch_kernel(stream_softmax_kernel, dim3((unsigned)p.rows), dim3(kBlock), s, ev, true, true, p);
  return hipGetLastError();
}

hipError_t launch_stream_read(const float* x, int64_t n, uint32_t* out, hipStream_t s,
                              const LaunchEvents& ev) {
  const int64_t n4 = n / 4;
  if (n4 <= 0) return hipSuccess;
  // 256 work-groups (one per CU) unless a share would exceed 16 vectors per
  // thread; NV rounded up to an instantiated size
  int64_t grid = n4 < (int64_t)kBlock * 256 ? (n4 + kBlock - 1) / kBlock : 256;
  while ((n4 + grid - 1) / grid > (int64_t)16 * kBlock) grid *= 2;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int64_t chunk = (n4 + grid - 1) / grid;
  const int per = (int)((chunk + kBlock - 1) / kBlock);
  const float4* x4 = reinterpret_cast<const float4*>(x);
  const dim3 g((unsigned)grid), blk(kBlock);
#define DSS_READ_NV(N)                                                                \
  if (per <= N) {                                                                     \
    launch_kernel(stream_read_kernel<N>, g, blk, s, ev, true, true, x4, n4, chunk, out); \
    return hipGetLastError();                                                         \
  }
  DSS_READ_NV(1) DSS_READ_NV(2) DSS_READ_NV(4) DSS_READ_NV(6) DSS_READ_NV(8) DSS_READ_NV(10)
  DSS_READ_NV(12) DSS_READ_NV(16)
#undef DSS_READ_NV
  return hipErrorInvalidValue;
}

}  // namespace dss
