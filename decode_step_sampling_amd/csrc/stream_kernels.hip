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

template <int KIND>
__global__ __launch_bounds__(kBlock) void stream_renorm_kernel(RenormParams P) {
  __shared__ RedSmem red;
  const int row = blockIdx.x;
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
