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

__global__ __launch_bounds__(kBlock) void stream_minp_kernel(SampleParams P) {
  __shared__ SampleSmem sm;
  sample_row_minp(P, blockIdx.x, sm);
}

template <int KIND>
__global__ __launch_bounds__(kBlock) void stream_renorm_kernel(RenormParams P) {
  __shared__ RedSmem red;
  renorm_row<KIND>(P, blockIdx.x, red);
}

// Top-k selection, one work-group per row (select_row, stream_device.h).
__global__ __launch_bounds__(kBlock) void stream_select_kernel(SelectParams Q) {
  __shared__ SelectSmem sm;
  select_row(Q, blockIdx.x, sm);
}

// Probabilities from logits, one work-group per row (softmax_row,
// stream_device.h); the same arithmetic as the resident kernel.
__global__ __launch_bounds__(kBlock) void stream_softmax_kernel(SoftmaxParams Q) {
  __shared__ RedSmem red;
  const int row = blockIdx.x;
  const float T = Q.temp_arr ? Q.temp_arr[row] : Q.temp;
  const bool ok = softmax_row(Q.in + (int64_t)row * Q.vocab, Q.out + (int64_t)row * Q.vocab,
                              Q.vocab, T, Q.vec_ok != 0, red);
  if (Q.row_status && threadIdx.x == 0) Q.row_status[row] = ok ? 0 : 1;
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

hipError_t launch_stream_minp(const SampleParams& p, hipStream_t s, const LaunchEvents& ev) {
  const dim3 grid((unsigned)p.num_outputs), block(kBlock);
  launch_kernel(stream_minp_kernel, grid, block, s, ev, true, true, p);
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

// Plain streaming read for the bench's achievable-read reference: the batch
// is read once and its largest bit pattern folded into *out
// (order-independent).  Nothing else happens to
// the data, so its time is the read rate the GPU reaches at this size.
// The read reference: a grid-stride loop over 2048 work-groups of 256
// threads, one 16-byte load per thread per iteration.  Among the shapes
// measured on this GPU for a cold 38.9 MB batch (grid-stride and
// one-chunk-per-work-group loops, 256..1024 threads, 1..16 loads in flight
// per thread, with and without the non-temporal hint) this was the fastest:
// about 8 MB in flight over the whole GPU reads faster than issuing every
// load of a chunk at once (which measured 2.4 times slower).
constexpr int kReadBlock = 256;
constexpr int kReadGrid = 2048;
__global__ __launch_bounds__(kReadBlock) void stream_read_kernel(const float4* x, int64_t n4,
                                                                 uint32_t* out) {
  const gptr<const float4> src = as_global(x);
  const int64_t stride = (int64_t)gridDim.x * kReadBlock;
  uint32_t mx = 0u;
  for (int64_t q = (int64_t)blockIdx.x * kReadBlock + threadIdx.x; q < n4; q += stride) {
    const float4 a = load_f4(src + q);
    mx = max(mx, max(max(__float_as_uint(a.x), __float_as_uint(a.y)),
                     max(__float_as_uint(a.z), __float_as_uint(a.w))));
  }
  __shared__ uint32_t wm[kReadBlock / kWave];
  mx = wave_max(mx);
  if ((threadIdx.x & (kWave - 1)) == 0) wm[threadIdx.x / kWave] = mx;
  __syncthreads();
  if (threadIdx.x < kWave) {
    const uint32_t m = wave_max(threadIdx.x < kReadBlock / kWave ? wm[threadIdx.x] : 0u);
    // Atomics on one address serialise in the L2 (about 10 ns each), so a
    // work-group whose maximum the word already reaches skips its atomic:
    // the word only grows, so the result is the same maximum.
    if (threadIdx.x == 0 && m > vload(out))
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
  const int64_t need = (n4 + kReadBlock - 1) / kReadBlock;
  const unsigned grid = (unsigned)(need < kReadGrid ? need : kReadGrid);
  launch_kernel(stream_read_kernel, dim3(grid), dim3(kReadBlock), s, ev, true, true,
                reinterpret_cast<const float4*>(x), n4, out);
  return hipGetLastError();
}

}  // namespace dss
