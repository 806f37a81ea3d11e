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
