// C ABI of libdss.so (declared in include/dss.h): argument validation on the
// host, device check, choice of engine, launch on the caller's stream.
// Validation happens before the first HIP runtime call, so every error path
// can be exercised on a machine without a GPU.
#include <atomic>
#include <cmath>
#include <cstring>

#include "dss_internal.h"

#define DSS_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<void*> g_ev_start{nullptr}, g_ev_stop{nullptr};  // dss_set_timing_events
std::atomic<uint64_t> g_spin_ticks{dss::kDefaultSpinTicks};  // dss_set_spin_limit
std::atomic<int32_t> g_handoff_test{0};                       // dss_set_handoff_test
std::atomic<int> g_split_slices{0};                            // dss_set_split_slices

dss::LaunchEvents timing_events() {
  return dss::LaunchEvents{static_cast<hipEvent_t>(g_ev_start.load(std::memory_order_relaxed)),
                           static_cast<hipEvent_t>(g_ev_stop.load(std::memory_order_relaxed))};
}

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSS_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DSS_ERR_DEVICE;
  int st = g_device_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DSS_ERR_HIP;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? DSS_OK : DSS_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int sample_common(int op, const float* probs, int32_t rows, int32_t vocab, const int32_t* indices,
                  int32_t num_outputs, const uint64_t* seed_arr, uint64_t seed,
                  const uint64_t* offset_arr, uint64_t offset, const int32_t* top_k_arr,
                  int32_t top_k, const float* top_p_arr, float top_p, const float* min_p_arr,
                  float min_p, int32_t* samples, uint8_t* valid, int32_t* rounds, uint32_t flags,
                  void* workspace, size_t workspace_bytes, void* stream,
                  const dss::LaunchEvents& ev, bool check_only = false,
                  bool repair_slots = false, const float* temp_arr = nullptr,
                  float temp = 1.0f, float* prob_buf = nullptr) {
  // prob_buf set: `probs` holds logits, sampled through softmax(z / T) on the
  // split engine (the caller has checked that its plan applies)
  if (flags & ~DSS_FLAGS_ALL) return DSS_ERR_INVALID_ARG;
  // the joint order only exists for the combined filter; the engines know it
  // as an op of its own (the public op id still sizes the workspace)
  if ((flags & DSS_FLAG_ORDER_JOINT) && op != dss::kOpTopKTopP) return DSS_ERR_UNSUPPORTED;
  const int eop = (flags & DSS_FLAG_ORDER_JOINT) ? dss::kOpTopKTopPJoint : op;
  if (rows < 0 || vocab <= 0 || num_outputs < 0) return DSS_ERR_INVALID_ARG;
  if (vocab > DSS_MAX_VOCAB) return DSS_ERR_UNSUPPORTED;
  if (!indices && num_outputs != rows) return DSS_ERR_INVALID_ARG;
  if (num_outputs == 0) return DSS_OK;
  if (!probs || !samples) return DSS_ERR_INVALID_ARG;
  const int vec_ok = (vocab % 4 == 0) && aligned16(probs);
  dss::SplitPlan plan = dss::plan_split(eop, rows, vocab, num_outputs, flags, vec_ok);
  if (plan.W > 0 && !top_k_arr && (eop == dss::kOpTopK || eop == dss::kOpTopKTopP) &&
      (top_k > dss::kSplitKCapHost || (int64_t)top_k * plan.W > dss::kSplitScalarKW))
    plan = dss::SplitPlan{0, 0, 0, 0, 0, 0};
  dss::SplitPlan rplan = plan.W > 0 ? dss::SplitPlan{0, 0, 0, 0, 0, 0}
                                    : dss::plan_resident(eop, vocab, num_outputs, flags, vec_ok, true,
                                                         dss::resident_pairs(eop, top_k_arr, top_k, vocab));
  // Plain and min-p sampling of a batch the resident engine would take in
  // more than one launch: one work-group per output keeps HBM busier than
  // launches that each wait at row barriers.  Plain sampling reads the row
  // twice (tile masses, then one tile); min-p reads it for the tile maxima
  // and again only where a tile holds a kept value (172 / 185 outputs of
  // V = 128256: 19 / 27 us instead of 41 / 44 us).  Batches that fit one
  // launch (up to 64 outputs of V = 151936) stay resident, where the chip's
  // every compute unit shares each row.
  const bool wide_stream = rplan.W > 0 && rplan.chunk < num_outputs &&
                           (eop == dss::kOpNone || eop == dss::kOpMinP);
  const bool minp_streams = wide_stream && eop == dss::kOpMinP;
  if (wide_stream) rplan = dss::SplitPlan{0, 0, 0, 0, 0, 0};
  const size_t need = dss_workspace_size(op, rows, vocab, num_outputs, flags);
  if (workspace_bytes < need || (need > 0 && !workspace)) return DSS_ERR_WORKSPACE;
  // and whatever the chosen plan itself uses (never past the caller's buffer)
  const size_t used = plan.W > 0 ? plan.workspace : rplan.W > 0 ? rplan.workspace : 0;
  if (workspace_bytes < used || (used > 0 && !workspace)) return DSS_ERR_WORKSPACE;
  if (check_only) return DSS_OK;
  const int dev = check_device();
  if (dev != DSS_OK) return dev;

  dss::SampleParams p;
  p.probs = probs;
  p.rows = rows;
  p.vocab = vocab;
  p.indices = indices;
  p.num_outputs = num_outputs;
  p.seed_arr = seed_arr;
  p.seed = seed;
  p.offset_arr = offset_arr;
  p.offset = offset;
  p.top_k_arr = top_k_arr;
  p.top_k = top_k;
  p.top_p_arr = top_p_arr;
  p.top_p = top_p;
  p.min_p_arr = min_p_arr;
  p.min_p = min_p;
  p.samples = samples;
  p.valid = valid;
  p.rounds = rounds;
  p.vec_ok = vec_ok;
  p.single_pivot = (flags & DSS_FLAG_SINGLE_PIVOT) ? 1 : 0;
  p.temp_arr = temp_arr;
  p.temp = temp;
  p.prob_buf = prob_buf;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (prob_buf) {
    if (plan.W == 0) return DSS_ERR_INVALID_ARG;
    return dss::launch_split_logits(eop, p, plan, workspace, st, ev) == hipSuccess ? DSS_OK
                                                                                 : DSS_ERR_HIP;
  }
  if (repair_slots && plan.W == 0 && rplan.W > 0 &&
      dss::launch_resident_repair(workspace, st) != hipSuccess)
    return DSS_ERR_HIP;
  const hipError_t e =
      plan.W > 0     ? dss::launch_split_sample(eop, p, plan, workspace, st, ev)
      : rplan.W > 0  ? dss::launch_resident_sample(eop, p, rplan, workspace, st, ev)
      : minp_streams ? dss::launch_stream_minp(p, st, ev)
                     : dss::launch_stream_sample(eop, p, st, ev);
  return e == hipSuccess ? DSS_OK : DSS_ERR_HIP;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Whether top-k-then-top-p sampling from logits runs fused on the split
// engine (the plan sample_common would take for the same shape, sequential
// order only); otherwise probabilities are written first and sampled.
bool logits_fused(int32_t rows, int32_t vocab, int32_t num_outputs, const int32_t* top_k_arr,
                  int32_t top_k, uint32_t flags, int vec_ok) {
  if (flags & DSS_FLAG_ORDER_JOINT) return false;
  const dss::SplitPlan plan =
      dss::plan_split(dss::kOpTopKTopP, rows, vocab, num_outputs, flags, vec_ok);
  if (plan.W == 0) return false;
  return top_k_arr || (top_k <= dss::kSplitKCapHost && (int64_t)top_k * plan.W <= dss::kSplitScalarKW);
}

// Workspace of the logits path: the engines' area (the softmax kernel's and
// the sampling call's share one), then the probabilities.  The probabilities
// start past the fixed region (control words and resident slots) even when
// neither engine needs it for this call, so a shared workspace keeps every
// word that other calls expect at zero.
size_t logits_engine_bytes(int32_t rows, int32_t vocab, int32_t num_outputs, uint32_t flags) {
  const size_t a = dss_workspace_size(DSS_OP_TOP_K_TOP_P, rows, vocab, num_outputs, flags);
  const size_t b = dss::plan_softmax(rows, vocab, flags, vocab % 4 == 0).workspace;
  const size_t c = align256(dss::kFixedRegionBytes);
  const size_t m = a > b ? a : b;
  return align256(m > c ? m : c);
}

int renorm_common(int kind, int op_id, const float* in, float* out, int32_t rows, int32_t vocab,
                  const int32_t* top_k_arr, int32_t top_k, const float* top_p_arr, float top_p,
                  uint8_t* row_status, uint32_t flags, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (flags & ~DSS_FLAGS_ALL) return DSS_ERR_INVALID_ARG;
  if (flags & DSS_FLAG_ORDER_JOINT) return DSS_ERR_UNSUPPORTED;
  if (rows < 0 || vocab <= 0) return DSS_ERR_INVALID_ARG;
  if (vocab > DSS_MAX_VOCAB) return DSS_ERR_UNSUPPORTED;
  if (rows == 0) return DSS_OK;
  if (!in || !out) return DSS_ERR_INVALID_ARG;
  const int vec_ok = (vocab % 4 == 0) && aligned16(in) && aligned16(out);
  const dss::SplitPlan plan = dss::plan_split_renorm(kind, rows, vocab, flags, vec_ok);
  const dss::SplitPlan rplan = kind == dss::kRenormTopP
                                   ? dss::plan_resident(dss::kOpTopP, vocab, rows, flags, vec_ok)
                                   : dss::SplitPlan{0, 0, 0, 0, 0, 0};
  const size_t need = dss_workspace_size(op_id, rows, vocab, rows, flags);
  if (workspace_bytes < need || (need > 0 && !workspace)) return DSS_ERR_WORKSPACE;
  const int dev = check_device();
  if (dev != DSS_OK) return dev;

  dss::RenormParams p;
  p.in = in;
  p.out = out;
  p.rows = rows;
  p.vocab = vocab;
  p.top_k_arr = top_k_arr;
  p.top_k = top_k;
  p.top_p_arr = top_p_arr;
  p.top_p = top_p;
  p.row_status = row_status;
  p.vec_ok = vec_ok;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e =
      plan.W > 0    ? dss::launch_split_renorm(kind, p, plan, workspace, st, timing_events())
      : rplan.W > 0 ? dss::launch_resident_renorm(p, rplan, workspace, st, timing_events())
                    : dss::launch_stream_renorm(kind, p, st, timing_events());
  return e == hipSuccess ? DSS_OK : DSS_ERR_HIP;
}

}  // namespace

namespace dss {
uint64_t spin_limit_ticks() { return g_spin_ticks.load(std::memory_order_relaxed); }
int handoff_test_mode() { return g_handoff_test.load(std::memory_order_relaxed); }
int forced_split_slices() { return g_split_slices.load(std::memory_order_relaxed); }
}  // namespace dss

// Scratch of the allocation-free entry point: one array per GPU the library
// runs on, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol); it
// uses the device address that hipGetSymbolAddress returns for the current
// device, looked up once per device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (nullptr on failure).
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}
}  // namespace

DSS_EXPORT int dss_sampling_from_probs(const float* probs, int32_t rows, int32_t vocab,
                                       const int32_t* indices, int32_t num_outputs,
                                       const uint64_t* seed_arr, uint64_t seed,
                                       const uint64_t* offset_arr, uint64_t offset,
                                       int32_t* samples, uint8_t* valid, int32_t* rounds,
                                       uint32_t flags, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  return sample_common(dss::kOpNone, probs, rows, vocab, indices, num_outputs, seed_arr, seed,
                       offset_arr, offset, nullptr, 0, nullptr, 0.0f, nullptr, 0.0f, samples,
                       valid, rounds, flags, workspace, workspace_bytes, stream, timing_events());
}

DSS_EXPORT int dss_top_k_sampling_from_probs(const float* probs, int32_t rows, int32_t vocab,
                                             const int32_t* indices, int32_t num_outputs,
                                             const uint64_t* seed_arr, uint64_t seed,
                                             const uint64_t* offset_arr, uint64_t offset,
                                             const int32_t* top_k_arr, int32_t top_k,
                                             int32_t* samples, uint8_t* valid, int32_t* rounds,
                                             uint32_t flags, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  return sample_common(dss::kOpTopK, probs, rows, vocab, indices, num_outputs, seed_arr, seed,
                       offset_arr, offset, top_k_arr, top_k, nullptr, 0.0f, nullptr, 0.0f,
                       samples, valid, rounds, flags, workspace, workspace_bytes, stream, timing_events());
}

DSS_EXPORT int dss_top_p_sampling_from_probs(const float* probs, int32_t rows, int32_t vocab,
                                             const int32_t* indices, int32_t num_outputs,
                                             const uint64_t* seed_arr, uint64_t seed,
                                             const uint64_t* offset_arr, uint64_t offset,
                                             const float* top_p_arr, float top_p,
                                             int32_t* samples, uint8_t* valid, int32_t* rounds,
                                             uint32_t flags, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  return sample_common(dss::kOpTopP, probs, rows, vocab, indices, num_outputs, seed_arr, seed,
                       offset_arr, offset, nullptr, 0, top_p_arr, top_p, nullptr, 0.0f,
                       samples, valid, rounds, flags, workspace, workspace_bytes, stream, timing_events());
}

DSS_EXPORT int dss_min_p_sampling_from_probs(const float* probs, int32_t rows, int32_t vocab,
                                             const int32_t* indices, int32_t num_outputs,
                                             const uint64_t* seed_arr, uint64_t seed,
                                             const uint64_t* offset_arr, uint64_t offset,
                                             const float* min_p_arr, float min_p,
                                             int32_t* samples, uint8_t* valid, int32_t* rounds,
                                             uint32_t flags, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  return sample_common(dss::kOpMinP, probs, rows, vocab, indices, num_outputs, seed_arr, seed,
                       offset_arr, offset, nullptr, 0, nullptr, 0.0f, min_p_arr, min_p,
                       samples, valid, rounds, flags, workspace, workspace_bytes, stream, timing_events());
}

DSS_EXPORT int dss_top_k_top_p_sampling_from_probs(
    const float* probs, int32_t rows, int32_t vocab, const int32_t* indices, int32_t num_outputs,
    const uint64_t* seed_arr, uint64_t seed, const uint64_t* offset_arr, uint64_t offset,
    const int32_t* top_k_arr, int32_t top_k, const float* top_p_arr, float top_p,
    int32_t* samples, uint8_t* valid, int32_t* rounds, uint32_t flags, void* workspace,
    size_t workspace_bytes, void* stream) {
  return sample_common(dss::kOpTopKTopP, probs, rows, vocab, indices, num_outputs, seed_arr,
                       seed, offset_arr, offset, top_k_arr, top_k, top_p_arr, top_p, nullptr,
                       0.0f, samples, valid, rounds, flags, workspace, workspace_bytes, stream, timing_events());
}

DSS_EXPORT int dss_top_k_top_p_sampling_from_probs_noalloc(
    const float* probs, int32_t rows, int32_t vocab, const int32_t* indices, int32_t num_outputs,
    const uint64_t* seed_arr, uint64_t seed, const uint64_t* offset_arr, uint64_t offset,
    const int32_t* top_k_arr, int32_t top_k, const float* top_p_arr, float top_p,
    int32_t* samples, uint8_t* valid, int32_t* rounds, uint32_t flags, void* stream) {
  // every host check of the call first (no HIP call; the workspace pointer
  // is only tested for NULL there), then the scratch's size
  const int chk = sample_common(dss::kOpTopKTopP, probs, rows, vocab, indices, num_outputs,
                                seed_arr, seed, offset_arr, offset, top_k_arr, top_k, top_p_arr,
                                top_p, nullptr, 0.0f, samples, valid, rounds, flags,
                                reinterpret_cast<void*>(static_cast<uintptr_t>(256)),
                                SIZE_MAX, stream, timing_events(), true);
  if (chk != DSS_OK || num_outputs == 0) return chk;
  if (dss_workspace_size(DSS_OP_TOP_K_TOP_P, rows, vocab, num_outputs, flags) > kScratchBytes)
    return DSS_ERR_WORKSPACE;
  const int dev = check_device();
  if (dev != DSS_OK) return dev;
  void* ws = scratch_address();
  if (ws == nullptr) return DSS_ERR_HIP;
  return sample_common(dss::kOpTopKTopP, probs, rows, vocab, indices, num_outputs, seed_arr, seed,
                       offset_arr, offset, top_k_arr, top_k, top_p_arr, top_p, nullptr, 0.0f,
                       samples, valid, rounds, flags, ws, kScratchBytes, stream, timing_events(),
                       false, true);
}

DSS_EXPORT int dss_top_k_renorm_probs(const float* probs, float* out, int32_t rows, int32_t vocab,
                                      const int32_t* top_k_arr, int32_t top_k,
                                      uint8_t* row_status, uint32_t flags, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return renorm_common(dss::kRenormTopK, DSS_OP_TOP_K_RENORM, probs, out, rows, vocab, top_k_arr,
                       top_k, nullptr, 0.0f, row_status, flags, workspace, workspace_bytes,
                       stream);
}

DSS_EXPORT int dss_top_p_renorm_probs(const float* probs, float* out, int32_t rows, int32_t vocab,
                                      const float* top_p_arr, float top_p, uint8_t* row_status,
                                      uint32_t flags, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return renorm_common(dss::kRenormTopP, DSS_OP_TOP_P_RENORM, probs, out, rows, vocab, nullptr,
                       0, top_p_arr, top_p, row_status, flags, workspace, workspace_bytes,
                       stream);
}

DSS_EXPORT int dss_top_k_mask_logits(const float* logits, float* out, int32_t rows,
                                     int32_t vocab, const int32_t* top_k_arr, int32_t top_k,
                                     uint8_t* row_status, uint32_t flags, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return renorm_common(dss::kMaskLogits, DSS_OP_TOP_K_MASK_LOGITS, logits, out, rows, vocab,
                       top_k_arr, top_k, nullptr, 0.0f, row_status, flags, workspace,
                       workspace_bytes, stream);
}

DSS_EXPORT int dss_softmax(const float* logits, float* probs, int32_t rows, int32_t vocab,
                           const float* temperature_arr, float temperature, uint8_t* row_status,
                           uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (flags & ~DSS_FLAGS_ALL) return DSS_ERR_INVALID_ARG;
  if (rows < 0 || vocab <= 0) return DSS_ERR_INVALID_ARG;
  if (vocab > DSS_MAX_VOCAB) return DSS_ERR_UNSUPPORTED;
  if (rows == 0) return DSS_OK;
  if (!logits || !probs) return DSS_ERR_INVALID_ARG;
  const int vec_ok = (vocab % 4 == 0) && aligned16(logits) && aligned16(probs);
  const size_t need = dss_workspace_size(DSS_OP_SOFTMAX, rows, vocab, rows, flags);
  if (workspace_bytes < need || (need > 0 && !workspace)) return DSS_ERR_WORKSPACE;
  const int dev = check_device();
  if (dev != DSS_OK) return dev;
  const dss::SoftmaxParams q{logits, probs, rows, vocab, temperature_arr, temperature, row_status,
                             vec_ok};
  return dss::launch_softmax(q, dss::plan_softmax(rows, vocab, flags, vec_ok), workspace,
                             static_cast<hipStream_t>(stream), timing_events()) == hipSuccess
             ? DSS_OK
             : DSS_ERR_HIP;
}

DSS_EXPORT int dss_top_k_top_p_sampling_from_logits(
    const float* logits, int32_t rows, int32_t vocab, const int32_t* indices, int32_t num_outputs,
    const uint64_t* seed_arr, uint64_t seed, const uint64_t* offset_arr, uint64_t offset,
    const int32_t* top_k_arr, int32_t top_k, const float* top_p_arr, float top_p,
    const float* temperature_arr, float temperature, int32_t* samples, uint8_t* valid,
    int32_t* rounds, uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (flags & ~DSS_FLAGS_ALL) return DSS_ERR_INVALID_ARG;
  if (rows < 0 || vocab <= 0 || num_outputs < 0) return DSS_ERR_INVALID_ARG;
  if (vocab > DSS_MAX_VOCAB) return DSS_ERR_UNSUPPORTED;
  if (!indices && num_outputs != rows) return DSS_ERR_INVALID_ARG;
  if (num_outputs == 0) return DSS_OK;
  if (!logits || !samples) return DSS_ERR_INVALID_ARG;
  const size_t eng = logits_engine_bytes(rows, vocab, num_outputs, flags);
  const size_t need = dss_workspace_size(DSS_OP_TOP_K_TOP_P_FROM_LOGITS, rows, vocab, num_outputs,
                                         flags);
  if (workspace_bytes < need || !workspace) return DSS_ERR_WORKSPACE;
  float* probs = reinterpret_cast<float*>(static_cast<char*>(workspace) + eng);
  const dss::LaunchEvents ev = timing_events();
  const int vec_ok = (vocab % 4 == 0) && aligned16(logits);
  if (logits_fused(rows, vocab, num_outputs, top_k_arr, top_k, flags, vec_ok)) {
    // one kernel: the softmax rides inside the split engine's pass (the
    // probabilities area only takes rows that fall back)
    return sample_common(dss::kOpTopKTopP, logits, rows, vocab, indices, num_outputs, seed_arr,
                         seed, offset_arr, offset, top_k_arr, top_k, top_p_arr, top_p, nullptr,
                         0.0f, samples, valid, rounds, flags, workspace, eng, stream, ev, false,
                         false, temperature_arr, temperature, probs);
  }
  // every check of the sampling call before anything is enqueued
  const int chk = sample_common(dss::kOpTopKTopP, probs, rows, vocab, indices, num_outputs, seed_arr,
                                seed, offset_arr, offset, top_k_arr, top_k, top_p_arr, top_p,
                                nullptr, 0.0f, samples, valid, rounds, flags, workspace, eng,
                                stream, ev, true);
  if (chk != DSS_OK) return chk;
  const int dev = check_device();
  if (dev != DSS_OK) return dev;
  // probabilities into the workspace (invalid rows come out NaN-filled, which
  // the sampling call reports as invalid outputs), then the sampling call;
  // the timing events span both kernels
  const dss::SoftmaxParams q{logits, probs, rows, vocab, temperature_arr, temperature, nullptr,
                             vec_ok};
  const hipError_t e = dss::launch_softmax(q, dss::plan_softmax(rows, vocab, flags, vec_ok),
                                           workspace, static_cast<hipStream_t>(stream),
                                           dss::LaunchEvents{ev.start, nullptr});
  if (e != hipSuccess) return DSS_ERR_HIP;
  return sample_common(dss::kOpTopKTopP, probs, rows, vocab, indices, num_outputs, seed_arr, seed,
                       offset_arr, offset, top_k_arr, top_k, top_p_arr, top_p, nullptr, 0.0f,
                       samples, valid, rounds, flags, workspace, eng, stream,
                       dss::LaunchEvents{nullptr, ev.stop});
}

DSS_EXPORT int dss_top_k(const float* x, int32_t rows, int32_t vocab, int32_t k, float* values,
                         int32_t* indices, uint8_t* row_status, uint32_t flags, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (flags & ~DSS_FLAGS_ALL) return DSS_ERR_INVALID_ARG;
  if (rows < 0 || vocab <= 0 || k < 1 || k > vocab) return DSS_ERR_INVALID_ARG;
  if (vocab > DSS_MAX_VOCAB || k > dss::kSelectMax) return DSS_ERR_UNSUPPORTED;
  if (rows == 0) return DSS_OK;
  if (!x || !values || !indices) return DSS_ERR_INVALID_ARG;
  const int vec = (vocab % 4 == 0) && aligned16(x);
  const dss::SplitPlan plan = dss::plan_split_select(rows, vocab, k, flags, vec);
  if (workspace_bytes < plan.workspace || (plan.workspace > 0 && !workspace))
    return DSS_ERR_WORKSPACE;
  const int dev = check_device();
  if (dev != DSS_OK) return dev;
  const dss::SelectParams q{x, values, indices, rows, vocab, k, row_status, vec};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (plan.W > 0) {
    e = dss::launch_split_select(q, plan, workspace, s, timing_events());
  } else {
    e = dss::launch_select(q, s, timing_events());
  }
  return e == hipSuccess ? DSS_OK : DSS_ERR_HIP;
}

DSS_EXPORT int dss_chain_speculative_sampling(
    const float* draft_probs, const int32_t* draft_token_ids, const float* target_probs,
    int32_t rows, int32_t num_draft, int32_t vocab, const uint64_t* seed_arr, uint64_t seed,
    const uint64_t* offset_arr, uint64_t offset, int32_t* output_tokens, int32_t* accepted,
    uint8_t* valid, uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (flags & ~DSS_FLAGS_ALL) return DSS_ERR_INVALID_ARG;
  if (rows < 0 || vocab <= 0 || num_draft < 0) return DSS_ERR_INVALID_ARG;
  if (vocab > DSS_MAX_VOCAB || num_draft > dss::kSpecMaxN) return DSS_ERR_UNSUPPORTED;
  if (rows == 0) return DSS_OK;
  if (!target_probs || !output_tokens || !accepted) return DSS_ERR_INVALID_ARG;
  if (num_draft > 0 && (!draft_probs || !draft_token_ids)) return DSS_ERR_INVALID_ARG;
  const int vec = vocab % 4 == 0 && aligned16(target_probs) &&
                  (num_draft == 0 || aligned16(draft_probs));
  const dss::SpecPlan plan = dss::plan_spec(rows, vocab, num_draft, vec);
  if (plan.W == 0) return DSS_ERR_UNSUPPORTED;
  if (workspace_bytes < plan.workspace || (plan.workspace > 0 && !workspace))
    return DSS_ERR_WORKSPACE;
  const int dev = check_device();
  if (dev != DSS_OK) return dev;
  const dss::SpecParams sp{draft_probs, draft_token_ids, target_probs, rows, num_draft, vocab,
                           seed_arr, seed, offset_arr, offset, output_tokens, accepted, valid};
  return dss::launch_spec(sp, plan, workspace, static_cast<hipStream_t>(stream),
                          timing_events()) == hipSuccess
             ? DSS_OK
             : DSS_ERR_HIP;
}

DSS_EXPORT size_t dss_workspace_size(int32_t op, int32_t rows, int32_t vocab,
                                     int32_t num_outputs, uint32_t flags) {
  // sized for 16-byte aligned rows; an unaligned call runs the streaming
  // engine, which needs none
  if (vocab <= 0) return 0;
  const int vec = vocab % 4 == 0;
  if (op == DSS_OP_TOP_K_RENORM || op == DSS_OP_TOP_K_MASK_LOGITS) {
    if (rows <= 0) return 0;
    const int kind = op == DSS_OP_TOP_K_RENORM ? dss::kRenormTopK : dss::kMaskLogits;
    return dss::plan_split_renorm(kind, rows, vocab, flags, vec).workspace;
  }
  if (op == DSS_OP_CHAIN_SPECULATIVE) {
    // num_outputs is the number of draft tokens per row here
    if (rows <= 0) return 0;
    return dss::plan_spec(rows, vocab, num_outputs, vec).workspace;
  }
  if (op == DSS_OP_TOP_K_SELECT) {
    if (rows <= 0) return 0;
    return dss::plan_split_select(rows, vocab, 1, flags, vec).workspace;
  }
  if (op == DSS_OP_TOP_P_RENORM) {
    if (rows <= 0) return 0;
    return dss::plan_resident(dss::kOpTopP, vocab, rows, flags, vec).workspace;
  }
  if (op == DSS_OP_SOFTMAX) {
    if (rows <= 0) return 0;
    return dss::plan_softmax(rows, vocab, flags, vec).workspace;
  }
  if (op == DSS_OP_TOP_K_TOP_P_FROM_LOGITS) {
    // the engines' area, then probabilities: one row per input row (written
    // before sampling), or per output (the fused path's fallback rows)
    if (rows <= 0 || num_outputs <= 0) return 0;
    const size_t n = (size_t)(rows > num_outputs ? rows : num_outputs);
    return logits_engine_bytes(rows, vocab, num_outputs, flags) + align256(n * (size_t)vocab * 4);
  }
  if (op < DSS_OP_SAMPLING || op > DSS_OP_TOP_K_TOP_P || num_outputs <= 0) return 0;
  // top-k ops may run on either engine (the choice can depend on k)
  const dss::SplitPlan plan = dss::plan_split(op, rows, vocab, num_outputs, flags, vec);
  size_t res = dss::plan_resident(op, vocab, num_outputs, flags, vec).workspace;
  // top-k then top-p with a scalar k may take the pair search's plans, which
  // reach larger vocabularies
  if (op == DSS_OP_TOP_K_TOP_P) {
    const size_t rp =
        dss::plan_resident(dss::kOpTopKTopP, vocab, num_outputs, flags, vec, true, true).workspace;
    res = rp > res ? rp : res;
  }
  return plan.W > 0 && plan.workspace > res ? plan.workspace : res;
}

DSS_EXPORT int32_t dss_set_timing_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return DSS_ERR_INVALID_ARG;
  g_ev_start.store(start, std::memory_order_relaxed);
  g_ev_stop.store(stop, std::memory_order_relaxed);
  return DSS_OK;
}

DSS_EXPORT int32_t dss_set_spin_limit(uint64_t ticks) {
  g_spin_ticks.store(ticks == UINT64_MAX ? dss::kDefaultSpinTicks : ticks,
                     std::memory_order_relaxed);
  return DSS_OK;
}

DSS_EXPORT int32_t dss_set_handoff_test(int32_t mode) {
  if (mode != 0 && mode != 1) return DSS_ERR_INVALID_ARG;
  g_handoff_test.store(mode, std::memory_order_relaxed);
  return DSS_OK;
}

DSS_EXPORT int32_t dss_set_split_slices(int32_t slices) {
  if (slices != 0 && (slices < 1 || slices > 16 || (slices & (slices - 1)) != 0))
    return DSS_ERR_INVALID_ARG;
  g_split_slices.store(slices, std::memory_order_relaxed);
  return DSS_OK;
}

DSS_EXPORT int32_t dss_workspace_status(const void* workspace, size_t workspace_bytes,
                                        uint8_t* broken, void* stream) {
  if (workspace_bytes > 0 && workspace == nullptr) return DSS_ERR_INVALID_ARG;
  const int slots = workspace_bytes >= dss::kFixedRegionBytes ? dss::kResidentSlots : 0;
  if (broken) std::memset(broken, 0, dss::kResidentSlots);
  if (slots == 0) return 0;
  const int dev = check_device();
  if (dev != DSS_OK) return dev;
  // the arrival counter of every resident slot (its first word), strided
  uint32_t ctr[dss::kResidentSlots];
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpy2DAsync(ctr, sizeof(uint32_t),
                       static_cast<const char*>(workspace) + dss::kCtlRegionBytes,
                       dss::kResidentSlotBytes, sizeof(uint32_t), slots, hipMemcpyDeviceToHost,
                       st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return DSS_ERR_HIP;
  int n = 0;
  for (int q = 0; q < slots; ++q) {
    const bool b = (ctr[q] & 0x80000000u) != 0u;
    n += b ? 1 : 0;
    if (broken) broken[q] = b ? 1 : 0;
  }
  return n;
}

DSS_EXPORT int32_t dss_stream_read_reference(const float* x, int64_t n, uint32_t* out_max,
                                             void* stream) {
  if (n < 0 || (n % 4) != 0 || (n > 0 && (x == nullptr || !aligned16(x))) || out_max == nullptr)
    return DSS_ERR_INVALID_ARG;
  const int dst = check_device();
  if (dst != DSS_OK) return dst;
  return dss::launch_stream_read(x, n, out_max, static_cast<hipStream_t>(stream),
                                timing_events()) == hipSuccess
             ? DSS_OK
             : DSS_ERR_HIP;
}

DSS_EXPORT const char* dss_strerror(int32_t status) {
  switch (status) {
    case DSS_OK: return "ok";
    case DSS_ERR_INVALID_ARG: return "invalid argument";
    case DSS_ERR_WORKSPACE: return "workspace missing or too small";
    case DSS_ERR_UNSUPPORTED: return "unsupported configuration";
    case DSS_ERR_HIP: return "HIP runtime error";
    case DSS_ERR_DEVICE: return "current device is not gfx950";
    default: return "unknown status";
  }
}

DSS_EXPORT int32_t dss_version(void) { return 100; }
