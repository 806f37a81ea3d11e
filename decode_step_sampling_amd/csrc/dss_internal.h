// Internal declarations shared by the host ABI and the kernel translation
// units of libdss.so.  Not installed; the public interface is include/dss.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dss.h"
#include "dss_hooks.h"

namespace dss {

// Filter ids used as template parameters by the sampling kernels.
enum Op : int {
  kOpNone = 0,      // plain inverse-transform sampling
  kOpTopK = 1,
  kOpTopP = 2,
  kOpMinP = 3,
  kOpTopKTopP = 4,  // top-k first, then top-p inside the top-k set
  kOpTopKTopPJoint = 5,  // both checks in every round, top-p against the row's mass
};

// Everything a sampling kernel reads or writes.  Pointer fields are device
// memory; a NULL parameter array means "use the scalar".
struct SampleParams {
  const float* probs;
  int32_t rows;
  int32_t vocab;
  const int32_t* indices;
  int32_t num_outputs;
  const uint64_t* seed_arr;
  uint64_t seed;
  const uint64_t* offset_arr;
  uint64_t offset;
  const int32_t* top_k_arr;
  int32_t top_k;
  const float* top_p_arr;
  float top_p;
  const float* min_p_arr;
  float min_p;
  int32_t* samples;
  uint8_t* valid;
  int32_t* rounds;
  int32_t vec_ok;   // rows may be read with 16-byte loads
  int32_t single_pivot;  // streaming loop: low <- pivot1 after each rejection
  // sampling from logits (split engine): `probs` holds logits z, the filters
  // apply to softmax(z / T), T per row (temp_arr) or one scalar
  const float* temp_arr;
  float temp;
  float* prob_buf;  // [num_outputs][vocab] probabilities of an output that falls back
};

enum RenormKind : int { kRenormTopK = 0, kRenormTopP = 1, kMaskLogits = 2 };

struct RenormParams {
  const float* in;
  float* out;
  int32_t rows;
  int32_t vocab;
  const int32_t* top_k_arr;
  int32_t top_k;
  const float* top_p_arr;
  float top_p;
  uint8_t* row_status;
  int32_t vec_ok;
};

// Optional kernel-timing events (dss_set_timing_events): the first kernel of
// a call records `start` when it begins executing and the last records
// `stop` when it ends (hipExtLaunchKernel dispatch events).  NULL: none.
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};

// Longest wait of a resident row barrier, in ticks of the 100 MHz constant
// clock (dss_set_spin_limit; 50 ms unless changed).
uint64_t spin_limit_ticks();
// 1 (dss_set_handoff_test): every split-engine hand-off is treated as
// foreign, so its outputs take the in-kernel fallback (a test setting)
int handoff_test_mode();
constexpr uint64_t kDefaultSpinTicks = 5000000ull;
// Slices per output the split engine must use (dss_set_split_slices; 0: its
// own choice).
int forced_split_slices();

// Launch kernel on stream s, attaching the dispatch events of ev that apply
// (start if first, stop if last).
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t s, const LaunchEvents& ev,
                          bool first, bool last, Args... args) {
  hipEvent_t a = first ? ev.start : nullptr, b = last ? ev.stop : nullptr;
  if (a || b) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, a, b, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  }
}

// Streaming engine: one 1024-thread work-group per output (or row), every
// pass reads the row from global memory.  Returns a hipError_t.
hipError_t launch_stream_sample(int op, const SampleParams& p, hipStream_t s, const LaunchEvents& ev);
// min-p sampling in two reads of each row (per-tile maxima first; tiles that
// hold no kept value are not read again), one draw, rounds = 1
hipError_t launch_stream_minp(const SampleParams& p, hipStream_t s, const LaunchEvents& ev);
hipError_t launch_stream_renorm(int kind, const RenormParams& p, hipStream_t s,
                                const LaunchEvents& ev);

// Split-row engine (top-k and top-k-then-top-p sampling): W work-groups per
// output on one XCD, one HBM read of the row, candidates handed to the last
// work-group through the caller's workspace.  W == 0 means "not eligible".
struct SplitPlan {
  int W;             // slices per output
  int L;             // slice length (values, multiple of 4)
  int nv;            // 16-byte loads per thread per slice
  int chunk;         // outputs per launch
  size_t handoff;    // bytes of the hand-off area (counters, headers, lists)
  size_t workspace;  // bytes of workspace needed in all (hand-off + results)
};
SplitPlan plan_split(int op, int rows, int vocab, int num_outputs, uint32_t flags, int vec_ok);
hipError_t launch_split_sample(int op, const SampleParams& p, const SplitPlan& plan,
                               void* workspace, hipStream_t s, const LaunchEvents& ev);

// Top-k-then-top-p sampling from logits on the split engine, softmax fused:
// the slices' maxima and sums of exponentials ride with the hand-off, and
// the finishing work-group turns the candidates into probabilities.  Plans
// as plan_split; the workspace also holds p.prob_buf (logits_fallback_bytes).
hipError_t launch_split_logits(int op, const SampleParams& p, const SplitPlan& plan,
                               void* workspace, hipStream_t s, const LaunchEvents& ev);

// Split-row top-k renormalisation / logit masking (kind kRenormTopK or
// kMaskLogits): the split engine finds tau_k and Z_k per row, a second kernel
// writes the rows.  W == 0 means "not eligible" (streaming engine instead).
SplitPlan plan_split_renorm(int kind, int rows, int vocab, uint32_t flags, int vec_ok);
hipError_t launch_split_renorm(int kind, const RenormParams& p, const SplitPlan& plan,
                               void* workspace, hipStream_t s, const LaunchEvents& ev);

// Workspace layout shared by every op, so that calls of any kind can use one
// workspace: [0, kCtlRegionBytes) the split engine's arrival counters and
// generation numbers; then kResidentSlots per-output slots of the resident
// engine (zero between calls); then the split engine's hand-off area and
// per-row results (written before they are read).
constexpr size_t kCtlRegionBytes = 16384;
constexpr int kResidentSlots = 256;  // outputs (and work-groups) of one resident launch at most
constexpr size_t kResidentSlotBytes = 67840;
// A scalar top-k whose sets would crowd the split engine's lists goes to the
// resident engine: k above the split cap (2048), or k * W above half of the
// 8192 candidates a row's merge holds (flat rows would overflow them).
constexpr int kSplitKCapHost = 2048;
constexpr int kSplitScalarKW = 4096;
constexpr int kResidentSegKeys = 8192;  // boundary-bin keys one work-group may publish
constexpr size_t kFixedRegionBytes = kCtlRegionBytes + (size_t)kResidentSlots * kResidentSlotBytes +
                                     (size_t)kResidentSlots * kResidentSegKeys * 4;
// The split-row hand-off area after the fixed region: per output and slice a
// header of kSplitHdrWords words, then a list of kSplitListEntries entries;
// at most kSplitChunk outputs per launch (the arrival counters and
// generation numbers of the control region).
constexpr int kSplitHdrWords = 32;
constexpr int kSplitListEntries = 4096;
constexpr int kSplitChunk = 2048;

// Resident-slice engine (plain, top-p and min-p sampling; top-p
// renormalisation): W work-groups per output on one XCD keep the row in
// registers and meet at row barriers.  W == 0 means "not eligible".
// sample: the plan of a sampling call (plain, top-p and min-p may then hold
// 64 values per thread); renormalisation and the softmax keep at most 48.
// pairs: top-k then top-p by the one search on (count, mass) pairs
// (resident_pairs), which may hold 64 values per thread too.
SplitPlan plan_resident(int op, int vocab, int num_outputs, uint32_t flags, int vec_ok,
                        bool sample = false, bool pairs = false);
// Top-k then top-p on the resident engine by the one search on (count,
// mass) pairs: a scalar k whose values above the top-k boundary bin (fewer
// than k) fit one key list, and a row of fewer than 2^20 values (a bin's
// count fills 20 bits of the packed pair).
inline bool resident_pairs(int op, const int32_t* top_k_arr, int top_k, int vocab) {
  return op == kOpTopKTopP && top_k_arr == nullptr && top_k <= kResidentSegKeys && vocab < (1 << 20);
}
hipError_t launch_resident_sample(int op, const SampleParams& p, const SplitPlan& plan,
                                  void* workspace, hipStream_t s, const LaunchEvents& ev);
hipError_t launch_resident_renorm(const RenormParams& p, const SplitPlan& plan, void* workspace,
                                  hipStream_t s, const LaunchEvents& ev);
// Zero the slots of workspace whose row barrier was given up (broken mark).
hipError_t launch_resident_repair(void* workspace, hipStream_t s);

// Probabilities from logits with a temperature, p = softmax(z / T) per row
// (T per row or one scalar); invalid rows are NaN-filled with status 1.
struct SoftmaxParams {
  const float* in;
  float* out;
  int32_t rows;
  int32_t vocab;
  const float* temp_arr;
  float temp;
  uint8_t* row_status;
  int32_t vec_ok;
};
// W == 0: the one-work-group-per-row streaming kernel runs instead
SplitPlan plan_softmax(int rows, int vocab, uint32_t flags, int vec_ok);
hipError_t launch_softmax(const SoftmaxParams& p, const SplitPlan& plan, void* workspace,
                          hipStream_t s, const LaunchEvents& ev);
hipError_t launch_stream_softmax(const SoftmaxParams& p, hipStream_t s, const LaunchEvents& ev);

// Top-k selection: per row the k largest values (descending, equal values by
// ascending index) and their indices; one work-group per row.
constexpr int kSelectMax = 4096;
struct SelectParams {
  const float* in;
  float* values;    // [rows][k]
  int32_t* indices; // [rows][k]
  int32_t rows;
  int32_t vocab;
  int32_t k;
  uint8_t* row_status;
  int32_t vec_ok;
};
hipError_t launch_select(const SelectParams& p, hipStream_t s, const LaunchEvents& ev);

// Chain speculative verification (spec_kernels.hip).
constexpr int kSpecMaxN = 64;             // draft tokens per row (one lane each)
constexpr int kSpecMaxW = 16;             // slices per row
constexpr int kSpecRowsPerLaunch = 2048;  // the split engine's counter block
struct SpecParams {
  const float* q;          // [rows][n][vocab] draft probabilities
  const int32_t* ids;      // [rows][n] draft tokens
  const float* p;          // [rows][n + 1][vocab] target probabilities
  int32_t rows, n, vocab;
  const uint64_t* seed_arr;
  uint64_t seed;
  const uint64_t* offset_arr;
  uint64_t offset;
  int32_t* tokens;         // [rows][n + 1]
  int32_t* accepted;       // [rows]
  uint8_t* valid;          // [rows], nullable
};
struct SpecPlan {
  int W;              // slices per row (0: not supported)
  int Lv;             // slice length in 16-byte vectors
  int CH;             // vectors of one wave's chunk
  int per_launch;     // rows per launch
  size_t workspace;   // bytes
  uint32_t* ctr;      // [kSpecRowsPerLaunch] arrival counters (zero between calls)
  uint32_t* gen;      // [kSpecRowsPerLaunch] generation numbers
  uint32_t* hdr;      // [per_launch][W][4]
  double* masses;     // [per_launch][W][16]
};
SpecPlan plan_spec(int rows, int vocab, int n, int vec_ok);
hipError_t launch_spec(const SpecParams& sp, const SpecPlan& plan, void* workspace,
                       hipStream_t s, const LaunchEvents& ev);
// Top-k selection on the split engine (k <= 2048): the top-k set that the
// engine gathers, sorted; rows whose lists overflow fall back to the
// one-work-group selection inside the same kernel.  W == 0: not eligible.
SplitPlan plan_split_select(int rows, int vocab, int k, uint32_t flags, int vec_ok);
hipError_t launch_split_select(const SelectParams& q, const SplitPlan& plan, void* workspace,
                               hipStream_t s, const LaunchEvents& ev);

// plain streaming read of n floats (n a multiple of 4, x 16-byte aligned);
// folds their maximum bit pattern into *out
hipError_t launch_stream_read(const float* x, int64_t n, uint32_t* out, hipStream_t s,
                              const LaunchEvents& ev);

}  // namespace dss
