/*
 * dss_hooks.h -- measurement and test hooks of libdss.so.
 *
 * Not part of the sampling ops (include/dss.h): these calls exist so that a
 * benchmark can time kernels without a profiler, compare the sampling
 * kernels with a plain read of the same bytes, and so that tests can force
 * the bounded waits to give up and the split engine's hand-off checks to
 * fail while every kernel still exits normally.  All are process-wide and take effect for later calls.
 */
#ifndef DSS_HOOKS_H
#define DSS_HOOKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Profiling hook (not part of the sampling path).  With two hipEvent_t
 * handles (passed as void*, both non-NULL), every later call of this process
 * attaches them to its kernels as dispatch events (hipExtLaunchKernel): the
 * first kernel of the call records `start` when it begins executing, the
 * last records `stop` when it ends, so hipEventElapsedTime(start, stop) is
 * the call's kernel time as a kernel-trace profiler reports it.  (NULL,
 * NULL) switches the hook off.  Process-wide; the caller owns the events
 * and must keep them alive while the hook is on.  Returns DSS_ERR_INVALID_ARG
 * if exactly one handle is NULL. */
int32_t dss_set_timing_events(void* start, void* stop);

/* Measurement aid (not part of the sampling path): one plain streaming read
 * of n floats at x (device, 16-byte aligned, n a multiple of 4): a
 * grid-stride loop of up to 2048 work-groups of 256 threads, one 16-byte
 * load per thread per iteration, folding the largest float32 bit
 * pattern into *out_max (device uint32, caller-initialised; atomicMax).
 * Its time is the read rate this GPU reaches for that many bytes, the
 * reference beside the sampling kernels' HBM fraction.  Enqueued on
 * `stream`.  DSS_ERR_INVALID_ARG for a bad size, pointer or alignment. */
int32_t dss_stream_read_reference(const float* x, int64_t n, uint32_t* out_max, void* stream);

/* Longest wait of a resident row barrier, and of a split-engine finishing
 * work-group for its slices, in ticks of the GPU's 100 MHz constant clock
 * (default 5,000,000 = 50 ms).  UINT64_MAX restores the default.  A small
 * limit makes waits give up: a resident output is reported invalid and its
 * control block marked broken (see dss.h "Co-residency"); a finishing
 * work-group samples its output with the exact one-work-group passes
 * instead.  0 makes every such wait give up at once.  For tests of those
 * paths only.  Always DSS_OK. */
int32_t dss_set_spin_limit(uint64_t ticks);

/* 1 makes every hand-off of the split-row engine look foreign (as if a
 * slice's header carried another generation or XCD), so every output whose
 * slices published lists or histograms is computed instead by the in-kernel
 * fallback of one work-group (the exact passes for top-k sampling, the
 * streaming engine otherwise); 0 restores normal hand-offs.  For tests that
 * the fallback fires and is correct; process-wide.  DSS_ERR_INVALID_ARG for
 * other values. */
int32_t dss_set_handoff_test(int32_t mode);

/* Slices per output of the split-row engine (a power of two, 1..16), for
 * measuring other choices than its own (about 256 work-groups in all); 0
 * restores its own choice.  A value the vocabulary needs more slices than
 * is raised to that minimum; the engine still halves it while a slice would
 * be empty.  Also applies to dss_workspace_size, so query the workspace
 * after setting it.  DSS_ERR_INVALID_ARG for other values. */
int32_t dss_set_split_slices(int32_t slices);

#ifdef __cplusplus
}
#endif

#endif /* DSS_HOOKS_H */
