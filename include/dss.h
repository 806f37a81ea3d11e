/*
 * dss.h -- sorting-free decode-step sampling on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libdss.so.  Plain pointers and sizes only.  Pages cited:
 *   [Blog] FlashInfer blog "Sorting-Free GPU Kernels for LLM Sampling"
 *          (Chinese translation "面向 LLM 采样的免排序 GPU 内核");
 *   [F4]   gpu-kernel-drills note "F4 讲解：不排序的 top-k / top-p";
 *   [Expl] charlestar explainer on FlashInfer Sorting-Free Sampling.
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ---------------------------------------------------------------------------
 * Memory.  Every array argument is DEVICE memory of the current HIP device:
 *   probabilities / logits, outputs, per-output parameter arrays, index maps,
 *   seed and offset arrays.  The caller allocates and owns all of them; the
 *   library keeps no pointer after it returns and allocates nothing.
 *   Row-major contiguous [rows, vocab] float32; row r starts at
 *   probs + (int64)r * vocab.  Any alignment is accepted; 16-byte aligned rows
 *   (vocab % 4 == 0 and a 16-byte aligned base) take the vector-load path.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Work is enqueued asynchronously; nothing synchronises the host.
 *
 * Workspace.  `workspace` / `workspace_bytes` is caller-owned device scratch
 *   of at least dss_workspace_size(...) bytes (NULL is fine when that is 0):
 *   the split-row engine's hand-off area (top-k and top-k-then-top-p
 *   sampling, top-k selection, chain speculative verification) and its
 *   per-row results (top-k renormalisation and top-k logit masking), and the
 *   resident engine's per-output control blocks and key lists (plain, top-p
 *   and min-p sampling, top-p renormalisation, and top-k sampling with one
 *   scalar k that would crowd the split engine's lists).  It must
 *   be zero-filled once when it is allocated; every call leaves its counters
 *   and control blocks at zero again when its kernels end (the rest is
 *   written before it is read), so a workspace can be reused by later calls
 *   on the same stream without clearing.  Two calls that run concurrently
 *   (different streams) need different workspaces.
 *
 * Co-residency.  The resident engine's work-groups of one output wait for
 *   each other inside the kernel, so each of its launches holds no more
 *   work-groups than the device keeps resident at once.  Work that runs
 *   concurrently on other streams can still hold compute units; a
 *   work-group that waits more than 50 ms reports its output invalid
 *   (sample -1, valid 0; renorm rows NaN) instead of hanging, and marks its
 *   control block broken: every later output that uses that block comes
 *   out invalid as well (never counted against stale state) until the
 *   workspace is zero-filled again; dss_workspace_status reports such
 *   blocks.  Callers that overlap other kernels with these ops can pass
 *   DSS_FLAG_STREAMING, whose engine never waits.
 *   The split engine waits in one case only: with per-output k arrays, a
 *   launch of more slices than one work-group per compute unit ends with one
 *   finishing work-group per output that waits for that output's slices
 *   (all placed before it in the grid) when its k is above 2048.  That wait
 *   is bounded too (50 ms); a finisher that gives up samples its output
 *   with the exact one-work-group passes instead, and leaves the control
 *   words balanced for later calls.
 *
 * Outputs of the sampling ops (length num_outputs):
 *   samples[i]  token id in [0, vocab), or -1 when output i is invalid;
 *   valid[i]    1 / 0 (nullable: pass NULL to skip) [Expl "退化分布必须可报告"];
 *   rounds[i]   number of draws the rejection loop used (nullable).
 *
 * Rows and outputs.  indices[i] maps output i to a probability row
 *   ([Expl "动态 batch 中的 RNG 所有权": several outputs may share a row); with
 *   indices == NULL, output i reads row i and num_outputs must equal rows.
 *   Per-output parameters: if the array pointer (top_k_arr, top_p_arr,
 *   min_p_arr) is non-NULL it holds num_outputs values (one per output,
 *   not per row); otherwise the scalar applies to every output.
 *
 * Random numbers ([Expl "Seed、offset 与 deterministic 的边界"]).  Each output
 *   owns the stream
 *     key = (seed_i, 0), counter = (offset_i, sid_i, r / 4, 0),
 *     u_r = (word[r % 4] of Philox4x64-10(counter, key)) >> 11, times 2^-53,
 *   for draws r = 0, 1, 2, ... (Philox4x64-10: Salmon et al., SC'11).
 *   seed_i = seed_arr ? seed_arr[i] : seed, offset_i likewise; sid_i = 0 when
 *   seed_arr is given (the stream then depends only on the request's own
 *   seed and offset, not on its batch position) and sid_i = i when one scalar
 *   seed serves the call.  The library never advances offsets: the caller
 *   must give every call a new offset.  Identical inputs and streams give
 *   identical outputs (fixed reduction order, no floating-point atomics).
 *
 * Data problems are reported per output / row, never as an error status:
 *   a row containing NaN, +-inf or any value with the sign bit set
 *   (including -0.0), or whose total is zero; top_k <= 0; NaN top_p / min_p;
 *   indices[i] outside [0, rows).  Sampling: samples[i] = -1, valid[i] = 0.
 *   Renorm / mask: the output row is NaN-filled and row_status[r] = 1
 *   (row_status nullable, 0 for good rows).
 *
 * Filter semantics (value-based, ties kept: the kept set is always the upper
 * set {x >= tau}; [F4 §⑥], [Expl "Tie 需要明确定义"]):
 *   top_k   tau = k-th largest value; k >= vocab keeps every token.
 *   top_p   tau = v_(m), m = min{r >= 1 : v_(1) + ... + v_(r) >= p * Z},
 *           v_(1) >= v_(2) >= ... the sorted row, Z its total
 *           ([Expl "Top-p"], [F4 §①-②]); p clamped to [0, 1].
 *   min_p   tau = min_p * max(row), exact product ([Blog "Min-P"]);
 *           min_p clamped to [0, 1].
 *   top_k_top_p (top-k first, [Blog] footnote 1, [Expl "Top-k 与 top-p 的组合
 *           顺序会改变分布"]): top-p applied inside the top-k set, Z being the
 *           top-k mass.
 *   The sampled distribution is p~_i = x_i / sum_{x_j >= tau} x_j on the kept
 *   set ([Expl "采样流水线究竟在计算什么"]); zero-probability tokens are never
 *   drawn.  Rows need not sum to one.
 *
 * Status codes (host validation runs before any HIP call):
 */
#ifndef DSS_H
#define DSS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSS_OK                  0
#define DSS_ERR_INVALID_ARG   (-1)  /* NULL required pointer, negative size, ... */
#define DSS_ERR_WORKSPACE     (-2)  /* workspace smaller than dss_workspace_size */
#define DSS_ERR_UNSUPPORTED   (-3)  /* vocab above DSS_MAX_VOCAB, joint order    */
#define DSS_ERR_HIP           (-4)  /* a HIP runtime call or launch failed       */
#define DSS_ERR_DEVICE        (-5)  /* current device is not gfx950             */

#define DSS_MAX_VOCAB  (1 << 20)

/* flags */
#define DSS_FLAG_ORDER_JOINT   0x1u  /* joint top-k/top-p order ([Blog] footnote 1):
                                        top_k_top_p sampling only, any other op
                                        returns DSS_ERR_UNSUPPORTED */
#define DSS_FLAG_FROM_ZERO     0x2u  /* run the rejection loop exactly as the
                                        blog's listing starts it: low = 0,
                                        high = max, whole row (no certified
                                        starting interval, no split rows)     */
#define DSS_FLAG_STREAMING     0x4u  /* force the one-work-group-per-row
                                        streaming engine                       */
#define DSS_FLAG_SINGLE_PIVOT  0x8u  /* sampling ops: single-pivot rounds
                                        ([Blog] "拒绝采样"; [Expl] "如何在不知道
                                        top-k 边界时拒绝错误样本"): from low = 0,
                                        low <- the rejected value, streaming
                                        engine; for comparing round counts
                                        with the dual-pivot loop.  Ignored by
                                        the renorm / mask ops                 */
#define DSS_FLAGS_ALL          0xFu

/* op ids for dss_workspace_size */
#define DSS_OP_SAMPLING          0
#define DSS_OP_TOP_K_SAMPLING    1
#define DSS_OP_TOP_P_SAMPLING    2
#define DSS_OP_MIN_P_SAMPLING    3
#define DSS_OP_TOP_K_TOP_P       4
#define DSS_OP_TOP_K_RENORM      5
#define DSS_OP_TOP_P_RENORM      6
#define DSS_OP_TOP_K_MASK_LOGITS 7
#define DSS_OP_TOP_K_TOP_P_FROM_LOGITS 8
#define DSS_OP_SOFTMAX           9
#define DSS_OP_TOP_K_SELECT     10
#define DSS_OP_CHAIN_SPECULATIVE 11  /* num_outputs = draft tokens per row */

/* Inverse-transform sampling from each output's row ([Blog "逆变换采样"],
 * [Expl "不带过滤时：inverse transform sampling"]): u ~ U[0,1) (draw r = 0),
 * return the first token j with F_j > u * Z, F the prefix sums in index order,
 * Z the row total.  rounds[i] = 1. */
int dss_sampling_from_probs(const float* probs, int32_t rows, int32_t vocab,
                            const int32_t* indices, int32_t num_outputs,
                            const uint64_t* seed_arr, uint64_t seed,
                            const uint64_t* offset_arr, uint64_t offset,
                            int32_t* samples, uint8_t* valid, int32_t* rounds,
                            uint32_t flags, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Top-k sampling by dual-pivot rejection sampling ([Blog "双枢轴拒绝采样"],
 * [Expl "Dual Pivot 怎样收缩范围"]); the output law is x_j / Z_k on the top-k
 * set ([Blog "拒绝采样器正确性的理论证明"]). */
int dss_top_k_sampling_from_probs(const float* probs, int32_t rows, int32_t vocab,
                                  const int32_t* indices, int32_t num_outputs,
                                  const uint64_t* seed_arr, uint64_t seed,
                                  const uint64_t* offset_arr, uint64_t offset,
                                  const int32_t* top_k_arr, int32_t top_k,
                                  int32_t* samples, uint8_t* valid, int32_t* rounds,
                                  uint32_t flags, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Top-p (nucleus) sampling by dual-pivot rejection sampling ([Blog "拒绝采样",
 * "双枢轴拒绝采样"]). */
int dss_top_p_sampling_from_probs(const float* probs, int32_t rows, int32_t vocab,
                                  const int32_t* indices, int32_t num_outputs,
                                  const uint64_t* seed_arr, uint64_t seed,
                                  const uint64_t* offset_arr, uint64_t offset,
                                  const float* top_p_arr, float top_p,
                                  int32_t* samples, uint8_t* valid, int32_t* rounds,
                                  uint32_t flags, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Min-p sampling ([Blog "Min-P"], [Expl "Min-p"]) through the same loop. */
int dss_min_p_sampling_from_probs(const float* probs, int32_t rows, int32_t vocab,
                                  const int32_t* indices, int32_t num_outputs,
                                  const uint64_t* seed_arr, uint64_t seed,
                                  const uint64_t* offset_arr, uint64_t offset,
                                  const float* min_p_arr, float min_p,
                                  int32_t* samples, uint8_t* valid, int32_t* rounds,
                                  uint32_t flags, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Fused top-k-then-top-p sampling ([Blog] footnote 1 "Top-K First"; [Expl
 * "Top-k 与 top-p 的组合顺序会改变分布"]): top-p applies inside the top-k set,
 * its mass target p * Z_k.  With DSS_FLAG_ORDER_JOINT both checks run
 * together in every rejection round ([Blog] footnote 1 "Joint"; [Expl], same
 * section) and the top-p target is p times the whole row's mass: the kept
 * set is {x >= max(tau_k, tau_p)}, tau_p the top-p threshold of the row. */
int dss_top_k_top_p_sampling_from_probs(const float* probs, int32_t rows, int32_t vocab,
                                        const int32_t* indices, int32_t num_outputs,
                                        const uint64_t* seed_arr, uint64_t seed,
                                        const uint64_t* offset_arr, uint64_t offset,
                                        const int32_t* top_k_arr, int32_t top_k,
                                        const float* top_p_arr, float top_p,
                                        int32_t* samples, uint8_t* valid, int32_t* rounds,
                                        uint32_t flags, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Allocation-free variant of dss_top_k_top_p_sampling_from_probs, for
 * callers that cannot allocate device memory or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, semantics and outputs (token for token: the same kernels
 * and streams) without workspace / workspace_bytes; the kernels' scratch is
 * a static device array of the library, 64 MiB on every GPU the library runs
 * on, held until the process ends.  A call whose
 * dss_workspace_size(DSS_OP_TOP_K_TOP_P, rows, vocab, num_outputs, flags)
 * exceeds 64 MiB returns DSS_ERR_WORKSPACE before anything is enqueued (the
 * headline shape, 64 rows of 151936, needs 34.2 MB; up to about 1000 slices
 * of the split engine fit).  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); the first call on a device looks
 * up the array's device address once.  Every call on one GPU shares the
 * array: calls that overlap on one GPU (concurrent streams, threads) race
 * and must be serialised by the caller.  The array is zero when the library
 * loads and the kernels leave it so; a resident control block whose wait
 * was given up ("Co-residency") is zeroed again by a small kernel before
 * the next call that uses the resident engine. */
int dss_top_k_top_p_sampling_from_probs_noalloc(const float* probs, int32_t rows, int32_t vocab,
                                                const int32_t* indices, int32_t num_outputs,
                                                const uint64_t* seed_arr, uint64_t seed,
                                                const uint64_t* offset_arr, uint64_t offset,
                                                const int32_t* top_k_arr, int32_t top_k,
                                                const float* top_p_arr, float top_p,
                                                int32_t* samples, uint8_t* valid, int32_t* rounds,
                                                uint32_t flags, void* stream);

/* Top-k renormalisation ([F4 §②-④], [Expl "只过滤/归一化"]):
 * out[r, i] = x_i / Z_kept if x_i >= tau_k else 0.  top_k_arr has `rows`
 * entries (per row).  out may equal probs (in place). */
int dss_top_k_renorm_probs(const float* probs, float* out, int32_t rows, int32_t vocab,
                           const int32_t* top_k_arr, int32_t top_k,
                           uint8_t* row_status, uint32_t flags,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Top-p renormalisation by a monotone threshold search on the float32 bit
 * pattern ([F4 §②-③, §⑤]).  top_p_arr has `rows` entries.  In place allowed. */
int dss_top_p_renorm_probs(const float* probs, float* out, int32_t rows, int32_t vocab,
                           const float* top_p_arr, float top_p,
                           uint8_t* row_status, uint32_t flags,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Keep the k largest logits, set the rest to -inf ([Expl "只过滤/归一化"]);
 * negative logits are ordered by value, not raw bits ([F4 §⑧]); ties at the
 * k-th value are kept; -0.0 equals +0.0.  A NaN logit invalidates the row;
 * +-inf logits are ordinary values.  top_k_arr has `rows` entries.  In place
 * allowed. */
int dss_top_k_mask_logits(const float* logits, float* out, int32_t rows, int32_t vocab,
                          const int32_t* top_k_arr, int32_t top_k,
                          uint8_t* row_status, uint32_t flags,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Probabilities from logits with a temperature ([Expl "采样流水线究竟在计算什么"]):
 * probs[r, i] = exp(z_i / T_r) / sum_j exp(z_j / T_r), computed as
 * float32((exp((z_i - m) / T) / S)) with m the row's largest logit and the
 * differences, exponentials and their sum S in float64 (subtracting m keeps
 * the exponentials in range; the formula is unchanged).  temperature_arr has
 * `rows` entries (NULL: the scalar for every row).  A NaN or +inf logit, a
 * row without a finite logit, or a temperature that is not a finite positive
 * number give a NaN row with row_status 1 (nullable); -inf logits get
 * probability 0.  probs may equal logits (in place).  The workspace is the
 * one of dss_workspace_size(DSS_OP_SOFTMAX, rows, vocab, rows, flags); only
 * DSS_FLAG_STREAMING changes anything (one work-group per row). */
int dss_softmax(const float* logits, float* probs, int32_t rows, int32_t vocab,
                const float* temperature_arr, float temperature, uint8_t* row_status,
                uint32_t flags, void* workspace, size_t workspace_bytes, void* stream);

/* Top-k-then-top-p sampling from logits with a temperature
 * (temperature_arr per ROW, `rows` entries): the softmax of [Expl
 * "采样流水线究竟在计算什么"] followed by the filters and the draw of
 * dss_top_k_top_p_sampling_from_probs, with the same indices, seeds,
 * parameters and flags.
 * Sequential order (the default), on the split engine: one kernel.  Top-k,
 * top-p and the draw compare values only with each other and with
 * fractions of their sums, so they are unchanged when every value is scaled
 * by one constant; the kernel ranks the logits themselves and applies the
 * filters to the softmax's weights w_i = float32(exp((z_i - m) / T)) (m the
 * row's largest logit) of its candidates only, never forming the normaliser
 * S.  Kept sets equal those of the float32 probabilities w_i / S except
 * where the one rounding of each makes or breaks a tie.
 * The joint order, DSS_FLAG_STREAMING / FROM_ZERO / SINGLE_PIVOT, a ragged
 * or unaligned row, and scalar k beyond the split engine's reach: dss_softmax
 * into the workspace first, then the sampling call on those probabilities.
 * An output the fused kernel cannot finish alone (k above 2048, overflowing
 * candidate lists) gets its row's probabilities written to the workspace and
 * is sampled exactly from them, inside the same kernel.
 * A NaN or +inf logit, no finite logit, or a temperature that is not a
 * finite positive number make the output invalid.  Workspace:
 * dss_workspace_size(DSS_OP_TOP_K_TOP_P_FROM_LOGITS, ...) bytes (the
 * engines' area, then max(rows, num_outputs) rows of probabilities),
 * zero-filled once like every workspace. */
int dss_top_k_top_p_sampling_from_logits(const float* logits, int32_t rows, int32_t vocab,
                                         const int32_t* indices, int32_t num_outputs,
                                         const uint64_t* seed_arr, uint64_t seed,
                                         const uint64_t* offset_arr, uint64_t offset,
                                         const int32_t* top_k_arr, int32_t top_k,
                                         const float* top_p_arr, float top_p,
                                         const float* temperature_arr, float temperature,
                                         int32_t* samples, uint8_t* valid, int32_t* rounds,
                                         uint32_t flags, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* Top-k selection ([Expl "选择 top-k 值本身"]: the values and indices, not a
 * sample): for every row the k largest entries, values[r, 0..k) in
 * descending order with equal values by ascending index (-0.0 equals +0.0),
 * indices[r, 0..k) their positions in the row; values and indices are
 * [rows, k] device arrays.  Any float32 input (probabilities or logits,
 * +-inf allowed); a NaN makes the row invalid (NaN values, index -1,
 * row_status 1, nullable).  1 <= k <= vocab, else DSS_ERR_INVALID_ARG;
 * k > 4096 is DSS_ERR_UNSUPPORTED.  For k <= 2048 on 16-byte aligned rows
 * of at least 1024 values the split engine runs (one read of the row, the
 * top-k set gathered as in sampling, then sorted); it needs the workspace of
 * dss_workspace_size(DSS_OP_TOP_K_SELECT, rows, vocab, rows, flags).
 * Otherwise, or with DSS_FLAG_STREAMING, one work-group per row (no
 * workspace).  Other flags are ignored. */
int dss_top_k(const float* x, int32_t rows, int32_t vocab, int32_t k, float* values,
              int32_t* indices, uint8_t* row_status, uint32_t flags, void* workspace,
              size_t workspace_bytes, void* stream);

/* Chain speculative verification ([Blog "社区采用和其他应用"] names chain
 * speculative sampling as a use of the same rejection sampling; the pages
 * give no algorithm, so the standard one is taken: Leviathan, Kalman &
 * Matias 2023, Chen et al. 2023).  Row r holds num_draft draft tokens
 * draft_token_ids[r, j] with draft distributions draft_probs[r, j, :] (q_j)
 * and num_draft + 1 target distributions target_probs[r, j, :] (p_j), all
 * C-contiguous device arrays, probabilities float32.  For j = 0, 1, ... the
 * draft d_j is accepted iff u_j * q_j(d_j) < p_j(d_j) (decided exactly),
 * u_j = draw r = j of the row's stream; at the first rejection j* one token
 * is drawn (draw r = num_draft) by inverse transform from the residual
 * max(0, p_j* - q_j*) (differences in float64), or from p_j* if that
 * residual is zero everywhere; if every draft is accepted the bonus token is
 * drawn (draw r = num_draft) from p_{num_draft}.  output_tokens[r, :]
 * (num_draft + 1 entries) = d_0 .. d_{j*-1}, the drawn token, then -1;
 * accepted[r] = j* (num_draft with the bonus); valid[r] = 1 (nullable).
 * Seeds and offsets as in the sampling calls (per row).  A draft id outside
 * [0, vocab), a negative / NaN / inf value among the examined p_j(d_j),
 * q_j(d_j) or in the rows the final draw reads, or a final row with zero
 * mass make the row invalid: tokens -1, accepted 0, valid 0.
 * 0 <= num_draft <= 64, else DSS_ERR_UNSUPPORTED; vocab % 4 == 0 and 16-byte
 * aligned probability arrays, else DSS_ERR_UNSUPPORTED.  Workspace:
 * dss_workspace_size(DSS_OP_CHAIN_SPECULATIVE, rows, vocab, num_draft,
 * flags); flags are reserved (pass 0).  Reads per row: 2 num_draft single
 * values, then the one row (bonus) or two rows (residual) the draw needs. */
int dss_chain_speculative_sampling(const float* draft_probs, const int32_t* draft_token_ids,
                                   const float* target_probs, int32_t rows, int32_t num_draft,
                                   int32_t vocab, const uint64_t* seed_arr, uint64_t seed,
                                   const uint64_t* offset_arr, uint64_t offset,
                                   int32_t* output_tokens, int32_t* accepted, uint8_t* valid,
                                   uint32_t flags, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Bytes of workspace an op needs for these sizes and flags (0 if none). */
size_t dss_workspace_size(int32_t op, int32_t rows, int32_t vocab,
                          int32_t num_outputs, uint32_t flags);

/* State of a workspace's resident control blocks: the number of slots
 * (0 .. 256) whose row barrier was given up (see "Co-residency" above);
 * broken (nullable, host memory of 256 bytes) receives one flag per slot.
 * Outputs that a later call maps to such a slot (output index modulo the
 * launch's chunk) come out invalid until the workspace is zero-filled again.
 * Reads the workspace on `stream` and waits for it (host-synchronous).
 * Returns a negative status for a NULL workspace with nonzero size or a
 * HIP failure; 0 for a workspace too small to hold the slots. */
int32_t dss_workspace_status(const void* workspace, size_t workspace_bytes, uint8_t* broken,
                             void* stream);

/* Static description of a status code. */
const char* dss_strerror(int32_t status);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t dss_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSS_H */
