/*
 * radamw.h -- C ABI of libradamw.so, the fused AdamW / AMSGrad optimizer
 * step for AMD Instinct MI355X (gfx950).
 *
 * Page abbreviations used in the citations below:
 *   FA-ja  = RUDA docs page "実験的なデバイス上の融合 AdamW / AMSGrad"
 *   FA-zh  = RUDA docs page "实验性融合 AdamW / AMSGrad"
 *   TR-zh  = RUDA docs page "训练与状态保存"
 *
 * General conventions (all entry points):
 *   - Every array pointer is a DEVICE pointer (hipMalloc / torch CUDA
 *     memory) unless the argument says "host".  Host pointers are rejected
 *     (FA-ja "サポートされている契約": no arbitrary host pointers).
 *   - Arrays are dense and contiguous, 1-D, indexed 0..n-1.  Parameters and
 *     moments are FP32; gradients are FP32, FP16 or BF16 (FA-zh
 *     "增加的实际能力").  Pointers must be aligned to their element size.
 *   - All device work is enqueued on `stream` (a hipStream_t; NULL is the
 *     legacy default stream) and is asynchronous: a RADAMW_OK return means
 *     the work was SUBMITTED, not that it completed (FA-ja "低レベルの使用").
 *     The caller keeps every buffer alive until the stream has passed the
 *     work, and synchronises before reading results or saving a checkpoint.
 *   - Any non-zero return other than RADAMW_ERR_HIP and RADAMW_ERR_DECISION
 *     means nothing was launched and nothing (device memory, state structs,
 *     step counts, output flags) was modified (FA-ja "低レベルの使用": validation leaves
 *     every input unchanged).  RADAMW_ERR_HIP reports a failing HIP runtime
 *     call; a multi-kernel entry point may have submitted earlier kernels,
 *     and the caller should treat the device state as unconfirmed (FA-ja
 *     "低レベルの使用": discard unconfirmed outputs after a device fault).
 *     The library keeps no pointer after a call returns, except a
 *     persistent tensor list (radamw_list_create), which keeps its
 *     segments' pointers until radamw_list_destroy.
 *   - There is no device-side step counter: the completed-step count lives
 *     in host memory owned by the caller, and the bias-correction
 *     coefficients are computed on the host for every call, so a captured
 *     graph replay would repeat one step's coefficients (FA-zh
 *     "增加的实际能力"); graph capture is not supported: a stream being
 *     captured is refused with RADAMW_ERR_INVALID before anything is
 *     launched or recorded.
 *   - Thread safety: calls may come from several host threads; each call is
 *     independent apart from the launch counter and the per-device caches
 *     (segment-table staging, the mapped report page, the second update
 *     stream), which are internally locked.  Multi-tensor calls on
 *     different caller streams of one device share that device's second
 *     stream, so their update launches may wait for one another.
 */
#ifndef RADAMW_H
#define RADAMW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t without requiring the HIP headers in C callers. */
typedef struct ihipStream_t *radamw_stream_t;

/* ----------------------------------------------------------- status codes */
enum {
    RADAMW_OK = 0,
    RADAMW_ERR_INVALID = -1, /* null pointer, n < 0, unknown dtype, host pointer,
                                pointer of another device, an array running
                                past the end of its allocation, hyper-
                                parameter out of range, non-finite or
                                non-positive gradient_scale, flag not 0/1,
                                a stream being captured into a graph          */
    RADAMW_ERR_STATE = -2,   /* AMSGrad flag and v_max presence disagree, or
                                the step count would overflow                 */
    RADAMW_ERR_ALIAS = -3,   /* a written range overlaps another range         */
    RADAMW_ERR_ALIGN = -4,   /* pointer not aligned to its element size        */
    RADAMW_ERR_RANGE = -5,   /* row count / capacity / scratch size out of
                                range; an element count above 2^48 (any
                                entry point taking n)                         */
    RADAMW_ERR_HIP = -6,     /* a HIP runtime call failed (see
                                radamw_last_hip_error)                         */
    RADAMW_ERR_DECISION = -7 /* fused steps only: the host's skip / clip
                                decision from the read-back report differs
                                from the one the device took and applied (a
                                library fault; never expected).  Unlike the
                                other errors the step DID run as the device
                                decided: the result struct and the step count
                                follow the device's decision.                 */
};

/* Gradient storage type (FA-zh "增加的实际能力"). */
typedef enum {
    RADAMW_F32 = 0,
    RADAMW_F16 = 1,  /* IEEE binary16 */
    RADAMW_BF16 = 2  /* bfloat16: the upper 16 bits of a binary32 */
} radamw_dtype;

/*
 * Hyper-parameters of the update (FA-ja "この演算子を使用する理由": formula
 * and defaults; FA-ja "低レベルの使用": the options struct).  Checked:
 * lr >= 0, eps >= 0, weight_decay >= 0, 0 <= beta1, beta2 < 1, all finite;
 * amsgrad and maximize are 0 or 1.
 */
typedef struct {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;
    int32_t amsgrad;
    int32_t maximize;
} radamw_options;

/*
 * Per-call control (FA-ja "低レベルの使用": StepControl).  The stored
 * gradient is divided by gradient_scale (finite, > 0).  skip_update = 1 is
 * the caller's found_inf decision: no launch, no write, no step increment
 * (FA-zh "增加的实际能力").  The library never scans for non-finite values
 * inside the update itself.
 */
typedef struct {
    double gradient_scale;
    int32_t skip_update;
} radamw_control;

/*
 * Optimizer state of one tensor (FA-ja "低レベルの使用": the state exposes
 * the step and the moment buffers).  step is the number of completed
 * updates; step == 0 is the pages' "no state yet": the next update is t = 1
 * and initialises the moments inside the kernel without reading them
 * (FA-zh "增加的实际能力").  exp_avg / exp_avg_sq / max_exp_avg_sq are
 * device FP32 arrays of n elements; max_exp_avg_sq is non-NULL exactly when
 * AMSGrad is on.
 */
typedef struct {
    uint64_t step;
    float *exp_avg;
    float *exp_avg_sq;
    float *max_exp_avg_sq;
} radamw_state;

/* One contiguous tensor of a multi-tensor update (in place). */
typedef struct {
    float *param;
    const void *grad;
    float *exp_avg;
    float *exp_avg_sq;
    float *max_exp_avg_sq; /* NULL unless AMSGrad */
    int64_t n;
} radamw_segment;

/*
 * 12-byte gradient-statistics record (TR-zh "在 ruda:0 上进行原生 PyTorch
 * 训练": a 12-byte report is read back before the update).  Layout chosen
 * here (the pages fix only the size): w[0] | w[1] << 32 is the IEEE binary64
 * sum of squares of the finite stored gradient values; w[2] is the count of
 * non-finite values, saturating at 2^32 - 1.  The same record is used for
 * the per-workgroup rows, the intermediate merge levels and the report.
 */
typedef struct {
    uint32_t w[3];
} radamw_stats;

/* Result of radamw_fused_step_multi (host struct). */
typedef struct {
    int32_t updated;     /* 1 when the update was launched                  */
    int32_t found_inf;   /* 1 when the report counted non-finite values     */
    uint32_t nonfinite;  /* the report's non-finite count                   */
    uint32_t reserved;
    double sumsq;        /* the report's sum of squares (stored scale)      */
    double total_norm;   /* sqrt(sumsq) / gradient_scale                    */
    double clip_coef;    /* min(1, max_norm / (total_norm + 1e-6)), or 1    */
} radamw_fused_result;

/* Defaults of FA-ja "この演算子を使用する理由": betas (0.9, 0.999),
 * eps 1e-5, weight decay 1e-4; lr 1e-3 as in the pages' usage examples;
 * amsgrad = maximize = 0.  Returns the struct by value. */
radamw_options radamw_options_default(void);

/*
 * Out-of-place update of one tensor (FA-ja "低レベルの使用": adamw_step;
 * FA-ja "割り当てとパフォーマンスのモデル": out-of-place outputs).
 *   p, g      : inputs, n elements; g has dtype gdt.  Never written.
 *   in        : host struct; in->step completed steps.  When in->step == 0
 *               the input moment pointers are not read (may be NULL).
 *   p_out     : output params (device, n FP32), caller-allocated.
 *   out       : host struct with caller-allocated output moment arrays
 *               (n FP32 each; max_exp_avg_sq iff amsgrad).  On launch,
 *               out->step = in->step + 1; otherwise out is not touched.
 *   updated   : host int32, set to 1 on launch, 0 on skip / n == 0.
 * No output range may overlap any input or other output (RADAMW_ERR_ALIAS).
 * skip_update or n == 0: nothing is launched or written (FA-zh
 * "增加的实际能力"), so the caller may allocate outputs only after a call
 * with ctrl->skip_update known to be 0.
 */
int radamw_step(const float *p, const void *g, radamw_dtype gdt, int64_t n,
                const radamw_state *in, float *p_out, radamw_state *out,
                const radamw_options *opts, const radamw_control *ctrl,
                radamw_stream_t stream, int32_t *updated);

/*
 * In-place update over caller-owned storage (FA-ja "ネイティブ PyTorch
 * ストレージと階層統計": the storage kernel adamw_scaled).  p, st->exp_avg,
 * st->exp_avg_sq (and st->max_exp_avg_sq iff AMSGrad) are read and written;
 * g is read only.  st->step is incremented only when the kernel is launched.
 */
int radamw_step_inplace(float *p, const void *g, radamw_dtype gdt, int64_t n,
                        radamw_state *st, const radamw_options *opts,
                        const radamw_control *ctrl, radamw_stream_t stream,
                        int32_t *updated);

/*
 * The staged (unfused) baseline, for measurement only (FA-ja
 * "割り当てとパフォーマンスのモデル", FA-zh "优化点与边界": a benchmark-only
 * baseline of four kernels, five with AMSGrad, that re-reads the gradient
 * and goes through a delta buffer; 48 bytes per parameter instead of 28, 60
 * instead of 36).  Same arguments and semantics as radamw_step_inplace,
 * plus delta: a caller-owned device scratch array of n FP32 (written).  The
 * per-element arithmetic is the fused kernel's, split across the launches
 * m -> v -> [v_max] -> delta -> p, so results are identical to
 * radamw_step_inplace.  Every array must be 16-byte aligned (RADAMW_ERR_ALIGN),
 * gradients of 16-bit types 8-byte aligned.
 */
/*
 * Placement of the streams of one flattened bucket (FA-ja
 * "サポートされている契約": a pre-flattened bucket whose elements share the
 * options and the step count) in a single allocation.  The update's
 * bandwidth depends on where its streams lie relative to one another in
 * HBM: on MI355X, p, g, m and v of a 2^28-element bucket exactly 1 GiB apart
 * update at ~6.44-6.55 TB/s, in separate allocations at ~6.54-6.59 TB/s,
 * and back to back in one allocation with each stream's start shifted by a
 * further 12 KiB at ~6.76-6.83 TB/s (3-4.5% faster for AdamW, AMSGrad and
 * 16-bit gradients; 3.6% at 1e8+7 elements).  The gain is for streams up to
 * about 1 GiB: streams of 5-27 GB came within +-2% of separate allocations.
 * The rule is measured, not derived: stream k starts at byte offset
 * k * pitch, with pitch = (n * max element size rounded up to 2 MiB) +
 * 12 KiB.
 *   n              : elements of every stream (0 <= n <= 2^48).
 *   element_bytes  : host array of nstreams element sizes (1, 2, 4 or 8),
 *                    in the order the caller wants the streams placed
 *                    (for example p, g, m, v, v_max); 1 <= nstreams <= 16.
 *   offsets        : host array of nstreams byte offsets (written).
 *   arena_bytes    : host, the allocation size the layout needs (written).
 * The arena's base should be 2 MiB-aligned (large hipMalloc allocations
 * are).  Host only; allocates nothing.  Any layout of the streams gives the
 * same results; this one is only faster.
 */
int radamw_bucket_layout(int64_t n, const int32_t *element_bytes, int32_t nstreams, int64_t *offsets,
                         int64_t *arena_bytes);

/*
 * Streaming ceiling, for measurement only.  FA-ja "残りゲート" asks that
 * performance work follow measured profiles rather than the traffic model;
 * this call measures what the memory system gives the update's access
 * pattern.  It moves nreads FP32 read streams and nwrites FP32 write streams
 * of n elements with the update kernel's geometry, cache hints and
 * occupancy rule, and one add per stream instead of the optimizer's
 * arithmetic: out[w][i] = ((in[0][i] + in[1][i]) + ...) + w (the empty sum
 * is 0).  AdamW with an FP32 gradient is the 4-read / 3-write pattern,
 * AMSGrad 5 / 4, a first step 2 / 3.
 *   in        : host array of nreads device pointers (0 <= nreads <= 5).
 *   out       : host array of max(nwrites, 1) device pointers
 *               (0 <= nwrites <= 4).  With nwrites == 0, out[0] is a sink of
 *               n floats that is never written in practice (a store guarded
 *               by a comparison with NaN keeps the loads live).
 *   n         : elements per stream, a multiple of 4; every array 16-byte
 *               aligned (RADAMW_ERR_ALIGN).
 *   cap_per_cu: resident workgroups per compute unit, 1..32, or 0 for the
 *               update kernels' own rule applied to 4 * (nreads + nwrites)
 *               bytes per element.
 * nreads + nwrites >= 1.  An output may be exactly one of the inputs
 * (in place, as the in-place update writes p, m and v: every element is
 * loaded before the same lane stores it); otherwise written arrays may
 * overlap nothing (RADAMW_ERR_ALIAS).  Read arrays may overlap each other.
 * n == 0 launches nothing.  radamw_time_next_update applies to this launch.
 */
int radamw_stream_probe(const float *const *in, int32_t nreads, float *const *out, int32_t nwrites,
                        int64_t n, int32_t cap_per_cu, radamw_stream_t stream);

int radamw_step_staged_inplace(float *p, const void *g, radamw_dtype gdt, int64_t n,
                               radamw_state *st, float *delta, const radamw_options *opts,
                               const radamw_control *ctrl, radamw_stream_t stream,
                               int32_t *updated);

/*
 * In-place update of a list of tensors that share one options struct and
 * one step count (FA-ja "サポートされている契約": a pre-flattened bucket
 * works only when every element shares the options and the step count).  A
 * flattened bucket is nseg == 1.  Launches: every tensor of at least 2^22
 * elements gets a launch of its own and all smaller tensors share a single
 * launch, so a list of many small tensors costs one launch, while large
 * tensors keep the single-tensor kernel (which measured faster than sharing
 * a launch).  All launches use the same constants and the step count
 * advances once.  With two or more launches, every other one runs on a
 * second stream the library keeps per device, so that the drain of one
 * launch overlaps the start of the next: that stream first waits for all
 * work queued on `stream` before the call, and `stream` waits for all of it
 * before anything queued after the call, so the call still orders on
 * `stream` exactly like a single launch.  The fused and list entry points
 * below submit their update launches the same way.
 *   segs  : host array of nseg descriptors (device pointers inside).
 *   step  : host, the shared completed-step count; incremented on launch.
 * Segments with n == 0 are ignored; when every segment is empty nothing is
 * launched and *step is unchanged.  No written range may overlap any other
 * range of any segment (RADAMW_ERR_ALIAS).  nseg >= 0.
 */
int radamw_step_multi(const radamw_segment *segs, int32_t nseg, radamw_dtype gdt,
                      uint64_t *step, const radamw_options *opts,
                      const radamw_control *ctrl, radamw_stream_t stream,
                      int32_t *updated);

/*
 * radamw_step_multi that also writes a 16-bit model copy of the updated
 * parameters in the same pass: models[i] (device, segs[i].n elements of
 * model_dtype, written) receives segs[i].param after the update, rounded to
 * nearest even (the FP16 / BF16 model weights of an FP32-master optimizer,
 * TR-zh "训练与状态保存": FP32 master parameters, 16-bit model storage).
 * models[i] may be NULL (no copy for that tensor).  model_dtype is
 * RADAMW_F16 or RADAMW_BF16.  Adds 2 bytes per parameter of traffic; the
 * update itself is identical to radamw_step_multi's.  Copies may overlap
 * nothing (RADAMW_ERR_ALIAS).
 */
int radamw_step_multi_writeback(const radamw_segment *segs, void *const *models, int32_t nseg,
                                radamw_dtype gdt, radamw_dtype model_dtype, uint64_t *step,
                                const radamw_options *opts, const radamw_control *ctrl,
                                radamw_stream_t stream, int32_t *updated);

/*
 * Merge plan for rows statistics records (FA-ja "ネイティブ PyTorch
 * ストレージと階層統計": StatsPlan; TR-zh "在 ruda:0 上进行原生 PyTorch
 * 训练": fan-in 1024, at most two extra merge kernels, at most 49,200 bytes
 * of reusable scratch).  rows must be in 1..4,194,304 (else
 * RADAMW_ERR_RANGE).  *scratch_elements receives the FP32-element count of
 * the intermediate levels (3 per record; initial rows and final report not
 * included); *extra_merge_kernels the number of fan-in-1024 levels before
 * the final merge (0 when rows <= 1024).  Host only; no device access.
 */
int radamw_stats_plan(int64_t rows, int64_t *scratch_elements,
                      int32_t *extra_merge_kernels);

/* Number of records one radamw_grad_stats call writes for n elements of
 * dtype gdt (a deterministic function of n and gdt alone; 0 when n == 0).
 * Returns a negative status for n < 0 or an unknown dtype.  Host only. */
int64_t radamw_grad_stats_rows(int64_t n, radamw_dtype gdt);

/*
 * Read-only analysis of one gradient (FA-ja "ネイティブ PyTorch ストレージと
 * 階層統計": analyze_gradient; TR-zh: gradient storage stays unchanged).
 * Writes radamw_grad_stats_rows(n, gdt) records to rows_out (device), each
 * the sum of squares of the finite values and the non-finite count of one
 * workgroup's share.  rows_capacity < that count -> RADAMW_ERR_RANGE.
 * *rows_written (host) receives the count (0 when n == 0: nothing launched).
 * The reduction order is fixed, so repeated calls give identical bits.
 */
int radamw_grad_stats(const void *g, radamw_dtype gdt, int64_t n,
                      radamw_stats *rows_out, int64_t rows_capacity,
                      int64_t *rows_written, radamw_stream_t stream);

/*
 * Reduce nrows records to the 12-byte report (FA-ja "ネイティブ PyTorch
 * ストレージと階層統計": merge_gradient_stats_chunks then
 * merge_gradient_stats; TR-zh: hierarchical fan-in 1024 changes only the
 * reduction order).  nrows in 1..4,194,304.
 *   hierarchical = 1: the radamw_stats_plan levels, each reducing groups of
 *     up to 1024 records into scratch, then one final merge into report.
 *     scratch (device, FP32 elements, 4-byte aligned) must hold
 *     scratch_elements >= the plan's count; it may be NULL when that count
 *     is 0.
 *   hierarchical = 0: one final merge over all rows (scratch unused).
 * Counts are bit-identical between the two modes; sums differ only by
 * FP64 rounding order.  report: 12 device bytes owned by the caller.
 */
int radamw_merge_stats(const radamw_stats *rows, int64_t nrows, float *scratch,
                       int64_t scratch_elements, radamw_stats *report,
                       int32_t hierarchical, radamw_stream_t stream);

/*
 * Read a device report back to the host (hipMemcpyAsync through a pinned
 * staging buffer, then stream synchronisation): the read-back of the step
 * composed from separate calls (TR-zh: the report is read back before any
 * update).  host_report: host struct.
 */
int radamw_read_report(const radamw_stats *report, radamw_stats *host_report,
                       radamw_stream_t stream);

/*
 * Host decision after the report (TR-zh "在 ruda:0 上进行原生 PyTorch 训练":
 * any non-finite gradient skips the whole step; optional global L2 clipping
 * after unscaling).  norm = sqrt(sumsq) / gradient_scale; clip = min(1,
 * max_grad_norm / (norm + 1e-6)) when max_grad_norm > 0, else 1.
 * Fills ctrl: skip_update = (count > 0); gradient_scale = gradient_scale /
 * clip (exactly gradient_scale when clip == 1).  result (optional, may be
 * NULL) receives the decoded report and the decision.  Host only.
 */
int radamw_decide(const radamw_stats *host_report, double gradient_scale,
                  double max_grad_norm, radamw_control *ctrl,
                  radamw_fused_result *result);

/*
 * The check every fused step makes after its read-back (TR-zh "在 ruda:0 上
 * 进行原生 PyTorch 训练": the report read back decides whether and how the
 * step updates): the host's decision from host_report (radamw_decide) must
 * equal the device's, device_decision = {skip, bits of the FP32 unscale
 * factor 1 / (gradient_scale / clip)} as the final merge wrote it.  result
 * (host, required) is filled from the report as by radamw_decide, with
 * result->updated taken from the DEVICE's decision, which is the one the
 * queued update kernels applied.  Returns RADAMW_OK when the two agree
 * (same skip; for an update, the same FP32 factor bit for bit) and
 * RADAMW_ERR_DECISION otherwise.  Host only.
 */
int radamw_check_decision(const radamw_stats *host_report, const uint32_t *device_decision,
                          double gradient_scale, double max_grad_norm,
                          radamw_fused_result *result);

/*
 * The whole fused step over a tensor list, the ruda_torch.AdamW
 * fused_step path of TR-zh: statistics of every active gradient ->
 * (hierarchical) merge -> 12-byte report read back -> skip or clip decision
 * -> the in-place update of radamw_step_multi.
 *   workspace : device, >= radamw_fused_workspace_bytes(...) bytes, 8-byte
 *               aligned (RADAMW_ERR_ALIGN otherwise), caller-owned: the
 *               rows, the merge scratch and a decision slot in its last 12
 *               bytes (an 8-byte record at an 8-byte boundary).
 *   max_grad_norm <= 0 disables clipping.
 *   result    : host struct, always filled on RADAMW_OK.
 * The final merge writes the report into host memory the library maps for
 * the device, and takes the same skip / clip decision as radamw_decide on
 * the device as well (the same binary64 operations, each correctly
 * rounded), writing it to the decision slot.  The update launches are
 * queued right behind the merge and read that slot, so the GPU never waits
 * for the host; the host waits once, for the merge, reads the report, takes
 * the decision itself and advances *step when the update ran.  When the
 * report counts a non-finite value the queued update kernels write nothing
 * (they have already issued their reads, so a skipped step costs one read
 * pass of the update's inputs; skips are rare).  The two decisions always
 * agree (radamw_check_decision); if they did not, the call returns
 * RADAMW_ERR_DECISION with *step and *result following the decision the
 * device applied.  The workspace stays in use until the stream has passed
 * the update kernels.
 */
int64_t radamw_fused_workspace_bytes(const radamw_segment *segs, int32_t nseg,
                                     radamw_dtype gdt);
int radamw_fused_step_multi(const radamw_segment *segs, int32_t nseg,
                            radamw_dtype gdt, uint64_t *step,
                            const radamw_options *opts, double gradient_scale,
                            double max_grad_norm, int32_t hierarchical,
                            void *workspace, int64_t workspace_bytes,
                            radamw_stream_t stream, radamw_fused_result *result);

/*
 * The fused step for callers that cannot allocate device memory: tight
 * serving loops, harnesses that forbid hipMalloc, and programs that replay
 * captured HIP graphs around it and may not allocate between replays.  The
 * call itself waits for its stream (it reads the report back), so it cannot
 * be recorded into a graph.
 * radamw_fused_step_multi over ONE flattened bucket (nseg <= 1; more is
 * RADAMW_ERR_RANGE) with no workspace argument: the statistics rows, merge
 * scratch, decision slot and report live in a static device array of the
 * library (98,560 bytes per device, held until the process ends), which fits
 * every bucket the library accepts (a tensor writes at most 8192 statistics
 * rows).  The call allocates no device or pinned host memory (its host-side
 * validation uses small host containers); on its first call on a device it
 * looks up that device's copy of the array.  Same arguments, checks,
 * arithmetic and results as radamw_fused_step_multi, bit for bit; the update
 * is one launch on `stream`.  The report and the device's decision are read
 * back behind the update, so the call returns when the step has completed
 * on the GPU.  Calls on one device share the array and are serialised by a
 * lock inside the library; work of another process has its own copy.
 * Nothing in the array needs clearing between calls: every call writes the
 * rows, records and report it reads.
 */
int radamw_fused_step_multi_noalloc(const radamw_segment *segs, int32_t nseg,
                                    radamw_dtype gdt, uint64_t *step,
                                    const radamw_options *opts, double gradient_scale,
                                    double max_grad_norm, int32_t hierarchical,
                                    radamw_stream_t stream, radamw_fused_result *result);

/*
 * Persistent tensor lists.  A training run updates the same tensors step
 * after step, and validating a list of a few hundred separately allocated
 * tensors (two HIP pointer queries per allocation, the overlap sweep)
 * costs about 0.6 ms of host time per call before the first kernel can
 * start.  radamw_list_create validates a segment list once and computes
 * everything that depends only on the tensors: the launch split of
 * radamw_step_multi, the update descriptors, the statistics rows of
 * radamw_fused_step_multi and their coarse indexes.  The device tables, the
 * statistics rows and the merge scratch live in one device allocation the
 * list owns, so a step only launches.  The arithmetic, the launch policy and
 * every result are those of radamw_step_multi / radamw_step_multi_writeback
 * / radamw_fused_step_multi on the same segments, bit for bit.
 *
 * OWNERSHIP (the one exception to "the library keeps no pointer"): a list
 * keeps the segment and model-copy pointers it was created with.  The
 * caller keeps every one of those buffers allocated, at the same address
 * and size, until radamw_list_destroy; stepping a list whose buffers were
 * freed or moved is undefined (the kernels would touch freed memory).  A
 * gradient that moves to a new buffer needs a new list.
 *
 * radamw_list_create(segs, nseg, gdt, amsgrad, models, model_dtype, stream,
 *                    list_out)
 *   segs, nseg, gdt : as radamw_step_multi (host array, device buffers,
 *                     in place); validated here exactly as there, with the
 *                     AMSGrad flag `amsgrad` (0/1) fixed for the list.
 *   models          : host array of nseg device pointers to FP16 / BF16
 *                     model copies (entries may be NULL), or NULL for none;
 *                     model_dtype is then RADAMW_F16 or RADAMW_BF16.
 *   stream          : fixes the device; the tables are uploaded on it
 *                     from pinned memory the list keeps (the call does not
 *                     wait for the stream).
 *   list_out        : host; receives the handle.  Allocates device memory
 *                     (tables + 12 B per statistics row + merge scratch).
 *   Errors as radamw_step_multi, plus RADAMW_ERR_RANGE when the rows exceed
 *   the merge plan's limit.  On error nothing is allocated.
 *
 * radamw_list_step(list, step, opts, ctrl, stream, updated)
 *   radamw_step_multi (or the write-back variant, when the list has model
 *   copies) over the list's segments.  opts->amsgrad must equal the list's
 *   flag (RADAMW_ERR_STATE otherwise); the stream must be on the list's
 *   device (RADAMW_ERR_INVALID otherwise).
 *
 * radamw_list_fused_step(list, step, opts, gradient_scale, max_grad_norm,
 *                        hierarchical, stream, result)
 *   radamw_fused_step_multi over the list's segments, using the list's own
 *   rows, scratch and decision slot as the workspace; the host waits once,
 *   for the final merge.
 *
 * Calls on one list serialise on a lock inside it, and each step's first
 * kernel waits (hipStreamWaitEvent) for the list's previous work, the table
 * upload or the last update, even when that went to another stream; calls
 * on different lists are independent.  radamw_time_next_update applies to the update
 * launches of a list step as to radamw_step_multi's.
 *
 * radamw_list_destroy(list): waits for the last submitted kernel that reads
 * the list's device memory, frees it and the handle.  NULL is accepted.
 */
typedef struct radamw_list_s *radamw_list;

int radamw_list_create(const radamw_segment *segs, int32_t nseg, radamw_dtype gdt,
                       int32_t amsgrad, void *const *models, radamw_dtype model_dtype,
                       radamw_stream_t stream, radamw_list *list_out);
int radamw_list_step(radamw_list list, uint64_t *step, const radamw_options *opts,
                     const radamw_control *ctrl, radamw_stream_t stream, int32_t *updated);
int radamw_list_fused_step(radamw_list list, uint64_t *step, const radamw_options *opts,
                           double gradient_scale, double max_grad_norm,
                           int32_t hierarchical, radamw_stream_t stream,
                           radamw_fused_result *result);
int radamw_list_destroy(radamw_list list);

/*
 * One fused step over several lists that take one decision together: the
 * parameter groups of a torch optimizer (for example weights with weight
 * decay and norms without), each with its own options and step count, under
 * one global-norm clip and one non-finite skip (TR-zh "在 ruda:0 上进行原生
 * PyTorch 训练": the statistics of every active group are reduced before any
 * parameter is updated).
 *
 * radamw_lists_fused_step(lists, nlists, steps, opts, gradient_scale,
 *                         max_grad_norm, hierarchical, stream, result)
 *   lists  : host array of nlists distinct list handles (1..65536), all on
 *            the stream's device.
 *   steps  : host array of nlists completed-step counts, one per list; a
 *            list that updates advances its own entry by one.
 *   opts   : host array of nlists option structs; opts[k].amsgrad must
 *            equal list k's flag.
 *   Every list's gradients are analysed (one launch per list); each list's
 *   rows are merged to one record (with the fan-in-1024 levels when
 *   hierarchical = 1), and those records, in array order, take one final
 *   merge into the report.  With a single non-empty list this is exactly
 *   radamw_list_fused_step.  The decision is taken once on that report
 *   (on the device by the final merge, into the first non-empty list's
 *   decision slot, which every list's queued update kernels read; and on
 *   the host after the one wait): a non-finite value anywhere skips every
 *   list; otherwise every list updates with the same clipped scale and its
 *   own options and step.
 *   Lists with no non-empty tensor neither launch nor step.
 *   Errors as radamw_list_fused_step, checked for every list before any
 *   launch; a handle given twice is RADAMW_ERR_INVALID.
 */
int radamw_lists_fused_step(const radamw_list *lists, int32_t nlists, uint64_t *steps,
                            const radamw_options *opts, double gradient_scale,
                            double max_grad_norm, int32_t hierarchical,
                            radamw_stream_t stream, radamw_fused_result *result);

/*
 * The FP32 constants one update launches with, formed on the host in FP64
 * and cast (FA-ja "この演算子を使用する理由": bias corrections by an FP64
 * integer power, cast to FP32), for update number t >= 1:
 *   out9 = {beta1, 1 - beta1, beta2, 1 - beta2, (maximize ? -1 : 1) /
 *           gradient_scale, 1 - lr * weight_decay, lr / (1 - beta1^t),
 *           1 / (1 - beta2^t), eps}.
 * Host only (out9: host array of 9 floats); lets the coefficients be
 * checked without a device.
 */
int radamw_host_coefficients(const radamw_options *opts, uint64_t t, double gradient_scale,
                             float *out9);

/* Utilities. */
const char *radamw_status_string(int status);
/* Last HIP error code seen by this thread inside the library (0 = none). */
int radamw_last_hip_error(void);
/* Total kernel launches made by the library in this process (test hook:
 * proves skip / empty calls launch nothing). */
uint64_t radamw_launch_count(void);

/*
 * Measurement hook (not part of the method): the next radamw_step,
 * radamw_step_inplace, radamw_step_multi, radamw_fused_step_multi or list
 * step call on this thread that launches an update records start_event
 * when its first update kernel starts (hipExtLaunchKernelGGL), so the
 * host's submission latency is not timed, and stop_event when its update
 * kernels have ended: at the end of a single launch, or, when the launches
 * are spread over two streams, on the caller's stream right after it has
 * joined the second one.
 * The events are caller-created hipEvent_t of the stream's device; passing
 * NULL, NULL clears the request.  Always returns RADAMW_OK.
 */
int radamw_time_next_update(void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* RADAMW_H */
