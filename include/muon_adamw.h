/*
 * muon_adamw.h -- C ABI of the MI355X (gfx950) hybrid MuonAdamW optimizer step.
 *
 * The method is the one described on the OpenDM training-stack page
 * ("VLA训练栈深度揭秘：OpenDM的MuonAdamW优化器、FSDP分布式训练与混合精度策略"):
 *   - its Muon/AdamW hybrid section, table on how parameters are split
 *     (routing, reproduced by muon_adamw_plan);
 *   - the Newton-Schulz paragraph of that section (a fixed number of quintic
 *     Newton-Schulz steps stand in for the zeroth power of each whole matrix);
 *   - the hyperparameter table of the optimizer config and the sentence after
 *     it (momentum 0.95, Nesterov, 5 steps, moonlight coefficient 0.2, base
 *     lr 2.5e-5, Muon lr = lr * muon_lr_scale * 0.2 * sqrt(max(shape)));
 *   - the MuonShardPlan paragraph (the plan records full shapes before any
 *     wrapping; NS acts on whole matrices -- on one GPU every matrix is whole);
 *   - the defaults quick-reference table (max_grad_norm 1.0).
 *
 * Conventions shared by every entry point:
 *   - Return 0 (MA_OK) on success, a negative MA_ERR_* code otherwise; the
 *     thread-local muon_adamw_last_error() then holds a message.
 *   - Arguments are validated before anything is launched: an error return
 *     means no kernel ran and no buffer changed.
 *   - No C++ exception crosses this boundary.
 *   - Parameters, gradients and optimizer states are float32, contiguous,
 *     row-major, in device memory owned by the caller.  The library never
 *     allocates device memory; its scratch lives in a caller-provided
 *     workspace.
 *   - Device work is asynchronous on the caller's HIP stream; device faults
 *     surface at the caller's next synchronisation (HIP semantics).  The
 *     host blocks in a step only when it runs more than four steps of the
 *     same plan ahead of the device: each eager step stages its descriptor
 *     tables in one of four pinned host buffers used in turn, and waits
 *     until the device has read the one it reuses.  Part of
 *     a step may run on streams the library creates on the same device
 *     (default priority, one set per plan and device, released by
 *     muon_adamw_plan_free); they fork from the caller's stream and are
 *     joined back into it before the step's work ends, so the caller's
 *     stream order covers the whole step, under graph capture too.
 */
#ifndef MUON_ADAMW_H_
#define MUON_ADAMW_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MA_OK                 0
#define MA_ERR_INVALID_ARG   (-1)  /* null pointer, bad count, bad value   */
#define MA_ERR_SHAPE         (-2)  /* non-positive or overflowing shape    */
#define MA_ERR_UNSUPPORTED   (-3)  /* ndim > 8, ns_steps < 1, bad mode ... */
#define MA_ERR_WORKSPACE     (-4)  /* workspace null, small or misaligned  */
#define MA_ERR_HIP           (-5)  /* a HIP runtime call failed            */
#define MA_ERR_CAPTURE       (-6)  /* upload needed under stream capture   */

/* ---- groups, modes, precisions ------------------------------------------ */
#define MA_GROUP_MUON   0
#define MA_GROUP_ADAMW  1
#define MA_GROUP_NONE   2      /* frozen: no update, not in the clip norm */

#define MA_MODE_MUON_ADAMW 0   /* the hybrid (optim = muon_adamw)          */
#define MA_MODE_ADAMW      1   /* every trainable tensor to AdamW          */

#define MA_NS_BF16 0           /* bf16 MFMA operands, fp32 accumulation    */
#define MA_NS_FP32 1           /* fp32 MFMA throughout                     */

/* ---- learning-rate schedules (defaults table of the page) ---------------- */
#define MA_LR_CONSTANT   0     /* lr every step                            */
#define MA_LR_COSINE_MIN 1     /* cosine_with_min_lr                       */

/* ---- parameter storage (precision policies of the page) ---------------- */
#define MA_PARAM_FP32 0        /* fp32_mixed: float32 weights              */
#define MA_PARAM_BF16 1        /* bf16_mixed: the model stored in bfloat16 */

#define MA_MAX_NDIM 8

/* One model parameter, in the caller's order.  `name` is the dotted module
 * path (UTF-8, NUL-terminated), `shape` holds `ndim` positive sizes,
 * `trainable` is 0 for frozen parameters.  Borrowed for the duration of the
 * muon_adamw_plan call only. */
typedef struct {
    const char*    name;
    int32_t        ndim;
    const int64_t* shape;
    int32_t        trainable;
} ma_param_desc;

/* `overlap_groups` = 1 runs the AdamW group beside the Muon group: one
 * workgroup per CU on a library-owned second stream of the same device
 * (default priority) streams AdamW chunks while the Muon kernels run on the
 * caller's stream -- its waves are small enough to share each SIMD with a
 * Newton-Schulz GEMM wave -- and after the Newton-Schulz launches a second
 * AdamW launch on the caller's stream finishes whatever chunks are left.
 * Chunks are claimed from a counter in the workspace; AdamW is elementwise,
 * so the results are bitwise those of overlap 0.  The side stream is joined
 * back into the caller's stream before the step's work ends.  With bf16
 * Newton-Schulz products the Muon matrices then also run in smaller batches
 * (each through all of its iterations; about 160 MB of operands per batch),
 * which leaves more HBM bandwidth to the AdamW stream.
 *
 * In both modes the Newton-Schulz GEMMs run in batches of matrices that
 * alternate between the caller's stream and a second library-owned stream;
 * every matrix's iterations stay in order on one stream, so the results do
 * not depend on the batching.  0 runs AdamW on the caller's stream, in order
 * before the Muon group.
 *
 * param_dtype: how every trainable parameter and its gradient are stored
 * (the page's precision policies: bf16_mixed, the default there, stores the
 * model in bfloat16; fp32_mixed keeps fp32 weights).  MA_PARAM_FP32 (0):
 * float32.  MA_PARAM_BF16 (1): bfloat16; the step reads them as bf16,
 * computes in float32 exactly as for float32 storage and rounds the new
 * parameter once to bf16 (round to nearest, ties to even).  Optimizer states
 * (Muon momentum, AdamW moments) and muon_update_out are float32 either way.
 * With no float32 master copy an update below half a bf16 spacing leaves a
 * parameter unchanged, as it does for any bf16-stored weight.
 *
 * A NULL opts means mode MA_MODE_MUON_ADAMW, moonlight 0.2, overlap 0,
 * float32 parameters. */
typedef struct {
    int32_t mode;                  /* MA_MODE_*                            */
    double  moonlight_coefficient; /* 0.2 on the page                      */
    int32_t overlap_groups;        /* 1: AdamW beside the Muon group       */
    int32_t param_dtype;           /* MA_PARAM_FP32 / MA_PARAM_BF16        */
} ma_plan_opts;

typedef struct ma_plan ma_plan;    /* opaque, immutable once built         */

/* What the plan decided for one entry.  For a Muon matrix stored m x n,
 * (r, c) = (min, max) is its canonical orientation (Gram matrix r x r),
 * `transposed` is 1 when m > n, `bucket` numbers the distinct (r, c) in order
 * of first appearance, `lr_shape_scale` is the float32 rounding of
 * moonlight_coefficient * sqrt(max(m, n)) computed in double.  For an AdamW
 * tensor, `adam_offset` is its start in the concatenation of all AdamW
 * tensors in table order.  Unused fields are 0 (-1 for bucket, adam_offset). */
typedef struct {
    int32_t group;
    int32_t bucket;
    int64_t m, n, r, c;
    int32_t transposed;
    float   lr_shape_scale;
    int64_t numel;
    int64_t adam_offset;
} ma_plan_entry;

/* Caller-owned optimizer state, arrays indexed like the plan's entries.
 * muon_momentum[i] (m x n) for Muon entries, adam_m[i] / adam_v[i] (numel)
 * for AdamW entries; other slots are ignored and may be NULL.  `step` counts
 * completed steps; muon_adamw_step uses t = step+1 for the schedule and the
 * bias corrections and increments it on success.  All tensors start at zero
 * for a fresh run.
 *
 * device_step (nullable): a device int64 that counts completed steps
 * instead of `step`, which is then neither read nor changed.  Each step
 * reads it on the device, uses t = *device_step + 1 and stores t back, in
 * stream order.  Every launch of such a step takes the same arguments for
 * any t.  Every eager step uploads its descriptor tables (the tensor
 * addresses and tile lists) into the workspace; a step under stream capture
 * cannot, and reads the tables the last eager step of this plan with
 * device_step set put there.  So after one eager step, a step with the same
 * pointers and workspace can be captured in a HIP graph and replayed, each
 * replay advancing *device_step, provided nothing else writes that
 * workspace between that eager step and the replays. */
typedef struct {
    float* const* muon_momentum;
    float* const* adam_m;
    float* const* adam_v;
    int64_t       step;
    int64_t*      device_step;
} ma_state;

/* Hyperparameters of one step.  muon_adamw_default_hparams fills the page's
 * defaults (lr 2.5e-5, muon_lr_scale 1, momentum 0.95, Nesterov on, 5 NS
 * steps, clip 1.0) and the readings where the page is silent: NS coefficients
 * (3.2608, -3.6447, 1.3650), NS epsilon 1e-7, AdamW betas (0.9, 0.999), eps
 * 1e-8, decay 0.01, Muon decay 0, bf16 NS.  max_grad_norm <= 0 turns the
 * global clip off.  ns_coeffs (a, b, c) define X <- a X + (b A + c A^2) X.
 * Scalars are double: derived constants (1 - beta, bias corrections, the
 * scheduled rate, lr * shape factor) are formed in double -- those that
 * depend on the step number on the device, at the start of the step -- and
 * rounded once to the float32 the kernels compute in.
 *
 * lr_schedule (the page's defaults table: cosine_with_min_lr, min_lr_rate
 * 0.1; default MA_LR_CONSTANT) sets the rate of optimizer step t (step + 1,
 * or the device counter + 1) for both groups to lr * f(t - 1):
 * MA_LR_CONSTANT f = 1; MA_LR_COSINE_MIN
 * f(k) = k / warmup_steps for k < warmup_steps, else min_lr_rate +
 * (1 - min_lr_rate) (1 + cos(pi p)) / 2 with p = (k - warmup_steps) /
 * max(1, total_steps - warmup_steps) held at 1 past the end.  It needs
 * total_steps >= 1, 0 <= warmup_steps <= total_steps and min_lr_rate in
 * [0, 1]. */
typedef struct {
    double  lr;
    double  muon_lr_scale;
    double  muon_momentum;
    int32_t muon_nesterov;
    int32_t muon_ns_steps;
    double  ns_coeffs[3];
    int32_t ns_precision;      /* MA_NS_BF16 or MA_NS_FP32 */
    double  ns_eps;
    double  beta1;
    double  beta2;
    double  eps;
    double  weight_decay;
    double  muon_weight_decay;
    double  max_grad_norm;
    int32_t lr_schedule;       /* MA_LR_CONSTANT or MA_LR_COSINE_MIN */
    int64_t warmup_steps;
    int64_t total_steps;
    double  min_lr_rate;
} ma_hparams;

/* Fill *hp with the defaults listed above.  Errors: INVALID_ARG if hp is
 * NULL. */
int muon_adamw_default_hparams(ma_hparams* hp);

/* Build the routing/shape plan of a parameter table (the page's routing
 * rule: a trainable matrix whose name has a component containing
 * 'action_expert', then a component 'layers', ends in '.weight' and contains
 * none of 'embed', 'lm_head', 'norm' (case-insensitive) is Muon; any other
 * trainable tensor is AdamW; frozen tensors are NONE).  Host only: touches no
 * GPU.  On success *out owns a plan to be released with muon_adamw_plan_free.
 * Errors: INVALID_ARG (null table/out/name, n < 1, bad mode, coefficient not
 * finite and positive), UNSUPPORTED (ndim < 0 or > 8), SHAPE (a size < 1,
 * an element count above 2^62, or a Muon matrix whose canonical r x c,
 * each side rounded up to a multiple of 256, exceeds (2^31 - 1) / 4
 * elements: its fp32 Newton-Schulz operand must stay below 2 GiB). */
int muon_adamw_plan(const ma_param_desc* table, int32_t n,
                    const ma_plan_opts* opts, ma_plan** out);

/* Number of entries (equal to the table length).  Errors: INVALID_ARG. */
int muon_adamw_plan_size(const ma_plan* plan, int32_t* n_entries);

/* Decision for entry i.  Errors: INVALID_ARG (null, i out of range). */
int muon_adamw_plan_entry(const ma_plan* plan, int32_t i, ma_plan_entry* e);

/* Canonical text of the plan (header, one line per bucket, one line per
 * entry; format documented with the oracle that produces the same bytes).
 * Writes at most cap bytes (NUL-terminated when it fits) and sets *len to the
 * full length without the NUL; call with buf = NULL, cap = 0 to size it.
 * Errors: INVALID_ARG (null plan or len), WORKSPACE if cap is too small
 * (buf untouched, *len set). */
int muon_adamw_plan_dump(const ma_plan* plan, char* buf, size_t cap, size_t* len);

/* Bytes of device workspace one muon_adamw_step call needs for this plan
 * and NS precision.  The caller allocates it (256-byte aligned) and may
 * reuse it across steps.  An eager step writes everything it reads there
 * (its descriptor tables included), so between eager steps the contents are
 * scratch and the caller may use or free the memory; only replays of a
 * captured step depend on what an earlier eager step left in it (see
 * ma_state.device_step).
 * Errors: INVALID_ARG (null, bad precision). */
int muon_adamw_workspace_size(const ma_plan* plan, int32_t ns_precision, size_t* bytes);

/* One optimizer step on `stream` (a hipStream_t; NULL = the null stream).
 *
 *   1. N = sqrt(sum of g^2 over every trainable gradient);
 *      coef = max_grad_norm > 0 ? min(1, max_grad_norm / (N + 1e-6)) : 1
 *      (gradients are read-only: coef is applied on the fly).
 *   2. AdamW entries: g' = coef g; p *= 1 - lr wd; m = b1 m + (1-b1) g';
 *      v = b2 v + (1-b2) g'^2; p -= lr/(1-b1^t) * m / (sqrt(v)/sqrt(1-b2^t) + eps).
 *   3. Muon entries (m x n): buf = mu buf + coef g; u = coef g + mu buf
 *      (Nesterov; u = buf otherwise); X = u (transposed if m > n) / (||u||_F
 *      + ns_eps); ns_steps times { A = X X^T; B = b A + c A A; X = a X + B X };
 *      delta = lr * muon_lr_scale * lr_shape_scale * X (back in m x n);
 *      p = p (1 - lr muon_wd) - delta.
 *
 * params[i], grads[i]: entry i's tensors (NULL allowed for NONE entries):
 *   float32, or bfloat16 for a plan built with MA_PARAM_BF16 (the pointer
 *   types stay float*; they then address 2-byte elements).
 * grad_norm_out: optional device float receiving N.
 * muon_update_out: optional array (indexed like entries) of device m x n
 *   float buffers receiving delta for Muon entries; the array itself or any
 *   slot may be NULL.
 * workspace / ws_bytes: device scratch of at least muon_adamw_workspace_size
 *   bytes for hp->ns_precision, 256-byte aligned.
 * Errors (nothing launched): INVALID_ARG (null plan/state/hp, a required
 * pointer NULL, hp values out of range, or two of the buffers the step
 * touches overlapping: parameters, gradients, states, update outputs,
 * grad_norm_out, device_step and the workspace must be pairwise disjoint,
 * as address ranges), UNSUPPORTED (ns_steps < 1 or > 64,
 * unknown precision), WORKSPACE (null, too small, misaligned), CAPTURE (the
 * stream is capturing and the descriptor tables would have to be uploaded:
 * run one eager step with the same pointers and workspace first, with
 * state->device_step set), HIP (a launch or copy failed; state->step is then
 * not advanced). */
int muon_adamw_step(const ma_plan* plan,
                    float* const* params,
                    const float* const* grads,
                    ma_state* state,
                    const ma_hparams* hp,
                    void* workspace, size_t ws_bytes,
                    void* stream,
                    float* grad_norm_out,
                    float* const* muon_update_out);

/* Number of events muon_adamw_step_profiled records. */
#define MA_PROFILE_EVENTS 5

/* muon_adamw_step, plus measurement: phase_events (nullable) is an array of
 * MA_PROFILE_EVENTS hipEvent_t created by the caller, recorded on `stream`
 * at [0] the start of the step, [1] after the clip norm, [2] after the AdamW
 * group, [3] after the Muon momentum/normalise pass, [4] at the end of the
 * step.  Without overlap_groups each interval is exactly its phase's
 * kernels ([1] -> [2] is the one AdamW launch; [3] -> [4] spans the
 * Newton-Schulz launches on both of its streams).  With overlap_groups, [2] is
 * recorded on the side stream after its AdamW launch and the remaining
 * AdamW chunks run between [3] and [4], so only [0] -> [4] is meaningful.
 * Same errors as muon_adamw_step. */
int muon_adamw_step_profiled(const ma_plan* plan,
                             float* const* params,
                             const float* const* grads,
                             ma_state* state,
                             const ma_hparams* hp,
                             void* workspace, size_t ws_bytes,
                             void* stream,
                             float* grad_norm_out,
                             float* const* muon_update_out,
                             void* const* phase_events);

/* Largest workspace (bytes) of a plan that muon_adamw_step_noalloc accepts:
 * the size of its per-device scratch. */
#define MA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* muon_adamw_step for callers that cannot allocate memory (code in tight
 * serving loops, or harnesses that forbid allocation calls): the same
 * computation, arguments and errors, with the workspace replaced by a
 * device scratch array that the library holds in its code object -- one
 * copy of MA_NOALLOC_SCRATCH_BYTES on every GPU it runs on, kept until the
 * process ends.  This call allocates nothing: no device or pinned memory,
 * and no streams or events (every kernel of the step runs on `stream`; the
 * AdamW group does not run beside the Muon group and Newton-Schulz batches
 * run one after another, so it is slower than muon_adamw_step with
 * overlap).  Its descriptor tables travel in kernel arguments.
 *
 * All calls on one GPU share that GPU's scratch, which keeps the last call's
 * contents; each call writes every part of it that it reads before reading
 * it, so no state carries over.  Calls that overlap on one GPU (on
 * different streams or host threads) race on the scratch and give wrong
 * results: callers must order them.  A step under stream capture is refused
 * (a replay could meet another plan's data in the shared scratch).
 *
 * Errors: as muon_adamw_step, plus WORKSPACE when the plan's workspace
 * (muon_adamw_workspace_size for hp->ns_precision) exceeds
 * MA_NOALLOC_SCRATCH_BYTES, and CAPTURE under stream capture; nothing is
 * launched then. */
int muon_adamw_step_noalloc(const ma_plan* plan,
                            float* const* params,
                            const float* const* grads,
                            ma_state* state,
                            const ma_hparams* hp,
                            void* stream,
                            float* grad_norm_out,
                            float* const* muon_update_out);

/* Release a plan (NULL is a no-op).  Must not race with a step using it;
 * device work already queued does not reference plan memory after the step
 * returns... except the library's pinned staging buffers, which are freed
 * only after their last copy completed. */
void muon_adamw_plan_free(ma_plan* plan);

/* Message of the last error on this thread ("" if none). */
const char* muon_adamw_last_error(void);

/* Library version string. */
const char* muon_adamw_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_ADAMW_H_ */
