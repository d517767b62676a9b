/*
 * dpstep.h -- C ABI of the data-parallel gradient reduce + AdamW step for
 * MI355X (gfx950).
 *
 * The step, as the pages define it:
 *  - every replica r holds the full model and sums its own gradients over
 *    a micro-steps into g_r, exchanging nothing until the last one
 *    ("Distributed Training: Split along the Four Axes of Data, Tensor,
 *    Pipeline, and State", ai-knowledge-map.com: averaging-formula paragraph
 *    and the b=4, a=8, n=8 worked example);
 *  - the replicas are averaged, g_bar = (sum_r g_r) / n, and every replica
 *    applies the same update with it (same page: data-parallel all-reduce and
 *    averaging-formula paragraphs);
 *  - the update keeps a higher-precision master copy and Adam's two moments
 *    beside the low-precision weights, 16 bytes per parameter in all (same
 *    page, mixed-precision paragraph; "Data vs Tensor vs Pipeline
 *    Parallelism: When to Use Each", abhik.ai, section "What each one splits
 *    / Data parallelism");
 *  - under ZeRO a rank updates only its shard of the state, with the same
 *    result as the unsharded update (first page, ZeRO paragraph; second page,
 *    same section: 16*Psi/N bytes per GPU).
 *
 * Here the n replicas are n buffers in one GPU's memory and a shard is a
 * range [shard_begin, shard_end) of the flat parameter space: the
 * concatenation of the plan's tensors in list order.
 *
 * Conventions for every entry point:
 *  - Pointers named device point to GPU memory the caller owns (allocated by
 *    any means, for example by torch); the library never frees them.  Pointers
 *    named host point to host memory, read during the call only.
 *  - Compute calls are asynchronous on the caller's stream, never synchronise
 *    and never allocate, except where a comment says otherwise.
 *  - Every call returns a dp_status.  On failure nothing was launched and
 *    dp_last_error() returns a message for the calling thread.  A failed HIP
 *    call inside the library is reported there, and hipGetLastError() is
 *    reset, so the caller's own HIP error checks do not see it again.  Faults inside
 *    kernels surface at the next synchronising call (dp_read_state).
 *  - Calls on one plan may be issued on different streams, one after
 *    another: the caller orders them (for example with events), as the data
 *    one call writes is read by the next.  The library orders only its own
 *    pointer-table uploads across streams.  A HIP graph of captured calls is
 *    ordered like any other launch on the stream it is launched on.
 *    Distinct plans are independent.
 *  - A plan belongs to the device that is current at its first GPU call
 *    (binding per-tensor pointers, preparing a range, dp_state_init).  Every
 *    later GPU call checks that this device is current, and fails with
 *    DP_ERR_STATE otherwise.
 */
#ifndef DPSTEP_H
#define DPSTEP_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DP_ABI_VERSION 3
#define DP_MAX_REPLICAS 16
#define DP_DEFAULT_CHUNK 16384
/* dp_reduce_adam_step_noalloc: the largest flat space it takes, and the bytes
 * of the static device array that holds its scratch on each GPU. */
#define DP_STATIC_MAX_PARAMS (INT64_C(1) << 30)
#define DP_STATIC_SCRATCH_BYTES 51920896

typedef enum dp_status {
    DP_OK = 0,
    DP_ERR_INVALID_ARG = 1, /* null pointer, unknown enum value, bad size */
    DP_ERR_BAD_LAYOUT = 2,  /* layout rejected by dp_plan_create */
    DP_ERR_UNBOUND = 3,     /* a role the call reads or writes has no memory bound */
    DP_ERR_RANGE = 4,       /* range not inside [0, P) or begin > end */
    DP_ERR_STATE = 5,       /* call out of order (see each call) */
    DP_ERR_OOM = 6,         /* a library allocation failed */
    DP_ERR_HIP = 7,         /* a HIP call failed; dp_last_error() has its text */
    DP_ERR_IO = 8,          /* a file system call failed (dpckpt.h) */
    DP_ERR_CORRUPT = 9      /* a checkpoint file failed its checks (dpckpt.h) */
} dp_status;

typedef enum dp_dtype { DP_F32 = 0, DP_F16 = 1, DP_BF16 = 2 } dp_dtype;

/* Memory roles.  All roles are laid out like the flat parameter space.
 * MASTER, EXP_AVG and EXP_AVG_SQ have two banks (the replica argument of the
 * bind calls, 0 or 1).  Bank 0 is required; bank 1 only by
 * dp_reduce_adam_step, which reads the current bank and writes the other.
 * dp_step_state.bank says which bank is current. */
typedef enum dp_role {
    DP_ROLE_PARAM = 0,      /* low-precision parameters (param dtype); written by dp_adam_step */
    DP_ROLE_MASTER = 1,     /* binary32 master weights (two banks) */
    DP_ROLE_EXP_AVG = 2,    /* binary32 first moment m (two banks) */
    DP_ROLE_EXP_AVG_SQ = 3, /* binary32 second moment v (two banks) */
    DP_ROLE_GRAD = 4,       /* per replica: the micro-step gradient, or the incoming partial (grad dtype) */
    DP_ROLE_ACC = 5,        /* per replica: binary32 accumulator g_r */
    DP_ROLE_GBAR = 6        /* binary32 averaged gradient g_bar; with n = 1 it defaults to ACC[0] */
} dp_role;

typedef enum dp_scaler_mode {
    DP_SCALER_NONE = 0,    /* scale 1; a non-finite gradient still skips the step */
    DP_SCALER_STATIC = 1,  /* fixed scale; a non-finite gradient skips the step */
    DP_SCALER_DYNAMIC = 2  /* skip and back off on a non-finite gradient, grow after growth_interval clean steps */
} dp_scaler_mode;

/* Ragged tensor list.  numel is host memory, copied by dp_plan_create. */
typedef struct dp_layout {
    int32_t num_tensors;   /* >= 0 */
    int32_t n_replicas;    /* 1 .. DP_MAX_REPLICAS */
    const int64_t* numel;  /* host: [num_tensors], each >= 0 */
    dp_dtype grad_dtype;   /* DP_F16 or DP_BF16 */
    dp_dtype param_dtype;  /* DP_F16 or DP_BF16 */
    int32_t chunk_elems;   /* 0 = DP_DEFAULT_CHUNK; else a power of two in [256, 2^26] */
    int32_t reserved;
} dp_layout;

typedef struct dp_state_cfg {
    double beta1, beta2;       /* Adam's moment decay rates */
    int32_t scaler_mode;       /* dp_scaler_mode */
    int32_t growth_interval;   /* dynamic: clean steps before the scale grows (> 0) */
    double init_scale;         /* static / dynamic: initial loss scale (> 0) */
    double backoff;            /* dynamic: factor on a skipped step, in (0, 1) */
    double growth;             /* dynamic: growth factor, >= 1 */
} dp_state_cfg;

typedef struct dp_adam_hparams {
    double lr;            /* learning rate */
    double eps;           /* added to sqrt of the bias-corrected second moment */
    double weight_decay;  /* decoupled: w <- w * (1 - lr * weight_decay) */
} dp_adam_hparams;

/* The per-run scalar state, as held on the device. */
typedef struct dp_step_state {
    int64_t t;               /* applied updates */
    int64_t iter;            /* steps taken, applied or skipped */
    int64_t growth_tracker;  /* consecutive applied steps since the last scale change */
    double beta1_pow;        /* beta1^t */
    double beta2_pow;        /* beta2^t */
    double scale;            /* loss scale the next step's gradients must carry */
    int32_t found_inf;       /* the last finalised g_bar held an inf or NaN: the step was skipped */
    int32_t bank;            /* state bank (0 or 1) holding the current master, m and v */
    double sumsq;            /* sum of squares of the last (scaled) g_bar */
    double norm;             /* L2 norm of the last unscaled g_bar */
    double clip;             /* global-norm clip factor applied (1 when off or not needed) */
    double gscale;           /* clip / scale: multiplies the stored g_bar in the update */
} dp_step_state;

typedef struct dp_plan_info {
    int64_t params;          /* P */
    int64_t num_chunks;      /* chunks covering [0, P) */
    int32_t num_tensors;
    int32_t n_replicas;
    int32_t chunk_elems;
    int32_t reserved;
    double state_bytes;      /* 16 * P: param + grad (2 + 2) + master, m, v (4 + 4 + 4) */
    /* algorithmic HBM bytes of one call over the full range */
    double bytes_accumulate_first;  /* read g, write g_r */
    double bytes_accumulate;        /* read g and g_r, write g_r */
    double bytes_reduce_acc;        /* read n accumulators, write g_bar */
    double bytes_reduce_partials;   /* read n low-precision partials, write g_bar */
    double bytes_accumulate_reduce; /* read n accumulators and n gradients, write g_bar */
    double bytes_stats_scan;        /* read g_bar */
    double bytes_adam;              /* read g_bar, w, m, v; write w, m, v, p */
    /* dp_reduce_adam_step: read n accumulators and n gradients (or n
     * partials), w, m, v; write w, m, v, p (g_bar is not stored) */
    double bytes_reduce_adam;
    double bytes_reduce_adam_partials;
} dp_plan_info;

/* One entry of a chunk table: a piece of one tensor, at most chunk_elems long. */
typedef struct dp_chunk {
    int64_t flat;    /* flat index of the chunk's first element */
    int64_t offset;  /* index of that element inside its tensor */
    int32_t tensor;  /* tensor index */
    int32_t len;     /* elements */
} dp_chunk;

typedef struct dp_plan dp_plan;

int dp_abi_version(void);
const char* dp_status_string(dp_status s);
/* Message of the calling thread's last failure ("" if none).  Valid until the
 * thread's next failing call. */
const char* dp_last_error(void);

/* Builds a plan over a ragged tensor list: prefix sums of the flat space and
 * the chunk table of [0, P) (host work only; no GPU is touched).  Rejects
 * negative sizes, bad dtypes, n_replicas outside [1, DP_MAX_REPLICAS] and bad
 * chunk sizes with DP_ERR_BAD_LAYOUT.  *out receives the plan. */
dp_status dp_plan_create(const dp_layout* layout, dp_plan** out);

/* Frees the library's device memory (tables, partials, state) and the plan.
 * Synchronises the plan's device first.  Null is accepted. */
dp_status dp_plan_destroy(dp_plan* plan);

dp_status dp_plan_info_get(const dp_plan* plan, dp_plan_info* out);

/* Copies entries [first, first + cap) of the chunk table of [begin, end) into
 * host array out and the table's length into *count (host work only). */
dp_status dp_plan_chunks(const dp_plan* plan, int64_t begin, int64_t end, int64_t first, int64_t cap,
                         dp_chunk* out, int64_t* count);

/* Binds one contiguous device buffer to a role: tensor i starts at element
 * prefix[i] of it.  replica selects the GRAD / ACC buffer, or the bank (0, 1)
 * of MASTER / EXP_AVG / EXP_AVG_SQ; 0 for PARAM and GBAR.  Host work only
 * (a role's pointer-table ring, if it has one, is kept for later per-tensor
 * bindings); rebinding is cheap and may happen between any two calls. */
dp_status dp_plan_bind_flat(dp_plan* plan, dp_role role, int32_t replica, void* device_base);

/* Binds one device pointer per tensor (host array ptrs[num_tensors]).  The
 * kernels read the pointers from a device table.  Each role keeps a ring of
 * four such tables; the first per-tensor binding of a role allocates the ring
 * (device memory and pinned host staging), which lasts until
 * dp_plan_destroy.  A rebinding copies ptrs into the next slot's staging
 * memory and returns without synchronising: the next compute call that
 * reads the role uploads the table on its own stream before its launch,
 * and calls on other streams wait for that upload.  Work already launched
 * with an earlier table keeps reading it undisturbed.  A slot is rewritten
 * only four rebindings later, after the launches that read it have finished
 * (the rebinding waits for them then, if they have not).  Rebinding the
 * pointers already bound does nothing.  Suited to rebinding per micro-step,
 * for example gradients in per-tensor buffers that change every step.
 * Under HIP graph capture a call must find its tables uploaded by an earlier
 * uncaptured call (DP_ERR_STATE otherwise: make one uncaptured call after
 * rebinding; replays are then ordered after it like after any prior work),
 * and roles whose calls were captured must not be rebound while the graph
 * may replay, since the graph reads the tables current at capture. */
dp_status dp_plan_bind_tensors(dp_plan* plan, dp_role role, int32_t replica, void* const* ptrs);

/* Checks that [begin, end) lies in [0, P) (DP_ERR_RANGE) and sets up the
 * plan's device chunk table of [0, P) if no GPU call has done so yet (the
 * plan's one-time set-up: allocates and synchronises then).  A shard range
 * needs no table of its own: dp_adam_step runs on the pieces of the [0, P)
 * table that overlap its range, clipped to it. */
dp_status dp_plan_prepare_range(dp_plan* plan, int64_t begin, int64_t end);

/* Does nothing and returns DP_OK: shard ranges hold no tables or other state
 * of their own, so a caller whose shard ranges change over a run has nothing
 * to release.  Kept so that such callers need no change. */
dp_status dp_plan_drop_ranges(dp_plan* plan);

/* The per-run scalar state of the step: the applied-step count t and the
 * bias-correction powers of Adam, and the loss scale with its growth
 * tracker.  The pages count loss scaling among the training state a
 * checkpoint must hold, beside the optimizer's ("Distributed Training: Split
 * along the Four Axes of Data, Tensor, Pipeline, and State",
 * ai-knowledge-map.com: checkpoint-contents paragraph), and ask that it stay
 * aligned with the baseline when runs are compared (same page, evaluation
 * paragraph on training semantics).  The scaler policies themselves
 * (dp_scaler_mode: skip on a non-finite gradient, back off, grow after a
 * run of clean steps) are not on the pages; they follow the workloads this
 * library is built for, which name a static and a dynamic loss scale.
 *
 * Allocates the device state and statistics scratch on the current device
 * (first call), and sets t = 0, beta powers = 1, scale = init_scale (1 with
 * DP_SCALER_NONE), growth tracker 0, asynchronously on stream. */
dp_status dp_state_init(dp_plan* plan, const dp_state_cfg* cfg, hipStream_t stream);

/* Micro-step accumulation [first page, averaging formula]: over [0, P),
 * ACC[replica] = GRAD[replica] when first != 0, else ACC[replica] + GRAD[replica],
 * in binary32.  emit_stats != 0 (only with n_replicas == 1, where g_bar is
 * ACC[0]) also writes the per-chunk statistics of the result, so the last
 * micro-step replaces the scan of dp_grad_stats.  DP_ERR_STATE: first == 0 on
 * a replica with no first micro-step since the last reduction. */
dp_status dp_accumulate(dp_plan* plan, int32_t replica, int32_t first, int32_t emit_stats, hipStream_t stream);

/* Every replica's micro-step at once: the same as dp_accumulate(r, first, 0)
 * for r = 0 .. n-1 in one launch.  The pages have every micro-step run on all
 * n devices at the same time [first page, averaging formula paragraph]; here
 * the n replicas' gradients are n buffers (GRAD[r]) of one GPU.  DP_ERR_STATE
 * if the replicas are at different micro-steps, or first == 0 before a first
 * micro-step. */
dp_status dp_accumulate_all(dp_plan* plan, int32_t first, hipStream_t stream);

/* dp_accumulate_all over one bucket [begin, end) of the flat space, so each
 * micro-step's accumulation can follow its backward pass bucket by bucket and
 * a bucket's gradient buffer is free for reuse as soon as it is added in [first
 * page, averaging formula paragraph: the a micro-steps of each device are
 * summed before the exchange].  The bucket rules are those of
 * dp_accumulate_reduce_range: each end a tensor start, P, or a multiple of 256
 * elements into its tensor (DP_ERR_INVALID_ARG); the buckets of one
 * micro-step come in any order and on several streams, do not overlap
 * (DP_ERR_STATE) and take the same first flag (DP_ERR_INVALID_ARG).  Once they
 * cover [0, P) the micro-step is complete and the accumulators hold, bit for
 * bit, what dp_accumulate_all(first) leaves.  Until then every other
 * accumulation, reduction, statistics or single-pass call returns
 * DP_ERR_STATE.  DP_ERR_STATE as for dp_accumulate_all for the micro-step
 * counts. */
dp_status dp_accumulate_all_range(dp_plan* plan, int32_t first, int64_t begin, int64_t end, hipStream_t stream);

/* The last micro-step fused with the replica average: GBAR = (sum_r
 * (ACC[r] + GRAD[r])) / n in the order of dp_reduce_replicas, plus the
 * per-chunk statistics; bit for bit the result of dp_accumulate on every
 * replica followed by dp_reduce_replicas(DP_ROLE_ACC), but ACC[r] is read and
 * not written back (it keeps the sum of the earlier micro-steps).  With no
 * earlier micro-step since the last reduction (a = 1, or incoming partials)
 * it is GBAR = (sum_r GRAD[r]) / n.  DP_ERR_STATE if the replicas are at
 * different micro-steps or before dp_state_init. */
dp_status dp_accumulate_reduce(dp_plan* plan, hipStream_t stream);

/* dp_accumulate_reduce over one bucket [begin, end) of the flat space, so the
 * reduction can start on the gradients the backward pass has finished while
 * it still computes the others -- the bucketed gradient all-reduce overlapped
 * with the backward pass that the pages describe for data parallelism (first
 * page, data-parallel all-reduce paragraph; "Data vs Tensor vs Pipeline
 * Parallelism: When to Use Each", abhik.ai, section "What each one splits /
 * Data parallelism").  A bucket's ends must each be a tensor start, P, or a
 * multiple of 256 elements into their tensor (DP_ERR_INVALID_ARG otherwise).
 * The buckets of one reduction may come in any order and on several streams;
 * they must not overlap (DP_ERR_STATE), and together they cover [0, P).  The
 * reduction is complete when they do: it then gives, bit for bit, the
 * g_bar and the per-chunk statistics of dp_accumulate_reduce.  Until then
 * dp_grad_stats, the accumulation calls and the other reductions return
 * DP_ERR_STATE.  The caller orders dp_grad_stats after every bucket's
 * launch, for example with events when the buckets run on other streams. */
dp_status dp_accumulate_reduce_range(dp_plan* plan, int64_t begin, int64_t end, hipStream_t stream);

/* dp_reduce_replicas over one bucket [begin, end): GBAR = (sum_r src[r]) / n
 * in the fixed order, from the accumulators after all micro-steps (src =
 * DP_ROLE_ACC) or from n incoming partials (src = DP_ROLE_GRAD), plus the
 * bucket's per-chunk statistics.  The bucketed reduction of the same
 * paragraphs as dp_accumulate_reduce_range, for callers that accumulate the
 * last micro-step separately or receive partials in pieces.  The bucket
 * rules, the completion once the buckets cover [0, P) and the DP_ERR_STATE
 * of the other calls until then are those of dp_accumulate_reduce_range; the
 * complete reduction gives, bit for bit, the g_bar and statistics of
 * dp_reduce_replicas(src).  Every bucket of one reduction takes the same
 * sources, including across the two bucket calls (DP_ERR_INVALID_ARG).
 * DP_ERR_STATE with DP_ROLE_ACC when the replicas accumulated different
 * numbers of micro-steps, or none. */
dp_status dp_reduce_replicas_range(dp_plan* plan, dp_role src, int64_t begin, int64_t end, hipStream_t stream);

/* Replica average [first page, averaging formula and reduction-order
 * paragraph]: GBAR = (sum_r SRC[r]) / n over [0, P) with a fixed pairwise order
 * (adjacent pairs by levels, an odd last term carried, binary32 partial sums),
 * and the per-chunk statistics of GBAR.  src is DP_ROLE_ACC (the
 * accumulators; every replica must have the same number of micro-steps, else
 * DP_ERR_STATE) or DP_ROLE_GRAD (n low-precision partials, a = 1). */
dp_status dp_reduce_replicas(dp_plan* plan, dp_role src, hipStream_t stream);

/* Global statistics and per-step scalars of g_bar: its sum of squares and
 * whether it holds an inf or NaN, then the step's scalars.  The pages ask
 * that the reduction's numerics be aligned between runs, naming loss
 * scaling and reduction precision together ("Distributed Training ...":
 * evaluation paragraph on training semantics, and the reduction-order
 * paragraph: the summation order changes the bits), and count loss scaling
 * as state (checkpoint-contents paragraph).  The sum of squares is kept in
 * binary64 in a fixed order.  Global-norm clipping (max_norm) is not on the
 * pages: it comes from the workloads this library is built for, which clip
 * at 1.0; the norm is the unscaled one over the whole plan, so a shard's
 * update equals the unsharded one (same page, ZeRO paragraph).
 *
 * scan != 0 first reads GBAR to
 * write the per-chunk statistics; scan == 0 uses those written by
 * dp_reduce_replicas or dp_accumulate(emit_stats) (DP_ERR_STATE if there are
 * none).  Then, on the device: norm = sqrt(sum g_bar^2) / scale; if any entry
 * of g_bar is inf or NaN the step is skipped (iter += 1, a dynamic scale backs
 * off); otherwise clip = max_norm / norm when max_norm > 0 and norm >
 * max_norm (else 1), gscale = clip / scale, t += 1, the beta powers advance,
 * iter += 1, and a dynamic scale grows after growth_interval clean steps.
 * DP_ERR_STATE before dp_state_init. */
dp_status dp_grad_stats(dp_plan* plan, int32_t scan, double max_norm, hipStream_t stream);

/* The fused update over [shard_begin, shard_end) [first page,
 * mixed-precision and ZeRO paragraphs; Adam with bias correction and
 * decoupled weight decay]: one read of GBAR, MASTER, EXP_AVG, EXP_AVG_SQ and
 * one write of MASTER, EXP_AVG, EXP_AVG_SQ, PARAM per element:
 *   g = g_bar * gscale
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2
 *   w = w (1 - lr wd) - lr / (1 - beta1^t) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 *   p = w rounded to nearest-even in the param dtype
 * computed in binary64 and stored in binary32.  Nothing is written when the
 * finalised step was skipped.  Any partition of [0, P) into ranges gives the
 * same result as one call on [0, P).  DP_ERR_STATE if dp_grad_stats has not
 * run since the last accumulation or reduction.  No range needs a table of
 * its own, so no range allocates: with every role bound flat the launch
 * covers the range's own pieces, otherwise the pieces of the [0, P) chunk
 * table that overlap it, each clipped to the range. */
dp_status dp_adam_step(dp_plan* plan, const dp_adam_hparams* hp, int64_t shard_begin, int64_t shard_end,
                       hipStream_t stream);

/* The whole step after the micro-steps, in one pass over memory, for runs
 * without gradient clipping.  It reads the sources of dp_accumulate_reduce
 * (ACC[r] + GRAD[r], or GRAD[r] alone with no earlier micro-step since the last
 * reduction) and the current state bank once.  It writes the other bank and
 * PARAM once.  g_bar is never stored.
 *
 * Without clipping, the statistics of g_bar change the update only through the
 * skip decision [first page, loss scaling as part of the training state].  So
 * every element's update is computed before that decision is known, with the
 * scalars the step has if it is applied: gscale = 1 / scale and t + 1.  The
 * finalisation of dp_grad_stats(scan = 0, max_norm = 0) then runs on the
 * device.  If the step is applied, the written bank becomes current.  If it is
 * skipped, the current bank stays as it was and PARAM is emitted again from
 * its master.
 *
 * The result, bit for bit, is that of dp_accumulate_reduce, dp_grad_stats(0,
 * 0) and dp_adam_step over [0, P): the same state and the same scalars.  This
 * assumes PARAM held the round-to-nearest-even image of the current master
 * before the call, as dp_adam_step leaves it.
 *
 * Needs both banks of MASTER, EXP_AVG and EXP_AVG_SQ (DP_ERR_UNBOUND).
 * DP_ERR_STATE if the replicas are at different micro-steps or before
 * dp_state_init.  Afterwards dp_adam_step returns DP_ERR_STATE until the next
 * step's statistics. */
dp_status dp_reduce_adam_step(dp_plan* plan, const dp_adam_hparams* hp, hipStream_t stream);

/* For callers that cannot allocate device memory -- work recorded under HIP
 * graph capture, allocation-free serving loops, harnesses that forbid
 * hipMalloc: dp_reduce_adam_step for a plan of one tensor of P elements with
 * every role bound flat and the default chunk size, without a plan.  Nothing
 * is allocated.  The scratch the kernels need (statistics slots, the fold's
 * second level, the chunk table) is one static device array of
 * DP_STATIC_SCRATCH_BYTES (49.5 MiB) that each GPU holds from the library's
 * first use there until the process ends; P may not exceed
 * DP_STATIC_MAX_PARAMS (2^30; DP_ERR_INVALID_ARG beyond).
 *
 * The caller passes every input and output:
 *  - grads: host array [n] of device pointers, replica r's last micro-step
 *    (or incoming partial) in the grad dtype, P elements each;
 *  - accs: host array [n] of device pointers to binary32 accumulators that
 *    hold the sum of the earlier micro-steps (read, not written), or NULL when
 *    there were none;
 *  - master, exp_avg, exp_avg_sq: host arrays [2] of device pointers, the two
 *    binary32 banks of each; param: device, P elements of the param dtype;
 *  - state: device memory holding a dp_step_state (8-byte aligned), read and
 *    written.  The caller sets it up once, for example by copying a host
 *    struct with t = iter = growth_tracker = 0, beta1_pow = beta2_pow = 1,
 *    scale = the initial loss scale (1 without a scaler), bank = 0 and
 *    found_inf = 0; state->bank then says which bank is current;
 *  - cfg: the scaler and the betas, as for dp_state_init; hp as for
 *    dp_reduce_adam_step.
 *
 * The result, the two banks, the parameters and the state block, equals bit
 * for bit what dp_reduce_adam_step leaves on such a plan in the same state.
 * On a skipped step the current bank stays current and PARAM is emitted
 * again from it.
 *
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind.  The call clears what has to start at zero itself, but calls that
 * overlap on one GPU (on different streams, or from different threads) race
 * on the array and give wrong results.  The first call on each device
 * resolves the array's device address (hipGetSymbolAddress): make it outside
 * graph capture.  Asynchronous on stream. */
dp_status dp_reduce_adam_step_noalloc(int64_t P, int32_t n, dp_dtype grad_dtype, dp_dtype param_dtype,
                                      void* const* grads, void* const* accs, void* const* master,
                                      void* const* exp_avg, void* const* exp_avg_sq, void* param,
                                      dp_step_state* state, const dp_state_cfg* cfg, const dp_adam_hparams* hp,
                                      hipStream_t stream);

/* dp_reduce_adam_step in buckets: the single pass over one bucket [begin,
 * end) of the flat space, so the update of the parameters whose gradients
 * (or incoming partials) are complete can run while the backward pass, or
 * the exchange, still produces the others (the bucketed overlap of the
 * pages' data-parallel all-reduce, as for dp_accumulate_reduce_range).  The
 * bucket rules are those of dp_accumulate_reduce_range: ends on the piece
 * grid (DP_ERR_INVALID_ARG), no overlap (DP_ERR_STATE), any order, any
 * streams.  Every bucket of one step takes the same hp (DP_ERR_INVALID_ARG
 * otherwise).  Each bucket updates its elements into the other state bank
 * with the scalars of an applied step and writes its statistics; nothing is
 * committed until dp_reduce_adam_finish.  Until then every other step call
 * returns DP_ERR_STATE. */
dp_status dp_reduce_adam_range(dp_plan* plan, const dp_adam_hparams* hp, int64_t begin, int64_t end,
                               hipStream_t stream);

/* Completes a bucketed single pass once its buckets cover [0, P)
 * (DP_ERR_STATE before): the statistics fold and the commit or skip of the
 * step, with the parameters emitted again after a skip, exactly as at the
 * end of dp_reduce_adam_step.  The result equals dp_reduce_adam_step bit
 * for bit.  The caller orders this call after every bucket's launch, for
 * example with events when the buckets ran on other streams. */
dp_status dp_reduce_adam_finish(dp_plan* plan, hipStream_t stream);

/* Copies the device scalar state into host struct out after the stream's
 * previous work (synchronises the stream). */
dp_status dp_read_state(dp_plan* plan, dp_step_state* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DPSTEP_H */
