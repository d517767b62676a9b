/*
 * dpckpt.h -- checkpoint and resume of the data-parallel step's state, with
 * resharding, for the library of dpstep.h.
 *
 * What a checkpoint holds.  Every piece of the training state the step reads
 * back:
 *  - the optimizer state (master, m, v);
 *  - the low-precision parameters;
 *  - the scalar state: t, the beta powers, the loss scale and its growth
 *    tracker.
 * The pages list the optimizer state and the loss-scaling state as part of
 * what a checkpoint must keep ("Distributed Training: Split along the Four
 * Axes of Data, Tensor, Pipeline, and State", ai-knowledge-map.com: checkpoint
 * contents and loss-scaling paragraphs).  Under ZeRO each rank holds only its
 * shard of that state (same page, ZeRO paragraph), so a checkpoint is written
 * shard by shard.  It can be read back over any other partition of the flat
 * parameter space: that is resharding, for example 8 shards restored as 4.
 *
 * Layout on disk, one directory per run.
 *  - Shard files "g<generation>-<begin>-<end>.dpshard".  Each has a 256-byte
 *    header, a table of 64-bit block checksums (one per 2^20 elements of each
 *    array), then master, m, v (binary32) and the parameters (param dtype) of
 *    [begin, end), each array starting on a 4096-byte boundary.
 *  - The manifest "manifest.dpck", a text file.  It holds the tensor layout,
 *    the scalar state and optimizer settings (doubles as exact bit patterns),
 *    and the list of shard files of one generation.  It ends with a checksum
 *    line.
 *
 * The commit protocol.  Shard files are written under a temporary name,
 * flushed, then renamed.  The manifest is replaced the same way, by one
 * rename.  Until that rename, a reader sees the previous generation whole.
 * A process killed at any point leaves either the old or the new generation
 * readable, never a mix.  Files of other generations are removed only after a
 * commit.
 *
 * Integrity.  Reads verify the checksums of every block they touch, the
 * header checks and the manifest checksum (DP_ERR_CORRUPT on a mismatch).  The
 * checksums detect corruption; they are not cryptographic.
 *
 * Conventions: as in dpstep.h.  Every call here is synchronous, and does host
 * file I/O; none is meant for the step's hot loop.
 */
#ifndef DPCKPT_H
#define DPCKPT_H

#include "dpstep.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ---- host layer: host memory only, no GPU is touched ------------------- */

/* Writes shard [begin, end) of generation `generation` into directory dir
 * (which must exist).  The data comes from host arrays master, exp_avg and
 * exp_avg_sq (binary32) and param (layout->param_dtype), each holding end -
 * begin elements.  layout gives the tensor list, which is checked on commit
 * and on read.  Nothing refers to the file until dp_ckpt_commit.
 * DP_ERR_RANGE if [begin, end) is not inside [0, P); DP_ERR_IO on a file
 * system error. */
dp_status dp_ckpt_write_shard(const char* dir, int64_t generation, const dp_layout* layout, int64_t begin,
                              int64_t end, const float* master, const float* exp_avg, const float* exp_avg_sq,
                              const void* param);

/* Commits generation `generation` of dir.  Its shard files must tile [0, P)
 * exactly, with no gap and no overlap; empty shards are allowed.  Their
 * headers must match layout.  The manifest records scalars (host) and cfg
 * (host).  Shard files of every other generation are removed afterwards.
 * DP_ERR_STATE if the shards do not tile the range; DP_ERR_CORRUPT on a bad
 * header; DP_ERR_IO on a file system error. */
dp_status dp_ckpt_commit(const char* dir, int64_t generation, const dp_layout* layout, const dp_step_state* scalars,
                         const dp_state_cfg* cfg);

/* Reads [begin, end) of the committed generation of dir into the host arrays.
 * Any array pointer may be null, and that array is then skipped.  The range
 * may cross any number of shard files, so any partition of [0, P) can be read
 * back from any partition that was written.  The scalar state, the optimizer
 * settings and the generation number go to *scalars, *cfg and *generation;
 * each of these may be null.
 * DP_ERR_STATE if dir holds no committed checkpoint; DP_ERR_BAD_LAYOUT if
 * layout (tensor list, param dtype) differs from the checkpoint's;
 * DP_ERR_CORRUPT on a checksum mismatch; DP_ERR_IO on a file system error. */
dp_status dp_ckpt_read(const char* dir, const dp_layout* layout, int64_t begin, int64_t end, float* master,
                       float* exp_avg, float* exp_avg_sq, void* param, dp_step_state* scalars, dp_state_cfg* cfg,
                       int64_t* generation);

/* ---- device layer: a plan's bound memory ------------------------------- */

/* Writes shard [begin, end) of the plan's current state bank (MASTER,
 * EXP_AVG, EXP_AVG_SQ) and PARAM, as dp_ckpt_write_shard.  It runs between
 * steps: it synchronises stream first, then copies through pinned host
 * buffers of at most 64 MiB, which it allocates and frees.  The roles may be
 * bound flat or per tensor.  DP_ERR_STATE before dp_state_init. */
dp_status dp_checkpoint_save(dp_plan* plan, const char* dir, int64_t generation, int64_t begin, int64_t end,
                             hipStream_t stream);

/* Commits generation `generation` with the plan's device scalar state and
 * optimizer settings, as dp_ckpt_commit (synchronises stream). */
dp_status dp_checkpoint_commit(dp_plan* plan, const char* dir, int64_t generation, hipStream_t stream);

/* Restores [begin, end) of the committed checkpoint into the current bank of
 * MASTER, EXP_AVG, EXP_AVG_SQ and into PARAM; the current bank stays current,
 * and the plan's state outside [begin, end) is left as it was.  A plan that
 * resumes a run restores every range it updates.  restore_scalars != 0 also
 * sets the device scalar state: t, iter, the beta powers, the scale and the
 * growth tracker.  The plan's optimizer settings (dp_state_init) must then
 * equal the checkpoint's, else DP_ERR_STATE.  Accumulation restarts: the next
 * call must be a first micro-step.  The call synchronises stream, and
 * allocates and frees pinned host buffers.  Errors are those of dp_ckpt_read,
 * plus DP_ERR_STATE before dp_state_init.  A layout, range or settings
 * mismatch is found in the manifest before any of the plan's memory is
 * written; a corrupt shard block or a generation committed by another writer
 * during the load (DP_ERR_STATE) can leave the range partly restored. */
dp_status dp_checkpoint_load(dp_plan* plan, const char* dir, int64_t begin, int64_t end, int32_t restore_scalars,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DPCKPT_H */
