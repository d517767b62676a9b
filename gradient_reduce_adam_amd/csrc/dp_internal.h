// Internal interface between the C-ABI layer (api.cpp) and the gfx950
// kernels (kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dpstep.h"

namespace dpk {

constexpr int kBlock = 256;              // threads per workgroup: 4 wave64s
constexpr int64_t kMaxBlocksPerLaunch = 1 << 20;

// Where one role's memory is: a flat base (tensor i at element prefix[i]) or
// a device table of per-tensor pointers.
struct RoleRef {
    void* base;        // flat binding, or nullptr
    void* const* tab;  // device array [num_tensors] of per-tensor pointers, or nullptr
};

struct Srcs {
    RoleRef r[DP_MAX_REPLICAS];
};

// Device copy of the scalar state; the layout equals dp_step_state so the
// host reads it back with one copy.
struct DevState {
    int64_t t, iter, growth_tracker;
    double beta1_pow, beta2_pow, scale;
    int32_t found_inf, reserved;
    double sumsq, norm, clip, gscale;
};
static_assert(sizeof(DevState) == sizeof(dp_step_state), "DevState must mirror dp_step_state");

// Per-chunk statistics of g_bar: binary64 sum of squares and the count of
// non-finite entries.  Index = position of the chunk in the [0, P) table.
struct StatsBuf {
    double* sumsq;
    uint32_t* bad;
};

// Second level of the statistics fold: one entry per group of kFoldGroup
// chunk partials (used when a table has more than kFoldGroup chunks).
constexpr int64_t kFoldGroup = 4096;
struct FoldBuf {
    double* sumsq;
    uint64_t* bad;
};

struct AdamArgs {
    double lr, eps, weight_decay, beta1, beta2;
};

struct ScalerArgs {
    double beta1, beta2, backoff, growth, max_norm;
    int32_t mode, growth_interval;
};

hipError_t launch_accumulate(dp_dtype gdt, bool first, bool stats, const dp_chunk* chunks, int64_t nchunks,
                             RoleRef grad, RoleRef acc, StatsBuf sb, hipStream_t stream);
hipError_t launch_accumulate_all(dp_dtype gdt, bool first, int n, const dp_chunk* chunks, int64_t nchunks,
                                 const Srcs& grads, const Srcs& accs, hipStream_t stream);

// What each replica contributes to the reduction.
enum class ReduceMode {
    kAccumulators,  // acc_r (binary32)
    kGradients,     // g_r (the gradient dtype): partials, or a single micro-step
    kAccPlusGrad    // acc_r + g_r: the last micro-step fused, acc_r not written back
};
hipError_t launch_reduce(ReduceMode mode, dp_dtype gdt, int n, const dp_chunk* chunks, int64_t nchunks,
                         const Srcs& accs, const Srcs& grads, RoleRef gbar, StatsBuf sb, hipStream_t stream);
hipError_t launch_stats(const dp_chunk* chunks, int64_t nchunks, RoleRef gbar, StatsBuf sb, hipStream_t stream);
hipError_t launch_finalize(StatsBuf sb, int64_t nparts, FoldBuf fold, DevState* st, const ScalerArgs& args,
                           hipStream_t stream);
hipError_t launch_adamw(dp_dtype pdt, const dp_chunk* chunks, int64_t nchunks, RoleRef gbar, RoleRef w, RoleRef m,
                        RoleRef v, RoleRef p, const DevState* st, const AdamArgs& args, hipStream_t stream);
hipError_t launch_state_init(DevState* st, double scale, hipStream_t stream);

}  // namespace dpk
