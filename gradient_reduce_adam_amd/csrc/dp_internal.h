// Internal interface between the C-ABI layer (api.cpp) and the gfx950
// kernels (kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dpstep.h"

namespace dpk {

constexpr int kWave = 64;                 // threads per streaming workgroup: one wave64
constexpr int kPiece = 4 * kWave;         // elements per streaming workgroup: 4 per lane
constexpr int kFoldThreads = 256;         // threads of the statistics fold workgroups
// workgroups per dispatch: gridDim.x * kWave must stay below 2^32, so one call
// covers up to 2^26 pieces (17e9 elements) in a single dispatch
constexpr int64_t kMaxBlocksPerLaunch = (int64_t{1} << 26) - 1;

// The pieces of one call's range [begin, end), as the kernels see them.
//  flat:  every role of the call is one flat buffer; piece p covers flat
//         elements [floor4(begin) + p * kPiece, ... + kPiece) within the range
//  table: the chunk table of the range; npieces = chunks << log2s, piece p is
//         piece (p & (2^log2s - 1)) of chunk (p >> log2s) (pieces past a short
//         chunk's end are empty)
struct Table {
    const dp_chunk* chunks;
    int64_t begin, end;
    int64_t npieces;
    int log2s;  // log2(chunk_elems / kPiece)
    bool flat;
};

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

// Per-piece statistics of g_bar: binary64 sum of squares and the count of
// non-finite entries.  Index = position of the piece in the [0, P) table.
struct StatsBuf {
    double* sumsq;
    uint32_t* bad;
};

// Second level of the statistics fold: one entry per group of kFoldGroup
// piece partials (used when a table has more than kFoldGroup pieces).
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

hipError_t launch_accumulate(dp_dtype gdt, bool first, bool stats, const Table& t, RoleRef grad, RoleRef acc,
                             StatsBuf sb, hipStream_t stream);
hipError_t launch_accumulate_all(dp_dtype gdt, bool first, int n, const Table& t, const Srcs& grads, const Srcs& accs,
                                 hipStream_t stream);

// What each replica contributes to the reduction.
enum class ReduceMode {
    kAccumulators,  // acc_r (binary32)
    kGradients,     // g_r (the gradient dtype): partials, or a single micro-step
    kAccPlusGrad    // acc_r + g_r: the last micro-step fused, acc_r not written back
};
hipError_t launch_reduce(ReduceMode mode, dp_dtype gdt, int n, const Table& t, const Srcs& accs, const Srcs& grads,
                         RoleRef gbar, StatsBuf sb, hipStream_t stream);
hipError_t launch_stats(const Table& t, RoleRef gbar, StatsBuf sb, hipStream_t stream);
hipError_t launch_finalize(StatsBuf sb, int64_t nparts, FoldBuf fold, DevState* st, const ScalerArgs& args,
                           hipStream_t stream);
hipError_t launch_adamw(dp_dtype pdt, const Table& t, RoleRef gbar, RoleRef w, RoleRef m, RoleRef v, RoleRef p,
                        const DevState* st, const AdamArgs& args, hipStream_t stream);
hipError_t launch_state_init(DevState* st, double scale, hipStream_t stream);

}  // namespace dpk
