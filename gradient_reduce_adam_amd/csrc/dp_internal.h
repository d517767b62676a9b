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
    int32_t found_inf, bank;
    double sumsq, norm, clip, gscale;
};
static_assert(sizeof(DevState) == sizeof(dp_step_state), "DevState must mirror dp_step_state");

// Per-piece statistics of g_bar: binary64 sum of squares and the count of
// non-finite entries of piece p of the [0, P) table, at slot
// (p % 8) * ceil(npieces / 8) + p / 8.  Consecutive workgroups go round-robin
// to the 8 XCDs, so this keeps the slots one XCD writes contiguous in its own
// L2 and they leave it as whole lines.  The fold adds the slots in slot order;
// the few slots no piece maps to stay zero.
struct StatsBuf {
    double* sumsq;
    uint32_t* bad;
};
inline int64_t stats_slots(int64_t npieces) { return 8 * ((npieces + 7) / 8); }

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
    int32_t flip_bank;  // an applied step makes the other state bank current
};

// The optimizer state in two banks: bank st->bank is current.  The two-pass
// update works in place on the current bank; the single-pass update reads it
// and writes the other one.  Bank 1 is unbound (null) unless the caller gave
// one.
struct StateRefs {
    RoleRef w[2], m[2], v[2];
};

hipError_t launch_accumulate(dp_dtype gdt, bool first, bool stats, const Table& t, RoleRef grad, RoleRef acc,
                             StatsBuf sb, hipStream_t stream);

// What each replica contributes to the reduction.
enum class ReduceMode {
    kAccumulators,  // acc_r (binary32)
    kGradients,     // g_r (the gradient dtype): partials, or a single micro-step
    kAccPlusGrad    // acc_r + g_r: the last micro-step fused, acc_r not written back
};
// Pieces [p0, p1) of a table: the whole table, or one bucket of it.
struct PieceSpan {
    int64_t p0, p1;
};
// Every replica's micro-step over pieces [p0, p1) of the table (flat pieces
// only for the first micro-step).
hipError_t launch_accumulate_all(dp_dtype gdt, bool first, int n, const Table& t, PieceSpan sp, const Srcs& grads,
                                 const Srcs& accs, hipStream_t stream);
hipError_t launch_reduce(ReduceMode mode, dp_dtype gdt, int n, const Table& t, PieceSpan sp, const Srcs& accs,
                         const Srcs& grads, RoleRef gbar, StatsBuf sb, hipStream_t stream);
hipError_t launch_stats(const Table& t, RoleRef gbar, StatsBuf sb, hipStream_t stream);
hipError_t launch_finalize(StatsBuf sb, int64_t nparts, FoldBuf fold, DevState* st, const ScalerArgs& args,
                           hipStream_t stream);
// The update over pieces [p0, p1): flat pieces of the call's range, or the
// pieces of the [0, P) table that overlap the range [t.begin, t.end), each
// clipped to it.
hipError_t launch_adamw(dp_dtype pdt, const Table& t, PieceSpan sp, RoleRef gbar, const StateRefs& s, RoleRef p,
                        const DevState* st, const AdamArgs& args, hipStream_t stream);
// Single pass: the replica average of launch_reduce (same sources, order and
// statistics) feeding the update of every element, from the current bank into
// the other, with the scalars the step will have if it is applied (no clip).
// Pieces [p0, p1) of the table: the whole table, or one bucket of it.
hipError_t launch_reduce_adamw(ReduceMode mode, dp_dtype gdt, dp_dtype pdt, int n, const Table& t, PieceSpan sp,
                               const Srcs& accs, const Srcs& grads, const StateRefs& s, RoleRef p, StatsBuf sb,
                               const DevState* st, const AdamArgs& args, hipStream_t stream);
// After a skipped single-pass step: p = RNE(w) from the current bank again
// (does nothing when the step was applied).
hipError_t launch_restore_param(dp_dtype pdt, const Table& t, const StateRefs& s, RoleRef p, const DevState* st,
                                hipStream_t stream);
hipError_t launch_state_init(DevState* st, double scale, hipStream_t stream);

// Copies of per-tensor pointer tables from pinned host memory (readable by
// the device) into device tables, all of one launch's pending ones at once:
// tables [0, count), T pointers each.
constexpr int kMaxUploads = 2 * DP_MAX_REPLICAS + 8;
struct TableUploads {
    const void* const* src[kMaxUploads];
    void** dst[kMaxUploads];
    int32_t count;
    int32_t T;
};
hipError_t launch_upload_tables(const TableUploads& u, hipStream_t stream);
// The chunk table of one tensor [0, P) (chunks of 2^log2c elements) into
// device memory `chunks`, and zeros in the statistics slots that no piece of
// its npieces maps to (the fold adds them).
hipError_t launch_flat_table(dp_chunk* chunks, int64_t P, int log2c, StatsBuf sb, int64_t npieces,
                             hipStream_t stream);

}  // namespace dpk
