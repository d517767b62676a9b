// Kernel launchers for a host-only build of the C-ABI layer (api.cpp,
// checkpoint.cpp) under a sanitizer: every launch reports hipErrorNotSupported.
// Only the calls that never reach a launch (plans, chunk tables, bindings,
// argument and order checks, the checkpoint host layer) are meant to run in
// such a build.
#include "dp_internal.h"

namespace dpk {

hipError_t launch_accumulate(dp_dtype, bool, bool, const Table&, RoleRef, RoleRef, StatsBuf, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_accumulate_all(dp_dtype, bool, int, const Table&, PieceSpan, const Srcs&, const Srcs&, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_reduce(ReduceMode, dp_dtype, int, const Table&, PieceSpan, const Srcs&, const Srcs&, RoleRef,
                         StatsBuf, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_stats(const Table&, RoleRef, StatsBuf, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_finalize(StatsBuf, int64_t, FoldBuf, DevState*, const ScalerArgs&, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_adamw(dp_dtype, const Table&, PieceSpan, RoleRef, const StateRefs&, RoleRef, const DevState*,
                        const AdamArgs&, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_reduce_adamw(ReduceMode, dp_dtype, dp_dtype, int, const Table&, PieceSpan, const Srcs&,
                               const Srcs&, const StateRefs&, RoleRef, StatsBuf, const DevState*, const AdamArgs&,
                               hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_restore_param(dp_dtype, const Table&, const StateRefs&, RoleRef, const DevState*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_state_init(DevState*, double, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_upload_tables(const TableUploads&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace dpk
