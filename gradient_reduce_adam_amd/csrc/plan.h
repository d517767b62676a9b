// The plan object behind the C ABI, shared by the files that implement it
// (api.cpp: plans, bindings, the step; checkpoint.cpp: save and restore).
#pragma once

#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "dp_internal.h"
#include "dpstep.h"

namespace dpapi {

constexpr int kNumRoles = 7;

// Per-tensor pointer tables of one role live in a ring of kRingSlots device
// tables.  A rebinding fills the next slot's pinned staging copy on the host
// and returns; the next launch that reads the role uploads it on that
// launch's own stream, ahead of itself (one small kernel copies every table
// the launch finds pending), and launches on other streams wait for that
// upload.  Launches still reading an earlier slot are undisturbed.
// A slot is written again only kRingSlots rebindings later, after the
// launches that read it (events recorded behind each) have finished.
constexpr int kRingSlots = 4;

// Events shared by the pointer-table slots: one is recorded behind each
// launch that reads per-tensor tables and one behind each upload of tables,
// and every slot involved holds a reference, so a launch adds at most two
// event records to its stream however many tables it reads.  An event
// returns to the free list when its last reference goes.
struct EventPool {
    std::vector<hipEvent_t> ev;
    std::vector<int> refs;
    std::vector<int> free_list;
};

// Where one role's memory is: one flat buffer, or one pointer per tensor
// (kept on the host and mirrored in the current slot of the device ring).
struct Binding {
    void* flat = nullptr;
    std::vector<void*> tensors;  // host copy of the per-tensor pointers
    void** dev_table = nullptr;  // device table of the current slot; null for a flat binding
    bool bound = false;

    void** ring_dev = nullptr;   // kRingSlots device tables of T pointers (first per-tensor binding)
    void** ring_host = nullptr;  // their pinned staging copies
    void** ring_host_dev = nullptr;  // the staging copies' device-side address
    int slot = -1;               // current slot
    bool pending = false;        // the current slot's staging copy is not on the device yet
    // events of the plan's pool (EventPool indices, -1: none) that a slot
    // holds: behind its upload, and per stream behind the last launch there
    // that read it
    int uploaded[kRingSlots] = {-1, -1, -1, -1};
    hipStream_t upload_stream[kRingSlots] = {};
    std::vector<std::pair<hipStream_t, int>> uses[kRingSlots];

    dpk::RoleRef ref() const { return dpk::RoleRef{flat, dev_table}; }
};

struct DeviceTable {
    int64_t begin = 0, end = 0, count = 0;  // count: chunks
    dp_chunk* dev = nullptr;
    int log2s = 0;

    // pieces of a launch over this range: direct flat pieces when every role
    // of the call is flat-bound, else pieces of the chunks
    int64_t npieces(bool flat) const {
        if (!flat) return count << log2s;
        const int64_t lo = begin & ~int64_t{3};
        return end > begin ? (end - lo + dpk::kPiece - 1) / dpk::kPiece : 0;
    }
    dpk::Table table(bool flat) const { return dpk::Table{dev, begin, end, npieces(flat), log2s, flat}; }
};

// Records the message of a failure for dp_last_error() and returns s; for
// DP_ERR_OOM and DP_ERR_HIP it also resets the runtime's last error.
dp_status fail(dp_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dp_status hip_fail(hipError_t e, const char* what);
extern thread_local std::string g_last_error;

}  // namespace dpapi

struct dp_plan {
    std::vector<int64_t> numel, prefix;
    int64_t P = 0;
    int32_t T = 0, n = 1, chunk = DP_DEFAULT_CHUNK;
    dp_dtype gdt = DP_BF16, pdt = DP_BF16;

    dpapi::Binding roles[dpapi::kNumRoles][DP_MAX_REPLICAS];
    dpapi::EventPool events;  // of the per-tensor pointer-table rings

    // device resources (allocated by the first GPU call: dp_state_init, prepare_range or bind_tensors)
    int device = -1;
    dpk::DevState* state = nullptr;
    dpk::StatsBuf stats{nullptr, nullptr};
    dpk::FoldBuf fold{nullptr, nullptr};
    dpapi::DeviceTable full;
    std::vector<dp_chunk> full_host;  // host copy of the [0, P) chunk table

    // ordering state
    bool state_ready = false;
    dp_state_cfg cfg{};
    std::vector<int32_t> micro;   // micro-steps accumulated per replica since the last reduction
    bool partials_valid = false;  // piece statistics of the current g_bar exist
    int64_t partials_count = 0;   // how many (they follow the launch that wrote them)
    bool stats_current = false;   // dp_grad_stats ran on the current g_bar
    // a call issued in buckets: the element ranges done so far, until they
    // cover [0, P).  bucket_mode 1: reduction buckets
    // (dp_accumulate_reduce_range, dp_reduce_replicas_range), all from the
    // same sources, complete once they cover [0, P); 2:
    // single-pass buckets (dp_reduce_adam_range), with the update
    // hyperparameters of the first one, complete at dp_reduce_adam_finish;
    // 3: buckets of one micro-step of every replica (dp_accumulate_all_range),
    // with the `first` flag of the first one, complete once they cover [0, P)
    std::vector<std::pair<int64_t, int64_t>> buckets;
    int64_t bucket_elems = 0;
    int bucket_mode = 0;
    dp_adam_hparams bucket_hp{};
    int32_t bucket_first = 0;
    int bucket_src = 0;  // mode 1: 0 the last micro-step fused, else the role reduced
};

namespace dpapi {
// Binds the plan to the current device on first use; DP_ERR_STATE if another
// device is current later.
dp_status ensure_device(dp_plan* p);
}  // namespace dpapi
