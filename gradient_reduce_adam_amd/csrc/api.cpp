// C ABI of the data-parallel gradient reduce + AdamW step: plans, chunk
// tables, bindings, argument checks and the ordering rules between calls.
// The kernels live in kernels.hip; this file only validates and launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "dp_internal.h"
#include "dpstep.h"
#include "plan.h"

namespace dpapi {

thread_local std::string g_last_error;

dp_status fail(dp_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    // The error now belongs to this call's status and message.  Reset the
    // runtime's per-thread last error, or the caller's next HIP error check
    // (torch makes one after its own allocations and launches) would report
    // it again as its own.
    if (s == DP_ERR_OOM || s == DP_ERR_HIP) (void)hipGetLastError();
    return s;
}

dp_status hip_fail(hipError_t e, const char* what) {
    return fail(DP_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
}

dp_status ensure_device(dp_plan* p) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (p->device >= 0 && p->device != dev)
        return fail(DP_ERR_STATE, "plan was set up on device %d, current device is %d", p->device, dev);
    p->device = dev;
    return DP_OK;
}

}  // namespace dpapi

using dpapi::Binding;
using dpapi::DeviceTable;
using dpapi::ensure_device;
using dpapi::fail;
using dpapi::hip_fail;
using dpapi::kNumRoles;

namespace {

int log2_exact(int64_t x) {
    int k = 0;
    while ((int64_t{1} << k) < x) ++k;
    return k;
}

size_t esize(dp_dtype d) { return d == DP_F32 ? 4 : 2; }

}  // namespace

namespace {

// Both banks of the optimizer state (bank 1 null when unbound).
dpk::StateRefs state_refs(const dp_plan* p) {
    dpk::StateRefs s{};
    for (int b = 0; b < 2; ++b) {
        s.w[b] = p->roles[DP_ROLE_MASTER][b].ref();
        s.m[b] = p->roles[DP_ROLE_EXP_AVG][b].ref();
        s.v[b] = p->roles[DP_ROLE_EXP_AVG_SQ][b].ref();
    }
    return s;
}

// Chunk table of [begin, end): every tensor piece inside the range, split at
// multiples of chunk_elems counted from the tensor's start (so a chunk keeps
// the tensor's alignment), in flat order.
void build_chunks(const dp_plan* p, int64_t begin, int64_t end, std::vector<dp_chunk>* out) {
    out->clear();
    if (begin >= end) return;
    int32_t t = static_cast<int32_t>(std::upper_bound(p->prefix.begin(), p->prefix.end(), begin) - p->prefix.begin()) - 1;
    for (; t < p->T && p->prefix[t] < end; ++t) {
        const int64_t t0 = p->prefix[t], t1 = p->prefix[t + 1];
        const int64_t lo = std::max(begin, t0), hi = std::min(end, t1);
        if (lo >= hi) continue;
        int64_t off = lo - t0;
        while (off < hi - t0) {
            const int64_t next = (off / p->chunk + 1) * p->chunk;
            const int64_t stop = std::min(next, hi - t0);
            out->push_back(dp_chunk{t0 + off, off, t, static_cast<int32_t>(stop - off)});
            off = stop;
        }
    }
}

dp_status upload_table(dp_plan* p, int64_t begin, int64_t end, DeviceTable* out,
                       std::vector<dp_chunk>* keep = nullptr) {
    std::vector<dp_chunk> tmp;
    std::vector<dp_chunk>& host = keep ? *keep : tmp;
    build_chunks(p, begin, end, &host);
    out->begin = begin;
    out->end = end;
    out->count = static_cast<int64_t>(host.size());
    out->dev = nullptr;
    out->log2s = log2_exact(p->chunk / dpk::kPiece);
    if (host.empty()) return DP_OK;
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&out->dev), host.size() * sizeof(dp_chunk));
    if (e != hipSuccess) return fail(DP_ERR_OOM, "hipMalloc of a %zu-entry chunk table: %s", host.size(), hipGetErrorString(e));
    e = hipMemcpy(out->dev, host.data(), host.size() * sizeof(dp_chunk), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(out->dev);
        out->dev = nullptr;
        return hip_fail(e, "hipMemcpy of a chunk table");
    }
    return DP_OK;
}

// Every compute call passes through here: the plan's device must be current
// (kernels get pointers into its memory), and the [0, P) table must exist.
dp_status ensure_full(dp_plan* p) {
    dp_status s = ensure_device(p);
    if (s != DP_OK) return s;
    if (p->full.dev || p->P == 0 || p->full.count > 0) return DP_OK;
    return upload_table(p, 0, p->P, &p->full, &p->full_host);
}

// The piece of the [0, P) table that holds flat element x (0 <= x < P).
int64_t piece_holding(const dp_plan* p, int64_t x) {
    const auto& ch = p->full_host;
    const auto it = std::upper_bound(ch.begin(), ch.end(), x, [](int64_t v, const dp_chunk& c) { return v < c.flat; });
    const int64_t c = static_cast<int64_t>(it - ch.begin()) - 1;
    return (c << p->full.log2s) + (x - ch[static_cast<size_t>(c)].flat) / dpk::kPiece;
}

bool role_ok(dp_role r) { return r >= DP_ROLE_PARAM && r <= DP_ROLE_GBAR; }
bool per_replica(dp_role r) { return r == DP_ROLE_GRAD || r == DP_ROLE_ACC; }
bool banked(dp_role r) { return r == DP_ROLE_MASTER || r == DP_ROLE_EXP_AVG || r == DP_ROLE_EXP_AVG_SQ; }

const Binding* gbar_binding(const dp_plan* p) {
    const Binding* b = &p->roles[DP_ROLE_GBAR][0];
    if (!b->bound && p->n == 1) b = &p->roles[DP_ROLE_ACC][0];
    return b;
}

Binding* gbar_binding(dp_plan* p) { return const_cast<Binding*>(gbar_binding(static_cast<const dp_plan*>(p))); }

dp_status need(const Binding* b, const char* what) {
    if (!b->bound) return fail(DP_ERR_UNBOUND, "role %s is not bound", what);
    return DP_OK;
}

dp_status check_launch(hipError_t e, const char* what) { return e == hipSuccess ? DP_OK : hip_fail(e, what); }

bool all_flat(std::initializer_list<dpk::RoleRef> refs) {
    for (const dpk::RoleRef& r : refs)
        if (r.tab) return false;
    return true;
}

bool all_flat(const dpk::Srcs& s, int n) {
    for (int i = 0; i < n; ++i)
        if (s.r[i].tab) return false;
    return true;
}

bool all_flat(const dpk::StateRefs& s) {
    for (int b = 0; b < 2; ++b)
        if (s.w[b].tab || s.m[b].tab || s.v[b].tab) return false;
    return true;
}

const char* bucket_kind(int mode) {
    switch (mode) {
        case 1: return "reduction (dp_accumulate_reduce_range or dp_reduce_replicas_range)";
        case 2: return "single pass (dp_reduce_adam_range, then dp_reduce_adam_finish)";
        case 3: return "micro-step (dp_accumulate_all_range)";
    }
    return "call";
}

// Calls on whole accumulators or on g_bar may not run while a bucketed call
// is half done; a bucketed call may not start while buckets of another kind
// are open (mode: the caller's kind, 0 for a whole-space call).
dp_status no_open_buckets(const dp_plan* p, const char* where, int mode = 0) {
    if (!p->buckets.empty() && p->bucket_mode != mode)
        return fail(DP_ERR_STATE, "%s while a bucketed %s covers %lld of %lld elements", where,
                    bucket_kind(p->bucket_mode), static_cast<long long>(p->bucket_elems),
                    static_cast<long long>(p->P));
    return DP_OK;
}

// Replicas must be at the same micro-step; with first == 0, past the first.
dp_status same_micro_step(const dp_plan* p, bool first) {
    for (int32_t r = 0; r < p->n; ++r) {
        if (!first && p->micro[r] == 0)
            return fail(DP_ERR_STATE, "replica %d: first == 0 without a first micro-step since the last reduction", r);
        if (p->micro[r] != p->micro[0])
            return fail(DP_ERR_STATE, "replicas are at different micro-steps (replica %d: %d, replica 0: %d)", r,
                        p->micro[r], p->micro[0]);
    }
    return DP_OK;
}

// The piece of the [0, P) table that starts at flat element x, or -1 if no
// piece starts there (x must be a tensor start, or a multiple of 256 elements
// into its tensor); P maps to the table's end.
int64_t piece_at(const dp_plan* p, int64_t x) {
    const int64_t np = p->full.npieces(false);
    if (x == p->P) return np;
    const auto& ch = p->full_host;
    const auto it = std::upper_bound(ch.begin(), ch.end(), x,
                                     [](int64_t v, const dp_chunk& c) { return v < c.flat; });
    if (it == ch.begin()) return -1;
    const dp_chunk& c = *(it - 1);
    const int64_t off = x - c.flat;
    if (off >= c.len || off % dpk::kPiece != 0) return -1;
    return (static_cast<int64_t>(it - 1 - ch.begin()) << p->full.log2s) + off / dpk::kPiece;
}

// A bucket [begin, end) of a bucketed call: inside [0, P), both ends on the
// piece grid of the [0, P) table, and disjoint from the buckets already done.
// Its pieces go to *p0, *p1 (when not null).
dp_status bucket_span(dp_plan* p, int64_t begin, int64_t end, int64_t* p0, int64_t* p1) {
    if (begin < 0 || end > p->P || begin > end)
        return fail(DP_ERR_RANGE, "bucket [%lld, %lld) not inside [0, %lld)", static_cast<long long>(begin),
                    static_cast<long long>(end), static_cast<long long>(p->P));
    dp_status s = ensure_full(p);
    if (s != DP_OK) return s;
    const int64_t q0 = piece_at(p, begin), q1 = piece_at(p, end);
    if (q0 < 0 || q1 < 0)
        return fail(DP_ERR_INVALID_ARG,
                    "bucket [%lld, %lld): each end must be a tensor start, P, or a multiple of 256 elements into "
                    "its tensor",
                    static_cast<long long>(begin), static_cast<long long>(end));
    for (const auto& b : p->buckets)
        if (begin < b.second && b.first < end)
            return fail(DP_ERR_STATE, "bucket [%lld, %lld) overlaps bucket [%lld, %lld) of this reduction",
                        static_cast<long long>(begin), static_cast<long long>(end),
                        static_cast<long long>(b.first), static_cast<long long>(b.second));
    if (p0) *p0 = q0;
    if (p1) *p1 = q1;
    return DP_OK;
}

// ---- per-tensor pointer tables: the ring of device slots -------------------
// The bindings one launch reads; the per-tensor ones among them get their
// pending upload before the launch and an event behind it.
constexpr int kMaxReads = dpk::kMaxUploads;
struct Reads {
    Binding* b[kMaxReads];
    int n = 0;
    void add(Binding* x) {
        if (n < kMaxReads) b[n++] = x;
    }
    void replicas(dp_plan* p, dp_role role) {
        for (int32_t r = 0; r < p->n; ++r) add(&p->roles[role][r]);
    }
    void state(dp_plan* p) {
        for (int role = DP_ROLE_MASTER; role <= DP_ROLE_EXP_AVG_SQ; ++role)
            for (int bank = 0; bank < 2; ++bank) add(&p->roles[role][bank]);
    }
};

// The plan's shared events (EventPool).
hipError_t ev_take(dp_plan* p, int* out) {
    dpapi::EventPool& pool = p->events;
    if (!pool.free_list.empty()) {
        *out = pool.free_list.back();
        pool.free_list.pop_back();
        return hipSuccess;
    }
    hipEvent_t e = nullptr;
    hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (r != hipSuccess) return r;
    pool.ev.push_back(e);
    pool.refs.push_back(0);
    *out = static_cast<int>(pool.ev.size()) - 1;
    return hipSuccess;
}

void ev_ref(dp_plan* p, int i) { ++p->events.refs[i]; }

void ev_unref(dp_plan* p, int i) {
    if (i < 0) return;
    if (--p->events.refs[i] == 0) p->events.free_list.push_back(i);
}

// Before a launch on `stream`: upload every per-tensor table that a
// rebinding left pending (one kernel for all of them, one event behind it),
// and make the stream wait for uploads issued on other streams.
dp_status stage_tables(dp_plan* p, const Reads& rd, hipStream_t stream) {
    const int32_t T = p->T;
    if (T == 0) return DP_OK;
    dpk::TableUploads up{};
    up.T = T;
    Binding* pend[dpk::kMaxUploads];
    for (int i = 0; i < rd.n; ++i) {
        Binding& b = *rd.b[i];
        if (!b.bound || !b.dev_table) continue;
        const int k = b.slot;
        if (b.pending) {
            bool seen = false;  // a binding listed twice is uploaded once
            for (int j = 0; j < up.count; ++j) seen = seen || pend[j] == &b;
            if (seen) continue;
            up.src[up.count] = b.ring_host_dev + static_cast<size_t>(k) * T;
            up.dst[up.count] = b.dev_table;
            pend[up.count++] = &b;
        } else if (b.upload_stream[k] != stream && b.uploaded[k] >= 0) {
            hipError_t e = hipStreamWaitEvent(stream, p->events.ev[b.uploaded[k]], 0);
            if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent on a pointer table's upload");
        }
    }
    if (up.count == 0) return DP_OK;
    hipError_t e = dpk::launch_upload_tables(up, stream);
    if (e != hipSuccess) return hip_fail(e, "upload of rebound pointer tables");
    int ev = -1;
    e = ev_take(p, &ev);
    if (e == hipSuccess) e = hipEventRecord(p->events.ev[ev], stream);
    if (e != hipSuccess) {
        if (ev >= 0 && p->events.refs[ev] == 0) p->events.free_list.push_back(ev);
        return hip_fail(e, "event behind a pointer table upload");
    }
    for (int j = 0; j < up.count; ++j) {
        Binding& b = *pend[j];
        const int k = b.slot;
        ev_unref(p, b.uploaded[k]);
        b.uploaded[k] = ev;
        ev_ref(p, ev);
        b.upload_stream[k] = stream;
        b.pending = false;
    }
    return DP_OK;
}

// After a launch on `stream` that read at least one per-tensor table: one event
// behind it, held by every per-tensor table slot the launch read.
dp_status note_reads(dp_plan* p, const Reads& rd, hipStream_t stream) {
    int ev = -1;
    hipError_t e = ev_take(p, &ev);
    if (e == hipSuccess) e = hipEventRecord(p->events.ev[ev], stream);
    if (e != hipSuccess) {
        if (ev >= 0 && p->events.refs[ev] == 0) p->events.free_list.push_back(ev);
        return hip_fail(e, "event behind a launch");
    }
    for (int i = 0; i < rd.n; ++i) {
        Binding& b = *rd.b[i];
        if (!b.bound || !b.dev_table) continue;
        auto& uses = b.uses[b.slot];
        bool found = false;
        for (auto& u : uses)
            if (u.first == stream) {
                found = true;
                if (u.second != ev) {
                    ev_unref(p, u.second);
                    u.second = ev;
                    ev_ref(p, ev);
                }
            }
        if (!found) {
            uses.emplace_back(stream, ev);
            ev_ref(p, ev);
        }
    }
    return DP_OK;
}

// The sources of a replica reduction in `mode`, and g_bar.
Reads reduction_reads(dp_plan* p, dpk::ReduceMode mode) {
    Reads rd;
    if (mode != dpk::ReduceMode::kGradients) rd.replicas(p, DP_ROLE_ACC);
    if (mode != dpk::ReduceMode::kAccumulators) rd.replicas(p, DP_ROLE_GRAD);
    rd.add(gbar_binding(p));
    return rd;
}

// Under HIP graph capture the per-tensor tables a launch reads must already
// have been uploaded by an uncaptured call: a captured upload would copy the
// staging slot at every replay, after later rebindings rewrote it, and an
// event recorded during a capture marks nothing on the stream itself.  So a
// captured call whose tables are pending fails, and its reads are not
// tracked (a plan whose calls were captured must not rebind those roles
// while the graph may replay).  The upload is prior work like any other the
// graph reads: the caller orders the replays after it.
dp_status tables_ready_for_capture(const Reads& rd) {
    for (int i = 0; i < rd.n; ++i) {
        const Binding& b = *rd.b[i];
        if (b.bound && b.dev_table && b.pending)
            return fail(DP_ERR_STATE,
                        "a per-tensor pointer table rebound since the last uncaptured call would be uploaded inside a "
                        "graph capture; make one uncaptured call that reads it first");
    }
    return DP_OK;
}

// A launch that reads per-tensor tables: stage them, launch, note the reads.
// A launch that reads no per-tensor table (flat bindings) skips all of it.
template <typename F>
dp_status with_tables(dp_plan* p, const Reads& rd, hipStream_t stream, const char* what, F&& launch) {
    bool tables = false;
    for (int i = 0; i < rd.n && !tables; ++i) tables = rd.b[i]->bound && rd.b[i]->dev_table;
    if (!tables) return check_launch(launch(), what);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    const bool capturing = cs != hipStreamCaptureStatusNone;
    dp_status s = capturing ? tables_ready_for_capture(rd) : stage_tables(p, rd, stream);
    if (s != DP_OK) return s;
    s = check_launch(launch(), what);
    if (s != DP_OK) return s;
    return capturing ? DP_OK : note_reads(p, rd, stream);
}

// Slot k may be written again once its upload and every launch that read it
// have finished (waits only when kRingSlots rebindings are still in flight).
dp_status release_slot(dp_plan* p, Binding& b, int k) {
    hipError_t e = hipSuccess;
    if (b.uploaded[k] >= 0) {
        e = hipEventSynchronize(p->events.ev[b.uploaded[k]]);
        ev_unref(p, b.uploaded[k]);
        b.uploaded[k] = -1;
    }
    for (auto& u : b.uses[k]) {
        if (e == hipSuccess) e = hipEventSynchronize(p->events.ev[u.second]);
        ev_unref(p, u.second);
    }
    b.uses[k].clear();
    b.upload_stream[k] = nullptr;
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize before reusing a pointer table slot");
    return DP_OK;
}

void free_ring(Binding& b) {
    if (b.ring_dev) (void)hipFree(b.ring_dev);
    if (b.ring_host) (void)hipHostFree(b.ring_host);
    b.ring_dev = nullptr;
    b.ring_host = nullptr;
}

}  // namespace

extern "C" {

int dp_abi_version(void) { return DP_ABI_VERSION; }

const char* dp_status_string(dp_status s) {
    switch (s) {
        case DP_OK: return "ok";
        case DP_ERR_INVALID_ARG: return "invalid argument";
        case DP_ERR_BAD_LAYOUT: return "bad layout";
        case DP_ERR_UNBOUND: return "role not bound";
        case DP_ERR_RANGE: return "range out of bounds";
        case DP_ERR_STATE: return "call out of order";
        case DP_ERR_OOM: return "out of memory";
        case DP_ERR_HIP: return "HIP error";
        case DP_ERR_IO: return "file system error";
        case DP_ERR_CORRUPT: return "checkpoint corrupt";
    }
    return "unknown status";
}

const char* dp_last_error(void) { return dpapi::g_last_error.c_str(); }

dp_status dp_plan_create(const dp_layout* L, dp_plan** out) {
    if (!L || !out) return fail(DP_ERR_INVALID_ARG, "dp_plan_create: null argument");
    *out = nullptr;
    if (L->num_tensors < 0) return fail(DP_ERR_BAD_LAYOUT, "num_tensors %d < 0", L->num_tensors);
    if (L->num_tensors > 0 && !L->numel) return fail(DP_ERR_BAD_LAYOUT, "numel is null");
    if (L->n_replicas < 1 || L->n_replicas > DP_MAX_REPLICAS)
        return fail(DP_ERR_BAD_LAYOUT, "n_replicas %d outside [1, %d]", L->n_replicas, DP_MAX_REPLICAS);
    if (L->grad_dtype != DP_F16 && L->grad_dtype != DP_BF16)
        return fail(DP_ERR_BAD_LAYOUT, "grad_dtype must be DP_F16 or DP_BF16");
    if (L->param_dtype != DP_F16 && L->param_dtype != DP_BF16)
        return fail(DP_ERR_BAD_LAYOUT, "param_dtype must be DP_F16 or DP_BF16");
    int32_t chunk = L->chunk_elems == 0 ? DP_DEFAULT_CHUNK : L->chunk_elems;
    if (chunk < dpk::kPiece || chunk > (1 << 26) || (chunk & (chunk - 1)) != 0)
        return fail(DP_ERR_BAD_LAYOUT, "chunk_elems %d must be a power of two in [256, 2^26]", L->chunk_elems);
    dp_plan* p = new (std::nothrow) dp_plan();
    if (!p) return fail(DP_ERR_OOM, "dp_plan_create: host allocation failed");
    p->T = L->num_tensors;
    p->n = L->n_replicas;
    p->gdt = L->grad_dtype;
    p->pdt = L->param_dtype;
    p->chunk = chunk;
    p->numel.assign(L->numel, L->numel + L->num_tensors);
    p->prefix.assign(static_cast<size_t>(p->T) + 1, 0);
    for (int32_t i = 0; i < p->T; ++i) {
        if (p->numel[i] < 0) {
            delete p;
            return fail(DP_ERR_BAD_LAYOUT, "numel[%d] = %lld < 0", i, static_cast<long long>(L->numel[i]));
        }
        if (p->prefix[i] > INT64_MAX / 2 - p->numel[i]) {
            delete p;
            return fail(DP_ERR_BAD_LAYOUT, "total parameter count overflows");
        }
        p->prefix[i + 1] = p->prefix[i] + p->numel[i];
    }
    p->P = p->prefix[p->T];
    p->micro.assign(p->n, 0);
    *out = p;
    return DP_OK;
}

dp_status dp_plan_destroy(dp_plan* p) {
    if (!p) return DP_OK;
    if (p->device >= 0) {
        // free on the plan's device, after its work has drained
        int cur = -1;
        const bool switched = hipGetDevice(&cur) == hipSuccess && cur != p->device &&
                              hipSetDevice(p->device) == hipSuccess;
        (void)hipDeviceSynchronize();
        for (auto& row : p->roles)
            for (auto& b : row) free_ring(b);
        for (hipEvent_t ev : p->events.ev) (void)hipEventDestroy(ev);
        if (p->full.dev) (void)hipFree(p->full.dev);
        if (p->state) (void)hipFree(p->state);
        if (p->stats.sumsq) (void)hipFree(p->stats.sumsq);
        if (p->stats.bad) (void)hipFree(p->stats.bad);
        if (p->fold.sumsq) (void)hipFree(p->fold.sumsq);
        if (p->fold.bad) (void)hipFree(p->fold.bad);
        if (switched) (void)hipSetDevice(cur);
    }
    delete p;
    return DP_OK;
}

dp_status dp_plan_info_get(const dp_plan* p, dp_plan_info* out) {
    if (!p || !out) return fail(DP_ERR_INVALID_ARG, "dp_plan_info_get: null argument");
    std::vector<dp_chunk> tmp;
    build_chunks(p, 0, p->P, &tmp);
    const double P = static_cast<double>(p->P);
    const double sg = static_cast<double>(esize(p->gdt)), sp = static_cast<double>(esize(p->pdt));
    out->params = p->P;
    out->num_chunks = static_cast<int64_t>(tmp.size());
    out->num_tensors = p->T;
    out->n_replicas = p->n;
    out->chunk_elems = p->chunk;
    out->reserved = 0;
    out->state_bytes = 16.0 * P;
    out->bytes_accumulate_first = P * (sg + 4.0);
    out->bytes_accumulate = P * (sg + 8.0);
    out->bytes_reduce_acc = P * (4.0 * p->n + 4.0);
    out->bytes_reduce_partials = P * (sg * p->n + 4.0);
    out->bytes_accumulate_reduce = P * ((sg + 4.0) * p->n + 4.0);
    out->bytes_stats_scan = P * 4.0;
    out->bytes_adam = P * (16.0 + 12.0 + sp);
    out->bytes_reduce_adam = P * ((sg + 4.0) * p->n + 12.0 + 12.0 + sp);
    out->bytes_reduce_adam_partials = P * (sg * p->n + 12.0 + 12.0 + sp);
    return DP_OK;
}

dp_status dp_plan_chunks(const dp_plan* p, int64_t begin, int64_t end, int64_t first, int64_t cap, dp_chunk* out,
                         int64_t* count) {
    if (!p || !count || (cap > 0 && !out) || first < 0 || cap < 0)
        return fail(DP_ERR_INVALID_ARG, "dp_plan_chunks: bad argument");
    if (begin < 0 || end > p->P || begin > end)
        return fail(DP_ERR_RANGE, "range [%lld, %lld) not inside [0, %lld)", static_cast<long long>(begin),
                    static_cast<long long>(end), static_cast<long long>(p->P));
    std::vector<dp_chunk> tmp;
    build_chunks(p, begin, end, &tmp);
    *count = static_cast<int64_t>(tmp.size());
    for (int64_t i = 0; i < cap && first + i < *count; ++i) out[i] = tmp[static_cast<size_t>(first + i)];
    return DP_OK;
}

static dp_status bind_check(dp_plan* p, dp_role role, int32_t replica) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "bind: null plan");
    if (!role_ok(role)) return fail(DP_ERR_INVALID_ARG, "bind: unknown role %d", static_cast<int>(role));
    const int32_t lim = per_replica(role) ? p->n : (banked(role) ? 2 : 1);
    if (replica < 0 || replica >= lim)
        return fail(DP_ERR_INVALID_ARG, "bind: replica %d outside [0, %d) for role %d", replica, lim, static_cast<int>(role));
    return DP_OK;
}

dp_status dp_plan_bind_flat(dp_plan* p, dp_role role, int32_t replica, void* base) {
    dp_status s = bind_check(p, role, replica);
    if (s != DP_OK) return s;
    if (!base && p->P > 0) return fail(DP_ERR_INVALID_ARG, "bind_flat: null base");
    Binding& b = p->roles[role][replica];
    b.flat = base;
    b.tensors.clear();
    b.dev_table = nullptr;  // the ring stays for a later per-tensor binding
    b.pending = false;
    b.bound = true;
    return DP_OK;
}

dp_status dp_plan_bind_tensors(dp_plan* p, dp_role role, int32_t replica, void* const* ptrs) {
    dp_status s = bind_check(p, role, replica);
    if (s != DP_OK) return s;
    if (p->T > 0 && !ptrs) return fail(DP_ERR_INVALID_ARG, "bind_tensors: null pointer array");
    for (int32_t i = 0; i < p->T; ++i)
        if (!ptrs[i] && p->numel[i] > 0) return fail(DP_ERR_INVALID_ARG, "bind_tensors: tensor %d has a null pointer", i);
    s = ensure_device(p);
    if (s != DP_OK) return s;
    Binding& b = p->roles[role][replica];
    const size_t T = static_cast<size_t>(p->T);
    if (T == 0) {
        b.flat = nullptr;
        b.tensors.clear();
        b.dev_table = nullptr;
        b.bound = true;
        return DP_OK;
    }
    // the same pointers as the current table: nothing to do
    if (b.bound && b.dev_table && std::equal(b.tensors.begin(), b.tensors.end(), ptrs)) return DP_OK;
    if (!b.ring_dev) {  // first per-tensor binding of this role: the ring's memory
        hipError_t e = hipMalloc(reinterpret_cast<void**>(&b.ring_dev), sizeof(void*) * T * dpapi::kRingSlots);
        if (e == hipSuccess)
            e = hipHostMalloc(reinterpret_cast<void**>(&b.ring_host), sizeof(void*) * T * dpapi::kRingSlots,
                              hipHostMallocDefault);
        if (e == hipSuccess) e = hipHostGetDevicePointer(reinterpret_cast<void**>(&b.ring_host_dev), b.ring_host, 0);
        if (e != hipSuccess) {
            if (b.ring_dev) (void)hipFree(b.ring_dev);
            if (b.ring_host) (void)hipHostFree(b.ring_host);
            b.ring_dev = nullptr;
            b.ring_host = nullptr;
            b.ring_host_dev = nullptr;
            return fail(DP_ERR_OOM, "allocation of a pointer table ring: %s", hipGetErrorString(e));
        }
    }
    const int k = (b.slot + 1) % dpapi::kRingSlots;
    s = release_slot(p, b, k);
    if (s != DP_OK) return s;
    std::copy(ptrs, ptrs + T, b.ring_host + k * T);
    b.slot = k;
    b.pending = true;
    b.dev_table = b.ring_dev + k * T;
    b.tensors.assign(ptrs, ptrs + T);
    b.flat = nullptr;
    b.bound = true;
    return DP_OK;
}

dp_status dp_plan_prepare_range(dp_plan* p, int64_t begin, int64_t end) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "prepare_range: null plan");
    if (begin < 0 || end > p->P || begin > end)
        return fail(DP_ERR_RANGE, "range [%lld, %lld) not inside [0, %lld)", static_cast<long long>(begin),
                    static_cast<long long>(end), static_cast<long long>(p->P));
    return ensure_full(p);  // a range needs no table of its own
}

// The state block and the statistics scratch, all or nothing: on a failure
// nothing stays allocated and p->state stays null.
static dp_status alloc_device_state(dp_plan* p) {
    // statistics are always written on table pieces of [0, P): one slot per
    // piece, grouped by XCD; the slots no piece maps to stay zero
    const size_t np = static_cast<size_t>(dpk::stats_slots(std::max<int64_t>(p->full.npieces(false), 1)));
    const size_t ng = (np + dpk::kFoldGroup - 1) / dpk::kFoldGroup;
    void* mem[5] = {};
    const size_t bytes[5] = {sizeof(dpk::DevState), np * sizeof(double), np * sizeof(uint32_t), ng * sizeof(double),
                             ng * sizeof(uint64_t)};
    hipError_t e = hipSuccess;
    for (int i = 0; i < 5 && e == hipSuccess; ++i) e = hipMalloc(&mem[i], bytes[i]);
    if (e == hipSuccess) e = hipMemset(mem[1], 0, bytes[1]);
    if (e == hipSuccess) e = hipMemset(mem[2], 0, bytes[2]);
    if (e != hipSuccess) {
        for (void* m : mem)
            if (m) (void)hipFree(m);
        return fail(e == hipErrorOutOfMemory ? DP_ERR_OOM : DP_ERR_HIP,
                    "allocation of the state block and statistics scratch: %s", hipGetErrorString(e));
    }
    p->state = static_cast<dpk::DevState*>(mem[0]);
    p->stats.sumsq = static_cast<double*>(mem[1]);
    p->stats.bad = static_cast<uint32_t*>(mem[2]);
    p->fold.sumsq = static_cast<double*>(mem[3]);
    p->fold.bad = static_cast<uint64_t*>(mem[4]);
    return DP_OK;
}

dp_status dp_plan_drop_ranges(dp_plan* p) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "dp_plan_drop_ranges: null plan");
    return DP_OK;  // ranges hold no state of their own
}

dp_status dp_state_init(dp_plan* p, const dp_state_cfg* cfg, hipStream_t stream) {
    if (!p || !cfg) return fail(DP_ERR_INVALID_ARG, "dp_state_init: null argument");
    if (cfg->scaler_mode < DP_SCALER_NONE || cfg->scaler_mode > DP_SCALER_DYNAMIC)
        return fail(DP_ERR_INVALID_ARG, "unknown scaler_mode %d", cfg->scaler_mode);
    if (!(cfg->beta1 >= 0.0 && cfg->beta1 < 1.0 && cfg->beta2 >= 0.0 && cfg->beta2 < 1.0))
        return fail(DP_ERR_INVALID_ARG, "betas must lie in [0, 1)");
    if (cfg->scaler_mode != DP_SCALER_NONE && !(cfg->init_scale > 0.0))
        return fail(DP_ERR_INVALID_ARG, "init_scale must be > 0");
    if (cfg->scaler_mode == DP_SCALER_DYNAMIC &&
        (!(cfg->backoff > 0.0 && cfg->backoff < 1.0) || !(cfg->growth >= 1.0) || cfg->growth_interval <= 0))
        return fail(DP_ERR_INVALID_ARG, "dynamic scaler needs backoff in (0,1), growth >= 1, growth_interval > 0");
    dp_status s = ensure_device(p);
    if (s != DP_OK) return s;
    s = ensure_full(p);
    if (s != DP_OK) return s;
    if (!p->state) {
        s = alloc_device_state(p);
        if (s != DP_OK) return s;
    }
    const double scale = cfg->scaler_mode == DP_SCALER_NONE ? 1.0 : cfg->init_scale;
    s = check_launch(dpk::launch_state_init(p->state, scale, stream), "state init launch");
    if (s != DP_OK) return s;
    p->cfg = *cfg;
    p->state_ready = true;
    std::fill(p->micro.begin(), p->micro.end(), 0);
    p->partials_valid = false;
    p->stats_current = false;
    p->buckets.clear();
    p->bucket_elems = 0;
    p->bucket_mode = 0;
    return DP_OK;
}

dp_status dp_accumulate(dp_plan* p, int32_t replica, int32_t first, int32_t emit_stats, hipStream_t stream) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "dp_accumulate: null plan");
    {
        dp_status g = no_open_buckets(p, "dp_accumulate");
        if (g != DP_OK) return g;
    }
    if (replica < 0 || replica >= p->n) return fail(DP_ERR_INVALID_ARG, "replica %d outside [0, %d)", replica, p->n);
    if (emit_stats && p->n != 1)
        return fail(DP_ERR_INVALID_ARG, "emit_stats needs n_replicas == 1 (g_bar is then the accumulator)");
    const Binding& g = p->roles[DP_ROLE_GRAD][replica];
    const Binding& a = p->roles[DP_ROLE_ACC][replica];
    dp_status s = need(&g, "GRAD");
    if (s == DP_OK) s = need(&a, "ACC");
    if (s != DP_OK) return s;
    if (emit_stats) {
        const Binding* gb = gbar_binding(p);
        if (gb->flat != a.flat || gb->dev_table != a.dev_table)
            return fail(DP_ERR_STATE, "emit_stats needs GBAR to be ACC[0] (leave GBAR unbound)");
        if (!p->state_ready) return fail(DP_ERR_STATE, "emit_stats before dp_state_init");
    }
    if (!first && p->micro[replica] == 0)
        return fail(DP_ERR_STATE, "replica %d: first == 0 without a first micro-step since the last reduction", replica);
    s = ensure_full(p);
    if (s != DP_OK) return s;
    const dpk::Table t = p->full.table(first && !emit_stats && all_flat({g.ref(), a.ref()}));
    if (t.npieces > 0) {
        Reads rd;
        rd.add(&p->roles[DP_ROLE_GRAD][replica]);
        rd.add(&p->roles[DP_ROLE_ACC][replica]);
        s = with_tables(p, rd, stream, "accumulate launch", [&] {
            return dpk::launch_accumulate(p->gdt, first != 0, emit_stats != 0, t, g.ref(), a.ref(), p->stats, stream);
        });
        if (s != DP_OK) return s;
    }
    p->micro[replica] = first ? 1 : p->micro[replica] + 1;
    p->stats_current = false;
    p->partials_valid = emit_stats != 0;
    p->partials_count = t.npieces;
    return DP_OK;
}

static dp_status bound_replicas(dp_plan* p, dp_role role, dpk::Srcs* out) {
    for (int32_t r = 0; r < p->n; ++r) {
        const Binding& b = p->roles[role][r];
        if (!b.bound)
            return fail(DP_ERR_UNBOUND, "role %s of replica %d is not bound", role == DP_ROLE_ACC ? "ACC" : "GRAD", r);
        out->r[r] = b.ref();
    }
    return DP_OK;
}

static dp_status reduce_common(dp_plan* p, dpk::ReduceMode mode, const dpk::Srcs& accs, const dpk::Srcs& grads,
                               hipStream_t stream) {
    const Binding* gb = gbar_binding(p);
    if (!gb->bound) return fail(DP_ERR_UNBOUND, "role GBAR is not bound");
    dp_status s = ensure_full(p);
    if (s != DP_OK) return s;
    const dpk::Table t = p->full.table(false);  // statistics: table pieces
    if (t.npieces > 0) {
        s = with_tables(p, reduction_reads(p, mode), stream, "reduce launch", [&] {
            return dpk::launch_reduce(mode, p->gdt, p->n, t, dpk::PieceSpan{0, t.npieces}, accs, grads, gb->ref(),
                                      p->stats, stream);
        });
        if (s != DP_OK) return s;
    }
    std::fill(p->micro.begin(), p->micro.end(), 0);
    p->partials_valid = true;
    p->partials_count = t.npieces;
    p->stats_current = false;
    return DP_OK;
}

dp_status dp_reduce_replicas(dp_plan* p, dp_role src, hipStream_t stream) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "dp_reduce_replicas: null plan");
    {
        dp_status g = no_open_buckets(p, "dp_reduce_replicas");
        if (g != DP_OK) return g;
    }
    if (src != DP_ROLE_ACC && src != DP_ROLE_GRAD)
        return fail(DP_ERR_INVALID_ARG, "src must be DP_ROLE_ACC or DP_ROLE_GRAD");
    if (!p->state_ready) return fail(DP_ERR_STATE, "dp_reduce_replicas before dp_state_init");
    dpk::Srcs accs{}, grads{};
    dp_status s = bound_replicas(p, src, src == DP_ROLE_ACC ? &accs : &grads);
    if (s != DP_OK) return s;
    if (src == DP_ROLE_ACC) {
        for (int32_t r = 0; r < p->n; ++r)
            if (p->micro[r] != p->micro[0] || p->micro[r] == 0)
                return fail(DP_ERR_STATE, "replicas accumulated different numbers of micro-steps (replica %d: %d, replica 0: %d)",
                            r, p->micro[r], p->micro[0]);
    }
    return reduce_common(p, src == DP_ROLE_ACC ? dpk::ReduceMode::kAccumulators : dpk::ReduceMode::kGradients, accs,
                         grads, stream);
}

dp_status dp_accumulate_all(dp_plan* p, int32_t first, hipStream_t stream) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "dp_accumulate_all: null plan");
    {
        dp_status g = no_open_buckets(p, "dp_accumulate_all");
        if (g != DP_OK) return g;
    }
    dpk::Srcs grads{}, accs{};
    dp_status s = bound_replicas(p, DP_ROLE_GRAD, &grads);
    if (s == DP_OK) s = bound_replicas(p, DP_ROLE_ACC, &accs);
    if (s != DP_OK) return s;
    s = same_micro_step(p, first != 0);
    if (s != DP_OK) return s;
    s = ensure_full(p);
    if (s != DP_OK) return s;
    // Addressing (flat pieces or chunk-table pieces, see kernels.hip), as
    // measured on MI355X: micro-steps after the first (read-modify-write of
    // the accumulators) always go through the chunk table -- the table load
    // each wave does before its first access staggers the waves' start and
    // moves 7-8% more bytes per second on this pass -- while the write-mostly
    // first micro-step is 15% faster on flat pieces.  Every kernel that
    // writes statistics uses table pieces, so the summation order of the
    // statistics does not depend on how the roles are bound.
    const dpk::Table t = p->full.table(first && all_flat(grads, p->n) && all_flat(accs, p->n));
    if (t.npieces > 0) {
        Reads rd;
        rd.replicas(p, DP_ROLE_GRAD);
        rd.replicas(p, DP_ROLE_ACC);
        s = with_tables(p, rd, stream, "accumulate launch", [&] {
            return dpk::launch_accumulate_all(p->gdt, first != 0, p->n, t, dpk::PieceSpan{0, t.npieces}, grads, accs,
                                              stream);
        });
        if (s != DP_OK) return s;
    }
    for (int32_t r = 0; r < p->n; ++r) p->micro[r] = first ? 1 : p->micro[r] + 1;
    p->stats_current = false;
    p->partials_valid = false;
    return DP_OK;
}

dp_status dp_accumulate_all_range(dp_plan* p, int32_t first, int64_t begin, int64_t end, hipStream_t stream) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "dp_accumulate_all_range: null plan");
    dp_status s = no_open_buckets(p, "dp_accumulate_all_range", 3);
    if (s != DP_OK) return s;
    if (p->bucket_mode == 3 && !p->buckets.empty() && (first != 0) != (p->bucket_first != 0))
        return fail(DP_ERR_INVALID_ARG, "the buckets of one micro-step take the same first flag (%d here, %d before)",
                    first != 0, p->bucket_first != 0);
    dpk::Srcs grads{}, accs{};
    s = bound_replicas(p, DP_ROLE_GRAD, &grads);
    if (s == DP_OK) s = bound_replicas(p, DP_ROLE_ACC, &accs);
    if (s != DP_OK) return s;
    s = same_micro_step(p, first != 0);
    if (s != DP_OK) return s;
    int64_t p0 = 0, p1 = 0;
    s = bucket_span(p, begin, end, &p0, &p1);
    if (s != DP_OK) return s;
    // The addressing of dp_accumulate_all: flat pieces of [begin, end) for a
    // first micro-step on flat bindings, else the bucket's span of table
    // pieces.  The adds are elementwise, so the pieces a bucket is cut into
    // never change the bits.
    if (p1 > p0) {
        const bool flat = first && all_flat(grads, p->n) && all_flat(accs, p->n);
        DeviceTable bucket;
        bucket.begin = begin;
        bucket.end = end;
        bucket.log2s = p->full.log2s;
        const dpk::Table t = flat ? bucket.table(true) : p->full.table(false);
        const dpk::PieceSpan sp = flat ? dpk::PieceSpan{0, t.npieces} : dpk::PieceSpan{p0, p1};
        Reads rd;
        rd.replicas(p, DP_ROLE_GRAD);
        rd.replicas(p, DP_ROLE_ACC);
        s = with_tables(p, rd, stream, "accumulate launch", [&] {
            return dpk::launch_accumulate_all(p->gdt, first != 0, p->n, t, sp, grads, accs, stream);
        });
        if (s != DP_OK) return s;
    }
    if (end > begin) {
        if (p->buckets.empty()) p->bucket_first = first != 0;
        p->buckets.emplace_back(begin, end);
        p->bucket_elems += end - begin;
        p->bucket_mode = 3;
    }
    p->stats_current = false;
    p->partials_valid = false;
    if (p->bucket_elems == p->P) {  // the buckets cover [0, P): the micro-step is complete
        p->buckets.clear();
        p->bucket_elems = 0;
        p->bucket_mode = 0;
        for (int32_t r = 0; r < p->n; ++r) p->micro[r] = first ? 1 : p->micro[r] + 1;
    }
    return DP_OK;
}

// One bucket of a bucketed reduction from the given sources; every bucket of
// one reduction takes the same kind (src: 0 the last micro-step fused, else
// the role reduced alone).
static dp_status reduction_bucket(dp_plan* p, int src, int64_t begin, int64_t end, hipStream_t stream,
                                  const char* where) {
    if (!p->state_ready) return fail(DP_ERR_STATE, "%s before dp_state_init", where);
    dp_status s = no_open_buckets(p, where, 1);
    if (s != DP_OK) return s;
    if (p->bucket_mode == 1 && !p->buckets.empty() && p->bucket_src != src)
        return fail(DP_ERR_INVALID_ARG, "%s: the buckets of one reduction take the same sources", where);
    int64_t p0 = 0, p1 = 0;
    s = bucket_span(p, begin, end, &p0, &p1);
    if (s != DP_OK) return s;
    const Binding* gb = gbar_binding(p);
    if (!gb->bound) return fail(DP_ERR_UNBOUND, "role GBAR is not bound");
    dpk::Srcs grads{}, accs{};
    dpk::ReduceMode mode = dpk::ReduceMode::kGradients;
    if (src == DP_ROLE_ACC) {
        s = bound_replicas(p, DP_ROLE_ACC, &accs);
        if (s != DP_OK) return s;
        for (int32_t r = 0; r < p->n; ++r)
            if (p->micro[r] != p->micro[0] || p->micro[r] == 0)
                return fail(DP_ERR_STATE,
                            "replicas accumulated different numbers of micro-steps (replica %d: %d, replica 0: %d)", r,
                            p->micro[r], p->micro[0]);
        mode = dpk::ReduceMode::kAccumulators;
    } else {
        s = bound_replicas(p, DP_ROLE_GRAD, &grads);
        if (s != DP_OK) return s;
        if (src == 0) {
            s = same_micro_step(p, true);
            if (s != DP_OK) return s;
            if (p->micro[0] > 0) {
                s = bound_replicas(p, DP_ROLE_ACC, &accs);
                if (s != DP_OK) return s;
                mode = dpk::ReduceMode::kAccPlusGrad;
            }
        }
    }
    const dpk::Table t = p->full.table(false);  // statistics: table pieces, the slots of the whole reduction
    if (p1 > p0) {
        s = with_tables(p, reduction_reads(p, mode), stream, "reduce launch", [&] {
            return dpk::launch_reduce(mode, p->gdt, p->n, t, dpk::PieceSpan{p0, p1}, accs, grads, gb->ref(), p->stats,
                                      stream);
        });
        if (s != DP_OK) return s;
    }
    if (end > begin) {
        if (p->buckets.empty()) p->bucket_src = src;
        p->buckets.emplace_back(begin, end);
        p->bucket_elems += end - begin;
        p->bucket_mode = 1;
    }
    p->partials_valid = false;
    p->stats_current = false;
    if (p->bucket_elems == p->P) {  // the buckets cover [0, P): the reduction is complete
        p->buckets.clear();
        p->bucket_elems = 0;
        p->bucket_mode = 0;
        std::fill(p->micro.begin(), p->micro.end(), 0);
        p->partials_valid = true;
        p->partials_count = t.npieces;
    }
    return DP_OK;
}

dp_status dp_accumulate_reduce_range(dp_plan* p, int64_t begin, int64_t end, hipStream_t stream) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "dp_accumulate_reduce_range: null plan");
    return reduction_bucket(p, 0, begin, end, stream, "dp_accumulate_reduce_range");
}

dp_status dp_reduce_replicas_range(dp_plan* p, dp_role src, int64_t begin, int64_t end, hipStream_t stream) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "dp_reduce_replicas_range: null plan");
    if (src != DP_ROLE_ACC && src != DP_ROLE_GRAD)
        return fail(DP_ERR_INVALID_ARG, "src must be DP_ROLE_ACC or DP_ROLE_GRAD");
    return reduction_bucket(p, src, begin, end, stream, "dp_reduce_replicas_range");
}

dp_status dp_accumulate_reduce(dp_plan* p, hipStream_t stream) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "dp_accumulate_reduce: null plan");
    {
        dp_status g = no_open_buckets(p, "dp_accumulate_reduce");
        if (g != DP_OK) return g;
    }
    if (!p->state_ready) return fail(DP_ERR_STATE, "dp_accumulate_reduce before dp_state_init");
    dpk::Srcs grads{}, accs{};
    dp_status s = bound_replicas(p, DP_ROLE_GRAD, &grads);
    if (s != DP_OK) return s;
    for (int32_t r = 0; r < p->n; ++r)
        if (p->micro[r] != p->micro[0])
            return fail(DP_ERR_STATE, "replicas are at different micro-steps (replica %d: %d, replica 0: %d)", r,
                        p->micro[r], p->micro[0]);
    const bool with_acc = p->micro[0] > 0;
    if (with_acc) {
        s = bound_replicas(p, DP_ROLE_ACC, &accs);
        if (s != DP_OK) return s;
    }
    return reduce_common(p, with_acc ? dpk::ReduceMode::kAccPlusGrad : dpk::ReduceMode::kGradients, accs, grads,
                         stream);
}

dp_status dp_grad_stats(dp_plan* p, int32_t scan, double max_norm, hipStream_t stream) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "dp_grad_stats: null plan");
    {
        dp_status g = no_open_buckets(p, "dp_grad_stats");
        if (g != DP_OK) return g;
    }
    if (!p->state_ready) return fail(DP_ERR_STATE, "dp_grad_stats before dp_state_init");
    if (!(max_norm >= 0.0)) return fail(DP_ERR_INVALID_ARG, "max_norm must be >= 0 (0 disables clipping)");
    dp_status s = ensure_full(p);
    if (s != DP_OK) return s;
    if (scan) {
        const Binding* gb = gbar_binding(p);
        s = need(gb, "GBAR");
        if (s != DP_OK) return s;
        const dpk::Table t = p->full.table(false);  // statistics: table pieces
        if (t.npieces > 0) {
            Reads rd;
            rd.add(gbar_binding(p));
            s = with_tables(p, rd, stream, "stats launch",
                            [&] { return dpk::launch_stats(t, gb->ref(), p->stats, stream); });
            if (s != DP_OK) return s;
        }
        p->partials_count = t.npieces;
    } else if (!p->partials_valid && p->full.count > 0) {
        return fail(DP_ERR_STATE, "no fused statistics for the current g_bar: reduce first, or pass scan = 1");
    }
    dpk::ScalerArgs a{p->cfg.beta1, p->cfg.beta2, p->cfg.backoff, p->cfg.growth, max_norm,
                      p->cfg.scaler_mode, p->cfg.growth_interval, 0};
    const int64_t nparts = p->full.count > 0 ? p->partials_count : 0;
    s = check_launch(dpk::launch_finalize(p->stats, nparts, p->fold, p->state, a, stream), "finalize launch");
    if (s != DP_OK) return s;
    p->partials_valid = false;
    p->stats_current = true;
    std::fill(p->micro.begin(), p->micro.end(), 0);
    return DP_OK;
}

dp_status dp_adam_step(dp_plan* p, const dp_adam_hparams* hp, int64_t begin, int64_t end, hipStream_t stream) {
    if (!p || !hp) return fail(DP_ERR_INVALID_ARG, "dp_adam_step: null argument");
    if (begin < 0 || end > p->P || begin > end)
        return fail(DP_ERR_RANGE, "shard [%lld, %lld) not inside [0, %lld)", static_cast<long long>(begin),
                    static_cast<long long>(end), static_cast<long long>(p->P));
    if (!(hp->lr >= 0.0) || !(hp->eps > 0.0) || !(hp->weight_decay >= 0.0))
        return fail(DP_ERR_INVALID_ARG, "need lr >= 0, eps > 0, weight_decay >= 0");
    if (!p->stats_current) return fail(DP_ERR_STATE, "dp_adam_step before dp_grad_stats on the current g_bar");
    const Binding* gb = gbar_binding(p);
    dp_status s = need(gb, "GBAR");
    if (s == DP_OK) s = need(&p->roles[DP_ROLE_MASTER][0], "MASTER");
    if (s == DP_OK) s = need(&p->roles[DP_ROLE_EXP_AVG][0], "EXP_AVG");
    if (s == DP_OK) s = need(&p->roles[DP_ROLE_EXP_AVG_SQ][0], "EXP_AVG_SQ");
    if (s == DP_OK) s = need(&p->roles[DP_ROLE_PARAM][0], "PARAM");
    if (s != DP_OK) return s;
    if (begin == end) return DP_OK;
    s = ensure_full(p);
    if (s != DP_OK) return s;
    dpk::AdamArgs a{hp->lr, hp->eps, hp->weight_decay, p->cfg.beta1, p->cfg.beta2};
    const dpk::StateRefs sr = state_refs(p);
    const dpk::RoleRef pr = p->roles[DP_ROLE_PARAM][0].ref();
    const bool flat = all_flat(sr) && all_flat({gb->ref(), pr});
    // No table of the range's own: flat pieces of [begin, end), or the pieces
    // of the [0, P) table that overlap it, each clipped to it in the kernel
    dpk::Table t;
    dpk::PieceSpan sp;
    if (flat) {
        DeviceTable r;
        r.begin = begin;
        r.end = end;
        r.log2s = p->full.log2s;
        t = r.table(true);
        sp = dpk::PieceSpan{0, t.npieces};
    } else {
        t = p->full.table(false);
        t.begin = begin;
        t.end = end;
        sp = dpk::PieceSpan{piece_holding(p, begin), piece_holding(p, end - 1) + 1};
    }
    Reads rd;
    rd.add(gbar_binding(p));
    rd.state(p);
    rd.add(&p->roles[DP_ROLE_PARAM][0]);
    return with_tables(p, rd, stream, "adamw launch", [&] {
        return dpk::launch_adamw(p->pdt, t, sp, gb->ref(), sr, pr, p->state, a, stream);
    });
}

// The single pass's sources (every replica's last micro-step, plus its
// accumulator after earlier micro-steps) and the state it reads and writes
// (both banks and the parameters), checked before any launch.
static dp_status single_pass_sources(dp_plan* p, dpk::Srcs* grads, dpk::Srcs* accs, bool* with_acc) {
    dp_status s = bound_replicas(p, DP_ROLE_GRAD, grads);
    if (s != DP_OK) return s;
    for (int32_t r = 0; r < p->n; ++r)
        if (p->micro[r] != p->micro[0])
            return fail(DP_ERR_STATE, "replicas are at different micro-steps (replica %d: %d, replica 0: %d)", r,
                        p->micro[r], p->micro[0]);
    *with_acc = p->micro[0] > 0;
    if (*with_acc) {
        s = bound_replicas(p, DP_ROLE_ACC, accs);
        if (s != DP_OK) return s;
    }
    static const char* const names[] = {"MASTER", "EXP_AVG", "EXP_AVG_SQ"};
    for (int role = DP_ROLE_MASTER; role <= DP_ROLE_EXP_AVG_SQ; ++role)
        for (int b = 0; b < 2; ++b)
            if (!p->roles[role][b].bound)
                return fail(DP_ERR_UNBOUND, "role %s bank %d is not bound (the single pass writes the other bank)",
                            names[role - DP_ROLE_MASTER], b);
    return need(&p->roles[DP_ROLE_PARAM][0], "PARAM");
}

static bool valid_hparams(const dp_adam_hparams* hp) {
    return hp->lr >= 0.0 && hp->eps > 0.0 && hp->weight_decay >= 0.0;
}

// The single pass over pieces [p0, p1) of the [0, P) table.
static dp_status single_pass_launch(dp_plan* p, const dp_adam_hparams* hp, bool with_acc, const dpk::Srcs& grads,
                                    const dpk::Srcs& accs, int64_t p0, int64_t p1, hipStream_t stream) {
    if (p1 <= p0) return DP_OK;
    const dpk::AdamArgs a{hp->lr, hp->eps, hp->weight_decay, p->cfg.beta1, p->cfg.beta2};
    Reads rd;
    rd.replicas(p, DP_ROLE_GRAD);
    if (with_acc) rd.replicas(p, DP_ROLE_ACC);
    rd.state(p);
    rd.add(&p->roles[DP_ROLE_PARAM][0]);
    return with_tables(p, rd, stream, "reduce + adamw launch", [&] {
        return dpk::launch_reduce_adamw(with_acc ? dpk::ReduceMode::kAccPlusGrad : dpk::ReduceMode::kGradients, p->gdt,
                                        p->pdt, p->n, p->full.table(false), dpk::PieceSpan{p0, p1}, accs, grads,
                                        state_refs(p), p->roles[DP_ROLE_PARAM][0].ref(), p->stats, p->state, a,
                                        stream);
    });
}

// The end of a single pass: the statistics fold and the commit of the step
// (the written bank becomes current if it is applied), then the parameters
// emitted again from the current bank if it was skipped.
static dp_status single_pass_commit(dp_plan* p, hipStream_t stream) {
    const dpk::StateRefs sr = state_refs(p);
    const dpk::RoleRef pr = p->roles[DP_ROLE_PARAM][0].ref();
    const dpk::ScalerArgs sc{p->cfg.beta1, p->cfg.beta2, p->cfg.backoff, p->cfg.growth, 0.0,
                             p->cfg.scaler_mode, p->cfg.growth_interval, 1};
    dp_status s = check_launch(dpk::launch_finalize(p->stats, p->full.npieces(false), p->fold, p->state, sc, stream),
                               "finalize launch");
    if (s != DP_OK) return s;
    Reads rd;
    rd.state(p);
    rd.add(&p->roles[DP_ROLE_PARAM][0]);
    s = with_tables(p, rd, stream, "parameter restore launch", [&] {
        return dpk::launch_restore_param(p->pdt, p->full.table(all_flat(sr) && all_flat({pr})), sr, pr, p->state,
                                         stream);
    });
    if (s != DP_OK) return s;
    std::fill(p->micro.begin(), p->micro.end(), 0);
    p->partials_valid = false;
    p->stats_current = false;
    return DP_OK;
}

dp_status dp_reduce_adam_step(dp_plan* p, const dp_adam_hparams* hp, hipStream_t stream) {
    if (!p || !hp) return fail(DP_ERR_INVALID_ARG, "dp_reduce_adam_step: null argument");
    {
        dp_status g = no_open_buckets(p, "dp_reduce_adam_step");
        if (g != DP_OK) return g;
    }
    if (!valid_hparams(hp)) return fail(DP_ERR_INVALID_ARG, "need lr >= 0, eps > 0, weight_decay >= 0");
    if (!p->state_ready) return fail(DP_ERR_STATE, "dp_reduce_adam_step before dp_state_init");
    dpk::Srcs grads{}, accs{};
    bool with_acc = false;
    dp_status s = single_pass_sources(p, &grads, &accs, &with_acc);
    if (s != DP_OK) return s;
    s = ensure_full(p);
    if (s != DP_OK) return s;
    s = single_pass_launch(p, hp, with_acc, grads, accs, 0, p->full.npieces(false), stream);
    if (s != DP_OK) return s;
    return single_pass_commit(p, stream);
}

dp_status dp_reduce_adam_range(dp_plan* p, const dp_adam_hparams* hp, int64_t begin, int64_t end,
                               hipStream_t stream) {
    if (!p || !hp) return fail(DP_ERR_INVALID_ARG, "dp_reduce_adam_range: null argument");
    if (!valid_hparams(hp)) return fail(DP_ERR_INVALID_ARG, "need lr >= 0, eps > 0, weight_decay >= 0");
    if (!p->state_ready) return fail(DP_ERR_STATE, "dp_reduce_adam_range before dp_state_init");
    {
        dp_status g = no_open_buckets(p, "dp_reduce_adam_range", 2);
        if (g != DP_OK) return g;
    }
    if (p->bucket_mode == 2 && !p->buckets.empty()) {
        const dp_adam_hparams& h = p->bucket_hp;
        if (h.lr != hp->lr || h.eps != hp->eps || h.weight_decay != hp->weight_decay)
            return fail(DP_ERR_INVALID_ARG, "the buckets of one step take the same lr, eps and weight_decay");
    }
    int64_t p0 = 0, p1 = 0;
    dp_status s = bucket_span(p, begin, end, &p0, &p1);
    if (s != DP_OK) return s;
    dpk::Srcs grads{}, accs{};
    bool with_acc = false;
    s = single_pass_sources(p, &grads, &accs, &with_acc);
    if (s != DP_OK) return s;
    s = single_pass_launch(p, hp, with_acc, grads, accs, p0, p1, stream);
    if (s != DP_OK) return s;
    if (end > begin) {
        if (p->buckets.empty()) p->bucket_hp = *hp;
        p->buckets.emplace_back(begin, end);
        p->bucket_elems += end - begin;
        p->bucket_mode = 2;
    }
    p->partials_valid = false;
    p->stats_current = false;
    return DP_OK;
}

dp_status dp_reduce_adam_finish(dp_plan* p, hipStream_t stream) {
    if (!p) return fail(DP_ERR_INVALID_ARG, "dp_reduce_adam_finish: null plan");
    if (!p->state_ready) return fail(DP_ERR_STATE, "dp_reduce_adam_finish before dp_state_init");
    {
        dp_status g = no_open_buckets(p, "dp_reduce_adam_finish", 2);
        if (g != DP_OK) return g;
    }
    if (p->bucket_elems != p->P)
        return fail(DP_ERR_STATE, "dp_reduce_adam_finish: the buckets cover %lld of %lld elements",
                    static_cast<long long>(p->bucket_elems), static_cast<long long>(p->P));
    static const char* const names[] = {"MASTER", "EXP_AVG", "EXP_AVG_SQ"};
    for (int role = DP_ROLE_MASTER; role <= DP_ROLE_EXP_AVG_SQ; ++role)
        for (int b = 0; b < 2; ++b)
            if (!p->roles[role][b].bound)
                return fail(DP_ERR_UNBOUND, "role %s bank %d is not bound", names[role - DP_ROLE_MASTER], b);
    dp_status s = need(&p->roles[DP_ROLE_PARAM][0], "PARAM");
    if (s == DP_OK) s = ensure_full(p);
    if (s != DP_OK) return s;
    s = single_pass_commit(p, stream);
    if (s != DP_OK) return s;
    p->buckets.clear();
    p->bucket_elems = 0;
    p->bucket_mode = 0;
    return DP_OK;
}

dp_status dp_read_state(dp_plan* p, dp_step_state* out, hipStream_t stream) {
    if (!p || !out) return fail(DP_ERR_INVALID_ARG, "dp_read_state: null argument");
    if (!p->state) return fail(DP_ERR_STATE, "dp_read_state before dp_state_init");
    dp_status s = ensure_device(p);
    if (s != DP_OK) return s;
    hipError_t e = hipMemcpyAsync(out, p->state, sizeof(dp_step_state), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync of the state block");
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    return DP_OK;
}

}  // extern "C"
