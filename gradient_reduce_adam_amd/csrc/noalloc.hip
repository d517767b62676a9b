// dp_reduce_adam_step_noalloc: the single pass of dp_reduce_adam_step over one
// flat tensor, for callers that cannot allocate device memory.  Everything the
// kernels need beyond the caller's inputs and outputs -- the per-piece
// statistics slots, the fold's second level and the chunk table -- lives in
// one static device array, `scratch`, that each GPU holds from the library's
// load until the process ends.  Its size fixes the largest call:
// DP_STATIC_MAX_PARAMS elements.
//
// In host code `scratch` names a host-side stand-in, not device memory.  The
// device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device (with that device current) on the first call there, and only that
// address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dp_internal.h"
#include "dpstep.h"
#include "plan.h"

using dpapi::fail;
using dpapi::hip_fail;

namespace {

constexpr int kLog2Chunk = 14;  // DP_DEFAULT_CHUNK elements per chunk
static_assert((1 << kLog2Chunk) == DP_DEFAULT_CHUNK, "chunk size");
constexpr int kLog2PiecesPerChunk = kLog2Chunk - 8;  // 256-element pieces
static_assert((1 << 8) == dpk::kPiece, "piece size");

constexpr int64_t kMaxChunks = DP_STATIC_MAX_PARAMS >> kLog2Chunk;
constexpr int64_t kMaxPieces = kMaxChunks << kLog2PiecesPerChunk;
constexpr int64_t kMaxSlots = 8 * ((kMaxPieces + 7) / 8);
constexpr int64_t kMaxGroups = (kMaxSlots + dpk::kFoldGroup - 1) / dpk::kFoldGroup;

// Layout of the array: statistics slots (binary64 sums, then counts), the
// fold's group sums and counts, the chunk table.
constexpr size_t kOffSumsq = 0;
constexpr size_t kOffBad = kOffSumsq + kMaxSlots * sizeof(double);
constexpr size_t kOffFoldSumsq = kOffBad + kMaxSlots * sizeof(uint32_t);
constexpr size_t kOffFoldBad = kOffFoldSumsq + kMaxGroups * sizeof(double);
constexpr size_t kOffChunks = kOffFoldBad + kMaxGroups * sizeof(uint64_t);
constexpr size_t kScratchBytes = kOffChunks + kMaxChunks * sizeof(dp_chunk);
static_assert(kOffBad % 256 == 0 && kOffFoldSumsq % 256 == 0 && kOffFoldBad % 256 == 0 && kOffChunks % 256 == 0,
              "every part of the scratch starts 256-byte aligned");
static_assert(kScratchBytes == DP_STATIC_SCRATCH_BYTES, "the header states the scratch size");

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The device address of the current device's copy of `scratch`.
dp_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DP_ERR_INVALID_ARG, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the static scratch");
        if (!ptr) return fail(DP_ERR_HIP, "hipGetSymbolAddress gave a null address for the static scratch");
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return DP_OK;
}

dp_status launched(hipError_t e, const char* what) { return e == hipSuccess ? DP_OK : hip_fail(e, what); }

}  // namespace

extern "C" dp_status dp_reduce_adam_step_noalloc(int64_t P, int32_t n, dp_dtype grad_dtype, dp_dtype param_dtype,
                                                 void* const* grads, void* const* accs, void* const* master,
                                                 void* const* exp_avg, void* const* exp_avg_sq, void* param,
                                                 dp_step_state* state, const dp_state_cfg* cfg,
                                                 const dp_adam_hparams* hp, hipStream_t stream) {
    if (!cfg || !hp || !state) return fail(DP_ERR_INVALID_ARG, "dp_reduce_adam_step_noalloc: null argument");
    if (P < 0) return fail(DP_ERR_INVALID_ARG, "P = %lld < 0", static_cast<long long>(P));
    if (P > DP_STATIC_MAX_PARAMS)
        return fail(DP_ERR_INVALID_ARG,
                    "P = %lld exceeds DP_STATIC_MAX_PARAMS = %lld, the size of the static scratch; use "
                    "dp_reduce_adam_step on a plan",
                    static_cast<long long>(P), static_cast<long long>(DP_STATIC_MAX_PARAMS));
    if (n < 1 || n > DP_MAX_REPLICAS) return fail(DP_ERR_INVALID_ARG, "n = %d outside [1, %d]", n, DP_MAX_REPLICAS);
    if ((grad_dtype != DP_F16 && grad_dtype != DP_BF16) || (param_dtype != DP_F16 && param_dtype != DP_BF16))
        return fail(DP_ERR_INVALID_ARG, "grad_dtype and param_dtype must be DP_F16 or DP_BF16");
    if (cfg->scaler_mode < DP_SCALER_NONE || cfg->scaler_mode > DP_SCALER_DYNAMIC)
        return fail(DP_ERR_INVALID_ARG, "unknown scaler_mode %d", cfg->scaler_mode);
    if (!(cfg->beta1 >= 0.0 && cfg->beta1 < 1.0 && cfg->beta2 >= 0.0 && cfg->beta2 < 1.0))
        return fail(DP_ERR_INVALID_ARG, "betas must lie in [0, 1)");
    if (cfg->scaler_mode == DP_SCALER_DYNAMIC &&
        (!(cfg->backoff > 0.0 && cfg->backoff < 1.0) || !(cfg->growth >= 1.0) || cfg->growth_interval <= 0))
        return fail(DP_ERR_INVALID_ARG, "dynamic scaler needs backoff in (0,1), growth >= 1, growth_interval > 0");
    if (!(hp->lr >= 0.0) || !(hp->eps > 0.0) || !(hp->weight_decay >= 0.0))
        return fail(DP_ERR_INVALID_ARG, "need lr >= 0, eps > 0, weight_decay >= 0");
    if ((reinterpret_cast<uintptr_t>(state) & 7) != 0)
        return fail(DP_ERR_INVALID_ARG, "state must be 8-byte aligned");
    if (P > 0) {
        if (!grads || !master || !exp_avg || !exp_avg_sq || !param)
            return fail(DP_ERR_INVALID_ARG, "dp_reduce_adam_step_noalloc: null pointer array or param");
        for (int32_t r = 0; r < n; ++r)
            if (!grads[r] || (accs && !accs[r]))
                return fail(DP_ERR_INVALID_ARG, "replica %d: null gradient or accumulator pointer", r);
        for (int b = 0; b < 2; ++b)
            if (!master[b] || !exp_avg[b] || !exp_avg_sq[b])
                return fail(DP_ERR_INVALID_ARG, "bank %d: null master, exp_avg or exp_avg_sq pointer", b);
    }
    void* base = nullptr;
    dp_status s = scratch_address(&base);
    if (s != DP_OK) return s;
    unsigned char* mem = static_cast<unsigned char*>(base);
    const dpk::StatsBuf sb{reinterpret_cast<double*>(mem + kOffSumsq), reinterpret_cast<uint32_t*>(mem + kOffBad)};
    const dpk::FoldBuf fold{reinterpret_cast<double*>(mem + kOffFoldSumsq),
                            reinterpret_cast<uint64_t*>(mem + kOffFoldBad)};
    dp_chunk* chunks = reinterpret_cast<dp_chunk*>(mem + kOffChunks);

    // The [0, P) table of a one-tensor plan with the default chunk size, as
    // dp_reduce_adam_step reads it: the same pieces, slots and fold order.
    const int64_t nchunks = (P + DP_DEFAULT_CHUNK - 1) >> kLog2Chunk;
    const int64_t npieces = nchunks << kLog2PiecesPerChunk;
    const dpk::Table table{chunks, 0, P, npieces, kLog2PiecesPerChunk, false};
    const dpk::Table flat{nullptr, 0, P, (P + dpk::kPiece - 1) / dpk::kPiece, kLog2PiecesPerChunk, true};

    dpk::Srcs g{}, a{};
    dpk::StateRefs sr{};
    if (P > 0) {
        for (int32_t r = 0; r < n; ++r) {
            g.r[r] = dpk::RoleRef{grads[r], nullptr};
            if (accs) a.r[r] = dpk::RoleRef{accs[r], nullptr};
        }
        for (int b = 0; b < 2; ++b) {
            sr.w[b] = dpk::RoleRef{master[b], nullptr};
            sr.m[b] = dpk::RoleRef{exp_avg[b], nullptr};
            sr.v[b] = dpk::RoleRef{exp_avg_sq[b], nullptr};
        }
    }
    const dpk::RoleRef pr{param, nullptr};
    dpk::DevState* st = reinterpret_cast<dpk::DevState*>(state);
    const dpk::AdamArgs args{hp->lr, hp->eps, hp->weight_decay, cfg->beta1, cfg->beta2};
    const dpk::ScalerArgs sc{cfg->beta1, cfg->beta2, cfg->backoff, cfg->growth, 0.0,
                             cfg->scaler_mode, cfg->growth_interval, 1};

    s = launched(dpk::launch_flat_table(chunks, P, kLog2Chunk, sb, npieces, stream), "chunk table launch");
    if (s != DP_OK) return s;
    if (npieces > 0) {
        s = launched(dpk::launch_reduce_adamw(accs ? dpk::ReduceMode::kAccPlusGrad : dpk::ReduceMode::kGradients,
                                              grad_dtype, param_dtype, n, table, dpk::PieceSpan{0, npieces}, a, g, sr,
                                              pr, sb, st, args, stream),
                     "reduce + adamw launch");
        if (s != DP_OK) return s;
    }
    s = launched(dpk::launch_finalize(sb, npieces, fold, st, sc, stream), "finalize launch");
    if (s != DP_OK) return s;
    return launched(dpk::launch_restore_param(param_dtype, flat, sr, pr, st, stream), "parameter restore launch");
}
