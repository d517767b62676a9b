// gfx950 kernels of the data-parallel gradient reduce + AdamW step.
//
// Work decomposition.  Every streaming kernel runs one wave64 workgroup per
// 256-element piece.  A lane moves 4 consecutive elements, so each binary32
// stream is one 16-byte access per lane and one contiguous KiB per wave, and a
// 16-bit stream one 8-byte access per lane.  Pieces are found in one of two
// ways:
//  - flat (every role of the call bound as one flat buffer): piece p covers
//    flat elements [lo, lo + 256) with lo = floor4(begin) + 256 p, clipped to
//    [begin, end); no table is read, so the first memory access of a wave
//    depends on nothing but its indices;
//  - table: the plan's chunk table splits the range into chunks of at most
//    chunk_elems elements inside one tensor, and piece p is piece (p & (S-1))
//    of chunk (p >> log2 S), S = chunk_elems / 256.  Needed when a role is
//    bound per tensor; also used for every kernel that writes statistics (so
//    their summation order does not depend on the bindings) and for the
//    read-modify-write accumulation (see api.cpp for the measurements).
// Thousands of one-shot single-wave workgroups keep the addresses in flight
// dense and spread over all HBM channels; measured on MI355X this beats
// larger workgroups and persistent grid-stride loops by 10-25% on these
// read-modify-write streams.  A piece whose pointers are not aligned, and the
// ragged end of a chunk, take a per-element path.
//
// Reductions are fixed-order trees: a wave64 butterfly per piece writes one
// binary64 partial, folded later in a fixed order, so results are bitwise
// reproducible run to run.  No floating-point atomics are used.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dp_internal.h"

namespace dpk {
namespace {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Memory access through the global address space (global_load / global_store
// rather than flat_*: the pointers come from tables, so the compiler cannot
// infer the address space itself).  _nt variants set the nontemporal hint for
// data streamed once.
#define DP_GLOBAL __attribute__((address_space(1)))

template <typename V>
__device__ __forceinline__ V ldg(const void* p, int64_t i) { return ((const DP_GLOBAL V*)p)[i]; }
template <typename V>
__device__ __forceinline__ void stg(void* p, int64_t i, V x) { ((DP_GLOBAL V*)p)[i] = x; }
template <typename V>
__device__ __forceinline__ V ldg_nt(const void* p, int64_t i) {
    return __builtin_nontemporal_load(((const DP_GLOBAL V*)p) + i);
}
template <typename V>
__device__ __forceinline__ void stg_nt(void* p, int64_t i, V x) {
    __builtin_nontemporal_store(x, ((DP_GLOBAL V*)p) + i);
}

__device__ __forceinline__ bool aligned(const void* p, uintptr_t bytes) {
    return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0;
}

// ---- the piece a workgroup owns ----------------------------------------------
// Element i of the piece (0 <= i < kPiece) is at offset i from the piece's
// pointers; elements [vlo, vhi) belong to the call's range.
struct Piece {
    int32_t tensor;  // table mode: tensor of the chunk
    int64_t flat;    // flat index of element 0
    int64_t offset;  // table mode: index of element 0 inside its tensor
    int vlo, vhi;
};

template <bool kFlat>
__device__ __forceinline__ Piece piece_of(const Table& t, int64_t p) {
    Piece q;
    if constexpr (kFlat) {
        const int64_t lo = (t.begin & ~int64_t{3}) + p * kPiece;
        q.tensor = 0;
        q.flat = lo;
        q.offset = 0;
        q.vlo = t.begin > lo ? static_cast<int>(t.begin - lo) : 0;
        const int64_t rest = t.end - lo;
        q.vhi = rest < kPiece ? static_cast<int>(rest) : kPiece;
    } else {
        const dp_chunk c = t.chunks[p >> t.log2s];
        const int start = static_cast<int>(p & ((int64_t{1} << t.log2s) - 1)) * kPiece;
        q.tensor = c.tensor;
        q.flat = c.flat + start;
        q.offset = c.offset + start;
        q.vlo = 0;
        const int rest = c.len - start;
        q.vhi = rest < 0 ? 0 : (rest < kPiece ? rest : kPiece);
    }
    return q;
}

// Piece p of the [0, P) chunk table with its elements clipped to the call's
// range [t.begin, t.end): an update over a shard runs on the pieces of the
// whole table that overlap the shard, so a shard needs no table of its own.
// Over [0, P) the clip changes nothing.
__device__ __forceinline__ Piece piece_of_clipped(const Table& t, int64_t p) {
    Piece q = piece_of<false>(t, p);
    const int64_t lo = t.begin - q.flat, hi = t.end - q.flat;
    if (lo > q.vlo) q.vlo = lo < kPiece ? static_cast<int>(lo) : kPiece;
    if (hi < q.vhi) q.vhi = hi > 0 ? static_cast<int>(hi) : 0;
    return q;
}

template <typename T>
__device__ __forceinline__ T* elem_ptr(const RoleRef& r, const Piece& q) {
    if (r.tab) return static_cast<T*>(r.tab[q.tensor]) + q.offset;
    return static_cast<T*>(r.base) + q.flat;
}

// The 4 elements of this lane: all in range (vector path) or the in-range
// subset [lo, hi) of [e0, e0 + 4) (per-element path).
struct LaneSpan {
    int e0, lo, hi;
    bool full;
};

__device__ __forceinline__ LaneSpan lane_span(const Piece& q) {
    LaneSpan l;
    l.e0 = static_cast<int>(threadIdx.x) * 4;
    l.lo = l.e0 > q.vlo ? l.e0 : q.vlo;
    l.hi = l.e0 + 4 < q.vhi ? l.e0 + 4 : q.vhi;
    l.full = l.e0 >= q.vlo && l.e0 + 4 <= q.vhi;
    return l;
}

// ---- low-precision formats --------------------------------------------------
// kind: 1 = binary16, 2 = bfloat16 (dp_dtype values)
template <int kind>
__device__ __forceinline__ float widen1(uint16_t b) {
    if constexpr (kind == 2) return __uint_as_float(static_cast<uint32_t>(b) << 16);
    else return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

template <int kind>
__device__ __forceinline__ f32x4 widen4(u32x2 q) {
    if constexpr (kind == 2) {
        return f32x4{__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xFFFF0000u), __uint_as_float(q.y << 16),
                     __uint_as_float(q.y & 0xFFFF0000u)};
    } else {
        return __builtin_convertvector(__builtin_bit_cast(f16x4, q), f32x4);
    }
}

// binary32 -> low precision, round to nearest even (hardware conversion).
template <int kind>
__device__ __forceinline__ uint16_t narrow1(float x) {
    if constexpr (kind == 2) return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
    else return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

__device__ __forceinline__ uint32_t nonfinite(float x) {
    return (__float_as_uint(x) & 0x7F800000u) == 0x7F800000u ? 1u : 0u;
}

__device__ __forceinline__ void add_stats(float y, double& ss, uint32_t& bad) {
    ss += static_cast<double>(y) * static_cast<double>(y);
    bad += nonfinite(y);
}

// Fixed-order wave64 butterfly of (sumsq, bad); lane 0 writes the partial of
// piece p (of npieces) to its XCD-grouped slot.
__device__ __forceinline__ void wave_stats_store(double ss, uint32_t bad, int64_t p, int64_t npieces, StatsBuf sb) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        ss += __shfl_xor(ss, off, 64);
        bad += __shfl_xor(bad, off, 64);
    }
    if (threadIdx.x == 0) {
        const int64_t slot = (p & 7) * ((npieces + 7) >> 3) + (p >> 3);
        sb.sumsq[slot] = ss;
        sb.bad[slot] = bad;
    }
}

// ---- fixed-order replica tree ---------------------------------------------
// Level-wise pairwise sum: (0+1), (2+3), ...; an odd last term is carried to
// the next level unchanged.  Every partial sum is a binary32 add.
template <int Cnt>
struct TreeLevel {
    template <int N>
    __device__ __forceinline__ static void run(float (&b)[N]) {
#pragma unroll
        for (int j = 0; j < Cnt / 2; ++j) b[j] = b[2 * j] + b[2 * j + 1];
        if constexpr (Cnt & 1) b[Cnt / 2] = b[Cnt - 1];
        constexpr int next = Cnt / 2 + (Cnt & 1);
        if constexpr (next > 1) TreeLevel<next>::run(b);
    }
};

template <int N>
__device__ __forceinline__ float tree_sum(float (&b)[N]) {
    if constexpr (N > 1) TreeLevel<N>::run(b);
    return b[0];
}

// Division by n, rounded once to binary32: for n a power of two the binary32
// reciprocal is exact and so is the product; otherwise one binary64 division
// (binary64 then binary32 is correctly rounded: 53 >= 2 * 24 + 2).
template <int N>
__device__ __forceinline__ float average(float s) {
    if constexpr ((N & (N - 1)) == 0) return s * (1.0f / static_cast<float>(N));
    else return static_cast<float>(static_cast<double>(s) / static_cast<double>(N));
}

// ============================================================================
// micro-step accumulation: acc = g (first) or acc + g
// ============================================================================
template <int kGrad, bool kFirst, bool kStats>
__device__ __forceinline__ void accumulate_piece(const Piece& q, RoleRef grad, RoleRef acc, double& ss,
                                                 uint32_t& bad) {
    const uint16_t* __restrict__ g = elem_ptr<const uint16_t>(grad, q);
    float* __restrict__ a = elem_ptr<float>(acc, q);
    const LaneSpan l = lane_span(q);
    if (l.full && aligned(g, 8) && aligned(a, 16)) {
        const int lane = threadIdx.x;
        f32x4 r = widen4<kGrad>(ldg_nt<u32x2>(g, lane));
        // the first micro-step only writes acc: a nontemporal store, as for
        // every write-only stream (on table pieces a plain one streamed 20%
        // slower on MI355X); the read-modify-write keeps the plain store
        if constexpr (kFirst) {
            stg_nt<f32x4>(a, lane, r);
        } else {
            r = ldg<f32x4>(a, lane) + r;
            stg<f32x4>(a, lane, r);
        }
        if constexpr (kStats) {
#pragma unroll
            for (int e = 0; e < 4; ++e) add_stats(r[e], ss, bad);
        }
    } else {
        for (int i = l.lo; i < l.hi; ++i) {
            const float gi = widen1<kGrad>(ldg<uint16_t>(g, i));
            const float r = kFirst ? gi : ldg<float>(a, i) + gi;
            stg<float>(a, i, r);
            if constexpr (kStats) add_stats(r, ss, bad);
        }
    }
}

// one replica; with kStats the piece statistics of the result (n = 1: it is g_bar)
template <bool kFlat, int kGrad, bool kFirst, bool kStats>
__global__ void __launch_bounds__(kWave) k_accumulate(Table t, int64_t base, RoleRef grad, RoleRef acc, StatsBuf sb) {
    const int64_t p = base + blockIdx.x;
    const Piece q = piece_of<kFlat>(t, p);
    double ss = 0.0;
    uint32_t bad = 0;
    accumulate_piece<kGrad, kFirst, kStats>(q, grad, acc, ss, bad);
    if constexpr (kStats) wave_stats_store(ss, bad, p, t.npieces, sb);
}

// every replica's micro-step in one launch: blockIdx.y is the replica (the
// dispatcher walks x fastest, so each replica's buffers stream in order)
template <bool kFlat, int kGrad, bool kFirst>
__global__ void __launch_bounds__(kWave) k_accumulate_all(Table t, int64_t base, Srcs grads, Srcs accs) {
    const Piece q = piece_of<kFlat>(t, base + blockIdx.x);
    double ss = 0.0;
    uint32_t bad = 0;
    accumulate_piece<kGrad, kFirst, false>(q, grads.r[blockIdx.y], accs.r[blockIdx.y], ss, bad);
}

// ============================================================================
// replica reduction: gbar = tree(x_0..x_{N-1}) / N, plus piece statistics
//   kMode 0: x_r = acc_r                 (binary32 accumulators)
//   kMode 1: x_r = g_r                   (low-precision gradients or partials)
//   kMode 2: x_r = acc_r + g_r           (the last micro-step fused: acc_r is
//                                         not written back)
// ============================================================================
template <int kMode, int kGrad, int N>
struct ReduceSrc {
    const float* ap[N];
    const uint16_t* gp[N];
    bool ok;  // every source pointer of the piece allows the vector path

    __device__ __forceinline__ ReduceSrc(const Piece& q, const Srcs& accs, const Srcs& grads) {
        ok = true;
#pragma unroll
        for (int r = 0; r < N; ++r) {
            if constexpr (kMode != 1) {
                ap[r] = elem_ptr<const float>(accs.r[r], q);
                ok = ok && aligned(ap[r], 16);
            }
            if constexpr (kMode != 0) {
                gp[r] = elem_ptr<const uint16_t>(grads.r[r], q);
                ok = ok && aligned(gp[r], 8);
            }
        }
    }

    // the average of this lane's 4 elements (vector path)
    __device__ __forceinline__ f32x4 vec(int lane) const {
        float x[4][N];
#pragma unroll
        for (int r = 0; r < N; ++r) {
            f32x4 t;
            if constexpr (kMode == 0) t = ldg_nt<f32x4>(ap[r], lane);
            else if constexpr (kMode == 1) t = widen4<kGrad>(ldg_nt<u32x2>(gp[r], lane));
            else t = ldg_nt<f32x4>(ap[r], lane) + widen4<kGrad>(ldg_nt<u32x2>(gp[r], lane));
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e][r] = t[e];
        }
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = average<N>(tree_sum<N>(x[e]));
        return y;
    }

    // the average of element i (per-element path)
    __device__ __forceinline__ float elem(int i) const {
        float x[N];
#pragma unroll
        for (int r = 0; r < N; ++r) {
            if constexpr (kMode == 0) x[r] = ldg<float>(ap[r], i);
            else if constexpr (kMode == 1) x[r] = widen1<kGrad>(ldg<uint16_t>(gp[r], i));
            else x[r] = ldg<float>(ap[r], i) + widen1<kGrad>(ldg<uint16_t>(gp[r], i));
        }
        return average<N>(tree_sum<N>(x));
    }
};

template <bool kFlat, int kMode, int kGrad, int N>
__global__ void __launch_bounds__(kWave) k_reduce(Table t, int64_t base, Srcs accs, Srcs grads, RoleRef gbar,
                                                    StatsBuf sb) {
    const int64_t p = base + blockIdx.x;
    const Piece q = piece_of<kFlat>(t, p);
    const ReduceSrc<kMode, kGrad, N> src(q, accs, grads);
    float* __restrict__ out = elem_ptr<float>(gbar, q);
    const LaneSpan l = lane_span(q);
    double ss = 0.0;
    uint32_t bad = 0;
    if (l.full && src.ok && aligned(out, 16)) {
        const f32x4 y = src.vec(threadIdx.x);
#pragma unroll
        for (int e = 0; e < 4; ++e) add_stats(y[e], ss, bad);
        stg_nt<f32x4>(out, threadIdx.x, y);
    } else {
        for (int i = l.lo; i < l.hi; ++i) {
            const float y = src.elem(i);
            stg<float>(out, i, y);
            add_stats(y, ss, bad);
        }
    }
    wave_stats_store(ss, bad, p, t.npieces, sb);
}

// ============================================================================
// statistics scan of gbar (when not fused into the producer)
// ============================================================================
template <bool kFlat>
__global__ void __launch_bounds__(kWave) k_stats(Table t, int64_t base, RoleRef gbar, StatsBuf sb) {
    const int64_t p = base + blockIdx.x;
    const Piece q = piece_of<kFlat>(t, p);
    const float* __restrict__ x = elem_ptr<const float>(gbar, q);
    const LaneSpan l = lane_span(q);
    double ss = 0.0;
    uint32_t bad = 0;
    if (l.full && aligned(x, 16)) {
        const f32x4 v = ldg_nt<f32x4>(x, threadIdx.x);
#pragma unroll
        for (int e = 0; e < 4; ++e) add_stats(v[e], ss, bad);
    } else {
        for (int i = l.lo; i < l.hi; ++i) add_stats(ldg<float>(x, i), ss, bad);
    }
    wave_stats_store(ss, bad, p, t.npieces, sb);
}

// ============================================================================
// pass 2: the statistics slots are folded in slot order -- by groups of
// kFoldGroup when there are many -- and one workgroup updates the scalar state
// ============================================================================
// The fixed order: thread t adds slots lo + t, lo + t + 256, ... in turn;
// then s[t] += s[t + w] for w = 128, 64, ..., 1.  The slots were written from
// every XCD and miss this one's L2, so a thread issues a batch of loads before
// it adds them (same order), and the levels below the wave size run as wave-0
// butterflies: lane t < w then adds s[t] + s[t + w] exactly as the tree does,
// and lane 0 ends with the tree's sum, bit for bit.  Result in thread 0.
constexpr int kFoldBatch = 16;  // loads in flight per thread (kFoldGroup / kFoldThreads)
static_assert(kFoldThreads == 4 * kWave, "the fold has four waves");

template <typename Count>
__device__ __forceinline__ void block_fold(const double* __restrict__ ss_in, const Count* __restrict__ bad_in,
                                           int64_t lo, int64_t hi, double& ss_out, uint64_t& bad_out) {
    __shared__ double s_ss[kFoldThreads];
    __shared__ uint64_t s_bad[kFoldThreads];
    const int tid = threadIdx.x;
    double ss = 0.0;
    uint64_t bad = 0;
    for (int64_t base = lo + tid; base < hi; base += int64_t{kFoldBatch} * kFoldThreads) {
        double v[kFoldBatch];
        uint64_t c[kFoldBatch];
#pragma unroll
        for (int j = 0; j < kFoldBatch; ++j) {
            const int64_t i = base + int64_t{j} * kFoldThreads;
            v[j] = i < hi ? ss_in[i] : 0.0;
            c[j] = i < hi ? static_cast<uint64_t>(bad_in[i]) : 0;
        }
#pragma unroll
        for (int j = 0; j < kFoldBatch; ++j) {
            if (base + int64_t{j} * kFoldThreads < hi) {
                ss += v[j];
                bad += c[j];
            }
        }
    }
    s_ss[tid] = ss;
    s_bad[tid] = bad;
    __syncthreads();
#pragma unroll
    for (int w = kFoldThreads / 2; w >= kWave; w >>= 1) {
        if (tid < w) {
            s_ss[tid] = s_ss[tid] + s_ss[tid + w];
            s_bad[tid] = s_bad[tid] + s_bad[tid + w];
        }
        __syncthreads();
    }
    if (tid < kWave) {
        ss = s_ss[tid];
        bad = s_bad[tid];
#pragma unroll
        for (int w = kWave / 2; w > 0; w >>= 1) {
            // lane t < w: s[t] + s[t + w]; the other lanes only mirror it
            const double o = __shfl_xor(ss, w, kWave);
            const uint64_t ob = __shfl_xor(bad, w, kWave);
            ss = (tid & w) ? o + ss : ss + o;
            bad += ob;
        }
    }
    ss_out = ss;
    bad_out = bad;
}

__global__ void __launch_bounds__(kFoldThreads) k_fold(StatsBuf sb, int64_t nslots, FoldBuf fold) {
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * kFoldGroup;
    const int64_t hi = lo + kFoldGroup < nslots ? lo + kFoldGroup : nslots;
    double ss;
    uint64_t bad;
    block_fold(sb.sumsq, sb.bad, lo, hi, ss, bad);
    if (threadIdx.x == 0) {
        fold.sumsq[blockIdx.x] = ss;
        fold.bad[blockIdx.x] = bad;
    }
}

template <typename Count>
__global__ void __launch_bounds__(kFoldThreads) k_finalize(const double* __restrict__ ss_in,
                                                             const Count* __restrict__ bad_in, int64_t nslots,
                                                             DevState* __restrict__ st, ScalerArgs args) {
    double sumsq;
    uint64_t badsum;
    block_fold(ss_in, bad_in, 0, nslots, sumsq, badsum);
    if (threadIdx.x != 0) return;
    DevState s = *st;
    s.sumsq = sumsq;
    s.found_inf = badsum != 0 ? 1 : 0;
    s.norm = sqrt(sumsq) / s.scale;
    if (s.found_inf) {
        s.clip = 1.0;
        s.gscale = 0.0;
        if (args.mode == DP_SCALER_DYNAMIC) {
            s.scale *= args.backoff;
            s.growth_tracker = 0;
        }
    } else {
        s.clip = (args.max_norm > 0.0 && s.norm > args.max_norm) ? args.max_norm / s.norm : 1.0;
        s.gscale = s.clip / s.scale;
        s.t += 1;
        s.beta1_pow *= args.beta1;
        s.beta2_pow *= args.beta2;
        if (args.flip_bank) s.bank ^= 1;
        if (args.mode == DP_SCALER_DYNAMIC) {
            s.growth_tracker += 1;
            if (s.growth_tracker == args.growth_interval) {
                s.scale *= args.growth;
                s.growth_tracker = 0;
            }
        }
    }
    s.iter += 1;
    *st = s;
}

__global__ void k_state_init(DevState* __restrict__ st, double scale) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    DevState s;
    s.t = 0;
    s.iter = 0;
    s.growth_tracker = 0;
    s.beta1_pow = 1.0;
    s.beta2_pow = 1.0;
    s.scale = scale;
    s.found_inf = 0;
    s.bank = 0;
    s.sumsq = 0.0;
    s.norm = 0.0;
    s.clip = 1.0;
    s.gscale = 0.0;
    *st = s;
}

// ============================================================================
// fused AdamW: one read of gbar, w, m, v and one write of w, m, v, p per
// element; binary64 arithmetic, binary32 storage
// ============================================================================
struct AdamCoef {
    double gscale, b1, omb1, b2, omb2, step, sqrt_bc2, eps, dec;
};

// The coefficients of the update with gradient factor gscale and bias
// corrections 1 - b1p, 1 - b2p (b1p = beta1^t, b2p = beta2^t of the step).
__device__ __forceinline__ AdamCoef adam_coef(double gscale, double b1p, double b2p, const AdamArgs& args) {
#pragma clang fp contract(off)
    AdamCoef k;
    k.gscale = gscale;
    k.b1 = args.beta1;
    k.omb1 = 1.0 - args.beta1;
    k.b2 = args.beta2;
    k.omb2 = 1.0 - args.beta2;
    k.step = args.lr / (1.0 - b1p);
    k.sqrt_bc2 = sqrt(1.0 - b2p);
    k.eps = args.eps;
    k.dec = 1.0 - args.lr * args.weight_decay;
    return k;
}

// One element of the update.  Every operation is a separately rounded IEEE
// binary64 operation in the order written (no contraction into fused
// multiply-adds), so the result depends on the inputs only, not on the
// instruction selection.
__device__ __forceinline__ void adam1(float gb, float& w, float& m, float& v, const AdamCoef& k) {
#pragma clang fp contract(off)
    const double g = static_cast<double>(gb) * k.gscale;
    const double mi = k.b1 * static_cast<double>(m) + k.omb1 * g;
    const double vi = k.b2 * static_cast<double>(v) + k.omb2 * (g * g);
    const double denom = sqrt(vi) / k.sqrt_bc2 + k.eps;
    const double wi = static_cast<double>(w) * k.dec - k.step * (mi / denom);
    m = static_cast<float>(mi);
    v = static_cast<float>(vi);
    w = static_cast<float>(wi);
}

template <int kParam>
__device__ __forceinline__ u32x2 narrow4(const float (&w)[4]) {
    return u32x2{static_cast<uint32_t>(narrow1<kParam>(w[0])) | (static_cast<uint32_t>(narrow1<kParam>(w[1])) << 16),
                 static_cast<uint32_t>(narrow1<kParam>(w[2])) | (static_cast<uint32_t>(narrow1<kParam>(w[3])) << 16)};
}

// The state of one piece: read from bank rd, written to bank wr (the same
// bank for the in-place update).
struct StatePtrs {
    const float* w_in;
    const float* m_in;
    const float* v_in;
    float* w_out;
    float* m_out;
    float* v_out;
    uint16_t* p;
    bool ok;  // the vector path is allowed

    __device__ __forceinline__ StatePtrs(const StateRefs& s, RoleRef pr, int rd, int wr, const Piece& q) {
        w_in = elem_ptr<const float>(s.w[rd], q);
        m_in = elem_ptr<const float>(s.m[rd], q);
        v_in = elem_ptr<const float>(s.v[rd], q);
        w_out = elem_ptr<float>(s.w[wr], q);
        m_out = elem_ptr<float>(s.m[wr], q);
        v_out = elem_ptr<float>(s.v[wr], q);
        p = elem_ptr<uint16_t>(pr, q);
        ok = aligned(w_in, 16) && aligned(m_in, 16) && aligned(v_in, 16) && aligned(w_out, 16) &&
             aligned(m_out, 16) && aligned(v_out, 16) && aligned(p, 8);
    }

    // this lane's 4 elements with gradient G (vector path)
    template <int kParam>
    __device__ __forceinline__ void update4(f32x4 G, int lane, const AdamCoef& k) const {
        const f32x4 W = ldg_nt<f32x4>(w_in, lane);
        const f32x4 M = ldg_nt<f32x4>(m_in, lane);
        const f32x4 V = ldg_nt<f32x4>(v_in, lane);
        float w4[4] = {W[0], W[1], W[2], W[3]};
        float m4[4] = {M[0], M[1], M[2], M[3]};
        float v4[4] = {V[0], V[1], V[2], V[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) adam1(G[e], w4[e], m4[e], v4[e], k);
        stg_nt<f32x4>(w_out, lane, f32x4{w4[0], w4[1], w4[2], w4[3]});
        stg_nt<f32x4>(m_out, lane, f32x4{m4[0], m4[1], m4[2], m4[3]});
        stg_nt<f32x4>(v_out, lane, f32x4{v4[0], v4[1], v4[2], v4[3]});
        stg_nt<u32x2>(p, lane, narrow4<kParam>(w4));
    }

    // element i with gradient g (per-element path)
    template <int kParam>
    __device__ __forceinline__ void update1(float g, int i, const AdamCoef& k) const {
        float w = ldg<float>(w_in, i), m = ldg<float>(m_in, i), v = ldg<float>(v_in, i);
        adam1(g, w, m, v, k);
        stg<float>(w_out, i, w);
        stg<float>(m_out, i, m);
        stg<float>(v_out, i, v);
        stg<uint16_t>(p, i, narrow1<kParam>(w));
    }
};

// two-pass update, in place on the current bank, with the finalised scalars
template <bool kFlat, int kParam>
__global__ void __launch_bounds__(kWave) k_adamw(Table t, int64_t base, RoleRef gbar, StateRefs sr, RoleRef pr,
                                                   const DevState* __restrict__ st, AdamArgs args) {
    if (st->found_inf) return;
    const AdamCoef k = adam_coef(st->gscale, st->beta1_pow, st->beta2_pow, args);
    const int bank = st->bank;
    const Piece q = kFlat ? piece_of<true>(t, base + blockIdx.x) : piece_of_clipped(t, base + blockIdx.x);
    const float* __restrict__ gp = elem_ptr<const float>(gbar, q);
    const StatePtrs sp(sr, pr, bank, bank, q);
    const LaneSpan l = lane_span(q);
    if (l.full && sp.ok && aligned(gp, 16)) {
        sp.update4<kParam>(ldg_nt<f32x4>(gp, threadIdx.x), threadIdx.x, k);
    } else {
        for (int i = l.lo; i < l.hi; ++i) sp.update1<kParam>(ldg<float>(gp, i), i, k);
    }
}

// ============================================================================
// single pass: replica average, statistics and the update of every element
// in one read of the sources and the state.  Without clipping the update of
// a step depends on the statistics only through the skip decision, so it is
// computed with the scalars the step has if applied (gscale = 1 / scale, t + 1)
// into the other bank; the finalisation makes that bank current only when the
// step is applied.  Table pieces, as k_reduce, so the statistics are the same.
// ============================================================================
template <int kMode, int kGrad, int N, int kParam>
__global__ void __launch_bounds__(kWave) k_reduce_adamw(Table t, int64_t base, Srcs accs, Srcs grads, StateRefs sr,
                                                          RoleRef pr, StatsBuf sb, const DevState* __restrict__ st,
                                                          AdamArgs args) {
    AdamCoef k;
    {
#pragma clang fp contract(off)
        k = adam_coef(1.0 / st->scale, st->beta1_pow * args.beta1, st->beta2_pow * args.beta2, args);
    }
    const int bank = st->bank;
    const int64_t p = base + blockIdx.x;
    const Piece q = piece_of<false>(t, p);
    const ReduceSrc<kMode, kGrad, N> src(q, accs, grads);
    const StatePtrs sp(sr, pr, bank, bank ^ 1, q);
    const LaneSpan l = lane_span(q);
    double ss = 0.0;
    uint32_t bad = 0;
    if (l.full && src.ok && sp.ok) {
        const f32x4 y = src.vec(threadIdx.x);
#pragma unroll
        for (int e = 0; e < 4; ++e) add_stats(y[e], ss, bad);
        sp.update4<kParam>(y, threadIdx.x, k);
    } else {
        for (int i = l.lo; i < l.hi; ++i) {
            const float y = src.elem(i);
            add_stats(y, ss, bad);
            sp.update1<kParam>(y, i, k);
        }
    }
    wave_stats_store(ss, bad, p, t.npieces, sb);
}

// After a skipped single-pass step the parameters hold the discarded update:
// emit them again from the current bank's master.  A grid-stride loop over the
// pieces, so the launch costs a few microseconds when there is nothing to do.
constexpr unsigned kRestoreBlocks = 4096;

template <bool kFlat, int kParam>
__global__ void __launch_bounds__(kWave) k_restore_param(Table t, StateRefs sr, RoleRef pr,
                                                           const DevState* __restrict__ st) {
    if (!st->found_inf) return;
    const int bank = st->bank;
    for (int64_t pc = blockIdx.x; pc < t.npieces; pc += gridDim.x) {
        const Piece q = piece_of<kFlat>(t, pc);
        const float* __restrict__ w = elem_ptr<const float>(sr.w[bank], q);
        uint16_t* __restrict__ pp = elem_ptr<uint16_t>(pr, q);
        const LaneSpan l = lane_span(q);
        if (l.full && aligned(w, 16) && aligned(pp, 8)) {
            const f32x4 W = ldg<f32x4>(w, threadIdx.x);
            const float w4[4] = {W[0], W[1], W[2], W[3]};
            stg<u32x2>(pp, threadIdx.x, narrow4<kParam>(w4));
        } else {
            for (int i = l.lo; i < l.hi; ++i) stg<uint16_t>(pp, i, narrow1<kParam>(ldg<float>(w, i)));
        }
    }
}

// The chunk table of one tensor of P elements, [0, P) in chunks of 2^log2c
// elements, written into caller-provided device memory; and zeros in the
// statistics slots that no piece of that table maps to.  Those slots are the
// ones of pieces [npieces, 8 ceil(npieces / 8)): a fold adds them, and memory
// that an earlier call with another size used may hold other values there.
__global__ void __launch_bounds__(256) k_flat_table(dp_chunk* __restrict__ chunks, int64_t P, int log2c,
                                                      int64_t nchunks, StatsBuf sb, int64_t npieces) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < nchunks) {
        const int64_t flat = i << log2c;
        const int64_t rest = P - flat;
        const int64_t c = int64_t{1} << log2c;
        chunks[i] = dp_chunk{flat, flat, 0, static_cast<int32_t>(rest < c ? rest : c)};
    }
    const int64_t per = (npieces + 7) >> 3;
    const int64_t p = npieces + i;
    if (p < 8 * per) {
        const int64_t slot = (p & 7) * per + (p >> 3);
        sb.sumsq[slot] = 0.0;
        sb.bad[slot] = 0;
    }
}

// Workgroup b copies table b of the list: T pointers from pinned host memory
// into its device table.
__global__ void __launch_bounds__(256) k_upload_tables(TableUploads u) {
    const void* const* __restrict__ src = u.src[blockIdx.x];
    void** __restrict__ dst = u.dst[blockIdx.x];
    for (int32_t i = static_cast<int32_t>(threadIdx.x); i < u.T; i += 256) dst[i] = const_cast<void*>(src[i]);
}

// ---- launch helpers ---------------------------------------------------------
// Launches `launch(base, grid)` over pieces [p0, p1), one workgroup each, in
// slices of at most kMaxBlocksPerLaunch (gridDim.y = ny); base is the piece
// of the slice's first workgroup.
template <typename F>
hipError_t for_span(int64_t p0, int64_t p1, unsigned ny, F&& launch) {
    for (int64_t b = p0; b < p1; b += kMaxBlocksPerLaunch) {
        const int64_t cnt = p1 - b < kMaxBlocksPerLaunch ? p1 - b : kMaxBlocksPerLaunch;
        launch(b, dim3(static_cast<unsigned>(cnt), ny));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename F>
hipError_t for_pieces(int64_t npieces, unsigned ny, F&& launch) {
    return for_span(0, npieces, ny, static_cast<F&&>(launch));
}

template <bool kFlat, int kMode, int kGrad, int N>
hipError_t reduce_n(const Table& t, PieceSpan sp, const Srcs& accs, const Srcs& grads, RoleRef gbar, StatsBuf sb,
                    hipStream_t s) {
    return for_span(sp.p0, sp.p1, 1, [&](int64_t b, dim3 grid) {
        hipLaunchKernelGGL((k_reduce<kFlat, kMode, kGrad, N>), grid, dim3(kWave), 0, s, t, b, accs, grads, gbar, sb);
    });
}

template <bool kFlat, int kMode, int kGrad>
hipError_t reduce_dispatch(int n, const Table& t, PieceSpan sp, const Srcs& accs, const Srcs& grads, RoleRef gbar,
                           StatsBuf sb, hipStream_t s) {
    switch (n) {
#define DP_CASE(K) \
    case K: return reduce_n<kFlat, kMode, kGrad, K>(t, sp, accs, grads, gbar, sb, s);
        DP_CASE(1) DP_CASE(2) DP_CASE(3) DP_CASE(4) DP_CASE(5) DP_CASE(6) DP_CASE(7) DP_CASE(8)
        DP_CASE(9) DP_CASE(10) DP_CASE(11) DP_CASE(12) DP_CASE(13) DP_CASE(14) DP_CASE(15) DP_CASE(16)
#undef DP_CASE
        default: return hipErrorInvalidValue;
    }
}

template <bool kFlat>
hipError_t reduce_modes(ReduceMode mode, dp_dtype gdt, int n, const Table& t, PieceSpan sp, const Srcs& accs,
                        const Srcs& grads, RoleRef gbar, StatsBuf sb, hipStream_t s) {
    if (mode == ReduceMode::kAccumulators) return reduce_dispatch<kFlat, 0, 2>(n, t, sp, accs, grads, gbar, sb, s);
    if (mode == ReduceMode::kGradients) {
        if (gdt == DP_F16) return reduce_dispatch<kFlat, 1, 1>(n, t, sp, accs, grads, gbar, sb, s);
        return reduce_dispatch<kFlat, 1, 2>(n, t, sp, accs, grads, gbar, sb, s);
    }
    if (gdt == DP_F16) return reduce_dispatch<kFlat, 2, 1>(n, t, sp, accs, grads, gbar, sb, s);
    return reduce_dispatch<kFlat, 2, 2>(n, t, sp, accs, grads, gbar, sb, s);
}

template <bool kFlat>
hipError_t accumulate_t(dp_dtype gdt, bool first, bool stats, const Table& t, RoleRef grad, RoleRef acc, StatsBuf sb,
                        hipStream_t s) {
    return for_pieces(t.npieces, 1, [&](int64_t b, dim3 grid) {
        const dim3 blk(kWave);
#define DP_ACC(G, F, S) hipLaunchKernelGGL((k_accumulate<kFlat, G, F, S>), grid, blk, 0, s, t, b, grad, acc, sb)
        if constexpr (kFlat) {
            if (gdt == DP_BF16) DP_ACC(2, true, false); else DP_ACC(1, true, false);
        } else if (gdt == DP_BF16) {
            if (first) { if (stats) DP_ACC(2, true, true); else DP_ACC(2, true, false); }
            else { if (stats) DP_ACC(2, false, true); else DP_ACC(2, false, false); }
        } else {
            if (first) { if (stats) DP_ACC(1, true, true); else DP_ACC(1, true, false); }
            else { if (stats) DP_ACC(1, false, true); else DP_ACC(1, false, false); }
        }
#undef DP_ACC
    });
}

template <bool kFlat>
hipError_t accumulate_all_t(dp_dtype gdt, bool first, int n, const Table& t, PieceSpan sp, const Srcs& grads,
                            const Srcs& accs, hipStream_t s) {
    return for_span(sp.p0, sp.p1, static_cast<unsigned>(n), [&](int64_t b, dim3 grid) {
        const dim3 blk(kWave);
#define DP_ALL(G, F) hipLaunchKernelGGL((k_accumulate_all<kFlat, G, F>), grid, blk, 0, s, t, b, grads, accs)
        if constexpr (kFlat) {
            if (gdt == DP_BF16) DP_ALL(2, true); else DP_ALL(1, true);
        } else if (gdt == DP_BF16) {
            if (first) DP_ALL(2, true); else DP_ALL(2, false);
        } else {
            if (first) DP_ALL(1, true); else DP_ALL(1, false);
        }
#undef DP_ALL
    });
}

template <bool kFlat>
hipError_t adamw_t(dp_dtype pdt, const Table& t, PieceSpan sp, RoleRef gbar, const StateRefs& sr, RoleRef p,
                   const DevState* st, const AdamArgs& args, hipStream_t s) {
    return for_span(sp.p0, sp.p1, 1, [&](int64_t b, dim3 grid) {
        if (pdt == DP_BF16)
            hipLaunchKernelGGL((k_adamw<kFlat, 2>), grid, dim3(kWave), 0, s, t, b, gbar, sr, p, st, args);
        else
            hipLaunchKernelGGL((k_adamw<kFlat, 1>), grid, dim3(kWave), 0, s, t, b, gbar, sr, p, st, args);
    });
}

template <int kMode, int kGrad, int N>
hipError_t reduce_adamw_n(dp_dtype pdt, const Table& t, PieceSpan sp, const Srcs& accs, const Srcs& grads,
                          const StateRefs& sr, RoleRef p, StatsBuf sb, const DevState* st, const AdamArgs& args,
                          hipStream_t s) {
    return for_span(sp.p0, sp.p1, 1, [&](int64_t b, dim3 grid) {
        if (pdt == DP_BF16)
            hipLaunchKernelGGL((k_reduce_adamw<kMode, kGrad, N, 2>), grid, dim3(kWave), 0, s, t, b, accs, grads, sr,
                               p, sb, st, args);
        else
            hipLaunchKernelGGL((k_reduce_adamw<kMode, kGrad, N, 1>), grid, dim3(kWave), 0, s, t, b, accs, grads, sr,
                               p, sb, st, args);
    });
}

template <int kMode, int kGrad>
hipError_t reduce_adamw_dispatch(dp_dtype pdt, int n, const Table& t, PieceSpan sp, const Srcs& accs,
                                 const Srcs& grads, const StateRefs& sr, RoleRef p, StatsBuf sb, const DevState* st,
                                 const AdamArgs& args, hipStream_t s) {
    switch (n) {
#define DP_CASE(K) \
    case K: return reduce_adamw_n<kMode, kGrad, K>(pdt, t, sp, accs, grads, sr, p, sb, st, args, s);
        DP_CASE(1) DP_CASE(2) DP_CASE(3) DP_CASE(4) DP_CASE(5) DP_CASE(6) DP_CASE(7) DP_CASE(8)
        DP_CASE(9) DP_CASE(10) DP_CASE(11) DP_CASE(12) DP_CASE(13) DP_CASE(14) DP_CASE(15) DP_CASE(16)
#undef DP_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Flat pieces serve only the first micro-step (no statistics) and the update;
// everything else runs on table pieces (the host decides, see api.cpp).
hipError_t launch_accumulate(dp_dtype gdt, bool first, bool stats, const Table& t, RoleRef grad, RoleRef acc,
                             StatsBuf sb, hipStream_t s) {
    if (t.flat && (!first || stats)) return hipErrorInvalidValue;
    return t.flat ? accumulate_t<true>(gdt, true, false, t, grad, acc, sb, s)
                  : accumulate_t<false>(gdt, first, stats, t, grad, acc, sb, s);
}

hipError_t launch_accumulate_all(dp_dtype gdt, bool first, int n, const Table& t, PieceSpan sp, const Srcs& grads,
                                 const Srcs& accs, hipStream_t s) {
    if ((t.flat && !first) || sp.p0 < 0 || sp.p1 > t.npieces || sp.p0 > sp.p1) return hipErrorInvalidValue;
    return t.flat ? accumulate_all_t<true>(gdt, true, n, t, sp, grads, accs, s)
                  : accumulate_all_t<false>(gdt, first, n, t, sp, grads, accs, s);
}

hipError_t launch_reduce(ReduceMode mode, dp_dtype gdt, int n, const Table& t, PieceSpan sp, const Srcs& accs,
                         const Srcs& grads, RoleRef gbar, StatsBuf sb, hipStream_t s) {
    if (t.flat || sp.p0 < 0 || sp.p1 > t.npieces || sp.p0 > sp.p1) return hipErrorInvalidValue;
    return reduce_modes<false>(mode, gdt, n, t, sp, accs, grads, gbar, sb, s);
}

hipError_t launch_stats(const Table& t, RoleRef gbar, StatsBuf sb, hipStream_t s) {
    if (t.flat) return hipErrorInvalidValue;
    return for_pieces(t.npieces, 1, [&](int64_t b, dim3 grid) {
        hipLaunchKernelGGL(k_stats<false>, grid, dim3(kWave), 0, s, t, b, gbar, sb);
    });
}

hipError_t launch_finalize(StatsBuf sb, int64_t nparts, FoldBuf fold, DevState* st, const ScalerArgs& args,
                           hipStream_t s) {
    const int64_t nslots = nparts > 0 ? stats_slots(nparts) : 0;
    if (nslots <= kFoldGroup) {
        hipLaunchKernelGGL(k_finalize<uint32_t>, dim3(1), dim3(kFoldThreads), 0, s, sb.sumsq, sb.bad, nslots, st, args);
        return hipGetLastError();
    }
    const int64_t groups = (nslots + kFoldGroup - 1) / kFoldGroup;
    hipLaunchKernelGGL(k_fold, dim3(static_cast<unsigned>(groups)), dim3(kFoldThreads), 0, s, sb, nslots, fold);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_finalize<uint64_t>, dim3(1), dim3(kFoldThreads), 0, s, fold.sumsq, fold.bad, groups, st,
                       args);
    return hipGetLastError();
}

hipError_t launch_adamw(dp_dtype pdt, const Table& t, PieceSpan sp, RoleRef gbar, const StateRefs& sr, RoleRef p,
                        const DevState* st, const AdamArgs& args, hipStream_t s) {
    if (sp.p0 < 0 || sp.p1 > t.npieces || sp.p0 > sp.p1) return hipErrorInvalidValue;
    return t.flat ? adamw_t<true>(pdt, t, sp, gbar, sr, p, st, args, s)
                  : adamw_t<false>(pdt, t, sp, gbar, sr, p, st, args, s);
}

hipError_t launch_reduce_adamw(ReduceMode mode, dp_dtype gdt, dp_dtype pdt, int n, const Table& t, PieceSpan sp,
                               const Srcs& accs, const Srcs& grads, const StateRefs& sr, RoleRef p, StatsBuf sb,
                               const DevState* st, const AdamArgs& args, hipStream_t s) {
    // statistics: table pieces, and a span inside the table
    if (t.flat || sp.p0 < 0 || sp.p1 > t.npieces || sp.p0 > sp.p1) return hipErrorInvalidValue;
    if (mode == ReduceMode::kGradients) {
        if (gdt == DP_F16) return reduce_adamw_dispatch<1, 1>(pdt, n, t, sp, accs, grads, sr, p, sb, st, args, s);
        return reduce_adamw_dispatch<1, 2>(pdt, n, t, sp, accs, grads, sr, p, sb, st, args, s);
    }
    if (mode == ReduceMode::kAccPlusGrad) {
        if (gdt == DP_F16) return reduce_adamw_dispatch<2, 1>(pdt, n, t, sp, accs, grads, sr, p, sb, st, args, s);
        return reduce_adamw_dispatch<2, 2>(pdt, n, t, sp, accs, grads, sr, p, sb, st, args, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_restore_param(dp_dtype pdt, const Table& t, const StateRefs& sr, RoleRef p, const DevState* st,
                                hipStream_t s) {
    if (t.npieces == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(t.npieces < kRestoreBlocks ? t.npieces : kRestoreBlocks));
    if (t.flat) {
        if (pdt == DP_BF16) hipLaunchKernelGGL((k_restore_param<true, 2>), grid, dim3(kWave), 0, s, t, sr, p, st);
        else hipLaunchKernelGGL((k_restore_param<true, 1>), grid, dim3(kWave), 0, s, t, sr, p, st);
    } else {
        if (pdt == DP_BF16) hipLaunchKernelGGL((k_restore_param<false, 2>), grid, dim3(kWave), 0, s, t, sr, p, st);
        else hipLaunchKernelGGL((k_restore_param<false, 1>), grid, dim3(kWave), 0, s, t, sr, p, st);
    }
    return hipGetLastError();
}

hipError_t launch_flat_table(dp_chunk* chunks, int64_t P, int log2c, StatsBuf sb, int64_t npieces, hipStream_t s) {
    const int64_t nchunks = (P + (int64_t{1} << log2c) - 1) >> log2c;
    const int64_t work = nchunks > 8 ? nchunks : 8;
    hipLaunchKernelGGL(k_flat_table, dim3(static_cast<unsigned>((work + 255) / 256)), dim3(256), 0, s, chunks, P,
                       log2c, nchunks, sb, npieces);
    return hipGetLastError();
}

hipError_t launch_upload_tables(const TableUploads& u, hipStream_t s) {
    if (u.count <= 0 || u.count > kMaxUploads || u.T <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_upload_tables, dim3(static_cast<unsigned>(u.count)), dim3(256), 0, s, u);
    return hipGetLastError();
}

hipError_t launch_state_init(DevState* st, double scale, hipStream_t s) {
    hipLaunchKernelGGL(k_state_init, dim3(1), dim3(kWave), 0, s, st, scale);
    return hipGetLastError();
}

}  // namespace dpk
