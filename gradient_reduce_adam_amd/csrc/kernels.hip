// gfx950 kernels of the data-parallel gradient reduce + AdamW step.
//
// Every streaming kernel walks a chunk table: workgroup b processes chunk
// (base + b), a contiguous piece of one tensor of at most chunk_elems
// elements.  A chunk whose pointers are all 16-byte aligned goes through
// 16-byte vector loads and stores (wave64 reads 1 KiB contiguous per
// instruction); any other chunk, and the ragged end of every chunk, takes a
// scalar loop.  All reductions are fixed-order trees (wavefront butterflies,
// then LDS across the four waves, then one partial per chunk), so results are
// bitwise reproducible run to run; no floating-point atomics are used.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dp_internal.h"

namespace dpk {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <typename T>
__device__ __forceinline__ T* elem_ptr(const RoleRef& r, const dp_chunk& c) {
    if (r.tab) return static_cast<T*>(r.tab[c.tensor]) + c.offset;
    return static_cast<T*>(r.base) + c.flat;
}

__device__ __forceinline__ bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Memory access through the global address space (global_load / global_store
// rather than flat_*: the pointers come from tables, so the compiler cannot
// infer the address space itself).  _nt variants set the nontemporal hint
// for data streamed once.
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

// ---- low-precision formats --------------------------------------------------
// kind: 1 = binary16, 2 = bfloat16 (dp_dtype values)
template <int kind>
__device__ __forceinline__ float widen1(uint16_t b) {
    if constexpr (kind == 2) return __uint_as_float(static_cast<uint32_t>(b) << 16);
    else return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

template <int kind>
__device__ __forceinline__ f32x8 widen8(u32x4 q) {
    if constexpr (kind == 2) {
        f32x8 f;
        f[0] = __uint_as_float(q.x << 16); f[1] = __uint_as_float(q.x & 0xFFFF0000u);
        f[2] = __uint_as_float(q.y << 16); f[3] = __uint_as_float(q.y & 0xFFFF0000u);
        f[4] = __uint_as_float(q.z << 16); f[5] = __uint_as_float(q.z & 0xFFFF0000u);
        f[6] = __uint_as_float(q.w << 16); f[7] = __uint_as_float(q.w & 0xFFFF0000u);
        return f;
    } else {
        return __builtin_convertvector(__builtin_bit_cast(f16x8, q), f32x8);
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

// ---- deterministic block reduction of (sumsq, bad) -----------------------
__device__ __forceinline__ void block_stats_store(double ss, uint32_t bad, int64_t cid, StatsBuf sb) {
    __shared__ double s_ss[kBlock / 64];
    __shared__ uint32_t s_bad[kBlock / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        ss += __shfl_xor(ss, off, 64);
        bad += __shfl_xor(bad, off, 64);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        s_ss[wave] = ss;
        s_bad[wave] = bad;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        sb.sumsq[cid] = (s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3]);
        sb.bad[cid] = s_bad[0] + s_bad[1] + s_bad[2] + s_bad[3];
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
__device__ __forceinline__ void accumulate_chunk(const dp_chunk& c, RoleRef grad, RoleRef acc, double& ss,
                                                 uint32_t& bad) {
    const uint16_t* __restrict__ g = elem_ptr<const uint16_t>(grad, c);
    float* __restrict__ a = elem_ptr<float>(acc, c);
    const int len = c.len, tid = threadIdx.x;
    const int nvec = (aligned16(g) && aligned16(a)) ? (len >> 3) : 0;  // 8 elements per vector
    constexpr int U = 2;
    for (int v0 = 0; v0 < nvec; v0 += kBlock * U) {
        u32x4 gq[U];
        f32x4 a0[U], a1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kBlock + tid;
            if (v < nvec) {
                gq[u] = ldg_nt<u32x4>(g, v);
                if constexpr (!kFirst) {
                    a0[u] = ldg<f32x4>(a, 2 * v);
                    a1[u] = ldg<f32x4>(a, 2 * v + 1);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kBlock + tid;
            if (v < nvec) {
                const f32x8 gf = widen8<kGrad>(gq[u]);
                f32x4 r0 = {gf[0], gf[1], gf[2], gf[3]};
                f32x4 r1 = {gf[4], gf[5], gf[6], gf[7]};
                if constexpr (!kFirst) {
                    r0 = a0[u] + r0;
                    r1 = a1[u] + r1;
                }
                stg<f32x4>(a, 2 * v, r0);
                stg<f32x4>(a, 2 * v + 1, r1);
                if constexpr (kStats) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ss += static_cast<double>(r0[e]) * static_cast<double>(r0[e]);
                        bad += nonfinite(r0[e]);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ss += static_cast<double>(r1[e]) * static_cast<double>(r1[e]);
                        bad += nonfinite(r1[e]);
                    }
                }
            }
        }
    }
    for (int i = nvec * 8 + tid; i < len; i += kBlock) {
        const float gi = widen1<kGrad>(ldg<uint16_t>(g, i));
        const float r = kFirst ? gi : ldg<float>(a, i) + gi;
        stg<float>(a, i, r);
        if constexpr (kStats) {
            ss += static_cast<double>(r) * static_cast<double>(r);
            bad += nonfinite(r);
        }
    }
}

// one replica; with kStats the chunk statistics of the result (n = 1: it is g_bar)
template <int kGrad, bool kFirst, bool kStats>
__global__ void __launch_bounds__(kBlock) k_accumulate(const dp_chunk* __restrict__ chunks, int64_t base,
                                                         RoleRef grad, RoleRef acc, StatsBuf sb) {
    const int64_t cid = base + blockIdx.x;
    const dp_chunk c = chunks[cid];
    double ss = 0.0;
    uint32_t bad = 0;
    accumulate_chunk<kGrad, kFirst, kStats>(c, grad, acc, ss, bad);
    if constexpr (kStats) block_stats_store(ss, bad, cid, sb);
}

// every replica's micro-step in one launch: workgroup b handles replica
// b / nchunks, chunk b % nchunks (replica-major, so each replica's buffers are
// streamed in order)
template <int kGrad, bool kFirst>
__global__ void __launch_bounds__(kBlock) k_accumulate_all(const dp_chunk* __restrict__ chunks, int64_t nchunks,
                                                             int64_t base, Srcs grads, Srcs accs) {
    const int64_t b = base + blockIdx.x;
    const int r = static_cast<int>(b / nchunks);
    const dp_chunk c = chunks[b - static_cast<int64_t>(r) * nchunks];
    double ss = 0.0;
    uint32_t bad = 0;
    accumulate_chunk<kGrad, kFirst, false>(c, grads.r[r], accs.r[r], ss, bad);
}

// ============================================================================
// replica reduction: gbar = tree(x_0..x_{N-1}) / N, plus chunk statistics
//   kMode 0: x_r = acc_r                 (binary32 accumulators)
//   kMode 1: x_r = g_r                   (low-precision gradients or partials)
//   kMode 2: x_r = acc_r + g_r           (the last micro-step fused: acc_r is
//                                         not written back)
// Modes 0 and 2 move 4 elements per lane (one dwordx4 of each binary32
// stream, a wave reads 1 KiB contiguous); mode 1 moves 8.
// ============================================================================
template <int N>
__device__ __forceinline__ void reduce_store(float (&x)[4][N], float* out, int64_t q, double& ss, uint32_t& bad) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        y[e] = average<N>(tree_sum<N>(x[e]));
        ss += static_cast<double>(y[e]) * static_cast<double>(y[e]);
        bad += nonfinite(y[e]);
    }
    stg_nt<f32x4>(out, q, f32x4{y[0], y[1], y[2], y[3]});
}

template <int kind>
__device__ __forceinline__ f32x4 widen4(u32x2 q) {
    if constexpr (kind == 2) {
        return f32x4{__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xFFFF0000u), __uint_as_float(q.y << 16),
                     __uint_as_float(q.y & 0xFFFF0000u)};
    } else {
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        return __builtin_convertvector(__builtin_bit_cast(f16x4, q), f32x4);
    }
}

template <int kMode, int kGrad, int N>
__global__ void __launch_bounds__(kBlock) k_reduce(const dp_chunk* __restrict__ chunks, int64_t base, Srcs accs,
                                                     Srcs grads, RoleRef gbar, StatsBuf sb) {
    const int64_t cid = base + blockIdx.x;
    const dp_chunk c = chunks[cid];
    const int len = c.len, tid = threadIdx.x;
    const float* ap[N];
    const uint16_t* gp[N];
    bool ok = true;
#pragma unroll
    for (int r = 0; r < N; ++r) {
        if constexpr (kMode != 1) {
            ap[r] = elem_ptr<const float>(accs.r[r], c);
            ok = ok && aligned16(ap[r]);
        }
        if constexpr (kMode != 0) {
            gp[r] = elem_ptr<const uint16_t>(grads.r[r], c);
            ok = ok && (reinterpret_cast<uintptr_t>(gp[r]) & (kMode == 1 ? 15u : 7u)) == 0;
        }
    }
    float* __restrict__ out = elem_ptr<float>(gbar, c);
    ok = ok && aligned16(out);
    constexpr int kVec = kMode == 1 ? 8 : 4;  // elements per lane and iteration
    constexpr int U = ((kMode == 0 && N <= 8) || (kMode == 2 && N <= 4)) ? 2 : 1;
    const int nvec = ok ? len / kVec : 0;
    double ss = 0.0;
    uint32_t bad = 0;
    for (int v0 = 0; v0 < nvec; v0 += kBlock * U) {
        if constexpr (kMode != 1) {
            f32x4 q[U][N];
            u32x2 h[U][N];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * kBlock + tid;
                if (v < nvec) {
#pragma unroll
                    for (int r = 0; r < N; ++r) {
                        q[u][r] = ldg_nt<f32x4>(ap[r], v);
                        if constexpr (kMode == 2) h[u][r] = ldg_nt<u32x2>(gp[r], v);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * kBlock + tid;
                if (v < nvec) {
                    float x[4][N];
#pragma unroll
                    for (int r = 0; r < N; ++r) {
                        f32x4 t = q[u][r];
                        if constexpr (kMode == 2) t = t + widen4<kGrad>(h[u][r]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e][r] = t[e];
                    }
                    reduce_store<N>(x, out, v, ss, bad);
                }
            }
        } else {
            const int v = v0 + tid;
            if (v < nvec) {
                f32x8 f[N];
#pragma unroll
                for (int r = 0; r < N; ++r) f[r] = widen8<kGrad>(ldg_nt<u32x4>(gp[r], v));
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    float x[4][N];
#pragma unroll
                    for (int r = 0; r < N; ++r)
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e][r] = f[r][4 * hh + e];
                    reduce_store<N>(x, out, 2 * static_cast<int64_t>(v) + hh, ss, bad);
                }
            }
        }
    }
    for (int i = nvec * kVec + tid; i < len; i += kBlock) {
        float x[N];
#pragma unroll
        for (int r = 0; r < N; ++r) {
            if constexpr (kMode == 0) x[r] = ldg<float>(ap[r], i);
            else if constexpr (kMode == 1) x[r] = widen1<kGrad>(ldg<uint16_t>(gp[r], i));
            else x[r] = ldg<float>(ap[r], i) + widen1<kGrad>(ldg<uint16_t>(gp[r], i));
        }
        const float y = average<N>(tree_sum<N>(x));
        stg<float>(out, i, y);
        ss += static_cast<double>(y) * static_cast<double>(y);
        bad += nonfinite(y);
    }
    block_stats_store(ss, bad, cid, sb);
}

// ============================================================================
// statistics scan of gbar (when not fused into the producer)
// ============================================================================
__global__ void __launch_bounds__(kBlock) k_stats(const dp_chunk* __restrict__ chunks, int64_t base, RoleRef gbar,
                                                    StatsBuf sb) {
    const int64_t cid = base + blockIdx.x;
    const dp_chunk c = chunks[cid];
    const float* __restrict__ x = elem_ptr<const float>(gbar, c);
    const int len = c.len, tid = threadIdx.x;
    const int nvec = aligned16(x) ? (len >> 2) : 0;
    double ss = 0.0;
    uint32_t bad = 0;
    for (int v = tid; v < nvec; v += kBlock) {
        const f32x4 q = ldg_nt<f32x4>(x, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ss += static_cast<double>(q[e]) * static_cast<double>(q[e]);
            bad += nonfinite(q[e]);
        }
    }
    for (int i = nvec * 4 + tid; i < len; i += kBlock) {
        const float y = ldg<float>(x, i);
        ss += static_cast<double>(y) * static_cast<double>(y);
        bad += nonfinite(y);
    }
    block_stats_store(ss, bad, cid, sb);
}

// ============================================================================
// pass 2: the chunk partials are folded in a fixed order -- by groups of
// kFoldGroup when there are many -- and one workgroup updates the scalar state
// ============================================================================
template <typename Count>
__device__ __forceinline__ void block_fold(const double* __restrict__ ss_in, const Count* __restrict__ bad_in,
                                           int64_t lo, int64_t hi, double& ss_out, uint64_t& bad_out) {
    __shared__ double s_ss[kBlock];
    __shared__ uint64_t s_bad[kBlock];
    const int tid = threadIdx.x;
    double ss = 0.0;
    uint64_t bad = 0;
    for (int64_t i = lo + tid; i < hi; i += kBlock) {
        ss += ss_in[i];
        bad += bad_in[i];
    }
    s_ss[tid] = ss;
    s_bad[tid] = bad;
    __syncthreads();
    for (int w = kBlock / 2; w > 0; w >>= 1) {
        if (tid < w) {
            s_ss[tid] = s_ss[tid] + s_ss[tid + w];
            s_bad[tid] = s_bad[tid] + s_bad[tid + w];
        }
        __syncthreads();
    }
    ss_out = s_ss[0];
    bad_out = s_bad[0];
}

__global__ void __launch_bounds__(kBlock) k_fold(StatsBuf sb, int64_t nparts, FoldBuf fold) {
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * kFoldGroup;
    const int64_t hi = lo + kFoldGroup < nparts ? lo + kFoldGroup : nparts;
    double ss;
    uint64_t bad;
    block_fold(sb.sumsq, sb.bad, lo, hi, ss, bad);
    if (threadIdx.x == 0) {
        fold.sumsq[blockIdx.x] = ss;
        fold.bad[blockIdx.x] = bad;
    }
}

template <typename Count>
__global__ void __launch_bounds__(kBlock) k_finalize(const double* __restrict__ ss_in, const Count* __restrict__ bad_in,
                                                       int64_t nparts, DevState* __restrict__ st, ScalerArgs args) {
    double sumsq;
    uint64_t badsum;
    block_fold(ss_in, bad_in, 0, nparts, sumsq, badsum);
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
    s.reserved = 0;
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
__global__ void __launch_bounds__(kBlock) k_adamw(const dp_chunk* __restrict__ chunks, int64_t base, RoleRef gbar,
                                                    RoleRef wr, RoleRef mr, RoleRef vr, RoleRef pr,
                                                    const DevState* __restrict__ st, AdamArgs args) {
    if (st->found_inf) return;
    AdamCoef k;
    {
#pragma clang fp contract(off)
        k.gscale = st->gscale;
        k.b1 = args.beta1;
        k.omb1 = 1.0 - args.beta1;
        k.b2 = args.beta2;
        k.omb2 = 1.0 - args.beta2;
        k.step = args.lr / (1.0 - st->beta1_pow);
        k.sqrt_bc2 = sqrt(1.0 - st->beta2_pow);
        k.eps = args.eps;
        k.dec = 1.0 - args.lr * args.weight_decay;
    }

    const int64_t cid = base + blockIdx.x;
    const dp_chunk c = chunks[cid];
    const float* __restrict__ gp = elem_ptr<const float>(gbar, c);
    float* __restrict__ wp = elem_ptr<float>(wr, c);
    float* __restrict__ mp = elem_ptr<float>(mr, c);
    float* __restrict__ vp = elem_ptr<float>(vr, c);
    uint16_t* __restrict__ pp = elem_ptr<uint16_t>(pr, c);
    const int len = c.len, tid = threadIdx.x;
    const bool ok = aligned16(gp) && aligned16(wp) && aligned16(mp) && aligned16(vp) &&
                    (reinterpret_cast<uintptr_t>(pp) & 7u) == 0;
    const int nvec = ok ? (len >> 2) : 0;  // 4 elements per vector
    constexpr int U = 2;
    for (int v0 = 0; v0 < nvec; v0 += kBlock * U) {
        f32x4 G[U], W[U], M[U], V[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = v0 + u * kBlock + tid;
            if (q < nvec) {
                G[u] = ldg_nt<f32x4>(gp, q);
                W[u] = ldg_nt<f32x4>(wp, q);
                M[u] = ldg_nt<f32x4>(mp, q);
                V[u] = ldg_nt<f32x4>(vp, q);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = v0 + u * kBlock + tid;
            if (q < nvec) {
                float w4[4] = {W[u][0], W[u][1], W[u][2], W[u][3]};
                float m4[4] = {M[u][0], M[u][1], M[u][2], M[u][3]};
                float v4[4] = {V[u][0], V[u][1], V[u][2], V[u][3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) adam1(G[u][e], w4[e], m4[e], v4[e], k);
                stg_nt<f32x4>(wp, q, f32x4{w4[0], w4[1], w4[2], w4[3]});
                stg_nt<f32x4>(mp, q, f32x4{m4[0], m4[1], m4[2], m4[3]});
                stg_nt<f32x4>(vp, q, f32x4{v4[0], v4[1], v4[2], v4[3]});
                const uint32_t p01 = static_cast<uint32_t>(narrow1<kParam>(w4[0])) |
                                     (static_cast<uint32_t>(narrow1<kParam>(w4[1])) << 16);
                const uint32_t p23 = static_cast<uint32_t>(narrow1<kParam>(w4[2])) |
                                     (static_cast<uint32_t>(narrow1<kParam>(w4[3])) << 16);
                stg_nt<u32x2>(pp, q, u32x2{p01, p23});
            }
        }
    }
    for (int i = nvec * 4 + tid; i < len; i += kBlock) {
        float w = ldg<float>(wp, i), m = ldg<float>(mp, i), v = ldg<float>(vp, i);
        adam1(ldg<float>(gp, i), w, m, v, k);
        stg<float>(wp, i, w);
        stg<float>(mp, i, m);
        stg<float>(vp, i, v);
        stg<uint16_t>(pp, i, narrow1<kParam>(w));
    }
}

// ---- launch helpers ---------------------------------------------------------
template <typename F>
hipError_t for_pieces(int64_t nchunks, F&& launch) {
    for (int64_t b = 0; b < nchunks; b += kMaxBlocksPerLaunch) {
        const int64_t cnt = nchunks - b < kMaxBlocksPerLaunch ? nchunks - b : kMaxBlocksPerLaunch;
        launch(b, dim3(static_cast<unsigned>(cnt)));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int kMode, int kGrad, int N>
hipError_t reduce_n(const dp_chunk* chunks, int64_t nchunks, const Srcs& accs, const Srcs& grads, RoleRef gbar,
                    StatsBuf sb, hipStream_t s) {
    return for_pieces(nchunks, [&](int64_t b, dim3 grid) {
        hipLaunchKernelGGL((k_reduce<kMode, kGrad, N>), grid, dim3(kBlock), 0, s, chunks, b, accs, grads, gbar, sb);
    });
}

template <int kMode, int kGrad>
hipError_t reduce_dispatch(int n, const dp_chunk* chunks, int64_t nchunks, const Srcs& accs, const Srcs& grads,
                           RoleRef gbar, StatsBuf sb, hipStream_t s) {
    switch (n) {
#define DP_CASE(K) \
    case K: return reduce_n<kMode, kGrad, K>(chunks, nchunks, accs, grads, gbar, sb, s);
        DP_CASE(1) DP_CASE(2) DP_CASE(3) DP_CASE(4) DP_CASE(5) DP_CASE(6) DP_CASE(7) DP_CASE(8)
        DP_CASE(9) DP_CASE(10) DP_CASE(11) DP_CASE(12) DP_CASE(13) DP_CASE(14) DP_CASE(15) DP_CASE(16)
#undef DP_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_accumulate(dp_dtype gdt, bool first, bool stats, const dp_chunk* chunks, int64_t nchunks,
                             RoleRef grad, RoleRef acc, StatsBuf sb, hipStream_t s) {
    return for_pieces(nchunks, [&](int64_t b, dim3 grid) {
        const dim3 blk(kBlock);
#define DP_ACC(G, F, S) hipLaunchKernelGGL((k_accumulate<G, F, S>), grid, blk, 0, s, chunks, b, grad, acc, sb)
        if (gdt == DP_BF16) {
            if (first) { if (stats) DP_ACC(2, true, true); else DP_ACC(2, true, false); }
            else { if (stats) DP_ACC(2, false, true); else DP_ACC(2, false, false); }
        } else {
            if (first) { if (stats) DP_ACC(1, true, true); else DP_ACC(1, true, false); }
            else { if (stats) DP_ACC(1, false, true); else DP_ACC(1, false, false); }
        }
#undef DP_ACC
    });
}

hipError_t launch_accumulate_all(dp_dtype gdt, bool first, int n, const dp_chunk* chunks, int64_t nchunks,
                                 const Srcs& grads, const Srcs& accs, hipStream_t s) {
    return for_pieces(nchunks * n, [&](int64_t b, dim3 grid) {
        const dim3 blk(kBlock);
        if (gdt == DP_BF16) {
            if (first) hipLaunchKernelGGL((k_accumulate_all<2, true>), grid, blk, 0, s, chunks, nchunks, b, grads, accs);
            else hipLaunchKernelGGL((k_accumulate_all<2, false>), grid, blk, 0, s, chunks, nchunks, b, grads, accs);
        } else {
            if (first) hipLaunchKernelGGL((k_accumulate_all<1, true>), grid, blk, 0, s, chunks, nchunks, b, grads, accs);
            else hipLaunchKernelGGL((k_accumulate_all<1, false>), grid, blk, 0, s, chunks, nchunks, b, grads, accs);
        }
    });
}

hipError_t launch_reduce(ReduceMode mode, dp_dtype gdt, int n, const dp_chunk* chunks, int64_t nchunks,
                         const Srcs& accs, const Srcs& grads, RoleRef gbar, StatsBuf sb, hipStream_t s) {
    if (mode == ReduceMode::kAccumulators) return reduce_dispatch<0, 2>(n, chunks, nchunks, accs, grads, gbar, sb, s);
    if (mode == ReduceMode::kGradients) {
        if (gdt == DP_F16) return reduce_dispatch<1, 1>(n, chunks, nchunks, accs, grads, gbar, sb, s);
        return reduce_dispatch<1, 2>(n, chunks, nchunks, accs, grads, gbar, sb, s);
    }
    if (gdt == DP_F16) return reduce_dispatch<2, 1>(n, chunks, nchunks, accs, grads, gbar, sb, s);
    return reduce_dispatch<2, 2>(n, chunks, nchunks, accs, grads, gbar, sb, s);
}

hipError_t launch_stats(const dp_chunk* chunks, int64_t nchunks, RoleRef gbar, StatsBuf sb, hipStream_t s) {
    return for_pieces(nchunks, [&](int64_t b, dim3 grid) {
        hipLaunchKernelGGL(k_stats, grid, dim3(kBlock), 0, s, chunks, b, gbar, sb);
    });
}

hipError_t launch_finalize(StatsBuf sb, int64_t nparts, FoldBuf fold, DevState* st, const ScalerArgs& args,
                           hipStream_t s) {
    if (nparts <= kFoldGroup) {
        hipLaunchKernelGGL(k_finalize<uint32_t>, dim3(1), dim3(kBlock), 0, s, sb.sumsq, sb.bad, nparts, st, args);
        return hipGetLastError();
    }
    const int64_t groups = (nparts + kFoldGroup - 1) / kFoldGroup;
    hipLaunchKernelGGL(k_fold, dim3(static_cast<unsigned>(groups)), dim3(kBlock), 0, s, sb, nparts, fold);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_finalize<uint64_t>, dim3(1), dim3(kBlock), 0, s, fold.sumsq, fold.bad, groups, st, args);
    return hipGetLastError();
}

hipError_t launch_adamw(dp_dtype pdt, const dp_chunk* chunks, int64_t nchunks, RoleRef gbar, RoleRef w, RoleRef m,
                        RoleRef v, RoleRef p, const DevState* st, const AdamArgs& args, hipStream_t s) {
    return for_pieces(nchunks, [&](int64_t b, dim3 grid) {
        if (pdt == DP_BF16)
            hipLaunchKernelGGL(k_adamw<2>, grid, dim3(kBlock), 0, s, chunks, b, gbar, w, m, v, p, st, args);
        else
            hipLaunchKernelGGL(k_adamw<1>, grid, dim3(kBlock), 0, s, chunks, b, gbar, w, m, v, p, st, args);
    });
}

hipError_t launch_state_init(DevState* st, double scale, hipStream_t s) {
    hipLaunchKernelGGL(k_state_init, dim3(1), dim3(64), 0, s, st, scale);
    return hipGetLastError();
}

}  // namespace dpk
