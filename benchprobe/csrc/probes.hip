// Benchmark-only kernels; none of them is part of the method.
//  - bandwidth references shaped like the library's streaming kernels: a copy,
//    a read, and "stream mixes" that read and write exactly the arrays one of
//    the library's kernels streams, with the same access shape (one-shot wave64
//    workgroups over 256-element pieces, 16 bytes per lane per binary32 stream
//    and 8 per 16-bit stream, nontemporal hints where the library uses them)
//    and no arithmetic beyond a sum, so their rate is what that mix of
//    streams can reach on this GPU;
//  - a matrix-core load standing in for the compute of a backward pass.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define PROBE_GLOBAL __attribute__((address_space(1)))

template <typename V>
__device__ __forceinline__ V ld_nt(const void* p, int64_t i) {
    return __builtin_nontemporal_load(((const PROBE_GLOBAL V*)p) + i);
}
template <typename V>
__device__ __forceinline__ V ld(const void* p, int64_t i) { return ((const PROBE_GLOBAL V*)p)[i]; }
template <typename V>
__device__ __forceinline__ void st_nt(void* p, int64_t i, V x) {
    __builtin_nontemporal_store(x, ((PROBE_GLOBAL V*)p) + i);
}
template <typename V>
__device__ __forceinline__ void st(void* p, int64_t i, V x) { ((PROBE_GLOBAL V*)p)[i] = x; }

// ---- copy and read --------------------------------------------------------
// The copy moves one KiB per wave; the read takes four KiB per wave (a single
// KiB leaves it bound by how fast waves launch), sums them and stores only
// when the sum equals a value the caller's data never holds.
__global__ void __launch_bounds__(64) stream_copy(const f32x4* src, f32x4* dst, int64_t nvec) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x;
    if (i < nvec) st_nt<f32x4>(dst, i, ld_nt<f32x4>(src, i));
}

__global__ void __launch_bounds__(64) stream_read(const f32x4* src, int64_t nvec, float* sink) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t i = base + 64 * j;
        if (i < nvec) {
            const f32x4 v = ld_nt<f32x4>(src, i);
            s += (v.x + v.y) + (v.z + v.w);
        }
    }
    if (s == -1.0f && sink != nullptr) sink[0] = s;
}

// ---- stream mixes ------------------------------------------------------------
constexpr int kMaxStreams = 16;
struct MixPtrs {
    const void* r16[kMaxStreams];  // 16-bit streams read (nontemporal)
    const void* r32[kMaxStreams];  // binary32 streams read
    void* w32[kMaxStreams];        // binary32 streams written
    void* w16[kMaxStreams];        // 16-bit streams written (nontemporal)
};

// Piece p (one wave) covers elements [256 p, 256 p + 256); n is a multiple of
// 256.  With kRmw the first binary32 stream is read and written in place with
// plain accesses (the accumulator of a read-modify-write); every other access
// is nontemporal.  With a start table (stag != null) each wave first loads
// the entry of its group of 64 pieces and offsets its index by it (the
// entries are zero): the dependent scalar load the library's chunk table puts
// before a wave's first access, which staggers the waves' starts.
template <int R16, int R32, int W32, int W16, bool kRmw>
__global__ void __launch_bounds__(64) stream_mix(MixPtrs q, const int64_t* __restrict__ stag) {
    int64_t lane = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x;
    if (stag) lane += stag[blockIdx.x >> 6];
    f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < R16; ++k) {
        const u32x2 b = ld_nt<u32x2>(q.r16[k], lane);
        s += f32x4{__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u), __uint_as_float(b.y << 16),
                   __uint_as_float(b.y & 0xFFFF0000u)};
    }
#pragma unroll
    for (int k = 0; k < R32; ++k) s += (kRmw && k == 0) ? ld<f32x4>(q.r32[k], lane) : ld_nt<f32x4>(q.r32[k], lane);
#pragma unroll
    for (int k = 0; k < W32; ++k) {
        if (kRmw && k == 0) st<f32x4>(q.w32[k], lane, s);
        else st_nt<f32x4>(q.w32[k], lane, s + static_cast<float>(k));
    }
#pragma unroll
    for (int k = 0; k < W16; ++k) {
        const u32x2 b = {(__float_as_uint(s.x) >> 16) | (__float_as_uint(s.y) & 0xFFFF0000u),
                         (__float_as_uint(s.z) >> 16) | (__float_as_uint(s.w) & 0xFFFF0000u)};
        st_nt<u32x2>(q.w16[k], lane, b);
    }
}

template <int R16, int R32, int W32, int W16, bool kRmw>
hipError_t mix_launch(const MixPtrs& q, int64_t n, const int64_t* stag, hipStream_t s) {
    hipLaunchKernelGGL((stream_mix<R16, R32, W32, W16, kRmw>), dim3(static_cast<unsigned>(n / 256)), dim3(64), 0, s,
                       q, stag);
    return hipGetLastError();
}

// ---- matrix-core load ------------------------------------------------------
// Every wave chains `iters` bf16 products of 32x32x8 (16384 flops each) on
// register tiles, reading and writing no memory; the sum of the result feeds
// a comparison that never holds, so the products are not removed.
constexpr int kBusyThreads = 256;
constexpr unsigned kBusyBlocks = 1024;
constexpr double kFlopsPerProduct = 2.0 * 32 * 32 * 8;

__global__ void __launch_bounds__(kBusyThreads) busy_mfma(int64_t iters, float* sink) {
    const short v = static_cast<short>(threadIdx.x);
    const s16x4 a = {v, 1, 2, 3};
    const s16x4 b = {3, 2, 1, v};
    f32x16 acc = {};
    for (int64_t i = 0; i < iters; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, acc, 0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[e];
    if (s == -1.0f && sink != nullptr) sink[0] = s;
}

}  // namespace

extern "C" {

// One pass of a copy or read reference over `bytes` bytes (a multiple of
// 1024): kind 0 copies src to dst, kind 1 reads src (dst unused).  Returns 0,
// -1 on a bad argument, or the HIP error code.
int probe_stream(int kind, const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    if (src == nullptr || bytes <= 0 || bytes % 1024 != 0 || (kind == 0 && dst == nullptr) || kind < 0 || kind > 1)
        return -1;
    const int64_t nvec = bytes / 16;
    const int64_t blocks = kind == 0 ? nvec / 64 : (nvec + 255) / 256;
    if (blocks > (int64_t{1} << 31) - 1) return -1;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (kind == 0)
        hipLaunchKernelGGL(stream_copy, grid, dim3(64), 0, stream, static_cast<const f32x4*>(src),
                           static_cast<f32x4*>(dst), nvec);
    else
        hipLaunchKernelGGL(stream_read, grid, dim3(64), 0, stream, static_cast<const f32x4*>(src), nvec, nullptr);
    return static_cast<int>(hipGetLastError());
}

// One pass of a stream mix over n elements (a multiple of 256, at most
// 2^31 * 256): the streams of one of the library's kernels, given as host
// arrays of device pointers.  Supported mixes (r16, r32, w32, w16, rmw):
//   (1, 1, 1, 0, 1)  read-modify-write accumulation: gradient + accumulator in place
//   (n, 0, 1, 0, 0)  reduction of n partials into g_bar (n = 1 .. 16)
//   (n, n, 1, 0, 0)  last micro-step fused with the reduction (n = 1 .. 16)
//   (0, 4, 3, 1, 0)  two-pass AdamW: g_bar, w, m, v in; w, m, v, p out
//   (n, 3, 3, 1, 0)  single pass from n partials: out to the other bank
//   (n, n + 3, 3, 1, 0)  single pass after earlier micro-steps (n = 1 .. 13)
// stag: null, or device memory of ceil(n / 16384) zero int64 entries (the
// start table).  Returns 0, -1 for an unsupported mix or bad argument, or the
// HIP error code.
int probe_mix(int r16, int r32, int w32, int w16, int rmw, const void* const* p16, const void* const* p32,
              void* const* q32, void* const* q16, int64_t n, const int64_t* stag, hipStream_t stream) {
    if (n <= 0 || n % 256 != 0 || n / 256 > (int64_t{1} << 31) - 1 || r16 < 0 || r32 < 0 || w32 < 0 || w16 < 0 ||
        r16 > kMaxStreams || r32 > kMaxStreams || w32 > kMaxStreams || w16 > kMaxStreams)
        return -1;
    MixPtrs q{};
    for (int k = 0; k < r16; ++k) q.r16[k] = p16[k];
    for (int k = 0; k < r32; ++k) q.r32[k] = p32[k];
    for (int k = 0; k < w32; ++k) q.w32[k] = q32[k];
    for (int k = 0; k < w16; ++k) q.w16[k] = q16[k];
    for (int k = 0; k < r16; ++k)
        if (!q.r16[k]) return -1;
    for (int k = 0; k < r32; ++k)
        if (!q.r32[k]) return -1;
    for (int k = 0; k < w32; ++k)
        if (!q.w32[k]) return -1;
    for (int k = 0; k < w16; ++k)
        if (!q.w16[k]) return -1;
    if (rmw) {
        if (r16 == 1 && r32 == 1 && w32 == 1 && w16 == 0 && q.r32[0] == q.w32[0])
            return static_cast<int>(mix_launch<1, 1, 1, 0, true>(q, n, stag, stream));
        return -1;
    }
#define PROBE_N(N)                                                                          \
    case N:                                                                                 \
        if (r32 == 0 && w32 == 1 && w16 == 0) return mix_launch<N, 0, 1, 0, false>(q, n, stag, stream);   \
        if (r32 == N && w32 == 1 && w16 == 0) return mix_launch<N, N, 1, 0, false>(q, n, stag, stream);   \
        if (r32 == 3 && w32 == 3 && w16 == 1) return mix_launch<N, 3, 3, 1, false>(q, n, stag, stream);   \
        if (N <= 13 && r32 == N + 3 && w32 == 3 && w16 == 1)                                      \
            return mix_launch<N, (N <= 13 ? N + 3 : 3), 3, 1, false>(q, n, stag, stream);                 \
        return -1;
    switch (r16) {
        case 0:
            if (r32 == 4 && w32 == 3 && w16 == 1) return mix_launch<0, 4, 3, 1, false>(q, n, stag, stream);
            return -1;
        PROBE_N(1) PROBE_N(2) PROBE_N(3) PROBE_N(4) PROBE_N(5) PROBE_N(6) PROBE_N(7) PROBE_N(8)
        PROBE_N(9) PROBE_N(10) PROBE_N(11) PROBE_N(12) PROBE_N(13) PROBE_N(14) PROBE_N(15) PROBE_N(16)
        default: return -1;
    }
#undef PROBE_N
}

// Occupies the matrix cores with about `flops` floating-point operations
// (bf16 products, rounded up to whole products per wave) on `stream`: the
// compute of a synthetic backward pass.  Returns 0, -1 on a bad argument, or
// the HIP error code.
int probe_busy(double flops, hipStream_t stream) {
    if (!(flops >= 0.0)) return -1;
    const double waves = static_cast<double>(kBusyBlocks) * (kBusyThreads / 64);
    const int64_t iters = static_cast<int64_t>(flops / (waves * kFlopsPerProduct) + 0.999999);
    if (iters == 0) return 0;
    hipLaunchKernelGGL(busy_mfma, dim3(kBusyBlocks), dim3(kBusyThreads), 0, stream, iters, nullptr);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
