// Seeded synthetic inputs, device side: the bit-identical twin of
// synth_host.c (same definition: SplitMix64 output function over a counter,
// Irwin-Hall(4) integer, one binary32 multiply, round-to-nearest-even into the
// output format).  This is input generation for tests and benchmarks only; it
// holds none of the update step's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__device__ __forceinline__ float value_at(uint64_t key, int64_t i, float c) {
    uint64_t h = mix64(key + static_cast<uint64_t>(i + 1) * kGolden);
    int32_t s = static_cast<int32_t>(h & 0xFFFFu) + static_cast<int32_t>((h >> 16) & 0xFFFFu) +
                static_cast<int32_t>((h >> 32) & 0xFFFFu) + static_cast<int32_t>((h >> 48) & 0xFFFFu);
    return __fmul_rn(static_cast<float>(s - 131070), c);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return static_cast<uint16_t>((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return static_cast<uint16_t>((u + 0x7FFFu + lsb) >> 16);
}

__device__ __forceinline__ uint16_t to_f16(float x) {
    uint32_t u = __float_as_uint(x);
    uint16_t sign = static_cast<uint16_t>((u >> 16) & 0x8000u);
    uint32_t e = (u >> 23) & 0xFFu;
    uint32_t mant = u & 0x007FFFFFu;
    if (e == 0xFFu) return static_cast<uint16_t>(sign | 0x7C00u | (mant ? 0x0200u : 0u));
    int32_t ue = static_cast<int32_t>(e) - 127;
    if (ue > 15) return static_cast<uint16_t>(sign | 0x7C00u);
    if (ue >= -14) {
        uint32_t v = (static_cast<uint32_t>(ue + 15) << 10) | (mant >> 13);
        uint32_t rem = mant & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (v & 1u))) v += 1u;
        return static_cast<uint16_t>(sign | v);
    }
    if (e == 0u) return sign;
    uint32_t m24 = mant | 0x00800000u;
    int32_t shift = -ue - 1;
    if (shift > 24) return sign;
    uint32_t v = m24 >> shift;
    uint32_t rem = m24 & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (v & 1u))) v += 1u;
    return static_cast<uint16_t>(sign | v);
}

template <int kDtype>
__global__ void __launch_bounds__(256) gen_normal(uint64_t key, int64_t start, int64_t count, float c,
                                                  void* __restrict__ out) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < count; j += stride) {
        float x = value_at(key, start + j, c);
        if constexpr (kDtype == 0) {
            static_cast<float*>(out)[j] = x;
        } else if constexpr (kDtype == 1) {
            static_cast<uint16_t*>(out)[j] = to_f16(x);
        } else {
            static_cast<uint16_t*>(out)[j] = to_bf16(x);
        }
    }
}

// The same for several streams at once, one per blockIdx.y: out[y][j] is
// position start + j of keys[y] (all with the constant c).
constexpr int kMaxStreams = 16;
struct MultiOut {
    uint64_t keys[kMaxStreams];
    void* outs[kMaxStreams];
};

template <int kDtype>
__global__ void __launch_bounds__(256) gen_normal_multi(MultiOut m, int64_t start, int64_t count, float c) {
    const uint64_t key = m.keys[blockIdx.y];
    void* __restrict__ out = m.outs[blockIdx.y];
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < count; j += stride) {
        float x = value_at(key, start + j, c);
        if constexpr (kDtype == 0) {
            static_cast<float*>(out)[j] = x;
        } else if constexpr (kDtype == 1) {
            static_cast<uint16_t*>(out)[j] = to_f16(x);
        } else {
            static_cast<uint16_t*>(out)[j] = to_bf16(x);
        }
    }
}

__global__ void poke_u16(uint16_t* p, uint32_t bits) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = static_cast<uint16_t>(bits);
}

}  // namespace

extern "C" {

// Overwrites one 16-bit element (used to inject a non-finite gradient value).
int synth_poke_u16(void* p, uint32_t bits, hipStream_t stream) {
    if (p == nullptr) return -1;
    hipLaunchKernelGGL(poke_u16, dim3(1), dim3(64), 0, stream, static_cast<uint16_t*>(p), bits);
    return static_cast<int>(hipGetLastError());
}

// Fills out[0, count) with stream positions [start, start + count) of `key`.
// dtype: 0 binary32, 1 binary16, 2 bfloat16.  Asynchronous on `stream`.
// Returns 0 on success, -1 on a bad argument, or the HIP error code.
int synth_normal_device(uint64_t key, int64_t start, int64_t count, float c, int dtype, void* out,
                        hipStream_t stream) {
    if (count < 0 || (count > 0 && out == nullptr) || dtype < 0 || dtype > 2) return -1;
    if (count == 0) return 0;
    int64_t blocks64 = (count + 255) / 256;
    if (blocks64 > 65536) blocks64 = 65536;
    dim3 grid(static_cast<unsigned>(blocks64)), block(256);
    switch (dtype) {
        case 0: hipLaunchKernelGGL(gen_normal<0>, grid, block, 0, stream, key, start, count, c, out); break;
        case 1: hipLaunchKernelGGL(gen_normal<1>, grid, block, 0, stream, key, start, count, c, out); break;
        default: hipLaunchKernelGGL(gen_normal<2>, grid, block, 0, stream, key, start, count, c, out); break;
    }
    return static_cast<int>(hipGetLastError());
}

// synth_normal_device for n streams (keys[i] into outs[i], host arrays of n
// entries, n <= 16) in one launch.
int synth_normal_device_multi(const uint64_t* keys, const void* const* outs, int n, int64_t start, int64_t count,
                              float c, int dtype, hipStream_t stream) {
    if (n < 1 || n > kMaxStreams || !keys || !outs || count < 0 || dtype < 0 || dtype > 2) return -1;
    MultiOut m{};
    for (int i = 0; i < n; ++i) {
        if (count > 0 && outs[i] == nullptr) return -1;
        m.keys[i] = keys[i];
        m.outs[i] = const_cast<void*>(outs[i]);
    }
    if (count == 0) return 0;
    int64_t blocks64 = (count + 255) / 256;
    if (blocks64 > 65536 / n) blocks64 = 65536 / n > 0 ? 65536 / n : 1;
    dim3 grid(static_cast<unsigned>(blocks64), static_cast<unsigned>(n)), block(256);
    switch (dtype) {
        case 0: hipLaunchKernelGGL(gen_normal_multi<0>, grid, block, 0, stream, m, start, count, c); break;
        case 1: hipLaunchKernelGGL(gen_normal_multi<1>, grid, block, 0, stream, m, start, count, c); break;
        default: hipLaunchKernelGGL(gen_normal_multi<2>, grid, block, 0, stream, m, start, count, c); break;
    }
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
