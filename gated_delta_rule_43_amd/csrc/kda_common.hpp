// kda_common.hpp -- element conversions and small device helpers shared by the
// KDA kernels for gfx950.  Internal to libkda.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace kda {

// Raises a kernel's dynamic LDS limit to `bytes` once per device (bit d of
// `done` records device d): the attribute persists, and setting it on every
// launch would cost host time on every call.
inline hipError_t ensure_dynamic_lds(const void *fn, int bytes, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (1ull << dev) : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

// bf16 is carried as its 16-bit pattern; widening to fp32 is exact.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

// fp32 -> bf16 with round-to-nearest-even (quiet NaN kept as NaN).
__device__ __forceinline__ bf16_t from_f32_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    bf16_t r;
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
        r.bits = static_cast<uint16_t>((u >> 16) | 0x0040u);
    } else {
        u += 0x7fffu + ((u >> 16) & 1u);
        r.bits = static_cast<uint16_t>(u >> 16);
    }
    return r;
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return from_f32_bf16(f); }

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Sequence bounds of packed sequence n, clamped so that malformed offsets can
// never produce an out-of-range token index.
__device__ __forceinline__ void seq_bounds(const int32_t *cu, int n, int fixedT, int totalT,
                                           int &bos, int &eos) {
    if (cu) {
        int a = cu[n], b = cu[n + 1];
        a = a < 0 ? 0 : (a > totalT ? totalT : a);
        b = b < a ? a : (b > totalT ? totalT : b);
        bos = a;
        eos = b;
    } else {
        bos = n * fixedT;
        eos = bos + fixedT;
    }
}

}  // namespace kda
