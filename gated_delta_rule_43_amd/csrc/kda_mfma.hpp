// kda_mfma.hpp -- MFMA fragment helpers shared by the bf16 chunked kernels (gfx950).
// Internal to libkda.so.
#pragma once

#include "kda_common.hpp"

namespace kda {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Fragment layouts (verified on gfx950): for v_mfma_f32_16x16x32_f16 lane l
// holds row (l & 15) of A (column of B) and k = 8 (l >> 4) .. +7; for
// v_mfma_f32_16x16x16_f16, k = 4 (l >> 4) .. +3; the 16 x 16 result puts
// rows 4 (l >> 4) + i, column l & 15 in element i of lane l.
__device__ __forceinline__ floatx4 mma32(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma16(half4 a, half4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// 16x16x32 operand fragment of rows row0..row0+15, k = k0..k0+31 from a
// row-major [rows][k] fp16 tile: lane holds row (lane & 15), k = k0 + 8 (lane >> 4) .. +7.
__device__ __forceinline__ half8 frag8(const _Float16 *base, int pitch, int row0, int k0,
                                       int lane) {
    return *reinterpret_cast<const half8 *>(base + (row0 + (lane & 15)) * pitch + k0 +
                                            8 * (lane >> 4));
}
// 16x16x16 operand fragment: lane holds row (lane & 15), k = k0 + 4 (lane >> 4) .. +3.
__device__ __forceinline__ half4 frag4(const _Float16 *base, int pitch, int row0, int k0,
                                       int lane) {
    return *reinterpret_cast<const half4 *>(base + (row0 + (lane & 15)) * pitch + k0 +
                                            4 * (lane >> 4));
}
// An accumulator block (rows 4 (lane >> 4) + i, column lane & 15) as fp16: this
// is also the B fragment of a following 16x16x16 product with k = those rows.
__device__ __forceinline__ half4 to_half4(floatx4 x) {
    half4 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = (_Float16)x[i];
    return h;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ void unpack8(const uint4 &u, float *x) {
    x[0] = bf16lo(u.x); x[1] = bf16hi(u.x); x[2] = bf16lo(u.y); x[3] = bf16hi(u.y);
    x[4] = bf16lo(u.z); x[5] = bf16hi(u.z); x[6] = bf16lo(u.w); x[7] = bf16hi(u.w);
}


}  // namespace kda
