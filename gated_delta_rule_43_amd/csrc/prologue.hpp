// prologue.hpp -- optional input prologue of the KDA kernels (gfx950).
// Internal to libkda.so.
//
// "Kimi K3: Open Frontier Intelligence and Implementation Framework", section
// "Hybrid Attention Mechanism": KDA's forget gate is channel-wise and its decay
// is lower-bounded.  The parameterisation taken here makes the decay
// g = -g_lb * sigmoid(x) of gate logits x (so g lies in [-g_lb, 0] and
// alpha = exp(g) in [exp(-g_lb), 1]) and beta = sigmoid(b), and the
// recurrence reads L2-normalised queries and keys.  With the prologue the
// kernels take those raw projections and apply the three maps while loading,
// instead of a caller running them as separate elementwise passes over HBM:
//   q <- q (sum_c q_c^2 + eps)^-1/2,  k likewise   (0 when the sum is 0)
//   g <- -g_lb sigmoid(x),   beta <- sigmoid(b)
// each under its own flag bit (the values of KDA_PROLOGUE_* in kda.h).
#pragma once

#include "kda_common.hpp"

namespace kda {

constexpr unsigned PRO_NORM_QK = 1u;     // q, k are raw; L2-normalise per (token, head)
constexpr unsigned PRO_GATE_LOGIT = 2u;  // g holds logits x; g = -g_lb sigmoid(x)
constexpr unsigned PRO_BETA_LOGIT = 4u;  // beta holds logits b; beta = sigmoid(b)
constexpr unsigned PRO_ALL = PRO_NORM_QK | PRO_GATE_LOGIT | PRO_BETA_LOGIT;

struct Prologue {
    unsigned flags = 0;
    float glb = 0.f;  // g_lb
    float eps = 0.f;  // added to the sum of squares
};

// Which maps a kernel instantiation applies: none, all three (fixed at compile
// time, so the maps share basic blocks with the code around them), or those
// that pro.flags selects at run time.
enum ProMode { PRO_OFF = 0, PRO_FULL = 1, PRO_RUNTIME = 2 };

template <int PM>
__device__ __forceinline__ bool pro_on(const Prologue &p, unsigned bit) {
    return PM == PRO_FULL || (PM == PRO_RUNTIME && (p.flags & bit) != 0);
}

inline int pro_mode(const Prologue &p) {
    return p.flags == 0 ? PRO_OFF : (p.flags == PRO_ALL ? PRO_FULL : PRO_RUNTIME);
}

// bf16 bit pattern of -inf: a gate or beta logit that maps to exactly 0, used
// for the padding rows of a partial chunk (which must add nothing).
constexpr uint32_t BF16_NEG_INF_PAIR = 0xFF80FF80u;

// 1 / (1 + exp(-x)); exact limits 0 at -inf and 1 at +inf.
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.f + fast_exp(-x));
}

__device__ __forceinline__ float gate_from_logit(float x, float glb) { return -glb * sigmoid_f(x); }

__device__ __forceinline__ float inv_norm(float sumsq, float eps) {
    const float s = sumsq + eps;
    return s > 0.f ? rsqrtf(s) : 0.f;
}

// Sum over the 16 lanes of a DPP row (lanes 16 j .. 16 j + 15), every lane
// receiving the total: swaps within quads, then across the quads of a half
// row (row_half_mirror), then across the halves (row_mirror).
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    return x;
}

// Sum of squares of eight bf16 values packed in a uint4.
__device__ __forceinline__ float sumsq_bf16x8(const uint4 &u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = __uint_as_float(w[i] << 16), b = __uint_as_float(w[i] & 0xffff0000u);
        s += a * a + b * b;
    }
    return s;
}

__device__ __forceinline__ float sumsq8(const float *x) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += x[e] * x[e];
    return s;
}

}  // namespace kda
