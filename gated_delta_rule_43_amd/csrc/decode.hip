// decode.hip -- one recurrent KDA decode step on gfx950.
//
// "Kimi K3: Open Frontier Intelligence and Implementation Framework", section
// "Inference Serving": serving keeps one KDA recurrent state per sequence.
// A decode step feeds one token per sequence through the recurrence of
// section "Hybrid Attention Mechanism" (delta rule, channel-wise forget gate):
//
//   S'  = Diag(alpha) S                  (row c scaled by exp(g[c]))
//   r_k = S'^T k,   r_q = S'^T q         (column reductions over key channels)
//   u   = beta (v - r_k)
//   S   = S' + k u^T                      (written back in place)
//   o   = S^T q = r_q + (k . q) u
//
// The step is a pure stream over the fp32 state (K*V*4 bytes read and written
// per head, no reuse), so it is HBM-bound and uses the vector ALUs only.  One
// workgroup owns one (sequence, head) state: each thread keeps its rows of
// four consecutive columns in registers between the read and the write-back,
// so the state crosses HBM exactly twice.  Loads are 16-byte and a wavefront
// covers whole rows, so every access is fully coalesced.  The write-back uses
// non-temporal stores: the new state is not read again within the step, and
// streaming it past the caches lifts the read+write stream from about 5.0 to
// 6.7 TB/s on MI355X (non-temporal loads, by contrast, slow it down).
#include "kda_common.hpp"
#include "prologue.hpp"

namespace kda {

// One workgroup of NT threads per (sequence, head): thread (cg, rg) keeps
// rows rg, rg + RG, .. (RPT of them) of columns 4 cg .. 4 cg + 3 of the state.
template <int K, int V, int NT>
struct DecodeShape {
    static constexpr int CG = V / 4;    // column groups of four floats
    static constexpr int RG = NT / CG;  // row groups
    static constexpr int RPT = K / RG;  // rows per thread
    static constexpr int NW = NT / 64;  // wavefronts per workgroup
    static_assert(V % 4 == 0 && CG <= 64 && 64 % CG == 0, "column groups must tile a wave");
    static_assert(NT % CG == 0 && K % RG == 0, "rows must tile the workgroup");
};

template <int K, int V, int NT>
struct DecodeLds {
    float sq[K], sk[K], sa[K];
    float4 red[DecodeShape<K, V, NT>::NW][DecodeShape<K, V, NT>::CG][2];
    float skq;
};

// One token through the recurrence for the workgroup's (sequence, head):
// scales this thread's rows s[0 .. RPT) by alpha in place, writes o (row group 0) and
// returns u for its four columns; the new state is s + k_r u on row r.
// q, k, g point at the token's [K] vectors, v at its [V] vector.  Leaves
// lds.sk valid for the caller; callers that run another token first pass a
// barrier (every thread is done reading lds).  PRO: the input prologue
// (prologue.hpp) applies as pro.flags selects; wave 0 then normalises q and k
// (a wave-wide sum of squares) while the other waves fill in the decay.
template <int K, int V, int NT, typename TIn, typename TOut, bool PRO>
__device__ __forceinline__ float4 decode_token(float4 *s, const TIn *q, const TIn *k, const TIn *g,
                                               const TIn *beta, const TIn *v, TOut *o,
                                               DecodeLds<K, V, NT> &lds, const Prologue &pro) {
    using D = DecodeShape<K, V, NT>;
    const int t = threadIdx.x;
    const int cg = t % D::CG, rg = t / D::CG;
    const int lane = t & 63, w = t >> 6;
    const bool gate_logit = PRO && (pro.flags & PRO_GATE_LOGIT);
    if (PRO && (pro.flags & PRO_NORM_QK)) {
        if (w == 0) {
            constexpr int CPL = (K + 63) / 64;  // channels per lane
            float qv[CPL], kv[CPL], sq = 0.f, sk = 0.f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = lane + 64 * i;
                qv[i] = c < K ? to_f32(q[c]) : 0.f;
                kv[i] = c < K ? to_f32(k[c]) : 0.f;
                sq += qv[i] * qv[i];
                sk += kv[i] * kv[i];
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                sq += __shfl_xor(sq, off);
                sk += __shfl_xor(sk, off);
            }
            const float iq = inv_norm(sq, pro.eps), ik = inv_norm(sk, pro.eps);
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = lane + 64 * i;
                if (c < K) {
                    lds.sq[c] = qv[i] * iq;
                    lds.sk[c] = kv[i] * ik;
                }
            }
        }
        for (int c = t; c < K; c += NT) {
            const float x = to_f32(g[c]);
            lds.sa[c] = fast_exp(gate_logit ? gate_from_logit(x, pro.glb) : x);
        }
    } else {
        for (int c = t; c < K; c += NT) {
            lds.sq[c] = to_f32(q[c]);
            lds.sk[c] = to_f32(k[c]);
            const float x = to_f32(g[c]);
            lds.sa[c] = fast_exp(gate_logit ? gate_from_logit(x, pro.glb) : x);
        }
    }
    __syncthreads();
    if (w == 0) {
        float p = 0.f;
        for (int c = lane; c < K; c += 64) p += lds.sk[c] * lds.sq[c];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
        if (lane == 0) lds.skq = p;
    }

    float4 rk = make_float4(0.f, 0.f, 0.f, 0.f), rq = rk;
#pragma unroll
    for (int i = 0; i < D::RPT; ++i) {
        const int r = rg + i * D::RG;
        const float a = lds.sa[r], kr = lds.sk[r], qr = lds.sq[r];
        s[i].x *= a; s[i].y *= a; s[i].z *= a; s[i].w *= a;
        rk.x += kr * s[i].x; rk.y += kr * s[i].y; rk.z += kr * s[i].z; rk.w += kr * s[i].w;
        rq.x += qr * s[i].x; rq.y += qr * s[i].y; rq.z += qr * s[i].z; rq.w += qr * s[i].w;
    }
    // Lanes of one wave holding the same columns differ by multiples of CG.
#pragma unroll
    for (int off = D::CG; off < 64; off <<= 1) {
        rk.x += __shfl_xor(rk.x, off); rk.y += __shfl_xor(rk.y, off);
        rk.z += __shfl_xor(rk.z, off); rk.w += __shfl_xor(rk.w, off);
        rq.x += __shfl_xor(rq.x, off); rq.y += __shfl_xor(rq.y, off);
        rq.z += __shfl_xor(rq.z, off); rq.w += __shfl_xor(rq.w, off);
    }
    if (lane < D::CG) {
        lds.red[w][lane][0] = rk;
        lds.red[w][lane][1] = rq;
    }
    __syncthreads();
    float4 RK = lds.red[0][cg][0], RQ = lds.red[0][cg][1];
#pragma unroll
    for (int ww = 1; ww < D::NW; ++ww) {
        const float4 a = lds.red[ww][cg][0], b = lds.red[ww][cg][1];
        RK.x += a.x; RK.y += a.y; RK.z += a.z; RK.w += a.w;
        RQ.x += b.x; RQ.y += b.y; RQ.z += b.z; RQ.w += b.w;
    }
    float b = to_f32(beta[0]);
    if (PRO && (pro.flags & PRO_BETA_LOGIT)) b = sigmoid_f(b);
    const TIn *vp = v + 4 * cg;
    float4 u;
    u.x = b * (to_f32(vp[0]) - RK.x);
    u.y = b * (to_f32(vp[1]) - RK.y);
    u.z = b * (to_f32(vp[2]) - RK.z);
    u.w = b * (to_f32(vp[3]) - RK.w);
    if (rg == 0) {
        const float kq = lds.skq;
        TOut *op = o + 4 * cg;
        op[0] = from_f32<TOut>(RQ.x + kq * u.x);
        op[1] = from_f32<TOut>(RQ.y + kq * u.y);
        op[2] = from_f32<TOut>(RQ.z + kq * u.z);
        op[3] = from_f32<TOut>(RQ.w + kq * u.w);
    }
    return u;
}

typedef float f4v __attribute__((ext_vector_type(4)));

// Writes this thread's rows of the new state s + k_r u to S (non-temporal).
template <int K, int V, int NT>
__device__ __forceinline__ void store_state(float4 *S, const float4 *s, const float4 &u,
                                            const float *sk) {
    using D = DecodeShape<K, V, NT>;
    const int cg = threadIdx.x % D::CG, rg = threadIdx.x / D::CG;
#pragma unroll
    for (int i = 0; i < D::RPT; ++i) {
        const int r = rg + i * D::RG;
        const float kr = sk[r];
        const f4v x = {s[i].x + kr * u.x, s[i].y + kr * u.y, s[i].z + kr * u.z, s[i].w + kr * u.w};
        __builtin_nontemporal_store(x, reinterpret_cast<f4v *>(&S[r * D::CG + cg]));
    }
}

// One decode step.  PAGED: the states live in pool slots (slot_in /
// slot_out); otherwise the unit's own entry of a dense [N, H, K, V] array is
// updated in place.  PRO: with the input prologue.
template <int K, int V, int NT, typename TIn, typename TOut, bool PAGED, bool PRO>
__global__ __launch_bounds__(NT) void decode_step_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const TIn *__restrict__ g, const TIn *__restrict__ beta, float *__restrict__ state,
    const int32_t *__restrict__ slot_in, const int32_t *__restrict__ slot_out, int pool_slots,
    int H, Prologue pro, TOut *__restrict__ o) {
    using D = DecodeShape<K, V, NT>;
    __shared__ DecodeLds<K, V, NT> lds;

    const size_t unit = blockIdx.x;  // n * H + h
    const int t = threadIdx.x;
    const int cg = t % D::CG, rg = t / D::CG;

    // The state is read from Sin and written to Sout: the unit's own entry of
    // a dense [N, H, K, V] array, or slots slot_in[n] / slot_out[n] of a pool
    // (equal slots update in place; an input slot outside the pool reads as
    // zeros, an output slot outside it is not written).
    const float4 *Sin = reinterpret_cast<const float4 *>(state + unit * (size_t)(K * V));
    float4 *Sout = reinterpret_cast<float4 *>(state + unit * (size_t)(K * V));
    if constexpr (PAGED) {
        const int n = (int)(unit / H), h = (int)(unit % H);
        const int si = slot_in[n], so = slot_out[n];
        Sin = si >= 0 && si < pool_slots
                  ? reinterpret_cast<const float4 *>(state + ((size_t)si * H + h) * (K * V))
                  : nullptr;
        Sout = so >= 0 && so < pool_slots
                   ? reinterpret_cast<float4 *>(state + ((size_t)so * H + h) * (K * V))
                   : nullptr;
    }

    // Issue the state loads first; the small per-head vectors follow.
    float4 s[D::RPT];
    if (!PAGED || Sin) {
#pragma unroll
        for (int i = 0; i < D::RPT; ++i) s[i] = Sin[(rg + i * D::RG) * D::CG + cg];
    } else {
#pragma unroll
        for (int i = 0; i < D::RPT; ++i) s[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float4 u = decode_token<K, V, NT, TIn, TOut, PRO>(s, q + unit * K, k + unit * K,
                                                            g + unit * K, beta + unit, v + unit * V,
                                                            o + unit * V, lds, pro);
    if (!PAGED || Sout) store_state<K, V, NT>(Sout, s, u, lds.sk);
}

// T consecutive tokens per sequence in one pass over each state (the
// verification step of speculative decoding): tokens are [N, T, H, *]; the
// state is read once from slot_in[n], kept in registers, advanced token by
// token, and after token j written to slot slot_out[n * T + j] when that slot
// lies in the pool (so the caller keeps exactly the prefixes it may accept).
template <int K, int V, int NT, typename TIn, typename TOut, bool PRO>
__global__ __launch_bounds__(NT) void decode_multi_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const TIn *__restrict__ g, const TIn *__restrict__ beta, float *__restrict__ pool,
    const int32_t *__restrict__ slot_in, const int32_t *__restrict__ slot_out, int pool_slots,
    int T, int H, Prologue pro, TOut *__restrict__ o) {
    using D = DecodeShape<K, V, NT>;
    __shared__ DecodeLds<K, V, NT> lds;

    const int unit = blockIdx.x;  // n * H + h
    const int n = unit / H, h = unit % H;
    const int t = threadIdx.x;
    const int cg = t % D::CG, rg = t / D::CG;
    auto slot_ptr = [&](int sl) {
        return sl >= 0 && sl < pool_slots ? reinterpret_cast<float4 *>(pool + ((size_t)sl * H + h) * (K * V))
                                          : nullptr;
    };

    const float4 *Sin = slot_ptr(slot_in[n]);
    float4 s[D::RPT];
    if (Sin) {
#pragma unroll
        for (int i = 0; i < D::RPT; ++i) s[i] = Sin[(rg + i * D::RG) * D::CG + cg];
    } else {
#pragma unroll
        for (int i = 0; i < D::RPT; ++i) s[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int j = 0; j < T; ++j) {
        if (j > 0) __syncthreads();  // every thread is done with the previous token's lds
        const size_t tok = ((size_t)n * T + j) * H + h;
        const float4 u = decode_token<K, V, NT, TIn, TOut, PRO>(s, q + tok * K, k + tok * K,
                                                                g + tok * K, beta + tok, v + tok * V,
                                                                o + tok * V, lds, pro);
        float4 *Sout = slot_ptr(slot_out[(size_t)n * T + j]);
        if (Sout) store_state<K, V, NT>(Sout, s, u, lds.sk);
        // the new state stays in registers for the next token
#pragma unroll
        for (int i = 0; i < D::RPT; ++i) {
            const float kr = lds.sk[rg + i * D::RG];
            s[i].x += kr * u.x; s[i].y += kr * u.y; s[i].z += kr * u.z; s[i].w += kr * u.w;
        }
    }
}

// Slot arrays null: dense states [N, H, K, V] updated in place.
struct DecodeStates {
    float *state;
    const int32_t *slot_in, *slot_out;
    int pool_slots;
};

template <int K, int V, int NT, typename TIn, typename TOut, bool PAGED, bool PRO>
static void launch_step(const void *q, const void *k, const void *v, const void *g,
                        const void *beta, const DecodeStates &st, const Prologue &pro, void *o,
                        int units, int H, hipStream_t stream) {
    hipLaunchKernelGGL((decode_step_kernel<K, V, NT, TIn, TOut, PAGED, PRO>), dim3(units), dim3(NT),
                       0, stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                       static_cast<const TIn *>(v), static_cast<const TIn *>(g),
                       static_cast<const TIn *>(beta), st.state, PAGED ? st.slot_in : nullptr,
                       PAGED ? st.slot_out : nullptr, PAGED ? st.pool_slots : 0, H, pro,
                       static_cast<TOut *>(o));
}

template <int K, int V, int NT, typename TIn, typename TOut>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, const DecodeStates &st, const Prologue &pro,
                                  void *o, int units, int H, hipStream_t stream) {
    if (st.slot_in) {
        if (pro.flags) launch_step<K, V, NT, TIn, TOut, true, true>(q, k, v, g, beta, st, pro, o, units, H, stream);
        else launch_step<K, V, NT, TIn, TOut, true, false>(q, k, v, g, beta, st, pro, o, units, H, stream);
    } else {
        if (pro.flags) launch_step<K, V, NT, TIn, TOut, false, true>(q, k, v, g, beta, st, pro, o, units, H, stream);
        else launch_step<K, V, NT, TIn, TOut, false, false>(q, k, v, g, beta, st, pro, o, units, H, stream);
    }
    return hipGetLastError();
}

template <int K, int V, int NT>
static hipError_t launch_decode_kv(const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, const DecodeStates &st, const Prologue &pro,
                                   void *o, int units, int H, bool in_bf16, bool out_bf16,
                                   hipStream_t stream) {
    if (in_bf16) {
        return out_bf16 ? launch_decode_t<K, V, NT, bf16_t, bf16_t>(q, k, v, g, beta, st, pro, o, units, H, stream)
                        : launch_decode_t<K, V, NT, bf16_t, float>(q, k, v, g, beta, st, pro, o, units, H, stream);
    }
    return out_bf16 ? launch_decode_t<K, V, NT, float, bf16_t>(q, k, v, g, beta, st, pro, o, units, H, stream)
                    : launch_decode_t<K, V, NT, float, float>(q, k, v, g, beta, st, pro, o, units, H, stream);
}

// Internal launcher: shapes were validated by the caller.  slot_in / slot_out
// null: state is a dense [N, H, K, V] array updated in place; else state is a
// pool of pool_slots slots.
hipError_t launch_decode(const void *q, const void *k, const void *v, const void *g,
                         const void *beta, float *state, const int32_t *slot_in,
                         const int32_t *slot_out, int pool_slots, const Prologue &pro, void *o,
                         int N, int H, int K, int V, bool in_bf16, bool out_bf16,
                         hipStream_t stream) {
    const int units = N * H;
    if (units == 0) return hipSuccess;
    const DecodeStates st{state, slot_in, slot_out, pool_slots};
    if (K == 128 && V == 128)
        return launch_decode_kv<128, 128, 256>(q, k, v, g, beta, st, pro, o, units, H, in_bf16, out_bf16, stream);
    if (K == 32 && V == 32)
        return launch_decode_kv<32, 32, 64>(q, k, v, g, beta, st, pro, o, units, H, in_bf16, out_bf16, stream);
    return hipErrorInvalidValue;
}

struct MultiArgs {
    float *pool;
    const int32_t *slot_in, *slot_out;
    int pool_slots, N, T, H;
};

template <int K, int V, int NT, typename TIn, typename TOut>
static hipError_t launch_multi_t(const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, const MultiArgs &a, const Prologue &pro,
                                 void *o, hipStream_t stream) {
    if (pro.flags)
        hipLaunchKernelGGL((decode_multi_kernel<K, V, NT, TIn, TOut, true>), dim3(a.N * a.H), dim3(NT),
                           0, stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                           static_cast<const TIn *>(v), static_cast<const TIn *>(g),
                           static_cast<const TIn *>(beta), a.pool, a.slot_in, a.slot_out,
                           a.pool_slots, a.T, a.H, pro, static_cast<TOut *>(o));
    else
        hipLaunchKernelGGL((decode_multi_kernel<K, V, NT, TIn, TOut, false>), dim3(a.N * a.H), dim3(NT),
                           0, stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                           static_cast<const TIn *>(v), static_cast<const TIn *>(g),
                           static_cast<const TIn *>(beta), a.pool, a.slot_in, a.slot_out,
                           a.pool_slots, a.T, a.H, pro, static_cast<TOut *>(o));
    return hipGetLastError();
}

template <int K, int V, int NT>
static hipError_t launch_multi_kv(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, const MultiArgs &a, const Prologue &pro,
                                  void *o, bool in_bf16, bool out_bf16, hipStream_t stream) {
    if (in_bf16)
        return out_bf16 ? launch_multi_t<K, V, NT, bf16_t, bf16_t>(q, k, v, g, beta, a, pro, o, stream)
                        : launch_multi_t<K, V, NT, bf16_t, float>(q, k, v, g, beta, a, pro, o, stream);
    return out_bf16 ? launch_multi_t<K, V, NT, float, bf16_t>(q, k, v, g, beta, a, pro, o, stream)
                    : launch_multi_t<K, V, NT, float, float>(q, k, v, g, beta, a, pro, o, stream);
}

// Internal launcher of the multi-token step: shapes were validated by the caller.
hipError_t launch_decode_multi(const void *q, const void *k, const void *v, const void *g,
                               const void *beta, float *pool, const int32_t *slot_in,
                               const int32_t *slot_out, int pool_slots, const Prologue &pro,
                               void *o, int N, int T, int H, int K, int V, bool in_bf16,
                               bool out_bf16, hipStream_t stream) {
    if (N == 0 || T == 0) return hipSuccess;
    const MultiArgs a{pool, slot_in, slot_out, pool_slots, N, T, H};
    if (K == 128 && V == 128)
        return launch_multi_kv<128, 128, 256>(q, k, v, g, beta, a, pro, o, in_bf16, out_bf16, stream);
    if (K == 32 && V == 32)
        return launch_multi_kv<32, 32, 64>(q, k, v, g, beta, a, pro, o, in_bf16, out_bf16, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
