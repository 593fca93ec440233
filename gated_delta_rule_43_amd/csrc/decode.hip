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

namespace kda {

// PAGED: the states live in pool slots (slot_in / slot_out); otherwise the
// unit's own entry of a dense [N, H, K, V] array is updated in place.
template <int K, int V, int NT, typename TIn, typename TOut, bool PAGED>
__global__ __launch_bounds__(NT) void decode_step_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const TIn *__restrict__ g, const TIn *__restrict__ beta, float *__restrict__ state,
    const int32_t *__restrict__ slot_in, const int32_t *__restrict__ slot_out, int pool_slots,
    int H, TOut *__restrict__ o) {
    constexpr int CG = V / 4;    // column groups of four floats
    constexpr int RG = NT / CG;  // row groups
    constexpr int RPT = K / RG;  // rows per thread
    constexpr int NW = NT / 64;  // wavefronts per workgroup
    static_assert(V % 4 == 0 && CG <= 64 && 64 % CG == 0, "column groups must tile a wave");
    static_assert(NT % CG == 0 && K % RG == 0, "rows must tile the workgroup");

    __shared__ float sq[K], sk[K], sa[K];
    __shared__ float4 red[NW][CG][2];
    __shared__ float skq;

    const size_t unit = blockIdx.x;  // n * H + h
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    const int lane = t & 63, w = t >> 6;

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
    float4 s[RPT];
    if (!PAGED || Sin) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) s[i] = Sin[(rg + i * RG) * CG + cg];
    } else {
#pragma unroll
        for (int i = 0; i < RPT; ++i) s[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    for (int c = t; c < K; c += NT) {
        sq[c] = to_f32(q[unit * K + c]);
        sk[c] = to_f32(k[unit * K + c]);
        sa[c] = fast_exp(to_f32(g[unit * K + c]));
    }
    __syncthreads();
    if (w == 0) {
        float p = 0.f;
        for (int c = lane; c < K; c += 64) p += sk[c] * sq[c];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
        if (lane == 0) skq = p;
    }

    float4 rk = make_float4(0.f, 0.f, 0.f, 0.f), rq = rk;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + i * RG;
        const float a = sa[r], kr = sk[r], qr = sq[r];
        s[i].x *= a; s[i].y *= a; s[i].z *= a; s[i].w *= a;
        rk.x += kr * s[i].x; rk.y += kr * s[i].y; rk.z += kr * s[i].z; rk.w += kr * s[i].w;
        rq.x += qr * s[i].x; rq.y += qr * s[i].y; rq.z += qr * s[i].z; rq.w += qr * s[i].w;
    }
    // Lanes of one wave holding the same columns differ by multiples of CG.
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
        rk.x += __shfl_xor(rk.x, off); rk.y += __shfl_xor(rk.y, off);
        rk.z += __shfl_xor(rk.z, off); rk.w += __shfl_xor(rk.w, off);
        rq.x += __shfl_xor(rq.x, off); rq.y += __shfl_xor(rq.y, off);
        rq.z += __shfl_xor(rq.z, off); rq.w += __shfl_xor(rq.w, off);
    }
    if (lane < CG) {
        red[w][lane][0] = rk;
        red[w][lane][1] = rq;
    }
    __syncthreads();
    float4 RK = red[0][cg][0], RQ = red[0][cg][1];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) {
        const float4 a = red[ww][cg][0], b = red[ww][cg][1];
        RK.x += a.x; RK.y += a.y; RK.z += a.z; RK.w += a.w;
        RQ.x += b.x; RQ.y += b.y; RQ.z += b.z; RQ.w += b.w;
    }
    const float b = to_f32(beta[unit]);
    const TIn *vp = v + unit * V + 4 * cg;
    float4 u;
    u.x = b * (to_f32(vp[0]) - RK.x);
    u.y = b * (to_f32(vp[1]) - RK.y);
    u.z = b * (to_f32(vp[2]) - RK.z);
    u.w = b * (to_f32(vp[3]) - RK.w);

    typedef float f4v __attribute__((ext_vector_type(4)));
    if (!PAGED || Sout) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + i * RG;
            const float kr = sk[r];
            const f4v x = {s[i].x + kr * u.x, s[i].y + kr * u.y, s[i].z + kr * u.z, s[i].w + kr * u.w};
            __builtin_nontemporal_store(x, reinterpret_cast<f4v *>(&Sout[r * CG + cg]));
        }
    }
    if (rg == 0) {
        const float kq = skq;
        TOut *op = o + unit * V + 4 * cg;
        op[0] = from_f32<TOut>(RQ.x + kq * u.x);
        op[1] = from_f32<TOut>(RQ.y + kq * u.y);
        op[2] = from_f32<TOut>(RQ.z + kq * u.z);
        op[3] = from_f32<TOut>(RQ.w + kq * u.w);
    }
}

// Slot arrays null: dense states [N, H, K, V] updated in place.
struct DecodeStates {
    float *state;
    const int32_t *slot_in, *slot_out;
    int pool_slots;
};

template <int K, int V, int NT, typename TIn, typename TOut>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, const DecodeStates &st, void *o, int units,
                                  int H, hipStream_t stream) {
    if (st.slot_in)
        hipLaunchKernelGGL((decode_step_kernel<K, V, NT, TIn, TOut, true>), dim3(units), dim3(NT),
                           0, stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                           static_cast<const TIn *>(v), static_cast<const TIn *>(g),
                           static_cast<const TIn *>(beta), st.state, st.slot_in, st.slot_out,
                           st.pool_slots, H, static_cast<TOut *>(o));
    else
        hipLaunchKernelGGL((decode_step_kernel<K, V, NT, TIn, TOut, false>), dim3(units), dim3(NT),
                           0, stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                           static_cast<const TIn *>(v), static_cast<const TIn *>(g),
                           static_cast<const TIn *>(beta), st.state, nullptr, nullptr, 0, H,
                           static_cast<TOut *>(o));
    return hipGetLastError();
}

template <int K, int V, int NT>
static hipError_t launch_decode_kv(const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, const DecodeStates &st, void *o, int units,
                                   int H, bool in_bf16, bool out_bf16, hipStream_t stream) {
    if (in_bf16) {
        return out_bf16 ? launch_decode_t<K, V, NT, bf16_t, bf16_t>(q, k, v, g, beta, st, o, units, H, stream)
                        : launch_decode_t<K, V, NT, bf16_t, float>(q, k, v, g, beta, st, o, units, H, stream);
    }
    return out_bf16 ? launch_decode_t<K, V, NT, float, bf16_t>(q, k, v, g, beta, st, o, units, H, stream)
                    : launch_decode_t<K, V, NT, float, float>(q, k, v, g, beta, st, o, units, H, stream);
}

// Internal launcher: shapes were validated by the caller.  slot_in / slot_out
// null: state is a dense [N, H, K, V] array updated in place; else state is a
// pool of pool_slots slots.
hipError_t launch_decode(const void *q, const void *k, const void *v, const void *g,
                         const void *beta, float *state, const int32_t *slot_in,
                         const int32_t *slot_out, int pool_slots, void *o, int N, int H, int K,
                         int V, bool in_bf16, bool out_bf16, hipStream_t stream) {
    const int units = N * H;
    if (units == 0) return hipSuccess;
    const DecodeStates st{state, slot_in, slot_out, pool_slots};
    if (K == 128 && V == 128)
        return launch_decode_kv<128, 128, 256>(q, k, v, g, beta, st, o, units, H, in_bf16, out_bf16, stream);
    if (K == 32 && V == 32)
        return launch_decode_kv<32, 32, 64>(q, k, v, g, beta, st, o, units, H, in_bf16, out_bf16, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
