// chunk_valu.hip -- chunked KDA forward pass in fp32 on the vector ALUs (gfx950).
//
// Serves fp32 inputs, whose tolerance leaves no room for half-precision
// operands.  Every decay factor exp(G_r - G_s) is evaluated exactly, so any
// g <= 0 is accepted; speed is secondary here (the bf16 path is chunk_mfma.hip).
//
// Chunked form of the recurrence of "Kimi K3: Open Frontier Intelligence and
// Implementation Framework", section "Hybrid Attention Mechanism" (delta rule
// with a channel-wise forget gate).  For one chunk of L tokens starting from
// state S, with G_r the inclusive running sum of g inside the chunk:
//
//   A_rs = beta_r sum_c k_rc k_sc exp(G_rc - G_sc)      (s < r, strictly lower)
//   (I + A) U = Diag(beta) (V - (K * exp(G)) S)         (forward substitution)
//   P_rs = sum_c q_rc k_sc exp(G_rc - G_sc)             (s <= r)
//   O    = (Q * exp(G)) S + P U
//   S   <- Diag(exp(G_L)) S + (K * exp(G_L - G))^T U
//
// U holds the per-token pseudo-values u_r = beta_r (v_r - (Diag(alpha_r) S_{r-1})^T k_r),
// so the chunk reproduces the token-by-token recurrence exactly up to rounding.
//
// One workgroup handles one (sequence, head, V-column tile); the tile of S
// stays in LDS for the whole sequence.  Columns of the state evolve
// independently, so V-tiles need no communication.
#include "kda_common.hpp"
#include "prologue.hpp"
#include "state_io.hpp"

namespace kda {

template <int K, int V, int C, int VT, int NT>
struct ValuSmem {
    static constexpr int floats = 3 * C * K + 2 * C * C + 2 * C * VT + K * VT + C;
    static constexpr size_t bytes = sizeof(float) * floats;
};

// PRO: the input prologue (prologue.hpp) applies, as pro.flags selects.
template <int K, int V, int C, int VT, int NT, typename TIn, typename TOut, bool PRO>
__global__ __launch_bounds__(NT) void chunk_valu_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const TIn *__restrict__ g, const TIn *__restrict__ beta, StateIO io, Prologue pro,
    TOut *__restrict__ o, const int32_t *__restrict__ cu, int fixedT, int H, int totalT) {
    const bool gate_logit = PRO && (pro.flags & PRO_GATE_LOGIT);
    const bool beta_logit = PRO && (pro.flags & PRO_BETA_LOGIT);
    const bool norm_qk = PRO && (pro.flags & PRO_NORM_QK);
    extern __shared__ float smem[];
    float *sQ = smem;            // [C][K]
    float *sK = sQ + C * K;      // [C][K]
    float *sG = sK + C * K;      // [C][K]  running sum of g inside the chunk
    float *sA = sG + C * K;      // [C][C]
    float *sP = sA + C * C;      // [C][C]
    float *sV = sP + C * C;      // [C][VT]
    float *sU = sV + C * VT;     // [C][VT]
    float *sS = sU + C * VT;     // [K][VT] state tile
    float *sB = sS + K * VT;     // [C]

    const int t = threadIdx.x;
    const int vt = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    // element (r, c) of this tile of a state is at [r * V + vt * VT + c]
    const float *s0p = state_in(io, n, h, H, K * V);
    SnapCursor snap;
    snap.init(io, n);

    for (int i = t; i < K * VT; i += NT) {
        const int r = i / VT, c = i % VT;
        sS[i] = s0p ? s0p[r * V + vt * VT + c] : 0.f;
    }

    for (int c0 = bos; c0 < eos; c0 += C) {
        const int L = min(C, eos - c0);
        __syncthreads();
        for (int i = t; i < C * K; i += NT) {
            const int r = i / K, c = i % K;
            const bool in = r < L;
            const size_t off = ((size_t)(c0 + r) * H + h) * K + c;
            sQ[i] = in ? to_f32(q[off]) : 0.f;
            sK[i] = in ? to_f32(k[off]) : 0.f;
            float gv = in ? to_f32(g[off]) : 0.f;
            if (gate_logit && in) gv = gate_from_logit(gv, pro.glb);
            sG[i] = gv;
        }
        for (int i = t; i < C * VT; i += NT) {
            const int r = i / VT, c = i % VT;
            sV[i] = r < L ? to_f32(v[((size_t)(c0 + r) * H + h) * V + (size_t)vt * VT + c]) : 0.f;
        }
        for (int r = t; r < C; r += NT) {
            float b = r < L ? to_f32(beta[(size_t)(c0 + r) * H + h]) : 0.f;
            if (beta_logit && r < L) b = sigmoid_f(b);
            sB[r] = b;
        }
        __syncthreads();

        // Prologue: unit-norm rows of Q and K (padding rows stay zero).
        if (norm_qk) {
            for (int r = t; r < C; r += NT) {
                float sq = 0.f, sk = 0.f;
                for (int c = 0; c < K; ++c) {
                    sq += sQ[r * K + c] * sQ[r * K + c];
                    sk += sK[r * K + c] * sK[r * K + c];
                }
                const float iq = inv_norm(sq, pro.eps), ik = inv_norm(sk, pro.eps);
                for (int c = 0; c < K; ++c) {
                    sQ[r * K + c] *= iq;
                    sK[r * K + c] *= ik;
                }
            }
        }

        // Running sum of the log-decay per key channel (padding rows add 0).
        for (int c = t; c < K; c += NT) {
            float acc = 0.f;
            for (int r = 0; r < C; ++r) {
                acc += sG[r * K + c];
                sG[r * K + c] = acc;
            }
        }
        __syncthreads();

        // A (strictly lower, beta-scaled rows) and P (lower with diagonal).
        for (int i = t; i < C * C; i += NT) {
            const int r = i / C, s = i % C;
            float a = 0.f, p = 0.f;
            if (s <= r) {
                for (int c = 0; c < K; ++c) {
                    const float ks = sK[s * K + c] * fast_exp(sG[r * K + c] - sG[s * K + c]);
                    a += sK[r * K + c] * ks;
                    p += sQ[r * K + c] * ks;
                }
            }
            sA[i] = s < r ? sB[r] * a : 0.f;
            sP[i] = p;
        }
        // Right-hand side beta (V - (K * exp(G)) S).
        for (int i = t; i < C * VT; i += NT) {
            const int r = i / VT, j = i % VT;
            float x = 0.f;
            for (int c = 0; c < K; ++c) x += sK[r * K + c] * fast_exp(sG[r * K + c]) * sS[c * VT + j];
            sU[i] = sB[r] * (sV[i] - x);
        }
        __syncthreads();

        // Forward substitution (I + A) U = RHS, one row at a time.
        for (int r = 1; r < L; ++r) {
            for (int j = t; j < VT; j += NT) {
                float acc = sU[r * VT + j];
                for (int s = 0; s < r; ++s) acc -= sA[r * C + s] * sU[s * VT + j];
                sU[r * VT + j] = acc;
            }
            __syncthreads();
        }

        // Output O = (Q * exp(G)) S + P U.
        for (int i = t; i < C * VT; i += NT) {
            const int r = i / VT, j = i % VT;
            if (r < L) {
                float acc = 0.f;
                for (int c = 0; c < K; ++c) acc += sQ[r * K + c] * fast_exp(sG[r * K + c]) * sS[c * VT + j];
                for (int s = 0; s <= r; ++s) acc += sP[r * C + s] * sU[s * VT + j];
                o[((size_t)(c0 + r) * H + h) * V + (size_t)vt * VT + j] = from_f32<TOut>(acc);
            }
        }
        __syncthreads();

        // State advance to the end of the chunk.
        for (int i = t; i < K * VT; i += NT) {
            const int c = i / VT, j = i % VT;
            const float gl = sG[(L - 1) * K + c];
            float acc = fast_exp(gl) * sS[i];
            for (int s = 0; s < L; ++s) acc += sK[s * K + c] * fast_exp(gl - sG[s * K + c]) * sU[s * VT + j];
            sS[i] = acc;
        }
        // prefix snapshot when the state now covers a boundary (each thread
        // copies the elements it has just advanced)
        if (snap.due(c0 - bos + L)) {
            float *sp = snap.dest(io, h, H, K * V);
            snap.advance(io);
            if (sp) {
                for (int i = t; i < K * VT; i += NT) sp[(i / VT) * V + vt * VT + i % VT] = sS[i];
            }
        }
    }
    __syncthreads();
    float *sTp = state_out(io, n, h, H, K * V);
    if (sTp) {
        for (int i = t; i < K * VT; i += NT) {
            const int r = i / VT, c = i % VT;
            sTp[r * V + vt * VT + c] = sS[i];
        }
    }
}

template <int K, int V, int C, int VT, typename TIn, typename TOut, bool PRO>
static hipError_t launch_valu_t(const void *q, const void *k, const void *v, const void *g,
                                const void *beta, const StateIO &io, const Prologue &pro, void *o,
                                const int32_t *cu, int N, int fixedT, int totalT, int H,
                                hipStream_t stream) {
    constexpr int NT = 256;
    using SM = ValuSmem<K, V, C, VT, NT>;
    auto kern = chunk_valu_kernel<K, V, C, VT, NT, TIn, TOut, PRO>;
    if (SM::bytes > 64 * 1024) {
        static std::atomic<uint64_t> lds_set{0};
        hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(kern),
                                          static_cast<int>(SM::bytes), lds_set);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(V / VT, H, N), dim3(NT), SM::bytes, stream,
                       static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                       static_cast<const TIn *>(v), static_cast<const TIn *>(g),
                       static_cast<const TIn *>(beta), io, pro, static_cast<TOut *>(o), cu, fixedT,
                       H, totalT);
    return hipGetLastError();
}

template <int K, int V, int C, int VT, bool PRO>
static hipError_t launch_valu_pro(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, const StateIO &io, const Prologue &pro,
                                  void *o, const int32_t *cu, int N, int fixedT, int totalT, int H,
                                  bool in_bf16, bool out_bf16, hipStream_t stream) {
    if (in_bf16)
        return out_bf16 ? launch_valu_t<K, V, C, VT, bf16_t, bf16_t, PRO>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, stream)
                        : launch_valu_t<K, V, C, VT, bf16_t, float, PRO>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, stream);
    return out_bf16 ? launch_valu_t<K, V, C, VT, float, bf16_t, PRO>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, stream)
                    : launch_valu_t<K, V, C, VT, float, float, PRO>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, stream);
}

template <int K, int V, int C, int VT>
static hipError_t launch_valu_kvc(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, const StateIO &io, const Prologue &pro,
                                  void *o, const int32_t *cu, int N, int fixedT, int totalT, int H,
                                  bool in_bf16, bool out_bf16, hipStream_t stream) {
    if (pro.flags)
        return launch_valu_pro<K, V, C, VT, true>(q, k, v, g, beta, io, pro, o, cu, N, fixedT,
                                                  totalT, H, in_bf16, out_bf16, stream);
    return launch_valu_pro<K, V, C, VT, false>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT,
                                               H, in_bf16, out_bf16, stream);
}

// Internal launcher.  cu == nullptr means fixed-length sequences of fixedT tokens.
hipError_t launch_chunk_valu(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, const StateIO &io, const Prologue &pro, void *o,
                             const int32_t *cu, int N, int fixedT, int totalT, int H, int K, int V,
                             int C, bool in_bf16, bool out_bf16, hipStream_t stream) {
    if (N == 0 || H == 0) return hipSuccess;
    if (K == 32 && V == 32 && C == 16)
        return launch_valu_kvc<32, 32, 16, 32>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, in_bf16, out_bf16, stream);
    if (K == 128 && V == 128 && C == 64)
        return launch_valu_kvc<128, 128, 64, 16>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, in_bf16, out_bf16, stream);
    return hipErrorInvalidValue;
}

size_t chunk_valu_smem_bytes(int K, int V, int C) {
    if (K == 32 && V == 32 && C == 16) return ValuSmem<32, 32, 16, 32, 256>::bytes;
    if (K == 128 && V == 128 && C == 64) return ValuSmem<128, 128, 64, 16, 256>::bytes;
    return 0;
}

}  // namespace kda
