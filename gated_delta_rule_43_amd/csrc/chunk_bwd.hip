// chunk_bwd.hip -- chunked KDA backward pass on gfx950 (fp32, vector ALUs).
//
// Gradients of the recurrence of "Kimi K3: Open Frontier Intelligence and
// Implementation Framework", section "Hybrid Attention Mechanism" (delta rule
// with a channel-wise forget gate), for the loss sum(do * o) + sum(dsT * S_T).
//
// Per chunk of L tokens (G the running sum of g inside the chunk, G_m its
// value at the middle row m, E = exp(G - G_m), S the state at the chunk's
// start, S' = Diag(exp(G_m)) S, F = Diag(exp(G_{L-1} - G_m))):
//   Kp = K * E,  Km = K / E,  Qp = Q * E,  Gk = strict_lower(Kp Km^T),
//   P = lower(Qp Km^T),  T = (I + Diag(beta) Gk)^-1,
//   R = V - Kp S',  U = T Diag(beta) R,  O = Qp S' + P U,  S_end = F (S' + Km^T U).
// Reverse mode through these products, with dS_end the gradient at the
// chunk's end and X = F dS_end:
//   dU = Km X + P^T dO,   dY = T^T dU,   dA = -strict_lower(dY U^T),   dP = lower(dO U^T)
//   dS' = X + Qp^T dO - Kp^T Diag(beta) dY,   dS_start = Diag(exp(G_m)) dS'
//   dV = Diag(beta) dY,   dbeta = rowsum(R * dY) + rowsum(Gk * dA)
//   dKp = -Diag(beta) dY S'^T + Diag(beta) dA Km,   dQp = dO S'^T + dP Km
//   dKm = U X^T + (Diag(beta) dA)^T Kp + dP^T Qp
//   dK = dKp E + dKm / E,   dQ = dQp E
//   D = dKp * Kp - dKm * Km + dQp * Qp  (+ rowsum(S_end * dS_end) on row L-1),
//   dg = reverse running sum of D over the chunk's rows.
// G_m cancels from the forward result, so its own gradient is zero and it is
// treated as a constant.
//
// Five launches:
//   bwd_prep_kernel    (chunk, head), all chunks at once: Kp, Km, Qp, E, Gk,
//                      P, T, beta, F, exp(G_m) into the chunk's record;
//   bwd_trans_kernel   (chunk, head): the chunk's state transition
//                      S_end = MM S_start + NN and the adjoint's constant NB;
//   bwd_states_kernel  (sequence, head, value tile): the forward state chain,
//                      one [K][K] product per chunk, leaving every chunk's
//                      start state in the workspace;
//   bwd_dstate_kernel  (sequence, head, value tile): the reverse chain
//                      dS_start = MM^T dS_end + NB, chunk after chunk from
//                      the last, and ds0;
//   bwd_grads_kernel   (chunk, head): every input gradient of the chunk.
// The state chains are column-separable (value tiles need no communication);
// the gradients of q, k, g and beta sum over all value columns, so the last
// pass loops over the columns in sub-tiles and accumulates in registers.
#include "kda_common.hpp"

namespace kda {
namespace {

constexpr int BNT = 256;  // threads per workgroup of the state-chain kernels
constexpr int PNT = 512;  // threads per workgroup of the record and transition kernels (one
                          // workgroup per CU by LDS; eight waves hide LDS latency)

// Record of one (chunk, head), in floats.  MM, NN, NB: the chunk's state
// transition S_end = MM S_start + NN and its adjoint dS_start = MM^T dS_end + NB.
template <int K, int V, int C>
struct BwdRec {
    static constexpr size_t KP = 0, KM = KP + C * K, QP = KM + C * K, EE = QP + C * K;
    static constexpr size_t GK = EE + C * K, PP = GK + C * C, TT = PP + C * C;
    static constexpr size_t BETA = TT + C * C, FF = BETA + C, EGM = FF + K;
    static constexpr size_t MM = EGM + K, NN = MM + K * K, NB = NN + K * V;
    static constexpr size_t floats = NB + K * V;
};

__device__ __forceinline__ int chunks_of(const int32_t *cu, int n, int fixedT, int totalT, int C) {
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    return (eos - bos + C - 1) / C;
}

// Index of sequence n's first chunk in the packed chunk list (all NT threads;
// red holds NT ints).
template <int NT>
__device__ int first_chunk(const int32_t *cu, int n, int fixedT, int totalT, int C, int *red) {
    if (!cu) return n * ((fixedT + C - 1) / C);
    int s = 0;
    for (int m = threadIdx.x; m < n; m += NT) s += chunks_of(cu, m, fixedT, totalT, C);
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = NT / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    const int r = red[0];
    __syncthreads();
    return r;
}

// Sequence and local chunk of packed chunk gc; n = -1 past the last chunk
// (all NT threads; red holds NT ints).
template <int NT>
__device__ void locate_chunk(const int32_t *cu, int N, int fixedT, int totalT, int C, int gc,
                             int &n, int &i, int *red) {
    if (!cu) {
        const int cps = (fixedT + C - 1) / C;
        n = cps > 0 ? gc / cps : -1;
        i = cps > 0 ? gc % cps : 0;
        if (n >= N) n = -1;
        return;
    }
    // contiguous ranges of sequences per thread, an exclusive scan of their
    // chunk counts, then the owning thread walks its range
    const int t = threadIdx.x;
    const int lo = (int)((long long)N * t / NT), hi = (int)((long long)N * (t + 1) / NT);
    int cnt = 0;
    for (int m = lo; m < hi; ++m) cnt += chunks_of(cu, m, fixedT, totalT, C);
    red[t] = cnt;
    __syncthreads();
    for (int d = 1; d < NT; d <<= 1) {
        const int x = t >= d ? red[t - d] : 0;
        __syncthreads();
        red[t] += x;
        __syncthreads();
    }
    const int incl = red[t], excl = incl - cnt;
    __syncthreads();
    if (t == 0) {
        red[0] = -1;
        red[1] = 0;
    }
    __syncthreads();
    if (gc >= excl && gc < incl) {
        int base = excl;
        for (int m = lo; m < hi; ++m) {
            const int c = chunks_of(cu, m, fixedT, totalT, C);
            if (gc < base + c) {
                red[0] = m;
                red[1] = gc - base;
                break;
            }
            base += c;
        }
    }
    __syncthreads();
    n = red[0];
    i = red[1];
    __syncthreads();
}

// A [K][K] fp32 matrix as float4 pieces, MQ per thread, held in registers so
// that the next chunk's copy is in flight while this chunk's is used.
template <int K, int NT>
struct MatPrefetch {
    static constexpr int MQ = K * K / 4 / NT;
    static_assert(K * K % (4 * NT) == 0, "matrix must split evenly");
    float4 m[MQ];
    __device__ __forceinline__ void load(const float *src) {
#pragma unroll
        for (int i = 0; i < MQ; ++i)
            m[i] = reinterpret_cast<const float4 *>(src)[threadIdx.x + NT * i];
    }
    // to LDS with row pitch P (one 16-byte store when P keeps rows aligned)
    template <int P>
    __device__ __forceinline__ void store(float *dst) const {
#pragma unroll
        for (int i = 0; i < MQ; ++i) {
            const int e = 4 * (threadIdx.x + NT * i), r = e / K, c = e % K;
            float *d = dst + r * P + c;
            if constexpr (P % 4 == 0) {
                *reinterpret_cast<float4 *>(d) = m[i];
            } else {
                d[0] = m[i].x;
                d[1] = m[i].y;
                d[2] = m[i].z;
                d[3] = m[i].w;
            }
        }
    }
};

// Copies a contiguous [R][D] fp32 block to LDS with row pitch P, float4 loads
// (all of a thread's loads issued before its stores).
template <int R, int D, int P, int NT>
__device__ __forceinline__ void rows_to_lds(float *dst, const float *src) {
    constexpr int Q = R * D / 4, PER = (Q + NT - 1) / NT;
    static_assert(D % 4 == 0, "rows must split into float4");
    float4 x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int qi = threadIdx.x + NT * i;
        if (qi < Q) x[i] = reinterpret_cast<const float4 *>(src)[qi];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int qi = threadIdx.x + NT * i;
        if (qi < Q) {
            const int e = 4 * qi, r = e / D, c = e % D;
            float *d = dst + r * P + c;
            d[0] = x[i].x;
            d[1] = x[i].y;
            d[2] = x[i].z;
            d[3] = x[i].w;
        }
    }
}

// ------------------------------------------------------------------ pass 0
template <int K, int V, int C, typename TIn>
__global__ __launch_bounds__(PNT) void bwd_prep_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ g,
    const TIn *__restrict__ beta, const int32_t *__restrict__ cu, int N, int fixedT, int totalT,
    int H, float *__restrict__ ws) {
    using Rc = BwdRec<K, V, C>;
    extern __shared__ float smem[];
    constexpr int PK = K + 1;     // row pitch: a wave reading one column hits distinct banks
    float *sKp = smem;             // [C][PK]
    float *sKm = sKp + C * PK;     // [C][PK]
    float *sQp = sKm + C * PK;     // [C][PK]
    float *sX = sQp + C * PK;      // [C][K]: G, later Gk [C][C] and T [C][C]
    float *sB = sX + C * K;        // [C]
    float *sGm = sB + C;           // [K]
    int *red = reinterpret_cast<int *>(sGm + K);  // [PNT]
    static_assert(2 * C * C <= C * K, "Gk and T must fit the G buffer");

    const int gc = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    int n, ci;
    locate_chunk<PNT>(cu, N, fixedT, totalT, C, gc, n, ci, red);
    if (n < 0) return;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + ci * C, L = min(C, eos - c0);
    const int m = min(C / 2 - 1, L - 1);  // reference row
    float *rec = ws + ((size_t)gc * H + h) * Rc::floats;

    for (int e = t; e < C * K; e += PNT) {
        const int r = e / K, c = e % K;
        sX[e] = r < L ? to_f32(g[((size_t)(c0 + r) * H + h) * K + c]) : 0.f;
    }
    for (int r = t; r < C; r += PNT) sB[r] = r < L ? to_f32(beta[(size_t)(c0 + r) * H + h]) : 0.f;
    __syncthreads();
    for (int c = t; c < K; c += PNT) {  // running sum down each channel
        float acc = 0.f;
        for (int r = 0; r < C; ++r) {
            acc += sX[r * K + c];
            sX[r * K + c] = acc;
        }
    }
    __syncthreads();
    for (int c = t; c < K; c += PNT) {
        const float gm = sX[m * K + c];
        sGm[c] = gm;
        rec[Rc::FF + c] = fast_exp(sX[(L - 1) * K + c] - gm);
        rec[Rc::EGM + c] = fast_exp(gm);
    }
    for (int r = t; r < C; r += PNT) rec[Rc::BETA + r] = sB[r];
    __syncthreads();
    for (int e = t; e < C * K; e += PNT) {
        const int r = e / K, c = e % K;
        const float d = sX[e] - sGm[c];
        const float ep = fast_exp(d), em = fast_exp(-d);
        const size_t off = ((size_t)(c0 + r) * H + h) * K + c;
        const float kv = r < L ? to_f32(k[off]) : 0.f, qv = r < L ? to_f32(q[off]) : 0.f;
        sKp[r * PK + c] = kv * ep;
        sKm[r * PK + c] = kv * em;
        sQp[r * PK + c] = qv * ep;
        rec[Rc::KP + e] = kv * ep;
        rec[Rc::KM + e] = kv * em;
        rec[Rc::QP + e] = qv * ep;
        rec[Rc::EE + e] = ep;
    }
    __syncthreads();
    // Gram blocks: Gk strictly lower, P lower with the diagonal
    float *sGk = sX, *sT = sX + C * C;
    for (int e = t; e < C * C; e += PNT) {
        const int r = e / C, s = e % C;
        float a = 0.f, p = 0.f;
        if (s <= r) {
            for (int c = 0; c < K; ++c) {
                const float km = sKm[s * PK + c];
                a += sKp[r * PK + c] * km;
                p += sQp[r * PK + c] * km;
            }
        }
        const float gk = s < r ? a : 0.f;
        sGk[e] = gk;
        rec[Rc::GK + e] = gk;
        rec[Rc::PP + e] = p;
    }
    __syncthreads();
    // T = (I + Diag(beta) Gk)^-1, row by row: T_r = e_r - beta_r sum_{s<r} Gk_rs T_s
    for (int e = t; e < C * C; e += PNT) sT[e] = (e / C == e % C) ? 1.f : 0.f;
    __syncthreads();
    for (int r = 1; r < C; ++r) {
        for (int col = t; col < r; col += PNT) {
            float acc = 0.f;
            for (int s = col; s < r; ++s) acc += sGk[r * C + s] * sT[s * C + col];
            sT[r * C + col] = -sB[r] * acc;
        }
        __syncthreads();
    }
    for (int e = t; e < C * C; e += PNT) rec[Rc::TT + e] = sT[e];
}

// -------------------------------------------------------------- pass 0b
// The chunk's transition: with W = T Diag(beta) Kp, U~ = T Diag(beta) V and
// Q^ = Qp - P W (so that U = U~ - W S' and O = Q^ S' + P U~),
//   MM = F (I - Km^T W) Diag(exp(G_m)),   NN = F Km^T U~,
//   NB = Diag(exp(G_m)) Q^T dO            (dS_start = MM^T dS_end + NB).
// Three [C][D+1] buffers are reused in turn (pitch D+1: rows fall on
// different banks when a wave reads one column).
template <int K, int V, int C, typename TIn>
__global__ __launch_bounds__(PNT) void bwd_trans_kernel(
    const TIn *__restrict__ v, const float *__restrict__ dout, const int32_t *__restrict__ cu,
    int N, int fixedT, int totalT, int H, float *__restrict__ recs) {
    using Rc = BwdRec<K, V, C>;
    static_assert(K == V, "one buffer pitch for key and value tiles");
    constexpr int PD = K + 1, PC = C + 1, RB = 4;  // RB output rows per thread
    extern __shared__ float smem[];
    float *b0 = smem, *b1 = b0 + C * PD, *b2 = b1 + C * PD;
    float *sT = b2 + C * PD, *sP = sT + C * PC;
    float *sB = sP + C * PC, *sF = sB + C, *sE = sF + K;
    int *red = reinterpret_cast<int *>(sE + K);

    const int gc = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    int n, ci;
    locate_chunk<PNT>(cu, N, fixedT, totalT, C, gc, n, ci, red);
    if (n < 0) return;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + ci * C, L = min(C, eos - c0);
    float *rec = recs + ((size_t)gc * H + h) * Rc::floats;

    auto load_rows = [&](float *dst, size_t src_off) {
        rows_to_lds<C, K, PD, PNT>(dst, rec + src_off);
    };
    // out[r][j] = sum_{s<=r} T[r][s] beta_s in[s][j]   (r < C, j < K)
    auto tri_apply = [&](float *out, const float *in) {
        for (int e = t; e < C * K; e += PNT) {
            const int r = e / K, j = e % K;
            float acc = 0.f;
            for (int s2 = 0; s2 <= r; ++s2) acc += sT[r * PC + s2] * sB[s2] * in[s2 * PD + j];
            out[r * PD + j] = acc;
        }
    };
    // out[c][j] = sum_r a[r][c] b[r][j] for RB consecutive c per thread
    auto at_b = [&](const float *a, const float *b, auto &&store) {
        for (int e = t; e < (K / RB) * K; e += PNT) {
            const int cb = (e / K) * RB, j = e % K;
            float acc[RB] = {};
            for (int r = 0; r < C; ++r) {
                const float bv = b[r * PD + j];
#pragma unroll
                for (int i = 0; i < RB; ++i) acc[i] += a[r * PD + cb + i] * bv;
            }
#pragma unroll
            for (int i = 0; i < RB; ++i) store(cb + i, j, acc[i]);
        }
    };

    for (int e = t; e < C * C; e += PNT) {
        sT[(e / C) * PC + e % C] = rec[Rc::TT + e];
        sP[(e / C) * PC + e % C] = rec[Rc::PP + e];
    }
    for (int r = t; r < C; r += PNT) sB[r] = rec[Rc::BETA + r];
    for (int c = t; c < K; c += PNT) {
        sF[c] = rec[Rc::FF + c];
        sE[c] = rec[Rc::EGM + c];
    }
    load_rows(b0, Rc::KP);
    __syncthreads();
    tri_apply(b1, b0);  // W
    __syncthreads();
    load_rows(b0, Rc::QP);
    __syncthreads();
    for (int e = t; e < C * K; e += PNT) {  // Q^ = Qp - P W
        const int r = e / K, j = e % K;
        float acc = b0[r * PD + j];
        for (int s2 = 0; s2 <= r; ++s2) acc -= sP[r * PC + s2] * b1[s2 * PD + j];
        b2[r * PD + j] = acc;
    }
    __syncthreads();
    for (int e = t; e < C * V; e += PNT) {
        const int r = e / V, j = e % V;
        b0[r * PD + j] = r < L ? dout[((size_t)(c0 + r) * H + h) * V + j] : 0.f;
    }
    __syncthreads();
    at_b(b2, b0, [&](int c, int j, float x) { rec[Rc::NB + (size_t)c * V + j] = sE[c] * x; });
    __syncthreads();
    load_rows(b0, Rc::KM);
    __syncthreads();
    at_b(b0, b1, [&](int c, int j, float x) {
        rec[Rc::MM + (size_t)c * K + j] = sF[c] * ((c == j ? 1.f : 0.f) - x) * sE[j];
    });
    __syncthreads();
    for (int e = t; e < C * V; e += PNT) {
        const int r = e / V, j = e % V;
        b1[r * PD + j] = r < L ? to_f32(v[((size_t)(c0 + r) * H + h) * V + j]) : 0.f;
    }
    __syncthreads();
    tri_apply(b2, b1);  // U~
    __syncthreads();
    at_b(b0, b2, [&](int c, int j, float x) { rec[Rc::NN + (size_t)c * V + j] = sF[c] * x; });
}

// ------------------------------------------------------------------ pass 1
// Forward state chain of one value tile, S <- MM S + NN chunk after chunk:
// writes the start state of every chunk of the sequence to Sst[chunk][h].
// RB rows of one column per thread; MM staged with row pitch K + 1 (the four
// row blocks a wave reads fall on different banks; unpadded rows with
// 16-byte reads measured 2.3x slower).
template <int K, int V, int C, int VT>
__global__ __launch_bounds__(BNT) void bwd_states_kernel(
    const float *__restrict__ s0, const int32_t *__restrict__ cu, int fixedT, int totalT, int H,
    const float *__restrict__ recs, float *__restrict__ Sst) {
    using Rc = BwdRec<K, V, C>;
    constexpr int PK = K + 1, RB = K * VT / BNT;
    static_assert(K * VT % BNT == 0 && BNT % VT == 0, "tile must cover the workgroup");
    extern __shared__ float smem[];
    float *sM = smem;            // [K][K + 1]
    float *sS = sM + K * PK;     // [K][VT]
    int *red = reinterpret_cast<int *>(sS + K * VT);

    const int vt = blockIdx.x, h = blockIdx.y, n = blockIdx.z, t = threadIdx.x;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int nch = (eos - bos + C - 1) / C;
    const int first = first_chunk<BNT>(cu, n, fixedT, totalT, C, red);
    const int j = t % VT, cb = (t / VT) * RB;  // this thread's column and first row
    float S[RB], nn[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
        S[i] = s0 ? s0[((size_t)n * H + h) * K * V + (size_t)(cb + i) * V + vt * VT + j] : 0.f;
    MatPrefetch<K, BNT> pm;
    auto fetch = [&](int ci) {  // chunk ci's MM and this thread's NN entries
        const float *rec = recs + ((size_t)(first + ci) * H + h) * Rc::floats;
        pm.load(rec + Rc::MM);
#pragma unroll
        for (int i = 0; i < RB; ++i) nn[i] = rec[Rc::NN + (size_t)(cb + i) * V + vt * VT + j];
    };
    if (nch > 0) fetch(0);
    for (int ci = 0; ci < nch; ++ci) {
        const int gc = first + ci;
        float *dst = Sst + ((size_t)gc * H + h) * K * V + vt * VT + j;
#pragma unroll
        for (int i = 0; i < RB; ++i) dst[(size_t)(cb + i) * V] = S[i];
        __syncthreads();
        pm.template store<PK>(sM);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            sS[(cb + i) * VT + j] = S[i];
            S[i] = nn[i];
        }
        __syncthreads();
        if (ci + 1 < nch) fetch(ci + 1);
        for (int c2 = 0; c2 < K; ++c2) {
            const float sv = sS[c2 * VT + j];
#pragma unroll
            for (int i = 0; i < RB; ++i) S[i] += sM[(cb + i) * PK + c2] * sv;
        }
    }
}

// ------------------------------------------------------------------ pass 2
// Reverse chain of the state gradient for one value tile, dS <- MM^T dS + NB
// chunk after chunk from the last: writes the gradient at the end of every
// chunk to dSe[chunk][h] and the gradient of S_0 to ds0.
template <int K, int V, int C, int VT>
__global__ __launch_bounds__(BNT) void bwd_dstate_kernel(
    const float *__restrict__ dsT, float *__restrict__ ds0, const int32_t *__restrict__ cu,
    int fixedT, int totalT, int H, const float *__restrict__ recs, float *__restrict__ dSe) {
    using Rc = BwdRec<K, V, C>;
    constexpr int PK = K + 1, RB = K * VT / BNT;
    static_assert(K * VT % BNT == 0 && BNT % VT == 0, "tile must cover the workgroup");
    extern __shared__ float smem[];
    float *sM = smem;            // [K][K + 1]
    float *sS = sM + K * PK;     // [K][VT]
    int *red = reinterpret_cast<int *>(sS + K * VT);

    const int vt = blockIdx.x, h = blockIdx.y, n = blockIdx.z, t = threadIdx.x;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int nch = (eos - bos + C - 1) / C;
    const int first = first_chunk<BNT>(cu, n, fixedT, totalT, C, red);
    const int j = t % VT, cb = (t / VT) * RB;
    const size_t sbase = ((size_t)n * H + h) * K * V + vt * VT + j;
    float D[RB], nb[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) D[i] = dsT ? dsT[sbase + (size_t)(cb + i) * V] : 0.f;
    MatPrefetch<K, BNT> pm;
    auto fetch = [&](int ci) {  // chunk ci's MM and this thread's NB entries
        const float *rec = recs + ((size_t)(first + ci) * H + h) * Rc::floats;
        pm.load(rec + Rc::MM);
#pragma unroll
        for (int i = 0; i < RB; ++i) nb[i] = rec[Rc::NB + (size_t)(cb + i) * V + vt * VT + j];
    };
    if (nch > 0) fetch(nch - 1);
    for (int ci = nch - 1; ci >= 0; --ci) {
        const int gc = first + ci;
        float *dst = dSe + ((size_t)gc * H + h) * K * V + vt * VT + j;
#pragma unroll
        for (int i = 0; i < RB; ++i) dst[(size_t)(cb + i) * V] = D[i];
        __syncthreads();
        pm.template store<PK>(sM);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            sS[(cb + i) * VT + j] = D[i];
            D[i] = nb[i];
        }
        __syncthreads();
        if (ci > 0) fetch(ci - 1);
        for (int c2 = 0; c2 < K; ++c2) {
            const float dv = sS[c2 * VT + j];
#pragma unroll
            for (int i = 0; i < RB; ++i) D[i] += sM[c2 * PK + cb + i] * dv;
        }
    }
    if (ds0)
#pragma unroll
        for (int i = 0; i < RB; ++i) ds0[sbase + (size_t)(cb + i) * V] = D[i];
}

// ------------------------------------------------------------------ pass 3
// GNT threads: 512 at d = 128 (the per-thread accumulators stay in registers),
// 256 at d = 32.
template <int K, int V, int C, int VS, int GNT, typename TIn>
__global__ __launch_bounds__(GNT) void bwd_grads_kernel(
    const TIn *__restrict__ v, const float *__restrict__ dout, const int32_t *__restrict__ cu,
    int N, int fixedT, int totalT, int H, const float *__restrict__ recs,
    const float *__restrict__ Sst, const float *__restrict__ dSe, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dg,
    float *__restrict__ dbeta) {
    using Rc = BwdRec<K, V, C>;
    // thread t owns elements t + GNT i of the [C][K] and [C][C] accumulators:
    // channel (or column) t % K (t % C) of rows t / K + RK i (t / C + RC i)
    constexpr int MCK = C * K / GNT, MCC = C * C / GNT, RK = GNT / K, RC = GNT / C;
    static_assert(C * K % GNT == 0 && C * C % GNT == 0 && GNT % K == 0 && GNT % C == 0,
                  "ownership must tile the workgroup");
    extern __shared__ float smem[];
    // row pitches PK = K + 1, PC = C + 1, PS = VS + 1: a wave reading one
    // column of a tile touches distinct banks
    constexpr int PK = K + 1, PC = C + 1, PS = VS + 1;
    float *sKp = smem;           // [C][PK]  (finally D)
    float *sKm = sKp + C * PK;   // [C][PK]
    float *sQp = sKm + C * PK;   // [C][PK]
    float *sT = sQp + C * PK;    // [C][PC]  (finally Gk)
    float *sP = sT + C * PC;     // [C][PC]  (finally dA)
    float *sS = sP + C * PC;     // [K][PS] S'
    float *sX = sS + K * PS;     // [K][PS] X = F dS_end
    float *sR = sX + K * PS;     // [C][VS] R = V - Kp S'
    float *sO = sR + C * VS;     // [C][VS] dO
    float *sU = sO + C * VS;     // [C][VS] U
    float *sDU = sU + C * VS;    // [C][VS] dU
    float *sDY = sDU + C * VS;   // [C][VS] dY
    float *sB = sDY + C * VS;    // [C]
    float *sF = sB + C;          // [K]
    float *sE = sF + K;          // [K]
    float *sH = sE + K;          // [K]   rowsum(S_end * dS_end)
    float *sDb = sH + K;         // [C]   dbeta
    int *red = reinterpret_cast<int *>(sDb + C);
    float *sDp = sS;             // [C][PC] dP, over the column buffers after the loop
    static_assert(C * PC <= 2 * K * PS + 5 * C * VS, "dP must fit the column buffers");

    const int gc = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    int n, ci;
    locate_chunk<GNT>(cu, N, fixedT, totalT, C, gc, n, ci, red);
    if (n < 0) return;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + ci * C, L = min(C, eos - c0);
    const float *rec = recs + ((size_t)gc * H + h) * Rc::floats;
    const float *S0c = Sst + ((size_t)gc * H + h) * K * V;
    const float *dSc = dSe + ((size_t)gc * H + h) * K * V;

    rows_to_lds<C, K, PK, GNT>(sKp, rec + Rc::KP);
    rows_to_lds<C, K, PK, GNT>(sKm, rec + Rc::KM);
    rows_to_lds<C, K, PK, GNT>(sQp, rec + Rc::QP);
    rows_to_lds<C, C, PC, GNT>(sT, rec + Rc::TT);
    rows_to_lds<C, C, PC, GNT>(sP, rec + Rc::PP);
    for (int r = t; r < C; r += GNT) {
        sB[r] = rec[Rc::BETA + r];
        sDb[r] = 0.f;
    }
    for (int c = t; c < K; c += GNT) {
        sF[c] = rec[Rc::FF + c];
        sE[c] = rec[Rc::EGM + c];
        sH[c] = 0.f;
    }

    // owned accumulators: element e = t + GNT * i of a [C][K] (or [C][C]) array
    float aQ[MCK], aKp[MCK], aKm[MCK], aA[MCC], aP[MCC];
#pragma unroll
    for (int i = 0; i < MCK; ++i) aQ[i] = aKp[i] = aKm[i] = 0.f;
#pragma unroll
    for (int i = 0; i < MCC; ++i) aA[i] = aP[i] = 0.f;

    for (int j0 = 0; j0 < V; j0 += VS) {
        __syncthreads();
        for (int e = t; e < K * VS; e += GNT) {
            const int c = e / VS, j = e % VS;
            sS[c * PS + j] = sE[c] * S0c[(size_t)c * V + j0 + j];
            sX[c * PS + j] = sF[c] * dSc[(size_t)c * V + j0 + j];
        }
        for (int e = t; e < C * VS; e += GNT) {
            const int r = e / VS, j = e % VS;
            const size_t off = ((size_t)(c0 + r) * H + h) * V + j0 + j;
            sR[e] = r < L ? to_f32(v[off]) : 0.f;
            sO[e] = r < L ? dout[off] : 0.f;
        }
        __syncthreads();
        for (int e = t; e < C * VS; e += GNT) {  // R = V - Kp S'
            const int r = e / VS, j = e % VS;
            float acc = sR[e];
            #pragma unroll 4
            for (int c = 0; c < K; ++c) acc -= sKp[r * PK + c] * sS[c * PS + j];
            sR[e] = acc;
        }
        __syncthreads();
        for (int e = t; e < C * VS; e += GNT) {  // U = T Diag(beta) R;  dU = P^T dO
            const int r = e / VS, j = e % VS;
            float u = 0.f, du = 0.f;
            for (int s = 0; s <= r; ++s) u += sT[r * PC + s] * sB[s] * sR[s * VS + j];
            for (int s = r; s < C; ++s) du += sP[s * PC + r] * sO[s * VS + j];
            sU[e] = u;
            sDU[e] = du;
        }
        __syncthreads();
        for (int e = t; e < C * VS; e += GNT) {  // dU += Km X
            const int r = e / VS, j = e % VS;
            float acc = sDU[e];
            #pragma unroll 4
            for (int c = 0; c < K; ++c) acc += sKm[r * PK + c] * sX[c * PS + j];
            sDU[e] = acc;
        }
        // h[c] += sum_j S_end[c][j] dS_end[c][j], with S_end = F (S' + Km^T U), X = F dS_end
        for (int c = t; c < K; c += GNT) {
            float acc = 0.f;
            for (int j = 0; j < VS; ++j) {
                float se = sS[c * PS + j];
                #pragma unroll 4
                for (int r = 0; r < C; ++r) se += sKm[r * PK + c] * sU[r * VS + j];
                acc += se * sX[c * PS + j];
            }
            sH[c] += acc;
        }
        __syncthreads();
        for (int e = t; e < C * VS; e += GNT) {  // dY = T^T dU
            const int r = e / VS, j = e % VS;
            float acc = 0.f;
            #pragma unroll 4
            for (int s = r; s < C; ++s) acc += sT[s * PC + r] * sDU[s * VS + j];
            sDY[e] = acc;
        }
        __syncthreads();
        for (int e = t; e < C * VS; e += GNT) {  // dv = beta dY
            const int r = e / VS, j = e % VS;
            if (r < L) dv[((size_t)(c0 + r) * H + h) * V + j0 + j] = sB[r] * sDY[e];
        }
        for (int r = t; r < C; r += GNT) {  // dbeta += rowsum(R * dY)
            float acc = 0.f;
            for (int j = 0; j < VS; ++j) acc += sR[r * VS + j] * sDY[r * VS + j];
            sDb[r] += acc;
        }
        // owned [C][K] elements: dQp += dO S'^T, dKp -= beta dY S'^T, dKm += U X^T
        // (column by column: the thread's channel operands are loaded once)
        {
            const int c = t % K, r0 = t / K;
#pragma unroll 1
            for (int j = 0; j < VS; ++j) {
                const float sv = sS[c * PS + j], xv = sX[c * PS + j];
#pragma unroll
                for (int i = 0; i < MCK; ++i) {
                    const int r = r0 + RK * i;
                    aQ[i] += sO[r * VS + j] * sv;
                    aKp[i] -= sB[r] * sDY[r * VS + j] * sv;
                    aKm[i] += sU[r * VS + j] * xv;
                }
            }
        }
        // owned [C][C] elements: dA -= dY U^T, dP += dO U^T
        {
            const int sc = t % C, r0 = t / C;
#pragma unroll 1
            for (int j = 0; j < VS; ++j) {
                const float u = sU[sc * VS + j];
#pragma unroll
                for (int i = 0; i < MCC; ++i) {
                    const int r = r0 + RC * i;
                    aA[i] -= sDY[r * VS + j] * u;
                    aP[i] += sO[r * VS + j] * u;
                }
            }
        }
    }
    __syncthreads();
    // masked dA (strictly lower) and dP (lower) to LDS; Gk over T
#pragma unroll
    for (int i = 0; i < MCC; ++i) {
        const int e = t + GNT * i, r = e / C, s = e % C;
        sP[r * PC + s] = s < r ? aA[i] : 0.f;
        sDp[r * PC + s] = s <= r ? aP[i] : 0.f;
    }
    rows_to_lds<C, C, PC, GNT>(sT, rec + Rc::GK);
    __syncthreads();
    for (int r = t; r < C; r += GNT) {  // dbeta += rowsum(Gk * dA)
        float acc = sDb[r];
        for (int s = 0; s < r; ++s) acc += sT[r * PC + s] * sP[r * PC + s];
        if (r < L) dbeta[(size_t)(c0 + r) * H + h] = acc;
    }
    // dKp += beta dA Km,  dQp += dP Km,  dKm += (beta dA)^T Kp + dP^T Qp
    {
        const int c = t % K, r0 = t / K;
#pragma unroll 1
        for (int s = 0; s < C; ++s) {
            const float kms = sKm[s * PK + c], bkp = sB[s] * sKp[s * PK + c], qps = sQp[s * PK + c];
#pragma unroll
            for (int i = 0; i < MCK; ++i) {
                const int r = r0 + RK * i;
                aKp[i] += sB[r] * sP[r * PC + s] * kms;
                aQ[i] += sDp[r * PC + s] * kms;
                aKm[i] += sP[s * PC + r] * bkp + sDp[s * PC + r] * qps;
            }
        }
    }
    // dq, dk, and D = dKp Kp - dKm Km + dQp Qp (+ h on the last row)
    float D[MCK];
#pragma unroll
    for (int i = 0; i < MCK; ++i) {
        const int e = t + GNT * i, r = e / K, c = e % K;
        D[i] = aKp[i] * sKp[r * PK + c] - aKm[i] * sKm[r * PK + c] + aQ[i] * sQp[r * PK + c] +
               (r == L - 1 ? sH[c] : 0.f);
        if (r < L) {
            const float ep = rec[Rc::EE + e];
            const size_t off = ((size_t)(c0 + r) * H + h) * K + c;
            dq[off] = aQ[i] * ep;
            dk[off] = aKp[i] * ep + aKm[i] / ep;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MCK; ++i) {
        const int e = t + GNT * i;
        sKp[(e / K) * PK + e % K] = D[i];
    }
    __syncthreads();
    for (int c = t; c < K; c += GNT) {  // dg = reverse running sum of D down each channel
        float acc = 0.f;
        for (int r = L - 1; r >= 0; --r) {
            acc += sKp[r * PK + c];
            dg[((size_t)(c0 + r) * H + h) * K + c] = acc;
        }
    }
}

template <int K, int V, int C>
size_t rec_bytes() { return sizeof(float) * BwdRec<K, V, C>::floats; }

// Upper bound on the packed chunk count of N sequences over total_T tokens.
size_t chunk_cap(int N, int totalT, int fixedT, bool packed, int C) {
    if (!packed) return (size_t)N * ((fixedT + C - 1) / C);
    return ((size_t)totalT + (size_t)(C - 1) * N) / C;
}

template <int K, int V, int C>
size_t bwd_ws_bytes(size_t cap, int H) {
    return cap * H * (rec_bytes<K, V, C>() + 2 * sizeof(float) * K * V);
}

template <int K, int V, int C, int VT, int VS, int GNT, typename TIn>
hipError_t launch_bwd_t(const void *q, const void *k, const void *v, const void *g,
                        const void *beta, const float *s0, const float *dout, const float *dsT,
                        float *dq, float *dk, float *dv, float *dg, float *dbeta, float *ds0,
                        const int32_t *cu, int N, int fixedT, int totalT, int H, void *workspace,
                        hipStream_t stream) {
    const size_t cap = chunk_cap(N, totalT, fixedT, cu != nullptr, C);
    float *recs = static_cast<float *>(workspace);
    float *Sst = recs + cap * H * BwdRec<K, V, C>::floats;
    float *dSe = Sst + cap * H * (size_t)K * V;
    const size_t red = sizeof(int) * BNT, redP = sizeof(int) * PNT, red3 = sizeof(int) * GNT;
    const size_t lds0 = sizeof(float) * (3 * C * (K + 1) + C * K + C + K) + redP;
    const size_t ldsT = sizeof(float) * (3 * C * (K + 1) + 2 * C * (C + 1) + C + 2 * K) + redP;
    const size_t lds1 = sizeof(float) * (K * (K + 1) + K * VT) + red;
    const size_t lds2 = lds1;
    const size_t lds3 = sizeof(float) * (3 * C * (K + 1) + 2 * C * (C + 1) + 2 * K * (VS + 1) +
                                         5 * C * VS + 2 * C + 3 * K) + red3;
    static std::atomic<uint64_t> set0{0}, setT{0}, set1{0}, set2{0}, set3{0};
    auto k0 = bwd_prep_kernel<K, V, C, TIn>;
    auto kT = bwd_trans_kernel<K, V, C, TIn>;
    auto k1 = bwd_states_kernel<K, V, C, VT>;
    auto k2 = bwd_dstate_kernel<K, V, C, VT>;
    auto k3 = bwd_grads_kernel<K, V, C, VS, GNT, TIn>;
    hipError_t e;
    if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(k0), (int)lds0, set0)) != hipSuccess) return e;
    if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(kT), (int)ldsT, setT)) != hipSuccess) return e;
    if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(k1), (int)lds1, set1)) != hipSuccess) return e;
    if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(k2), (int)lds2, set2)) != hipSuccess) return e;
    if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(k3), (int)lds3, set3)) != hipSuccess) return e;
    const TIn *tq = static_cast<const TIn *>(q), *tk = static_cast<const TIn *>(k);
    const TIn *tv = static_cast<const TIn *>(v), *tg = static_cast<const TIn *>(g);
    const TIn *tb = static_cast<const TIn *>(beta);
    if (cap > 0) {
        hipLaunchKernelGGL(k0, dim3((unsigned)cap, H), dim3(PNT), lds0, stream, tq, tk, tg, tb, cu, N,
                           fixedT, totalT, H, recs);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(kT, dim3((unsigned)cap, H), dim3(PNT), ldsT, stream, tv, dout, cu, N,
                           fixedT, totalT, H, recs);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(k1, dim3(V / VT, H, N), dim3(BNT), lds1, stream, s0, cu, fixedT,
                           totalT, H, recs, Sst);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k2, dim3(V / VT, H, N), dim3(BNT), lds2, stream, dsT, ds0, cu, fixedT,
                       totalT, H, recs, dSe);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (cap > 0) {
        hipLaunchKernelGGL(k3, dim3((unsigned)cap, H), dim3(GNT), lds3, stream, tv, dout, cu, N,
                           fixedT, totalT, H, recs, Sst, dSe, dq, dk, dv, dg, dbeta);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

bool chunk_bwd_supported(int K, int V, int C) {
    return (K == 32 && V == 32 && C == 16) || (K == 128 && V == 128 && C == 64);
}

size_t chunk_bwd_workspace_bytes(int N, int totalT, int fixedT, bool packed, int H, int K, int V,
                                 int C) {
    const size_t cap = chunk_cap(N, totalT, fixedT, packed, C);
    if (K == 32 && V == 32 && C == 16) return bwd_ws_bytes<32, 32, 16>(cap, H);
    if (K == 128 && V == 128 && C == 64) return bwd_ws_bytes<128, 128, 64>(cap, H);
    return 0;
}

hipError_t launch_chunk_bwd(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const float *s0, const float *dout,
                            const float *dsT, float *dq, float *dk, float *dv, float *dg,
                            float *dbeta, float *ds0, const int32_t *cu, int N, int fixedT,
                            int totalT, int H, int K, int V, int C, bool in_bf16,
                            void *workspace, hipStream_t stream) {
    if (N == 0 || H == 0) return hipSuccess;
    if (K == 128 && V == 128 && C == 64)
        return in_bf16 ? launch_bwd_t<128, 128, 64, 4, 8, 512, bf16_t>(q, k, v, g, beta, s0, dout, dsT, dq, dk, dv, dg, dbeta, ds0, cu, N, fixedT, totalT, H, workspace, stream)
                       : launch_bwd_t<128, 128, 64, 4, 8, 512, float>(q, k, v, g, beta, s0, dout, dsT, dq, dk, dv, dg, dbeta, ds0, cu, N, fixedT, totalT, H, workspace, stream);
    if (K == 32 && V == 32 && C == 16)
        return in_bf16 ? launch_bwd_t<32, 32, 16, 16, 8, 256, bf16_t>(q, k, v, g, beta, s0, dout, dsT, dq, dk, dv, dg, dbeta, ds0, cu, N, fixedT, totalT, H, workspace, stream)
                       : launch_bwd_t<32, 32, 16, 16, 8, 256, float>(q, k, v, g, beta, s0, dout, dsT, dq, dk, dv, dg, dbeta, ds0, cu, N, fixedT, totalT, H, workspace, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
