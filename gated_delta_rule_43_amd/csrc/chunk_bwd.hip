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
// Six launches:
//   bwd_prep_kernel    (chunk, head), all chunks at once: Kp, Km, Qp, E, Gk,
//                      P, T, beta, F, exp(G_m) into the chunk's record;
//   bwd_trans_kernel   (chunk, head): the chunk's state transition
//                      S_end = MM S_start + NN and the adjoint's constant NB;
//   bwd_states_kernel  (sequence, head, value tile): the forward state chain,
//                      one [K][K] product per chunk, leaving every chunk's
//                      start state in the workspace;
//   bwd_dstate_kernel  (sequence, head, value tile): the reverse chain
//                      dS_start = MM^T dS_end + NB, chunk after chunk from
//                      the last, and ds0 (at d = 128 both chains run as
//                      bwd_chain_mfma_kernel, on the matrix cores);
//   bwd_udy_kernel     (chunk, head), value tile after value tile: R, U,
//                      dU, dY and dv, and each tile's shares of dbeta and
//                      rowsum(S_end * dS_end);
//   bwd_kgrad_kernel   (chunk, head): the gradients that sum over all value
//                      columns (of q, k, g and beta), as register-tiled
//                      products over value slices.
// The state chains are column-separable (value tiles need no communication).
#include <type_traits>

#include "kda_mfma.hpp"

namespace kda {
namespace {

constexpr int BNT = 256;  // threads per workgroup of the state-chain kernels
constexpr int PNT = 512;  // threads per workgroup of the record, transition and column
                          // passes (one workgroup per CU by LDS; eight waves hide LDS latency)

// Record of one (chunk, head), in floats.  MM, NN, NB: the chunk's state
// transition S_end = MM S_start + NN and its adjoint dS_start = MM^T dS_end + NB.
template <int K, int V, int C>
struct BwdRec {
    static constexpr size_t KP = 0, KM = KP + C * K, QP = KM + C * K, EE = QP + C * K;
    static constexpr size_t GK = EE + C * K, PP = GK + C * C, TT = PP + C * C;
    static constexpr size_t BETA = TT + C * C, FF = BETA + C, EGM = FF + K;
    static constexpr size_t MM = EGM + K, NN = MM + K * K, NB = NN + K * V;
    // MM and MM^T as fp32 MFMA A fragments (16x16x4): [K/16 row blocks][K/4
    // k-steps][64 lanes], lane l holding row 16 rb + (l % 16), column
    // 4 ks + l / 16, so that a wave reads a fragment as one contiguous 256 B
    static constexpr size_t MMA = NB + K * V, MMTA = MMA + K * K;
    static constexpr size_t floats = MMTA + K * K;
    __host__ __device__ static constexpr size_t frag(int row, int col) {
        return ((size_t)(row / 16) * (K / 4) + col / 4) * 64 + (row % 16) + 16 * (col % 4);
    }
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

// Chunks of sequence [bos, eos) that a state chain walks, clamped so that
// its records [first, first + nch) stay inside the workspace's cap chunks:
// with malformed (non-monotone) cu_seqlens the per-sequence counts can sum
// past cap, and those chunks are then skipped rather than addressed.
__device__ __forceinline__ int chain_chunks(int bos, int eos, int C, int first, int cap) {
    const int nch = (eos - bos + C - 1) / C;
    const int room = cap - first;
    return nch < room ? nch : (room > 0 ? room : 0);
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

// 16-byte piece of a row of TIn values, widened to fp32 (8 values for bf16, 4 for fp32).
__device__ __forceinline__ void widen(const uint4 &x, const bf16_t *, float *o) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void widen(const uint4 &x, const float *, float *o) {
    o[0] = __uint_as_float(x.x);
    o[1] = __uint_as_float(x.y);
    o[2] = __uint_as_float(x.z);
    o[3] = __uint_as_float(x.w);
}

// A chunk's [C][D] tile of a token-major [tokens, H, D] tensor (rows c0 ..,
// head h; rows at or past L read as 0) to LDS as fp32 with row pitch P.
// 16-byte loads, every one issued before the first store.
template <int C, int D, int P, int NT, typename TIn>
__device__ __forceinline__ void token_tile_to_lds(float *dst, const TIn *src, int c0, int L, int H,
                                                  int h) {
    constexpr int EP = 16 / sizeof(TIn), Q = C * D / EP, PER = (Q + NT - 1) / NT;
    static_assert(D % EP == 0, "rows must split into 16-byte pieces");
    uint4 x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int qi = threadIdx.x + NT * i, r = qi * EP / D, c = qi * EP % D;
        x[i] = make_uint4(0u, 0u, 0u, 0u);
        if (qi < Q && r < L)
            x[i] = *reinterpret_cast<const uint4 *>(src + ((size_t)(c0 + r) * H + h) * D + c);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int qi = threadIdx.x + NT * i, r = qi * EP / D, c = qi * EP % D;
        if (qi < Q) {
            float f[EP];
            widen(x[i], src, f);
#pragma unroll
            for (int u = 0; u < EP; ++u) dst[r * P + c + u] = f[u];
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
    constexpr int PK = K + 4;     // row pitch: the 16 rows x 4 columns of a fragment read hit distinct banks
    float *sKp = smem;             // [C][PK]
    float *sKm = sKp + C * PK;     // [C][PK]
    float *sQp = sKm + C * PK;     // [C][PK]
    float *sX = sQp + C * PK;      // [C][K]: G, later Gk [C][C]
    float *sB = sX + C * K;        // [C]
    float *sGm = sB + C;           // [K]
    int *red = reinterpret_cast<int *>(sGm + K);  // [PNT]
    static_assert(C <= K, "Gk must fit the G buffer");

    const int gc = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    int n, ci;
    locate_chunk<PNT>(cu, N, fixedT, totalT, C, gc, n, ci, red);
    if (n < 0) return;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + ci * C, L = min(C, eos - c0);
    const int m = min(C / 2 - 1, L - 1);  // reference row
    float *rec = ws + ((size_t)gc * H + h) * Rc::floats;

    token_tile_to_lds<C, K, K, PNT>(sX, g, c0, L, H, h);
    token_tile_to_lds<C, K, PK, PNT>(sKp, k, c0, L, H, h);  // raw k and q until scaled below
    token_tile_to_lds<C, K, PK, PNT>(sQp, q, c0, L, H, h);
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
        const float kv = sKp[r * PK + c], qv = sQp[r * PK + c];
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
    float *sGk = sX;
    if constexpr (K == 128 && C == 64 && PNT == 512) {
        // on the matrix cores: wave w forms tiles 2 w and 2 w + 1 (row block
        // tile / 4, column block tile % 4) of both blocks; tiles above the
        // diagonal are zero
        const int lane = t & 63, w = t >> 6, lr = lane & 15, lq = lane >> 4;
        const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tt = 2 * w + u, ar = tt / 4, as = tt % 4;
            floatx4 a = z, p = z;
            if (as <= ar) {
#pragma unroll 8
                for (int ks = 0; ks < K / 4; ++ks) {
                    const int c = 4 * ks + lq;
                    const float km = sKm[(16 * as + lr) * PK + c];
                    a = __builtin_amdgcn_mfma_f32_16x16x4f32(sKp[(16 * ar + lr) * PK + c], km, a, 0, 0, 0);
                    p = __builtin_amdgcn_mfma_f32_16x16x4f32(sQp[(16 * ar + lr) * PK + c], km, p, 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * ar + 4 * lq + i, s2 = 16 * as + lr;
                const float gk = s2 < r ? a[i] : 0.f;
                sGk[r * C + s2] = gk;
                rec[Rc::GK + r * C + s2] = gk;
                rec[Rc::PP + r * C + s2] = s2 <= r ? p[i] : 0.f;
            }
        }
    } else {
    for (int e = t; e < C * C; e += PNT) {
        const int r = e / C, s = e % C;
        float a = 0.f, p = 0.f;
        if (s <= r) {
            float a4[4] = {}, p4[4] = {};  // four partial sums: shorter dependency chains
            for (int c = 0; c < K; c += 4) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float km = sKm[s * PK + c + u];
                    a4[u] += sKp[r * PK + c + u] * km;
                    p4[u] += sQp[r * PK + c + u] * km;
                }
            }
            a = (a4[0] + a4[1]) + (a4[2] + a4[3]);
            p = (p4[0] + p4[1]) + (p4[2] + p4[3]);
        }
        const float gk = s < r ? a : 0.f;
        sGk[e] = gk;
        rec[Rc::GK + e] = gk;
        rec[Rc::PP + e] = p;
    }
    }
    __syncthreads();
    // T = (I + Diag(beta) Gk)^-1 by forward substitution, one column per lane
    // of wave 0 held in registers: column j solves (I + Diag(beta) Gk) x = e_j,
    // x_r = [r == j] - beta_r sum_{s<r} Gk_rs x_s.  Entries not yet formed are
    // 0 and Gk is 0 on and above the diagonal, so each row's sum may run over
    // whole groups of four.
    static_assert(C <= 64 && C % 4 == 0, "one column per lane of a wave");
    if (t < C) {
        float x[C];
#pragma unroll
        for (int r = 0; r < C; ++r) x[r] = 0.f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int s4 = 0; s4 < (r + 3) / 4; ++s4) {
                const float4 gv = *reinterpret_cast<const float4 *>(sGk + r * C + 4 * s4);
                a0 += gv.x * x[4 * s4] + gv.z * x[4 * s4 + 2];
                a1 += gv.y * x[4 * s4 + 1] + gv.w * x[4 * s4 + 3];
            }
            x[r] = (r == t ? 1.f : 0.f) - sB[r] * (a0 + a1);
        }
#pragma unroll
        for (int r = 0; r < C; ++r) rec[Rc::TT + r * C + t] = x[r];
    }
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
            float a0 = 0.f, a1 = 0.f;
            int s2 = 0;
            for (; s2 + 1 <= r; s2 += 2) {
                a0 += sT[r * PC + s2] * sB[s2] * in[s2 * PD + j];
                a1 += sT[r * PC + s2 + 1] * sB[s2 + 1] * in[(s2 + 1) * PD + j];
            }
            if (s2 == r) a0 += sT[r * PC + r] * sB[r] * in[r * PD + j];
            out[r * PD + j] = a0 + a1;
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
        float a0 = 0.f, a1 = 0.f;
        int s2 = 0;
        for (; s2 + 1 <= r; s2 += 2) {
            a0 += sP[r * PC + s2] * b1[s2 * PD + j];
            a1 += sP[r * PC + s2 + 1] * b1[(s2 + 1) * PD + j];
        }
        if (s2 == r) a0 += sP[r * PC + r] * b1[r * PD + j];
        b2[r * PD + j] = b0[r * PD + j] - (a0 + a1);
    }
    __syncthreads();
    token_tile_to_lds<C, V, PD, PNT>(b0, dout, c0, L, H, h);
    __syncthreads();
    at_b(b2, b0, [&](int c, int j, float x) { rec[Rc::NB + (size_t)c * V + j] = sE[c] * x; });
    __syncthreads();
    load_rows(b0, Rc::KM);
    __syncthreads();
    at_b(b0, b1, [&](int c, int j, float x) {
        const float m = sF[c] * ((c == j ? 1.f : 0.f) - x) * sE[j];
        rec[Rc::MM + (size_t)c * K + j] = m;
        rec[Rc::MMA + Rc::frag(c, j)] = m;
        rec[Rc::MMTA + Rc::frag(j, c)] = m;
    });
    __syncthreads();
    token_tile_to_lds<C, V, PD, PNT>(b1, v, c0, L, H, h);
    __syncthreads();
    tri_apply(b2, b1);  // U~
    __syncthreads();
    at_b(b0, b2, [&](int c, int j, float x) { rec[Rc::NN + (size_t)c * V + j] = sF[c] * x; });
}

// Matrix-core variant of the transition pass at d = 128: the same six
// products on v_mfma_f32_16x16x4_f32 with eight waves.  In the [C][K]
// products (W, Q^, U~) wave w owns column block w for the four row blocks and
// skips the k-steps above the diagonal of the triangular factor; in the
// [K][K] products (NB, MM, NN) it owns row block w for all eight column
// blocks, one A fragment serving the eight.  Tiles carry row pitch K + 16 and
// the [C][C] factors C + 4, so that the lanes of a fragment read fall on
// distinct banks.
template <int K, int V, int C, typename TIn>
__global__ __launch_bounds__(PNT) void bwd_trans_mfma_kernel(
    const TIn *__restrict__ v, const float *__restrict__ dout, const int32_t *__restrict__ cu,
    int N, int fixedT, int totalT, int H, float *__restrict__ recs) {
    using Rc = BwdRec<K, V, C>;
    static_assert(K == 128 && V == K && C == 64 && PNT == 512, "eight waves over 128 x 128 tiles");
    constexpr int PD = K + 16, PC = C + 4, RB = C / 16, CB = K / 16, KS = C / 4;
    extern __shared__ float smem[];
    float *b0 = smem, *b1 = b0 + C * PD, *b2 = b1 + C * PD;
    float *sT = b2 + C * PD, *sP = sT + C * PC;
    float *sB = sP + C * PC, *sF = sB + C, *sE = sF + K;
    int *red = reinterpret_cast<int *>(sE + K);

    const int gc = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const int lane = t & 63, w = t >> 6, lr = lane & 15, lq = lane >> 4;
    int n, ci;
    locate_chunk<PNT>(cu, N, fixedT, totalT, C, gc, n, ci, red);
    if (n < 0) return;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + ci * C, L = min(C, eos - c0);
    float *rec = recs + ((size_t)gc * H + h) * Rc::floats;
    const floatx4 z = {0.f, 0.f, 0.f, 0.f};

    rows_to_lds<C, C, PC, PNT>(sT, rec + Rc::TT);
    rows_to_lds<C, C, PC, PNT>(sP, rec + Rc::PP);
    rows_to_lds<C, K, PD, PNT>(b0, rec + Rc::KP);
    rows_to_lds<C, K, PD, PNT>(b2, rec + Rc::QP);
    for (int r = t; r < C; r += PNT) sB[r] = rec[Rc::BETA + r];
    for (int c = t; c < K; c += PNT) {
        sF[c] = rec[Rc::FF + c];
        sE[c] = rec[Rc::EGM + c];
    }
    __syncthreads();
    // acc[b] = rows 16 b .. 16 b + 15, columns 16 w .. 16 w + 15 of L in, with
    // L lower triangular (T Diag(beta), or P): block b needs only s <= 16 b + 15
    auto tri = [&](const float *lo, bool scale, const float *in, floatx4(&acc)[RB]) {
#pragma unroll
        for (int b = 0; b < RB; ++b) acc[b] = z;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int s = 4 * ks + lq;
            const float bv = in[s * PD + 16 * w + lr], bs = scale ? sB[s] : 1.f;
#pragma unroll
            for (int b = 0; b < RB; ++b)
                if (b >= ks / 4)
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(lo[(16 * b + lr) * PC + s] * bs, bv,
                                                                  acc[b], 0, 0, 0);
        }
    };
    // acc[jb] = rows 16 w .. 16 w + 15, columns 16 jb .. 16 jb + 15 of a^T bm
    auto at_b = [&](const float *a, const float *bm, floatx4(&acc)[CB]) {
#pragma unroll
        for (int jb = 0; jb < CB; ++jb) acc[jb] = z;
#pragma unroll 4
        for (int ks = 0; ks < KS; ++ks) {
            const int s = 4 * ks + lq;
            const float av = a[s * PD + 16 * w + lr];
#pragma unroll
            for (int jb = 0; jb < CB; ++jb)
                acc[jb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bm[s * PD + 16 * jb + lr], acc[jb],
                                                               0, 0, 0);
        }
    };
    floatx4 acc[RB], accU[RB], accM[CB];
    tri(sT, true, b0, acc);  // W = T Diag(beta) Kp
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) b1[(16 * b + 4 * lq + i) * PD + 16 * w + lr] = acc[b][i];
    __syncthreads();
    tri(sP, false, b1, acc);  // Q^ = Qp - P W, in place (each lane owns its elements)
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) b2[(16 * b + 4 * lq + i) * PD + 16 * w + lr] -= acc[b][i];
    __syncthreads();
    token_tile_to_lds<C, V, PD, PNT>(b0, dout, c0, L, H, h);
    __syncthreads();
    at_b(b2, b0, accM);  // NB = Diag(exp(G_m)) Q^T dO
#pragma unroll
    for (int jb = 0; jb < CB; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 16 * w + 4 * lq + i, j = 16 * jb + lr;
            rec[Rc::NB + (size_t)c * V + j] = sE[c] * accM[jb][i];
        }
    __syncthreads();
    rows_to_lds<C, K, PD, PNT>(b0, rec + Rc::KM);
    token_tile_to_lds<C, V, PD, PNT>(b2, v, c0, L, H, h);
    __syncthreads();
    tri(sT, true, b2, accU);  // U~ = T Diag(beta) V
    at_b(b0, b1, accM);       // MM = F (I - Km^T W) Diag(exp(G_m))
#pragma unroll
    for (int jb = 0; jb < CB; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 16 * w + 4 * lq + i, j = 16 * jb + lr;
            const float m = sF[c] * ((c == j ? 1.f : 0.f) - accM[jb][i]) * sE[j];
            // only the fragment-ordered copies: the matrix-core chains read
            // those, and nothing reads the row-major MM at this size
            rec[Rc::MMA + Rc::frag(c, j)] = m;
            rec[Rc::MMTA + Rc::frag(j, c)] = m;
        }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) b1[(16 * b + 4 * lq + i) * PD + 16 * w + lr] = accU[b][i];
    __syncthreads();
    at_b(b0, b1, accM);  // NN = F Km^T U~
#pragma unroll
    for (int jb = 0; jb < CB; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 16 * w + 4 * lq + i, j = 16 * jb + lr;
            rec[Rc::NN + (size_t)c * V + j] = sF[c] * accM[jb][i];
        }
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
    int cap, const float *__restrict__ recs, float *__restrict__ Sst) {
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
    const int first = first_chunk<BNT>(cu, n, fixedT, totalT, C, red);
    const int nch = chain_chunks(bos, eos, C, first, cap);
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
        float S2[RB] = {};  // odd columns: a second dependency chain per row
        for (int c2 = 0; c2 < K; c2 += 2) {
            const float sv = sS[c2 * VT + j], sw = sS[(c2 + 1) * VT + j];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                S[i] += sM[(cb + i) * PK + c2] * sv;
                S2[i] += sM[(cb + i) * PK + c2 + 1] * sw;
            }
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) S[i] += S2[i];
    }
}

// ------------------------------------------------------------------ pass 2
// Reverse chain of the state gradient for one value tile, dS <- MM^T dS + NB
// chunk after chunk from the last: writes the gradient at the end of every
// chunk to dSe[chunk][h] and the gradient of S_0 to ds0.
template <int K, int V, int C, int VT>
__global__ __launch_bounds__(BNT) void bwd_dstate_kernel(
    const float *__restrict__ dsT, float *__restrict__ ds0, const int32_t *__restrict__ cu,
    int fixedT, int totalT, int H, int cap, const float *__restrict__ recs,
    float *__restrict__ dSe) {
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
    const int first = first_chunk<BNT>(cu, n, fixedT, totalT, C, red);
    const int nch = chain_chunks(bos, eos, C, first, cap);
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
        float D2[RB] = {};  // odd rows of MM: a second dependency chain per column
        for (int c2 = 0; c2 < K; c2 += 2) {
            const float dv = sS[c2 * VT + j], dw = sS[(c2 + 1) * VT + j];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                D[i] += sM[c2 * PK + cb + i] * dv;
                D2[i] += sM[(c2 + 1) * PK + cb + i] * dw;
            }
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) D[i] += D2[i];
    }
    if (ds0)
#pragma unroll
        for (int i = 0; i < RB; ++i) ds0[sbase + (size_t)(cb + i) * V] = D[i];
}

// ------------------------------------------------- passes 1 and 2, d = 128
// Both state chains on the matrix cores (v_mfma_f32_16x16x4_f32: exact fp32
// products, fp32 accumulation), one workgroup of eight waves per (sequence,
// head, 16-column value tile).  Wave w owns row block w of the tile (two per
// SIMD, so that one wave's fragment loads overlap the other's matrix
// instructions); the tile goes through LDS each chunk to serve as
// the B operand of every wave (two LDS copies by step parity, so one barrier
// per step suffices: a wave writes a copy in step s + 1 only after every wave
// has passed step s's barrier, and with it finished reading that copy in step
// s - 1), and the chunk's A fragments (MM, or MM^T for the adjoint, stored
// fragment-ordered in the record) stream from memory into registers ahead of
// use.
//   ADJ = false: S <- MM S + NN from s0, writing each chunk's start state;
//   ADJ = true:  dS <- MM^T dS + NB from dsT, chunk after chunk from the last,
//                writing each chunk's end-state gradient and finally ds0.
template <int K, int V, int C, bool ADJ>
__device__ __forceinline__ void chain_mfma(int vt, int h, int n, const float *__restrict__ init,
                                           float *__restrict__ fin, const int32_t *__restrict__ cu,
                                           int fixedT, int totalT, int H, int cap,
                                           const float *__restrict__ recs, float *__restrict__ out) {
    using Rc = BwdRec<K, V, C>;
    constexpr int NW = 8, KS = K / 4, RBW = K / (16 * NW);  // waves; k-steps; row blocks per wave
    static_assert(K == 128 && V % 16 == 0 && RBW == 1, "eight waves of one 16-row block");
    __shared__ float sS[2][K * 16];
    __shared__ int red[64 * NW];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int first = first_chunk<64 * NW>(cu, n, fixedT, totalT, C, red);
    const int nch = chain_chunks(bos, eos, C, first, cap);
    const int col = vt * 16 + (lane & 15);
    const size_t sbase = ((size_t)n * H + h) * K * V + col;
    const size_t fofs = ADJ ? Rc::MMTA : Rc::MMA, aofs = ADJ ? Rc::NB : Rc::NN;

    floatx4 acc[RBW];
#pragma unroll
    for (int b = 0; b < RBW; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * (RBW * w + b) + 4 * (lane >> 4) + i;
            acc[b][i] = init ? init[sbase + (size_t)row * V] : 0.f;
        }
    // The chunks' A fragments and addends are fetched DEPTH steps ahead into a
    // ring of register stages: one step's products take far less time than a
    // load's latency, so a one-step lookahead left every step waiting on its
    // loads.
    constexpr int DEPTH = 4;
    float cur[RBW][KS], nxt[DEPTH][RBW][KS], add[DEPTH][RBW][4];
    auto fetch = [&](int ci, float (&fr)[RBW][KS], float (&fa)[RBW][4]) {
        const float *rec = recs + ((size_t)(first + ci) * H + h) * Rc::floats;
#pragma unroll
        for (int b = 0; b < RBW; ++b) {
            const int rb = RBW * w + b;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) fr[b][ks] = rec[fofs + ((size_t)rb * KS + ks) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[b][i] = rec[aofs + (size_t)(16 * rb + 4 * (lane >> 4) + i) * V + col];
        }
    };
    auto chunk_of = [&](int step) { return ADJ ? nch - 1 - step : step; };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (d < nch) fetch(chunk_of(d), nxt[d], add[d]);
    for (int step0 = 0; step0 < nch; step0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int step = step0 + d;
            if (step >= nch) break;
            const int ci = chunk_of(step);
            float *dst = out + ((size_t)(first + ci) * H + h) * K * V + col;
#pragma unroll
            for (int b = 0; b < RBW; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * (RBW * w + b) + 4 * (lane >> 4) + i;
                    dst[(size_t)row * V] = acc[b][i];
                    sS[step & 1][row * 16 + (lane & 15)] = acc[b][i];
                }
            float ad[RBW][4];
#pragma unroll
            for (int b = 0; b < RBW; ++b) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) cur[b][ks] = nxt[d][b][ks];
#pragma unroll
                for (int i = 0; i < 4; ++i) ad[b][i] = add[d][b][i];
            }
            __syncthreads();
            if (step + DEPTH < nch) fetch(chunk_of(step + DEPTH), nxt[d], add[d]);
            // even and odd k-steps in two accumulators: two dependency chains
            floatx4 acc2[RBW];
#pragma unroll
            for (int b = 0; b < RBW; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[b][i] = ad[b][i];
                    acc2[b][i] = 0.f;
                }
#pragma unroll
            for (int ks = 0; ks < KS; ks += 2) {
                const float bv = sS[step & 1][64 * ks + lane];  // B[k = 4 ks + lane / 16][lane % 16]
                const float bw = sS[step & 1][64 * (ks + 1) + lane];
#pragma unroll
                for (int b = 0; b < RBW; ++b) {
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur[b][ks], bv, acc[b], 0, 0, 0);
                    acc2[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur[b][ks + 1], bw, acc2[b], 0, 0, 0);
                }
            }
#pragma unroll
            for (int b = 0; b < RBW; ++b) acc[b] += acc2[b];
        }
    }
    if (ADJ && fin)
#pragma unroll
        for (int b = 0; b < RBW; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * (RBW * w + b) + 4 * (lane >> 4) + i;
                fin[sbase + (size_t)row * V] = acc[b][i];
            }
}

// Both chains in one launch (they read different parts of the record and
// write different buffers, and each alone fills a quarter of the CUs at most
// on one sequence): grid (V / 16, H, 2 N) (launched in z slices from z0), z < N
// the state chain of sequence z, z >= N the state-gradient chain of sequence
// z - N.  Workgroups are dealt
// to the eight XCDs round-robin in dispatch order; when there are eight value
// tiles and the (head, z) pairs come in eights, the tiles of one pair are
// mapped to one XCD, so that their reads of the chunk's fragments share that
// XCD's L2.
template <int K, int V, int C>
__global__ __launch_bounds__(512) void bwd_chain_mfma_kernel(
    const float *__restrict__ s0, const float *__restrict__ dsT, float *__restrict__ ds0,
    const int32_t *__restrict__ cu, int N, int z0, int fixedT, int totalT, int H, int cap,
    const float *__restrict__ recs, float *__restrict__ Sst, float *__restrict__ dSe) {
    int vt = blockIdx.x, hz = blockIdx.y + gridDim.y * blockIdx.z;
    if (gridDim.x == 8 && (gridDim.y * gridDim.z) % 8 == 0) {
        const int id = blockIdx.x + 8 * hz;  // dispatch order
        vt = (id / 8) % 8;
        hz = id % 8 + 8 * (id / 64);
    }
    const int h = hz % gridDim.y, z = z0 + hz / gridDim.y;
    if (z < N)
        chain_mfma<K, V, C, false>(vt, h, z, s0, nullptr, cu, fixedT, totalT, H, cap, recs, Sst);
    else
        chain_mfma<K, V, C, true>(vt, h, z - N, dsT, ds0, cu, fixedT, totalT, H, cap, recs, dSe);
}

// ------------------------------------------------------------------ pass 3
// Per (chunk, head): the column-separable part of the chunk's gradient, one
// VT-column value tile after another with the chunk's operands staged once and
// the next tile's inputs loaded into registers while the current one is
// processed.  With S' = Diag(exp(G_m)) S_start and X = F dS_end on the tile:
//   R = V - Kp S',  U = T Diag(beta) R,  dU = Km X + P^T dO,  dY = T^T dU,
//   dv = Diag(beta) dY,
// the tile's share of dbeta (rowsum(R * dY)) and of rowsum(S_end * dS_end)
// (S_end = F (S' + Km^T U)), and U, dY stored transposed ([V][C] per
// (chunk, head)) for pass 4.
template <int K, int V, int C, int VT, typename TIn>
__global__ __launch_bounds__(PNT) void bwd_udy_kernel(
    const TIn *__restrict__ v, const float *__restrict__ dout, const int32_t *__restrict__ cu,
    int N, int fixedT, int totalT, int H, const float *__restrict__ recs,
    const float *__restrict__ Sst, const float *__restrict__ dSe, float *__restrict__ UT,
    float *__restrict__ dYT, float *__restrict__ dbp, float *__restrict__ hp,
    float *__restrict__ dv) {
    using Rc = BwdRec<K, V, C>;
    constexpr int PK = K + 1, PC = C + 1, PV = VT + 1, NVT = V / VT;
    constexpr int QS = (K * VT + PNT - 1) / PNT, QV = (C * VT + PNT - 1) / PNT;  // per-thread loads
    extern __shared__ float smem[];
    float *sKp = smem, *sKm = sKp + C * PK;              // [C][PK]
    float *sT = sKm + C * PK, *sP = sT + C * PC;         // [C][PC]
    float *sS = sP + C * PC, *sX = sS + K * PV;          // [K][PV]  S' (then S' + Km^T U), X
    float *sR = sX + K * PV, *sO = sR + C * PV;          // [C][PV]  R, dO
    float *sU = sO + C * PV, *sDU = sU + C * PV, *sDY = sDU + C * PV;  // [C][PV]
    float *sB = sDY + C * PV, *sF = sB + C, *sE = sF + K;
    int *red = reinterpret_cast<int *>(sE + K);

    const int gc = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    int n, ci;
    locate_chunk<PNT>(cu, N, fixedT, totalT, C, gc, n, ci, red);
    if (n < 0) return;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + ci * C, L = min(C, eos - c0);
    const size_t unit = (size_t)gc * H + h;
    const float *rec = recs + unit * Rc::floats;
    const float *S0c = Sst + unit * K * V, *dSc = dSe + unit * K * V;

    float pS[QS], pX[QS], pV[QV], pO[QV];
    auto fetch = [&](int j0) {  // tile inputs in registers
#pragma unroll
        for (int i = 0; i < QS; ++i) {
            const int e = t + PNT * i;
            if (e < K * VT) {
                const int c = e / VT, j = e % VT;
                pS[i] = S0c[(size_t)c * V + j0 + j];
                pX[i] = dSc[(size_t)c * V + j0 + j];
            }
        }
#pragma unroll
        for (int i = 0; i < QV; ++i) {
            const int e = t + PNT * i;
            if (e < C * VT) {
                const int r = e / VT, j = e % VT;
                const size_t off = ((size_t)(c0 + r) * H + h) * V + j0 + j;
                pV[i] = r < L ? to_f32(v[off]) : 0.f;
                pO[i] = r < L ? dout[off] : 0.f;
            }
        }
    };
    fetch(0);
    rows_to_lds<C, K, PK, PNT>(sKp, rec + Rc::KP);
    rows_to_lds<C, K, PK, PNT>(sKm, rec + Rc::KM);
    rows_to_lds<C, C, PC, PNT>(sT, rec + Rc::TT);
    rows_to_lds<C, C, PC, PNT>(sP, rec + Rc::PP);
    for (int r = t; r < C; r += PNT) sB[r] = rec[Rc::BETA + r];
    for (int c = t; c < K; c += PNT) {
        sF[c] = rec[Rc::FF + c];
        sE[c] = rec[Rc::EGM + c];
    }
    __syncthreads();
    for (int vt = 0; vt < NVT; ++vt) {
        const int j0 = vt * VT;
        if (vt > 0) __syncthreads();  // the previous tile's buffers are free
#pragma unroll
        for (int i = 0; i < QS; ++i) {
            const int e = t + PNT * i;
            if (e < K * VT) {
                const int c = e / VT, j = e % VT;
                sS[c * PV + j] = sE[c] * pS[i];
                sX[c * PV + j] = sF[c] * pX[i];
            }
        }
#pragma unroll
        for (int i = 0; i < QV; ++i) {
            const int e = t + PNT * i;
            if (e < C * VT) {
                const int r = e / VT, j = e % VT;
                sR[r * PV + j] = pV[i];
                sO[r * PV + j] = pO[i];
            }
        }
        __syncthreads();
        if (vt + 1 < NVT) fetch(j0 + VT);
        {  // R = V - Kp S';  dU = P^T dO + Km X.  Column jj, rows rr + RS m per thread
           // (one read of S' and X serves every row), four partial sums per dot
            constexpr int RS = PNT / VT, MR3 = (C + RS - 1) / RS;
            const int jj = t % VT, rr = t / VT;
            float a[MR3][4] = {}, d[MR3][4] = {};
            for (int c = 0; c < K; c += 4) {
                float sv[4], xv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    sv[u] = sS[(c + u) * PV + jj];
                    xv[u] = sX[(c + u) * PV + jj];
                }
#pragma unroll
                for (int m = 0; m < MR3; ++m) {
                    const int r = rr + RS * m;
                    if (r < C) {
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            a[m][u] += sKp[r * PK + c + u] * sv[u];
                            d[m][u] += sKm[r * PK + c + u] * xv[u];
                        }
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MR3; ++m) {
                const int r = rr + RS * m;
                if (r < C) {
                    float du = (d[m][0] + d[m][1]) + (d[m][2] + d[m][3]);
                    for (int s2 = r; s2 < C; ++s2) du += sP[s2 * PC + r] * sO[s2 * PV + jj];
                    sR[r * PV + jj] = sR[r * PV + jj] - ((a[m][0] + a[m][1]) + (a[m][2] + a[m][3]));
                    sDU[r * PV + jj] = du;
                }
            }
        }
        __syncthreads();
        for (int e = t; e < C * VT; e += PNT) {  // U = T Diag(beta) R;  dY = T^T dU
            const int r = e / VT, j = e % VT;
            float u0 = 0.f, u1 = 0.f, y0 = 0.f, y1 = 0.f;
            int s2 = 0;
            for (; s2 + 1 <= r; s2 += 2) {
                u0 += sT[r * PC + s2] * sB[s2] * sR[s2 * PV + j];
                u1 += sT[r * PC + s2 + 1] * sB[s2 + 1] * sR[(s2 + 1) * PV + j];
            }
            if (s2 == r) u0 += sT[r * PC + r] * sB[r] * sR[r * PV + j];
            for (s2 = r; s2 + 1 < C; s2 += 2) {
                y0 += sT[s2 * PC + r] * sDU[s2 * PV + j];
                y1 += sT[(s2 + 1) * PC + r] * sDU[(s2 + 1) * PV + j];
            }
            if (s2 < C) y0 += sT[s2 * PC + r] * sDU[s2 * PV + j];
            const float dy = y0 + y1;
            sU[r * PV + j] = u0 + u1;
            sDY[r * PV + j] = dy;
            if (r < L) dv[((size_t)(c0 + r) * H + h) * V + j0 + j] = sB[r] * dy;
        }
        __syncthreads();
        for (int e = t; e < K * VT; e += PNT) {  // S' + Km^T U, in place
            const int c = e / VT, j = e % VT;
            float a[4] = {};
            for (int r = 0; r < C; r += 4) {
#pragma unroll
                for (int u = 0; u < 4; ++u) a[u] += sKm[(r + u) * PK + c] * sU[(r + u) * PV + j];
            }
            sS[c * PV + j] += (a[0] + a[1]) + (a[2] + a[3]);
        }
        for (int r = t; r < C; r += PNT) {  // this tile's share of dbeta
            float acc = 0.f;
            for (int j = 0; j < VT; ++j) acc += sR[r * PV + j] * sDY[r * PV + j];
            dbp[(unit * NVT + vt) * C + r] = acc;
        }
        for (int e = t; e < C * VT; e += PNT) {  // U and dY transposed: [V][C]
            const int j = e / C, r = e % C;
            UT[unit * V * C + (size_t)(j0 + j) * C + r] = sU[r * PV + j];
            dYT[unit * V * C + (size_t)(j0 + j) * C + r] = sDY[r * PV + j];
        }
        __syncthreads();
        for (int c = t; c < K; c += PNT) {  // and of rowsum(S_end * dS_end) = rowsum((S' + Km^T U) * X)
            float acc = 0.f;
            for (int j = 0; j < VT; ++j) acc += sS[c * PV + j] * sX[c * PV + j];
            hp[(unit * NVT + vt) * K + c] = acc;
        }
    }
}

// ------------------------------------------------- pass 3, d = 128 (matrix cores)
// The column pass with every product on v_mfma_f32_16x16x4_f32 (exact fp32
// products).  Eight waves per (chunk, head): waves 0-3 form R = V - Kp S' and
// then U = (T Diag(beta)) R for row block w; waves 4-7 form dU = Km X + P^T dO
// and then dY = T^T dU for row block w - 4; then every wave forms one 16-row
// block of S' + Km^T U (for rowsum(S_end * dS_end)).  The chunk's A fragments
// (Kp, Km, T Diag(beta), P^T, T^T, Km^T) are loaded into registers once and
// serve all the value tiles; the tiles' B operands come from LDS.
template <int K, int V, int C, int VT>
__global__ __launch_bounds__(512) void bwd_udy_mfma_kernel(
    const bf16_t *__restrict__ vb, const float *__restrict__ vf, bool in_bf16,
    const float *__restrict__ dout, const int32_t *__restrict__ cu, int N, int fixedT,
    int totalT, int H, const float *__restrict__ recs, const float *__restrict__ Sst,
    const float *__restrict__ dSe, float *__restrict__ UT, float *__restrict__ dYT,
    float *__restrict__ dbp, float *__restrict__ hp, float *__restrict__ dv) {
    using Rc = BwdRec<K, V, C>;
    constexpr int PV = VT + 1, NVT = V / VT, KSK = K / 4, KSC = C / 4;
    static_assert(K == 128 && C == 64 && VT == 16, "eight waves: four row blocks of C, eight of K");
    __shared__ float sS[K * PV], sX[K * PV];                  // S', X (F dS_end)
    __shared__ float sO[C * PV], sR[C * PV], sDU[C * PV];     // dO, R, dU
    __shared__ float sU[C * PV], sDY[C * PV];                 // U, dY
    __shared__ float sF[K], sE[K], sB[C];
    __shared__ int red[512];

    const int gc = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const int lane = t & 63, w = t >> 6, rb = w & 3, lr = lane & 15, lq = lane >> 4;
    int n, ci;
    locate_chunk<512>(cu, N, fixedT, totalT, C, gc, n, ci, red);
    if (n < 0) return;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + ci * C, L = min(C, eos - c0);
    const size_t unit = (size_t)gc * H + h;
    const float *rec = recs + unit * Rc::floats;
    const float *S0c = Sst + unit * K * V, *dSc = dSe + unit * K * V;
    for (int r = t; r < C; r += 512) sB[r] = rec[Rc::BETA + r];
    for (int c = t; c < K; c += 512) {
        sF[c] = rec[Rc::FF + c];
        sE[c] = rec[Rc::EGM + c];
    }
    // A fragments: lane holds row 16 blk + lr, column 4 ks + lq
    float a1[KSK], a2[KSC], a3[KSC];
    const int arow = 16 * rb + lr;
    if (w < 4) {  // Kp (for R), T Diag(beta) (for U)
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks) a1[ks] = rec[Rc::KP + (size_t)arow * K + 4 * ks + lq];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            const int s2 = 4 * ks + lq;
            a2[ks] = rec[Rc::TT + (size_t)arow * C + s2] * rec[Rc::BETA + s2];
            a3[ks] = 0.f;
        }
    } else {      // Km (for dU), P^T (for dU), T^T (for dY)
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks) a1[ks] = rec[Rc::KM + (size_t)arow * K + 4 * ks + lq];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            const int s2 = 4 * ks + lq;
            a2[ks] = rec[Rc::PP + (size_t)s2 * C + arow];
            a3[ks] = rec[Rc::TT + (size_t)s2 * C + arow];
        }
    }
    float a4[KSC];  // Km^T, rows 16 w .. of K
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) a4[ks] = rec[Rc::KM + (size_t)(4 * ks + lq) * K + 16 * w + lr];
    __syncthreads();

    // Each value tile's inputs (its columns of S_start, dS_end, V and dO) are
    // loaded into registers one tile ahead, so their latency overlaps the
    // previous tile's products instead of stalling every tile.
    constexpr int NS = K * VT / 512, NR = C * VT / 512;
    static_assert(NS * 512 == K * VT && NR * 512 == C * VT, "tile elements per thread");
    float pS[NS], pX[NS], pR[NR], pO[NR];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int e = t + 512 * i, c = e / VT, j = e % VT;
            pS[i] = S0c[(size_t)c * V + j0 + j];
            pX[i] = dSc[(size_t)c * V + j0 + j];
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int e = t + 512 * i, r = e / VT, j = e % VT;
            const size_t off = ((size_t)(c0 + r) * H + h) * V + j0 + j;
            pR[i] = r < L ? (in_bf16 ? to_f32(vb[off]) : vf[off]) : 0.f;
            pO[i] = r < L ? dout[off] : 0.f;
        }
    };
    fetch(0);
    for (int vt = 0; vt < NVT; ++vt) {
        const int j0 = vt * VT;
        if (vt > 0) __syncthreads();
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int e = t + 512 * i, c = e / VT, j = e % VT;
            sS[c * PV + j] = sE[c] * pS[i];
            sX[c * PV + j] = sF[c] * pX[i];
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int e = t + 512 * i, r = e / VT, j = e % VT;
            sR[r * PV + j] = pR[i];
            sO[r * PV + j] = pO[i];
        }
        if (vt + 1 < NVT) fetch(j0 + VT);
        __syncthreads();
        // phase A: R (waves 0-3) or dU (waves 4-7) for row block rb
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        const float *bk = w < 4 ? sS : sX;
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[ks], bk[(4 * ks + lq) * PV + lr], acc, 0, 0, 0);
        if (w >= 4) {
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a2[ks], sO[(4 * ks + lq) * PV + lr], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rb + 4 * lq + i;
            if (w < 4) sR[r * PV + lr] = sR[r * PV + lr] - acc[i];
            else sDU[r * PV + lr] = acc[i];
        }
        __syncthreads();
        // phase B: U = (T Diag(beta)) R (waves 0-3), dY = T^T dU (waves 4-7)
        acc = floatx4{0.f, 0.f, 0.f, 0.f};
        const float *bb = w < 4 ? sR : sDU;
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(w < 4 ? a2[ks] : a3[ks],
                                                       bb[(4 * ks + lq) * PV + lr], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rb + 4 * lq + i;
            if (w < 4) {
                sU[r * PV + lr] = acc[i];
            } else {
                sDY[r * PV + lr] = acc[i];
                if (r < L) dv[((size_t)(c0 + r) * H + h) * V + j0 + lr] = sB[r] * acc[i];
            }
        }
        __syncthreads();
        // phase C: S' + Km^T U for rows 16 w .. of K, then this tile's share of
        // rowsum(S_end * dS_end) (a 16-lane sum per row)
        acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[ks], sU[(4 * ks + lq) * PV + lr], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 16 * w + 4 * lq + i;
            float x = (sS[c * PV + lr] + acc[i]) * sX[c * PV + lr];
            x += __shfl_xor(x, 1);
            x += __shfl_xor(x, 2);
            x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8);
            if (lr == 0) hp[(unit * NVT + vt) * K + c] = x;
        }
        for (int r = t; r < C; r += 512) {  // this tile's share of dbeta
            float s = 0.f;
            for (int j = 0; j < VT; ++j) s += sR[r * PV + j] * sDY[r * PV + j];
            dbp[(unit * NVT + vt) * C + r] = s;
        }
        for (int e = t; e < C * VT; e += 512) {  // U and dY transposed: [V][C]
            const int j = e / C, r = e % C;
            UT[unit * V * C + (size_t)(j0 + j) * C + r] = sU[r * PV + j];
            dYT[unit * V * C + (size_t)(j0 + j) * C + r] = sDY[r * PV + j];
        }
    }
}

// ------------------------------------------------------------------ pass 4
// Per (chunk, head): the gradients that sum over all value columns,
//   dQp = dO S'^T + dP Km,  dKp = -Diag(beta) dY S'^T + Diag(beta) dA Km,
//   dKm = U X^T + (Diag(beta) dA)^T Kp + dP^T Qp,
//   dA = -strict_lower(dY U^T),  dP = lower(dO U^T),
// then dq, dk, dg and dbeta.  The products over the value columns run on
// VB-column slices staged transposed in LDS, each thread holding an MR x MC
// tile of the [C][K] sums and an AR x AC tile of the [C][C] sums.
template <int K, int V, int C, int VT, int VB, int NT, int MR, int MC, int AR, int AC,
          typename TIn>
__global__ __launch_bounds__(NT) void bwd_kgrad_kernel(
    const float *__restrict__ dout, const int32_t *__restrict__ cu, int N, int fixedT,
    int totalT, int H, const float *__restrict__ recs, const float *__restrict__ Sst,
    const float *__restrict__ dSe, const float *__restrict__ UT, const float *__restrict__ dYT,
    const float *__restrict__ dbp, const float *__restrict__ hp, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dg, float *__restrict__ dbeta) {
    using Rc = BwdRec<K, V, C>;
    constexpr int NVT = V / VT, PK = K + 1, PC = C + 1, PTC = C + 4, PTK = K + 4;
    constexpr int CG = K / MC, ACG = C / AC;  // column groups
    static_assert((C / MR) * CG == NT && (C / AR) * ACG == NT, "tiles must cover the workgroup");
    static_assert(V % VB == 0, "value slices");
    extern __shared__ float smem[];
    // value-column phase
    float *sOT = smem, *sYT = sOT + VB * PTC, *sUT = sYT + VB * PTC;  // [VB][PTC]
    float *sST = sUT + VB * PTC, *sXT = sST + VB * PTK;               // [VB][PTK]
    // final phase (over the same space)
    float *sKp = smem, *sKm = sKp + C * PK, *sQp = sKm + C * PK;      // [C][PK]
    float *sA = sQp + C * PK, *sDp = sA + C * PC, *sG = sDp + C * PC; // [C][PC]
    float *sB = sG + C * PC, *sH = sB + C, *sF = sH + K, *sE = sF + K;
    int *red = reinterpret_cast<int *>(sE + K);
    static_assert(3 * VB * PTC + 2 * VB * PTK <= 3 * C * PK + 3 * C * PC, "slices fit");

    const int gc = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    int n, ci;
    locate_chunk<NT>(cu, N, fixedT, totalT, C, gc, n, ci, red);
    if (n < 0) return;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + ci * C, L = min(C, eos - c0);
    const size_t unit = (size_t)gc * H + h;
    const float *rec = recs + unit * Rc::floats;
    const float *S0c = Sst + unit * K * V, *dSc = dSe + unit * K * V;
    const float *Uc = UT + unit * V * C, *dYc = dYT + unit * V * C;
    for (int r = t; r < C; r += NT) sB[r] = rec[Rc::BETA + r];
    for (int c = t; c < K; c += NT) {
        sF[c] = rec[Rc::FF + c];
        sE[c] = rec[Rc::EGM + c];
    }

    const int r0 = (t / CG) * MR, cc0 = (t % CG) * MC;    // [C][K] tile
    const int ar0 = (t / ACG) * AR, as0 = (t % ACG) * AC; // [C][C] tile
    float aQ[MR][MC] = {}, aKp[MR][MC] = {}, aKm[MR][MC] = {}, aA[AR][AC] = {}, aP[AR][AC] = {};
    // transposed staging of a VB-column slice: 16-byte loads along the value
    // columns, all issued before the stores
    constexpr int QO = (C * VB / 4 + NT - 1) / NT, QS = (K * VB / 4 + NT - 1) / NT;
    for (int jb = 0; jb < V; jb += VB) {
        __syncthreads();
        float4 xo[QO], xs[QS], xx[QS];
#pragma unroll
        for (int i = 0; i < QO; ++i) {
            const int qi = t + NT * i, r = qi * 4 / VB, j = qi * 4 % VB;
            xo[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (qi < C * VB / 4 && r < L)
                xo[i] = *reinterpret_cast<const float4 *>(dout + ((size_t)(c0 + r) * H + h) * V + jb + j);
        }
#pragma unroll
        for (int i = 0; i < QS; ++i) {
            const int qi = t + NT * i, c = qi * 4 / VB, j = qi * 4 % VB;
            if (qi < K * VB / 4) {
                xs[i] = *reinterpret_cast<const float4 *>(S0c + (size_t)c * V + jb + j);
                xx[i] = *reinterpret_cast<const float4 *>(dSc + (size_t)c * V + jb + j);
            }
        }
        rows_to_lds<VB, C, PTC, NT>(sYT, dYc + (size_t)jb * C);
        rows_to_lds<VB, C, PTC, NT>(sUT, Uc + (size_t)jb * C);
#pragma unroll
        for (int i = 0; i < QO; ++i) {
            const int qi = t + NT * i, r = qi * 4 / VB, j = qi * 4 % VB;
            if (qi < C * VB / 4) {
                sOT[j * PTC + r] = xo[i].x;
                sOT[(j + 1) * PTC + r] = xo[i].y;
                sOT[(j + 2) * PTC + r] = xo[i].z;
                sOT[(j + 3) * PTC + r] = xo[i].w;
            }
        }
#pragma unroll
        for (int i = 0; i < QS; ++i) {
            const int qi = t + NT * i, c = qi * 4 / VB, j = qi * 4 % VB;
            if (qi < K * VB / 4) {
                const float e = sE[c], f = sF[c];
                sST[j * PTK + c] = e * xs[i].x;
                sST[(j + 1) * PTK + c] = e * xs[i].y;
                sST[(j + 2) * PTK + c] = e * xs[i].z;
                sST[(j + 3) * PTK + c] = e * xs[i].w;
                sXT[j * PTK + c] = f * xx[i].x;
                sXT[(j + 1) * PTK + c] = f * xx[i].y;
                sXT[(j + 2) * PTK + c] = f * xx[i].z;
                sXT[(j + 3) * PTK + c] = f * xx[i].w;
            }
        }
        __syncthreads();
#pragma unroll 2
        for (int j = 0; j < VB; ++j) {
            float o[MR], y[MR], u[MR], sv[MC], xv[MC];
#pragma unroll
            for (int i = 0; i < MR; ++i) {
                o[i] = sOT[j * PTC + r0 + i];
                y[i] = sYT[j * PTC + r0 + i];
                u[i] = sUT[j * PTC + r0 + i];
            }
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                sv[m] = sST[j * PTK + cc0 + m];
                xv[m] = sXT[j * PTK + cc0 + m];
            }
#pragma unroll
            for (int i = 0; i < MR; ++i)
#pragma unroll
                for (int m = 0; m < MC; ++m) {
                    aQ[i][m] += o[i] * sv[m];
                    aKp[i][m] += y[i] * sv[m];
                    aKm[i][m] += u[i] * xv[m];
                }
            float yy[AR], oo[AR], uu[AC];
#pragma unroll
            for (int i = 0; i < AR; ++i) {
                yy[i] = sYT[j * PTC + ar0 + i];
                oo[i] = sOT[j * PTC + ar0 + i];
            }
#pragma unroll
            for (int m = 0; m < AC; ++m) uu[m] = sUT[j * PTC + as0 + m];
#pragma unroll
            for (int i = 0; i < AR; ++i)
#pragma unroll
                for (int m = 0; m < AC; ++m) {
                    aA[i][m] -= yy[i] * uu[m];
                    aP[i][m] += oo[i] * uu[m];
                }
        }
    }
    __syncthreads();
    // final phase: record operands, masked dA and dP, Gk, the tiles' partial sums
    rows_to_lds<C, K, PK, NT>(sKp, rec + Rc::KP);
    rows_to_lds<C, K, PK, NT>(sKm, rec + Rc::KM);
    rows_to_lds<C, K, PK, NT>(sQp, rec + Rc::QP);
    rows_to_lds<C, C, PC, NT>(sG, rec + Rc::GK);
#pragma unroll
    for (int i = 0; i < AR; ++i)
#pragma unroll
        for (int m = 0; m < AC; ++m) {
            const int r = ar0 + i, s2 = as0 + m;
            sA[r * PC + s2] = s2 < r ? aA[i][m] : 0.f;
            sDp[r * PC + s2] = s2 <= r ? aP[i][m] : 0.f;
        }
    for (int c = t; c < K; c += NT) {
        float acc = 0.f;
        for (int w = 0; w < NVT; ++w) acc += hp[(unit * NVT + w) * K + c];
        sH[c] = acc;
    }
    __syncthreads();
    for (int r = t; r < C; r += NT) {  // dbeta = tiles' rowsum(R * dY) + rowsum(Gk * dA)
        float acc = 0.f;
        for (int w = 0; w < NVT; ++w) acc += dbp[(unit * NVT + w) * C + r];
        for (int s2 = 0; s2 < r; ++s2) acc += sG[r * PC + s2] * sA[r * PC + s2];
        if (r < L) dbeta[(size_t)(c0 + r) * H + h] = acc;
    }
    // dKp = beta (dA Km - dY S'^T),  dQp += dP Km,  dKm += (beta dA)^T Kp + dP^T Qp
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int m = 0; m < MC; ++m) aKp[i][m] = -aKp[i][m];
    for (int s2 = 0; s2 < C; ++s2) {
        float km[MC], kp[MC], qp[MC];
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            km[m] = sKm[s2 * PK + cc0 + m];
            kp[m] = sB[s2] * sKp[s2 * PK + cc0 + m];
            qp[m] = sQp[s2 * PK + cc0 + m];
        }
#pragma unroll
        for (int i = 0; i < MR; ++i) {
            const int r = r0 + i;
            const float a = sA[r * PC + s2], p = sDp[r * PC + s2];
            const float at = sA[s2 * PC + r], pt = sDp[s2 * PC + r];
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                aKp[i][m] += a * km[m];
                aQ[i][m] += p * km[m];
                aKm[i][m] += at * kp[m] + pt * qp[m];
            }
        }
    }
    float D[MR][MC];
#pragma unroll
    for (int i = 0; i < MR; ++i) {
        const int r = r0 + i;
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            const int c = cc0 + m;
            const float dKp = sB[r] * aKp[i][m];
            D[i][m] = dKp * sKp[r * PK + c] - aKm[i][m] * sKm[r * PK + c] +
                      aQ[i][m] * sQp[r * PK + c] + (r == L - 1 ? sH[c] : 0.f);
            if (r < L) {
                const float ep = rec[Rc::EE + (size_t)r * K + c];
                const size_t off = ((size_t)(c0 + r) * H + h) * K + c;
                dq[off] = aQ[i][m] * ep;
                dk[off] = dKp * ep + aKm[i][m] / ep;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int m = 0; m < MC; ++m) sKp[(r0 + i) * PK + cc0 + m] = D[i][m];
    __syncthreads();
    for (int c = t; c < K; c += NT) {  // dg = reverse running sum of D down each channel
        float acc = 0.f;
        for (int r = L - 1; r >= 0; --r) {
            acc += sKp[r * PK + c];
            dg[((size_t)(c0 + r) * H + h) * K + c] = acc;
        }
    }
}

// ------------------------------------------------- pass 4, d = 128 (matrix cores)
// The cross-column gradients with every product on v_mfma_f32_16x16x4_f32.
// Eight waves; wave w owns column block w of the three [C][K] sums (all four
// row blocks) and two 16 x 16 tiles of each [C][C] sum.  The value-column
// contractions read their fragments from 32-column slices staged transposed
// in LDS; the C-contractions of the final phase read them from the staged
// record tiles.
template <int K, int V, int C, int VT, int VB>
__global__ __launch_bounds__(512) void bwd_kgrad_mfma_kernel(
    const float *__restrict__ dout, const int32_t *__restrict__ cu, int N, int fixedT,
    int totalT, int H, const float *__restrict__ recs, const float *__restrict__ Sst,
    const float *__restrict__ dSe, const float *__restrict__ UT, const float *__restrict__ dYT,
    const float *__restrict__ dbp, const float *__restrict__ hp, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dg, float *__restrict__ dbeta) {
    using Rc = BwdRec<K, V, C>;
    constexpr int NT = 512, NVT = V / VT, PK = K + 1, PC = C + 1, PTC = C + 4, PTK = K + 4;
    constexpr int RB = C / 16;  // row blocks
    static_assert(K == 128 && C == 64 && V % VB == 0 && VB % 4 == 0, "eight waves, one column block each");
    extern __shared__ float smem[];
    float *sOT = smem, *sYT = sOT + VB * PTC, *sUT = sYT + VB * PTC;  // [VB][PTC]
    float *sST = sUT + VB * PTC, *sXT = sST + VB * PTK;               // [VB][PTK]
    float *sKp = smem, *sKm = sKp + C * PK, *sQp = sKm + C * PK;      // [C][PK]
    float *sA = sQp + C * PK, *sDp = sA + C * PC, *sG = sDp + C * PC; // [C][PC]
    float *sB = sG + C * PC, *sH = sB + C, *sF = sH + K, *sE = sF + K;
    int *red = reinterpret_cast<int *>(sE + K);

    const int gc = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const int lane = t & 63, w = t >> 6, lr = lane & 15, lq = lane >> 4;
    int n, ci;
    locate_chunk<NT>(cu, N, fixedT, totalT, C, gc, n, ci, red);
    if (n < 0) return;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + ci * C, L = min(C, eos - c0);
    const size_t unit = (size_t)gc * H + h;
    const float *rec = recs + unit * Rc::floats;
    const float *S0c = Sst + unit * K * V, *dSc = dSe + unit * K * V;
    const float *Uc = UT + unit * V * C, *dYc = dYT + unit * V * C;
    for (int r = t; r < C; r += NT) sB[r] = rec[Rc::BETA + r];
    for (int c = t; c < K; c += NT) {
        sF[c] = rec[Rc::FF + c];
        sE[c] = rec[Rc::EGM + c];
    }
    const int cb = w;                       // this wave's column block of the [C][K] sums
    const int t0 = 2 * w, t1 = 2 * w + 1;   // its two [C][C] tiles (row block t / 4, column block t % 4)
    floatx4 aQ[RB], aKp[RB], aKm[RB], aA[2], aP[2];
    const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < RB; ++b) aQ[b] = aKp[b] = aKm[b] = z;
    aA[0] = aA[1] = aP[0] = aP[1] = z;

    // Each value slice's inputs are loaded into registers one slice ahead
    // (issued once the slice before is staged, in flight during its
    // products), then staged transposed in LDS.
    constexpr int QO = (C * VB / 4 + NT - 1) / NT, QS = (K * VB / 4 + NT - 1) / NT;
    constexpr int QR = (VB * C / 4 + NT - 1) / NT;
    float4 xo[QO], xs[QS], xx[QS], xy[QR], xu[QR];
    auto load_slice = [&](int jb) {
#pragma unroll
        for (int i = 0; i < QO; ++i) {
            const int qi = t + NT * i, r = qi * 4 / VB, j = qi * 4 % VB;
            xo[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (qi < C * VB / 4 && r < L)
                xo[i] = *reinterpret_cast<const float4 *>(dout + ((size_t)(c0 + r) * H + h) * V + jb + j);
        }
#pragma unroll
        for (int i = 0; i < QS; ++i) {
            const int qi = t + NT * i, c = qi * 4 / VB, j = qi * 4 % VB;
            if (qi < K * VB / 4) {
                xs[i] = *reinterpret_cast<const float4 *>(S0c + (size_t)c * V + jb + j);
                xx[i] = *reinterpret_cast<const float4 *>(dSc + (size_t)c * V + jb + j);
            }
        }
#pragma unroll
        for (int i = 0; i < QR; ++i) {
            const int qi = t + NT * i;
            if (qi < VB * C / 4) {
                xy[i] = reinterpret_cast<const float4 *>(dYc + (size_t)jb * C)[qi];
                xu[i] = reinterpret_cast<const float4 *>(Uc + (size_t)jb * C)[qi];
            }
        }
    };
    load_slice(0);
    for (int jb = 0; jb < V; jb += VB) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < QR; ++i) {  // the slice's dY^T and U^T rows, [VB][C] at pitch PTC
            const int qi = t + NT * i;
            if (qi < VB * C / 4) {
                const int e = 4 * qi, r = e / C, c = e % C;
                float *dy = sYT + r * PTC + c, *du = sUT + r * PTC + c;
                dy[0] = xy[i].x;
                dy[1] = xy[i].y;
                dy[2] = xy[i].z;
                dy[3] = xy[i].w;
                du[0] = xu[i].x;
                du[1] = xu[i].y;
                du[2] = xu[i].z;
                du[3] = xu[i].w;
            }
        }
#pragma unroll
        for (int i = 0; i < QO; ++i) {
            const int qi = t + NT * i, r = qi * 4 / VB, j = qi * 4 % VB;
            if (qi < C * VB / 4) {
                sOT[j * PTC + r] = xo[i].x;
                sOT[(j + 1) * PTC + r] = xo[i].y;
                sOT[(j + 2) * PTC + r] = xo[i].z;
                sOT[(j + 3) * PTC + r] = xo[i].w;
            }
        }
#pragma unroll
        for (int i = 0; i < QS; ++i) {
            const int qi = t + NT * i, c = qi * 4 / VB, j = qi * 4 % VB;
            if (qi < K * VB / 4) {
                const float e = sE[c], f = sF[c];
                sST[j * PTK + c] = e * xs[i].x;
                sST[(j + 1) * PTK + c] = e * xs[i].y;
                sST[(j + 2) * PTK + c] = e * xs[i].z;
                sST[(j + 3) * PTK + c] = e * xs[i].w;
                sXT[j * PTK + c] = f * xx[i].x;
                sXT[(j + 1) * PTK + c] = f * xx[i].y;
                sXT[(j + 2) * PTK + c] = f * xx[i].z;
                sXT[(j + 3) * PTK + c] = f * xx[i].w;
            }
        }
        __syncthreads();
        if (jb + VB < V) load_slice(jb + VB);
#pragma unroll 2
        for (int ks = 0; ks < VB / 4; ++ks) {
            const int jr = 4 * ks + lq;  // the k (value column) this lane supplies
            const float bS = sST[jr * PTK + 16 * cb + lr], bX = sXT[jr * PTK + 16 * cb + lr];
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const float o = sOT[jr * PTC + 16 * b + lr], y = sYT[jr * PTC + 16 * b + lr];
                const float u = sUT[jr * PTC + 16 * b + lr];
                aQ[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(o, bS, aQ[b], 0, 0, 0);
                aKp[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(y, bS, aKp[b], 0, 0, 0);
                aKm[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(u, bX, aKm[b], 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int tt = q ? t1 : t0, ar = tt / 4, as = tt % 4;
                const float bU = sUT[jr * PTC + 16 * as + lr];
                aA[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(sYT[jr * PTC + 16 * ar + lr], bU, aA[q], 0, 0, 0);
                aP[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(sOT[jr * PTC + 16 * ar + lr], bU, aP[q], 0, 0, 0);
            }
        }
    }
    __syncthreads();
    // final phase: record tiles, masked dA = -dY U^T and dP = dO U^T, Gk, partial sums
    rows_to_lds<C, K, PK, NT>(sKp, rec + Rc::KP);
    rows_to_lds<C, K, PK, NT>(sKm, rec + Rc::KM);
    rows_to_lds<C, K, PK, NT>(sQp, rec + Rc::QP);
    rows_to_lds<C, C, PC, NT>(sG, rec + Rc::GK);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int tt = q ? t1 : t0, ar = tt / 4, as = tt % 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ar + 4 * lq + i, s2 = 16 * as + lr;
            sA[r * PC + s2] = s2 < r ? -aA[q][i] : 0.f;
            sDp[r * PC + s2] = s2 <= r ? aP[q][i] : 0.f;
        }
    }
    for (int c = t; c < K; c += NT) {
        float acc = 0.f;
        for (int w2 = 0; w2 < NVT; ++w2) acc += hp[(unit * NVT + w2) * K + c];
        sH[c] = acc;
    }
    __syncthreads();
    for (int r = t; r < C; r += NT) {  // dbeta = tiles' rowsum(R * dY) + rowsum(Gk * dA)
        float acc = 0.f;
        for (int w2 = 0; w2 < NVT; ++w2) acc += dbp[(unit * NVT + w2) * C + r];
        for (int s2 = 0; s2 < r; ++s2) acc += sG[r * PC + s2] * sA[r * PC + s2];
        if (r < L) dbeta[(size_t)(c0 + r) * H + h] = acc;
    }
    // aKp <- dA Km - dY S'^T (times beta per row below); aQ += dP Km;
    // aKm += (Diag(beta) dA)^T Kp + dP^T Qp; contractions over the C tokens
#pragma unroll
    for (int b = 0; b < RB; ++b) aKp[b] = -aKp[b];
#pragma unroll 2
    for (int ks = 0; ks < C / 4; ++ks) {
        const int sr = 4 * ks + lq;  // the token this lane supplies
        const float bKm = sKm[sr * PK + 16 * cb + lr], bKp = sKp[sr * PK + 16 * cb + lr];
        const float bQp = sQp[sr * PK + 16 * cb + lr], bs = sB[sr];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const int ar = 16 * b + lr;
            aKp[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[ar * PC + sr], bKm, aKp[b], 0, 0, 0);
            aQ[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(sDp[ar * PC + sr], bKm, aQ[b], 0, 0, 0);
            aKm[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(bs * sA[sr * PC + ar], bKp, aKm[b], 0, 0, 0);
            aKm[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(sDp[sr * PC + ar], bQp, aKm[b], 0, 0, 0);
        }
    }
    // dq, dk and D = dKp Kp - dKm Km + dQp Qp (+ h on the last row)
    float D[RB][4];
    const int c = 16 * cb + lr;
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * b + 4 * lq + i;
            const float dKp = sB[r] * aKp[b][i];
            D[b][i] = dKp * sKp[r * PK + c] - aKm[b][i] * sKm[r * PK + c] +
                      aQ[b][i] * sQp[r * PK + c] + (r == L - 1 ? sH[c] : 0.f);
            if (r < L) {
                const float ep = rec[Rc::EE + (size_t)r * K + c];
                const size_t off = ((size_t)(c0 + r) * H + h) * K + c;
                dq[off] = aQ[b][i] * ep;
                dk[off] = dKp * ep + aKm[b][i] / ep;
            }
        }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) sKp[(16 * b + 4 * lq + i) * PK + c] = D[b][i];
    __syncthreads();
    for (int c2 = t; c2 < K; c2 += NT) {  // dg = reverse running sum of D down each channel
        float acc = 0.f;
        for (int r = L - 1; r >= 0; --r) {
            acc += sKp[r * PK + c2];
            dg[((size_t)(c0 + r) * H + h) * K + c2] = acc;
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

constexpr int VT3 = 16;  // value columns per workgroup of pass 3

// Per (chunk, head): the record, the start state and end-state gradient, U and
// dY transposed, and pass 3's per-tile partial sums of dbeta and h.
template <int K, int V, int C>
size_t bwd_ws_bytes(size_t cap, int H) {
    return cap * H * (rec_bytes<K, V, C>() +
                      sizeof(float) * (2 * K * V + 2 * C * V + (V / VT3) * (C + K)));
}

// VT: value columns per chain workgroup; VB, NT4, MR, MC, AR, AC: pass 4's
// value slice, threads and per-thread tiles.
template <int K, int V, int C, int VT, int VB, int NT4, int MR, int MC, int AR, int AC,
          typename TIn>
hipError_t launch_bwd_t(const void *q, const void *k, const void *v, const void *g,
                        const void *beta, const float *s0, const float *dout, const float *dsT,
                        float *dq, float *dk, float *dv, float *dg, float *dbeta, float *ds0,
                        const int32_t *cu, int N, int fixedT, int totalT, int H, void *workspace,
                        hipStream_t stream) {
    const size_t cap = chunk_cap(N, totalT, fixedT, cu != nullptr, C);
    float *recs = static_cast<float *>(workspace);
    float *Sst = recs + cap * H * BwdRec<K, V, C>::floats;
    float *dSe = Sst + cap * H * (size_t)K * V;
    float *UTb = dSe + cap * H * (size_t)K * V;
    float *dYTb = UTb + cap * H * (size_t)C * V;
    float *dbp = dYTb + cap * H * (size_t)C * V;
    float *hpb = dbp + cap * H * (size_t)(V / VT3) * C;
    const size_t red = sizeof(int) * BNT, redP = sizeof(int) * PNT, red4 = sizeof(int) * NT4;
    const size_t lds0 = sizeof(float) * (3 * C * (K + 4) + C * K + C + K) + redP;
    const size_t ldsT = sizeof(float) * (3 * C * (K + 1) + 2 * C * (C + 1) + C + 2 * K) + redP;
    const size_t lds1 = sizeof(float) * (K * (K + 1) + K * VT) + red;
    const size_t lds2 = lds1;
    const size_t lds3 = sizeof(float) * (2 * C * (K + 1) + 2 * C * (C + 1) + 2 * K * (VT3 + 1) +
                                         5 * C * (VT3 + 1) + C + 2 * K) + redP;
    const size_t lds4 = sizeof(float) * (3 * C * (K + 1) + 3 * C * (C + 1) + C + 3 * K) + red4;
    static std::atomic<uint64_t> set0{0}, setT{0}, set1{0}, set2{0}, set3{0}, set4{0};
    auto k0 = bwd_prep_kernel<K, V, C, TIn>;
    auto kT = bwd_trans_kernel<K, V, C, TIn>;
    auto k1 = bwd_states_kernel<K, V, C, VT>;
    auto k2 = bwd_dstate_kernel<K, V, C, VT>;
    auto k3 = bwd_udy_kernel<K, V, C, VT3, TIn>;
    auto k4 = bwd_kgrad_kernel<K, V, C, VT3, VB, NT4, MR, MC, AR, AC, TIn>;
    hipError_t e;
    if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(k0), (int)lds0, set0)) != hipSuccess) return e;
    if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(kT), (int)ldsT, setT)) != hipSuccess) return e;
    if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(k1), (int)lds1, set1)) != hipSuccess) return e;
    if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(k2), (int)lds2, set2)) != hipSuccess) return e;
    if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(k3), (int)lds3, set3)) != hipSuccess) return e;
    if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(k4), (int)lds4, set4)) != hipSuccess) return e;
    const TIn *tq = static_cast<const TIn *>(q), *tk = static_cast<const TIn *>(k);
    const TIn *tv = static_cast<const TIn *>(v), *tg = static_cast<const TIn *>(g);
    const TIn *tb = static_cast<const TIn *>(beta);
    if (cap > 0) {
        hipLaunchKernelGGL(k0, dim3((unsigned)cap, H), dim3(PNT), lds0, stream, tq, tk, tg, tb, cu, N,
                           fixedT, totalT, H, recs);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if constexpr (K == 128) {
            auto kTm = bwd_trans_mfma_kernel<K, V, C, TIn>;
            static std::atomic<uint64_t> setTm{0};
            const size_t ldsTm = sizeof(float) * (3 * C * (K + 16) + 2 * C * (C + 4) + C + 2 * K) + redP;
            if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(kTm), (int)ldsTm, setTm)) != hipSuccess)
                return e;
            hipLaunchKernelGGL(kTm, dim3((unsigned)cap, H), dim3(PNT), ldsTm, stream, tv, dout, cu, N,
                               fixedT, totalT, H, recs);
        } else {
            hipLaunchKernelGGL(kT, dim3((unsigned)cap, H), dim3(PNT), ldsT, stream, tv, dout, cu, N,
                               fixedT, totalT, H, recs);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if constexpr (K != 128) {
            hipLaunchKernelGGL(k1, dim3(V / VT, H, N), dim3(BNT), lds1, stream, s0, cu, fixedT,
                               totalT, H, (int)cap, recs, Sst);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if constexpr (K == 128) {
        // both chains in one grid; z slices of at most 65535 workgroups
        for (int z0 = 0; z0 < 2 * N; z0 += 65535) {
            const int nz = std::min(65535, 2 * N - z0);
            hipLaunchKernelGGL((bwd_chain_mfma_kernel<K, V, C>), dim3(V / 16, H, nz), dim3(512), 0,
                               stream, s0, dsT, ds0, cu, N, z0, fixedT, totalT, H, (int)cap, recs,
                               Sst, dSe);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    } else {
        hipLaunchKernelGGL(k2, dim3(V / VT, H, N), dim3(BNT), lds2, stream, dsT, ds0, cu, fixedT,
                           totalT, H, (int)cap, recs, dSe);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (cap > 0) {
        if constexpr (K == 128)
            hipLaunchKernelGGL((bwd_udy_mfma_kernel<K, V, C, VT3>), dim3((unsigned)cap, H), dim3(512),
                               0, stream, reinterpret_cast<const bf16_t *>(v),
                               reinterpret_cast<const float *>(v), std::is_same<TIn, bf16_t>::value,
                               dout, cu, N, fixedT, totalT, H, recs, Sst, dSe, UTb, dYTb, dbp, hpb,
                               dv);
        else
            hipLaunchKernelGGL(k3, dim3((unsigned)cap, H), dim3(PNT), lds3, stream, tv, dout,
                               cu, N, fixedT, totalT, H, recs, Sst, dSe, UTb, dYTb, dbp, hpb, dv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if constexpr (K == 128) {
            auto k4m = bwd_kgrad_mfma_kernel<K, V, C, VT3, VB>;
            static std::atomic<uint64_t> set4m{0};
            const size_t lds4m = sizeof(float) * (3 * C * (K + 1) + 3 * C * (C + 1) + C + 3 * K) +
                                 sizeof(int) * 512;
            if ((e = ensure_dynamic_lds(reinterpret_cast<const void *>(k4m), (int)lds4m, set4m)) != hipSuccess)
                return e;
            hipLaunchKernelGGL(k4m, dim3((unsigned)cap, H), dim3(512), lds4m, stream, dout, cu, N,
                               fixedT, totalT, H, recs, Sst, dSe, UTb, dYTb, dbp, hpb, dq, dk, dg,
                               dbeta);
        } else {
            hipLaunchKernelGGL(k4, dim3((unsigned)cap, H), dim3(NT4), lds4, stream, dout, cu, N,
                               fixedT, totalT, H, recs, Sst, dSe, UTb, dYTb, dbp, hpb, dq, dk, dg,
                               dbeta);
        }
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
        return in_bf16 ? launch_bwd_t<128, 128, 64, 4, 32, 512, 4, 4, 2, 4, bf16_t>(q, k, v, g, beta, s0, dout, dsT, dq, dk, dv, dg, dbeta, ds0, cu, N, fixedT, totalT, H, workspace, stream)
                       : launch_bwd_t<128, 128, 64, 4, 32, 512, 4, 4, 2, 4, float>(q, k, v, g, beta, s0, dout, dsT, dq, dk, dv, dg, dbeta, ds0, cu, N, fixedT, totalT, H, workspace, stream);
    if (K == 32 && V == 32 && C == 16)
        return in_bf16 ? launch_bwd_t<32, 32, 16, 16, 16, 256, 1, 2, 1, 1, bf16_t>(q, k, v, g, beta, s0, dout, dsT, dq, dk, dv, dg, dbeta, ds0, cu, N, fixedT, totalT, H, workspace, stream)
                       : launch_bwd_t<32, 32, 16, 16, 16, 256, 1, 2, 1, 1, float>(q, k, v, g, beta, s0, dout, dsT, dq, dk, dv, dg, dbeta, ds0, cu, N, fixedT, totalT, H, workspace, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
