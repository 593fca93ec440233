// chunk_split.hip -- two-pass bf16 KDA forward for few (sequence, head) units.
//
// Same recurrence and chunk algebra as chunk_mfma.hip ("Kimi K3: Open
// Frontier Intelligence and Implementation Framework", section "Hybrid
// Attention Mechanism": delta rule with a channel-wise forget gate whose
// lower-bounded decay lets intra- and inter-chunk tiles run as dense
// products), reorganised for workloads whose sequential chains are too few to
// fill the GPU.  Everything that does not depend on the state is computed
// first, for all chunks at once; the sequential pass is then a short chain.
//
// With Kp, Km, Qp, A, P, G_m and G_C as in chunk_mfma.hip and
// T = (I + A)^-1 Diag(beta) (never formed):
//   W  = T Kp,   U~ = T V,   Q^ = Qp - P W,   O^ = P U~          (pass 1)
//   S' = Diag(exp(G_m)) S
//   U  = U~ - W S',   O = Q^ S' + O^,   S <- Diag(exp(G_C - G_m)) (S' + Km^T U)   (pass 2)
// (substituting U into O = Qp S' + P U gives the pass-2 form).
//
// Pass 1 (chunk_prep_kernel): one workgroup of 4 waves per (chunk, head),
// all chunks in parallel.  Pass 2 (chunk_state_kernel): one workgroup per
// (sequence, head, 16-column value tile); one state wave runs the chain with
// the state in registers while seven loader waves stream the next chunk's
// W, Q^, Km^T tiles into double-buffered LDS with direct loads.
// Intermediates live in the caller's workspace.
#include "kda_mfma.hpp"

namespace kda {
namespace {

constexpr int C = 64, KD = 128, VD = 128;
constexpr int STATE_WAVES = 1;   // state waves per workgroup in pass 2
constexpr int LOADER_WAVES = 7;  // tile-streaming waves per workgroup in pass 2
constexpr int PK = 136;  // LDS pitch (halves), [64][128] fp16 tiles
constexpr int PC = 72;   // LDS pitch (halves), [128][64] tiles read as 16-byte fragments
constexpr int P4 = 76;   // LDS pitch (halves), [64][64] tiles read as 8-byte fragments
constexpr int PI = 20;   // LDS pitch (halves), 16 x 16 fp16 blocks
constexpr int PF = 17;   // LDS pitch (floats), 16 x 16 fp32 blocks
constexpr int VTP = 68;  // LDS pitch (bf16), V^T staging tile [128][64]

// Per-(chunk, head) record in the workspace (bytes).  The contraction index
// of W, Q^ (c) and Km^T (s) is stored permuted within each 32-wide block,
// see kperm_pos below.  The first 33 KB are what the state pass streams.
constexpr size_t R_W = 0;             // fp16 [64][128]  W     [r][c]
constexpr size_t R_KMT = 16384;       // fp16 [128][64]  Diag(f) Km^T [c][s], f = the R_FC factor
constexpr size_t R_FM = 32768;        // fp32 [128]      exp(G_m)
constexpr size_t R_FC = 33280;        // fp32 [128]      exp(G_C - G_m + G_m of the next chunk)
constexpr size_t R_UT = 33792;        // fp16 [128][64]  U~    [j][r]
constexpr size_t R_QH = 50176;        // fp16 [64][128]  Q^    [r][c]
constexpr size_t R_P = 66560;         // fp16 [64][64]   P     [r][s], zero above the diagonal
constexpr size_t R_SP = 74752;        // fp16 S' as MFMA B fragments [8 tiles][4 ks][64 lanes][8]
constexpr size_t REC = 107520;
constexpr size_t OFFS_BYTES = 512;    // int32 chunk offsets, up to 127 sequences

// The pass-2 products contract over an index (c for W S' and Q^ S', s for
// Km^T U) whose right operand comes straight out of MFMA accumulators: lane l
// holds rows 4 (l >> 4) .. +3 of each 16-row block.  A 16x16x32 B fragment
// wants 8 k values per lane; taking the lane's rows of blocks 2 ks and
// 2 ks + 1 as those 8 values leaves the state in registers, provided the left
// operand's k values are laid out in the same order.  Within each 32-wide
// block, stored position 8 g + t holds logical index 4 g + t (t < 4) or
// 16 + 4 g + t - 4 (t >= 4); kperm_pos gives the stored position of the
// logical 4-group [4 q, 4 q + 4).
__device__ __forceinline__ int kperm_pos(int q) {
    return 32 * (q >> 3) + 8 * (q & 3) + 4 * ((q >> 2) & 1);
}

// W and Km^T rows and U~ columns are stored with their 16-byte blocks
// XOR-permuted by (row or column index & 7): the state pass copies them into
// LDS unchanged (linear, fully coalesced direct loads), where the permutation
// makes the 16 rows of an MFMA fragment read land in distinct banks.
// swz(x, r): stored half offset of logical half offset x within row r.
__device__ __forceinline__ int swz(int x, int r) { return (((x >> 3) ^ (r & 7)) << 3) | (x & 7); }

// ---------------------------------------------------------------- offsets
// offs[n] = first chunk of sequence n in the packed chunk list, clamped so that
// the list never exceeds `cap` chunks (malformed offsets cannot overrun the
// workspace).
__global__ void chunk_offsets_kernel(const int32_t *cu, int fixedT, int N, int totalT, int cap,
                                     int32_t *offs) {
    if (threadIdx.x != 0) return;
    int acc = 0;
    offs[0] = 0;
    for (int n = 0; n < N; ++n) {
        int bos, eos;
        seq_bounds(cu, n, fixedT, totalT, bos, eos);
        acc += (eos - bos + C - 1) / C;
        if (acc > cap) acc = cap;
        offs[n + 1] = acc;
    }
}

// Locating chunks: for N fixed-length sequences the chunk list is regular
// (sequence n owns chunks [n cps, (n + 1) cps)) and no offset table is built;
// packed sequences read the table chunk_offsets_kernel wrote.
struct ChunkMap {
    const int32_t *offs;  // nullptr for fixed-length sequences
    int cps;              // chunks per sequence (fixed length)
    __device__ __forceinline__ int first(int n) const { return offs ? offs[n] : n * cps; }
    // sequence holding packed chunk gc (gc < first(N))
    __device__ __forceinline__ int seq_of(int gc, int N) const {
        if (!offs) return gc / cps;
        int n = 0;
        while (n + 1 < N && offs[n + 1] <= gc) ++n;
        return n;
    }
};

__device__ __forceinline__ ChunkMap chunk_map(const int32_t *cu, int fixedT, const unsigned char *ws) {
    ChunkMap m;
    m.offs = cu ? reinterpret_cast<const int32_t *>(ws) : nullptr;
    m.cps = (fixedT + C - 1) / C;
    return m;
}

// ---------------------------------------------------------------- pass 1
struct PrepSmem {
    _Float16 kp[C * PK];    // Kp [s][c]
    _Float16 qp[C * PK];    // Qp [s][c], then Q^ in place
    _Float16 km[C * PK];    // Km [s][c], then W
    _Float16 a16[C * P4];   // A [r][s], off-diagonal lower blocks
    _Float16 p[C * P4];     // P [r][s], lower blocks
    _Float16 tii[4][16 * PI];
    float ad[4][16 * PF];   // diagonal A blocks, fp32
    float beta[C];
    float gsum[4][KD];      // per-wave channel sums of g
    float gnext[2][KD];     // per-wave sums of the next chunk's first 32 rows of g
};

__device__ __forceinline__ floatx4 block32(const _Float16 *lhs, const _Float16 *rhs, int bi, int bj,
                                           int lane) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        acc = mma32(frag8(lhs, PK, 16 * bi, 32 * ks, lane), frag8(rhs, PK, 16 * bj, 32 * ks, lane), acc);
    return acc;
}

__global__ __launch_bounds__(256) void chunk_prep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ g,
    const uint16_t *__restrict__ beta, const int32_t *__restrict__ cu, int fixedT, int N, int H,
    int totalT, unsigned char *__restrict__ ws) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PrepSmem &sm = *reinterpret_cast<PrepSmem *>(smem_raw);
    const ChunkMap cm = chunk_map(cu, fixedT, ws);
    const int gc = blockIdx.x, h = blockIdx.y;
    if (gc >= cm.first(N)) return;
    const int n = cm.seq_of(gc, N);
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + (gc - cm.first(n)) * C;
    const int L = min(C, eos - c0);
    // records of one head are contiguous, in chunk order
    unsigned char *rec = ws + OFFS_BYTES + ((size_t)h * gridDim.x + gc) * REC;

    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int cg = t & 15, rg = t >> 4;  // channels 8 cg .., rows 4 rg .. 4 rg + 3

    // ---- loads and the running log-decay sum
    uint4 rq[4], rk[4], rgv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = 4 * rg + u;
        rq[u] = make_uint4(0u, 0u, 0u, 0u);
        rk[u] = rq[u];
        rgv[u] = rq[u];
        if (r < L) {
            const size_t off = ((size_t)(c0 + r) * H + h) * KD + 8 * cg;
            rq[u] = *reinterpret_cast<const uint4 *>(q + off);
            rk[u] = *reinterpret_cast<const uint4 *>(k + off);
            rgv[u] = *reinterpret_cast<const uint4 *>(g + off);
        }
    }
    uint4 rv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = 4 * rg + u;
        rv[u] = make_uint4(0u, 0u, 0u, 0u);
        if (r < L) rv[u] = *reinterpret_cast<const uint4 *>(v + ((size_t)(c0 + r) * H + h) * VD + 8 * cg);
    }
    if (t < C) sm.beta[t] = t < L ? __uint_as_float((uint32_t)beta[(size_t)(c0 + t) * H + h] << 16) : 0.f;
    // The first half of the next chunk of this sequence (if any): its G_m is
    // folded into this chunk's end-of-chunk scale factor.
    uint4 rgn[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = C + 4 * rg + u;
        rgn[u] = make_uint4(0u, 0u, 0u, 0u);
        if (w < 2 && c0 + r < eos)
            rgn[u] = *reinterpret_cast<const uint4 *>(g + ((size_t)(c0 + r) * H + h) * KD + 8 * cg);
    }

    float G[4][8], ex[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) unpack8(rgv[u], G[u]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        G[1][e] += G[0][e];
        G[2][e] += G[1][e];
        G[3][e] += G[2][e];
        const float tot = G[3][e];
        float s = tot;
        float x = __shfl_up(s, 16);
        if (lg >= 1) s += x;
        x = __shfl_up(s, 32);
        if (lg >= 2) s += x;
        ex[e] = s - tot;
        if (lg == 3) sm.gsum[w][8 * cg + e] = s;
    }
    // V^T staging copy (bf16 [column][row], pitch VTP) in the A/P tiles, which
    // are not used before the Gram phase: the two waves that solve for U~
    // read it back in their MFMA accumulator layout
    {
        uint16_t *vst = reinterpret_cast<uint16_t *>(sm.a16);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint16_t c4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t wv = (&rv[u].x)[e >> 1];
                c4[u] = (uint16_t)((e & 1) ? (wv >> 16) : (wv & 0xffffu));
            }
            uint2 pk;
            pk.x = (uint32_t)c4[0] | ((uint32_t)c4[1] << 16);
            pk.y = (uint32_t)c4[2] | ((uint32_t)c4[3] << 16);
            *reinterpret_cast<uint2 *>(&vst[(8 * cg + e) * VTP + 4 * rg]) = pk;
        }
    }
    if (w < 2) {
        float gn[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) unpack8(rgn[u], gn[u]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = gn[0][e] + gn[1][e] + gn[2][e] + gn[3][e];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            if (lg == 0) sm.gnext[w][8 * cg + e] = x;
        }
    }
    __syncthreads();
    // V in the accumulator layout of waves 2, 3 (rows 16 i + 4 lg + e, column
    // 64 (w & 1) + 16 b + l16)
    uint2 vz[4][4];
    if (w >= 2) {
        const uint16_t *vst = reinterpret_cast<const uint16_t *>(sm.a16);
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vz[b][i] = *reinterpret_cast<const uint2 *>(&vst[(64 * (w & 1) + 16 * b + l16) * VTP + 16 * i + 4 * lg]);
    }
    {
        float kv[4][8], qv[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            unpack8(rk[u], kv[u]);
            unpack8(rq[u], qv[u]);
        }
        half4 kmT[8];
        half8 kpr[4], qpr[4], kmr[4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ch = 8 * cg + e;
            const float s0w = sm.gsum[0][ch], s1w = sm.gsum[1][ch], s2w = sm.gsum[2][ch],
                        s3w = sm.gsum[3][ch];
            const float gm = s0w + s1w;                 // G at token 31 (end of wave 1's rows)
            const float gcl = gm + s2w + s3w;           // G at token 63
            float pre = ex[e] - gm;
            if (w >= 1) pre += s0w;
            if (w >= 2) pre += s1w;
            if (w >= 3) pre += s2w;
            // end-of-chunk factor: exp(G_C - G_m + G_m of the next chunk)
            const float fe = fast_exp(gcl - gm + sm.gnext[0][ch] + sm.gnext[1][ch]);
            if (rg == 0) {
                reinterpret_cast<float *>(rec + R_FM)[ch] = fast_exp(gm);
                reinterpret_cast<float *>(rec + R_FC)[ch] = fe;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float f = fast_exp(pre + G[u][e]);  // exp(G - G_m)
                const float fi = __builtin_amdgcn_rcpf(f);
                kpr[u][e] = (_Float16)(kv[u][e] * f);
                qpr[u][e] = (_Float16)(qv[u][e] * f);
                kmr[u][e] = (_Float16)(kv[u][e] * fi);
                kmT[e][u] = (_Float16)(kv[u][e] * fi * fe);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 4 * rg + u;
            *reinterpret_cast<half8 *>(&sm.kp[r * PK + 8 * cg]) = kpr[u];
            *reinterpret_cast<half8 *>(&sm.qp[r * PK + 8 * cg]) = qpr[u];
            *reinterpret_cast<half8 *>(&sm.km[r * PK + 8 * cg]) = kmr[u];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 8 * cg + e;
            *reinterpret_cast<half4 *>(rec + R_KMT + 2 * ((size_t)c * C + swz(kperm_pos(rg), c))) = kmT[e];
        }
    }
    __syncthreads();

    // ---- Gram / query-key blocks: wave w takes the diagonal blocks (w, w) and
    // three of the twelve off-diagonal blocks, then inverts I + A_ww.
    {
        const floatx4 a = block32(sm.kp, sm.km, w, w, lane);
        float *ad = sm.ad[w];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lg + i;
            ad[r * PF + l16] = l16 < r ? sm.beta[16 * w + r] * a[i] : 0.f;
        }
        const floatx4 pq = block32(sm.qp, sm.km, w, w, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lg + i;
            sm.p[(16 * w + r) * P4 + 16 * w + l16] = (_Float16)(l16 <= r ? pq[i] : 0.f);
        }
#pragma unroll
        for (int tsk = 0; tsk < 3; ++tsk) {
            const int o = 3 * w + tsk, oo = o % 6;
            const bool gram = o < 6;
            const int bi = oo < 1 ? 1 : (oo < 3 ? 2 : 3);
            const int bj = oo < 1 ? 0 : (oo < 3 ? oo - 1 : oo - 3);
            const floatx4 acc = block32(gram ? sm.kp : sm.qp, sm.km, bi, bj, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * bi + 4 * lg + i, s = 16 * bj + l16;
                if (gram)
                    sm.a16[r * P4 + s] = (_Float16)(sm.beta[r] * acc[i]);
                else
                    sm.p[r * P4 + s] = (_Float16)acc[i];
            }
        }
        // (I + A_ww)^-1: quad 4j..4j+3 owns column j, lane q sums s = q (mod 4)
        const int j = lane >> 2, qd = lane & 3;
        float coef[4][16];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) coef[m][r] = (4 * m < r) ? ad[r * PF + 4 * m + qd] : 0.f;
        float t_own[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float part = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                if (4 * m < r) part += coef[m][r] * t_own[m];
            part += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, part), 0xB1, 0xF, 0xF, true));
            part += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, part), 0x4E, 0xF, 0xF, true));
            const float tr = (r == j ? 1.f : 0.f) - part;
            if ((r & 3) == qd) t_own[r >> 2] = tr;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) sm.tii[w][(4 * m + qd) * PI + j] = (_Float16)t_own[m];
    }
    __syncthreads();

    // ---- (I + A) [W | U~] = Diag(beta) [Kp | V] by 16-row block substitution.
    // Waves 0, 1 solve for the Kp columns (W), waves 2, 3 for the V columns (U~);
    // each wave owns four 16-column blocks.
    const bool wside = w < 2;
    // Right-hand sides for all (i, b) first (their LDS reads all in flight
    // together), then row block i outer, the four independent column blocks
    // inner.
    float zx[4][4][4];  // [i][b][e]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * i + 4 * lg + e, col = 64 * (w & 1) + 16 * b + l16;
                const uint32_t vw = (e < 2) ? vz[b][i].x : vz[b][i].y;
                zx[i][b][e] = wside ? (float)sm.kp[r * PK + col]
                                    : __uint_as_float((e & 1) ? (vw & 0xffff0000u) : (vw << 16));
            }
    half4 Xh[4][4];  // [column block][row block]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const floatx4 bt = *reinterpret_cast<const floatx4 *>(&sm.beta[16 * i + 4 * lg]);
        const half4 ti = frag4(sm.tii[i], PI, 0, 0, lane);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            floatx4 z;
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] = bt[e] * zx[i][b][e];
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < i; ++jj) acc = mma16(frag4(sm.a16, P4, 16 * i, 16 * jj, lane), Xh[b][jj], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] -= acc[e];
            Xh[b][i] = to_half4(mma16(ti, to_half4(z), floatx4{0.f, 0.f, 0.f, 0.f}));
        }
    }
    // ---- Q^ = Qp - P W (waves 0, 1, in place over Qp; W into the Km tile).
    // The product is formed transposed, (P W)^T = W^T P^T: a lane's W
    // accumulator block read as a 16x16x16 A operand is a block of W^T, and
    // P's row fragment serves as the B operand, so each lane ends up with four
    // consecutive columns of one row: one 8-byte read-modify-write of Qp.
    if (wside) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i <= rb; ++i) acc = mma16(Xh[b][i], frag4(sm.p, P4, 16 * rb, 16 * i, lane), acc);
                _Float16 *qrow = &sm.qp[(16 * rb + l16) * PK + 64 * (w & 1) + 16 * b + 4 * lg];
                half4 qv = *reinterpret_cast<const half4 *>(qrow);
#pragma unroll
                for (int e = 0; e < 4; ++e) qv[e] = (_Float16)((float)qv[e] - acc[e]);
                *reinterpret_cast<half4 *>(qrow) = qv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.km[(16 * rb + 4 * lg + e) * PK + 64 * (w & 1) + 16 * b + l16] = Xh[b][rb][e];
            }
        }
    }
    __syncthreads();
    // U~ (waves 2, 3) into a staging copy laid out as in the record, over the
    // Kp tile (no longer read), for linear global stores below
    if (!wside) {
        _Float16 *stage = sm.kp;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int col = 64 * (w & 1) + 16 * b + l16;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
                *reinterpret_cast<half4 *>(&stage[col * C + swz(16 * rb + 4 * lg, col)]) = Xh[b][rb];
        }
    }
    // ---- W and Q^ rows to the workspace, k-permuted (16-byte stores: stored
    // block b of a row takes logical 4-groups 8 (b >> 2) + (b & 3) and that + 4)
    // (stored 16-byte block bp of a W row holds logical block bp ^ (r & 7))
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = 256 * e + t, r = idx >> 4, bp = idx & 15;
        half8 wv, qv;
        {
            const int b = bp ^ (r & 7), l0 = 32 * (b >> 2) + 4 * (b & 3), l1 = l0 + 16;
            const half4 w0 = *reinterpret_cast<const half4 *>(&sm.km[r * PK + l0]);
            const half4 w1 = *reinterpret_cast<const half4 *>(&sm.km[r * PK + l1]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wv[i] = w0[i];
                wv[4 + i] = w1[i];
            }
        }
        {
            const int l0 = 32 * (bp >> 2) + 4 * (bp & 3), l1 = l0 + 16;
            const half4 q0 = *reinterpret_cast<const half4 *>(&sm.qp[r * PK + l0]);
            const half4 q1 = *reinterpret_cast<const half4 *>(&sm.qp[r * PK + l1]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qv[i] = q0[i];
                qv[4 + i] = q1[i];
            }
        }
        *reinterpret_cast<half8 *>(rec + R_W + 2 * ((size_t)r * KD + 8 * bp)) = wv;
        *reinterpret_cast<half8 *>(rec + R_QH + 2 * ((size_t)r * KD + 8 * bp)) = qv;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = 256 * e + t;
        *reinterpret_cast<uint4 *>(rec + R_UT + 16 * idx) = *reinterpret_cast<const uint4 *>(&sm.kp[8 * idx]);
    }
    // ---- P rows, with the blocks above the diagonal zeroed (16-byte stores)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int idx = 256 * e + t, r = idx >> 3, b = idx & 7;
        half8 pv;
        if ((b >> 1) > (r >> 4)) {
#pragma unroll
            for (int i = 0; i < 8; ++i) pv[i] = (_Float16)0.f;
        } else {
            const half4 p0 = *reinterpret_cast<const half4 *>(&sm.p[r * P4 + 8 * b]);
            const half4 p1 = *reinterpret_cast<const half4 *>(&sm.p[r * P4 + 8 * b + 4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[i] = p0[i];
                pv[4 + i] = p1[i];
            }
        }
        *reinterpret_cast<half8 *>(rec + R_P + 2 * ((size_t)r * C + 8 * b)) = pv;
    }
}

// ---------------------------------------------------------------- pass 2
// One chunk's state-pass operands in LDS, for a workgroup owning VT = 16 NSW
// value columns: W ([64][128] fp16) and Km^T ([128][64] fp16) without padding,
// each row's 16-byte blocks XOR-permuted by (row & 7) as stored (swz); the
// scale factors; then the workgroup's columns of U~ (blocks permuted by the
// column index).  Loader waves copy it with direct global-to-LDS loads in
// wave-wide 1 KB segments.
template <int NSW>
struct ChunkTiles {
    _Float16 w[C * KD];
    _Float16 kmt[KD * C];
    float fmc[2 * KD];
    _Float16 ut[16 * NSW * C];  // [j][r]
};
static_assert(sizeof(ChunkTiles<1>) == 35 * 1024, "segment count");

// NSW state waves own 16 value columns each; NLW loader waves stream the
// tiles (one CU sustains its highest direct-load rate only with several
// waves' loads in flight).
template <int NSW, int NLW>
struct StateSmem {
    ChunkTiles<NSW> buf[3];  // chunk ci in buf[ci % 3]
};

// Workgroup barrier for the loader waves, which touch LDS only through their
// direct loads and wait for those explicitly: no fence, so the compiler adds
// no waits of its own.
__device__ __forceinline__ void loader_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Global source of LDS slot p (16-byte units) of a ChunkTiles<NSW> image for
// value columns [col0, col0 + 16 NSW): the record's first 33 KB (W, Km^T,
// scale factors) and the tile's U~ columns, both copied linearly.
template <int NSW>
__device__ __forceinline__ const unsigned char *tile_source(const unsigned char *rec, int p,
                                                            int col0) {
    constexpr int HEAD = (int)(R_UT / 16);  // 2112
    return p < HEAD ? rec + 16 * p : rec + R_UT + 128 * col0 + 16 * (p - HEAD);
}

// One direct global-to-LDS load: 16 bytes per lane from `src`, landing at
// lds + 16 lane (lds is wave-uniform).
__device__ __forceinline__ void lds_dma16(const unsigned char *src, unsigned char *lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }

template <int NSW, int NLW>
__device__ __forceinline__ void load_tiles(unsigned char *dst, const unsigned char *rec, int col0,
                                           int lw, int lane) {
    constexpr int SEGMENTS = (int)(sizeof(ChunkTiles<NSW>) / 1024);
#pragma unroll
    for (int s = lw; s < SEGMENTS; s += NLW) {
        const unsigned char *src = tile_source<NSW>(rec, 64 * s + lane, col0);
        lds_dma16(src, dst + 1024 * s);
    }
}

// 16x16x32 fragment from a swizzled tile with `rowlen` halves per row.
__device__ __forceinline__ half8 frag8_sw(const _Float16 *base, int rowlen, int row0, int ks,
                                          int lane) {
    const int r = row0 + (lane & 15);
    const int kb = (4 * ks + (lane >> 4)) ^ (r & 7);
    return *reinterpret_cast<const half8 *>(base + r * rowlen + 8 * kb);
}

// B fragment of a k-permuted product from accumulator blocks 2 ks, 2 ks + 1.
__device__ __forceinline__ half8 bfrag(const floatx4 &lo, const floatx4 &hi) {
    half8 b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b[i] = (_Float16)lo[i];
        b[4 + i] = (_Float16)hi[i];
    }
    return b;
}

// W fragments of one chunk for the state wave: 16x16x32 A operands for the
// four row blocks and four k-steps.
template <int NSW>
__device__ __forceinline__ void load_w(half8 (&a)[4][4], const ChunkTiles<NSW> &tl, int lane) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) a[ks][rb] = frag8_sw(tl.w, KD, 16 * rb, ks, lane);
}

// One chunk of the state chain for state wave `sw` (16 value columns), all in
// registers: the left operands and U~ come from the LDS tiles, the right
// operands are the wave's own accumulators, which hold S' = Diag(exp(G_m)) S
// on entry.  S' is published (as the
// fp16 B fragments the output product needs) to the chunk's record.  Each
// phase's LDS reads are issued as a group ahead of the arithmetic that
// consumes them.
template <int NSW>
__device__ __forceinline__ void state_chunk(floatx4 (&S)[8], const ChunkTiles<NSW> &tl,
                                            unsigned char *sp_out, int sw, int lane) {
    const int lg = lane >> 4, j = 16 * sw + (lane & 15);
    half8 a[4][4];
    load_w<NSW>(a, tl, lane);
    floatx4 f[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) f[cb] = *reinterpret_cast<const floatx4 *>(&tl.fmc[KD + 16 * cb + 4 * lg]);
    half4 ut[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const int blk = (2 * rb + (lg >> 1)) ^ (j & 7);
        ut[rb] = *reinterpret_cast<const half4 *>(&tl.ut[j * C + 8 * blk + 4 * (lg & 1)]);
    }
    __builtin_amdgcn_sched_barrier(0);  // all of the reads above in flight before the products
    half8 bs[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bs[ks] = bfrag(S[2 * ks], S[2 * ks + 1]);
    // X = W S'
    floatx4 X[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) X[rb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) X[rb] = mma32(a[ks][rb], bs[ks], X[rb]);
    half8 k2[2][8];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) k2[ks][cb] = frag8_sw(tl.kmt, C, 16 * cb, ks, lane);
    // Diag(f) S', the accumulator the state update adds onto (off the chain,
    // while the products above run)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[cb][i] *= f[cb][i];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        *reinterpret_cast<half8 *>(sp_out + 1024 * ks + 16 * lane) = bs[ks];
    __builtin_amdgcn_sched_barrier(0);
    // U = U~ - X
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) X[rb][e] = (float)ut[rb][e] - X[rb][e];
    half8 bu[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) bu[ks] = bfrag(X[2 * ks], X[2 * ks + 1]);
    // S'' = Diag(f) (S' + Km^T U) = Diag(f) S' + (Diag(f) Km^T) U with
    // f = exp(G_C - G_m + G_m'): the next chunk's S' (G_m' its mid-chunk
    // reference; for a sequence's last chunk f = exp(G_C - G_m), which leaves S
    // itself).  The record holds Km^T already scaled by f.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) S[cb] = mma32(k2[ks][cb], bu[ks], S[cb]);
}

// Grid: one workgroup per (unit, value tile), XCD-aware: workgroup b runs on
// XCD b mod 8, and all value tiles of a unit share that XCD (and its L2),
// which serves their common W, Km^T tiles.  Waves: NSW state waves, NLW
// loader waves; one barrier per chunk.
template <int NSW, int NLW>
__global__ __launch_bounds__(64 * (NSW + NLW)) void chunk_state_kernel(
    const float *s0, float *sT, const int32_t *__restrict__ cu, int fixedT, int N, int H,
    int totalT, int cap, unsigned char *__restrict__ ws) {
    constexpr int VTILE = 16 * NSW, NVT = VD / VTILE;
    constexpr int SEGS = (int)(sizeof(ChunkTiles<NSW>) / 1024);
    extern __shared__ __align__(16) unsigned char smem_raw[];
    StateSmem<NSW, NLW> &sm = *reinterpret_cast<StateSmem<NSW, NLW> *>(smem_raw);
    const ChunkMap cm = chunk_map(cu, fixedT, ws);
    const int b = blockIdx.x, slot = b >> 3;
    const int vt = slot % NVT;
    const int unit = (slot / NVT) * 8 + (b & 7);
    if (unit >= N * H) return;
    const int n = unit / H, h = unit - n * H;
    const int ch0 = cm.first(n);
    const int nchunks = cm.first(n + 1) - ch0;
    unsigned char *recs = ws + OFFS_BYTES;
    auto rec = [&](int ci) { return recs + ((size_t)h * cap + ch0 + ci) * REC; };
    const int col0 = vt * VTILE;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lg = lane >> 4;

    if (w < NSW) {
        const int jcol = col0 + 16 * w + (lane & 15);  // this lane's value column
        const size_t sbase = (size_t)unit * (KD * VD) + jcol;
        const int tile = (col0 >> 4) + w;                // 16-column tile of the S' record
        floatx4 S[8];
        if (s0) {
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[cb][i] = s0[sbase + (size_t)(16 * cb + 4 * lg + i) * VD];
        } else {
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) S[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();
        if (nchunks > 0) {
            // S' of the first chunk; later chunks receive theirs from the
            // previous chunk's end-of-chunk factor
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const floatx4 f = *reinterpret_cast<const floatx4 *>(&sm.buf[0].fmc[16 * cb + 4 * lg]);
#pragma unroll
                for (int i = 0; i < 4; ++i) S[cb][i] *= f[i];
            }
        }
        for (int ci = 0; ci < nchunks; ++ci) {
            state_chunk<NSW>(S, sm.buf[ci % 3], rec(ci) + R_SP + 4096 * tile, w, lane);
            __syncthreads();
        }
        if (sT) {
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) sT[sbase + (size_t)(16 * cb + 4 * lg + i) * VD] = S[cb][i];
        }
    } else {
        // Loader waves, three buffers: while the state waves work on chunk ci,
        // chunk ci + 2 is issued into the buffer chunk ci - 1 used, and the
        // loads of chunk ci + 1 (issued one chunk earlier) must land before the
        // barrier that ends chunk ci; loads complete in issue order, so a wave
        // waits until no more than its ci + 2 loads are outstanding.  Each load
        // thus has two chunk times to arrive.
        static_assert(SEGS % NLW == 0, "equal load counts per loader wave");
        constexpr int PER_WAVE = SEGS / NLW;
        const int lw = w - NSW;
        auto issue = [&](int ci) {
            load_tiles<NSW, NLW>(reinterpret_cast<unsigned char *>(&sm.buf[ci % 3]), rec(ci), col0, lw, lane);
        };
        for (int c = 0; c < 2 && c < nchunks; ++c) issue(c);
        if (nchunks > 1)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_WAVE));  // chunk 0 landed
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        for (int ci = 0; ci < nchunks; ++ci) {
            if (ci + 2 < nchunks) {
                issue(ci + 2);
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_WAVE));
            } else {
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
            loader_barrier();
        }
    }
}

template <int NSW, int NLW>
hipError_t launch_state(const float *s0, float *sT, const int32_t *cu, int N, int fixedT,
                        int totalT, int H, int cap, unsigned char *ws, hipStream_t stream) {
    auto kern = chunk_state_kernel<NSW, NLW>;
    constexpr int smem = (int)sizeof(StateSmem<NSW, NLW>);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    const int groups = (N * H + 7) / 8;
    hipLaunchKernelGGL(kern, dim3(groups * 8 * (VD / (16 * NSW))), dim3(64 * (NSW + NLW)), smem,
                       stream, s0, sT, cu, fixedT, N, H, totalT, cap, ws);
    return hipGetLastError();
}

// ---------------------------------------------------------------- pass 3
// O = Q^ S' + P U~ for every (chunk, head) at once: one workgroup of 4 waves
// per record, wave w producing value tiles 2 w and 2 w + 1 (16 columns each).
// Operands are read as MFMA fragments straight from the record (Q^ with its
// permuted contraction index matching the S' fragments; P and U~ in natural
// order); outputs leave through a buffer resource spanning the chunk's valid
// rows.
__device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t r, int off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
}
__device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t r, int off, bf16_t x) {
    __builtin_amdgcn_raw_buffer_store_b16(x.bits, r, off, 0, 0);
}

template <typename TOut>
__global__ __launch_bounds__(256) void chunk_output_kernel(TOut *__restrict__ o,
                                                           const int32_t *__restrict__ cu,
                                                           int fixedT, int N, int H, int totalT,
                                                           const unsigned char *__restrict__ ws) {
    const ChunkMap cm = chunk_map(cu, fixedT, ws);
    const int gc = blockIdx.x, h = blockIdx.y;
    if (gc >= cm.first(N)) return;
    const int n = cm.seq_of(gc, N);
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + (gc - cm.first(n)) * C;
    const int L = min(C, eos - c0);
    const unsigned char *rec = ws + OFFS_BYTES + ((size_t)h * gridDim.x + gc) * REC;

    const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    half8 aq[4][4], ap[2][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            aq[ks][rb] = *reinterpret_cast<const half8 *>(rec + R_QH + 2 * ((16 * rb + l16) * KD + 8 * (4 * ks + lg)));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            ap[ks][rb] = *reinterpret_cast<const half8 *>(rec + R_P + 2 * ((16 * rb + l16) * C + 32 * ks + 8 * lg));
    const int row_bytes = H * VD * (int)sizeof(TOut);
    __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        o + (size_t)c0 * H * VD, 0, L * row_bytes, 0x00020000);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int tile = 2 * w + tt, j = 16 * tile + l16;
        half8 bs[4], bu[2];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            bs[ks] = *reinterpret_cast<const half8 *>(rec + R_SP + 4096 * tile + 1024 * ks + 16 * lane);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            bu[ks] = *reinterpret_cast<const half8 *>(rec + R_UT + 2 * (j * C + swz(32 * ks + 8 * lg, j)));
        floatx4 Y[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) Y[rb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) Y[rb] = mma32(ap[ks][rb], bu[ks], Y[rb]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) Y[rb] = mma32(aq[ks][rb], bs[ks], Y[rb]);
        const int lane_off = ((4 * lg * H + h) * VD + j) * (int)sizeof(TOut);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                store_elem(orsrc, lane_off + (16 * rb + e) * row_bytes, from_f32<TOut>(Y[rb][e]));
    }
}

int max_chunks(int N, int totalT, int fixedT, bool varlen) {
    if (!varlen) return N * ((fixedT + C - 1) / C);
    return (int)(((long long)totalT + (long long)(C - 1) * N + C - 1) / C);
}

}  // namespace

// The two-pass path serves bf16 inputs with (K, V, C) = (128, 128, 64) and
// fewer than 127 sequences.  It beats the single-pass kernel while its pass-2
// workgroups (8 per unit) leave the GPU underfilled and sequences are long
// enough to amortise the extra launches: up to 32 units, at least 8 chunks
// per sequence on average.
bool chunk_split_supported(int N, int H, int K, int V, int Cc) {
    return K == KD && V == VD && Cc == C && N > 0 && N < 127 && H > 0;
}

bool chunk_split_recommended(int N, int totalT, int H, int K, int V, int Cc) {
    return chunk_split_supported(N, H, K, V, Cc) && (long long)N * H <= 32 &&
           (long long)totalT >= 8LL * C * N;
}

size_t chunk_split_workspace_bytes(int N, int totalT, int H) {
    return OFFS_BYTES + (size_t)max_chunks(N, totalT, 0, true) * H * REC;
}

hipError_t launch_chunk_split(const void *q, const void *k, const void *v, const void *g,
                              const void *beta, const float *s0, void *o, float *sT,
                              const int32_t *cu, int N, int fixedT, int totalT, int H,
                              bool out_bf16, void *workspace, hipStream_t stream) {
    if (N == 0 || H == 0) return hipSuccess;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const int cap = max_chunks(N, totalT, fixedT, cu != nullptr);
    hipError_t e;
    if (cu) {
        hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(64), 0, stream, cu, fixedT, N,
                           totalT, cap, reinterpret_cast<int32_t *>(ws));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (cap > 0) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(chunk_prep_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(PrepSmem));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(chunk_prep_kernel, dim3(cap, H), dim3(256), sizeof(PrepSmem), stream,
                           static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                           static_cast<const uint16_t *>(v), static_cast<const uint16_t *>(g),
                           static_cast<const uint16_t *>(beta), cu, fixedT, N, H, totalT, ws);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    e = launch_state<STATE_WAVES, LOADER_WAVES>(s0, sT, cu, N, fixedT, totalT, H, cap, ws, stream);
    if (e != hipSuccess || cap == 0) return e;
    if (out_bf16)
        hipLaunchKernelGGL(chunk_output_kernel<bf16_t>, dim3(cap, H), dim3(256), 0, stream,
                           static_cast<bf16_t *>(o), cu, fixedT, N, H, totalT, ws);
    else
        hipLaunchKernelGGL(chunk_output_kernel<float>, dim3(cap, H), dim3(256), 0, stream,
                           static_cast<float *>(o), cu, fixedT, N, H, totalT, ws);
    return hipGetLastError();
}

}  // namespace kda
