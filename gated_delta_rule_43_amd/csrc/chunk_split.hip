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
// With Kp, Km, Qp, A, P, G_m and G_C as in chunk_mfma.hip, S the state at
// the chunk's start, E = Diag(exp(G_m)) and T = (I + A)^-1 Diag(beta) (never
// formed):
//   W  = T Kp,   U~ = T V,   Q^ = (Qp - P W) E,   O^ = P U~,
//   M' = -Diag(exp(G_C - G_m)) Km^T W E,
//   N  =  Diag(exp(G_C - G_m)) Km^T U~,   f = exp(G_C)                 (pass 1)
//   S <- Diag(f) S + M' S + N                                          (pass 2)
//   O  = Q^ S + O^                                                     (pass 3)
// which is the chunk update S <- Diag(exp(G_C)) S + Diag(exp(G_C - G_m))
// Km^T (U~ - W E S) and output O = (Qp - P W) E S + P U~ regrouped.  The
// mid-chunk reference G_m keeps Kp, Km and Qp (fp16 MFMA operands) within
// e^+-8; the column factor E is applied in fp32 before the one rounding of
// Q^ and M' to fp16, whose entries then have magnitude of at most those of
// q and of an undecayed update.  Each chunk's records depend on that chunk
// alone.
//
// Pass 1 (chunk_prep_kernel): one workgroup of 4 waves per (chunk, head), all
// chunks in parallel.  Pass 2 (chunk_state_kernel): one workgroup per
// (sequence, head, 16-column value tile); four state waves run the chain with
// the state in registers (one 128 x 128 x 16 product per chunk) while four
// loader waves stream the next chunks' M', N and f into LDS with direct loads.
// Pass 3 (chunk_output_kernel): one workgroup per (chunk, head).
// Intermediates live in the caller's workspace.
#include "kda_mfma.hpp"
#include "prologue.hpp"
#include "state_io.hpp"

namespace kda {
namespace {

constexpr int C = 64, KD = 128, VD = 128;
constexpr int STATE_WAVES = 4;   // pass-2 waves running the chain (128 / STATE_WAVES state rows each)
constexpr int LOADER_WAVES = 4;  // pass-2 waves streaming the tiles
constexpr int RBW = 8 / STATE_WAVES;  // 16-row blocks of the state per state wave
constexpr int KSW = 4 / STATE_WAVES;  // k-steps whose B fragments a state wave owns
constexpr int NBUF = 4;          // pass-2 LDS buffers (chunk ci in buffer ci % 4)
constexpr int PK = 136;  // LDS pitch (halves), [64][128] fp16 tiles
constexpr int P4 = 76;   // LDS pitch (halves), [64][64] tiles read as 8-byte fragments
constexpr int PI = 20;   // LDS pitch (halves), 16 x 16 fp16 blocks
constexpr int PF = 17;   // LDS pitch (floats), 16 x 16 fp32 blocks
constexpr int VTP = 68;  // LDS pitch (bf16), V^T staging tile [128][64]

// Per-(chunk, head) record in the workspace (bytes).  "A order" / "B order":
// MFMA 16x16x32 operand fragments stored lane by lane, [block][k-step][64
// lanes][8 halves], so that a wave reads a fragment as one contiguous 1 KB.
// Q^'s contraction index is stored permuted within each 32-wide block (see
// kperm_pos).  M', f and one value tile's 4 KB of N (36.5 KB) are what the
// state pass streams per chunk.
constexpr size_t R_M = 0;         // fp16 M' in A order [8 row blocks][4 k-steps]
constexpr size_t R_N = 32768;     // fp16 N as accumulators [8 value tiles][8 row blocks][64 lanes][4]
constexpr size_t R_FC = 65536;    // fp32 [128]  f
constexpr size_t R_OH = 66048;    // fp16 O^ as accumulators [8 value tiles][4 row blocks][64 lanes][4]
constexpr size_t R_QH = 82432;    // fp16 Q^ in A order [4 row blocks][4 k-steps]
constexpr size_t R_SP = 98816;    // fp16 S (chunk-start state) in B order [8 value tiles][4 k-steps]
constexpr size_t REC = 131584;

// Several products take an operand straight out of MFMA accumulators, where
// lane l holds rows 4 (l >> 4) .. +3 of each 16-row block: the state S (in
// M' S and Q^ S), and W and U~ (in M' and N).  A 16x16x32 fragment wants 8
// k values per lane; taking the lane's rows of blocks 2 ks and 2 ks + 1 as
// those 8 values keeps the operand in registers, provided the other operand's
// k values are laid out in the same order.  Within each 32-wide block, stored
// position 8 g + t holds logical index 4 g + t (t < 4) or 16 + 4 g + t - 4
// (t >= 4); kperm_pos gives the stored position of the logical 4-group
// [4 q, 4 q + 4).
__device__ __forceinline__ int kperm_pos(int q) {
    return 32 * (q >> 3) + 8 * (q & 3) + 4 * ((q >> 2) & 1);
}

// ---------------------------------------------------------------- chunk map
// Fixed-length sequences own regular ranges of the chunk list (sequence n:
// [n cps, (n + 1) cps)).  For packed sequences every wave derives the map from
// cu itself: lane l counts the chunks of sequences l and l + 64, a wave-wide
// inclusive scan turns the counts into each sequence's end chunk, and lookups
// read one lane (the index is wave-uniform) or count lanes with a ballot.  End
// chunks are clamped to cap, the list's capacity, so malformed offsets cannot
// overrun the workspace.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    return x;
}

struct ChunkMap {
    bool packed;
    int cps;             // chunks per sequence (fixed length)
    int N;
    int end_lo, end_hi;  // end chunk of sequences lane and lane + 64 (packed)
    __device__ __forceinline__ int first(int n) const {
        if (!packed) return n * cps;
        if (n <= 0) return 0;
        const int m = n - 1;  // first(n) = end of sequence n - 1
        return m < 64 ? __builtin_amdgcn_readlane(end_lo, m) : __builtin_amdgcn_readlane(end_hi, m - 64);
    }
    // sequence holding chunk gc (gc < first(N)): the number of sequences
    // ending at or before it
    __device__ __forceinline__ int seq_of(int gc) const {
        if (!packed) return gc / cps;
        const int lane = __lane_id();
        return __popcll(__ballot(lane < N && end_lo <= gc)) +
               __popcll(__ballot(lane + 64 < N && end_hi <= gc));
    }
};

__device__ __forceinline__ ChunkMap chunk_map(const int32_t *cu, int fixedT, int N, int totalT,
                                              int cap) {
    ChunkMap m;
    m.packed = cu != nullptr;
    m.cps = (fixedT + C - 1) / C;
    m.N = N;
    m.end_lo = m.end_hi = 0;
    if (m.packed) {
        const int lane = __lane_id();
        int c_lo = 0, c_hi = 0, bos, eos;
        if (lane < N) {
            seq_bounds(cu, lane, 0, totalT, bos, eos);
            c_lo = (eos - bos + C - 1) / C;
        }
        if (lane + 64 < N) {
            seq_bounds(cu, lane + 64, 0, totalT, bos, eos);
            c_hi = (eos - bos + C - 1) / C;
        }
        const int s_lo = wave_incl_scan(c_lo, lane);
        m.end_lo = min(s_lo, cap);
        if (N > 64) {
            const int s_hi = wave_incl_scan(c_hi, lane) + __builtin_amdgcn_readlane(s_lo, 63);
            m.end_hi = min(s_hi, cap);
        }
    }
    return m;
}

// ---------------------------------------------------------------- pass 1
// Diag(f) Km^T tile of pass 1 ([128][64] fp16, no padding): half offset of the
// logical 4-group q of row c (the contraction index s permuted as kperm_pos
// says, then the row's 16-byte blocks XOR-permuted by kt_swz(c)), and of the
// 16x16x32 fragment (rows 16 cb .. +15, k-step ks) a lane reads.  The rows of
// a fragment read (16 consecutive c) and of one write instruction (c = 8 cg +
// e for 16 values of cg) both get 8 distinct swizzles, so neither piles onto
// one bank group.
__device__ __forceinline__ int kt_swz(int c) { return (c ^ (c >> 3)) & 7; }
__device__ __forceinline__ int kt_off(int c, int q) {
    const int pos = kperm_pos(q);
    return c * C + (((pos >> 3) ^ kt_swz(c)) << 3) + (pos & 7);
}
__device__ __forceinline__ int kt_frag_off(int cb, int ks, int lane) {
    const int c = 16 * cb + (lane & 15);
    return c * C + (((4 * ks + (lane >> 4)) ^ kt_swz(c)) << 3);
}
// Two accumulator blocks (16 rows each) of one lane as the 8 k values of a
// 16x16x32 fragment in permuted order (block 2 ks first, then 2 ks + 1).
__device__ __forceinline__ half8 pair8(half4 lo, half4 hi) {
    half8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = lo[i];
        r[4 + i] = hi[i];
    }
    return r;
}

struct PrepSmem {
    _Float16 kp[C * PK];    // Kp [s][c], then Diag(f) Km^T (see kt_off)
    _Float16 qp[C * PK];    // Qp [s][c], then Q^ in place
    _Float16 km[C * PK];    // Km [s][c]
    _Float16 a16[C * P4];   // A [r][s], off-diagonal lower blocks
    _Float16 p[C * P4];     // P [r][s], lower blocks
    _Float16 tii[4][16 * PI];
    float ad[4][16 * PF];   // diagonal A blocks, fp32
    float beta[C];
    float gsum[4][KD];      // per-wave channel sums of g
    float egm[KD];          // exp(G_m)
};

__device__ __forceinline__ floatx4 block32(const _Float16 *lhs, const _Float16 *rhs, int bi, int bj,
                                           int lane) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        acc = mma32(frag8(lhs, PK, 16 * bi, 32 * ks, lane), frag8(rhs, PK, 16 * bj, 32 * ks, lane), acc);
    return acc;
}

template <int PM>
__global__ __launch_bounds__(256) void chunk_prep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ g,
    const uint16_t *__restrict__ beta, const int32_t *__restrict__ cu, int fixedT, int N, int H,
    int totalT, Prologue pro, unsigned char *__restrict__ ws) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PrepSmem &sm = *reinterpret_cast<PrepSmem *>(smem_raw);
    const ChunkMap cm = chunk_map(cu, fixedT, N, totalT, gridDim.x);
    const int gc = blockIdx.x, h = blockIdx.y;
    if (gc >= cm.first(N)) return;
    const int n = cm.seq_of(gc);
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + (gc - cm.first(n)) * C;
    const int L = min(C, eos - c0);
    // records of one head are contiguous, in chunk order
    unsigned char *rec = ws + ((size_t)h * gridDim.x + gc) * REC;

    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int cg = t & 15, rg = t >> 4;  // channels 8 cg .., rows 4 rg .. 4 rg + 3

    // ---- loads, issued unconditionally (rows past the chunk's end re-read
    // its last row and are zeroed afterwards) and in the order they are
    // needed: g (the gate scan and every decay factor), then k and q (the
    // scaled operands), then v (staged last), so that the scan and the
    // exponentials run while the later rows are still arriving.
    uint4 rq[4], rk[4], rgv[4], rv[4];
    size_t off[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) off[u] = ((size_t)(c0 + min(4 * rg + u, L - 1)) * H + h) * KD + 8 * cg;
    // beta of row t & 63 (every wave loads it, so that no wave waits on a
    // load of its own before issuing the rest; wave 0 stores it)
    const uint16_t bt_raw = beta[(size_t)(c0 + min(t & 63, L - 1)) * H + h];
#pragma unroll
    for (int u = 0; u < 4; ++u) rgv[u] = *reinterpret_cast<const uint4 *>(g + off[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) rk[u] = *reinterpret_cast<const uint4 *>(k + off[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) rq[u] = *reinterpret_cast<const uint4 *>(q + off[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) rv[u] = *reinterpret_cast<const uint4 *>(v + off[u]);
    const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
    // padding rows: zeros, and gate logits that map to g = 0
    const uint32_t gpad = pro_on<PM>(pro, PRO_GATE_LOGIT) ? BF16_NEG_INF_PAIR : 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (4 * rg + u >= L) {
            rq[u] = zero4;
            rk[u] = zero4;
            rgv[u] = make_uint4(gpad, gpad, gpad, gpad);
            rv[u] = zero4;
        }
    }

    // ---- running log-decay sum: within the thread's 4 rows, then across the
    // wave's 4 row groups (two shuffles, all 8 channels together), then across
    // waves through LDS
    float G[4][8], ex[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) unpack8(rgv[u], G[u]);
    if (pro_on<PM>(pro, PRO_GATE_LOGIT)) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) G[u][e] = gate_from_logit(G[u][e], pro.glb);
    }
    float sc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        G[1][e] += G[0][e];
        G[2][e] += G[1][e];
        G[3][e] += G[2][e];
        sc[e] = G[3][e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = __shfl_up(sc[e], 16);
        if (lg >= 1) sc[e] += x;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = __shfl_up(sc[e], 32);
        if (lg >= 2) sc[e] += x;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ex[e] = sc[e] - G[3][e];
    if (lg == 3) {
        *reinterpret_cast<floatx4 *>(&sm.gsum[w][8 * cg]) = floatx4{sc[0], sc[1], sc[2], sc[3]};
        *reinterpret_cast<floatx4 *>(&sm.gsum[w][8 * cg + 4]) = floatx4{sc[4], sc[5], sc[6], sc[7]};
    }
    if (w == 0) {
        float b = __uint_as_float((uint32_t)bt_raw << 16);
        if (pro_on<PM>(pro, PRO_BETA_LOGIT)) b = sigmoid_f(b);
        sm.beta[t] = t < L ? b : 0.f;
    }
    __syncthreads();

    // ---- decay factors of this thread's rows and channels (g only):
    // f = exp(G - G_m) and its reciprocal; per channel exp(G_C - G_m) (the row
    // factor of M' and N), exp(G_m) and f of the state pass, exp(G_C)
    float fx[4][8], fr[4][8], fe[8];
    {
        floatx4 gs[4][2];  // the four waves' channel sums for channels 8 cg ..
#pragma unroll
        for (int wi = 0; wi < 4; ++wi)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) gs[wi][hh] = *reinterpret_cast<const floatx4 *>(&sm.gsum[wi][8 * cg + 4 * hh]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ch = 8 * cg + e;
            const float s0w = gs[0][e >> 2][e & 3], s1w = gs[1][e >> 2][e & 3], s2w = gs[2][e >> 2][e & 3],
                        s3w = gs[3][e >> 2][e & 3];
            const float gm = s0w + s1w;                 // G at token 31 (end of wave 1's rows)
            const float gcl = gm + s2w + s3w;           // G at token 63
            float pre = ex[e] - gm;
            if (w >= 1) pre += s0w;
            if (w >= 2) pre += s1w;
            if (w >= 3) pre += s2w;
            fe[e] = fast_exp(gcl - gm);
            if (rg == 0) {
                sm.egm[ch] = fast_exp(gm);
                reinterpret_cast<float *>(rec + R_FC)[ch] = fast_exp(gcl);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                fx[u][e] = fast_exp(pre + G[u][e]);  // exp(G - G_m)
                fr[u][e] = __builtin_amdgcn_rcpf(fx[u][e]);
            }
        }
    }
    // ---- Kp, Qp, Km (and Diag(f) Km^T, kept in registers for this thread's
    // channels 8 cg + e and rows 4 rg .. 4 rg + 3 until the tile it goes to
    // is free)
    half4 kmT[8];
    {
        half8 kpr[4], qpr[4], kmr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float kv[8], qv[8];
            unpack8(rk[u], kv);
            unpack8(rq[u], qv);
            if (pro_on<PM>(pro, PRO_NORM_QK)) {  // a row's 128 channels lie in one DPP row
                const float ik = inv_norm(row16_sum(sumsq8(kv)), pro.eps);
                const float iq = inv_norm(row16_sum(sumsq8(qv)), pro.eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    kv[e] *= ik;
                    qv[e] *= iq;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kpr[u][e] = (_Float16)(kv[e] * fx[u][e]);
                qpr[u][e] = (_Float16)(qv[e] * fx[u][e]);
                const float km = kv[e] * fr[u][e];
                kmr[u][e] = (_Float16)km;
                kmT[e][u] = (_Float16)(km * fe[e]);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 4 * rg + u;
            *reinterpret_cast<half8 *>(&sm.kp[r * PK + 8 * cg]) = kpr[u];
            *reinterpret_cast<half8 *>(&sm.qp[r * PK + 8 * cg]) = qpr[u];
            *reinterpret_cast<half8 *>(&sm.km[r * PK + 8 * cg]) = kmr[u];
        }
    }
    // ---- V^T staging copy (bf16 [column][row], pitch VTP) in the A/P tiles,
    // which are not used before the Gram phase: each wave reads back its U~
    // blocks' columns in the MFMA accumulator layout
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
    __syncthreads();
    // V in the accumulator layout of this wave's U~ blocks (rows 16 i + 4 lg + e,
    // column 32 w + 16 b + l16); the Gram phase overwrites the staging tile
    // after the barrier that follows
    uint2 vz[2][4];
    {
        const uint16_t *vst = reinterpret_cast<const uint16_t *>(sm.a16);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vz[b][i] = *reinterpret_cast<const uint2 *>(&vst[(32 * w + 16 * b + l16) * VTP + 16 * i + 4 * lg]);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the staging reads are done
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
    // Wave w owns column blocks 2 w, 2 w + 1 of both: Xh[0..1] are W's
    // (Kp columns 32 w .. 32 w + 31), Xh[2..3] U~'s (V columns likewise), so
    // that the products which follow (Q^ from W, M' from W, N from U~) split
    // evenly over the four waves.
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
                const int r = 16 * i + 4 * lg + e, col = 32 * w + 16 * (b & 1) + l16;
                if (b < 2) {
                    zx[i][b][e] = (float)sm.kp[r * PK + col];
                } else {
                    const uint32_t vw = (e < 2) ? vz[b - 2][i].x : vz[b - 2][i].y;
                    zx[i][b][e] = __uint_as_float((e & 1) ? (vw & 0xffff0000u) : (vw << 16));
                }
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
    // ---- Q^ = (Qp - P W) E (each wave its two W blocks, in place over Qp).
    // The product is formed transposed, (P W)^T = W^T P^T: a lane's W
    // accumulator block read as a 16x16x16 A operand is a block of W^T, and
    // P's row fragment serves as the B operand, so each lane ends up with four
    // consecutive columns of one row: one 8-byte read-modify-write of Qp.
    // The lane's key channels here (32 w + 16 b + 4 lg + e) are also those of
    // its M' elements below: their exp(G_m) factors, read once.
    floatx4 ecol[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) ecol[b] = *reinterpret_cast<const floatx4 *>(&sm.egm[32 * w + 16 * b + 4 * lg]);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i <= rb; ++i) acc = mma16(Xh[b][i], frag4(sm.p, P4, 16 * rb, 16 * i, lane), acc);
            _Float16 *qrow = &sm.qp[(16 * rb + l16) * PK + 32 * w + 16 * b + 4 * lg];
            half4 qv = *reinterpret_cast<const half4 *>(qrow);
#pragma unroll
            for (int e = 0; e < 4; ++e) qv[e] = (_Float16)(((float)qv[e] - acc[e]) * ecol[b][e]);
            *reinterpret_cast<half4 *>(qrow) = qv;
        }
    }
    __syncthreads();
    // ---- Diag(f) Km^T into the Kp tile (no longer read): [c][s], s permuted
    // as the contraction index, 16-byte blocks of a row XOR-permuted by (c & 7)
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<half4 *>(&sm.kp[kt_off(8 * cg + e, rg)]) = kmT[e];
    // ---- Q^ to the workspace as A fragments, k-permuted: wave w writes row
    // block w, one whole 1 KB fragment per k-step (a lane's 8 values are
    // logical k 32 ks + 4 lg .. +3 and that + 16 of row 16 w + l16)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int r = 16 * w + l16, l0 = 32 * ks + 4 * lg;
        const half4 q0 = *reinterpret_cast<const half4 *>(&sm.qp[r * PK + l0]);
        const half4 q1 = *reinterpret_cast<const half4 *>(&sm.qp[r * PK + l0 + 16]);
        *reinterpret_cast<half8 *>(rec + R_QH + 16 * ((w * 4 + ks) * 64 + lane)) = pair8(q0, q1);
    }
    __syncthreads();
    // ---- M' = -Diag(f) Km^T W E (from Xh[0..1]) and N = Diag(f) Km^T U~
    // (from Xh[2..3]), f = exp(G_C - G_m) here, contracting over s with the
    // accumulator blocks as operands.  M' is formed transposed
    // (M'^T = -E W^T (Diag(f) Km^T)^T): each lane then holds four consecutive
    // contraction indices of one row of M' (key channels 32 w + 4 lg + i and
    // that + 16, whose E factors are ecol), which is what its A-order fragment
    // takes; this wave's two W blocks are the two halves of k-step w.
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
        half8 kt[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) kt[ks] = *reinterpret_cast<const half8 *>(&sm.kp[kt_frag_off(cb, ks, lane)]);
        floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            a0 = mma32(pair8(Xh[0][2 * ks], Xh[0][2 * ks + 1]), kt[ks], a0);
            a1 = mma32(pair8(Xh[1][2 * ks], Xh[1][2 * ks + 1]), kt[ks], a1);
        }
        half8 mv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mv[i] = (_Float16)(-a0[i] * ecol[0][i]);
            mv[4 + i] = (_Float16)(-a1[i] * ecol[1][i]);
        }
        *reinterpret_cast<half8 *>(rec + R_M + 16 * ((cb * 4 + w) * 64 + lane)) = mv;
#pragma unroll
        for (int b = 2; b < 4; ++b) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                acc = mma32(kt[ks], pair8(Xh[b][2 * ks], Xh[b][2 * ks + 1]), acc);
            const int jt = 2 * w + b - 2;
            *reinterpret_cast<half4 *>(rec + R_N + 8 * ((jt * 8 + cb) * 64 + lane)) = to_half4(acc);
        }
    }
    // ---- O^ = P U~ for this wave's U~ blocks (value tiles 2 w, 2 w + 1), stored
    // as the output pass's accumulators.  P's A fragments take the permuted
    // contraction order of the U~ pairs: logical s = 32 ks + 4 lg .. +3 and
    // that + 16, from the [r][s] tile; blocks above P's diagonal block are
    // zero (their LDS is never written).
    half8 pf[4][2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const _Float16 *prow = &sm.p[(16 * rb + l16) * P4 + 32 * ks + 4 * lg];
            const half4 lo = 2 * ks > rb ? half4{0, 0, 0, 0} : *reinterpret_cast<const half4 *>(prow);
            const half4 hi = 2 * ks + 1 > rb ? half4{0, 0, 0, 0} : *reinterpret_cast<const half4 *>(prow + 16);
            pf[rb][ks] = pair8(lo, hi);
        }
#pragma unroll
    for (int b = 2; b < 4; ++b) {
        const int jt = 2 * w + b - 2;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (2 * ks <= rb) acc = mma32(pf[rb][ks], pair8(Xh[b][2 * ks], Xh[b][2 * ks + 1]), acc);
            *reinterpret_cast<half4 *>(rec + R_OH + 8 * ((jt * 4 + rb) * 64 + lane)) = to_half4(acc);
        }
    }
}

// ---------------------------------------------------------------- pass 2
// One chunk's state-pass operands in LDS for a workgroup owning one 16-column
// value tile, as copied from the record: M' in A order, the tile's N, f and
// exp(G_m).  Loader waves copy it with direct global-to-LDS loads in
// wave-wide 1 KB segments.
struct ChunkTiles {
    _Float16 m[8 * 4 * 64 * 8];  // M' fragments [row block][k-step][lane][8]
    _Float16 n[8 * 64 * 4];      // N [row block][lane][4], accumulator layout
    float fc[KD];                // f
};
// The tiles are copied in 1 KB segments (16 bytes per lane); the last one, f,
// is half a segment.
constexpr int SLOTS = (int)(sizeof(ChunkTiles) / 16);  // 2336
constexpr int SEGS = (SLOTS + 63) / 64;                 // 37
static_assert(SLOTS == 36 * 64 + 32, "segment count");

struct StateSmem {
    ChunkTiles buf[NBUF];
    _Float16 xb[2][4][64 * 8];  // S B fragments exchanged between the state waves [parity][k-step]
};

// Workgroup barrier without a memory fence: waves that must see each other's
// LDS writes wait for them explicitly, so the compiler adds no waits of its
// own (direct loads in flight and fragment reads stay in flight across it).
__device__ __forceinline__ void loader_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Global source of LDS slot p (16-byte units) of a ChunkTiles image for value
// tile jt: M' (2048 slots), the tile's N (256), then f (32).
__device__ __forceinline__ const unsigned char *tile_source(const unsigned char *rec, int p, int jt) {
    return p < 2048 ? rec + R_M + 16 * p
         : p < 2304 ? rec + R_N + 4096 * jt + 16 * (p - 2048)
                    : rec + R_FC + 16 * (p - 2304);
}

// One direct global-to-LDS load: 16 bytes per lane from `src`, landing at
// lds + 16 lane (lds is wave-uniform).
__device__ __forceinline__ void lds_dma16(const unsigned char *src, unsigned char *lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }

// Loader wave lw copies segments lw, lw + LOADER_WAVES, ... (PW of them);
// HALF_LAST: its last one is the half segment (lanes 0-31 only).
template <int PW, bool HALF_LAST>
__device__ __forceinline__ void load_tiles(unsigned char *dst, const unsigned char *rec, int jt,
                                           int lw, int lane) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int sg = lw + LOADER_WAVES * i;
        if (!(HALF_LAST && i == PW - 1) || lane < 32)
            lds_dma16(tile_source(rec, 64 * sg + lane, jt), dst + 1024 * sg);
    }
}

// The loader waves' side of the pipeline.  Chunk ci is copied into buffer
// ci % 4.  Barrier ci (early in the state waves' chunk ci) certifies that
// chunk ci + 1 has landed (if there is one); after it chunk ci + 3 is issued into the
// buffer chunk ci - 1 used, which the state wave finished reading before
// barrier ci - 1.  Loads complete in issue order, so "chunk ci + 1 landed" is
// "at most the loads of chunk ci + 2 outstanding": each chunk has two chunk
// times to arrive.
template <int PW, bool HALF_LAST>
__device__ __forceinline__ void loader_loop(StateSmem &sm, const unsigned char *recs, int cap,
                                            int h, int ch0, int nchunks, int jt, int lw, int lane) {
    auto issue = [&](int ci) {
        load_tiles<PW, HALF_LAST>(reinterpret_cast<unsigned char *>(&sm.buf[ci % NBUF]),
                       recs + ((size_t)h * cap + ch0 + ci) * REC, jt, lw, lane);
    };
    for (int c = 0; c < 3 && c < nchunks; ++c) issue(c);
    if (nchunks > 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PW));  // chunk 0 landed
    else if (nchunks > 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(PW));
    else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    for (int ci = 0; ci < nchunks; ++ci) {
        if (ci + 2 < nchunks)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(PW));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        loader_barrier();
        if (ci + 3 < nchunks) issue(ci + 3);
    }
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

// M' fragments of k-step ks for the row blocks [RBW sw, RBW sw + RBW).
__device__ __forceinline__ void read_m(half8 (&a)[RBW], const ChunkTiles &tl, int sw, int ks, int lane) {
#pragma unroll
    for (int r = 0; r < RBW; ++r)
        a[r] = *reinterpret_cast<const half8 *>(&tl.m[8 * (((RBW * sw + r) * 4 + ks) * 64 + lane)]);
}
// The tile's N and f of a chunk for those row blocks, in the accumulator layout.
__device__ __forceinline__ void read_nf(half4 (&nv)[RBW], floatx4 (&fv)[RBW], const ChunkTiles &tl,
                                        int sw, int lane) {
    const int lg = lane >> 4;
#pragma unroll
    for (int r = 0; r < RBW; ++r) {
        const int cb = RBW * sw + r;
        nv[r] = *reinterpret_cast<const half4 *>(&tl.n[4 * (cb * 64 + lane)]);
        fv[r] = *reinterpret_cast<const floatx4 *>(&tl.fc[16 * cb + 4 * lg]);
    }
}
// MFMAs of one k-step on this wave's rows: S += M'[own rows, ks block] * b.
__device__ __forceinline__ void mfma_step(floatx4 (&S)[RBW], const half8 (&a)[RBW], const half8 &b) {
#pragma unroll
    for (int r = 0; r < RBW; ++r) S[r] = mma32(a[r], b, S[r]);
}

// Grid: one workgroup per (unit, value tile), XCD-aware: workgroup b runs on
// XCD b mod 8, and all value tiles of a unit share that XCD (and its L2),
// which serves their common M' tiles.  Waves [0, STATE_WAVES) are the state
// waves, the rest the loaders.
//
// State wave sw keeps RBW row blocks of the tile's 128 x 16 slice of S in
// accumulators: the rows of its k-steps KSW sw .. KSW sw + KSW - 1.  Per chunk
// it converts them to those k-steps' fp16 B fragments, publishes them (for
// the output pass) and hands them to the other state waves through LDS;
// barrier ci makes all of them visible.  It then forms Diag(f) S + N on its
// rows and adds the products of its own k-steps first and the others' after
// (cyclic order from its own), reading M' fragments one k-step ahead and the
// next chunk's first ones after this chunk's last; the exchanged fragments
// have the own k-steps' products to arrive.
// SNAP: the call writes prefix snapshots (a separate instantiation, so that
// calls without them keep the check off the chain).
template <bool SNAP>
__global__ __launch_bounds__(64 * (STATE_WAVES + LOADER_WAVES)) void chunk_state_kernel(
    StateIO io, const int32_t *__restrict__ cu, int fixedT, int N, int H, int totalT, int cap,
    unsigned char *__restrict__ ws) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    StateSmem &sm = *reinterpret_cast<StateSmem *>(smem_raw);
    const ChunkMap cm = chunk_map(cu, fixedT, N, totalT, cap);
    const int b = blockIdx.x, slot = b >> 3;
    const int jt = slot % 8;                   // 16-column value tile
    const int unit = (slot / 8) * 8 + (b & 7);
    if (unit >= N * H) return;
    const int n = unit / H, h = unit - n * H;
    const int ch0 = cm.first(n);
    const int nchunks = cm.first(n + 1) - ch0;
    unsigned char *recs = ws;
    auto rec = [&](int ci) { return recs + ((size_t)h * cap + ch0 + ci) * REC; };

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lg = lane >> 4;

    if (w < STATE_WAVES) {
        const int sw = w;
        auto korder = [&](int t) { return (KSW * sw + t) & 3; };  // k-step order, own first
        const int jcol = 16 * jt + (lane & 15);                    // this lane's value column
        // element (row, jcol) of a state is at [row * VD + jcol]; this lane's
        // rows are 16 (RBW sw + r) + 4 lg + i
        auto elem = [&](int r, int i) { return (16 * (RBW * sw + r) + 4 * lg + i) * VD + jcol; };
        const float *s0p = state_in(io, n, h, H, KD * VD);
        int bos, eos;
        seq_bounds(cu, n, fixedT, totalT, bos, eos);
        const int len = eos - bos;
        SnapCursor snap;
        if (SNAP) snap.init(io, n);
        floatx4 S[RBW];  // rows 16 (RBW sw + r) + 4 lg + i
        if (s0p) {
#pragma unroll
            for (int r = 0; r < RBW; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[r][i] = s0p[elem(r, i)];
        } else {
#pragma unroll
            for (int r = 0; r < RBW; ++r) S[r] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();
        half8 a[RBW], bq[RBW];
        half4 nv[RBW];
        floatx4 fv[RBW];
        if (nchunks > 0) {
            read_m(a, sm.buf[0], sw, korder(0), lane);
            read_nf(nv, fv, sm.buf[0], sw, lane);
        }
        for (int ci = 0; ci < nchunks; ++ci) {
            const ChunkTiles &tl = sm.buf[ci % NBUF];
            unsigned char *sp = rec(ci) + R_SP + 4096 * jt;
            half8 bk[4];  // B fragments in this wave's k-step order
#pragma unroll
            for (int t = 0; t < KSW; ++t) {
                bk[t] = bfrag(S[2 * t], S[2 * t + 1]);
                *reinterpret_cast<half8 *>(&sm.xb[ci & 1][korder(t)][8 * lane]) = bk[t];
                // an ordinary (L2-resident) store: the output pass reads the
                // snapshot back shortly; a non-temporal one costs ~6% of the call
                *reinterpret_cast<half8 *>(sp + 1024 * korder(t) + 16 * lane) = bk[t];
            }
            // Barrier ci: all of S exchanged, chunk ci + 1 landed, and every
            // read of this wave from earlier chunks' buffers done.
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            loader_barrier();
#pragma unroll
            for (int t = KSW; t < 4; ++t)
                bk[t] = *reinterpret_cast<const half8 *>(&sm.xb[ci & 1][korder(t)][8 * lane]);
            read_m(bq, tl, sw, korder(1), lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < RBW; ++r) {
#pragma unroll
                for (int i = 0; i < 4; ++i) S[r][i] = __builtin_fmaf(fv[r][i], S[r][i], (float)nv[r][i]);
                S[r] = mma32(a[r], bk[0], S[r]);
            }
            __builtin_amdgcn_sched_barrier(0);
            read_m(a, tl, sw, korder(2), lane);
            mfma_step(S, bq, bk[1]);
            __builtin_amdgcn_sched_barrier(0);
            read_m(bq, tl, sw, korder(3), lane);
            mfma_step(S, a, bk[2]);
            __builtin_amdgcn_sched_barrier(0);
            // the next chunk's first fragments, N and f (unused after the last chunk)
            const ChunkTiles &nx = sm.buf[(ci + 1) % NBUF];
            read_m(a, nx, sw, korder(0), lane);
            read_nf(nv, fv, nx, sw, lane);
            mfma_step(S, bq, bk[3]);
            // prefix snapshot when the state now covers a boundary
            if (SNAP && snap.due(min(C * (ci + 1), len))) {
                float *sp = snap.dest(io, h, H, KD * VD);
                snap.advance(io);
                if (sp) {
                    // one 16-byte store per row block: after the quad
                    // transpose a lane holds row 4 lg + (lane & 3), columns
                    // 4 ((lane & 15) >> 2) .. +3 of the tile
#pragma unroll
                    for (int r = 0; r < RBW; ++r) {
                        const floatx4 t = quad_transpose(S[r], lane);
                        *reinterpret_cast<floatx4 *>(&sp[(16 * (RBW * sw + r) + 4 * lg + (lane & 3)) * VD +
                                                          16 * jt + 4 * ((lane & 15) >> 2)]) = t;
                    }
                }
            }
        }
        float *sTp = state_out(io, n, h, H, KD * VD);
        if (sTp) {
#pragma unroll
            for (int r = 0; r < RBW; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) sTp[elem(r, i)] = S[r][i];
        }
    } else {
        // Segments per loader wave: the first SEGS % LOADER_WAVES waves take one more.
        constexpr int PW = SEGS / LOADER_WAVES;
        static_assert(SEGS % LOADER_WAVES == 1, "segment split");
        const int lw = w - STATE_WAVES;
        if (lw == 0)
            loader_loop<PW + 1, true>(sm, recs, cap, h, ch0, nchunks, jt, lw, lane);
        else
            loader_loop<PW, false>(sm, recs, cap, h, ch0, nchunks, jt, lw, lane);
    }
}

hipError_t launch_state(const StateIO &io, const int32_t *cu, int N, int fixedT, int totalT,
                        int H, int cap, unsigned char *ws, hipStream_t stream) {
    constexpr int smem = (int)sizeof(StateSmem);
    auto kern = io.snap ? chunk_state_kernel<true> : chunk_state_kernel<false>;
    static std::atomic<uint64_t> lds_set[2];
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(kern), smem,
                                      lds_set[io.snap ? 1 : 0]);
    if (e != hipSuccess) return e;
    const int groups = (N * H + 7) / 8;
    hipLaunchKernelGGL(kern, dim3(groups * 8 * 8), dim3(64 * (STATE_WAVES + LOADER_WAVES)), smem,
                       stream, io, cu, fixedT, N, H, totalT, cap, ws);
    return hipGetLastError();
}

// ---------------------------------------------------------------- pass 3
// O = Q^ S + O^ for every (chunk, head) at once: one workgroup of 4 waves
// per record, wave w producing value tiles 2 w and 2 w + 1 (16 columns each).
// The accumulators start from O^; Q^ (contraction index permuted to match the
// S fragments) and the chunk-start state S are read as MFMA fragments
// straight from the record;
// outputs leave through a buffer resource spanning the chunk's valid rows,
// as non-temporal stores (nothing in the call reads them back).
constexpr int CPOL_NT = 2;
// Four consecutive columns of one output row: 16 bytes (fp32) or 8 (bf16).
__device__ __forceinline__ void store_row4(__amdgpu_buffer_rsrc_t r, int off, const floatx4 &y, float) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const i32x4 b = {(int)__float_as_uint(y[0]), (int)__float_as_uint(y[1]), (int)__float_as_uint(y[2]),
                     (int)__float_as_uint(y[3])};
    __builtin_amdgcn_raw_buffer_store_b128(b, r, off, 0, CPOL_NT);
}
__device__ __forceinline__ void store_row4(__amdgpu_buffer_rsrc_t r, int off, const floatx4 &y, bf16_t) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    const i32x2 b = {(int)(from_f32<bf16_t>(y[0]).bits | ((uint32_t)from_f32<bf16_t>(y[1]).bits << 16)),
                     (int)(from_f32<bf16_t>(y[2]).bits | ((uint32_t)from_f32<bf16_t>(y[3]).bits << 16))};
    __builtin_amdgcn_raw_buffer_store_b64(b, r, off, 0, CPOL_NT);
}

template <typename TOut>
__global__ __launch_bounds__(256) void chunk_output_kernel(TOut *__restrict__ o,
                                                           const int32_t *__restrict__ cu,
                                                           int fixedT, int N, int H, int totalT,
                                                           const unsigned char *__restrict__ ws) {
    const ChunkMap cm = chunk_map(cu, fixedT, N, totalT, gridDim.x);
    const int gc = blockIdx.x, h = blockIdx.y;
    if (gc >= cm.first(N)) return;
    const int n = cm.seq_of(gc);
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int c0 = bos + (gc - cm.first(n)) * C;
    const int L = min(C, eos - c0);
    const unsigned char *rec = ws + ((size_t)h * gridDim.x + gc) * REC;

    const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Q^ (A fragments, 16 KB) is shared by the four waves: each copies four of
    // its fragments into LDS with direct loads
    __shared__ __align__(16) unsigned char qs[16 * 1024];
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(rec + R_QH + 1024 * (4 * w + i) + 16 * lane, qs + 1024 * (4 * w + i));
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    half8 aq[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            aq[ks][rb] = *reinterpret_cast<const half8 *>(qs + 1024 * (rb * 4 + ks) + 16 * lane);
    const int row_bytes = H * VD * (int)sizeof(TOut);
    __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        o + (size_t)c0 * H * VD, 0, L * row_bytes, 0x00020000);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int tile = 2 * w + tt, j = 16 * tile + l16;
        half8 bs[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            bs[ks] = *reinterpret_cast<const half8 *>(rec + R_SP + 4096 * tile + 1024 * ks + 16 * lane);
        floatx4 Y[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const half4 oh = *reinterpret_cast<const half4 *>(rec + R_OH + 8 * ((tile * 4 + rb) * 64 + lane));
#pragma unroll
            for (int e = 0; e < 4; ++e) Y[rb][e] = (float)oh[e];
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) Y[rb] = mma32(aq[ks][rb], bs[ks], Y[rb]);
        // after a 4 x 4 transpose inside each quad of lanes, a lane holds row
        // 4 lg + (lane & 3) of each row block, columns j - (lane & 3) .. +3
        const int lane_off = (((4 * lg + (lane & 3)) * H + h) * VD + j - (lane & 3)) * (int)sizeof(TOut);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            store_row4(orsrc, lane_off + 16 * rb * row_bytes, quad_transpose(Y[rb], lane), TOut{});
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
// enough to amortise the extra launches (MI355X, warm): up to 24 units, or 32
// when sequences average at most 16 chunks (at 32 units: 42 vs 51 us at
// T = 1024, 194 vs 178 us at T = 4096), and at least 4 chunks per sequence on
// average.
bool chunk_split_supported(int N, int H, int K, int V, int Cc) {
    return K == KD && V == VD && Cc == C && N > 0 && N < 127 && H > 0;
}

bool chunk_split_recommended(int N, int totalT, int H, int K, int V, int Cc) {
    if (!chunk_split_supported(N, H, K, V, Cc) || (long long)totalT < 4LL * C * N) return false;
    const long long units = (long long)N * H;
    return units <= 24 || (units <= 32 && (long long)totalT <= 16LL * C * N);
}

size_t chunk_split_workspace_bytes(int N, int totalT, int H) {
    return (size_t)max_chunks(N, totalT, 0, true) * H * REC;
}

hipError_t launch_chunk_split(const void *q, const void *k, const void *v, const void *g,
                              const void *beta, const StateIO &io, const Prologue &pro, void *o,
                              const int32_t *cu, int N, int fixedT, int totalT, int H,
                              bool out_bf16, void *workspace, hipStream_t stream) {
    if (N == 0 || H == 0) return hipSuccess;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const int cap = max_chunks(N, totalT, fixedT, cu != nullptr);
    hipError_t e;
    if (cap > 0) {
        static std::atomic<uint64_t> lds_set[3];
        const int pm = pro_mode(pro);
        auto kern = pm == PRO_FULL      ? chunk_prep_kernel<PRO_FULL>
                    : pm == PRO_RUNTIME ? chunk_prep_kernel<PRO_RUNTIME>
                                        : chunk_prep_kernel<PRO_OFF>;
        e = ensure_dynamic_lds(reinterpret_cast<const void *>(kern), (int)sizeof(PrepSmem),
                               lds_set[pm]);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(cap, H), dim3(256), sizeof(PrepSmem), stream,
                           static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                           static_cast<const uint16_t *>(v), static_cast<const uint16_t *>(g),
                           static_cast<const uint16_t *>(beta), cu, fixedT, N, H, totalT, pro, ws);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    e = launch_state(io, cu, N, fixedT, totalT, H, cap, ws, stream);
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
