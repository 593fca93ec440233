// chunk_mfma.hip -- bf16-input chunked KDA forward on the gfx950 matrix cores.
//
// "Kimi K3: Open Frontier Intelligence and Implementation Framework", section
// "Hybrid Attention Mechanism": KDA is the delta rule with a channel-wise
// forget gate, and its lower-bounded decay lets both the diagonal
// (intra-chunk) and off-diagonal (inter-chunk) tiles run as dense matrix
// products.  This kernel is that chunked forward pass for K = V = 128 and
// chunk C = 64.
//
// Algebra for one chunk (rows r, s = tokens; G = running sum of g inside the
// chunk, per key channel; m = 31 the reference row; Q, K, V the chunk tiles):
//   Kp = K * exp(G - G_m),  Km = K * exp(G_m - G),  Qp = Q * exp(G - G_m)
//   A  = Diag(beta) strict_lower(Kp Km^T)      P = lower(Qp Km^T)
//   S' = Diag(exp(G_m)) S
//   (I + A) U = Diag(beta) (V - Kp S')         O = Qp S' + P U
//   S  <- Diag(exp(G_C - G_m)) (S' + Km^T U)
// Kp Km^T and Qp Km^T carry exp(G_r - G_s) <= 1 for s <= r.  With
// -g_lb <= g <= 0 and g_lb * C / 2 <= 8 every factor stays within e^8, inside
// fp16 range: this is where the lower bound on the decay is used.
//
// Mapping onto CDNA4.  One workgroup of 12 wavefronts owns one (sequence,
// head, 64-column V tile); the two tiles of a head run side by side on two
// CUs of one XCD.  Two wave groups run concurrently, separated by two
// workgroup barriers per chunk:
//  * state waves 0-3: wave w owns value columns 16 w .. 16 w + 15 and keeps the
//    128 x 16 fp32 state slice in MFMA accumulators for the whole sequence
//    (rows in the order that makes two accumulator blocks one fp16 B
//    fragment).  Per chunk (phase A) it forms S', takes its B fragments
//    straight from the accumulators and forms Kp S' and, transposed,
//    (Qp S')^T with v_mfma_f32_16x16x32_f16; then (phase B) it solves
//    (I + A) U = Y by 16-row block substitution in registers (the 16x16
//    accumulator layout is the B layout of v_mfma_f32_16x16x16_f16), advances
//    the state with Km^T U (Km^T read from the Km tile by the transposing LDS
//    read ds_read_b64_tr_b16), adds (P U)^T to the transposed output and
//    stages it in LDS.
//  * prep waves 4-11: prep wave p owns tokens 8p .. 8p + 7 of a chunk (a
//    lane holds two channels of all eight).  In phase A they form the current
//    chunk's Gram and query-key blocks and the 16 x 16 diagonal inverses
//    (I + A_ii)^-1 (a product form on the matrix cores), and waves 4-7 the
//    next chunk's per-channel factors; in phase B they build the next chunk's
//    fp16 operand tiles (exponentials of the running decay sums), take the
//    running decay sums of the chunk after it, refill their input registers
//    from buffer loads as the old contents are consumed, and waves 4-7 store
//    the previous chunk's staged output as whole rows (each store instruction
//    then covers whole cache lines, where the accumulator layout gives a
//    quarter row per lane group).
// Packed sequences are dealt to workgroups longest first.
#include "kda_mfma.hpp"
#include "prologue.hpp"
#include "state_io.hpp"

namespace kda {
namespace {

constexpr int C = 64;    // chunk length
constexpr int KD = 128;  // key dimension
constexpr int VD = 128;  // value dimension
constexpr int VT = 64;   // value columns per workgroup
constexpr int NT = 768;  // threads per workgroup: 4 state waves + 8 prep waves
constexpr int NP = 8;    // prep waves
constexpr int PK = 144;  // LDS pitch (halves) of [64][128] fp16 tiles
constexpr int P4 = 68;   // LDS pitch (halves) of [64][64] fp16 tiles read as 8-byte fragments
constexpr int PI = 20;   // LDS pitch (halves) of 16 x 16 fp16 blocks
constexpr int PV = 72;   // LDS pitch (halves) of the V tile
constexpr int PO = 68;   // LDS pitch (floats) of the output staging tile

// State rows.  Accumulator block cb of a state wave holds, in lane group
// g = lane >> 4, element i, the state row (key channel)
//   sigma(cb, g, i) = 32 (cb >> 1) + 8 g + 4 (cb & 1) + i,
// so that blocks 2 k and 2 k + 1 of lane group g together hold channels
// 32 k + 8 g .. 32 k + 8 g + 7: exactly the contraction indices of a 16x16x32
// B fragment.  The state thus serves as the B operand of Kp S' and Qp S'
// straight from the accumulators while Kp, Qp and Km keep their channels in
// natural order (the layout every reader of the tiles expects).
__device__ __forceinline__ int sigma(int cb, int g, int i) {
    return 32 * (cb >> 1) + 8 * g + 4 * (cb & 1) + i;
}

struct Smem {
    _Float16 kp[C * PK];        // Kp [s][c]
    _Float16 qp[C * PK];        // Qp [s][c]
    _Float16 km[2][C * PK];     // Km [s][c] by chunk parity: Gram / query-key B operand, and
                                // (read transposed) the state-advance A operand
    _Float16 a16[C * P4];       // A [r][s], lower blocks
    _Float16 p[C * P4];         // P [r][s], lower blocks
    _Float16 tii[4][16 * PI];   // (I + A_ii)^-1, diagonal blocks
    uint16_t vr[C * PV];        // bf16 V tile [r][j]
    float beta[C];
    float fm[2][KD];            // exp(G_m) times the previous chunk's exp(G_C - G_m): the
                                // state's scaling at a chunk's start, by chunk parity
    float fc[2][KD];            // exp(G_C - G_m), by chunk parity
    float gsum[2][NP][KD];      // prep waves: per-wave channel sums of g, by chunk parity
    float woff[2][NP][KD];      // log2(e) (G at prep wave p's first token - G_m), by parity
    float ost[2][C * PO];       // the chunk's output tile [r][j], staged for whole-row stores,
                                // by chunk parity
};

typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Transposing LDS read (ds_read_b64_tr_b16): in each 16-lane group, lane j
// receives as element i the (j & 3)-th 16-bit value of the 8 bytes addressed
// by lane 4 i + (j >> 2) of its group.
__device__ __forceinline__ short4v read_tr(const void *addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v *)(const_cast<void *>(addr)));
}

// Km^T A fragment of state block cb, contraction half ks: lane (l16, g) gets
// row sigma(cb, l16 >> 2, l16 & 3) (a key channel) and, as contraction
// positions 8 g .. 8 g + 7, the tokens 32 ks + 4 g + t and 32 ks + 16 + 4 g + t
// (t < 4): the order in which two 16-row U blocks serve as a B fragment.
__device__ __forceinline__ half8 frag_kmT(const _Float16 *km, int cb, int ks, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int c = 32 * (cb >> 1) + 8 * (j & 3) + 4 * (cb & 1);
    const int t = 32 * ks + 4 * g + (j >> 2);
    const half4 lo = __builtin_bit_cast(half4, read_tr(km + t * PK + c));
    const half4 hi = __builtin_bit_cast(half4, read_tr(km + (t + 16) * PK + c));
    half8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = lo[i];
        r[i + 4] = hi[i];
    }
    return r;
}

__device__ __forceinline__ half8 cat8(half4 a, half4 b) {
    half8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = a[i];
        r[i + 4] = b[i];
    }
    return r;
}

// One chunk's inputs, held in a prep wave's registers ahead of use.
// Lane l of prep wave p holds channels 2 l and 2 l + 1 of tokens 8 p .. 8 p + 7
// (one 4-byte load per token row, each instruction reading one whole 256-byte
// row), so the running decay sum over a wave's tokens stays inside the lane.
// The loads go through buffer resources whose extent ends at the chunk's last
// token, so rows past a short chunk's end read as zero without touching
// memory, and all address arithmetic but one scalar base per chunk is fixed
// for the whole kernel.
struct Raw {
    uint32_t q[8], k[8];  // token 8 p + t: bf16 channels 2 l (low half) and 2 l + 1
    uint4 v;              // V tile piece: row 8 p + (l >> 3), columns 8 (l & 7) .. + 7
    uint32_t beta;        // beta of token lane (used by prep wave 4, which finishes its phases early)
    int L;                // the chunk's length
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes from base (raw addressing; accesses past
// the extent return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t extent(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Byte offsets, inside a chunk, of one lane's loads (the same for every chunk;
// the whole offset is in the lane's register, where the extent check sees it).
struct LaneOffs {
    uint32_t row[8];  // q / k / g: token 8p + t, channels 2 l, 2 l + 1
    uint32_t v;       // V: token 8 p + (l >> 3), columns 8 (l & 7) .. + 7
    uint32_t beta;    // beta: token lane
};

__device__ __forceinline__ LaneOffs lane_offsets(int H, int p, int lane) {
    LaneOffs o;
#pragma unroll
    for (int t = 0; t < 8; ++t) o.row[t] = (uint32_t)((8 * p + t) * H * KD * 2 + 4 * lane);
    o.v = (uint32_t)((8 * p + (lane >> 3)) * H * VD * 2 + 16 * (lane & 7));
    o.beta = (uint32_t)(lane * H * 2);
    return o;
}

__device__ __forceinline__ void load_g(uint32_t *rg, const uint16_t *g, int c0, int L, int H, int h,
                                       const LaneOffs &lof) {
    const auto r = extent(g + ((size_t)c0 * H + h) * KD, (uint32_t)(L * H * KD * 2));
#pragma unroll
    for (int t = 0; t < 8; ++t) rg[t] = load4(r, lof.row[t]);
}

__device__ __forceinline__ void load_raw(Raw &R, const uint16_t *q, const uint16_t *k,
                                         const uint16_t *v, const uint16_t *beta, int c0, int L,
                                         int H, int h, int vt, int p, const LaneOffs &lof) {
    const size_t cb = ((size_t)c0 * H + h) * KD;
    const uint32_t rows = (uint32_t)(L * H * KD * 2);
    const auto rq = extent(q + cb, rows), rk = extent(k + cb, rows);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        R.q[t] = load4(rq, lof.row[t]);
        R.k[t] = load4(rk, lof.row[t]);
    }
    const auto rv = extent(v + ((size_t)c0 * H + h) * VD + vt * VT,
                           (uint32_t)((L - 1) * H * VD * 2 + 2 * VT));
    R.v = load16(rv, lof.v);
    const auto rb = extent(beta + (size_t)c0 * H + h, (uint32_t)((L - 1) * H * 2 + 2));
    R.beta = p == 4 ? __builtin_amdgcn_raw_buffer_load_b16(rb, lof.beta, 0, 0) : 0u;
    R.L = L;
}

// Extents of one chunk's inputs, from which a prep wave refills its input
// registers as soon as their previous contents are used (spreading the loads
// over the work rather than issuing them in one burst).
struct Src {
    __amdgpu_buffer_rsrc_t q, k, v, beta;
    int L;
};

__device__ __forceinline__ Src chunk_src(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                         const uint16_t *beta, int c0, int L, int H, int h, int vt,
                                         int p) {
    const size_t cb = ((size_t)c0 * H + h) * KD;
    const uint32_t rows = (uint32_t)(L * H * KD * 2);
    Src s;
    s.q = extent(q + cb, rows);
    s.k = extent(k + cb, rows);
    s.v = extent(v + ((size_t)c0 * H + h) * VD + vt * VT, (uint32_t)((L - 1) * H * VD * 2 + 2 * VT));
    s.beta = extent(beta + (size_t)c0 * H + h, (uint32_t)((L - 1) * H * 2 + 2));
    s.L = L;
    return s;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gate_src(const uint16_t *g, int c0, int L, int H,
                                                           int h) {
    return extent(g + ((size_t)c0 * H + h) * KD, (uint32_t)(L * H * KD * 2));
}

// Prep wave p, first half of the running log-decay sum: lc[t] = sum of g over
// tokens 8p .. 8p + t for this lane's two channels (inside the lane), and the
// wave's channel totals to LDS.  Rows at or past L read as `pad`.
// PM (a ProMode): rg holds gate logits when the prologue's gate map applies.
template <int PM>
__device__ __forceinline__ void scan_partials(Smem &sm, uint32_t *rg, int L, uint32_t pad,
                                              int par, int p, int lane, float (*lc)[2],
                                              const Prologue &pro, __amdgpu_buffer_rsrc_t gnext,
                                              const LaneOffs &lof) {
    // rows past the end loaded as zero: no decay, except through the gate map
    const bool gl = pro_on<PM>(pro, PRO_GATE_LOGIT);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t w = gl && 8 * p + t >= L ? pad : rg[t];
        lc[t][0] = bf16lo(w);
        lc[t][1] = bf16hi(w);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 8; ++t) rg[t] = load4(gnext, lof.row[t]);  // the next chunk's gates
    __builtin_amdgcn_sched_barrier(0);
    if (gl) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            lc[t][0] = gate_from_logit(lc[t][0], pro.glb);
            lc[t][1] = gate_from_logit(lc[t][1], pro.glb);
        }
    }
#pragma unroll
    for (int t = 1; t < 8; ++t) {
        lc[t][0] += lc[t - 1][0];
        lc[t][1] += lc[t - 1][1];
    }
    *reinterpret_cast<float2 *>(&sm.gsum[par][p][2 * lane]) = make_float2(lc[7][0], lc[7][1]);
}

// From the prep waves' channel totals of parity par, the chunk's per-channel
// factors exp(G_m) and exp(G_C - G_m) and each prep wave's offset to the
// reference row, log2(e) (G_{8p - 1} - G_m) (minus the totals of waves p..3,
// or plus those of waves 4..p-1), for channel c.
__device__ __forceinline__ void chunk_factors(Smem &sm, int par, int c, bool first) {
    constexpr float LOG2E = 1.4426950408889634f;
    {
        float x[NP];
#pragma unroll
        for (int ww = 0; ww < NP; ++ww) x[ww] = sm.gsum[par][ww][c];
        float below = 0.f;  // - sum of waves p..3, built downward from p = 3
#pragma unroll
        for (int ww = 3; ww >= 0; --ww) {
            below -= x[ww];
            sm.woff[par][ww][c] = LOG2E * below;
        }
        const float gm = -below;
        float above = 0.f;  // sum of waves 4..p-1
#pragma unroll
        for (int ww = 4; ww < NP; ++ww) {
            sm.woff[par][ww][c] = LOG2E * above;
            above += x[ww];
        }
        // the end-of-chunk scaling of the previous chunk is folded into this
        // chunk's start scaling (the state is kept without it in between)
        sm.fm[par][c] = fast_exp(gm) * (first ? 1.f : sm.fc[par ^ 1][c]);
        sm.fc[par][c] = fast_exp(above);
    }
}


// Sums over the 64 lanes of a wave of eight values per lane, by halving
// exchanges: lanes 32 apart (v_permlane32_swap) leave four sums per lane,
// 16-lane rows (v_permlane16_swap) two, lanes 8 apart (DPP row rotate) one,
// then quad and half-row DPP steps finish the 8-lane groups.  Lane
// 8 j + i ends with the total of value j.  The totals are returned as
// wave-uniform values read from lanes 0, 8, .., 56.
__device__ __forceinline__ void wave_sums8(const float *x, float *tot, int lane) {
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[j]), __float_as_uint(x[j + 4]), false, false);
        y[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // lanes < 32: value j, else j + 4
    }
    float z[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y[j]), __float_as_uint(y[j + 2]), false, false);
        z[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // even rows: j (+4), odd rows: j + 2 (+4)
    }
    const bool up = (lane & 8) != 0;
    const float keep = up ? z[1] : z[0], give = up ? z[0] : z[1];
    // row_ror:8 -- lane l of a row reads lane (l + 8) mod 16 of it
    float u = keep + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, give), 0x128, 0xF, 0xF, false));
    u += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, u), 0xB1, 0xF, 0xF, false));
    u += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, u), 0x4E, 0xF, 0xF, false));
    u += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, u), 0x141, 0xF, 0xF, false));
    // lane 8 j holds value (4 (j >= 4) + 2 (j & 2 ? 1 : 0) + (j & 1)) = j
#pragma unroll
    for (int j = 0; j < 8; ++j) tot[j] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(u), 8 * j));
}

// Prep wave p, second half: exp(G - G_m) for this lane's tokens from the
// running sums and the wave's offset to the reference row, and the fp16
// operand tiles of the chunk (after the prologue's normalisation of q and k,
// whose 128 channels of a token are spread over the wave's 64 lanes).
template <int PM>
__device__ __forceinline__ void build_operands(Smem &sm, Raw &R, uint32_t bpad, int par,
                                               int p, int lane, const float (*lc)[2],
                                               const Prologue &pro, const Src &nx,
                                               const LaneOffs &lof) {
    const int L = R.L;
    const int c = 2 * lane;
    // this wave's offset to the reference row m = 31 (the end of wave 3's
    // tokens), in log2 units
    const float2 wo = *reinterpret_cast<const float2 *>(&sm.woff[par][p][c]);
    constexpr float LOG2E = 1.4426950408889634f;
    float ik[8], iq[8];
    if (pro_on<PM>(pro, PRO_NORM_QK)) {
        float sk[8], sq[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float k0 = bf16lo(R.k[t]), k1 = bf16hi(R.k[t]);
            const float q0 = bf16lo(R.q[t]), q1 = bf16hi(R.q[t]);
            sk[t] = __builtin_fmaf(k1, k1, k0 * k0);
            sq[t] = __builtin_fmaf(q1, q1, q0 * q0);
        }
        float tk[8], tq[8];
        wave_sums8(sk, tk, lane);
        wave_sums8(sq, tq, lane);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            ik[t] = inv_norm(tk[t], pro.eps);
            iq[t] = inv_norm(tq[t], pro.eps);
        }
    }
    // four token rows at a time (fewer live registers)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        float kv[4][2], qv[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            kv[t][0] = bf16lo(R.k[4 * hh + t]);  // zero past the chunk's end
            kv[t][1] = bf16hi(R.k[4 * hh + t]);
            qv[t][0] = bf16lo(R.q[4 * hh + t]);
            qv[t][1] = bf16hi(R.q[4 * hh + t]);
        }
        // refill with the next chunk's rows, pinned here (after the last use
        // of the old contents) so the loop-carried registers stay in place
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            R.k[4 * hh + t] = load4(nx.k, lof.row[4 * hh + t]);
            R.q[4 * hh + t] = load4(nx.q, lof.row[4 * hh + t]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int tt = 4 * hh + t;
            if (pro_on<PM>(pro, PRO_NORM_QK)) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    kv[t][j] *= ik[tt];
                    qv[t][j] *= iq[tt];
                }
            }
            half2v hkp, hkm, hqp;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float f = __builtin_amdgcn_exp2f(__builtin_fmaf(lc[tt][j], LOG2E, j ? wo.y : wo.x));
                const float i = __builtin_amdgcn_rcpf(f);
                hkp[j] = (_Float16)(kv[t][j] * f);
                hkm[j] = (_Float16)(kv[t][j] * i);
                hqp[j] = (_Float16)(qv[t][j] * f);
            }
            const int rb = (8 * p + tt) * PK + c;
            *reinterpret_cast<half2v *>(&sm.kp[rb]) = hkp;
            *reinterpret_cast<half2v *>(&sm.km[par][rb]) = hkm;
            *reinterpret_cast<half2v *>(&sm.qp[rb]) = hqp;
        }
    }
    // V: rows 8p .. 8p + 7, eight lanes per row (zero past the end)
    *reinterpret_cast<uint4 *>(&sm.vr[(8 * p + (lane >> 3)) * PV + 8 * (lane & 7)]) = R.v;
    __builtin_amdgcn_sched_barrier(0);
    R.v = load16(nx.v, lof.v);
    __builtin_amdgcn_sched_barrier(0);
    if (p == 4) {
        const bool bl = pro_on<PM>(pro, PRO_BETA_LOGIT);
        const float b = __uint_as_float((bl && lane >= L ? bpad : R.beta) << 16);
        R.beta = __builtin_amdgcn_raw_buffer_load_b16(nx.beta, lof.beta, 0, 0);
        sm.beta[lane] = pro_on<PM>(pro, PRO_BETA_LOGIT) ? sigmoid_f(b) : b;
    }
    R.L = nx.L;
}
// Block product: lane (l16, lg) receives element i =
// (lhs rhs^T)[16 bi + 4 lg + i][16 bj + l16].
__device__ __forceinline__ floatx4 block_product(const _Float16 *lhs, const _Float16 *rhs, int bi,
                                                 int bj, int lane) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        acc = mma32(frag8(lhs, PK, 16 * bi, 32 * ks, lane), frag8(rhs, PK, 16 * bj, 32 * ks, lane), acc);
    return acc;
}

// Transposed block product: lane (l16, lg) receives element i =
// (lhs rhs^T)[16 bi + l16][16 bj + 4 lg + i], i.e. one row of the block and
// four consecutive columns (which an 8-byte store keeps together).
__device__ __forceinline__ floatx4 block_product_t(const _Float16 *lhs, const _Float16 *rhs,
                                                   int bi, int bj, int lane) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        acc = mma32(frag8(rhs, PK, 16 * bj, 32 * ks, lane), frag8(lhs, PK, 16 * bi, 32 * ks, lane), acc);
    return acc;
}

// Prep wave p: the chunk's Gram / query-key blocks.  Waves 0-3 take the
// diagonal blocks (p, p) and the inverse (I + A_pp)^-1; waves 4-7 the
// off-diagonal blocks of the Gram and query-key products.
__device__ __forceinline__ void prep_blocks(Smem &sm, int par, int p, int lane) {
    const _Float16 *km = sm.km[par];
    const int l16 = lane & 15, lg = lane >> 4;
    if (p < 4) {
        // A_pp = Diag(beta) strict_lower(Kp Km^T) on this block, held twice:
        // in the A layout (lane: row l16, columns 4 lg .. +3; the transposed
        // product) and in the B layout (lane: column l16, rows 4 lg .. +3)
        const floatx4 at = block_product_t(sm.kp, km, p, p, lane);
        const floatx4 ab = block_product(sm.kp, km, p, p, lane);
        const float br = sm.beta[16 * p + l16];
        const floatx4 bc = *reinterpret_cast<const floatx4 *>(&sm.beta[16 * p + 4 * lg]);
        half4 LA, LB;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            LA[i] = (_Float16)(4 * lg + i < l16 ? br * at[i] : 0.f);
            LB[i] = (_Float16)(l16 < 4 * lg + i ? bc[i] * ab[i] : 0.f);
        }
        const floatx4 pq = block_product_t(sm.qp, km, p, p, lane);
        half4 ph;
#pragma unroll
        for (int i = 0; i < 4; ++i) ph[i] = (_Float16)(4 * lg + i <= l16 ? pq[i] : 0.f);
        *reinterpret_cast<half4 *>(&sm.p[(16 * p + l16) * P4 + 16 * p + 4 * lg]) = ph;
        // (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8) for the strictly lower
        // 16 x 16 block L (L^16 = 0), as 16x16x16 products.  A product Z = X Y
        // from X in the A layout and Y in the B layout gives Z in the B layout
        // (accumulator = B fragment); Z^T = Y^T X^T from the same registers,
        // operands swapped, gives Z in the A layout.
        const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
        half4 eye;
#pragma unroll
        for (int i = 0; i < 4; ++i) eye[i] = (_Float16)(4 * lg + i == l16 ? 1.f : 0.f);
        const half4 L2B = to_half4(mma16(LA, LB, z4)), L2A = to_half4(mma16(LB, LA, z4));
        const half4 L4B = to_half4(mma16(L2A, L2B, z4)), L4A = to_half4(mma16(L2B, L2A, z4));
        const half4 L8B = to_half4(mma16(L4A, L4B, z4));
        const half4 R1A = to_half4(mma16(eye + L2B, eye - LA, z4));   // ((I - L)(I + L^2))^T
        const half4 R2A = to_half4(mma16(eye + L4B, R1A, z4));        // (R1 (I + L^4))^T
        const half4 TA = to_half4(mma16(eye + L8B, R2A, z4));         // (R2 (I + L^8))^T
        *reinterpret_cast<half4 *>(&sm.tii[p][l16 * PI + 4 * lg]) = TA;
    } else if (p < 6) {
        // waves 4 and 5: rows 32-63 x columns 0-31 of the Gram (wave 4) or
        // query-key (wave 5) product -- blocks (2,0), (2,1), (3,0), (3,1) --
        // as one 32x32 tile (half the LDS reads of four 16x16 blocks),
        // transposed: lane l gets row 32 + (l & 31), columns
        // 8 q + 4 (l >> 5) .. + 3 in registers 4 q .. 4 q + 3
        const bool gram = p == 4;
        const _Float16 *lhs = gram ? sm.kp : sm.qp;
        const int r32 = lane & 31, kh = 8 * (lane >> 5);
        floatx16 acc = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const half8 a = *reinterpret_cast<const half8 *>(&km[r32 * PK + 16 * ks + kh]);
            const half8 b = *reinterpret_cast<const half8 *>(&lhs[(32 + r32) * PK + 16 * ks + kh]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
        }
        const float sc = gram ? sm.beta[32 + r32] : 1.f;
        _Float16 *dst = gram ? sm.a16 : sm.p;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            half4 hv;
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = (_Float16)(sc * acc[4 * qq + i]);
            *reinterpret_cast<half4 *>(&dst[(32 + r32) * P4 + 8 * qq + 4 * (lane >> 5)]) = hv;
        }
    } else {
        // waves 6 and 7: blocks (1,0) and (3,2) of the Gram (wave 6) or
        // query-key (wave 7) product
        const bool gram = p == 6;
#pragma unroll
        for (int tsk = 0; tsk < 2; ++tsk) {
            const int bi = tsk ? 3 : 1, bj = tsk ? 2 : 0;
            const floatx4 acc = block_product_t(gram ? sm.kp : sm.qp, km, bi, bj, lane);
            const float sc = gram ? sm.beta[16 * bi + l16] : 1.f;
            half4 hv;
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = (_Float16)(sc * acc[i]);
            _Float16 *dst = gram ? sm.a16 : sm.p;
            *reinterpret_cast<half4 *>(&dst[(16 * bi + l16) * P4 + 16 * bj + 4 * lg]) = hv;
        }
    }
}

// The packed sequence of rank rho when sequences are ordered by length,
// longest first (ties in index order): every thread of the workgroup takes
// part (two workgroup barriers); scratch holds SORT_MAX + 1 ints of LDS.
constexpr int SORT_MAX = 256;
__device__ __forceinline__ int sequence_of_rank(const int32_t *cu, int N, int totalT, int rho,
                                             int *scratch) {
    const int t = threadIdx.x;
    for (int m = t; m < N; m += NT) {
        int a, e;
        seq_bounds(cu, m, 0, totalT, a, e);
        scratch[m] = e - a;
    }
    __syncthreads();
    if (t < N) {
        const int len = scratch[t];
        int rank = 0;
        for (int m = 0; m < N; ++m) {
            const int lm = scratch[m];
            rank += (lm > len || (lm == len && m < t)) ? 1 : 0;
        }
        if (rank == rho) scratch[SORT_MAX] = t;
    }
    __syncthreads();
    return scratch[SORT_MAX];
}

template <typename TOut>
__device__ __forceinline__ void store4(TOut *dst, floatx4 v);
template <>
__device__ __forceinline__ void store4<float>(float *dst, floatx4 v) {
    *reinterpret_cast<floatx4 *>(dst) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *dst, floatx4 v) {
    // round to nearest even by the packed hardware conversion
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    uint2 w;
    w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){v[0], v[1]}, b2));
    w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){v[2], v[3]}, b2));
    *reinterpret_cast<uint2 *>(dst) = w;
}

// Prep wave 4 + j: rows 16 j .. 16 j + 15 of a chunk's staged output tile to
// o, four whole rows (the workgroup's 64 columns) per store instruction:
// lane holds row 16 j + 4 s + (lane >> 4), columns 4 (lane & 15) .. + 3.
template <typename TOut>
__device__ __forceinline__ void store_output(const Smem &sm, int par, TOut *o, int c0, int L, int H,
                                             int h, int vt, int j, int lane) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int r = 16 * j + 4 * s + (lane >> 4);
        const floatx4 x = *reinterpret_cast<const floatx4 *>(&sm.ost[par][r * PO + 4 * (lane & 15)]);
        if (r < L) store4<TOut>(o + ((size_t)(c0 + r) * H + h) * VD + vt * VT + 4 * (lane & 15), x);
    }
}

template <typename TOut, int PM>
__global__ __launch_bounds__(NT) void chunk_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ g,
    const uint16_t *__restrict__ beta, StateIO io, Prologue pro, TOut *__restrict__ o,
    const int32_t *__restrict__ cu, int fixedT, int N, int H, int totalT) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem &sm = *reinterpret_cast<Smem *>(smem_raw);

    // Both V tiles of a head land on the same XCD (workgroups are dealt to the
    // 8 XCDs round-robin), so their shared q/k/g reads meet in one L2.
    const int b = blockIdx.x;
    const int xcd = b & 7, slot = b >> 3;
    const int vt = slot & 1;
    const int unit = (slot >> 1) * 8 + xcd;  // position in the work order
    if (unit >= N * H) return;
    const int h = unit % H;
    // Packed sequences run longest first: workgroups are dispatched in
    // order, so the longest chains start earliest and the short ones fill in
    int n = unit / H;
    if (cu && N > 1 && N <= SORT_MAX)
        n = sequence_of_rank(cu, N, totalT, n, reinterpret_cast<int *>(sm.kp));

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const bool state_wave = w < 4;
    const int l16 = lane & 15, lg = lane >> 4;
    int bos, eos;
    seq_bounds(cu, n, fixedT, totalT, bos, eos);
    const int nchunks = (eos - bos + C - 1) / C;

    // The two wave groups run separate loops with the same barrier sequence
    // (three before the loop, two per chunk), so their registers never overlap.
    if (state_wave) {
        // S[cb] holds rows c = 16 cb + 4 lg + i, column 16 w + l16 of the tile;
        // element (c, column) of a state is at [c * VD + column]
        const int col = vt * VT + 16 * w + l16;
        const float *s0p = state_in(io, n, h, H, KD * VD);
        SnapCursor snap;
        snap.init(io, n);
        floatx4 S[8];
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[cb][i] = s0p ? s0p[sigma(cb, lg, i) * VD + col] : 0.f;
        // the initial state has landed before the loop, so the loop's waits
        // never cover the previous chunk's output stores
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        __syncthreads();
        __syncthreads();
        for (int ci = 0; ci < nchunks; ++ci) {
            const int c0 = bos + ci * C;
            const int L = min(C, eos - c0);
            const int par = ci & 1;

            // straight from the accumulators, the inter-chunk products Kp S'
            // and Qp S', and Y = Diag(beta) (V - Kp S')
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const floatx4 f = *reinterpret_cast<const floatx4 *>(&sm.fm[par][sigma(cb, lg, 0)]);
#pragma unroll
                for (int i = 0; i < 4; ++i) S[cb][i] *= f[i];
            }
            half8 bs[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) bs[ks] = cat8(to_half4(S[2 * ks]), to_half4(S[2 * ks + 1]));
            // the four row blocks advance together (eight independent
            // accumulation chains); each fragment register is refilled with the
            // next k-step's fragment as soon as its product has issued.  The
            // output is accumulated transposed, O^T = S'^T Qp^T (the same
            // fragments with the operand roles swapped), so that a lane ends
            // with four consecutive columns of one output row
            floatx4 X[4], O[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) X[rb] = O[rb] = floatx4{0.f, 0.f, 0.f, 0.f};
            half8 fk[4], fq[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                fk[rb] = frag8(sm.kp, PK, 16 * rb, 0, lane);
                fq[rb] = frag8(sm.qp, PK, 16 * rb, 0, lane);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    X[rb] = mma32(fk[rb], bs[ks], X[rb]);
                    if (ks < 3) fk[rb] = frag8(sm.kp, PK, 16 * rb, 32 * (ks + 1), lane);
                    O[rb] = mma32(bs[ks], fq[rb], O[rb]);
                    if (ks < 3) fq[rb] = frag8(sm.qp, PK, 16 * rb, 32 * (ks + 1), lane);
                }
            }
            floatx4 Y[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                // V rows 16 rb + 4 lg + i of column 16 w + l16, transposed on read
                const short4v vv = read_tr(&sm.vr[(16 * rb + 4 * lg + (l16 >> 2)) * PV + 16 * w + 4 * (l16 & 3)]);
                const floatx4 bb = *reinterpret_cast<const floatx4 *>(&sm.beta[16 * rb + 4 * lg]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Y[rb][i] = bb[i] * (__uint_as_float((uint32_t)(uint16_t)vv[i] << 16) - X[rb][i]);
            }
            __syncthreads();
            // ---- phase B: (I + A) U = Y by 16-row blocks,
            // U_i = T_ii (Y_i - sum_{j<i} A_ij U_j), all in registers; the
            // fragments of A, of the inverses and of the first half of Km^T are
            // loaded before the substitution starts
            half4 Aij[6], Tii[4];
#pragma unroll
            for (int i = 1, x = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < i; ++j, ++x) Aij[x] = frag4(sm.a16, P4, 16 * i, 16 * j, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) Tii[i] = frag4(sm.tii[i], PI, 0, 0, lane);
            half8 km[8];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                km[2 * cb] = frag_kmT(sm.km[par], cb, 0, lane);
                km[2 * cb + 1] = frag_kmT(sm.km[par], cb, 1, lane);
            }
            half4 U[4];
#pragma unroll
            for (int i = 0, x = 0; i < 4; ++i) {
                floatx4 z = Y[i];
                if (i > 0) {
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < i; ++j, ++x) acc = mma16(Aij[x], U[j], acc);
#pragma unroll
                    for (int e = 0; e < 4; ++e) z[e] -= acc[e];
                }
                U[i] = to_half4(mma16(Tii[i], to_half4(z), floatx4{0.f, 0.f, 0.f, 0.f}));
            }
            // S = Diag(exp(G_C - G_m)) (S' + Km^T U), U as B fragments straight
            // from the accumulators (the Km^T fragment registers refilled with
            // the second half's as they issue); O^T += U^T P^T
            const half8 bu0 = cat8(U[0], U[1]), bu1 = cat8(U[2], U[3]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                S[cb] = mma32(km[2 * cb], bu0, S[cb]);
                km[2 * cb] = frag_kmT(sm.km[par], cb + 4, 0, lane);
                S[cb] = mma32(km[2 * cb + 1], bu1, S[cb]);
                km[2 * cb + 1] = frag_kmT(sm.km[par], cb + 4, 1, lane);
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int i = 0; i <= rb; ++i) O[rb] = mma16(U[i], frag4(sm.p, P4, 16 * rb, 16 * i, lane), O[rb]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                S[cb + 4] = mma32(km[2 * cb], bu0, S[cb + 4]);
                S[cb + 4] = mma32(km[2 * cb + 1], bu1, S[cb + 4]);
            }
            // O^T blocks to the staging tile (a lane holds chunk row
            // 16 rb + l16, columns 16 w + 4 lg .. + 3); prep waves 4-7 store
            // it at the end of the next phase B as whole rows
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int r = 16 * rb + l16;
                if (r < L)
                    *reinterpret_cast<floatx4 *>(&sm.ost[par][(16 * rb + l16) * PO + 16 * w + 4 * lg]) = O[rb];
            }
            // S now holds S' + Km^T U; its end-of-chunk scaling
            // Diag(exp(G_C - G_m)) is applied with the next chunk's start
            // scaling (and here only to the copies that leave the kernel)
            // prefix snapshot when the state now covers a boundary
            if (snap.due(c0 - bos + L)) {
                float *sp = snap.dest(io, h, H, KD * VD);
                snap.advance(io);
                if (sp) {
                    // one 16-byte store per row block: after the quad
                    // transpose a lane holds row 4 lg + (lane & 3), columns
                    // col - (lane & 3) .. +3
#pragma unroll
                    for (int cb = 0; cb < 8; ++cb) {
                        const floatx4 f = *reinterpret_cast<const floatx4 *>(&sm.fc[par][sigma(cb, lg, 0)]);
                        const floatx4 t = quad_transpose(S[cb] * f, lane);
                        *reinterpret_cast<floatx4 *>(&sp[sigma(cb, lg, lane & 3) * VD + col - (lane & 3)]) = t;
                    }
                }
            }
            __syncthreads();
        }
        float *sTp = state_out(io, n, h, H, KD * VD);
        if (sTp && nchunks > 0) {
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const floatx4 f = *reinterpret_cast<const floatx4 *>(&sm.fc[(nchunks - 1) & 1][sigma(cb, lg, 0)]);
                S[cb] *= f;
            }
        }
        if (sTp) {
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) sTp[sigma(cb, lg, i) * VD + col] = S[cb][i];
        }
    } else {
        const int p = w - 4;
        // Waves are issued oldest first: prep waves 0-3 would always win the
        // vector ALU against waves 4-7 on the same SIMD, and the chunk waits
        // for the slowest prep wave; raising 4-7 (from the start of each
        // phase A to the end of their operand build) evens the two out.
        const uint32_t gpad = pro_on<PM>(pro, PRO_GATE_LOGIT) ? BF16_NEG_INF_PAIR : 0u;
        const uint32_t bpad = pro_on<PM>(pro, PRO_BETA_LOGIT) ? (BF16_NEG_INF_PAIR & 0xFFFFu) : 0u;
        const LaneOffs lof = lane_offsets(H, p, lane);
        Raw R;
        uint32_t rg[8];
        float lc[8][2];
        // chunk i of the sequence, clamped to the last one (a chunk past the
        // end is loaded as the last one again and never used)
        const int last = nchunks > 0 ? nchunks - 1 : 0;
        auto cstart = [&](int i) { return bos + min(i, last) * C; };
        auto clen = [&](int i) { return min(C, eos - cstart(i)); };
        // Pipeline: in the iteration that handles chunk ci, the prep waves form
        // chunk ci's Gram / query-key blocks (phase A), then chunk ci + 1's
        // operands and chunk ci + 2's decay sums (phase B), and issue the loads
        // of chunk ci + 2's inputs and chunk ci + 3's gates, which are used one
        // iteration later.
        auto src = [&](int i) { return chunk_src(q, k, v, beta, cstart(i), clen(i), H, h, vt, p); };
        auto gsrc = [&](int i) { return gate_src(g, cstart(i), clen(i), H, h); };
        if (nchunks > 0) {
            load_g(rg, g, cstart(0), clen(0), H, h, lof);
            load_raw(R, q, k, v, beta, cstart(0), clen(0), H, h, vt, p, lof);
            scan_partials<PM>(sm, rg, clen(0), gpad, 0, p, lane, lc, pro, gsrc(1), lof);
        }
        __syncthreads();
        if (p >= 6) chunk_factors(sm, 0, 64 * (p - 6) + lane, true);  // chunk 0's (its channel totals are in)
        __syncthreads();
        if (nchunks > 0) {
            build_operands<PM>(sm, R, bpad, 0, p, lane, lc, pro, src(1), lof);
            scan_partials<PM>(sm, rg, clen(1), gpad, 1, p, lane, lc, pro, gsrc(2), lof);
        }
        __syncthreads();
        for (int ci = 0; ci < nchunks; ++ci) {
            // ---- phase A: this chunk's Gram / query-key blocks and diagonal inverses
            if (p >= 4) __builtin_amdgcn_s_setprio(1);
            prep_blocks(sm, ci & 1, p, lane);
            // the next chunk's factors and offsets (its channel totals landed
            // one iteration ago), for phase B: waves 6 and 7, whose blocks
            // finish first
            if (p >= 6) chunk_factors(sm, (ci & 1) ^ 1, 64 * (p - 6) + lane, false);
            __syncthreads();
            // ---- phase B: the next chunk's operands and the decay sums of the
            // chunk after it; their input registers are refilled (for chunks
            // ci + 2 and ci + 3) as they are consumed.  Both run in every
            // iteration (unconditional register refills keep the loop-carried
            // inputs in place): past the last chunk they rework the last
            // chunk's inputs into buffers that are not read again.
            build_operands<PM>(sm, R, bpad, (ci & 1) ^ 1, p, lane, lc, pro, src(ci + 2), lof);
            // waves 4-7 give way to 0-3 (their phase-B work is the longer
            // path) until the next phase A
            if (p >= 4) __builtin_amdgcn_s_setprio(0);
            scan_partials<PM>(sm, rg, clen(ci + 2), gpad, ci & 1, p, lane, lc, pro, gsrc(ci + 3), lof);
            // the previous chunk's output (staged by the state waves in its
            // phase B): waves 4-7 finish this phase early
            if (p >= 4 && ci > 0)
                store_output<TOut>(sm, (ci & 1) ^ 1, o, cstart(ci - 1), clen(ci - 1), H, h, vt, p - 4, lane);
            __syncthreads();
        }
        // the last chunk's output (its staging tile is complete after the
        // loop's last barrier)
        if (p >= 4 && nchunks > 0)
            store_output<TOut>(sm, (nchunks - 1) & 1, o, cstart(nchunks - 1), clen(nchunks - 1), H, h, vt, p - 4, lane);
    }
}

template <typename TOut, int PM>
hipError_t launch_t(const void *q, const void *k, const void *v, const void *g, const void *beta,
                    const StateIO &io, const Prologue &pro, void *o, const int32_t *cu, int N,
                    int fixedT, int totalT, int H, hipStream_t stream) {
    auto kern = chunk_mfma_kernel<TOut, PM>;
    const size_t smem = sizeof(Smem);
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(kern), (int)smem, lds_set);
    if (e != hipSuccess) return e;
    const int units = N * H;
    const int grid = ((units + 7) / 8) * 16;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), smem, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), static_cast<const uint16_t *>(g),
                       static_cast<const uint16_t *>(beta), io, pro, static_cast<TOut *>(o), cu,
                       fixedT, N, H, totalT);
    return hipGetLastError();
}

}  // namespace

bool chunk_mfma_supported(int K, int V, int Cc) { return K == KD && V == VD && Cc == C; }

hipError_t launch_chunk_mfma(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, const StateIO &io, const Prologue &pro, void *o,
                             const int32_t *cu, int N, int fixedT, int totalT, int H,
                             bool out_bf16, hipStream_t stream) {
    if (N == 0 || H == 0) return hipSuccess;
    switch (pro_mode(pro)) {
        case PRO_FULL:
            return out_bf16 ? launch_t<bf16_t, PRO_FULL>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, stream)
                            : launch_t<float, PRO_FULL>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, stream);
        case PRO_RUNTIME:
            return out_bf16 ? launch_t<bf16_t, PRO_RUNTIME>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, stream)
                            : launch_t<float, PRO_RUNTIME>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, stream);
        default:
            return out_bf16 ? launch_t<bf16_t, PRO_OFF>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, stream)
                            : launch_t<float, PRO_OFF>(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, stream);
    }
}

size_t chunk_mfma_smem_bytes() { return sizeof(Smem); }

}  // namespace kda
