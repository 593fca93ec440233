// kda_api.hip -- the C ABI of libkda.so (declared in include/kda.h).
//
// Host side only: argument validation (before any HIP call, so argument errors
// never enqueue work), dispatch to the kernels by (K, V, chunk, dtype), and
// mapping of HIP errors to kda_status_t.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/kda.h"
#include "prologue.hpp"
#include "state_io.hpp"

namespace kda {
hipError_t launch_decode(const void *q, const void *k, const void *v, const void *g,
                         const void *beta, float *state, const int32_t *slot_in,
                         const int32_t *slot_out, int pool_slots, const Prologue &pro, void *o,
                         int N, int H, int K, int V, bool in_bf16, bool out_bf16,
                         hipStream_t stream);
hipError_t launch_decode_multi(const void *q, const void *k, const void *v, const void *g,
                               const void *beta, float *pool, const int32_t *slot_in,
                               const int32_t *slot_out, int pool_slots, const Prologue &pro,
                               void *o, int N, int T, int H, int K, int V, bool in_bf16,
                               bool out_bf16, hipStream_t stream);
hipError_t launch_chunk_valu(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, const StateIO &io, const Prologue &pro, void *o,
                             const int32_t *cu, int N, int fixedT, int totalT, int H, int K, int V,
                             int C, bool in_bf16, bool out_bf16, hipStream_t stream);
hipError_t launch_chunk_mfma(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, const StateIO &io, const Prologue &pro, void *o,
                             const int32_t *cu, int N, int fixedT, int totalT, int H,
                             bool out_bf16, hipStream_t stream);
bool chunk_mfma_supported(int K, int V, int C);
bool chunk_bwd_supported(int K, int V, int C);
size_t chunk_bwd_workspace_bytes(int N, int totalT, int fixedT, bool packed, int H, int K, int V,
                                 int C);
hipError_t launch_chunk_bwd(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const float *s0, const float *dout,
                            const float *dsT, float *dq, float *dk, float *dv, float *dg,
                            float *dbeta, float *ds0, const int32_t *cu, int N, int fixedT,
                            int totalT, int H, int K, int V, int C, bool in_bf16,
                            void *workspace, hipStream_t stream);
bool chunk_split_supported(int N, int H, int K, int V, int C);
bool chunk_split_recommended(int N, int totalT, int H, int K, int V, int C);
size_t chunk_split_workspace_bytes(int N, int totalT, int H);
hipError_t launch_chunk_split(const void *q, const void *k, const void *v, const void *g,
                              const void *beta, const StateIO &io, const Prologue &pro, void *o,
                              const int32_t *cu, int N, int fixedT, int totalT, int H,
                              bool out_bf16, void *workspace, hipStream_t stream);
}  // namespace kda

namespace {

bool dtype_ok(kda_dtype_t d) { return d == KDA_F32 || d == KDA_BF16; }

bool chunk_shape_supported(int K, int V, int C) {
    return (K == 32 && V == 32 && C == 16) || (K == 128 && V == 128 && C == 64);
}

// Elements of a [rows, H, D] tensor must stay below 2^31 (kernels index
// tiles with 32-bit arithmetic on top of 64-bit bases).
bool fits(long long rows, long long H, long long D) {
    return rows >= 0 && rows * H * D < (long long)INT_MAX;
}

kda_status_t from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// Range checks of the prologue's scalars.
kda_status_t make_prologue(unsigned flags, float glb, float eps, kda::Prologue &pro) {
    if (flags & ~kda::PRO_ALL) return KDA_ERR_VALUE;
    if (!std::isfinite(eps) || eps < 0.f) return KDA_ERR_VALUE;
    if (flags & kda::PRO_GATE_LOGIT) {
        if (!std::isfinite(glb) || glb < 0.f) return KDA_ERR_VALUE;
    }
    pro.flags = flags;
    pro.glb = glb;
    pro.eps = eps;
    return KDA_OK;
}

kda_status_t validate_fwd(const void *q, const void *k, const void *v, const void *g,
                          const void *beta, const void *o, int N, int totalT, int H, int K,
                          int V, int chunk, kda_dtype_t in_dtype, kda_dtype_t out_dtype) {
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_DTYPE;
    if (N < 0 || totalT < 0 || H <= 0 || K <= 0 || V <= 0 || chunk <= 0) return KDA_ERR_SHAPE;
    if (!fits(totalT, H, K > V ? K : V) || !fits(N, H, (long long)K * V)) return KDA_ERR_SHAPE;
    if (!chunk_shape_supported(K, V, chunk)) return KDA_ERR_UNSUPPORTED;
    if (totalT > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL;
    return KDA_OK;
}

// The workspace is optional: a workspace of at least
// kda_two_pass_workspace_bytes() selects the two-pass bf16 path (when that
// size is nonzero), none selects the single-pass kernels; a nonzero workspace
// that is too small is an error.
kda_status_t check_workspace(const void *workspace, size_t workspace_bytes, size_t need,
                             bool &two_pass) {
    two_pass = false;
    if (workspace_bytes == 0) return KDA_OK;
    if (!workspace) return KDA_ERR_NULL;
    if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
    two_pass = need > 0;
    return KDA_OK;
}

kda_status_t run_fwd(const void *q, const void *k, const void *v, const void *g,
                     const void *beta, const kda::StateIO &io, const kda::Prologue &pro, void *o,
                     const int32_t *cu, int N, int fixedT, int totalT, int H, int K, int V,
                     int chunk, kda_dtype_t in_dtype, kda_dtype_t out_dtype, void *workspace,
                     bool two_pass, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool in_bf16 = in_dtype == KDA_BF16, out_bf16 = out_dtype == KDA_BF16;
    // A declared gate bound beyond what the fp16 decay factors of the bf16
    // chunked kernels hold (g_lb * chunk / 2 > 8) sends the call to the
    // exact-decay kernel, which reads the same bf16 inputs.
    const bool steep = (pro.flags & kda::PRO_GATE_LOGIT) && (double)pro.glb * chunk > 16.0;
    hipError_t e;
    if (steep)
        e = kda::launch_chunk_valu(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, K, V,
                                   chunk, in_bf16, out_bf16, st);
    else if (in_bf16 && two_pass && kda::chunk_split_supported(N, H, K, V, chunk))
        e = kda::launch_chunk_split(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H,
                                    out_bf16, workspace, st);
    else if (in_bf16 && kda::chunk_mfma_supported(K, V, chunk))
        e = kda::launch_chunk_mfma(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H,
                                   out_bf16, st);
    else
        e = kda::launch_chunk_valu(q, k, v, g, beta, io, pro, o, cu, N, fixedT, totalT, H, K, V,
                                   chunk, in_bf16, out_bf16, st);
    return from_hip(e);
}

kda::StateIO dense_states(const float *s0, float *sT) {
    kda::StateIO io;
    io.s0 = s0;
    io.sT = sT;
    return io;
}

// A pool of pool_slots slots of H K x V fp32 states must be addressable.
bool pool_ok(int pool_slots, int H, int K, int V) {
    return pool_slots >= 1 && (long long)pool_slots * H <= LLONG_MAX / 4 / ((long long)K * V);
}

// Scratch of kda_varlen_fwd_noalloc: a file-scope device array of
// KDA_NOALLOC_SCRATCH_BYTES, one copy per GPU the library is loaded on, held
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it only stands for the symbol): the device address is
// looked up once per device with hipGetSymbolAddress and kept below.
constexpr size_t kScratchBytes = (size_t)80 << 20;
static_assert(kScratchBytes == KDA_NOALLOC_SCRATCH_BYTES, "scratch size and its documented value");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
hipError_t scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = __atomic_load_n(&g_scratch_ptr[dev], __ATOMIC_ACQUIRE);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev];
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            __atomic_store_n(&g_scratch_ptr[dev], p, __ATOMIC_RELEASE);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

int kda_version(void) { return 105; }

const char *kda_status_str(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: invalid or oversized dimensions";
        case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unknown dtype";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: (K, V, chunk) or dtype not supported";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace too small (or, without a workspace argument, the call needs more than the library's scratch)";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP runtime error";
        case KDA_ERR_VALUE: return "KDA_ERR_VALUE: scalar argument out of range";
    }
    return "KDA_ERR_UNKNOWN";
}

size_t kda_two_pass_workspace_bytes(int N, int total_T, int H, int K, int V, int chunk) {
    if (N <= 0 || total_T < 0 || H <= 0 || !kda::chunk_split_supported(N, H, K, V, chunk)) return 0;
    return kda::chunk_split_workspace_bytes(N, total_T, H);
}

size_t kda_workspace_bytes(int N, int total_T, int H, int K, int V, int chunk) {
    if (N <= 0 || total_T < 0 || H <= 0 || !kda::chunk_split_recommended(N, total_T, H, K, V, chunk))
        return 0;
    return kda::chunk_split_workspace_bytes(N, total_T, H);
}

kda_status_t kda_chunk_fwd_prologue(const void *q, const void *k, const void *v, const void *g,
                                    const void *beta, const float *s0, void *o, float *sT, int B,
                                    int T, int H, int K, int V, int chunk, kda_dtype_t in_dtype,
                                    kda_dtype_t out_dtype, void *workspace,
                                    size_t workspace_bytes, unsigned prologue,
                                    float gate_lower_bound, float norm_eps, void *stream) {
    if (B < 0 || T < 0) return KDA_ERR_SHAPE;
    const long long total = (long long)B * T;
    if (total > INT_MAX) return KDA_ERR_SHAPE;
    kda_status_t s = validate_fwd(q, k, v, g, beta, o, B, (int)total, H, K, V, chunk, in_dtype,
                                  out_dtype);
    if (s != KDA_OK) return s;
    kda::Prologue pro;
    s = make_prologue(prologue, gate_lower_bound, norm_eps, pro);
    if (s != KDA_OK) return s;
    bool two_pass;
    s = check_workspace(workspace, workspace_bytes,
                        kda_two_pass_workspace_bytes(B, (int)total, H, K, V, chunk), two_pass);
    if (s != KDA_OK) return s;
    if (B == 0) return KDA_OK;
    if (T == 0 && !sT) return KDA_OK;
    return run_fwd(q, k, v, g, beta, dense_states(s0, sT), pro, o, nullptr, B, T, (int)total, H,
                   K, V, chunk, in_dtype, out_dtype, workspace, two_pass, stream);
}

kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const float *s0, void *o, float *sT, int B,
                           int T, int H, int K, int V, int chunk, kda_dtype_t in_dtype,
                           kda_dtype_t out_dtype, void *workspace, size_t workspace_bytes,
                           void *stream) {
    return kda_chunk_fwd_prologue(q, k, v, g, beta, s0, o, sT, B, T, H, K, V, chunk, in_dtype,
                                  out_dtype, workspace, workspace_bytes, 0u, 0.f, 0.f, stream);
}

kda_status_t kda_varlen_fwd_prologue(const void *q, const void *k, const void *v, const void *g,
                                     const void *beta, const float *s0, void *o, float *sT,
                                     const int32_t *cu_seqlens, int N, int total_T, int H, int K,
                                     int V, int chunk, kda_dtype_t in_dtype,
                                     kda_dtype_t out_dtype, void *workspace,
                                     size_t workspace_bytes, unsigned prologue,
                                     float gate_lower_bound, float norm_eps, void *stream) {
    kda_status_t s = validate_fwd(q, k, v, g, beta, o, N, total_T, H, K, V, chunk, in_dtype,
                                  out_dtype);
    if (s != KDA_OK) return s;
    kda::Prologue pro;
    s = make_prologue(prologue, gate_lower_bound, norm_eps, pro);
    if (s != KDA_OK) return s;
    if (N > 0 && !cu_seqlens) return KDA_ERR_NULL;
    bool two_pass;
    s = check_workspace(workspace, workspace_bytes,
                        kda_two_pass_workspace_bytes(N, total_T, H, K, V, chunk), two_pass);
    if (s != KDA_OK) return s;
    if (N == 0) return KDA_OK;
    return run_fwd(q, k, v, g, beta, dense_states(s0, sT), pro, o, cu_seqlens, N, 0, total_T, H,
                   K, V, chunk, in_dtype, out_dtype, workspace, two_pass, stream);
}

kda_status_t kda_varlen_fwd(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const float *s0, void *o, float *sT,
                            const int32_t *cu_seqlens, int N, int total_T, int H, int K, int V,
                            int chunk, kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                            void *workspace, size_t workspace_bytes, void *stream) {
    return kda_varlen_fwd_prologue(q, k, v, g, beta, s0, o, sT, cu_seqlens, N, total_T, H, K, V,
                                   chunk, in_dtype, out_dtype, workspace, workspace_bytes, 0u,
                                   0.f, 0.f, stream);
}

kda_status_t kda_varlen_fwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                                    const void *beta, const float *s0, void *o, float *sT,
                                    const int32_t *cu_seqlens, int N, int total_T, int H, int K,
                                    int V, int chunk, kda_dtype_t in_dtype,
                                    kda_dtype_t out_dtype, void *stream) {
    kda_status_t s = validate_fwd(q, k, v, g, beta, o, N, total_T, H, K, V, chunk, in_dtype,
                                  out_dtype);
    if (s != KDA_OK) return s;
    if (N > 0 && !cu_seqlens) return KDA_ERR_NULL;
    if (N == 0) return KDA_OK;
    if (in_dtype != KDA_BF16 || !kda::chunk_split_supported(N, H, K, V, chunk))
        return KDA_ERR_UNSUPPORTED;
    const size_t need = kda::chunk_split_workspace_bytes(N, total_T, H);
    if (need > kScratchBytes) return KDA_ERR_WORKSPACE;
    void *ws = nullptr;
    hipError_t e = scratch_of_current_device(&ws);
    if (e != hipSuccess) return KDA_ERR_HIP;
    kda::Prologue pro;
    return run_fwd(q, k, v, g, beta, dense_states(s0, sT), pro, o, cu_seqlens, N, 0, total_T, H,
                   K, V, chunk, in_dtype, out_dtype, ws, true, stream);
}

kda_status_t kda_varlen_fwd_paged_prologue(
    const void *q, const void *k, const void *v, const void *g, const void *beta, float *pool,
    int pool_slots, const int32_t *s0_slot, const int32_t *sT_slot, const int32_t *start_pos,
    const int32_t *block_table, int table_stride, int snap_tokens, int page_tokens, void *o,
    const int32_t *cu_seqlens, int N, int total_T, int H, int K, int V, int chunk,
    kda_dtype_t in_dtype, kda_dtype_t out_dtype, void *workspace, size_t workspace_bytes,
    unsigned prologue, float gate_lower_bound, float norm_eps, void *stream) {
    kda_status_t s = validate_fwd(q, k, v, g, beta, o, N, total_T, H, K, V, chunk, in_dtype,
                                  out_dtype);
    if (s != KDA_OK) return s;
    kda::Prologue pro;
    s = make_prologue(prologue, gate_lower_bound, norm_eps, pro);
    if (s != KDA_OK) return s;
    if (!pool) return KDA_ERR_NULL;
    if (!pool_ok(pool_slots, H, K, V)) return KDA_ERR_SHAPE;
    if (block_table &&
        (table_stride < 1 || snap_tokens < 1 || snap_tokens % chunk != 0 || page_tokens < 1 ||
         page_tokens % snap_tokens != 0))
        return KDA_ERR_SHAPE;
    if (N > 0 && !cu_seqlens) return KDA_ERR_NULL;
    bool two_pass;
    s = check_workspace(workspace, workspace_bytes,
                        kda_two_pass_workspace_bytes(N, total_T, H, K, V, chunk), two_pass);
    if (s != KDA_OK) return s;
    if (N == 0) return KDA_OK;
    kda::StateIO io;
    io.s0 = s0_slot ? pool : nullptr;
    io.s0_slot = s0_slot;
    io.sT = sT_slot ? pool : nullptr;
    io.sT_slot = sT_slot;
    if (block_table) {
        io.snap = pool;
        io.block_table = block_table;
        io.table_stride = table_stride;
        io.snap_tokens = snap_tokens;
        io.page_tokens = page_tokens;
        io.snaps_per_page = page_tokens / snap_tokens;
    }
    io.start_pos = start_pos;
    io.pool_slots = pool_slots;
    return run_fwd(q, k, v, g, beta, io, pro, o, cu_seqlens, N, 0, total_T, H, K, V, chunk,
                   in_dtype, out_dtype, workspace, two_pass, stream);
}

kda_status_t kda_varlen_fwd_paged(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, float *pool, int pool_slots,
                                  const int32_t *s0_slot, const int32_t *sT_slot,
                                  const int32_t *start_pos, const int32_t *block_table,
                                  int table_stride, int snap_tokens, int page_tokens, void *o,
                                  const int32_t *cu_seqlens, int N, int total_T, int H, int K,
                                  int V, int chunk, kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    return kda_varlen_fwd_paged_prologue(q, k, v, g, beta, pool, pool_slots, s0_slot, sT_slot,
                                         start_pos, block_table, table_stride, snap_tokens,
                                         page_tokens, o, cu_seqlens, N, total_T, H, K, V, chunk,
                                         in_dtype, out_dtype, workspace, workspace_bytes, 0u, 0.f,
                                         0.f, stream);
}

kda_status_t kda_decode_step_prologue(const void *q, const void *k, const void *v, const void *g,
                                      const void *beta, float *state, void *o, int N, int H,
                                      int K, int V, kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                                      unsigned prologue, float gate_lower_bound, float norm_eps,
                                      void *stream) {
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_DTYPE;
    if (N < 0 || H <= 0 || K <= 0 || V <= 0) return KDA_ERR_SHAPE;
    if (!fits(N, H, (long long)K * V)) return KDA_ERR_SHAPE;
    if (!((K == 128 && V == 128) || (K == 32 && V == 32))) return KDA_ERR_UNSUPPORTED;
    kda::Prologue pro;
    kda_status_t s = make_prologue(prologue, gate_lower_bound, norm_eps, pro);
    if (s != KDA_OK) return s;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL;
    return from_hip(kda::launch_decode(q, k, v, g, beta, state, nullptr, nullptr, 0, pro, o, N,
                                       H, K, V, in_dtype == KDA_BF16, out_dtype == KDA_BF16,
                                       static_cast<hipStream_t>(stream)));
}

kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, float *state, void *o, int N, int H, int K,
                             int V, kda_dtype_t in_dtype, kda_dtype_t out_dtype, void *stream) {
    return kda_decode_step_prologue(q, k, v, g, beta, state, o, N, H, K, V, in_dtype, out_dtype,
                                    0u, 0.f, 0.f, stream);
}

kda_status_t kda_decode_step_paged_prologue(const void *q, const void *k, const void *v,
                                            const void *g, const void *beta, float *pool,
                                            int pool_slots, const int32_t *slot_in,
                                            const int32_t *slot_out, void *o, int N, int H,
                                            int K, int V, kda_dtype_t in_dtype,
                                            kda_dtype_t out_dtype, unsigned prologue,
                                            float gate_lower_bound, float norm_eps,
                                            void *stream) {
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_DTYPE;
    if (N < 0 || H <= 0 || K <= 0 || V <= 0) return KDA_ERR_SHAPE;
    if (!fits(N, H, (long long)K * V)) return KDA_ERR_SHAPE;
    if (!((K == 128 && V == 128) || (K == 32 && V == 32))) return KDA_ERR_UNSUPPORTED;
    if (!pool_ok(pool_slots, H, K, V)) return KDA_ERR_SHAPE;
    kda::Prologue pro;
    kda_status_t s = make_prologue(prologue, gate_lower_bound, norm_eps, pro);
    if (s != KDA_OK) return s;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !pool || !slot_in || !slot_out || !o) return KDA_ERR_NULL;
    return from_hip(kda::launch_decode(q, k, v, g, beta, pool, slot_in, slot_out, pool_slots, pro,
                                       o, N, H, K, V, in_dtype == KDA_BF16, out_dtype == KDA_BF16,
                                       static_cast<hipStream_t>(stream)));
}

kda_status_t kda_decode_step_paged(const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, float *pool, int pool_slots,
                                   const int32_t *slot_in, const int32_t *slot_out, void *o,
                                   int N, int H, int K, int V, kda_dtype_t in_dtype,
                                   kda_dtype_t out_dtype, void *stream) {
    return kda_decode_step_paged_prologue(q, k, v, g, beta, pool, pool_slots, slot_in, slot_out,
                                          o, N, H, K, V, in_dtype, out_dtype, 0u, 0.f, 0.f,
                                          stream);
}

kda_status_t kda_decode_multi_paged_prologue(const void *q, const void *k, const void *v,
                                             const void *g, const void *beta, float *pool,
                                             int pool_slots, const int32_t *slot_in,
                                             const int32_t *slot_out, void *o, int N, int T,
                                             int H, int K, int V, kda_dtype_t in_dtype,
                                             kda_dtype_t out_dtype, unsigned prologue,
                                             float gate_lower_bound, float norm_eps,
                                             void *stream) {
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_DTYPE;
    if (N < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0) return KDA_ERR_SHAPE;
    if (!fits((long long)N * T, H, K > V ? K : V)) return KDA_ERR_SHAPE;
    if (!((K == 128 && V == 128) || (K == 32 && V == 32))) return KDA_ERR_UNSUPPORTED;
    if (!pool_ok(pool_slots, H, K, V)) return KDA_ERR_SHAPE;
    kda::Prologue pro;
    kda_status_t s = make_prologue(prologue, gate_lower_bound, norm_eps, pro);
    if (s != KDA_OK) return s;
    if (N == 0 || T == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !pool || !slot_in || !slot_out || !o) return KDA_ERR_NULL;
    return from_hip(kda::launch_decode_multi(q, k, v, g, beta, pool, slot_in, slot_out, pool_slots,
                                             pro, o, N, T, H, K, V, in_dtype == KDA_BF16,
                                             out_dtype == KDA_BF16, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_decode_multi_paged(const void *q, const void *k, const void *v, const void *g,
                                    const void *beta, float *pool, int pool_slots,
                                    const int32_t *slot_in, const int32_t *slot_out, void *o,
                                    int N, int T, int H, int K, int V, kda_dtype_t in_dtype,
                                    kda_dtype_t out_dtype, void *stream) {
    return kda_decode_multi_paged_prologue(q, k, v, g, beta, pool, pool_slots, slot_in, slot_out,
                                           o, N, T, H, K, V, in_dtype, out_dtype, 0u, 0.f, 0.f,
                                           stream);
}

size_t kda_bwd_workspace_bytes(int N, int total_T, int H, int K, int V, int chunk) {
    if (N < 0 || total_T < 0 || H <= 0 || !kda::chunk_bwd_supported(K, V, chunk)) return 0;
    return kda::chunk_bwd_workspace_bytes(N, total_T, 0, true, H, K, V, chunk);
}

}  // extern "C"

namespace {

kda_status_t run_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                     const float *s0, const float *dout, const float *dsT, float *dq, float *dk,
                     float *dv, float *dg, float *dbeta, float *ds0, const int32_t *cu, int N,
                     int fixedT, int totalT, int H, int K, int V, int chunk, kda_dtype_t in_dtype,
                     void *workspace, size_t workspace_bytes, void *stream) {
    if (!dtype_ok(in_dtype)) return KDA_ERR_DTYPE;
    if (N < 0 || totalT < 0 || H <= 0 || K <= 0 || V <= 0 || chunk <= 0) return KDA_ERR_SHAPE;
    if (!fits(totalT, H, K > V ? K : V) || !fits(N, H, (long long)K * V)) return KDA_ERR_SHAPE;
    if (!kda::chunk_bwd_supported(K, V, chunk)) return KDA_ERR_UNSUPPORTED;
    if (totalT > 0 && (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta))
        return KDA_ERR_NULL;
    if (cu == nullptr && N > 0 && fixedT < 0) return KDA_ERR_SHAPE;
    const size_t need = kda::chunk_bwd_workspace_bytes(N, totalT, 0, true, H, K, V, chunk);
    if (need > 0 && !workspace) return KDA_ERR_NULL;
    if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
    if (N == 0) return KDA_OK;
    return from_hip(kda::launch_chunk_bwd(q, k, v, g, beta, s0, dout, dsT, dq, dk, dv, dg, dbeta,
                                          ds0, cu, N, fixedT, totalT, H, K, V, chunk,
                                          in_dtype == KDA_BF16, workspace,
                                          static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_bwd(const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const float *s0, const float *do_, const float *dsT,
                           float *dq, float *dk, float *dv, float *dg, float *dbeta, float *ds0,
                           int B, int T, int H, int K, int V, int chunk, kda_dtype_t in_dtype,
                           void *workspace, size_t workspace_bytes, void *stream) {
    if (B < 0 || T < 0) return KDA_ERR_SHAPE;
    const long long total = (long long)B * T;
    if (total > INT_MAX) return KDA_ERR_SHAPE;
    return run_bwd(q, k, v, g, beta, s0, do_, dsT, dq, dk, dv, dg, dbeta, ds0, nullptr, B, T,
                   (int)total, H, K, V, chunk, in_dtype, workspace, workspace_bytes, stream);
}

kda_status_t kda_varlen_bwd(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const float *s0, const float *do_,
                            const float *dsT, float *dq, float *dk, float *dv, float *dg,
                            float *dbeta, float *ds0, const int32_t *cu_seqlens, int N,
                            int total_T, int H, int K, int V, int chunk, kda_dtype_t in_dtype,
                            void *workspace, size_t workspace_bytes, void *stream) {
    if (N > 0 && !cu_seqlens) return KDA_ERR_NULL;
    return run_bwd(q, k, v, g, beta, s0, do_, dsT, dq, dk, dv, dg, dbeta, ds0, cu_seqlens, N, 0,
                   total_T, H, K, V, chunk, in_dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"
