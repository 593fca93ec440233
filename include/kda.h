/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library, libkda.so.
 *
 * The operation.  "Kimi K3: Open Frontier Intelligence and Implementation
 * Framework" (gemslabs.io), section "Hybrid Attention Mechanism", describes
 * Kimi Delta Attention (KDA) as the delta-rule recurrence extended with a
 * channel-wise forget gate, whose lower-bounded decay lets both the diagonal
 * (intra-chunk) and off-diagonal (inter-chunk) tiles run as dense matrix
 * products.  Per sequence and head, with S a K x V fp32 matrix whose rows are
 * key channels:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,            alpha_t = exp(g_t)
 *
 * The gate is passed as g = log(alpha), one value per (token, head, key
 * channel); beta is one scalar per (token, head); no query scale is applied.
 * Section "Inference Serving" of the same page keeps KDA recurrent states
 * per sequence: the state S_T returned by a forward call is exactly the
 * state to resume from (pass it back as s0), and the decode step updates a
 * persistent state in place.
 *
 * Layouts (row-major, contiguous; "tokens" is B*T or total_T):
 *   q, k, g : [tokens, H, K]        v, o : [tokens, H, V]     beta : [tokens, H]
 *   s0, sT  : [N, H, K, V] fp32 (row index = key channel)
 * q, k, v, g and beta all have in_dtype; o has out_dtype.
 *
 * Supported set: (K, V, chunk) = (32, 32, 16) or (128, 128, 64);
 * in_dtype KDA_F32 or KDA_BF16; out_dtype KDA_F32 or KDA_BF16.  Anything
 * else returns KDA_ERR_UNSUPPORTED before any GPU work.
 *
 * Numerical precondition (the lower-bounded decay): -g_lb <= g <= 0 with
 * g_lb * chunk / 2 <= 8 (g_lb = 0.25 at chunk 64, 1.0 at chunk 16).  The
 * bf16 chunked kernels factor the intra-chunk decay around the middle of the
 * chunk and hold the factors in fp16; outside this bound results are
 * unspecified (but every access stays in bounds).  The fp32-input kernels
 * evaluate every decay factor exactly and accept any g <= 0: a model whose
 * decay goes below -0.25 per token (at chunk 64) must pass fp32 inputs, or
 * bf16 gate logits with its bound through a _prologue entry point (below).
 *
 * Magnitudes on the bf16 d = 128 kernels.  Their matrix-core operands are
 * fp16 (11-bit significand, normal range 6.1e-5 .. 6.5e4); accumulation, the
 * state between calls and the outputs are fp32.  The single-pass kernel
 * (workspace_bytes == 0) also rounds the running state, scaled by
 * exp(G_m) <= 1, to fp16 once per chunk, so values and states far below
 * unit scale fall into fp16's subnormal range and lose relative precision:
 * with unit-norm q and k its largest error stays within 2e-2 of the
 * output's RMS (the accuracy the bf16 kernels are held to against an fp64
 * evaluation of the recurrence) for value and state scales from 1e-2 to 1e3
 * (at 1e-3 it is about 3e-2).  The two-pass path advances the state in fp32
 * (decay and value terms), rounding it to fp16 only for the key-correction
 * product, and stays within 2e-2 from 1e-4 to 1e3.  For smaller scales use
 * the two-pass path or fp32 inputs, or rescale v and s0 (the recurrence is
 * linear in them).
 *
 * Ownership and ordering.  The caller allocates every buffer; the library
 * allocates no device memory, keeps no state between calls and is
 * thread-safe (one exception: kda_varlen_fwd_noalloc below uses a static
 * scratch array that the library's code object holds on each GPU).  Every
 * pointer argument is a device pointer (cu_seqlens, slot lists and block
 * tables included).  Every call validates its arguments on the host,
 * then enqueues its kernels on `stream` (a hipStream_t; NULL = the default
 * stream) and returns without synchronising.  Results are ready when the
 * stream is.  A call issues no memset, copy or host-device
 * synchronisation, so calls may be captured into a HIP graph; the first call
 * of each kernel on a device sets its LDS attribute, so make one call of each
 * entry point in use before capturing.
 *
 * Aliasing.  q, k, v, g, beta and o must not overlap each other or the
 * states.  sT == s0 is allowed (in place); otherwise sT and s0 must not overlap.
 *
 * Errors.  Argument errors are detected before any launch: a nonzero status
 * is returned and nothing is enqueued.  A failed launch returns KDA_ERR_HIP.
 * Device-side precondition violations (non-monotone cu_seqlens, g outside
 * the bound, non-finite inputs) give unspecified values but never
 * out-of-bounds accesses: kernels clamp sequence bounds to [0, total_T].
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL                     */
    KDA_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be,
                                or the tensor would exceed 2^31 elements       */
    KDA_ERR_DTYPE = 3,       /* unknown dtype enum                             */
    KDA_ERR_UNSUPPORTED = 4, /* (K, V, chunk) or dtype combination not built   */
    KDA_ERR_WORKSPACE = 5,   /* workspace smaller than kda_workspace_bytes()   */
    KDA_ERR_HIP = 6,         /* the HIP runtime reported an error              */
    KDA_ERR_VALUE = 7        /* a scalar argument out of its range (prologue
                                flags, gate lower bound, normalisation eps)    */
} kda_status_t;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;

/*
 * Chunked forward pass over a fixed-length batch: B sequences of T tokens,
 * tensors [B, T, H, *] (the same as the packed call with cu_seqlens =
 * {0, T, 2T, .., B*T}).
 *   s0 : [B, H, K, V] initial states, or NULL for zeros.
 *   o  : [B, T, H, V] output, out_dtype.
 *   sT : [B, H, K, V] final states, or NULL if not wanted.  May equal s0.
 *   chunk : 16 or 64, as fixed by (K, V) above.
 *   workspace : optional device scratch that selects the implementation:
 *               workspace_bytes == 0 (workspace ignored, may be NULL) runs the
 *               single-pass kernels; workspace_bytes >=
 *               kda_two_pass_workspace_bytes(B, B*T, H, K, V, chunk) > 0 runs
 *               the two-pass bf16 path (intra-chunk pass over all chunks,
 *               then the sequential state pass), which is faster when few
 *               (sequence, head) units leave the GPU underfilled;
 *               kda_workspace_bytes() gives the size to pass for the
 *               recommended choice.  A nonzero workspace_bytes smaller than
 *               kda_two_pass_workspace_bytes() fails with KDA_ERR_WORKSPACE,
 *               and a NULL workspace with nonzero workspace_bytes with
 *               KDA_ERR_NULL.  The caller owns it; concurrent calls need
 *               separate workspaces; its contents are scratch.
 * T = 0 or B = 0 is allowed: sT receives s0 (or zeros) and o is untouched.
 */
kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const float *s0, void *o, float *sT,
                           int B, int T, int H, int K, int V, int chunk,
                           kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Chunked forward pass over N packed sequences of different lengths.
 *   cu_seqlens : DEVICE int32 [N + 1], cu[0] = 0, nondecreasing, cu[N] = total_T.
 *                Sequence n holds tokens [cu[n], cu[n+1]); chunks restart at
 *                every sequence start and the last chunk of each is partial.
 *   s0, sT     : [N, H, K, V] as above; zero-length sequences get sT = s0.
 */
kda_status_t kda_varlen_fwd(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const float *s0, void *o, float *sT,
                            const int32_t *cu_seqlens, int N, int total_T, int H, int K,
                            int V, int chunk, kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_varlen_fwd without allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the two-pass bf16 path of kda_varlen_fwd, with the
 * library's own static scratch in place of the caller's workspace.  The
 * scratch is a device array of KDA_NOALLOC_SCRATCH_BYTES (80 MiB), one copy
 * on every GPU the library is loaded on, held until the process ends; the
 * call itself allocates nothing.  Arguments, layouts and results are those of
 * kda_varlen_fwd with a two-pass-sized workspace (bit-identical output).
 * Limits, checked before any launch: bf16 inputs, (K, V, chunk) =
 * (128, 128, 64) and 1 <= N <= 126, else KDA_ERR_UNSUPPORTED; a call whose
 * two-pass workspace (kda_two_pass_workspace_bytes) exceeds the scratch,
 * KDA_ERR_WORKSPACE.  The scratch found on the CURRENT device is used, so
 * the stream must belong to the current device.  Every call on a GPU shares
 * that GPU's one scratch: calls that overlap in time on one GPU (other
 * streams, other host threads) race and give undefined results; calls
 * ordered on one stream are safe.  Nothing in the scratch needs clearing
 * between calls (every byte read is written earlier in the same call).
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)
kda_status_t kda_varlen_fwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                                    const void *beta, const float *s0, void *o, float *sT,
                                    const int32_t *cu_seqlens, int N, int total_T, int H, int K,
                                    int V, int chunk, kda_dtype_t in_dtype,
                                    kda_dtype_t out_dtype, void *stream);

/*
 * One recurrent decode step: one new token for each of N sequences.
 *   q, k, g : [N, H, K]; v : [N, H, V]; beta : [N, H]   (in_dtype)
 *   state   : [N, H, K, V] fp32, read and updated in place (S_{t-1} -> S_t)
 *   o       : [N, H, V] (out_dtype)
 * Supported (K, V): (32, 32) and (128, 128).
 */
kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, float *state, void *o, int N, int H, int K,
                             int V, kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                             void *stream);

/*
 * Paged states for prefix caching.  Section "Inference Serving" of the page
 * above keeps KDA recurrent states in one paged pool shared with the
 * attention KV cache, and lets a request hit a cached prefix at 512-token
 * boundaries even inside 6144-token physical blocks.  Here a pool is a
 * caller-owned fp32 array of pool_slots slots; slot s holds the H states
 * [H, K, V] of one sequence at one point in time, at pool + s*H*K*V.
 *
 * kda_varlen_fwd_paged: kda_varlen_fwd with the states in a pool, and prefix
 * snapshots.
 *   s0_slot     : DEVICE int32 [N], slot of each sequence's initial state
 *                 (< 0 or >= pool_slots: zeros), or NULL for all zeros.
 *   sT_slot     : DEVICE int32 [N], slot receiving each final state (< 0 or
 *                 >= pool_slots: not written), or NULL for none.
 *                 sT_slot[n] == s0_slot[n] updates in place.
 *   start_pos   : DEVICE int32 [N], absolute position of each sequence's first
 *                 token in this call (its cached prefix length), or NULL for
 *                 all 0.  Must be a multiple of chunk for snapshots to be
 *                 written (boundaries off the chunk grid are skipped).
 *   block_table : DEVICE int32 [N, table_stride], or NULL for no snapshots.
 *                 Entry b is the physical page holding the sequence's
 *                 absolute tokens [b*page_tokens, (b+1)*page_tokens), or < 0.
 *   snap_tokens, page_tokens : boundary interval (a multiple of chunk; 512)
 *                 and page size (a multiple of snap_tokens; 6144), so a page
 *                 holds page_tokens/snap_tokens slots.
 * For every boundary p = j*snap_tokens with start_pos[n] < p <=
 * start_pos[n] + len_n, the state after the sequence's first p tokens is
 * written to slot page*(page_tokens/snap_tokens) + ((p-1) % page_tokens) /
 * snap_tokens, page = block_table[n*table_stride + (p-1)/page_tokens]; the
 * boundary at a page's end belongs to that page.  Blocks at or past
 * table_stride, negative pages and slots at or past pool_slots are skipped.
 * Slots written by one call (final states and snapshots) must be distinct
 * from each other and from every slot the call reads, except a sequence's
 * own in-place sT_slot.  Everything else is as for kda_varlen_fwd (o,
 * workspace and implementation choice, supported set, errors).
 */
kda_status_t kda_varlen_fwd_paged(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, float *pool, int pool_slots,
                                  const int32_t *s0_slot, const int32_t *sT_slot,
                                  const int32_t *start_pos, const int32_t *block_table,
                                  int table_stride, int snap_tokens, int page_tokens, void *o,
                                  const int32_t *cu_seqlens, int N, int total_T, int H, int K,
                                  int V, int chunk, kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_decode_step_paged: kda_decode_step with the states in a pool.
 * Sequence n reads its state from slot slot_in[n] (< 0 or >= pool_slots:
 * zeros) and writes the new state to slot slot_out[n] (< 0 or >= pool_slots:
 * not written); slot_in and slot_out are DEVICE int32 [N].  Equal slots
 * update in place; different slots leave the old state in place, e.g. as the
 * snapshot at a boundary, or to branch a sequence.  Output slots must be
 * distinct from each other and from the input slots of other sequences.
 */
kda_status_t kda_decode_step_paged(const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, float *pool, int pool_slots,
                                   const int32_t *slot_in, const int32_t *slot_out, void *o,
                                   int N, int H, int K, int V, kda_dtype_t in_dtype,
                                   kda_dtype_t out_dtype, void *stream);

/*
 * kda_decode_multi_paged: T consecutive tokens per sequence in one pass over
 * each state, the verification step of speculative decoding (section
 * "Inference Serving" of the page above pairs KDA serving with speculative
 * drafts).  The outputs are those of T decode steps in a row; the state is
 * read once and, after token j of sequence n, written to a slot the caller
 * picks, so that whichever draft prefix is accepted, its state is ready with
 * no second pass.
 *   q, k, g : [N, T, H, K]; v : [N, T, H, V]; beta : [N, T, H]   (in_dtype)
 *   o       : [N, T, H, V] (out_dtype)
 *   slot_in : DEVICE int32 [N], slot of each sequence's state before the
 *             drafts (< 0 or >= pool_slots: zeros)
 *   slot_out: DEVICE int32 [N, T], slot receiving the state after token j
 *             (< 0 or >= pool_slots: not written)
 * The slots written must be distinct from each other and from the input
 * slots of other sequences; a sequence's own input slot may be among its
 * output slots (it is read before anything is written).  T = 1 matches
 * kda_decode_step_paged bit for bit.  Supported (K, V): (32, 32), (128, 128).
 */
kda_status_t kda_decode_multi_paged(const void *q, const void *k, const void *v, const void *g,
                                    const void *beta, float *pool, int pool_slots,
                                    const int32_t *slot_in, const int32_t *slot_out, void *o,
                                    int N, int T, int H, int K, int V, kda_dtype_t in_dtype,
                                    kda_dtype_t out_dtype, void *stream);

/*
 * Input prologue.  The same section describes KDA's decay as lower-bounded
 * and its gate as channel-wise; the parameterisation taken here computes the
 * decay from gate logits x as g = -g_lb * sigmoid(x), which keeps g in
 * [-g_lb, 0], beta as sigmoid(b) of beta logits, and feeds the recurrence
 * L2-normalised queries and keys.  The *_prologue entry points take those
 * raw projections and apply the selected maps inside the kernels' input
 * loads, in fp32, so that a model layer needs no separate elementwise passes
 * (the bytes moved are the same).  prologue is a bitwise OR of:
 *   KDA_PROLOGUE_NORM_QK    q and k are raw: every [K] vector of q and of k
 *                           is scaled by (sum of its squares + norm_eps)^-1/2
 *                           (a vector whose sum is 0 stays 0);
 *   KDA_PROLOGUE_GATE_LOGIT g holds logits x; the decay used is
 *                           g = -gate_lower_bound * sigmoid(x);
 *   KDA_PROLOGUE_BETA_LOGIT beta holds logits b; the value used is sigmoid(b).
 * prologue = 0 is the plain entry point.  Range checks (KDA_ERR_VALUE):
 * unknown bits; norm_eps negative or not finite; with GATE_LOGIT,
 * gate_lower_bound negative or not finite.  With GATE_LOGIT and
 * gate_lower_bound * chunk > 16 (a decay steeper than the bf16 chunked
 * kernels' fp16 factors hold, see the numerical precondition above), a
 * chunked call runs the exact-decay kernel whatever in_dtype is (fp32
 * arithmetic, every decay factor evaluated exactly: correct for any bound,
 * slower), so bf16 inputs with, for example, g_lb = 2 at chunk 64 are served.
 * Everything else (shapes, layouts, states, workspace, errors) is as for the
 * entry point of the same name without the suffix.
 */
typedef enum {
    KDA_PROLOGUE_NORM_QK = 1,
    KDA_PROLOGUE_GATE_LOGIT = 2,
    KDA_PROLOGUE_BETA_LOGIT = 4
} kda_prologue_flags_t;

kda_status_t kda_chunk_fwd_prologue(const void *q, const void *k, const void *v, const void *g,
                                    const void *beta, const float *s0, void *o, float *sT,
                                    int B, int T, int H, int K, int V, int chunk,
                                    kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                                    void *workspace, size_t workspace_bytes,
                                    unsigned prologue, float gate_lower_bound, float norm_eps,
                                    void *stream);

kda_status_t kda_varlen_fwd_prologue(const void *q, const void *k, const void *v, const void *g,
                                     const void *beta, const float *s0, void *o, float *sT,
                                     const int32_t *cu_seqlens, int N, int total_T, int H, int K,
                                     int V, int chunk, kda_dtype_t in_dtype,
                                     kda_dtype_t out_dtype, void *workspace,
                                     size_t workspace_bytes, unsigned prologue,
                                     float gate_lower_bound, float norm_eps, void *stream);

kda_status_t kda_varlen_fwd_paged_prologue(
    const void *q, const void *k, const void *v, const void *g, const void *beta, float *pool,
    int pool_slots, const int32_t *s0_slot, const int32_t *sT_slot, const int32_t *start_pos,
    const int32_t *block_table, int table_stride, int snap_tokens, int page_tokens, void *o,
    const int32_t *cu_seqlens, int N, int total_T, int H, int K, int V, int chunk,
    kda_dtype_t in_dtype, kda_dtype_t out_dtype, void *workspace, size_t workspace_bytes,
    unsigned prologue, float gate_lower_bound, float norm_eps, void *stream);

kda_status_t kda_decode_step_prologue(const void *q, const void *k, const void *v, const void *g,
                                      const void *beta, float *state, void *o, int N, int H,
                                      int K, int V, kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                                      unsigned prologue, float gate_lower_bound, float norm_eps,
                                      void *stream);

kda_status_t kda_decode_step_paged_prologue(const void *q, const void *k, const void *v,
                                            const void *g, const void *beta, float *pool,
                                            int pool_slots, const int32_t *slot_in,
                                            const int32_t *slot_out, void *o, int N, int H,
                                            int K, int V, kda_dtype_t in_dtype,
                                            kda_dtype_t out_dtype, unsigned prologue,
                                            float gate_lower_bound, float norm_eps,
                                            void *stream);

kda_status_t kda_decode_multi_paged_prologue(const void *q, const void *k, const void *v,
                                             const void *g, const void *beta, float *pool,
                                             int pool_slots, const int32_t *slot_in,
                                             const int32_t *slot_out, void *o, int N, int T,
                                             int H, int K, int V, kda_dtype_t in_dtype,
                                             kda_dtype_t out_dtype, unsigned prologue,
                                             float gate_lower_bound, float norm_eps,
                                             void *stream);

/*
 * Backward pass: the gradients of the loss L = sum(do * o) + sum(dsT * S_T)
 * with respect to every input of the forward call with the same arguments
 * (the recurrence above, differentiated through the same chunked algebra in
 * reverse: the per-chunk products, then the state gradient carried from each
 * chunk's end to its start, chunk after chunk from the last).
 *   do_   : [tokens, H, V] fp32, the gradient of o.
 *   dsT   : [N, H, K, V] fp32, the gradient of S_T, or NULL for zeros.
 *   s0    : the forward's initial states, or NULL for zeros.
 *   dq, dk, dg : [tokens, H, K] fp32;  dv : [tokens, H, V] fp32;
 *   dbeta : [tokens, H] fp32;  ds0 : [N, H, K, V] fp32, or NULL if not wanted.
 * Every gradient is written in full (rows of every token).  All arithmetic is
 * fp32 (bf16 inputs are widened exactly).  The workspace is required: at
 * least kda_bwd_workspace_bytes(N, total_T, ...) bytes (a per-(chunk, head)
 * record of the chunk's products plus each chunk's start state and end-state
 * gradient); NULL with a nonzero requirement is KDA_ERR_NULL, too small is
 * KDA_ERR_WORKSPACE.  Numerical precondition: that of the bf16 forward
 * (-g_lb <= g <= 0 with g_lb * chunk / 2 <= 8), for both input dtypes, since
 * the decay factors are factored around the middle of each chunk.
 * Supported (K, V, chunk): (32, 32, 16) and (128, 128, 64).
 */
kda_status_t kda_chunk_bwd(const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const float *s0, const float *do_, const float *dsT,
                           float *dq, float *dk, float *dv, float *dg, float *dbeta, float *ds0,
                           int B, int T, int H, int K, int V, int chunk, kda_dtype_t in_dtype,
                           void *workspace, size_t workspace_bytes, void *stream);

kda_status_t kda_varlen_bwd(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const float *s0, const float *do_,
                            const float *dsT, float *dq, float *dk, float *dv, float *dg,
                            float *dbeta, float *ds0, const int32_t *cu_seqlens, int N,
                            int total_T, int H, int K, int V, int chunk, kda_dtype_t in_dtype,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of a backward call over N sequences and total_T tokens
 * (an upper bound for any lengths; 0 for an unsupported shape). */
size_t kda_bwd_workspace_bytes(int N, int total_T, int H, int K, int V, int chunk);

/* Workspace bytes for the recommended implementation of a forward call over
 * N sequences, total_T tokens: nonzero (the two-pass size) when the two-pass
 * path is supported and expected to be faster (bf16 inputs assumed; at least
 * 4 chunks per sequence on average, and at most 24 (sequence, head) units, or
 * 32 when sequences average at most 16 chunks), else 0. */
size_t kda_workspace_bytes(int N, int total_T, int H, int K, int V, int chunk);

/* Workspace bytes that select the two-pass path whenever it is supported:
 * (K, V, chunk) = (128, 128, 64), 1 <= N <= 126; 0 when it is not.  The
 * two-pass path runs for bf16 inputs only; fp32 inputs ignore the workspace.
 * Size: ceil((total_T + 63 N) / 64) * H * 131584 bytes. */
size_t kda_two_pass_workspace_bytes(int N, int total_T, int H, int K, int V, int chunk);

/* Static, human-readable name of a status code. */
const char *kda_status_str(kda_status_t status);

/* Library ABI version (major * 100 + minor). */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
