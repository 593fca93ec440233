// state_io.hpp -- where a forward or decode call finds and leaves its states.
//
// Dense calls pass s0 / sT as [N, H, K, V] arrays.  Paged calls keep states in
// slots of a pool: slot s holds the H consecutive K x V fp32 states of one
// sequence at one point in time, at pool + s * H * K * V.  Section "Inference
// Serving" of "Kimi K3: Open Frontier Intelligence and Implementation
// Framework" keeps KDA recurrent states in one paged pool and lets requests
// hit a cached prefix at 512-token boundaries inside 6144-token physical
// blocks; a forward call can therefore also leave a snapshot of each
// sequence's state at every multiple of snap_tokens absolute tokens, in the
// slot that the sequence's block table gives for that boundary:
//
//   boundary p (the state after the first p tokens), p = j * snap_tokens:
//     page = block_table[n * table_stride + (p - 1) / page_tokens]
//     slot = page * (page_tokens / snap_tokens) + ((p - 1) % page_tokens) / snap_tokens
//
// (a 6144-token page with 512-token boundaries holds 12 slots; the boundary
// at a page's end belongs to that page).  Entries < 0, blocks at or past
// table_stride and slots at or past pool_slots are skipped, so a bad table
// never writes outside the pool.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

namespace kda {

struct StateIO {
    const float *s0 = nullptr;             // dense [N,H,K,V], or the pool when s0_slot is set; null: zeros
    float *sT = nullptr;                   // dense, or the pool when sT_slot is set; null: not written
    const int32_t *s0_slot = nullptr;      // [N] slot of each initial state (< 0: zeros)
    const int32_t *sT_slot = nullptr;      // [N] slot for each final state (< 0: not written)
    float *snap = nullptr;                 // pool receiving prefix snapshots; null: none
    const int32_t *block_table = nullptr;  // [N, table_stride] physical page of each logical block
    const int32_t *start_pos = nullptr;    // [N] absolute position of each sequence's first token; null: 0
    int pool_slots = 0;                    // slots in the pool (paged states and snapshots)
    int table_stride = 0, snap_tokens = 0, page_tokens = 0;
    int snaps_per_page = 0;                // page_tokens / snap_tokens
};

// Initial state of (n, h): kv consecutive floats, or null for zeros.
__device__ __forceinline__ const float *state_in(const StateIO &io, int n, int h, int H, int kv) {
    if (!io.s0) return nullptr;
    long long s = n;
    if (io.s0_slot) {
        s = io.s0_slot[n];
        if (s < 0 || s >= io.pool_slots) return nullptr;
    }
    return io.s0 + ((size_t)s * H + h) * (size_t)kv;
}

// Destination of the final state of (n, h), or null when it is not wanted.
__device__ __forceinline__ float *state_out(const StateIO &io, int n, int h, int H, int kv) {
    if (!io.sT) return nullptr;
    long long s = n;
    if (io.sT_slot) {
        s = io.sT_slot[n];
        if (s < 0 || s >= io.pool_slots) return nullptr;
    }
    return io.sT + ((size_t)s * H + h) * (size_t)kv;
}

// Walks the boundaries of one sequence.  After each chunk the caller reports
// how many of the sequence's tokens (rel, counted from its first token in this
// call) the state now includes; due(rel) says whether that is the next
// boundary, dest() gives its slot and advance() moves to the one after.  The
// divisions happen once, in init(); the chain only compares and increments.
// init() also loads the sequence's first 128 block-table entries into two
// registers per lane (call it with the whole wave active, next to the initial
// state's loads), so that dest() reads a lane instead of waiting on memory.
// rel grows by whole chunks and boundaries are multiples of the chunk when
// start positions are, so each boundary is met exactly once; a start position
// off the chunk grid meets none (those snapshots are skipped).
struct SnapCursor {
    int next = INT_MAX;  // rel of the next boundary
    int block = 0;       // its logical block (page_tokens tokens each)
    int idx = 0;         // its slot index inside the page
    int pages_lo = -1, pages_hi = -1;  // block-table entries lane and lane + 64
    const int32_t *row = nullptr;      // the sequence's block-table row

    __device__ __forceinline__ void init(const StateIO &io, int n) {
        if (!io.snap) return;
        row = io.block_table + (size_t)n * io.table_stride;
        const int lane = __lane_id();
        if (lane < io.table_stride) pages_lo = row[lane];
        if (lane + 64 < io.table_stride) pages_hi = row[lane + 64];
        long long start = io.start_pos ? io.start_pos[n] : 0;
        if (start < 0) start = 0;
        const long long p = (start / io.snap_tokens + 1) * io.snap_tokens;  // first boundary
        next = p - start > INT_MAX ? INT_MAX : (int)(p - start);
        const long long b = (p - 1) / io.page_tokens;
        block = b > INT_MAX ? INT_MAX : (int)b;
        idx = (int)(((p - 1) % io.page_tokens) / io.snap_tokens);
    }
    __device__ __forceinline__ bool due(int rel) const { return rel == next; }
    // Destination of (n, h) for the current boundary, or null.
    __device__ __forceinline__ float *dest(const StateIO &io, int h, int H, int kv) const {
        if (block >= io.table_stride) return nullptr;
        const long long page = block < 64    ? __builtin_amdgcn_readlane(pages_lo, block)
                               : block < 128 ? __builtin_amdgcn_readlane(pages_hi, block - 64)
                                             : row[block];
        if (page < 0) return nullptr;
        const long long slot = page * io.snaps_per_page + idx;
        if (slot >= io.pool_slots) return nullptr;
        return io.snap + ((size_t)slot * H + h) * (size_t)kv;
    }
    __device__ __forceinline__ void advance(const StateIO &io) {
        next = next > INT_MAX - io.snap_tokens ? INT_MAX : next + io.snap_tokens;
        if (++idx == io.snaps_per_page) {
            idx = 0;
            ++block;
        }
    }
};

// 4 x 4 transpose inside each group of 4 lanes: lane s of a quad holds
// column s of a 4 x 4 block (v[i] = row i) and receives row s (v[j] = column
// j).  Two exchange stages, with the quad's partner s ^ 2, then s ^ 1, each
// sending two of the lane's values and keeping two.
__device__ __forceinline__ float quad_xor2(float x) {  // the value of lane s ^ 2
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor1(float x) {  // the value of lane s ^ 1
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}
template <typename F4>
__device__ __forceinline__ F4 quad_transpose(F4 v, int lane) {
    const bool hi2 = lane & 2, hi1 = lane & 1;
    float r0 = quad_xor2(hi2 ? v[0] : v[2]), r1 = quad_xor2(hi2 ? v[1] : v[3]);
    if (hi2) {
        v[0] = r0;
        v[1] = r1;
    } else {
        v[2] = r0;
        v[3] = r1;
    }
    r0 = quad_xor1(hi1 ? v[0] : v[1]);
    r1 = quad_xor1(hi1 ? v[2] : v[3]);
    if (hi1) {
        v[0] = r0;
        v[2] = r1;
    } else {
        v[1] = r0;
        v[3] = r1;
    }
    return v;
}

}  // namespace kda
