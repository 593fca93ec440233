"""GPU parity of the paged-state entry points (prefix caching) against the oracle.

kda_varlen_fwd_paged reads initial states from pool slots, writes final states
to pool slots and leaves a snapshot of each sequence's state at every
snap_tokens boundary in the slot its block table gives; kda_decode_step_paged
reads and writes states through slot indices.  Expected values: the oracle's
outputs and final states, and for a snapshot at boundary p the oracle's final
state over the sequence's first p - start_pos tokens (the definition of the
state after p tokens).  Slots the call must not touch are compared bit for bit
with their contents before the call.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_43_amd import inputs, kda
from oracle import oracle
from tests.parity import TOL, rel_err, report, to_gpu

pytestmark = pytest.mark.gpu


def _pool(seed, slots, H, K, V):
    rng = np.random.default_rng(seed)
    return torch.from_numpy((0.1 * rng.standard_normal((slots, H, K, V))).astype(np.float32))


def _slot_of(table, n, p, snap, page):
    pg = table[n][(p - 1) // page] if (p - 1) // page < len(table[n]) else -1
    return None if pg < 0 else pg * (page // snap) + ((p - 1) % page) // snap


def _expected_paged_fwd(d, cu, pool0, s0_slot, start, table, snap, page):
    """Reference o, final states and {slot: snapshot} for one paged call."""
    N = len(cu) - 1
    H, K, V = pool0.shape[1:]
    s0 = np.zeros((N, H, K, V))
    for n in range(N):
        if s0_slot[n] >= 0:
            s0[n] = pool0[s0_slot[n]].double().numpy()
    o_ref, s_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, s0)
    snaps = {}
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        first = (start[n] // snap + 1) * snap
        for p in range(first, start[n] + (b - a) + 1, snap):
            slot = _slot_of(table, n, p, snap, page)
            if slot is None:
                continue
            r = p - start[n]
            sl = {x: d[x][a:a + r] for x in ("q", "k", "v", "g", "beta")}
            _, st = oracle.recurrence(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"],
                                      np.array([0, r]), s0[n:n + 1])
            snaps[slot] = st[0]
    return o_ref, s_ref, snaps


# (dtype, K, two_pass): the bf16 d=128 two-pass and single-pass kernels, and the
# fp32-arithmetic kernel at both supported shapes
IMPLS = [("bf16", 128, True), ("bf16", 128, False), ("f32", 128, None), ("f32", 32, None),
         ("bf16", 32, None)]


@pytest.mark.parametrize("dtype,K,two_pass", IMPLS)
def test_paged_prefill_snapshots(dtype, K, two_pass):
    C = 16 if K == 32 else 64
    f = C / 64
    snap, page = int(256 * f), int(1024 * f)          # 4 slots per page
    lengths = [int(700 * f), int(337 * f), int(1024 * f), 0]
    start = [0, int(1536 * f), int(448 * f), int(512 * f)]   # multiples of the chunk
    H = 2
    table = [[2, -1], [-1, 0], [1, 3], [-1, -1]]
    s0_slot = [-1, 16, 17, 18]
    sT_slot = [19, 16, 20, 21]                        # sequence 1 updates in place
    slots = 22
    print(f"[case] paged prefill {dtype} K={K} two_pass={two_pass} lengths={lengths} "
          f"start={start}", flush=True)
    d = inputs.draw_varlen(21, H=H, K=K, V=K, dtype=dtype, lengths=lengths)
    cu = d["cu_seqlens"].numpy().astype(np.int64)
    pool0 = _pool(22, slots, H, K, K)
    o_ref, s_ref, snaps = _expected_paged_fwd(d, cu, pool0, s0_slot, start, table, snap, page)
    assert len(snaps) == 7  # 2 + 1 + 4 boundaries, all mapped

    x = to_gpu(d)
    pool = pool0.cuda()
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    o = kda.varlen_fwd_paged(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"], pool,
                             s0_slot=i32(s0_slot), sT_slot=i32(sT_slot), start_pos=i32(start),
                             block_table=i32(table), snap_tokens=snap, page_tokens=page,
                             two_pass=two_pass)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    errs = {"o": rel_err(o, o_ref)}
    for n in range(4):
        errs[f"sT{n}"] = rel_err(pool[sT_slot[n]], s_ref[n])
    for slot, ref in snaps.items():
        errs[f"snap{slot}"] = rel_err(pool[slot], ref)
    report(f"paged_prefill_{dtype}_K{K}_{two_pass}", **errs)
    assert all(e <= tol for e in errs.values()), errs
    written = set(snaps) | set(sT_slot)
    for s in range(slots):
        if s not in written:
            assert torch.equal(pool[s].cpu(), pool0[s]), f"slot {s} was modified"


@pytest.mark.parametrize("two_pass", [True, False])
def test_resume_from_snapshot(two_pass):
    """A prefix hit: restarting at a cached boundary from its snapshot gives the
    same outputs, final state and later snapshots as the uninterrupted run."""
    H, K, T, snap, page = 2, 128, 1024, 256, 1024
    print(f"[case] resume from snapshot two_pass={two_pass}", flush=True)
    d = inputs.draw_varlen(23, H=H, K=K, V=K, dtype="bf16", lengths=[T])
    x = to_gpu(d)
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    pool = torch.zeros(2 * 4 + 2, H, K, K, device="cuda")
    # full run: snapshots into page 0 (slots 0-3), final state to slot 8
    o_full = kda.varlen_fwd_paged(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"],
                                  pool, sT_slot=i32([8]), block_table=i32([[0]]),
                                  snap_tokens=snap, page_tokens=page, two_pass=two_pass)
    # resume at token 512 from its snapshot (slot 1), snapshots into page 1 (slots 4-7)
    h = 512
    sl = {k: x[k][h:].contiguous() for k in ("q", "k", "v", "g", "beta")}
    o_tail = kda.varlen_fwd_paged(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"],
                                  i32([0, T - h]), pool, s0_slot=i32([1]), sT_slot=i32([9]),
                                  start_pos=i32([h]), block_table=i32([[1]]), snap_tokens=snap,
                                  page_tokens=page, two_pass=two_pass)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                     np.array([0, T]))
    tol = TOL["bf16"]
    errs = {"o_full": rel_err(o_full, o_ref), "o_tail": rel_err(o_tail, o_ref[h:]),
            "sT_full": rel_err(pool[8], s_ref[0]), "sT_tail": rel_err(pool[9], s_ref[0])}
    # boundaries 768 and 1024 are slots 2, 3 (first run) and 6, 7 (resumed run)
    for a, b in ((2, 6), (3, 7)):
        errs[f"snap{b}_vs_{a}"] = rel_err(pool[b], pool[a].cpu().double().numpy())
    report(f"resume_two_pass={two_pass}", **errs)
    assert all(e <= tol for e in errs.values()), errs
    assert torch.count_nonzero(pool[4]) == 0 and torch.count_nonzero(pool[5]) == 0


@pytest.mark.parametrize("dtype,K", [("bf16", 128), ("f32", 128), ("bf16", 32)])
def test_paged_decode(dtype, K):
    N, H = 4, 2
    slots = 8
    slot_in = [0, 1, 2, -1]      # the last sequence starts from zeros
    slot_out = [0, 5, 6, 7]      # in place, then three copy-on-write steps
    print(f"[case] paged decode {dtype} K={K}", flush=True)
    pool0 = _pool(24, slots, H, K, K)
    step = inputs.draw_decode_step(25, 0, N, H, K, K, dtype)
    st_in = np.zeros((N, H, K, K))
    for n in range(N):
        if slot_in[n] >= 0:
            st_in[n] = pool0[slot_in[n]].double().numpy()
    o_ref, st_ref = oracle.decode_step(step["q"], step["k"], step["v"], step["g"],
                                       step["beta"], st_in)
    x = to_gpu(step)
    pool = pool0.cuda()
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    o = kda.decode_step_paged(x["q"], x["k"], x["v"], x["g"], x["beta"], pool, i32(slot_in),
                              i32(slot_out))
    torch.cuda.synchronize()
    tol = TOL[dtype]
    errs = {"o": rel_err(o, o_ref)}
    for n in range(N):
        errs[f"s{n}"] = rel_err(pool[slot_out[n]], st_ref[n])
    report(f"paged_decode_{dtype}_K{K}", **errs)
    assert all(e <= tol for e in errs.values()), errs
    for s in (1, 2, 3, 4):       # inputs of copy-on-write steps and unused slots
        assert torch.equal(pool[s].cpu(), pool0[s]), f"slot {s} was modified"


def test_paged_decode_matches_dense_decode():
    """The same step through slots (in place) and through the dense entry point
    gives bit-identical outputs and states."""
    N, H, K = 3, 2, 128
    print("[case] paged vs dense decode", flush=True)
    pool0 = _pool(26, N, H, K, K)
    step = to_gpu(inputs.draw_decode_step(27, 0, N, H, K, K, "bf16"))
    dense = pool0.cuda()
    o_d = kda.decode_step(step["q"], step["k"], step["v"], step["g"], step["beta"], dense)
    pool = pool0.cuda()
    ids = torch.arange(N, dtype=torch.int32, device="cuda")
    o_p = kda.decode_step_paged(step["q"], step["k"], step["v"], step["g"], step["beta"], pool,
                                ids, ids)
    torch.cuda.synchronize()
    assert torch.equal(o_d, o_p) and torch.equal(dense, pool)


@pytest.mark.parametrize("dtype,K", [("bf16", 128), ("f32", 128), ("bf16", 32)])
def test_multi_token_decode(dtype, K):
    """T draft tokens per sequence in one pass: outputs equal T decode steps, and
    the state after token j lands in slot_out[n][j] (the oracle's state after
    that prefix); a sequence may end in its own input slot."""
    N, T, H = 3, 5, 2
    slots = 16
    slot_in = [0, -1, 2]
    slot_out = [[3, -1, 4, -1, 0],
                [5, 6, 7, 8, 9],
                [-1, -1, -1, -1, 10]]
    print(f"[case] multi-token decode {dtype} K={K} N={N} T={T}", flush=True)
    pool0 = _pool(28, slots, H, K, K)
    d = inputs.draw_varlen(29, H=H, K=K, V=K, dtype=dtype, lengths=[T] * N)
    cu = np.arange(N + 1) * T
    s0 = np.zeros((N, H, K, K))
    for n in range(N):
        if slot_in[n] >= 0:
            s0[n] = pool0[slot_in[n]].double().numpy()
    o_ref, _ = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, s0)
    ref_states = {}
    for n in range(N):
        for j in range(T):
            if slot_out[n][j] >= 0:
                sl = {x: d[x][n * T:n * T + j + 1] for x in ("q", "k", "v", "g", "beta")}
                _, st = oracle.recurrence(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"],
                                          np.array([0, j + 1]), s0[n:n + 1])
                ref_states[slot_out[n][j]] = st[0]
    x = to_gpu(d)
    shp = lambda t, D: t.reshape(N, T, H, D) if D else t.reshape(N, T, H)
    pool = pool0.cuda()
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    o = kda.decode_multi_paged(shp(x["q"], K), shp(x["k"], K), shp(x["v"], K), shp(x["g"], K),
                               shp(x["beta"], 0), pool, i32(slot_in), i32(slot_out))
    torch.cuda.synchronize()
    tol = TOL[dtype]
    errs = {"o": rel_err(o.reshape(N * T, H, K), o_ref)}
    for slot, ref in ref_states.items():
        errs[f"s{slot}"] = rel_err(pool[slot], ref)
    report(f"multi_decode_{dtype}_K{K}", **errs)
    assert all(e <= tol for e in errs.values()), errs
    for s in set(range(slots)) - set(ref_states):
        assert torch.equal(pool[s].cpu(), pool0[s]), f"slot {s} was modified"


def test_multi_token_decode_one_token_equals_single_step():
    N, H, K = 4, 2, 128
    print("[case] multi-token decode T=1 vs single paged step", flush=True)
    pool0 = _pool(30, 2 * N, H, K, K)
    step = to_gpu(inputs.draw_decode_step(31, 0, N, H, K, K, "bf16"))
    ids = torch.arange(N, dtype=torch.int32, device="cuda")
    outs = ids + N
    pa = pool0.cuda()
    o_a = kda.decode_step_paged(step["q"], step["k"], step["v"], step["g"], step["beta"], pa, ids,
                                outs)
    pb = pool0.cuda()
    u = lambda t: t.unsqueeze(1).contiguous()
    o_b = kda.decode_multi_paged(u(step["q"]), u(step["k"]), u(step["v"]), u(step["g"]),
                                 u(step["beta"]), pb, ids, outs.reshape(N, 1).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b[:, 0]) and torch.equal(pa, pb)
