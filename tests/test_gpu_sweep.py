"""Seeded combinational sweeps of the entry points against the oracle: the
packed forward, the paged forward, the backward pass and multi-token decode.

The other GPU tests vary one property at a time (length, head count, path,
output type, prologue map); here each case draws all of them together from
its own seed, so that combinations no single test names are still compared
element by element with the sequential fp64 recurrence: implementation
(two-pass, single-pass or the library's choice for bf16 d = 128; the fp32 and
d = 32 kernels), packed lengths mixing chunk-edge values and zeros with
random ones, head count, initial state or none, fp32 or bf16 output, and the
input prologue with a random subset of its maps.  Bounds as everywhere:
max|err| / RMS(ref) <= 1e-4 (fp32 inputs) or 2e-2 (bf16 inputs), a bf16
output allowed its own rounding on top.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_43_amd import inputs, kda
from oracle import oracle
from tests.parity import TOL, rel_err, rel_err_rounded, report, to_gpu

pytestmark = pytest.mark.gpu

G_LB = 0.25  # decay bound of the draws and of the gate map (the bf16 kernels' at chunk 64)
CASES = 40


def _case(seed):
    rng = np.random.default_rng(9000 + seed)
    kind = rng.choice(["bf16-128", "bf16-128", "bf16-128", "bf16-128", "bf16-32", "f32-32",
                       "f32-128"])
    dtype, K = kind.split("-")
    K = int(K)
    C = 64 if K == 128 else 16
    N = int(rng.integers(1, 10))
    edge = [0, 1, C - 1, C, C + 1, 2 * C + 3, 5 * C]
    lengths = [int(rng.choice(edge)) if rng.random() < 0.4 else int(rng.integers(0, 600 if K == 128 else 200))
               for _ in range(N)]
    if dtype == "f32" and K == 128:
        lengths = [min(x, 200) for x in lengths]
    H = int(rng.choice([1, 2, 3, 5]))
    two_pass = None
    if kind == "bf16-128":
        two_pass = [None, True, False][int(rng.integers(0, 3))]
    s0 = bool(rng.random() < 0.6)
    out_bf16 = bool(rng.random() < 0.3)
    flags = int(rng.integers(1, 8)) if rng.random() < 0.4 else 0
    return dict(dtype=dtype, K=K, lengths=lengths, H=H, two_pass=two_pass, s0=s0,
                out_bf16=out_bf16, flags=flags)


@pytest.mark.parametrize("seed", range(CASES))
def test_forward_sweep(seed):
    c = _case(seed)
    print(f"[case] sweep seed={seed} {c}", flush=True)
    dtype, K, H = c["dtype"], c["K"], c["H"]
    s0_std = 0.1 if c["s0"] else None
    p = None
    if c["flags"]:
        f = c["flags"]
        raw = inputs.draw_raw_varlen(500 + seed, H, K, K, dtype, c["lengths"], s0_std=s0_std)
        plain = inputs.draw_varlen(700 + seed, H, K, K, dtype, lengths=c["lengths"], g_lb=G_LB)
        d = dict(raw)
        if not f & 1:
            d["q"], d["k"] = plain["q"], plain["k"]
        if not f & 2:
            d["g"] = plain["g"]
        if not f & 4:
            d["beta"] = plain["beta"]
        p = kda.Prologue(normalize_qk=bool(f & 1), gate_lower_bound=G_LB if f & 2 else None,
                         beta_logits=bool(f & 4), norm_eps=1e-6 if f & 1 else 0.0)
        q, k, g, b = oracle.prologue(d["q"], d["k"], d["g"], d["beta"],
                                     normalize_qk=p.normalize_qk,
                                     gate_lower_bound=p.gate_lower_bound,
                                     beta_logits=p.beta_logits, norm_eps=p.norm_eps)
        ref_in = (q, k, oracle.as_f64(d["v"]), g, b)
    else:
        d = inputs.draw_varlen(500 + seed, H, K, K, dtype, lengths=c["lengths"], s0_std=s0_std,
                               g_lb=G_LB)
        ref_in = tuple(d[x] for x in ("q", "k", "v", "g", "beta"))
    cu = d["cu_seqlens"].numpy().astype(np.int64)
    s0_ref = oracle.as_f64(d["s0"]) if d["s0"] is not None else None
    o_ref, s_ref = oracle.recurrence(*ref_in, cu, s0_ref)
    x = to_gpu(d)
    out_dtype = torch.bfloat16 if c["out_bf16"] else torch.float32
    o, sT = kda.varlen_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"], x["s0"],
                           out_dtype=out_dtype, two_pass=c["two_pass"], prologue=p)
    torch.cuda.synchronize()
    eo = rel_err_rounded(o, o_ref, 2.0 ** -8) if c["out_bf16"] else rel_err(o, o_ref)
    es = rel_err(sT, s_ref)
    report(f"sweep_{seed}", o=eo, sT=es)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


# The paged prefill (prefix-cache snapshots): each seeded case draws the
# implementation, packed lengths, start positions on the chunk grid, a block
# table with unmapped pages, initial states from slots or none, final states in
# place or in fresh slots, and a random subset of the prologue maps; expected
# values: the oracle's outputs and final states, and for a snapshot at
# boundary p the oracle's state after the sequence's first p - start tokens;
# slots the call must not write stay bit-identical.
PAGED_IMPLS = [("bf16", 128, True), ("bf16", 128, False), ("bf16", 128, None), ("f32", 128, None),
               ("f32", 32, None), ("bf16", 32, None)]
PAGED_CASES = 16


def _paged_case(seed):
    rng = np.random.default_rng(9500 + seed)
    dtype, K, two_pass = PAGED_IMPLS[int(rng.integers(0, len(PAGED_IMPLS)))]
    C = 16 if K == 32 else 64
    f = C // 16 if K == 32 else 4
    snap, page = 64 * f, 256 * f                     # 4 snapshot slots per page
    N = int(rng.integers(1, 6))
    cap = 300 if (dtype == "f32" and K == 128) else 3 * page
    lengths = [int(rng.choice([0, 1, C - 1, C, snap, snap + 1, page])) if rng.random() < 0.4
               else int(rng.integers(0, cap)) for _ in range(N)]
    start = [int(rng.integers(0, 3 * page // C)) * C for _ in range(N)]
    per = page // snap
    pages_used, table = 0, []
    nblk = max((s + L) // page + 1 for s, L in zip(start, lengths))
    for n in range(N):
        row = []
        for b in range(nblk):
            if rng.random() < 0.75:
                row.append(pages_used)
                pages_used += 1
            else:
                row.append(-1)
        table.append(row)
    nxt = pages_used * per                            # state slots after the pages
    s0_slot, sT_slot = [], []
    for n in range(N):
        if rng.random() < 0.6:
            s0_slot.append(nxt)
            nxt += 1
        else:
            s0_slot.append(-1)
        if s0_slot[-1] >= 0 and rng.random() < 0.5:
            sT_slot.append(s0_slot[-1])               # in place
        else:
            sT_slot.append(nxt)
            nxt += 1
    flags = int(rng.integers(1, 8)) if rng.random() < 0.4 else 0
    return dict(dtype=dtype, K=K, two_pass=two_pass, snap=snap, page=page, lengths=lengths,
                start=start, table=table, s0_slot=s0_slot, sT_slot=sT_slot, slots=nxt + 1,
                H=int(rng.choice([1, 2, 3])), flags=flags)


@pytest.mark.parametrize("seed", range(PAGED_CASES))
def test_paged_prefill_sweep(seed):
    from tests.test_gpu_paged import _expected_paged_fwd, _pool
    c = _paged_case(seed)
    print(f"[case] paged sweep seed={seed} {c}", flush=True)
    dtype, K, H = c["dtype"], c["K"], c["H"]
    p = None
    if c["flags"]:
        fl = c["flags"]
        raw = inputs.draw_raw_varlen(600 + seed, H, K, K, dtype, c["lengths"])
        plain = inputs.draw_varlen(800 + seed, H, K, K, dtype, lengths=c["lengths"], g_lb=G_LB)
        d = dict(raw)
        if not fl & 1:
            d["q"], d["k"] = plain["q"], plain["k"]
        if not fl & 2:
            d["g"] = plain["g"]
        if not fl & 4:
            d["beta"] = plain["beta"]
        p = kda.Prologue(normalize_qk=bool(fl & 1), gate_lower_bound=G_LB if fl & 2 else None,
                         beta_logits=bool(fl & 4), norm_eps=1e-6 if fl & 1 else 0.0)
        q, k, g, b = oracle.prologue(d["q"], d["k"], d["g"], d["beta"],
                                     normalize_qk=p.normalize_qk,
                                     gate_lower_bound=p.gate_lower_bound,
                                     beta_logits=p.beta_logits, norm_eps=p.norm_eps)
        ref_in = dict(q=q, k=k, v=oracle.as_f64(d["v"]), g=g, beta=b)
    else:
        d = inputs.draw_varlen(600 + seed, H, K, K, dtype, lengths=c["lengths"], g_lb=G_LB)
        ref_in = {x: oracle.as_f64(d[x]) for x in ("q", "k", "v", "g", "beta")}
    cu = d["cu_seqlens"].numpy().astype(np.int64)
    pool0 = _pool(700 + seed, c["slots"], H, K, K)
    o_ref, s_ref, snaps = _expected_paged_fwd(ref_in, cu, pool0, c["s0_slot"], c["start"],
                                              c["table"], c["snap"], c["page"])
    x = to_gpu(d)
    pool = pool0.cuda()
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    o = kda.varlen_fwd_paged(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"], pool,
                             s0_slot=i32(c["s0_slot"]), sT_slot=i32(c["sT_slot"]),
                             start_pos=i32(c["start"]), block_table=i32(c["table"]),
                             snap_tokens=c["snap"], page_tokens=c["page"],
                             two_pass=c["two_pass"], prologue=p)
    torch.cuda.synchronize()
    errs = {"o": rel_err(o, o_ref)}
    for n, sl in enumerate(c["sT_slot"]):
        errs[f"sT{n}"] = rel_err(pool[sl], s_ref[n])
    for slot, ref in snaps.items():
        errs[f"snap{slot}"] = rel_err(pool[slot], ref)
    report(f"paged_sweep_{seed}", **{k2: v2 for k2, v2 in list(errs.items())[:6]})
    assert all(e <= TOL[dtype] for e in errs.values()), errs
    written = set(snaps) | set(c["sT_slot"])
    for s in range(c["slots"]):
        if s not in written:
            assert torch.equal(pool[s].cpu(), pool0[s]), f"slot {s} was modified"


# The backward pass: each seeded case draws the input dtype and head size,
# packed lengths (zeros and chunk edges among them), head count, and whether
# an initial state and a final-state gradient are given; every gradient is
# compared with the oracle's (autograd of the plain fp64 recurrence).
BWD_CASES = 12


def _bwd_case(seed):
    rng = np.random.default_rng(9700 + seed)
    dtype, K = [("bf16", 128), ("bf16", 128), ("f32", 128), ("f32", 32), ("bf16", 32)][
        int(rng.integers(0, 5))]
    C = 64 if K == 128 else 16
    N = int(rng.integers(1, 5))
    hi = 260 if K == 128 else 120
    lengths = [int(rng.choice([0, 1, C - 1, C, C + 1])) if rng.random() < 0.4
               else int(rng.integers(0, hi)) for _ in range(N)]
    return dict(dtype=dtype, K=K, lengths=lengths, H=int(rng.choice([1, 2, 3])),
                s0=bool(rng.random() < 0.6), dsT=bool(rng.random() < 0.6))


@pytest.mark.parametrize("seed", range(BWD_CASES))
def test_backward_sweep(seed):
    from tests.test_gpu_bwd import _grads_case
    c = _bwd_case(seed)
    print(f"[case] backward sweep seed={seed} {c}", flush=True)
    dtype, K, H, lengths = c["dtype"], c["K"], c["H"], c["lengths"]
    d = inputs.draw_varlen(900 + seed, H, K, K, dtype, lengths=lengths,
                           s0_std=0.1 if c["s0"] else None, g_lb=G_LB)
    rng = np.random.default_rng(950 + seed)
    tot = int(sum(lengths))
    do = torch.from_numpy(rng.standard_normal((tot, H, K)).astype(np.float32))
    dsT = (torch.from_numpy(rng.standard_normal((len(lengths), H, K, K)).astype(np.float32))
           if c["dsT"] else None)
    _grads_case(f"bwd_sweep_{seed}", d, d["cu_seqlens"].numpy(), dtype, do, dsT)


# Multi-token decode through state slots (T = 1 is the single paged step):
# each seeded case draws dtype and head size, T, the input slots (none, own,
# or one shared by two sequences that branch from it), which token states are
# kept and where (fresh slots, or the sequence's own input slot for its last
# token), and prologue maps; outputs and every kept state are compared with
# the oracle, and every other slot must stay bit-identical.
DEC_CASES = 12


def _decode_case(seed):
    rng = np.random.default_rng(9900 + seed)
    dtype, K = [("bf16", 128), ("f32", 128), ("bf16", 32), ("f32", 32)][int(rng.integers(0, 4))]
    N, T, H = int(rng.integers(1, 7)), int(rng.integers(1, 6)), int(rng.choice([1, 2, 3]))
    nxt = 0
    slot_in = []
    for n in range(N):
        r = rng.random()
        if r < 0.2:
            slot_in.append(-1)
        elif r < 0.35 and n > 0 and slot_in[-1] >= 0:
            slot_in.append(slot_in[-1])               # branch from the previous sequence's state
        else:
            slot_in.append(nxt)
            nxt += 1
    shared = {s for s in slot_in if s >= 0 and slot_in.count(s) > 1}
    slot_out = []
    for n in range(N):
        row = []
        for j in range(T):
            if j == T - 1 and slot_in[n] >= 0 and slot_in[n] not in shared and rng.random() < 0.5:
                row.append(slot_in[n])                # the accepted state back in place
            elif rng.random() < 0.5:
                row.append(nxt + 100)                 # fresh slots, numbered after the inputs
                nxt += 1
            else:
                row.append(-1)
        slot_out.append(row)
    n_in = max([s for s in slot_in if s >= 0] + [-1]) + 1
    slot_out = [[s - 100 + n_in if s >= 100 else s for s in row] for row in slot_out]
    flags = int(rng.integers(1, 8)) if rng.random() < 0.4 else 0
    return dict(dtype=dtype, K=K, N=N, T=T, H=H, slot_in=slot_in, slot_out=slot_out,
                slots=nxt + n_in + 1, flags=flags)


@pytest.mark.parametrize("seed", range(DEC_CASES))
def test_decode_sweep(seed):
    from tests.test_gpu_paged import _pool
    c = _decode_case(seed)
    print(f"[case] decode sweep seed={seed} {c}", flush=True)
    dtype, K, N, T, H = c["dtype"], c["K"], c["N"], c["T"], c["H"]
    lengths = [T] * N
    p = None
    if c["flags"]:
        fl = c["flags"]
        raw = inputs.draw_raw_varlen(1000 + seed, H, K, K, dtype, lengths)
        plain = inputs.draw_varlen(1100 + seed, H, K, K, dtype, lengths=lengths, g_lb=G_LB)
        d = dict(raw)
        if not fl & 1:
            d["q"], d["k"] = plain["q"], plain["k"]
        if not fl & 2:
            d["g"] = plain["g"]
        if not fl & 4:
            d["beta"] = plain["beta"]
        p = kda.Prologue(normalize_qk=bool(fl & 1), gate_lower_bound=G_LB if fl & 2 else None,
                         beta_logits=bool(fl & 4), norm_eps=1e-6 if fl & 1 else 0.0)
        q, k, g, b = oracle.prologue(d["q"], d["k"], d["g"], d["beta"],
                                     normalize_qk=p.normalize_qk,
                                     gate_lower_bound=p.gate_lower_bound,
                                     beta_logits=p.beta_logits, norm_eps=p.norm_eps)
        r = dict(q=q, k=k, v=oracle.as_f64(d["v"]), g=g, beta=b)
    else:
        d = inputs.draw_varlen(1000 + seed, H, K, K, dtype, lengths=lengths, g_lb=G_LB)
        r = {x: oracle.as_f64(d[x]) for x in ("q", "k", "v", "g", "beta")}
    pool0 = _pool(1200 + seed, c["slots"], H, K, K)
    s0 = np.zeros((N, H, K, K))
    for n in range(N):
        if c["slot_in"][n] >= 0:
            s0[n] = pool0[c["slot_in"][n]].double().numpy()
    cu = np.arange(N + 1) * T
    o_ref, _ = oracle.recurrence(r["q"], r["k"], r["v"], r["g"], r["beta"], cu, s0)
    kept = {}
    for n in range(N):
        for j in range(T):
            if c["slot_out"][n][j] >= 0:
                sl = {x: r[x][n * T:n * T + j + 1] for x in r}
                _, st = oracle.recurrence(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"],
                                          np.array([0, j + 1]), s0[n:n + 1])
                kept[c["slot_out"][n][j]] = st[0]
    x = to_gpu(d)
    shp = lambda t, D: t.reshape(N, T, H, D) if D else t.reshape(N, T, H)
    pool = pool0.cuda()
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    o = kda.decode_multi_paged(shp(x["q"], K), shp(x["k"], K), shp(x["v"], K), shp(x["g"], K),
                               shp(x["beta"], 0), pool, i32(c["slot_in"]), i32(c["slot_out"]),
                               prologue=p)
    torch.cuda.synchronize()
    errs = {"o": rel_err(o.reshape(N * T, H, K), o_ref)}
    for slot, ref in kept.items():
        errs[f"s{slot}"] = rel_err(pool[slot], ref)
    report(f"decode_sweep_{seed}", **{k2: v2 for k2, v2 in list(errs.items())[:6]})
    assert all(e <= TOL[dtype] for e in errs.values()), errs
    for s in set(range(c["slots"])) - set(kept):
        assert torch.equal(pool[s].cpu(), pool0[s]), f"slot {s} was modified"
