#!/usr/bin/env python3
"""KDA forward throughput on one MI355X: chunked prefill and recurrent decode.

One JSON line on stdout.  A step is one chunked forward pass over a prefill
workload (bf16 inputs, d_k = d_v = 128, chunk 64, fp32 state, accumulation and
output) on the implementation the library recommends for it
(kda_workspace_bytes: 0 bytes runs the single-pass fused kernel, a workspace
the two-pass path).  The headline workload is the largest one that fits one
GPU: 64 packed sequences with log-uniform lengths in [16, 32768] (seed 3:
219,348 tokens), 16 heads, run through kda_varlen_fwd from zero initial
states; `value` is its tokens/s, from the median of per-call HIP-event
timings with a 512 MiB cache flush before every call.  The batched workload
(B=4, H=32, T=8192) and the small prefill workload (B=1, H=8, T=4096) are
reported alongside under "prefill_legs", together with the prefix-cache,
prologue and backward legs on the small workload, and the decode leg (one
token for each of 256 sequences x 32 heads, persistent fp32 state,
kda_decode_step) under "decode".

Inputs are synthetic and already resident in HBM when the timed region starts.
The roofline objects price the ALGORITHMIC bytes (and flops) of one forward
call against MI355X peaks (HBM 8 TB/s; dense fp16/bf16 MFMA 2.5 PFLOP/s);
call time comes from HIP events on the stream the kernels run on.
roofline_mfma also gives the ceiling the algorithmic flops have at the HBM
floor and, from the committed rocprofv3 counter summary of the same kernel
source, the executed matrix-core rate.
The cpu_baseline leg times the fp64 oracle on the host cores over the whole
headline workload, and compares its result with the timed GPU call's outputs
(max|err|/RMS on o and S_T).
"""

import argparse
import hashlib
import glob
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
PREFILL = "prefill_bf16_B1_H8_T4096"
DECODE = "decode_bf16_N256_H32"
DECODE_TAG = "decode_N256_H32"


def prefill_alg_bytes(B, T, H, K, V, in_bytes=2, out_bytes=4, s0=False, sT=True):
    """q, k, g [B,T,H,K], v [B,T,H,V], beta [B,T,H] read; o [B,T,H,V] written;
    S_0 read and S_T written at K*V*4 bytes per (sequence, head)."""
    th = B * T * H
    b = th * ((3 * K + V) * in_bytes + in_bytes + V * out_bytes)
    b += B * H * K * V * 4 * (int(s0) + int(sT))
    return b


def prefill_alg_flops(B, T, H, K, V, C):
    """Algorithmic flops of the chunked form per token-head: C(C-1)K (strictly
    lower Gram), 2C(C+1)(K+V) over the chunk for the triangular intra-chunk
    products, C^3/3 for the triangular solve, all divided by C; plus 6KV for
    the three state contractions (K S, Q S, K^T U)."""
    per_chunk = C * (C - 1) * K + 2 * C * (C + 1) * (K + V) + C ** 3 / 3.0
    return B * T * H * (per_chunk / C + 6 * K * V)


def bwd_alg_bytes(B, T, H, K, V, in_bytes=2):
    """Algorithmic HBM bytes of one backward call: q, k, v, g, beta read once,
    do (fp32) read once, dq, dk, dv, dg, dbeta (fp32) written once, dsT read and
    ds0 written (fp32 states)."""
    th = B * T * H
    return (th * ((3 * K + V) * in_bytes + in_bytes + V * 4 + (3 * K + V) * 4 + 4)
            + 2 * B * H * K * V * 4)


def decode_alg_bytes(N, H, K, V, in_bytes=2, out_bytes=4):
    """State read + written (2 K V 4), q, k, g, v, beta read, o written."""
    return N * H * (2 * K * V * 4 + (3 * K + V + 1) * in_bytes + V * out_bytes)


# The sources each profiled kernel is built from (a change elsewhere in the
# library leaves its counter summary valid).
_COMMON = ["kda_common.hpp", "kda_mfma.hpp", "prologue.hpp", "state_io.hpp"]
PROFILE_SOURCES = {
    "kda_chunk_fwd_two_pass": ["chunk_split.hip"] + _COMMON,
    "chunk_mfma_kernel": ["chunk_mfma.hip"] + _COMMON,
    "decode_step_kernel": ["decode.hip"] + _COMMON,
    "kda_chunk_bwd": ["chunk_bwd.hip", "kda_common.hpp"],
}


def kernel_source_hash(stem=None):
    """sha256 prefix of the kernel sources behind profile `stem` (all of
    csrc/ when stem is None or unknown)."""
    csrc = os.path.join(ROOT, "gated_delta_rule_43_amd", "csrc")
    names = next((v for k, v in PROFILE_SOURCES.items() if stem and stem.startswith(k)), None)
    files = ([os.path.join(csrc, n) for n in names] if names
             else sorted(glob.glob(os.path.join(csrc, "*"))))
    h = hashlib.sha256()
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(stem):
    """HBM bytes per call from the committed rocprofv3 counter summary
    (profiles/<stem>_traffic.md: FETCH_SIZE + WRITE_SIZE summed over the
    call's kernels, scaled by the plain-copy calibration), or None when that
    summary was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{stem}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source hash:\s*`?([0-9a-f]+)`?", text)
    b = re.search(r"HBM bytes per launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != kernel_source_hash(stem):
        return None
    return float(b.group(1))


def measured_mfma_flops(stem):
    """Executed matrix-core flops per call from the committed rocprofv3 counter
    summary (profiles/<stem>_mfma.md: the MFMA operation counters, in units of
    512 flops, summed over the call's kernels), or None when that summary was
    taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{stem}_mfma.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source hash:\s*`?([0-9a-f]+)`?", text)
    f = re.search(r"executed MFMA flops per launch:\s*([0-9.eE+]+)", text)
    if not m or not f or m.group(1) != kernel_source_hash(stem):
        return None
    return float(f.group(1))


def time_launches(fn, steps, warmup, stream):
    """Mean ms per call of `steps` back-to-back calls after `warmup` calls (one
    event pair around the loop: the warm, pipelined rate)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


class CacheFlush:
    """Writes a 512 MiB buffer (twice the 256 MB Infinity Cache) between timed
    calls, so that each call starts with its inputs in HBM only."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        self.i = 0

    def __call__(self):
        self.i += 1
        self.buf.fill_(self.i & 0xFF)


def time_calls(fn, steps, warmup, stream, flush=None):
    """Each of `steps` calls timed by its own HIP event pair on `stream` (the
    stream the kernels run on), after `warmup` untimed calls; with `flush`, the
    cache is flushed before every call, outside its events.  Returns per-call
    statistics in ms and the wall time of the timed region."""
    import torch
    for _ in range(warmup):
        if flush:
            flush()
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        if flush:
            flush()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return {"median_ms": ms[len(ms) // 2] if len(ms) % 2 else 0.5 * (ms[len(ms) // 2 - 1] + ms[len(ms) // 2]),
            "min_ms": ms[0], "mean_ms": sum(ms) / len(ms), "max_ms": ms[-1],
            "cold": flush is not None, "wall_s": wall}


def settle_clock(stream, fills=1000):
    """Keep the GPU busy for ~50 ms (1000 writes of 256 MiB) so that it reaches
    its steady clock before anything is timed (the first ~50 short calls
    otherwise run slower)."""
    import torch
    buf = torch.empty(256 << 20, dtype=torch.uint8, device=stream.device)
    for i in range(fills):
        buf.fill_(i & 0xFF)
    torch.cuda.synchronize()


def rel_err(x, ref):
    """max|x - ref| / RMS(ref) over a whole tensor (the parity measure)."""
    import numpy as np
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(x - ref))) if x.size else 0.0
    return err / rms if rms > 0.0 else err


def cpu_baseline(d, cu, H, what, gpu_out=None, max_passes=3, wall_budget_s=8.0):
    """fp64 oracle over the whole packed workload d (all (sequence, head)
    units), repeated while the wall budget lasts (at most max_passes); input
    conversion is outside the timing.  With gpu_out = (o, sT) of the timed
    GPU call on the same inputs, the oracle's result also gives that call's
    max|err| / RMS on o and on S_T (after the timing)."""
    from oracle import oracle
    q, k, v, g, beta = (oracle.as_f64(d[x]) for x in ("q", "k", "v", "g", "beta"))
    s0 = oracle.as_f64(d["s0"]) if d.get("s0") is not None else None
    threads = oracle.host_threads()
    units = (len(cu) - 1) * H
    used = min(threads, units)
    times = []
    while len(times) < max_passes and sum(times) < wall_budget_s:
        t0 = time.perf_counter()
        ref = oracle.recurrence(q, k, v, g, beta, cu, s0, nthreads=used)
        times.append(time.perf_counter() - t0)
    dt = sum(times) / len(times)
    tokens = int(cu[-1])
    res = {"value": tokens / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": f"{what}: the whole workload, {tokens} tokens x {H} heads ({len(times)} "
                     f"pass(es), mean {dt:.2f} s wall each, ~{sum(times) * used:.0f} core-s in "
                     f"total), parallel over its {units} (sequence, head) units; {threads} "
                     f"host threads available"}
    if gpu_out is not None:
        o_ref, s_ref = ref
        del ref
        o = gpu_out[0].detach().cpu().double().numpy().reshape(o_ref.shape)
        e_o = rel_err(o, o_ref)
        del o, o_ref
        e_s = rel_err(gpu_out[1].detach().cpu().double().numpy().reshape(s_ref.shape), s_ref)
        res["parity_of_timed_call"] = {"o": e_o, "sT": e_s, "measure": "max|err|/RMS(ref), whole tensors",
                                       "bound": 2e-2}
    return res


def decode_leg(args, dev, stream):
    """Decode workload: persistent fp32 state [256, 32, 128, 128], a fresh token per
    sequence each step (8 pre-drawn steps cycled), one kda_decode_step per step."""
    import torch
    from gated_delta_rule_43_amd import inputs, kda
    wd = inputs.WORKLOADS[DECODE]
    state = inputs.draw_decode_state(wd.seed, wd.N, wd.H, wd.K, wd.V, wd.s0_std).to(dev)
    nin = 8
    steps_in = [{k2: v2.to(dev) for k2, v2 in
                 inputs.draw_decode_step(wd.seed, s, wd.N, wd.H, wd.K, wd.V, wd.dtype).items()}
                for s in range(nin)]
    od = torch.empty(wd.N, wd.H, wd.V, device=dev)
    ctr = [0]

    def dstep():
        xi = steps_in[ctr[0] % nin]
        ctr[0] += 1
        kda.decode_step(xi["q"], xi["k"], xi["v"], xi["g"], xi["beta"], state, out=od)

    if args.only == "decode":
        for _ in range(args.steps):
            dstep()
        torch.cuda.synchronize()
        return {"only": "decode", "workload": DECODE, "launches": args.steps}
    dms, dwall = time_launches(dstep, args.decode_steps, 20, stream)
    db = decode_alg_bytes(wd.N, wd.H, wd.K, wd.V)
    dach = db / (dms * 1e-3) / 1e9
    # the same step on states kept in pool slots (slot n in place)
    slots = torch.arange(wd.N, dtype=torch.int32, device=dev)

    def dstep_paged():
        xi = steps_in[ctr[0] % nin]
        ctr[0] += 1
        kda.decode_step_paged(xi["q"], xi["k"], xi["v"], xi["g"], xi["beta"], state, slots, slots,
                              out=od)

    pms, _ = time_launches(dstep_paged, args.decode_steps, 20, stream)

    # the same step from raw projections: q/k L2 normalisation and the gate and
    # beta logit maps inside the kernel (kda_decode_step_prologue)
    raw = [{k2: v2.to(dev) for k2, v2 in
            inputs.draw_raw_varlen(wd.seed + 100 + s, wd.H, wd.K, wd.V, wd.dtype, [1] * wd.N).items()
            if isinstance(v2, torch.Tensor) and v2.dim() >= 2} for s in range(2)]
    pro = kda.Prologue(normalize_qk=True, gate_lower_bound=0.25, beta_logits=True, norm_eps=1e-6)

    def dstep_pro():
        xi = raw[ctr[0] % 2]
        ctr[0] += 1
        kda.decode_step(xi["q"], xi["k"], xi["v"], xi["g"], xi["beta"], state, out=od, prologue=pro)

    proms, _ = time_launches(dstep_pro, args.decode_steps, 20, stream)

    # draft verification: 4 tokens per sequence in one pass over each state
    # (kda_decode_multi_paged), keeping the state after every draft token in
    # its own slot, or only the last one, in place
    td = 4
    dd = inputs.draw_varlen(wd.seed + 1, H=wd.H, K=wd.K, V=wd.V, dtype=wd.dtype, lengths=[td] * wd.N)
    sh = lambda t: t.to(dev).reshape(wd.N, td, *t.shape[1:])
    dq, dk, dv, dg, dbt = (sh(dd[key]) for key in ("q", "k", "v", "g", "beta"))
    mpool = torch.empty(wd.N * (1 + td), wd.H, wd.K, wd.V, device=dev)
    mpool[:wd.N].copy_(state)
    m_in = torch.arange(wd.N, dtype=torch.int32, device=dev)
    keep_all = (wd.N + torch.arange(wd.N * td, dtype=torch.int32, device=dev)).reshape(wd.N, td)
    keep_last = torch.full((wd.N, td), -1, dtype=torch.int32, device=dev)
    keep_last[:, -1] = m_in
    mo = torch.empty(wd.N, td, wd.H, wd.V, device=dev)

    def verify(slots_out):
        return lambda: kda.decode_multi_paged(dq, dk, dv, dg, dbt, mpool, m_in, slots_out, out=mo)

    vms_all, _ = time_launches(verify(keep_all), args.decode_steps, 10, stream)
    vms_last, _ = time_launches(verify(keep_last), args.decode_steps, 10, stream)

    # the workload's whole 1000-step loop, one launch per step, and the same
    # steps as a HIP graph of the 8 pre-drawn steps replayed 125 times (the
    # library allocates nothing and launches only on the caller's stream, so
    # its calls can be captured)
    n_loop = 1000

    def timed(run):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def eager_loop():
        for _ in range(n_loop):
            dstep()

    loop_ms = timed(eager_loop)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for xi in steps_in:
            kda.decode_step(xi["q"], xi["k"], xi["v"], xi["g"], xi["beta"], state, out=od)
    graph.replay()

    def graph_loop():
        for _ in range(n_loop // nin):
            graph.replay()

    graph_ms = timed(graph_loop)
    return {
        "workload": DECODE, "value": wd.N / (dms * 1e-3), "unit": "tokens/s",
        "ms_per_step": dms, "steps": args.decode_steps,
        "roofline": {"bound": "hbm", "achieved": dach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dach / HBM_PEAK_GBS,
                     "traffic": measured_traffic(f"decode_step_kernel_{DECODE_TAG}"),
                     "kernel": "decode_step_kernel", "alg_bytes_per_launch": db},
        "paged_ms_per_step": pms,
        "prologue_ms_per_step": proms,
        "loop_1000": {"steps": n_loop, "eager_ms_total": loop_ms, "eager_ms_per_step": loop_ms / n_loop,
                      "graph_ms_total": graph_ms, "graph_ms_per_step": graph_ms / n_loop,
                      "graph": f"{nin} steps per graph, replayed {n_loop // nin} times"},
        "draft_verify": {"draft_tokens": td, "ms_keep_every_state": vms_all,
                         "ms_keep_last_state": vms_last,
                         "tokens_per_s_keep_last": wd.N * td / (vms_last * 1e-3),
                         "ms_same_tokens_as_single_steps": td * dms},
    }


def _tag(name):
    """Profile-file tag of a workload name."""
    return (name.replace("prefill_bf16_", "prefill_").replace("batched_bf16_", "batched_")
            .replace("varlen_bf16_", "varlen_"))


def load_prefill(w, dev):
    """The workload's inputs on the GPU, as a packed call: flat [tokens, H, *]
    tensors and cu_seqlens (fixed-length batches are run through their own
    entry point, kda_chunk_fwd, with [B, T, H, *] views)."""
    import torch
    from gated_delta_rule_43_amd import inputs
    if w.kind == "varlen":
        d = inputs.draw_varlen(w.seed, w.H, w.K, w.V, w.dtype, N=w.N, len_min=w.len_min,
                               len_max=w.len_max, s0_std=w.s0_std)
        cu = d["cu_seqlens"].numpy().astype("int64")
    else:
        d = inputs.draw_fixed(w.seed, w.B, w.T, w.H, w.K, w.V, w.dtype, s0_std=w.s0_std)
        for key in ("q", "k", "v", "g", "beta"):
            d[key] = d[key].reshape(w.B * w.T, *d[key].shape[2:])
        import numpy as np
        cu = np.arange(w.B + 1, dtype="int64") * w.T
    x = {key: (val.to(dev) if isinstance(val, torch.Tensor) else val) for key, val in d.items()}
    x["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=dev)
    return d, x, cu


def prefill_call(w, x, cu, dev):
    """The benchmarked call: the library's recommended implementation for the
    workload (kda_workspace_bytes), outputs preallocated."""
    import torch
    from gated_delta_rule_43_amd import kda
    N, tokens = len(cu) - 1, int(cu[-1])
    o = torch.empty(tokens, w.H, w.V, device=dev)
    sT = torch.empty(N, w.H, w.K, w.V, device=dev)
    nws = kda.workspace_bytes(N, tokens, w.H, w.K, w.V, w.chunk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    if w.kind == "varlen":
        def fn():
            kda.varlen_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"], x["s0"],
                           chunk=w.chunk, final_state=sT, out=o, workspace=ws)
    else:
        v4 = {key: x[key].view(w.B, w.T, *x[key].shape[1:]) for key in ("q", "k", "v", "g", "beta")}
        o4 = o.view(w.B, w.T, w.H, w.V)

        def fn():
            kda.chunk_fwd(v4["q"], v4["k"], v4["v"], v4["g"], v4["beta"], x["s0"], chunk=w.chunk,
                          final_state=sT, out=o4, workspace=ws)
    kernels = ("chunk_prep_kernel + chunk_state_kernel + chunk_output_kernel" if nws
               else "chunk_mfma_kernel")
    return fn, ("two-pass" if nws else "fused single-pass"), kernels, (o, sT, ws)


def prefill_leg(w, args, dev, stream, flush, steps, warmup):
    """Cold per-call timing (median, min) with the cache flushed between calls,
    and the warm back-to-back rate, of one prefill workload; roofline of the
    call against HBM (algorithmic bytes) and the MFMA peak (algorithmic flops)."""
    d, x, cu = load_prefill(w, dev)
    fn, path, kernels, _bufs = prefill_call(w, x, cu, dev)
    cold = time_calls(fn, steps, warmup, stream, flush=flush)
    warm_ms, _ = time_launches(fn, steps, 2, stream)
    N, tokens = len(cu) - 1, int(cu[-1])
    ms = cold["median_ms"]
    alg_b = prefill_alg_bytes(1, tokens, w.H, w.K, w.V, s0=w.s0_std is not None, sT=True)
    alg_b += (N - 1) * w.H * w.K * w.V * 4 * (int(w.s0_std is not None) + 1)
    alg_f = prefill_alg_flops(1, tokens, w.H, w.K, w.V, w.chunk)
    achieved = alg_b / (ms * 1e-3) / 1e9
    stem = ("kda_chunk_fwd_two_pass_" if path == "two-pass" else "chunk_mfma_kernel_") + _tag(w.name)
    leg = {
        "workload": w.name, "tokens": tokens, "sequences": N, "heads": w.H,
        "value": tokens / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
        "timing": {**cold, "warm_mean_ms": warm_ms,
                   "flush": "512 MiB written between timed calls (cold); warm = back-to-back loop"},
        "path": path,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(stem),
                     "kernel": f"kda_{'varlen' if w.kind == 'varlen' else 'chunk'}_fwd {path}: {kernels}",
                     "alg_bytes_per_launch": alg_b},
        "roofline_mfma": {"achieved": alg_f / (ms * 1e-3) / 1e12, "peak": MFMA_F16_PEAK_TFLOPS,
                          "unit": "TFLOP/s",
                          "frac": alg_f / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                          "flops": "algorithmic", "alg_flops_per_launch": alg_f,
                          # the most the algorithmic flops can reach: the call
                          # running at the HBM floor of its algorithmic bytes
                          "ceiling_frac_at_hbm_floor":
                              alg_f / (alg_b / (HBM_PEAK_GBS * 1e9)) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                          "target_frac": 0.40},
    }
    ex = measured_mfma_flops(stem)
    if ex is not None:
        leg["roofline_mfma"]["executed"] = {
            "flops_per_launch": ex, "achieved": ex / (ms * 1e-3) / 1e12,
            "frac": ex / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "source": f"profiles/{stem}_mfma.md (rocprofv3 MFMA operation counters)"}
    return leg, d, cu, _bufs[:2]


def next_legs(args, dev, stream):
    """Prefix-cache snapshots, the fused input prologue and the backward pass,
    on the 8-head prefill workload (B=1, H=8, T=4096)."""
    import torch
    from gated_delta_rule_43_amd import inputs, kda
    w = inputs.WORKLOADS[PREFILL]
    d = inputs.draw_fixed(w.seed, w.B, w.T, w.H, w.K, w.V, w.dtype, s0_std=w.s0_std)
    x = {key: (val.to(dev) if val is not None else None) for key, val in d.items()}
    o = torch.empty(w.B, w.T, w.H, w.V, device=dev)
    sT = torch.empty(w.B, w.H, w.K, w.V, device=dev)
    nws = kda.workspace_bytes(w.B, w.B * w.T, w.H, w.K, w.V, w.chunk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    steps = max(10, args.steps)

    # the same call through the paged entry point, leaving a state snapshot
    # every 512 tokens (prefix caching: one 6144-token page per sequence)
    snap, page = 512, 6144
    per_page = page // snap
    pages = -(-w.T // page)
    pool = torch.zeros(w.B * pages * per_page + w.B, w.H, w.K, w.V, device=dev)
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    table = i32([[b * pages + j for j in range(pages)] for b in range(w.B)])
    sT_slot = i32([w.B * pages * per_page + b for b in range(w.B)])
    cu = i32([b * w.T for b in range(w.B + 1)])
    flat = {key: x[key].reshape(w.B * w.T, *x[key].shape[2:]) for key in ("q", "k", "v", "g", "beta")}
    o_flat = o.view(w.B * w.T, w.H, w.V)

    def step_plain():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], chunk=w.chunk,
                      final_state=sT, out=o, workspace=ws)

    def step_snap():
        kda.varlen_fwd_paged(flat["q"], flat["k"], flat["v"], flat["g"], flat["beta"], cu, pool,
                             sT_slot=sT_slot, block_table=table, snap_tokens=snap,
                             page_tokens=page, chunk=w.chunk, out=o_flat,
                             workspace=ws if nws else None, two_pass=bool(nws))

    ms_plain, _ = time_launches(step_plain, steps, 20, stream)
    ms_snap, _ = time_launches(step_snap, steps, 20, stream)

    # raw projections (unnormalised q and k, gate logits, beta logits): the maps
    # run inside the kernels' loads (kda_chunk_fwd_prologue), against running
    # them first as separate elementwise passes in torch and then the plain call
    r = inputs.draw_raw_fixed(w.seed + 100, w.B, w.T, w.H, w.K, w.V, w.dtype, s0_std=w.s0_std)
    xr = {key: (val.to(dev) if val is not None else None) for key, val in r.items()}
    pro = kda.Prologue(normalize_qk=True, gate_lower_bound=0.25, beta_logits=True, norm_eps=1e-6)

    def step_pro():
        kda.chunk_fwd(xr["q"], xr["k"], xr["v"], xr["g"], xr["beta"], xr["s0"], chunk=w.chunk,
                      final_state=sT, out=o, workspace=ws, prologue=pro)

    def step_torch_prologue():
        def unit(t):
            t32 = t.float()
            return (t32 * torch.rsqrt((t32 * t32).sum(-1, keepdim=True) + 1e-6)).to(t.dtype)
        gq, gk = unit(xr["q"]), unit(xr["k"])
        gg = (-0.25 * torch.sigmoid(xr["g"].float())).to(xr["g"].dtype)
        gb = torch.sigmoid(xr["beta"].float()).to(xr["beta"].dtype)
        kda.chunk_fwd(gq, gk, xr["v"], gg, gb, xr["s0"], chunk=w.chunk, final_state=sT, out=o,
                      workspace=ws)

    ms_pro, _ = time_launches(step_pro, steps, 20, stream)
    ms_torch_pro, _ = time_launches(step_torch_prologue, steps, 20, stream)

    # backward of the same call (kda_chunk_bwd): gradients of every input for
    # a given do and dsT, workspace preallocated
    do = torch.randn(w.B, w.T, w.H, w.V, device=dev, generator=torch.Generator(dev).manual_seed(7))
    dsT = torch.randn(w.B, w.H, w.K, w.V, device=dev, generator=torch.Generator(dev).manual_seed(8))
    bws = torch.empty(kda.bwd_workspace_bytes(w.B, w.B * w.T, w.H, w.K, w.V, w.chunk),
                      dtype=torch.uint8, device=dev)

    def step_bwd():
        kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, initial_state=x["s0"],
                      dsT=dsT, chunk=w.chunk, workspace=bws)

    ms_bwd, _ = time_launches(step_bwd, max(20, steps), 5, stream)
    bwd_b = bwd_alg_bytes(w.B, w.T, w.H, w.K, w.V)
    tokens = w.B * w.T
    return {
        "prefix_cache": {"workload": w.name, "ms_per_step_plain": ms_plain,
                         "ms_per_step_with_snapshots": ms_snap, "snap_tokens": snap,
                         "page_tokens": page, "snapshots_per_call": w.B * w.H * (w.T // snap)},
        "prologue": {"workload": w.name, "ms_per_step_fused_maps": ms_pro,
                     "ms_per_step_torch_maps_then_plain_call": ms_torch_pro,
                     "maps": "q, k L2-normalised (eps 1e-6); g = -0.25 sigmoid(gate logits); "
                             "beta = sigmoid(beta logits)"},
        "backward": {"workload": w.name, "ms_per_step": ms_bwd,
                     "tokens_per_s": tokens / (ms_bwd * 1e-3),
                     "kernels": "bwd_prep_kernel + bwd_trans_mfma_kernel + bwd_chain_mfma_kernel "
                                "(both chains) + bwd_udy_mfma_kernel + bwd_kgrad_mfma_kernel "
                                "(fp32, MFMA at d = 128)",
                     "alg_bytes_per_call": bwd_b,
                     "achieved_GBps": bwd_b / (ms_bwd * 1e-3) / 1e9,
                     "hbm_frac": bwd_b / (ms_bwd * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }


PREFILL_WORKLOADS = ["varlen_bf16_N64_H16", "batched_bf16_B4_H32_T8192", "prefill_bf16_B1_H8_T4096"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="time the headline workload (and decode) only")
    ap.add_argument("--prefill-workload", default=PREFILL_WORKLOADS[0], choices=PREFILL_WORKLOADS)
    ap.add_argument("--only", choices=["prefill", "decode", "copy", "backward"], default=None,
                    help="profiling mode: launch only this call --steps times and print "
                         "nothing else (copy = a 512 MiB device copy for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the KDA path here runs on a single MI355X and "
              f"--gpus {args.gpus} is not supported (each (sequence, head) unit is "
              f"independent, so N GPUs would each run this same kernel on 1/N of the units).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_43_amd import inputs, kda
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_43_amd import build
        build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.only == "copy":
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_per_copy": src.numel()}), flush=True)
        return
    if args.only == "decode":
        print(json.dumps(decode_leg(args, dev, stream)), flush=True)
        return
    if args.only == "prefill":
        w = inputs.WORKLOADS[args.prefill_workload]
        d, x, cu = load_prefill(w, dev)
        fn, path, kernels, _bufs = prefill_call(w, x, cu, dev)
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        print(json.dumps({"only": "prefill", "workload": w.name, "path": path,
                          "kernels": kernels, "launches": args.steps}), flush=True)
        return
    if args.only == "backward":
        w = inputs.WORKLOADS[PREFILL]
        d = inputs.draw_fixed(w.seed, w.B, w.T, w.H, w.K, w.V, w.dtype)
        x = {key: (val.to(dev) if val is not None else None) for key, val in d.items()}
        do = torch.randn(w.B, w.T, w.H, w.V, device=dev)
        for _ in range(args.steps):
            kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, chunk=w.chunk)
        torch.cuda.synchronize()
        print(json.dumps({"only": "backward", "workload": w.name, "launches": args.steps}),
              flush=True)
        return

    settle_clock(stream)
    flush = CacheFlush(dev)
    w = inputs.WORKLOADS[args.prefill_workload]
    head, d_head, cu_head, out_head = prefill_leg(w, args, dev, stream, flush, args.steps,
                                                  args.warmup)
    cfg = {"workload": w.name, "sequences": head["sequences"], "tokens": head["tokens"],
           "H": w.H, "d_k": w.K, "d_v": w.V, "chunk": w.chunk, "global_batch": head["sequences"],
           "seq_len": (w.T if w.kind == "fixed" else f"log-uniform [{w.len_min}, {w.len_max}]"),
           "parallelism": "none (1 GPU)"}
    result = {
        "metric": "KDA fwd tokens/s (prefill, decode) + % of MFMA/HBM roofline, 1 MI355X",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, f16 MFMA operands, f32 accumulate/state/out",
        "data": "synthetic",
        "config": cfg,
        "roofline": head["roofline"],
        "roofline_mfma": head["roofline_mfma"],
        "timing": head["timing"],
        "path": head["path"],
    }
    if not args.no_legs:
        legs = {}
        for name in PREFILL_WORKLOADS:
            if name != w.name:
                leg, _, _, _ = prefill_leg(inputs.WORKLOADS[name], args, dev, stream, flush,
                                        args.steps, args.warmup)
                legs[name] = leg
        result["prefill_legs"] = legs
        result.update(next_legs(args, dev, stream))
    if not args.no_decode:
        result["decode"] = decode_leg(args, dev, stream)
    del flush
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d_head, cu_head, w.H, w.name, gpu_out=out_head)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
