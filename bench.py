#!/usr/bin/env python3
"""KDA forward throughput on one MI355X: chunked prefill and recurrent decode.

One JSON line on stdout.  A step is one chunked forward pass (kda_chunk_fwd)
over the prefill workload B=1, H=8, T=4096, d_k=d_v=128, chunk 64, bf16
inputs with fp32 state, accumulation and output, on the implementation the
library recommends for it (kda_workspace_bytes > 0: the two-pass path, three
launches: the intra-chunk pass over all chunks, the sequential state pass, the
output pass over all chunks); `value` is its tokens/s.  The single-pass fused kernel's time on
the same workload is reported alongside.  The decode leg (one token for each
of 256 sequences x 32 heads, persistent fp32 state, kda_decode_step) is
reported in the same line under "decode".

Inputs are synthetic and already resident in HBM when the timed region starts.
The roofline objects price the ALGORITHMIC bytes (and flops) of one forward
call against MI355X peaks (HBM 8 TB/s; dense fp16/bf16 MFMA 2.5 PFLOP/s);
call time comes from HIP events on the stream the kernels run on.
The cpu_baseline leg times the fp64 oracle on the host cores.
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


def time_launches(fn, steps, warmup, stream):
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


def cpu_baseline(d, w, wall_budget_s=2.5):
    """fp64 oracle over the whole prefill workload (all heads), repeated until
    about wall_budget_s of wall time (at most 20 passes); input conversion is
    outside the timing."""
    from oracle import oracle
    q, k, v, g, beta = (oracle.as_f64(d[x]) for x in ("q", "k", "v", "g", "beta"))
    threads = oracle.host_threads()
    used = min(threads, w.B * w.H)
    times = []
    while len(times) < 20 and sum(times) < wall_budget_s:
        t0 = time.perf_counter()
        oracle.fixed(q, k, v, g, beta, nthreads=used)
        times.append(time.perf_counter() - t0)
    dt = sum(times) / len(times)
    return {"value": w.B * w.T / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"whole prefill workload B={w.B} H={w.H} T={w.T} ({len(times)} passes, "
                      f"mean {dt:.3f} s wall each, ~{sum(times) * used:.0f} core-s in total), "
                      f"parallel over the {w.B * w.H} (sequence, head) units; "
                      f"{threads} host threads available"}


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
    return {
        "workload": DECODE, "value": wd.N / (dms * 1e-3), "unit": "tokens/s",
        "ms_per_step": dms, "steps": args.decode_steps,
        "roofline": {"bound": "hbm", "achieved": dach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dach / HBM_PEAK_GBS,
                     "traffic": measured_traffic(f"decode_step_kernel_{DECODE_TAG}"),
                     "kernel": "decode_step_kernel", "alg_bytes_per_launch": db},
        "paged_ms_per_step": pms,
        "prologue_ms_per_step": proms,
        "draft_verify": {"draft_tokens": td, "ms_keep_every_state": vms_all,
                         "ms_keep_last_state": vms_last,
                         "tokens_per_s_keep_last": wd.N * td / (vms_last * 1e-3),
                         "ms_same_tokens_as_single_steps": td * dms},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU reaches its steady clock after ~100 prefill calls (~7 ms)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--prefill-workload", default=PREFILL,
                    choices=["prefill_bf16_B1_H8_T4096", "batched_bf16_B4_H32_T8192"])
    ap.add_argument("--only", choices=["prefill", "decode", "copy", "backward"], default=None,
                    help="profiling mode: launch only this kernel --steps times and print "
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

    # ---- prefill: the step
    w = inputs.WORKLOADS[args.prefill_workload]
    d = inputs.draw_fixed(w.seed, w.B, w.T, w.H, w.K, w.V, w.dtype, s0_std=w.s0_std)
    x = {key: (val.to(dev) if val is not None else None) for key, val in d.items()}
    o = torch.empty(w.B, w.T, w.H, w.V, device=dev)
    sT = torch.empty(w.B, w.H, w.K, w.V, device=dev)
    nws = kda.workspace_bytes(w.B, w.B * w.T, w.H, w.K, w.V, w.chunk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    path = "two-pass" if nws else "fused single-pass"
    kernels = ("chunk_prep_kernel + chunk_state_kernel + chunk_output_kernel" if nws
               else "chunk_mfma_kernel")

    def step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], chunk=w.chunk,
                      final_state=sT, out=o, workspace=ws)

    def step_fused():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], chunk=w.chunk,
                      final_state=sT, out=o, two_pass=False)

    if args.only == "backward":
        do = torch.randn(w.B, w.T, w.H, w.V, device=dev)
        for _ in range(args.steps):
            kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, initial_state=x["s0"],
                          chunk=w.chunk)
        torch.cuda.synchronize()
        print(json.dumps({"only": "backward", "workload": w.name, "launches": args.steps}),
              flush=True)
        return
    if args.only == "prefill":
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"only": "prefill", "workload": w.name, "launches": args.steps}),
              flush=True)
        return

    ms, wall = time_launches(step, args.steps, args.warmup, stream)
    ms_fused, _ = time_launches(step_fused, max(5, args.steps // 5), 2, stream) if nws else (ms, 0)

    # the same step through the paged entry point, leaving a state snapshot
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
    nws_p = kda.workspace_bytes(w.B, w.B * w.T, w.H, w.K, w.V, w.chunk)

    def step_snap():
        kda.varlen_fwd_paged(flat["q"], flat["k"], flat["v"], flat["g"], flat["beta"], cu, pool,
                             sT_slot=sT_slot, block_table=table, snap_tokens=snap,
                             page_tokens=page, chunk=w.chunk, out=o_flat,
                             workspace=ws if nws_p else None, two_pass=bool(nws_p))

    ms_snap, _ = time_launches(step_snap, args.steps, 20, stream)

    # the same step from raw projections (unnormalised q and k, gate logits,
    # beta logits): the maps run inside the kernels' loads
    # (kda_chunk_fwd_prologue), against a model-side version that first runs
    # them as separate elementwise passes in torch and then makes the plain call
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

    ms_pro, _ = time_launches(step_pro, args.steps, 20, stream)
    ms_torch_pro, _ = time_launches(step_torch_prologue, args.steps, 20, stream)

    # backward of the same step (kda_chunk_bwd): gradients of every input for
    # a given do and dsT, workspace preallocated
    do = torch.randn(w.B, w.T, w.H, w.V, device=dev, generator=torch.Generator(dev).manual_seed(7))
    dsT = torch.randn(w.B, w.H, w.K, w.V, device=dev, generator=torch.Generator(dev).manual_seed(8))
    bws = torch.empty(kda.bwd_workspace_bytes(w.B, w.B * w.T, w.H, w.K, w.V, w.chunk),
                      dtype=torch.uint8, device=dev)

    def step_bwd():
        kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, initial_state=x["s0"],
                      dsT=dsT, chunk=w.chunk, workspace=bws)

    ms_bwd, _ = time_launches(step_bwd, max(5, args.steps // 5), 3, stream)
    bwd_b = bwd_alg_bytes(w.B, w.T, w.H, w.K, w.V)
    tokens = w.B * w.T
    alg_b = prefill_alg_bytes(w.B, w.T, w.H, w.K, w.V, s0=w.s0_std is not None, sT=True)
    alg_f = prefill_alg_flops(w.B, w.T, w.H, w.K, w.V, w.chunk)
    achieved = alg_b / (ms * 1e-3) / 1e9
    tag = w.name.replace("prefill_bf16_", "prefill_").replace("batched_bf16_", "batched_")
    traffic = measured_traffic(("kda_chunk_fwd_two_pass_" if nws else "chunk_mfma_kernel_") + tag)
    result = {
        "metric": "KDA fwd tokens/s (prefill, decode) + % of MFMA/HBM roofline, 1 MI355X",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, f16 MFMA operands, f32 accumulate/state/out",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "d_k": w.K, "d_v": w.V,
                   "chunk": w.chunk, "global_batch": w.B, "seq_len": w.T,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": f"kda_chunk_fwd {path}: {kernels}",
                     "alg_bytes_per_launch": alg_b},
        "roofline_mfma": {"achieved": alg_f / (ms * 1e-3) / 1e12, "peak": MFMA_F16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": alg_f / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                          "flops": "algorithmic", "alg_flops_per_launch": alg_f},
        "wall_s_timed_region": wall,
        "path": path,
        "fused_single_pass_ms_per_step": ms_fused,
        "prefix_cache": {"ms_per_step_with_snapshots": ms_snap, "snap_tokens": snap,
                         "page_tokens": page, "snapshots_per_call": w.B * w.H * (w.T // snap)},
        "backward": {"ms_per_step": ms_bwd, "tokens_per_s": tokens / (ms_bwd * 1e-3),
                     "kernels": "bwd_prep_kernel + bwd_trans_mfma_kernel + bwd_chain_mfma_kernel (both chains) + "
                                "bwd_udy_mfma_kernel + bwd_kgrad_mfma_kernel (fp32, MFMA at d = 128)",
                     "alg_bytes_per_call": bwd_b,
                     "achieved_GBps": bwd_b / (ms_bwd * 1e-3) / 1e9,
                     "hbm_frac": bwd_b / (ms_bwd * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "prologue": {"ms_per_step_fused_maps": ms_pro,
                     "ms_per_step_torch_maps_then_plain_call": ms_torch_pro,
                     "maps": "q, k L2-normalised (eps 1e-6); g = -0.25 sigmoid(gate logits); "
                             "beta = sigmoid(beta logits)"},
    }

    # ---- decode leg
    if not args.no_decode:
        result["decode"] = decode_leg(args, dev, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
