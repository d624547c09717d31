"""Benchmark of the joint-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--legs all|none]

A step is one dense bf16 joint-attention forward (QK^T, online softmax, PV,
epilogue -- the whole hot path of dit_attn_fwd_ws: the attention kernel and,
for the query blocks of its last partial round, the merge of their split key
ranges) over the 2048x2048-image DiT shape with its CFG pair: B=2, H=24,
N=512 text + 16384 image = 16896 tokens, D=128, 1% of key rows x8 (inputs
already resident in HBM).  `value` is the algorithmic TFLOP/s of that step
(4 N^2 D flops per (b, h)).  The same forward without the split
(dit_attn_fwd) is timed beside it as `ms_no_split`.

In the same run and on the same stream, timed the same way (W warm-ups, then
K timed launches between HIP events), the other configurations are reported
as legs: the fp8 recipe (quantisation pass + fp8 attention) and the
block-sparse kernel at the 2048^2 shape with B=1, the block-mask selection
(tau = 1, on inputs with spatial locality) and block-sparse attention on the
mask it selects at that shape, the dense kernel at the
1024^2 shape and on the image-to-image joint sequence, and the tiny shape
(launch-bound: its time per launch comes from a HIP graph of many launches,
so host-side call overhead is not counted).  For the step, launch_stats adds
per-launch min / median times and one cold-cache launch.  The fp64 CPU
oracle is timed on a bounded sample of rows of the headline workload (the
CPU baseline); the same leg checks the fp8 leg's output against the oracle
on rows of every work-group (cosine and relative L2 against the exact
attention and against the oracle's fp8 recipe), outside every timed region.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "joint-attention TFLOP/s at 2048² DiT shape (bf16, fp8); % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
PROFILE_DIR = os.path.join(ROOT, "profiles")


def _flops_dense(B, H, N, D=128):
    return 4.0 * B * H * N * N * D


def _time_launches(fn, steps, warmup, torch):
    """Average ms per launch of fn() between HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _launch_stats(fn, steps, torch, flush_mib=512):
    """Per-launch times (an event pair around each of `steps` launches, so a
    little slower than the bracketed average) -> min and median, plus one
    launch after a write of `flush_mib` MiB that evicts L2 and the
    infinity cache (cold-cache time)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    ts = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    junk = torch.empty(flush_mib << 18, dtype=torch.float32, device="cuda")
    junk.fill_(1.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    del junk
    return {"min_ms": round(ts[0], 4), "median_ms": round(ts[len(ts) // 2], 4),
            "cold_ms": round(e0.elapsed_time(e1), 4), "per_launch_samples": steps}


def _source_sha(*names):
    """sha256[:16] of the kernel sources with comments and blank space
    removed, so that an edit to a comment keeps the counters' record valid
    while any change to the code voids it."""
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "joint_attention_non_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic(kernel_key: str, sha: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; otherwise None."""
    path = os.path.join(PROFILE_DIR, "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec.get("bytes_per_launch")


def _cpu_baseline(w, q, k, v, budget_s=18.0):
    """The fp64 oracle on the host cores, on a bounded sample of query rows of
    the headline workload (every key of the row's (b, h) slice): a probe of a
    few hundred rows sizes the sample to about budget_s seconds."""
    import oracle
    from workloads import sample_rows
    qd, kd, vd = (t.double().numpy() for t in (q, k, v))
    n_probe, dt = 512, 0.0
    while True:
        probe = sample_rows(w.batch, w.heads, w.seqlen, n_probe, seed=1)
        t0 = time.perf_counter()
        oracle.attn(qd, kd, vd, w.scale, rows=probe)
        dt = time.perf_counter() - t0
        if dt >= 0.5 or n_probe >= 65536:
            break
        n_probe *= 4
    n = int(max(64, min(400000, len(probe) * budget_s / max(dt, 1e-6))))
    rows = sample_rows(w.batch, w.heads, w.seqlen, n, seed=2)
    t0 = time.perf_counter()
    oracle.attn(qd, kd, vd, w.scale, rows=rows)
    dt = time.perf_counter() - t0
    flops = len(rows) * 4.0 * w.seqlen * w.head_dim
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{len(rows)} random query rows of {w.name} (all {w.seqlen} keys each), "
                      f"fp64, {dt:.1f} s"}


def _graph_us_per_launch(call, n, torch):
    """GPU time per launch of call() from a HIP graph holding n launches."""
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            call()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n)


def _fp8_split_plan(B, H, N, cus):
    """(first split block, ranges) of the fp8 attention grid on `cus` compute
    units: 256-row query blocks, the last partial round cut into key ranges
    of 128-key tiles (none when the grid is whole rounds or smaller than one)."""
    units = B * H * ((N + 255) // 256)
    full, r = divmod(units, cus)
    split = min(cus // r, (N + 127) // 128) if (full >= 1 and r > 0) else 1
    return (units - r, split) if split >= 2 else (units, 1)


def _fp8_accuracy(wf, rows, got, cus):
    """Part of the oracle leg: the fp8 output on `rows` (first, last and one
    random row of every 256-row work-group) against the oracle's exact
    attention on the unquantised inputs, against its fp8 recipe, and against
    the recipe as the library applies it (rows of the split last round: the
    recipe cut into the same key ranges, merged exactly)."""
    import numpy as np
    import oracle
    from workloads import make_workload_inputs
    q, k, v, _ = make_workload_inputs(wf, seed=0)
    ref, _ = oracle.attn(q, k, v, wf.scale, rows=rows)
    q8, sq = oracle.fp8_quantize(q)
    k8, sk = oracle.fp8_quantize(k)
    v8, sv = oracle.fp8_quantize(v)
    rec, _ = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, wf.scale, rows=rows)
    first, split = _fp8_split_plan(wf.batch, wf.heads, wf.seqlen, cus)
    nqb = (wf.seqlen + 255) // 256
    r = rows.numpy()
    in_split = (r // wf.seqlen) * nqb + (r % wf.seqlen) // 256 >= first
    rec_lib = rec.copy()
    if in_split.any():
        rec_lib[in_split], _ = oracle.attn_fp8_recipe(q8, k8, v8, sq, sk, sv, wf.scale, rows=rows[in_split],
                                                      nsplit=split)
    a = got.double().numpy().ravel()

    def cmp(b):
        b = b.ravel()
        return {"cos": round(float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b))), 6),
                "rel_l2": round(float(np.linalg.norm(a - b) / np.linalg.norm(b)), 5)}
    e_ref, e_rec = cmp(ref), cmp(rec)
    rr = rec.ravel()
    b = ref.ravel()
    return {"rows": int(rows.numel()), "vs_exact": e_ref, "vs_recipe": e_rec,
            "vs_recipe_as_applied": dict(cmp(rec_lib), split_rows=int(in_split.sum()), ranges=split),
            "recipe_vs_exact_rel_l2": round(float(np.linalg.norm(rr - b) / np.linalg.norm(b)), 5),
            "gate": {"cos_min": 0.99, "rel_l2_max": 0.05,
                     "cos_met": e_ref["cos"] >= 0.99, "rel_l2_met": e_ref["rel_l2"] <= 0.05}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--legs", default="all", choices=["all", "none"],
                    help="also time the fp8, block-sparse, mask-selection, 1024^2, image-to-image "
                         "and tiny legs")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="after timing, run one device-to-device copy of MIB MiB (a kernel of "
                         "known traffic, to scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the joint-attention kernel is measured on one "
              "GPU's share; multi-GPU runs are not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch

    import joint_attention_non_amd as dit
    from workloads import WORKLOADS, block_rows, make_local_qkv, make_workload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dit.load()

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    # ---- headline: dense bf16 at 2048^2 with the CFG pair ----
    w = WORKLOADS["img2048"]
    log(f"[bench] generating {w.name} inputs")
    q, k, v, _ = make_workload_inputs(w, seed=0)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    wsb = dit.fwd_workspace(qd)
    log(f"[bench] timing {w.name}: warmup {args.warmup}, steps {args.steps}, "
        f"tail-split workspace {dit.fwd_workspace_bytes(qd)} bytes")
    torch.cuda.synchronize()
    step = lambda: dit.attn_fwd(qd, kd, vd, out=o, workspace=wsb)
    ms = _time_launches(step, args.steps, args.warmup, torch)
    ms_plain = _time_launches(lambda: dit.attn_fwd(qd, kd, vd, out=o), args.steps, args.warmup, torch)
    flops = _flops_dense(w.batch, w.heads, w.seqlen, w.head_dim)
    tflops = flops / (ms * 1e-3) / 1e12
    sha = _source_sha("attn_bf16.hip", "device_common.h")
    traffic = _traffic("attn_bf16_img2048", sha)
    stats = _launch_stats(step, args.steps, torch)
    stats["ms_no_split"] = round(ms_plain, 4)
    log(f"[bench] {w.name}: per-launch {stats}")
    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": "attn_dense_kernel<false>",
                "flops_per_launch": flops,
                # achieved HBM rate: the counted bytes over the timed step
                "traffic_gbs": None if traffic is None else round(traffic / (ms * 1e-3) / 1e9, 1),
                "traffic_frac_of_hbm": None if traffic is None else round(traffic / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    log(f"[bench] {w.name}: {ms:.3f} ms  {tflops:.1f} TFLOP/s  {100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak"
        f"  (without the tail split {ms_plain:.3f} ms)")
    del o, wsb

    legs = {}
    fp8_inputs = None
    if args.legs == "all":
        # fp8 recipe at 2048^2, B=1
        wf = WORKLOADS["img2048_fp8"]
        log(f"[bench] leg {wf.name}")
        qf, kf, vf, _ = make_workload_inputs(wf, seed=0)
        qf, kf, vf = (t.to(dev) for t in (qf, kf, vf))
        of = torch.empty_like(qf)
        ws = torch.empty(dit.fp8_workspace_bytes(qf), dtype=torch.uint8, device=dev)
        ms_f = _time_launches(lambda: dit.attn_fwd_fp8(qf, kf, vf, workspace=ws, out=of),
                              args.steps, args.warmup, torch)
        ms_q = _time_launches(lambda: dit.fp8_quantize(qf, kf, vf, workspace=ws),
                              args.steps, args.warmup, torch)
        # dit_attn_fwd_fp8 quantises K and V in its pass (Q inside the
        # attention kernel); the timed quantise-only call does Q, K and V, so
        # the pass inside the call moves 2/3 of its bytes (HBM-bound).
        ms_a = ms_f - ms_q * 2.0 / 3.0
        fp8_rows = block_rows(wf.batch, wf.heads, wf.seqlen, 256, seed=5)
        fp8_out = of.reshape(-1, wf.head_dim)[fp8_rows.to(dev)].float().cpu()
        fp8_inputs = (wf, fp8_rows, fp8_out)
        ff = _flops_dense(wf.batch, wf.heads, wf.seqlen, wf.head_dim)
        nbq = (wf.seqlen + 127) // 128
        qbytes = (3 * qf.numel() * 2                                  # bf16 Q, K, V read
                  + 3 * wf.batch * wf.heads * nbq * 128 * wf.head_dim  # e4m3 codes written
                  + 3 * wf.batch * wf.heads * nbq * 4)                 # fp32 scales written
        legs[wf.name] = {
            "ms_total": round(ms_f, 4),
            "tflops_total": round(ff / (ms_f * 1e-3) / 1e12, 2),
            "frac_total": round(ff / (ms_f * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "ms_quantize_qkv": round(ms_q, 4),
            "ms_attention_est": round(ms_a, 4),
            "attention_est": {"bound": "mfma", "achieved": round(ff / (ms_a * 1e-3) / 1e12, 2),
                              "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(ff / (ms_a * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                              "how": "ms_total - 2/3 ms_quantize_qkv (the call's own pass quantises K, V; "
                                     "Q is quantised inside the attention kernel)"},
            "quantize_qkv": {"bound": "hbm", "achieved": round(qbytes / (ms_q * 1e-3) / 1e9, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(qbytes / (ms_q * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "bytes_per_launch": qbytes},
        }
        log(f"[bench] {wf.name}: {legs[wf.name]}")
        del qf, kf, vf, of, ws

        # block-sparse at 2048^2, B=1
        wsp = WORKLOADS["img2048_sparse"]
        log(f"[bench] leg {wsp.name}")
        qs, ks, vs, mask = make_workload_inputs(wsp, seed=0)
        active = int(mask.sum())
        qs, ks, vs, md = (t.to(dev) for t in (qs, ks, vs, mask))
        os_ = torch.empty_like(qs)
        ms_s = _time_launches(lambda: dit.attn_fwd_blocksparse(qs, ks, vs, md, out=os_),
                              args.steps, args.warmup, torch)
        fs = 4.0 * wsp.batch * wsp.heads * active * 128 * 128 * wsp.head_dim
        legs[wsp.name] = {"ms": round(ms_s, 4), "active_blocks": active,
                          "total_blocks": int(mask.numel()),
                          "bound": "mfma", "achieved": round(fs / (ms_s * 1e-3) / 1e12, 2),
                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(fs / (ms_s * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "flops_counted": "active 128x128 blocks only"}
        log(f"[bench] {wsp.name}: {legs[wsp.name]}")
        del qs, ks, vs, md, os_

        # mask selection at 2048^2, B=1 (tau = 1, inputs with spatial locality),
        # then block-sparse attention on the selected mask
        log("[bench] leg img2048_select")
        qs, ks, vs = (t.to(dev) for t in make_local_qkv(wsp.batch, wsp.heads, wsp.seqlen,
                                                         wsp.text_tokens, seed=0))
        nbs = (wsp.seqlen + 127) // 128
        msel = torch.empty((wsp.batch, wsp.heads, nbs, nbs), dtype=torch.uint8, device=dev)
        wsel = torch.empty(dit.select_blocks_workspace_bytes(qs), dtype=torch.uint8, device=dev)
        os_ = torch.empty_like(qs)
        ms_sel = _time_launches(lambda: dit.select_blocks(qs, ks, 1.0, wsp.text_tokens, out=msel,
                                                          workspace=wsel),
                                max(args.steps, 50), args.warmup, torch)
        active = int(msel.sum())
        ms_ss = _time_launches(lambda: dit.attn_fwd_blocksparse(qs, ks, vs, msel, out=os_),
                               args.steps, args.warmup, torch)
        fs = 4.0 * active * 128 * 128 * wsp.head_dim
        sel_bytes = 2 * qs.numel() * 2 + msel.numel()      # Q, K read once; mask written
        legs["img2048_select"] = {
            "tau": 1.0, "inputs": "make_local_qkv (amp 16, length 8), seed 0",
            "ms_select": round(ms_sel, 4), "active_blocks": active, "total_blocks": int(msel.numel()),
            "density": round(active / msel.numel(), 4),
            "select": {"bound": "hbm", "achieved": round(sel_bytes / (ms_sel * 1e-3) / 1e9, 1),
                       "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": round(sel_bytes / (ms_sel * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                       "bytes_per_launch": sel_bytes},
            "ms_sparse_attention": round(ms_ss, 4),
            "sparse_attention": {"bound": "mfma", "achieved": round(fs / (ms_ss * 1e-3) / 1e12, 2),
                                 "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(fs / (ms_ss * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "ms_select_plus_attention": round(ms_sel + ms_ss, 4),
        }
        log(f"[bench] img2048_select: {legs['img2048_select']}")
        del qs, ks, vs, msel, wsel, os_

        for wname in ("img1024", "i2i2048"):
            w1 = WORKLOADS[wname]
            log(f"[bench] leg {w1.name}")
            q1, k1, v1, _ = make_workload_inputs(w1, seed=0)
            q1, k1, v1 = (t.to(dev) for t in (q1, k1, v1))
            o1 = torch.empty_like(q1)
            ws1 = dit.fwd_workspace(q1)
            ms_1 = _time_launches(lambda: dit.attn_fwd(q1, k1, v1, out=o1, workspace=ws1),
                                  max(args.steps, 50) if w1.seqlen < 8192 else args.steps,
                                  args.warmup, torch)
            f1 = _flops_dense(w1.batch, w1.heads, w1.seqlen, w1.head_dim)
            legs[w1.name] = {"ms": round(ms_1, 4), "achieved": round(f1 / (ms_1 * 1e-3) / 1e12, 2),
                             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(f1 / (ms_1 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                             "shape": f"B{w1.batch} H{w1.heads} N{w1.seqlen}"}
            log(f"[bench] {w1.name}: {legs[w1.name]}")
            del q1, k1, v1, o1, ws1

        # the tiny shape is launch-bound: time a graph of many launches
        wt = WORKLOADS["tiny"]
        log(f"[bench] leg {wt.name}")
        qt, kt, vt, _ = make_workload_inputs(wt, seed=0)
        qt, kt, vt = (t.to(dev) for t in (qt, kt, vt))
        ot = torch.empty_like(qt)
        wst = dit.fwd_workspace(qt)
        tiny = {}
        for label, call in (("us_per_launch", lambda: dit.attn_fwd(qt, kt, vt, out=ot, workspace=wst)),
                            ("us_per_launch_no_split", lambda: dit.attn_fwd(qt, kt, vt, out=ot))):
            tiny[label] = round(_graph_us_per_launch(call, 200, torch), 2)
        ft = _flops_dense(wt.batch, wt.heads, wt.seqlen, wt.head_dim)
        tiny["achieved_tflops"] = round(ft / (tiny["us_per_launch"] * 1e-6) / 1e12, 3)
        tiny["timing"] = "HIP graph of 200 back-to-back launches, replayed; graph time / 200"
        tiny["shape"] = f"B{wt.batch} H{wt.heads} N{wt.seqlen}"
        legs[wt.name] = tiny
        log(f"[bench] {wt.name}: {tiny}")
        del qt, kt, vt, ot, wst

    if args.calib_copy:
        n = args.calib_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {args.calib_copy} MiB read + {args.calib_copy} MiB written")
        del src, dst

    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline (bounded sample)")
        cpu = _cpu_baseline(w, q, k, v)
        log(f"[bench] cpu: {cpu}")
        if fp8_inputs is not None:
            log("[bench] fp8 accuracy against the oracle (rows of every work-group)")
            legs["img2048_fp8"]["accuracy"] = _fp8_accuracy(
                *fp8_inputs, torch.cuda.get_device_properties(0).multi_processor_count)
            log(f"[bench] fp8 accuracy: {legs['img2048_fp8']['accuracy']}")

    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": dict(w.describe(), softmax_scale="1/sqrt(128)", seed=0),
        "roofline": roofline, "cpu_baseline": cpu, "launch_stats": stats, "legs": legs,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
