#!/usr/bin/env python3
"""Benchmark of the tree-verification step on one MI355X.

One step = tv_tree_verify_attn -> tv_lmhead_argmax -> tv_accept_compact
(acceptance and KV compaction in one launch; with --paged, tv_tree_accept ->
tv_kv_compact_paged) on one stream, over one batch of synthetic inputs already
resident in HBM (the Qwen3-8B-shaped layer with a 1024-token prefix and a
64-node draft tree by default).  Prints one JSON line with verified tree
nodes/s of the step captured once as a HIP graph and replayed, the step
time, the roofline fraction of the dominant kernel (the LM head, whose
per-launch time is taken with HIP events on the launch stream in eager
steps), and the fp64 oracle timed on this host's cores as a CPU baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--paged PAGE_SIZE] [--model qwen3_8b] [--tree CONFIG]
                    [--decode STEPS --model qwen3_8b] [--compact-stack LAYERS]

--paged keeps the key/value caches in pages of a shared pool (placed by a
seeded random permutation) and runs the paged attention and compaction calls.
--model runs the whole multi-layer verification step instead (36 Qwen3-8B-
shaped layers with synthetic weights, LM head, acceptance, one compaction
launch for every layer), captured once as a graph and replayed.
--tree times draft-tree construction from a path-conditioned draft head
(tv_tree_build_level per depth + tv_tree_build_finish) on a named
configuration (e.g. quickstart_d20_w7_n128), with the one-launch per-depth
tv_tree_build beside it.
--decode runs STEPS steps of ragged speculative decoding with the model
(tree construction, multi-layer pass, acceptance, compaction per step) and
reports generated tokens per second of device time.
--compact-stack times one tv_kv_compact_layers launch over LAYERS stacked
layers of the ragged-batch geometry (8 sequences, 8 KV heads of 128, prefixes
512-8192, 64-node trees of depth <= 12), each sequence accepting the root
path of its deepest node, with L2 and the infinity cache evicted (by a
1 GiB read) before each launch: the bandwidth evidence for compaction, whose
single-layer launches are too small to say anything but latency.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
FP32_VEC_TFLOPS = 157.3
METRIC = "verified tree nodes/s + verify-step µs on 1 MI355X; % of HBM/MFMA roofline"
DEFAULT_WORKLOAD = "qwen3_30b_a3b_B4_L4096_N1024"
# (multi-layer pass, decode loop) workloads of each synthetic model's geometry
MODEL_WORKLOADS = {"qwen3_8b": ("qwen3_8b_L1024_N64", "qwen3_8b_ragged8_N64")}
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
LMHEAD_SOURCES = [os.path.join(ROOT, "tree_draft_verification_amd", "csrc", f)
                  for f in ("lmhead.hip", "gemm.hip", "tv_internal.h")]
COMPACT_SOURCES = [os.path.join(ROOT, "tree_draft_verification_amd", "csrc", f)
                   for f in ("compact.hip", "accept_core.h", "tv_internal.h")]


def kernel_source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_work(wl, a, path, path_len, slots=False):
    """Bytes and flops each part must move / compute (not what it wastes).
    With slots (a slot table), the commit reads and writes each sequence's
    N-entry table window and its length instead of moving rows."""
    e = 2 if wl.dtype == "bf16" else 4
    L = a["seq_lens"].astype(np.int64)
    depth = a["depth"].astype(np.int64)
    attn_bytes = int((2 * L * wl.Hkv * wl.D * e).sum()
                     + wl.B * wl.N * (2 * wl.Hq * wl.D * e + 2 * wl.Hkv * wl.D * e + 4))
    attn_flops = int(4 * wl.Hq * wl.D * (L[:, None] + depth + 1).sum())
    lm_bytes = int(wl.V * wl.hidden * e + wl.M * wl.hidden * e + 4 * wl.M)
    lm_flops = int(2 * wl.M * wl.hidden * wl.V)
    moved = sum(int((path[b, :path_len[b]] != np.arange(path_len[b])).sum())
                for b in range(wl.B))
    compact_bytes = (int(8 * wl.B * wl.N + 8 * wl.B) if slots
                     else int(4 * moved * wl.Hkv * wl.D * e + 8 * wl.B))
    accept_bytes = int(12 * wl.B * wl.N + 4 * wl.B * (path.shape[1] + 2))
    return dict(attn=(attn_bytes, attn_flops), lmhead=(lm_bytes, lm_flops),
                accept=(accept_bytes, 0), compact=(compact_bytes, 0),
                accept_compact=(accept_bytes + compact_bytes, 0))


def gemm8_plan(M, V):
    """W tiles of each width (384-row tiles first, then 256-row ones) that the
    library's LM head takes from 256 rows on: the split with the fewest rounds
    of 256 workgroups, a 384-row round counting 1.425 of a 256-row one and a
    second launch 0.05; on equal cost the most 384-row tiles."""
    nmt = -(-M // 256)

    def rounds(t):
        return -(-(nmt * t) // 256)

    best, cost = (0, -(-V // 256)), rounds(-(-V // 256))
    a = -(-V // 384)
    if rounds(a) * 1.425 < cost:
        best, cost = (a, 0), rounds(a) * 1.425
    n = 1
    while 384 * n < V:
        tail = -(-(V - 384 * n) // 256)
        c = rounds(n) * 1.425 + rounds(tail) + 0.05
        if c <= cost:
            best, cost = (n, tail), c
        n += 1
    return best


def lmhead_kernel_name(M, V, dtype):
    """Name of the kernel the library runs for the LM head at these sizes
    (the label only; it follows the library's host-side choice: the
    streaming kernel up to 64 rows, the eight-wavefront product from 256
    rows, in one or two launches by W tile width as gemm8_plan splits the
    vocabulary)."""
    if dtype != "bf16":
        return "lmhead_f32_kernel"
    if M <= 64:
        return "lmhead_stream_kernel (packed W)"
    if M >= 256:
        n384, n256 = gemm8_plan(M, V)
        nt = "true" if M <= 256 else "false"  # one H slice: non-temporal W loads
        names = ([f"gemm8_argmax_kernel<384, {nt}>"] if n384 else []) + \
            ([f"gemm8_argmax_kernel<256, {nt}>"] if n256 else [])
        return " + ".join(names + ["argmax_reduce_kernel"])
    return "gemm32_kernel + argmax_reduce_kernel"


def roof_entry(nbytes, flops, us, dtype):
    t = us * 1e-6
    gbs = nbytes / t / 1e9
    tflops = flops / t / 1e12
    peak_f = BF16_DENSE_TFLOPS if dtype == "bf16" else FP32_VEC_TFLOPS
    t_roof = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (peak_f * 1e12))
    bound = "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (peak_f * 1e12) else "mfma"
    return dict(us=round(us, 2), bytes=nbytes, flops=flops, gbs=round(gbs, 1),
                tflops=round(tflops, 2), bound=bound, roof_us=round(t_roof * 1e6, 2),
                frac=round(t_roof / t, 4))


def cpu_baseline(wl, a, lm, coins, budget_s=20.0):
    """The fp64 oracle, as it stands, on verification steps of the same
    workload, repeated until about budget_s seconds have passed.  Batches of
    more than 1024 nodes are sampled one sequence at a time (its attention,
    its LM-head rows, its acceptance and compaction), cycling through the
    batch."""
    import oracle
    from workloads import draft_tokens
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    per_seq = wl.M > 1024
    reps, spent, nodes = 0, 0.0, 0
    while reps < 20 and (reps == 0 or spent < budget_s):
        if per_seq:
            b = reps % wl.B
            sb = slice(b, b + 1)
            att = {k: (a[k][sb] if k in ("q", "k_cache", "v_cache", "seq_lens", "parent", "depth")
                       else a[k]) for k in a}
            hid = lm["hidden"][b * wl.N:(b + 1) * wl.N]
            co = {k: v[sb] for k, v in coins.items()}
        else:
            att, hid, co = a, lm["hidden"], coins
        nb = att["parent"].shape[0]
        t0 = time.perf_counter()
        oracle.tree_attention(att["q"], att["k_cache"], att["v_cache"], att["seq_lens"],
                              att["parent"], att["scale"], wl.dtype)
        ref = oracle.lm_head_argmax(hid, lm["w"], wl.dtype)
        t1 = time.perf_counter()
        tgt = ref["argmax"].reshape(nb, wl.N)
        draft = draft_tokens(att["parent"], co, tgt)           # drafter input, untimed
        t2 = time.perf_counter()
        acc = oracle.tree_accept(att["parent"], draft, tgt, 32)
        oracle.kv_compact(att["k_cache"], att["v_cache"], att["seq_lens"], acc["path"],
                          acc["path_len"])
        t3 = time.perf_counter()
        spent += (t1 - t0) + (t3 - t2)
        nodes += nb * wl.N
        reps += 1
    what = (f"{reps} single-sequence verification step(s) of {wl.name}" if per_seq
            else f"{reps} whole verification step(s) of {wl.name}")
    return dict(value=round(nodes / spent, 3), unit="nodes/s", cores=int(cores),
                kind="oracle",
                sample=f"{what} ({wl.N} nodes each, {spent:.1f} s of fp64 numpy)")


def copy_calibration(nbytes: int, reps: int = 5) -> None:
    """A plain device copy of known size, to scale HBM counters against."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help=f"workload (default {DEFAULT_WORKLOAD}; with --model, the model's own: "
                         "its 64-node step for the pass, its ragged batch for --decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--paged", type=int, default=0,
                    help="page size of a paged key/value cache (0: contiguous caches)")
    ap.add_argument("--model", default=None,
                    help="time the multi-layer pass of this synthetic model (e.g. qwen3_8b)")
    ap.add_argument("--decode", type=int, default=0,
                    help="steps of multi-step speculative decoding (with --model)")
    ap.add_argument("--tree-depth", type=int, default=20)
    ap.add_argument("--tree-width", type=int, default=7)
    ap.add_argument("--tree-budget", type=int, default=63)
    ap.add_argument("--tree", default=None,
                    help="time draft-tree construction on this configuration")
    ap.add_argument("--compact-stack", type=int, default=0,
                    help="time layered KV compaction over this many stacked layers")
    ap.add_argument("--compact-path-depth", type=int, default=20,
                    help="accepted paths of this depth through level-ordered trees of width 7 "
                         "(0: the deepest root paths of the workload's own trees)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time the LM head's plain product through torch.matmul (the "
                         "vendor GEMM library, no argmax) for comparison")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="only run a plain device copy of this many bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the step has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        copy_calibration(args.calibrate_copy)
        return
    if args.workload is None:
        if args.model:
            if args.model not in MODEL_WORKLOADS:
                print(f"bench.py: --model {args.model} needs a --workload of its attention geometry",
                      file=sys.stderr)
                sys.exit(2)
            args.workload = MODEL_WORKLOADS[args.model][1 if args.decode else 0]
        else:
            args.workload = DEFAULT_WORKLOAD
    if args.model and args.decode:
        decode_bench(args)
        return
    if args.model:
        model_bench(args)
        return
    if args.tree:
        tree_bench(args)
        return
    if args.compact_stack:
        compact_stack_bench(args)
        return

    import torch

    import tree_draft_verification_amd as tv
    from workloads import (WORKLOADS, attn_inputs, draft_coins, draft_tokens, lmhead_inputs,
                           paged_layout)

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    a = attn_inputs(wl)
    lm = lmhead_inputs(wl)
    coins = draft_coins(wl, a["depth"])

    def to_dev(x):
        x = np.ascontiguousarray(x)
        if wl.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)

    q = to_dev(a["q"])
    ps = args.paged
    if ps:
        pg = paged_layout(a["k_cache"], a["v_cache"], ps, seed=wl.seed + ps)
        kc, vc = to_dev(pg["k_pages"]), to_dev(pg["v_pages"])
        block_table = i32(pg["block_table"])
    else:
        kc, vc = to_dev(a["k_cache"]), to_dev(a["v_cache"])
    hid, w = to_dev(lm["hidden"]), to_dev(lm["w"])
    # The vocabulary projection is a static weight: repack it once, outside
    # the timed region, into the layout the LM-head kernel streams fastest.
    w_step = tv.tv_lmhead_pack_weights(w) if wl.dtype == "bf16" else w
    lens0 = i32(a["seq_lens"])
    lens = lens0.clone()
    parent = i32(a["parent"])
    max_len = int(a["seq_lens"].max())
    out = torch.empty_like(q)
    argmax = torch.empty(wl.M, dtype=torch.int32, device=dev)
    P = 32
    path = torch.empty((wl.B, P), dtype=torch.int32, device=dev)
    plen = torch.empty(wl.B, dtype=torch.int32, device=dev)
    bonus = torch.empty(wl.B, dtype=torch.int32, device=dev)
    dt = tv.TV_BF16 if wl.dtype == "bf16" else tv.TV_F32
    need = (tv.tv_tree_verify_attn_paged_workspace(wl.B, wl.N, wl.Hq, wl.Hkv, wl.D, max_len, ps, dt)
            if ps else tv.tv_tree_verify_attn_workspace(wl.B, wl.N, wl.Hq, wl.Hkv, wl.D, max_len, dt))
    attn_ws = torch.zeros(max(256, need), dtype=torch.uint8, device=dev)
    lm_ws = torch.zeros(tv.tv_lmhead_argmax_workspace(wl.M, wl.hidden, wl.V, dt),
                        dtype=torch.uint8, device=dev)

    # Draft tokens of the simulated drafter: they copy the target's greedy
    # token at the parent (from one untimed LM-head call) with the workload's
    # probability, else a random token.
    tv.tv_lmhead_argmax(hid, w_step, argmax, workspace=lm_ws)
    draft = i32(draft_tokens(a["parent"], coins, argmax.cpu().numpy().reshape(wl.B, wl.N)))
    torch.cuda.synchronize()

    # Contiguous caches: acceptance and compaction run as one launch
    # (tv_accept_compact); paged caches use the two calls.
    fused_tail = not ps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
          for _ in range(args.steps)]

    def step(events=None):
        lens.copy_(lens0)   # compaction advanced the lengths; restore the batch
        if events:
            events[0].record()
        if ps:
            tv.tv_tree_verify_attn_paged(q, kc, vc, block_table, lens, parent, out,
                                         max_seq_len=max_len, scale=a["scale"], workspace=attn_ws)
        else:
            tv.tv_tree_verify_attn(q, kc, vc, lens, parent, out, max_seq_len=max_len,
                                   scale=a["scale"], workspace=attn_ws)
        if events:
            events[1].record()
        tv.tv_lmhead_argmax(hid, w_step, argmax, workspace=lm_ws)
        if events:
            events[2].record()
        if fused_tail:
            tv.tv_accept_compact(parent, draft, argmax, kc, vc, lens, P, path=path, path_len=plen,
                                 bonus=bonus)
            if events:
                events[3].record()
        else:
            tv.tv_tree_accept(parent, draft, argmax, P, path=path, path_len=plen, bonus=bonus)
            if events:
                events[3].record()
            if ps == 1:   # slot table: the commit permutes table entries, no row moves
                tv.tv_kv_commit_slots(block_table, lens, path, plen, wl.N)
            else:
                tv.tv_kv_compact_paged(kc, vc, block_table, lens, path, plen)
        if events:
            events[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Eager steps, each call bracketed by HIP events on the stream it is
    # launched on: the per-kernel breakdown and the LM head's own time.
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()

    # The value: the same step captured once as a HIP graph and replayed
    # (no host launch gaps between the four calls).
    gs = torch.cuda.Stream()
    gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    with torch.cuda.stream(gs):
        step()
        gs.synchronize()
        tv.tv_graph_begin(gs)
        step()
        graph = tv.tv_graph_end(gs)
        for _ in range(args.warmup):
            graph.launch(gs)
        gs.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            gev[i][0].record(gs)
            graph.launch(gs)
            gev[i][1].record(gs)
        gs.synchronize()
        t1 = time.perf_counter()
    graph_per = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in gev])

    # For reference only: the same LM head reading the row-major weight.
    rm_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    rm_reps = 20
    rm_ev[0].record()
    for _ in range(rm_reps):
        tv.tv_lmhead_argmax(hid, w, argmax, workspace=lm_ws)
    rm_ev[1].record()
    torch.cuda.synchronize()
    lm_rowmajor_us = rm_ev[0].elapsed_time(rm_ev[1]) * 1e3 / rm_reps

    # For comparison only: the same product through the vendor GEMM library
    # (logits written in bf16, no argmax), after the step's own timing.
    lib_us = None
    if args.library_gemm and wl.dtype == "bf16":
        wt = w.t()
        for _ in range(3):
            lib_out = torch.matmul(hid, wt)
        torch.cuda.synchronize()
        rm_ev[0].record()
        for _ in range(rm_reps):
            lib_out = torch.matmul(hid, wt)
        rm_ev[1].record()
        torch.cuda.synchronize()
        lib_us = rm_ev[0].elapsed_time(rm_ev[1]) * 1e3 / rm_reps
        del lib_out

    names = ["attn", "lmhead", "accept", "compact"]
    per = {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
           * 1e3 for j, n in enumerate(names)}
    if fused_tail:  # one launch between events 2 and 4
        per = {"attn": per["attn"], "lmhead": per["lmhead"],
               "accept_compact": per["accept"] + per["compact"]}
        names = ["attn", "lmhead", "accept_compact"]
    eager_us = float(np.mean([ev[i][0].elapsed_time(ev[i][4]) for i in range(args.steps)])) * 1e3
    step_us = float(np.median(graph_per))
    wall_ms = (t1 - t0) * 1e3 / args.steps
    value = wl.M * args.steps / (t1 - t0)

    path_h, plen_h = path.cpu().numpy(), plen.cpu().numpy()
    work = algorithmic_work(wl, a, path_h, plen_h, slots=ps == 1)
    kernels = {n: roof_entry(work[n][0], work[n][1], per[n], wl.dtype) for n in names}

    # Dominant kernel: the LM head (one kernel launch per call).
    lm_b, lm_f = work["lmhead"]
    lm_us = per["lmhead"]
    traffic = None
    if os.path.exists(COUNTERS):
        with open(COUNTERS) as f:
            cnt = json.load(f).get(f"lmhead_argmax/{wl.name}", {})
        if cnt.get("source_digest") == kernel_source_digest(LMHEAD_SOURCES):
            traffic = cnt.get("traffic_bytes")
    mfma_bound = lm_f / (BF16_DENSE_TFLOPS * 1e12) > lm_b / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        achieved = lm_f / (lm_us * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=BF16_DENSE_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / BF16_DENSE_TFLOPS, 4),
                    traffic=traffic)
    else:
        achieved = lm_b / (lm_us * 1e-6) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic)
    roof.update(kernel=lmhead_kernel_name(wl.M, wl.V, wl.dtype),
                algorithmic_bytes=lm_b, launch_us=round(lm_us, 2))

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "nodes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded generator, Qwen3-shaped layers, simulated drafter)",
        "config": {"workload": wl.name, "batch": wl.B, "nodes": wl.N,
                   "prefix": [int(x) for x in a["seq_lens"]], "Hq": wl.Hq, "Hkv": wl.Hkv,
                   "head_dim": wl.D, "hidden": wl.hidden, "vocab": wl.V,
                   "kv_layout": ("slots" if ps == 1 else f"paged{ps}") if ps else "contiguous",
                   "parallelism": "none (1 GPU)"},
        "step_us": round(step_us, 2),
        "step_us_p10_p90": [round(float(np.percentile(graph_per, 10)), 2),
                            round(float(np.percentile(graph_per, 90)), 2)],
        "eager_step_us": round(eager_us, 2),
        "mean_path_len": float(plen_h.mean()),
        "roofline": roof,
        "kernels": kernels,
        "lmhead_rowmajor_us": round(lm_rowmajor_us, 2),
    }
    if lib_us is not None:
        res["library_gemm_us"] = round(lib_us, 2)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, a, lm, coins)
    print(json.dumps(res), flush=True)


def model_work(cfg, wl, seq_lens) -> dict:
    """Algorithmic HBM bytes and flops of one multi-layer pass: every weight
    read once, the prefix K/V of every layer read once, the tree rows and the
    activations between kernels (bf16 in, fp32 partial sums excluded: they
    are an implementation choice)."""
    Hd, I, Ly = cfg.hidden, cfg.inter, cfg.layers
    qkv = (cfg.Hq + 2 * cfg.Hkv) * cfg.D
    M = wl.B * wl.N
    w_layer = 2 * (qkv * Hd + Hd * cfg.Hq * cfg.D + 2 * I * Hd + Hd * I) + 2 * (2 * Hd + 2 * cfg.D)
    weights = Ly * w_layer + 2 * cfg.V * Hd + 2 * Hd + 2 * M * Hd
    kv = Ly * (2 * int(np.sum(seq_lens)) * cfg.Hkv * cfg.D * 2 + 2 * M * cfg.Hkv * cfg.D * 2)
    flops = 2 * M * (Ly * (qkv * Hd + Hd * cfg.Hq * cfg.D + 3 * I * Hd) + cfg.V * Hd)
    return dict(bytes=int(weights + kv), weight_bytes=int(weights), kv_bytes=int(kv),
                flops=int(flops))


_LAYER_KEYS = ("ln1", "w_qkv", "q_norm", "k_norm", "w_o", "ln2", "w_gu", "w_down")


def model_cpu_baseline(cfg, wl, w):
    """The fp64 oracle's pass on a bounded sample: the pass with one and with
    two of the model's layers (the rest of the pass unchanged), timed, and
    scaled to all layers: t = t1 + (t2 - t1) * (layers - 1)."""
    import oracle
    from workloads import model_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    xs = model_inputs(cfg, wl, layers=2)
    t = {}
    for n in (1, 2):
        wn = {k: (v[:n] if k in _LAYER_KEYS else v) for k, v in w.items()}
        t0 = time.perf_counter()
        oracle.verify_pass(cfg.dims(layers=n), wn, xs["tokens"], xs["parent"], xs["seq_lens"],
                           xs["k_cache"][:n], xs["v_cache"][:n], logit_rows=[0])
        t[n] = time.perf_counter() - t0
    t_pass = t[1] + max(t[2] - t[1], 0.0) * (cfg.layers - 1)
    M = wl.B * wl.N
    return dict(value=round(M / t_pass, 4), unit="nodes/s", cores=int(cores), kind="oracle",
                sample=f"fp64 oracle pass over {wl.name} with 1 and 2 of {cfg.layers} layers "
                       f"({t[1] + t[2]:.1f} s), scaled to {cfg.layers} layers")


def model_bench(args):
    import torch

    import tree_draft_verification_amd as tv
    from workloads import (MODELS, WORKLOADS, draft_coins, draft_tokens, model_inputs,
                           model_weights)

    cfg = MODELS[args.model]
    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    t_setup = time.perf_counter()

    def progress(msg):
        print(f"[bench] {time.perf_counter() - t_setup:6.1f} s  {msg}", file=sys.stderr, flush=True)

    w = model_weights(cfg)
    x = model_inputs(cfg, wl)
    progress("synthetic weights and caches drawn")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    model = tv.tv_model_pack(cfg.dims(), {k: bf(v) for k, v in w.items()})
    torch.cuda.synchronize()
    progress("weights packed on the device")
    k0, v0 = bf(x["k_cache"]), bf(x["v_cache"])
    k, v = k0.clone(), v0.clone()
    lens0 = i32(x["seq_lens"])
    lens = lens0.clone()
    parent = i32(x["parent"])
    msl = int(x["seq_lens"].max())
    M, P = wl.B * wl.N, 32
    arg = torch.empty(M, dtype=torch.int32, device=dev)
    path = torch.empty((wl.B, P), dtype=torch.int32, device=dev)
    plen = torch.empty(wl.B, dtype=torch.int32, device=dev)
    bonus = torch.empty(wl.B, dtype=torch.int32, device=dev)
    ws = torch.zeros(tv.tv_verify_pass_workspace(model, wl.B, wl.N, msl), dtype=torch.uint8,
                     device=dev)
    cws = torch.zeros(tv.tv_kv_compact_layers_workspace(wl.B), dtype=torch.uint8, device=dev)
    # The simulated drafter copies the target's greedy token at the parent
    # with the workload's probability; the target's tokens come from passes
    # of this model, one tree level settled per pass (setup, untimed).
    coins = draft_coins(wl, x["depth"])
    tok_h = x["tokens"].copy()
    for _ in range(int(x["depth"].max()) + 1):
        tokens = i32(tok_h)
        tv.tv_verify_pass(model, tokens, parent, lens0, k, v, arg, max_seq_len=msl, workspace=ws)
        new = draft_tokens(x["parent"], coins, arg.cpu().numpy().reshape(wl.B, wl.N))
        if (new == tok_h).all():
            break
        tok_h = new
    tokens = i32(tok_h)
    progress("draft tokens settled")

    def step():
        lens.copy_(lens0)   # compaction advanced the lengths; restore the batch
        tv.tv_verify_pass(model, tokens, parent, lens, k, v, arg, max_seq_len=msl, workspace=ws)
        tv.tv_tree_accept(parent, tokens, arg, P, path=path, path_len=plen, bonus=bonus)
        tv.tv_kv_compact_layers(k, v, lens, path, plen, workspace=cws)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
        s.synchronize()
        # eager step time (the same calls, launched one by one)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(5):
            step()
        e1.record(s)
        s.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / 5
        tv.tv_graph_begin(s)
        step()
        graph = tv.tv_graph_end(s)
        for _ in range(args.warmup):
            graph.launch(s)
        s.synchronize()
    setup_s = time.perf_counter() - t_setup
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(s):
        for i in range(args.steps):
            ev[i][0].record(s)
            graph.launch(s)
            ev[i][1].record(s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in ev])
    step_us = float(np.median(per))
    value = M * args.steps / (t1 - t0)
    plen_h = plen.cpu().numpy()
    work = model_work(cfg, wl, x["seq_lens"])
    achieved = work["bytes"] / (step_us * 1e-6) / 1e9
    res = {
        "metric": "verified tree nodes/s, whole multi-layer verification step (graph replay)",
        "value": round(value, 1), "unit": "nodes/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded weights and caches, simulated drafter)",
        "config": {"workload": f"{cfg.name} x {wl.name}", "layers": cfg.layers,
                   "hidden": cfg.hidden, "inter": cfg.inter, "batch": wl.B, "nodes": wl.N,
                   "prefix": [int(t) for t in x["seq_lens"]], "parallelism": "none (1 GPU)"},
        "step_us": round(step_us, 2),
        "step_us_p10_p90": [round(float(np.percentile(per, 10)), 2),
                            round(float(np.percentile(per, 90)), 2)],
        "eager_step_us": round(eager_us, 2),
        "mean_path_len": float(plen_h.mean()),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "whole step (graph): weights + KV streamed once",
                     "algorithmic_bytes": work["bytes"], "launch_us": round(step_us, 2)},
        "work": work,
        "setup_s": round(setup_s, 1),
    }
    progress("timed")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = model_cpu_baseline(cfg, wl, w)
        progress("cpu baseline timed")
    print(json.dumps(res), flush=True)


def tree_bench(args):
    """Draft-tree construction from a path-conditioned draft head: the level
    calls (one per depth, each reading one row per frontier node) and the
    finish call.  A first, untimed pass drives the levels with the synthetic
    drafter and keeps each level's rows resident; the timed steps replay the
    level calls on them, so the drafter itself is not timed; the timed build
    is captured once as a HIP graph and replayed (device time of its
    kernels), with the eagerly launched build and the one-launch builder on
    one row per depth beside it."""
    import torch

    import tree_draft_verification_amd as tv
    from workloads import TREE_BUILDS, PathDrafter, draft_logp

    cfg = TREE_BUILDS[args.tree]
    B, D, W, V = cfg.B, cfg.depth, cfg.width, cfg.V
    dev = torch.device("cuda:0")
    drafter = PathDrafter(V, cfg.seed, scale=cfg.scale, quantum=cfg.quantum)
    roots_h = drafter.roots(B)
    root = torch.from_numpy(roots_h).to(dev)
    N = cfg.budget + 1
    par = torch.empty((B, N), dtype=torch.int32, device=dev)
    tok = torch.empty((B, N), dtype=torch.int32, device=dev)
    fsrc = torch.empty((B, W), dtype=torch.int32, device=dev)
    ftok = torch.empty((B, W), dtype=torch.int32, device=dev)
    ws = torch.zeros(tv.tv_tree_build_level_workspace(B, D, V, W), dtype=torch.uint8, device=dev)
    rows = []
    paths = [[(int(roots_h[b]),)] for b in range(B)]
    for level in range(1, D + 1):
        r_h = np.zeros((B, W, V), np.float32)
        for b in range(B):
            for r, pth in enumerate(paths[b]):
                r_h[b, r] = drafter.row(b, pth)
        rows.append(torch.from_numpy(r_h).to(dev))
        tv.tv_tree_build_level(rows[-1], level, D, frontier_src=fsrc, frontier_tok=ftok,
                               workspace=ws)
        fs, ft = fsrc.cpu().numpy(), ftok.cpu().numpy()
        paths = [[paths[b][int(fs[b, r])] + (int(ft[b, r]),) for r in range(W)] for b in range(B)]

    def build():
        for level in range(1, D + 1):
            tv.tv_tree_build_level(rows[level - 1], level, D, frontier_src=fsrc, frontier_tok=ftok,
                                   workspace=ws)
        tv.tv_tree_build_finish(root, D, V, W, cfg.budget, parent=par, tokens=tok, workspace=ws)

    for _ in range(args.warmup):
        build()
    torch.cuda.synchronize()
    # eager: every level call launched from the host (host-bound)
    eager_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    eager_ev[0].record()
    for i in range(args.steps):
        build()
    eager_ev[1].record()
    torch.cuda.synchronize()
    eager_us = eager_ev[0].elapsed_time(eager_ev[1]) * 1e3 / args.steps
    # the value: the whole build captured once as a HIP graph and replayed,
    # i.e. the device time of the level and finish kernels back to back
    gs = torch.cuda.Stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    with torch.cuda.stream(gs):
        build()
        gs.synchronize()
        tv.tv_graph_begin(gs)
        build()
        graph = tv.tv_graph_end(gs)
        for _ in range(args.warmup):
            graph.launch(gs)
        gs.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(gs)
            graph.launch(gs)
            ev[i][1].record(gs)
        gs.synchronize()
        t1 = time.perf_counter()
    per = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in ev])
    us = float(np.median(per))
    # rows read: one at level 1, W at every other level
    nbytes = B * (1 + (D - 1) * W) * V * 4 + B * N * 8
    achieved = nbytes / (us * 1e-6) / 1e9

    # the one-launch builder, one row per depth (a branch-agnostic draft head)
    x = draft_logp(cfg)
    lp = torch.from_numpy(x["logp"]).to(dev)
    root1 = torch.from_numpy(x["root_tokens"]).to(dev)
    ws1 = torch.zeros(tv.tv_tree_build_workspace(B, D, V, W), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        tv.tv_tree_build(lp, root1, W, cfg.budget, parent=par, tokens=tok, workspace=ws1)
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev1[0].record()
    for _ in range(args.steps):
        tv.tv_tree_build(lp, root1, W, cfg.budget, parent=par, tokens=tok, workspace=ws1)
    ev1[1].record()
    torch.cuda.synchronize()
    depth_rows_us = ev1[0].elapsed_time(ev1[1]) * 1e3 / args.steps

    res = {
        "metric": "draft trees built/s (branch-conditioned accum_logp: tv_tree_build_level x depth "
                  "+ tv_tree_build_finish)",
        "value": round(B * args.steps / (t1 - t0), 1), "unit": "trees/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 (scores summed in f64)",
        "data": "synthetic (seeded path-conditioned draft log-probabilities, recorded per level)",
        "config": {"workload": cfg.name, "batch": B, "depth": D, "width": W,
                   "budget": cfg.budget, "vocab": V},
        "step_us": round(us, 2),
        "step_us_p10_p90": [round(float(np.percentile(per, 10)), 2),
                            round(float(np.percentile(per, 90)), 2)],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "whole build (top-k and level kernels per depth, finish kernel)",
                     "algorithmic_bytes": nbytes, "launch_us": round(us, 2)},
        "depth_rows_us": round(depth_rows_us, 2),
        "eager_us": round(eager_us, 2),
    }
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        reps = 0
        while reps < 20 and (reps == 0 or time.perf_counter() - t0 < 20.0):
            oracle.accum_logp_tree_paths(drafter.row, roots_h, D, W, cfg.budget)
            reps += 1
        spent = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            cores = 1
        res["cpu_baseline"] = dict(value=round(B * reps / spent, 3), unit="trees/s",
                                   cores=int(cores), kind="oracle",
                                   sample=f"{reps} full build(s) of {cfg.name} ({spent:.1f} s; "
                                          "draft rows cached)")
    print(json.dumps(res), flush=True)


def compact_stack_bench(args):
    """One tv_kv_compact_layers launch over many stacked layers."""
    import torch

    import tree_draft_verification_amd as tv
    from workloads import WORKLOADS, attn_inputs

    t_setup = time.perf_counter()

    def progress(msg):
        print(f"[bench] {time.perf_counter() - t_setup:6.1f} s  {msg}", file=sys.stderr, flush=True)

    wl = WORKLOADS["qwen3_8b_ragged8_N64"]
    layers = args.compact_stack
    a = attn_inputs(wl.replace(Hq=wl.Hkv, D=8))  # trees and prefix lengths only
    par, depth, lens_h = a["parent"], a["depth"], a["seq_lens"]
    B, Hkv, D, Lcap, P = wl.B, wl.Hkv, wl.D, wl.Lcap, 32
    path_h = np.full((B, P), -1, dtype=np.int32)
    plen_h = np.zeros(B, dtype=np.int32)
    pd, pw = args.compact_path_depth, 7
    if pd > 0:
        # accepted paths through level-ordered trees of depth pd and width
        # pw (the shape the level-by-level builder makes, node 0 then pw
        # nodes per level): node j of the path is drawn from level j
        if 1 + pd * pw > Lcap - int(lens_h.max()) or pd + 1 > P:
            raise SystemExit("bench.py: --compact-path-depth does not fit the caches")
        rng = np.random.default_rng(wl.seed + 7)
        for b in range(B):
            chain = [0] + [1 + (j - 1) * pw + int(rng.integers(pw)) for j in range(1, pd + 1)]
            path_h[b, :len(chain)] = chain
            plen_h[b] = len(chain)
        tree_rows = 1 + pd * pw
    else:
        for b in range(B):
            node = int(np.argmax(depth[b]))         # deepest node, smallest index
            chain = []
            while node >= 0:
                chain.append(node)
                node = int(par[b, node])
            chain.reverse()
            path_h[b, :len(chain)] = chain
            plen_h[b] = len(chain)
        tree_rows = wl.N
    moved = int(sum((path_h[b, :plen_h[b]] != np.arange(plen_h[b])).sum() for b in range(B)))
    e = 2
    nbytes = 4 * moved * Hkv * D * e * layers + 8 * B
    dev = torch.device("cuda:0")
    plane = (layers, B, Hkv, Lcap, D)
    progress(f"stacked caches: {layers} layers, "
             f"{2 * np.prod(plane) * e / 2**30:.1f} GiB")
    k = torch.empty(plane, dtype=torch.int16, device=dev)
    v = torch.empty(plane, dtype=torch.int16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)
    for b in range(B):   # only the tree rows are read; fill them with seeded bits
        L = int(lens_h[b])
        for c in (k, v):
            c[:, b, :, L:L + tree_rows].random_(-32768, 32767, generator=g)
    lens0 = torch.from_numpy(lens_h.astype(np.int32)).to(dev)
    lens = lens0.clone()
    path = torch.from_numpy(path_h).to(dev)
    plen = torch.from_numpy(plen_h).to(dev)
    ws = torch.zeros(tv.tv_kv_compact_layers_workspace(B), dtype=torch.uint8, device=dev)
    # Cold caches: a 1 GiB read before each launch evicts L2 and the 256 MB
    # infinity cache.  A read leaves no dirty lines behind; a write-based
    # flush would leave write-backs that compete with the timed kernel.
    flush = torch.zeros(1 << 27, dtype=torch.int64, device=dev)
    flush_out = torch.zeros((), dtype=torch.int64, device=dev)

    def evict():
        torch.sum(flush, dim=0, out=flush_out)

    kb, vb = k.view(torch.bfloat16), v.view(torch.bfloat16)

    # one launch checked against the moves done by indexing (bits)
    src = [torch.from_numpy(int(lens_h[b]) + path_h[b, :plen_h[b]].astype(np.int64)).to(dev)
           for b in range(B)]
    want_k = [k[:, b, :, src[b]].clone() for b in range(B)]
    want_v = [v[:, b, :, src[b]].clone() for b in range(B)]
    tv.tv_kv_compact_layers(kb, vb, lens, path, plen, workspace=ws)
    torch.cuda.synchronize()
    for b in range(B):
        L, n = int(lens_h[b]), int(plen_h[b])
        if not (torch.equal(k[:, b, :, L:L + n], want_k[b])
                and torch.equal(v[:, b, :, L:L + n], want_v[b])):
            raise SystemExit(f"bench.py: stacked compaction moved the wrong rows (sequence {b})")
    if not torch.equal(lens.cpu(), lens0.cpu() + plen.cpu()):
        raise SystemExit("bench.py: stacked compaction left wrong lengths")
    del want_k, want_v
    progress("stacked compaction checked")

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.warmup + args.steps):
        lens.copy_(lens0)
        evict()
        if i >= args.warmup:
            ev[i - args.warmup][0].record()
        tv.tv_kv_compact_layers(kb, vb, lens, path, plen, workspace=ws)
        if i >= args.warmup:
            ev[i - args.warmup][1].record()
    torch.cuda.synchronize()
    per = np.array([x[0].elapsed_time(x[1]) * 1e3 for x in ev])
    us = float(np.median(per))
    achieved = nbytes / (us * 1e-6) / 1e9
    # context: a plain device copy with the same bytes read and written,
    # timed the same way (cold, between events)
    half = nbytes // 2
    src_c = torch.empty(half, dtype=torch.uint8, device=dev)
    dst_c = torch.empty_like(src_c)
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.warmup + args.steps):
        evict()
        if i >= args.warmup:
            evc[i - args.warmup][0].record()
        dst_c.copy_(src_c)
        if i >= args.warmup:
            evc[i - args.warmup][1].record()
    torch.cuda.synchronize()
    copy_us = float(np.median([x[0].elapsed_time(x[1]) * 1e3 for x in evc]))
    workload = (f"{wl.name} geometry, {layers} stacked layers"
                + (f", depth-{pd} width-{pw} paths" if pd > 0 else ""))
    traffic = None
    if os.path.exists(COUNTERS):
        with open(COUNTERS) as f:
            cnt = json.load(f).get(f"compact_kernel_layered/{workload}", {})
        if cnt.get("source_digest") == kernel_source_digest(COMPACT_SOURCES):
            traffic = cnt.get("traffic_bytes")
    res = {
        "metric": "KV compaction bandwidth (tv_kv_compact_layers, one launch over stacked layers)",
        "value": round(achieved, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (bits)",
        "data": "synthetic (seeded trees and cache bits; cold caches)",
        "config": {"workload": workload,
                   "batch": B, "kv_heads": Hkv, "head_dim": D, "Lcap": Lcap,
                   "layers": layers, "moved_rows_per_layer": moved,
                   "path_lens": [int(x) for x in plen_h]},
        "step_us": round(us, 2),
        "step_us_p10_p90": [round(float(np.percentile(per, 10)), 2),
                            round(float(np.percentile(per, 90)), 2)],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "compact_kernel<false, false> (layered)",
                     "algorithmic_bytes": nbytes, "launch_us": round(us, 2)},
        "plain_copy_same_bytes": {"us": round(copy_us, 2),
                                  "gbs": round(nbytes / (copy_us * 1e-6) / 1e9, 1)},
    }
    print(json.dumps(res), flush=True)


def decode_bench(args):
    """Multi-step ragged speculative decoding at full size.  The simulated
    drafter knows the target's greedy continuation from the current state
    (one-token passes on a scratch copy of the caches); a tree node whose path
    follows it favours the next greedy token with probability 0.9.  Trees are
    built level by level (tv_tree_build_level, tv_tree_build_finish); the
    drafter and the host bookkeeping between levels and steps are not timed."""
    import torch

    import tree_draft_verification_amd as tv
    from workloads import MODELS, WORKLOADS, model_inputs, model_weights

    cfg = MODELS[args.model]
    wl = WORKLOADS[args.workload]
    steps, depth, width, budget = args.decode, args.tree_depth, args.tree_width, args.tree_budget
    N = budget + 1
    room = N + steps * (depth + 1)
    dev = torch.device("cuda:0")
    t_setup = time.perf_counter()

    def progress(msg):
        print(f"[bench] {time.perf_counter() - t_setup:6.1f} s  {msg}", file=sys.stderr, flush=True)

    w = model_weights(cfg)
    x = model_inputs(cfg, wl.replace(N=room))
    progress("synthetic weights and caches drawn")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    model = tv.tv_model_pack(cfg.dims(), {k: bf(v) for k, v in w.items()})
    del w
    k0, v0 = bf(x["k_cache"]), bf(x["v_cache"])
    del x["k_cache"], x["v_cache"]
    B, V = wl.B, cfg.V
    L0 = x["seq_lens"].copy()
    root0 = x["tokens"][:, 0].copy()
    Lcap = k0.shape[3]
    progress("weights packed, caches resident")

    k, v = k0.clone(), v0.clone()
    ks, vs = torch.empty_like(k0), torch.empty_like(v0)   # scratch of the simulated drafter
    lens = i32(L0)
    root = i32(root0)
    P = 32
    chain = torch.full((B, 1), -1, dtype=torch.int32, device=dev)
    ref = torch.empty((B, depth), dtype=torch.int32, device=dev)
    par = torch.empty((B, N), dtype=torch.int32, device=dev)
    tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    arg = torch.empty(B * N, dtype=torch.int32, device=dev)
    path = torch.empty((B, P), dtype=torch.int32, device=dev)
    plen = torch.empty(B, dtype=torch.int32, device=dev)
    bonus = torch.empty(B, dtype=torch.int32, device=dev)
    tb_ws = torch.zeros(tv.tv_tree_build_level_workspace(B, depth, V, width), dtype=torch.uint8,
                        device=dev)
    fsrc = torch.empty((B, width), dtype=torch.int32, device=dev)
    ftok = torch.empty((B, width), dtype=torch.int32, device=dev)
    lv_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    level_us = []
    pass_ws = torch.zeros(tv.tv_verify_pass_workspace(model, B, N, Lcap - N), dtype=torch.uint8,
                          device=dev)
    ar_ws = torch.zeros(tv.tv_verify_pass_workspace(model, B, 1, Lcap - 1), dtype=torch.uint8,
                        device=dev)
    cl_ws = torch.zeros(tv.tv_kv_compact_layers_workspace(B), dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    rng = np.random.default_rng(wl.seed)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    emitted = np.zeros(B, dtype=np.int64)
    plens = []
    cur = L0.copy()
    for s in range(steps):
        # simulated drafter (untimed): the target's greedy continuation from
        # the current state, by one-token passes on a scratch copy of the
        # caches; each depth favours that token with probability 0.9
        ks.copy_(k)
        vs.copy_(v)
        sl = lens.clone()
        t1 = root.reshape(B, 1).clone()
        for d in range(depth):
            a1 = tv.tv_verify_pass(model, t1, chain, sl, ks, vs, max_seq_len=int(cur.max()) + d,
                                   workspace=ar_ws)
            ref[:, d] = a1
            t1 = a1.reshape(B, 1).clone()
            sl += 1
        ref_h = ref.cpu().numpy()
        root_h = root.cpu().numpy()
        # the branch-conditioned tree, level by level: a frontier node whose
        # drafted tokens follow the greedy continuation favours the next one
        # with probability 0.9, any other node a token of its own; only the
        # level calls and the finish are timed
        paths = [[(int(root_h[b]),)] for b in range(B)]
        tb_us = 0.0
        for level in range(1, depth + 1):
            logits = torch.randn((B, width, V), generator=gen, device=dev)
            for b in range(B):
                for r, pth in enumerate(paths[b]):
                    d = len(pth) - 1
                    on_ref = list(pth[1:]) == [int(t) for t in ref_h[b, :d]]
                    t_ = (int(ref_h[b, d]) if on_ref and d < depth and rng.random() < 0.9
                          else int(rng.integers(V)))
                    logits[b, r, t_] += 12.0
            logp = torch.log_softmax(logits, dim=-1).contiguous()
            lv_ev[0].record()
            tv.tv_tree_build_level(logp, level, depth, frontier_src=fsrc, frontier_tok=ftok,
                                   workspace=tb_ws)
            lv_ev[1].record()
            fs, ft = fsrc.cpu().numpy(), ftok.cpu().numpy()
            tb_us += lv_ev[0].elapsed_time(lv_ev[1]) * 1e3
            paths = [[paths[b][int(fs[b, r])] + (int(ft[b, r]),) for r in range(width)]
                     for b in range(B)]
        torch.cuda.synchronize()
        ev[s][0].record()
        tv.tv_tree_build_finish(root, depth, V, width, budget, parent=par, tokens=tokens,
                                workspace=tb_ws)
        ev[s][1].record()
        tv.tv_verify_pass(model, tokens, par, lens, k, v, arg, max_seq_len=int(cur.max()),
                          workspace=pass_ws)
        ev[s][2].record()
        tv.tv_tree_accept(par, tokens, arg, P, path=path, path_len=plen, bonus=bonus)
        ev[s][3].record()
        tv.tv_kv_compact_layers(k, v, lens, path, plen, workspace=cl_ws)
        ev[s][4].record()
        root = bonus.clone()
        level_us.append(tb_us)
        plen_h = plen.cpu().numpy()
        plens.append(plen_h.tolist())
        emitted += plen_h
        cur = lens.cpu().numpy()
        progress(f"step {s}: path lengths {plen_h.tolist()}")
        if int(cur.max()) + N > Lcap:
            break
    torch.cuda.synchronize()
    done = len(plens)
    parts = np.array([[ev[s][j].elapsed_time(ev[s][j + 1]) * 1e3 for j in range(4)]
                      for s in range(done)])
    parts[:, 0] += np.array(level_us[:done])     # the level calls of each tree
    dev_s = parts.sum() * 1e-6
    res = {
        "metric": "generated tokens/s, multi-step ragged speculative decoding (device time)",
        "value": round(float(emitted.sum()) / dev_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": done, "warmup": 0, "ms_per_step": round(parts.sum(axis=1).mean() / 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded weights and caches, path-conditioned drafter favouring the "
                "greedy continuation)",
        "config": {"workload": f"{cfg.name} x {wl.name}", "batch": B,
                   "prefix": [int(t) for t in L0], "tree_depth": depth, "tree_width": width,
                   "tree_budget": budget, "parallelism": "none (1 GPU)"},
        "tokens_per_step": round(float(emitted.sum()) / done, 2),
        "mean_path_len": round(float(np.mean(plens)), 2),
        "step_us_breakdown": {"tree_build": round(float(parts[:, 0].mean()), 1),
                              "verify_pass": round(float(parts[:, 1].mean()), 1),
                              "accept": round(float(parts[:, 2].mean()), 1),
                              "compact_layers": round(float(parts[:, 3].mean()), 1)},
        "path_lens": plens,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
