"""Throughput of the DFlash2 draft-block head on one MI355X.

A step is one pass of the whole draft-head path over one batch of synthetic
input, inputs resident in HBM:
  walk workloads:  conv prepare + conv finish (one wrapped sublayer),
                   unary LM-head top-K, context projection + greedy walk;
  packed TF:       the same conv, unary top-K with gold logits, context
                   projection + teacher-forced scores and K-way CE.
The teacher-forced scorer is also timed on walk workloads (field "tf_ms").

Prints ONE JSON line (rank 0):  value = anchor blocks per second.
The roofline object covers the dominant op (LM head + top-K): algorithmic
bytes (or FLOPs) per launch over its average duration from HIP events on the
launch stream inside the timed region.  cpu_baseline is the CPU oracle timed
on a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DFlash2 draft-head blocks/s + % of HBM/MFMA roofline, Qwen3-8B shape"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
LMHEAD_SOURCES = ["lmhead.hip", "gemm.hpp", "common.hpp"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_1x8_h4096_v151936")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--selector", choices=("greedy", "sample"), default="greedy",
                    help="walk workloads: greedy walk, or the path sampled from softmax of the same scores "
                         "(temperature 1, a fixed generator key)")
    ap.add_argument("--train", action="store_true",
                    help="teacher-forced workloads: the step also runs the selector CE backward")
    ap.add_argument("--metrics", action="store_true",
                    help="the LM head also forms the full-vocabulary log-sum-exp and, on teacher-forced "
                         "workloads, the gold's probability and top-K hit (recall@K, target mass, coverage)")
    ap.add_argument("--output-multiplier", type=float, default=1.0)
    ap.add_argument("--softcap", type=float, default=0.0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    return ap.parse_args()


def lmhead_source_hash() -> str:
    h = hashlib.sha256()
    for f in LMHEAD_SOURCES:
        with open(os.path.join(ROOT, "block_draft_head_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def lmhead_work(w):
    """Algorithmic bytes and FLOPs of one LM-head + top-K launch: the weights
    stream once, activations are read once, ids and values are written once;
    logits never leave the chip."""
    es = 4 if w.dtype == "f32" else 2
    N = w.n_rows
    bytes_ = w.vocab * w.hidden * es + N * w.hidden * es + N * w.top_k * 8
    flops = 2.0 * N * w.vocab * w.hidden
    return bytes_, flops


def traffic_for(w, launches_key):
    """HBM bytes per launch from committed rocprofv3 counters, or None when
    they are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    e = t.get(launches_key)
    if not e or e.get("source_hash") != lmhead_source_hash():
        return None
    return e["fetch_kib"] * 1024.0 * e["fetch_scale"] + e["write_kib"] * 1024.0 * e["write_scale"]


def backward_report(w, ms):
    """Selector CE backward (context projection, per-row kernel, dW_H
    contraction): its algorithmic bytes and flops over its measured time.
    Bytes: h twice (projection and dW_H), W_H, g and dg written and read, the
    predecessor and K successor rows gathered, ids / logits / per-row scalars,
    and a read-modify-write of every touched float32 gradient row and of dW_H.
    Flops: the two N x r x H contractions (the per-row work is O(N K r))."""
    N, H, r, K = w.n_rows, w.hidden, w.rank, w.top_k
    es = 2 if w.dtype == "bf16" else 4
    nbytes = (2 * N * H * es + r * H * es + 4 * N * r * 4 + N * r * es + N * K * r * es + N * K * 8 + N * 17
              + 2 * (N * r + N * K * r) * 4 + 2 * r * H * 4)
    flops = 2 * (2 * N * r * H)
    s = ms * 1e-3
    return {"ms": ms, "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "hbm_frac": nbytes / s / (HBM_PEAK_GBS * 1e9), "gbs": nbytes / s / 1e9, "tflops": flops / s / 1e12}


def cpu_baseline(w, inp, budget_s):
    """The oracle as it stands, on the host: whole steps of the same workload
    on a bounded sample of anchor blocks (all blocks when they fit)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import dflash2_oracle as O

    bs = w.block_size
    blocks = 1
    t_all = 0.0
    reps = 0
    rows = slice(0, blocks * bs)
    while True:
        t0 = time.perf_counter()
        h = inp["h"][rows]
        xo, kp, _ = O.conv_prepare(h, inp["w_proj"], inp["base"], bs, w.taps, w.group_size, w.dtype)
        O.conv_finish(inp["y"][rows], kp, inp["base"], bs, w.taps, w.group_size, w.dtype)
        ids, vals, gl = O.unary_topk(h, inp["w_lm"], w.top_k, w.dtype,
                                     gold_ids=inp["gold"][rows] if w.mode == "tf" else None)
        g = O.context_projection(h, inp["w_h"], w.dtype)
        if w.mode == "tf":
            O.selector_score_tf(g, inp["cb_pred"], inp["cb_succ"], ids, vals, inp["pred"][rows], w.dtype,
                                gold_ids=inp["gold"][rows], force=inp["force"][rows], gold_logit=gl)
        else:
            O.selector_walk(g, inp["cb_pred"], inp["cb_succ"], ids, vals, inp["anchors"][:blocks], bs, w.dtype)
        t_all += time.perf_counter() - t0
        reps += 1
        if t_all >= budget_s or reps >= 50:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": reps * blocks / t_all, "unit": "blocks/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{reps} whole oracle step(s) on {blocks} anchor block(s) of {w.name} "
                  f"(float64 numpy, {t_all:.1f} s); host has {os.cpu_count()} CPUs",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no "
              f"multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_draft_head_amd import dflash2 as D
    from block_draft_head_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    inp = make_inputs(w)
    dev = {}
    for k, a in inp.items():
        if a.dtype == np.uint16:
            dev[k] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        else:
            dev[k] = torch.from_numpy(a).cuda()
    torch.cuda.synchronize()
    print("[bench] inputs resident on the GPU", file=sys.stderr, flush=True)

    bs, T, gs, K, r = w.block_size, w.taps, w.group_size, w.top_k, w.rank
    N, H, V = w.n_rows, w.hidden, w.vocab
    ws_topk = D.make_workspace(D.OP_UNARY_TOPK, N, H, V, 0, K, "cuda")
    ws_sel = D.make_workspace(D.OP_SELECTOR_WALK if w.mode != "tf" else D.OP_SELECTOR_TF, N, H, V, r, K, "cuda")
    ws_tf = D.make_workspace(D.OP_SELECTOR_TF, N, H, V, r, K, "cuda")
    tf_mode = w.mode == "tf"
    if args.train and not tf_mode:
        print("--train needs a teacher-forced workload", file=sys.stderr)
        sys.exit(2)
    if tf_mode:  # selector CE backward: gradient buffers accumulate across steps (no zeroing in the step)
        ws_bwd = D.make_workspace(D.OP_SELECTOR_CE_BACKWARD, N, H, V, r, K, "cuda")
        grads = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in ((V, r), (V, r), (r, H))]
        grad_ce = torch.full((N,), 1.0 / N, dtype=torch.float32, device="cuda")
    x_out = torch.empty_like(dev["h"])
    k_post = torch.empty((N, T, H // gs), dtype=torch.float32, device="cuda")
    y_out = torch.empty_like(dev["y"])
    gold = dev["gold"] if tf_mode else None

    def op_conv():
        D.conv_prepare(dev["h"], dev["w_proj"], dev["base"], bs, T, gs, out=x_out, k_post=k_post)
        D.conv_finish(dev["y"], k_post, dev["base"], bs, T, gs, out=y_out)

    transformed = args.metrics or args.output_multiplier != 1.0 or args.softcap != 0.0
    metrics_out = {}

    def op_lmhead():
        if not transformed:
            return D.unary_topk(dev["h"], dev["w_lm"], K, gold_ids=gold, workspace=ws_topk)
        ids, vals, gl, lse, prob, hit = D.unary_topk_ex(dev["h"], dev["w_lm"], K, gold_ids=gold,
                                                        output_multiplier=args.output_multiplier,
                                                        softcap=args.softcap, want_lse=args.metrics,
                                                        want_metrics=args.metrics, workspace=ws_topk)
        metrics_out.update(lse=lse, prob=prob, hit=hit)
        return ids, vals, gl

    def op_selector(ids, vals, gl):
        if tf_mode:
            return D.selector_score_tf(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals, dev["pred"],
                                       gold_ids=gold, force=dev["force"], gold_logit=gl, workspace=ws_sel)
        if args.selector == "sample":
            return D.selector_sample(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals,
                                     dev["anchors"], bs, temperature=1.0, seed=0x5EED, workspace=ws_sel)
        return D.selector_walk(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals, dev["anchors"],
                               bs, workspace=ws_sel)

    def op_backward(ids, vals, gl):
        return D.selector_ce_backward(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals, dev["pred"],
                                      gold, grad_ce, force=dev["force"], gold_logit=gl, grad_pred=grads[0],
                                      grad_succ=grads[1], grad_wh=grads[2], want_ce=False, workspace=ws_bwd)

    def step():
        op_conv()
        ids, vals, gl = op_lmhead()
        res = op_selector(ids, vals, gl)
        if args.train:
            op_backward(ids, vals, gl)
        return ids, vals, gl, res

    def timed(fn, n):
        """Device time of n back-to-back calls of `fn`, from events recorded on
        the launch stream (torch's current stream) at the two ends."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            out = fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n, out

    for _ in range(args.warmup):
        ids, vals, gl, res = step()
    torch.cuda.synchronize()

    # teacher-forced scoring of the walk's own path (walk workloads): the same
    # predecessors every step, so it can ride along in the attribution pass
    pred = None
    if not tf_mode:
        path = res[0]
        pred = torch.empty(N, dtype=torch.int32, device="cuda")
        pred.view(w.n_blocks, bs)[:, 1:] = path[:, :-1]
        pred.view(w.n_blocks, bs)[:, 0] = dev["anchors"]

    def op_tf(ids, vals):
        return D.selector_score_tf(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals, pred,
                                   workspace=ws_tf)

    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)

    # headline: whole steps, events only at the two ends of the timed region
    t0 = time.perf_counter()
    ms_per_step, (ids, vals, gl, res) = timed(step, args.steps)
    wall = time.perf_counter() - t0
    gpu_ms = ms_per_step * args.steps

    # attribution pass: the same steps with events between the ops.  The host
    # enqueues far faster than the GPU drains a step (the LM head alone is
    # hundreds of microseconds), so each op's events bracket its kernels as
    # the GPU runs them back to back; the LM-head figure feeds the roofline.
    names = ["conv", "lmhead", "selector"] + (["ce_backward"] if tf_mode else ["tf"])
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for e in evs:
        e[0].record()
        op_conv()
        e[1].record()
        i_, v_, g_ = op_lmhead()
        e[2].record()
        op_selector(i_, v_, g_)
        e[3].record()
        if not tf_mode:
            op_tf(i_, v_)
        else:
            op_backward(i_, v_, g_)
        e[4].record()
    torch.cuda.synchronize()
    op_ms = {k: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, k in enumerate(names)}
    tf_ms = op_ms.pop("tf", None)
    bwd_ms = op_ms.pop("ce_backward", None)
    if args.train:
        op_ms["ce_backward"] = bwd_ms
    replay_ok = None
    if not tf_mode and args.selector == "greedy":  # a sampled path is not the scores' argmax
        _, best, _, _ = op_tf(ids, vals)
        replay_ok = bool(torch.equal(best.view(w.n_blocks, bs)[:, 1:], res[0][:, 1:]))

    # achievable HBM rate on this device: a 1 GiB device-to-device copy (read
    # plus write bytes over its event time, best of 5), beside the 8 TB/s peak
    cs = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cd = torch.empty_like(cs)
    cd.copy_(cs)
    copy_ms = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        cd.copy_(cs)
        b.record()
        torch.cuda.synchronize()
        copy_ms.append(a.elapsed_time(b))
    copy_gbs = 2.0 * (1 << 30) / (min(copy_ms) * 1e-3) / 1e9
    del cs, cd

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    metrics = None
    if args.metrics:
        metrics = {"mean_log_sum_exp": float(metrics_out["lse"].mean())}
        if metrics_out.get("hit") is not None:
            hit = metrics_out["hit"].float()
            metrics.update({"recall_at_k": float(hit.mean()), "coverage": float(hit.mean()),
                            "target_mass": float(metrics_out["prob"].mean())})

    lm_bytes, lm_flops = lmhead_work(w)
    lm_ms = op_ms["lmhead"]
    mfma_bound = lm_flops / lm_bytes > (BF16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9) and w.dtype == "bf16"
    if mfma_bound:
        achieved = lm_flops / (lm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        achieved = lm_bytes / (lm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_for(w, w.name)
    roof["kernel"] = ("lmhead_dma_kernel + top-K merge" if N <= 8 and w.dtype == "bf16" else
                      "lmhead_stream_kernel + top-K merge" if N <= 8 else
                      "lmhead_big_kernel + top-K merge" if w.dtype == "bf16" else
                      "lmhead_tiled_kernel + top-K merge")
    roof["algorithmic_bytes"] = lm_bytes
    roof["avg_ms"] = lm_ms

    out = {
        "metric": METRIC,
        "value": w.n_blocks * args.steps / (gpu_ms * 1e-3),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "n_blocks": w.n_blocks, "block_size": bs, "hidden": H, "vocab": V,
                   "taps": T, "group_size": gs, "rank": r, "top_k": K, "mode": w.mode,
                   "selector": ("teacher-forced + CE backward" if args.train else "teacher-forced") if tf_mode
                   else args.selector,
                   "unary": {"output_multiplier": args.output_multiplier, "softcap": args.softcap,
                             "metrics": args.metrics}},
        "roofline": roof,
        "ops_ms": op_ms,
        "selector_plus_conv_over_lmhead": (op_ms["conv"] + op_ms["selector"]) / lm_ms,
        "tf_ms": tf_ms,
        "unary_metrics": metrics,
        "ce_backward": backward_report(w, bwd_ms) if tf_mode else None,
        "tf_replays_walk": replay_ok,
        "wall_s_timed": wall,
        "copy_gbs": copy_gbs,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
