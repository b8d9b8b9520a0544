"""Throughput of the DFlash2 draft-block head on one MI355X.

A step is one pass of the whole draft-head path over one batch of synthetic
input, inputs resident in HBM:
  walk workloads:  conv prepare + conv finish (one wrapped sublayer), the unary
                   LM-head top-K and the greedy walk (at most 8 rows, bf16:
                   dflash2_decode_head, whose LM-head kernel also streams the
                   context projection's rows; else the unary top-K whose
                   call also forms the context rows, W_H tiles on the
                   many-row kernel's stream (`--context-rows selector`: the
                   selector call forms them), then the walk);
  packed TF:       the same conv, unary top-K with gold logits and the
                   context rows, teacher-forced scores and K-way CE.
The context rows' share of the LM-head op is reported beside it
(`context_rows_ms`: the op with W_H minus the same op without).

Timing.  Every timed step is preceded, outside its events, by a 512 MiB write
that evicts the 256 MiB MALL, so small weights (the conv projection, the
context projection, codebook rows) come from HBM as they would after the rest
of a draft-verify cycle.  A step's time is the median over steps of HIP events
recorded on the launch stream (torch's current stream) around it.  The share
of each op is measured by difference, not by events between the ops (an event
record costs ~4 us of GPU time, more than the small ops themselves): the full
step, the step without the conv and the step without the selector are timed in
interleaved rounds, and conv = full - no_conv, selector = full - no_selector,
LM head = full - conv - selector.

Prints ONE JSON line: value = anchor blocks per second of the headline
workload; `workloads` carries the other configurations; the roofline object
covers the dominant op (LM head + top-K) timed back to back; cpu_baseline is
the CPU oracle timed on a bounded sample of the same workload on this host
(float64 sums, and beside it the same code with float32 sums).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DFlash2 draft-head blocks/s + % of HBM/MFMA roofline, Qwen3-8B shape"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
LMHEAD_SOURCES = ["lmhead.hip", "gemm.hpp", "common.hpp", "selector.hpp"]
FLUSH_MIB = 512              # > the 256 MiB MALL
TARGETS = {  # fractions of the op's roofline the workloads aim at
    "decode_1x8_h4096_v151936": 0.70, "packed_tf_512x8_h4096_v151936": 0.50}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_1x8_h4096_v151936")
    ap.add_argument("--attr-steps", type=int, default=0,
                    help="steps per variant in the attribution (default 200 for at most 8 rows, else 30)")
    ap.add_argument("--no-workloads", action="store_true", help="skip the other configurations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--selector", choices=("greedy", "sample"), default="greedy",
                    help="walk workloads: greedy walk, or the path sampled from softmax of the same scores "
                         "(temperature 1, a fixed generator key)")
    ap.add_argument("--train", action="store_true",
                    help="teacher-forced workloads: the step also runs the selector CE backward")
    ap.add_argument("--metrics", action="store_true",
                    help="the LM head also forms the full-vocabulary log-sum-exp and, on teacher-forced "
                         "workloads, the gold's probability and top-K hit (recall@K, target mass, coverage)")
    ap.add_argument("--context-rows", choices=("lmhead", "selector"), default="lmhead",
                    help="where the selector's context rows h W_H^T are formed outside the decode head: in the "
                         "LM head's call (W_H tiles on its weight stream), or by the selector call itself")
    ap.add_argument("--output-multiplier", type=float, default=1.0)
    ap.add_argument("--softcap", type=float, default=0.0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of each CPU-oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def lmhead_source_hash() -> str:
    h = hashlib.sha256()
    for f in LMHEAD_SOURCES:
        with open(os.path.join(ROOT, "block_draft_head_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def lmhead_work(w, ctx=False):
    """Algorithmic bytes and FLOPs of one LM-head + top-K op: the weights
    stream once, activations are read once, ids and values are written once;
    logits never leave the chip.  With ctx the op also forms the context rows
    h W_H^T: W_H streams once more and g [N, r] float32 is written."""
    es = 4 if w.dtype == "f32" else 2
    N = w.n_rows
    rows = w.vocab + (w.rank if ctx else 0)
    bytes_ = rows * w.hidden * es + N * w.hidden * es + N * w.top_k * 8 + (N * w.rank * 4 if ctx else 0)
    flops = 2.0 * N * rows * w.hidden
    return bytes_, flops


def small_op_floors(w, ops, launch_floor_us, path):
    """Conv and selector against their floors at decode size: each launch
    costs at least the measured back-to-back launch floor, and each byte
    moves at the HBM peak.  The conv wrapper is two launches (prepare before
    the sublayer, finish after it); it reads W_k, x, y and k_post and writes
    x_out, y_out and k_post.  The fused decode head runs the selector in the
    LM-head launches (W_H streams with W_lm, the walk in the merge launch), so
    its floor is bytes only: W_H plus the gathered codebook rows."""
    es = 4 if w.dtype == "f32" else 2
    N, H, T, G, r, K, bs = w.n_rows, w.hidden, w.taps, w.groups, w.rank, w.top_k, w.block_size
    conv_bytes = 2 * T * G * H * es + 4 * N * H * es + 2 * N * T * G * 4
    sel_bytes = r * H * es + 2 * (bs - 1) * K * r * es + N * r * 4
    sel_launches = 0 if path == "decode_head" else 2
    conv_floor = (2 * launch_floor_us + conv_bytes / (HBM_PEAK_GBS * 1e3)) * 1e-3
    sel_floor = (sel_launches * launch_floor_us + sel_bytes / (HBM_PEAK_GBS * 1e3)) * 1e-3
    lm = ops["lmhead"]
    return {"launch_floor_us": launch_floor_us,
            "conv": {"ms": ops["conv"], "launches": 2, "bytes": conv_bytes, "floor_ms": conv_floor,
                     "gap_ms": ops["conv"] - conv_floor},
            "selector": {"ms": ops["selector"], "launches": sel_launches, "bytes": sel_bytes, "floor_ms": sel_floor,
                         "gap_ms": ops["selector"] - sel_floor},
            "ratio_at_floors": (conv_floor + sel_floor) / lm if lm > 0 else None,
            "target_ratio": 0.05}


def traffic_for(key):
    """HBM bytes per launch from committed rocprofv3 counters, or None when
    they are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    e = t.get(key)
    if not e or e.get("source_hash") != lmhead_source_hash():
        return None
    return e["fetch_kib"] * 1024.0 * e["fetch_scale"] + e["write_kib"] * 1024.0 * e["write_scale"]


def backward_report(w, ms):
    """Selector CE backward: its algorithmic bytes and flops over its measured time.
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


def cpu_baseline(w, inp, budget_s, acc):
    """The oracle as it stands, on the host: whole steps of the same workload
    on one anchor block, repeated within the budget.  acc: the precision of
    the oracle's sums (numpy float64 is the oracle itself)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import dflash2_oracle as O

    bs = w.block_size
    rows = slice(0, bs)
    t_all, reps = 0.0, 0
    saved = O.ACC
    O.ACC = acc
    try:
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
                O.selector_walk(g, inp["cb_pred"], inp["cb_succ"], ids, vals, inp["anchors"][:1], bs, w.dtype)
            t_all += time.perf_counter() - t0
            reps += 1
            if t_all >= budget_s or reps >= 50:
                break
    finally:
        O.ACC = saved
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    name = "float64" if acc == np.float64 else "float32"
    return {
        "value": reps / t_all, "unit": "blocks/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{reps} whole oracle step(s) on 1 anchor block of {w.name} ({name} sums, numpy, {t_all:.1f} s); "
                  f"host has {os.cpu_count()} CPUs",
    }


class Timer:
    """Per-step device times with events on the launch stream; before each
    step (outside its events) a FLUSH_MIB write evicts the MALL."""

    def __init__(self, torch):
        self.torch = torch
        self.flush_buf = torch.empty(FLUSH_MIB << 20, dtype=torch.uint8, device="cuda")

    def steps(self, fn, n, flush=True):
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        out = None
        for a, b in ev:
            if flush:
                self.flush_buf.zero_()
            a.record()
            out = fn()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev], out

    def back_to_back(self, fn, n):
        """Mean device time of n calls between two events (no flush)."""
        torch = self.torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def attribution(self, variants, n, rounds=5):
        """Median step time of each variant, timed in interleaved rounds."""
        per = {k: [] for k in variants}
        m = max(1, math.ceil(n / rounds))
        for _ in range(rounds):
            for k, fn in variants.items():
                per[k] += self.steps(fn, m)[0]
        return {k: statistics.median(v) for k, v in per.items()}, m * rounds


def gpu_inputs(torch, w, seed=0):
    """The workload's fields with the distributions of the seeded recipe
    (block_draft_head_amd.inputs), drawn on the device: the configurations
    other than the headline are timed only, so their draws need not match
    the CPU generator's."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    N, H, V, T, G, r = w.n_rows, w.hidden, w.vocab, w.taps, w.groups, w.rank
    s = math.sqrt(256.0 / H)

    def normal(shape, std, mean=0.0):
        t = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).mul_(std)
        if mean:
            t.add_(mean)
        return t.to(dt)

    base = torch.randn((2, T, H), generator=g, device="cuda").mul_(0.05)
    base[:, 0, :] += 1.0
    ids = lambda n: torch.randint(0, V, (n,), generator=g, device="cuda", dtype=torch.int32)
    return {
        "h": normal((N, H), 1.0), "y": normal((N, H), 1.0), "w_lm": normal((V, H), 1.0 / math.sqrt(H)),
        "base": base.to(dt), "w_proj": normal((2 * T * G, H), 0.01 * s), "w_h": normal((r, H), 0.05 * s),
        "cb_pred": normal((V, r), 0.05), "cb_succ": normal((V, r), 0.05), "anchors": ids(w.n_blocks),
        "pred": ids(N), "gold": ids(N),
        "force": (torch.rand(N, generator=g, device="cuda") < 0.8).to(torch.uint8),
    }


class Path:
    """One workload's ops on device tensors, and the step variants."""

    def __init__(self, D, torch, w, dev, args):
        self.D, self.torch, self.w, self.dev, self.args = D, torch, w, dev, args
        bs, T, gs, K, r = w.block_size, w.taps, w.group_size, w.top_k, w.rank
        N, H, V = w.n_rows, w.hidden, w.vocab
        self.tf = w.mode == "tf"
        self.transformed = args.metrics or args.output_multiplier != 1.0 or args.softcap != 0.0
        self.fused = (not self.tf and not self.transformed and args.selector == "greedy" and w.dtype == "bf16"
                      and N <= 8 and H % 512 == 0)
        mk = lambda op, rr: D.make_workspace(op, N, H, V, rr, K, "cuda")
        if self.fused:
            self.ws_head = mk(D.OP_DECODE_HEAD, r)
            self.ws_lat = mk(D.OP_DECODE_HEAD, 0)
            self.head_out = (torch.empty((N, K), dtype=torch.int32, device="cuda"),
                             torch.empty((N, K), dtype=torch.float32, device="cuda"),
                             torch.empty((w.n_blocks, bs), dtype=torch.int32, device="cuda"),
                             torch.empty((w.n_blocks, bs), dtype=torch.float32, device="cuda"))
        # outside the decode head, the context rows ride on the LM head's call
        self.ctx = not self.fused and args.context_rows == "lmhead"
        self.g = torch.empty((N, r), dtype=torch.float32, device="cuda") if self.ctx else None
        self.ws_topk = mk(D.OP_UNARY_TOPK, 0)
        self.ws_sel = mk(D.OP_SELECTOR_TF if self.tf else D.OP_SELECTOR_WALK, r)
        if self.tf:
            self.ws_bwd = mk(D.OP_SELECTOR_CE_BACKWARD, r)
            self.grads = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in ((V, r), (V, r), (r, H))]
            self.grad_ce = torch.full((N,), 1.0 / N, dtype=torch.float32, device="cuda")
        self.x_out = torch.empty_like(dev["h"])
        self.k_post = torch.empty((N, T, H // gs), dtype=torch.float32, device="cuda")
        self.y_out = torch.empty_like(dev["y"])
        self.gold = dev["gold"] if self.tf else None
        self.metrics_out = {}
        self.last = None

    def conv(self):
        d, w = self.dev, self.w
        self.D.conv_prepare(d["h"], d["w_proj"], d["base"], w.block_size, w.taps, w.group_size, out=self.x_out,
                            k_post=self.k_post)
        self.D.conv_finish(d["y"], self.k_post, d["base"], w.block_size, w.taps, w.group_size, out=self.y_out)

    def lmhead(self):
        d, a, K = self.dev, self.args, self.w.top_k
        if self.fused:
            ids, vals, _, _ = self.D.decode_head(d["h"], d["w_lm"], K, workspace=self.ws_lat,
                                                 out=(self.head_out[0], self.head_out[1], None, None))
            return ids, vals, None
        if not self.transformed and not self.ctx:
            return self.D.unary_topk(d["h"], d["w_lm"], K, gold_ids=self.gold, workspace=self.ws_topk)
        ids, vals, gl, lse, prob, hit = self.D.unary_topk_ex(d["h"], d["w_lm"], K, gold_ids=self.gold,
                                                             output_multiplier=a.output_multiplier,
                                                             softcap=a.softcap, want_lse=a.metrics,
                                                             want_metrics=a.metrics, workspace=self.ws_topk,
                                                             w_h=d["w_h"] if self.ctx else None, g=self.g)
        self.metrics_out.update(lse=lse, prob=prob, hit=hit)
        return ids, vals, gl

    def selector(self, ids, vals, gl):
        d, w, D = self.dev, self.w, self.D
        # with the context rows formed by the LM head, h and W_H are not passed
        h, wh = (None, None) if self.ctx else (d["h"], d["w_h"])
        if self.tf:
            return D.selector_score_tf(h, wh, d["cb_pred"], d["cb_succ"], ids, vals, d["pred"], gold_ids=self.gold,
                                       force=d["force"], gold_logit=gl, workspace=self.ws_sel, g=self.g)
        if self.args.selector == "sample":
            return D.selector_sample(h, wh, d["cb_pred"], d["cb_succ"], ids, vals, d["anchors"], w.block_size,
                                     temperature=1.0, seed=0x5EED, workspace=self.ws_sel, g=self.g)
        return D.selector_walk(h, wh, d["cb_pred"], d["cb_succ"], ids, vals, d["anchors"], w.block_size,
                               workspace=self.ws_sel, g=self.g)

    def backward(self, ids, vals, gl):
        d = self.dev
        return self.D.selector_ce_backward(d["h"], d["w_h"], d["cb_pred"], d["cb_succ"], ids, vals, d["pred"],
                                           self.gold, self.grad_ce, force=d["force"], gold_logit=gl,
                                           grad_pred=self.grads[0], grad_succ=self.grads[1],
                                           grad_wh=self.grads[2], want_ce=False, workspace=self.ws_bwd)

    def head_with_selector(self):
        """LM head + selector: one call for the decode head, two otherwise."""
        d, w = self.dev, self.w
        if self.fused:
            ids, vals, path, ps = self.D.decode_head(d["h"], d["w_lm"], w.top_k, d["w_h"], d["cb_pred"],
                                                     d["cb_succ"], d["anchors"], w.block_size,
                                                     workspace=self.ws_head, out=self.head_out)
            self.last = (ids, vals, None, (path, ps))
            return self.last
        ids, vals, gl = self.lmhead()
        res = self.selector(ids, vals, gl)
        if self.args.train:
            self.backward(ids, vals, gl)
        self.last = (ids, vals, gl, res)
        return self.last

    def variants(self):
        def full():
            self.conv()
            return self.head_with_selector()

        def no_conv():
            return self.head_with_selector()

        def no_selector():
            self.conv()
            return self.lmhead()

        return {"full": full, "no_conv": no_conv, "no_selector": no_selector}

    def teeth(self):
        """Share of walk steps whose pick is not the unary argmax (slot 0)."""
        if self.tf or self.last is None:
            return None
        ids, _, _, res = self.last
        bs = self.w.block_size
        if bs < 2:
            return None
        path = res[0]
        first = ids.view(self.w.n_blocks, bs, -1)[:, 1:, 0]
        return float((path[:, 1:] != first).float().mean())


def roofline(w, lm_ms, key, ctx=False):
    lm_bytes, lm_flops = lmhead_work(w, ctx)
    mfma_bound = lm_flops / lm_bytes > (BF16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9) and w.dtype == "bf16"
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": lm_flops / (lm_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "algorithmic_flops": lm_flops}
    else:
        roof = {"bound": "hbm", "achieved": lm_bytes / (lm_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "algorithmic_bytes": lm_bytes}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_for(key)
    roof["avg_ms"] = lm_ms
    return roof


def measure(D, torch, timer, w, dev, args, steps, warmup, attr_steps):
    """Headline-style measurement of one workload."""
    p = Path(D, torch, w, dev, args)
    var = p.variants()
    for _ in range(warmup):
        var["full"]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    per, _ = timer.steps(var["full"], steps)
    wall = time.perf_counter() - t0
    teeth = p.teeth()
    med, n_attr = timer.attribution(var, attr_steps)
    conv = med["full"] - med["no_conv"]
    sel = med["full"] - med["no_selector"]
    lm = med["full"] - conv - sel
    # the LM-head op back to back (the weight stream exceeds the MALL, so no flush is needed)
    lm_b2b = timer.back_to_back(p.lmhead, 50 if w.n_rows <= 64 else 10)
    ctx_ms = None
    if p.ctx:
        # the context rows' share of the LM-head op: the op minus the same op
        # without W_H, both back to back in 5 interleaved rounds (median)
        d = p.dev
        plain = lambda: D.unary_topk(d["h"], d["w_lm"], w.top_k, gold_ids=p.gold, workspace=p.ws_topk)
        reps = 50 if w.n_rows <= 64 else 10
        diffs = [timer.back_to_back(p.lmhead, reps) - timer.back_to_back(plain, reps) for _ in range(5)]
        ctx_ms = statistics.median(diffs)
    kern = ("lmhead_dma_kernel + decode_tail_kernel" if p.fused else
            "lmhead_dma_kernel + top-K merge" if w.n_rows <= 8 and w.dtype == "bf16" else
            "lmhead_stream_kernel + top-K merge" if w.n_rows <= 8 else
            "lmhead_big_kernel + top-K merge" if w.dtype == "bf16" else "lmhead_tiled_kernel + top-K merge")
    if p.ctx:
        kern += (" (W_H tiles in the stream)" if w.dtype == "bf16" and w.n_rows > 8 else
                 " + context projection")
    roof = roofline(w, lm_b2b, w.name, p.ctx)
    roof["kernel"] = kern
    out = {
        "ms_per_step": statistics.median(per), "ms_per_step_mean": statistics.fmean(per),
        "blocks_per_s": w.n_blocks / (statistics.median(per) * 1e-3), "wall_s_timed": wall,
        "ops_ms": {"conv": conv, "lmhead": lm, "selector": sel},
        "selector_plus_conv_over_lmhead": (conv + sel) / lm if lm > 0 else None,
        "attribution_ms": {k: v for k, v in med.items()}, "attribution_steps_per_variant": n_attr,
        "roofline": roof, "teeth": teeth, "path": "decode_head" if p.fused else "unary_topk + selector",
        "context_rows": "decode head" if p.fused else "lm head" if p.ctx else "selector",
        "context_rows_ms": ctx_ms,
    }
    if w.name in TARGETS:
        out["roofline_target_frac"] = TARGETS[w.name]
    if p.tf:
        _, _, _, res = p.last
        out["tf_coverage"] = float(res[3].float().mean())
        if args.train:
            bwd = timer.back_to_back(lambda: p.backward(*p.last[:3]), 5)
            out["ce_backward"] = backward_report(w, bwd)
    if args.metrics and p.metrics_out.get("lse") is not None:
        m = {"mean_log_sum_exp": float(p.metrics_out["lse"].mean())}
        if p.metrics_out.get("hit") is not None:
            hit = p.metrics_out["hit"].float()
            m.update({"recall_at_k": float(hit.mean()), "coverage": float(hit.mean()),
                      "target_mass": float(p.metrics_out["prob"].mean())})
        out["unary_metrics"] = m
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no "
              f"multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_draft_head_amd import dflash2 as D
    from block_draft_head_amd.inputs import WORKLOAD_ORDER, WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    log(f"workload {w.name}: generating inputs")
    inp = make_inputs(w)
    dev = {}
    for k, a in inp.items():
        if a.dtype == np.uint16:
            dev[k] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        else:
            dev[k] = torch.from_numpy(a).cuda()
    torch.cuda.synchronize()
    log("inputs resident on the GPU")
    timer = Timer(torch)

    # floors of this device, measured in the same run
    timer.back_to_back(lambda: torch.cuda._sleep(1), 50)
    launch_floor = timer.back_to_back(lambda: torch.cuda._sleep(1), 1000) * 1e3
    ev = timer.steps(lambda: None, 200, flush=False)[0]
    event_overhead = statistics.median(ev) * 1e3

    attr = args.attr_steps or (200 if w.n_rows <= 8 else 30)
    log(f"timing {args.steps} steps after {args.warmup} warmup; attribution over {attr} steps per variant")
    head = measure(D, torch, timer, w, dev, args, args.steps, args.warmup, attr)

    # achievable HBM rate on this device: a 1 GiB device-to-device copy (read
    # plus write bytes over its event time, best of 5), beside the 8 TB/s peak
    cs = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cd = torch.empty_like(cs)
    cd.copy_(cs)
    copy_ms = min(timer.back_to_back(lambda: cd.copy_(cs), 1) for _ in range(5))
    copy_gbs = 2.0 * (1 << 30) / (copy_ms * 1e-3) / 1e9
    del cs, cd
    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ops = head["ops_ms"]
    out = {
        "metric": METRIC,
        "value": head["blocks_per_s"],
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "n_blocks": w.n_blocks, "block_size": w.block_size, "hidden": w.hidden,
                   "vocab": w.vocab, "taps": w.taps, "group_size": w.group_size, "rank": w.rank,
                   "top_k": w.top_k, "mode": w.mode,
                   "selector": ("teacher-forced + CE backward" if args.train else "teacher-forced")
                   if w.mode == "tf" else args.selector,
                   "unary": {"output_multiplier": args.output_multiplier, "softcap": args.softcap,
                             "metrics": args.metrics}},
        "roofline": head["roofline"],
        "timing": {"per_step": f"median of {args.steps} steps, each after a {FLUSH_MIB} MiB write that evicts "
                               f"the MALL (outside its events); HIP events on the launch stream",
                   "ms_per_step_mean": head["ms_per_step_mean"], "wall_s_timed": head["wall_s_timed"],
                   "event_overhead_us": event_overhead, "launch_floor_us": launch_floor,
                   "attribution": "full - no_conv = conv; full - no_selector = selector; medians of "
                                  f"{head['attribution_steps_per_variant']} flushed steps per variant, "
                                  "interleaved in 5 rounds",
                   "attribution_ms": head["attribution_ms"]},
        "path": head["path"],
        "context_rows": head["context_rows"],
        "context_rows_ms": head["context_rows_ms"],
        "ops_ms": ops,
        "selector_plus_conv_over_lmhead": head["selector_plus_conv_over_lmhead"],
        "conv_10_wrappers_ms": 10 * ops["conv"],
        "teeth": head["teeth"],
        "copy_gbs": copy_gbs,
    }
    for k in ("roofline_target_frac", "tf_coverage", "ce_backward", "unary_metrics"):
        if k in head:
            out[k] = head[k]
    out["timing"]["median_ms_flushed_steps"] = head["attribution_ms"]["full"]
    if w.n_rows <= 8:
        out["small_op_floors"] = small_op_floors(w, ops, launch_floor, head["path"])

    if not args.no_workloads:
        wl = {}
        # (timed steps, warmup, steps per attribution variant): the attribution
        # differences are small against the LM head, so they get more steps
        budget = {"tiny_fp32_16x8_h256_v4096": (50, 10, 50), "serve_64x8_h5120_v248320": (30, 5, 100),
                  "packed_tf_512x8_h4096_v151936": (15, 3, 40), "wide_256x16_h5120_v248320_t8_k64": (10, 3, 20),
                  "decode_1x8_h4096_v151936": (50, 10, 200)}
        sub = argparse.Namespace(**{**vars(args), "train": False, "metrics": False, "output_multiplier": 1.0,
                                    "softcap": 0.0, "selector": "greedy"})
        for name in WORKLOAD_ORDER:
            if name == w.name:
                continue
            wk = WORKLOADS[name]
            log(f"workload {name}")
            d2 = gpu_inputs(torch, wk)
            steps, warm, at = budget[name]
            r = measure(D, torch, timer, wk, d2, sub, steps, warm, at)
            wl[name] = {k: r[k] for k in ("ms_per_step", "blocks_per_s", "ops_ms", "selector_plus_conv_over_lmhead",
                                          "roofline", "teeth", "path", "attribution_steps_per_variant",
                                          "context_rows", "context_rows_ms")}
            for k in ("roofline_target_frac", "tf_coverage"):
                if k in r:
                    wl[name][k] = r[k]
            del d2
            torch.cuda.empty_cache()
        out["workloads"] = wl

    if not args.no_cpu_baseline:
        log("timing the CPU oracle (float64, then float32 sums)")
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds, np.float64)
        out["cpu_baseline_fp32"] = cpu_baseline(w, inp, args.cpu_seconds, np.float32)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
