"""GPU parity at the full workload sizes, in the launch configuration that
bench.py times (same shapes, same seeded inputs, same workspaces, the fused
decode head where bench.py uses it).

The oracle cannot redo a whole full-size pass in seconds, so each stage is
checked on what it can compute one by one:

* conv prepare / finish on sampled whole anchor blocks (the conv never
  crosses a block, so a block's rows are exact on their own), the first and
  last block among them, under the float32 error rule of tests/helpers.py;
* unary top-K against each checked row's exact logits over the full
  vocabulary (plus the gold logit on the teacher-forced workload): every row
  of the decode workload, and on the many-row workloads the first, the last
  and one random row of every 256-row tile (the many-row kernel's row tile).
  Every checked row's list is merged from every vocabulary slab's partial
  list, so each slab takes part in every checked row;
* outside the decode head, the context rows that the LM head's call forms
  (every element, within the float32 bound of tests/helpers.py);
* the selector on every block / row, fed those rows, the oracle fed the
  GPU's candidate ids with its own exact logits for them and its own exact
  context rows (stage-wise, so a top-K near-tie cannot cascade); the walks
  must override the unary pick somewhere.
"""
import numpy as np
import pytest
import torch

from block_draft_head_amd.inputs import WORKLOAD_ORDER, WORKLOADS, make_inputs
from oracle import dflash2_oracle as O
from tests.helpers import (act_ok, close, compare_grads, compare_tf, compare_topk, compare_walk, context_ok, conv_delta,
                           corr_abs, corr_ok, oracle_logits_rows, to_dev, to_np)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def D():
    from block_draft_head_amd import dflash2
    assert torch.cuda.is_available(), "no GPU visible"
    return dflash2


def log(msg):
    print(msg, flush=True)


def mismatch(gpu, ref, ok, dt):
    idx = np.argwhere(~ok)[:4]
    return [(tuple(map(int, i)), float(O.widen(gpu[tuple(i)], dt)), float(ref[tuple(i)])) for i in idx]


def sample(n, k, rng):
    """First, last and k - 2 random distinct indices of range(n)."""
    pick = {0, n - 1}
    while len(pick) < min(k, n):
        pick.add(int(rng.integers(0, n)))
    return sorted(pick)


def tile_rows(n, rng, tile=256):
    """Every row when n <= 8; else the first, the last and one random row of
    every `tile`-row tile."""
    if n <= 8:
        return list(range(n))
    pick = set()
    for t0 in range(0, n, tile):
        t1 = min(n, t0 + tile)
        pick |= {t0, t1 - 1, int(rng.integers(t0, t1))}
    return sorted(pick)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", [n for n in WORKLOAD_ORDER if not n.startswith("tiny")])
def test_full_size_workload(D, name):
    w = WORKLOADS[name]
    bs, T, gs, K, r = w.block_size, w.taps, w.group_size, w.top_k, w.rank
    N, H, V, dt = w.n_rows, w.hidden, w.vocab, w.dtype
    tf_mode = w.mode == "tf"
    rng = np.random.default_rng(1234)
    log(f"[{name}] generating inputs")
    inp = make_inputs(w)
    dev = {k: to_dev(v) for k, v in inp.items()}

    # ---- conv, on sampled whole blocks
    log(f"[{name}] conv")
    x_out = torch.empty_like(dev["h"])
    y_out = torch.empty_like(dev["y"])
    k_post = torch.empty((N, T, H // gs), dtype=torch.float32, device="cuda")
    D.conv_prepare(dev["h"], dev["w_proj"], dev["base"], bs, T, gs, out=x_out, k_post=k_post)
    D.conv_finish(dev["y"], k_post, dev["base"], bs, T, gs, out=y_out)
    blocks = sample(w.n_blocks, 16, rng)
    rows = np.concatenate([np.arange(b * bs, (b + 1) * bs) for b in blocks])
    xo, kp, yo = to_np(x_out[rows]), to_np(k_post[rows]), to_np(y_out[rows])
    hr = inp["h"][rows]
    _, kp_r, ex = O.conv_prepare(hr, inp["w_proj"], inp["base"], bs, T, gs, dt)
    c = O.conv_projection(hr, inp["w_proj"], T, gs, dt)
    A = corr_abs(hr, inp["w_proj"], T, gs, dt)
    assert close(kp, kp_r).all(), "k_post differs"
    if dt == "bf16":
        okc = corr_ok(kp, kp_r, A[:, 1])
        assert okc.all(), f"k_post beyond the float32 bound at {np.argwhere(~okc)[:3]}"
    ok = act_ok(xo, ex, dt, conv_delta(hr, c[:, 0], inp["base"][0], bs, gs, dt, A[:, 0]))
    assert ok.all(), f"x_out: {(~ok).sum()} mismatches in blocks {blocks}: {mismatch(xo, ex, ok, dt)}"
    _, ey = O.conv_finish(inp["y"][rows], kp, inp["base"], bs, T, gs, dt)
    ok = act_ok(yo, ey, dt, conv_delta(inp["y"][rows], kp, inp["base"][1], bs, gs, dt))
    assert ok.all(), f"y_out: {(~ok).sum()} mismatches in blocks {blocks}: {mismatch(yo, ey, ok, dt)}"

    # ---- unary top-K, on the checked rows against the exact full-vocabulary
    # logits (the decode workload through the fused decode head, as timed)
    log(f"[{name}] unary top-K")
    fused = w.mode == "walk" and N <= 8 and dt == "bf16" and H % 512 == 0
    gold = dev["gold"] if tf_mode else None
    if fused:
        ws = D.make_workspace(D.OP_DECODE_HEAD, N, H, V, r, K, "cuda")
        ids, vals, path, ps = D.decode_head(dev["h"], dev["w_lm"], K, dev["w_h"], dev["cb_pred"], dev["cb_succ"],
                                            dev["anchors"], bs, workspace=ws)
        gl = None
    else:
        # the context rows formed in the LM head's call, as bench.py does
        ws = D.make_workspace(D.OP_UNARY_TOPK, N, H, V, 0, K, "cuda")
        ids, vals, gl, g = D.unary_topk_ctx(dev["h"], dev["w_lm"], K, dev["w_h"], gold_ids=gold, workspace=ws)
    assert D.read_device_status(ws) == 0
    gids, gvals = to_np(ids), to_np(vals)
    srows = tile_rows(N, rng)
    U = oracle_logits_rows(inp["h"][srows], inp["w_lm"], dt)
    fails, flags, msgs = compare_topk(gids[srows], gvals[srows], U, K)
    log(f"[{name}] top-K on {len(srows)} rows: fails {fails} flags {flags}")
    assert fails == 0, msgs
    assert flags <= max(1, len(srows) // 20)
    if tf_mode:
        assert close(to_np(gl)[srows], U[np.arange(len(srows)), inp["gold"][srows]]).all(), "gold logit differs"

    # ---- selector, every block / row, oracle fed the GPU candidates
    log(f"[{name}] selector")
    u_at = O.logits_at(inp["h"], inp["w_lm"], gids, dt)
    g64 = O.context_projection(inp["h"], inp["w_h"], dt)
    if not fused:
        ok = context_ok(to_np(g), inp["h"], inp["w_h"], dt)
        assert ok.all(), f"context rows: {(~ok).sum()} outside the bound, first at {np.argwhere(~ok)[:3]}"
    if tf_mode:
        gold_exact = O.logits_at(inp["h"], inp["w_lm"], inp["gold"][:, None], dt)[:, 0]
        assert close(to_np(gl), gold_exact).all(), "gold logit differs"
        ws_sel = D.make_workspace(D.OP_SELECTOR_TF, N, H, V, r, K, "cuda")
        res = D.selector_score_tf(None, None, dev["cb_pred"], dev["cb_succ"], ids, vals, dev["pred"], gold_ids=gold,
                                  force=dev["force"], gold_logit=gl, workspace=ws_sel, g=g)
        gpu = tuple(to_np(t) for t in res)
        ref = O.selector_score_tf(g64, inp["cb_pred"], inp["cb_succ"], gids, u_at, inp["pred"], dt,
                                  gold_ids=inp["gold"], force=inp["force"], gold_logit=gold_exact)
        fails, flags, msgs = compare_tf(gpu, ref, gids)
        cov = float(np.mean(gpu[3]))
        log(f"[{name}] TF: fails {fails} flags {flags} coverage {cov:.4f}")
        assert fails == 0, msgs
        # forced rows always hold gold; the rest only when it is a candidate
        assert 0.75 < cov < 0.85
        # the selector CE's gradients, mean over the valid rows
        log(f"[{name}] selector CE backward")
        wgt = np.full(N, 1.0 / max(1, int(ref[3].sum())), np.float32)
        ws_b = D.make_workspace(D.OP_SELECTOR_CE_BACKWARD, N, H, V, r, K, "cuda")
        gp, gs, gw, ce, valid = D.selector_ce_backward(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids,
                                                       vals, dev["pred"], gold, to_dev(wgt), force=dev["force"],
                                                       gold_logit=gl, workspace=ws_b)
        assert D.read_device_status(ws_b) == 0
        dA, dB, dW, _, rvalid = O.selector_ce_backward(inp["h"], inp["w_h"], inp["cb_pred"], inp["cb_succ"], gids,
                                                       u_at, inp["pred"], dt, inp["gold"], inp["force"],
                                                       gold_exact, wgt.astype(np.float64))
        assert np.array_equal(to_np(valid), rvalid)
        fails, msgs = compare_grads({"dA": to_np(gp), "dB": to_np(gs), "dW": to_np(gw)},
                                    {"dA": dA, "dB": dB, "dW": dW})
        log(f"[{name}] CE backward: fails {fails}")
        assert fails == 0, msgs
    else:
        if not fused:
            ws_sel = D.make_workspace(D.OP_SELECTOR_WALK, N, H, V, r, K, "cuda")
            path, ps = D.selector_walk(None, None, dev["cb_pred"], dev["cb_succ"], ids, vals, dev["anchors"], bs,
                                       workspace=ws_sel, g=g)
            assert D.read_device_status(ws_sel) == 0
        fails, flags, teeth, msgs = compare_walk(to_np(path), to_np(ps), g64, inp["cb_pred"], inp["cb_succ"], gids,
                                                 u_at, inp["anchors"], bs, dt)
        steps = w.n_blocks * (bs - 1)
        log(f"[{name}] walk: {steps} steps, fails {fails} flags {flags} selector overrides {teeth}")
        assert fails == 0, msgs
        assert flags <= max(1, steps // 100)
        if steps >= 64:
            # the pair term overrides the unary pick on some steps (a few per
            # cent at these codebook scales): a selector that ignored it fails
            assert teeth > 0, "the selector never overrode the unary pick"
    torch.cuda.synchronize()
