"""GPU parity of the selector's context rows g = h W_Hᵀ formed inside the LM
head's call (dflash2_unary_topk_ex with W_H: extra tiles of the many-row
kernel's weight stream, its own launch in the other regimes) and of the
walk, sampling and teacher-forcing calls fed those rows in place of h and
W_H."""
import numpy as np
import pytest
import torch

from block_draft_head_amd.inputs import Workload, make_inputs
from oracle import dflash2_oracle as O
from tests.helpers import (close, compare_sample, compare_tf, compare_topk, compare_walk, context_ok, scale_codebooks,
                           to_dev, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    from block_draft_head_amd import dflash2
    assert torch.cuda.is_available(), "no GPU visible"
    return dflash2


def log(msg):
    print(msg, flush=True)


def inputs(nb, bs, H, V, r, K, dtype, seed):
    w = Workload("ctx", nb, bs, H, V, dtype, 2, 16, r, K, "walk+tf")
    return make_inputs(w, seed=seed, fields=["h", "w_lm", "w_h", "cb_pred", "cb_succ", "anchors", "pred", "gold",
                                             "force"])


CTX_CASES = [
    # (N, H, V, r, K, dtype, forced slabs): 256 x 256 MFMA tiles with one,
    # two and three context tiles (ragged ranks 40 and 520), row tiles with a
    # ragged tail, slabs that end in context tiles or hold only context
    # tiles (V 2000 is 8 vocabulary tiles; 8 slabs over 8 + 3 tiles leave the
    # last two with context tiles only), lists of 16 and 64; the LDS-streamed,
    # register-streamed and float32 tiled regimes, which form g in a launch of
    # their own
    (300, 256, 5000, 40, 16, "bf16", 0), (513, 512, 20011, 256, 16, "bf16", 0),
    (260, 256, 2000, 520, 16, "bf16", 8), (260, 256, 2000, 520, 64, "bf16", 8),
    (256, 1024, 9001, 264, 8, "bf16", 3), (600, 256, 70001, 512, 16, "bf16", 1),
    (8, 4096, 30011, 256, 16, "bf16", 0), (5, 320, 4099, 40, 16, "bf16", 0),
    (7, 256, 7001, 32, 16, "f32", 0), (100, 256, 3001, 264, 16, "f32", 0),
]


@pytest.mark.parametrize("N,H,V,r,K,dtype,slabs", CTX_CASES)
def test_unary_topk_forms_the_context_rows(D, N, H, V, r, K, dtype, slabs):
    log(f"topk+g N={N} H={H} V={V} r={r} K={K} {dtype} slabs={slabs or 'auto'}")
    inp = inputs(N, 1, H, V, r, K, dtype, 31)
    dev = {k: to_dev(inp[k]) for k in ("h", "w_lm", "w_h", "gold")}
    try:
        D.debug_force_slabs(slabs)
        ids, vals, gl, g = D.unary_topk_ctx(dev["h"], dev["w_lm"], K, dev["w_h"], gold_ids=dev["gold"])
        ref_ids, ref_vals, ref_gl = D.unary_topk(dev["h"], dev["w_lm"], K, gold_ids=dev["gold"])
        torch.cuda.synchronize()
    finally:
        D.debug_force_slabs(0)
    # the vocabulary tiles are the same with or without the context tiles
    assert torch.equal(ids, ref_ids) and torch.equal(vals, ref_vals) and torch.equal(gl, ref_gl)
    ok = context_ok(to_np(g), inp["h"], inp["w_h"], dtype)
    assert ok.all(), (np.argwhere(~ok)[:5], to_np(g)[~ok][:5])
    U = O.lm_logits(inp["h"], inp["w_lm"], dtype)
    fails, flags, msgs = compare_topk(to_np(ids), to_np(vals), U, K)
    log(f"  topk fails={fails} flags={flags}")
    assert fails == 0, msgs[:5]


def test_context_rows_are_written_in_full_each_call(D):
    # g filled with NaN first: every element is overwritten, on two calls
    # with the second one smaller, and nothing past N x r is touched
    N, H, V, r, K = 300, 256, 5000, 264, 16
    inp = inputs(N, 1, H, V, r, K, "bf16", 33)
    h, w_lm, w_h = (to_dev(inp[k]) for k in ("h", "w_lm", "w_h"))
    buf = torch.full((N * r + 64,), float("nan"), dtype=torch.float32, device="cuda")
    g = buf[:N * r].view(N, r)
    D.unary_topk_ctx(h, w_lm, K, w_h, g=g)
    torch.cuda.synchronize()
    assert context_ok(to_np(g), inp["h"], inp["w_h"], "bf16").all()
    assert torch.isnan(buf[N * r:]).all()
    n2 = 100
    buf.fill_(float("nan"))
    g2 = buf[:n2 * r].view(n2, r)
    D.unary_topk_ctx(h[:n2], w_lm, K, w_h, g=g2)
    torch.cuda.synchronize()
    assert context_ok(to_np(g2), inp["h"][:n2], inp["w_h"], "bf16").all()
    assert torch.isnan(buf[n2 * r:]).all()


WALK_CASES = [
    # (n_blocks, bs, H, V, r, K, dtype): the many-row bf16 kernel (g from its
    # context tiles) and float32 tiles (g from the projection's own launch)
    (40, 8, 512, 5000, 256, 16, "bf16"), (20, 16, 256, 3001, 520, 64, "bf16"), (6, 8, 256, 2000, 40, 16, "f32"),
]


@pytest.mark.parametrize("nb,bs,H,V,r,K,dtype", WALK_CASES)
def test_selector_calls_take_the_context_rows(D, nb, bs, H, V, r, K, dtype):
    log(f"walk/sample/tf from g nb={nb} bs={bs} H={H} V={V} r={r} K={K} {dtype}")
    inp = inputs(nb, bs, H, V, r, K, dtype, 37)
    scale_codebooks(inp, r, dtype)
    dev = {k: to_dev(v) for k, v in inp.items()}
    N = nb * bs
    ids, vals, _, g = D.unary_topk_ctx(dev["h"], dev["w_lm"], K, dev["w_h"])
    cb = (dev["cb_pred"], dev["cb_succ"])
    path, ps = D.selector_walk(None, None, *cb, ids, vals, dev["anchors"], bs, g=g)
    # h and W_H given beside g are not read
    path_b, ps_b = D.selector_walk(dev["h"], dev["w_h"], *cb, ids, vals, dev["anchors"], bs, g=g)
    path_na, ps_na = D.selector_walk_noalloc(None, None, *cb, ids, vals, dev["anchors"], bs, g=g)
    torch.cuda.synchronize()
    assert torch.equal(path_b, path) and torch.equal(path_na, path)
    assert torch.equal(ps_b.nan_to_num(0.0), ps.nan_to_num(0.0)) and torch.equal(ps_na.nan_to_num(0.0),
                                                                                 ps.nan_to_num(0.0))
    U = O.lm_logits(inp["h"], inp["w_lm"], dtype)
    gids = to_np(ids)
    u64 = U[np.arange(N)[:, None], gids]
    g64 = O.context_projection(inp["h"], inp["w_h"], dtype)
    fails, flags, teeth, msgs = compare_walk(to_np(path), to_np(ps), g64, inp["cb_pred"], inp["cb_succ"], gids, u64,
                                             inp["anchors"], bs, dtype)
    log(f"  walk fails={fails} flags={flags} teeth={teeth}/{nb * (bs - 1)}")
    assert fails == 0, msgs[:5]
    assert teeth > 0
    # sampling
    seed = 0x51ED2700 + nb
    sp, sps = D.selector_sample(None, None, *cb, ids, vals, dev["anchors"], bs, temperature=0.7, seed=seed, g=g)
    fails, flags, msgs = compare_sample(to_np(sp), to_np(sps), g64, inp["cb_pred"], inp["cb_succ"], gids, u64,
                                        inp["anchors"], bs, dtype, 0.7, seed)
    log(f"  sample fails={fails} flags={flags}")
    assert fails == 0, msgs[:5]
    # teacher forcing with gold ids, forcing and the gold logits
    gold = inp["gold"].copy()
    gold[::3] = gids[::3, K // 2]
    glog = U[np.arange(N), gold].astype(np.float32)
    gpu = D.selector_score_tf(None, None, *cb, ids, vals, dev["pred"], gold_ids=to_dev(gold), force=dev["force"],
                              gold_logit=to_dev(glog), g=g)
    ref = O.selector_score_tf(g64, inp["cb_pred"], inp["cb_succ"], gids, u64, inp["pred"], dtype, gold_ids=gold,
                              force=inp["force"], gold_logit=glog.astype(np.float64))
    fails, flags, msgs = compare_tf(tuple(to_np(t) for t in gpu), ref, gids)
    log(f"  tf fails={fails} flags={flags}")
    assert fails == 0, msgs[:5]


def test_walk_from_context_rows_clears_the_status(D):
    # a walk that flags an out-of-range anchor, then one from g on the same
    # workspace: the status word is cleared although no projection runs
    nb, bs, H, V, r, K = 4, 8, 256, 2000, 32, 16
    inp = inputs(nb, bs, H, V, r, K, "bf16", 41)
    dev = {k: to_dev(v) for k, v in inp.items()}
    ids, vals, _, g = D.unary_topk_ctx(dev["h"], dev["w_lm"], K, dev["w_h"])
    ws = D.make_workspace(D.OP_SELECTOR_WALK, nb * bs, H, V, r, K, "cuda")
    bad = dev["anchors"].clone()
    bad[2] = V + 5
    path, _ = D.selector_walk(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals, bad, bs, workspace=ws)
    assert D.read_device_status(ws) == 8 and (path[2] == -1).all()
    path, _ = D.selector_walk(None, None, dev["cb_pred"], dev["cb_succ"], ids, vals, dev["anchors"], bs,
                              workspace=ws, g=g)
    assert D.read_device_status(ws) == 0 and (path >= 0).all()


LSE_CASES = [
    # (N, H, V, r, K, dtype, forced slabs): 256 x 256 tiles with two slabs of
    # context tiles only; the LDS-streamed and the float32 register-streamed
    # decode regimes, where g is its own launch beside the log-sum-exp kernels
    (260, 256, 2000, 520, 16, "bf16", 8), (8, 4096, 30011, 256, 16, "bf16", 0), (5, 256, 7001, 32, 16, "f32", 0),
]


@pytest.mark.parametrize("N,H,V,r,K,dtype,slabs", LSE_CASES)
def test_context_rows_leave_the_log_sum_exp_and_metrics_alone(D, N, H, V, r, K, dtype, slabs):
    # slabs holding only context tiles contribute empty lists and an empty
    # log-sum-exp partial; the transformed top-K, the log-sum-exp and the gold
    # metrics match the oracle as without W_H
    log(f"topk_ex+g+lse N={N} H={H} V={V} r={r} K={K} {dtype} slabs={slabs or 'auto'}")
    mult, cap = 1.3, 6.0
    inp = inputs(N, 1, H, V, r, K, dtype, 43)
    gold = inp["gold"].copy()
    U = O.lm_logits(inp["h"], inp["w_lm"], dtype)
    gold[::3] = np.argmax(U[::3], axis=1)
    dev = {k: to_dev(inp[k]) for k in ("h", "w_lm", "w_h")}
    g = torch.empty((N, r), dtype=torch.float32, device="cuda")
    try:
        D.debug_force_slabs(slabs)
        ids, vals, gl, lse, prob, hit = D.unary_topk_ex(dev["h"], dev["w_lm"], K, gold_ids=to_dev(gold),
                                                        output_multiplier=mult, softcap=cap, want_lse=True,
                                                        want_metrics=True, w_h=dev["w_h"], g=g)
        torch.cuda.synchronize()
    finally:
        D.debug_force_slabs(0)
    rids, rvals, rlse, rgl, rprob, rhit = O.unary_topk_ex(inp["h"], inp["w_lm"], K, dtype, gold_ids=gold,
                                                          output_multiplier=mult, softcap=cap)
    fails, flags, msgs = compare_topk(to_np(ids), to_np(vals), O.transform_logits(U, mult, cap), K)
    assert fails == 0, msgs[:5]
    assert close(to_np(gl), rgl).all() and close(to_np(lse), rlse).all()
    assert close(to_np(prob), rprob, atol=1e-6).all()
    assert np.array_equal(to_np(hit), (to_np(ids) == gold[:, None]).any(1).astype(np.uint8))
    assert context_ok(to_np(g), inp["h"], inp["w_h"], dtype).all()
