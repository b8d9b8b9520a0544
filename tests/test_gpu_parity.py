"""GPU parity: the HIP library, called through the C ABI, against the CPU
oracle on the same seeded inputs.  Sizes span several tiles with ragged tails
in both kernel regimes (weight streaming for <= 8 rows, LDS-tiled MFMA for
more); full-size workloads are in test_gpu_workloads.py."""
import numpy as np
import pytest
import torch

from block_draft_head_amd.inputs import Workload, make_inputs, to_storage
from oracle import dflash2_oracle as O
from tests.helpers import (act_ok, close, compare_grads, compare_sample, compare_tf, compare_topk, compare_walk, conv_delta,
                           corr_abs, corr_ok, scale_codebooks, to_dev, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    from block_draft_head_amd import dflash2
    assert torch.cuda.is_available(), "no GPU visible"
    return dflash2


def wl(name="t", n_blocks=4, block_size=8, hidden=256, vocab=4096, dtype="bf16", taps=2, group_size=16,
       rank=32, top_k=16, mode="walk+tf"):
    return Workload(name, n_blocks, block_size, hidden, vocab, dtype, taps, group_size, rank, top_k, mode)


def log(msg):
    print(msg, flush=True)


# --------------------------------------------------------------------- conv

CONV_CASES = [
    # (n_blocks, bs, H, T, gs, dtype): streaming (N <= 8) and tiled, ragged row tiles
    (1, 8, 256, 2, 16, "bf16"), (1, 8, 256, 2, 16, "f32"), (2, 4, 512, 3, 8, "bf16"),
    (1, 4, 256, 1, 64, "bf16"), (1, 8, 256, 8, 32, "bf16"),
    (17, 8, 256, 2, 16, "bf16"), (17, 8, 256, 2, 16, "f32"), (9, 16, 384, 8, 32, "bf16"),
    (40, 4, 256, 3, 4, "bf16"), (5, 16, 256, 16, 16, "bf16"),
    # bf16 grids of 64 x 64 tiles (at least 256 of them), tap bounds 2, 4, 8
    (512, 8, 1024, 2, 8, "bf16"), (256, 16, 1024, 4, 8, "bf16"), (128, 16, 1024, 8, 32, "bf16"),
]


@pytest.mark.parametrize("nb,bs,H,T,gs,dtype", CONV_CASES)
def test_conv_prepare_and_finish(D, nb, bs, H, T, gs, dtype):
    log(f"conv nb={nb} bs={bs} H={H} T={T} gs={gs} {dtype}")
    w = wl(n_blocks=nb, block_size=bs, hidden=H, taps=T, group_size=gs, dtype=dtype)
    # a larger projection so the dynamic part is well above rounding noise
    inp = make_inputs(w, seed=3, fields=["h", "y", "base", "w_proj"])
    if dtype == "f32":
        inp["w_proj"] = inp["w_proj"] * np.float32(4.0)
    xo, kp = D.conv_prepare(to_dev(inp["h"]), to_dev(inp["w_proj"]), to_dev(inp["base"]), bs, T, gs)
    xo_r, kp_r, ex = O.conv_prepare(inp["h"], inp["w_proj"], inp["base"], bs, T, gs, dtype)
    c = O.conv_projection(inp["h"], inp["w_proj"], T, gs, dtype)
    A = corr_abs(inp["h"], inp["w_proj"], T, gs, dtype)
    # k_post, the output half of the same float32 projection, within the
    # ulps the x_out rule allows the input half
    assert close(to_np(kp), kp_r).all()
    if dtype == "bf16":
        okc = corr_ok(to_np(kp), kp_r, A[:, 1])
        assert okc.all(), f"k_post beyond the float32 bound at {np.argwhere(~okc)[:3]}"
    ok = act_ok(to_np(xo), ex, dtype, conv_delta(inp["h"], c[:, 0], inp["base"][0], bs, gs, dtype, A[:, 0]))
    assert ok.all(), f"{(~ok).sum()} x_out mismatches, first at {np.argwhere(~ok)[:3]}"
    # finish, fed the same float32 k_post on both sides: only the taps round
    kp32 = kp_r.astype(np.float32)
    yo = D.conv_finish(to_dev(inp["y"]), to_dev(kp32), to_dev(inp["base"]), bs, T, gs)
    _, ey = O.conv_finish(inp["y"], kp32, inp["base"], bs, T, gs, dtype)
    ok = act_ok(to_np(yo), ey, dtype, conv_delta(inp["y"], kp32, inp["base"][1], bs, gs, dtype))
    assert ok.all(), f"{(~ok).sum()} y_out mismatches"


@pytest.mark.parametrize("nb,bs", [(1, 8), (16, 8)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_identity_init_is_exact_on_device(D, nb, bs, dtype):
    H, T, gs = 256, 2, 16
    w = wl(n_blocks=nb, block_size=bs, hidden=H, taps=T, group_size=gs, dtype=dtype)
    inp = make_inputs(w, seed=4, fields=["h", "y"])
    f = torch.float32 if dtype == "f32" else torch.bfloat16
    base = torch.zeros((2, T, H), dtype=f, device="cuda")
    base[:, 0] = 1
    wp = torch.zeros((2 * T * (H // gs), H), dtype=f, device="cuda")
    x = to_dev(inp["h"])
    xo, kp = D.conv_prepare(x, wp, base, bs, T, gs)
    assert torch.equal(xo.float(), x.float()) and not kp.any()
    y = to_dev(inp["y"])
    assert torch.equal(D.conv_finish(y, kp, base, bs, T, gs).float(), y.float())


def test_conv_does_not_leak_across_blocks_on_device(D):
    nb, bs, H, T, gs = 6, 8, 256, 3, 16
    w = wl(n_blocks=nb, block_size=bs, hidden=H, taps=T, group_size=gs)
    inp = make_inputs(w, seed=5, fields=["h", "y", "base", "w_proj"])
    x, y, base, wp = (to_dev(inp[k]) for k in ("h", "y", "base", "w_proj"))
    xo, kp = D.conv_prepare(x, wp, base, bs, T, gs)
    yo = D.conv_finish(y, kp, base, bs, T, gs)
    for blk in range(1, nb):
        x2, y2 = x.clone(), y.clone()
        x2[: blk * bs] = 100 * torch.randn_like(x2[: blk * bs].float()).to(x2.dtype)
        y2[: blk * bs] = -100 * torch.randn_like(y2[: blk * bs].float()).to(y2.dtype)
        xo2, kp2 = D.conv_prepare(x2, wp, base, bs, T, gs)
        yo2 = D.conv_finish(y2, kp, base, bs, T, gs)
        sl = slice(blk * bs, None)
        assert torch.equal(xo2[sl], xo[sl]) and torch.equal(kp2[sl], kp[sl]) and torch.equal(yo2[sl], yo[sl])


# --------------------------------------------------------------- unary top-K

TOPK_CASES = [
    # (N, H, V, K, dtype): streaming for N <= 8, tiled above; ragged vocab tails
    (1, 256, 4133, 16, "bf16"), (8, 256, 4133, 16, "bf16"), (5, 512, 3001, 64, "bf16"),
    (8, 256, 4096, 1, "f32"), (3, 256, 2000, 16, "f32"), (8, 1024, 20000, 16, "bf16"),
    (9, 256, 3000, 16, "bf16"), (128, 256, 4096, 16, "f32"), (300, 256, 5000, 64, "bf16"),
    (130, 512, 2999, 7, "bf16"), (64, 256, 16, 16, "bf16"),
    # bf16, N <= 8, H a multiple of 512: weights streamed through LDS; several
    # ring turns per tile and several tiles per wave, ragged per-wave ranges
    (8, 4096, 30011, 16, "bf16"), (1, 4096, 5003, 64, "bf16"), (3, 2048, 70001, 5, "bf16"),
    # many rows whose 32 lists of 32 keys (1024) one wave merges in two chunks
    (1800, 256, 9000, 20, "bf16"),
    # many rows, lists of 32 and 64 keys over slabs of several tiles (the
    # scan's hits inserted into the lists between tiles)
    (300, 256, 70000, 64, "bf16"), (300, 256, 70000, 24, "bf16"),
    # many rows, an odd number of 64-deep k-tiles (5, 1, 3): the k loop's
    # last tile alone, with and without the weight-row touches
    (40, 320, 5003, 16, "bf16"), (300, 64, 4000, 16, "bf16"), (64, 192, 3001, 64, "bf16"),
]


@pytest.mark.parametrize("N,H,V,K,dtype", TOPK_CASES)
def test_unary_topk(D, N, H, V, K, dtype):
    log(f"topk N={N} H={H} V={V} K={K} {dtype}")
    w = wl(n_blocks=N, block_size=1, hidden=H, vocab=V, top_k=K, dtype=dtype)
    inp = make_inputs(w, seed=6, fields=["h", "w_lm", "gold"])
    ids, vals, gl = D.unary_topk(to_dev(inp["h"]), to_dev(inp["w_lm"]), K, gold_ids=to_dev(inp["gold"]))
    U = O.lm_logits(inp["h"], inp["w_lm"], dtype)
    fails, flags, msgs = compare_topk(to_np(ids), to_np(vals), U, K)
    log(f"  fails={fails} flags={flags}")
    assert fails == 0, msgs[:5]
    assert flags <= max(1, N // 50)
    assert close(to_np(gl), U[np.arange(N), inp["gold"]]).all()


TOPK_EX_CASES = [
    # (N, H, V, K, dtype, multiplier, softcap): every kernel regime (LDS-streamed
    # bf16 with K splits 4 / 2 / 1, register-streamed, 256 x 256 MFMA tiles
    # with lists of 8 / 16 / 64, float32 tiles), ragged vocabulary tails
    (8, 4096, 30011, 16, "bf16", 1.0, 30.0), (3, 1024, 20000, 16, "bf16", 1.7, 0.0),
    (5, 512, 5003, 64, "bf16", 0.8, 8.0), (8, 320, 4099, 8, "bf16", 1.0, 0.0), (5, 256, 7001, 16, "f32", 2.0, 3.0),
    (300, 256, 5000, 16, "bf16", 1.0, 30.0), (40, 512, 9001, 64, "bf16", 0.5, 0.0),
    (600, 256, 70001, 5, "bf16", 1.3, 4.0), (100, 256, 3001, 16, "f32", 1.0, 1.5),
    # K = V (every id a candidate); K = 1 under a tight cap
    (1, 256, 64, 64, "bf16", 1.0, 5.0), (9, 256, 100, 1, "f32", 2.0, 0.5),
]


@pytest.mark.parametrize("N,H,V,K,dtype,mult,cap", TOPK_EX_CASES)
def test_unary_topk_ex_transforms_and_metrics(D, N, H, V, K, dtype, mult, cap):
    log(f"topk_ex N={N} H={H} V={V} K={K} {dtype} mult={mult} cap={cap}")
    w = wl(n_blocks=N, block_size=1, hidden=H, vocab=V, top_k=K, dtype=dtype)
    inp = make_inputs(w, seed=8, fields=["h", "w_lm", "gold"])
    gold = inp["gold"].copy()
    U = O.lm_logits(inp["h"], inp["w_lm"], dtype)
    # a third of the golds are in the top K, so the hit flag takes both values
    gold[::3] = np.argmax(U[::3], axis=1)
    ids, vals, gl, lse, prob, hit = D.unary_topk_ex(to_dev(inp["h"]), to_dev(inp["w_lm"]), K, gold_ids=to_dev(gold),
                                                    output_multiplier=mult, softcap=cap, want_lse=True,
                                                    want_metrics=True)
    rids, rvals, rlse, rgl, rprob, rhit = O.unary_topk_ex(inp["h"], inp["w_lm"], K, dtype, gold_ids=gold,
                                                          output_multiplier=mult, softcap=cap)
    Ut = O.transform_logits(U, mult, cap)
    fails, flags, msgs = compare_topk(to_np(ids), to_np(vals), Ut, K)
    log(f"  fails={fails} flags={flags}")
    assert fails == 0, msgs[:5]
    assert close(to_np(gl), rgl).all()
    assert close(to_np(lse), rlse).all(), (to_np(lse)[:4], rlse[:4])
    assert close(to_np(prob), rprob, atol=1e-6).all()
    gi, gh = to_np(ids), to_np(hit)
    # the hit flag is the GPU's own candidate set; the oracle's agrees unless
    # that row's set was flagged as a boundary near-tie
    assert np.array_equal(gh, (gi == gold[:, None]).any(1).astype(np.uint8))
    assert 0 < gh.sum() < N or N < 3
    assert int((gh != rhit).sum()) <= flags
    # the plain call gives the same ids; with no transform, the same values
    if mult == 1.0 and cap == 0.0:
        ids0, vals0, _ = D.unary_topk(to_dev(inp["h"]), to_dev(inp["w_lm"]), K, gold_ids=to_dev(gold))
        assert torch.equal(ids0, ids) and torch.equal(vals0, vals)


@pytest.mark.parametrize("N", [8, 40])
def test_unary_topk_exact_ties_take_the_lower_id(D, N):
    H, V, K = 256, 1000, 16
    h = torch.randn(N, H, device="cuda").bfloat16()
    row = torch.randn(H, device="cuda").bfloat16()
    w = torch.randn(V, H, device="cuda").bfloat16() * 0.01
    tied = torch.tensor([977, 3, 500, 41, 42, 700, 5, 999], device="cuda")
    w[tied] = row
    h[:, :] = row  # every row's best direction is the tied one
    ids, vals, _ = D.unary_topk(h, w, K)
    want = torch.sort(tied).values.int()
    assert torch.equal(ids[:, :8], want.expand(N, 8))
    assert torch.equal(vals[:, :8], vals[:, :1].expand(N, 8))


@pytest.mark.parametrize("N,V,K", [(40, 6000, 8), (300, 6001, 16), (260, 5000, 64), (16, 777, 7)])
def test_unary_topk_rising_logits_take_every_fallback(D, N, V, K):
    """Weight rows whose norm grows with the id: every vocabulary tile beats
    the thresholds the earlier tiles set, so in the many-row kernel rows
    overflow their candidate slots on nearly every tile and the tiles are
    formed again and scanned exactly."""
    log(f"rising topk N={N} V={V} K={K}")
    H = 256
    w = wl(n_blocks=N, block_size=1, hidden=H, vocab=V, top_k=K)
    inp = make_inputs(w, seed=11, fields=["h", "gold"])
    rng = np.random.default_rng(11)
    scale = (1.0 + 3.0 * np.arange(V) / V).astype(np.float32)[:, None]
    w_lm = to_storage(torch.from_numpy((rng.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32) * scale), "bf16")
    ids, vals, gl = D.unary_topk(to_dev(inp["h"]), to_dev(w_lm), K, gold_ids=to_dev(inp["gold"]))
    U = O.lm_logits(inp["h"], w_lm, "bf16")
    fails, flags, msgs = compare_topk(to_np(ids), to_np(vals), U, K)
    log(f"  fails={fails} flags={flags}")
    assert fails == 0, msgs[:5]
    assert flags <= max(1, N // 50)
    assert close(to_np(gl), U[np.arange(N), inp["gold"]]).all()


@pytest.mark.parametrize("N,K", [(24, 16), (300, 8), (40, 64)])
def test_unary_topk_repeated_rows_tie_everywhere(D, N, K):
    """Five distinct weight rows repeated over the vocabulary: every tile
    holds exact ties at the thresholds, and the K best must be the lowest ids
    of the best value(s)."""
    H, V = 256, 3001
    w = wl(n_blocks=N, block_size=1, hidden=H, vocab=V, top_k=K)
    inp = make_inputs(w, seed=12, fields=["h", "w_lm"])
    w_lm = inp["w_lm"][np.arange(V) % 5].copy()
    ids, vals, _ = D.unary_topk(to_dev(inp["h"]), to_dev(w_lm), K)
    U = O.lm_logits(inp["h"], w_lm, "bf16")
    fails, flags, msgs = compare_topk(to_np(ids), to_np(vals), U, K)
    assert fails == 0, msgs[:5]
    # with only 5 distinct values per row the K best are fixed exactly (no
    # near-tie is possible between distinct values of this size)
    order = np.lexsort((np.broadcast_to(np.arange(V), U.shape), -U), axis=1)[:, :K]
    assert np.array_equal(to_np(ids), order.astype(np.int32))


def test_unary_topk_is_deterministic(D):
    w = wl(n_blocks=300, block_size=1, hidden=256, vocab=7000, top_k=16)
    inp = make_inputs(w, seed=8, fields=["h", "w_lm"])
    h, wl_ = to_dev(inp["h"]), to_dev(inp["w_lm"])
    a = D.unary_topk(h, wl_, 16)
    b = D.unary_topk(h, wl_, 16)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("N,H,V,K,dtype", [
    (300, 256, 7000, 16, "bf16"),   # many rows: 256 x 256 MFMA tiles
    (300, 256, 7000, 16, "f32"),    # many rows, float32 tiles
    (8, 512, 20011, 16, "bf16"),    # at most 8 rows, weights through LDS
    (5, 256, 5000, 64, "f32"),      # at most 8 rows, float32 register stream
    (300, 256, 70000, 64, "bf16"),  # many rows, 64-key lists: one slab of 274 tiles down to one tile per slab
])
def test_slab_count_does_not_change_the_lists(D, N, H, V, K, dtype):
    """The vocabulary split (the number of partial lists per row, forced by the
    debug knob) changes neither the ids nor the values; nor the fused decode
    head's lattice and path."""
    w = wl(n_blocks=1, block_size=N, hidden=H, vocab=V, top_k=K, rank=64, dtype=dtype)
    inp = make_inputs(w, seed=17, fields=["h", "w_lm", "w_h", "cb_pred", "cb_succ"])
    dev = {k: to_dev(v) for k, v in inp.items()}
    anchors = torch.tensor([3], dtype=torch.int32, device="cuda")
    fused = dtype == "bf16" and N <= 8

    def run():
        ids, vals, _ = D.unary_topk(dev["h"], dev["w_lm"], K)
        out = [ids, vals]
        if fused:
            out += list(D.decode_head(dev["h"], dev["w_lm"], K, dev["w_h"], dev["cb_pred"], dev["cb_succ"], anchors,
                                      N))
        torch.cuda.synchronize()
        return out

    ref = run()
    try:
        for n in (1, 3, 17, 255, 1024):
            D.debug_force_slabs(n)
            log(f"slabs {n}: workspace {D.workspace_bytes(D.OP_UNARY_TOPK, N, H, V, 0, K)} B")
            got = run()
            assert all(torch.equal(torch.nan_to_num(a, nan=0.0), torch.nan_to_num(b, nan=0.0))
                       for a, b in zip(got, ref)), f"slab count {n} changed the result"
    finally:
        D.debug_force_slabs(0)
    U = O.lm_logits(inp["h"], inp["w_lm"], dtype)
    fails, _, msgs = compare_topk(to_np(ref[0]), to_np(ref[1]), U, K)
    assert fails == 0, msgs


@pytest.mark.parametrize("N,K", [(8, 16), (5, 64), (1, 1)])
def test_reused_workspace_gives_identical_results(D, N, K):
    """A workspace reused call after call (any contents) gives the same result."""
    w = wl(n_blocks=1, block_size=N, hidden=512, vocab=20011, top_k=K, rank=64)
    inp = make_inputs(w, seed=9)
    dev = {k: to_dev(v) for k, v in inp.items()}
    ws = D.make_workspace(D.OP_UNARY_TOPK, N, 512, 20011, 0, K, "cuda").fill_(0xA5)
    wsw = D.make_workspace(D.OP_SELECTOR_WALK, N, 512, 20011, 64, K, "cuda").fill_(0x5A)
    ref = None
    for _ in range(4):
        ids, vals, _ = D.unary_topk(dev["h"], dev["w_lm"], K, workspace=ws)
        path, ps = D.selector_walk(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals,
                                   dev["anchors"], N, workspace=wsw)
        out = (ids.clone(), vals.clone(), path.clone(), ps.clone())
        if ref is None:
            ref = out
        assert all(torch.equal(a, b) for a, b in zip(out, ref))
    U = O.lm_logits(inp["h"], inp["w_lm"], "bf16")
    fails, _, msgs = compare_topk(to_np(ref[0]), to_np(ref[1]), U, K)
    assert fails == 0, msgs


# ------------------------------------------------------------------ selector

def rand_cands(rng, N, V, K):
    ids = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
    vals = (-np.sort(-rng.standard_normal((N, K)), axis=1)).astype(np.float32)
    return ids, vals


WALK_CASES = [
    # (n_blocks, bs, H, V, r, K, dtype)
    (1, 8, 256, 1000, 32, 16, "f32"), (3, 8, 256, 1000, 256, 16, "bf16"), (16, 8, 256, 4096, 32, 16, "f32"),
    (5, 16, 256, 3000, 40, 20, "bf16"), (4, 16, 512, 5000, 512, 64, "bf16"), (7, 2, 256, 500, 64, 1, "bf16"),
    (2, 3, 256, 800, 256, 33, "bf16"), (64, 8, 256, 2000, 256, 16, "bf16"),
    # 128 blocks or more (bf16): the walk that follows one pick at a time, with
    # padded LDS rows (r a multiple of 512) and packed ones, ragged K
    (128, 8, 256, 3000, 512, 20, "bf16"), (130, 4, 256, 2000, 40, 64, "bf16"), (200, 2, 256, 500, 256, 1, "bf16"),
    (129, 16, 256, 4000, 1024, 33, "bf16"),
]


@pytest.mark.parametrize("nb,bs,H,V,r,K,dtype", WALK_CASES)
def test_selector_walk_and_tf(D, nb, bs, H, V, r, K, dtype):
    log(f"walk nb={nb} bs={bs} H={H} V={V} r={r} K={K} {dtype}")
    w = wl(n_blocks=nb, block_size=bs, hidden=H, vocab=V, rank=r, top_k=K, dtype=dtype)
    inp = make_inputs(w, seed=9, fields=["h", "w_h", "cb_pred", "cb_succ", "anchors", "pred", "gold", "force"])
    scale_codebooks(inp, r, dtype)
    rng = np.random.default_rng(nb * 1000 + K)
    N = nb * bs
    ids, vals = rand_cands(rng, N, V, K)
    dev = {k: to_dev(v) for k, v in inp.items()}
    path, ps = D.selector_walk(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids), to_dev(vals),
                               dev["anchors"], bs)
    g64 = O.context_projection(inp["h"], inp["w_h"], dtype)
    u64 = vals.astype(np.float64)
    fails, flags, teeth, msgs = compare_walk(to_np(path), to_np(ps), g64, inp["cb_pred"], inp["cb_succ"], ids, u64,
                                             inp["anchors"], bs, dtype)
    log(f"  walk fails={fails} flags={flags} teeth={teeth}/{nb * (bs - 1)}")
    assert fails == 0, msgs[:5]
    # one candidate leaves nothing to override; otherwise the pair term must
    # have overridden the unary pick somewhere
    assert teeth == 0 if K == 1 else teeth > 0
    if flags == 0:
        ref_path, _ = O.selector_walk(g64, inp["cb_pred"], inp["cb_succ"], ids, u64, inp["anchors"], bs, dtype)
        assert np.array_equal(to_np(path), ref_path)
    # teacher forcing with random predecessors, gold ids and forcing
    gold = inp["gold"].copy()
    gold[::3] = ids[::3, K // 2]  # a third of the rows have the gold in the set
    glog = rng.standard_normal(N).astype(np.float32)
    gpu = D.selector_score_tf(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids), to_dev(vals),
                              dev["pred"], gold_ids=to_dev(gold), force=dev["force"], gold_logit=to_dev(glog))
    ref = O.selector_score_tf(g64, inp["cb_pred"], inp["cb_succ"], ids, u64, inp["pred"], dtype, gold_ids=gold,
                              force=inp["force"], gold_logit=glog.astype(np.float64))
    fails, flags, msgs = compare_tf(tuple(to_np(t) for t in gpu), ref, ids)
    log(f"  tf fails={fails} flags={flags}")
    assert fails == 0, msgs[:5]
    # replay: the walk's own predecessors through teacher forcing give the walk
    pred = np.zeros(N, np.int32)
    P = to_np(path)
    for b in range(nb):
        pred[b * bs + 1:(b + 1) * bs] = P[b, :-1]
    pred[::bs] = inp["anchors"]  # position 0 is not scored by the walk
    sc, best, _, _ = D.selector_score_tf(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids),
                                         to_dev(vals), to_dev(pred))
    best, sc = to_np(best).reshape(nb, bs), to_np(sc).reshape(nb, bs, K)
    assert np.array_equal(best[:, 1:], P[:, 1:])
    assert np.array_equal(sc.max(axis=2)[:, 1:], to_np(ps)[:, 1:])  # bit-exact replay


SAMPLE_CASES = [
    # (n_blocks, bs, H, V, r, K, dtype, temperature)
    (3, 8, 256, 1000, 256, 16, "bf16", 1.0), (16, 8, 256, 4096, 32, 16, "f32", 0.5),
    (4, 16, 512, 5000, 512, 64, "bf16", 2.0), (2, 3, 256, 800, 256, 33, "bf16", 1.0),
    (64, 8, 256, 2000, 256, 16, "bf16", 1.0),
]


@pytest.mark.parametrize("nb,bs,H,V,r,K,dtype,temp", SAMPLE_CASES)
def test_selector_sample(D, nb, bs, H, V, r, K, dtype, temp):
    log(f"sample nb={nb} bs={bs} H={H} V={V} r={r} K={K} {dtype} T={temp}")
    w = wl(n_blocks=nb, block_size=bs, hidden=H, vocab=V, rank=r, top_k=K, dtype=dtype)
    inp = make_inputs(w, seed=19, fields=["h", "w_h", "cb_pred", "cb_succ", "anchors"])
    if dtype == "f32":
        inp["cb_pred"] *= np.float32(6)
        inp["cb_succ"] *= np.float32(6)
    rng = np.random.default_rng(nb * 1000 + K + 7)
    ids, vals = rand_cands(rng, nb * bs, V, K)
    dev = {k: to_dev(v) for k, v in inp.items()}
    seed = 0x9E3779B97F4A7C15 ^ (nb * 131 + K)
    path, ps = D.selector_sample(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids), to_dev(vals),
                                 dev["anchors"], bs, temperature=temp, seed=seed)
    g64 = O.context_projection(inp["h"], inp["w_h"], dtype)
    u64 = vals.astype(np.float64)
    fails, flags, msgs = compare_sample(to_np(path), to_np(ps), g64, inp["cb_pred"], inp["cb_succ"], ids, u64,
                                        inp["anchors"], bs, dtype, temp, seed)
    log(f"  sample fails={fails} flags={flags}")
    assert fails == 0, msgs[:5]
    if flags == 0:
        ref, _ = O.selector_sample(g64, inp["cb_pred"], inp["cb_succ"], ids, u64, inp["anchors"], bs, dtype, temp,
                                   seed)
        assert np.array_equal(to_np(path), ref)
    # the same seed draws the same path; another seed another one
    path2, _ = D.selector_sample(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids), to_dev(vals),
                                 dev["anchors"], bs, temperature=temp, seed=seed)
    assert torch.equal(path, path2)
    if nb * (bs - 1) >= 16:
        path3, _ = D.selector_sample(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids),
                                     to_dev(vals), dev["anchors"], bs, temperature=temp, seed=seed + 1)
        assert not torch.equal(path, path3)


def test_sampling_at_vanishing_temperature_follows_the_greedy_walk(D):
    nb, bs, H, V, r, K = 32, 8, 256, 2000, 256, 16
    w = wl(n_blocks=nb, block_size=bs, hidden=H, vocab=V, rank=r, top_k=K)
    inp = make_inputs(w, seed=21, fields=["h", "w_h", "cb_pred", "cb_succ", "anchors"])
    rng = np.random.default_rng(5)
    ids, vals = rand_cands(rng, nb * bs, V, K)
    args = [to_dev(inp[k]) for k in ("h", "w_h", "cb_pred", "cb_succ")] + [to_dev(ids), to_dev(vals),
                                                                           to_dev(inp["anchors"]), bs]
    gp, gps = D.selector_walk(*args)
    sp, sps = D.selector_sample(*args, temperature=1e-6, seed=3)
    same = (to_np(gp) == to_np(sp)).all(axis=1)
    # a block may part only where two of the greedy scores lie within the noise's reach
    assert same.mean() > 0.9, same.mean()
    assert np.array_equal(to_np(gps)[same], to_np(sps)[same])


def test_gpu_draws_follow_the_softmax_of_the_scores(D):
    # Zero successor codebook: every position scores the same three unary
    # values log(1, 2, 5); each (block, position) is one draw.
    nb, bs, H, V, r, K = 2048, 8, 256, 64, 32, 3
    w = wl(n_blocks=nb, block_size=bs, hidden=H, vocab=V, rank=r, top_k=K)
    inp = make_inputs(w, seed=22, fields=["h", "w_h", "cb_pred", "anchors"])
    N = nb * bs
    ids = np.tile(np.array([5, 9, 17], np.int32), (N, 1))
    vals = np.tile(np.log([1.0, 2.0, 5.0]).astype(np.float32), (N, 1))
    zero_b = torch.zeros((V, r), dtype=torch.bfloat16, device="cuda")
    for temp, p in ((1.0, np.array([1, 2, 5]) / 8), (2.0, np.sqrt([1, 2, 5]) / np.sqrt([1, 2, 5]).sum())):
        path, _ = D.selector_sample(to_dev(inp["h"]), to_dev(inp["w_h"]), to_dev(inp["cb_pred"]), zero_b,
                                    to_dev(ids), to_dev(vals), to_dev(inp["anchors"]), bs, temperature=temp,
                                    seed=11)
        picks = to_np(path)[:, 1:].ravel()
        freq = np.array([(picks == i).mean() for i in (5, 9, 17)])
        sd = np.sqrt(p * (1 - p) / picks.size)
        log(f"  T={temp} freq={freq} want={p}")
        assert np.all(np.abs(freq - p) < 4 * sd), (temp, freq, p)


def test_zero_successor_codebook_walks_the_unary_argmax(D):
    nb, bs, H, V, r, K = 8, 8, 256, 1000, 64, 16
    w = wl(n_blocks=nb, block_size=bs, hidden=H, vocab=V, rank=r, top_k=K)
    inp = make_inputs(w, seed=10, fields=["h", "w_h", "cb_pred", "anchors"])
    rng = np.random.default_rng(1)
    ids, vals = rand_cands(rng, nb * bs, V, K)
    zero_b = torch.zeros((V, r), dtype=torch.bfloat16, device="cuda")
    path, ps = D.selector_walk(to_dev(inp["h"]), to_dev(inp["w_h"]), to_dev(inp["cb_pred"]), zero_b, to_dev(ids),
                               to_dev(vals), to_dev(inp["anchors"]), bs)
    P = to_np(path)
    assert np.array_equal(P[:, 1:], ids.reshape(nb, bs, K)[:, 1:, 0])
    assert np.array_equal(to_np(ps)[:, 1:], vals.reshape(nb, bs, K)[:, 1:, 0])


def test_out_of_range_ids_are_flagged_not_read(D):
    nb, bs, H, V, r, K = 4, 8, 256, 1000, 32, 16
    w = wl(n_blocks=nb, block_size=bs, hidden=H, vocab=V, rank=r, top_k=K)
    inp = make_inputs(w, seed=11, fields=["h", "w_h", "cb_pred", "cb_succ", "anchors", "w_lm"])
    rng = np.random.default_rng(2)
    ids, vals = rand_cands(rng, nb * bs, V, K)
    dev = {k: to_dev(v) for k, v in inp.items()}
    ws = D.make_workspace(D.OP_SELECTOR_WALK, nb * bs, H, V, r, K, "cuda")
    anchors = inp["anchors"].copy()
    anchors[1] = V + 5
    anchors[2] = -1
    path, ps = D.selector_walk(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids), to_dev(vals),
                               to_dev(anchors), bs, workspace=ws)
    assert D.read_device_status(ws) == 8
    P = to_np(path)
    assert np.all(P[1] == -1) and np.all(P[2] == -1) and np.all(P[0] >= 0) and np.all(P[3] >= 0)
    # a clean call on the same workspace clears the word
    D.selector_walk(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids), to_dev(vals),
                    dev["anchors"], bs, workspace=ws)
    assert D.read_device_status(ws) == 0
    # gold ids out of range in the LM head
    ws2 = D.make_workspace(D.OP_UNARY_TOPK, nb * bs, H, V, 0, K, "cuda")
    gold = np.arange(nb * bs, dtype=np.int32)
    gold[3] = V
    _, _, gl = D.unary_topk(dev["h"], dev["w_lm"], K, gold_ids=to_dev(gold), workspace=ws2)
    assert D.read_device_status(ws2) == 8 and torch.isnan(gl[3]) and not torch.isnan(gl[4])
    # predecessor out of range in teacher forcing
    ws3 = D.make_workspace(D.OP_SELECTOR_TF, nb * bs, H, V, r, K, "cuda")
    pred = np.zeros(nb * bs, np.int32)
    pred[5] = -7
    _, best, _, _ = D.selector_score_tf(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids),
                                        to_dev(vals), to_dev(pred), workspace=ws3)
    assert D.read_device_status(ws3) == 8 and int(best[5]) == -1 and int(best[4]) >= 0



@pytest.mark.parametrize("nb,bs,r,K", [(160, 8, 512, 16), (140, 6, 96, 24), (130, 16, 512, 64), (130, 8, 264, 40)])
def test_chased_walk_equals_pair_walk(D, nb, bs, r, K):
    """With 128 blocks or more (bf16) the walk follows one pick at a time;
    below that every adjacent pair is scored.  The first 127 blocks, walked
    alone, take the pair walk: both must give the same paths and bit-equal
    scores, also with candidate and anchor ids out of range."""
    H, V = 256, 2500
    log(f"chase vs pair nb={nb} bs={bs} r={r} K={K}")
    w = wl(n_blocks=nb, block_size=bs, hidden=H, vocab=V, rank=r, top_k=K, dtype="bf16")
    inp = make_inputs(w, seed=21, fields=["h", "w_h", "cb_pred", "cb_succ", "anchors"])
    rng = np.random.default_rng(nb + K)
    N = nb * bs
    ids, vals = rand_cands(rng, N, V, K)
    ids[bs + 2, 3] = V + 1  # invalid candidates in block 1 and the last block
    ids[(nb - 1) * bs + 1, 0] = -4
    anchors = inp["anchors"].copy()
    anchors[5] = -2
    dev = {k: to_dev(v) for k, v in inp.items()}
    outs = []
    for m in (nb, 127):
        ws = D.make_workspace(D.OP_SELECTOR_WALK, m * bs, H, V, r, K, "cuda")
        path, ps = D.selector_walk(dev["h"][:m * bs], dev["w_h"], dev["cb_pred"], dev["cb_succ"],
                                   to_dev(ids[:m * bs]), to_dev(vals[:m * bs]), to_dev(anchors[:m]), bs, workspace=ws)
        assert D.read_device_status(ws) == 8
        outs.append((to_np(path), to_np(ps)))
    (p_all, s_all), (p_pair, s_pair) = outs
    assert np.all(p_all[5] == -1) and np.all(np.isnan(s_all[5, 1:]))
    assert np.array_equal(p_all[:127], p_pair)
    assert np.array_equal(s_all[:127].view(np.uint32), s_pair.view(np.uint32))

# -------------------------------------------------------- selector CE backward

CE_BWD_CASES = [
    # (N, H, V, r, K, dtype): ragged rows, rank and vocab; ids shared by many rows
    (128, 256, 4096, 32, 16, "f32"), (200, 256, 1000, 256, 16, "bf16"), (333, 512, 3000, 40, 20, "bf16"),
    (64, 256, 500, 512, 64, "bf16"), (37, 256, 800, 264, 33, "f32"), (24, 256, 300, 8, 1, "bf16"),
    (1, 256, 100, 16, 5, "bf16"), (1000, 320, 2000, 256, 16, "bf16"),
    # the rank limit; every vocabulary id a candidate of every row
    (16, 256, 500, 4096, 8, "bf16"), (9, 256, 64, 8, 64, "f32"),
    # a vocabulary whose 2V + 1 counters span more than 1024 scan tiles
    (50, 256, 2_200_000, 8, 4, "bf16"),
    # a 50-token vocabulary: every id is a candidate of ~64 rows, so many
    # codebook rows gather more than one 64-entry chunk (chunks add atomically)
    (200, 256, 50, 32, 16, "bf16"),
]


def ce_bwd_inputs(N, H, V, r, K, dtype, seed):
    w = wl(n_blocks=N, block_size=1, hidden=H, vocab=V, rank=r, top_k=K, dtype=dtype)
    inp = make_inputs(w, seed=seed, fields=["h", "w_h", "cb_pred", "cb_succ", "pred", "gold", "force"])
    if dtype == "f32":
        inp["cb_pred"] *= np.float32(6)
        inp["cb_succ"] *= np.float32(6)
    rng = np.random.default_rng(seed + N)
    ids, vals = rand_cands(rng, N, V, K)
    gold = inp["gold"].copy()
    gold[::3] = ids[::3, K // 2]
    glog = rng.standard_normal(N).astype(np.float32)
    wgt = (rng.random(N) + 0.5).astype(np.float32)
    return inp, ids, vals, gold, glog, wgt


@pytest.mark.parametrize("N,H,V,r,K,dtype", CE_BWD_CASES)
def test_selector_ce_backward(D, N, H, V, r, K, dtype):
    log(f"ce backward N={N} H={H} V={V} r={r} K={K} {dtype}")
    inp, ids, vals, gold, glog, wgt = ce_bwd_inputs(N, H, V, r, K, dtype, seed=17)
    dev = {k: to_dev(v) for k, v in inp.items()}
    # the gradients are added into what the buffers hold
    rng = np.random.default_rng(5)
    pre = [(rng.standard_normal(s) * 1e-3).astype(np.float32) for s in ((V, r), (V, r), (r, H))]
    gp, gs, gw, ce, valid = D.selector_ce_backward(
        dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids), to_dev(vals), dev["pred"], to_dev(gold),
        to_dev(wgt), force=dev["force"], gold_logit=to_dev(glog), grad_pred=to_dev(pre[0]), grad_succ=to_dev(pre[1]),
        grad_wh=to_dev(pre[2]))
    dA, dB, dW, _, rvalid = O.selector_ce_backward(inp["h"], inp["w_h"], inp["cb_pred"], inp["cb_succ"], ids,
                                                   vals.astype(np.float64), inp["pred"], dtype, gold, inp["force"],
                                                   glog.astype(np.float64), wgt.astype(np.float64))
    got = {"dA": to_np(gp) - pre[0], "dB": to_np(gs) - pre[1], "dW": to_np(gw) - pre[2]}
    fails, msgs = compare_grads(got, {"dA": dA, "dB": dB, "dW": dW})
    assert np.array_equal(to_np(valid), rvalid)
    g64 = O.context_projection(inp["h"], inp["w_h"], dtype)
    _, _, rce, _ = O.selector_score_tf(g64, inp["cb_pred"], inp["cb_succ"], ids, vals.astype(np.float64),
                                       inp["pred"], dtype, gold_ids=gold, force=inp["force"],
                                       gold_logit=glog.astype(np.float64))
    assert close(to_np(ce), rce).all()
    log(f"  valid {int(rvalid.sum())}/{N} fails={fails}")
    assert fails == 0, msgs
    if K > 1 and rvalid.any():
        assert np.abs(dB).max() > 0 and np.abs(dW).max() > 0


def test_selector_ce_backward_with_every_row_excluded_adds_nothing(D):
    # no gold among the candidates and nothing forced: no CE, no gradient
    N, H, V, r, K = 40, 256, 600, 32, 8
    inp, ids, vals, _, glog, wgt = ce_bwd_inputs(N, H, V, r, K, "bf16", seed=29)
    gold = np.full(N, V - 1, np.int32)
    ids = ids % (V - 1)
    dev = {k: to_dev(v) for k, v in inp.items()}
    pre = [torch.full(sh, 0.25, dtype=torch.float32, device="cuda") for sh in ((V, r), (V, r), (r, H))]
    gp, gs, gw, ce, valid = D.selector_ce_backward(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids),
                                                   to_dev(vals), dev["pred"], to_dev(gold), to_dev(wgt),
                                                   grad_pred=pre[0], grad_succ=pre[1], grad_wh=pre[2])
    assert not to_np(valid).any() and not to_np(ce).any()
    assert all(bool((t == 0.25).all()) for t in (gp, gs, gw))


def test_selector_ce_backward_accumulates_and_skips_bad_rows(D):
    N, H, V, r, K = 96, 256, 700, 64, 8
    inp, ids, vals, gold, glog, wgt = ce_bwd_inputs(N, H, V, r, K, "bf16", seed=23)
    dev = {k: to_dev(v) for k, v in inp.items()}
    ws = D.make_workspace(D.OP_SELECTOR_CE_BACKWARD, N, H, V, r, K, "cuda")
    pred = inp["pred"].copy()
    pred[7] = V  # out of range: that row is excluded and flagged
    args = (dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], to_dev(ids), to_dev(vals), to_dev(pred),
            to_dev(gold), to_dev(wgt))
    gp, gs, gw, ce, valid = D.selector_ce_backward(*args, force=dev["force"], gold_logit=to_dev(glog), workspace=ws)
    assert D.read_device_status(ws) == 8 and int(valid[7]) == 0 and float(ce[7]) == 0.0
    # a second call adds the same gradient again
    D.selector_ce_backward(*args, force=dev["force"], gold_logit=to_dev(glog), grad_pred=gp, grad_succ=gs,
                           grad_wh=gw, want_ce=False, workspace=ws)
    pred_ok = pred.copy()
    pred_ok[7] = 0
    wz = wgt.copy()
    wz[7] = 0  # the excluded row carries no weight
    dA, dB, dW, _, rvalid = O.selector_ce_backward(inp["h"], inp["w_h"], inp["cb_pred"], inp["cb_succ"], ids,
                                                   vals.astype(np.float64), pred_ok, "bf16", gold, inp["force"],
                                                   glog.astype(np.float64), wz.astype(np.float64))
    fails, msgs = compare_grads({"dA": to_np(gp), "dB": to_np(gs), "dW": to_np(gw)},
                                {"dA": 2 * dA, "dB": 2 * dB, "dW": 2 * dW})
    assert fails == 0, msgs
    # no force given: rows whose gold is outside the set are excluded
    _, _, _, _, v2 = D.selector_ce_backward(*args[:6], dev["pred"], to_dev(gold), to_dev(wgt))
    assert np.array_equal(to_np(v2), np.isin(np.arange(N), np.flatnonzero((ids == gold[:, None]).any(1))))


# -------------------------------------------------------------- end to end

def test_tiny_fp32_workload_end_to_end(D):
    """16 blocks x 8, H 256, V 4096, fp32: the conv wrapper around an identity
    sublayer, LM head -> walk, the walk's own path replayed through teacher
    forcing, teacher forcing with gold ids, and the oracle's own pipeline (its
    top-K into its walk) against the GPU's, block by block."""
    from block_draft_head_amd.inputs import WORKLOADS
    w = WORKLOADS["tiny_fp32_16x8_h256_v4096"]
    inp = make_inputs(w)
    dev = {k: to_dev(v) for k, v in inp.items()}
    bs, T, gs, K, nb = w.block_size, w.taps, w.group_size, w.top_k, w.n_blocks
    N = nb * bs
    xo, kp = D.conv_prepare(dev["h"], dev["w_proj"], dev["base"], bs, T, gs)
    yo = D.conv_finish(xo, kp, dev["base"], bs, T, gs)
    _, kp_r, ex = O.conv_prepare(inp["h"], inp["w_proj"], inp["base"], bs, T, gs, "f32")
    assert act_ok(to_np(xo), ex, "f32").all() and close(to_np(kp), kp_r).all()
    _, ey = O.conv_finish(to_np(xo), to_np(kp), inp["base"], bs, T, gs, "f32")
    assert act_ok(to_np(yo), ey, "f32").all()
    # the whole wrapper against the oracle's, each side on its own data
    _, ey_all = O.conv_finish(ex.astype(np.float32), kp_r.astype(np.float32), inp["base"], bs, T, gs, "f32")
    assert act_ok(to_np(yo), ey_all, "f32").all()
    ids, vals, gl = D.unary_topk(dev["h"], dev["w_lm"], K, gold_ids=dev["gold"])
    U = O.lm_logits(inp["h"], inp["w_lm"], "f32")
    fails, flags, msgs = compare_topk(to_np(ids), to_np(vals), U, K)
    assert fails == 0, msgs[:5]
    gids = to_np(ids)
    u64 = U[np.arange(U.shape[0])[:, None], gids]
    g64 = O.context_projection(inp["h"], inp["w_h"], "f32")
    path, ps = D.selector_walk(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals, dev["anchors"], bs)
    P = to_np(path)
    fails, flags, teeth, msgs = compare_walk(P, to_np(ps), g64, inp["cb_pred"], inp["cb_succ"], gids, u64,
                                             inp["anchors"], bs, "f32")
    log(f"tiny walk fails={fails} flags={flags} teeth={teeth}")
    assert fails == 0, msgs[:5]
    assert teeth > 0
    # the walk's own predecessors through teacher forcing give the walk back
    pred = np.zeros(N, np.int32)
    for b in range(nb):
        pred[b * bs + 1:(b + 1) * bs] = P[b, :-1]
    pred[::bs] = inp["anchors"]
    sc, best, _, _ = D.selector_score_tf(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals,
                                         to_dev(pred))
    best, sc = to_np(best).reshape(nb, bs), to_np(sc).reshape(nb, bs, K)
    assert np.array_equal(best[:, 1:], P[:, 1:])
    assert np.array_equal(sc.max(axis=2)[:, 1:], to_np(ps)[:, 1:])
    # teacher forcing with gold ids and forcing
    gpu = D.selector_score_tf(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals, dev["pred"],
                              gold_ids=dev["gold"], force=dev["force"], gold_logit=gl)
    ref = O.selector_score_tf(g64, inp["cb_pred"], inp["cb_succ"], gids, u64, inp["pred"], "f32",
                              gold_ids=inp["gold"], force=inp["force"], gold_logit=U[np.arange(U.shape[0]), inp["gold"]])
    fails, flags, msgs = compare_tf(tuple(to_np(t) for t in gpu), ref, gids)
    assert fails == 0, msgs[:5]
    # end to end: the oracle's own top-K into its own walk.  A block may differ
    # from the GPU's only where the stage-wise comparison flagged a near-tie
    # in it (a top-K boundary or a selector argmax within the tie margin).
    o_ids, o_vals = O.topk_of(U, K)
    o_path, _ = O.selector_walk(g64, inp["cb_pred"], inp["cb_succ"], o_ids, o_vals, inp["anchors"], bs, "f32")
    same = tied = 0
    for b in range(nb):
        if np.array_equal(P[b], o_path[b]):
            same += 1
            continue
        rows = slice(b * bs, (b + 1) * bs)
        _, tf, _ = compare_topk(gids[rows], to_np(vals)[rows], U[rows], K)
        _, wf, _, _ = compare_walk(P, None, g64, inp["cb_pred"], inp["cb_succ"], gids, u64, inp["anchors"], bs, "f32",
                                   blocks=[b])
        assert tf + wf > 0, f"block {b}: GPU path {P[b]} vs oracle {o_path[b]} with no flagged tie"
        tied += 1
    log(f"end to end: {same} of {nb} blocks identical, {tied} differ through flagged ties")
    assert same + tied == nb and same >= nb - 2
