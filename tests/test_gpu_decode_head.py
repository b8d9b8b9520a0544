"""GPU parity of the fused decode head (dflash2_decode_head): the lattice
against the plain unary top-K (same kernel tiles, so bit-equal) and against
the oracle, the walk against the oracle fed the GPU's lattice, repeated calls
on one workspace, and the lattice-only form."""
import numpy as np
import pytest
import torch

from block_draft_head_amd.inputs import Workload, make_inputs
from oracle import dflash2_oracle as O
from tests.helpers import compare_topk, compare_walk, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    from block_draft_head_amd import dflash2
    assert torch.cuda.is_available(), "no GPU visible"
    return dflash2


def log(msg):
    print(msg, flush=True)


def inputs(nb, bs, H, V, r, K, seed, cb_scale):
    w = Workload("dh", nb, bs, H, V, "bf16", 2, 16, r, K, "walk")
    inp = make_inputs(w, seed=seed, fields=["h", "w_lm", "w_h", "cb_pred", "cb_succ", "anchors"])
    if cb_scale != 1:
        # larger codebooks: the pair term overrides the unary pick on a share of the steps
        for k in ("cb_pred", "cb_succ"):
            inp[k] = O.round_bf16(O.widen(inp[k], "bf16") * cb_scale)
    return inp


CASES = [
    # (n_blocks, bs, H, V, r, K, codebook scale): ragged vocabularies and
    # ranks (a partial last tile of 16 rows), every K split, 1-4 successor tiles
    (1, 8, 512, 4096, 32, 16, 6), (1, 8, 4096, 20000, 256, 16, 6), (2, 4, 1024, 5001, 64, 20, 6),
    (1, 8, 512, 3001, 256, 64, 4), (8, 1, 512, 1000, 16, 5, 1), (1, 5, 2048, 777, 40, 7, 6),
    (1, 8, 1536, 9999, 520, 33, 6), (4, 2, 512, 300, 8, 1, 1),
]


@pytest.mark.parametrize("nb,bs,H,V,r,K,cs", CASES)
def test_decode_head_matches_topk_and_oracle(D, nb, bs, H, V, r, K, cs):
    log(f"decode head nb={nb} bs={bs} H={H} V={V} r={r} K={K} cb x{cs}")
    inp = inputs(nb, bs, H, V, r, K, 5, cs)
    dev = {k: to_dev(v) for k, v in inp.items()}
    ws = D.make_workspace(D.OP_DECODE_HEAD, nb * bs, H, V, r, K, "cuda")
    ids, vals, path, ps = D.decode_head(dev["h"], dev["w_lm"], K, dev["w_h"], dev["cb_pred"], dev["cb_succ"],
                                        dev["anchors"], bs, workspace=ws)
    ref_ids, ref_vals, _ = D.unary_topk(dev["h"], dev["w_lm"], K)
    torch.cuda.synchronize()
    assert torch.equal(ids, ref_ids) and torch.equal(vals, ref_vals)
    assert D.read_device_status(ws) == 0
    U = O.lm_logits(inp["h"], inp["w_lm"], "bf16")
    fails, _, msgs = compare_topk(to_np(ids), to_np(vals), U, K)
    assert fails == 0, msgs
    gids = to_np(ids)
    u64 = U[np.arange(U.shape[0])[:, None], gids]
    g64 = O.context_projection(inp["h"], inp["w_h"], "bf16")
    fails, flags, teeth, msgs = compare_walk(to_np(path), to_np(ps), g64, inp["cb_pred"], inp["cb_succ"], gids, u64,
                                             inp["anchors"], bs, "bf16")
    log(f"  walk flags={flags} teeth={teeth}")
    assert fails == 0, msgs
    # the same call again on the same workspace, and the lattice alone
    ids2, vals2, path2, ps2 = D.decode_head(dev["h"], dev["w_lm"], K, dev["w_h"], dev["cb_pred"], dev["cb_succ"],
                                            dev["anchors"], bs, workspace=ws)
    ids3, vals3, p3, _ = D.decode_head(dev["h"], dev["w_lm"], K, workspace=ws)
    torch.cuda.synchronize()
    assert p3 is None
    assert torch.equal(ids2, ids) and torch.equal(vals2, vals) and torch.equal(path2, path)
    assert torch.equal(torch.nan_to_num(ps2, nan=0.0), torch.nan_to_num(ps, nan=0.0))
    assert torch.equal(ids3, ids) and torch.equal(vals3, vals)


def test_decode_head_teeth_at_decode_shape(D):
    # one block of 8 at H 4096, r 256 with codebooks scaled so the pair term
    # competes with the unary gaps: the selector must override some picks
    nb, bs, H, V, r, K = 1, 8, 4096, 20000, 256, 16
    total = 0
    for seed in range(3):
        inp = inputs(nb, bs, H, V, r, K, 11 + seed, 12)
        dev = {k: to_dev(v) for k, v in inp.items()}
        ids, vals, path, ps = D.decode_head(dev["h"], dev["w_lm"], K, dev["w_h"], dev["cb_pred"], dev["cb_succ"],
                                            dev["anchors"], bs)
        U = O.lm_logits(inp["h"], inp["w_lm"], "bf16")
        gids = to_np(ids)
        u64 = U[np.arange(U.shape[0])[:, None], gids]
        g64 = O.context_projection(inp["h"], inp["w_h"], "bf16")
        fails, flags, teeth, msgs = compare_walk(to_np(path), to_np(ps), g64, inp["cb_pred"], inp["cb_succ"], gids,
                                                 u64, inp["anchors"], bs, "bf16")
        assert fails == 0, msgs
        total += teeth
    log(f"teeth over 3 decode blocks: {total} of 21 steps")
    assert total > 0


def test_decode_head_flags_an_out_of_range_anchor(D):
    nb, bs, H, V, r, K = 1, 8, 512, 2000, 32, 8
    inp = inputs(nb, bs, H, V, r, K, 3, 1)
    dev = {k: to_dev(v) for k, v in inp.items()}
    ws = D.make_workspace(D.OP_DECODE_HEAD, nb * bs, H, V, r, K, "cuda")
    bad = torch.tensor([V + 3], dtype=torch.int32, device="cuda")
    ids, vals, path, ps = D.decode_head(dev["h"], dev["w_lm"], K, dev["w_h"], dev["cb_pred"], dev["cb_succ"], bad,
                                        bs, workspace=ws)
    assert D.read_device_status(ws) == 8
    assert (path == -1).all()
    ref_ids, _, _ = D.unary_topk(dev["h"], dev["w_lm"], K)
    assert torch.equal(ids, ref_ids)
    # the next call on the same workspace is clean again
    D.decode_head(dev["h"], dev["w_lm"], K, dev["w_h"], dev["cb_pred"], dev["cb_succ"], dev["anchors"], bs,
                  workspace=ws)
    assert D.read_device_status(ws) == 0


@pytest.mark.parametrize("kind,K", [("clustered", 16), ("clustered", 4), ("clustered", 6), ("tied", 16),
                                    ("one_list", 16)])
def test_decode_head_merge_fallbacks(D, kind, K):
    # lattices that defeat the fast merge: the top-K inside one workgroup's
    # slice (many keys of one list reach the bound; at small K nearly every
    # key of that list does), or every logit of a row tied (more survivors
    # than the sort holds); the exact paths must give the plain top-K bit for
    # bit
    nb, bs, H, V, r = 1, 8, 512, 6000, 32
    inp = inputs(nb, bs, H, V, r, K, 21, 1)
    w = O.widen(inp["w_lm"], "bf16")
    hh = O.widen(inp["h"], "bf16")
    if kind == "clustered":
        w[2000:2040] = hh[0] / np.linalg.norm(hh[0]) * np.linspace(1.0, 2.0, 40)[:, None]
    elif kind == "tied":
        w[:] = w[7]
    else:
        w[:] = 0.0
        w[3000:3020] = hh[:1] * 0.01
    inp["w_lm"] = O.round_bf16(w)
    dev = {k: to_dev(v) for k, v in inp.items()}
    ids, vals, path, ps = D.decode_head(dev["h"], dev["w_lm"], K, dev["w_h"], dev["cb_pred"], dev["cb_succ"],
                                        dev["anchors"], bs)
    ref_ids, ref_vals, _ = D.unary_topk(dev["h"], dev["w_lm"], K)
    torch.cuda.synchronize()
    assert torch.equal(ids, ref_ids) and torch.equal(vals, ref_vals)
    U = O.lm_logits(inp["h"], inp["w_lm"], "bf16")
    fails, _, msgs = compare_topk(to_np(ids), to_np(vals), U, K)
    assert fails == 0, msgs
    gids = to_np(ids)
    u64 = U[np.arange(U.shape[0])[:, None], gids]
    g64 = O.context_projection(inp["h"], inp["w_h"], "bf16")
    fails, _, _, msgs = compare_walk(to_np(path), to_np(ps), g64, inp["cb_pred"], inp["cb_succ"], gids, u64,
                                     inp["anchors"], bs, "bf16")
    assert fails == 0, msgs
