"""dflash2_selector_walk_noalloc against dflash2_selector_walk: the same
kernels with the workspace in the library's own device array, so paths and
path scores must be bit-equal.  Two calls in a row, the second smaller, and
both walk forms (every pair scored at once; one pick at a time with 128
blocks or more)."""
import numpy as np
import pytest
import torch

from block_draft_head_amd.inputs import Workload, make_inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    from block_draft_head_amd import dflash2
    assert torch.cuda.is_available(), "no GPU visible"
    return dflash2


def case(nb, bs, H, V, r, K, dtype, seed):
    w = Workload("na", nb, bs, H, V, dtype, 2, 16, r, K, "walk")
    inp = make_inputs(w, seed=seed, fields=["h", "w_h", "cb_pred", "cb_succ", "anchors"])
    if dtype == "f32":  # larger codebooks: the pair term overrides the unary pick more often
        inp["cb_pred"] *= np.float32(6)
        inp["cb_succ"] *= np.float32(6)
    rng = np.random.default_rng(seed)
    N = nb * bs
    ids = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
    vals = (-np.sort(-rng.standard_normal((N, K)), axis=1)).astype(np.float32)
    if N > 3:
        ids[3, 0] = V + 5  # an out-of-range candidate: both forms end that path the same way
    dev = {k: to_dev(v) for k, v in inp.items()}
    return dev, to_dev(ids), to_dev(vals)


# (n_blocks, bs, H, V, r, K, dtype): each pair runs big then small, in one process
PAIRS = [
    ((40, 8, 256, 4096, 256, 16, "bf16"), (3, 8, 256, 1000, 32, 8, "bf16")),
    ((130, 8, 256, 3000, 512, 20, "bf16"), (1, 8, 256, 2000, 64, 16, "bf16")),
    ((16, 8, 256, 4096, 32, 16, "f32"), (2, 4, 256, 500, 16, 3, "f32")),
]


@pytest.mark.parametrize("big,small", PAIRS)
def test_noalloc_walk_equals_workspace_walk(D, big, small):
    for shape, seed in ((big, 1), (small, 2)):
        nb, bs, H, V, r, K, dtype = shape
        print(f"noalloc walk nb={nb} bs={bs} H={H} V={V} r={r} K={K} {dtype}", flush=True)
        dev, ids, vals = case(nb, bs, H, V, r, K, dtype, seed)
        ref_p, ref_s = D.selector_walk(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals,
                                       dev["anchors"], bs)
        path = torch.full((nb, bs), -7, dtype=torch.int32, device="cuda")
        score = torch.full((nb, bs), 7.0, dtype=torch.float32, device="cuda")
        p, s = D.selector_walk_noalloc(dev["h"], dev["w_h"], dev["cb_pred"], dev["cb_succ"], ids, vals,
                                       dev["anchors"], bs, path=path, path_score=score)
        torch.cuda.synchronize()
        assert p.data_ptr() == path.data_ptr() and s.data_ptr() == score.data_ptr()
        assert torch.equal(p, ref_p)
        assert torch.equal(torch.nan_to_num(s, nan=-1e30), torch.nan_to_num(ref_s, nan=-1e30))
        assert (p[:, 0] == dev["anchors"]).all()


def test_noalloc_walk_rejects_a_walk_beyond_its_array(D):
    # 257 blocks of 16 at rank 512: the context rows alone exceed the array
    h = torch.zeros((257 * 16, 256), dtype=torch.bfloat16, device="cuda")
    wh = torch.zeros((512, 256), dtype=torch.bfloat16, device="cuda")
    cb = torch.zeros((100, 512), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((257 * 16, 4), dtype=torch.int32, device="cuda")
    vals = torch.zeros((257 * 16, 4), dtype=torch.float32, device="cuda")
    anchors = torch.zeros(257, dtype=torch.int32, device="cuda")
    with pytest.raises(D.DFlash2Error) as e:
        D.selector_walk_noalloc(h, wh, cb, cb, ids, vals, anchors, 16)
    assert e.value.status == 4  # DFLASH2_ERR_UNSUPPORTED, before anything is enqueued
