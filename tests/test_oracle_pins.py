"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test ties one oracle function to something other than itself: numbers
printed on the pages, hand-worked examples derived from the pages' equations
(tests/golden/), textbook or library special cases, invariants the pages
state, and brute force on tiny inputs.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dflash2_oracle as O

if os.environ.get("DFLASH2_ORACLE_MUTANT"):
    # Planted-mistake run (tests/test_oracle_mutants.py): swap in a copy of
    # the oracle with one source edit applied.
    import types
    _old, _new = json.loads(os.environ["DFLASH2_ORACLE_MUTANT"])
    _src = open(O.__file__).read()
    assert _src.count(_old) >= 1, _old
    O = types.ModuleType("dflash2_oracle_mutant")
    exec(compile(_src.replace(_old, _new), "dflash2_oracle_mutant", "exec"), O.__dict__)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bf16(a):
    return torch.tensor(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- formats

def test_round_bf16_matches_torch_rne_on_float32_values():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # exact midpoints between neighbouring bf16 values, both parities
    bits = rng.integers(0, 2**16, 20_000).astype(np.uint32) << 16
    bits = (bits & np.uint32(0x7F7F0000)) | np.uint32(0x8000)
    mid = bits.view(np.float32)
    x = np.concatenate([x, mid, -mid, np.float32([0.0, -0.0, 1e-40, -3e-39])])
    want = _bf16(x)
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_bf16_rounds_once_from_float64():
    # 1 + 2^-8 + 2^-40 sits just above the midpoint of 1.0 (0x3F80) and the
    # next bf16 (0x3F81).  Rounding through float32 first would drop 2^-40 and
    # then tie to even (0x3F80); one direct rounding gives 0x3F81.
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8 + 2.0 ** -40)])
    assert O.round_bf16(x).tolist() == [0x3F81, 0x3F80, 0x3F82, 0xBF81]


def test_widen_is_exact():
    u = np.arange(0, 2**16, 7, dtype=np.uint16)
    u = u[(u & 0x7F80) != 0x7F80]  # finite patterns only
    assert np.array_equal(O.round_bf16(O.widen(u, "bf16")), u)


# ------------------------------------------------------- parameter shapes

def test_param_shapes_reproduce_the_ablation_parameter_counts():
    fx = _load("ablation_param_counts.json")
    p, d = fx["printed"], fx["derived"]
    shapes = O.param_shapes(d["hidden"], d["vocab"], p["conv_kernel_size"],
                            p["conv_group_size"], p["selector_rank"])
    n = {k: int(np.prod(v)) for k, v in shapes.items()}
    conv = n["conv.w_proj"] + n["conv.base"]
    sel = n["selector.w_h"] + n["selector.cb_pred"] + n["selector.cb_succ"]
    assert d["wrapped_sublayers"] * conv + sel == p["DFLASH2_params"] - p["DFLASH_params"]
    # A bias on the projection, or a single base kernel shared by the two
    # convolutions, would break the count.
    G = d["hidden"] // p["conv_group_size"]
    assert d["wrapped_sublayers"] * (conv + 2 * p["conv_kernel_size"] * G) + sel != p["DFLASH2_params"] - p["DFLASH_params"]
    assert d["wrapped_sublayers"] * (conv - p["conv_kernel_size"] * d["hidden"]) + sel != p["DFLASH2_params"] - p["DFLASH_params"]


def test_param_shapes_match_the_explainer_conv_count():
    fx = _load("ablation_param_counts.json")["explainer_conv_params"]
    shapes = O.param_shapes(fx["hidden"], 1, 2, 16, 1)
    per_wrapper = int(np.prod(shapes["conv.w_proj"])) + int(np.prod(shapes["conv.base"]))
    total = fx["layers"] * 2 * per_wrapper
    assert round(total / 1e6, 1) == fx["printed_millions"]


def test_config_rules_raise():
    ok = dict(hidden=64, vocab=100, block_size=8, taps=2, group_size=16, rank=4, top_k=16)
    O.check_config(**ok)
    for bad in [dict(taps=0), dict(taps=9), dict(group_size=5), dict(rank=0),
                dict(top_k=0), dict(top_k=101)]:
        with pytest.raises(ValueError):
            O.check_config(**{**ok, **bad})
    x = np.zeros((12, 64), np.float32)
    with pytest.raises(ValueError):  # not a whole number of blocks
        O.conv_prepare(x, np.zeros((16, 64), np.float32), np.zeros((2, 2, 64), np.float32), 8, 2, 16, "f32")


# ------------------------------------------------------------------ conv

@pytest.mark.parametrize("case", _load("conv_worked_example.json")["cases"], ids=lambda c: c["name"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_worked_examples(case, dtype):
    f = (lambda a: np.asarray(a, np.float32)) if dtype == "f32" else _bf16
    bs, T, gs = case["block_size"], case["taps"], case["group_size"]
    xo, kp, ex = O.conv_prepare(f(case["x"]), f(case["w_proj"]), f(case["base"]), bs, T, gs, dtype)
    assert np.array_equal(ex, np.asarray(case["x_out"], np.float64))
    assert np.array_equal(kp, np.asarray(case["k_post"], np.float64))
    yo, ey = O.conv_finish(f(case["y"]), kp, f(case["base"]), bs, T, gs, dtype)
    assert np.array_equal(ey, np.asarray(case["y_out"], np.float64))
    assert np.array_equal(O.widen(yo, dtype), ey)


def _rand_conv(rng, N, H, T, gs, dtype, scale=0.3):
    G = H // gs
    f = (lambda a: a.astype(np.float32)) if dtype == "f32" else _bf16
    x = f(rng.standard_normal((N, H)))
    w = f(rng.standard_normal((2 * T * G, H)) * scale)
    base = f(rng.standard_normal((2, T, H)) * scale + np.eye(T, 1)[None, :, :])
    y = f(rng.standard_normal((N, H)))
    return x, w, base, y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 2, 3])
def test_conv_identity_init_is_exact_passthrough(dtype, T):
    # tap 0 = 1, later taps 0, projection 0 -> exact no-op (pull request
    # 'Two deltas', item 2; SpecForge 'Architecture').
    rng = np.random.default_rng(T)
    N, H, gs, bs = 24, 32, 8, 4
    x, _, _, y = _rand_conv(rng, N, H, T, gs, dtype)
    f = (lambda a: a.astype(np.float32)) if dtype == "f32" else _bf16
    w = f(np.zeros((2 * T * (H // gs), H)))
    base = np.zeros((2, T, H))
    base[:, 0, :] = 1.0
    base = f(base)
    xo, kp, _ = O.conv_prepare(x, w, base, bs, T, gs, dtype)
    assert np.array_equal(O.widen(xo, dtype), O.widen(x, dtype))
    assert not kp.any()
    yo, _ = O.conv_finish(y, kp, base, bs, T, gs, dtype)
    assert np.array_equal(O.widen(yo, dtype), O.widen(y, dtype))


def test_conv_never_reads_across_a_block_boundary():
    rng = np.random.default_rng(7)
    N, H, T, gs, bs = 32, 16, 3, 4, 8
    x, w, base, y = _rand_conv(rng, N, H, T, gs, "f32")
    _, kp, ex = O.conv_prepare(x, w, base, bs, T, gs, "f32")
    _, ey = O.conv_finish(y, kp, base, bs, T, gs, "f32")
    for blk in range(1, N // bs):
        x2, y2 = x.copy(), y.copy()
        x2[: blk * bs] = rng.standard_normal((blk * bs, H)) * 100
        y2[: blk * bs] = rng.standard_normal((blk * bs, H)) * 100
        _, kp2, ex2 = O.conv_prepare(x2, w, base, bs, T, gs, "f32")
        _, ey2 = O.conv_finish(y2, kp, base, bs, T, gs, "f32")
        sl = slice(blk * bs, N)
        assert np.array_equal(ex2[sl], ex[sl]) and np.array_equal(ey2[sl], ey[sl])
        assert np.array_equal(kp2[sl], kp[sl])
    # the first position of a block only sees its own row: k_0 * x_n
    c = O.conv_projection(x, w, T, gs, "f32")
    g_of_h = np.arange(H) // gs
    for n in range(0, N, bs):
        k0 = O.widen(base, "f32")[0, 0] + c[n, 0, 0, g_of_h]
        assert np.array_equal(ex[n], k0 * O.widen(x, "f32")[n])


@pytest.mark.parametrize("T", [1, 2, 4])
def test_conv_with_zero_projection_is_a_per_block_depthwise_conv1d(T):
    # Library special case: with no dynamic part the op is a textbook causal
    # depthwise convolution, run block by block with zero left padding.
    rng = np.random.default_rng(11 + T)
    N, H, gs, bs = 32, 12, 4, 8
    x, _, base, y = _rand_conv(rng, N, H, T, gs, "f32")
    w0 = np.zeros((2 * T * (H // gs), H), np.float32)
    _, kp, ex = O.conv_prepare(x, w0, base, bs, T, gs, "f32")
    _, ey = O.conv_finish(y, kp, base, bs, T, gs, "f32")
    for s, (inp, got) in enumerate([(x, ex), (y, ey)]):
        # conv1d is a cross-correlation: weight index T-1-j multiplies x[t-j]
        wt = torch.tensor(base[s].T[:, ::-1].copy(), dtype=torch.float64).unsqueeze(1)  # [H,1,T]
        for b in range(N // bs):
            blk = torch.tensor(inp[b * bs:(b + 1) * bs].T, dtype=torch.float64).unsqueeze(0)  # [1,H,bs]
            ref = torch.nn.functional.conv1d(torch.nn.functional.pad(blk, (T - 1, 0)), wt, groups=H)
            np.testing.assert_allclose(got[b * bs:(b + 1) * bs], ref[0].T.numpy(), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("T,gs,bs", [(1, 2, 1), (2, 2, 4), (3, 4, 4), (4, 1, 4)])
def test_conv_matches_scalar_brute_force(T, gs, bs):
    rng = np.random.default_rng(100 + T * 10 + gs)
    N, H = 3 * bs, 8
    G = H // gs
    x, w, base, y = _rand_conv(rng, N, H, T, gs, "f32", scale=0.5)
    xo, kp, ex = O.conv_prepare(x, w, base, bs, T, gs, "f32")
    _, ey = O.conv_finish(y, kp, base, bs, T, gs, "f32")
    X, W, Bk, Y = (np.asarray(a, np.float64) for a in (x, w, base, y))
    for n in range(N):
        blk_start = (n // bs) * bs
        for h in range(H):
            g = h // gs
            acc_x = acc_y = 0.0
            for j in range(T):
                if n - j < blk_start:
                    continue
                c_pre = sum(W[(0 * T + j) * G + g, i] * X[n, i] for i in range(H))
                c_post = sum(W[(1 * T + j) * G + g, i] * X[n, i] for i in range(H))
                acc_x += (Bk[0, j, h] + c_pre) * X[n - j, h]
                acc_y += (Bk[1, j, h] + c_post) * Y[n - j, h]
            assert abs(acc_x - ex[n, h]) < 1e-12 and abs(acc_y - ey[n, h]) < 1e-12
    # the output is rounded once, to nearest
    assert np.array_equal(xo, ex.astype(np.float32))


# ------------------------------------------------------------- unary top-K

def test_unary_topk_matches_selection_by_brute_force():
    rng = np.random.default_rng(3)
    N, H, V, K = 5, 16, 40, 7
    h = rng.standard_normal((N, H)).astype(np.float32)
    W = rng.standard_normal((V, H)).astype(np.float32)
    gold = rng.integers(0, V, N).astype(np.int32)
    ids, vals, gl = O.unary_topk(h, W, K, "f32", gold_ids=gold)
    for n in range(N):
        U = [sum(float(h[n, i]) * float(W[v, i]) for i in range(H)) for v in range(V)]
        left = list(range(V))
        for k in range(K):
            best = left[0]
            for v in left[1:]:
                if U[v] > U[best]:
                    best = v
            assert ids[n, k] == best and abs(vals[n, k] - U[best]) < 1e-12
            left.remove(best)
        assert abs(gl[n] - U[gold[n]]) < 1e-12


def test_unary_topk_agrees_with_torch_topk_and_breaks_ties_by_lower_id():
    rng = np.random.default_rng(4)
    N, H, V, K = 6, 32, 500, 16
    h = _bf16(rng.standard_normal((N, H)))
    W = rng.standard_normal((V, H))
    # row n's best direction appears at four ids, one of them lower than the
    # first copy: an exact four-way tie at the top of row n
    dup = {}
    for n in range(N):
        ids_n = [400 - 7 * n, 100 + n, 300 + 3 * n, 11 + n]
        W[ids_n] = 6.0 * O.widen(h, "bf16")[n]
        dup[n] = sorted(ids_n)
    Wb = _bf16(W)
    ids, vals, _ = O.unary_topk(h, Wb, K, "bf16")
    U = O.widen(h, "bf16") @ O.widen(Wb, "bf16").T
    tv, ti = torch.topk(torch.tensor(U), K, dim=1)
    np.testing.assert_array_equal(vals, tv.numpy())
    for n in range(N):
        assert set(ids[n].tolist()) == set(ti[n].tolist()) or (vals[n, -1] == vals[n, -2])
        assert ids[n, :4].tolist() == dup[n]
        for k in range(K - 1):
            if vals[n, k] == vals[n, k + 1]:
                assert ids[n, k] < ids[n, k + 1]


def test_logits_at_and_context_projection_match_brute_force():
    rng = np.random.default_rng(5)
    N, H, V, r = 4, 12, 30, 5
    h = _bf16(rng.standard_normal((N, H)))
    W = _bf16(rng.standard_normal((V, H)))
    Wh = _bf16(rng.standard_normal((r, H)))
    hf, Wf, Whf = (O.widen(a, "bf16") for a in (h, W, Wh))
    ids = rng.integers(0, V, (N, 3))
    got = O.logits_at(h, W, ids, "bf16")
    g = O.context_projection(h, Wh, "bf16")
    for n in range(N):
        for k in range(3):
            assert abs(got[n, k] - sum(hf[n, i] * Wf[ids[n, k], i] for i in range(H))) < 1e-12
        for rho in range(r):
            assert abs(g[n, rho] - sum(Whf[rho, i] * hf[n, i] for i in range(H))) < 1e-12


# --------------------------------------------------------------- selector

def test_selector_worked_example():
    fx = _load("selector_worked_example.json")
    f = lambda a: np.asarray(a, np.float32)
    A, B, g = f(fx["cb_pred"]), f(fx["cb_succ"]), np.asarray(fx["g"], np.float64)
    ids = np.asarray(fx["cand_ids"], np.int32)
    U = np.asarray(fx["cand_u"], np.float64)
    path, ps = O.selector_walk(g, A, B, ids, U, np.array([fx["anchor"]]), fx["block_size"], "f32")
    assert path[0].tolist() == fx["path"]
    assert ps[0].tolist() == fx["path_score"]
    gold = np.asarray(fx["gold"], np.int32)
    gl = np.asarray(fx["gold_logit"], np.float64)
    pred = np.asarray(fx["tf_pred"], np.int32)
    for force, row2_valid in [(np.ones(3, np.uint8), 1), (np.zeros(3, np.uint8), 0)]:
        sc, best, ce, valid = O.selector_score_tf(g, A, B, ids, U, pred, "f32",
                                                  gold_ids=gold, force=force, gold_logit=gl)
        assert sc[1:].tolist() == fx["tf_scores_rows_1_2"]
        assert best[1:].tolist() == fx["tf_best_rows_1_2"]
        sp = [math.log1p(math.exp(z)) for z in fx["ce_softplus_arg_rows_1_2_forced"]]
        assert valid[1] == 1 and abs(ce[1] - sp[0]) < 1e-12
        assert valid[2] == row2_valid
        assert abs(ce[2] - (sp[1] if row2_valid else 0.0)) < 1e-12


def _rand_selector(rng, N, V, r, K, dtype="f32"):
    f = (lambda a: a.astype(np.float32)) if dtype == "f32" else _bf16
    A = f(rng.standard_normal((V, r)) * 0.7)
    B = f(rng.standard_normal((V, r)) * 0.7)
    g = rng.standard_normal((N, r))
    ids = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
    U = -np.sort(-rng.standard_normal((N, K)), axis=1)
    return A, B, g, ids, U


def test_selector_matches_brute_force_on_tiny_vocab():
    # V <= 8 and K = V: every pair is a candidate pair.
    rng = np.random.default_rng(21)
    V, r, bs, nb = 6, 3, 5, 4
    N = nb * bs
    A, B, g, ids, U = _rand_selector(rng, N, V, r, V)
    anchors = rng.integers(0, V, nb)
    path, ps = O.selector_walk(g, A, B, ids, U, anchors, bs, "f32")
    Af, Bf = A.astype(np.float64), B.astype(np.float64)

    def S(n, a, k):
        b = ids[n, k]
        tot = U[n, k]
        for rho in range(r):
            tot += Af[a, rho] * g[n, rho] * Bf[b, rho]
        return tot

    for blk in range(nb):
        a = anchors[blk]
        assert path[blk, 0] == a
        for t in range(1, bs):
            n = blk * bs + t
            vals = [S(n, a, k) for k in range(V)]
            kbest = max(range(V), key=lambda k: (vals[k], -k))
            assert path[blk, t] == ids[n, kbest] and abs(ps[blk, t] - vals[kbest]) < 1e-12
            a = ids[n, kbest]
    pred = rng.integers(0, V, N)
    sc, best, _, _ = O.selector_score_tf(g, A, B, ids, U, pred, "f32")
    for n, k in itertools.product(range(N), range(V)):
        assert abs(sc[n, k] - S(n, pred[n], k)) < 1e-12


@pytest.mark.parametrize("zero", ["succ", "pred", "ctx"])
def test_zero_factor_reduces_the_walk_to_the_unary_argmax(zero):
    # A zero successor codebook preserves the unary scores (SpecForge
    # 'Architecture'); a zero predecessor codebook or context does the same.
    rng = np.random.default_rng(31)
    V, r, K, bs, nb = 50, 8, 6, 8, 5
    N = nb * bs
    A, B, g, ids, U = _rand_selector(rng, N, V, r, K)
    if zero == "succ":
        B = np.zeros_like(B)
    elif zero == "pred":
        A = np.zeros_like(A)
    else:
        g = np.zeros_like(g)
    path, ps = O.selector_walk(g, A, B, ids, U, rng.integers(0, V, nb), bs, "f32")
    for blk in range(nb):
        for t in range(1, bs):
            n = blk * bs + t
            assert path[blk, t] == ids[n, 0] and ps[blk, t] == U[n, 0]


def test_exact_ties_in_the_walk_go_to_the_lowest_slot():
    rng = np.random.default_rng(36)
    V, r, K, bs, nb = 40, 4, 5, 6, 3
    A, B, g, ids, _ = _rand_selector(rng, nb * bs, V, r, K)
    U = np.zeros((nb * bs, K))
    U[:, :3] = 2.0  # three equal leaders, the rest lower; no pair term
    path, ps = O.selector_walk(g, A, np.zeros_like(B), ids, U, rng.integers(0, V, nb), bs, "f32")
    assert np.array_equal(path[:, 1:], ids.reshape(nb, bs, K)[:, 1:, 0])


def test_top1_candidate_set_makes_any_selector_follow_the_unary_pick():
    rng = np.random.default_rng(32)
    V, r, bs, nb = 30, 4, 8, 3
    A, B, g, ids, U = _rand_selector(rng, nb * bs, V, r, 1)
    path, _ = O.selector_walk(g, A, B, ids, U, rng.integers(0, V, nb), bs, "f32")
    assert np.array_equal(path[:, 1:], ids.reshape(nb, bs)[:, 1:])


def test_replaying_the_walk_through_teacher_forcing_reproduces_it():
    # Pull request 'Selector training objective': the vectorised scorer fed
    # with the sequential trace's own predecessors gives the same path.
    rng = np.random.default_rng(33)
    V, r, K, bs, nb = 200, 16, 8, 8, 12
    N = nb * bs
    A, B, g, ids, U = _rand_selector(rng, N, V, r, K, "bf16")
    anchors = rng.integers(0, V, nb)
    path, ps = O.selector_walk(g, A, B, ids, U, anchors, bs, "bf16")
    pred = np.zeros(N, np.int32)
    for blk in range(nb):
        pred[blk * bs + 1: (blk + 1) * bs] = path[blk, :-1]
    sc, best, _, _ = O.selector_score_tf(g, A, B, ids, U, pred, "bf16")
    for blk in range(nb):
        for t in range(1, bs):
            n = blk * bs + t
            assert best[n] == path[blk, t] and sc[n].max() == ps[blk, t]
    # the selector has teeth on these inputs: it overrides the unary pick
    assert (path[:, 1:] != ids.reshape(nb, bs, K)[:, 1:, 0]).any()


def test_ce_closed_forms():
    rng = np.random.default_rng(34)
    V, r, N = 40, 4, 10
    # K = 1 with the gold in the set: CE = 0
    A, B, g, ids, U = _rand_selector(rng, N, V, r, 1)
    _, _, ce, valid = O.selector_score_tf(g, A, B, ids, U, rng.integers(0, V, N), "f32", gold_ids=ids[:, 0])
    assert valid.all() and np.all(ce == 0)
    # equal scores over K candidates: CE = ln K
    K = 5
    A, B, g, ids, U = _rand_selector(rng, N, V, r, K)
    Uc = np.full((N, K), 0.25)
    _, best, ce, valid = O.selector_score_tf(g, A, np.zeros_like(B), ids, Uc, rng.integers(0, V, N), "f32", gold_ids=ids[:, 2])
    np.testing.assert_allclose(ce, math.log(K), rtol=0, atol=1e-14)
    assert np.array_equal(best, ids[:, 0])  # exact tie: the lowest slot wins
    # adding a per-row constant to U leaves CE and the argmax unchanged
    pred = rng.integers(0, V, N)
    s1, b1, ce1, _ = O.selector_score_tf(g, A, B, ids, U, pred, "f32", gold_ids=ids[:, 3])
    s2, b2, ce2, _ = O.selector_score_tf(g, A, B, ids, U + rng.standard_normal((N, 1)) * 5, pred, "f32", gold_ids=ids[:, 3])
    assert np.array_equal(b1, b2)
    np.testing.assert_allclose(ce1, ce2, rtol=1e-12, atol=1e-12)


def test_forced_gold_takes_the_weakest_slot_and_coverage_follows():
    rng = np.random.default_rng(35)
    N, H, V, K, r = 4096, 64, 4096, 16, 8
    h = rng.standard_normal((N, H)).astype(np.float32)
    W = (rng.standard_normal((V, H)) / 8).astype(np.float32)
    gold = rng.integers(0, V, N).astype(np.int32)
    force = (rng.random(N) < 0.8).astype(np.uint8)
    ids, vals, gl = O.unary_topk(h, W, K, "f32", gold_ids=gold)
    A, B, g, _, _ = _rand_selector(rng, N, V, r, K)
    pred = rng.integers(0, V, N)
    sc, best, ce, valid = O.selector_score_tf(g, A, B, ids, vals, pred, "f32", gold_ids=gold, force=force, gold_logit=gl)
    in_set = (ids == gold[:, None]).any(1)
    assert np.array_equal(valid.astype(bool), in_set | (force == 1))
    cov = valid.mean()
    assert abs(cov - (0.8 + 0.2 * K / V)) < 0.03
    # a forced row's CE uses the gold at slot K-1 with its own logit
    n = int(np.flatnonzero(~in_set & (force == 1))[0])
    s2 = sc[n].copy()
    s2[K - 1] = gl[n] + (O.widen(A, "f32")[pred[n]] * g[n]) @ O.widen(B, "f32")[gold[n]]
    m = s2.max()
    assert abs(ce[n] - (m + math.log(np.exp(s2 - m).sum()) - s2[K - 1])) < 1e-12
    # excluded rows contribute no CE
    assert np.all(ce[valid == 0] == 0)


# ---------------------------------------------------------------- sampling walk

def test_philox4x32_10_reproduces_the_published_known_answers():
    # Known-answer vectors of Philox4x32-10 (Salmon et al., SC 2011, as
    # distributed with the authors' Random123 library): counter, key -> output.
    kat = [
        ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
         (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
         (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, want in kat:
        got = O.philox4x32_10(np.array(ctr, np.uint64), np.array(key, np.uint64))
        assert tuple(int(v) for v in got) == want


def test_walk_uniforms_are_open_24_bit_grid_points():
    u = O.walk_uniform(3, 5, np.arange(4096), 0xDEADBEEF12345678)
    assert u.min() > 0 and u.max() < 1
    assert np.all(((u * 2 ** 24) - 0.5) == np.floor(u * 2 ** 24))
    # distinct counters give distinct draws; the same counter the same draw
    assert len(np.unique(u)) > 4000
    assert np.array_equal(u, O.walk_uniform(3, 5, np.arange(4096), 0xDEADBEEF12345678))
    assert not np.array_equal(u, O.walk_uniform(3, 6, np.arange(4096), 0xDEADBEEF12345678))
    assert not np.array_equal(u, O.walk_uniform(3, 5, np.arange(4096), 0xDEADBEEF12345679))


def test_sampling_at_vanishing_temperature_is_the_greedy_walk():
    rng = np.random.default_rng(41)
    V, r, K, bs, nb = 200, 16, 8, 8, 12
    A, B, g, ids, U = _rand_selector(rng, nb * bs, V, r, K)
    anchors = rng.integers(0, V, nb)
    path, ps = O.selector_walk(g, A, B, ids, U, anchors, bs, "f32")
    spath, sps = O.selector_sample(g, A, B, ids, U, anchors, bs, "f32", 1e-9, 7)
    assert np.array_equal(path, spath) and np.array_equal(ps, sps)
    # at temperature 1 the draws depart from the greedy path
    spath1, _ = O.selector_sample(g, A, B, ids, U, anchors, bs, "f32", 1.0, 7)
    assert not np.array_equal(path, spath1)


def test_sampled_picks_follow_the_softmax_of_the_scores():
    # Gumbel-max: the first argmax of S / temperature + Gumbel noise is
    # distributed as softmax(S / temperature).  Zero successor codebook: S is
    # the unary row, the same at every position, so every (block, position)
    # is an independent draw from one known distribution.
    rng = np.random.default_rng(42)
    V, r, K, bs, nb = 64, 4, 3, 8, 2000
    N = nb * bs
    A, B, g, _, _ = _rand_selector(rng, N, V, r, K)
    ids = np.tile(np.array([5, 9, 17], np.int32), (N, 1))
    U = np.tile(np.log([1.0, 2.0, 5.0]), (N, 1))
    for temp, p in ((1.0, np.array([1, 2, 5]) / 8), (2.0, np.sqrt([1, 2, 5]) / np.sqrt([1, 2, 5]).sum())):
        path, ps = O.selector_sample(g, A, np.zeros_like(B), ids, U, rng.integers(0, V, nb), bs, "f32", temp, 99)
        picks = path[:, 1:].ravel()
        freq = np.array([(picks == i).mean() for i in (5, 9, 17)])
        sd = np.sqrt(p * (1 - p) / picks.size)
        assert np.all(np.abs(freq - p) < 4 * sd), (temp, freq, p)
        # the reported score is the picked candidate's S, noise excluded
        assert np.allclose(ps[:, 1:].ravel(), np.log([1.0, 2.0, 5.0])[np.searchsorted([5, 9, 17], picks)])


def test_temperature_divides_the_scores_not_the_noise():
    rng = np.random.default_rng(43)
    V, r, K, bs, nb = 100, 8, 6, 8, 10
    A, B, g, ids, U = _rand_selector(rng, nb * bs, V, r, K)
    anchors = rng.integers(0, V, nb)
    # scores doubled at temperature 2 give the same draws as the scores at 1
    p1, s1 = O.selector_sample(g, A, np.zeros_like(B), ids, U, anchors, bs, "f32", 1.0, 5)
    p2, s2 = O.selector_sample(g, A, np.zeros_like(B), ids, 2.0 * U, anchors, bs, "f32", 2.0, 5)
    assert np.array_equal(p1, p2) and np.allclose(2.0 * s1, s2)


# ---------------------------------------------------------------- selector CE backward

def _grid(rng, shape, scale, q=8):
    # values on a 2^-q grid, so that x +/- 2^-(q+4) is exact in float32
    return (np.rint(rng.standard_normal(shape) * scale * 2 ** q) / 2 ** q).astype(np.float32)


def _ce_case(rng, N=14, H=6, V=12, r=4, K=5):
    """Small case with every row kind: gold in the set, gold forced into the
    weakest slot, gold excluded; repeated predecessors and candidate ids
    shared by rows, so the scatter-adds collide."""
    h = _grid(rng, (N, H), 1.0)
    w_h = _grid(rng, (r, H), 0.5)
    A = _grid(rng, (V, r), 0.8)
    B = _grid(rng, (V, r), 0.8)
    ids = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
    U = -np.sort(-rng.standard_normal((N, K)), axis=1)
    pred = rng.integers(0, 3, N).astype(np.int32)
    gold = ids[np.arange(N), rng.integers(0, K, N)].copy()
    out = np.flatnonzero(rng.random(N) < 0.5)
    for n in out:
        gold[n] = rng.choice(np.setdiff1d(np.arange(V), ids[n]))
    force = (rng.random(N) < 0.6).astype(np.uint8)
    force[out[::2]], force[out[1::2]] = 0, 1
    gl = rng.standard_normal(N)
    w = rng.random(N) + 0.25
    return h, w_h, A, B, ids, U, pred, gold, force, gl, w


def _weighted_ce(h, w_h, A, B, ids, U, pred, gold, force, gl, w, g=None):
    if g is None:
        g = O.context_projection(h, w_h, "f32")
    _, _, ce, valid = O.selector_score_tf(g, A, B, ids, U, pred, "f32", gold_ids=gold, force=force, gold_logit=gl)
    return float(np.sum(w * ce)), valid


def test_ce_backward_matches_central_differences_of_the_forward():
    # Every entry of dA, dB and dW_H against a central difference of the
    # weighted teacher-forced CE (the forward pinned above); dg against a
    # difference in g itself.  The step 2^-12 is exact on the 2^-8 grid.
    rng = np.random.default_rng(41)
    case = _ce_case(rng)
    h, w_h, A, B, ids, U, pred, gold, force, gl, w = case
    dA, dB, dW, dg, valid = O.selector_ce_backward(h, w_h, A, B, ids, U, pred, "f32", gold, force, gl, w)
    base, valid_f = _weighted_ce(*case)
    assert np.array_equal(valid, valid_f)
    assert 0 < valid.sum() < len(valid)     # some rows excluded
    eps = 2.0 ** -12
    for name, pos, grad in (("A", 2, dA), ("B", 3, dB), ("W", 1, dW)):
        for idx in np.ndindex(grad.shape):
            args_p, args_m = list(case), list(case)
            xp, xm = case[pos].copy(), case[pos].copy()
            xp[idx] += np.float32(eps)
            xm[idx] -= np.float32(eps)
            assert xp[idx] - case[pos][idx] == eps      # the step is exact
            args_p[pos], args_m[pos] = xp, xm
            fd = (_weighted_ce(*args_p)[0] - _weighted_ce(*args_m)[0]) / (2 * eps)
            assert abs(fd - grad[idx]) < 2e-6 * (1 + abs(fd)), (name, idx, fd, grad[idx])
    g = O.context_projection(h, w_h, "f32")
    for idx in np.ndindex(g.shape):
        gp, gm = g.copy(), g.copy()
        gp[idx] += 1e-6
        gm[idx] -= 1e-6
        fd = (_weighted_ce(*case, g=gp)[0] - _weighted_ce(*case, g=gm)[0]) / 2e-6
        assert abs(fd - dg[idx]) < 1e-6 * (1 + abs(fd))
    # untouched codebook rows get no gradient
    assert np.all(dA[np.setdiff1d(np.arange(len(A)), pred[valid == 1])] == 0)


def test_ce_backward_obeys_the_euler_identity_of_the_trilinear_pair_term():
    # The pair term is linear in each of A, B and W_H (g = W_H h), so
    # d/dlambda L(lambda X) at lambda = 1 is the same for X = A, B or W_H:
    # <dA, A> = <dB, B> = <dW_H, W_H> = <dg, g>, and it is nonzero.
    rng = np.random.default_rng(42)
    N, H, V, r, K = 64, 32, 300, 16, 8
    h = _bf16(rng.standard_normal((N, H)))
    w_h = _bf16(rng.standard_normal((r, H)) * 0.2)
    A = _bf16(rng.standard_normal((V, r)) * 0.7)
    B = _bf16(rng.standard_normal((V, r)) * 0.7)
    ids = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
    U = -np.sort(-rng.standard_normal((N, K)), axis=1)
    pred = rng.integers(0, V, N).astype(np.int32)
    gold = rng.integers(0, V, N).astype(np.int32)
    gold[::2] = ids[::2, 3]
    force = (rng.random(N) < 0.8).astype(np.uint8)
    gl = rng.standard_normal(N)
    dA, dB, dW, dg, valid = O.selector_ce_backward(h, w_h, A, B, ids, U, pred, "bf16", gold, force, gl, np.ones(N))
    g = O.context_projection(h, w_h, "bf16")
    e = [np.sum(dA * O.widen(A, "bf16")), np.sum(dB * O.widen(B, "bf16")), np.sum(dW * O.widen(w_h, "bf16")),
         np.sum(dg * g)]
    assert abs(e[0]) > 1e-2
    np.testing.assert_allclose(e, e[0], rtol=1e-10, atol=0)


def test_ce_backward_closed_forms():
    rng = np.random.default_rng(43)
    N, H, V, r, K = 9, 5, 40, 3, 4
    h, w_h = _grid(rng, (N, H), 1.0), _grid(rng, (r, H), 0.5)
    A, B = _grid(rng, (V, r), 0.8), _grid(rng, (V, r), 0.8)
    ids = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
    pred = rng.integers(0, V, N).astype(np.int32)
    w = rng.random(N) + 0.5
    # K = 1, gold in the set: the CE is identically 0, so is every gradient
    z = O.selector_ce_backward(h, w_h, A, B, ids[:, :1], np.zeros((N, 1)), pred, "f32", ids[:, 0], None, None, w)
    assert all(np.all(t == 0) for t in z[:4]) and z[4].all()
    # zero successor codebook, equal unary logits: the softmax is uniform, so
    # the successor gradient of row n is w (1/K - [k = gold]) (A[p] * g), and
    # nothing else moves (v = 0)
    kg = rng.integers(0, K, N)
    Z = np.zeros_like(B)
    dA, dB, dW, dg, valid = O.selector_ce_backward(h, w_h, A, Z, ids, np.full((N, K), 0.5), pred, "f32",
                                                   ids[np.arange(N), kg], None, None, w)
    assert valid.all() and np.all(dA == 0) and np.all(dW == 0) and np.all(dg == 0)
    g = O.context_projection(h, w_h, "f32")
    want = np.zeros((V, r))
    for n in range(N):
        for k in range(K):
            want[ids[n, k]] += w[n] * (1 / K - (k == kg[n])) * A[pred[n]].astype(np.float64) * g[n]
    np.testing.assert_allclose(dB, want, rtol=1e-12, atol=1e-15)
    # excluded rows (gold outside the set, not forced) contribute nothing
    far = np.full(N, V - 1, np.int32)
    ids2 = ids % (V - 1)
    z = O.selector_ce_backward(h, w_h, A, B, ids2, np.zeros((N, K)), pred, "f32", far, np.zeros(N, np.uint8),
                               np.zeros(N), w)
    assert not z[4].any() and all(np.all(t == 0) for t in z[:4])


# ---------------------------------------------------------------- unary transforms and metrics

def _lm_case(rng, N=6, H=16, V=40, scale=1.0):
    h = rng.standard_normal((N, H)).astype(np.float32)
    w = (rng.standard_normal((V, H)) * scale).astype(np.float32)
    return h, w


def test_untransformed_ex_is_the_plain_candidate_lattice():
    rng = np.random.default_rng(51)
    h, w = _lm_case(rng)
    gold = rng.integers(0, 40, 6)
    ids, vals, gl = O.unary_topk(h, w, 7, "f32", gold_ids=gold)
    ids2, vals2, lse, gl2, prob, hit = O.unary_topk_ex(h, w, 7, "f32", gold_ids=gold)
    assert np.array_equal(ids, ids2) and np.array_equal(vals, vals2) and np.array_equal(gl, gl2)


def test_softcap_is_bounded_odd_and_linear_near_zero():
    x = np.linspace(-400, 400, 2001)
    for m, c in ((1.0, 30.0), (2.5, 10.0), (0.5, 50.0)):
        y = O.transform_logits(x, m, c)
        assert np.all(np.abs(y) <= c)                       # the cap bounds the final logits
        assert np.allclose(y, -O.transform_logits(-x, m, c), rtol=0, atol=1e-12)
        assert np.all(np.diff(y) >= 0)
        small = np.abs(m * x) < 1e-3 * c
        assert np.allclose(y[small], m * x[small], rtol=1e-6, atol=0)
    # a vanishing cap is off, a huge cap is the multiplier alone
    assert np.array_equal(O.transform_logits(x, 3.0, 0.0), 3.0 * x)
    assert np.allclose(O.transform_logits(x, 3.0, 1e9), 3.0 * x, rtol=1e-9, atol=0)
    # tanh(1) at x = c / m
    assert abs(O.transform_logits(np.array([4.0]), 2.5, 10.0)[0] - 10.0 * math.tanh(1.0)) < 1e-12


def test_transforms_keep_the_candidates_and_rescale_the_values():
    rng = np.random.default_rng(52)
    h, w = _lm_case(rng, N=8, V=60, scale=3.0)
    gold = rng.integers(0, 60, 8)
    ids0, vals0, _ = O.unary_topk(h, w, 10, "f32", gold_ids=gold)
    for m, c in ((2.0, 0.0), (1.0, 5.0), (0.3, 2.0)):
        ids, vals, lse, gl, prob, hit = O.unary_topk_ex(h, w, 10, "f32", gold_ids=gold, output_multiplier=m,
                                                        softcap=c)
        assert np.array_equal(ids, ids0)
        want = m * vals0 if c == 0 else c * np.tanh(m * vals0 / c)
        np.testing.assert_allclose(vals, want, rtol=1e-13, atol=1e-13)
    with pytest.raises(ValueError):
        O.unary_topk_ex(h, w, 10, "f32", output_multiplier=-1.0)
    with pytest.raises(ValueError):
        O.unary_topk_ex(h, w, 10, "f32", softcap=-2.0)


def test_metrics_by_brute_force_on_a_tiny_vocabulary():
    # target probabilities over every possible gold sum to one; the hit flag,
    # the log-sum-exp and the probability by scalar loops
    rng = np.random.default_rng(53)
    N, H, V, K = 3, 5, 9, 4
    h, w = _lm_case(rng, N, H, V, scale=2.0)
    for m, c in ((1.0, 0.0), (1.7, 3.0)):
        total = np.zeros(N)
        for g in range(V):
            gold = np.full(N, g)
            ids, vals, lse, gl, prob, hit = O.unary_topk_ex(h, w, K, "f32", gold_ids=gold, output_multiplier=m,
                                                            softcap=c)
            total += prob
            for n in range(N):
                logits = [m * sum(float(h[n, i]) * float(w[v, i]) for i in range(H)) for v in range(V)]
                if c:
                    logits = [c * math.tanh(x / c) for x in logits]
                z = sum(math.exp(x) for x in logits)
                assert abs(lse[n] - math.log(z)) < 1e-12
                assert abs(prob[n] - math.exp(logits[g]) / z) < 1e-12
                ranked = sorted(range(V), key=lambda v: (-logits[v], v))[:K]
                assert hit[n] == (g in ranked)
        np.testing.assert_allclose(total, 1.0, rtol=0, atol=1e-12)


def test_log_sum_exp_of_equal_logits_and_of_a_dominant_one():
    U = np.zeros((2, 1000))
    U[1, 7] = 800.0   # would overflow without the shift
    lse = O.logsumexp_rows(U)
    assert abs(lse[0] - math.log(1000)) < 1e-12
    assert abs(lse[1] - 800.0) < 1e-12
