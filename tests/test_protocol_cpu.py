"""The comparison protocol itself, checked on the CPU."""
import numpy as np

from oracle import dflash2_oracle as O
from block_draft_head_amd.inputs import WORKLOADS, make_inputs
from tests.helpers import CORR_ULPS, act_ok, bf16_bracketed, compare_topk, context_ok, conv_delta, corr_abs


def test_bf16_bracket_accepts_both_neighbours_and_nothing_else():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(50_000) * 10.0 ** rng.integers(-3, 4, 50_000)
    rne = O.round_bf16(ref).astype(np.int64)
    for d, want in [(0, True), (1, None), (-1, None), (2, False), (-2, False)]:
        cand = (rne + d).astype(np.uint16)
        got = bf16_bracketed(cand, ref)
        if want is None:
            # exactly one of the two one-step neighbours of the nearest value
            # also brackets the reference (the one on the reference's side)
            continue
        assert np.all(got == want), (d, np.flatnonzero(got != want)[:5])
    up = bf16_bracketed((rne + 1).astype(np.uint16), ref)
    dn = bf16_bracketed((rne - 1).astype(np.uint16), ref)
    exact = O.widen(rne.astype(np.uint16), "bf16") == ref
    assert np.all((up ^ dn) | exact)


def test_topk_comparison_flags_near_ties_and_fails_real_errors():
    U = np.array([[5.0, 4.0, 3.0, 2.9995, 1.0]])
    assert compare_topk(np.array([[0, 1, 2]]), np.array([[5.0, 4.0, 3.0]]), U, 3)[:2] == (0, 0)
    assert compare_topk(np.array([[0, 1, 3]]), np.array([[5.0, 4.0, 2.9995]]), U, 3)[:2] == (0, 1)
    assert compare_topk(np.array([[0, 1, 4]]), np.array([[5.0, 4.0, 1.0]]), U, 3)[:2] == (1, 0)
    assert compare_topk(np.array([[0, 1, 2]]), np.array([[5.0, 4.0, 3.1]]), U, 3)[:2] == (1, 0)


def _float32_prepare(w, blocks):
    """A float32 evaluation of conv prepare (float32 projection, float32 taps,
    one rounding) on the given blocks, beside the exact value and the rule's delta."""
    inp = make_inputs(w, fields=["h", "w_proj", "base"])
    bs, T, gs = w.block_size, w.taps, w.group_size
    rows = np.concatenate([np.arange(b * bs, (b + 1) * bs) for b in blocks])
    h = inp["h"][rows]
    _, _, ex = O.conv_prepare(h, inp["w_proj"], inp["base"], bs, T, gs, "bf16")
    c64 = O.conv_projection(h, inp["w_proj"], T, gs, "bf16")
    x32 = O.widen(h, "bf16").astype(np.float32)
    c32 = (x32 @ O.widen(inp["w_proj"], "bf16").astype(np.float32).T).reshape(c64.shape)
    b32 = O.widen(inp["base"], "bf16").astype(np.float32)
    gh = np.arange(w.hidden) // gs
    f32 = np.zeros_like(x32)
    for n in range(len(rows)):
        for j in range(min(T - 1, n % bs) + 1):
            f32[n] = f32[n] + (b32[0, j] + c32[n, 0, j, gh]) * x32[n - j]
    A = corr_abs(h, inp["w_proj"], T, gs, "bf16")
    delta = conv_delta(h, c64[:, 0], inp["base"][0], bs, gs, "bf16", A[:, 0])
    S = conv_delta(h, c64[:, 0], inp["base"][0], bs, gs, "bf16") * 2.0 ** 24 / (2 * T + 1)
    return O.round_bf16(f32.astype(np.float64)), ex, delta, S, (c32, c64, A)


def test_conv_rule_accepts_a_float32_sum_and_rejects_a_wrong_ulp():
    """The float32 evaluation passes the conv rule everywhere, including where
    the taps nearly cancel; moving any output one bf16 step further from the
    exact value fails it wherever the float32 error bound is below half a bf16
    step; the float32 projection stays within the rule's ulps of its terms;
    and the rule is tighter than 2^-16 of the terms' magnitudes away from
    cancellation."""
    for name, blocks in (("serve_64x8_h5120_v248320", (0, 24, 62, 63)),
                         ("wide_256x16_h5120_v248320_t8_k64", (0, 100, 255))):
        w = WORKLOADS[name]
        got, ex, delta, S, (c32, c64, A) = _float32_prepare(w, blocks)
        assert np.all(np.abs(c32 - c64) <= CORR_ULPS * 2.0 ** -24 * A)
        assert not bf16_bracketed(got, ex).all()  # the strict bracket alone rejects a correct float32 sum here
        assert act_ok(got, ex, "bf16", delta).all()
        # one step further out from the exact value
        g = O.widen(got, "bf16")
        away = np.where((g >= ex) == (g >= 0), 1, -1)  # +1 grows the magnitude
        worse = (got.astype(np.int64) + away).astype(np.uint16)
        far = delta < np.abs(ex) * 2.0 ** -10
        assert far.mean() > 0.98
        assert not act_ok(worse, ex, "bf16", delta)[far & (g != ex)].any()
        # away from cancellation the bound is below 2^-16 S (2.6x at two taps)
        big = np.abs(ex) > 0.25 * S
        assert np.median(delta[big] / (2.0 ** -16 * S[big])) < (0.5 if w.taps == 2 else 1.0)


def test_conv_rule_fails_a_shifted_tap():
    """A planted mistake in the float32 evaluation (tap 1 reads the row after,
    not the row before, and so is missing at the block's last position) fails
    the rule on most rows past a block's first; the first rows still pass."""
    w = WORKLOADS["serve_64x8_h5120_v248320"]
    inp = make_inputs(w, fields=["h", "w_proj", "base"])
    bs, T, gs = w.block_size, w.taps, w.group_size
    h = inp["h"][: 2 * bs]
    _, _, ex = O.conv_prepare(h, inp["w_proj"], inp["base"], bs, T, gs, "bf16")
    c64 = O.conv_projection(h, inp["w_proj"], T, gs, "bf16")
    x = O.widen(h, "bf16")
    b = O.widen(inp["base"], "bf16")
    gh = np.arange(w.hidden) // gs
    bad = np.zeros_like(x)
    for n in range(2 * bs):
        p = n % bs
        bad[n] = (b[0, 0] + c64[n, 0, 0, gh]) * x[n]
        if 1 <= p < bs - 1:
            bad[n] += (b[0, 1] + c64[n, 0, 1, gh]) * x[n + 1]
    A = corr_abs(h, inp["w_proj"], T, gs, "bf16")
    delta = conv_delta(h, c64[:, 0], inp["base"][0], bs, gs, "bf16", A[:, 0])
    ok = act_ok(O.round_bf16(bad), ex, "bf16", delta)
    tapped = np.array([n % bs >= 1 for n in range(2 * bs)])
    assert (~ok[tapped]).mean() > 0.9 and ok[~tapped].all()


def test_context_rule_accepts_a_float32_product_and_fails_a_dropped_term():
    """The float32 product h W_Hᵀ passes the context-row bound at H 5120; the
    same product with one of its H terms dropped (one column of W_H zeroed)
    fails it on nearly every element, and so does the product through a W_H
    whose rows are off by one."""
    rng = np.random.default_rng(3)
    N, H, r = 64, 5120, 48
    h = O.round_bf16(rng.standard_normal((N, H)))
    w_h = O.round_bf16(rng.standard_normal((r, H)) * 0.02)
    x32, w32 = O.widen(h, "bf16").astype(np.float32), O.widen(w_h, "bf16").astype(np.float32)
    assert context_ok(x32 @ w32.T, h, w_h, "bf16").all()
    dropped = w32.copy()
    dropped[:, 1234] = 0.0
    assert (~context_ok(x32 @ dropped.T, h, w_h, "bf16")).mean() > 0.9
    assert not context_ok(x32 @ np.roll(w32, 1, axis=0).T, h, w_h, "bf16").any()
