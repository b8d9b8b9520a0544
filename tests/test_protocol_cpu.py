"""The comparison protocol itself, checked on the CPU."""
import numpy as np

from oracle import dflash2_oracle as O
from tests.helpers import bf16_bracketed, compare_topk


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
