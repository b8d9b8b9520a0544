"""The oracle's pins have teeth: each plausible mistake planted in a copy of
the oracle (one source edit, on the CPU) makes the pin suite fail."""
import json
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "tap reads the next row": ("out[n] += k * v[n - j]", "out[n] += k * v[min(n + j, N - 1)]"),
    "interleaved channel groups": ("g_of_h = np.arange(H) // group_size", "g_of_h = np.arange(H) % (H // group_size)"),
    "taps cross the block start": ("for j in range(min(T - 1, p) + 1):", "for j in range(min(T - 1, n) + 1):"),
    "kernel taken from the tapped row": ("k = base_s[j] + corr[n, j, g_of_h]", "k = base_s[j] + corr[n - j, j, g_of_h]"),
    "base kernel dropped": ("k = base_s[j] + corr[n, j, g_of_h]", "k = corr[n, j, g_of_h]"),
    "finish gets the input kernel": ("return round_to(exact, dtype), c[:, 1].copy(), exact", "return round_to(exact, dtype), c[:, 0].copy(), exact"),
    "projection layout (g, s, j)": ("return c.reshape(N, 2, taps, G)", "return c.reshape(N, G, 2, taps).transpose(0, 2, 3, 1)"),
    "finish uses the input base": ("widen(base, dtype)[1], block_size, group_size)", "widen(base, dtype)[0], block_size, group_size)"),
    "bf16 output truncated": ("np.rint(np.ldexp(x, -q))", "np.trunc(np.ldexp(x, -q))"),
    "top-K ties to the higher id": ("np.lexsort((vid, -U[n]))", "np.lexsort((-vid, -U[n]))"),
    "top-K ascending": ("np.lexsort((vid, -U[n]))", "np.lexsort((vid, U[n]))"),
    "codebooks swapped": ("a_row = widen(cb_pred[pred_id], dtype)\n    b_rows = widen(cb_succ[", "a_row = widen(cb_succ[pred_id], dtype)\n    b_rows = widen(cb_pred["),
    "context projection ignored": ("b_rows @ (a_row * g_row)", "b_rows @ a_row"),
    "unary term dropped": ("np.asarray(cand_u, dtype=np.float64) + b_rows", "0.0 * np.asarray(cand_u, dtype=np.float64) + b_rows"),
    "selector ties to the last slot": ("np.flatnonzero(s == s.max())[0]", "np.flatnonzero(s == s.max())[-1]"),
    "walk keeps the anchor as predecessor": ("a = int(cand_ids[n, j])", "a = a"),
    "gold forced into slot 0": ("kg = K - 1", "kg = 0"),
    "CE sign flipped": ("ce[n] = lse - s2[kg]", "ce[n] = s2[kg] - lse"),
    "gold outside the set always kept": ("elif force is not None and force[n]:", "elif True:"),
    "context projection transposed": ("return widen(h, dtype) @ widen(w_h, dtype).T", "return widen(h, dtype) @ widen(w_h, dtype).T[::-1]"),
    "Philox round multipliers swapped": ("p0 = np.uint64(_PHILOX_M[0]) * c0", "p0 = np.uint64(_PHILOX_M[1]) * c0"),
    "Philox key not advanced": ("k0 = (k0 + np.uint64(_PHILOX_W[0])) & mask", "k0 = k0"),
    "Gumbel noise with the wrong sign": ("return -np.log(-np.log(walk_uniform(", "return np.log(-np.log(walk_uniform("),
    "temperature multiplies the scores": ("z = s / temperature + gumbel_noise(", "z = s * temperature + gumbel_noise("),
    "sampled score reported with its noise": ("pscore[b, t] = s[j]\n            allz[b, t] = z", "pscore[b, t] = z[j]\n            allz[b, t] = z"),
    "noise shared by every slot": ("gumbel_noise(b, t, np.arange(K), seed)", "gumbel_noise(b, t, np.zeros(K, np.int64), seed)"),
    "backward drops the gold one-hot": ("d[kg] -= 1.0", "d[kg] -= 0.0"),
    "backward ignores the forced gold": ("ids[kg] = gold\n            u[kg] = float(", "ids[kg] = ids[kg]\n            u[kg] = float("),
    "backward ignores the upstream gradient": ("d *= float(grad_ce[n])", "d *= 1.0"),
    "predecessor gradient without the context": ("dA[p] += g[n] * v", "dA[p] += v"),
    "successor gradient sent to the predecessor row": ("np.add.at(dB, ids, d[:, None]", "np.add.at(dB, np.full_like(ids, p), d[:, None]"),
    "projection gradient against the wrong factor": ("dg[n] = A[p] * v", "dg[n] = g[n] * v"),
    "softcap before the multiplier": ("    x = np.asarray(U, dtype=np.float64) * float(output_multiplier)\n    if softcap > 0:\n        x = float(softcap) * np.tanh(x / float(softcap))", "    x = np.asarray(U, dtype=np.float64)\n    if softcap > 0:\n        x = float(softcap) * np.tanh(x / float(softcap))\n    x = x * float(output_multiplier)"),
    "softcap without the inner divide": ("x = float(softcap) * np.tanh(x / float(softcap))", "x = float(softcap) * np.tanh(x)"),
    "log-sum-exp without its shift added back": ("return m + np.log(np.exp(X - m[:, None]).sum(axis=1))", "return np.log(np.exp(X - m[:, None]).sum(axis=1))"),
    "target mass against the wrong normaliser": ("prob = np.exp(gl - lse)", "prob = np.exp(gl - lse) * U.shape[1] / (U.shape[1] + 1)"),
    "hit taken over the first candidate only": ("hit = (ids == g[:, None]).any(axis=1)", "hit = (ids[:, :1] == g[:, None]).any(axis=1)"),
    "backward keeps rows the forward excludes": ("        else:\n            continue\n        valid[n] = 1\n        ag", "        else:\n            pass\n        valid[n] = 1\n        ag"),
}


def _run(item):
    name, (old, new) = item
    env = dict(os.environ, DFLASH2_ORACLE_MUTANT=json.dumps([old, new]))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin():
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_run, MUTANTS.items()))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    broken = [(n, out) for n, rc, out in results if rc not in (0, 1)]
    assert not broken, broken
    assert not survivors, [n for n, _ in survivors]
