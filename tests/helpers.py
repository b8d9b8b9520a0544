"""Comparison protocol between the HIP library and the CPU oracle.

* Activations: float32 outputs within |gpu - ref| <= 2e-3 + 1e-3 |ref|; bf16
  outputs must be one of the two bf16 values that bracket the exact float64
  reference (one rounding, either way at a midpoint).
* Logits and scores: rtol 1e-3, atol 2e-3 against the oracle's exact value.
* Token ids: bit-exact, except near-ties (gap <= 1e-3 in the oracle's exact
  values) at a top-K boundary or a selector argmax, which are flagged, not
  failed.  The selector is checked stage-wise: the oracle scores the GPU's own
  candidate ids with its own exact unary logits, and replays the GPU's path so
  a flagged step cannot cascade.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import dflash2_oracle as O

RTOL, ATOL, TIE = 1e-3, 2e-3, 1e-3


def to_dev(a: np.ndarray, dtype: str = None, device="cuda") -> torch.Tensor:
    """numpy storage -> device tensor (uint16 arrays are bf16 bit patterns)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bracketed(gpu_bits: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """True where the bf16 value lies on the reference or is adjacent to it
    with no bf16 value strictly between."""
    g = O.widen(gpu_bits, "bf16")
    b = gpu_bits.astype(np.int64)
    up = ref > g
    neg = (b & 0x8000) != 0
    mag = b & 0x7FFF
    # one ulp from g toward ref, in sign-magnitude bf16
    toward_larger_mag = up != neg
    nmag = np.where(toward_larger_mag, mag + 1, mag - 1)
    crosses = nmag < 0  # stepping down from +-0 crosses to the other sign
    nb = np.where(crosses, (b ^ 0x8000) & 0x8000 | 1, (b & 0x8000) | np.maximum(nmag, 0))
    n = O.widen(nb.astype(np.uint16), "bf16")
    adjacent = np.where(up, n >= ref, n <= ref)
    return (g == ref) | adjacent


def act_ok(gpu: np.ndarray, ref: np.ndarray, dtype: str, delta: np.ndarray = None) -> np.ndarray:
    """Conv outputs.  bf16: the GPU value must be one of the two bf16 values
    bracketing the exact one, or the round-to-nearest-even of some value
    within delta of it (conv_delta: the float32 error the kernel's arithmetic
    can make).  Where the float32 error is below half a bf16 ulp this is the
    one-ulp bracket; where the taps nearly cancel a correct float32 sum can
    round one bf16 step further out."""
    if dtype == "f32":
        return np.abs(gpu.astype(np.float64) - ref) <= 2e-3 + 1e-3 * np.abs(ref)
    ok = bf16_bracketed(gpu, ref)
    if delta is None:
        return ok
    # the values a round-to-nearest-even of any x in [ref - d, ref + d] can take
    d = np.asarray(delta, np.float64)
    g = O.widen(gpu, "bf16")
    lo, hi = O.widen(O.round_bf16(ref - d), "bf16"), O.widen(O.round_bf16(ref + d), "bf16")
    return ok | ((g >= lo) & (g <= hi))


# Float32 error model of a conv output (x_out or y_out), used as delta above.
# The kernel forms the dynamic correction c = W x as a float32 sum of H
# products (exact bf16 products), then sum_j fma(base_j + c_j, v_{n-j}, acc)
# in float32.  Each of the 2T + 1 roundings of the tap chain (base + c, then
# each fma) is at most 2^-24 of the sum of the terms' magnitudes, S =
# sum_j |k_j v_{n-j}|; an error e_j in c_j adds |e_j| |v_{n-j}|.  A float32
# sum of H terms is taken as within CORR_ULPS ulps of the sum of their
# magnitudes, A_j = sum_h |W_jh x_h|; the GPU tests check that bound on the
# corrections the kernel returns (k_post, the other half of the same
# projection), so it is pinned, not assumed.  numpy's float32 product stays
# under 0.4 of those ulps at H = 4096 and 5120.
CORR_ULPS = 8


def corr_abs(x, w_proj, taps: int, group_size: int, dtype: str) -> np.ndarray:
    """A = sum_h |W_k[(s T + j) G + g, h] x[n, h]|  -> [N, 2, T, G] float64."""
    X, W = np.abs(O.widen(x, dtype)), np.abs(O.widen(w_proj, dtype))
    G = X.shape[1] // group_size
    return (X @ W.T).reshape(X.shape[0], 2, taps, G)


def corr_ok(gpu_corr, exact, absum) -> np.ndarray:
    """A float32 correction (k_post) within CORR_ULPS ulps of its terms' magnitudes."""
    return np.abs(np.asarray(gpu_corr, np.float64) - exact) <= CORR_ULPS * 2.0 ** -24 * absum


def conv_delta(v, corr, base_s, block_size: int, group_size: int, dtype: str, corr_absum=None) -> np.ndarray:
    """delta = (2T + 1) 2^-24 S + CORR_ULPS 2^-24 sum_j A_j |v_{n-j}| for each
    output, with the taps inside the block.  v and base_s in storage dtype,
    corr float [N, T, G] (the exact corrections, or the GPU's own k_post when
    it is fed to the oracle: then corr_absum is None and only the tap chain
    counts)."""
    Vv = np.abs(O.widen(v, dtype))
    Bs = O.widen(base_s, dtype)
    N, H = Vv.shape
    T = Bs.shape[0]
    gh = np.arange(H) // group_size
    C = np.asarray(corr, np.float64)
    S = np.zeros((N, H), np.float64)
    E = np.zeros((N, H), np.float64)
    for n in range(N):
        for j in range(min(T - 1, n % block_size) + 1):
            S[n] += np.abs(Bs[j] + C[n, j, gh]) * Vv[n - j]
            if corr_absum is not None:
                E[n] += np.asarray(corr_absum, np.float64)[n, j, gh] * Vv[n - j]
    return 2.0 ** -24 * ((2 * T + 1) * S + CORR_ULPS * E)


def close(gpu, ref, rtol=RTOL, atol=ATOL) -> np.ndarray:
    gpu = np.asarray(gpu, np.float64)
    return np.abs(gpu - ref) <= atol + rtol * np.abs(ref)


def scale_codebooks(inp, r, dtype):
    """Larger codebooks, so that the pair term overrides the unary pick on
    20-50 % of the steps against the N(0, 1) candidate logits (x6 at rank <= 64
    and in float32, x3 above): both terms then decide picks."""
    s = 6 if dtype == "f32" or r <= 64 else 3
    for k in ("cb_pred", "cb_succ"):
        inp[k] = inp[k] * np.float32(s) if dtype == "f32" else O.round_bf16(O.widen(inp[k], "bf16") * s)


def context_ok(gpu_g, h, w_h, dtype: str) -> np.ndarray:
    """The float32 context rows g = h W_Hᵀ (a sum of H products each) within
    CORR_ULPS ulps of the sum of their magnitudes, as the conv corrections."""
    exact = O.context_projection(h, w_h, dtype)
    absum = np.abs(O.widen(h, dtype)) @ np.abs(O.widen(w_h, dtype)).T
    return np.abs(np.asarray(gpu_g, np.float64) - exact) <= CORR_ULPS * 2.0 ** -24 * absum


def oracle_logits_rows(h: np.ndarray, w_lm: np.ndarray, dtype: str, chunk: int = 16384) -> np.ndarray:
    """The oracle's exact logits for a few rows, vocabulary chunk by chunk
    (keeps the float64 copy of a large LM head out of memory)."""
    V = w_lm.shape[0]
    out = np.empty((h.shape[0], V), np.float64)
    for v0 in range(0, V, chunk):
        out[:, v0:v0 + chunk] = O.lm_logits(h, w_lm[v0:v0 + chunk], dtype)
    return out


def compare_topk(gpu_ids, gpu_vals, U_rows, K):
    """gpu_ids/gpu_vals [n, K] for the rows whose exact logits are U_rows [n, V].
    Returns (fails, flags, messages)."""
    ref_ids, ref_vals = O.topk_of(U_rows, K)
    fails, flags, msgs = 0, 0, []
    V = U_rows.shape[1]
    for n in range(U_rows.shape[0]):
        g = gpu_ids[n]
        if np.any(g < 0) or np.any(g >= V) or len(set(g.tolist())) != K:
            fails += 1
            msgs.append(f"row {n}: invalid ids {g}")
            continue
        ug = U_rows[n, g]
        if not np.all(close(gpu_vals[n], ug)):
            fails += 1
            msgs.append(f"row {n}: values {gpu_vals[n]} vs exact {ug}")
            continue
        if np.array_equal(g, ref_ids[n]):
            continue
        kth = ref_vals[n, -1]
        missing = np.setdiff1d(ref_ids[n], g)
        ok = (ug.min() >= kth - TIE and np.all(ug[:-1] >= ug[1:] - TIE)
              and (missing.size == 0 or U_rows[n, missing].max() <= ug.min() + TIE))
        if ok:
            flags += 1
        else:
            fails += 1
            msgs.append(f"row {n}: ids {g} vs oracle {ref_ids[n]}")
    return fails, flags, msgs


def compare_walk(gpu_path, gpu_ps, g64, A, B, cand_ids, cand_u, anchors, bs, dtype, blocks=None):
    """Replays the GPU path through the oracle's transition scores.
    Returns (fails, flags, teeth, messages); teeth counts steps where the
    selector's pick differs from the unary argmax (slot 0)."""
    fails = flags = teeth = 0
    msgs = []
    blocks = range(gpu_path.shape[0]) if blocks is None else blocks
    for b in blocks:
        if gpu_path[b, 0] != anchors[b]:
            fails += 1
            msgs.append(f"block {b}: position 0 {gpu_path[b, 0]} != anchor {anchors[b]}")
            continue
        for t in range(1, bs):
            n = b * bs + t
            s = O.transition_scores(g64[n], A, B, int(gpu_path[b, t - 1]), cand_ids[n], cand_u[n], dtype)
            hits = np.flatnonzero(cand_ids[n] == gpu_path[b, t])
            if hits.size == 0:
                fails += 1
                msgs.append(f"block {b} t {t}: picked {gpu_path[b, t]} is not a candidate")
                continue
            jg, jo = int(hits[0]), O.first_argmax(s)
            teeth += jg != 0
            if jg != jo:
                if s[jo] - s[jg] <= TIE:
                    flags += 1
                else:
                    fails += 1
                    msgs.append(f"block {b} t {t}: slot {jg} (score {s[jg]}) vs oracle slot {jo} ({s[jo]})")
            if gpu_ps is not None and not close(gpu_ps[b, t], s[jg]):
                fails += 1
                msgs.append(f"block {b} t {t}: path score {gpu_ps[b, t]} vs {s[jg]}")
    return fails, flags, teeth, msgs


def compare_sample(gpu_path, gpu_ps, g64, A, B, cand_ids, cand_u, anchors, bs, dtype, temperature, seed):
    """Replays a sampled GPU path through the oracle: at each step the oracle's
    scores S for the GPU's predecessor, the noisy scores z = S / temperature +
    G (float64 Gumbel noise from the same generator), and the GPU's pick must
    be the first argmax of z, or within TIE / temperature + 1e-4 of it (the
    kernel forms S and the noise in float32: flagged, not failed).
    Returns (fails, flags, messages)."""
    fails = flags = 0
    msgs = []
    for b in range(gpu_path.shape[0]):
        if gpu_path[b, 0] != anchors[b]:
            fails += 1
            msgs.append(f"block {b}: position 0 {gpu_path[b, 0]} != anchor {anchors[b]}")
            continue
        for t in range(1, bs):
            n = b * bs + t
            s = O.transition_scores(g64[n], A, B, int(gpu_path[b, t - 1]), cand_ids[n], cand_u[n], dtype)
            z = s / temperature + O.gumbel_noise(b, t, np.arange(len(s)), seed)
            hits = np.flatnonzero(cand_ids[n] == gpu_path[b, t])
            if hits.size == 0:
                fails += 1
                msgs.append(f"block {b} t {t}: picked {gpu_path[b, t]} is not a candidate")
                continue
            jg, jo = int(hits[0]), O.first_argmax(z)
            if jg != jo:
                if z[jo] - z[jg] <= TIE / temperature + 1e-4:
                    flags += 1
                else:
                    fails += 1
                    msgs.append(f"block {b} t {t}: slot {jg} (z {z[jg]}) vs oracle slot {jo} ({z[jo]})")
            if gpu_ps is not None and not close(gpu_ps[b, t], s[jg]):
                fails += 1
                msgs.append(f"block {b} t {t}: path score {gpu_ps[b, t]} vs {s[jg]}")
    return fails, flags, msgs


def compare_tf(gpu, ref, cand_ids):
    """gpu/ref = (scores, best_ids, ce, valid) of the same rows."""
    gs, gb, gce, gv = gpu
    rs, rb, rce, rv = ref
    fails = flags = 0
    msgs = []
    bad = ~close(gs, rs)
    if bad.any():
        fails += int(bad.any(axis=1).sum())
        msgs.append(f"scores differ in rows {np.flatnonzero(bad.any(axis=1))[:10]}")
    for n in np.flatnonzero(gb != rb):
        hits = np.flatnonzero(cand_ids[n] == gb[n])
        jo = O.first_argmax(rs[n])
        if hits.size and rs[n, jo] - rs[n, hits[0]] <= TIE:
            flags += 1
        else:
            fails += 1
            msgs.append(f"row {n}: best {gb[n]} vs oracle {rb[n]}")
    if rv is not None:
        if not np.array_equal(gv, rv):
            fails += int((gv != rv).sum())
            msgs.append(f"valid differs in rows {np.flatnonzero(gv != rv)[:10]}")
        m = rv == 1
        badce = ~close(gce[m], rce[m])
        if badce.any():
            fails += int(badce.sum())
            msgs.append(f"ce differs: {gce[m][badce][:5]} vs {rce[m][badce][:5]}")
        if not np.all(gce[~m] == 0):
            fails += 1
            msgs.append("excluded rows carry a CE")
    return fails, flags, msgs


# Gradient tolerance.  The GPU sums in float32 (scores, softmax, atomics in
# any order, the MFMA contraction over rows): its error is ~1e-7 of the terms,
# at most ~1e-5 of the tensor's largest entry after N ~ 4096 row sums, and
# sums that cancel keep that absolute error.  So an entry passes within
# GRAD_RTOL of itself plus GRAD_SCALE_ATOL of the tensor's largest magnitude.
GRAD_RTOL, GRAD_SCALE_ATOL = 1e-3, 2e-5


def compare_grads(gpu: dict, ref: dict):
    """gpu/ref: name -> array.  Returns (fails, messages)."""
    fails, msgs = 0, []
    for k, r in ref.items():
        g = np.asarray(gpu[k], np.float64)
        scale = float(np.abs(r).max()) if r.size else 0.0
        ok = np.abs(g - r) <= GRAD_RTOL * np.abs(r) + GRAD_SCALE_ATOL * scale
        if not ok.all():
            bad = np.argwhere(~ok)
            fails += len(bad)
            i = tuple(bad[0])
            msgs.append(f"{k}: {len(bad)} entries off, e.g. {i}: {g[i]} vs {r[i]} (scale {scale})")
    return fails, msgs
