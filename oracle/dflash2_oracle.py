"""CPU oracle for the DFlash2 draft-block head.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import or run this module; the
library never routes through it.  It shares no code with the HIP library and
imports nothing from it.

Plain numpy, every sum taken in float64.  bf16 inputs arrive as uint16 bit
patterns and are widened exactly; float32 inputs are widened exactly.  For
bf16 x bf16 products float64 is exact and the summation error is ~1e-16
relative, so the results here stand for the exact values of the definitions.

Sources (cited by page title and section):

* [Speculators]  "DFlash2" page of the vLLM Speculators user guide
  (sections "Local Convolution", "Candidate Selector", "Training Objective",
  "Key Parameters").
* [SpecForge]    "DFlash2" concept page of the SpecForge docs
  (sections "Architecture", the ``dflash_config`` JSON and its validity rules,
  "Selector objective and schedule").
* [verl PR]      "feat: add DFlash2 drafter training backend" (verl-SpeCo pull
  request 62; sections "What DFlash2 adds", "Two deltas over the upstream
  inference implementation", "Selector training objective", "Real-data
  ablation").
* [Explainer]    "DFlash 2 Explanation" (sections "Component Breakdown",
  "Problem 1 - Independent picks are incoherent", "Problem 2 - Suffix decay is
  local", the "One Cycle, Step by Step" sequence diagram).

Readings taken where the pages leave a step open are marked READING below.
Pins that tie each function to the pages live in ``tests/test_oracle_*.py``;
every function here is pinned (none is "parity unpinned") except the absolute
values of random-input scores, which rest on the definitions themselves.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

DTYPES = ("f32", "bf16")

# Precision the storage arrays are widened to, and so of every sum.  float64
# is the oracle.  The benchmark's second CPU line times the same steps with
# float32 sums by setting this to np.float32 around its calls; no pin and no
# parity test ever runs with anything but float64.
ACC = np.float64


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64 (ACC), exactly.  bf16 is the high half of a float32."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(ACC)
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(ACC)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), one round-to-nearest-even.

    Rounds straight from float64 (no detour through float32, which could round
    twice).  bf16 keeps 8 significant bits and float32's exponent range, so the
    quantum of a value in [2^(e-1), 2^e) is 2^(e-8), never below 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)  # np.rint: ties to even
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    y = np.where(np.abs(y) > big, np.copysign(np.inf, y), y)
    y = np.where(np.isfinite(x), y, x)
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage dtype, one round-to-nearest-even (READING: the conv
    computes exactly and rounds its output once; the pages fix no precision)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# configuration rules and parameter shapes
# --------------------------------------------------------------------------

def check_config(hidden: int, vocab: int, block_size: int, taps: int,
                 group_size: int, rank: int, top_k: int) -> None:
    """The DFlash2 draft-config validity rules ([SpecForge], the rules under
    the ``dflash_config`` JSON): taps in [1, block_size], group size divides
    hidden, rank >= 1, top-K in [1, vocab]."""
    if block_size < 1:
        raise ValueError("block_size must be positive")
    if not (1 <= taps <= block_size):
        raise ValueError("conv_kernel_size must be in [1, block_size]")
    if group_size < 1 or hidden % group_size != 0:
        raise ValueError("conv_group_size must divide hidden_size")
    if rank < 1:
        raise ValueError("selector_rank must be positive")
    if not (1 <= top_k <= vocab):
        raise ValueError("selector_top_k must be in [1, vocab_size]")


def param_shapes(hidden: int, vocab: int, taps: int, group_size: int,
                 rank: int) -> Dict[str, Tuple[int, ...]]:
    """Shapes of the DFlash2 parameters this oracle accepts.

    * one conv wrapper: a bias-free projection from the hidden state to
      2*T*G dynamic coefficients (pre and post kernels from one projection,
      [verl PR] "What DFlash2 adds"; [Speculators] "Local Convolution") and a
      per-channel base kernel for each of the two convolutions;
    * the selector: a bias-free context projection H of width r and two
      materialised [V, r] codebooks ([Speculators] "Training Objective").

    These are pinned by the trainable-parameter counts of the [verl PR]
    "Real-data ablation" table.
    """
    G = hidden // group_size
    return {
        "conv.w_proj": (2 * taps * G, hidden),
        "conv.base": (2, taps, hidden),
        "selector.w_h": (rank, hidden),
        "selector.cb_pred": (vocab, rank),
        "selector.cb_succ": (vocab, rank),
    }


def _need_shape(name: str, a: np.ndarray, shape) -> None:
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(a.shape)} != {tuple(shape)}")


def _check_blocked(n_rows: int, block_size: int) -> int:
    """The draft length must be a whole number of blocks, else raise
    ([verl PR] "Two deltas ...", item 1)."""
    if block_size < 1 or n_rows % block_size != 0:
        raise ValueError("draft length is not a multiple of block_size")
    return n_rows // block_size


# --------------------------------------------------------------------------
# a1-a3: grouped dynamic causal convolution
# --------------------------------------------------------------------------

def conv_projection(x: np.ndarray, w_proj: np.ndarray, taps: int,
                    group_size: int, dtype: str) -> np.ndarray:
    """Dynamic corrections c[n, s, j, g] = sum_h W[(s*T + j)*G + g, h] x[n, h].

    s = 0 is the kernel for the sublayer input, s = 1 the one for its output
    ([Speculators] "Local Convolution": one projection of the current hidden
    state gives both).  READING: linear, no bias, no activation; the row
    layout (s, j, g) is this library's own.
    """
    X = widen(x, dtype)
    N, H = X.shape
    G = H // group_size
    _need_shape("w_proj", w_proj, (2 * taps * G, H))
    c = X @ widen(w_proj, dtype).T
    return c.reshape(N, 2, taps, G)


def depthwise_taps(v: np.ndarray, corr: np.ndarray, base_s: np.ndarray,
                   block_size: int, group_size: int) -> np.ndarray:
    """out[n, h] = sum_{j <= min(T-1, p(n))} (base_s[j, h] + corr[n, j, h // gs]) * v[n - j, h].

    The two-tap form k_{t,0} x_t + k_{t,1} x_{t-1} ([verl PR] "What DFlash2
    adds"; [Explainer] "Problem 2") generalised to T taps.  p(n) = n mod bs is
    the position inside the anchor block; a tap that would reach before the
    block start reads zero, so no tap crosses a block ([verl PR] "Two deltas",
    item 1; [Speculators] "Local Convolution").  The kernel at output row n is
    built from row n's own correction (READING of "computed from the current
    hidden state", [Explainer] "Problem 2").  Channels of one contiguous group
    of gs share the correction ([verl PR] "What DFlash2 adds").
    """
    N, H = v.shape
    T = base_s.shape[0]
    g_of_h = np.arange(H) // group_size
    out = np.zeros((N, H), dtype=np.float64)
    for n in range(N):
        p = n % block_size
        for j in range(min(T - 1, p) + 1):
            k = base_s[j] + corr[n, j, g_of_h]
            out[n] += k * v[n - j]
    return out


def conv_prepare(x, w_proj, base, block_size: int, taps: int, group_size: int,
                 dtype: str):
    """Pre-sublayer half of the wrapper: returns (x_out in storage dtype,
    k_post float64 [N, T, G], x_out float64 before rounding).

    ``prepare`` convolves the sublayer input and also hands ``finish`` the
    dynamic part of the output kernel ([verl PR] "What DFlash2 adds").
    """
    X = widen(x, dtype)
    N, H = X.shape
    _check_blocked(N, block_size)
    check_config(H, 1, block_size, taps, group_size, 1, 1)
    _need_shape("base", base, (2, taps, H))
    c = conv_projection(x, w_proj, taps, group_size, dtype)
    exact = depthwise_taps(X, c[:, 0], widen(base, dtype)[0], block_size, group_size)
    return round_to(exact, dtype), c[:, 1].copy(), exact


def conv_finish(y, k_post, base, block_size: int, taps: int, group_size: int,
                dtype: str):
    """Post-sublayer half: returns (y_out in storage dtype, y_out float64).

    Applies base[1] + k_post to the sublayer output y with the same block-local
    taps.  ``k_post`` may be float64 or float32; it is widened exactly.
    """
    Y = widen(y, dtype)
    N, H = Y.shape
    _check_blocked(N, block_size)
    check_config(H, 1, block_size, taps, group_size, 1, 1)
    _need_shape("base", base, (2, taps, H))
    _need_shape("k_post", k_post, (N, taps, H // group_size))
    exact = depthwise_taps(Y, np.asarray(k_post, dtype=np.float64),
                           widen(base, dtype)[1], block_size, group_size)
    return round_to(exact, dtype), exact


# --------------------------------------------------------------------------
# a4-a5: unary logits and per-position top-K
# --------------------------------------------------------------------------

def lm_logits(h, w_lm, dtype: str) -> np.ndarray:
    """U[n, v] = <h[n], W_lm[v]> over the full vocabulary: the shared LM head's
    raw logits ([Explainer] "Component Breakdown"; [Speculators] requires the
    full verifier vocabulary).  READING: raw logits, no softmax or transform."""
    return widen(h, dtype) @ widen(w_lm, dtype).T


def logits_at(h, w_lm, ids: np.ndarray, dtype: str) -> np.ndarray:
    """U[n, ids[n, k]] for given ids, one exact dot product each."""
    Hm = widen(h, dtype)
    ids = np.asarray(ids)
    out = np.empty(ids.shape, dtype=np.float64)
    for n in range(ids.shape[0]):
        out[n] = widen(w_lm[ids[n]], dtype) @ Hm[n]
    return out


def topk_of(U: np.ndarray, top_k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per row, the top_k entries ordered by value descending, lower id first
    on exact ties (READING: the pages fix no tie order)."""
    N, V = U.shape
    ids = np.empty((N, top_k), dtype=np.int32)
    vals = np.empty((N, top_k), dtype=np.float64)
    vid = np.arange(V)
    for n in range(N):
        order = np.lexsort((vid, -U[n]))[:top_k]
        ids[n] = order
        vals[n] = U[n, order]
    return ids, vals


def unary_topk(h, w_lm, top_k: int, dtype: str, gold_ids=None):
    """Candidate lattice: selector_top_k candidates per position from the
    unary logits ([Speculators] "Candidate Selector"; [Explainer] "Problem 1").

    Returns (ids int32 [N, K], vals float64 [N, K], gold_logit float64 [N] or
    None, where gold_logit[n] = U[n, gold_ids[n]]).
    """
    U = lm_logits(h, w_lm, dtype)
    if not (1 <= top_k <= U.shape[1]):
        raise ValueError("selector_top_k must be in [1, vocab_size]")
    ids, vals = topk_of(U, top_k)
    gl = None
    if gold_ids is not None:
        g = np.asarray(gold_ids)
        gl = U[np.arange(U.shape[0]), g]
    return ids, vals, gl


# --------------------------------------------------------------------------
# a6-a10: candidate selector
# --------------------------------------------------------------------------

def context_projection(h, w_h, dtype: str) -> np.ndarray:
    """g[n] = H(h_n) = W_H h_n ([verl PR] "What DFlash2 adds": H projects the
    backbone hidden state).  READING: linear, no bias, no gate nonlinearity."""
    return widen(h, dtype) @ widen(w_h, dtype).T


def transition_scores(g_row, cb_pred, cb_succ, pred_id, cand_ids, cand_u, dtype):
    """S(a, b) = U(b) + <A(a) * H(h), B(b)> for one predecessor a and the
    candidate ids b ([verl PR] "What DFlash2 adds", selector equation;
    [Explainer] "Problem 1"; [Speculators] "Candidate Selector")."""
    a_row = widen(cb_pred[pred_id], dtype)
    b_rows = widen(cb_succ[np.asarray(cand_ids)], dtype)
    return np.asarray(cand_u, dtype=np.float64) + b_rows @ (a_row * g_row)


def first_argmax(s: np.ndarray) -> int:
    """Index of the maximum, lowest index on ties (READING: the lowest slot,
    i.e. the higher unary candidate, wins an exact tie)."""
    return int(np.flatnonzero(s == s.max())[0])


def selector_walk(g, cb_pred, cb_succ, cand_ids, cand_u, anchors, block_size: int,
                  dtype: str, return_scores: bool = False):
    """Greedy path per anchor block.

    Position 0 holds the anchor, the last verified token ([Explainer]
    "Component Breakdown", block attention mask).  For t = 1 .. bs-1 the token
    picked at t-1 is the predecessor and the best-scoring candidate of row t is
    picked ([Speculators] "Candidate Selector"; [Explainer] sequence diagram:
    candidate lists plus last verified token in, one path out).

    Returns (path int32 [n_b, bs] with path[:, 0] = anchor, path_score float64
    [n_b, bs] with 0 at position 0[, scores float64 [n_b, bs, K], row 0 zero]).
    """
    cand_ids = np.asarray(cand_ids)
    N, K = cand_ids.shape
    nb = _check_blocked(N, block_size)
    anchors = np.asarray(anchors)
    _need_shape("anchors", anchors, (nb,))
    path = np.zeros((nb, block_size), dtype=np.int32)
    pscore = np.zeros((nb, block_size), dtype=np.float64)
    allsc = np.zeros((nb, block_size, K), dtype=np.float64)
    for b in range(nb):
        a = int(anchors[b])
        path[b, 0] = a
        for t in range(1, block_size):
            n = b * block_size + t
            s = transition_scores(g[n], cb_pred, cb_succ, a, cand_ids[n], cand_u[n], dtype)
            j = first_argmax(s)
            a = int(cand_ids[n, j])
            path[b, t] = a
            pscore[b, t] = s[j]
            allsc[b, t] = s
    if return_scores:
        return path, pscore, allsc
    return path, pscore


def selector_score_tf(g, cb_pred, cb_succ, cand_ids, cand_u, pred_ids,
                      dtype: str, gold_ids=None, force=None, gold_logit=None):
    """Teacher-forced scoring of every row in one shot ([verl PR] "Selector
    training objective": the predecessor is the given previous token).

    * scores[n, k] = S(pred[n], cand[n, k]) over the strict candidate set, and
      best_ids[n] its first argmax.
    * With gold ids: the forced set C' replaces the weakest slot K-1 by
      (gold, U(gold)) when force[n] and gold is not in C ([Speculators]
      "Training Objective"); other rows whose gold is outside C are excluded
      ([SpecForge] "Selector objective and schedule"; [verl PR]).  READING:
      both rules, chosen per row by ``force``.  valid[n] = gold in C', and
      ce[n] = logsumexp_k S'[n, k] - S'[n, k_gold] (0 where not valid).

    Returns (scores [N, K], best_ids [N], ce [N] or None, valid [N] or None).
    """
    cand_ids = np.asarray(cand_ids)
    N, K = cand_ids.shape
    scores = np.empty((N, K), dtype=np.float64)
    best = np.empty(N, dtype=np.int32)
    ce = valid = None
    if gold_ids is not None:
        ce = np.zeros(N, dtype=np.float64)
        valid = np.zeros(N, dtype=np.uint8)
        if force is not None and gold_logit is None:
            raise ValueError("forcing the gold id needs its logit")
    for n in range(N):
        p = int(pred_ids[n])
        s = transition_scores(g[n], cb_pred, cb_succ, p, cand_ids[n], cand_u[n], dtype)
        scores[n] = s
        best[n] = cand_ids[n, first_argmax(s)]
        if gold_ids is None:
            continue
        gold = int(gold_ids[n])
        hits = np.flatnonzero(cand_ids[n] == gold)
        s2 = s.copy()
        if hits.size:
            kg = int(hits[0])
        elif force is not None and force[n]:
            kg = K - 1
            s2[kg] = transition_scores(g[n], cb_pred, cb_succ, p, [gold],
                                       [gold_logit[n]], dtype)[0]
        else:
            continue
        m = s2.max()
        lse = m + np.log(np.sum(np.exp(s2 - m)))
        ce[n] = lse - s2[kg]
        valid[n] = 1
    return scores, best, ce, valid


# --------------------------------------------------------------------------
# sampling walk
# --------------------------------------------------------------------------
#
# [Explainer] "Problem 1 - Independent picks are incoherent" (the paragraph
# after the selector equation) and the "Draft-Verify Cycle" flowchart (the
# walk node): besides the greedy walk, the path may be sampled from the same
# scores.  The pages fix no distribution or generator.  READINGS:
#   * a_t is drawn from softmax over the candidates of row t of
#     S_t(a_{t-1}, .) / temperature (temperature 1: the scores as they are);
#   * the draw is the Gumbel-max form: the first argmax over j of
#     S_t(a_{t-1}, c_{t,j}) / temperature + G[b, t, j], with G standard
#     Gumbel noise (Gumbel-max: this argmax is distributed exactly as the
#     softmax draw), so, as in the greedy walk, every predecessor's pick is
#     defined before the path is known;
#   * G[b, t, j] = -log(-log(u)) with u = (x / 256 + 1/2) / 2^24, x the first
#     word of Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
#     numbers: as easy as 1, 2, 3", SC 2011) at counter (j, t, b, 0) under the
#     key (seed mod 2^32, seed / 2^32): one counter-based generator, defined
#     by its publication and implemented separately on each side.

_PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # round multipliers
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # key schedule (Weyl) increments


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds (the SC 2011 definition): each round takes
    (c0, c1, c2, c3) to (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
    lo(M0 c0)) and the key advances by the Weyl constants between rounds.
    counter: uint array [..., 4]; key: uint array [..., 2] (broadcast).
    Returns uint32 [..., 4]."""
    c = np.asarray(counter, dtype=np.uint64) & 0xFFFFFFFF
    k = np.asarray(key, dtype=np.uint64) & 0xFFFFFFFF
    c0, c1, c2, c3 = (c[..., i] for i in range(4))
    k0, k1 = k[..., 0], k[..., 1]
    mask = np.uint64(0xFFFFFFFF)
    for r in range(10):
        p0 = np.uint64(_PHILOX_M[0]) * c0   # exact: a 32 x 32-bit product fits 64 bits
        p1 = np.uint64(_PHILOX_M[1]) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + np.uint64(_PHILOX_W[0])) & mask
        k1 = (k1 + np.uint64(_PHILOX_W[1])) & mask
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def walk_uniform(block: int, t: int, slots, seed: int) -> np.ndarray:
    """u[j] in (0, 1) for the given slots of position t of anchor block
    `block` (READING above): 24 bits of the first Philox word, centred."""
    slots = np.asarray(slots, dtype=np.uint64)
    ctr = np.stack([slots, np.full_like(slots, t), np.full_like(slots, block), np.zeros_like(slots)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    x = philox4x32_10(ctr, key)[..., 0].astype(np.float64)
    return (np.floor(x / 256.0) + 0.5) / 2.0 ** 24


def gumbel_noise(block: int, t: int, slots, seed: int) -> np.ndarray:
    """Standard Gumbel noise -log(-log(u)) for the given slots."""
    return -np.log(-np.log(walk_uniform(block, t, slots, seed)))


def selector_sample(g, cb_pred, cb_succ, cand_ids, cand_u, anchors, block_size: int,
                    dtype: str, temperature: float, seed: int, return_scores: bool = False):
    """Sampled path per anchor block: as selector_walk, with the pick at t the
    first argmax of S_t(a_{t-1}, .) / temperature + G[b, t, .] (READINGS above).
    path_score holds the picked candidate's S (without the noise).

    Returns (path int32 [n_b, bs], path_score float64 [n_b, bs][, z float64
    [n_b, bs, K]: the noisy scores the picks maximise])."""
    if not temperature > 0:
        raise ValueError("temperature must be positive")
    cand_ids = np.asarray(cand_ids)
    N, K = cand_ids.shape
    nb = _check_blocked(N, block_size)
    anchors = np.asarray(anchors)
    _need_shape("anchors", anchors, (nb,))
    path = np.zeros((nb, block_size), dtype=np.int32)
    pscore = np.zeros((nb, block_size), dtype=np.float64)
    allz = np.zeros((nb, block_size, K), dtype=np.float64)
    for b in range(nb):
        a = int(anchors[b])
        path[b, 0] = a
        for t in range(1, block_size):
            n = b * block_size + t
            s = transition_scores(g[n], cb_pred, cb_succ, a, cand_ids[n], cand_u[n], dtype)
            z = s / temperature + gumbel_noise(b, t, np.arange(K), seed)
            j = first_argmax(z)
            a = int(cand_ids[n, j])
            path[b, t] = a
            pscore[b, t] = s[j]
            allz[b, t] = z
    if return_scores:
        return path, pscore, allz
    return path, pscore


# --------------------------------------------------------------------------
# selector CE backward
# --------------------------------------------------------------------------
#
# [verl PR] "Selector training objective": the selector's inputs are
# detached, so its CE trains only its own parameters; [SpecForge] "Selector
# objective and schedule" (the stop-gradient switch detaches both inputs,
# the unary logits and the hidden states).  With L = sum_n w[n] CE[n] over the
# rows that carry a CE (w the upstream gradient dL/dCE[n]) and d[n, k] =
# w[n] (softmax(S'[n])_k - [k = k_gold]) on the forced set C' of
# selector_score_tf:
#   dL/dB[c'_k]   += d[n, k] (A[p_n] * g[n])
#   dL/dA[p_n]    += g[n] * v[n],          v[n] = sum_k d[n, k] B[c'_k]
#   dL/dg[n]       = A[p_n] * v[n]
#   dL/dW_H        = sum_n dL/dg[n] (outer) h[n]      (g = W_H h)
# READING: h and U (the forced gold's logit included) are constants.

def selector_ce_backward(h, w_h, cb_pred, cb_succ, cand_ids, cand_u, pred_ids, dtype: str,
                         gold_ids, force, gold_logit, grad_ce):
    """Gradients of sum_n grad_ce[n] CE[n] (the CE of selector_score_tf) with
    respect to the predecessor codebook A, the successor codebook B and the
    context projection W_H.  Returns (dA [V, r], dB [V, r], dW_H [r, H],
    dg [N, r], valid [N]) in float64."""
    cand_ids = np.asarray(cand_ids)
    N, K = cand_ids.shape
    g = context_projection(h, w_h, dtype)
    A, B = widen(cb_pred, dtype), widen(cb_succ, dtype)
    dA, dB = np.zeros_like(A), np.zeros_like(B)
    dg = np.zeros_like(g)
    valid = np.zeros(N, dtype=np.uint8)
    for n in range(N):
        p = int(pred_ids[n])
        ids = cand_ids[n].astype(np.int64).copy()
        u = np.asarray(cand_u[n], dtype=np.float64).copy()
        gold = int(gold_ids[n])
        hits = np.flatnonzero(ids == gold)
        if hits.size:
            kg = int(hits[0])
        elif force is not None and force[n]:
            kg = K - 1
            ids[kg] = gold
            u[kg] = float(gold_logit[n])
        else:
            continue
        valid[n] = 1
        ag = A[p] * g[n]
        s = u + B[ids] @ ag
        e = np.exp(s - s.max())
        d = e / e.sum()
        d[kg] -= 1.0
        d *= float(grad_ce[n])
        v = d @ B[ids]
        dg[n] = A[p] * v
        dA[p] += g[n] * v
        np.add.at(dB, ids, d[:, None] * ag[None, :])
    dW = dg.T @ widen(h, dtype)
    return dA, dB, dW, dg, valid


# --------------------------------------------------------------------------
# unary-logit transforms and candidate metrics
# --------------------------------------------------------------------------
#
# [SpecForge] "Export and serve": the optional output_multiplier and
# final_logit_softcapping of the draft config act on the unary logits, in
# local generation and in serving alike.  The page names them and fixes no
# formula.  READINGS:
#   * the multiplier scales the raw logit; the softcap then maps x to
#     c tanh(x / c) (c > 0; 0 = off), so that the cap bounds the final logits;
#   * candidates, their values and the gold logit are those of the
#     transformed logits (the transform is increasing for a positive
#     multiplier, so it never reorders distinct logits).
# [Explainer] "Problem 1" (recall@1 / recall@16 per position) and
# [SpecForge] "Selector objective and schedule" (selector_coverage: how often
# the gold is in the strict unary top-k set): hit[n] = [gold in top-K].
# [verl PR] "What DFlash2 adds" (validation reports unary candidate recall
# and target mass): READING: the target mass is the unary softmax
# probability of the gold token over the full vocabulary,
# exp(U'(gold) - logsumexp_v U'(v)).

def transform_logits(U, output_multiplier: float = 1.0, softcap: float = 0.0) -> np.ndarray:
    """U' = softcap(output_multiplier * U), softcap(x) = c tanh(x / c) for
    c > 0 and the identity for c = 0."""
    x = np.asarray(U, dtype=np.float64) * float(output_multiplier)
    if softcap > 0:
        x = float(softcap) * np.tanh(x / float(softcap))
    return x


def logsumexp_rows(X: np.ndarray) -> np.ndarray:
    """log sum_v exp(X[n, v]) per row, shifted by the row maximum."""
    m = X.max(axis=1)
    return m + np.log(np.exp(X - m[:, None]).sum(axis=1))


def unary_topk_ex(h, w_lm, top_k: int, dtype: str, gold_ids=None, output_multiplier: float = 1.0,
                  softcap: float = 0.0):
    """The candidate lattice over the transformed logits, with the metrics
    of the same pass.  Returns (ids [N, K], vals [N, K], lse [N], gold_logit,
    gold_prob, hit), the last three None without gold ids."""
    if not (output_multiplier > 0 and np.isfinite(output_multiplier)):
        raise ValueError("output_multiplier must be positive and finite")
    if not (softcap >= 0 and np.isfinite(softcap)):
        raise ValueError("final_logit_softcapping must be >= 0 and finite")
    U = transform_logits(lm_logits(h, w_lm, dtype), output_multiplier, softcap)
    if not (1 <= top_k <= U.shape[1]):
        raise ValueError("selector_top_k must be in [1, vocab_size]")
    ids, vals = topk_of(U, top_k)
    lse = logsumexp_rows(U)
    gl = prob = hit = None
    if gold_ids is not None:
        g = np.asarray(gold_ids)
        gl = U[np.arange(U.shape[0]), g]
        prob = np.exp(gl - lse)
        hit = (ids == g[:, None]).any(axis=1).astype(np.uint8)
    return ids, vals, lse, gl, prob, hit
