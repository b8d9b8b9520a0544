"""Seeded synthetic inputs for the DFlash2 draft-block head.

This module only draws random tensors and describes workload shapes.  It holds
none of the method's arithmetic, so the CPU oracle (under ``oracle/``) and the
HIP library can both consume exactly the same bytes.

Recipe (every workload, default seed 0):

* every field has its own ``torch.Generator`` seeded with
  ``seed * 1000 + field_index`` (field order below), so a field's values do not
  depend on which other fields were drawn;
* normal draws are torch's CPU ``randn`` in float32, scaled by the standard
  deviation (the second argument of ``N(mean, std)``) and shifted by the mean;
* bf16 workloads round each float32 draw to nearest-even once; both sides
  consume those bf16 bit patterns, kept here as ``uint16``;
* integer ids are torch ``randint`` on ``[0, vocab)``; the force mask is a
  Bernoulli(0.8) draw.

Field order and distributions (H hidden, V vocab, T taps, G = H / group_size,
r rank, N = n_blocks * block_size):

====  ==========  ==========  ==============================================
 idx  field       shape       distribution
====  ==========  ==========  ==============================================
  0   h           [N, H]      N(0, 1)           drafter hidden state
  1   y           [N, H]      N(0, 1)           a sublayer's output (finish input)
  2   w_lm        [V, H]      N(0, 1/sqrt(H))   shared LM head
  3   base        [2, T, H]   tap 0: 1 + N(0, 0.05); other taps N(0, 0.05)
  4   w_proj      [2TG, H]    N(0, 0.01 * sqrt(256/H))   conv kernel projection
  5   w_h         [r, H]      N(0, 0.05 * sqrt(256/H))   context projection H
  6   cb_pred     [V, r]      N(0, 0.05)        predecessor codebook A
  7   cb_succ     [V, r]      N(0, 0.05)        successor codebook B
  8   anchors     [n_blocks]  uniform ids       last verified token per block
  9   pred        [N]         uniform ids       teacher-forced predecessors
 10   gold        [N]         uniform ids       gold next tokens
 11   force       [N]         Bernoulli(0.8)    rows whose gold is forced in
====  ==========  ==========  ==============================================

The 1/sqrt(H) scaling keeps every projection that reads h variance-preserving
at any hidden size (at H = 256 it gives the tiny workload's own values).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and dtype of one synthetic workload."""

    name: str
    n_blocks: int
    block_size: int
    hidden: int
    vocab: int
    dtype: str  # "f32" or "bf16": activations and weights alike
    taps: int
    group_size: int
    rank: int
    top_k: int
    mode: str  # "walk", "tf" or "walk+tf"

    @property
    def n_rows(self) -> int:
        return self.n_blocks * self.block_size

    @property
    def groups(self) -> int:
        return self.hidden // self.group_size

    @property
    def proj_out(self) -> int:
        return 2 * self.taps * self.groups

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Workloads on Qwen3-shaped sizes.  Names state what they are and their sizes.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_fp32_16x8_h256_v4096", 16, 8, 256, 4096, "f32", 2, 16, 32, 16, "walk+tf"),
        Workload("decode_1x8_h4096_v151936", 1, 8, 4096, 151936, "bf16", 2, 16, 256, 16, "walk"),
        Workload("serve_64x8_h5120_v248320", 64, 8, 5120, 248320, "bf16", 2, 16, 256, 16, "walk"),
        Workload("packed_tf_512x8_h4096_v151936", 512, 8, 4096, 151936, "bf16", 2, 16, 256, 16, "tf"),
        Workload("wide_256x16_h5120_v248320_t8_k64", 256, 16, 5120, 248320, "bf16", 8, 32, 512, 64, "walk"),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)

FIELDS = ["h", "y", "w_lm", "base", "w_proj", "w_h", "cb_pred", "cb_succ",
          "anchors", "pred", "gold", "force"]


def _gen(seed: int, field: str) -> torch.Generator:
    return torch.Generator().manual_seed(seed * 1000 + FIELDS.index(field))


def _normal(seed: int, field: str, shape, std: float, mean: float = 0.0) -> torch.Tensor:
    t = torch.randn(*shape, generator=_gen(seed, field), dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t


def to_storage(t: torch.Tensor, dtype: str) -> np.ndarray:
    """float32 tensor -> numpy storage: float32, or bf16 bit patterns as uint16
    (one round-to-nearest-even, done by torch's own conversion)."""
    if dtype == "f32":
        return t.numpy()
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, seed: int = 0, fields=None) -> Dict[str, np.ndarray]:
    """Draw the named fields (all by default) of workload ``w``.

    Float fields come back as numpy float32 (``w.dtype == "f32"``) or uint16
    bf16 bit patterns; ids as int32; the force mask as uint8.
    """
    want = FIELDS if fields is None else list(fields)
    N, H, V, T, G, r = w.n_rows, w.hidden, w.vocab, w.taps, w.groups, w.rank
    s = math.sqrt(256.0 / H)
    out: Dict[str, np.ndarray] = {}
    for f in want:
        if f == "h":
            t = _normal(seed, f, (N, H), 1.0)
        elif f == "y":
            t = _normal(seed, f, (N, H), 1.0)
        elif f == "w_lm":
            t = _normal(seed, f, (V, H), 1.0 / math.sqrt(H))
        elif f == "base":
            t = _normal(seed, f, (2, T, H), 0.05)
            t[:, 0, :] += 1.0
        elif f == "w_proj":
            t = _normal(seed, f, (2 * T * G, H), 0.01 * s)
        elif f == "w_h":
            t = _normal(seed, f, (r, H), 0.05 * s)
        elif f in ("cb_pred", "cb_succ"):
            t = _normal(seed, f, (V, r), 0.05)
        elif f == "anchors":
            out[f] = torch.randint(0, V, (w.n_blocks,), generator=_gen(seed, f)).numpy().astype(np.int32)
            continue
        elif f in ("pred", "gold"):
            out[f] = torch.randint(0, V, (N,), generator=_gen(seed, f)).numpy().astype(np.int32)
            continue
        elif f == "force":
            u = torch.rand(N, generator=_gen(seed, f))
            out[f] = (u < 0.8).numpy().astype(np.uint8)
            continue
        else:
            raise KeyError(f)
        out[f] = to_storage(t, w.dtype)
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact widening)."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def small_workload(base: Optional[Workload] = None, **kw) -> Workload:
    """A reduced workload for parity tests (shape overrides on top of ``base``)."""
    b = base if base is not None else WORKLOADS["tiny_fp32_16x8_h256_v4096"]
    return b.scaled(name=kw.pop("name", b.name + "_scaled"), **kw)
