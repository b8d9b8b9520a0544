"""Python binding of libdflash2.so (the DFlash2 draft-block head for gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch device tensors; outputs and workspaces are allocated with
torch (device memory is torch's), and work goes on torch's current stream.
The names mirror the C entry points declared in include/dflash2.h.
There is no fallback: if the library is not built, importing raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

# DFLASH2_LIBRARY names another build of the same ABI (the host-only,
# sanitizer-instrumented build the ABI tests load); default: the in-tree one.
_LIB_PATH = os.environ.get("DFLASH2_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                              "libdflash2.so")

STATUS = {
    0: "DFLASH2_OK", 1: "DFLASH2_ERR_NULL", 2: "DFLASH2_ERR_SHAPE", 3: "DFLASH2_ERR_DTYPE",
    4: "DFLASH2_ERR_UNSUPPORTED", 5: "DFLASH2_ERR_ALIAS", 6: "DFLASH2_ERR_WORKSPACE",
    7: "DFLASH2_ERR_LAUNCH", 8: "DFLASH2_ERR_DEVICE_ID_RANGE",
}
OP_UNARY_TOPK, OP_SELECTOR_WALK, OP_SELECTOR_TF, OP_SELECTOR_CE_BACKWARD, OP_DECODE_HEAD = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
MAX_TOP_K, MAX_TAPS, MAX_BLOCK_SIZE, MAX_RANK = 64, 16, 64, 4096
NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024 + 256

EXPORTS = ["dflash2_conv_prepare", "dflash2_conv_finish", "dflash2_unary_topk", "dflash2_unary_topk_ex",
           "dflash2_selector_walk", "dflash2_selector_walk_noalloc", "dflash2_selector_sample", "dflash2_selector_score_tf",
           "dflash2_selector_ce_backward", "dflash2_decode_head", "dflash2_workspace_bytes",
           "dflash2_status_str", "dflash2_read_device_status", "dflash2_debug_force_slabs", "dflash2_version"]


class DFlash2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_str(status)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m block_draft_head_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "dflash2_conv_prepare": [ctypes.c_int, I64, I32, I32, I32, I32, P, P, P, P, P, P],
        "dflash2_conv_finish": [ctypes.c_int, I64, I32, I32, I32, I32, P, P, P, P, P],
        "dflash2_unary_topk": [ctypes.c_int, I64, I32, I32, I32, P, P, P, P, P, P, P, SZ, P],
        "dflash2_unary_topk_ex": [ctypes.c_int, I64, I32, I32, I32, P, P, P, ctypes.c_float, ctypes.c_float, P, I32,
                                  P, P, P, P, P, P, P, P, SZ, P],
        "dflash2_selector_walk": [ctypes.c_int, I32, I32, I32, I32, I32, I32] + [P] * 11 + [SZ, P],
        "dflash2_selector_walk_noalloc": [ctypes.c_int, I32, I32, I32, I32, I32, I32] + [P] * 11,
        "dflash2_selector_sample": [ctypes.c_int, I32, I32, I32, I32, I32, I32] + [P] * 8 +
                                   [ctypes.c_float, ctypes.c_uint64, P, P, P, SZ, P],
        "dflash2_selector_score_tf": [ctypes.c_int, I64, I32, I32, I32, I32] + [P] * 16 + [SZ, P],
        "dflash2_selector_ce_backward": [ctypes.c_int, I64, I32, I32, I32, I32] + [P] * 16 + [P, SZ, P],
        "dflash2_decode_head": [ctypes.c_int, I32, I32, I32, I32, I32, I32] + [P] * 10 + [P, SZ, P],
        "dflash2_workspace_bytes": [ctypes.c_int, I64, I32, I32, I32, I32],
        "dflash2_status_str": [ctypes.c_int],
        "dflash2_read_device_status": [P, P],
        "dflash2_debug_force_slabs": [I32],
        "dflash2_version": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.dflash2_workspace_bytes.restype = SZ
    lib.dflash2_status_str.restype = ctypes.c_char_p
    lib.dflash2_version.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib_path() -> str:
    return _LIB_PATH


def version() -> str:
    return _lib.dflash2_version().decode()


def status_str(status: int) -> str:
    return _lib.dflash2_status_str(int(status)).decode()


def debug_force_slabs(n_slabs: int) -> None:
    """Fixes the LM-head kernels' vocabulary slab count (0 = automatic); a
    determinism knob.  Size workspaces after changing it."""
    _check(_lib.dflash2_debug_force_slabs(int(n_slabs)), "dflash2_debug_force_slabs")


def workspace_bytes(op: int, n_rows: int, hidden: int = 0, vocab: int = 0, rank: int = 0, top_k: int = 0) -> int:
    return int(_lib.dflash2_workspace_bytes(op, n_rows, hidden, vocab, rank, top_k))


# ---------------------------------------------------------------- helpers

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DFlash2Error(status, where)


def _same_dtype(ref: torch.Tensor, *ts: torch.Tensor) -> None:
    for t in ts:
        if t.dtype != ref.dtype:
            raise TypeError(f"dtype mismatch: {t.dtype} vs {ref.dtype}")


def _ids(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return t


def make_workspace(op: int, n_rows: int, hidden: int, vocab: int, rank: int, top_k: int, device) -> torch.Tensor:
    return torch.empty(max(workspace_bytes(op, n_rows, hidden, vocab, rank, top_k), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- operations

def conv_prepare(x: torch.Tensor, w_proj: torch.Tensor, base: torch.Tensor, block_size: int, taps: int,
                 group_size: int, out: Optional[torch.Tensor] = None,
                 k_post: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """x [N, H] -> (x_out [N, H], k_post [N, T, G] float32).  See dflash2_conv_prepare."""
    _same_dtype(x, w_proj, base)
    N, H = x.shape
    G = H // group_size if group_size > 0 else 0
    if out is None:
        out = torch.empty_like(x)
    if k_post is None:
        k_post = torch.empty((N, taps, max(G, 1)), dtype=torch.float32, device=x.device)
    st = _lib.dflash2_conv_prepare(_dtype_code(x), N, block_size, H, taps, group_size, _ptr(x), _ptr(w_proj),
                                   _ptr(base), _ptr(out), _ptr(k_post), _stream(x.device))
    _check(st, "dflash2_conv_prepare")
    return out, k_post


def conv_finish(y: torch.Tensor, k_post: torch.Tensor, base: torch.Tensor, block_size: int, taps: int,
                group_size: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [N, H], k_post [N, T, G] -> y_out [N, H].  See dflash2_conv_finish."""
    _same_dtype(y, base)
    if k_post.dtype != torch.float32:
        raise TypeError("k_post must be float32")
    N, H = y.shape
    if out is None:
        out = torch.empty_like(y)
    st = _lib.dflash2_conv_finish(_dtype_code(y), N, block_size, H, taps, group_size, _ptr(y), _ptr(k_post),
                                  _ptr(base), _ptr(out), _stream(y.device))
    _check(st, "dflash2_conv_finish")
    return out


def unary_topk(h: torch.Tensor, w_lm: torch.Tensor, top_k: int, gold_ids: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None):
    """h [N, H], w_lm [V, H] -> (ids [N, K] int32, vals [N, K] float32, gold_logit [N] or None)."""
    _same_dtype(h, w_lm)
    N, H = h.shape
    V = w_lm.shape[0]
    dev = h.device
    ids = torch.empty((N, top_k), dtype=torch.int32, device=dev)
    vals = torch.empty((N, top_k), dtype=torch.float32, device=dev)
    gl = torch.empty(N, dtype=torch.float32, device=dev) if gold_ids is not None else None
    if gold_ids is not None:
        _ids(gold_ids, "gold_ids")
    if workspace is None:
        workspace = make_workspace(OP_UNARY_TOPK, N, H, V, 0, top_k, dev)
    st = _lib.dflash2_unary_topk(_dtype_code(h), N, H, V, top_k, _ptr(h), _ptr(w_lm), _ptr(gold_ids), _ptr(ids),
                                 _ptr(vals), _ptr(gl), _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "dflash2_unary_topk")
    return ids, vals, gl


def unary_topk_ex(h: torch.Tensor, w_lm: torch.Tensor, top_k: int, gold_ids: Optional[torch.Tensor] = None,
                  output_multiplier: float = 1.0, softcap: float = 0.0, want_lse: bool = False,
                  want_metrics: bool = False, workspace: Optional[torch.Tensor] = None,
                  w_h: Optional[torch.Tensor] = None, g: Optional[torch.Tensor] = None):
    """unary_topk over softcap(output_multiplier * U).  -> (ids, vals, gold_logit or None, lse [N] or None,
    gold_prob [N] or None, gold_hit [N] uint8 or None); the gold metrics need gold_ids and want_metrics.
    With w_h [r, H] and g [N, r] float32, g also receives the context projection h w_hᵀ."""
    _same_dtype(h, w_lm)
    if (w_h is None) != (g is None):
        raise ValueError("w_h and g come together")
    r = 0
    if w_h is not None:
        _same_dtype(h, w_h)
        r = w_h.shape[0]
        if g.dtype != torch.float32 or tuple(g.shape) != (h.shape[0], r):
            raise TypeError("g must be float32 [N, r]")
    N, H = h.shape
    V = w_lm.shape[0]
    dev = h.device
    ids = torch.empty((N, top_k), dtype=torch.int32, device=dev)
    vals = torch.empty((N, top_k), dtype=torch.float32, device=dev)
    gl = prob = hit = None
    if gold_ids is not None:
        _ids(gold_ids, "gold_ids")
        gl = torch.empty(N, dtype=torch.float32, device=dev)
        if want_metrics:
            prob = torch.empty(N, dtype=torch.float32, device=dev)
            hit = torch.empty(N, dtype=torch.uint8, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev) if want_lse else None
    if workspace is None:
        workspace = make_workspace(OP_UNARY_TOPK, N, H, V, 0, top_k, dev)
    st = _lib.dflash2_unary_topk_ex(_dtype_code(h), N, H, V, top_k, _ptr(h), _ptr(w_lm), _ptr(gold_ids),
                                    float(output_multiplier), float(softcap), _ptr(w_h), r, _ptr(ids), _ptr(vals),
                                    _ptr(gl), _ptr(lse), _ptr(prob), _ptr(hit), _ptr(g), _ptr(workspace),
                                    workspace.numel(), _stream(dev))
    _check(st, "dflash2_unary_topk_ex")
    return ids, vals, gl, lse, prob, hit


def unary_topk_ctx(h: torch.Tensor, w_lm: torch.Tensor, top_k: int, w_h: torch.Tensor,
                   gold_ids: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   g: Optional[torch.Tensor] = None):
    """The unary top-K and the selector's context rows in one call (dflash2_unary_topk_ex with w_h).
    -> (ids, vals, gold_logit or None, g [N, r] float32)."""
    if g is None:
        g = torch.empty((h.shape[0], w_h.shape[0]), dtype=torch.float32, device=h.device)
    ids, vals, gl, _, _, _ = unary_topk_ex(h, w_lm, top_k, gold_ids=gold_ids, workspace=workspace, w_h=w_h, g=g)
    return ids, vals, gl, g


def _selector_shapes(h, w_h, g, cb_pred, cb_succ):
    """(N, H) of the selector's rows; h and w_h may be None when the context rows g are given."""
    _same_dtype(cb_pred, *[t for t in (h, w_h, cb_succ) if t is not None])
    if g is not None:
        if g.dtype != torch.float32 or g.dim() != 2 or g.shape[1] != cb_pred.shape[1]:
            raise TypeError("g must be float32 [N, r]")
        return g.shape[0], (h.shape[1] if h is not None else 64)
    if h is None or w_h is None:
        raise ValueError("h and w_h are needed without g")
    return h.shape


def selector_walk(h, w_h, cb_pred, cb_succ, cand_ids, cand_vals, anchor_ids, block_size: int,
                  workspace: Optional[torch.Tensor] = None, want_scores: bool = True, g=None):
    """-> (path [n_blocks, bs] int32, path_score [n_blocks, bs] float32 or None).  g: the context
    rows formed beforehand (unary_topk_ctx), or None to form them from h and w_h."""
    _ids(cand_ids, "cand_ids")
    _ids(anchor_ids, "anchor_ids")
    N, H = _selector_shapes(h, w_h, g, cb_pred, cb_succ)
    V, r = cb_pred.shape
    K = cand_ids.shape[1]
    nb = anchor_ids.shape[0]
    dev = cb_pred.device
    path = torch.empty((nb, block_size), dtype=torch.int32, device=dev)
    ps = torch.empty((nb, block_size), dtype=torch.float32, device=dev) if want_scores else None
    if workspace is None:
        workspace = make_workspace(OP_SELECTOR_WALK, nb * block_size, H, V, r, K, dev)
    st = _lib.dflash2_selector_walk(_dtype_code(cb_pred), nb, block_size, H, V, r, K, _ptr(h), _ptr(w_h), _ptr(g),
                                    _ptr(cb_pred),
                                    _ptr(cb_succ), _ptr(cand_ids), _ptr(cand_vals), _ptr(anchor_ids), _ptr(path),
                                    _ptr(ps), _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "dflash2_selector_walk")
    return path, ps


def selector_walk_noalloc(h, w_h, cb_pred, cb_succ, cand_ids, cand_vals, anchor_ids, block_size: int,
                          path: Optional[torch.Tensor] = None, path_score: Optional[torch.Tensor] = None,
                          want_scores: bool = True, g=None):
    """selector_walk without a workspace (the library's own device array; see
    dflash2_selector_walk_noalloc).  Outputs may be passed in, so that a
    caller that cannot allocate allocates nothing here either.
    -> (path [n_blocks, bs] int32, path_score [n_blocks, bs] float32 or None)."""
    _ids(cand_ids, "cand_ids")
    _ids(anchor_ids, "anchor_ids")
    N, H = _selector_shapes(h, w_h, g, cb_pred, cb_succ)
    V, r = cb_pred.shape
    K = cand_ids.shape[1]
    nb = anchor_ids.shape[0]
    dev = cb_pred.device
    if path is None:
        path = torch.empty((nb, block_size), dtype=torch.int32, device=dev)
    if path_score is None and want_scores:
        path_score = torch.empty((nb, block_size), dtype=torch.float32, device=dev)
    st = _lib.dflash2_selector_walk_noalloc(_dtype_code(cb_pred), nb, block_size, H, V, r, K, _ptr(h), _ptr(w_h),
                                            _ptr(g), _ptr(cb_pred), _ptr(cb_succ), _ptr(cand_ids), _ptr(cand_vals),
                                            _ptr(anchor_ids), _ptr(path), _ptr(path_score), _stream(dev))
    _check(st, "dflash2_selector_walk_noalloc")
    return path, path_score


def selector_sample(h, w_h, cb_pred, cb_succ, cand_ids, cand_vals, anchor_ids, block_size: int,
                    temperature: float = 1.0, seed: int = 0, workspace: Optional[torch.Tensor] = None,
                    want_scores: bool = True, g=None):
    """-> (path [n_blocks, bs] int32, path_score [n_blocks, bs] float32 or None), the
    path drawn from softmax(S / temperature) with the counter-based generator keyed by seed."""
    _ids(cand_ids, "cand_ids")
    _ids(anchor_ids, "anchor_ids")
    N, H = _selector_shapes(h, w_h, g, cb_pred, cb_succ)
    V, r = cb_pred.shape
    K = cand_ids.shape[1]
    nb = anchor_ids.shape[0]
    dev = cb_pred.device
    path = torch.empty((nb, block_size), dtype=torch.int32, device=dev)
    ps = torch.empty((nb, block_size), dtype=torch.float32, device=dev) if want_scores else None
    if workspace is None:
        workspace = make_workspace(OP_SELECTOR_WALK, nb * block_size, H, V, r, K, dev)
    st = _lib.dflash2_selector_sample(_dtype_code(cb_pred), nb, block_size, H, V, r, K, _ptr(h), _ptr(w_h), _ptr(g),
                                      _ptr(cb_pred),
                                      _ptr(cb_succ), _ptr(cand_ids), _ptr(cand_vals), _ptr(anchor_ids),
                                      float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(path), _ptr(ps),
                                      _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "dflash2_selector_sample")
    return path, ps


def decode_head(h, w_lm, top_k: int, w_h=None, cb_pred=None, cb_succ=None, anchor_ids=None,
                block_size: Optional[int] = None, workspace: Optional[torch.Tensor] = None, want_scores: bool = True,
                out=None):
    """The decode step in one launch: h [N, H] (N <= 8, bf16), w_lm [V, H] -> (ids [N, K], vals [N, K],
    path [n_blocks, bs] or None, path_score or None).  With w_h, cb_pred, cb_succ and anchor_ids the greedy
    walk of every block (block_size = N / n_blocks) runs in the same launch; without them only the lattice
    is formed.  `out` may pass (ids, vals, path, path_score) to write into."""
    _same_dtype(h, w_lm)
    N, H = h.shape
    V = w_lm.shape[0]
    dev = h.device
    sel = w_h is not None
    r = 0
    nb, bs = 1, N
    if sel:
        _same_dtype(h, w_h, cb_pred, cb_succ)
        _ids(anchor_ids, "anchor_ids")
        r = cb_pred.shape[1]
        nb = anchor_ids.shape[0]
        bs = block_size if block_size is not None else N // max(nb, 1)
    if out is not None:
        ids, vals, path, ps = out
    else:
        ids = torch.empty((N, top_k), dtype=torch.int32, device=dev)
        vals = torch.empty((N, top_k), dtype=torch.float32, device=dev)
        path = torch.empty((nb, bs), dtype=torch.int32, device=dev) if sel else None
        ps = torch.empty((nb, bs), dtype=torch.float32, device=dev) if sel and want_scores else None
    if workspace is None:
        workspace = make_workspace(OP_DECODE_HEAD, N, H, V, r, top_k, dev)
    st = _lib.dflash2_decode_head(_dtype_code(h), nb, bs, H, V, r, top_k, _ptr(h), _ptr(w_lm), _ptr(w_h),
                                  _ptr(cb_pred), _ptr(cb_succ), _ptr(anchor_ids), _ptr(ids), _ptr(vals), _ptr(path),
                                  _ptr(ps), _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "dflash2_decode_head")
    return ids, vals, path, ps


def selector_score_tf(h, w_h, cb_pred, cb_succ, cand_ids, cand_vals, pred_ids, gold_ids=None, force=None,
                      gold_logit=None, workspace: Optional[torch.Tensor] = None, g=None):
    """-> (scores [N, K] float32, best_ids [N] int32, ce [N] float32 or None, valid [N] uint8 or None)."""
    _ids(cand_ids, "cand_ids")
    _ids(pred_ids, "pred_ids")
    N, H = _selector_shapes(h, w_h, g, cb_pred, cb_succ)
    V, r = cb_pred.shape
    K = cand_ids.shape[1]
    dev = cb_pred.device
    scores = torch.empty((N, K), dtype=torch.float32, device=dev)
    best = torch.empty(N, dtype=torch.int32, device=dev)
    ce = valid = None
    if gold_ids is not None:
        _ids(gold_ids, "gold_ids")
        ce = torch.empty(N, dtype=torch.float32, device=dev)
        valid = torch.empty(N, dtype=torch.uint8, device=dev)
    if force is not None and force.dtype != torch.uint8:
        raise TypeError("force must be uint8")
    if workspace is None:
        workspace = make_workspace(OP_SELECTOR_TF, N, H, V, r, K, dev)
    st = _lib.dflash2_selector_score_tf(_dtype_code(cb_pred), N, H, V, r, K, _ptr(h), _ptr(w_h), _ptr(g),
                                        _ptr(cb_pred),
                                        _ptr(cb_succ), _ptr(cand_ids), _ptr(cand_vals), _ptr(pred_ids),
                                        _ptr(gold_ids), _ptr(force), _ptr(gold_logit), _ptr(scores), _ptr(best),
                                        _ptr(ce), _ptr(valid), _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "dflash2_selector_score_tf")
    return scores, best, ce, valid


def selector_ce_backward(h, w_h, cb_pred, cb_succ, cand_ids, cand_vals, pred_ids, gold_ids, grad_ce, force=None,
                         gold_logit=None, grad_pred=None, grad_succ=None, grad_wh=None, want_ce=True,
                         workspace: Optional[torch.Tensor] = None):
    """Adds the gradients of sum_n grad_ce[n] CE[n] into (grad_pred [V, r], grad_succ [V, r], grad_wh [r, H]),
    float32, allocated zeroed when not given.  -> (grad_pred, grad_succ, grad_wh, ce [N] or None,
    valid [N] or None)."""
    _same_dtype(h, w_h, cb_pred, cb_succ)
    _ids(cand_ids, "cand_ids")
    _ids(pred_ids, "pred_ids")
    _ids(gold_ids, "gold_ids")
    N, H = h.shape
    V, r = cb_pred.shape
    K = cand_ids.shape[1]
    dev = h.device
    if force is not None and force.dtype != torch.uint8:
        raise TypeError("force must be uint8")
    if grad_ce.dtype != torch.float32:
        raise TypeError("grad_ce must be float32")
    grads = []
    for t, shape in ((grad_pred, (V, r)), (grad_succ, (V, r)), (grad_wh, (r, H))):
        if t is None:
            t = torch.zeros(shape, dtype=torch.float32, device=dev)
        elif t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise TypeError(f"gradient buffers must be contiguous float32 {shape}")
        grads.append(t)
    ce = torch.empty(N, dtype=torch.float32, device=dev) if want_ce else None
    valid = torch.empty(N, dtype=torch.uint8, device=dev) if want_ce else None
    if workspace is None:
        workspace = make_workspace(OP_SELECTOR_CE_BACKWARD, N, H, V, r, K, dev)
    st = _lib.dflash2_selector_ce_backward(_dtype_code(h), N, H, V, r, K, _ptr(h), _ptr(w_h), _ptr(cb_pred),
                                           _ptr(cb_succ), _ptr(cand_ids), _ptr(cand_vals), _ptr(pred_ids),
                                           _ptr(gold_ids), _ptr(force), _ptr(gold_logit), _ptr(grad_ce),
                                           _ptr(grads[0]), _ptr(grads[1]), _ptr(grads[2]), _ptr(ce), _ptr(valid),
                                           _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "dflash2_selector_ce_backward")
    return grads[0], grads[1], grads[2], ce, valid


def read_device_status(workspace: torch.Tensor) -> int:
    """Synchronises the current stream; returns the status code of the last call using `workspace`."""
    return int(_lib.dflash2_read_device_status(_ptr(workspace), _stream(workspace.device)))
