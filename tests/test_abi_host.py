"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/dflash2.h declares, and host validation returns the documented
status before anything reaches the device (all pointers here are fake and are
never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash2.h")

D = pytest.importorskip("block_draft_head_amd.dflash2", reason="libdflash2.so not built")
L = D._lib

import torch  # noqa: E402

# The validation tests pass fake device pointers and rely on every call being
# rejected on the host.  Never run them where a GPU is visible.
no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake-pointer host checks run only without a GPU")
P = ctypes.c_void_p
OK, NULL, SHAPE, DTYPE, UNSUP, ALIAS, WS = 0, 1, 2, 3, 4, 5, 6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash2_[a-z_]+)\s*\(", text)))


def test_every_declared_entry_point_is_exported():
    names = declared_functions()
    assert len(names) == 15, names
    assert sorted(D.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name, val in [("DFLASH2_MAX_TOP_K", D.MAX_TOP_K), ("DFLASH2_MAX_TAPS", D.MAX_TAPS),
                      ("DFLASH2_MAX_BLOCK_SIZE", D.MAX_BLOCK_SIZE), ("DFLASH2_MAX_RANK", D.MAX_RANK)]:
        assert re.search(rf"#define {name} {val}\b", text)
    for code, name in D.STATUS.items():
        assert re.search(rf"{name} = {code}\b", text)


def test_status_strings_and_version():
    assert D.version().startswith("dflash2-gfx950")
    for code in range(9):
        assert D.status_str(code) and D.status_str(code) != "unknown status"
    assert D.status_str(99) == "unknown status"


def fake(i):
    """Fake device pointer i: 64 MiB apart, so only the overlaps a test
    plants exist."""
    return P(0x4000000 * (i + 1))


def prep(dtype=1, n=16, bs=8, h=256, t=2, gs=16, x=fake(0), w=fake(1), b=fake(2), xo=fake(3), kp=fake(4)):
    return L.dflash2_conv_prepare(dtype, n, bs, h, t, gs, x, w, b, xo, kp, None)


def fin(dtype=1, n=16, bs=8, h=256, t=2, gs=16, y=fake(0), kp=fake(1), b=fake(2), yo=fake(3)):
    return L.dflash2_conv_finish(dtype, n, bs, h, t, gs, y, kp, b, yo, None)


@no_gpu
@pytest.mark.parametrize("call", [prep, fin])
def test_conv_rules(call):
    assert call(n=12) == SHAPE           # draft length not a whole number of blocks
    assert call(t=0) == SHAPE and call(t=9) == SHAPE   # taps outside [1, block_size]
    assert call(gs=24) == SHAPE          # group size must divide hidden
    assert call(n=0) == SHAPE and call(bs=0) == SHAPE and call(h=0) == SHAPE
    assert call(dtype=2) == DTYPE
    assert call(h=96, gs=16) == UNSUP    # hidden not a multiple of 64
    assert call(n=34, bs=17, t=17) == UNSUP  # taps above the kernel limit


@no_gpu
def test_conv_pointer_and_alias_rules():
    assert prep(x=None) == NULL and prep(kp=None) == NULL and prep(w=None) == NULL
    assert fin(yo=None) == NULL and fin(kp=None) == NULL
    assert prep(xo=fake(0)) == ALIAS     # output on the input
    assert prep(xo=P(0x4000000 + 64)) == ALIAS  # partial overlap
    assert prep(xo=fake(2)) == ALIAS     # output on base
    assert prep(kp=fake(1)) == ALIAS     # k_post on the projection weight
    assert prep(kp=fake(3)) == ALIAS     # k_post on x_out
    assert fin(yo=fake(0)) == ALIAS
    assert fin(yo=fake(2)) == ALIAS      # output on base
    assert fin(yo=fake(1)) == ALIAS      # output on k_post


def topk(dtype=1, n=8, h=256, v=4096, k=16, hp=fake(0), w=fake(1), gold=None, ids=fake(2), vals=fake(3),
         gl=None, ws=fake(4), wsb=None):
    if wsb is None:
        wsb = D.workspace_bytes(D.OP_UNARY_TOPK, n, h, v, 0, k) if n > 0 else 1 << 20
    return L.dflash2_unary_topk(dtype, n, h, v, k, hp, w, gold, ids, vals, gl, ws, wsb, None)


@no_gpu
def test_unary_topk_rules():
    assert topk(k=0) == SHAPE and topk(k=4097) == SHAPE and topk(v=0) == SHAPE and topk(n=0) == SHAPE
    assert topk(k=65) == UNSUP and topk(h=100) == UNSUP
    assert topk(dtype=-1) == DTYPE
    assert topk(hp=None) == NULL and topk(ws=None) == NULL and topk(ids=None) == NULL
    assert topk(gold=fake(5), gl=None) == NULL
    assert topk(wsb=16) == WS
    assert topk(ids=fake(3)) == ALIAS    # ids on vals
    assert topk(ids=fake(0)) == ALIAS and topk(vals=fake(1)) == ALIAS  # outputs on h, on the LM head
    assert topk(gold=fake(5), gl=fake(5)) == ALIAS  # the gold logit over the gold ids
    assert topk(gold=fake(5), gl=fake(4)) == ALIAS  # and over the workspace
    assert topk(ws=fake(1)) == ALIAS     # the workspace over the LM head


def topk_ex(dtype=1, n=8, h=256, v=4096, k=16, hp=fake(0), w=fake(1), gold=None, mult=1.0, cap=0.0, ids=fake(2),
            vals=fake(3), gl=None, lse=None, prob=None, hit=None, ws=fake(4), wsb=None, wh=None, r=0, g=None):
    if wsb is None:
        wsb = D.workspace_bytes(D.OP_UNARY_TOPK, n, h, v, 0, k) if n > 0 else 1 << 20
    return L.dflash2_unary_topk_ex(dtype, n, h, v, k, hp, w, gold, mult, cap, wh, r, ids, vals, gl, lse, prob, hit, g,
                                   ws, wsb, None)


@no_gpu
def test_unary_topk_ex_rules():
    # the plain call's rules
    assert topk_ex(k=0) == SHAPE and topk_ex(k=65) == UNSUP and topk_ex(h=100) == UNSUP and topk_ex(dtype=-1) == DTYPE
    assert topk_ex(hp=None) == NULL and topk_ex(ws=None) == NULL and topk_ex(wsb=16) == WS
    # a positive finite multiplier, a non-negative finite cap
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert topk_ex(mult=bad) == SHAPE
    for bad in (-0.5, float("inf"), float("nan")):
        assert topk_ex(cap=bad) == SHAPE
    # gold metrics need gold ids; gold ids need the gold logit
    assert topk_ex(prob=fake(6)) == NULL and topk_ex(hit=fake(7)) == NULL
    assert topk_ex(gold=fake(5)) == NULL
    # outputs overlap neither each other nor the workspace
    assert topk_ex(lse=fake(3)) == ALIAS and topk_ex(gold=fake(5), gl=fake(6), hit=fake(6)) == ALIAS
    assert topk_ex(lse=fake(4)) == ALIAS
    assert topk_ex(lse=fake(0)) == ALIAS and topk_ex(gold=fake(5), gl=fake(6), prob=fake(5)) == ALIAS
    # the context rows: W_H and g together, a rank the selector supports
    assert topk_ex(wh=fake(8), r=32) == NULL and topk_ex(g=fake(9), r=32) == NULL
    ctx = dict(wh=fake(8), r=32, g=fake(9))
    assert topk_ex(**{**ctx, "r": 0}) == SHAPE
    assert topk_ex(**{**ctx, "r": 12}) == UNSUP and topk_ex(**{**ctx, "r": 4104}) == UNSUP
    assert topk_ex(**ctx, mult=0.0) == SHAPE             # the other rules still hold
    assert topk_ex(**{**ctx, "g": fake(3)}) == ALIAS      # g over the values
    assert topk_ex(**{**ctx, "g": fake(4)}) == ALIAS      # over the workspace
    assert topk_ex(**{**ctx, "g": fake(8)}) == ALIAS      # over W_H
    assert topk_ex(**{**ctx, "g": fake(0)}) == ALIAS      # over h
    assert topk_ex(**{**ctx, "ids": fake(8)}) == ALIAS    # an output over W_H
    # without g the rank is not read
    assert topk_ex(r=12) == topk_ex(r=-5) == topk_ex()

def walk(dtype=1, nb=2, bs=8, h=256, v=1000, r=32, k=16, ws=fake(9), wsb=None, path=fake(7), anchors=fake(6), ps=None,
         hp=fake(0), wh=fake(1), g=None):
    if wsb is None:
        wsb = D.workspace_bytes(D.OP_SELECTOR_WALK, nb * bs, h, v, r, k) if nb * bs > 0 else 1 << 20
    return L.dflash2_selector_walk(dtype, nb, bs, h, v, r, k, hp, wh, g, fake(2), fake(3), fake(4), fake(5),
                                   anchors, path, ps, ws, wsb, None)


@no_gpu
def test_selector_walk_rules():
    assert walk(k=0) == SHAPE and walk(k=1001) == SHAPE and walk(r=0) == SHAPE and walk(nb=0) == SHAPE
    assert walk(k=65) == UNSUP and walk(bs=65) == UNSUP and walk(r=12) == UNSUP and walk(h=96) == UNSUP
    assert walk(r=4104) == UNSUP  # rank limit
    assert walk(bs=64, r=4096, k=64) != UNSUP
    assert walk(dtype=5) == DTYPE
    assert walk(path=None) == NULL and walk(anchors=None) == NULL and walk(ws=None) == NULL
    assert walk(wsb=100) == WS
    assert walk(ps=fake(7)) == ALIAS
    # outputs and workspace overlap no input: candidate ids, values, anchors, codebooks
    assert walk(path=fake(4)) == ALIAS and walk(ps=fake(5)) == ALIAS
    assert walk(path=fake(6)) == ALIAS and walk(ws=fake(2)) == ALIAS and walk(ps=fake(0)) == ALIAS
    # precomputed context rows stand in for h and W_H; without them both are needed
    assert walk(hp=None) == NULL and walk(wh=None) == NULL and walk(hp=None, wh=None) == NULL
    rows = walk(hp=None, wh=None, g=fake(11))
    assert rows not in (NULL, ALIAS, SHAPE, UNSUP) and walk(g=fake(11)) == rows
    assert walk(hp=None, wh=None, g=fake(11), path=fake(11)) == ALIAS  # an output over g
    assert walk(hp=None, wh=None, g=fake(11), ws=fake(11)) == ALIAS    # the workspace over g
    assert walk(hp=None, wh=None, g=fake(7)) == ALIAS                  # g under the path

def walk_na(dtype=1, nb=2, bs=8, h=256, v=1000, r=32, k=16, path=fake(10), ps=None, anchors=fake(6), hp=fake(0),
            wh=fake(1), g=None):
    return L.dflash2_selector_walk_noalloc(dtype, nb, bs, h, v, r, k, hp, wh, g, fake(2), fake(3), fake(4),
                                           fake(5), anchors, path, ps, None)


@no_gpu
def test_selector_walk_noalloc_rules():
    # the walk's rules, with the library's array in place of a workspace
    assert walk_na(k=0) == SHAPE and walk_na(nb=0) == SHAPE and walk_na(r=0) == SHAPE
    assert walk_na(k=65) == UNSUP and walk_na(bs=65) == UNSUP and walk_na(r=12) == UNSUP
    assert walk_na(dtype=5) == DTYPE
    # the status word and the float32 context rows must fit the array
    cap = D.NOALLOC_SCRATCH_BYTES
    assert D.workspace_bytes(D.OP_SELECTOR_WALK, 256 * 16, 5120, 248320, 512, 64) <= cap  # the wide walk fits
    assert walk_na(nb=257, bs=16, h=5120, v=248320, r=512, k=64) == UNSUP                 # one block more does not
    assert walk_na(path=None) == NULL and walk_na(anchors=None) == NULL
    assert walk_na(ps=fake(10)) == ALIAS
    assert walk_na(path=fake(4)) == ALIAS and walk_na(ps=fake(6)) == ALIAS and walk_na(path=fake(3)) == ALIAS
    assert walk_na(hp=None) == NULL and walk_na(hp=None, wh=None, g=fake(11), path=fake(11)) == ALIAS

def dhead(dtype=1, nb=1, bs=8, h=512, v=1000, r=32, k=16, wh=fake(2), A=fake(3), B=fake(4), anchors=fake(5),
          ids=fake(10), vals=fake(11), path=fake(12), ps=None, ws=fake(20), wsb=None):
    if wsb is None:
        wsb = D.workspace_bytes(D.OP_DECODE_HEAD, max(nb * bs, 1), h, v, r if wh else 0, k) or 1 << 20
    return L.dflash2_decode_head(dtype, nb, bs, h, v, r, k, fake(0), fake(1), wh, A, B, anchors, ids, vals, path, ps,
                                 ws, wsb, None)


@no_gpu
def test_decode_head_rules():
    assert dhead(k=0) == SHAPE and dhead(k=1001) == SHAPE and dhead(nb=0) == SHAPE and dhead(r=0) == SHAPE
    assert dhead(dtype=0) == UNSUP                 # bf16 only
    assert dhead(nb=2, bs=8) == UNSUP              # at most 8 rows
    assert dhead(h=256) == UNSUP                   # hidden a multiple of 512
    assert dhead(k=65) == UNSUP and dhead(r=12) == UNSUP
    assert dhead(dtype=7) == DTYPE
    # the selector's arguments come all together or not at all
    assert dhead(A=None) == NULL and dhead(anchors=None) == NULL and dhead(path=None) == NULL
    assert dhead(wh=None) == NULL                  # others given without w_h
    assert dhead(ids=None) == NULL and dhead(ws=None) == NULL
    assert dhead(wsb=100) == WS
    assert dhead(vals=fake(10)) == ALIAS and dhead(path=fake(20)) == ALIAS and dhead(ps=fake(12)) == ALIAS
    assert dhead(ids=fake(0)) == ALIAS             # an output over h
    assert dhead(vals=fake(1)) == ALIAS and dhead(path=fake(5)) == ALIAS and dhead(ps=fake(3)) == ALIAS
    assert dhead(ws=fake(2)) == ALIAS              # the workspace over W_H
    # without the selector the workspace holds no context rows
    assert (D.workspace_bytes(D.OP_DECODE_HEAD, 8, 4096, 151936, 0, 16)
            < D.workspace_bytes(D.OP_DECODE_HEAD, 8, 4096, 151936, 256, 16))


def sample(dtype=1, nb=2, bs=8, h=256, v=1000, r=32, k=16, temp=1.0, path=fake(10), ps=None, anchors=fake(6),
           ws=fake(12), wsb=None, hp=fake(0), wh=fake(1), g=None):
    if wsb is None:
        wsb = D.workspace_bytes(D.OP_SELECTOR_WALK, max(nb * bs, 1), h, v, r, k) if nb > 0 else 1 << 20
    return L.dflash2_selector_sample(dtype, nb, bs, h, v, r, k, hp, wh, g, fake(2), fake(3), fake(4), fake(5),
                                     anchors, temp, 0x1234, path, ps, ws, wsb, None)


@no_gpu
def test_selector_sample_rules():
    # the walk's rules, plus a positive, finite temperature
    assert sample(k=0) == SHAPE and sample(nb=0) == SHAPE and sample(k=65) == UNSUP and sample(r=12) == UNSUP
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert sample(temp=bad) == SHAPE
    assert sample(dtype=5) == DTYPE
    assert sample(path=None) == NULL and sample(anchors=None) == NULL and sample(ws=None) == NULL
    assert sample(wsb=100) == WS
    assert sample(ps=fake(10)) == ALIAS
    assert sample(path=fake(5)) == ALIAS and sample(ps=fake(4)) == ALIAS and sample(ws=fake(6)) == ALIAS
    assert sample(wh=None) == NULL and sample(hp=None, wh=None, g=fake(11), ws=fake(11)) == ALIAS

def tf(dtype=1, n=16, h=256, v=1000, r=32, k=16, gold=None, force=None, gl=None, ce=None, valid=None, ws=fake(12),
       wsb=None, scores=fake(13), best=fake(14), hp=fake(0), wh=fake(1), g=None):
    if wsb is None:
        wsb = D.workspace_bytes(D.OP_SELECTOR_TF, n, h, v, r, k) if n > 0 else 1 << 20
    return L.dflash2_selector_score_tf(dtype, n, h, v, r, k, hp, wh, g, fake(2), fake(3), fake(4), fake(5),
                                       fake(6), gold, force, gl, scores, best, ce, valid, ws, wsb, None)


@no_gpu
def test_selector_tf_rules():
    assert tf(k=0) == SHAPE and tf(n=0) == SHAPE and tf(k=2000) == SHAPE
    assert tf(k=100) == UNSUP and tf(r=20) == UNSUP
    assert tf(force=fake(8)) == NULL                       # force needs gold ids
    assert tf(gold=fake(7), force=fake(8), ce=fake(10), valid=fake(11)) == NULL  # and the gold logits
    assert tf(gold=fake(7)) == NULL                        # gold ids need ce and valid outputs
    assert tf(scores=None) == NULL and tf(ws=None) == NULL
    assert tf(wsb=8) == WS
    assert tf(scores=fake(14)) == ALIAS
    assert tf(scores=fake(4)) == ALIAS and tf(best=fake(6)) == ALIAS and tf(ws=fake(5)) == ALIAS
    full = dict(gold=fake(7), force=fake(8), gl=fake(9), ce=fake(10), valid=fake(11))
    assert tf(**{**full, "valid": fake(8)}) == ALIAS   # valid over force
    assert tf(**{**full, "ce": fake(9)}) == ALIAS      # ce over the gold logits
    assert tf(**{**full, "ce": fake(7)}) == ALIAS      # ce over the gold ids
    assert tf(hp=None) == NULL and tf(hp=None, wh=None, g=fake(15)) not in (NULL, ALIAS)
    assert tf(hp=None, wh=None, g=fake(15), scores=fake(15)) == ALIAS  # scores over g
    assert tf(g=fake(15), best=fake(15)) == ALIAS                      # with h and W_H given too

def bwd(dtype=1, n=16, h=256, v=1000, r=32, k=16, gold=fake(7), force=None, gl=None, gce=fake(9), gp=fake(20),
        gs=fake(40), gw=fake(60), ce=None, valid=None, ws=fake(12), wsb=None, hp=fake(0)):
    if wsb is None:
        wsb = D.workspace_bytes(D.OP_SELECTOR_CE_BACKWARD, n, h, v, r, k) if n > 0 else 1 << 20
    return L.dflash2_selector_ce_backward(dtype, n, h, v, r, k, hp, fake(1), fake(2), fake(3), fake(4), fake(5),
                                          fake(6), gold, force, gl, gce, gp, gs, gw, ce, valid, ws, wsb, None)


@no_gpu
def test_selector_ce_backward_rules():
    # the scorer's size rules
    assert bwd(k=0) == SHAPE and bwd(n=0) == SHAPE and bwd(k=2000) == SHAPE
    assert bwd(k=100) == UNSUP and bwd(r=20) == UNSUP and bwd(h=96) == UNSUP
    assert bwd(dtype=4) == DTYPE
    # gold ids, the upstream gradient and all three gradient buffers are required
    for kw in ("gold", "gce", "gp", "gs", "gw", "ws", "hp"):
        assert bwd(**{kw: None}) == NULL, kw
    assert bwd(force=fake(8)) == NULL            # forcing needs the gold logits
    assert bwd(wsb=8) == WS
    # the three gradients are distinct and overlap no input and no output
    assert bwd(gs=fake(20)) == ALIAS             # dB on dA
    assert bwd(gw=fake(20)) == ALIAS             # dW on dA
    assert bwd(gp=fake(2)) == ALIAS              # dA on the predecessor codebook
    assert bwd(gw=fake(0)) == ALIAS              # dW on h
    assert bwd(gs=fake(12)) == ALIAS             # dB on the workspace
    assert bwd(ce=fake(9)) == ALIAS              # ce on grad_ce


def off(i, b):
    """fake(i) moved by b bytes"""
    return P(0x4000000 * (i + 1) + b)


@no_gpu
def test_alignment_rules():
    """Floating-point arrays and the workspace off a 16-byte boundary, or
    int32 arrays off a 4-byte one, are refused before anything is enqueued."""
    assert prep(x=off(0, 8)) == UNSUP and prep(kp=off(4, 4)) == UNSUP and prep(b=off(2, 2)) == UNSUP
    assert fin(y=off(0, 2)) == UNSUP and fin(yo=off(3, 8)) == UNSUP and fin(kp=off(1, 4)) == UNSUP
    assert topk(hp=off(0, 2)) == UNSUP and topk(w=off(1, 8)) == UNSUP and topk(vals=off(3, 4)) == UNSUP
    assert topk(ws=off(4, 8)) == UNSUP and topk(ids=off(2, 2)) == UNSUP
    assert topk(gold=off(5, 2), gl=fake(6)) == UNSUP and topk(gold=fake(5), gl=off(6, 4)) == UNSUP
    assert topk_ex(wh=fake(8), r=32, g=off(9, 4)) == UNSUP and topk_ex(lse=off(7, 4)) == UNSUP
    assert walk(ps=off(8, 4)) == UNSUP and walk(path=off(7, 2)) == UNSUP and walk(anchors=off(6, 1)) == UNSUP
    assert walk(hp=None, wh=None, g=off(11, 8)) == UNSUP and walk(ws=off(9, 8)) == UNSUP
    assert walk_na(anchors=off(6, 2)) == UNSUP and walk_na(hp=off(0, 2)) == UNSUP
    assert sample(ps=off(11, 4)) == UNSUP and sample(ws=off(12, 4)) == UNSUP
    assert dhead(vals=off(11, 4)) == UNSUP and dhead(ws=off(20, 8)) == UNSUP and dhead(ids=off(10, 2)) == UNSUP
    assert dhead(A=off(3, 2)) == UNSUP and dhead(ps=off(13, 4)) == UNSUP
    assert tf(scores=off(13, 4)) == UNSUP and tf(best=off(14, 2)) == UNSUP and tf(hp=off(0, 8)) == UNSUP
    assert bwd(gp=off(20, 4)) == UNSUP and bwd(gce=off(9, 8)) == UNSUP and bwd(gold=off(7, 2)) == UNSUP
    # uint8 arrays may sit anywhere: a misplaced one is still caught by another rule
    assert tf(gold=fake(7), force=off(8, 1), gl=None) == NULL


def test_debug_slab_knob_changes_the_lm_head_workspace():
    assert L.dflash2_debug_force_slabs(-1) == SHAPE and L.dflash2_debug_force_slabs(4097) == SHAPE
    auto_dma = D.workspace_bytes(D.OP_UNARY_TOPK, 8, 4096, 151936, 0, 16)
    auto_big = D.workspace_bytes(D.OP_UNARY_TOPK, 4096, 4096, 151936, 0, 16)
    auto_dh = D.workspace_bytes(D.OP_DECODE_HEAD, 8, 4096, 151936, 256, 16)
    # the decode head streams 151936 / 16 + 256 / 16 = 9512 tiles; its automatic
    # grid is the fewest workgroups that keep the largest share at
    # ceil(9512 / 256) = 38 tiles: ceil(9512 / 38) = 251
    tiles = 151936 // 16 + 256 // 16
    grid = -(-tiles // -(-tiles // 256))
    assert grid == 251
    try:
        D.debug_force_slabs(7)
        # 8 rows: 7 lists of 16 keys per row instead of 251 (plus the status
        # header, the log-sum-exp partials and the context rows)
        assert D.workspace_bytes(D.OP_UNARY_TOPK, 8, 4096, 151936, 0, 16) < auto_dma
        # (the lists and their heads; each region rounded up to 256 bytes)
        up = lambda x: (x + 255) // 256 * 256
        lists = lambda n: up(8 * n * 16 * 8) + up(8 * n * 8)
        assert D.workspace_bytes(D.OP_DECODE_HEAD, 8, 4096, 151936, 256, 16) == auto_dh - lists(grid) + lists(7)
        assert D.workspace_bytes(D.OP_UNARY_TOPK, 4096, 4096, 151936, 0, 16) < auto_big
        D.debug_force_slabs(100000 // 100)  # clamped to each kernel's limit (256 stream workgroups)
        assert D.workspace_bytes(D.OP_DECODE_HEAD, 8, 4096, 151936, 256, 16) == auto_dh + lists(256) - lists(grid)
    finally:
        D.debug_force_slabs(0)
    assert D.workspace_bytes(D.OP_UNARY_TOPK, 8, 4096, 151936, 0, 16) == auto_dma
    assert D.workspace_bytes(D.OP_UNARY_TOPK, 4096, 4096, 151936, 0, 16) == auto_big


def test_workspace_sizes():
    # walk / TF: status header plus the float32 context projection
    assert D.workspace_bytes(D.OP_SELECTOR_WALK, 8, 4096, 151936, 256, 16) == 256 + 8 * 256 * 4
    assert D.workspace_bytes(D.OP_SELECTOR_TF, 4096, 4096, 151936, 256, 16) == 256 + 4096 * 256 * 4
    # CE backward: g (then gv), ag and dg rows; per-entry weight, target and
    # order for N (K + 1) entries; counts and offsets over 2V + 1 targets; scan
    # tile prefixes; each part rounded up to 256 bytes
    up = lambda x: (x + 255) // 256 * 256
    N, V, r, K = 4096, 151936, 256, 16
    want = 256 + 3 * up(N * r * 4) + 3 * up(N * (K + 1) * 4) + 2 * up((2 * V + 1) * 4) + up(-(-(2 * V + 1) // 4096) * 4)
    assert D.workspace_bytes(D.OP_SELECTOR_CE_BACKWARD, N, 4096, V, r, K) == want
    # top-K: one sorted list of K 8-byte keys per row per vocabulary slice
    b = D.workspace_bytes(D.OP_UNARY_TOPK, 8, 4096, 151936, 0, 16)
    assert b > 256 and (b - 256) % (8 * 16 * 8) == 0
    assert D.workspace_bytes(D.OP_UNARY_TOPK, 0, 4096, 151936, 0, 16) == 0
    assert D.workspace_bytes(7, 8, 4096, 151936, 0, 16) == 0
