"""bench.py's host-side contract, without a GPU: more than one GPU is refused
with a message, and the algorithmic work and floors it reports follow from the
workload's shape."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from block_draft_head_amd.inputs import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name", ["decode_1x8_h4096_v151936", "packed_tf_512x8_h4096_v151936"])
def test_lmhead_work_counts_the_stream_and_the_context_rows(name):
    w = WORKLOADS[name]
    b0, f0 = bench.lmhead_work(w)
    b1, f1 = bench.lmhead_work(w, ctx=True)
    N, H, V, K, r = w.n_rows, w.hidden, w.vocab, w.top_k, w.rank
    assert b0 == V * H * 2 + N * H * 2 + N * K * 8 and f0 == 2.0 * N * V * H
    # W_H streams once more and the float32 context rows are written
    assert b1 - b0 == r * H * 2 + N * r * 4 and f1 - f0 == 2.0 * N * r * H


def test_small_op_floors_at_decode():
    w = WORKLOADS["decode_1x8_h4096_v151936"]
    ops = {"conv": 0.007, "selector": 0.0075, "lmhead": 0.199}
    f = bench.small_op_floors(w, ops, 2.8, "decode_head")
    # two conv launches plus their bytes at 8 TB/s; the fused selector has no launch of its own
    assert f["conv"]["launches"] == 2 and f["selector"]["launches"] == 0
    assert abs(f["conv"]["floor_ms"] - (2 * 2.8 + f["conv"]["bytes"] / 8e6) * 1e-3) < 1e-12
    assert f["ratio_at_floors"] == pytest.approx((f["conv"]["floor_ms"] + f["selector"]["floor_ms"]) / 0.199)
