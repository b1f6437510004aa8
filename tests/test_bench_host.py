"""Host logic of bench.py (no GPU): the graph length that times exactly --steps steps, the
algorithmic byte and FLOP counts the roofline fractions divide by, and the refusal of more than
one GPU."""
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dfkv_workloads import GEOMS  # noqa: E402


@pytest.mark.parametrize("K,d", [(1, 1), (7, 7), (8, 8), (9, 9), (11, 11), (16, 8), (20, 10), (24, 8),
                                 (48, 8), (100, 10), (200, 8)])
def test_graph_steps(K, d):
    """Steps per graph: the smallest divisor of K that is at least 8, else K; K/d replays time K steps."""
    assert bench.graph_steps(K) == d
    assert K % d == 0


def _wl(cfg, rows):
    return types.SimpleNamespace(geom=GEOMS[cfg], n_rows=rows)


def test_algorithmic_dense_bs1():
    """Dense drafter, 4 rows (bs=1, width 4), one accepted row, counted by hand from the geometry:
    k_in = 3 x 4096, H = 4096, O = 5 layers x 2 x 8 heads x 128."""
    a = bench.algorithmic(_wl(1, 4), accepted_rows=1)
    K, H, O = 12288, 4096, 10240
    assert a["fc_bytes"] == 2 * H * K + 2 * 4 * K + 2 * 4 * H + 4 * (H // 16) * 4 == 100_798_464
    weights = 2 * (H * K + H + O * H + 5 * 128)
    row = 2 * 5 * (8 * 128) * 2            # K and V, every layer, bf16
    assert a["step_bytes"] == weights + 2 * 4 * K + row == 184_677_632
    assert a["fc_flops"] == 2.0 * 4 * K * H
    assert a["flops"] == 2.0 * 4 * (K * H + H * O)


def test_algorithmic_dense_bs64_and_mla():
    a = bench.algorithmic(_wl(2, 1024), accepted_rows=452)
    assert a["flops"] == 2.0 * 1024 * (12288 * 4096 + 4096 * 10240) == 188_978_561_024.0
    assert a["fc_flops"] == 2.0 * 1024 * 12288 * 4096
    # MLA: one latent (512) plus a rope part (64) per layer, three layers, one pool per layer
    m = bench.algorithmic(_wl(3, 4), accepted_rows=2)
    K, H, O = 3 * 7168, 7168, 3 * 576
    assert m["step_bytes"] == 2 * (H * K + H + O * H + 3 * 512) + 2 * 4 * K + 2 * (2 * 3 * 576)


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
