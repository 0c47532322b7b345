"""Host logic of bench.py that needs no GPU: the algorithmic-work count that feeds the roofline
(flops and K/V bytes of the computed tiles, from the mask at the start of a step), the linear fit
of step time against the computed fraction, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
from workloads import derive, get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def mask_of(bits):
    """[B, H, Tq, Tk] booleans (True = skipped) -> int32 words [B, H, Tq, W], bit j%32 of word
    j//32, packed with numpy independently of the code under test."""
    b, h, tq, tk = bits.shape
    w = (tk + 31) // 32
    words = np.zeros((b, h, tq, w), dtype=np.uint32)
    for j in range(tk):
        words[..., j // 32] |= bits[..., j].astype(np.uint32) << np.uint32(j % 32)
    return torch.from_numpy(words.view(np.int32))


def brute_work(bits, cfg):
    n, bq, bk, d = cfg.seq_len, cfg.tile_q, cfg.tile_k, cfg.head_dim
    flops = kv = 0.0
    elt = 2 if cfg.dtype == torch.bfloat16 else 4
    for idx in np.ndindex(*bits.shape):
        if bits[idx]:
            continue
        i, j = idx[2], idx[3]
        rows = min(bq, n - i * bq)
        cols = min(bk, n - j * bk)
        flops += 4.0 * rows * cols * d
        kv += 2.0 * cols * d * elt
    return flops, kv, float(bits.mean())


@pytest.mark.parametrize("name", ["tiny_ref", "stress_edge"])
def test_computed_work_matches_a_tile_by_tile_count(name):
    cfg = get_config(name)
    if name != "tiny_ref":   # N = 1000: ragged last tiles in both dimensions
        cfg = derive(cfg, heads=[0, 9], grid=(1, 10, 100))
    n = cfg.seq_len
    tq, tk = -(-n // cfg.tile_q), -(-n // cfg.tile_k)
    rng = np.random.default_rng(7)
    for density in (0.0, 0.3, 1.0):
        bits = rng.random((cfg.batch, cfg.heads, tq, tk)) < density
        got = bench.computed_work(mask_of(bits), cfg, tq, tk)
        want = brute_work(bits, cfg)
        assert got[0] == pytest.approx(want[0], rel=1e-12)
        assert got[1] == pytest.approx(want[1], rel=1e-12)
        assert got[2] == pytest.approx(want[2], rel=1e-12)
    # the empty mask is the dense step: 4 B H N^2 D flops
    empty = np.zeros((cfg.batch, cfg.heads, tq, tk), dtype=bool)
    assert bench.computed_work(mask_of(empty), cfg, tq, tk)[0] == pytest.approx(
        4.0 * cfg.batch * cfg.heads * n * n * cfg.head_dim, rel=1e-12)


def test_linear_fit_recovers_a_line_and_rejects_a_single_point():
    xs = [0.1, 0.4, 0.55, 1.0]
    a, b, r2 = bench.linear_fit(xs, [3.0 * x + 0.5 for x in xs])
    assert a == pytest.approx(3.0) and b == pytest.approx(0.5) and r2 == pytest.approx(1.0)
    assert bench.linear_fit([0.5], [1.0]) == (None, None, None)
    assert bench.linear_fit([0.5, 0.5], [1.0, 2.0]) == (None, None, None)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_host_cpu_names_the_processor():
    h = bench.host_cpu()
    assert h["nproc"] == os.cpu_count()
    assert h["model"] is None or isinstance(h["model"], str)
