"""The benchmark's FLOP count: live 64x64 tiles of the sliding-window causal mask (five GEMMs
of 2*64*64*128 FLOP each per live tile), checked against closed forms and brute force."""

import os

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def brute_live_tiles(S, W, grid=64):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    vis = (i - j >= 0) & (i - j < W)
    n = -(-S // grid)
    return sum(bool(vis[a * grid:(a + 1) * grid, b * grid:(b + 1) * grid].any()) for a in range(n) for b in range(n))


def test_causal_closed_form():
    for S in (64, 128, 8192):
        n = S // 64
        assert bench.live_tiles_window(S, S) == n * (n + 1) // 2
    assert bench.live_tiles_window(8192, 8192) == 8256      # per head; 528384 over 64 heads


def test_window_brute_force():
    for S, W in ((128, 64), (200, 17), (520, 300), (333, 333), (300, 1), (2048, 128)):
        assert bench.live_tiles_window(S, W) == brute_live_tiles(S, W), (S, W)


def test_headline_counted_flops():
    from masked_attention_backward_amd import workloads as W
    wl = W.WORKLOADS["large_causal"]
    total, per_head = bench.counted_flops(wl)
    assert per_head == 8256 * 5 * 2 * 64 * 64 * 128
    assert total == 528384 * 5 * 2 * 64 * 64 * 128
    assert abs(total - 2.7703e12) / 2.7703e12 < 1e-4


def test_bench_refuses_more_than_one_gpu():
    """The library is measured on one GPU: `bench.py --gpus 2` exits with status 2 and says so,
    before touching any device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
