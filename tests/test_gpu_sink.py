"""GPU parity of the sink + sliding-window path against the fp64 oracle.

Inputs come from the seeded generator; O and lse come from the oracle's forward (rounded
to the activation dtype and to fp32), never from the GPU.  Every element of dQ, dK, dV,
dsink (and Delta) must pass the gate in ``parity.py``.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from masked_attention_backward_amd import workloads as W
from parity import check, ATOL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def api():
    from masked_attention_backward_amd import api as a
    return a


def with_oracle_forward(wl, x):
    o, lse = oracle.sink_attention_forward(x["q"], x["k"], x["v"], x["sink"], wl.window, wl.scale)
    x["o"] = torch.from_numpy(o).to(wl.dtype)
    x["lse"] = torch.from_numpy(lse).to(torch.float32)
    return x


PATHS = ("ds_bank", "recompute")


def gpu_bwd(wl, x, path="ds_bank"):
    """One backward call; `path` picks the workspace size: the dS-bank size (dK/dV stores dS,
    dQ is one GEMM per block) or the minimum (dQ recomputes S and dP)."""
    g = {k: v.to(DEV) for k, v in x.items()}
    a = api()
    print(f"[gpu] attn_sink_bwd ({path}) {wl.name} B{wl.B} Hq{wl.Hq} Hkv{wl.Hkv} S{wl.Sq} W{wl.window} {wl.dtype}",
          flush=True)
    ws = None
    if path == "recompute":
        ws = torch.empty(a.attn_sink_bwd_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq), dtype=torch.uint8, device=DEV)
    out = a.attn_sink_bwd(g["q"], g["k"], g["v"], g["o"], g["do"], g["lse"], g["sink"], wl.window, wl.scale,
                          workspace=ws, return_delta=True)
    torch.cuda.synchronize()
    return out


def check_all(wl, x, ref, paths=PATHS, delta=True):
    """Both dQ paths against the oracle: every element of dQ, dK, dV, dsink (and Delta)."""
    for path in paths:
        dq, dk, dv, dsink, dl = gpu_bwd(wl, x, path)
        if delta:
            check(f"{path} delta", dl, ref["delta"], wl.dtype)
        check(f"{path} dsink", dsink, ref["dsink"], wl.dtype)
        check(f"{path} dq", dq, ref["dq"], wl.dtype)
        check(f"{path} dk", dk, ref["dk"], wl.dtype)
        check(f"{path} dv", dv, ref["dv"], wl.dtype)


SMALL = [
    W.WORKLOADS["tiny"],
    W.custom_sink("s192_causal", 1, 2, 2, 192, 192, torch.float16, seed_base=101),
    W.custom_sink("s200_w17_bf16", 2, 4, 2, 200, 17, torch.bfloat16, seed_base=102),
    W.custom_sink("s300_w1", 1, 8, 1, 300, 1, torch.float16, seed_base=103),
    W.custom_sink("s64_wbig", 1, 2, 1, 64, 100000, torch.float16, seed_base=104),
    W.custom_sink("s1", 1, 2, 1, 1, 1, torch.bfloat16, seed_base=105),
    W.custom_sink("s520_w300_bf16", 1, 4, 4, 520, 300, torch.bfloat16, seed_base=106),
    W.custom_sink("s77_w5", 3, 6, 3, 77, 5, torch.float16, seed_base=107),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_bwd_small(wl):
    x = with_oracle_forward(wl, W.make_inputs(wl))
    ref = oracle.sink_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["sink"], wl.window,
                                         wl.scale)
    check_all(wl, x, ref)


def test_bwd_no_sink_equals_causal():
    """sink = -inf: dsink is exactly 0 and the rest matches the oracle (plain causal attention)."""
    wl = W.custom_sink("nosink", 1, 4, 2, 160, 160, torch.float16, seed_base=110)
    x = W.make_inputs(wl)
    x["sink"] = torch.full((wl.Hq,), float("-inf"))
    x = with_oracle_forward(wl, x)
    ref = oracle.sink_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["sink"], wl.window,
                                         wl.scale)
    for path in PATHS:
        dq, dk, dv, dsink, _ = gpu_bwd(wl, x, path)
        assert torch.all(dsink.cpu() == 0)
        check(f"{path} dq", dq, ref["dq"], wl.dtype)
        check(f"{path} dk", dk, ref["dk"], wl.dtype)
        check(f"{path} dv", dv, ref["dv"], wl.dtype)


def test_bwd_paired_tiles():
    """Wide window with enough heads that both kernels run tile p together with tile n-1-p."""
    wl = W.custom_sink("paired", 4, 16, 16, 1024, 1024, torch.float16, seed_base=111)
    x = with_oracle_forward(wl, W.make_inputs(wl))
    ref = oracle.sink_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["sink"], wl.window,
                                         wl.scale)
    check_all(wl, x, ref, delta=False)


# Dense windows with too few key tiles to fill the GPU: with the dS-bank workspace key tiles
# are split by query heads over several dK/dV workgroups (fp32 partials, added in chunk
# order).  A sliding window, two sequences, a ragged last key tile, a window far shorter than
# the sequence, and one K/V head shared by eight query heads under a causal window, whose last
# key tiles split into 6 chunks over 8 heads (uneven); the small narrow-window shapes of the
# other tests split too.
HEAD_SPLIT = [
    W.custom_sink("split_s600_causal", 1, 8, 2, 600, 600, torch.float16, seed_base=120),
    W.custom_sink("split_s700_w400_bf16", 1, 6, 2, 700, 400, torch.bfloat16, seed_base=121),
    W.custom_sink("split_b2_s1024_causal", 2, 8, 2, 1024, 1024, torch.float16, seed_base=122),
    W.custom_sink("split_s2048_w300_mqa", 1, 8, 1, 2048, 300, torch.float16, seed_base=123),
    W.custom_sink("split_s2048_causal_mqa_bf16", 1, 8, 1, 2048, 2048, torch.bfloat16, seed_base=124),
]


@pytest.mark.parametrize("wl", HEAD_SPLIT, ids=lambda w: w.name)
def test_bwd_head_split(wl):
    x = with_oracle_forward(wl, W.make_inputs(wl))
    ref = oracle.sink_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["sink"], wl.window,
                                         wl.scale)
    check_all(wl, x, ref)


def random_sink_shapes(n=12, seed=20261203):
    """Seeded random small shapes: batch 1-2, 1-4 K/V heads in groups of 1-4, lengths 1-700
    (ragged tails), windows from 1 to past the sequence (narrow, wide, split and paired
    launches), both dtypes."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        Hkv = int(rng.integers(1, 5))
        Hq = Hkv * int(rng.integers(1, 5))
        S = int(rng.integers(1, 701))
        win = int(rng.choice([1, int(rng.integers(1, 300)), int(rng.integers(256, 800)), S, S + 37]))
        dt = torch.float16 if rng.integers(0, 2) == 0 else torch.bfloat16
        out.append((B, Hq, Hkv, S, max(1, win), dt))
    return out


@pytest.mark.parametrize("shape", random_sink_shapes(), ids=lambda t: "B%d_Hq%d_Hkv%d_S%d_W%d_%s" % (
    t[0], t[1], t[2], t[3], t[4], "f16" if t[5] == torch.float16 else "bf16"))
def test_bwd_random_shapes(shape):
    """Both dQ paths against the oracle, every element, on seeded random shapes."""
    B, Hq, Hkv, S, win, dt = shape
    wl = W.custom_sink("rand", B, Hq, Hkv, S, win, dt, seed_base=130 + S % 17)
    x = with_oracle_forward(wl, W.make_inputs(wl))
    ref = oracle.sink_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["sink"], wl.window,
                                         wl.scale)
    check_all(wl, x, ref)


def test_head_split_deterministic_and_fully_written():
    """Head-split launch: three runs bit-identical; outputs and workspace (partials included)
    pre-filled with 0xFF are fully overwritten / never read before written."""
    wl = HEAD_SPLIT[0]
    x = with_oracle_forward(wl, W.make_inputs(wl))
    g = {k: v.to(DEV) for k, v in x.items()}
    a = api()
    nbytes = a.attn_sink_bwd_ds_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.window)
    assert nbytes > a.attn_sink_bwd_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq) + \
        wl.B * wl.Hq * 2048 * ((wl.Sq + 31) // 32) * ((wl.Sq + 31) // 32 + 1) // 2   # room for partials
    outs = []
    for _ in range(3):
        dq = torch.full_like(g["q"], float("nan"))
        dk = torch.full_like(g["k"], float("nan"))
        dv = torch.full_like(g["v"], float("nan"))
        dsink = torch.full((wl.Hq,), float("nan"), device=DEV)
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
        print(f"[gpu] attn_sink_bwd (head split) {wl.name}", flush=True)
        st = a.lib.attn_sink_bwd(*(ctypes.c_void_p(t.data_ptr()) for t in (
            g["q"], g["k"], g["v"], g["o"], g["do"], g["lse"], g["sink"], dq, dk, dv, dsink, ws)),
            nbytes, wl.B, wl.Hq, wl.Hkv, wl.Sq, 128, wl.window, wl.scale, a.MA_F16,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (dq, dk, dv, dsink)])
        # The split ran: the fp32 partials after the dS bank (causal window: the lower triangle
        # of ceil(S/32) 32 x 32 blocks per head, 2 KiB each) were written.
        nb = (wl.Sq + 31) // 32
        part0 = a.attn_sink_bwd_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq) + \
            (wl.B * wl.Hq * nb * (nb + 1) // 2 * 2048 + 255) // 256 * 256
        assert bool((ws[part0:] != 0xFF).any())
    for t in outs[0]:
        assert torch.isfinite(t.float()).all()
    for other in outs[1:]:
        for u, v in zip(outs[0], other):
            assert torch.equal(u.view(torch.int16) if u.dtype != torch.float32 else u.view(torch.int32),
                               v.view(torch.int16) if v.dtype != torch.float32 else v.view(torch.int32))


@pytest.mark.parametrize("wl", [SMALL[0], SMALL[2], SMALL[6], W.custom_sink("f_causal", 1, 4, 1, 333, 333,
                                                                             torch.float16, seed_base=112)],
                         ids=lambda w: w.name)
def test_fwd(wl):
    x = W.make_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    print(f"[gpu] attn_sink_fwd {wl.name}", flush=True)
    o, lse = api().attn_sink_fwd(g["q"], g["k"], g["v"], g["sink"], wl.window, wl.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.sink_attention_forward(x["q"], x["k"], x["v"], x["sink"], wl.window, wl.scale)
    check("o", o, ro, wl.dtype)
    err = np.abs(lse.cpu().double().numpy() - rl)
    assert np.all(err <= 1e-5 + 1e-5 * np.abs(rl)), err.max()


def test_mid_config():
    wl = W.WORKLOADS["mid"]
    x = with_oracle_forward(wl, W.make_inputs(wl))
    ref = oracle.sink_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["sink"], wl.window,
                                         wl.scale)
    check_all(wl, x, ref)


@pytest.mark.parametrize("path", PATHS)
def test_deterministic_and_fully_written(path):
    """Three runs are bit-identical, and outputs and workspace pre-filled with 0xFF (NaN) are
    fully overwritten / never read before written (both dQ paths)."""
    wl = W.custom_sink("det", 2, 8, 2, 333, 100, torch.bfloat16, seed_base=113)
    x = with_oracle_forward(wl, W.make_inputs(wl))
    g = {k: v.to(DEV) for k, v in x.items()}
    a = api()
    outs = []
    for _ in range(3):
        dq = torch.full_like(g["q"], float("nan"))
        dk = torch.full_like(g["k"], float("nan"))
        dv = torch.full_like(g["v"], float("nan"))
        dsink = torch.full((wl.Hq,), float("nan"), device=DEV)
        nbytes = (a.attn_sink_bwd_ds_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.window) if path == "ds_bank"
                  else a.attn_sink_bwd_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq))
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
        st = a.lib.attn_sink_bwd(*(ctypes.c_void_p(t.data_ptr()) for t in (
            g["q"], g["k"], g["v"], g["o"], g["do"], g["lse"], g["sink"], dq, dk, dv, dsink, ws)),
            nbytes, wl.B, wl.Hq, wl.Hkv, wl.Sq, 128, wl.window, wl.scale, a.MA_BF16,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (dq, dk, dv, dsink)])
    for t in outs[0]:
        assert torch.isfinite(t.float()).all()
    for other in outs[1:]:
        for u, v in zip(outs[0], other):
            assert torch.equal(u.view(torch.int16) if u.dtype != torch.float32 else u.view(torch.int32),
                               v.view(torch.int16) if v.dtype != torch.float32 else v.view(torch.int32))


@pytest.mark.slow
def test_large_window128_full():
    wl = W.WORKLOADS["large_w128"]
    x = with_oracle_forward(wl, W.make_inputs(wl))
    ref = oracle.sink_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["sink"], wl.window,
                                         wl.scale)
    check_all(wl, x, ref, delta=False)


@pytest.mark.slow
def test_large_causal_full():
    """The benchmarked launch (B1 Hq64 Hkv8 S8192, window = S, bf16): every element of dQ, dK,
    dV, dsink and Delta against the oracle."""
    wl = W.WORKLOADS["large_causal"]
    x = with_oracle_forward(wl, W.make_inputs(wl))
    ref = oracle.sink_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["sink"], wl.window,
                                         wl.scale)
    check_all(wl, x, ref)


# The sink page's kernel-table shape: batch 1, 64 query heads, groups of 8 (8 K/V heads),
# 4096 tokens, head dimension 128, fp16; the window is read as the whole sequence (causal).
PAGES_SHAPE = W.WORKLOADS["pages_h64_s4096"]


@pytest.mark.slow
def test_pages_shape_forward_full():
    """Forward at the sink page's table shape (the paired-tile dense forward: 32 tiles of 128
    query rows per head, tile p with tile 31 - p): every O and lse element against the oracle."""
    wl = PAGES_SHAPE
    x = W.make_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    print(f"[gpu] attn_sink_fwd {wl.name}", flush=True)
    o, lse = api().attn_sink_fwd(g["q"], g["k"], g["v"], g["sink"], wl.window, wl.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.sink_attention_forward(x["q"], x["k"], x["v"], x["sink"], wl.window, wl.scale)
    check("o", o, ro, wl.dtype)
    err = np.abs(lse.cpu().double().numpy() - rl)
    assert np.all(err <= 1e-5 + 1e-5 * np.abs(rl)), err.max()


@pytest.mark.slow
def test_pages_shape_backward_full():
    """Backward at the sink page's table shape: every element of dQ, dK, dV, dsink, Delta."""
    wl = PAGES_SHAPE
    x = with_oracle_forward(wl, W.make_inputs(wl))
    ref = oracle.sink_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["sink"], wl.window,
                                         wl.scale)
    check_all(wl, x, ref)
