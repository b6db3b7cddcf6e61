"""GPU parity of the block-sparse path: tables bit-exact, forward and backward against the oracle."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from masked_attention_backward_amd import workloads as W
from parity import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def api():
    from masked_attention_backward_amd import api as a
    return a


def with_oracle_forward(wl, x):
    o, lse = oracle.blocksparse_attention_forward(x["q"], x["k"], x["v"], x["block_mask"], wl.bx, wl.by, wl.scale)
    x["o"] = torch.from_numpy(o).to(wl.dtype)
    x["lse"] = torch.from_numpy(lse).to(torch.float32)
    return x


def gpu_bwd(wl, x, path="default"):
    """path "default": the binding's workspace (the dS bank); "recompute": the minimum
    workspace (dQ recomputes S and dP)."""
    g = {k: v.to(DEV) for k, v in x.items()}
    print(f"[gpu] blocksparse_attn_bwd {wl.name} B{wl.B} N{wl.Hq} Sq{wl.Sq} Skv{wl.Skv} bx{wl.bx} by{wl.by} {path}",
          flush=True)
    ws = None
    if path == "recompute":
        a = api()
        ws = torch.empty(a.blocksparse_attn_bwd_workspace_bytes(wl.B, wl.Hq, wl.Sq, wl.Skv, wl.bx, wl.by),
                         dtype=torch.uint8, device=DEV)
    out = api().blocksparse_attn_bwd(g["q"], g["k"], g["v"], g["o"], g["do"], g["lse"], g["block_mask"], wl.bx,
                                     wl.by, wl.scale, workspace=ws)
    torch.cuda.synchronize()
    return out


def banked(wl):
    return wl.bx % 16 == 0 and wl.by % 16 == 0


@pytest.mark.parametrize("name", ["bigbird", "ragged"])
def test_tables_bit_exact_workload_masks(name):
    wl = W.WORKLOADS[name]
    m = W.make_block_mask(wl)
    print(f"[gpu] blocksparse_build_tables {name}", flush=True)
    got = api().blocksparse_build_tables(m.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.build_block_tables(m)
    for k in ("mask_t", "sel_q", "cnt_q", "sel_k", "cnt_k"):
        assert np.array_equal(got[k].cpu().numpy(), ref[k]), k


@pytest.mark.parametrize("shape,density", [((1, 1, 1, 1), 1.0), ((2, 3, 5, 7), 0.4), ((1, 2, 130, 67), 0.3),
                                           ((1, 1, 64, 200), 0.0), ((1, 1, 129, 1), 0.5)])
def test_tables_bit_exact_random(shape, density):
    rng = np.random.default_rng(sum(shape))
    m = ((rng.random(shape) < density) * rng.integers(1, 256, size=shape)).astype(np.uint8)
    print(f"[gpu] blocksparse_build_tables {shape}", flush=True)
    got = api().blocksparse_build_tables(torch.from_numpy(m).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.build_block_tables(m)
    for k in ("mask_t", "sel_q", "cnt_q", "sel_k", "cnt_k"):
        assert np.array_equal(got[k].cpu().numpy(), ref[k]), k


SMALL = [
    W.custom_blocksparse("b64_bigbird", 1, 2, 512, 512, 64, 64, "bigbird", seed_base=201),
    W.custom_blocksparse("b48x80_ragged", 1, 2, 300, 300, 48, 80, "ragged", seed_base=202),
    W.custom_blocksparse("b16x16_random", 1, 2, 200, 170, 16, 16, "random", density=0.3, seed_base=203),
    W.custom_blocksparse("b128x32_random", 2, 1, 400, 333, 128, 32, "random", density=0.5, seed_base=204),
    W.custom_blocksparse("b32x128_causal_bf16", 1, 2, 384, 384, 32, 128, "causal", dtype=torch.bfloat16,
                         seed_base=205),
    W.custom_blocksparse("b80x48_dense", 1, 1, 250, 260, 80, 48, "dense", seed_base=206),
    W.custom_blocksparse("b64x96_random_emptyrows", 1, 2, 320, 300, 64, 96, "random", density=0.2, seed_base=207),
    W.custom_blocksparse("b48x80_ragged_bf16", 2, 2, 290, 310, 48, 80, "ragged", dtype=torch.bfloat16,
                         seed_base=208),
    W.custom_blocksparse("b96x64_random_bf16", 1, 3, 260, 200, 96, 64, "random", dtype=torch.bfloat16,
                         density=0.5, seed_base=209),
    W.custom_blocksparse("b64_window200_bf16", 1, 2, 450, 450, 64, 64, "window", dtype=torch.bfloat16,
                         seed_base=210, window=200),
    W.custom_blocksparse("b32x16_window100", 2, 1, 333, 333, 32, 16, "window", seed_base=211, window=100),
    # Shapes whose key blocks can be selected by more than 64 query blocks split them over
    # several dK/dV workgroups of at most 32 (fp32 partials summed in chunk order): two chunks
    # (random, about 48 of 69), three (dense), and bigbird's global columns (three chunks) next
    # to single-chunk key blocks.
    W.custom_blocksparse("b16x32_random_2chunks", 1, 2, 1100, 300, 16, 32, "random", density=0.7, seed_base=212),
    W.custom_blocksparse("b16x64_dense_3chunks_bf16", 1, 1, 1100, 200, 16, 64, "dense", dtype=torch.bfloat16,
                         seed_base=213),
    W.custom_blocksparse("b64_bigbird_chunked", 1, 1, 4200, 4200, 64, 64, "bigbird", seed_base=214),
    # bx = 48: two selected query blocks can share a 32-row query half (one dS bank entry), and a
    # chunk boundary between them moves past the second.  Random: 67 query blocks at density
    # 0.7, two chunks per key block with boundaries at random entries; GQA dense: 35 query
    # blocks per head, so the boundary at entry 64 falls on the second head's block 29, which
    # shares a half with its block 28.
    W.custom_blocksparse("b48x64_random_chunked", 1, 2, 3200, 700, 48, 64, "random", density=0.7,
                         seed_base=215),
    W.custom_blocksparse("b48x80_dense_gqa_chunked_bf16", 1, 2, 1680, 400, 48, 80, "dense", dtype=torch.bfloat16,
                         seed_base=216, Nkv=1),
]


# Every block size runs both dQ paths (dS bank, recompute).
SMALL_PATHS = [(wl, p) for wl in SMALL for p in (("default", "recompute") if banked(wl) else ("default",))]


@pytest.mark.parametrize("wl,path", SMALL_PATHS, ids=lambda v: v if isinstance(v, str) else v.name)
def test_bwd_small(wl, path):
    x = with_oracle_forward(wl, W.make_inputs(wl))
    dq, dk, dv = gpu_bwd(wl, x, path)
    ref = oracle.blocksparse_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["block_mask"],
                                                wl.bx, wl.by, wl.scale)
    check("dq", dq, ref["dq"], wl.dtype)
    check("dk", dk, ref["dk"], wl.dtype)
    check("dv", dv, ref["dv"], wl.dtype)


@pytest.mark.parametrize("wl", [SMALL[0], SMALL[1], SMALL[3], SMALL[6]], ids=lambda w: w.name)
def test_fwd(wl):
    x = W.make_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    print(f"[gpu] blocksparse_attn_fwd {wl.name}", flush=True)
    o, lse = api().blocksparse_attn_fwd(g["q"], g["k"], g["v"], g["block_mask"], wl.bx, wl.by, wl.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.blocksparse_attention_forward(x["q"], x["k"], x["v"], x["block_mask"], wl.bx, wl.by, wl.scale)
    check("o", o, ro, wl.dtype)
    lg = lse.cpu().double().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.all(np.abs(lg[fin] - rl[fin]) <= 1e-5 + 1e-5 * np.abs(rl[fin]))


def test_bwd_empty_block_shares_tile():
    """bx = 48: a query block with no kept key block shares a 64-row tile with a live one, so its
    rows (lse = -inf) sit next to visible rows in the same dK/dV tile; they must contribute 0."""
    wl = W.custom_blocksparse("b48x80_empty_in_tile", 1, 2, 200, 190, 48, 80, "random", density=0.4,
                              seed_base=991)
    x = W.make_inputs(wl)
    x["block_mask"][0, 1, 2, :] = 0
    x = with_oracle_forward(wl, x)
    assert np.isneginf(x["lse"].numpy()).any()
    dq, dk, dv = gpu_bwd(wl, x)
    ref = oracle.blocksparse_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["block_mask"],
                                                wl.bx, wl.by, wl.scale)
    check("dq", dq, ref["dq"], wl.dtype)
    check("dk", dk, ref["dk"], wl.dtype)
    check("dv", dv, ref["dv"], wl.dtype)


GQA = [
    W.custom_blocksparse("gqa_b64_bigbird_4to2", 1, 4, 320, 320, 64, 64, "bigbird", seed_base=301, Nkv=2),
    W.custom_blocksparse("gqa_b48x80_random_6to2_bf16", 2, 6, 250, 230, 48, 80, "random", dtype=torch.bfloat16,
                         density=0.4, seed_base=302, Nkv=2),
    W.custom_blocksparse("gqa_b32x128_causal_8to1", 1, 8, 300, 300, 32, 128, "causal", seed_base=303, Nkv=1),
    # The group's 4 query heads select key block 0 76 times (three chunks), the last one 4 times.
    W.custom_blocksparse("gqa_b32_causal_chunked_4to1", 1, 4, 600, 600, 32, 32, "causal", seed_base=304, Nkv=1),
]


@pytest.mark.parametrize("wl", GQA, ids=lambda w: w.name)
def test_bwd_gqa(wl):
    """Grouped K/V heads: dK/dV of a K/V head sum over its query heads, each with its own mask."""
    x = with_oracle_forward(wl, W.make_inputs(wl))
    assert x["k"].shape[1] == wl.Hkv < wl.Hq
    dq, dk, dv = gpu_bwd(wl, x)
    ref = oracle.blocksparse_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["block_mask"],
                                                wl.bx, wl.by, wl.scale)
    check("dq", dq, ref["dq"], wl.dtype)
    check("dk", dk, ref["dk"], wl.dtype)
    check("dv", dv, ref["dv"], wl.dtype)


@pytest.mark.parametrize("wl", GQA[:2], ids=lambda w: w.name)
def test_fwd_gqa(wl):
    x = W.make_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    print(f"[gpu] blocksparse_attn_fwd (gqa) {wl.name}", flush=True)
    o, lse = api().blocksparse_attn_fwd(g["q"], g["k"], g["v"], g["block_mask"], wl.bx, wl.by, wl.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.blocksparse_attention_forward(x["q"], x["k"], x["v"], x["block_mask"], wl.bx, wl.by, wl.scale)
    check("o", o, ro, wl.dtype)
    lg = lse.cpu().double().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.all(np.abs(lg[fin] - rl[fin]) <= 1e-5 + 1e-5 * np.abs(rl[fin]))


def test_ragged_config_full():
    wl = W.WORKLOADS["ragged"]
    x = with_oracle_forward(wl, W.make_inputs(wl))
    dq, dk, dv = gpu_bwd(wl, x)
    ref = oracle.blocksparse_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["block_mask"],
                                                wl.bx, wl.by, wl.scale)
    check("dq", dq, ref["dq"], wl.dtype)
    check("dk", dk, ref["dk"], wl.dtype)
    check("dv", dv, ref["dv"], wl.dtype)


def test_deterministic_and_fully_written():
    wl = SMALL[6]
    x = with_oracle_forward(wl, W.make_inputs(wl))
    g = {k: v.to(DEV) for k, v in x.items()}
    a = api()
    outs = []
    for _ in range(3):
        dq = torch.full_like(g["q"], float("nan"))
        dk = torch.full_like(g["k"], float("nan"))
        dv = torch.full_like(g["v"], float("nan"))
        nbytes = a.blocksparse_attn_bwd_workspace_bytes(wl.B, wl.Hq, wl.Sq, wl.Skv, wl.bx, wl.by)
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
        st = a.lib.blocksparse_attn_bwd(*(ctypes.c_void_p(t.data_ptr()) for t in (
            g["q"], g["k"], g["v"], g["o"], g["do"], g["lse"], g["block_mask"], dq, dk, dv, ws)),
            nbytes, wl.B, wl.Hq, wl.Sq, wl.Skv, 128, wl.bx, wl.by, wl.scale, a.MA_F16,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (dq, dk, dv)])
    for t in outs[0]:
        assert torch.isfinite(t.float()).all()
    for other in outs[1:]:
        for u, v in zip(outs[0], other):
            assert torch.equal(u.view(torch.int16), v.view(torch.int16))


@pytest.mark.slow
def test_bigbird_config_full():
    """The bigbird configuration (B1 N16 S8192, bx = by = 64, fp16): every element of dQ, dK, dV."""
    wl = W.WORKLOADS["bigbird"]
    x = with_oracle_forward(wl, W.make_inputs(wl))
    dq, dk, dv = gpu_bwd(wl, x)
    ref = oracle.blocksparse_attention_backward(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["block_mask"],
                                                wl.bx, wl.by, wl.scale)
    check("dq", dq, ref["dq"], wl.dtype)
    check("dk", dk, ref["dk"], wl.dtype)
    check("dv", dv, ref["dv"], wl.dtype)
