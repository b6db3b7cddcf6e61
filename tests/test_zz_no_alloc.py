"""The allocation-free backward (attn_sink_bwd_noalloc, scratch in the library's static device
array) against attn_sink_bwd with a caller workspace of the minimum size (the same dQ path,
where dQ recomputes S and dP), through the C ABI: two calls in a row,
the second on a smaller problem, each compared bit for bit (same kernels, same order) and
with outputs pre-filled with NaN so every element must be written."""

import ctypes

import pytest
import torch

from masked_attention_backward_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    W.custom_sink("noalloc_big", 2, 16, 4, 1500, 700, torch.bfloat16, seed_base=130),
    W.custom_sink("noalloc_small", 1, 4, 2, 333, 90, torch.float16, seed_base=131),
]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_noalloc_matches_workspace_call_twice():
    from masked_attention_backward_amd import api
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for wl in CASES:
        x = W.make_inputs(wl)
        g = {k: v.to(DEV) for k, v in x.items()}
        code = api.MA_BF16 if wl.dtype == torch.bfloat16 else api.MA_F16
        print(f"[gpu] attn_sink_fwd + attn_sink_bwd + attn_sink_bwd_noalloc {wl.name} B{wl.B} Hq{wl.Hq} "
              f"Hkv{wl.Hkv} S{wl.Sq} W{wl.window} {wl.dtype}", flush=True)
        o, lse = api.attn_sink_fwd(g["q"], g["k"], g["v"], g["sink"], wl.window, wl.scale)
        ws = torch.empty(api.attn_sink_bwd_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq), dtype=torch.uint8,
                         device=DEV)
        want = api.attn_sink_bwd(g["q"], g["k"], g["v"], o, g["do"], lse, g["sink"], wl.window, wl.scale,
                                 workspace=ws)
        dq = torch.full_like(g["q"], float("nan"))
        dk = torch.full_like(g["k"], float("nan"))
        dv = torch.full_like(g["v"], float("nan"))
        dsink = torch.full((wl.Hq,), float("nan"), device=DEV)
        st = api.lib.attn_sink_bwd_noalloc(_ptr(g["q"]), _ptr(g["k"]), _ptr(g["v"]), _ptr(o), _ptr(g["do"]),
                                           _ptr(lse), _ptr(g["sink"]), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsink),
                                           wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.D, wl.window, wl.scale, code, stream)
        assert st == 0, api.lib.maskattn_strerror(st)
        torch.cuda.synchronize()
        for name, got, ref in zip(("dq", "dk", "dv", "dsink"), (dq, dk, dv, dsink), want):
            assert torch.isfinite(got.float()).all(), name
            assert torch.equal(_bits(got), _bits(ref)), name


def test_noalloc_binding_and_scratch_limit():
    """The binding of the same name, and a problem over the static scratch limit is refused."""
    from masked_attention_backward_amd import api
    wl = CASES[1]
    x = W.make_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    print(f"[gpu] attn_sink_bwd_noalloc binding {wl.name}", flush=True)
    o, lse = api.attn_sink_fwd(g["q"], g["k"], g["v"], g["sink"], wl.window, wl.scale)
    got = api.attn_sink_bwd_noalloc(g["q"], g["k"], g["v"], o, g["do"], lse, g["sink"], wl.window, wl.scale)
    ws = torch.empty(api.attn_sink_bwd_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq), dtype=torch.uint8, device=DEV)
    want = api.attn_sink_bwd(g["q"], g["k"], g["v"], o, g["do"], lse, g["sink"], wl.window, wl.scale, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        assert torch.equal(_bits(a), _bits(b))
    big = torch.empty((1, 64, 65536, 128), dtype=torch.float16, device=DEV)
    kv = torch.empty((1, 8, 65536, 128), dtype=torch.float16, device=DEV)
    l64 = torch.empty((1, 64, 65536), dtype=torch.float32, device=DEV)
    s64 = torch.zeros(64, dtype=torch.float32, device=DEV)
    with pytest.raises(api.MaskAttnError) as e:
        api.attn_sink_bwd_noalloc(big, kv, kv, big, big, l64, s64, 128)
    assert e.value.status == 5
