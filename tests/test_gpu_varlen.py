"""GPU parity of sink attention over packed variable-length sequences.

Inputs come from the seeded packed generator; O and lse come from the oracle's forward
(rounded to the activation dtype and to fp32), never from the GPU.  Layout: q, o, dO, dq
[Hq, total, D]; k, v, dk, dv [Hkv, total, D]; lse [Hq, total]; cu_seqlens [B + 1] int32.
"""

import numpy as np
import pytest
import torch

import oracle
from masked_attention_backward_amd import workloads as W
from parity import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCALE = 1.0 / np.sqrt(128.0)


def api():
    from masked_attention_backward_amd import api as a
    return a


def with_oracle_forward(x, window, dtype):
    o, lse = oracle.sink_attention_forward_varlen(x["q"], x["k"], x["v"], x["sink"], x["cu_seqlens"].numpy(),
                                                  window, SCALE)
    x["o"] = torch.from_numpy(o).to(dtype)
    x["lse"] = torch.from_numpy(lse).to(torch.float32)
    return x


def gpu_bwd(name, x, window, path="ds_bank"):
    """One packed backward; `path` picks the workspace size as in the dense tests (the dS-bank
    size, or the minimum: dQ recomputes S and dP)."""
    g = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in x.items()}
    a = api()
    print(f"[gpu] attn_sink_bwd_varlen ({path}) {name} Hq{x['q'].shape[0]} Hkv{x['k'].shape[0]} "
          f"total{x['q'].shape[1]} max{x['max_seqlen']} W{window} {x['q'].dtype}", flush=True)
    ws = None
    if path == "recompute":
        nb = len(x["cu_seqlens"]) - 1
        ws = torch.empty(a.attn_sink_bwd_workspace_bytes(nb, x["q"].shape[0], x["k"].shape[0], x["max_seqlen"]),
                         dtype=torch.uint8, device=DEV)
    out = a.attn_sink_bwd_varlen(g["q"], g["k"], g["v"], g["o"], g["do"], g["lse"], g["sink"], g["cu_seqlens"],
                                 g["max_seqlen"], window, SCALE, workspace=ws)
    torch.cuda.synchronize()
    return out


# (name, lengths, Hq, Hkv, window, dtype, seed): ragged lengths spanning several 128-row
# tiles, a one-row and an empty sequence, windows narrower than a tile and causal.
SMALL = [
    ("mixed_causal", [200, 1, 0, 333, 128, 64], 4, 2, 100000, torch.float16, 401),
    ("mixed_w70_bf16", [200, 1, 0, 333, 128, 64], 4, 2, 70, torch.bfloat16, 402),
    ("g8_w17", [129, 64, 65, 300], 8, 1, 17, torch.float16, 403),
    ("one_seq_causal_bf16", [257], 2, 2, 257, torch.bfloat16, 404),
    ("many_short", [3, 7, 1, 31, 64, 63, 65, 2, 0, 5], 2, 1, 100000, torch.float16, 405),
    ("g4_causal_bf16", [190, 64, 0, 257, 1], 8, 2, 100000, torch.bfloat16, 408),
    ("g6_w100", [300, 129, 40], 6, 1, 100, torch.float16, 409),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_bwd_small(case):
    name, lengths, hq, hkv, window, dtype, seed = case
    x = with_oracle_forward(W.varlen_inputs(lengths, hq, hkv, dtype, seed_base=seed), window, dtype)
    ref = oracle.sink_attention_backward_varlen(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["sink"],
                                                x["cu_seqlens"].numpy(), window, SCALE)
    for path in ("ds_bank", "recompute"):
        dq, dk, dv, dsink = gpu_bwd(name, x, window, path)
        check(f"{path} dsink", dsink, ref["dsink"], dtype)
        check(f"{path} dq", dq, ref["dq"], dtype)
        check(f"{path} dk", dk, ref["dk"], dtype)
        check(f"{path} dv", dv, ref["dv"], dtype)


@pytest.mark.parametrize("case", [SMALL[0], SMALL[1], SMALL[2]], ids=lambda c: c[0])
def test_fwd_small(case):
    name, lengths, hq, hkv, window, dtype, seed = case
    x = W.varlen_inputs(lengths, hq, hkv, dtype, seed_base=seed)
    o_ref, lse_ref = oracle.sink_attention_forward_varlen(x["q"], x["k"], x["v"], x["sink"],
                                                          x["cu_seqlens"].numpy(), window, SCALE)
    g = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in x.items()}
    print(f"[gpu] attn_sink_fwd_varlen {name}", flush=True)
    o, lse = api().attn_sink_fwd_varlen(g["q"], g["k"], g["v"], g["sink"], g["cu_seqlens"], g["max_seqlen"],
                                        window, SCALE)
    torch.cuda.synchronize()
    check("o", o, o_ref, dtype)
    check("lse", lse, lse_ref, dtype)


@pytest.mark.parametrize("hq,hkv,path", [(2, 2, "ds_bank"), (4, 2, "recompute")], ids=["mha_bank", "gqa_recompute"])
def test_equal_lengths_bit_identical_to_dense(hq, hkv, path):
    """B sequences of one length S are the dense [B, H, S, D] call relaid to [H, B*S, D]: the
    same tiles in the same order, so every output is bit-identical, wherever the dense call
    does not split its key tiles by query heads (one query head per K/V head, or the minimum
    workspace; a split dense call sums dK/dV in another order and agrees to rounding)."""
    B, S, window, dtype = 3, 200, 90, torch.float16
    x = with_oracle_forward(W.varlen_inputs([S] * B, hq, hkv, dtype, seed_base=406), window, dtype)
    dq, dk, dv, dsink = gpu_bwd("equal_lengths", x, window, path)

    def dense(t):   # [H, B*S, ...] -> [B, H, S, ...]
        return t.reshape(t.shape[0], B, S, *t.shape[2:]).transpose(0, 1).contiguous().to(DEV)

    print(f"[gpu] attn_sink_bwd dense twin ({path})", flush=True)
    a = api()
    ws = None
    if path == "recompute":
        ws = torch.empty(a.attn_sink_bwd_workspace_bytes(B, hq, hkv, S), dtype=torch.uint8, device=DEV)
    r = a.attn_sink_bwd(dense(x["q"]), dense(x["k"]), dense(x["v"]), dense(x["o"]), dense(x["do"]),
                        dense(x["lse"]), x["sink"].to(DEV), window, SCALE, workspace=ws)
    fo, flse = a.attn_sink_fwd_varlen(*(x[n].to(DEV) for n in ("q", "k", "v", "sink", "cu_seqlens")), S,
                                      window, SCALE)
    ro, rlse = a.attn_sink_fwd(dense(x["q"]), dense(x["k"]), dense(x["v"]), x["sink"].to(DEV), window, SCALE)
    torch.cuda.synchronize()
    for got, want in ((dq, r[0]), (dk, r[1]), (dv, r[2]), (fo, ro), (flse, rlse)):
        assert torch.equal(dense(got.cpu()), want)
    assert torch.equal(dsink, r[3])


def test_deterministic_and_rows_outside_untouched():
    """Two runs give identical bits; rows before cu[0] and after cu[B] keep their contents."""
    lengths, hq, hkv, window, dtype = [150, 0, 90], 4, 2, 100000, torch.bfloat16
    x = with_oracle_forward(W.varlen_inputs(lengths, hq, hkv, dtype, seed_base=407), window, dtype)
    outs = [gpu_bwd("repeat", x, window) for _ in range(2)]
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    # Offsets 5 .. 245 inside 250 rows: rows 0-4 and 245-249 belong to no sequence.
    cu = torch.tensor([5, 155, 155, 245], dtype=torch.int32)
    total = 250
    g = {n: torch.randn((x[n].shape[0], total, 128)).to(dtype).to(DEV) for n in ("q", "k", "v", "o", "do")}
    lse = torch.randn((hq, total), dtype=torch.float32, device=DEV) + 5.0
    a = api()
    dq = torch.full((hq, total, 128), 7.0, dtype=dtype, device=DEV)
    dk = torch.full((hkv, total, 128), 7.0, dtype=dtype, device=DEV)
    dv = torch.full((hkv, total, 128), 7.0, dtype=dtype, device=DEV)
    dsink = torch.empty(hq, dtype=torch.float32, device=DEV)
    ws = torch.empty(a.attn_sink_bwd_workspace_bytes(3, hq, hkv, 150), dtype=torch.uint8, device=DEV)
    print("[gpu] attn_sink_bwd_varlen offset table", flush=True)
    st = a.lib.attn_sink_bwd_varlen(a._ptr(g["q"]), a._ptr(g["k"]), a._ptr(g["v"]), a._ptr(g["o"]), a._ptr(g["do"]),
                                    a._ptr(lse), a._ptr(x["sink"].to(DEV)), a._ptr(cu.to(DEV)), a._ptr(dq),
                                    a._ptr(dk), a._ptr(dv), a._ptr(dsink), a._ptr(ws), ws.numel(), 3, total, 150, hq,
                                    hkv, 128, window, float(SCALE), a._dtype_code(g["q"]), a._stream(DEV))
    torch.cuda.synchronize()
    assert st == 0
    for t in (dq, dk, dv):
        assert torch.all(t[:, :5] == 7.0) and torch.all(t[:, 245:] == 7.0)
        assert torch.all(torch.isfinite(t[:, 5:245].float()))


@pytest.mark.slow
def test_pages_varlen_workload_sampled():
    """The varlen row of the sink page's kernel table at full size: 8 sequences of up to 2048
    tokens, 64 query heads, 4 K/V heads, fp16, causal within each sequence; sampled rows of
    two sequences checked against the dense oracle on that sequence (the two definitions
    agree per sequence), dsink against the sum over all sequences."""
    lengths = W.varlen_lengths(8, 2048)
    hq, hkv, dtype = 64, 4, torch.float16
    window = 2048
    x = W.varlen_inputs(lengths, hq, hkv, dtype, seed_base=300)
    cu = x["cu_seqlens"].numpy().astype(np.int64)
    # O and lse one sequence at a time (the dense definition on each sequence's rows equals the
    # packed one there; far cheaper than the packed form at this size).
    o = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:2], dtype=torch.float32)
    for b in range(len(lengths)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        ob, lb = oracle.sink_attention_forward(x["q"][None, :, s0:s1], x["k"][None, :, s0:s1],
                                               x["v"][None, :, s0:s1], x["sink"], window, SCALE)
        o[:, s0:s1] = torch.from_numpy(ob[0]).to(dtype)
        lse[:, s0:s1] = torch.from_numpy(lb[0]).to(torch.float32)
    x["o"], x["lse"] = o, lse
    dq, dk, dv, dsink = gpu_bwd("pages_varlen", x, window)
    rng = np.random.default_rng(9)
    dsink_ref = np.zeros(hq)
    for b in range(len(lengths)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        L = s1 - s0
        sl = lambda t: t[None, :, s0:s1]
        sample = b in (0, 5)
        rows = sorted(set([0, 127, 128, L - 1] + list(rng.integers(0, L, 6)))) if sample else [0]
        qs = [(0, h, int(i)) for i in rows for h in ((0, 33, 63) if sample else (0,))]
        ks = [(0, h, int(j)) for j in rows for h in ((0, 3) if sample else (0,))]
        ref = oracle.sink_attention_backward_sampled(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["o"]), sl(x["do"]),
                                                     sl(x["lse"]), x["sink"], window, SCALE, qs, ks)
        dsink_ref += ref["dsink"]
        if sample:
            check(f"dq[seq {b}]", torch.stack([dq[h, s0 + i] for _, h, i in qs]), ref["dq"], dtype)
            check(f"dk[seq {b}]", torch.stack([dk[h, s0 + j] for _, h, j in ks]), ref["dk"], dtype)
            check(f"dv[seq {b}]", torch.stack([dv[h, s0 + j] for _, h, j in ks]), ref["dv"], dtype)
    check("dsink", dsink, dsink_ref, dtype)


@pytest.mark.slow
def test_pages_varlen_forward_two_sequences():
    """The sink page's varlen forward row at full size (8 sequences of up to 2048 tokens, 64 query
    heads, 4 K/V heads, fp16, causal within each sequence): every O and lse row of two of the
    sequences against the dense oracle on that sequence's rows."""
    lengths = W.varlen_lengths(8, 2048)
    hq, hkv, dtype, window = 64, 4, torch.float16, 2048
    x = W.varlen_inputs(lengths, hq, hkv, dtype, seed_base=310)
    g = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in x.items()}
    print("[gpu] attn_sink_fwd_varlen pages workload", flush=True)
    o, lse = api().attn_sink_fwd_varlen(g["q"], g["k"], g["v"], g["sink"], g["cu_seqlens"], g["max_seqlen"], window,
                                        SCALE)
    torch.cuda.synchronize()
    cu = x["cu_seqlens"].numpy().astype(np.int64)
    for b in (0, 6):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        ro, rl = oracle.sink_attention_forward(x["q"][None, :, s0:s1], x["k"][None, :, s0:s1], x["v"][None, :, s0:s1],
                                               x["sink"], window, SCALE)
        check(f"o[seq {b}]", o[:, s0:s1], ro[0], dtype)
        check(f"lse[seq {b}]", lse[:, s0:s1], rl[0], dtype)


@pytest.mark.slow
def test_pages_varlen_equal_lengths_full():
    """The sink page's varlen row under its plain reading: 8 sequences of exactly 2048 tokens,
    64 query heads, 4 K/V heads, fp16, causal within each sequence.  Every element of dQ, dK,
    dV and dsink against the dense oracle applied to each sequence (equal to the packed
    definition on that sequence's rows; dsink sums over the sequences)."""
    vw = W.VARLEN["varlen_8x2048"]
    lengths, hq, hkv, dtype, window = list(vw.lengths), vw.Hq, vw.Hkv, vw.dtype, vw.window
    x = vw.inputs()
    cu = x["cu_seqlens"].numpy().astype(np.int64)
    o = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:2], dtype=torch.float32)
    for b in range(len(lengths)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        ob, lb = oracle.sink_attention_forward(x["q"][None, :, s0:s1], x["k"][None, :, s0:s1],
                                               x["v"][None, :, s0:s1], x["sink"], window, SCALE)
        o[:, s0:s1] = torch.from_numpy(ob[0]).to(dtype)
        lse[:, s0:s1] = torch.from_numpy(lb[0]).to(torch.float32)
    x["o"], x["lse"] = o, lse
    dq_ref = np.zeros(tuple(x["q"].shape))
    dk_ref = np.zeros(tuple(x["k"].shape))
    dv_ref = np.zeros(tuple(x["v"].shape))
    dsink_ref = np.zeros(hq)
    for b in range(len(lengths)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        sl = lambda t: t[None, :, s0:s1]
        ref = oracle.sink_attention_backward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["o"]), sl(x["do"]),
                                             sl(x["lse"]), x["sink"], window, SCALE)
        dq_ref[:, s0:s1] = ref["dq"][0]
        dk_ref[:, s0:s1] = ref["dk"][0]
        dv_ref[:, s0:s1] = ref["dv"][0]
        dsink_ref += ref["dsink"]
    for path in ("ds_bank", "recompute"):
        dq, dk, dv, dsink = gpu_bwd("pages_varlen_8x2048", x, window, path)
        check(f"{path} dsink", dsink, dsink_ref, dtype)
        check(f"{path} dq", dq, dq_ref, dtype)
        check(f"{path} dk", dk, dk_ref, dtype)
        check(f"{path} dv", dv, dv_ref, dtype)
