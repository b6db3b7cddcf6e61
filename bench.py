#!/usr/bin/env python3
"""Benchmark of the masked attention backward on one MI355X.

Default workload: GQA sink attention backward, B=1 Hq=64 Hkv=8 S=8192 D=128, window = S
(full causal), bf16 -- the dense-window configuration, the only one whose live tiles make
it MFMA-bound.  One step = one whole backward call (preprocess + dsink reduce + dK/dV +
dQ; for block-sparse workloads also the table build) on inputs already resident in HBM.
O and lse come from the library's own forward (untimed).

Metric: TFLOP/s counted over live tiles only, 5 GEMMs of 2*Br*Bc*D per live tile (64x64
counting grid for the window path; the mask blocks, edges clipped, for block-sparse).

Prints ONE JSON line.  The roofline object describes the dominant kernel (dK/dV), timed
live with HIP events recorded by the library between its stages on the launch stream.
The cpu_baseline leg times the fp64 oracle's backward on a bounded sample of the same
workload (a few query heads) on the host cores.
"""

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_16BIT = 2516.6   # TFLOP/s, dense fp16/bf16 MFMA, 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM = 8000.0          # GB/s

# HBM bytes per launch of the dominant kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# (scaled by a copy kernel of known size), valid only for the kernel sources they were taken on.
HBM_PROFILE = os.path.join(ROOT, "profiles", "dkdv_kernel_large_causal_bf16_hbm.md")
KERNEL_SOURCES = ["attn_bwd_kernels.h", "attn_bwd.hip", "attn_bwd_variant.hip", "ma_tiles.h", "ma_device.h",
                  "ma_launch.h", "capi.hip"]


def code_digest(texts):
    """SHA-256 of source texts with // comments, trailing blanks and empty lines removed (so a
    comment-only edit does not invalidate counters taken on the same code)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for text in texts:
        for line in text.splitlines():
            line = re.sub(r"//.*$", "", line).rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def kernel_source_digest():
    texts = []
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "masked_attention_backward_amd", "csrc", f)) as fh:
            texts.append(fh.read())
    return code_digest(texts)


def profiled_traffic():
    """Counter-measured bytes per launch of the dominant kernel, or None if they are stale."""
    try:
        with open(HBM_PROFILE) as fh:
            text = fh.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and line.split(":", 1)[0] in ("traffic-bytes-per-launch", "source-sha256"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    if fields.get("source-sha256") != kernel_source_digest():
        return None
    try:
        return int(fields["traffic-bytes-per-launch"])
    except (KeyError, ValueError):
        return None


def live_tiles_window(S, W, grid=64):
    """Count 64x64 (query-tile, key-tile) pairs holding at least one visible (i, j)."""
    n = (S + grid - 1) // grid
    count = 0
    for qi in range(n):
        q0, q1 = qi * grid, min(S, qi * grid + grid) - 1
        for kj in range(n):
            k0, k1 = kj * grid, min(S, kj * grid + grid) - 1
            if q1 - k0 >= 0 and q0 - k1 < W:
                count += 1
    return count


def counted_flops(wl, mask=None):
    D = wl.D
    if wl.kind == "sink":
        per_head = live_tiles_window(wl.Sq, min(wl.window, wl.Sq)) * 5 * 2 * 64 * 64 * D
        return per_head * wl.B * wl.Hq, per_head
    m = mask.numpy()
    rows = [min(wl.bx, wl.Sq - i * wl.bx) for i in range(wl.nqb)]
    cols = [min(wl.by, wl.Skv - j * wl.by) for j in range(wl.nkb)]
    import numpy as np
    area = (np.array(rows)[:, None] * np.array(cols)[None, :]) * (m != 0)
    total = float(area.sum()) * 5 * 2 * D
    return total, total / (wl.B * wl.Hq)


class HipEvents:
    """Minimal hipEvent wrapper (ctypes on libamdhip64) for events handed to the library."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e)
        return evs

    def elapsed(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def cpu_baseline(wl, x, budget_s):
    """Time the oracle backward on whole query heads until about budget_s seconds of work."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    heads, spent = 0, 0.0
    g = wl.Hq // wl.Hkv
    while spent < budget_s and heads < wl.Hq:
        h = heads
        sl = slice(h, h + 1)
        q, do = x["q"][:1, sl], x["do"][:1, sl]
        if wl.kind == "sink":
            k, v = x["k"][:1, h // g:h // g + 1], x["v"][:1, h // g:h // g + 1]
            sink = x["sink"][sl]
            o, lse = oracle.sink_attention_forward(q, k, v, sink, wl.window, wl.scale)
            t0 = time.perf_counter()
            oracle.sink_attention_backward(q, k, v, o, do, lse, sink, wl.window, wl.scale)
            spent += time.perf_counter() - t0
        else:
            k, v, m = x["k"][:1, sl], x["v"][:1, sl], x["block_mask"][:1, sl]
            o, lse = oracle.blocksparse_attention_forward(q, k, v, m, wl.bx, wl.by, wl.scale)
            t0 = time.perf_counter()
            oracle.blocksparse_attention_backward(q, k, v, o, do, lse, m, wl.bx, wl.by, wl.scale)
            spent += time.perf_counter() - t0
        heads += 1
    return heads, spent, cores


def bench_varlen(args):
    """The sink page's varlen row: 8 packed sequences of up to 2048 tokens, 64 query heads, 4 K/V
    heads (16 per group), D=128, fp16, causal within each sequence.  One step = one
    attn_sink_bwd_varlen call; the FLOP count sums each sequence's live tiles."""
    import torch
    from masked_attention_backward_amd import api, workloads as W

    dev = torch.device("cuda:0")
    lengths = W.varlen_lengths(8, 2048)
    hq, hkv, window = 64, 4, 2048
    x = W.varlen_inputs(lengths, hq, hkv, torch.float16)
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in x.items()}
    smax, scale = g["max_seqlen"], 1.0 / math.sqrt(128)
    o, lse = api.attn_sink_fwd_varlen(g["q"], g["k"], g["v"], g["sink"], g["cu_seqlens"], smax, window, scale)
    ws = torch.empty(api.attn_sink_bwd_workspace_bytes(len(lengths), hq, hkv, smax), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        api.attn_sink_bwd_varlen(g["q"], g["k"], g["v"], o, g["do"], lse, g["sink"], g["cu_seqlens"], smax, window,
                                 scale, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    flops = sum(live_tiles_window(L, min(window, L)) for L in lengths) * 5 * 2 * 64 * 64 * 128 * hq
    tflops = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": "attn-bwd TFLOP/s over unmasked tiles (% fp16 MFMA peak) + bwd ms",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic (seeded N(0,1) inputs, seeded lengths; O, lse from the library forward)",
        "config": {"workload": "varlen", "B": len(lengths), "Hq": hq, "Hkv": hkv, "lengths": lengths, "D": 128,
                   "window": window, "mask": "causal within each packed sequence + sink"},
        "pct_peak_mfma": round(100.0 * tflops / PEAK_MFMA_16BIT, 2),
        "counted_tflop": round(flops / 1e12, 4),
        "roofline": {"kernel": "whole backward call", "bound": "mfma", "achieved": round(tflops, 2),
                     "peak": PEAK_MFMA_16BIT, "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_16BIT, 4),
                     "traffic": None},
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_causal",
                    help="a registered workload name, or varlen (packed sequences of the sink page's varlen row)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle timing sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--with-copy-probe", action="store_true",
                    help="also run one 256 MiB device-to-device copy (a kernel of known traffic, used to scale "
                         "hardware byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this library runs and is measured on one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is "
              "not supported (sharding by (batch, kv-head) needs no communication and is described in the design "
              "notes, but no multi-GPU figure is produced).", file=sys.stderr)
        sys.exit(2)

    if args.workload == "varlen":
        bench_varlen(args)
        return

    import torch
    from masked_attention_backward_amd import api, workloads as W

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    x = W.make_inputs(wl)
    g = {k: v.to(dev) for k, v in x.items()}
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    dtype_code = api.MA_BF16 if wl.dtype == torch.bfloat16 else api.MA_F16

    if wl.kind == "sink":
        o, lse = api.attn_sink_fwd(g["q"], g["k"], g["v"], g["sink"], wl.window, wl.scale)
        nbytes = api.attn_sink_bwd_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq)
    else:
        o, lse = api.blocksparse_attn_fwd(g["q"], g["k"], g["v"], g["block_mask"], wl.bx, wl.by, wl.scale)
        nbytes = api.blocksparse_attn_bwd_workspace_bytes(wl.B, wl.Hq, wl.Sq, wl.Skv, wl.bx, wl.by)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
    dsink = torch.empty(wl.Hq, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    if wl.kind == "sink":
        call_args = [P(g["q"]), P(g["k"]), P(g["v"]), P(o), P(g["do"]), P(lse), P(g["sink"]), P(dq), P(dk), P(dv),
                     P(dsink), P(ws), nbytes, wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.D, wl.window, wl.scale, dtype_code, sp]
        fn, fn_timed = api.lib.attn_sink_bwd, api.lib.attn_sink_bwd_timed
    else:
        call_args = [P(g["q"]), P(g["k"]), P(g["v"]), P(o), P(g["do"]), P(lse), P(g["block_mask"]), P(dq), P(dk),
                     P(dv), P(ws), nbytes, wl.B, wl.Hq, wl.Sq, wl.Skv, wl.D, wl.bx, wl.by, wl.scale, dtype_code, sp]
        fn, fn_timed = api.lib.blocksparse_attn_bwd, api.lib.blocksparse_attn_bwd_timed

    def step():
        st = fn(*call_args)
        if st != 0:
            raise RuntimeError(f"backward failed with status {st}")

    if args.with_copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # Timed region: exactly K whole backward calls.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.4f} ms/step (wall {wall:.3f} s)", file=sys.stderr,
          flush=True)

    # Per-stage device time (events recorded by the library between its kernels).
    hip = HipEvents()
    evs = hip.create(4 * args.steps)
    arr = (ctypes.c_void_p * (4 * args.steps))(*[e.value for e in evs])
    for i in range(args.steps):
        st = fn_timed(*call_args, ctypes.cast(ctypes.byref(arr, 4 * i * ctypes.sizeof(ctypes.c_void_p)),
                                              ctypes.c_void_p))
        if st != 0:
            raise RuntimeError(f"timed backward failed with status {st}")
    torch.cuda.synchronize()
    pre = [hip.elapsed(evs[4 * i], evs[4 * i + 1]) for i in range(args.steps)]
    kdkv = [hip.elapsed(evs[4 * i + 1], evs[4 * i + 2]) for i in range(args.steps)]
    kdq = [hip.elapsed(evs[4 * i + 2], evs[4 * i + 3]) for i in range(args.steps)]
    hip.destroy(evs)
    mean = lambda v: sum(v) / len(v)  # noqa: E731

    # The forward that makes O and lse (support, not part of the step): timed for reference.
    def forward():
        if wl.kind == "sink":
            return api.attn_sink_fwd(g["q"], g["k"], g["v"], g["sink"], wl.window, wl.scale)
        return api.blocksparse_attn_fwd(g["q"], g["k"], g["v"], g["block_mask"], wl.bx, wl.by, wl.scale)

    forward()
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(3):
        forward()
    f1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = f0.elapsed_time(f1) / 3

    total_flops, per_head = counted_flops(wl, x.get("block_mask"))
    tflops = total_flops / (ms_per_step * 1e-3) / 1e12
    dkdv_alg = 0.8 * total_flops          # S, dP, dV, dK of the five counted GEMMs
    dkdv_ms = mean(kdkv)
    achieved = dkdv_alg / (dkdv_ms * 1e-3) / 1e12

    rec = {
        "metric": "attn-bwd TFLOP/s over unmasked tiles (% fp16 MFMA peak) + bwd ms",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f16",
        "data": "synthetic (seeded N(0,1) inputs; O, lse from the library forward)",
        "config": {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "Sq": wl.Sq, "Skv": wl.Skv, "D": wl.D,
                   "window": wl.window if wl.kind == "sink" else None, "bx": wl.bx or None, "by": wl.by or None,
                   "mask": wl.pattern or "sliding-window causal + sink"},
        "pct_peak_mfma": round(100.0 * tflops / PEAK_MFMA_16BIT, 2),
        "counted_tflop": round(total_flops / 1e12, 4),
        "kernels_ms": {"preprocess": round(mean(pre), 4), "dkdv": round(dkdv_ms, 4), "dq": round(mean(kdq), 4)},
        "fwd_ms_untimed_support": round(fwd_ms, 4),
        "roofline": {"kernel": "dkdv_kernel", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_MFMA_16BIT, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_MFMA_16BIT, 4),
                     "traffic": profiled_traffic() if wl.name == "large_causal" else None},
    }
    if not args.no_cpu_baseline:
        heads, spent, cores = cpu_baseline(wl, x, args.cpu_seconds)
        rec["cpu_baseline"] = {"value": round(per_head * heads / spent / 1e12, 6), "unit": "TFLOP/s",
                               "cores": cores, "kind": "oracle",
                               "sample": f"fp64 oracle backward of {heads} of {wl.B * wl.Hq} (batch, query head) "
                                         f"slices of {wl.name}, {spent:.1f} s; rate over that sample's live tiles"}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
