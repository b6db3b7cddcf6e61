#!/usr/bin/env python3
"""Benchmark of the masked attention backward on one MI355X.

Default workload: GQA sink attention backward, B=1 Hq=64 Hkv=8 S=8192 D=128, window = S
(full causal), bf16 -- the dense-window configuration, the only one whose live tiles make
it MFMA-bound.  One step = one whole backward call (preprocess + dK/dV with the dsink reduce +
dQ; for block-sparse workloads also the table build) on inputs already resident in HBM.
O and lse come from the library's own forward (untimed).

Metric: TFLOP/s counted over live tiles only, 5 GEMMs of 2*Br*Bc*D per live tile (64x64
counting grid for the window path; the mask blocks, edges clipped, for block-sparse).

Prints ONE JSON line.  `value` / `ms_per_step` time K back-to-back calls of the chosen
workload.  The roofline object describes the dominant kernel (dK/dV), timed live with HIP
events recorded by the library between its stages on the launch stream.  The cpu_baseline
leg times the fp64 oracle's backward on a bounded sample of the same workload.

The `configs` object (skipped with --no-configs) covers every synthetic configuration:
5 warm-up calls, then 5 interleaved rounds of 4 calls each (20 per configuration), every
call preceded by a 512 MiB write on the same stream (outside its events) so no input is
still cached; per-call median and minimum, TFLOP/s and the fraction of the bound the
configuration's arithmetic intensity sets (MFMA peak or 8 TB/s over the algorithmic bytes),
the back-to-back (warm) mean, the oracle's rate on a bounded sample, and the shader clock
sampled while the headline backward runs.
"""

import argparse
import ctypes
import json
import math
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_16BIT = 2516.6   # TFLOP/s, dense fp16/bf16 MFMA, 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_CLOCK_MHZ = 2400.0
PEAK_HBM = 8000.0          # GB/s
METRIC = "attn-bwd TFLOP/s over unmasked tiles (% fp16 MFMA peak) + bwd ms"

# HBM bytes per launch of the dominant kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# (scaled by a copy kernel of known size), valid only for the kernel sources they were taken on.
HBM_PROFILE = os.path.join(ROOT, "profiles", "dkdv_kernel_large_causal_bf16_hbm.md")
KERNEL_SOURCES = ["attn_bwd_kernels.h", "attn_bwd.hip", "attn_bwd_variant.hip", "ma_tiles.h", "ma_device.h",
                  "ma_launch.h", "capi.hip"]

# Which roofline bounds each configuration at its arithmetic intensity (counted FLOP against
# algorithmic bytes at 2516.6 TFLOP/s and 8 TB/s).
BOUND = {"tiny": "launch", "mid": "hbm", "large_w128": "hbm", "large_causal": "mfma", "bigbird": "hbm",
         "ragged": "mfma", "pages_h64_s4096": "mfma", "pages_h64_s4096_fwd": "mfma", "varlen_8x2048": "mfma",
         "varlen_mixed": "mfma"}
# Workspace size that selects the dQ path ("ds_bank": the dK/dV kernel stores dS and dQ is one
# GEMM per block; "recompute": the minimum workspace, dQ recomputes S and dP).
DQ_PATH = "ds_bank"
CONFIG_ORDER = ["tiny", "mid", "large_w128", "large_causal", "bigbird", "ragged", "pages_h64_s4096",
                "pages_h64_s4096_fwd", "varlen_8x2048", "varlen_mixed"]


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


def algorithmic_bytes(B, Hq, Hkv, Sq, Skv, D=128, elem=2, block_mask_bytes=0):
    """Bytes a backward call must move at least once: q, o, dO, k, v, lse in; dq, dk, dv out."""
    qsz = B * Hq * Sq * D * elem
    kvsz = B * Hkv * Skv * D * elem
    return 4 * qsz + 4 * kvsz + 4 * B * Hq * Sq + block_mask_bytes


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


# ------------------------------------------------------------------------------ oracle timing

def blas_threads():
    """Threads the oracle's BLAS may use: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when that is set (the host's CPU share for this process)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def oracle_sample(case, budget_s):
    """Time the fp64 oracle's backward on whole (batch, query head) slices of the case until
    about budget_s seconds of work; returns (slices, total slices, seconds, counted FLOP)."""
    import oracle
    x, kind = case.host, case.kind
    done, spent, flop = 0, 0.0, 0.0
    if kind == "varlen":
        vw = case.wl
        g = vw.Hq // vw.Hkv
        cu = x["cu_seqlens"].numpy()
        total = vw.Hq
        while spent < budget_s and done < total:
            h = done
            q, do = x["q"][h:h + 1], x["do"][h:h + 1]
            k, v = x["k"][h // g:h // g + 1], x["v"][h // g:h // g + 1]
            sink = x["sink"][h:h + 1]
            o, lse = oracle.sink_attention_forward_varlen(q, k, v, sink, cu, vw.window, vw.scale)
            t0 = time.perf_counter()
            oracle.sink_attention_backward_varlen(q, k, v, o, do, lse, sink, cu, vw.window, vw.scale)
            spent += time.perf_counter() - t0
            flop += case.flops / vw.Hq
            done += 1
        return done, total, spent, flop
    wl = case.wl
    g = wl.Hq // wl.Hkv
    total = wl.B * wl.Hq
    while spent < budget_s and done < total:
        b, h = divmod(done, wl.Hq)
        q, do = x["q"][b:b + 1, h:h + 1], x["do"][b:b + 1, h:h + 1]
        k, v = x["k"][b:b + 1, h // g:h // g + 1], x["v"][b:b + 1, h // g:h // g + 1]
        if wl.kind == "sink":
            sink = x["sink"][h:h + 1]
            o, lse = oracle.sink_attention_forward(q, k, v, sink, wl.window, wl.scale)
            t0 = time.perf_counter()
            oracle.sink_attention_backward(q, k, v, o, do, lse, sink, wl.window, wl.scale)
            spent += time.perf_counter() - t0
            flop += case.flops / total
        else:
            m = x["block_mask"][b:b + 1, h:h + 1]
            o, lse = oracle.blocksparse_attention_forward(q, k, v, m, wl.bx, wl.by, wl.scale)
            t0 = time.perf_counter()
            oracle.blocksparse_attention_backward(q, k, v, o, do, lse, m, wl.bx, wl.by, wl.scale)
            spent += time.perf_counter() - t0
            flop += counted_flops(wl.with_(B=1, Hq=1, Hkv=1), m)[0]
        done += 1
    return done, total, spent, flop


def oracle_rate(case, budget_s, threads):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=threads):
        done, total, spent, flop = oracle_sample(case, budget_s)
    return {"value": round(flop / spent / 1e12, 6) if spent > 0 else None, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 oracle backward of {done} of {total} query-head slices of {case.name} "
                      f"({'packed sequences, ' if case.kind == 'varlen' else ''}{spent:.1f} s); rate over that "
                      f"sample's counted FLOP"}


# --------------------------------------------------------------------------- clock sampling

CLOCK_PROBE = r"""
import json, sys, time
import amdsmi
amdsmi.amdsmi_init()
hs = amdsmi.amdsmi_get_processor_handles()
out = {"samples": [[] for _ in hs], "bdf": []}
for h in hs:
    try:
        out["bdf"].append(amdsmi.amdsmi_get_gpu_device_bdf(h))
    except Exception:
        out["bdf"].append(None)
t_end = time.time() + float(sys.argv[1])
while time.time() < t_end:
    for i, h in enumerate(hs):
        try:
            clk = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"]
            act = amdsmi.amdsmi_get_gpu_activity(h)["gfx_activity"]
            out["samples"][i].append([clk, act])
        except Exception:
            pass
    time.sleep(0.02)
amdsmi.amdsmi_shut_down()
print(json.dumps(out))
"""


def sample_clock_during(run_seconds, launch_loop):
    """Shader (GFX) clock sampled by amdsmi in a child process while launch_loop() keeps the
    GPU busy; the GPU with the highest mean activity is taken as this one.  None when amdsmi
    is unavailable."""
    try:
        p = subprocess.Popen([sys.executable, "-c", CLOCK_PROBE, str(run_seconds)], stdout=subprocess.PIPE,
                             stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    time.sleep(0.3)
    launch_loop()
    try:
        out, _ = p.communicate(timeout=run_seconds + 20)
        data = json.loads(out)
    except Exception:
        p.kill()
        return None
    best = None
    for i, smp in enumerate(data["samples"]):
        busy = [c for c, a in smp if a is not None and a >= 50]
        if not smp:
            continue
        act = statistics.mean(a for _, a in smp)
        if busy and (best is None or act > best[0]):
            best = (act, i, busy)
    if best is None:
        return None
    act, i, busy = best
    return {"mhz_median": statistics.median(busy), "mhz_min": min(busy), "mhz_max": max(busy),
            "samples": len(busy), "gfx_activity_mean_pct": round(act, 1), "bdf": data["bdf"][i],
            "source": "amdsmi GFX clock, sampled every 20 ms while the headline backward ran back to back"}


# ------------------------------------------------------------------------------------ cases

class Case:
    """One configuration on the device: inputs resident, O and lse from the library forward,
    outputs and workspace allocated; run() enqueues one call through the C ABI."""

    def __init__(self, name, kind, wl, host, run, flops, alg_bytes, dtype, config, run_timed=None):
        self.name, self.kind, self.wl, self.host = name, kind, wl, host
        self.run, self.run_timed = run, run_timed
        self.flops, self.alg_bytes, self.dtype, self.config = flops, alg_bytes, dtype, config


def dq_path_of(case):
    """The dQ path a backward case runs (None for the forward)."""
    if case.kind in ("sink", "varlen", "blocksparse"):
        return DQ_PATH
    return None


def make_case(name, dev):
    import torch
    from masked_attention_backward_amd import api, workloads as W

    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def status(fn):
        def call(*a):
            st = fn(*a)
            if st != 0:
                raise RuntimeError(f"{fn.__name__} failed with status {st}")
        return call

    if name in W.VARLEN:
        vw = W.VARLEN[name]
        x = vw.inputs()
        g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in x.items()}
        smax = g["max_seqlen"]
        o, lse = api.attn_sink_fwd_varlen(g["q"], g["k"], g["v"], g["sink"], g["cu_seqlens"], smax, vw.window, vw.scale)
        B, T = len(vw.lengths), sum(vw.lengths)
        nbytes = (api.attn_sink_bwd_ds_workspace_bytes(B, vw.Hq, vw.Hkv, smax, vw.window) if DQ_PATH == "ds_bank"
                  else api.attn_sink_bwd_workspace_bytes(B, vw.Hq, vw.Hkv, smax))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
        dsink = torch.empty(vw.Hq, dtype=torch.float32, device=dev)
        args = [P(g["q"]), P(g["k"]), P(g["v"]), P(o), P(g["do"]), P(lse), P(g["sink"]), P(g["cu_seqlens"]), P(dq),
                P(dk), P(dv), P(dsink), P(ws), nbytes, B, T, smax, vw.Hq, vw.Hkv, vw.D, vw.window, vw.scale,
                api.MA_F16 if vw.dtype == torch.float16 else api.MA_BF16, sp]
        fn = status(api.lib.attn_sink_bwd_varlen)
        flops = sum(live_tiles_window(L, min(vw.window, L)) for L in vw.lengths) * 5 * 2 * 64 * 64 * vw.D * vw.Hq
        keep = (g, o, lse, ws, dq, dk, dv, dsink)
        run = lambda: fn(*args) or keep  # noqa: E731
        cfg = {"workload": name, "B": B, "Hq": vw.Hq, "Hkv": vw.Hkv, "lengths": list(vw.lengths), "D": vw.D,
               "window": vw.window, "mask": "causal within each packed sequence + sink"}
        return Case(name, "varlen", vw, x, run, flops, algorithmic_bytes(1, vw.Hq, vw.Hkv, T, T, vw.D), "f16", cfg)

    fwd_only = name.endswith("_fwd")
    wl = W.WORKLOADS[name[:-4] if fwd_only else name]
    x = W.make_inputs(wl)
    g = {k: v.to(dev) for k, v in x.items()}
    dtype_code = api.MA_BF16 if wl.dtype == torch.bfloat16 else api.MA_F16
    dts = "bf16" if wl.dtype == torch.bfloat16 else "f16"
    total_flops, _ = counted_flops(wl, x.get("block_mask"))
    cfg = {"workload": name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "Sq": wl.Sq, "Skv": wl.Skv, "D": wl.D,
           "window": wl.window if wl.kind == "sink" else None, "bx": wl.bx or None, "by": wl.by or None,
           "mask": wl.pattern or "sliding-window causal + sink"}
    if fwd_only:
        o = torch.empty_like(g["q"])
        lse = torch.empty((wl.B, wl.Hq, wl.Sq), dtype=torch.float32, device=dev)
        args = [P(g["q"]), P(g["k"]), P(g["v"]), P(g["sink"]), P(o), P(lse), wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.D,
                wl.window, wl.scale, dtype_code, sp]
        fn = status(api.lib.attn_sink_fwd)
        keep = (g, o, lse)
        cfg["pass"] = "forward (2 GEMMs per live tile counted)"
        fl = total_flops * 2 / 5
        qsz, kvsz = wl.B * wl.Hq * wl.Sq * wl.D * 2, wl.B * wl.Hkv * wl.Skv * wl.D * 2
        return Case(name, "fwd", wl, x, lambda: fn(*args) or keep, fl, 2 * qsz + 2 * kvsz + 4 * wl.B * wl.Hq * wl.Sq,
                    dts, cfg)
    if wl.kind == "sink":
        o, lse = api.attn_sink_fwd(g["q"], g["k"], g["v"], g["sink"], wl.window, wl.scale)
        nbytes = (api.attn_sink_bwd_ds_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.window) if DQ_PATH == "ds_bank"
                  else api.attn_sink_bwd_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq))
    else:
        o, lse = api.blocksparse_attn_fwd(g["q"], g["k"], g["v"], g["block_mask"], wl.bx, wl.by, wl.scale)
        nbytes = (api.blocksparse_attn_bwd_ds_workspace_bytes(wl.B, wl.Hq, wl.Sq, wl.Skv, wl.bx, wl.by)
                  if DQ_PATH == "ds_bank" else api.blocksparse_attn_bwd_workspace_bytes(wl.B, wl.Hq, wl.Sq, wl.Skv,
                                                                                       wl.bx, wl.by))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
    dsink = torch.empty(wl.Hq, dtype=torch.float32, device=dev)
    if wl.kind == "sink":
        args = [P(g["q"]), P(g["k"]), P(g["v"]), P(o), P(g["do"]), P(lse), P(g["sink"]), P(dq), P(dk), P(dv),
                P(dsink), P(ws), nbytes, wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.D, wl.window, wl.scale, dtype_code, sp]
        fn, fn_timed = api.lib.attn_sink_bwd, api.lib.attn_sink_bwd_timed
        mbytes = 0
    else:
        args = [P(g["q"]), P(g["k"]), P(g["v"]), P(o), P(g["do"]), P(lse), P(g["block_mask"]), P(dq), P(dk), P(dv),
                P(ws), nbytes, wl.B, wl.Hq, wl.Sq, wl.Skv, wl.D, wl.bx, wl.by, wl.scale, dtype_code, sp]
        fn, fn_timed = api.lib.blocksparse_attn_bwd, api.lib.blocksparse_attn_bwd_timed
        mbytes = wl.B * wl.Hq * wl.nqb * wl.nkb
    keep = (g, o, lse, ws, dq, dk, dv, dsink)
    call, call_timed = status(fn), status(fn_timed)
    run = lambda: call(*args) or keep  # noqa: E731
    run_timed = lambda evp: call_timed(*args, evp) or keep  # noqa: E731
    return Case(name, wl.kind, wl, x, run, total_flops,
                algorithmic_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.Skv, wl.D, block_mask_bytes=mbytes), dts, cfg,
                run_timed)


def roofline_fracs(case, ms):
    tflops = case.flops / (ms * 1e-3) / 1e12
    gbs = case.alg_bytes / (ms * 1e-3) / 1e9
    bound = BOUND.get(case.name, "mfma")
    return tflops, gbs, bound


# ------------------------------------------------------------------------------------ sweep

def sweep(cases, rounds, calls, warm, dev):
    """Per-call device time with a 512 MiB flush write before every call (outside the
    events), configurations interleaved round by round."""
    import torch
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    times = {c.name: [] for c in cases}
    for c in cases:
        for _ in range(warm):
            flush.fill_(1)
            c.run()
    torch.cuda.synchronize()
    for r in range(rounds):
        pend = []
        for c in cases:
            for i in range(calls):
                flush.fill_(r + i)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                c.run()
                e1.record(stream)
                pend.append((c.name, e0, e1))
        torch.cuda.synchronize()
        for n, e0, e1 in pend:
            times[n].append(e0.elapsed_time(e1))
        print(f"[bench] configs: round {r + 1}/{rounds} done", file=sys.stderr, flush=True)
    warm_ms = {}
    for c in cases:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            c.run()
        e1.record(stream)
        torch.cuda.synchronize()
        warm_ms[c.name] = e0.elapsed_time(e1) / 10
    del flush
    return times, warm_ms


def config_record(case, times, warm_ms, clock_mhz, oracle):
    med, mn = statistics.median(times), min(times)
    tflops, gbs, bound = roofline_fracs(case, med)
    peak_clk = PEAK_MFMA_16BIT * (clock_mhz / PEAK_CLOCK_MHZ) if clock_mhz else None
    rec = {"config": case.config, "dtype": case.dtype, "calls": len(times), "ms_median": round(med, 4),
           "ms_min": round(mn, 4), "ms_warm_back_to_back": round(warm_ms, 4),
           "counted_tflop": round(case.flops / 1e12, 5), "tflops_median": round(tflops, 2),
           "pct_peak_mfma": round(100 * tflops / PEAK_MFMA_16BIT, 2),
           "pct_peak_mfma_at_clock": round(100 * tflops / peak_clk, 2) if peak_clk else None,
           "algorithmic_bytes": case.alg_bytes, "hbm_gbs_algorithmic": round(gbs, 1),
           "pct_hbm_8tbs": round(100 * gbs / PEAK_HBM, 2), "bound": bound,
           "frac_of_bound": round(tflops / PEAK_MFMA_16BIT if bound == "mfma" else gbs / PEAK_HBM, 4),
           "dq_path": dq_path_of(case)}
    if oracle is not None:
        rec["oracle"] = oracle
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_causal", help="the timed workload (a name in CONFIG_ORDER)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the headline oracle sample")
    ap.add_argument("--config-cpu-seconds", type=float, default=2.0, help="oracle budget per other configuration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration sweep")
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--calls", type=int, default=4, help="calls per configuration per round")
    ap.add_argument("--dq-path", choices=["ds_bank", "recompute"], default="ds_bank",
                    help="workspace size selecting how dQ is computed")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the shader-clock sample (about 2 s of back-to-back calls), e.g. under a profiler")
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
    if args.workload not in CONFIG_ORDER:
        print(f"bench.py: unknown workload {args.workload!r}; one of {CONFIG_ORDER}", file=sys.stderr)
        sys.exit(2)

    global DQ_PATH
    DQ_PATH = args.dq_path
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    head = make_case(args.workload, dev)
    torch.cuda.synchronize()

    if args.with_copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        head.run()
    torch.cuda.synchronize()
    print(f"[bench] {head.name}: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # Timed region: exactly K whole calls, back to back.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        head.run()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.4f} ms/step (wall {wall:.3f} s)", file=sys.stderr,
          flush=True)

    tflops = head.flops / (ms_per_step * 1e-3) / 1e12
    rec = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": head.dtype,
        "data": "synthetic (seeded N(0,1) inputs; O, lse from the library forward)",
        "config": head.config, "dq_path": dq_path_of(head),
        "pct_peak_mfma": round(100.0 * tflops / PEAK_MFMA_16BIT, 2),
        "counted_tflop": round(head.flops / 1e12, 4),
    }

    # Per-stage device time (events recorded by the library between its kernels).
    if head.run_timed is not None:
        hip = HipEvents()
        evs = hip.create(4 * args.steps)
        arr = (ctypes.c_void_p * (4 * args.steps))(*[e.value for e in evs])
        for i in range(args.steps):
            head.run_timed(ctypes.cast(ctypes.byref(arr, 4 * i * ctypes.sizeof(ctypes.c_void_p)), ctypes.c_void_p))
        torch.cuda.synchronize()
        pre = [hip.elapsed(evs[4 * i], evs[4 * i + 1]) for i in range(args.steps)]
        kdkv = [hip.elapsed(evs[4 * i + 1], evs[4 * i + 2]) for i in range(args.steps)]
        kdq = [hip.elapsed(evs[4 * i + 2], evs[4 * i + 3]) for i in range(args.steps)]
        hip.destroy(evs)
        dkdv_ms = statistics.mean(kdkv)
        achieved = 0.8 * head.flops / (dkdv_ms * 1e-3) / 1e12   # S, dP, dV, dK of the five counted GEMMs
        rec["kernels_ms"] = {"preprocess": round(statistics.mean(pre), 4), "dkdv": round(dkdv_ms, 4),
                             "dq": round(statistics.mean(kdq), 4)}
        rec["roofline"] = {"kernel": "dkdv_kernel", "bound": "mfma", "achieved": round(achieved, 2),
                           "peak": PEAK_MFMA_16BIT, "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_16BIT, 4),
                           "traffic": profiled_traffic() if head.name == "large_causal" else None}
    else:
        rec["roofline"] = {"kernel": "whole call", "bound": "mfma", "achieved": round(tflops, 2),
                           "peak": PEAK_MFMA_16BIT, "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_16BIT, 4),
                           "traffic": None}

    # Shader clock while the headline call runs back to back (about 2 s of work).
    n_loop = max(50, int(2000.0 / max(ms_per_step, 1e-3)))

    def loop():
        for _ in range(n_loop):
            head.run()
        torch.cuda.synchronize()

    clock = None if args.no_clock else sample_clock_during(n_loop * ms_per_step / 1000.0 + 0.5, loop)
    rec["clock"] = clock
    clock_mhz = clock["mhz_median"] if clock else None
    if clock_mhz:
        rec["pct_peak_mfma_at_clock"] = round(100.0 * tflops / (PEAK_MFMA_16BIT * clock_mhz / PEAK_CLOCK_MHZ), 2)

    threads = blas_threads()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = oracle_rate(head, args.cpu_seconds, threads)
        rec["cpu_baseline"]["host_cpus"] = os.cpu_count()

    if not args.no_configs:
        cases = [head if n == head.name else make_case(n, dev) for n in CONFIG_ORDER]
        torch.cuda.synchronize()
        times, warm = sweep(cases, args.rounds, args.calls, args.warmup, dev)
        out = {}
        for c in cases:
            orc = None
            if not args.no_cpu_baseline:
                orc = rec["cpu_baseline"] if c is head else oracle_rate(c, args.config_cpu_seconds, threads)
            out[c.name] = config_record(c, times[c.name], warm[c.name], clock_mhz, orc)
        rec["configs"] = out
        rec["configs_method"] = (f"{args.warmup} warm-up calls, then {args.rounds} interleaved rounds x {args.calls} "
                                 "calls per configuration, each call preceded by a 512 MiB write on the same stream "
                                 "(outside its HIP events); median and min per call; warm = mean of 10 back-to-back "
                                 "calls; frac_of_bound = TFLOP/s / 2516.6 (mfma) or algorithmic GB/s / 8000 (hbm)")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
