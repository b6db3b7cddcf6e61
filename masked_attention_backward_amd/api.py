"""Thin torch binding of ``libmaskattn.so`` (argument marshalling only).

Each function checks tensor shapes/dtypes/devices, allocates outputs and the workspace
with torch on the tensors' device, and calls the C ABI of the same name with raw device
pointers and torch's current HIP stream.  Every step of the computation runs in the HIP
kernels; nothing here computes attention.  Importing this module raises if the library
has not been built (``python -m masked_attention_backward_amd.build``).
"""

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmaskattn.so")

MA_F16, MA_BF16 = 0, 1
STATUS = {0: "MA_OK", 1: "MA_EINVAL", 2: "MA_EUNSUPPORTED", 3: "MA_EWORKSPACE", 4: "MA_ELAUNCH", 5: "MA_ESCRATCH"}
NOALLOC_SCRATCH_BYTES = 32 << 20   # MA_NOALLOC_SCRATCH_BYTES

EXPORTS = (
    "maskattn_strerror",
    "attn_sink_fwd",
    "attn_sink_bwd_workspace_bytes",
    "attn_sink_bwd",
    "blocksparse_build_tables",
    "blocksparse_attn_fwd",
    "blocksparse_attn_bwd_workspace_bytes",
    "blocksparse_attn_bwd",
    "attn_sink_bwd_timed",
    "blocksparse_attn_bwd_timed",
    "blocksparse_attn_fwd_gqa",
    "blocksparse_attn_bwd_gqa",
    "attn_sink_fwd_varlen",
    "attn_sink_bwd_varlen",
    "attn_sink_bwd_noalloc",
    "attn_sink_bwd_ds_workspace_bytes",
    "blocksparse_attn_bwd_ds_workspace_bytes",
)


class MaskAttnError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m masked_attention_backward_amd.build` "
                          "(the HIP library is the only implementation; there is no fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.maskattn_strerror.argtypes = [I]
    lib.maskattn_strerror.restype = ctypes.c_char_p
    lib.attn_sink_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, P]
    lib.attn_sink_fwd.restype = I
    lib.attn_sink_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.attn_sink_bwd_workspace_bytes.restype = Z
    lib.attn_sink_bwd.argtypes = [P] * 11 + [P, Z] + [I] * 6 + [F, I, P]
    lib.attn_sink_bwd.restype = I
    lib.blocksparse_build_tables.argtypes = [P, I, I, I, I, P, P, P, P, P, P]
    lib.blocksparse_build_tables.restype = I
    lib.blocksparse_attn_fwd.argtypes = [P, P, P, P, P, P, P, Z] + [I] * 7 + [F, I, P]
    lib.blocksparse_attn_fwd.restype = I
    lib.blocksparse_attn_bwd_workspace_bytes.argtypes = [I] * 7
    lib.blocksparse_attn_bwd_workspace_bytes.restype = Z
    lib.blocksparse_attn_bwd.argtypes = [P] * 10 + [P, Z] + [I] * 7 + [F, I, P]
    lib.blocksparse_attn_bwd.restype = I
    lib.attn_sink_bwd_timed.argtypes = lib.attn_sink_bwd.argtypes + [P]
    lib.attn_sink_bwd_timed.restype = I
    lib.blocksparse_attn_bwd_timed.argtypes = lib.blocksparse_attn_bwd.argtypes + [P]
    lib.blocksparse_attn_bwd_timed.restype = I
    lib.blocksparse_attn_fwd_gqa.argtypes = [P, P, P, P, P, P, P, Z] + [I] * 8 + [F, I, P]
    lib.blocksparse_attn_fwd_gqa.restype = I
    lib.blocksparse_attn_bwd_gqa.argtypes = [P] * 10 + [P, Z] + [I] * 8 + [F, I, P]
    lib.blocksparse_attn_bwd_gqa.restype = I
    lib.attn_sink_fwd_varlen.argtypes = [P] * 7 + [I] * 7 + [F, I, P]
    lib.attn_sink_fwd_varlen.restype = I
    lib.attn_sink_bwd_varlen.argtypes = [P] * 12 + [P, Z] + [I] * 7 + [F, I, P]
    lib.attn_sink_bwd_varlen.restype = I
    lib.attn_sink_bwd_noalloc.argtypes = [P] * 11 + [I] * 6 + [F, I, P]
    lib.attn_sink_bwd_noalloc.restype = I
    lib.attn_sink_bwd_ds_workspace_bytes.argtypes = [I] * 6
    lib.attn_sink_bwd_ds_workspace_bytes.restype = Z
    lib.blocksparse_attn_bwd_ds_workspace_bytes.argtypes = [I] * 7
    lib.blocksparse_attn_bwd_ds_workspace_bytes.restype = Z
    return lib


lib = _load()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float16:
        return MA_F16
    if t.dtype == torch.bfloat16:
        return MA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16")


def _check(fn, status):
    if status != 0:
        raise MaskAttnError(fn, status, lib.maskattn_strerror(status).decode())


def _need(t, name, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _workspace(nbytes, device, given=None):
    """The caller's workspace after checking it (uint8, contiguous, on `device`, at least
    `nbytes` bytes), or a new one of that size."""
    nbytes = int(nbytes)
    if given is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if not torch.is_tensor(given):
        raise TypeError("workspace: expected a torch.uint8 tensor")
    if given.dtype != torch.uint8:
        raise TypeError(f"workspace: expected torch.uint8, got {given.dtype}")
    if given.device != device:
        raise ValueError(f"workspace: expected device {device}, got {given.device}")
    if not given.is_contiguous():
        raise ValueError("workspace: must be contiguous")
    if given.numel() < nbytes:
        raise ValueError(f"workspace: {given.numel()} bytes, at least {nbytes} needed")
    return given


def _default_workspace(bank_bytes, min_bytes, device):
    """The workspace a call allocates when the caller gives none: the dS-bank size, unless that
    would take more than half of the device's free memory, then the minimum size (the library
    then recomputes S and dP for dQ instead of reading dS back)."""
    bank_bytes, min_bytes = int(bank_bytes), int(min_bytes)
    if bank_bytes > min_bytes:
        free, _ = torch.cuda.mem_get_info(device)
        if bank_bytes > free // 2:
            bank_bytes = min_bytes
    return _workspace(bank_bytes, device)


# --------------------------------------------------------------------------- sink path

def attn_sink_fwd(q, k, v, sink, window, scale=None):
    """Forward with sink and sliding window. q [B,Hq,S,128], k/v [B,Hkv,S,128], sink [Hq] fp32 -> (o, lse)."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    _need(k, "k", (B, Hkv, S, D), q.dtype, dev)
    _need(v, "v", (B, Hkv, S, D), q.dtype, dev)
    _need(sink, "sink", (Hq,), torch.float32, dev)
    _need(q, "q", (B, Hq, S, D), q.dtype, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    st = lib.attn_sink_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(o), _ptr(lse), B, Hq, Hkv, S, D, int(window),
                           scale, _dtype_code(q), _stream(dev))
    _check("attn_sink_fwd", st)
    return o, lse


def attn_sink_bwd_workspace_bytes(B, Hq, Hkv, S, D=128):
    return int(lib.attn_sink_bwd_workspace_bytes(B, Hq, Hkv, S, D))


def attn_sink_bwd_ds_workspace_bytes(B, Hq, Hkv, S, window, D=128):
    return int(lib.attn_sink_bwd_ds_workspace_bytes(B, Hq, Hkv, S, D, int(window)))


def attn_sink_bwd(q, k, v, o, do, lse, sink, window, scale=None, workspace=None, return_delta=False):
    """Backward with sink and sliding window -> (dq, dk, dv, dsink) [+ delta if return_delta].
    Without a workspace one of attn_sink_bwd_ds_workspace_bytes() is allocated (the dS-bank
    path), or of the minimum size when the bank would take more than half of the free device
    memory; a caller workspace of attn_sink_bwd_workspace_bytes() selects the recompute path."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    for name, t in (("q", q), ("o", o), ("do", do)):
        _need(t, name, (B, Hq, S, D), q.dtype, dev)
    _need(k, "k", (B, Hkv, S, D), q.dtype, dev)
    _need(v, "v", (B, Hkv, S, D), q.dtype, dev)
    _need(lse, "lse", (B, Hq, S), torch.float32, dev)
    _need(sink, "sink", (Hq,), torch.float32, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    ws = _workspace(attn_sink_bwd_workspace_bytes(B, Hq, Hkv, S, D), dev, workspace) if workspace is not None \
        else _default_workspace(attn_sink_bwd_ds_workspace_bytes(B, Hq, Hkv, S, window, D),
                                attn_sink_bwd_workspace_bytes(B, Hq, Hkv, S, D), dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dsink = torch.empty((Hq,), dtype=torch.float32, device=dev)
    st = lib.attn_sink_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(sink), _ptr(dq), _ptr(dk),
                           _ptr(dv), _ptr(dsink), _ptr(ws), ws.numel(), B, Hq, Hkv, S, D, int(window), scale,
                           _dtype_code(q), _stream(dev))
    _check("attn_sink_bwd", st)
    if return_delta:
        sp = (S + 63) // 64 * 64
        delta = ws[: B * Hq * sp * 4].view(torch.float32).view(B, Hq, sp)[..., :S]
        return dq, dk, dv, dsink, delta
    return dq, dk, dv, dsink


def attn_sink_bwd_noalloc(q, k, v, o, do, lse, sink, window, scale=None):
    """attn_sink_bwd without a workspace: the library's static scratch array holds Delta, lse*log2e
    and the dsink partials (calls that overlap on one GPU race) -> (dq, dk, dv, dsink)."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    for name, t in (("q", q), ("o", o), ("do", do)):
        _need(t, name, (B, Hq, S, D), q.dtype, dev)
    _need(k, "k", (B, Hkv, S, D), q.dtype, dev)
    _need(v, "v", (B, Hkv, S, D), q.dtype, dev)
    _need(lse, "lse", (B, Hq, S), torch.float32, dev)
    _need(sink, "sink", (Hq,), torch.float32, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dsink = torch.empty((Hq,), dtype=torch.float32, device=dev)
    st = lib.attn_sink_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(sink), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(dsink), B, Hq, Hkv, S, D, int(window), scale,
                                   _dtype_code(q), _stream(dev))
    _check("attn_sink_bwd_noalloc", st)
    return dq, dk, dv, dsink


def _varlen_shapes(q, k, cu_seqlens, max_seqlen):
    Hq, total, D = q.shape
    Hkv = k.shape[0]
    dev = q.device
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens: expected a 1-D int32 tensor of B + 1 offsets")
    _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32, dev)
    return cu_seqlens.numel() - 1, Hq, Hkv, total, D, int(max_seqlen), dev


def attn_sink_fwd_varlen(q, k, v, sink, cu_seqlens, max_seqlen, window, scale=None):
    """Forward over packed sequences. q [Hq,total,128], k/v [Hkv,total,128], cu_seqlens [B+1] int32
    (device), max_seqlen a host int -> (o [Hq,total,128], lse [Hq,total])."""
    B, Hq, Hkv, total, D, smax, dev = _varlen_shapes(q, k, cu_seqlens, max_seqlen)
    _need(q, "q", (Hq, total, D), q.dtype, dev)
    _need(k, "k", (Hkv, total, D), q.dtype, dev)
    _need(v, "v", (Hkv, total, D), q.dtype, dev)
    _need(sink, "sink", (Hq,), torch.float32, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, total), dtype=torch.float32, device=dev)
    st = lib.attn_sink_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(cu_seqlens), _ptr(o), _ptr(lse), B,
                                  total, smax, Hq, Hkv, D, int(window), scale, _dtype_code(q), _stream(dev))
    _check("attn_sink_fwd_varlen", st)
    return o, lse


def attn_sink_bwd_varlen(q, k, v, o, do, lse, sink, cu_seqlens, max_seqlen, window, scale=None, workspace=None):
    """Backward over packed sequences (layouts as attn_sink_fwd_varlen) -> (dq, dk, dv, dsink);
    workspace as attn_sink_bwd (dS-bank path by default)."""
    B, Hq, Hkv, total, D, smax, dev = _varlen_shapes(q, k, cu_seqlens, max_seqlen)
    for name, t in (("q", q), ("o", o), ("do", do)):
        _need(t, name, (Hq, total, D), q.dtype, dev)
    _need(k, "k", (Hkv, total, D), q.dtype, dev)
    _need(v, "v", (Hkv, total, D), q.dtype, dev)
    _need(lse, "lse", (Hq, total), torch.float32, dev)
    _need(sink, "sink", (Hq,), torch.float32, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    ws = _workspace(attn_sink_bwd_workspace_bytes(B, Hq, Hkv, smax, D), dev, workspace) if workspace is not None \
        else _default_workspace(attn_sink_bwd_ds_workspace_bytes(B, Hq, Hkv, smax, window, D),
                                attn_sink_bwd_workspace_bytes(B, Hq, Hkv, smax, D), dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dsink = torch.empty((Hq,), dtype=torch.float32, device=dev)
    st = lib.attn_sink_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(sink),
                                  _ptr(cu_seqlens), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsink), _ptr(ws), ws.numel(),
                                  B, total, smax, Hq, Hkv, D, int(window), scale, _dtype_code(q), _stream(dev))
    _check("attn_sink_bwd_varlen", st)
    return dq, dk, dv, dsink


# ---------------------------------------------------------------------- block-sparse

def blocksparse_build_tables(block_mask):
    """uint8 mask [B,N,nqb,nkb] -> dict(mask_t, sel_q, cnt_q, sel_k, cnt_k) built on the device."""
    B, N, nqb, nkb = block_mask.shape
    dev = block_mask.device
    _need(block_mask, "block_mask", (B, N, nqb, nkb), torch.uint8, dev)
    out = {
        "mask_t": torch.empty((B, N, nkb, nqb), dtype=torch.uint8, device=dev),
        "sel_q": torch.empty((B, N, nqb, nkb), dtype=torch.int32, device=dev),
        "cnt_q": torch.empty((B, N, nqb), dtype=torch.int32, device=dev),
        "sel_k": torch.empty((B, N, nkb, nqb), dtype=torch.int32, device=dev),
        "cnt_k": torch.empty((B, N, nkb), dtype=torch.int32, device=dev),
    }
    st = lib.blocksparse_build_tables(_ptr(block_mask), B, N, nqb, nkb, _ptr(out["mask_t"]), _ptr(out["sel_q"]),
                                      _ptr(out["cnt_q"]), _ptr(out["sel_k"]), _ptr(out["cnt_k"]), _stream(dev))
    _check("blocksparse_build_tables", st)
    return out


def blocksparse_attn_bwd_workspace_bytes(B, N, Sq, Skv, bx, by, D=128):
    return int(lib.blocksparse_attn_bwd_workspace_bytes(B, N, Sq, Skv, D, bx, by))


def blocksparse_attn_bwd_ds_workspace_bytes(B, N, Sq, Skv, bx, by, D=128):
    return int(lib.blocksparse_attn_bwd_ds_workspace_bytes(B, N, Sq, Skv, D, bx, by))


def _block_shapes(q, k, block_mask, bx, by):
    B, N, Sq, D = q.shape
    Nkv, Skv = k.shape[1], k.shape[2]
    nqb, nkb = -(-Sq // bx), -(-Skv // by)
    _need(block_mask, "block_mask", (B, N, nqb, nkb), torch.uint8, q.device)
    return B, N, Nkv, Sq, Skv, D


def blocksparse_attn_fwd(q, k, v, block_mask, bx, by, scale=None, workspace=None):
    """Block-sparse forward. q [B,N,Sq,128], k/v [B,Nkv,Skv,128] (N % Nkv == 0; Nkv < N groups
    the query heads as GQA) -> (o, lse); empty rows: o=0, lse=-inf."""
    B, N, Nkv, Sq, Skv, D = _block_shapes(q, k, block_mask, bx, by)
    dev = q.device
    _need(q, "q", (B, N, Sq, D), q.dtype, dev)
    _need(k, "k", (B, Nkv, Skv, D), q.dtype, dev)
    _need(v, "v", (B, Nkv, Skv, D), q.dtype, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    ws = _workspace(blocksparse_attn_bwd_workspace_bytes(B, N, Sq, Skv, bx, by, D), dev, workspace)
    o = torch.empty_like(q)
    lse = torch.empty((B, N, Sq), dtype=torch.float32, device=dev)
    if Nkv == N:
        st = lib.blocksparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(block_mask), _ptr(o), _ptr(lse), _ptr(ws),
                                      ws.numel(), B, N, Sq, Skv, D, bx, by, scale, _dtype_code(q), _stream(dev))
    else:
        st = lib.blocksparse_attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(block_mask), _ptr(o), _ptr(lse),
                                          _ptr(ws), ws.numel(), B, N, Nkv, Sq, Skv, D, bx, by, scale, _dtype_code(q),
                                          _stream(dev))
    _check("blocksparse_attn_fwd", st)
    return o, lse


def blocksparse_attn_bwd(q, k, v, o, do, lse, block_mask, bx, by, scale=None, workspace=None):
    """Block-sparse backward -> (dq, dk, dv); k/v (and dk/dv) may have fewer heads (GQA).

    Without a workspace one of blocksparse_attn_bwd_ds_workspace_bytes() is allocated (the
    dS-bank path), or of the minimum size when the bank would take more than half of the free
    device memory; a caller workspace of
    blocksparse_attn_bwd_workspace_bytes() selects the recompute path."""
    B, N, Nkv, Sq, Skv, D = _block_shapes(q, k, block_mask, bx, by)
    dev = q.device
    for name, t in (("q", q), ("o", o), ("do", do)):
        _need(t, name, (B, N, Sq, D), q.dtype, dev)
    _need(k, "k", (B, Nkv, Skv, D), q.dtype, dev)
    _need(v, "v", (B, Nkv, Skv, D), q.dtype, dev)
    _need(lse, "lse", (B, N, Sq), torch.float32, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    ws = _workspace(blocksparse_attn_bwd_workspace_bytes(B, N, Sq, Skv, bx, by, D), dev, workspace) \
        if workspace is not None else _default_workspace(blocksparse_attn_bwd_ds_workspace_bytes(B, N, Sq, Skv, bx, by, D),
                                                         blocksparse_attn_bwd_workspace_bytes(B, N, Sq, Skv, bx, by, D), dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if Nkv == N:
        st = lib.blocksparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(block_mask),
                                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), B, N, Sq, Skv, D, bx, by,
                                      scale, _dtype_code(q), _stream(dev))
    else:
        st = lib.blocksparse_attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(block_mask),
                                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), B, N, Nkv, Sq, Skv, D,
                                          bx, by, scale, _dtype_code(q), _stream(dev))
    _check("blocksparse_attn_bwd", st)
    return dq, dk, dv
