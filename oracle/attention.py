"""fp64 reference for attention with a sink logit, a sliding causal window or a block mask.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the product.

What is computed, and where the pages define it
------------------------------------------------
Page "[Example] Add GQA Sink Backward BHSD ..." (tilelang-ascend PR 1), "Files Added" and
the commit message of the 4->2 kernel revision: a forward pass with online softmax, an
attention sink and a sliding-window mask producing O and lse; a backward pass made of a
Delta phase (Delta = sum(O * dO)), a loop of five GEMMs with softmax and dS, and a dSink
phase; outputs dQ, dK, dV and dSinks.  GQA in BHSD layout (title; the H20 table row
"h=64, groups=8").

Page "knowledge(triton) ... #174" (cannbot-knowledge PR 174), BlockSparseAttentionGrad
runbooks, sections "task features" and "precision recipe": BNSD MHA with D=128, inputs
dO, O and the softmax statistics, a uint8 block mask [B,N,ceil(Sq/bx),ceil(Skv/by)], a
token-level ``where(mask)`` golden; p = exp(s - lse), ds = p * (dp - delta); a row with no
selected block gets 0.

Readings taken where the pages are silent (each is also listed in the design notes):
  * window: query i sees key j iff 0 <= i - j < window (window >= S is plain causal);
  * s_ij = scale * q_i . k_j, natural-log domain; the sink logit is not scaled;
  * lse includes the sink: lse_i = log(exp(sink_h) + sum_{j visible} exp(s_ij));
  * one fp32 sink logit per query head; dsink is summed over batch and rows;
  * GQA groups are contiguous: kv head = h // (Hq // Hkv);
  * a nonzero mask byte means "keep"; bx runs along queries, by along keys; edge
    blocks are clipped at the sequence end;
  * a query row with no visible key has P = 0, O = 0, dQ = 0 and lse = -inf.

The backward is the exact definition, evaluated from the stored inputs (q, k, v, o, dO,
lse, sink) as given, in fp64:
    D_i      = dO_i . o_i
    P_ij     = exp(s_ij - lse_i) if (i, j) visible else 0
    dP_ij    = dO_i . v_j
    dS_ij    = P_ij * (dP_ij - D_i)
    dQ_i     = scale * sum_j dS_ij k_j
    dK_j     = scale * sum_{h in group} sum_i dS_ij q_i
    dV_j     = sum_{h in group} sum_i P_ij dO_i
    dsink_h  = - sum_b sum_i exp(sink_h - lse_i) * D_i
The dsink line follows from treating the sink as one more logit whose value row is zero:
its dP is 0, so its dS is p_sink * (0 - D_i).

Rows are processed in chunks and only the span of visible key columns is touched; both
are plain restrictions of the sums above (no reordering of any single sum's terms beyond
what numpy's matmul does).
"""

import numpy as np

_CHUNK = 512


def _f64(x):
    """Return x as a float64 numpy array (accepts numpy arrays and torch tensors)."""
    if hasattr(x, "detach"):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _u8(x):
    if hasattr(x, "detach"):
        return x.detach().to("cpu").numpy().astype(np.uint8)
    return np.asarray(x, dtype=np.uint8)


# ----------------------------------------------------------------------------- masks

def window_visibility(rows, cols, window):
    """Sliding-window causal visibility: query i sees key j iff 0 <= i - j < window."""
    rows = np.asarray(rows)[:, None]
    cols = np.asarray(cols)[None, :]
    d = rows - cols
    return (d >= 0) & (d < window)


def block_visibility(block_mask_bn, bx, by, rows, cols):
    """Token visibility from one (b, n) slice of the uint8 block mask: M[i // bx, j // by] != 0."""
    m = np.asarray(block_mask_bn)
    qb = np.asarray(rows) // bx
    kb = np.asarray(cols) // by
    return m[qb[:, None], kb[None, :]] != 0


def _visible_span(vis):
    cols = np.flatnonzero(vis.any(axis=0))
    if cols.size == 0:
        return 0, 0
    return int(cols[0]), int(cols[-1]) + 1


def softmax_probabilities(s, lse, vis):
    """P_ij = exp(s_ij - lse_i) on visible entries, exactly 0 elsewhere and on rows with lse = -inf."""
    lse = np.asarray(lse, dtype=np.float64)
    ok = vis & np.isfinite(lse)[:, None]
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(s - lse[:, None])
    return np.where(ok, e, 0.0)


def _sink_probability(sink, lse):
    """p_sink_i = exp(sink - lse_i); 0 when the sink is -inf or the row is empty."""
    lse = np.asarray(lse, dtype=np.float64)
    if not np.isfinite(sink):
        return np.zeros_like(lse)
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp(sink - lse)
    return np.where(np.isfinite(lse), p, 0.0)


# ----------------------------------------------------------------- per-head kernels

def _head_forward(q, k, v, sink, vis_fn, scale):
    sq, skv = q.shape[0], k.shape[0]
    o = np.zeros((sq, v.shape[1]))
    lse = np.full(sq, -np.inf)
    all_cols = np.arange(skv)
    for r0 in range(0, sq, _CHUNK):
        rows = np.arange(r0, min(r0 + _CHUNK, sq))
        vis = vis_fn(rows, all_cols)
        c0, c1 = _visible_span(vis)
        vis = vis[:, c0:c1]
        s = scale * (q[rows] @ k[c0:c1].T)
        s = np.where(vis, s, -np.inf)
        # lse_i = log(e^sink + sum_vis e^s_ij), evaluated with the usual max shift.
        m = np.maximum(s.max(axis=1, initial=-np.inf), sink)
        shift = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - shift[:, None])
        z = e.sum(axis=1) + np.exp(sink - shift)
        with np.errstate(divide="ignore"):
            lse[rows] = shift + np.log(z)
        zsafe = np.where(z > 0, z, 1.0)
        p = np.where(z[:, None] > 0, e / zsafe[:, None], 0.0)
        o[rows] = p @ v[c0:c1]
    return o, lse


def _head_backward_rows(q, k, v, o, do, lse, vis_fn, scale, rows):
    """dQ for the given query rows of one head (plus this head's dK/dV contributions)."""
    skv = k.shape[0]
    all_cols = np.arange(skv)
    delta = (do[rows] * o[rows]).sum(axis=1)
    vis = vis_fn(rows, all_cols)
    c0, c1 = _visible_span(vis)
    vis = vis[:, c0:c1]
    s = scale * (q[rows] @ k[c0:c1].T)
    p = softmax_probabilities(s, lse[rows], vis)
    dp = do[rows] @ v[c0:c1].T
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k[c0:c1])
    dk = scale * (ds.T @ q[rows])
    dv = p.T @ do[rows]
    return dq, dk, dv, (c0, c1), delta


def _head_backward(q, k, v, o, do, lse, vis_fn, scale):
    sq, skv, d = q.shape[0], k.shape[0], q.shape[1]
    dq = np.zeros((sq, d))
    dk = np.zeros((skv, d))
    dv = np.zeros((skv, d))
    delta = np.zeros(sq)
    for r0 in range(0, sq, _CHUNK):
        rows = np.arange(r0, min(r0 + _CHUNK, sq))
        dq_r, dk_r, dv_r, (c0, c1), delta_r = _head_backward_rows(q, k, v, o, do, lse, vis_fn, scale, rows)
        dq[rows] = dq_r
        dk[c0:c1] += dk_r
        dv[c0:c1] += dv_r
        delta[rows] = delta_r
    return dq, dk, dv, delta


def _head_backward_cols(q, k, v, o, do, lse, vis_fn, scale, cols):
    """dK/dV contributions of one query head to the given key rows (all query rows summed)."""
    sq = q.shape[0]
    all_rows = np.arange(sq)
    vis = vis_fn(all_rows, cols)
    live = np.flatnonzero(vis.any(axis=1))
    d = q.shape[1]
    if live.size == 0:
        return np.zeros((len(cols), d)), np.zeros((len(cols), d))
    r0, r1 = int(live[0]), int(live[-1]) + 1
    rows = all_rows[r0:r1]
    vis = vis[r0:r1]
    delta = (do[rows] * o[rows]).sum(axis=1)
    s = scale * (q[rows] @ k[cols].T)
    p = softmax_probabilities(s, lse[rows], vis)
    dp = do[rows] @ v[cols].T
    ds = p * (dp - delta[:, None])
    dk = scale * (ds.T @ q[rows])
    dv = p.T @ do[rows]
    return dk, dv


# ---------------------------------------------------------------- path A: sink + window

def _window_fn(window):
    return lambda rows, cols: window_visibility(rows, cols, window)


def sink_attention_forward(q, k, v, sink, window, scale):
    """O [B,Hq,S,D] and lse [B,Hq,S] (fp64) for GQA attention with a sink logit and a window."""
    q, k, v, sink = _f64(q), _f64(k), _f64(v), _f64(sink)
    b_, hq, s_, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    o = np.zeros((b_, hq, s_, d))
    lse = np.zeros((b_, hq, s_))
    fn = _window_fn(window)
    for b in range(b_):
        for h in range(hq):
            o[b, h], lse[b, h] = _head_forward(q[b, h], k[b, h // g], v[b, h // g], float(sink[h]), fn, scale)
    return o, lse


def sink_attention_backward(q, k, v, o, do, lse, sink, window, scale):
    """dq, dk, dv, dsink and delta from the stored forward quantities (exact fp64 definition)."""
    q, k, v, o, do, lse, sink = (_f64(x) for x in (q, k, v, o, do, lse, sink))
    b_, hq, s_, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.zeros((b_, hq, s_))
    dsink = np.zeros(hq)
    fn = _window_fn(window)
    for b in range(b_):
        for h in range(hq):
            kvh = h // g
            dq_h, dk_h, dv_h, delta_h = _head_backward(q[b, h], k[b, kvh], v[b, kvh], o[b, h], do[b, h],
                                                       lse[b, h], fn, scale)
            dq[b, h] = dq_h
            dk[b, kvh] += dk_h
            dv[b, kvh] += dv_h
            delta[b, h] = delta_h
            dsink[h] -= (_sink_probability(float(sink[h]), lse[b, h]) * delta_h).sum()
    return {"dq": dq, "dk": dk, "dv": dv, "dsink": dsink, "delta": delta}


# ------------------------------------------------- path A over packed variable-length sequences

def packed_window_visibility(cu_seqlens, rows, cols, window):
    """Packed sequences (page 1's "GQA Sink ... VarLen" rows; layout [H, total, D] is this
    oracle's reading): row i sees row j iff both lie in one sequence b, cu[b] <= i, j <
    cu[b+1], and 0 <= i - j < window (the window counts within the sequence)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    # Sequence index of a row; rows outside [cu[0], cu[B]) belong to no sequence (-1).
    seg_r = np.searchsorted(cu, rows, side="right") - 1
    seg_c = np.searchsorted(cu, cols, side="right") - 1
    nseq = len(cu) - 1
    seg_r = np.where((rows >= cu[0]) & (rows < cu[-1]), seg_r, -1)
    seg_c = np.where((cols >= cu[0]) & (cols < cu[-1]), seg_c, -2)
    return (seg_r[:, None] == seg_c[None, :]) & (seg_r[:, None] >= 0) & (seg_r[:, None] < nseq) & \
        window_visibility(rows, cols, window)


def sink_attention_forward_varlen(q, k, v, sink, cu_seqlens, window, scale):
    """O [Hq,total,D] and lse [Hq,total] (fp64) over packed sequences: the sink-and-window
    definition with visibility restricted to each sequence."""
    q, k, v, sink = _f64(q), _f64(k), _f64(v), _f64(sink)
    hq, total, d = q.shape
    g = hq // k.shape[0]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    fn = lambda rows, cols: packed_window_visibility(cu, rows, cols, window)
    o = np.zeros((hq, total, d))
    lse = np.zeros((hq, total))
    for h in range(hq):
        o[h], lse[h] = _head_forward(q[h], k[h // g], v[h // g], float(sink[h]), fn, scale)
    return o, lse


def sink_attention_backward_varlen(q, k, v, o, do, lse, sink, cu_seqlens, window, scale):
    """dq, dk, dv [heads, total, D], dsink [Hq] and delta [Hq, total] over packed sequences;
    dsink sums over every row of every sequence."""
    q, k, v, o, do, lse, sink = (_f64(x) for x in (q, k, v, o, do, lse, sink))
    hq, total, d = q.shape
    g = hq // k.shape[0]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    fn = lambda rows, cols: packed_window_visibility(cu, rows, cols, window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.zeros((hq, total))
    dsink = np.zeros(hq)
    for h in range(hq):
        kvh = h // g
        dq[h], dk_h, dv_h, delta[h] = _head_backward(q[h], k[kvh], v[kvh], o[h], do[h], lse[h], fn, scale)
        dk[kvh] += dk_h
        dv[kvh] += dv_h
        dsink[h] -= (_sink_probability(float(sink[h]), lse[h]) * delta[h]).sum()
    return {"dq": dq, "dk": dk, "dv": dv, "dsink": dsink, "delta": delta}


def sink_attention_backward_sampled(q, k, v, o, do, lse, sink, window, scale, q_rows, kv_rows):
    """The same definition evaluated only at chosen outputs.

    q_rows:  iterable of (b, h, i)   -> dq[b, h, i, :]
    kv_rows: iterable of (b, kvh, j) -> dk[b, kvh, j, :], dv[b, kvh, j, :]
    dsink and delta are returned in full (they need only rowwise work).
    """
    q, k, v, o, do, lse, sink = (_f64(x) for x in (q, k, v, o, do, lse, sink))
    b_, hq, s_, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    fn = _window_fn(window)
    dq = np.zeros((len(q_rows), d))
    for n, (b, h, i) in enumerate(q_rows):
        dq_r, _, _, _, _ = _head_backward_rows(q[b, h], k[b, h // g], v[b, h // g], o[b, h], do[b, h],
                                               lse[b, h], fn, scale, np.array([i]))
        dq[n] = dq_r[0]
    dk = np.zeros((len(kv_rows), d))
    dv = np.zeros((len(kv_rows), d))
    for n, (b, kvh, j) in enumerate(kv_rows):
        for h in range(kvh * g, (kvh + 1) * g):
            dk_r, dv_r = _head_backward_cols(q[b, h], k[b, kvh], v[b, kvh], o[b, h], do[b, h], lse[b, h],
                                             fn, scale, np.array([j]))
            dk[n] += dk_r[0]
            dv[n] += dv_r[0]
    delta = (do * o).sum(axis=-1)
    dsink = np.zeros(hq)
    for h in range(hq):
        for b in range(b_):
            dsink[h] -= (_sink_probability(float(sink[h]), lse[b, h]) * delta[b, h]).sum()
    return {"dq": dq, "dk": dk, "dv": dv, "dsink": dsink, "delta": delta}


# ------------------------------------------------------------ path B: block-sparse attention
# MHA as on the block-sparse page; with fewer K/V heads than query heads (GQA, Hq % Hkv == 0)
# the grouping of path A applies: query head n reads K/V head n // (Hq // Hkv), the block mask
# is per query head, and dK/dV of a K/V head sum over its group.

def _block_fn(mask_bn, bx, by):
    return lambda rows, cols: block_visibility(mask_bn, bx, by, rows, cols)


def blocksparse_attention_forward(q, k, v, block_mask, bx, by, scale):
    """O [B,N,Sq,D] and lse [B,N,Sq] for block-sparse attention (no sink; empty rows: O=0,
    lse=-inf).  k, v: [B,Nkv,Skv,D] with N % Nkv == 0."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    m = _u8(block_mask)
    b_, n_, sq, d = q.shape
    g = n_ // k.shape[1]
    o = np.zeros((b_, n_, sq, d))
    lse = np.zeros((b_, n_, sq))
    for b in range(b_):
        for n in range(n_):
            o[b, n], lse[b, n] = _head_forward(q[b, n], k[b, n // g], v[b, n // g], -np.inf,
                                               _block_fn(m[b, n], bx, by), scale)
    return o, lse


def blocksparse_attention_backward(q, k, v, o, do, lse, block_mask, bx, by, scale):
    """dq, dk, dv, delta for block-sparse attention from the stored forward quantities."""
    q, k, v, o, do, lse = (_f64(x) for x in (q, k, v, o, do, lse))
    m = _u8(block_mask)
    b_, n_, sq, d = q.shape
    g = n_ // k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.zeros((b_, n_, sq))
    for b in range(b_):
        for n in range(n_):
            dq[b, n], dk_h, dv_h, delta[b, n] = _head_backward(
                q[b, n], k[b, n // g], v[b, n // g], o[b, n], do[b, n], lse[b, n], _block_fn(m[b, n], bx, by), scale)
            dk[b, n // g] += dk_h
            dv[b, n // g] += dv_h
    return {"dq": dq, "dk": dk, "dv": dv, "delta": delta}


def blocksparse_attention_backward_sampled(q, k, v, o, do, lse, block_mask, bx, by, scale, q_rows, kv_rows):
    """Block-sparse backward at chosen outputs: q_rows of (b, n, i) -> dq[b, n, i, :], kv_rows of
    (b, nkv, j) -> dk[b, nkv, j, :], dv[b, nkv, j, :]."""
    q, k, v, o, do, lse = (_f64(x) for x in (q, k, v, o, do, lse))
    m = _u8(block_mask)
    d = q.shape[-1]
    g = q.shape[1] // k.shape[1]
    dq = np.zeros((len(q_rows), d))
    for t, (b, n, i) in enumerate(q_rows):
        dq_r, _, _, _, _ = _head_backward_rows(q[b, n], k[b, n // g], v[b, n // g], o[b, n], do[b, n], lse[b, n],
                                               _block_fn(m[b, n], bx, by), scale, np.array([i]))
        dq[t] = dq_r[0]
    dk = np.zeros((len(kv_rows), d))
    dv = np.zeros((len(kv_rows), d))
    for t, (b, nkv, j) in enumerate(kv_rows):
        for n in range(nkv * g, (nkv + 1) * g):
            dk_r, dv_r = _head_backward_cols(q[b, n], k[b, nkv], v[b, nkv], o[b, n], do[b, n], lse[b, n],
                                             _block_fn(m[b, n], bx, by), scale, np.array([j]))
            dk[t] += dk_r[0]
            dv[t] += dv_r[0]
    return {"dq": dq, "dk": dk, "dv": dv}
