"""Plain definition of the block-mask transpose and the two selection tables.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the product.

Page "knowledge(triton) ... #174" (cannbot-knowledge PR 174), BlockSparseAttentionGrad
runbooks, "optimisation 1" / "optimisation 2" and the old handbook's "skeleton" and "pit 1":
the mask is transposed on the device (result bit-equal to ``mask.permute(0,1,3,2)``); a
q-major table lists, per query block row, the kept key-block columns and a kv-major table
lists, per key block, the kept query-block rows, each compacted by an exclusive prefix
count of the kept entries, so the columns appear in ascending order, followed by a count
that drives the kernel's loop.

Readings: the tables are indexed by mask block (not by a kernel tile); entries past the
count are -1; every array is int32 except the transposed mask (uint8).
"""

import numpy as np


def _u8(x):
    if hasattr(x, "detach"):
        return x.detach().to("cpu").numpy().astype(np.uint8)
    return np.asarray(x, dtype=np.uint8)


def _compact_rows(m):
    """For each row of m (..., R, C): ascending column ids with m != 0, then -1; and the count."""
    *lead, r, c = m.shape
    sel = np.full(m.shape, -1, dtype=np.int32)
    cnt = np.zeros((*lead, r), dtype=np.int32)
    flat = m.reshape(-1, r, c)
    sel_f = sel.reshape(-1, r, c)
    cnt_f = cnt.reshape(-1, r)
    for t in range(flat.shape[0]):
        for i in range(r):
            cols = np.flatnonzero(flat[t, i])
            sel_f[t, i, :cols.size] = cols
            cnt_f[t, i] = cols.size
    return sel, cnt


def build_block_tables(block_mask):
    """Return dict(mask_t, sel_q, cnt_q, sel_k, cnt_k) for a uint8 mask [B, N, nqb, nkb]."""
    m = _u8(block_mask)
    mask_t = np.ascontiguousarray(m.transpose(0, 1, 3, 2))
    sel_q, cnt_q = _compact_rows(m)
    sel_k, cnt_k = _compact_rows(mask_t)
    return {"mask_t": mask_t, "sel_q": sel_q, "cnt_q": cnt_q, "sel_k": sel_k, "cnt_k": cnt_k}


def block_mask_popcount(block_mask):
    """Number of kept blocks per (b, n)."""
    m = _u8(block_mask)
    return (m != 0).sum(axis=(-1, -2))
