"""Workload registry and seeded synthetic input generators.

This module holds no attention arithmetic: it only draws the random inputs (Q, K, V, dO,
sink logits, block masks) that both the GPU path and the CPU oracle consume, so neither
side depends on the other for its inputs.  O and lse are never produced here.

Workloads (shapes follow the synthetic configurations the pages' measurements are
quoted on; every tensor is ~N(0,1) drawn in float32 and rounded to nearest-even):

  tiny          GQA sink, B1 Hq4 Hkv1 S128 D128, window 64, fp16
  mid           GQA sink, B2 Hq32 Hkv8 S2048 D128, window 128, fp16
  large_w128    GQA sink, B1 Hq64 Hkv8 S8192 D128, window 128, bf16
  large_causal  GQA sink, B1 Hq64 Hkv8 S8192 D128, window = S (full causal), bf16
  pages_h64_s4096  GQA sink, B1 Hq64 Hkv8 S4096 D128, window = S, fp16 (the sink page's
                table shape)
  bigbird       block-sparse MHA, B1 N16 S8192 D128, bx=by=64, bigbird pattern, fp16
  ragged        block-sparse MHA, B2 N8 Sq=Skv=3000 D128, bx=48 by=80, Bernoulli(0.3)
                with the diagonal forced on, fp16

Packed variable-length sequences (``varlen_inputs``): q, dO [Hq, total, D], k, v
[Hkv, total, D], sink [Hq] and cu_seqlens [B + 1] int32.  The pages' varlen row gives batch
8, 64 heads, groups 16 (read as 16 query heads per K/V head: Hkv = 4) and 2048 tokens.
Two batches (``VARLEN``): ``varlen_8x2048``, eight sequences of exactly 2048 tokens (the
plain reading), and ``varlen_mixed``, lengths drawn uniformly from [1024, 2048] (t = 6)
with the first set to 2048.

Seeds: numpy ``default_rng(1000 * seed_base + t)`` with t = 0 for q, 1 k, 2 v, 3 dO,
4 sink, 5 mask, 6 sequence lengths.  The bigbird reading: for query block i keep {i}, the global columns
{0, 1} that lie at or before i, and 3 distinct columns drawn uniformly from [2, i-1]
(all of them when fewer exist).  The ragged reading: Bernoulli(0.3) per block, then every
key block whose token range overlaps the query block's token range is forced on, so no
query row is empty.
"""

from dataclasses import dataclass, replace
import math

import numpy as np
import torch

SINK = "sink"
BLOCKSPARSE = "blocksparse"


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str              # SINK or BLOCKSPARSE
    B: int
    Hq: int                # query heads (N for block-sparse)
    Hkv: int               # key/value heads (== Hq for block-sparse)
    Sq: int
    Skv: int
    D: int
    dtype: torch.dtype
    window: int = 0        # sink path; block path: band width (tokens) of the "window" pattern
    bx: int = 0            # block-sparse only
    by: int = 0
    pattern: str = ""      # "bigbird" | "ragged" | "random" | "dense" | "causal" | "window"
    density: float = 0.3
    seed_base: int = 0

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    @property
    def nqb(self):
        return -(-self.Sq // self.bx) if self.bx else 0

    @property
    def nkb(self):
        return -(-self.Skv // self.by) if self.by else 0

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", SINK, 1, 4, 1, 128, 128, 128, torch.float16, window=64, seed_base=1),
    "mid": Workload("mid", SINK, 2, 32, 8, 2048, 2048, 128, torch.float16, window=128, seed_base=2),
    "large_w128": Workload("large_w128", SINK, 1, 64, 8, 8192, 8192, 128, torch.bfloat16, window=128,
                           seed_base=3),
    "large_causal": Workload("large_causal", SINK, 1, 64, 8, 8192, 8192, 128, torch.bfloat16, window=8192,
                             seed_base=3),
    # The sink page's kernel-table shape (batch 1, 64 heads, groups of 8, 4096 tokens, d 128,
    # fp16); the window is read as the whole sequence.
    "pages_h64_s4096": Workload("pages_h64_s4096", SINK, 1, 64, 8, 4096, 4096, 128, torch.float16, window=4096,
                                seed_base=120),
    "bigbird": Workload("bigbird", BLOCKSPARSE, 1, 16, 16, 8192, 8192, 128, torch.float16, bx=64, by=64,
                        pattern="bigbird", seed_base=4),
    "ragged": Workload("ragged", BLOCKSPARSE, 2, 8, 8, 3000, 3000, 128, torch.float16, bx=48, by=80,
                       pattern="ragged", density=0.3, seed_base=5),
}


def _normal(seed, shape, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(dtype)


def bigbird_mask(rng, nqb, nkb):
    """Causal bigbird block pattern for one (b, n): diagonal + 2 global + 3 random columns per row."""
    m = np.zeros((nqb, nkb), dtype=np.uint8)
    for i in range(nqb):
        if i < nkb:
            m[i, i] = 1
        for g in (0, 1):
            if g <= i and g < nkb:
                m[i, g] = 1
        pool = np.arange(2, min(i, nkb))
        if pool.size <= 3:
            m[i, pool] = 1
        else:
            m[i, rng.choice(pool, size=3, replace=False)] = 1
    return m


def ragged_mask(rng, nqb, nkb, bx, by, sq, skv, density):
    """Bernoulli(density) blocks plus every key block overlapping the query block's token range."""
    m = (rng.random((nqb, nkb)) < density).astype(np.uint8)
    for i in range(nqb):
        q0, q1 = i * bx, min((i + 1) * bx, sq)
        for j in range(nkb):
            k0, k1 = j * by, min((j + 1) * by, skv)
            if max(q0, k0) < min(q1, k1):
                m[i, j] = 1
    return m


def make_block_mask(wl, seed=None):
    seed = (1000 * wl.seed_base + 5) if seed is None else seed
    rng = np.random.default_rng(seed)
    out = np.zeros((wl.B, wl.Hq, wl.nqb, wl.nkb), dtype=np.uint8)
    for b in range(wl.B):
        for n in range(wl.Hq):
            if wl.pattern == "bigbird":
                out[b, n] = bigbird_mask(rng, wl.nqb, wl.nkb)
            elif wl.pattern == "ragged":
                out[b, n] = ragged_mask(rng, wl.nqb, wl.nkb, wl.bx, wl.by, wl.Sq, wl.Skv, wl.density)
            elif wl.pattern == "random":
                out[b, n] = (rng.random((wl.nqb, wl.nkb)) < wl.density).astype(np.uint8)
            elif wl.pattern == "dense":
                out[b, n] = 1
            elif wl.pattern == "causal":
                qi = np.arange(wl.nqb)[:, None] * wl.bx
                kj = np.arange(wl.nkb)[None, :] * wl.by
                out[b, n] = (kj <= qi + wl.bx - 1).astype(np.uint8)
            elif wl.pattern == "window":
                # Blocks that meet the causal band 0 <= i - j < window of some row of the block.
                q0 = np.arange(wl.nqb)[:, None] * wl.bx
                q1 = np.minimum(q0 + wl.bx, wl.Sq) - 1
                k0 = np.arange(wl.nkb)[None, :] * wl.by
                k1 = np.minimum(k0 + wl.by, wl.Skv) - 1
                out[b, n] = ((k0 <= q1) & (k1 >= q0 - wl.window + 1)).astype(np.uint8)
            else:
                raise ValueError(f"unknown mask pattern {wl.pattern!r}")
    return torch.from_numpy(out)


def make_inputs(wl):
    """CPU tensors: q, k, v, do in wl.dtype; sink fp32 [Hq] (sink path); block_mask uint8 (block path)."""
    s = 1000 * wl.seed_base
    out = {
        "q": _normal(s + 0, (wl.B, wl.Hq, wl.Sq, wl.D), wl.dtype),
        "k": _normal(s + 1, (wl.B, wl.Hkv, wl.Skv, wl.D), wl.dtype),
        "v": _normal(s + 2, (wl.B, wl.Hkv, wl.Skv, wl.D), wl.dtype),
        "do": _normal(s + 3, (wl.B, wl.Hq, wl.Sq, wl.D), wl.dtype),
    }
    if wl.kind == SINK:
        out["sink"] = _normal(s + 4, (wl.Hq,), torch.float32)
    else:
        out["block_mask"] = make_block_mask(wl)
    return out


def custom_sink(name, B, Hq, Hkv, S, window, dtype=torch.float16, D=128, seed_base=100):
    return Workload(name, SINK, B, Hq, Hkv, S, S, D, dtype, window=window, seed_base=seed_base)


def custom_blocksparse(name, B, N, Sq, Skv, bx, by, pattern, dtype=torch.float16, D=128, density=0.3,
                       seed_base=200, Nkv=None, window=0):
    """Block-sparse workload with N query heads (the mask is per query head) and Nkv K/V heads
    (default N: MHA); `window` is the band width of the "window" pattern."""
    return Workload(name, BLOCKSPARSE, B, N, N if Nkv is None else Nkv, Sq, Skv, D, dtype, bx=bx, by=by,
                    pattern=pattern, density=density, seed_base=seed_base, window=window)


def varlen_lengths(B, max_len, seed_base=300):
    """B sequence lengths, uniform on [max(1, max_len // 2), max_len], the first one max_len."""
    rng = np.random.default_rng(1000 * seed_base + 6)
    n = rng.integers(max(1, max_len // 2), max_len + 1, size=B)
    n[0] = max_len
    return [int(x) for x in n]


def varlen_inputs(lengths, Hq, Hkv, dtype=torch.float16, D=128, seed_base=300):
    """CPU tensors of a packed batch with the given sequence lengths (zeros allowed):
    q, do [Hq, total, D], k, v [Hkv, total, D] in dtype, sink [Hq] fp32, cu_seqlens [B + 1]
    int32 and max_seqlen (int)."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    total = int(cu[-1])
    s = 1000 * seed_base
    return {
        "q": _normal(s + 0, (Hq, total, D), dtype),
        "k": _normal(s + 1, (Hkv, total, D), dtype),
        "v": _normal(s + 2, (Hkv, total, D), dtype),
        "do": _normal(s + 3, (Hq, total, D), dtype),
        "sink": _normal(s + 4, (Hq,), torch.float32),
        "cu_seqlens": torch.from_numpy(cu.astype(np.int32)),
        "max_seqlen": max(1, max(lengths)),
    }


@dataclass(frozen=True)
class VarlenWorkload:
    name: str
    lengths: tuple
    Hq: int
    Hkv: int
    window: int
    dtype: torch.dtype
    seed_base: int
    D: int = 128

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    def inputs(self):
        return varlen_inputs(list(self.lengths), self.Hq, self.Hkv, self.dtype, D=self.D, seed_base=self.seed_base)


VARLEN = {
    "varlen_8x2048": VarlenWorkload("varlen_8x2048", (2048,) * 8, 64, 4, 2048, torch.float16, 320),
    "varlen_mixed": VarlenWorkload("varlen_mixed", tuple(varlen_lengths(8, 2048)), 64, 4, 2048, torch.float16, 300),
}
