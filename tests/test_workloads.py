"""Input generators: mask patterns and packed-sequence lengths (CPU only)."""

import numpy as np
import torch

from masked_attention_backward_amd import workloads as W


def test_window_block_pattern_matches_token_band():
    """The "window" block pattern keeps exactly the blocks that hold a (q, k) with
    0 <= q - k < window, edge blocks clipped to Sq and Skv."""
    for Sq, Skv, bx, by, win in ((450, 450, 64, 64, 200), (333, 300, 32, 16, 100), (97, 130, 48, 80, 1)):
        wl = W.custom_blocksparse("t", 1, 1, Sq, Skv, bx, by, "window", window=win)
        m = W.make_block_mask(wl)[0, 0].numpy()
        i, j = np.arange(Sq)[:, None], np.arange(Skv)[None, :]
        band = (i - j >= 0) & (i - j < win)
        want = np.array([[band[a * bx:(a + 1) * bx, b * by:(b + 1) * by].any() for b in range(wl.nkb)]
                         for a in range(wl.nqb)])
        assert np.array_equal(m != 0, want), (Sq, Skv, bx, by, win)


def test_varlen_inputs_layout():
    lengths = W.varlen_lengths(8, 2048)
    assert lengths[0] == 2048 and all(1024 <= n <= 2048 for n in lengths)
    x = W.varlen_inputs([5, 0, 3], 4, 2, torch.bfloat16)
    assert x["q"].shape == (4, 8, 128) and x["k"].shape == (2, 8, 128)
    assert x["cu_seqlens"].tolist() == [0, 5, 5, 8] and x["cu_seqlens"].dtype == torch.int32
    assert x["max_seqlen"] == 5
