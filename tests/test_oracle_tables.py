"""Pins for the oracle's block tables: hand-worked fixture, brute force, CSR-transpose identity."""

import json
import os

import numpy as np
import torch

import oracle
from masked_attention_backward_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_fixture():
    with open(os.path.join(GOLDEN, "block_tables_3x4.json")) as f:
        fx = json.load(f)
    m = np.array(fx["mask"], dtype=np.uint8)[None, None]
    t = oracle.build_block_tables(m)
    assert t["mask_t"][0, 0].tolist() == fx["mask_t"]
    assert t["sel_q"][0, 0].tolist() == fx["sel_q"]
    assert t["cnt_q"][0, 0].tolist() == fx["cnt_q"]
    assert t["sel_k"][0, 0].tolist() == fx["sel_k"]
    assert t["cnt_k"][0, 0].tolist() == fx["cnt_k"]


def _brute(m):
    """Pure-Python loops, no numpy helpers beyond indexing."""
    r, c = len(m), len(m[0])
    sel_q = [[-1] * c for _ in range(r)]
    cnt_q = [0] * r
    for i in range(r):
        for j in range(c):
            if m[i][j]:
                sel_q[i][cnt_q[i]] = j
                cnt_q[i] += 1
    sel_k = [[-1] * r for _ in range(c)]
    cnt_k = [0] * c
    for j in range(c):
        for i in range(r):
            if m[i][j]:
                sel_k[j][cnt_k[j]] = i
                cnt_k[j] += 1
    return sel_q, cnt_q, sel_k, cnt_k


def test_brute_force_random_masks():
    rng = np.random.default_rng(0)
    for shape in [(1, 1, 1, 1), (2, 3, 5, 7), (1, 2, 13, 4), (1, 1, 65, 66)]:
        m = (rng.random(shape) < 0.4).astype(np.uint8) * rng.integers(1, 255, size=shape).astype(np.uint8)
        t = oracle.build_block_tables(m)
        for b in range(shape[0]):
            for n in range(shape[1]):
                sq, cq, sk, ck = _brute(m[b, n].tolist())
                assert t["sel_q"][b, n].tolist() == sq
                assert t["cnt_q"][b, n].tolist() == cq
                assert t["sel_k"][b, n].tolist() == sk
                assert t["cnt_k"][b, n].tolist() == ck
        assert np.array_equal(t["mask_t"], torch.from_numpy(m).permute(0, 1, 3, 2).numpy())
        pc = oracle.block_mask_popcount(m)
        assert np.array_equal(t["cnt_q"].sum(-1), pc)
        assert np.array_equal(t["cnt_k"].sum(-1), pc)


def test_csr_transpose_identity_on_workload_masks():
    for name in ("ragged",):
        wl = workloads.WORKLOADS[name]
        m = workloads.make_block_mask(wl).numpy()
        t = oracle.build_block_tables(m)
        b, n = 1, 5
        pairs_q = {(i, int(j)) for i in range(wl.nqb) for j in t["sel_q"][b, n, i, :t["cnt_q"][b, n, i]]}
        pairs_k = {(int(i), j) for j in range(wl.nkb) for i in t["sel_k"][b, n, j, :t["cnt_k"][b, n, j]]}
        assert pairs_q == pairs_k
        assert all(np.all(np.diff(t["sel_q"][b, n, i, :t["cnt_q"][b, n, i]]) > 0) for i in range(wl.nqb))


def test_workload_mask_readings():
    bb = workloads.WORKLOADS["bigbird"]
    m = workloads.make_block_mask(bb).numpy()
    # causal bigbird: 1 + 2 + 3 + 4 + 5 + 6 * 123 = 753 kept blocks per (b, n)
    assert np.all(oracle.block_mask_popcount(m) == 753)
    assert np.all(np.triu(m[0, 0], 1) == 0)
    rg = workloads.WORKLOADS["ragged"]
    m = workloads.make_block_mask(rg).numpy()
    # every query row of the ragged mask sees at least its own position
    for i in range(rg.Sq):
        assert m[0, 0, i // rg.bx, i // rg.by]
