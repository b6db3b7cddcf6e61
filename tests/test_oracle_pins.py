"""Pins for the fp64 oracle: each check comes from something other than the oracle itself.

* central finite differences of L = sum(dO * O) through the oracle's own forward;
* torch fp64 autograd through ``scaled_dot_product_attention`` (sink = -inf reductions:
  causal, windowed, dense, GQA via repeated K/V, token-expanded block mask);
* an augmented-key softmax in torch autograd (the sink as an extra logit with a zero
  value row) for lse and dsink;
* a closed form for one query and one key (a sigmoid);
* invariants of the softmax (row sums, shift invariance, sink-free column sums).
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loss_grads_fd(f, x, h_rel=1e-6):
    """Central differences of scalar f at every element of the array x (modified in place, restored)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        h = h_rel * max(1.0, abs(old))
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(1e-30, np.max(np.abs(b)))


# ------------------------------------------------------------------ finite differences

@pytest.mark.parametrize("window", [4, 9])
def test_fd_sink_window(window):
    rng = np.random.default_rng(7 + window)
    B, Hq, Hkv, S, D = 1, 2, 1, 9, 8
    scale = 1 / math.sqrt(D)
    q, k, v, do = _rand(rng, B, Hq, S, D), _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D), _rand(rng, B, Hq, S, D)
    sink = _rand(rng, Hq)

    def loss():
        o, _ = oracle.sink_attention_forward(q, k, v, sink, window, scale)
        return float((do * o).sum())

    o, lse = oracle.sink_attention_forward(q, k, v, sink, window, scale)
    g = oracle.sink_attention_backward(q, k, v, o, do, lse, sink, window, scale)
    for name, arr in (("dq", q), ("dk", k), ("dv", v), ("dsink", sink)):
        fd = _loss_grads_fd(loss, arr)
        assert _rel(g[name], fd) < 1e-7, name


def test_fd_blocksparse_with_empty_row():
    rng = np.random.default_rng(11)
    B, N, Sq, Skv, D, bx, by = 1, 2, 10, 11, 8, 3, 4
    scale = 1 / math.sqrt(D)
    nqb, nkb = -(-Sq // bx), -(-Skv // by)
    mask = (rng.random((B, N, nqb, nkb)) < 0.5).astype(np.uint8)
    mask[0, 0, 1, :] = 0          # query block 1 of head 0 sees nothing
    mask[0, 1, 0, 0] = 1
    q, k, v, do = _rand(rng, B, N, Sq, D), _rand(rng, B, N, Skv, D), _rand(rng, B, N, Skv, D), _rand(rng, B, N, Sq, D)

    def loss():
        o, _ = oracle.blocksparse_attention_forward(q, k, v, mask, bx, by, scale)
        return float((do * o).sum())

    o, lse = oracle.blocksparse_attention_forward(q, k, v, mask, bx, by, scale)
    assert np.all(np.isneginf(lse[0, 0, 3:6])) and np.all(o[0, 0, 3:6] == 0)
    g = oracle.blocksparse_attention_backward(q, k, v, o, do, lse, mask, bx, by, scale)
    assert np.all(g["dq"][0, 0, 3:6] == 0)
    for name, arr in (("dq", q), ("dk", k), ("dv", v)):
        fd = _loss_grads_fd(loss, arr)
        assert _rel(g[name], fd) < 1e-7, name


# ---------------------------------------------------------- torch SDPA reductions (sink = -inf)

def _sdpa_grads(q, k, v, do, scale, attn_mask=None, is_causal=False):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=attn_mask, is_causal=is_causal,
                                                         scale=scale)
    (o * torch.tensor(do)).sum().backward()
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def _oracle_sink(q, k, v, do, sink, window, scale):
    o, lse = oracle.sink_attention_forward(q, k, v, sink, window, scale)
    g = oracle.sink_attention_backward(q, k, v, o, do, lse, sink, window, scale)
    return o, lse, g


@pytest.mark.parametrize("S,window", [(37, 37), (37, 200), (40, 7)])
def test_sdpa_causal_and_window_reduction(S, window):
    rng = np.random.default_rng(S + window)
    B, H, D = 2, 3, 16
    scale = 0.3
    q, k, v, do = (_rand(rng, B, H, S, D) for _ in range(4))
    sink = np.full(H, -np.inf)
    o, lse, g = _oracle_sink(q, k, v, do, sink, window, scale)
    if window >= S:
        ref = _sdpa_grads(q, k, v, do, scale, is_causal=True)
    else:
        i = torch.arange(S)[:, None]
        j = torch.arange(S)[None, :]
        m = (j <= i) & (j > i - window)
        ref = _sdpa_grads(q, k, v, do, scale, attn_mask=m)
    for a, b in zip((o, g["dq"], g["dk"], g["dv"]), ref):
        assert np.max(np.abs(a - b)) < 1e-12 * max(1.0, np.max(np.abs(b)))
    assert np.all(g["dsink"] == 0)


def test_sdpa_gqa_reduction():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, S, D = 1, 6, 2, 33, 16
    scale = 1 / 4
    q, do = _rand(rng, B, Hq, S, D), _rand(rng, B, Hq, S, D)
    k, v = _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    sink = np.full(Hq, -np.inf)
    o, lse, g = _oracle_sink(q, k, v, do, sink, 12, scale)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    m = (j <= i) & (j > i - 12)
    ro, rdq, rdk, rdv = _sdpa_grads(q, kr, vr, do, scale, attn_mask=m)
    rdk = rdk.reshape(B, Hkv, Hq // Hkv, S, D).sum(axis=2)
    rdv = rdv.reshape(B, Hkv, Hq // Hkv, S, D).sum(axis=2)
    for a, b in zip((o, g["dq"], g["dk"], g["dv"]), (ro, rdq, rdk, rdv)):
        assert np.max(np.abs(a - b)) < 1e-12 * max(1.0, np.max(np.abs(b)))


@pytest.mark.parametrize("pattern", ["dense", "random"])
def test_sdpa_blocksparse_reduction(pattern):
    rng = np.random.default_rng(3)
    B, N, Sq, Skv, D, bx, by = 2, 2, 45, 50, 16, 16, 16
    scale = 0.2
    nqb, nkb = -(-Sq // bx), -(-Skv // by)
    if pattern == "dense":
        mask = np.ones((B, N, nqb, nkb), dtype=np.uint8)
    else:
        mask = (rng.random((B, N, nqb, nkb)) < 0.5).astype(np.uint8)
        mask[..., 0] = 1   # no empty rows (SDPA would give NaN there)
    q, do = _rand(rng, B, N, Sq, D), _rand(rng, B, N, Sq, D)
    k, v = _rand(rng, B, N, Skv, D), _rand(rng, B, N, Skv, D)
    o, lse = oracle.blocksparse_attention_forward(q, k, v, mask, bx, by, scale)
    g = oracle.blocksparse_attention_backward(q, k, v, o, do, lse, mask, bx, by, scale)
    tm = torch.tensor(mask, dtype=torch.bool)
    tok = tm.repeat_interleave(bx, dim=2)[:, :, :Sq].repeat_interleave(by, dim=3)[:, :, :, :Skv]
    ref = _sdpa_grads(q, k, v, do, scale, attn_mask=None if pattern == "dense" else tok)
    for a, b in zip((o, g["dq"], g["dk"], g["dv"]), ref):
        assert np.max(np.abs(a - b)) < 1e-12 * max(1.0, np.max(np.abs(b)))


def test_sdpa_blocksparse_gqa_reduction():
    """GQA block-sparse (per-query-head block mask, K/V shared by groups of query heads) equals
    SDPA on repeated K/V with the token-expanded mask, dK/dV summed over each group."""
    rng = np.random.default_rng(11)
    B, Hq, Hkv, Sq, Skv, D, bx, by = 2, 6, 2, 40, 37, 16, 16, 8
    g_ = Hq // Hkv
    scale = 0.25
    nqb, nkb = -(-Sq // bx), -(-Skv // by)
    mask = (rng.random((B, Hq, nqb, nkb)) < 0.5).astype(np.uint8)
    mask[..., 1] = 1   # no empty rows (SDPA would give NaN there)
    q, do = _rand(rng, B, Hq, Sq, D), _rand(rng, B, Hq, Sq, D)
    k, v = _rand(rng, B, Hkv, Skv, D), _rand(rng, B, Hkv, Skv, D)
    o, lse = oracle.blocksparse_attention_forward(q, k, v, mask, bx, by, scale)
    g = oracle.blocksparse_attention_backward(q, k, v, o, do, lse, mask, bx, by, scale)
    tm = torch.tensor(mask, dtype=torch.bool)
    tok = tm.repeat_interleave(bx, dim=2)[:, :, :Sq].repeat_interleave(by, dim=3)[:, :, :, :Skv]
    kr, vr = np.repeat(k, g_, axis=1), np.repeat(v, g_, axis=1)
    ro, rdq, rdk, rdv = _sdpa_grads(q, kr, vr, do, scale, attn_mask=tok)
    rdk = rdk.reshape(B, Hkv, g_, Skv, D).sum(axis=2)
    rdv = rdv.reshape(B, Hkv, g_, Skv, D).sum(axis=2)
    for a, b in zip((o, g["dq"], g["dk"], g["dv"]), (ro, rdq, rdk, rdv)):
        assert np.max(np.abs(a - b)) < 1e-12 * max(1.0, np.max(np.abs(b)))
    # the sampled form returns the same rows
    qs = [(1, 4, 0), (0, 5, 39), (1, 0, 17)]
    ks = [(0, 1, 0), (1, 0, 36), (1, 1, 20)]
    sm = oracle.blocksparse_attention_backward_sampled(q, k, v, o, do, lse, mask, bx, by, scale, qs, ks)
    for t, (b, n, i) in enumerate(qs):
        assert np.max(np.abs(sm["dq"][t] - g["dq"][b, n, i])) < 1e-12
    for t, (b, n, j) in enumerate(ks):
        assert np.max(np.abs(sm["dk"][t] - g["dk"][b, n, j])) < 1e-12
        assert np.max(np.abs(sm["dv"][t] - g["dv"][b, n, j])) < 1e-12


# ------------------------------------------------------------ augmented-key sink formulation

def test_augmented_key_sink_lse_and_dsink():
    rng = np.random.default_rng(17)
    B, Hq, Hkv, S, D, W = 2, 4, 2, 21, 8, 6
    scale = 0.37
    q, do = _rand(rng, B, Hq, S, D), _rand(rng, B, Hq, S, D)
    k, v = _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    sink = _rand(rng, Hq)
    o, lse, g = _oracle_sink(q, k, v, do, sink, W, scale)

    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ts = torch.tensor(sink, requires_grad=True)
    g_ = Hq // Hkv
    kr = tk.repeat_interleave(g_, dim=1)
    vr = tv.repeat_interleave(g_, dim=1)
    logits = scale * tq @ kr.transpose(-1, -2)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    vis = (j <= i) & (j > i - W)
    logits = logits.masked_fill(~vis, float("-inf"))
    sink_col = ts[None, :, None, None].expand(B, Hq, S, 1)
    aug = torch.cat([sink_col, logits], dim=-1)
    lse_ref = torch.logsumexp(aug, dim=-1)
    p = torch.softmax(aug, dim=-1)[..., 1:]          # the sink's value row is zero
    out = p @ vr
    (out * torch.tensor(do)).sum().backward()
    assert np.max(np.abs(lse - lse_ref.detach().numpy())) < 1e-12
    assert np.max(np.abs(o - out.detach().numpy())) < 1e-12
    for name, ref in (("dq", tq.grad), ("dk", tk.grad), ("dv", tv.grad), ("dsink", ts.grad)):
        ref = ref.numpy()
        assert np.max(np.abs(g[name] - ref)) < 1e-11 * max(1.0, np.max(np.abs(ref))), name


# ------------------------------------------------------------------------- closed form

def test_single_query_single_key_closed_form():
    """S = 1: P = sigmoid(s - sink), dsink = -P(1-P)(dO.v), dq = scale*P(1-P)(dO.v) k."""
    rng = np.random.default_rng(23)
    D = 8
    scale = 0.5
    q, k, v, do = (_rand(rng, 1, 1, 1, D) for _ in range(4))
    sink = np.array([0.7])
    o, lse, g = _oracle_sink(q, k, v, do, sink, 1, scale)
    s = scale * float(q[0, 0, 0] @ k[0, 0, 0])
    p = 1.0 / (1.0 + math.exp(-(s - 0.7)))
    dov = float(do[0, 0, 0] @ v[0, 0, 0])
    assert abs(lse[0, 0, 0] - math.log(math.exp(0.7) + math.exp(s))) < 1e-14
    assert np.allclose(o[0, 0, 0], p * v[0, 0, 0], rtol=0, atol=1e-14)
    assert abs(g["dsink"][0] + p * (1 - p) * dov) < 1e-14
    assert np.allclose(g["dq"][0, 0, 0], scale * p * (1 - p) * dov * k[0, 0, 0], rtol=0, atol=1e-14)
    assert np.allclose(g["dk"][0, 0, 0], scale * p * (1 - p) * dov * q[0, 0, 0], rtol=0, atol=1e-14)
    assert np.allclose(g["dv"][0, 0, 0], p * do[0, 0, 0], rtol=0, atol=1e-14)


def test_window_one_is_identity_attention():
    """window = 1: each query sees only itself, so O_i = sigmoid(s_ii - sink) v_i."""
    rng = np.random.default_rng(29)
    S, D = 6, 8
    q, k, v = (_rand(rng, 1, 1, S, D) for _ in range(3))
    sink = np.array([-0.4])
    o, lse = oracle.sink_attention_forward(q, k, v, sink, 1, 1.0)
    s = np.einsum("sd,sd->s", q[0, 0], k[0, 0])
    p = 1 / (1 + np.exp(-(s + 0.4)))
    assert np.allclose(o[0, 0], p[:, None] * v[0, 0], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- invariants

def test_softmax_invariants_sink_window():
    rng = np.random.default_rng(31)
    B, Hq, Hkv, S, D, W = 1, 4, 2, 50, 16, 13
    scale = 0.25
    q, do = _rand(rng, B, Hq, S, D), _rand(rng, B, Hq, S, D)
    k, v = _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    sink = _rand(rng, Hq)
    o, lse, g = _oracle_sink(q, k, v, do, sink, W, scale)
    for h in range(Hq):
        kvh = h // (Hq // Hkv)
        s = scale * q[0, h] @ k[0, kvh].T
        vis = oracle.window_visibility(np.arange(S), np.arange(S), W)
        p = oracle.softmax_probabilities(s, lse[0, h], vis)
        p_sink = np.exp(sink[h] - lse[0, h])
        assert np.max(np.abs(p.sum(1) + p_sink - 1)) < 1e-13
        dp = do[0, h] @ v[0, kvh].T
        delta = (do[0, h] * o[0, h]).sum(1)
        ds = p * (dp - delta[:, None])
        # softmax shift invariance: sum_j dS_ij + dS_sink_i = 0 with dS_sink = -p_sink D_i
        assert np.max(np.abs(ds.sum(1) - p_sink * delta)) < 1e-12
    assert np.max(np.abs(g["delta"] - (do * o).sum(-1))) < 1e-13


def test_sink_free_column_sums_blocksparse():
    rng = np.random.default_rng(37)
    B, N, Sq, Skv, D, bx, by = 1, 3, 40, 40, 8, 8, 16
    nqb, nkb = Sq // bx, -(-Skv // by)
    mask = (rng.random((B, N, nqb, nkb)) < 0.6).astype(np.uint8)
    mask[0, 0, 2, :] = 0
    q, do = _rand(rng, B, N, Sq, D), _rand(rng, B, N, Sq, D)
    k, v = _rand(rng, B, N, Skv, D), _rand(rng, B, N, Skv, D)
    o, lse = oracle.blocksparse_attention_forward(q, k, v, mask, bx, by, 0.3)
    g = oracle.blocksparse_attention_backward(q, k, v, o, do, lse, mask, bx, by, 0.3)
    nonempty = np.isfinite(lse)
    for n in range(N):
        assert np.max(np.abs(g["dk"][0, n].sum(0))) < 1e-12
        assert np.allclose(g["dv"][0, n].sum(0), do[0, n][nonempty[0, n]].sum(0), rtol=0, atol=1e-12)


# --------------------------------------------------------------- sampled == full at samples

def test_sampled_matches_full_sink():
    rng = np.random.default_rng(41)
    B, Hq, Hkv, S, D, W = 2, 4, 2, 70, 16, 20
    q, do = _rand(rng, B, Hq, S, D), _rand(rng, B, Hq, S, D)
    k, v = _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    sink = _rand(rng, Hq)
    o, lse, g = _oracle_sink(q, k, v, do, sink, W, 0.25)
    qs = [(0, 0, 0), (1, 3, 69), (1, 2, 33)]
    ks = [(0, 0, 0), (1, 1, 69), (0, 1, 50)]
    sm = oracle.sink_attention_backward_sampled(q, k, v, o, do, lse, sink, W, 0.25, qs, ks)
    for t, (b, h, i) in enumerate(qs):
        assert np.allclose(sm["dq"][t], g["dq"][b, h, i], rtol=0, atol=1e-12)
    for t, (b, h, j) in enumerate(ks):
        assert np.allclose(sm["dk"][t], g["dk"][b, h, j], rtol=0, atol=1e-12)
        assert np.allclose(sm["dv"][t], g["dv"][b, h, j], rtol=0, atol=1e-12)
    assert np.allclose(sm["dsink"], g["dsink"], rtol=0, atol=1e-12)


def test_sampled_matches_full_blocksparse():
    rng = np.random.default_rng(43)
    B, N, Sq, Skv, D, bx, by = 1, 2, 50, 45, 8, 16, 16
    mask = (rng.random((B, N, 4, 3)) < 0.5).astype(np.uint8)
    q, do = _rand(rng, B, N, Sq, D), _rand(rng, B, N, Sq, D)
    k, v = _rand(rng, B, N, Skv, D), _rand(rng, B, N, Skv, D)
    o, lse = oracle.blocksparse_attention_forward(q, k, v, mask, bx, by, 0.3)
    g = oracle.blocksparse_attention_backward(q, k, v, o, do, lse, mask, bx, by, 0.3)
    qs = [(0, 0, 0), (0, 1, 49), (0, 1, 20)]
    ks = [(0, 0, 0), (0, 1, 44), (0, 0, 17)]
    sm = oracle.blocksparse_attention_backward_sampled(q, k, v, o, do, lse, mask, bx, by, 0.3, qs, ks)
    for t, (b, n, i) in enumerate(qs):
        assert np.allclose(sm["dq"][t], g["dq"][b, n, i], rtol=0, atol=1e-12)
    for t, (b, n, j) in enumerate(ks):
        assert np.allclose(sm["dk"][t], g["dk"][b, n, j], rtol=0, atol=1e-12)
        assert np.allclose(sm["dv"][t], g["dv"][b, n, j], rtol=0, atol=1e-12)


# ------------------------------------------------------- packed variable-length sequences

def test_packed_visibility_brute_force():
    """Visibility over packed rows against a per-pair loop: same sequence and inside the
    window; empty sequences and rows outside every sequence (cu[0] > 0, cu[B] < total)."""
    cu = [2, 5, 5, 6, 11, 11]
    total, window = 13, 3
    rows = np.arange(total)
    vis = oracle.packed_window_visibility(cu, rows, rows, window)
    for i in range(total):
        for j in range(total):
            same = any(cu[b] <= i < cu[b + 1] and cu[b] <= j < cu[b + 1] for b in range(len(cu) - 1))
            assert vis[i, j] == (same and 0 <= i - j < window), (i, j)


@pytest.mark.parametrize("window", [4, 1000])
def test_varlen_equals_per_sequence_dense(window):
    """Every sequence of the packed definition is the dense definition on its own rows (B = 1),
    and dsink is the sum of the per-sequence dsinks; empty and one-row sequences included."""
    rng = np.random.default_rng(window)
    lengths = [7, 0, 19, 1, 12]
    Hq, Hkv, D, scale = 4, 2, 16, 0.35
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    q, do = _rand(rng, Hq, T, D), _rand(rng, Hq, T, D)
    k, v = _rand(rng, Hkv, T, D), _rand(rng, Hkv, T, D)
    sink = _rand(rng, Hq)
    o, lse = oracle.sink_attention_forward_varlen(q, k, v, sink, cu, window, scale)
    g = oracle.sink_attention_backward_varlen(q, k, v, o, do, lse, sink, cu, window, scale)
    dsink = np.zeros(Hq)
    for b in range(len(lengths)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 == s0:
            continue
        sl = lambda x: x[None, :, s0:s1]
        ro, rlse = oracle.sink_attention_forward(sl(q), sl(k), sl(v), sink, window, scale)
        assert np.max(np.abs(ro[0] - o[:, s0:s1])) < 1e-12
        assert np.max(np.abs(rlse[0] - lse[:, s0:s1])) < 1e-12
        rg = oracle.sink_attention_backward(sl(q), sl(k), sl(v), sl(o), sl(do), sl(lse), sink, window, scale)
        for name in ("dq", "dk", "dv", "delta"):
            assert np.max(np.abs(rg[name][0] - g[name][:, s0:s1])) < 1e-12, (b, name)
        dsink += rg["dsink"]
    assert np.max(np.abs(dsink - g["dsink"])) < 1e-12


def test_varlen_sdpa_block_diagonal():
    """Without a sink, the packed definition is SDPA (fp64 autograd) over the whole packed
    batch with a block-diagonal, windowed token mask, K/V repeated over each group and dK/dV
    summed back over it."""
    rng = np.random.default_rng(77)
    lengths, window = [9, 14, 3], 6
    Hq, Hkv, D, scale = 4, 1, 8, 0.5
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    q, do = _rand(rng, Hq, T, D), _rand(rng, Hq, T, D)
    k, v = _rand(rng, Hkv, T, D), _rand(rng, Hkv, T, D)
    sink = np.full(Hq, -np.inf)
    o, lse = oracle.sink_attention_forward_varlen(q, k, v, sink, cu, window, scale)
    g = oracle.sink_attention_backward_varlen(q, k, v, o, do, lse, sink, cu, window, scale)
    seg = np.repeat(np.arange(len(lengths)), lengths)
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    m = torch.from_numpy((seg[:, None] == seg[None, :]) & (i - j >= 0) & (i - j < window))
    kr, vr = np.repeat(k, Hq // Hkv, axis=0), np.repeat(v, Hq // Hkv, axis=0)
    ro, rdq, rdk, rdv = _sdpa_grads(q[None], kr[None], vr[None], do[None], scale, attn_mask=m)
    rdk = rdk[0].reshape(Hkv, Hq // Hkv, T, D).sum(axis=1)
    rdv = rdv[0].reshape(Hkv, Hq // Hkv, T, D).sum(axis=1)
    for a, b in zip((o, g["dq"], g["dk"], g["dv"]), (ro[0], rdq[0], rdk, rdv)):
        assert np.max(np.abs(a - b)) < 1e-12 * max(1.0, np.max(np.abs(b)))
    assert np.all(g["dsink"] == 0)
