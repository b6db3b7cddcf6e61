"""Tolerance gate shared by the GPU parity tests.

Every element must satisfy |got - ref| <= a + a*|ref| with a = 2e-3 for fp16 and
a = 1.6e-2 for bf16, and max |got - ref| <= 0.1; a non-finite element fails before the
tolerance is looked at (a NaN compares false against any bound).
"""

import numpy as np
import torch

ATOL = {torch.float16: 2e-3, torch.bfloat16: 1.6e-2}
MAX_ABS = 0.1


def to64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").double().numpy()


def check(name, got, ref, dtype):
    g = to64(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
    if not np.all(np.isfinite(g)):
        bad = np.argwhere(~np.isfinite(g))[:5]
        raise AssertionError(f"{name}: {np.count_nonzero(~np.isfinite(g))} non-finite elements, e.g. at {bad.tolist()}")
    a = ATOL[dtype]
    err = np.abs(g - r)
    bound = a + a * np.abs(r)
    ok = err <= bound
    worst = float((err / bound).max()) if err.size else 0.0
    if not ok.all() or (err.size and err.max() > MAX_ABS):
        idx = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{name}: {np.count_nonzero(~ok)} of {err.size} elements outside {a}+{a}|ref|; "
                             f"max abs err {err.max():.3e}; worst at {tuple(int(i) for i in idx)}: "
                             f"got {g[idx]:.6e} ref {r[idx]:.6e}")
    return {"max_abs": float(err.max()) if err.size else 0.0, "worst_ratio": worst}
