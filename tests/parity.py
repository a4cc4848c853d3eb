"""Element-wise comparison of GPU results with the fp64 oracle.

Tolerances come from the FAQ Q10 table (tests/golden/faq_q10_tolerances.txt):
|O_gpu - O_ref| <= atol + rtol * |O_ref| per element, fp16 1e-3/1e-3 and bf16
5e-3/5e-3; LSE within 1e-4 absolute where finite and exactly -inf where the
oracle has no visible key; no NaN anywhere.
"""
import numpy as np
import torch

import golden_io

TOL = golden_io.tolerances()
LSE_ATOL = 1e-4


def _np(x):
    if torch.is_tensor(x):
        return x.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def dtype_name(t):
    return {torch.float16: "fp16", torch.bfloat16: "bf16"}[t]


def assert_o_close(o_gpu, o_ref, dtype, where=""):
    atol, rtol = TOL[dtype_name(dtype) if not isinstance(dtype, str) else dtype]
    g = _np(o_gpu)
    r = np.asarray(o_ref, dtype=np.float64)
    assert g.shape == r.shape, f"{where}: shape {g.shape} vs {r.shape}"
    assert not np.isnan(g).any(), f"{where}: NaN in O"
    err = np.abs(g - r)
    bad = err > atol + rtol * np.abs(r)
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{where}: {int(bad.sum())} of {bad.size} O elements out of tolerance "
                             f"(max err {err.max():.3e}); first at {idx}")


def assert_lse_close(lse_gpu, lse_ref, where=""):
    g = _np(lse_gpu)
    r = np.asarray(lse_ref, dtype=np.float64)
    assert g.shape == r.shape, f"{where}: LSE shape {g.shape} vs {r.shape}"
    assert not np.isnan(g).any(), f"{where}: NaN in LSE"
    ninf = np.isneginf(r)
    assert np.array_equal(np.isneginf(g), ninf), f"{where}: -inf pattern of LSE differs"
    fin = ~ninf
    err = np.abs(g[fin] - r[fin])
    if err.size and err.max() > LSE_ATOL:
        raise AssertionError(f"{where}: LSE max err {err.max():.3e} > {LSE_ATOL}")
