"""Helpers that compare GPU results with the fp64 oracle (GSI-TS §2.1-§2.2).

Bar: gates bit-exact except for tokens whose oracle ratio lies within 1e-3
of eps; outputs within a per-token relative L2 tolerance (2e-2 for bf16
storage, 1e-5 for fp32).  A band token whose gate differs is compared with
the oracle output of the path the GPU actually took.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import gsi_oracle as orc

GATE_BAND = 1e-3
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def f64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


def eps32(eps: float) -> float:
    """The threshold as the library sees it (a float argument)."""
    return float(np.float32(eps))


def compare_tokens(W, V, X, eps, y_gpu, slow_gpu, rho_gpu, dtype, mode=orc.GATED, M=None,
                   rho_tol=None, what=""):
    """Check T tokens of one map against the oracle.

    W is [R][d]: either the whole weight or only the sampled output rows
    (then y_gpu holds the GPU output at those rows; row i of M = W V_k only
    needs row i of W).  Returns (worst relative error, band tokens whose gate
    differed).
    """
    tol = TOL[dtype]
    eps = eps32(eps)
    if M is None:
        M = orc.prepare(W, V)
    slow_g = np.asarray(slow_gpu).astype(bool)
    rho_g = np.asarray(rho_gpu, dtype=np.float64)
    y_g = np.asarray(y_gpu, dtype=np.float64)
    worst, n_band = 0.0, 0
    for t in range(X.shape[0]):
        x = X[t]
        ref = orc.linear_token(W, V, M, x, eps, mode)
        want = ref["y"]
        if bool(ref["slow"]) != bool(slow_g[t]):
            assert abs(ref["rho"] - eps) < GATE_BAND, (
                f"{what} token {t}: gate gpu={slow_g[t]} oracle={ref['slow']} rho={ref['rho']:.6f}")
            n_band += 1
            want = orc.slow_output(W, x) if slow_g[t] else orc.fast_output(M, ref["g"])
        if rho_tol is not None and np.isfinite(ref["rho"]):
            assert abs(rho_g[t] - ref["rho"]) <= rho_tol, (
                f"{what} token {t}: rho gpu {rho_g[t]:.6f} oracle {ref['rho']:.6f}")
        nw = np.linalg.norm(want)
        if not np.isfinite(nw):
            assert not np.isfinite(y_g[t]).all(), f"{what} token {t}: expected non-finite output"
            continue
        if nw == 0.0:
            assert np.all(y_g[t] == 0.0), f"{what} token {t}: expected zeros"
            continue
        err = np.linalg.norm(y_g[t] - want) / nw
        worst = max(worst, err)
        assert err <= tol, f"{what} token {t}: rel L2 {err:.3e} > {tol} (slow={slow_g[t]})"
    return worst, n_band
