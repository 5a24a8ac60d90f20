"""fp64 CPU oracle of the gated subspace linear map (test infrastructure).

This module is the checker, not the product.  Only the test suite, the
package smoke check and the CPU-baseline leg of the benchmark may import it;
the HIP library never calls it and shares no code with it.

Source: "Gated Subspace Inference for Transformer Acceleration" (S. J. Thomas,
2026), technical summary as rendered by gist.science, cited below as GSI-TS.

  * GSI-TS §2.1 (core decomposition): for a linear map W in R^{d_out x d}
    and an orthonormal basis V_k in R^{d x k}, an activation splits exactly
    into x = V_k V_k^T x + r, so y = W x = (W V_k)(V_k^T x) + W r = M g + W r
    with the cached image M = W V_k and the coordinates g = V_k^T x.
  * GSI-TS §2.2 (gated residual step): per token the residual ratio
    rho = ||r|| / ||x|| is compared with a threshold eps; below it the
    output is taken as M g (fast path), otherwise the full W x is computed
    (slow path).  Theorem 4 there bounds the fast-path error of a token by
    ||W||_2 * eps * ||x||.

Everything is plain numpy float64 on inputs already upcast exactly from their
storage dtype.  The residual r is formed explicitly.  No blocking, fusion or
reordering beyond the definitions is done, so each function can be read
against the pages.

Readings where the pages are silent (each is listed in the design notes):
  * tie rho == eps goes to the slow path (fast needs rho strictly below eps);
  * ||x|| == 0 gives rho := 0, hence the fast path, whose output M g = 0
    equals W x exactly;
  * a NaN/Inf token makes rho NaN; "rho < eps" is then false, so the token
    takes the slow path and W x carries the NaN as a dense layer would;
  * the slow path returns W x (the §2.2 statement), not M g + W r (equal in
    exact arithmetic, see the decomposition pin);
  * eps <= 0 or eps > 1 is applied literally.

Readings for chains of calls (an input read from an earlier output):
  * the input is the earlier output as stored, i.e. rounded to nearest-even
    in the storage type, not the exact value.

Every function here is pinned by tests that check it against closed forms,
special cases, identities, invariances or brute force (see tests/).
"""
from __future__ import annotations

import numpy as np

GATED, FORCE_FAST, FORCE_SLOW = 0, 1, 2


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def prepare(W, V) -> np.ndarray:
    """Cached low-rank image M = W V_k (GSI-TS §2.1), shape [d_out][k]."""
    return _f64(W) @ _f64(V)


def project(V, x) -> np.ndarray:
    """Subspace coordinates g = V_k^T x (GSI-TS §2.1), shape [k]."""
    return _f64(V).T @ _f64(x)


def residual(V, x, g) -> np.ndarray:
    """Explicit residual r = x - V_k g (GSI-TS §2.1), shape [d]."""
    return _f64(x) - _f64(V) @ _f64(g)


def residual_ratio(x, r) -> float:
    """rho = ||r|| / ||x|| (GSI-TS §2.2); 0 for x = 0, NaN for non-finite x."""
    nx = float(np.linalg.norm(_f64(x)))
    nr = float(np.linalg.norm(_f64(r)))
    if not np.isfinite(nx) or not np.isfinite(nr):
        return float("nan")
    if nx == 0.0:
        return 0.0
    return nr / nx


def takes_slow_path(rho: float, eps: float, mode: int = GATED) -> bool:
    """Gate (GSI-TS §2.2): fast iff rho < eps, slow otherwise (ties slow)."""
    if mode == FORCE_FAST:
        return False
    if mode == FORCE_SLOW:
        return True
    return not (rho < eps)


def fast_output(M, g) -> np.ndarray:
    """Fast path y = M g (GSI-TS §2.2)."""
    return _f64(M) @ _f64(g)


def slow_output(W, x) -> np.ndarray:
    """Slow path y = W x (GSI-TS §2.2)."""
    return _f64(W) @ _f64(x)


def linear_token(W, V, M, x, eps: float, mode: int = GATED) -> dict:
    """One token through the gated map: g, r, rho, slow flag and y."""
    g = project(V, x)
    r = residual(V, x, g)
    rho = residual_ratio(x, r)
    slow = takes_slow_path(rho, eps, mode)
    y = slow_output(W, x) if slow else fast_output(M, g)
    return {"g": g, "r": r, "rho": rho, "slow": slow, "y": y}


def linear(W, V, M, X, eps: float, mode: int = GATED) -> dict:
    """T tokens ([T][d]) through the gated map, one token at a time.

    Returns stacked arrays: g [T][k], r [T][d], rho [T], slow [T] (bool),
    y [T][d_out].
    """
    X = _f64(X)
    outs = [linear_token(W, V, M, X[t], eps, mode) for t in range(X.shape[0])]
    k = _f64(V).shape[1]
    d_out = _f64(W).shape[0]
    if not outs:
        return {"g": np.zeros((0, k)), "r": np.zeros((0, X.shape[1])), "rho": np.zeros(0),
                "slow": np.zeros(0, dtype=bool), "y": np.zeros((0, d_out))}
    return {
        "g": np.stack([o["g"] for o in outs]),
        "r": np.stack([o["r"] for o in outs]),
        "rho": np.array([o["rho"] for o in outs]),
        "slow": np.array([o["slow"] for o in outs], dtype=bool),
        "y": np.stack([o["y"] for o in outs]),
    }


def gate_batch(V, X, eps: float, mode: int = GATED) -> dict:
    """Gates of T tokens ([T][d]) at once (GSI-TS §2.1-§2.2), the same
    definitions as project / residual / residual_ratio / takes_slow_path
    written with matrix products over the token rows:
    G = X V_k (row t is g_t), R = X - G V_k^T (row t is r_t),
    rho_t = ||R_t|| / ||X_t||, with rho_t := 0 for a zero row and NaN for a
    row holding NaN or Inf; slow_t = not(rho_t < eps), or the forced mode.
    For checking long token sequences (every gate of a decode run).
    Returns g [T][k], rho [T], slow [T] (bool).
    """
    X = _f64(X)
    V = _f64(V)
    G = X @ V
    R = X - G @ V.T
    nx = np.linalg.norm(X, axis=1)
    nr = np.linalg.norm(R, axis=1)
    finite = np.isfinite(nx) & np.isfinite(nr)
    with np.errstate(invalid="ignore", divide="ignore"):
        rho = np.where(nx > 0.0, nr / np.where(nx > 0.0, nx, 1.0), 0.0)
    rho = np.where(finite, rho, np.nan)
    if mode == FORCE_FAST:
        slow = np.zeros(X.shape[0], dtype=bool)
    elif mode == FORCE_SLOW:
        slow = np.ones(X.shape[0], dtype=bool)
    else:
        with np.errstate(invalid="ignore"):
            slow = ~(rho < eps)
    return {"g": G, "rho": rho, "slow": slow}


def linear_rows(W_rows, V, x, eps: float, mode: int = GATED) -> dict:
    """One token, outputs restricted to a subset of rows of W.

    For maps too large to form M in full: the gate needs all of V_k and x,
    while each sampled output row i uses only row i of W, i.e. row i of
    M = W V_k.  Same definitions as linear_token, evaluated row by row.
    """
    g = project(V, x)
    r = residual(V, x, g)
    rho = residual_ratio(x, r)
    slow = takes_slow_path(rho, eps, mode)
    if slow:
        y = slow_output(W_rows, x)
    else:
        y = fast_output(prepare(W_rows, V), g)
    return {"g": g, "rho": rho, "slow": slow, "y": y}


def to_storage(y, dtype: str) -> np.ndarray:
    """The value a stored output holds: y rounded to nearest, ties to even, in
    the storage type ("fp32" or "bf16").

    bf16 keeps 8 significant bits and fp32's exponent range: normal values
    are rounded to 8 bits, values below 2**-126 to the subnormal grid of
    spacing 2**-133, and values that round to 2**128 or beyond overflow to
    infinity.  NaN and infinities are kept.
    """
    y = _f64(y)
    if dtype == "fp32":
        return y.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(f"unknown storage type {dtype!r}")
    with np.errstate(invalid="ignore", over="ignore"):
        m, e = np.frexp(y)  # y = m 2**e with 0.5 <= |m| < 1
        normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
        sub = np.ldexp(np.rint(np.ldexp(y, 133)), -133)
        out = np.where(np.abs(y) < 2.0 ** -126, sub, normal)
        out = np.where(np.abs(out) >= 2.0 ** 128, np.copysign(np.inf, y), out)
    return np.where(np.isfinite(y), out, y)


def chain(calls, dtype: str, mode: int = GATED) -> list:
    """Gated calls evaluated in order, where a call may read the output of an
    earlier one (the maps of consecutive transformer layers, GSI-TS §2.3 and
    §3: the gate is applied to every linear map, each fed by the ones before).

    Each call is a dict with W, V, M, eps and either "x" (its own token) or
    "src" = (j, offset): its input is the stored output of call j < i, i.e.
    to_storage(y_j, dtype), from element `offset` on, d elements long.
    Returns, per call, the linear_token result plus "x" (the input used).
    """
    out = []
    for i, c in enumerate(calls):
        if "src" in c:
            j, off = c["src"]
            if not 0 <= j < i:
                raise ValueError(f"call {i} reads call {j}, which does not come before it")
            d = _f64(c["V"]).shape[0]
            x = to_storage(out[j]["y"], dtype)[off:off + d]
            if x.shape[0] != d:
                raise ValueError(f"call {i}: slice [{off}, {off + d}) beyond the output of call {j}")
        else:
            x = _f64(c["x"])
        r = linear_token(c["W"], c["V"], c["M"], x, c["eps"], mode)
        r["x"] = x
        out.append(r)
    return out


def stack(calls, mode: int = GATED) -> list:
    """A sequence of independent gated calls (one per map of a decode step).

    `calls` holds dicts with keys W, V, M, X, eps.  GSI-TS §3 applies the gate
    to every linear map of the transformer; the calls here are independent,
    so the sequence is evaluated one call after the other.
    """
    return [linear(c["W"], c["V"], c["M"], c["X"], c["eps"], mode) for c in calls]


# ---- basis calibration (GSI-TS §2.3) ----------------------------------------
#
# The summary computes V_k once per layer from activations of a calibration
# pass, as the top-k subspace of those activations (the directions a full
# SVD would give), and starts layer l+1 from layer l's basis so that only
# small corrections, orthogonalised by DGKS, are needed.  Reading used here:
# V_k is the dominant k-dimensional left singular subspace of the sample
# matrix A^T (A = [n tokens][d]); it is reached by block subspace iteration
# V <- orth(A^T (A V)) from a starting basis V0 (random for a cold start, the
# previous layer's basis for the cascade), each sweep orthonormalising the
# new block column by column with DGKS (classical Gram-Schmidt, repeated
# while a column loses more than half its norm to the projection).


def dgks_orth(Y, eta: float = 1.0 / np.sqrt(2.0)) -> np.ndarray:
    """Orthonormal Q with span(Q) = span(Y) and Q^T Y upper triangular with a
    positive diagonal (the Q of Y = QR), by classical Gram-Schmidt with DGKS
    reorthogonalisation: a column's projection on the earlier columns is
    removed again while the removal shrinks its norm below eta times what it
    was."""
    Y = _f64(Y)
    d, k = Y.shape
    Q = np.zeros((d, k))
    for j in range(k):
        w = Y[:, j].copy()
        for _ in range(4):
            before = np.linalg.norm(w)
            w = w - Q[:, :j] @ (Q[:, :j].T @ w)
            if np.linalg.norm(w) > eta * before:
                break
        nw = np.linalg.norm(w)
        if not nw > 0.0:
            raise ValueError(f"column {j} of the block is dependent on the earlier ones")
        Q[:, j] = w / nw
    return Q


def subspace_iteration(A, V0, iters: int) -> np.ndarray:
    """`iters` sweeps of V <- orth(A^T (A V)) from V0 ([d][k]); A is [n][d]."""
    A = _f64(A)
    V = _f64(V0)
    for _ in range(iters):
        V = dgks_orth(A.T @ (A @ V))
    return V


def dominant_subspace(A, k: int) -> np.ndarray:
    """Top-k right singular vectors of A ([n][d]) via LAPACK SVD: the
    subspace the iteration converges to (reference only)."""
    _, _, vt = np.linalg.svd(_f64(A), full_matrices=False)
    return vt[:k].T


def principal_cosines(V1, V2) -> np.ndarray:
    """Cosines of the principal angles between span(V1) and span(V2)
    (orthonormal bases), largest first."""
    return np.linalg.svd(_f64(V1).T @ _f64(V2), compute_uv=False)


# ---- diagnostics (not compared against the GPU, used by pins) -------------

def rho_from_norms(x, g) -> float:
    """sqrt(max(0, 1 - ||g||^2/||x||^2)): equals rho when V_k is orthonormal."""
    nx2 = float(np.dot(_f64(x), _f64(x)))
    if nx2 == 0.0:
        return 0.0
    return float(np.sqrt(max(0.0, 1.0 - float(np.dot(_f64(g), _f64(g))) / nx2)))


def spectral_norm(W) -> float:
    """||W||_2 (largest singular value) via LAPACK SVD."""
    return float(np.linalg.norm(_f64(W), 2))


def gram_deviation(V) -> np.ndarray:
    """E = V_k^T V_k - I: how far the stored basis is from orthonormal (zero
    for the orthonormal V_k of GSI-TS §2.1)."""
    V = _f64(V)
    return V.T @ V - np.eye(V.shape[1])


def theorem4_bound(W, x, rho: float) -> float:
    """Fast-path error bound ||W||_2 * rho * ||x|| (GSI-TS §2.2, Theorem 4).

    With rho < eps on the fast path this is below ||W||_2 * eps * ||x||.
    """
    return spectral_norm(W) * rho * float(np.linalg.norm(_f64(x)))
