"""Pins of the fp64 oracle: checks against facts the oracle does not compute.

Each pin takes an oracle module (the real one, or a copy with a planted
mistake in tests/test_oracle_mutants.py) and raises AssertionError when the
oracle disagrees with a closed form, a special case, an identity, an
invariance or a brute-force computation.  References are to the technical
summary of "Gated Subspace Inference for Transformer Acceleration"
(S. J. Thomas, 2026), cited as GSI-TS.
"""
from __future__ import annotations

import numpy as np
import torch

from rank_gated_memory_amd import synth


def _rng(seed):
    return np.random.default_rng(seed)


def _orthonormal(rng, d, k):
    q, r = np.linalg.qr(rng.standard_normal((d, k)))
    return q * np.sign(np.diag(r))


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.allclose(a, b, rtol=rtol, atol=atol), f"{what}: max |diff| {np.max(np.abs(a - b))}"


def pin_identity_basis(orc):
    """V_k = first k columns of I: closed forms (GSI-TS §2.1, §2.2).

    g = x[:k], r = (0, x[k:]), rho = ||x[k:]|| / ||x||, M = W[:, :k],
    fast y = W[:, :k] x[:k], slow y = W x.
    """
    rng = _rng(11)
    d, d_out, k = 12, 7, 4
    W = rng.standard_normal((d_out, d))
    V = np.eye(d)[:, :k]
    X = rng.standard_normal((6, d))
    X[:3, k:] *= 1e-3          # three tokens with a tiny residual -> fast
    W_sq = rng.standard_normal((d, d))
    _close(orc.prepare(W_sq, V), W_sq[:, :k], 1e-15, 0, "M of a square W")
    M = orc.prepare(W, V)
    _close(M, W[:, :k], 1e-15, 0, "M")
    res = orc.linear(W, V, M, X, 0.05)
    _close(res["g"], X[:, :k], 1e-15, 0, "g")
    rho = np.array([np.sqrt(np.sum(x[k:] ** 2) / np.sum(x ** 2)) for x in X])
    _close(res["rho"], rho, 1e-13, 0, "rho")
    assert list(res["slow"]) == [False, False, False, True, True, True], res["slow"]
    for t in range(6):
        want = W @ X[t] if t >= 3 else W[:, :k] @ X[t, :k]
        _close(res["y"][t], want, 1e-13, 1e-15, f"y[{t}]")


def pin_full_rank(orc):
    """k = d: every x lies in the subspace, rho = 0 and M g = W x."""
    rng = _rng(12)
    d, d_out = 10, 6
    W = rng.standard_normal((d_out, d))
    V = _orthonormal(rng, d, d)
    X = rng.standard_normal((4, d))
    M = orc.prepare(W, V)
    res = orc.linear(W, V, M, X, 1e-6)
    assert np.all(res["rho"] < 1e-14), res["rho"]
    assert not res["slow"].any()
    for t in range(4):
        _close(res["y"][t], np.dot(W, X[t]), 1e-12, 1e-14, "y")


def pin_in_span_and_orthogonal(orc):
    """x in span(V_k) gives rho = 0 (fast); x orthogonal to V_k gives g = 0, rho = 1 (slow)."""
    rng = _rng(13)
    d, d_out, k = 20, 9, 5
    Q = _orthonormal(rng, d, k + 3)
    V, U = Q[:, :k], Q[:, k:]
    W = rng.standard_normal((d_out, d))
    M = orc.prepare(W, V)
    x_in = V @ rng.standard_normal(k)
    x_out = U @ rng.standard_normal(3)
    r = orc.linear(W, V, M, np.stack([x_in, x_out]), 1e-6)
    assert r["rho"][0] < 1e-14
    assert not r["slow"][0]
    _close(r["g"][1], np.zeros(k), 0, 1e-14, "g orthogonal")
    _close(r["rho"][1], 1.0, 1e-14, 0, "rho orthogonal")
    r2 = orc.linear(W, V, M, x_out[None], 0.99)
    assert r2["slow"][0]
    _close(r2["y"][0], np.dot(W, x_out), 1e-13, 1e-15, "slow y")


def pin_construction(orc):
    """Generator tokens with an orthogonal residual of known ratio (exact by construction)."""
    d, k, m = 64, 8, 16
    v, u = synth.orthonormal_frame(d, k, m, (99, 0, 0, synth.P_BASIS))
    mask = torch.zeros(12, dtype=torch.bool)
    mask[::2] = True
    X, rho_built = synth.tokens(v, u, mask, (99, 0, 0))
    V = v.numpy()
    W = _rng(14).standard_normal((5, d))
    res = orc.linear(W, V, orc.prepare(W, V), X.numpy(), 0.05)
    sl = mask.numpy()
    _close(res["rho"][sl], rho_built.numpy()[sl], 1e-12, 0, "constructed rho")
    assert res["slow"][sl].all()
    assert (res["rho"][~sl] < 0.0101).all() and not res["slow"][~sl].any()


def pin_decomposition(orc):
    """x = V_k g + r and M g + W r = W x (GSI-TS §2.1), in fp64."""
    rng = _rng(15)
    d, d_out, k = 48, 30, 7
    V = _orthonormal(rng, d, k)
    W = rng.standard_normal((d_out, d))
    M = orc.prepare(W, V)
    X = rng.standard_normal((5, d))
    res = orc.linear(W, V, M, X, 0.5)
    for t in range(5):
        _close(V @ res["g"][t] + res["r"][t], X[t], 1e-13, 1e-14, "x = Vg + r")
        _close(M @ res["g"][t] + W @ res["r"][t], np.dot(W, X[t]), 1e-12, 1e-13, "Mg + Wr = Wx")
        # r is orthogonal to the subspace (least-squares residual)
        _close(V.T @ res["r"][t], np.zeros(k), 0, 1e-13, "V^T r")


def pin_theorem4(orc):
    """Fast-path error <= ||W||_2 rho ||x|| < ||W||_2 eps ||x|| (GSI-TS §2.2, Theorem 4)."""
    rng = _rng(16)
    d, d_out, k = 40, 25, 6
    Q = _orthonormal(rng, d, k + 10)
    V, U = Q[:, :k], Q[:, k:]
    W = rng.standard_normal((d_out, d)) / np.sqrt(d)
    M = orc.prepare(W, V)
    # spectral norm from the eigenvalues of W^T W (independent of the oracle's SVD)
    w2 = float(np.sqrt(np.max(np.linalg.eigvalsh(W.T @ W))))
    eps = 0.2
    xs = []
    for rho in (0.0, 0.01, 0.05, 0.15, 0.19):
        z = rng.standard_normal(k)
        w = rng.standard_normal(10)
        c = rho * np.linalg.norm(z) / (np.linalg.norm(w) * np.sqrt(1 - rho * rho))
        xs.append(V @ z + c * (U @ w))
    X = np.stack(xs)
    res = orc.linear(W, V, M, X, eps, orc.FORCE_FAST)
    gated = orc.linear(W, V, M, X, eps)
    assert not gated["slow"].any()
    _close(orc.spectral_norm(W), w2, 1e-12, 0, "||W||_2 vs eigenvalues of W^T W")
    for t in range(len(xs)):
        err = np.linalg.norm(res["y"][t] - np.dot(W, X[t]))
        nx = np.linalg.norm(X[t])
        b = orc.theorem4_bound(W, X[t], res["rho"][t])
        _close(b, w2 * res["rho"][t] * nx, 1e-12, 1e-300, f"bound of token {t}")
        assert err <= b * (1 + 1e-10) + 1e-14, (t, err, b)
        assert err <= orc.theorem4_bound(W, X[t], eps)
    # the bound is attained when the residual lies on W's top right-singular direction
    _, s, vt = np.linalg.svd(W)
    top = vt[0] - V @ (V.T @ vt[0])
    top /= np.linalg.norm(top)
    # choose W so that its top right-singular vector is orthogonal to V
    W2 = np.outer(rng.standard_normal(d_out), top) * 3.0 + W @ (V @ V.T)
    M2 = orc.prepare(W2, V)
    x = V @ rng.standard_normal(k) + 0.1 * top
    r = orc.linear(W2, V, M2, x[None], 0.5)
    err = np.linalg.norm(r["y"][0] - np.dot(W2, x))
    w22 = float(np.sqrt(np.max(np.linalg.eigvalsh(W2.T @ W2))))
    bound = w22 * r["rho"][0] * np.linalg.norm(x)
    _close(orc.theorem4_bound(W2, x, r["rho"][0]), bound, 1e-12, 0, "nearly attained bound")
    assert err <= bound * (1 + 1e-10)
    assert err >= 0.5 * bound, (err, bound)


def pin_spectral_norm(orc):
    """||W||_2 in closed form: max |w_ii| for a diagonal W, ||a|| ||b|| for a
    rank-one W = a b^T, the scale for a scaled orthogonal W, and the square
    root of the largest eigenvalue of W^T W for a Gaussian W (independent of
    the oracle's SVD); the Theorem-4 bound is that norm times rho ||x||
    (GSI-TS §2.2)."""
    rng = _rng(31)
    D = np.diag([0.5, -3.25, 2.0, 1.0, 0.0])
    _close(orc.spectral_norm(D), 3.25, 1e-14, 0, "diagonal")
    a, b = rng.standard_normal(7), rng.standard_normal(11)
    _close(orc.spectral_norm(np.outer(a, b)), np.linalg.norm(a) * np.linalg.norm(b), 1e-13, 0, "rank one")
    Q = _orthonormal(rng, 9, 9)
    _close(orc.spectral_norm(2.5 * Q), 2.5, 1e-13, 0, "scaled orthogonal")
    G = rng.standard_normal((13, 6))
    _close(orc.spectral_norm(G), np.sqrt(np.max(np.linalg.eigvalsh(G.T @ G))), 1e-12, 0, "gaussian")
    x = np.array([3.0, 0.0, 4.0, 0.0, 0.0])
    _close(orc.theorem4_bound(D, x, 0.1), 3.25 * 0.1 * 5.0, 1e-14, 0, "bound of a diagonal map")
    _close(orc.theorem4_bound(D, 2.0 * x, 0.1), 3.25 * 0.1 * 10.0, 1e-14, 0, "bound scales with ||x||")
    assert orc.theorem4_bound(D, x, 0.0) == 0.0


def pin_gate_batch(orc):
    """The matrix form of the gate against closed forms (GSI-TS §2.1-§2.2):
    the identity basis (g = x[:k], rho = ||x[k:]|| / ||x||), tokens inside
    and orthogonal to the subspace (rho 0 and 1), constructed ratios, the
    least-squares residual, a zero token (rho 0, fast), NaN and Inf tokens
    (rho NaN, slow), the strict tie and the forced modes."""
    rng = _rng(32)
    d, k = 12, 4
    I = np.eye(d)[:, :k]
    X = rng.standard_normal((7, d))
    X[:3, k:] *= 1e-3
    X[5] = 0.0
    X[6, 2] = np.inf
    r = orc.gate_batch(I, X, 0.05)
    _close(r["g"][:6], X[:6, :k], 1e-15, 0, "identity g")
    want = np.array([np.linalg.norm(x[k:]) / np.linalg.norm(x) for x in X[:5]] + [0.0])
    _close(r["rho"][:6], want, 1e-13, 0, "identity rho")
    assert np.isnan(r["rho"][6])
    assert list(r["slow"]) == [False, False, False, True, True, False, True], r["slow"]
    # in span / orthogonal / constructed ratio
    Q = _orthonormal(rng, 30, 9)
    V, U = Q[:, :6], Q[:, 6:]
    z = rng.standard_normal(6)
    w = rng.standard_normal(3)
    rhos = [0.02, 0.3]
    toks = [V @ z, U @ w, np.full(30, np.nan)]
    for rho in rhos:
        c = rho * np.linalg.norm(z) / (np.linalg.norm(w) * np.sqrt(1 - rho * rho))
        toks.append(V @ z + c * (U @ w))
    r = orc.gate_batch(V, np.stack(toks), 0.05)
    assert r["rho"][0] < 1e-14 and not r["slow"][0]
    _close(r["g"][1], np.zeros(6), 0, 1e-14, "orthogonal g")
    _close(r["rho"][1], 1.0, 1e-14, 0, "orthogonal rho")
    assert np.isnan(r["rho"][2]) and r["slow"][2]
    _close(r["rho"][3:], rhos, 1e-12, 0, "constructed rho")
    assert list(r["slow"][3:]) == [False, True]
    # least squares (brute force) on a generic basis
    Y = rng.standard_normal((5, 30))
    r = orc.gate_batch(V, Y, 0.05)
    for t in range(5):
        sol, rss, _, _ = np.linalg.lstsq(V, Y[t], rcond=None)
        _close(r["g"][t], sol, 1e-12, 1e-14, "g vs lstsq")
        _close(r["rho"][t], np.sqrt(rss[0]) / np.linalg.norm(Y[t]), 1e-12, 0, "rho vs lstsq")
    # strict tie and forced modes
    x = (V @ z + 0.01 * (U @ w))[None]
    rho = float(orc.gate_batch(V, x, 0.5)["rho"][0])
    assert orc.gate_batch(V, x, rho)["slow"][0]
    assert not orc.gate_batch(V, x, float(np.nextafter(rho, np.inf)))["slow"][0]
    assert not orc.gate_batch(V, Y, 0.05, orc.FORCE_FAST)["slow"].any()
    assert orc.gate_batch(V, x, 0.5, orc.FORCE_SLOW)["slow"].all()


def pin_invariance(orc):
    """V_k -> V_k Q leaves rho and y unchanged; x -> a x keeps rho and scales y."""
    rng = _rng(17)
    d, d_out, k = 30, 11, 6
    V = _orthonormal(rng, d, k)
    Qk = _orthonormal(rng, k, k)
    W = rng.standard_normal((d_out, d))
    X = rng.standard_normal((4, d))
    X[:2] = (V @ rng.standard_normal((k, 2))).T + 1e-3 * rng.standard_normal((2, d))
    a = orc.linear(W, V, orc.prepare(W, V), X, 0.05)
    b = orc.linear(W, V @ Qk, orc.prepare(W, V @ Qk), X, 0.05)
    _close(a["rho"], b["rho"], 1e-12, 1e-15, "rho under V Q")
    _close(a["y"], b["y"], 1e-12, 1e-13, "y under V Q")
    c = orc.linear(W, V, orc.prepare(W, V), -2.5 * X, 0.05)
    _close(c["rho"], a["rho"], 1e-12, 1e-15, "rho under scaling")
    _close(c["y"], -2.5 * a["y"], 1e-12, 1e-13, "y under scaling")
    assert list(a["slow"]) == [False, False, True, True]


def pin_least_squares(orc):
    """Brute force: g and ||r|| from numpy's least-squares solve of V_k g ~ x."""
    rng = _rng(18)
    d, d_out, k = 25, 8, 5
    V = _orthonormal(rng, d, k)
    W = rng.standard_normal((d_out, d))
    X = rng.standard_normal((3, d))
    res = orc.linear(W, V, orc.prepare(W, V), X, 0.05)
    for t in range(3):
        sol, rss, rank, _ = np.linalg.lstsq(V, X[t], rcond=None)
        _close(res["g"][t], sol, 1e-12, 1e-14, "g vs lstsq")
        _close(res["rho"][t], np.sqrt(rss[0]) / np.linalg.norm(X[t]), 1e-12, 0, "rho vs lstsq")


def pin_gate_tie(orc):
    """Fast needs rho strictly below eps; rho == eps goes slow (GSI-TS §2.2)."""
    rng = _rng(19)
    d, d_out, k = 16, 6, 4
    V = _orthonormal(rng, d, k)
    W = rng.standard_normal((d_out, d))
    M = orc.prepare(W, V)
    x = V @ rng.standard_normal(k) + 0.05 * rng.standard_normal(d)
    rho = orc.linear(W, V, M, x[None], 0.5)["rho"][0]
    assert 0.0 < rho < 0.5
    at = orc.linear(W, V, M, x[None], float(rho))
    above = orc.linear(W, V, M, x[None], float(np.nextafter(rho, np.inf)))
    below = orc.linear(W, V, M, x[None], float(np.nextafter(rho, -np.inf)))
    assert at["slow"][0] and below["slow"][0] and not above["slow"][0]
    _close(at["y"][0], np.dot(W, x), 1e-13, 1e-14, "tie -> W x")
    _close(above["y"][0], M @ (V.T @ x), 1e-13, 1e-14, "above -> M g")


def pin_zero_token(orc):
    """x = 0: rho := 0, fast for eps > 0, y = 0; eps = 0 sends it slow, still y = 0."""
    rng = _rng(20)
    d, d_out, k = 10, 5, 3
    V = _orthonormal(rng, d, k)
    W = rng.standard_normal((d_out, d))
    M = orc.prepare(W, V)
    r = orc.linear(W, V, M, np.zeros((1, d)), 0.05)
    assert r["rho"][0] == 0.0 and not r["slow"][0]
    assert np.all(r["y"][0] == 0.0)
    r0 = orc.linear(W, V, M, np.zeros((1, d)), 0.0)
    assert r0["slow"][0] and np.all(r0["y"][0] == 0.0)


def pin_nonfinite(orc):
    """NaN or Inf in x: rho is NaN, the token goes slow and y carries it."""
    rng = _rng(21)
    d, d_out, k = 10, 5, 3
    V = _orthonormal(rng, d, k)
    W = rng.standard_normal((d_out, d))
    M = orc.prepare(W, V)
    X = rng.standard_normal((2, d))
    X[0, 4] = np.nan
    X[1, 2] = np.inf
    r = orc.linear(W, V, M, X, 0.05)
    assert np.isnan(r["rho"]).all()
    assert r["slow"].all()
    assert not np.isfinite(r["y"]).all(axis=1).any()


def pin_modes(orc):
    """Static projection (always fast) and dense (always slow) overrides."""
    rng = _rng(22)
    d, d_out, k = 14, 9, 5
    W = rng.standard_normal((d_out, d))
    V = np.eye(d)[:, :k]
    M = orc.prepare(W, V)
    X = rng.standard_normal((3, d))
    f = orc.linear(W, V, M, X, 0.05, orc.FORCE_FAST)
    s = orc.linear(W, V, M, X, 0.05, orc.FORCE_SLOW)
    assert not f["slow"].any() and s["slow"].all()
    for t in range(3):
        _close(f["y"][t], W[:, :k] @ X[t, :k], 1e-13, 1e-15, "force fast")
        _close(s["y"][t], np.dot(W, X[t]), 1e-13, 1e-15, "force slow")


def pin_batching(orc):
    """A batch equals its tokens one by one; row subsets equal full rows; stack equals calls."""
    rng = _rng(23)
    d, d_out, k = 18, 12, 4
    V = _orthonormal(rng, d, k)
    W = rng.standard_normal((d_out, d))
    M = orc.prepare(W, V)
    X = rng.standard_normal((5, d))
    X[:3] = (V @ rng.standard_normal((k, 3))).T + 1e-3 * rng.standard_normal((3, d))
    full = orc.linear(W, V, M, X, 0.05)
    assert full["y"].shape == (5, d_out) and full["rho"].shape == (5,)
    for t in range(5):
        one = orc.linear(W, V, M, X[t:t + 1], 0.05)
        _close(one["y"][0], full["y"][t], 0, 0, "token vs batch")
        rows = [0, 3, 11]
        sub = orc.linear_rows(W[rows], V, X[t], 0.05)
        assert sub["slow"] == bool(full["slow"][t])
        _close(sub["y"], full["y"][t, rows], 1e-13, 1e-15, "row subset")
    calls = [dict(W=W, V=V, M=M, X=X[:2], eps=0.05), dict(W=W[:5], V=V, M=M[:5], X=X[2:], eps=0.5)]
    st = orc.stack(calls)
    _close(st[0]["y"], full["y"][:2], 0, 0, "stack call 0")
    _close(st[1]["y"], orc.linear(W[:5], V, M[:5], X[2:], 0.5)["y"], 0, 0, "stack call 1")


def pin_norm_identity(orc):
    """For orthonormal V_k, rho also equals sqrt(1 - ||g||^2/||x||^2)."""
    rng = _rng(24)
    d, k = 64, 8
    V = _orthonormal(rng, d, k)
    W = rng.standard_normal((3, d))
    X = (V @ rng.standard_normal((k, 4))).T + 0.2 * rng.standard_normal((4, d))
    res = orc.linear(W, V, orc.prepare(W, V), X, 0.05)
    for t in range(4):
        _close(orc.rho_from_norms(X[t], res["g"][t]), res["rho"][t], 1e-10, 0, "pythagorean rho")


def pin_nested_bases(orc):
    """Growing a basis by more orthonormal columns never raises rho: with
    nested bases V_1 in V_2 in V_3, rho_3 <= rho_2 <= rho_1 for every token;
    a token inside span(V_2) has rho_2 = rho_3 = 0, and its rho_1 equals the
    norm of its coordinates on the columns V_2 adds, over ||x||."""
    rng = _rng(25)
    d = 48
    Q = _orthonormal(rng, d, 24)
    bases = [Q[:, :6], Q[:, :12], Q[:, :24]]
    X = rng.standard_normal((6, d))
    rhos = [[orc.residual_ratio(x, orc.residual(V, x, orc.project(V, x))) for x in X] for V in bases]
    for a, b in zip(rhos[:-1], rhos[1:]):
        assert all(rb <= ra + 1e-12 for ra, rb in zip(a, b)), "rho grew with the basis"
    c = rng.standard_normal(12)
    x = Q[:, :12] @ c
    r1 = orc.residual_ratio(x, orc.residual(bases[0], x, orc.project(bases[0], x)))
    _close(r1, np.linalg.norm(c[6:]) / np.linalg.norm(c), 1e-12, 0, "nested rho_1")
    for V in bases[1:]:
        assert orc.residual_ratio(x, orc.residual(V, x, orc.project(V, x))) < 1e-12


def pin_storage_rounding(orc):
    """Rounding into the storage type: torch's float32 -> bfloat16 conversion
    (round to nearest even) on float32 values across the whole exponent
    range, closed-form ties, subnormals, overflow and non-finite values."""
    rng = _rng(26)
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-88.0, 88.0, 20000))
    x = np.concatenate([x, rng.standard_normal(2000) * 2.0 ** -128])  # bf16 subnormal range
    x = x.astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    got = orc.to_storage(x, "bf16")
    assert np.array_equal(got, want), f"bf16: {np.sum(got != want)} values differ from torch"
    u = 2.0 ** -7  # spacing of bf16 in [1, 2)
    ties = {1 + u / 2: 1.0, 1 + 3 * u / 2: 1 + 2 * u, -(1 + u / 2): -1.0, 2.0 ** -133 * 1.5: 2.0 ** -132,
            2.0 ** -133 * 0.5: 0.0, (2 - u) * 2.0 ** 127: (2 - u) * 2.0 ** 127,
            (2 - u / 2) * 2.0 ** 127: np.inf, 1 + u / 4: 1.0, 1 + 3 * u / 4: 1 + u}
    for v, w in ties.items():
        assert orc.to_storage(np.array([v]), "bf16")[0] == w, f"bf16({v!r}) != {w!r}"
    sp = orc.to_storage(np.array([np.nan, np.inf, -np.inf, 0.0]), "bf16")
    assert np.isnan(sp[0]) and sp[1] == np.inf and sp[2] == -np.inf and sp[3] == 0.0
    y = rng.standard_normal(1000)
    assert np.array_equal(orc.to_storage(y, "fp32"), y.astype(np.float32).astype(np.float64))


def pin_chain(orc):
    """Calls reading earlier stored outputs (GSI-TS §2.3, §3).

    With k = d the gate is always fast and M g = W V V^T x = W x, so each
    output has the closed form W x with x the stored (rounded) slice of the
    producer's output; with the identity basis the gate of a chained call
    is decided by the tail of its stored input, rho = ||x[k:]|| / ||x||.
    """
    rng = _rng(27)
    d = 32
    for dt in ("fp32", "bf16"):
        W = [rng.standard_normal((2 * d, d)), rng.standard_normal((d, d)), rng.standard_normal((3 * d, d)),
             rng.standard_normal((d, d))]
        V = [_orthonormal(rng, d, d) for _ in W]
        x0 = rng.standard_normal(d)
        calls = [{"W": W[0], "V": V[0], "M": orc.prepare(W[0], V[0]), "eps": 0.05, "x": x0},
                 {"W": W[1], "V": V[1], "M": orc.prepare(W[1], V[1]), "eps": 0.05, "src": (0, d)},
                 {"W": W[2], "V": V[2], "M": orc.prepare(W[2], V[2]), "eps": 0.05, "src": (1, 0)},
                 {"W": W[3], "V": V[3], "M": orc.prepare(W[3], V[3]), "eps": 0.05, "src": (0, 0)}]
        res = orc.chain(calls, dt)
        y0 = W[0] @ x0
        x1 = orc.to_storage(y0, dt)[d:]
        y1 = W[1] @ x1
        x2 = orc.to_storage(y1, dt)
        y2 = W[2] @ x2
        x3 = orc.to_storage(y0, dt)[:d]
        y3 = W[3] @ x3
        for r, x, y, i in zip(res, (x0, x1, x2, x3), (y0, y1, y2, y3), range(4)):
            assert not r["slow"], f"{dt} call {i}: full-rank basis must take the fast path"
            assert np.array_equal(r["x"], x), f"{dt} call {i}: wrong input"
            _close(r["y"], y, 1e-12, 1e-12, f"{dt} chain call {i}")
        # identity basis: the chained call's gate follows the tail of its stored input
        k = d // 2
        E = np.eye(d)[:, :k]
        A = rng.standard_normal((d, d))
        B = rng.standard_normal((d, d))
        xa = np.concatenate([rng.standard_normal(k), 0.5 * rng.standard_normal(d - k)])
        cc = [{"W": A, "V": E, "M": orc.prepare(A, E), "eps": 0.05, "x": xa},
              {"W": B, "V": E, "M": orc.prepare(B, E), "eps": 0.05, "src": (0, 0)}]
        ra, rb = orc.chain(cc, dt)
        assert ra["slow"]
        _close(ra["y"], A @ xa, 1e-12, 1e-12, "slow producer")
        xb = orc.to_storage(A @ xa, dt)
        rho_b = np.linalg.norm(xb[k:]) / np.linalg.norm(xb)
        _close(rb["rho"], rho_b, 1e-12, 0, "chained rho")
        assert rb["slow"] == (not rho_b < 0.05)
        _close(rb["y"], B @ xb if rb["slow"] else B[:, :k] @ xb[:k], 1e-12, 1e-12, "chained output")
    for bad in ({"src": (1, 0)}, {"src": (0, 3 * d)}):
        c = [calls[0], dict(calls[1], **bad)]
        c[1].pop("x", None)
        try:
            orc.chain(c, "fp32")
        except ValueError:
            continue
        raise AssertionError(f"chain accepted {bad}")


def pin_gram_identity(orc):
    """For any basis V (orthonormal or not) and g = V^T x, the explicit
    residual satisfies ||x - V g||^2 = ||x||^2 - ||g||^2 + g^T E g with
    E = V^T V - I; E vanishes for an orthonormal basis and is diag(s^2 - 1)
    for columns scaled by s."""
    rng = _rng(28)
    d, k = 40, 6
    Q = _orthonormal(rng, d, k)
    assert np.max(np.abs(orc.gram_deviation(Q))) < 1e-13
    s = np.array([1.0, 0.5, 2.0, 1.01, 0.99, 3.0])
    _close(orc.gram_deviation(Q * s), np.diag(s * s - 1.0), 1e-12, 1e-12, "scaled columns")
    for V in (Q * s, Q + 0.05 * rng.standard_normal((d, k)), rng.standard_normal((d, k))):
        E = orc.gram_deviation(V)
        for _ in range(3):
            x = rng.standard_normal(d)
            g = orc.project(V, x)
            r = orc.residual(V, x, g)
            _close(np.dot(r, r), np.dot(x, x) - np.dot(g, g) + g @ E @ g, 1e-10, 1e-10, "gram identity")


def _spectral_samples(rng, n, d, spec):
    """n samples whose covariance has eigenvalues spec**2 along a random orthonormal frame."""
    F = _orthonormal(rng, d, len(spec))
    return (rng.standard_normal((n, len(spec))) * spec) @ F.T, F


def pin_dgks_orth(orc):
    """DGKS Gram-Schmidt gives the Q factor of Y = QR with diag(R) > 0:
    the same matrix as numpy's Householder QR after fixing its column signs,
    orthonormal to rounding even for an ill-conditioned block."""
    rng = _rng(29)
    for cond in (1.0, 1e6):
        U = _orthonormal(rng, 60, 8)
        Y = U @ np.diag(np.logspace(0, -np.log10(cond), 8)) @ _orthonormal(rng, 8, 8).T
        Q = orc.dgks_orth(Y)
        q, r = np.linalg.qr(Y)
        q = q * np.sign(np.diag(r))
        _close(Q, q, 1e-6 if cond > 1 else 1e-12, 1e-6 if cond > 1 else 1e-12, "dgks vs householder")
        assert np.max(np.abs(Q.T @ Q - np.eye(8))) < 1e-13
        R = Q.T @ Y
        assert np.all(np.diag(R) > 0) and np.max(np.abs(np.tril(R, -1))) < 1e-12 * np.abs(R).max()


def pin_subspace_iteration(orc):
    """The iteration converges to the top-k singular subspace (LAPACK SVD)
    at the rate of the spectral gap, keeps an exact top-k basis fixed, and
    from a nearby start (the cascade) needs fewer sweeps than from a random
    start to reach the same accuracy (GSI-TS §2.3)."""
    rng = _rng(30)
    d, k = 80, 6
    spec = np.concatenate([np.linspace(10.0, 6.0, k), np.linspace(2.0, 0.1, d - k)])
    A, F = _spectral_samples(rng, 400, d, spec)
    top = orc.dominant_subspace(A, k)
    assert orc.principal_cosines(top, F[:, :k]).min() > 0.95
    cold = orc.subspace_iteration(A, rng.standard_normal((d, k)), 30)
    assert 1.0 - orc.principal_cosines(cold, top).min() < 1e-12
    fixed = orc.subspace_iteration(A, top, 1)
    assert 1.0 - orc.principal_cosines(fixed, top).min() < 1e-13
    near = orc.dgks_orth(top + 0.05 * rng.standard_normal((d, k)))
    far = rng.standard_normal((d, k))

    def sweeps(V0, tol=1e-10):
        V = V0
        for it in range(1, 60):
            V = orc.subspace_iteration(A, V, 1)
            if 1.0 - orc.principal_cosines(V, top).min() < tol:
                return it
        return 60
    assert sweeps(near) < sweeps(far)


ALL_PINS = [
    pin_identity_basis, pin_full_rank, pin_in_span_and_orthogonal, pin_construction,
    pin_decomposition, pin_theorem4, pin_invariance, pin_least_squares, pin_gate_tie,
    pin_zero_token, pin_nonfinite, pin_modes, pin_batching, pin_norm_identity, pin_nested_bases,
    pin_storage_rounding, pin_chain, pin_gram_identity, pin_dgks_orth, pin_subspace_iteration,
    pin_spectral_norm, pin_gate_batch,
]
