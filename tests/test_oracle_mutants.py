"""Plant plausible mistakes in a private copy of the oracle (on the CPU) and
check that the pin suite catches every one of them.

A mutant counts as caught when at least one pin raises (an assertion or any
other error).  The real oracle module is never modified.
"""
import importlib.util
import os

import numpy as np
import pytest

from tests.oracle_pins import ALL_PINS

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "oracle", "gsi_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("gsi_oracle_mutant", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


f64 = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731

MUTANTS = {
    # prepare: columns of V_k taken in the wrong order / transposed W
    "prepare_column_order": ("prepare", lambda W, V: f64(W) @ f64(V)[:, ::-1]),
    "prepare_transposed_W": ("prepare", lambda W, V: f64(W).T @ f64(V)),
    # projection: dropped or reordered coordinates
    "project_reversed": ("project", lambda V, x: f64(V)[:, ::-1].T @ f64(x)),
    "project_drop_last": ("project", lambda V, x: np.concatenate([f64(V)[:, :-1].T @ f64(x), [0.0]])),
    # residual: wrong sign, dropped basis term
    "residual_sign": ("residual", lambda V, x, g: f64(x) + f64(V) @ f64(g)),
    "residual_drop_term": ("residual", lambda V, x, g: f64(x) - f64(V)[:, :-1] @ f64(g)[:-1]),
    # ratio: wrong denominator, squared, no zero guard
    "ratio_over_g": ("residual_ratio", lambda x, r: float(np.linalg.norm(r) / max(np.linalg.norm(x[:1]), 1e-300))),
    "ratio_squared": ("residual_ratio", lambda x, r: float(np.dot(r, r) / np.dot(x, x)) if np.dot(x, x) else 0.0),
    "ratio_no_zero_guard": ("residual_ratio", lambda x, r: float(np.float64(np.linalg.norm(r)) / np.float64(np.linalg.norm(x)))),
    # gate: tie goes fast, inverted, modes ignored
    "gate_tie_fast": ("takes_slow_path", lambda rho, eps, mode=0: (mode == 2) or (mode != 1 and rho > eps)),
    "gate_inverted": ("takes_slow_path", lambda rho, eps, mode=0: (mode == 2) or (mode != 1 and rho < eps)),
    "gate_ignores_modes": ("takes_slow_path", lambda rho, eps, mode=0: not (rho < eps)),
    # outputs: dropped terms, swapped path
    "fast_drop_term": ("fast_output", lambda M, g: f64(M)[:, :-1] @ f64(g)[:-1]),
    "slow_drop_term": ("slow_output", lambda W, x: f64(W)[:, :-1] @ f64(x)[:-1]),
    "slow_uses_image": ("linear_token", None),
    "batch_drops_token": ("linear", None),
    # storage rounding: truncation, ties away from zero, bf16 kept as fp32
    "storage_truncates": ("to_storage", None),
    "storage_ties_away": ("to_storage", None),
    "storage_bf16_as_fp32": ("to_storage", None),
    # chains: exact instead of stored input, offset ignored, wrong producer
    "chain_unrounded_input": ("chain", None),
    "chain_ignores_offset": ("chain", None),
    "chain_reads_previous_call": ("chain", None),
    # Gram deviation: no identity subtracted, transposed product
    "gram_no_identity": ("gram_deviation", lambda V: f64(V).T @ f64(V)),
    "gram_outer": ("gram_deviation", lambda V: f64(V) @ f64(V).T - np.eye(f64(V).shape[0])),
    # calibration: no reorthogonalisation pass, no normalisation, no block orthonormalisation
    "dgks_single_pass": ("dgks_orth", None),
    "dgks_unnormalised": ("dgks_orth", None),
    "iteration_one_sided": ("subspace_iteration", None),
    # Theorem-4 diagnostics: Frobenius instead of spectral norm, smallest
    # singular value, ||x|| squared or dropped in the bound
    "spectral_as_frobenius": ("spectral_norm", lambda W: float(np.linalg.norm(f64(W)))),
    "spectral_smallest": ("spectral_norm", lambda W: float(np.linalg.norm(f64(W), -2))),
    "bound_x_squared": ("theorem4_bound", lambda W, x, rho: float(np.linalg.norm(f64(W), 2)) * rho
                        * float(np.dot(f64(x), f64(x)))),
    "bound_drops_x": ("theorem4_bound", lambda W, x, rho: float(np.linalg.norm(f64(W), 2)) * rho),
    "bound_frobenius": ("theorem4_bound", lambda W, x, rho: float(np.linalg.norm(f64(W))) * rho
                        * float(np.linalg.norm(f64(x)))),
    # matrix-form gate: dropped basis column,
    # squared ratio, zero rows not guarded, tie sent fast, modes ignored
    "batch_gate_drop_column": ("gate_batch", None),
    "batch_gate_squared": ("gate_batch", None),
    "batch_gate_no_zero_guard": ("gate_batch", None),
    "batch_gate_tie_fast": ("gate_batch", None),
    "batch_gate_ignores_modes": ("gate_batch", None),
}


def _mutant_gate_batch(how):
    def gate_batch(V, X, eps, mode=0):
        X, V = f64(X), f64(V)
        Vu = V[:, :-1] if how == "drop" else V
        G = X @ V
        R = X - (X @ Vu) @ Vu.T
        nx = np.linalg.norm(X, axis=1)
        nr = np.linalg.norm(R, axis=1)
        with np.errstate(all="ignore"):
            if how == "noguard":
                rho = nr / nx
            else:
                rho = np.where(nx > 0, nr / np.where(nx > 0, nx, 1.0), 0.0)
            rho = np.where(np.isfinite(nx) & np.isfinite(nr), rho, np.nan)
            if how == "squared":
                rho = rho * rho
            slow = (rho > eps) if how == "tie" else ~(rho < eps)
        if how != "modes":
            if mode == 1:
                slow = np.zeros_like(slow)
            elif mode == 2:
                slow = np.ones_like(slow)
        return {"g": G, "rho": rho, "slow": slow}
    return gate_batch


def _mutant_dgks(how):
    def dgks_orth(Y, eta=0.7071):
        Y = f64(Y)
        d, k = Y.shape
        Q = np.zeros((d, k))
        for j in range(k):
            w = Y[:, j] - Q[:, :j] @ (Q[:, :j].T @ Y[:, j])
            Q[:, j] = w if how == "unnormalised" else w / np.linalg.norm(w)
        return Q
    return dgks_orth


def _mutant_iteration(mod):
    # columns normalised one by one instead of orthonormalised as a block:
    # every column drifts toward the top direction
    def subspace_iteration(A, V0, iters):
        V = f64(V0)
        for _ in range(iters):
            V = f64(A).T @ (f64(A) @ V)
            V = V / np.linalg.norm(V, axis=0)
        return V
    return subspace_iteration


def _mutant_to_storage(mod, how):
    orig = mod.to_storage

    def to_storage(y, dtype):
        y = f64(y)
        if dtype != "bf16" or how == "as_fp32":
            return y.astype(np.float32).astype(np.float64)
        m, e = np.frexp(y)
        t = np.ldexp(m, 8)
        r = np.trunc(t) if how == "trunc" else np.sign(t) * np.floor(np.abs(t) + 0.5)
        out = np.ldexp(r, e - 8)
        return np.where(np.isfinite(y), out, orig(y, dtype))
    return to_storage


def _mutant_chain(mod, how):
    def chain(calls, dtype, mode=0):
        out = []
        for i, c in enumerate(calls):
            if "src" in c:
                j, off = c["src"]
                if not 0 <= j < i:
                    raise ValueError("bad producer")
                if how == "previous":
                    j = i - 1
                if how == "no_offset":
                    off = 0
                d = f64(c["V"]).shape[0]
                y = out[j]["y"] if how == "unrounded" else mod.to_storage(out[j]["y"], dtype)
                x = y[off:off + d]
                if x.shape[0] != d:
                    raise ValueError("slice")
            else:
                x = f64(c["x"])
            r = mod.linear_token(c["W"], c["V"], c["M"], x, c["eps"], mode)
            r["x"] = x
            out.append(r)
        return out
    return chain


def _mutant_linear_token(mod):
    def linear_token(W, V, M, x, eps, mode=0):
        g = mod.project(V, x)
        r = mod.residual(V, x, g)
        rho = mod.residual_ratio(x, r)
        slow = mod.takes_slow_path(rho, eps, mode)
        return {"g": g, "r": r, "rho": rho, "slow": slow, "y": mod.fast_output(M, g)}
    return linear_token


def _mutant_linear(mod, orig):
    def linear(W, V, M, X, eps, mode=0):
        out = orig(W, V, M, X, eps, mode)
        if len(out["y"]) > 1:
            out["y"] = out["y"].copy()
            out["y"][-1] = out["y"][-2]
        return out
    return linear


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = fresh_oracle()
    attr, fn = MUTANTS[name]
    if name == "slow_uses_image":
        fn = _mutant_linear_token(mod)
    elif name == "batch_drops_token":
        fn = _mutant_linear(mod, mod.linear)
    elif name.startswith("storage_"):
        fn = _mutant_to_storage(mod, {"storage_truncates": "trunc", "storage_ties_away": "away",
                                      "storage_bf16_as_fp32": "as_fp32"}[name])
    elif name.startswith("dgks_"):
        fn = _mutant_dgks("unnormalised" if name == "dgks_unnormalised" else "single")
    elif name == "iteration_one_sided":
        fn = _mutant_iteration(mod)
    elif name.startswith("batch_gate_"):
        fn = _mutant_gate_batch({"batch_gate_drop_column": "drop", "batch_gate_squared": "squared",
                                 "batch_gate_no_zero_guard": "noguard", "batch_gate_tie_fast": "tie",
                                 "batch_gate_ignores_modes": "modes"}[name])
    elif name.startswith("chain_"):
        fn = _mutant_chain(mod, {"chain_unrounded_input": "unrounded", "chain_ignores_offset": "no_offset",
                                 "chain_reads_previous_call": "previous"}[name])
    setattr(mod, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in ALL_PINS:
            try:
                pin(mod)
            except Exception as e:  # noqa: BLE001 - any failure counts as caught
                caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} survived every pin"


def test_unmutated_copy_passes():
    mod = fresh_oracle()
    for pin in ALL_PINS:
        pin(mod)
