"""GPU parity at full size, in the launch configuration bench.py times.

* 28-layer GPT-J-6B-shaped stack (112 maps per step, cascaded bases, 5 % slow,
  512 decode steps) and 40-layer 13B-shaped stack (200 maps per step, 2 %
  slow, 256 steps): every step runs, and every call's gate and rho are
  checked against the oracle (57,344 and 51,200 calls), and every call's
  output on 64 sampled rows (row i of the fast output only needs row i of
  M = W V_k, which the oracle forms from row i of W).
* Batched map T=256, d=4096 -> 16384, k in {64, 256, 512} x slow share in
  {0, 10, 50, 100} %: every gate, every token on sampled rows, and the full
  output of a few tokens.
"""
import numpy as np
import pytest
import torch

from oracle import gsi_oracle as orc
from rank_gated_memory_amd import gsi, synth
from tests.parity import GATE_BAND, TOL, check_norm_form_rho, compare_tokens, eps32, f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ROWS = 64


def rows_for(d_out, key):
    g = torch.Generator().manual_seed(key)
    return torch.randperm(d_out, generator=g)[:ROWS].sort().values.numpy()


def run_all_steps(name):
    """Every decode step of a stack workload through gsi_stack, one launch per
    step in step order (the bench's launch configuration).  Returns the
    inputs, each map's outputs [steps][d_out], rho [steps] and slow [steps],
    and the status word after the run."""
    cfg, layers, roles, steps, rate, cascade = synth.STACKS[name]
    data = synth.stack_config(cfg, layers, roles, steps, rate, device=DEV, cascade=cascade)
    maps = [[gsi.Map(mi.W, mi.V) for mi in row] for row in data]
    for row in maps:
        for m in row:
            gsi.gsi_prepare(m)
    outs = [[(torch.empty((steps, mi.d_out), dtype=torch.bfloat16, device=DEV),
              torch.full((steps,), -1.0, dtype=torch.float32, device=DEV),
              torch.full((steps,), 7, dtype=torch.uint8, device=DEV)) for mi in row] for row in data]
    ws = None
    st_word = 0
    for s in range(steps):
        calls = [(m, mi.X[s], Y[s], 0.05, R[s:s + 1], S[s:s + 1])
                 for row, mrow, orow in zip(data, maps, outs)
                 for mi, m, (Y, R, S) in zip(row, mrow, orow)]
        st = gsi.Stack(calls, device=DEV)
        if ws is None:
            ws = gsi.workspace(st.ws_bytes, DEV)
        st.run(ws=ws)
        if s == steps - 1:
            torch.cuda.synchronize()
            st_word = st.status(ws)
    torch.cuda.synchronize()
    return data, outs, st_word


def check_every_gate(name):
    """Every call of every step: the gate against the oracle (bit-exact
    outside the 1e-3 band), rho against the oracle's explicit ratio through
    the Gram term of the stored basis, and the output of every call on 64
    sampled rows (row i of M g needs only row i of W); the constructed slow
    tokens are exactly the slow ones."""
    data, outs, st_word = run_all_steps(name)
    assert st_word == 0, f"status word {st_word:#x}"
    eps = eps32(0.05)
    calls = worst = band = slow_calls = 0
    worst_rho2 = 0.0
    for l, (row, orow) in enumerate(zip(data, outs)):
        for i, (mi, (Y, R, S)) in enumerate(zip(row, orow)):
            V = f64(mi.V)
            X = f64(mi.X)
            ref = orc.gate_batch(V, X, eps)
            slow_g = S.cpu().numpy()
            rho_g = R.cpu().numpy().astype(np.float64)
            assert set(np.unique(slow_g)) <= {0, 1}, f"{name} layer {l} map {mi.name}: unwritten gate"
            slow_g = slow_g.astype(bool)
            diff = slow_g != ref["slow"]
            if diff.any():
                assert np.all(np.abs(ref["rho"][diff] - eps) < GATE_BAND), (
                    f"{name} layer {l} {mi.name}: gates differ outside the band at steps "
                    f"{np.nonzero(diff)[0][:8].tolist()}")
            band += int(diff.sum())
            E = orc.gram_deviation(V)
            nx2 = np.einsum("td,td->t", X, X)
            q = np.einsum("tk,kl,tl->t", ref["g"], E, ref["g"]) / nx2
            worst_rho2 = max(worst_rho2, check_norm_form_rho(rho_g, ref["rho"], q, f"{name} layer {l} {mi.name}"))
            assert np.array_equal(slow_g, mi.slow_mask.cpu().numpy()), f"{name} layer {l} {mi.name}"
            rows = rows_for(mi.d_out, 1000 + l * 16 + i)
            W_rows = f64(mi.W[torch.as_tensor(rows, device=DEV)])
            M_rows = orc.prepare(W_rows, V)
            # the oracle output of the path the GPU took (equal to the
            # oracle's own path outside the band)
            want = np.where(slow_g[:, None], X @ W_rows.T, ref["g"] @ M_rows.T)
            got = f64(Y)[:, rows]
            err = np.linalg.norm(got - want, axis=1) / np.linalg.norm(want, axis=1)
            assert err.max() <= TOL[torch.bfloat16], (
                f"{name} layer {l} {mi.name}: rel L2 {err.max():.3e} at step {int(np.argmax(err))}")
            worst = max(worst, float(err.max()))
            calls += X.shape[0]
            slow_calls += int(slow_g.sum())
    print(f"{name}: {calls} calls, {slow_calls} slow, band {band}, worst rel L2 {worst:.2e} "
          f"(64 rows per call), worst |rho^2 - (rho_oracle^2 - q)| {worst_rho2:.1e}")
    return calls, slow_calls, data, outs


def test_gptj6b_28_layer_stack_every_gate():
    calls, slow_calls, data, outs = check_every_gate("gptj6b-28L")
    assert calls == 28 * 4 * 512 and slow_calls == 28 * 4 * 26
    # complete outputs of the slow calls of one step (y = W x needs no image)
    s = int(torch.nonzero(data[3][0].slow_mask)[0])
    for row, orow in zip(data, outs):
        for mi, (Y, _, S) in zip(row, orow):
            if int(S[s].item()):
                ref = f64(mi.W) @ f64(mi.X[s])
                err = np.linalg.norm(f64(Y[s]) - ref) / np.linalg.norm(ref)
                assert err <= TOL[torch.bfloat16], (mi.name, err)


def test_llama13b_40_layer_stack_every_gate():
    calls, slow_calls, _, _ = check_every_gate("llama13b-40L")
    assert calls == 40 * 5 * 256 and slow_calls == 40 * 5 * 5


@pytest.mark.parametrize("k", [64, 256, 512])
@pytest.mark.parametrize("frac", [0.0, 0.1, 0.5, 1.0])
def test_batched_t256(k, frac):
    mi = synth.config5(k, frac, device=DEV, w_device=DEV)
    m = gsi.Map(mi.W, mi.V)
    gsi.gsi_prepare(m)
    y, rho, slow = gsi.gsi_linear(m, mi.X, 0.05)
    torch.cuda.synchronize()
    T = mi.X.shape[0]
    assert int(slow.sum()) == int(round(frac * T))
    assert torch.equal(slow.bool().cpu(), mi.slow_mask.cpu())
    rows = rows_for(mi.d_out, 77 + k)
    W_rows = f64(mi.W[torch.as_tensor(rows, device=DEV)])
    V, X = f64(mi.V), f64(mi.X)
    yg = f64(y)
    worst, _ = compare_tokens(W_rows, V, X, 0.05, yg[:, rows], slow.cpu().numpy(), f64(rho),
                              torch.bfloat16, rho_tol="norm", what=f"T=256 k={k} slow={frac}")
    # full outputs of a few slow tokens (y = W x needs no image)
    W = f64(mi.W)
    for t in torch.nonzero(slow).flatten()[:3].tolist():
        ref = W @ X[t]
        err = np.linalg.norm(yg[t] - ref) / np.linalg.norm(ref)
        assert err <= 2e-2, (t, err)
    print(f"T=256 k={k} slow={frac}: worst rel L2 on sampled rows {worst:.2e}")
