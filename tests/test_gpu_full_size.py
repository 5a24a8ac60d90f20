"""GPU parity at full size, in the launch configuration bench.py times.

* 28-layer GPT-J-6B-shaped stack (112 maps per step, cascaded bases, 5 % slow)
  and 40-layer 13B-shaped stack (200 maps per step, 2 % slow): for sampled
  decode steps every call's gate is checked against the oracle, and every
  call's output on sampled rows (row i of the fast output only needs row i
  of M = W V_k, which the oracle forms from row i of W).
* Batched map T=256, d=4096 -> 16384, k in {64, 256, 512} x slow share in
  {0, 10, 50, 100} %: every gate, every token on sampled rows, and the full
  output of a few tokens.
"""
import numpy as np
import pytest
import torch

from oracle import gsi_oracle as orc
from rank_gated_memory_amd import gsi, synth
from tests.parity import compare_tokens, f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ROWS = 64


def rows_for(d_out, key):
    g = torch.Generator().manual_seed(key)
    return torch.randperm(d_out, generator=g)[:ROWS].sort().values.numpy()


def run_stack(name, sample_steps):
    cfg, layers, roles, steps, rate, cascade = synth.STACKS[name]
    data = synth.stack_config(cfg, layers, roles, steps, rate, device=DEV, cascade=cascade)
    maps = [[gsi.Map(mi.W, mi.V) for mi in row] for row in data]
    for row in maps:
        for m in row:
            gsi.gsi_prepare(m)
    results = {}
    ws = None
    for s in sample_steps:
        calls, outs = [], []
        for row, mrow in zip(data, maps):
            for mi, m in zip(row, mrow):
                y = torch.empty(mi.d_out, dtype=torch.bfloat16, device=DEV)
                r = torch.empty(1, dtype=torch.float32, device=DEV)
                sl = torch.empty(1, dtype=torch.uint8, device=DEV)
                calls.append((m, mi.X[s], y, 0.05, r, sl))
                outs.append((mi, y, r, sl))
        st = gsi.Stack(calls, device=DEV)
        if ws is None:
            ws = gsi.workspace(st.ws_bytes, DEV)
        st.run(ws=ws)
        torch.cuda.synchronize()
        results[s] = [(mi, y.cpu(), float(r.item()), int(sl.item())) for mi, y, r, sl in outs]
    return data, results


def check_stack(name, sample_steps):
    data, results = run_stack(name, sample_steps)
    worst, band, slow_calls = 0.0, 0, 0
    cache = {}
    for s, outs in results.items():
        for i, (mi, y, rho, sl) in enumerate(outs):
            if i not in cache:
                rows = rows_for(mi.d_out, 1000 + i)
                W_rows = f64(mi.W[torch.as_tensor(rows, device=DEV)])
                V = f64(mi.V)
                cache[i] = (rows, W_rows, V, orc.prepare(W_rows, V))
            rows, W_rows, V, M_rows = cache[i]
            x = f64(mi.X[s])[None]
            w, b = compare_tokens(W_rows, V, x, 0.05, f64(y)[rows][None], np.array([sl]),
                                  np.array([rho]), torch.bfloat16, M=M_rows, rho_tol=2e-2,
                                  what=f"{name} step {s} call {i} ({mi.name})")
            worst, band, slow_calls = max(worst, w), band + b, slow_calls + sl
            # the constructed slow tokens are exactly the slow ones
            assert bool(sl) == bool(mi.slow_mask[s].item()), (s, i)
    print(f"{name}: steps {sample_steps}, slow calls {slow_calls}, worst rel L2 {worst:.2e}, band {band}")
    return slow_calls


def slow_heavy_steps(name, n):
    """Steps with the most slow calls (from the constructed masks), plus step 0."""
    cfg, layers, roles, steps, rate, cascade = synth.STACKS[name]
    counts = torch.zeros(steps, dtype=torch.int64)
    for layer in range(layers):
        for ridx in range(len(roles)):
            counts += synth.pick_slow(steps, int(round(rate * steps)), (cfg, layer, ridx, synth.P_PICK)).long()
    top = torch.argsort(counts, descending=True)[:n].tolist()
    return sorted(set([0] + top))


def test_gptj6b_28_layer_stack():
    steps = slow_heavy_steps("gptj6b-28L", 2)
    assert check_stack("gptj6b-28L", steps) > 0


def test_llama13b_40_layer_stack():
    steps = slow_heavy_steps("llama13b-40L", 1)
    assert check_stack("llama13b-40L", steps) > 0


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
                              torch.bfloat16, rho_tol=2e-2, what=f"T=256 k={k} slow={frac}")
    # full outputs of a few slow tokens (y = W x needs no image)
    W = f64(mi.W)
    for t in torch.nonzero(slow).flatten()[:3].tolist():
        ref = W @ X[t]
        err = np.linalg.norm(yg[t] - ref) / np.linalg.norm(ref)
        assert err <= 2e-2, (t, err)
    print(f"T=256 k={k} slow={frac}: worst rel L2 on sampled rows {worst:.2e}")
