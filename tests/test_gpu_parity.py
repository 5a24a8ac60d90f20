"""GPU parity of the HIP path against the fp64 oracle (calls go through the C ABI).

Workloads follow the GSI technical summary's experiments, made synthetic:
a small fp32 map (d=256 -> 512, k=16, 32 tokens, 8 with a large residual),
the four GPT-J-6B-shaped maps in bf16 (1000 batch-1 tokens each, 50 slow),
ragged stacks, and the edge cases of the gate.
"""
import numpy as np
import pytest
import torch

from oracle import gsi_oracle as orc
from rank_gated_memory_amd import gsi, synth
from tests.parity import compare_tokens, eps32, f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def sync():
    torch.cuda.synchronize()


def new_map(W, V):
    m = gsi.Map(W.to(DEV).contiguous(), V.to(DEV).contiguous())
    gsi.gsi_prepare(m)
    return m


# ---------------------------------------------------------------- prepare ----

@pytest.mark.parametrize("d,d_out,k,dtype", [
    (256, 512, 16, torch.float32), (264, 200, 24, torch.float32), (4096, 4096, 256, torch.bfloat16),
    (512, 72, 8, torch.bfloat16), (1024, 1000, 320, torch.bfloat16), (2048, 640, 640, torch.bfloat16),
])
def test_prepare_image(d, d_out, k, dtype):
    W = synth.gaussian_weight(d_out, d, (90, d, d_out, k), dtype=dtype)
    v, _ = synth.orthonormal_frame(d, k, 0, (90, d, k, 1))
    V = v.to(dtype)
    m = new_map(W, V)
    sync()
    got = f64(m.image_rows())
    want = orc.prepare(f64(W), f64(V))
    rel = np.linalg.norm(got - want, axis=1) / np.linalg.norm(want, axis=1)
    tol = 1e-6 if dtype == torch.float32 else 4e-3
    assert rel.max() <= tol, rel.max()
    # padding rows of the last tile are zero
    tiles = (d_out + 63) // 64
    full = m.M[: tiles * 64 * k * W.element_size()].view(dtype)
    full = full.view(tiles, k * W.element_size() // 16, 64, 16 // W.element_size())
    full = full.permute(0, 2, 1, 3).reshape(tiles * 64, k)
    assert torch.all(full[d_out:] == 0)


# --------------------------------------------------------------- config 1 ----

def test_config1_single_tokens_and_batch():
    c = synth.config1()
    m = new_map(c.W, c.V)
    X = c.X.to(DEV)
    W, V, X64 = f64(c.W), f64(c.V), f64(c.X)
    # batched: all 32 tokens in one call
    y, rho, slow = gsi.gsi_linear(m, X, 0.05)
    sync()
    assert int(slow.sum()) == 8
    compare_tokens(W, V, X64, 0.05, f64(y), slow.cpu().numpy(), f64(rho), torch.float32,
                   rho_tol=1e-4, what="config1 batch")
    # one token per call
    ys, rhos, slows = [], [], []
    for t in range(X.shape[0]):
        y1, r1, s1 = gsi.gsi_linear(m, X[t:t + 1], 0.05)
        ys.append(y1)
        rhos.append(r1)
        slows.append(s1)
    sync()
    y1 = torch.cat(ys)
    compare_tokens(W, V, X64, 0.05, f64(y1), torch.cat(slows).cpu().numpy(), f64(torch.cat(rhos)),
                   torch.float32, rho_tol=1e-4, what="config1 T=1")
    # batching invariance
    assert torch.equal(torch.cat(slows), slow)
    assert torch.allclose(y1, y, rtol=1e-5, atol=1e-6)


# --------------------------------------------------------------- config 2 ----

GPTJ = {name: (d, d_out, k) for name, d, d_out, k in synth.GPTJ_MAPS}


@pytest.fixture(scope="module")
def config2_maps():
    return synth.config2(T=1000, device=DEV, w_device=DEV)


@pytest.mark.parametrize("idx", range(4), ids=[n for n, *_ in synth.GPTJ_MAPS])
def test_config2_map(config2_maps, idx):
    mi = config2_maps[idx]
    m = new_map(mi.W, mi.V)
    y, rho, slow = gsi.gsi_linear(m, mi.X, 0.05)
    sync()
    assert int(slow.sum()) == 50, int(slow.sum())
    assert torch.equal(slow.bool().cpu(), mi.slow_mask.cpu())
    W, V, X = f64(mi.W), f64(mi.V), f64(mi.X)
    M = orc.prepare(W, V)
    worst, band = compare_tokens(W, V, X, 0.05, f64(y), slow.cpu().numpy(), f64(rho),
                                 torch.bfloat16, M=M, rho_tol="norm", what=f"config2 {mi.name}")
    # 20 tokens one call each (batch-1 decode), incl. slow ones
    pick = torch.cat([torch.nonzero(mi.slow_mask).flatten()[:5],
                      torch.nonzero(~mi.slow_mask).flatten()[:15]]).cpu()
    ys, ss, rs = [], [], []
    for t in pick.tolist():
        a, b, c = gsi.gsi_linear(m, mi.X[t:t + 1], 0.05)
        ys.append(a)
        rs.append(b)
        ss.append(c)
    sync()
    compare_tokens(W, V, X[pick.numpy()], 0.05, f64(torch.cat(ys)), torch.cat(ss).cpu().numpy(),
                   f64(torch.cat(rs)), torch.bfloat16, M=M, rho_tol="norm", what=f"config2 {mi.name} T=1")
    print(f"{mi.name}: worst rel L2 {worst:.2e}, band tokens {band}")


def test_config2_stack(config2_maps):
    """The four maps x 8 tokens as one 32-call stack equals the oracle per call."""
    maps = [new_map(mi.W, mi.V) for mi in config2_maps]
    calls, outs = [], []
    for t in range(8):
        for mi, m in zip(config2_maps, maps):
            y = torch.empty(mi.d_out, dtype=torch.bfloat16, device=DEV)
            r = torch.empty(1, dtype=torch.float32, device=DEV)
            s = torch.empty(1, dtype=torch.uint8, device=DEV)
            calls.append((m, mi.X[t], y, 0.05, r, s))
            outs.append((mi, t, y, r, s))
    st = gsi.Stack(calls)
    ws = st.run()
    sync()
    for mi in config2_maps:
        W, V = f64(mi.W), f64(mi.V)
        M = orc.prepare(W, V)
        sel = [(t, y, r, s) for (mm, t, y, r, s) in outs if mm is mi]
        X = f64(mi.X[[t for t, *_ in sel]])
        compare_tokens(W, V, X, 0.05, np.stack([f64(y) for _, y, _, _ in sel]),
                       np.array([int(s.item()) for *_, s in sel]),
                       np.array([float(r.item()) for _, _, r, _ in sel]), torch.bfloat16, M=M,
                       rho_tol="norm", what=f"stack {mi.name}")
    # the workspace counters are back at zero: a second run gives identical bits
    y0 = [o[2].clone() for o in outs]
    st.run(ws=ws)
    sync()
    for (mi, t, y, r, s), yy in zip(outs, y0):
        assert torch.equal(y, yy)


# ------------------------------------------------------- ragged stacks -------

def ragged_stack_inputs(dtype, seed):
    shapes = [(264, 200, 24), (512, 72, 8), (1024, 1000, 64), (256, 8, 256), (2048, 1096, 128),
              (776, 520, 40)]
    items = []
    for i, (d, d_out, k) in enumerate(shapes):
        W = synth.gaussian_weight(d_out, d, (91, seed, i, 0), dtype=dtype)
        v, u = synth.orthonormal_frame(d, k, min(16, d - k) if d > k else 0, (91, seed, i, 1))
        if u.shape[1] == 0:
            u = torch.zeros((d, 1), dtype=torch.float64)
        mask = torch.tensor([i % 2 == 1 and d > k])
        X, _ = synth.tokens(v, u, mask, (91, seed, i))
        items.append((W, v.to(dtype), X.to(dtype)))
    return items


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_ragged_stack(dtype):
    items = ragged_stack_inputs(dtype, 1)
    calls, keep = [], []
    for W, V, X in items:
        m = new_map(W, V)
        y = torch.empty(W.shape[0], dtype=dtype, device=DEV)
        r = torch.empty(1, dtype=torch.float32, device=DEV)
        s = torch.empty(1, dtype=torch.uint8, device=DEV)
        xd = X[0].to(DEV)
        calls.append((m, xd, y, 0.05, r, s))
        keep.append((W, V, X, y, r, s))
    st = gsi.Stack(calls)
    st.run()
    sync()
    for i, (W, V, X, y, r, s) in enumerate(keep):
        compare_tokens(f64(W), f64(V), f64(X[:1]), 0.05, f64(y)[None], np.array([int(s.item())]),
                       np.array([float(r.item())]), dtype, rho_tol="norm", what=f"ragged {i}")


# ------------------------------------------------------------ edge cases -----

def small_map(dtype=torch.bfloat16, d=512, d_out=328, k=32, seed=5):
    W = synth.gaussian_weight(d_out, d, (92, seed, 0, 0), dtype=dtype)
    v, u = synth.orthonormal_frame(d, k, 16, (92, seed, 0, 1))
    return W, v, u


def test_zero_nan_and_thresholds():
    W, v, u = small_map()
    V = v.to(torch.bfloat16)
    m = new_map(W, V)
    X, _ = synth.tokens(v, u, torch.tensor([False, True, False, False]), (92, 5, 0))
    X = X.to(torch.bfloat16)
    X[2] = 0
    X[3, 7] = float("nan")
    Xd = X.to(DEV)
    y, rho, slow = gsi.gsi_linear(m, Xd, 0.05)
    sync()
    assert slow.tolist() == [0, 1, 0, 1]
    assert rho[2].item() == 0.0 and torch.all(y[2] == 0)
    assert torch.isnan(rho[3]) and not torch.isfinite(y[3]).all()
    compare_tokens(f64(W), f64(V), f64(X), 0.05, f64(y), slow.cpu().numpy(), f64(rho),
                   torch.bfloat16, what="edge")
    # eps <= 0: every token slow (x = 0 included, its output is still 0)
    _, _, s0 = gsi.gsi_linear(m, Xd, 0.0)
    # eps > 1: every finite token fast
    y2, _, s2 = gsi.gsi_linear(m, Xd, 2.0)
    sync()
    assert s0.tolist() == [1, 1, 1, 1]
    assert s2.tolist() == [0, 0, 0, 1]
    compare_tokens(f64(W), f64(V), f64(X), 2.0, f64(y2), s2.cpu().numpy(), np.zeros(4),
                   torch.bfloat16, what="eps>1")


def nonfinite_tokens(v, u, n_bad, n_good, seed):
    """n_bad tokens holding +Inf, -Inf or NaN in one element (cycling), then
    n_good ordinary fast tokens."""
    X, _ = synth.tokens(v, u, torch.zeros(n_bad + n_good, dtype=torch.bool), (92, seed, 1))
    X = X.to(torch.bfloat16)
    bad = (float("inf"), float("-inf"), float("nan"))
    for t in range(n_bad):
        X[t, (37 * t + 3) % X.shape[1]] = bad[t % 3]
    return X


@pytest.mark.parametrize("path", ["single", "batched-thin", "batched-wide", "stack"])
def test_nonfinite_tokens_every_path(path):
    """+Inf, -Inf and NaN tokens: rho NaN, slow path, outputs not finite
    (the oracle's reading), on every entry point that gates a token; the
    ordinary tokens around them are unaffected."""
    W, v, u = small_map(seed=9)
    V = v.to(torch.bfloat16)
    m = new_map(W, V)
    n_bad, n_good = {"single": (3, 2), "batched-thin": (6, 5), "batched-wide": (36, 6), "stack": (6, 3)}[path]
    X = nonfinite_tokens(v, u, n_bad, n_good, 11)
    T = X.shape[0]
    Xd = X.to(DEV)
    if path == "single":
        outs = [gsi.gsi_linear(m, Xd[t:t + 1], 0.05) for t in range(T)]
        y = torch.cat([o[0] for o in outs])
        rho = torch.cat([o[1] for o in outs])
        slow = torch.cat([o[2] for o in outs])
    elif path == "stack":
        y = torch.empty((T, W.shape[0]), dtype=torch.bfloat16, device=DEV)
        rho = torch.empty(T, dtype=torch.float32, device=DEV)
        slow = torch.empty(T, dtype=torch.uint8, device=DEV)
        st = gsi.Stack([(m, Xd[t], y[t], 0.05, rho[t:t + 1], slow[t:t + 1]) for t in range(T)])
        ws = st.run()
        sync()
        assert st.status(ws) == 0
    else:
        y, rho, slow = gsi.gsi_linear(m, Xd, 0.05)
    sync()
    assert slow.tolist() == [1] * n_bad + [0] * n_good, slow.tolist()
    assert torch.isnan(rho[:n_bad]).all()
    assert not torch.isfinite(y[:n_bad]).all(dim=1).any()
    compare_tokens(f64(W), f64(V), f64(X), 0.05, f64(y), slow.cpu().numpy(), f64(rho),
                   torch.bfloat16, rho_tol="norm", what=f"non-finite {path}")


def test_forced_modes_and_full_rank():
    W, v, u = small_map(torch.float32, d=256, d_out=136, k=256 - 16)
    V = v.to(torch.float32)
    m = new_map(W, V)
    X, _ = synth.tokens(v, u, torch.tensor([False, True, True]), (92, 6, 0))
    X = X.to(torch.float32)
    Xd = X.to(DEV)
    for mode in (gsi.FORCE_FAST, gsi.FORCE_SLOW):
        y, rho, slow = gsi.gsi_linear(m, Xd, 0.05, mode=mode)
        sync()
        assert slow.tolist() == ([0, 0, 0] if mode == gsi.FORCE_FAST else [1, 1, 1])
        compare_tokens(f64(W), f64(V), f64(X), 0.05, f64(y), slow.cpu().numpy(), f64(rho),
                       torch.float32, mode=mode, what=f"mode {mode}")
    # k = d: every token lies in the subspace; the fast output equals W x
    Wf = synth.gaussian_weight(64, 128, (92, 7, 0, 0), dtype=torch.float32)
    vf, _ = synth.orthonormal_frame(128, 128, 0, (92, 7, 0, 1))
    mf = new_map(Wf, vf.to(torch.float32))
    Xf = torch.randn(5, 128, generator=synth.generator("cpu", 92, 7, 0, 2)).to(torch.float32)
    y, rho, slow = gsi.gsi_linear(mf, Xf.to(DEV), 0.05)
    sync()
    assert slow.tolist() == [0] * 5 and float(rho.max()) < 1e-3
    ref = f64(Xf) @ f64(Wf).T
    assert np.allclose(f64(y), ref, rtol=1e-4, atol=1e-4)


def test_determinism_and_workspace_reuse():
    W, v, u = small_map(d=2048, d_out=1000, k=128)
    V = v.to(torch.bfloat16)
    m = new_map(W, V)
    mask = torch.zeros(64, dtype=torch.bool)
    mask[::7] = True
    X, _ = synth.tokens(v, u, mask, (92, 8, 0))
    Xd = X.to(torch.bfloat16).to(DEV)
    ws = gsi.workspace(gsi.gsi_linear_workspace(m, 64), DEV)
    a = gsi.gsi_linear(m, Xd, 0.05, ws=ws)
    b = gsi.gsi_linear(m, Xd, 0.05, ws=ws)
    sync()
    for p, q in zip(a, b):
        assert torch.equal(p.view(torch.uint8), q.view(torch.uint8))
    assert torch.equal(a[2].bool().cpu(), mask)


def test_empty_batch_is_noop():
    W, v, _ = small_map()
    m = new_map(W, v.to(torch.bfloat16))
    y = torch.full((0, W.shape[0]), 7.0, dtype=torch.bfloat16, device=DEV)
    x = torch.empty((0, W.shape[1]), dtype=torch.bfloat16, device=DEV)
    out = gsi.gsi_linear(m, x, 0.05, y=y)
    sync()
    assert out[0].shape == (0, W.shape[0])


def test_many_tokens_multiple_launches():
    """More tokens than one launch takes (4096): split launches, same results."""
    W = synth.gaussian_weight(64, 64, (93, 0, 0, 0), dtype=torch.float32)
    v, u = synth.orthonormal_frame(64, 8, 16, (93, 0, 0, 1))
    mask = torch.zeros(5000, dtype=torch.bool)
    mask[::10] = True
    X, _ = synth.tokens(v, u, mask, (93, 0, 0))
    X = X.to(torch.float32)
    m = new_map(W, v.to(torch.float32))
    y, rho, slow = gsi.gsi_linear(m, X.to(DEV), 0.05)
    sync()
    assert torch.equal(slow.bool().cpu(), mask)
    sel = np.r_[0:40, 4090:4110, 4980:5000]
    compare_tokens(f64(W), f64(v.to(torch.float32)), f64(X)[sel], 0.05, f64(y)[sel],
                   slow.cpu().numpy()[sel], f64(rho)[sel], torch.float32, what="T=5000")


# ------------------------------------------------------ batched (MFMA) path ---

@pytest.mark.parametrize("d,d_out,k,T", [
    (264, 200, 24, 2),       # smallest batch, ragged shapes, k not a multiple of 16
    (512, 72, 8, 3),         # k = 8, d_out below one 64-column tile
    (2048, 1096, 128, 97),   # ragged T and d_out
    (776, 520, 40, 300),     # T beyond one 256-token pass
    (256, 136, 256, 33),     # k = d
])
def test_batched_ragged(d, d_out, k, T):
    W = synth.gaussian_weight(d_out, d, (94, d, d_out, k), dtype=torch.bfloat16)
    extra = min(16, d - k)
    v, u = synth.orthonormal_frame(d, k, extra, (94, d, k, 1))
    if extra == 0:
        u = torch.zeros((d, 1), dtype=torch.float64)
    mask = torch.zeros(T, dtype=torch.bool)
    if extra:
        mask[1::3] = True
    X, _ = synth.tokens(v, u, mask, (94, d, k))
    X = X.to(torch.bfloat16)
    V = v.to(torch.bfloat16)
    m = new_map(W, V)
    for mode in (gsi.GATED, gsi.FORCE_FAST, gsi.FORCE_SLOW):
        y, rho, slow = gsi.gsi_linear(m, X.to(DEV), 0.05, mode=mode)
        sync()
        if mode == gsi.GATED:
            assert torch.equal(slow.bool().cpu(), mask)
        compare_tokens(f64(W), f64(V), f64(X), 0.05, f64(y), slow.cpu().numpy(), f64(rho),
                       torch.bfloat16, mode=mode, rho_tol="norm", what=f"batched {d},{d_out},{k},T={T},mode={mode}")


def test_batched_matches_single_token_calls():
    """A token's output does not depend on the batch it is in (batch vs. T=1 kernels)."""
    W, v, u = small_map(d=1024, d_out=640, k=64, seed=9)
    V = v.to(torch.bfloat16)
    m = new_map(W, V)
    mask = torch.zeros(40, dtype=torch.bool)
    mask[::4] = True
    X, _ = synth.tokens(v, u, mask, (92, 9, 0))
    Xd = X.to(torch.bfloat16).to(DEV)
    yb, rb, sb = gsi.gsi_linear(m, Xd, 0.05)
    ys = torch.cat([gsi.gsi_linear(m, Xd[t:t + 1], 0.05)[0] for t in range(40)])
    sync()
    assert torch.equal(sb.bool().cpu(), mask)
    err = (yb.double() - ys.double()).norm(dim=1) / ys.double().norm(dim=1)
    assert float(err.max()) < 1e-2


def test_batched_many_tokens_multiple_launches():
    """More tokens than one batched launch takes (4096)."""
    W = synth.gaussian_weight(96, 128, (95, 0, 0, 0), dtype=torch.bfloat16)
    v, u = synth.orthonormal_frame(128, 16, 16, (95, 0, 0, 1))
    mask = torch.zeros(4500, dtype=torch.bool)
    mask[::9] = True
    X, _ = synth.tokens(v, u, mask, (95, 0, 0))
    X = X.to(torch.bfloat16)
    V = v.to(torch.bfloat16)
    m = new_map(W, V)
    y, rho, slow = gsi.gsi_linear(m, X.to(DEV), 0.05)
    sync()
    assert torch.equal(slow.bool().cpu(), mask)
    sel = np.r_[0:30, 4080:4110, 4470:4500]
    compare_tokens(f64(W), f64(V), f64(X)[sel], 0.05, f64(y)[sel], slow.cpu().numpy()[sel],
                   f64(rho)[sel], torch.bfloat16, what="batched T=4500")


@pytest.mark.parametrize("T,n_slow", [(65, 32), (65, 33), (33, 0), (33, 33), (32, 32), (1, 1), (40, 20), (64, 32)])
def test_batched_thin_and_wide_kernels(T, n_slow):
    """A path with at most 32 tokens streams its matrix by rows, a larger one
    runs the wide items: both sides of that boundary, for both paths, and
    both paths streaming by rows in one call (T = 40 and 64: the output
    launch's row-stream items switch from the fast to the slow path), with
    d_out not a multiple of 16 (an odd number of row blocks: the last pair's
    second block lies past d_out) and k not a multiple of 32."""
    d, d_out, k = 1024, 200, 40
    W = synth.gaussian_weight(d_out, d, (97, T, n_slow, 0), dtype=torch.bfloat16)
    v, u = synth.orthonormal_frame(d, k, 16, (97, T, n_slow, 1))
    g = torch.Generator().manual_seed(97 * T + n_slow)
    mask = torch.zeros(T, dtype=torch.bool)
    mask[torch.randperm(T, generator=g)[:n_slow]] = True
    X, _ = synth.tokens(v, u, mask, (97, T, n_slow))
    X = X.to(torch.bfloat16)
    V = v.to(torch.bfloat16)
    m = new_map(W, V)
    y, rho, slow = gsi.gsi_linear(m, X.to(DEV), 0.05)
    sync()
    assert torch.equal(slow.bool().cpu(), mask)
    compare_tokens(f64(W), f64(V), f64(X), 0.05, f64(y), slow.cpu().numpy(), f64(rho),
                   torch.bfloat16, rho_tol="norm", what=f"batched T={T} slow={n_slow}")


@pytest.mark.parametrize("k", [128, 256])
@pytest.mark.parametrize("eps", [0.05, 0.10])
def test_spectral_tokens_operating_points(k, eps):
    """Power-law spectral tokens (the operating-point workload), nested bases:
    the gate is decided by the tokens' own residuals, many of them near eps.
    Batch-1 stack calls and the batched path, against the oracle."""
    d, d_out, T = 4096, 1000, 48
    v, u = synth.orthonormal_frame(d, 512, 256, (98, 0, 0, 1))
    X, _ = synth.spectral_tokens(v, u, T, (98, 0, 0))
    W = synth.gaussian_weight(d_out, d, (98, 0, 0, 0), dtype=torch.bfloat16)
    V = v[:, :k].to(torch.bfloat16)
    Xb = X.to(torch.bfloat16)
    m = new_map(W, V)
    Wf, Vf, Xf = f64(W), f64(V), f64(Xb)
    M = orc.prepare(Wf, Vf)
    # batched path
    y, rho, slow = gsi.gsi_linear(m, Xb.to(DEV), eps)
    sync()
    compare_tokens(Wf, Vf, Xf, eps, f64(y), slow.cpu().numpy(), f64(rho), torch.bfloat16, M=M,
                   rho_tol="norm", what=f"spectral batched k={k} eps={eps}")
    # batch-1: one stack of T single-token calls
    Xd = Xb.to(DEV)
    ys = torch.empty((T, d_out), dtype=torch.bfloat16, device=DEV)
    rs = torch.empty(T, dtype=torch.float32, device=DEV)
    ss = torch.empty(T, dtype=torch.uint8, device=DEV)
    st = gsi.Stack([(m, Xd[t], ys[t], eps, rs[t:t + 1], ss[t:t + 1]) for t in range(T)], device=DEV)
    st.run()
    sync()
    compare_tokens(Wf, Vf, Xf, eps, f64(ys), ss.cpu().numpy(), f64(rs), torch.bfloat16, M=M,
                   rho_tol="norm", what=f"spectral stack k={k} eps={eps}")
    share = 1.0 - float(ss.float().mean())
    print(f"k={k} eps={eps}: fast share {share:.2f}")
    assert 0.0 < share < 1.0 or eps == 0.10


# ------------------------------------------------ single launch vs phases ----

@pytest.mark.parametrize("n", [18, 4], ids=["18-calls", "4-calls"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_stack_single_launch_matches_two_phases(dtype, n):
    """gsi_stack (one persistent launch) gives the same bits as the two-launch
    form: 18 calls through the open list; 4 (one of them slow) through static
    output tickets, the form of a wave of at most four small calls."""
    items = (ragged_stack_inputs(dtype, 2) * 3)[:n]
    calls, outs = [], []
    for W, V, X in items:
        m = new_map(W, V)
        y = torch.empty(W.shape[0], dtype=dtype, device=DEV)
        r = torch.empty(1, dtype=torch.float32, device=DEV)
        s = torch.empty(1, dtype=torch.uint8, device=DEV)
        calls.append((m, X[0].to(DEV), y, 0.05, r, s))
        outs.append((y, r, s))
    st = gsi.Stack(calls)
    ws = gsi.workspace(st.ws_bytes, DEV)
    for mode in (gsi.GATED, gsi.FORCE_FAST, gsi.FORCE_SLOW):
        gsi.gsi_stack_phase(st, mode, gsi.PHASE_PROJECT, ws)
        gsi.gsi_stack_phase(st, mode, gsi.PHASE_APPLY, ws)
        sync()
        ref = [tuple(t.clone() for t in o) for o in outs]
        for o in outs:
            o[0].fill_(7)
        for _ in range(3):
            gsi.gsi_stack(st, mode, ws)
            sync()
            for (y, r, s), (y0, r0, s0) in zip(outs, ref):
                assert torch.equal(y, y0) and torch.equal(r, r0) and torch.equal(s, s0)
    assert st.status(ws) == 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_shared_projection_stack(dtype):
    """Calls reading one x with one basis share a projection (one set of
    projection units), yet each keeps its own threshold, gate and output:
    with rho ~ 0.029, eps = 0.05 takes the fast path and eps = 0.02 the slow
    one from the same rho.  Oracle parity, and the same bits as the
    two-launch form."""
    d, k = 512, 32
    v, u = synth.orthonormal_frame(d, k, 64, (93, 0, 0, 1))
    V = v.to(dtype).to(DEV).contiguous()
    mask = torch.tensor([False, True, False, False])
    X, _ = synth.tokens(v, u, mask, (93, 0, 0), rho_fast=0.03)
    Xd = X.to(dtype).to(DEV)
    outs_dims = (328, 200, 1000)
    epss = (0.05, 0.02, 0.05)
    maps = []
    for i, do in enumerate(outs_dims):
        W = synth.gaussian_weight(do, d, (93, 0, i, 2), dtype=dtype)
        m = gsi.Map(W.to(DEV), V)
        gsi.gsi_prepare(m)
        maps.append((m, W))
    calls, outs = [], []
    for t in range(4):
        for (m, W), eps in zip(maps, epss):
            y = torch.empty(m.d_out, dtype=dtype, device=DEV)
            r = torch.empty(1, dtype=torch.float32, device=DEV)
            s = torch.empty(1, dtype=torch.uint8, device=DEV)
            calls.append((m, Xd[t], y, eps, r, s))
            outs.append((t, W, eps, y, r, s))
    st = gsi.Stack(calls)
    ws = st.run()
    sync()
    Vf = f64(V)
    slow_seen = set()
    for t, W, eps, y, r, s in outs:
        compare_tokens(f64(W), Vf, f64(Xd[t:t + 1]), eps, f64(y)[None], np.array([int(s.item())]),
                       np.array([float(r.item())]), dtype, rho_tol="norm", what=f"shared t{t} eps{eps}")
        slow_seen.add((t, eps, int(s.item())))
    # one rho, two thresholds, two paths
    assert (0, 0.05, 0) in slow_seen and (0, 0.02, 1) in slow_seen
    assert st.status(ws) == 0
    ref = [o[3].clone() for o in outs]
    gsi.gsi_stack_phase(st, gsi.GATED, gsi.PHASE_PROJECT, ws)
    gsi.gsi_stack_phase(st, gsi.GATED, gsi.PHASE_APPLY, ws)
    sync()
    assert all(torch.equal(o[3], a) for o, a in zip(outs, ref))


# ------------------------------------------------ many projection units ----

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_many_projection_units(dtype):
    """Calls split into many projection units (d = 592: 37 units of 16
    rows; d = 536: 34 units, the last of 8 rows; d = 2048: 64 units of 32
    rows in a stack, 128 through gsi_linear, summed in two levels; d = 6400:
    100 (bf16) or 200 (fp32) units of 64 KiB in a stack, summed in two levels
    with a ragged last group).  Oracle parity through gsi_linear and through
    a stack of one call per wave, repeated runs on one workspace (the
    counters must return to zero), and the same bits from the two-launch
    form."""
    shapes = [(592, 200, 512), (536, 72, 512), (2048, 128, 512), (6400, 96, 512)]
    items = []
    for i, (d, d_out, k) in enumerate(shapes):
        W = synth.gaussian_weight(d_out, d, (95, 0, i, 0), dtype=dtype)
        v, u = synth.orthonormal_frame(d, k, 16, (95, 0, i, 1))
        mask = torch.tensor([False, True, False])
        X, _ = synth.tokens(v, u, mask, (95, 0, i))
        items.append((W, v.to(dtype), X.to(dtype)))
    maps = [new_map(W, V) for W, V, _ in items]
    for (W, V, X), m in zip(items, maps):
        Xd = X.to(DEV)
        lws = gsi.workspace(gsi.gsi_linear_workspace(m, 1), DEV)
        for _ in range(2):
            ys, rs, ss = [], [], []
            for t in range(X.shape[0]):
                y, r, s = gsi.gsi_linear(m, Xd[t:t + 1], 0.05, ws=lws)
                ys.append(y)
                rs.append(r)
                ss.append(s)
            sync()
            compare_tokens(f64(W), f64(V), f64(X), 0.05, f64(torch.cat(ys)), torch.cat(ss).cpu().numpy(),
                           f64(torch.cat(rs)), dtype, rho_tol="norm", what=f"linear d={W.shape[1]}")
    calls, outs = [], []
    for wave, ((W, V, X), m) in enumerate(zip(items, maps)):
        for t in range(X.shape[0]):
            y = torch.empty(W.shape[0], dtype=dtype, device=DEV)
            r = torch.empty(1, dtype=torch.float32, device=DEV)
            s = torch.empty(1, dtype=torch.uint8, device=DEV)
            calls.append((m, X[t].to(DEV), y, 0.05, r, s, wave))
            outs.append((W, V, X[t:t + 1], y, r, s))
    st = gsi.Stack(calls)
    ws = gsi.workspace(st.ws_bytes, DEV)
    ref = None
    for _ in range(3):
        gsi.gsi_stack(st, gsi.GATED, ws)
        sync()
        got = [tuple(t.clone() for t in o[3:]) for o in outs]
        if ref is None:
            ref = got
        assert all(all(torch.equal(a, b) for a, b in zip(g, r)) for g, r in zip(got, ref))
    for W, V, X, y, r, s in outs:
        compare_tokens(f64(W), f64(V), f64(X), 0.05, f64(y)[None], np.array([int(s.item())]),
                       np.array([float(r.item())]), dtype, rho_tol="norm", what=f"stack d={W.shape[1]}")
    assert st.status(ws) == 0
    # one wave (its unit sizes follow the whole wave's bytes): oracle parity,
    # and the single launch and the two-launch form give the same bits
    st1 = gsi.Stack([c[:6] for c in calls])
    ws1 = gsi.workspace(st1.ws_bytes, DEV)
    gsi.gsi_stack(st1, gsi.GATED, ws1)
    sync()
    one = [tuple(t.clone() for t in o[3:]) for o in outs]
    for W, V, X, y, r, s in outs:
        compare_tokens(f64(W), f64(V), f64(X), 0.05, f64(y)[None], np.array([int(s.item())]),
                       np.array([float(r.item())]), dtype, rho_tol="norm", what=f"one wave d={W.shape[1]}")
    for _ in range(2):
        gsi.gsi_stack_phase(st1, gsi.GATED, gsi.PHASE_PROJECT, ws1)
        gsi.gsi_stack_phase(st1, gsi.GATED, gsi.PHASE_APPLY, ws1)
        sync()
        two = [tuple(t.clone() for t in o[3:]) for o in outs]
        assert all(all(torch.equal(a, b) for a, b in zip(g, r)) for g, r in zip(two, one))
    assert st1.status(ws1) == 0


def test_stack_output_tickets_beyond_the_grid():
    """One wave of 48 calls (4 maps d = 1024 -> 8192, k = 64, x 12 tokens,
    every other one slow) whose output units (one 64-row image tile per fast
    unit, 128 rows of W per slow unit: several thousand) outnumber the
    workgroups many times over.  The eight ticket groups then run dry at
    different times and workgroups take tickets from other groups before
    they leave.  Every output row is written (y starts as NaN) and equals
    the oracle, and three runs on one workspace give the same bits with the
    status word 0."""
    dtype = torch.bfloat16
    d, d_out, k = 1024, 8192, 64
    items = []
    for i in range(4):
        W = synth.gaussian_weight(d_out, d, (97, 0, i, 0), dtype=dtype)
        v, u = synth.orthonormal_frame(d, k, 16, (97, 0, i, 1))
        mask = torch.tensor([t % 2 == 1 for t in range(12)])
        X, _ = synth.tokens(v, u, mask, (97, 0, i))
        items.append((W, v.to(dtype), X.to(dtype)))
    calls, outs = [], []
    for W, V, X in items:
        m = new_map(W, V)
        Xd = X.to(DEV)
        ys = torch.full((X.shape[0], d_out), float("nan"), dtype=dtype, device=DEV)
        rs = torch.empty(X.shape[0], dtype=torch.float32, device=DEV)
        ss = torch.empty(X.shape[0], dtype=torch.uint8, device=DEV)
        for t in range(X.shape[0]):
            calls.append((m, Xd[t], ys[t], 0.05, rs[t:t + 1], ss[t:t + 1]))
        outs.append((W, V, X, ys, rs, ss))
    st = gsi.Stack(calls)
    ws = gsi.workspace(st.ws_bytes, DEV)
    ref = None
    for _ in range(3):
        gsi.gsi_stack(st, gsi.GATED, ws)
        sync()
        assert st.status(ws) == 0
        got = [tuple(t.clone() for t in o[3:]) for o in outs]
        if ref is None:
            ref = got
        assert all(all(torch.equal(a, b) for a, b in zip(g, r)) for g, r in zip(got, ref))
    n_slow = 0
    for W, V, X, ys, rs, ss in outs:
        assert torch.isfinite(ys.float()).all(), "an output unit was never run"
        n_slow += int(ss.sum().item())
        compare_tokens(f64(W), f64(V), f64(X), 0.05, f64(ys), ss.cpu().numpy(), f64(rs), dtype,
                       rho_tol="norm", what="tickets beyond the grid")
    assert n_slow == 24


# ------------------------------------------------------------- maximum sizes -

@pytest.mark.parametrize("dtype,d,d_out,k", [
    (torch.bfloat16, 16384, 1032, 1024),   # d * 2 bytes = the 32 KiB row limit, k = the basis limit
    (torch.float32, 8192, 520, 1024),      # d * 4 bytes = the 32 KiB row limit
])
def test_maximum_sizes_every_entry_point(dtype, d, d_out, k):
    """The largest row (d * element size = 32 KiB) and basis (k = 1024) the
    library takes, through the single-token path, the batched path (bf16:
    a wide and a row-streaming output kernel; fp32: the batch-1 kernels) and
    a stack, against the oracle; every gate exact, every output within the
    bar."""
    W = synth.gaussian_weight(d_out, d, (97, d, k, 0), dtype=dtype)
    v, u = synth.orthonormal_frame(d, k, 16, (97, d, k, 1))
    mask = torch.zeros(48, dtype=torch.bool)
    mask[::6] = True  # 8 slow tokens (row stream), 40 fast (wide kernel)
    X, _ = synth.tokens(v, u, mask, (97, d, k))
    V = v.to(dtype)
    X = X.to(dtype)
    m = new_map(W, V)
    rt = "norm" if dtype == torch.bfloat16 else 1e-4
    Wf, Vf, Xf = f64(W), f64(V), f64(X)
    M = orc.prepare(Wf, Vf)
    Xd = X.to(DEV)
    y, rho, slow = gsi.gsi_linear(m, Xd, 0.05)
    sync()
    assert torch.equal(slow.bool().cpu(), mask)
    compare_tokens(Wf, Vf, Xf, 0.05, f64(y), slow.cpu().numpy(), f64(rho), dtype, M=M, rho_tol=rt,
                   what=f"max batched {d}x{k}")
    ys, rs, ss = zip(*[gsi.gsi_linear(m, Xd[t:t + 1], 0.05) for t in range(4)])
    sync()
    compare_tokens(Wf, Vf, Xf[:4], 0.05, np.concatenate([f64(a) for a in ys]), torch.cat(ss).cpu().numpy(),
                   f64(torch.cat(rs)), dtype, M=M, rho_tol=rt, what=f"max single {d}x{k}")
    Y = torch.empty((6, d_out), dtype=dtype, device=DEV)
    R = torch.empty(6, dtype=torch.float32, device=DEV)
    S = torch.empty(6, dtype=torch.uint8, device=DEV)
    st = gsi.Stack([(m, Xd[t], Y[t], 0.05, R[t:t + 1], S[t:t + 1]) for t in range(6)])
    st.run(check=True)
    compare_tokens(Wf, Vf, Xf[:6], 0.05, f64(Y), S.cpu().numpy(), f64(R), dtype, M=M, rho_tol=rt,
                   what=f"max stack {d}x{k}")
