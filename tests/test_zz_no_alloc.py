"""gsi_linear_static (no caller workspace, nothing allocated by the library)
against gsi_linear with a caller workspace: same kernels, so the results are
bitwise identical; two calls in a row, the second with a smaller input, on
the batched path, the single-token path and fp32; sizes beyond the static
array are rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from rank_gated_memory_amd import gsi, synth
from tests.parity import compare_tokens, f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def inputs(d, d_out, k, T, n_slow, dtype, key):
    W = synth.gaussian_weight(d_out, d, (95, key, 0, 0), dtype=dtype)
    v, u = synth.orthonormal_frame(d, k, 16, (95, key, 0, 1))
    mask = torch.zeros(T, dtype=torch.bool)
    mask[torch.randperm(T, generator=torch.Generator().manual_seed(key))[:n_slow]] = True
    X, _ = synth.tokens(v, u, mask, (95, key, 2))
    m = gsi.Map(W.to(DEV), v.to(dtype).to(DEV))
    gsi.gsi_prepare(m)
    return m, W, v.to(dtype), X.to(dtype).to(DEV)


def same(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("dtype,shape,calls", [
    (torch.bfloat16, (4096, 4096, 256), [(256, 26), (40, 35)]),    # batched: wide/thin, then smaller
    (torch.bfloat16, (1024, 1000, 64), [(1, 0), (1, 1)]),           # single token, fast then slow
    (torch.bfloat16, (2048, 3000, 128), [(300, 40), (3, 1)]),       # ragged d_out, batched then thin
    (torch.float32, (256, 512, 16), [(32, 8), (5, 2)]),             # fp32 batch-1 kernels
])
def test_static_matches_workspace_call(dtype, shape, calls):
    d, d_out, k = shape
    for i, (T, n_slow) in enumerate(calls):
        m, W, V, X = inputs(d, d_out, k, T, n_slow, dtype, 10 * d + i)
        print(f"static scratch: dtype={dtype} d={d} d_out={d_out} k={k} T={T} slow={n_slow}", flush=True)
        ys, rs, ss = gsi.gsi_linear_static(m, X, 0.05)
        yw, rw, sw = gsi.gsi_linear(m, X, 0.05)
        torch.cuda.synchronize()
        assert same(ys, yw), "outputs differ from the workspace call"
        assert same(rs, rw) and same(ss, sw)
        assert int(ss.sum()) == n_slow
        compare_tokens(f64(W), f64(V), f64(X), 0.05, f64(ys), ss.cpu().numpy(), f64(rs), dtype,
                       rho_tol="norm" if dtype == torch.bfloat16 else 1e-4, what=f"static T={T}")


def test_static_forced_modes_and_repeat():
    m, W, V, X = inputs(4096, 16384, 256, 64, 6, torch.bfloat16, 7)
    # each static call against the workspace call on the same tokens (a batch
    # of 7 runs the row-streaming kernels, one of 64 the wide ones)
    x7 = X[:7].contiguous()
    for mode in (gsi.FORCE_SLOW, gsi.FORCE_FAST, gsi.GATED):
        a = gsi.gsi_linear_static(m, X, 0.05, mode=mode)
        b = gsi.gsi_linear_static(m, x7, 0.05, mode=mode)
        c = gsi.gsi_linear(m, X, 0.05, mode=mode)
        c7 = gsi.gsi_linear(m, x7, 0.05, mode=mode)
        torch.cuda.synchronize()
        assert same(a[0], c[0]) and same(a[1], c[1]) and same(a[2], c[2])
        assert same(b[0], c7[0]) and same(b[1], c7[1]) and same(b[2], c7[2])
        compare_tokens(f64(W), f64(V), f64(x7), 0.05, f64(b[0]), b[2].cpu().numpy(), f64(b[1]),
                       torch.bfloat16, mode=mode, rho_tol="norm", what=f"static T=7 mode {mode}")


def test_static_rejects_beyond_the_array():
    # T = 4096 tokens at d = 16384, k = 1024 needs far more than 64 MiB
    W = torch.empty((64, 16384), dtype=torch.bfloat16, device=DEV)
    V = torch.empty((16384, 1024), dtype=torch.bfloat16, device=DEV)
    m = gsi.Map(W, V)
    assert gsi.gsi_static_scratch_bytes() == 64 << 20
    assert gsi.gsi_linear_workspace(m, 4096) > gsi.gsi_static_scratch_bytes()
    x = torch.empty((4096, 16384), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gsi.GsiError) as e:
        gsi.gsi_linear_static(m, x, 0.05)
    assert e.value.status == 5
    assert gsi.lib().gsi_linear_static(ctypes.byref(m.struct), 0, 0, 0, ctypes.c_float(0.05), 0, 0, 0, 0) == 0
