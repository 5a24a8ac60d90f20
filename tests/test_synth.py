"""Properties of the seeded input generator (CPU only)."""
import math

import numpy as np
import torch

from rank_gated_memory_amd import synth


def test_seeds_are_deterministic_and_distinct():
    assert synth.seed_for(1, 2, 3, 4) == synth.seed_for(1, 2, 3, 4)
    assert synth.seed_for(1, 2, 3, 4) != synth.seed_for(1, 2, 3, 5)
    a = synth.gaussian_weight(8, 16, (1, 0, 0, 0), dtype=torch.float32)
    b = synth.gaussian_weight(8, 16, (1, 0, 0, 0), dtype=torch.float32)
    assert torch.equal(a, b)


def test_frame_is_orthonormal():
    v, u = synth.orthonormal_frame(256, 16, 64, (1, 0, 0, synth.P_BASIS))
    q = torch.cat([v, u], 1)
    assert torch.allclose(q.T @ q, torch.eye(80, dtype=torch.float64), atol=1e-12)


def test_weight_scale():
    w = synth.gaussian_weight(512, 1024, (7, 0, 0, 0), dtype=torch.float32).double()
    assert abs(float(w.var()) * 1024 - 1.0) < 0.02


def test_exact_slow_count():
    m = synth.pick_slow(1000, 50, (2, 0, 0, synth.P_PICK))
    assert int(m.sum()) == 50
    m2 = synth.pick_slow(512, round(0.05 * 512), (3, 0, 0, synth.P_PICK))
    assert int(m2.sum()) == 26


def test_config1_shapes_and_dtypes():
    c = synth.config1()
    assert c.W.shape == (512, 256) and c.W.dtype == torch.float32
    assert c.V.shape == (256, 16) and c.X.shape == (32, 256)
    assert int(c.slow_mask.sum()) == 8
    rb = c.rho_built[c.slow_mask]
    assert bool(((rb >= 0.1) & (rb <= 0.5)).all())


def test_cascade_coherence():
    fr = synth.cascade_frames(1024, 64, 16, 4, (3, 0, 0, synth.P_CASCADE))
    for (v1, _), (v2, u2) in zip(fr[:-1], fr[1:]):
        c = synth.mean_principal_cosine(v1, v2)
        assert 0.90 < c < 0.995, c
        q = torch.cat([v2, u2], 1)
        assert torch.allclose(q.T @ q, torch.eye(80, dtype=torch.float64), atol=1e-12)


def test_cascade_coherence_at_full_width():
    # GPT-J-shaped roles: d=4096, k=256 and d=16384, k=512 (two layers each)
    for d, k in ((4096, 256),):
        fr = synth.cascade_frames(d, k, 64, 2, (3, 0, 9, synth.P_CASCADE))
        c = synth.mean_principal_cosine(fr[0][0], fr[1][0])
        assert 0.90 < c < 0.99, c


def test_spectral_tokens_follow_the_power_law():
    """Energy of the spectral tokens along the frame: E[(v_i^T x)^2] = i^-2 alpha on
    the head directions, the tail directions carry the remaining mass, and the
    outlier share is near the requested rate."""
    d, K, m, n, alpha = 512, 64, 64, 6000, 1.1
    v, u = synth.orthonormal_frame(d, K, m, (97, 1, 2, 3))
    X, out = synth.spectral_tokens(v, u, n, (97, 1, 2), alpha=alpha)
    assert X.shape == (n, d) and X.dtype == torch.float64
    assert abs(float(out.double().mean()) - 0.05) < 0.015
    keep = ~out
    head = ((X[keep] @ v) ** 2).mean(0)
    want = torch.arange(1, K + 1, dtype=torch.float64).pow(-2 * alpha)
    assert torch.allclose(head, want, rtol=0.12)
    tail = ((X[keep] @ u) ** 2).sum(1).mean()
    want_tail = torch.arange(K + 1, d + 1, dtype=torch.float64).pow(-2 * alpha).sum()
    assert abs(float(tail / want_tail) - 1.0) < 0.05
    # the part outside span([v | u]) is empty
    resid = X - (X @ v) @ v.T - (X @ u) @ u.T
    assert float(resid.norm() / X.norm()) < 1e-12


def test_subspace_map_carries_subspace_and_keeps_ratio():
    d_in, d_out, k_in, k_out = 256, 384, 16, 24
    v_in, u_in = synth.orthonormal_frame(d_in, k_in, 64, (8, 0, 0, 1))
    v_out, _ = synth.orthonormal_frame(d_out, k_out, 0, (8, 0, 0, 2))
    W = synth.subspace_map(v_in, v_out, (8, 0, 0, 3), dtype=torch.float32).double()
    # the basis of the input lands inside the basis of the output
    img = W @ v_in
    assert torch.linalg.matrix_norm(img - v_out @ (v_out.T @ img)) < 1e-5 * torch.linalg.matrix_norm(img)
    # tokens keep their residual ratio approximately
    mask = torch.tensor([False] * 20 + [True] * 20)
    X, rho_built = synth.tokens(v_in, u_in, mask, (8, 0, 0))
    Y = X @ W.T
    rho_in = torch.linalg.vector_norm(X - (X @ v_in) @ v_in.T, dim=1) / torch.linalg.vector_norm(X, dim=1)
    rho_out = torch.linalg.vector_norm(Y - (Y @ v_out) @ v_out.T, dim=1) / torch.linalg.vector_norm(Y, dim=1)
    ratio = rho_out / rho_in
    assert float(ratio.min()) > 0.5 and float(ratio.max()) < 2.0, ratio
