"""GPU basis calibration (gsi_calibrate) against the oracle's subspace
iteration with DGKS orthonormalisation (GSI-TS §2.3).

Both sides run the same sweeps V <- orth(A^T (A V)) from the same start; the
Q factor with a positive diagonal is unique, so the GPU basis (CholeskyQR2
in fp64, products with A in fp32) is compared with the oracle's column by
column.  Samples are synthetic: a planted k-dimensional head with a
spectral gap over a tail, as a calibration pass would give for a layer whose
activations lie near a subspace.
"""
import numpy as np
import pytest
import torch

from oracle import gsi_oracle as orc
from rank_gated_memory_amd import gsi, synth
from tests.parity import f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def sync():
    torch.cuda.synchronize()


def samples(d, k, n, key, gap=4.0, tail=64, frame=None):
    if frame is None:
        v, u = synth.orthonormal_frame(d, k, tail, key + (1,))
        frame = torch.cat([v, u], 1)
    spec = torch.cat([torch.linspace(2.0 * gap, gap, k, dtype=torch.float64),
                      torch.linspace(1.0, 0.2, frame.shape[1] - k, dtype=torch.float64)])
    return synth.frame_samples(frame, spec, n, key + (2,)), frame


@pytest.mark.parametrize("n,d,k,dtype,iters,tol", [
    (1024, 256, 16, torch.float32, 3, 2e-4),
    (600, 520, 40, torch.float32, 1, 2e-4),
    (2048, 4096, 256, torch.bfloat16, 3, 2e-2),
    # bf16 samples, d a multiple of 8 (matrix-core products) with n, d and k
    # all off the 64-wide tiles, so every zero-padded edge is used
    (600, 520, 40, torch.bfloat16, 2, 2e-2),
    # bf16 samples with the padded sample count at most d: Z^T = V^T A^T is
    # summed over two halves of K (the second ending inside a 64-wide
    # chunk) and k leaves a partial row tile
    (700, 1496, 72, torch.bfloat16, 2, 2e-2),
    # bf16 samples with d not a multiple of 8 (fp32 FMA products)
    (300, 260, 24, torch.bfloat16, 2, 2e-2),
])
def test_calibrate_matches_oracle_iteration(n, d, k, dtype, iters, tol):
    A, _ = samples(d, k, n, (100, d, k))
    A = A.to(dtype)
    V0 = synth.gaussian_block(d, k, (100, d, k, 3)).to(dtype)
    V, status = gsi.gsi_calibrate(A.to(DEV), V0.to(DEV), iters)
    sync()
    assert int(status.item()) == 0
    got = f64(V)
    want = orc.subspace_iteration(f64(A), f64(V0), iters)
    col_err = np.linalg.norm(got - want, axis=0)
    assert col_err.max() <= tol, f"worst column error {col_err.max():.2e}"
    orth = np.abs(got.T @ got - np.eye(k)).max()
    assert orth <= (1e-5 if dtype == torch.float32 else 1.5e-2), orth
    cos = orc.principal_cosines(orc.dgks_orth(got), want)
    assert 1.0 - cos.min() <= (1e-7 if dtype == torch.float32 else 1e-4), 1.0 - cos.min()
    print(f"n={n} d={d} k={k} {dtype}: worst column error {col_err.max():.2e}, orthogonality {orth:.2e}")


def test_calibration_converges_and_cascade_saves_sweeps():
    """Cold start from a Gaussian block converges to the samples' top-k
    subspace (LAPACK SVD of the same samples); the next layer, whose
    subspace is a rotated copy of this one (the depth cascade), starts from
    this layer's basis and is as accurate after 2 sweeps as a cold start
    after 8; each GPU basis matches the oracle run from the same start."""
    d, k, n = 1024, 64, 2048
    frames = synth.cascade_frames(d, k, 192, 2, (101, 0, 0))
    A0, _ = samples(d, k, n, (101, 0), frame=torch.cat(frames[0], 1))
    A1, _ = samples(d, k, n, (101, 1), frame=torch.cat(frames[1], 1))
    A0, A1 = A0.float(), A1.float()
    top0 = orc.dominant_subspace(f64(A0), k)
    top1 = orc.dominant_subspace(f64(A1), k)
    R0 = synth.gaussian_block(d, k, (101, 2)).float()
    V_l0, st0 = gsi.gsi_calibrate(A0.to(DEV), R0.to(DEV), 8)
    V_cold, st1 = gsi.gsi_calibrate(A1.to(DEV), R0.to(DEV), 8)
    V_warm, st2 = gsi.gsi_calibrate(A1.to(DEV), V_l0, 2)
    sync()
    assert int(st0.item()) == int(st1.item()) == int(st2.item()) == 0
    gap = lambda V, top: 1.0 - orc.principal_cosines(orc.dgks_orth(f64(V)), top).min()  # noqa: E731
    e0, ecold, ewarm = gap(V_l0, top0), gap(V_cold, top1), gap(V_warm, top1)
    # the oracle along the same path (its own layer-0 basis as the warm start)
    o0 = orc.subspace_iteration(f64(A0), f64(R0), 8)
    o1 = orc.subspace_iteration(f64(A1), o0, 2)
    assert np.linalg.norm(f64(V_l0) - o0, axis=0).max() <= 2e-4
    assert np.linalg.norm(f64(V_warm) - o1, axis=0).max() <= 2e-4
    print(f"layer 0 cold/8: {e0:.1e}; layer 1 cold/8: {ecold:.1e}, warm/2: {ewarm:.1e}")
    assert e0 < 1e-6 and ecold < 1e-6
    assert ewarm < 1e-6


def test_rank_deficient_block_sets_status():
    """Samples of rank 4 cannot give an 8-column basis: the Cholesky of the
    block meets a non-positive pivot, the run still ends, and the status
    word says so."""
    d, k, n = 64, 8, 32
    v, _ = synth.orthonormal_frame(d, 4, 0, (102, 0, 0, 1))
    A = synth.frame_samples(v, torch.ones(4, dtype=torch.float64), n, (102, 1)).float()
    V0 = synth.gaussian_block(d, k, (102, 2)).float()
    V, status = gsi.gsi_calibrate(A.to(DEV), V0.to(DEV), 2)
    sync()
    assert int(status.item()) != 0
