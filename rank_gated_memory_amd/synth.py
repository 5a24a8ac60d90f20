"""Seeded synthetic inputs for the gated subspace linear map.

This module only *builds inputs*: Gaussian weights W, orthonormal bases V_k
(plus an orthonormal complement block U used to place residuals), activation
tokens x with a prescribed residual ratio, and the choice of which tokens get
a large residual.  It never projects a vector onto a basis, never forms a
residual, a ratio, the image M = W V_k or an output; those belong to the
method and are computed independently by the CPU oracle and by the HIP
library.  Both of them consume what this module returns.

Every random draw comes from a torch.Generator seeded from
numpy.random.SeedSequence(20260506, spawn_key=(config, layer, map, purpose)),
so a tensor is a pure function of its key and of the device it is drawn on
(torch's CPU and GPU generators give different streams; small workloads are
drawn on the CPU and copied, large ones are drawn on the GPU).

Token recipe (workloads of the GSI technical summary's experiments, made
synthetic because no trained weights or text exist here):

* fast-path token: x = V_k z + c n with z ~ N(0, I_k), n ~ N(0, I_d)
  isotropic, c = rho_fast * ||z|| / ||n||; the realised ratio is close to
  rho_fast * sqrt(1 - k/d) (about 0.0097 for rho_fast = 0.01).
* slow-path token: x = V_k z + c U w with w ~ N(0, I_m), U orthonormal and
  orthogonal to V_k by construction (extra columns of the same QR), and
  c = rho * ||z|| / (||w|| sqrt(1 - rho^2)), so that the residual ratio is
  exactly rho (in exact arithmetic) with rho ~ U(rho_lo, rho_hi).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

ROOT_SEED = 20260506

# purpose codes (last element of a spawn key)
P_WEIGHT, P_BASIS, P_Z, P_NOISE, P_RESID, P_RHO, P_PICK, P_CASCADE, P_OUTLIER = range(9)

# Map roles of the two transformer shapes (d -> d_out, k).
GPTJ_MAPS = (
    ("qkv", 4096, 12288, 256),
    ("out", 4096, 4096, 256),
    ("fc_in", 4096, 16384, 256),
    ("fc_out", 16384, 4096, 512),
)
LLAMA13_MAPS = (
    ("qkv", 5120, 15360, 320),
    ("out", 5120, 5120, 320),
    ("gate", 5120, 13824, 320),
    ("up", 5120, 13824, 320),
    ("down", 13824, 5120, 640),
)


def seed_for(*key: int) -> int:
    """63-bit seed derived from the root seed and a spawn key."""
    ss = np.random.SeedSequence(ROOT_SEED, spawn_key=tuple(int(v) for v in key))
    a, b = ss.generate_state(2, dtype=np.uint32)
    return ((int(a) << 32) | int(b)) & ((1 << 63) - 1)


def generator(device, *key: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*key))
    return g


def gaussian_weight(d_out: int, d: int, key, device="cpu", dtype=torch.bfloat16):
    """W ~ N(0, 1/d), shape [d_out][d], rounded to the storage dtype."""
    g = generator(device, *key)
    w = torch.randn((d_out, d), generator=g, device=device, dtype=torch.float32)
    w.mul_(1.0 / math.sqrt(d))
    return w.to(dtype)


def orthonormal_frame(d: int, k: int, extra: int, key, device="cpu"):
    """fp64 (V [d][k], U [d][extra]) from the QR of a seeded Gaussian d x (k+extra).

    Column signs are fixed so that diag(R) > 0, which makes the frame a
    deterministic function of the Gaussian draw.
    """
    g = generator(device, *key)
    a = torch.randn((d, k + extra), generator=g, device=device, dtype=torch.float64)
    q, r = torch.linalg.qr(a)
    s = torch.sign(torch.diagonal(r))
    s[s == 0] = 1.0
    q = q * s
    return q[:, :k].contiguous(), q[:, k:].contiguous()


def cascade_frames(d: int, k: int, extra: int, layers: int, key, device="cpu",
                   tau: float = 0.33, rank1: int = 2, theta: float = 0.6):
    """Per-layer frames where layer l+1 grows out of layer l.

    Layer l+1 is the QR of (V_l + tau N) with N ~ N(0, 1/d), after `rank1`
    of its columns have been turned by the angle theta toward fresh Gaussian
    unit directions (rank-1 changes); the extra columns of the same QR give
    the complement block U.  This mimics the depth coherence the GSI
    technical summary reports for consecutive layers (§2.3) and is tuned so
    that the mean principal-angle cosine between neighbours stays above 0.90.
    """
    frames = [orthonormal_frame(d, k, extra, tuple(key) + (0,), device)]
    for layer in range(1, layers):
        g = generator(device, *tuple(key), layer)
        v_prev = frames[-1][0]
        a = v_prev + (tau / math.sqrt(d)) * torch.randn(
            (d, k), generator=g, device=device, dtype=torch.float64)
        cols = torch.randperm(k, generator=g, device=device)[:rank1]
        for c in cols.tolist():
            h = torch.randn(d, generator=g, device=device, dtype=torch.float64)
            h = h / torch.linalg.vector_norm(h)
            a[:, c] = math.cos(theta) * a[:, c] + math.sin(theta) * h * torch.linalg.vector_norm(a[:, c])
        fresh = torch.randn((d, extra), generator=g, device=device, dtype=torch.float64)
        q, r = torch.linalg.qr(torch.cat([a, fresh], dim=1))
        s = torch.sign(torch.diagonal(r))
        s[s == 0] = 1.0
        q = q * s
        frames.append((q[:, :k].contiguous(), q[:, k:].contiguous()))
    return frames


def subspace_map(v_in: torch.Tensor, v_out: torch.Tensor, key, device="cpu", dtype=torch.bfloat16):
    """A weight [d_out][d_in] that carries one activation subspace onto the next.

    v_in [d_in][k_in] and v_out [d_out][k_out] are orthonormal bases.  The
    weight is W = v_out B v_in^T + G (I - v_in v_in^T) with B ~ N(0, 1/k_out)
    and G ~ N(0, 1/d_out): a token v_in z + r (r orthogonal to v_in) maps to
    v_out (B z) + G r, whose two parts keep the norms of z and r in
    expectation, and G r falls almost entirely outside span(v_out) (a share
    k_out/d_out of its energy lands inside).  A chain of such maps thus keeps
    each token's residual ratio near where it started.  This stands in for
    the depth coherence of activation subspaces between consecutive layers
    that the GSI technical summary reports (§2.3), for dependency-chained
    stacks; drawn in fp32 and rounded to the storage dtype.
    """
    g = generator(device, *key)
    d_in, k_in = v_in.shape
    d_out, k_out = v_out.shape
    vi = v_in.to(device=device, dtype=torch.float32)
    vo = v_out.to(device=device, dtype=torch.float32)
    b = torch.randn((k_out, k_in), generator=g, device=device, dtype=torch.float32) / math.sqrt(k_out)
    w = torch.randn((d_out, d_in), generator=g, device=device, dtype=torch.float32) / math.sqrt(d_out)
    w -= (w @ vi) @ vi.T
    w += (vo @ b) @ vi.T
    return w.to(dtype)


@dataclass
class ChainLayer:
    """Maps of one GPT-J-style parallel block whose inputs are earlier outputs.

    qkv (d -> 3d) and fc_in (d -> f) read the layer input h; out (d -> d)
    reads the last third of qkv's output (the value part, which is what
    attention returns for a single cached position); fc_out (f -> d) reads
    fc_in's output and writes the next layer's input.  Each entry is (W, V).
    """
    maps: dict


def chain_config(d: int, k: int, f: int, kf: int, layers: int, key, device="cpu",
                 dtype=torch.bfloat16):
    """Bases and weights of a dependency-chained stack of GPT-J-style blocks.

    Activation spaces per layer l: h_l (layer input, d, basis k), o_l (the
    value part of qkv's output, d, k) and f_l (fc_in's output, f, kf).  The
    maps that feed a later map are subspace_maps between those spaces, so
    chained tokens keep their residual ratios; the Q and K parts of qkv and
    the out map (whose output nothing reads) are plain N(0, 1/d) weights.
    Returns (layers as ChainLayer, (V, U) frame of h_0 for drawing tokens).
    """
    key = tuple(key)
    h = [orthonormal_frame(d, k, 64 if l == 0 else 0, key + (l, 0, P_BASIS), device)
         for l in range(layers + 1)]
    out = []
    for l in range(layers):
        vo, _ = orthonormal_frame(d, k, 0, key + (l, 1, P_BASIS), device)
        vf, _ = orthonormal_frame(f, kf, 0, key + (l, 2, P_BASIS), device)
        vh, vh1 = h[l][0], h[l + 1][0]
        qk = gaussian_weight(2 * d, d, key + (l, 0, P_WEIGHT), device, dtype)
        qkv = torch.cat([qk, subspace_map(vh, vo, key + (l, 1, P_WEIGHT), device, dtype)])
        maps = {
            "qkv": (qkv, vh.to(dtype)),
            "fc_in": (subspace_map(vh, vf, key + (l, 2, P_WEIGHT), device, dtype), vh.to(dtype)),
            "out": (gaussian_weight(d, d, key + (l, 3, P_WEIGHT), device, dtype), vo.to(dtype)),
            "fc_out": (subspace_map(vf, vh1, key + (l, 4, P_WEIGHT), device, dtype), vf.to(dtype)),
        }
        out.append(ChainLayer(maps))
    return out, h[0]


def frame_samples(frame: torch.Tensor, spec: torch.Tensor, n: int, key, device="cpu") -> torch.Tensor:
    """n activation samples [n][d] = (Z * spec) frame^T with Z ~ N(0, I): the
    samples' covariance has eigenvalues spec^2 along the orthonormal columns
    of frame [d][m] (calibration inputs for the basis builder)."""
    g = generator(device, *key)
    z = torch.randn((n, frame.shape[1]), generator=g, device=device, dtype=torch.float64)
    return (z * spec.to(device=device, dtype=torch.float64)) @ frame.to(device=device, dtype=torch.float64).T


def gaussian_block(d: int, k: int, key, device="cpu") -> torch.Tensor:
    """A seeded Gaussian [d][k] block: the random start of a cold calibration."""
    g = generator(device, *key)
    return torch.randn((d, k), generator=g, device=device, dtype=torch.float64)


def pick_slow(n: int, count: int, key, device="cpu") -> torch.Tensor:
    """Boolean mask with exactly `count` True entries at seeded positions."""
    g = generator("cpu", *key)
    perm = torch.randperm(n, generator=g)
    mask = torch.zeros(n, dtype=torch.bool)
    mask[perm[:count]] = True
    return mask.to(device)


def tokens(v: torch.Tensor, u: torch.Tensor, slow_mask: torch.Tensor, key,
           rho_fast: float = 0.01, rho_slow=(0.1, 0.5)):
    """fp64 tokens [n][d] and the constructed ratio per token.

    Returns (X, rho_built) where rho_built is the exact construction ratio for
    slow tokens and NaN for fast tokens (whose isotropic noise has a small,
    unrecorded in-subspace part).
    """
    device = v.device
    d, k = v.shape
    m = u.shape[1]
    n = int(slow_mask.numel())
    gz = generator(device, *tuple(key), P_Z)
    gn = generator(device, *tuple(key), P_NOISE)
    gr = generator(device, *tuple(key), P_RESID)
    gp = generator(device, *tuple(key), P_RHO)
    z = torch.randn((n, k), generator=gz, device=device, dtype=torch.float64)
    x = z @ v.T
    zn = torch.linalg.vector_norm(z, dim=1)
    rho_built = torch.full((n,), float("nan"), dtype=torch.float64, device=device)
    slow_mask = slow_mask.to(device)
    fast_idx = torch.nonzero(~slow_mask).flatten()
    slow_idx = torch.nonzero(slow_mask).flatten()
    if fast_idx.numel():
        noise = torch.randn((fast_idx.numel(), d), generator=gn, device=device, dtype=torch.float64)
        c = rho_fast * zn[fast_idx] / torch.linalg.vector_norm(noise, dim=1)
        x[fast_idx] += c[:, None] * noise
    if slow_idx.numel():
        w = torch.randn((slow_idx.numel(), m), generator=gr, device=device, dtype=torch.float64)
        rho = rho_slow[0] + (rho_slow[1] - rho_slow[0]) * torch.rand(
            slow_idx.numel(), generator=gp, device=device, dtype=torch.float64)
        c = rho * zn[slow_idx] / (torch.linalg.vector_norm(w, dim=1) * torch.sqrt(1.0 - rho * rho))
        x[slow_idx] += c[:, None] * (w @ u.T)
        rho_built[slow_idx] = rho
    return x, rho_built


def spectral_tokens(v: torch.Tensor, u: torch.Tensor, n: int, key, alpha: float = 1.1,
                    outlier_rate: float = 0.05, outlier_scale=(4.0, 10.0)):
    """fp64 tokens [n][d] whose energy along the directions [v | u] decays as a power law.

    With K = v.shape[1] head directions and m = u.shape[1] tail directions
    (jointly orthonormal), x = v (s * z) + f u (t * w), z ~ N(0, I_K),
    w ~ N(0, I_m), where s_i = i^-alpha (i = 1..K) and t_j = s_{K+j} scaled so
    that the m tail directions carry the whole tail mass sum_{i>K}^{d} s_i^2.
    f = 1, except for a seeded share of outlier tokens with f ~ U(outlier_scale).
    A basis made of the first k columns of v then sees a residual ratio that
    falls as k grows, so the share of fast tokens depends on k and on the
    threshold instead of being prescribed.  Returns (X, outlier mask).
    """
    device = v.device
    d, K = v.shape
    m = u.shape[1]
    i = torch.arange(1, d + 1, dtype=torch.float64, device=device)
    s = i.pow(-alpha)
    head = s[:K]
    tail = s[K:K + m] * torch.sqrt((s[K:] ** 2).sum() / (s[K:K + m] ** 2).sum())
    gz = generator(device, *tuple(key), P_Z)
    gw = generator(device, *tuple(key), P_NOISE)
    go = generator(device, *tuple(key), P_OUTLIER)
    z = torch.randn((n, K), generator=gz, device=device, dtype=torch.float64) * head
    w = torch.randn((n, m), generator=gw, device=device, dtype=torch.float64) * tail
    out = torch.rand(n, generator=go, device=device, dtype=torch.float64) < outlier_rate
    f = outlier_scale[0] + (outlier_scale[1] - outlier_scale[0]) * torch.rand(
        n, generator=go, device=device, dtype=torch.float64)
    w = w * torch.where(out, f, torch.ones_like(f))[:, None]
    return z @ v.T + w @ u.T, out


# --------------------------------------------------------------------------
# Workload builders.  Each returns plain tensors in the storage dtype; the
# oracle receives their exact fp64 upcast.
# --------------------------------------------------------------------------

@dataclass
class MapInputs:
    name: str
    d: int
    d_out: int
    k: int
    W: torch.Tensor          # [d_out][d] storage dtype
    V: torch.Tensor          # [d][k]     storage dtype
    X: torch.Tensor          # [T][d]     storage dtype
    slow_mask: torch.Tensor  # [T] bool, constructed slow tokens
    rho_built: torch.Tensor  # [T] fp64, NaN for fast tokens
    extra: dict = field(default_factory=dict)


def single_map(cfg: int, layer: int, idx: int, name: str, d: int, d_out: int, k: int,
               T: int, n_slow: int, dtype, device="cpu", w_device=None, extra_cols: int = 64,
               frame=None, keep_fp64: bool = True) -> MapInputs:
    """One map with T tokens of which exactly n_slow are slow by construction."""
    w_device = device if w_device is None else w_device
    W = gaussian_weight(d_out, d, (cfg, layer, idx, P_WEIGHT), w_device, dtype)
    if frame is None:
        frame = orthonormal_frame(d, k, min(extra_cols, d - k), (cfg, layer, idx, P_BASIS), device)
    v64, u64 = frame
    mask = pick_slow(T, n_slow, (cfg, layer, idx, P_PICK), device)
    x64, rb = tokens(v64, u64, mask, (cfg, layer, idx))
    extra = {"V64": v64, "U64": u64, "X64": x64} if keep_fp64 else {}
    return MapInputs(name, d, d_out, k, W, v64.to(dtype), x64.to(dtype), mask, rb, extra=extra)


def config1(device="cpu") -> MapInputs:
    """fp32 map d=256 -> 512, k=16, T=32 tokens, 8 of them slow."""
    return single_map(1, 0, 0, "single", 256, 512, 16, 32, 8, torch.float32, device)


def config2(T: int = 1000, slow_rate: float = 0.05, device="cpu", w_device=None, maps=GPTJ_MAPS):
    """GPT-J-6B-shaped map set, bf16, T sequential batch-1 tokens per map."""
    out = []
    for idx, (name, d, d_out, k) in enumerate(maps):
        out.append(single_map(2, 0, idx, name, d, d_out, k, T, round(slow_rate * T),
                              torch.bfloat16, device, w_device))
    return out


def config5(k: int, slow_frac: float, T: int = 256, d: int = 4096, d_out: int = 16384,
            device="cpu", w_device=None) -> MapInputs:
    """Batched map T=256, d=4096 -> 16384, bf16, with round(slow_frac*T) slow tokens."""
    return single_map(5, k, int(round(slow_frac * 100)), "batched", d, d_out, k, T,
                      int(round(slow_frac * T)), torch.bfloat16, device, w_device)


# Map roles that read the same input as an earlier role of the same layer
# (follower index -> owner index): GPT-J's parallel block feeds qkv and
# fc_in from one layer norm; LLaMA's gate and up read one MLP input.
SHARED_INPUTS = {"gptj6b-28L": {2: 0}, "llama13b-40L": {3: 2}}


def stack_config(cfg: int, layers: int, maps, steps: int, slow_rate: float,
                 device="cpu", cascade: bool = True, extra_cols: int = 64, keep_fp64: bool = False,
                 share=None):
    """Layer stack: per map role a (cascaded or independent) basis per layer.

    Returns a list over layers of lists over roles of MapInputs whose X holds
    one token per decode step ([steps][d]).  share (follower role index ->
    owner role index): the follower reads the owner's tokens with the
    owner's basis (the same tensors) through its own weight, and carries
    shared=True.
    """
    share = share or {}
    n_slow = int(round(slow_rate * steps))
    frames = {}
    for ridx, (name, d, d_out, k) in enumerate(maps):
        if cascade:
            frames[ridx] = cascade_frames(d, k, extra_cols, layers, (cfg, 0, ridx, P_CASCADE), device)
    out = []
    for layer in range(layers):
        row = []
        for ridx, (name, d, d_out, k) in enumerate(maps):
            if ridx in share:
                o = row[share[ridx]]
                if (o.d, o.k) != (d, k):
                    raise ValueError(f"{name} cannot share the input of {o.name}")
                W = gaussian_weight(d_out, d, (cfg, layer, ridx, P_WEIGHT), device, torch.bfloat16)
                mi = MapInputs(name, d, d_out, k, W, o.V, o.X, o.slow_mask, o.rho_built, extra=o.extra)
                mi.shared = True
                row.append(mi)
                continue
            fr = frames[ridx][layer] if cascade else None
            row.append(single_map(cfg, layer, ridx, name, d, d_out, k, steps, n_slow,
                                  torch.bfloat16, device, device, extra_cols, frame=fr,
                                  keep_fp64=keep_fp64))
            if cascade and not keep_fp64:
                frames[ridx][layer] = None
        out.append(row)
    return out


def sweep_config(layers: int = 28, steps: int = 128, head: int = 1024, tail: int = 512,
                 alpha: float = 1.1, device="cpu"):
    """Operating-point workload: GPT-J-shaped maps whose tokens have a power-law spectrum.

    Per layer and map role: W, a frame of `head` nested basis directions plus
    `tail` complement directions, and `steps` spectral tokens.  A basis of
    size k is the first k columns of the frame (nested in k).  Returns a list
    over layers of lists over roles of dicts with W, the fp64 frame head V64
    [d][head] and the tokens X [steps][d] in bf16.
    """
    cfg = 6
    out = []
    for layer in range(layers):
        row = []
        for ridx, (name, d, d_out, k) in enumerate(GPTJ_MAPS):
            W = gaussian_weight(d_out, d, (cfg, layer, ridx, P_WEIGHT), device, torch.bfloat16)
            v, u = orthonormal_frame(d, head, tail, (cfg, layer, ridx, P_BASIS), device)
            x, outl = spectral_tokens(v, u, steps, (cfg, layer, ridx), alpha)
            row.append({"name": name, "d": d, "d_out": d_out, "k_ref": k, "W": W, "V64": v,
                        "X": x.to(torch.bfloat16), "outliers": outl})
        out.append(row)
    return out


STACKS = {
    # name: (config id, layers, map roles, decode steps, slow-token rate, cascaded bases)
    "gptj6b-28L": (3, 28, GPTJ_MAPS, 512, 0.05, True),
    "llama13b-40L": (4, 40, LLAMA13_MAPS, 256, 0.02, False),
}


def mean_principal_cosine(v1: torch.Tensor, v2: torch.Tensor) -> float:
    """Mean cosine of the principal angles between two orthonormal bases."""
    s = torch.linalg.svdvals(v1.T.to(torch.float64) @ v2.to(torch.float64))
    return float(s.mean())
