"""Byte and parameter accounting of the gated subspace linear map.

Pure host arithmetic used to report algorithmic HBM traffic and roofline
fractions; it computes nothing of the map itself.

GSI-TS = technical summary of "Gated Subspace Inference for Transformer
Acceleration" (S. J. Thomas, 2026).
"""
from __future__ import annotations

ESIZE = {"fp32": 4, "f32": 4, "bf16": 2}


def token_bytes(d: int, d_out: int, k: int, esize: int, slow: bool) -> int:
    """Algorithmic bytes moved for one token of one map at batch 1.

    Fast path (GSI-TS §2.2): read V_k (d*k) to form g and decide the gate,
    then the image M (d_out*k).  Slow path: V_k (the gate is decided first)
    and the full W (d_out*d).  Both read x (d) and write y (d_out).
    """
    body = d * k + (d * d_out if slow else d_out * k)
    return esize * (body + d + d_out)


def project_bytes(d: int, k: int, esize: int) -> int:
    """Bytes of the projection phase of one token: V_k and x."""
    return esize * (d * k + d)


def gram_bytes(k: int, esize: int) -> int:
    """Bytes of E = V_k^T V_k - I, read once per gate when the exact residual
    ratio is used (GSI-TS §2.2's ||r|| / ||x|| for the stored basis)."""
    return esize * k * k


def apply_bytes(d: int, d_out: int, k: int, esize: int, slow: bool) -> int:
    """Bytes of the output phase of one token: M (fast) or W and x (slow), plus y."""
    if slow:
        return esize * (d * d_out + d + d_out)
    return esize * (d_out * k + d_out)


def dense_bytes(d: int, d_out: int, esize: int) -> int:
    """Bytes of the dense y = W x at batch 1 (W, x and y)."""
    return esize * (d * d_out + d + d_out)


def token_flops(d: int, d_out: int, k: int, slow: bool) -> int:
    """Multiply-add flops (2 per MAC) of one token: projection plus the chosen path."""
    return 2 * d * k + (2 * d * d_out if slow else 2 * d_out * k)


def weight_read_speedup(d: int, k: int, slow_share: float) -> float:
    """Weight-read speedup of gating over dense reads, counting M against W.

    A fast token reads k columns' worth of the map (the image M) instead of
    d (GSI-TS §2.2); a slow token reads all d.  With a share s of slow
    tokens the ratio of dense to gated weight reads is 1 / ((1-s) k/d + s).
    This reconstruction reproduces the summary's printed speedups (§4).
    """
    return 1.0 / ((1.0 - slow_share) * k / d + slow_share)


def effective_parameters(total_params: float, d: int, k: int) -> float:
    """Parameters touched per token when every map reads k of d directions (GSI-TS §4)."""
    return total_params * k / d
