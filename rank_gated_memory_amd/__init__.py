"""Gated subspace linear maps on MI355X (gfx950).

The product path is the C-ABI library ``libgsi.so`` built from ``csrc/``;
``rank_gated_memory_amd.gsi`` is its Python binding (argument marshalling
only).  ``synth`` builds seeded synthetic inputs and ``accounting`` holds the
byte/flop bookkeeping used for roofline reports.
"""
__all__ = ["gsi", "synth", "accounting"]
