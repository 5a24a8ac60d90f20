"""CPU oracle of the gated subspace linear map (test infrastructure only).

Imported by tests, by the package smoke check and by the benchmark's CPU
baseline leg; never by the library's product path.
"""
from . import gsi_oracle  # noqa: F401
