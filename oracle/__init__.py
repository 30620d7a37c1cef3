"""fp64 CPU oracle for the KDA forward pass (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the GPU library and its Python binding never do.
"""
from .ref import kda_oracle, kda_oracle_np

__all__ = ["kda_oracle", "kda_oracle_np"]
