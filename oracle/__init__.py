"""Dense fp64 CPU oracle for block-sparse FlexAttention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
"""
from . import flex_oracle  # noqa: F401
