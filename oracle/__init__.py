"""CPU float64 oracle for exact attention: test infrastructure only.

Only the tests, the smoke check and the bench's CPU-baseline leg may import this package.
"""
from .attention import attention_fp64, attention_fp64_rows, attention_online_fp64, merge_partials

__all__ = ["attention_fp64", "attention_fp64_rows", "attention_online_fp64", "merge_partials"]
