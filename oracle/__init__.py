"""CPU float64 oracle for exact attention and the row softmax: test infrastructure only.

Only the tests, the smoke check and the bench's CPU-baseline leg may import this package.
"""
from .attention import attention_fp64, attention_fp64_rows, attention_online_fp64, merge_partials
from .softmax import softmax_online_fp64, softmax_rows_fp64

__all__ = ["attention_fp64", "attention_fp64_rows", "attention_online_fp64", "merge_partials",
           "softmax_rows_fp64", "softmax_online_fp64"]
