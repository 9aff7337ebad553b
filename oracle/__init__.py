"""CPU float64 oracle for exact attention, its gradients and the row softmax: test infrastructure only.

Only the tests, the smoke check and the bench's CPU-baseline leg may import this package.
"""
from .attention import attention_fp64, attention_fp64_rows, attention_online_fp64, merge_partials
from .attention_bwd import attention_bwd_fp64, attention_bwd_fp64_rows
from .softmax import softmax_online_fp64, softmax_rows_fp64

__all__ = ["attention_fp64", "attention_fp64_rows", "attention_online_fp64", "merge_partials",
           "attention_bwd_fp64", "attention_bwd_fp64_rows", "softmax_rows_fp64", "softmax_online_fp64"]
