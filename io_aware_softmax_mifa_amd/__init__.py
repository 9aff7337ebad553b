"""mifa: exact FlashAttention (forward and backward) for the AMD Instinct MI355X (gfx950).

The compute lives in a HIP shared library (`libmifa.so`, C ABI declared in include/mifa.h).
`binding` marshals torch tensors into that ABI, and `sdpa` registers torch custom ops with
autograd over it (a drop-in for scaled_dot_product_attention).  Importing this package does
not load the library, so the seeded input generator in `workloads` is usable on machines
without a GPU.
"""
import importlib

__all__ = ["binding", "sdpa", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
