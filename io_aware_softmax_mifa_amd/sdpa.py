"""A drop-in for torch.nn.functional.scaled_dot_product_attention on bf16 GPU tensors.

The Hacker News FlashAttention-3 thread names scaled_dot_product_attention as the user-facing
call that reaches fused attention; this module gives that call shape to the HIP library.  Two
torch custom ops carry the work -- ``mifa::attention_fwd`` (O in q's dtype and layout, plus
the float32 LSE) and ``mifa::attention_bwd`` (dq, dk, dv in the inputs' dtypes and layouts) --
and are tied together with ``register_autograd``, so ``loss.backward()`` runs the library's
backward.  Inputs are read in place through their strides ([B, H, N, d] tensors, including the
[B, N, H, d].transpose(1, 2) views that come out of one projection): no copies.

Semantics follow torch's function where they overlap: ``is_causal`` is the lower-triangular
mask (the square case; for Nq != Nk torch aligns that mask top-left, which this library does
not implement, so it raises), and ``attn_mask=torch.nn.attention.bias.causal_lower_right(Nq,
Nk)`` selects the bottom-right alignment (the queries are the last Nq positions), which it
does implement.  Dropout, other masks and grouped-query attention with 1 < Hk < Hq raise
NotImplementedError; Hk == 1 (multi-query) broadcasts the single key/value head through a
zero stride.
"""
from __future__ import annotations

import math

import torch
from torch.nn.attention.bias import CausalBias, CausalVariant

from . import binding

__all__ = ["scaled_dot_product_attention"]


@torch.library.custom_op("mifa::attention_fwd", mutates_args=(), device_types="cuda")
def attention_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool,
                  scale: float) -> tuple[torch.Tensor, torch.Tensor]:
    """O (q's dtype and layout) and LSE (float32 [B, H, Nq]) of exact attention."""
    out = torch.empty_like(q)
    return binding.attention(q, k, v, causal=causal, scale=scale, out=out)


@attention_fwd.register_fake
def _(q, k, v, causal, scale):
    B, H, Nq, _ = q.shape
    return torch.empty_like(q), q.new_empty((B, H, Nq), dtype=torch.float32)


@torch.library.custom_op("mifa::attention_bwd", mutates_args=(), device_types="cuda")
def attention_bwd(do: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                  lse: torch.Tensor, causal: bool, scale: float) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dq, dk, dv (dtypes and layouts of q, k, v) for the upstream gradient do."""
    if do.stride(3) != 1 or any(st % 8 for st in do.stride()[:3]):
        do = do.contiguous()
    # empty_like keeps a dense input's layout and makes an overlapping one (a broadcast head) dense
    grads = tuple(torch.empty_like(t) for t in (q, k, v))
    return binding.attention_backward(q, k, v, o, lse, do, causal=causal, scale=scale, grads=grads)


@attention_bwd.register_fake
def _(do, q, k, v, o, lse, causal, scale):
    return torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)


def _setup_context(ctx, inputs, output):
    q, k, v, causal, scale = inputs
    o, lse = output
    ctx.save_for_backward(q, k, v, o, lse)
    ctx.causal, ctx.scale = causal, scale
    ctx.mark_non_differentiable(lse)


def _backward(ctx, do, _dlse):
    q, k, v, o, lse = ctx.saved_tensors
    dq, dk, dv = attention_bwd(do, q, k, v, o, lse, ctx.causal, ctx.scale)
    return dq, dk, dv, None, None


attention_fwd.register_autograd(_backward, setup_context=_setup_context)


def scaled_dot_product_attention(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor, attn_mask=None,
                                 dropout_p: float = 0.0, is_causal: bool = False, scale: float | None = None,
                                 enable_gqa: bool = False) -> torch.Tensor:
    """softmax(scale q k^T [+ causal mask]) v for bf16 [B, H, N, d] GPU tensors, d = 64 or 128.

    Same arguments as torch.nn.functional.scaled_dot_product_attention; see the module
    docstring for what is supported.  Returns O in bf16 with query's layout; differentiable."""
    for name, t in (("query", query), ("key", key), ("value", value)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D [B, H, N, d] tensor")
        if t.dtype != torch.bfloat16 or t.device.type != "cuda":
            raise ValueError(f"{name} must be a bfloat16 GPU tensor")
    if dropout_p != 0.0:
        raise NotImplementedError("dropout is not implemented")
    B, Hq, Nq, d = query.shape
    Hk, Nk = key.shape[1], key.shape[2]
    if Hk != Hq:
        if not enable_gqa or Hk != 1 or value.shape[1] != 1:
            raise NotImplementedError("key/value heads must equal query heads, or be one head with enable_gqa")
        key = key.expand(B, Hq, Nk, d)
        value = value.expand(B, Hq, Nk, d)
    causal = False
    if attn_mask is not None:
        if is_causal:
            raise ValueError("give either attn_mask or is_causal, not both")
        if not isinstance(attn_mask, CausalBias):
            raise NotImplementedError("only the causal biases of torch.nn.attention.bias are implemented as masks")
        if (attn_mask.seq_len_q, attn_mask.seq_len_kv) != (Nq, Nk):
            raise ValueError("the causal bias does not match the query/key lengths")
        if attn_mask.variant == CausalVariant.LOWER_RIGHT or Nq == Nk:
            causal = True
        else:
            raise NotImplementedError("the top-left causal alignment with Nq != Nk is not implemented")
    elif is_causal:
        if Nq != Nk:
            raise NotImplementedError("is_causal with Nq != Nk aligns the mask top-left in torch, which is not "
                                      "implemented; pass attn_mask=causal_lower_right(Nq, Nk) for the bottom-right "
                                      "alignment")
        causal = True
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, _ = attention_fwd(query, key, value, causal, float(scale))
    return o
