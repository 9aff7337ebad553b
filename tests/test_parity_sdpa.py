"""GPU parity of the SDPA drop-in surface: strided layouts, bf16 O and gradients, the torch
custom ops with autograd, bottom-right causal for Nq != Nk, and one shared key/value head.

Everything is compared with the float64 CPU oracle (on dense copies of the same bf16 values).
Bars: float32 outputs keep the bars of the dense entry points (O max-abs 2e-2, mean-abs 2e-3,
LSE 1e-3; gradients max-abs 1e-2 max|ref|, RMS 5e-3 RMS(ref)).  A bf16 output adds one
rounding to nearest (at most u = 2^-8 relative, 8 significant bits): the O bars become
2e-2 + u max|ref| (max-abs) and 2e-3 + u mean|ref| (mean-abs); gradient bars become
(1e-2 + u) max|ref| and (5e-3 + u) RMS(ref).
"""
import numpy as np
import pytest
import torch

from io_aware_softmax_mifa_amd import workloads as W
from oracle import attention_bwd_fp64, attention_fp64

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


def say(msg):
    print(f"[parity-sdpa] {msg}", flush=True)


def check_o(o, lse, ro, rl, what, bf16):
    o = o.detach().float().cpu().double().numpy()
    lse = lse.cpu().double().numpy() if lse is not None else None
    err = np.abs(o - ro)
    mx = 2e-2 + (U * np.abs(ro).max() if bf16 else 0.0)
    mean = 2e-3 + (U * np.abs(ro).mean() if bf16 else 0.0)
    say(f"{what}: O max {err.max():.3e} (bar {mx:.2e}) mean {err.mean():.3e} (bar {mean:.2e})")
    assert np.isfinite(o).all()
    assert err.max() <= mx and err.mean() <= mean, what
    if lse is not None:
        lerr = np.abs(lse - rl).max()
        assert lerr <= 1e-3, (what, lerr)


def check_grads(got, ref, what, bf16):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.detach().float().cpu().double().numpy()
        err = np.abs(g - r)
        rms = np.sqrt((err ** 2).mean())
        ref_rms = np.sqrt((r ** 2).mean())
        mx_bar = (1e-2 + (U if bf16 else 0.0)) * np.abs(r).max()
        rms_bar = (5e-3 + (U if bf16 else 0.0)) * ref_rms
        say(f"{what}: {name} max {err.max():.3e} (bar {mx_bar:.2e}) rms {rms:.3e} (bar {rms_bar:.2e})")
        assert np.isfinite(g).all()
        assert err.max() <= mx_bar and rms <= rms_bar, (what, name)


def bnhd_views(B, H, Nq, Nk, d, seed):
    """q, k, v as [B, H, N, d] views of [B, N, H, d] storage (rows H*d apart), plus dense CPU copies."""
    q, k, v = W.make_rect_inputs(B, H, Nq, Nk, d, seed)
    views = []
    for t in (q, k, v):
        store = t.transpose(1, 2).contiguous().cuda()      # [B, N, H, d]
        views.append(store.transpose(1, 2))                 # [B, H, N, d] view, strides (N*H*d, d, H*d, 1)
    return (q, k, v), views


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_strided_forward(d, causal, out_dtype):
    from io_aware_softmax_mifa_amd import binding

    B, H, N = 2, 3, 333
    (q, k, v), (gq, gk, gv) = bnhd_views(B, H, N, N, d, 400 + d + causal)
    assert not gq.is_contiguous() and gq.stride(2) == H * d
    scale = W.fp32_scale(d)
    # O in the [B, N, H, d] layout too
    out = torch.empty((B, N, H, d), dtype=out_dtype, device="cuda").transpose(1, 2)
    o, lse = binding.attention(gq, gk, gv, causal=causal, scale=scale, out=out)
    torch.cuda.synchronize()
    ro, rl = attention_fp64(q, k, v, causal=causal, scale=scale)
    check_o(o, lse, ro, rl, f"strided fwd d={d} causal={causal} out={out_dtype}", out_dtype == torch.bfloat16)


def test_strided_forward_rect_and_broadcast():
    from io_aware_softmax_mifa_amd import binding

    B, H, Nq, Nk, d = 1, 4, 77, 300, 128
    (q, k, v), (gq, gk, gv) = bnhd_views(B, H, Nq, Nk, d, 410)
    scale = W.fp32_scale(d)
    o, lse = binding.attention(gq, gk, gv, causal=True, scale=scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = attention_fp64(q, k, v, causal=True, scale=scale)
    check_o(o, lse, ro, rl, "strided rect causal", True)
    # one key/value head broadcast over the query heads through a zero head stride
    k1, v1 = k[:, :1].contiguous(), v[:, :1].contiguous()
    ek, ev = k1.cuda().expand(B, H, Nk, d), v1.cuda().expand(B, H, Nk, d)
    assert ek.stride(1) == 0
    o, lse = binding.attention(gq, ek, ev, causal=False, scale=scale)
    torch.cuda.synchronize()
    ro, rl = attention_fp64(q, k1.expand(B, H, Nk, d), v1.expand(B, H, Nk, d), causal=False, scale=scale)
    check_o(o, lse, ro, rl, "broadcast kv head", False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("grad_dtype", [torch.float32, torch.bfloat16])
def test_strided_backward(d, grad_dtype):
    from io_aware_softmax_mifa_amd import binding

    B, H, N = 1, 3, 290
    (q, k, v), (gq, gk, gv) = bnhd_views(B, H, N, N, d, 420 + d)
    do = W.make_grad_output(B, H, N, d, 420 + d)
    gdo = do.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    scale = W.fp32_scale(d)
    o, lse = binding.attention(gq, gk, gv, causal=True, scale=scale, out_dtype=torch.bfloat16,
                               out=torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda").transpose(1, 2))
    grads = tuple(torch.empty((B, N, H, d), dtype=grad_dtype, device="cuda").transpose(1, 2) for _ in range(3))
    dq, dk, dv = binding.attention_backward(gq, gk, gv, o, lse, gdo, causal=True, scale=scale, grads=grads)
    torch.cuda.synchronize()
    ref = attention_bwd_fp64(q, k, v, do, causal=True, scale=scale)[:3]
    check_grads((dq, dk, dv), ref, f"strided bwd d={d} grads={grad_dtype} (bf16 O)", grad_dtype == torch.bfloat16)


@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
@pytest.mark.parametrize("causal", [True, False])
def test_custom_op_autograd(layout, causal):
    from io_aware_softmax_mifa_amd.sdpa import scaled_dot_product_attention as sdpa

    B, H, N, d = 2, 2, 200, 128
    q, k, v = W.make_inputs(B, H, N, d, 430 + causal)
    do = W.make_grad_output(B, H, N, d, 430 + causal)
    if layout == "bhnd":
        leaves = [t.cuda().requires_grad_() for t in (q, k, v)]
        args = leaves
    else:
        leaves = [t.transpose(1, 2).contiguous().cuda().requires_grad_() for t in (q, k, v)]
        args = [t.transpose(1, 2) for t in leaves]
    o = sdpa(*args, is_causal=causal)
    assert o.dtype == torch.bfloat16 and o.shape == (B, H, N, d)
    o.backward(do.cuda() if layout == "bhnd" else do.transpose(1, 2).contiguous().cuda().transpose(1, 2))
    torch.cuda.synchronize()
    scale = W.fp32_scale(d)  # the float32 value the library receives (reading R5)
    ro, rl = attention_fp64(q, k, v, causal=causal, scale=scale)
    check_o(o, None, ro, rl, f"sdpa {layout} causal={causal}", True)
    grads = [t.grad if layout == "bhnd" else t.grad.transpose(1, 2) for t in leaves]
    assert all(g.dtype == torch.bfloat16 for g in grads)
    ref = attention_bwd_fp64(q, k, v, do, causal=causal, scale=scale)[:3]
    check_grads(grads, ref, f"sdpa autograd {layout} causal={causal}", True)


def test_custom_op_lower_right_and_mqa():
    from torch.nn.attention.bias import causal_lower_right

    from io_aware_softmax_mifa_amd.sdpa import scaled_dot_product_attention as sdpa

    B, H, Nq, Nk, d = 1, 4, 50, 260, 64
    q, k, v = W.make_rect_inputs(B, H, Nq, Nk, d, 440)
    k1, v1 = k[:, :1].contiguous(), v[:, :1].contiguous()
    do = W.make_grad_output(B, H, Nq, d, 440)
    tq, tk, tv = (t.cuda().requires_grad_() for t in (q, k1, v1))
    o = sdpa(tq, tk, tv, attn_mask=causal_lower_right(Nq, Nk), enable_gqa=True, scale=0.2)
    o.backward(do.cuda())
    torch.cuda.synchronize()
    ek, ev = k1.expand(B, H, Nk, d), v1.expand(B, H, Nk, d)
    c = float(np.float32(0.2))  # the float32 value the library receives (reading R5)
    ro, rl = attention_fp64(q, ek, ev, causal=True, scale=c)
    check_o(o, None, ro, rl, "sdpa lower-right + one kv head", True)
    rdq, rdk, rdv, _ = attention_bwd_fp64(q, ek, ev, do, causal=True, scale=c)
    # the shared head's gradient is the sum over the query heads
    check_grads((tq.grad, tk.grad, tv.grad), (rdq, rdk.sum(axis=1, keepdims=True), rdv.sum(axis=1, keepdims=True)),
                "sdpa one kv head", True)


@pytest.mark.parametrize("d", [64, 128])
def test_strided_bf16_long_launch_shape(d):
    """[B, N, H, d] storage with bf16 O on the 8-wave launch (Nq > 1024, more than 256 query tiles
    of 256 rows), rectangular and causal.  Three heads against the oracle."""
    from io_aware_softmax_mifa_amd import binding

    B, H, Nq, Nk = 1, 64, 1100, 1300
    (q, k, v), (gq, gk, gv) = bnhd_views(B, H, Nq, Nk, d, 420 + d)
    scale = W.fp32_scale(d)
    out = torch.empty((B, Nq, H, d), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o, lse = binding.attention(gq, gk, gv, causal=True, scale=scale, out=out)
    torch.cuda.synchronize()
    for h in (0, 21, H - 1):
        ro, rl = attention_fp64(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], causal=True, scale=scale)
        check_o(o[:, h:h + 1], lse[:, h:h + 1], ro, rl, f"strided bf16 long d={d} head {h}", True)


@pytest.mark.parametrize("d", [64, 128])
def test_strided_bf16_key_split_pairs(d):
    """[B, N, H, d] storage with bf16 O through the key-split launch over tile pairs (causal,
    Nq > 1024, between 256 and 512 query tiles of 128 rows), rectangular: 24 heads of 1,500
    queries against 1,700 keys (288 tiles).  Three heads against the oracle."""
    from io_aware_softmax_mifa_amd import binding

    B, H, Nq, Nk = 1, 24, 1500, 1700
    (q, k, v), (gq, gk, gv) = bnhd_views(B, H, Nq, Nk, d, 430 + d)
    scale = W.fp32_scale(d)
    out = torch.empty((B, Nq, H, d), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o, lse = binding.attention(gq, gk, gv, causal=True, scale=scale, out=out)
    torch.cuda.synchronize()
    for h in (0, 11, H - 1):
        ro, rl = attention_fp64(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], causal=True, scale=scale)
        check_o(o[:, h:h + 1], lse[:, h:h + 1], ro, rl, f"strided bf16 key-split pairs d={d} head {h}", True)
