"""GPU check of the allocation-free split-KV entry point (mifa_attention_splitkv_noalloc) against
the workspace entry point (mifa_attention_splitkv), through the C ABI.

Both run the same kernels with the same key-range split, so the results must agree bit for bit;
the float64 oracle bar (O max-abs 2e-2, mean-abs 2e-3, LSE 1e-3) is checked on top, on sampled
rows.  Two calls in a row on the shared static array, the second with a smaller problem (different
head size, fewer ranges), then the first shape again: each call must see only its own partials.
"""
import numpy as np
import pytest
import torch

from io_aware_softmax_mifa_amd import binding
from io_aware_softmax_mifa_amd import workloads as W
from oracle import attention_fp64_rows

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


def say(msg):
    print(f"[noalloc] {msg}", flush=True)


def run_pair(B, H, Nq, Nk, d, causal, seed):
    q, k, v = W.make_rect_inputs(B, H, Nq, Nk, d, seed)
    scale = W.fp32_scale(d)
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    stream = torch.cuda.current_stream().cuda_stream
    need = binding.mifa_splitkv_workspace_bytes(B, H, Nq, Nk, d)
    assert 0 < need <= 32 << 20
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ws = torch.full((B, H, Nq, d), float("nan"), device="cuda")
    l_ws = torch.full((B, H, Nq), float("nan"), device="cuda")
    o_na, l_na = torch.full_like(o_ws, float("nan")), torch.full_like(l_ws, float("nan"))
    say(f"shape B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal}: partials {need} bytes")
    st = binding.mifa_attention_splitkv_raw(dq, dk, dv, o_ws, l_ws, B, H, Nq, Nk, d, causal, scale, ws, need, stream)
    assert st == 0, binding.mifa_status_string(st)
    st = binding.mifa_attention_splitkv_noalloc_raw(dq, dk, dv, o_na, l_na, B, H, Nq, Nk, d, causal, scale, stream)
    assert st == 0, binding.mifa_status_string(st)
    torch.cuda.synchronize()
    assert torch.isfinite(o_na).all() and torch.isfinite(l_na).all()
    assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), "noalloc differs from the workspace entry point"
    # the oracle bar on sampled rows
    rows = W.sample_rows(B, H, Nq, min(64, B * H * Nq), seed + 1000)
    ro, rl = attention_fp64_rows(q, k, v, rows, causal=causal, scale=scale)
    b, h, i = rows[:, 0], rows[:, 1], rows[:, 2]
    o = o_na.cpu().double().numpy()[b, h, i]
    lse = l_na.cpu().double().numpy()[b, h, i]
    err, lerr = np.abs(o - ro), np.abs(lse - rl)
    say(f"  O max {err.max():.3e} mean {err.mean():.3e}  LSE max {lerr.max():.3e}")
    assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr.max() <= LSE_MAX


def test_noalloc_matches_workspace_entry_point_twice_then_smaller():
    run_pair(1, 32, 16, 16384, 128, True, 501)   # one GPU's decode step: 32 key ranges
    run_pair(2, 4, 3, 3000, 64, True, 502)       # smaller, other head size, fewer ranges
    run_pair(1, 32, 16, 16384, 128, True, 503)   # the large shape again on the same array


def test_noalloc_single_range_and_limit():
    # Enough query tiles that one key range suffices: the static array is not used, and the
    # result is the plain forward's.
    B, H, Nq, Nk, d = 4, 32, 1024, 1024, 64
    q, k, v = (t.cuda() for t in W.make_rect_inputs(B, H, Nq, Nk, d, 505))
    scale = W.fp32_scale(d)
    o1, l1 = torch.empty(B, H, Nq, d, device="cuda"), torch.empty(B, H, Nq, device="cuda")
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    assert binding.mifa_attention_raw(q, k, v, o1, l1, B, H, Nq, Nk, d, True, scale, None) == 0
    assert binding.mifa_attention_splitkv_noalloc_raw(q, k, v, o2, l2, B, H, Nq, Nk, d, True, scale, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # partials beyond 32 MiB are refused before any launch
    big = (1, 8, 512, 65536, 128)
    assert binding.mifa_splitkv_workspace_bytes(*big) > 32 << 20
    t = torch.zeros(16, device="cuda")
    st = binding.mifa_attention_splitkv_noalloc_raw(t, t, t, t, t, *big, 1, 0.1, None)
    assert st == 11, binding.mifa_status_string(st)
