"""GPU parity of attention with Nq != Nk (mifa_attention) and of the split-KV path
(mifa_attention_splitkv) against the float64 CPU oracle, through the C ABI.

Tolerances as for the square forward (O max-abs 2e-2, mean-abs 2e-3, LSE 1e-3); the split path
adds one merge in fp32 (weights exp(LSE_s - max) and a division), far below the bar.
"""
import numpy as np
import pytest
import torch

from io_aware_softmax_mifa_amd import workloads as W
from oracle import attention_fp64

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


def say(msg):
    print(f"[decode parity] {msg}", flush=True)


def check(o, lse, ro, rl, what):
    o = o.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    err, lerr = np.abs(o - ro), np.abs(lse - rl)
    say(f"{what}: O max {err.max():.3e} mean {err.mean():.3e}  LSE max {lerr.max():.3e}")
    assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr.max() <= LSE_MAX, what


def run(fn, q, k, v, causal, scale, **kw):
    o, lse = fn(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, **kw)
    torch.cuda.synchronize()
    return o, lse


def case(B, H, Nq, Nk, d, causal, seed, split, dist="normal"):
    from io_aware_softmax_mifa_amd import binding

    q, k, v = W.make_rect_inputs(B, H, Nq, Nk, d, seed, dist)
    scale = W.fp32_scale(d)
    say(f"B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} split={split} dist={dist}")
    fn = binding.attention_splitkv if split else binding.attention
    o, lse = run(fn, q, k, v, causal, scale)
    ro, rl = attention_fp64(q, k, v, causal=causal, scale=scale)
    check(o, lse, ro, rl, f"Nq={Nq} Nk={Nk} d={d} causal={causal} split={split}")
    return q, k, v, o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 1000), (5, 300), (100, 129), (128, 4096), (257, 1000), (1000, 1001)])
def test_rectangular(nq, nk, d, causal):
    case(2, 2, nq, nk, d, causal, seed=nq * 7 + nk, split=False)


@pytest.mark.parametrize("d", [64, 128])
def test_more_queries_than_keys_noncausal(d):
    case(1, 3, 300, 200, d, False, seed=9, split=False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("b,h,nq,nk", [(2, 4, 1, 8192), (1, 8, 16, 16384), (2, 2, 64, 5000), (1, 3, 200, 3000),
                                       (3, 1, 7, 777)])
def test_splitkv(b, h, nq, nk, d, causal):
    case(b, h, nq, nk, d, causal, seed=b + h + nq + nk, split=True)


@pytest.mark.parametrize("d", [64, 128])
def test_splitkv_square_causal_has_empty_ranges(d):
    """Square causal through the split path: the early query tiles see only the first key
    ranges, so most of their ranges are empty and must contribute nothing to the merge."""
    case(1, 1, 4096, 4096, d, True, seed=44, split=True)


@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_large_logits(causal):
    """Logits of std 4: the ranges' LSEs differ widely and the merge rescales by them."""
    case(1, 4, 8, 12000, 128, causal, seed=45, split=True, dist="stress")


def test_splitkv_workspace_reuse_and_determinism():
    from io_aware_softmax_mifa_amd import binding

    q, k, v = W.make_rect_inputs(2, 4, 3, 20000, 128, seed=46)
    q2, k2, v2 = W.make_rect_inputs(1, 2, 1, 9000, 64, seed=47)
    need = max(binding.mifa_splitkv_workspace_bytes(2, 4, 3, 20000, 128),
               binding.mifa_splitkv_workspace_bytes(1, 2, 1, 9000, 64))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o1, l1 = run(binding.attention_splitkv, q, k, v, True, 0.1, workspace=ws)
    o2, l2 = run(binding.attention_splitkv, q2, k2, v2, False, 0.2, workspace=ws)
    o3, l3 = run(binding.attention_splitkv, q, k, v, True, 0.1, workspace=ws)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    ro, rl = attention_fp64(q2, k2, v2, causal=False, scale=float(np.float32(0.2)))
    check(o2, l2, ro, rl, "second call, smaller shape, same workspace")


def test_splitkv_rejects_small_workspace():
    from io_aware_softmax_mifa_amd import binding

    q, k, v = W.make_rect_inputs(1, 8, 1, 32768, 128, seed=48)
    need = binding.mifa_splitkv_workspace_bytes(1, 8, 1, 32768, 128)
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.MifaError) as e:
        run(binding.attention_splitkv, q, k, v, True, 0.1, workspace=ws)
    assert e.value.status == 9


@pytest.mark.parametrize("name", ["D1", "D2"])
def test_decode_workloads(name):
    w = W.decode_by_name(name)
    case(w.B, w.H, w.Nq, w.Nk, w.d, w.causal, w.seed, split=True, dist=w.dist)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_rectangular_long_launch_shape(d, causal):
    """Nq > 1024 with more than 256 query tiles of 256 rows takes the 8-wave launch; with Nq < Nk
    the causal diagonal is shifted by Nk - Nq, which decides where each wave stops.  Nq = 1100 also
    ends in a partial query tile and Nk = 1500 in a partial key block.  Three heads against the
    oracle."""
    from io_aware_softmax_mifa_amd import binding

    B, H, Nq, Nk = 1, 64, 1100, 1500
    q, k, v = W.make_rect_inputs(B, H, Nq, Nk, d, 31 + d, "normal")
    scale = W.fp32_scale(d)
    say(f"long rect: B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    o, lse = run(binding.attention, q, k, v, causal, scale)
    for h in (0, 37, H - 1):
        ro, rl = attention_fp64(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], causal=causal, scale=scale)
        check(o[:, h:h + 1], lse[:, h:h + 1], ro, rl, f"long rect d={d} causal={causal} head {h}")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
