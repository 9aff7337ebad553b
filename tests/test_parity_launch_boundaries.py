"""GPU parity at the edges of the forward's launch-shape rules: each case sits on one side of a
threshold the dispatcher compares against (N = 1024 for the long-sequence shapes, 256 CUs of
256-row tiles for the 8-wave launch, 256 and 512 tiles of 128 rows for the key-split launches),
so that every shape is exercised with the smallest and largest tile counts it accepts.  Two
heads (the first and the last) of every case are checked on every row against the float64
oracle, on NaN-filled outputs, so a tile the launch fails to write shows up as non-finite.

Tolerances as in test_parity.py: O max-abs 2e-2 and mean-abs 2e-3, LSE max-abs 1e-3.
"""
import numpy as np
import pytest
import torch

from io_aware_softmax_mifa_amd import workloads as W
from oracle import attention_fp64

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3

# (B, H, N, d, causal, the launch shape the rules pick)
CASES = [
    (1, 28, 1025, 128, True, "key split, 252 tiles of 128 rows (N > 1024)"),
    (1, 29, 1025, 128, True, "key split over tile pairs, 261 tiles"),
    (1, 51, 1025, 64, True, "key split over tile pairs, 459 tiles"),
    (1, 52, 1025, 64, True, "8-wave tile pairs, 260 tiles of 256 rows"),
    (1, 57, 1025, 128, True, "8-wave tile pairs, 285 tiles of 256 rows"),
    (2, 16, 1024, 64, True, "key split, 256 tiles (N = 1024)"),
    (1, 64, 1024, 128, False, "8-wave non-causal, exactly 256 tiles of 256 rows"),
    (1, 63, 1024, 128, False, "4-wave, 504 tiles (255 of 256 rows is too few)"),
    (1, 33, 1000, 64, True, "4-wave, 264 tiles, three workgroups per CU"),
    (2, 65, 513, 128, False, "4-wave, 650 tiles"),
]


def say(msg):
    print(f"[boundary] {msg}", flush=True)


@pytest.mark.parametrize("B,H,N,d,causal,shape", CASES, ids=[c[5] for c in CASES])
def test_launch_boundary(B, H, N, d, causal, shape):
    from io_aware_softmax_mifa_amd import binding

    q, k, v = W.make_inputs(B, H, N, d, seed=7000 + H + N + d)
    scale = W.fp32_scale(d)
    say(f"B={B} H={H} N={N} d={d} causal={causal}: {shape}")
    o = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    o, lse = binding.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), f"{shape}: non-finite output"
    for b, h in ((0, 0), (B - 1, H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ro, rl = attention_fp64(q[sl], k[sl], v[sl], causal=causal, scale=scale)
        err = np.abs(o[sl].double().numpy() - ro)
        lerr = np.abs(lse[sl].double().numpy() - rl)
        say(f"  head ({b}, {h}): O max {err.max():.3e} mean {err.mean():.3e}  LSE max {lerr.max():.3e}")
        assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr.max() <= LSE_MAX, (shape, b, h)
