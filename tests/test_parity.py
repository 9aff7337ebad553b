"""GPU parity: the HIP kernel (through the C ABI) against the float64 CPU oracle.

Tolerances: O max-abs 2e-2 and mean-abs 2e-3, LSE max-abs 1e-3 (fp32 outputs of bf16 inputs
against float64).  Expected error is far below the bar: products are exact, accumulation is
fp32 and the only deliberate rounding is bf16 softmax weights before the PV product, about
2^-8 relative per weight at most (bf16 keeps 8 significant bits).
"""
import math

import numpy as np
import pytest
import torch

from io_aware_softmax_mifa_amd import workloads as W
from oracle import attention_fp64, attention_fp64_rows

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


def say(msg):
    print(f"[parity] {msg}", flush=True)


def run_gpu(q, k, v, causal, scale, poison=False):
    from io_aware_softmax_mifa_amd import binding

    dq, dk, dv = (t.cuda() for t in (q, k, v))
    o = lse = None
    if poison:
        o = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    o, lse = binding.attention(dq, dk, dv, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(o_gpu, lse_gpu, o_ref, lse_ref, what):
    o_gpu = o_gpu.double().numpy() if hasattr(o_gpu, "numpy") else o_gpu
    lse_gpu = lse_gpu.double().numpy() if hasattr(lse_gpu, "numpy") else lse_gpu
    assert np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all(), f"{what}: non-finite output"
    err = np.abs(o_gpu - o_ref)
    lerr = np.abs(lse_gpu - lse_ref)
    say(f"{what}: O max {err.max():.3e} mean {err.mean():.3e}  LSE max {lerr.max():.3e}")
    assert err.max() <= O_MAX, f"{what}: O max-abs {err.max()}"
    assert err.mean() <= O_MEAN, f"{what}: O mean-abs {err.mean()}"
    assert lerr.max() <= LSE_MAX, f"{what}: LSE max-abs {lerr.max()}"


def full_case(B, H, N, d, causal, seed, dist="normal", scale=None):
    q, k, v = W.make_inputs(B, H, N, d, seed, dist)
    scale = W.fp32_scale(d) if scale is None else scale
    say(f"B={B} H={H} N={N} d={d} causal={causal} seed={seed} dist={dist} scale={scale}")
    o, lse = run_gpu(q, k, v, causal, scale)
    ro, rl = attention_fp64(q, k, v, causal=causal, scale=scale)
    check(o, lse, ro, rl, f"N={N} d={d} causal={causal}")
    return q, k, v, o, lse


# ---- the seeded workloads --------------------------------------------------------------

@pytest.mark.parametrize("name", ["C1-nc", "C1-c", "C2-nc", "C2-c"])
def test_small_configs_full(name):
    w = W.by_name(name)
    full_case(w.B, w.H, w.N, w.d, w.causal, w.seed, w.dist)


@pytest.mark.parametrize("name", ["C3", "C5"])
def test_large_configs_every_row(name):
    """Full-size launch in the benchmark's launch shape, every output row of every head against
    the float64 oracle (one head at a time, so the score matrix stays one head's size); the
    max-abs and mean-abs bars apply to all B*H*N*d outputs together."""
    w = W.by_name(name)
    q, k, v = W.make_workload_inputs(w)
    scale = W.fp32_scale(w.d)
    say(f"{name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} dist={w.dist}, every row")
    o, lse = run_gpu(q, k, v, w.causal, scale)
    o_np, lse_np = o.double().numpy(), lse.double().numpy()
    assert np.isfinite(o_np).all() and np.isfinite(lse_np).all(), f"{name}: non-finite output"
    err_max = err_sum = lerr_max = 0.0
    for b in range(w.B):
        for h in range(w.H):
            ho, hl = attention_fp64(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                    causal=w.causal, scale=scale)
            e = np.abs(o_np[b:b + 1, h:h + 1] - ho)
            err_max, err_sum = max(err_max, float(e.max())), err_sum + float(e.sum())
            lerr_max = max(lerr_max, float(np.abs(lse_np[b:b + 1, h:h + 1] - hl).max()))
    err_mean = err_sum / o_np.size
    say(f"{name} every row: O max {err_max:.3e} mean {err_mean:.3e}  LSE max {lerr_max:.3e}")
    assert err_max <= O_MAX and err_mean <= O_MEAN and lerr_max <= LSE_MAX, name


@pytest.mark.parametrize("name", ["C4", "C4-shard"])
def test_large_configs_sampled(name):
    """Full-size launch; 256 seeded sampled rows checked (the oracle of every row of the
    16,384-long heads would take minutes of host time)."""
    w = W.by_name(name)
    q, k, v = W.make_workload_inputs(w)
    scale = W.fp32_scale(w.d)
    say(f"{name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    o, lse = run_gpu(q, k, v, w.causal, scale)
    rows = W.sample_rows(w.B, w.H, w.N, 256, w.seed)
    ro, rl = attention_fp64_rows(q, k, v, rows, causal=w.causal, scale=scale)
    r = rows.numpy()
    check(o[r[:, 0], r[:, 1], r[:, 2]].double().numpy(), lse[r[:, 0], r[:, 1], r[:, 2]].double().numpy(), ro, rl,
          f"{name} 256 sampled rows")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


# ---- the long-sequence launch shape (8-wave workgroups, four K/V buffers) ----------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dist", ["normal", "stress"])
def test_long_sequence_launch_shape(d, causal, dist):
    """N > 1024 with more than 256 workgroups of 256 rows takes the 8-wave launch; N = 4133 also
    ends in a partial key block.  Two whole heads and 128 sampled rows against the oracle."""
    B, H, N = 1, 16, 4133
    q, k, v = W.make_inputs(B, H, N, d, seed=4133 + d, dist=dist)
    scale = W.fp32_scale(d)
    say(f"long: B={B} H={H} N={N} d={d} causal={causal} dist={dist}")
    o, lse = run_gpu(q, k, v, causal, scale)
    for h in (0, H - 1):
        ho, hl = attention_fp64(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], causal=causal, scale=scale)
        check(o[:, h:h + 1], lse[:, h:h + 1], ho, hl, f"long d={d} causal={causal} {dist} head {h}")
    rows = W.sample_rows(B, H, N, 128, seed=d + 7)
    ro, rl = attention_fp64_rows(q, k, v, rows, causal=causal, scale=scale)
    r = rows.numpy()
    check(o[r[:, 0], r[:, 1], r[:, 2]].double().numpy(), lse[r[:, 0], r[:, 1], r[:, 2]].double().numpy(), ro, rl,
          f"long d={d} causal={causal} {dist} sampled rows")


@pytest.mark.parametrize("d", [64, 128])
def test_non_causal_one_tile_per_cu(d):
    """Without the mask, exactly 256 query tiles of 256 rows take the 8-wave launch: B=4 H=16
    N=1024, and B=2 H=16 N=2000 (partial last tile); every row of every head checked."""
    for B, H, N in ((4, 16, 1024), (2, 16, 2000)):
        q, k, v = W.make_inputs(B, H, N, d, seed=5300 + N + d)
        scale = W.fp32_scale(d)
        say(f"non-causal, 256 tiles: B={B} H={H} N={N} d={d}")
        o, lse = run_gpu(q, k, v, False, scale, poison=True)
        ro, rl = attention_fp64(q, k, v, causal=False, scale=scale)
        check(o, lse, ro, rl, f"non-causal 256 tiles N={N} d={d}")


@pytest.mark.parametrize("causal", [False, True])
def test_d64_three_workgroups_per_cu(causal):
    """d = 64 with many 128-row tiles and N <= 1024 takes the 4-wave launch, three workgroups
    resident per CU (three waves per SIMD): 1,024 tiles causal, 640 with a ragged last tile
    non-causal; every row of every head checked."""
    B, H, N = (16, 16, 512) if causal else (8, 16, 600)
    q, k, v = W.make_inputs(B, H, N, 64, seed=5400 + N)
    scale = W.fp32_scale(64)
    say(f"d=64 4-wave, three per CU: B={B} H={H} N={N} causal={causal}")
    o, lse = run_gpu(q, k, v, causal, scale, poison=True)
    ro, rl = attention_fp64(q, k, v, causal=causal, scale=scale)
    check(o, lse, ro, rl, f"d=64 three per CU N={N} causal={causal}")


# ---- the key-split launch (few tiles: two wave groups per tile share the key blocks) --------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [512, 777, 1000, 2113])
def test_key_split_launch(N, d, causal):
    """At most one 128-row tile per CU and at least 512 keys: two groups of waves take the even
    and odd key blocks of a tile and merge at the end.  Odd and even block counts, partial last
    blocks, causal diagonals inside either group's blocks; every row of every head checked, on
    NaN-filled outputs."""
    B, H = 1, 3
    q, k, v = W.make_inputs(B, H, N, d, seed=5000 + N + d, dist="stress" if N == 777 else "normal")
    scale = W.fp32_scale(d)
    say(f"key split: B={B} H={H} N={N} d={d} causal={causal}")
    o, lse = run_gpu(q, k, v, causal, scale, poison=True)
    ro, rl = attention_fp64(q, k, v, causal=causal, scale=scale)
    check(o, lse, ro, rl, f"key split N={N} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", [(1, 24, 1536), (1, 19, 1900), (2, 9, 2000)])
def test_key_split_tile_pairs(B, H, N, d):
    """Causal, between one and two 128-row tiles per CU: the key-split launch over tile pairs
    (n-1-r, r).  24 heads take the XCD-grouped order with an even tile count; 19 and 18 heads
    the plain order with 15 and 16 tiles (15: the middle tile runs alone), ragged last tiles;
    every row of every head checked, on NaN-filled outputs."""
    q, k, v = W.make_inputs(B, H, N, d, seed=5200 + H + d)
    scale = W.fp32_scale(d)
    say(f"key split, tile pairs: B={B} H={H} N={N} d={d} causal=True")
    o, lse = run_gpu(q, k, v, True, scale, poison=True)
    ro, rl = attention_fp64(q, k, v, causal=True, scale=scale)
    check(o, lse, ro, rl, f"key split pairs B={B} H={H} N={N} d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_key_split_launch_rectangular(d):
    """Few queries against many keys through mifa_attention (no key-range partials): the newest
    70 positions of 2,500 with the causal mask, and without it."""
    from io_aware_softmax_mifa_amd import binding

    q, k, v = W.make_rect_inputs(2, 2, 70, 2500, d, seed=5100 + d)
    scale = W.fp32_scale(d)
    for causal in (False, True):
        o, lse = binding.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
        torch.cuda.synchronize()
        ro, rl = attention_fp64(q, k, v, causal=causal, scale=scale)
        check(o.cpu(), lse.cpu(), ro, rl, f"key split rect d={d} causal={causal}")


# ---- ragged and tiny sequence lengths --------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 17, 63, 64, 65, 127, 129, 130, 257, 1000])
def test_ragged_lengths(N, d, causal):
    full_case(2, 3, N, d, causal, seed=1000 + N)


@pytest.mark.parametrize("d", [64, 128])
def test_many_heads_xcd_grouping(d):
    """B*H a multiple of 8 takes the XCD-grouped tile order; 5 heads takes the plain order."""
    full_case(2, 8, 384, d, True, seed=77)
    full_case(1, 5, 384, d, True, seed=78)
    full_case(2, 4, 300, d, False, seed=79)


@pytest.mark.parametrize("d", [64, 128])
def test_stress_distribution_full(d):
    """Large logits (std 4): exercises the running-max rescale across blocks."""
    full_case(1, 4, 1024, d, True, seed=5, dist="stress")
    full_case(1, 4, 1024, d, False, seed=6, dist="stress")


def test_growing_maximum_forces_rescales():
    """Logits that grow along the key axis: every block raises the running max by more than
    the rescale slack, so the rescale path runs on every block."""
    N, d = 512, 128
    q = torch.ones(1, 2, N, d)
    k = (torch.arange(N, dtype=torch.float32) / 16.0)[None, None, :, None].expand(1, 2, N, d).contiguous()
    g = torch.Generator().manual_seed(3)
    v = torch.randn(1, 2, N, d, generator=g)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    c = float(np.float32(0.08))  # the float32 value the library receives (reading R5)
    for causal in (False, True):
        o, lse = run_gpu(q, k, v, causal, c)
        ro, rl = attention_fp64(q, k, v, causal=causal, scale=c)
        check(o, lse, ro, rl, f"growing max causal={causal}")


# ---- closed-form special cases on the GPU ---------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
def test_single_key(d):
    q, k, v = W.make_inputs(3, 2, 1, d, seed=11)
    o, lse = run_gpu(q, k, v, False, 0.3)
    assert (o - v.float()).abs().max().item() <= 1e-5 * max(1.0, v.float().abs().max().item())
    want = 0.3 * (q.double() * k.double()).sum(-1)
    assert (lse.double() - want).abs().max().item() < 1e-4


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(causal):
    q, k, _ = W.make_inputs(1, 2, 300, 128, seed=12, dist="stress")
    u = torch.linspace(-1, 1, 128).to(torch.bfloat16)
    v = u.expand(1, 2, 300, 128).contiguous()
    o, _ = run_gpu(q, k, v, causal, W.fp32_scale(128))
    assert (o - u.float()).abs().max().item() < 4e-3


@pytest.mark.parametrize("causal", [False, True])
def test_zero_logits_average_v(causal):
    """Q = 0 or scale = 0: uniform weights over the visible keys."""
    N, d = 200, 64
    _, k, v = W.make_inputs(1, 1, N, d, seed=13)
    counts = torch.arange(1, N + 1, dtype=torch.float64)
    for q, scale in ((torch.zeros(1, 1, N, d, dtype=torch.bfloat16), 0.125), (W.make_inputs(1, 1, N, d, 14)[0], 0.0)):
        o, lse = run_gpu(q, k, v, causal, scale)
        if causal:
            want_o = torch.cumsum(v[0, 0].double(), 0) / counts[:, None]
            want_l = torch.log(counts)
        else:
            want_o = v[0, 0].double().mean(0).expand(N, d)
            want_l = torch.full((N,), math.log(N), dtype=torch.float64)
        assert (o[0, 0].double() - want_o).abs().max().item() < 2e-2
        assert (lse[0, 0].double() - want_l).abs().max().item() < 1e-4


@pytest.mark.parametrize("d", [64, 128])
def test_negative_and_odd_scales(d):
    q, k, v = W.make_inputs(1, 2, 333, d, seed=15)
    for scale in (-0.2, 0.5, 1e-3, -1.0 / math.sqrt(d)):
        scale = float(np.float32(scale))  # the float32 value the library receives (reading R5)
        for causal in (False, True):
            o, lse = run_gpu(q, k, v, causal, scale)
            ro, rl = attention_fp64(q, k, v, causal=causal, scale=scale)
            check(o, lse, ro, rl, f"scale={scale} causal={causal}")


# ---- kernel hygiene ----------------------------------------------------------------------

def test_outputs_fully_overwritten():
    q, k, v = W.make_inputs(2, 3, 515, 128, seed=16)
    for causal in (False, True):
        o, lse = run_gpu(q, k, v, causal, W.fp32_scale(128), poison=True)
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_bitwise_deterministic():
    q, k, v = W.make_inputs(2, 4, 1000, 128, seed=17)
    a = run_gpu(q, k, v, True, W.fp32_scale(128))
    b = run_gpu(q, k, v, True, W.fp32_scale(128))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("cut", [0, 63, 100, 511])
def test_causal_prefix_bitwise_invariance(cut):
    """Rows <= cut never depend on keys/values after cut: changing those leaves rows <= cut
    bitwise identical (masked weights are exactly zero; blocks above the diagonal are not read)."""
    q, k, v = W.make_inputs(1, 2, 600, 128, seed=18)
    a_o, a_l = run_gpu(q, k, v, True, W.fp32_scale(128))
    k2, v2 = k.clone(), v.clone()
    k2[:, :, cut + 1:] = (torch.randn(k2[:, :, cut + 1:].shape) * 30).to(torch.bfloat16)
    v2[:, :, cut + 1:] = (torch.randn(v2[:, :, cut + 1:].shape) * 1000).to(torch.bfloat16)
    b_o, b_l = run_gpu(q, k2, v2, True, W.fp32_scale(128))
    assert torch.equal(a_o[:, :, : cut + 1], b_o[:, :, : cut + 1])
    assert torch.equal(a_l[:, :, : cut + 1], b_l[:, :, : cut + 1])


def test_side_stream_and_async_launch():
    """The launch goes on torch's current stream; results are right after syncing that stream."""
    from io_aware_softmax_mifa_amd import binding

    q, k, v = W.make_inputs(1, 4, 700, 64, seed=19)
    ro, rl = attention_fp64(q, k, v, causal=True, scale=0.125)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dq, dk, dv = (t.cuda(non_blocking=False) for t in (q, k, v))
        o, lse = binding.attention(dq, dk, dv, causal=True, scale=0.125)
    s.synchronize()
    check(o.cpu(), lse.cpu(), ro, rl, "side stream")


def test_raw_abi_pointers_and_errors():
    from io_aware_softmax_mifa_amd import binding

    q, k, v = (t.cuda() for t in W.make_inputs(1, 1, 64, 64, seed=20))
    o = torch.empty(1, 1, 64, 64, device="cuda")
    lse = torch.empty(1, 1, 64, device="cuda")
    st = binding.mifa_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 1, 64, 64,
                              0, 0.125, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    ro, rl = attention_fp64(q.cpu(), k.cpu(), v.cpu(), scale=0.125)
    check(o.cpu(), lse.cpu(), ro, rl, "raw ABI")
    with pytest.raises(binding.MifaError):
        binding.mifa_fwd(q, k, v, o, lse, 1, 1, 64, 96, 0, 0.125)
