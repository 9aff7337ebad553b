"""GPU parity of the row softmax (mifa_softmax_rows, through the C ABI) against the float64
CPU oracle.

Tolerances, derived from the arithmetic: the kernel works in fp32 (one FMA for c*x, v_exp_f32,
fp32 sums of at most 64 terms per thread then a tree, one reciprocal), so an fp32 output is
within a few 1e-6 relative of the exact value; the bar is 3e-5 relative.  A bf16 output adds
one round-to-nearest-even (at most 2^-8 relative: 8 significant bits), so its bar is 4e-3 relative.  LSE is fp32 with
the max exact up to the product rounding: 2e-5 absolute plus 1e-6 relative.  Outputs that
underflow fp32 are compared with an absolute floor of 1e-30.
"""
import numpy as np
import pytest
import torch

from io_aware_softmax_mifa_amd import workloads as W
from oracle import softmax_rows_fp64

pytestmark = pytest.mark.gpu

RTOL = {"f32": 3e-5, "bf16": 4e-3}
LSE_ATOL, LSE_RTOL = 2e-5, 1e-6


def say(msg):
    print(f"[softmax parity] {msg}", flush=True)


def check(y_gpu, lse_gpu, y_ref, lse_ref, dtype, what):
    y = y_gpu.float().cpu().double().numpy() if hasattr(y_gpu, "cpu") else y_gpu
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = np.abs(y - y_ref)
    bound = RTOL[dtype] * np.abs(y_ref) + 1e-30
    worst = (err / np.maximum(np.abs(y_ref), 1e-30)).max()
    say(f"{what}: max rel err {worst:.3e}")
    assert (err <= bound).all(), f"{what}: y error {err.max()} (worst relative {worst})"
    np.testing.assert_allclose(y.sum(axis=-1), 1.0, atol=max(1e-5, RTOL[dtype] * 2))
    if lse_gpu is not None:
        l = lse_gpu.cpu().double().numpy()
        lerr = np.abs(l - lse_ref)
        assert (lerr <= LSE_ATOL + LSE_RTOL * np.abs(lse_ref)).all(), f"{what}: lse error {lerr.max()}"


def run(x, scale, out=None, with_lse=True):
    from io_aware_softmax_mifa_amd import binding

    y, lse = binding.softmax_rows(x, scale=scale, out=out, with_lse=with_lse)
    torch.cuda.synchronize()
    return y, lse


def full_case(rows, cols, dtype, std, seed, scale=1.0):
    x = W.make_softmax_input(rows, cols, dtype, std, seed)
    scale = float(np.float32(scale))  # the float32 value the library receives
    say(f"rows={rows} cols={cols} dtype={dtype} std={std} seed={seed} scale={scale}")
    y, lse = run(x.cuda(), scale)
    yr, lr = softmax_rows_fp64(x, scale)
    check(y, lse, yr, lr, dtype, f"{rows}x{cols} {dtype}")


# ---- every launch shape and the ragged lengths around its limits ----------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cols", [1, 2, 7, 8, 63, 64, 65, 255, 256, 511, 512, 513, 1000, 2047, 2048, 4095, 4096,
                                  4097, 8191, 8192, 16383, 16384, 16385, 20000, 32767, 32768, 32769, 40000,
                                  65536, 65537, 100003, 131072, 131073])
def test_lengths(cols, dtype):
    full_case(5, cols, dtype, 2.0, seed=cols)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_row_counts_not_multiple_of_four(dtype):
    for rows in (1, 2, 3, 5, 7, 1023):
        full_case(rows, 300, dtype, 1.0, seed=rows)


# ---- the seeded workloads: full launch, sampled rows against the oracle -----------------------

@pytest.mark.parametrize("name", ["SM1", "SM2", "SM3", "SM4", "SM5"])
def test_workloads_sampled(name):
    w = W.softmax_by_name(name)
    x = W.make_softmax_input(w.rows, w.cols, w.dtype, w.std, w.seed)
    say(f"{name}: rows={w.rows} cols={w.cols} dtype={w.dtype}")
    y, lse = run(x.cuda(), w.scale)
    rows = W.sample_softmax_rows(w.rows, 64, w.seed)
    yr, lr = softmax_rows_fp64(x[rows], w.scale)
    check(y[rows.cuda()], lse[rows.cuda()], yr, lr, w.dtype, f"{name} 64 sampled rows")
    assert torch.isfinite(y).all() and torch.isfinite(lse).all()


# ---- special cases -----------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [0.0, -0.7, 1e-30, 3.0])
def test_scales(dtype, scale):
    full_case(4, 1500, dtype, 1.0, seed=11, scale=scale)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cols", [100, 3000, 20000])
def test_huge_logits(dtype, cols):
    """Logits of magnitude 1e4: exponentiating without the max shift would overflow."""
    full_case(3, cols, dtype, 1e4, seed=5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cols", [37, 3000, 20000])
def test_masked_entries(dtype, cols):
    """-inf entries take no weight, for positive, zero and negative scales."""
    x = W.make_softmax_input(4, cols, dtype, 1.0, seed=9)
    g = torch.Generator().manual_seed(3)
    mask = torch.rand(4, cols, generator=g) < 0.3
    mask[:, 0] = False
    x[mask] = float("-inf")
    for scale in (1.0, 0.0, -2.0):
        y, lse = run(x.cuda(), scale)
        yr, lr = softmax_rows_fp64(x, scale)
        assert (y.float().cpu()[mask] == 0).all()
        check(y, lse, yr, lr, dtype, f"masked cols={cols} scale={scale}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cols", [64, 4096, 16384, 20000, 65536, 140000])
def test_in_place_and_no_lse(dtype, cols):
    """y = x: every launch shape, including the 1024-thread resident rows (65,536) and the
    streamed rows (140,000: two passes over x, the second writing over it)."""
    x = W.make_softmax_input(6, cols, dtype, 2.0, seed=21)
    yr, lr = softmax_rows_fp64(x, 0.5)
    d = x.cuda()
    y, lse = run(d, 0.5, out=d, with_lse=False)
    assert lse is None and y.data_ptr() == d.data_ptr()
    check(y, None, yr, lr, dtype, f"in place cols={cols}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cols", [64, 4096, 20000])
def test_unaligned_base(dtype, cols):
    """A base address that is only element-aligned takes the element-load path."""
    x = W.make_softmax_input(1, 3 * cols + 1, dtype, 1.0, seed=31)
    d = x.cuda()[0, 1:].view(3, cols)  # one element past a 16-byte boundary
    assert d.data_ptr() % 16 != 0
    y, lse = run(d, 1.0)
    yr, lr = softmax_rows_fp64(x[0, 1:].view(3, cols), 1.0)
    check(y, lse, yr, lr, dtype, f"unaligned cols={cols}")


def test_bitwise_deterministic():
    x = W.make_softmax_input(64, 5000, "f32", 2.0, seed=41).cuda()
    y1, l1 = run(x, 1.0)
    y2, l2 = run(x, 1.0)
    assert torch.equal(y1, y2) and torch.equal(l1, l2)


def test_raw_abi_errors():
    from io_aware_softmax_mifa_amd import binding

    x = torch.zeros(4, 8, device="cuda")
    with pytest.raises(binding.MifaError) as e:
        binding.mifa_softmax_rows(x, x, None, 4, 8, 5, 1.0)
    assert e.value.status == 8
