"""The C ABI on a machine without a GPU: the library loads, exports every symbol the header
declares, and rejects every invalid argument before any HIP call (so no device is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mifa.h")
LIB = os.path.join(ROOT, "io_aware_softmax_mifa_amd", "libmifa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmifa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mifa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_api():
    assert declared_functions() == ["mifa_attention", "mifa_attention_splitkv", "mifa_attention_splitkv_noalloc",
                                    "mifa_attention_strided", "mifa_bwd",
                                    "mifa_bwd_strided", "mifa_bwd_workspace_bytes", "mifa_clock_probe", "mifa_fwd",
                                    "mifa_last_hip_error", "mifa_softmax_rows", "mifa_splitkv_workspace_bytes",
                                    "mifa_status_string", "mifa_version"]


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name


@pytest.fixture(scope="module")
def lib():
    from io_aware_softmax_mifa_amd import binding

    return binding


def test_version_and_status_strings(lib):
    assert lib.mifa_version().startswith("mifa ")
    assert "gfx950" in lib.mifa_version()
    for code in range(11):
        s = lib.mifa_status_string(code)
        assert s and s != "unknown status"
    assert lib.mifa_status_string(99) == "unknown status"
    assert lib.mifa_status_string(-1) == "unknown status"
    assert lib.mifa_last_hip_error() == 0


A = 1 << 20  # a fake, 16-byte aligned "device" address; never dereferenced on these paths


@pytest.mark.parametrize(
    "args,status",
    [
        ((0, A, A, A, A, 1, 1, 128, 64, 0, 0.125), 1),
        ((A, 0, A, A, A, 1, 1, 128, 64, 0, 0.125), 1),
        ((A, A, 0, A, A, 1, 1, 128, 64, 0, 0.125), 1),
        ((A, A, A, 0, A, 1, 1, 128, 64, 0, 0.125), 1),
        ((A, A, A, A, 0, 1, 1, 128, 64, 0, 0.125), 1),
        ((A, A, A, A, A, 0, 1, 128, 64, 0, 0.125), 2),
        ((A, A, A, A, A, 1, 0, 128, 64, 0, 0.125), 2),
        ((A, A, A, A, A, 1, 1, 0, 64, 0, 0.125), 2),
        ((A, A, A, A, A, -3, 1, 128, 64, 0, 0.125), 2),
        ((A, A, A, A, A, 1, 1, 128, 32, 0, 0.125), 3),
        ((A, A, A, A, A, 1, 1, 128, 96, 1, 0.125), 3),
        ((A, A, A, A, A, 1, 1, 128, 256, 0, 0.125), 3),
        ((A + 2, A, A, A, A, 1, 1, 128, 64, 0, 0.125), 4),
        ((A, A + 8, A, A, A, 1, 1, 128, 64, 0, 0.125), 4),
        ((A, A, A + 4, A, A, 1, 1, 128, 64, 0, 0.125), 4),
        ((A, A, A, A + 12, A, 1, 1, 128, 64, 0, 0.125), 4),
        ((A, A, A, A, A + 2, 1, 1, 128, 64, 0, 0.125), 4),
        ((A, A, A, A, A, 1, 1, 128, 64, 0, float("nan")), 5),
        ((A, A, A, A, A, 1, 1, 128, 64, 1, float("inf")), 5),
        ((A, A, A, A, A, 1, 1, 128, 64, 0, float("-inf")), 5),
        ((A, A, A, A, A, 1, 1, 1 << 24, 128, 0, 0.1), 6),
        ((A, A, A, A, A, 1 << 20, 1 << 12, 1 << 10, 64, 0, 0.1), 6),
    ],
)
def test_validation_rejects_before_any_hip_call(lib, args, status):
    got = lib.mifa_fwd_raw(*args, None)
    assert got == status, (args, got, lib.mifa_status_string(got))


def test_validation_order_null_before_shape(lib):
    # Several problems at once: the first failing check in the documented order wins.
    assert lib.mifa_fwd_raw(0, A, A, A, A, 0, 0, 0, 7, 0, float("nan"), None) == 1
    assert lib.mifa_fwd_raw(A, A, A, A, A, 0, 1, 1, 7, 0, float("nan"), None) == 2
    assert lib.mifa_fwd_raw(A, A, A, A, A, 1, 1, 1, 7, 0, float("nan"), None) == 3
    assert lib.mifa_fwd_raw(A + 1, A, A, A, A, 1, 1, 1, 64, 0, float("nan"), None) == 4


def test_binding_python_checks(lib):
    import torch

    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lib.attention(q, q, q)  # CPU tensors are rejected before any call


# ---- mifa_softmax_rows ------------------------------------------------------------------------

@pytest.mark.parametrize(
    "args,status",
    [
        ((0, A, A, 4, 64, 0, 1.0), 1),
        ((A, 0, A, 4, 64, 0, 1.0), 1),
        ((A, A, A, 0, 64, 0, 1.0), 2),
        ((A, A, A, 4, 0, 1, 1.0), 2),
        ((A, A, A, -1, 64, 0, 1.0), 2),
        ((A, A, A, 4, 64, 2, 1.0), 8),
        ((A, A, A, 4, 64, -1, 1.0), 8),
        ((A + 1, A, A, 4, 64, 0, 1.0), 4),
        ((A, A + 2, A, 4, 64, 1, 1.0), 4),
        ((A, A, A + 2, 4, 64, 0, 1.0), 4),
        ((A, A, A, 4, 64, 0, float("nan")), 5),
        ((A, A, A, 4, 64, 1, float("inf")), 5),
        ((A, A, A, 1 << 31, 64, 0, 1.0), 6),
        ((A, A, A, 4, 1 << 31, 1, 1.0), 6),
    ],
)
def test_softmax_validation_rejects_before_any_hip_call(lib, args, status):
    got = lib.mifa_softmax_rows_raw(*args, None)
    assert got == status, (args, got, lib.mifa_status_string(got))


def test_softmax_validation_order(lib):
    assert lib.mifa_softmax_rows_raw(0, A, A, 0, 0, 9, float("nan"), None) == 1
    assert lib.mifa_softmax_rows_raw(A, A, A, 0, 1, 9, float("nan"), None) == 2
    assert lib.mifa_softmax_rows_raw(A, A, A, 1, 1, 9, float("nan"), None) == 8
    assert lib.mifa_softmax_rows_raw(A + 1, A, A, 1, 1, 0, float("nan"), None) == 4
    # bf16 needs 2-byte alignment only; an odd address is rejected, an even one passes this check
    assert lib.mifa_softmax_rows_raw(A + 2, A, A, 1, 1, 0, float("nan"), None) == 5
    # a NULL lse is allowed (the check moves on to the scale)
    assert lib.mifa_softmax_rows_raw(A, A, 0, 1, 1, 1, float("nan"), None) == 5


def test_softmax_binding_python_checks(lib):
    import torch

    with pytest.raises(ValueError):
        lib.softmax_rows(torch.zeros(2, 8))  # CPU tensors are rejected before any call


# ---- mifa_attention and mifa_attention_splitkv -----------------------------------------------

@pytest.mark.parametrize(
    "args,status",
    [
        ((0, A, A, A, A, 1, 1, 4, 64, 64, 0, 0.125), 1),
        ((A, A, A, A, A, 1, 1, 0, 64, 64, 0, 0.125), 2),
        ((A, A, A, A, A, 1, 1, 4, 0, 64, 0, 0.125), 2),
        ((A, A, A, A, A, 1, 1, 65, 64, 64, 1, 0.125), 2),   # causal needs Nq <= Nk
        ((A, A, A, A, A, 1, 1, 4, 64, 96, 0, 0.125), 3),
        ((A, A, A + 4, A, A, 1, 1, 4, 64, 64, 0, 0.125), 4),
        ((A, A, A, A, A, 1, 1, 4, 64, 64, 0, float("nan")), 5),
        ((A, A, A, A, A, 1, 1, 4, 1 << 24, 128, 0, 0.1), 6),
    ],
)
def test_attention_validation(lib, args, status):
    got = lib.mifa_attention_raw(*args, None)
    assert got == status, (args, got, lib.mifa_status_string(got))
    got = lib.mifa_attention_splitkv_raw(*args, A, 1 << 40, None)
    assert got == status, (args, got, lib.mifa_status_string(got))


def test_attention_accepts_rectangular_noncausal_more_queries(lib):
    # Nq > Nk is fine without the causal mask: validation passes up to the workspace check
    assert lib.mifa_attention_splitkv_raw(A, A, A, A, A, 1, 1, 100, 10, 64, 0, 0.1, 0, 0, None) == 9


def test_splitkv_workspace_checks(lib):
    need = lib.mifa_splitkv_workspace_bytes(1, 8, 1, 32768, 128)
    assert need > 0
    args = (A, A, A, A, A, 1, 8, 1, 32768, 128, 1, 0.1)
    assert lib.mifa_attention_splitkv_raw(*args, 0, need, None) == 9          # NULL
    assert lib.mifa_attention_splitkv_raw(*args, A + 8, need, None) == 9      # misaligned
    assert lib.mifa_attention_splitkv_raw(*args, A, need - 1, None) == 9      # too small
    # argument errors come first
    assert lib.mifa_attention_splitkv_raw(A, A, A, A, A, 1, 8, 2, 1, 128, 1, 0.1, 0, 0, None) == 2


def test_splitkv_noalloc_checks(lib):
    # argument errors first, then the 32 MiB limit of the static scratch array (no HIP call before)
    assert lib.mifa_attention_splitkv_noalloc_raw(0, A, A, A, A, 1, 8, 1, 32768, 128, 1, 0.1, None) == 1
    assert lib.mifa_attention_splitkv_noalloc_raw(A, A, A, A, A, 1, 8, 2, 1, 128, 1, 0.1, None) == 2
    big = (1, 8, 512, 65536, 128)
    assert lib.mifa_splitkv_workspace_bytes(*big) > 32 << 20
    assert lib.mifa_attention_splitkv_noalloc_raw(A, A, A, A, A, *big, 1, 0.1, None) == 11
    assert "32 MiB" in lib.mifa_status_string(11)


def test_clock_probe_checks(lib):
    # null pointers, the span's range and alignment are checked before any HIP call
    assert lib.mifa_clock_probe_raw(0, 1000, None) == (1, 0)
    assert lib.mifa_clock_probe_raw(A, 0, None) == (2, 0)
    assert lib.mifa_clock_probe_raw(A, 2_000_001, None) == (2, 0)
    assert lib.mifa_clock_probe_raw(A + 4, 1000, None) == (4, 0)


def test_splitkv_workspace_bytes(lib):
    assert lib.mifa_splitkv_workspace_bytes(0, 1, 1, 10, 64) == 0
    assert lib.mifa_splitkv_workspace_bytes(1, 1, 1, 10, 96) == 0
    # few queries, many keys: several ranges, each holding O (d floats) and LSE per row
    n = lib.mifa_splitkv_workspace_bytes(2, 4, 3, 65536, 64)
    assert n > 0 and n % (2 * 4 * 3 * (64 + 1) * 4) == 0


# ---- mifa_bwd --------------------------------------------------------------------------------

def _bwd(lib, q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A, B=1, H=2, Nq=100, Nk=100, d=128, causal=1,
         scale=0.1, ws=A, wsb=1 << 40):
    return lib.mifa_bwd_raw(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nk, d, causal, scale, ws, wsb, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=0), 1), (dict(o=0), 1), (dict(lse=0), 1), (dict(do=0), 1), (dict(dq=0), 1), (dict(dk=0), 1),
        (dict(dv=0), 1),
        (dict(B=0), 2), (dict(Nq=0), 2), (dict(Nk=0), 2), (dict(Nq=101), 2),
        (dict(d=96), 3),
        (dict(do=A + 8), 4), (dict(dk=A + 4), 4), (dict(o=A + 2), 4), (dict(lse=A + 2), 4),
        (dict(scale=float("inf")), 5),
        (dict(Nq=1 << 24, Nk=1 << 24), 6),
        (dict(ws=0), 9), (dict(ws=A + 8), 9), (dict(wsb=2 * 100 * 8 - 1), 9),
    ],
)
def test_bwd_validation(lib, kw, status):
    got = _bwd(lib, **kw)
    assert got == status, (kw, got, lib.mifa_status_string(got))


def test_bwd_validation_order(lib):
    assert _bwd(lib, q=0, Nq=0, ws=0) == 1      # NULL before shape
    assert _bwd(lib, Nq=0, d=96) == 2            # shape before d
    assert _bwd(lib, d=96, q=A + 2) == 3         # d before alignment
    assert _bwd(lib, scale=float("nan"), ws=0) == 5  # arguments before the workspace
    assert _bwd(lib, causal=0, Nq=101, ws=0) == 9    # Nq > Nk is fine without the causal mask


def test_bwd_workspace_bytes(lib):
    assert lib.mifa_bwd_workspace_bytes(0, 1, 1) == 0
    assert lib.mifa_bwd_workspace_bytes(2, 3, 5) == 2 * 3 * 5 * 8


# ---- the strided entry points ----------------------------------------------------------------

def _dense(H, Nq, Nk, d):
    sq, sk = [H * Nq * d, Nq * d, d], [H * Nk * d, Nk * d, d]
    return sq, sk


def _fwd_strided(lib, strides="dense", o_dtype=1, q=A, Nq=100, Nk=100, d=128, causal=1, scale=0.1):
    if strides == "dense":
        sq, sk = _dense(2, Nq, Nk, d)
        strides = sq + sk + sk + sq
    return lib.mifa_attention_strided_raw(q, A, A, A, A, 1, 2, Nq, Nk, d, strides, o_dtype, causal, scale, None)


def test_attention_strided_validation(lib):
    sq, sk = _dense(2, 100, 100, 128)
    assert _fwd_strided(lib, strides=None) == 1                  # NULL strides
    assert _fwd_strided(lib, q=0) == 1
    assert _fwd_strided(lib, Nq=101) == 2                        # causal needs Nq <= Nk
    assert _fwd_strided(lib, d=96) == 3
    assert _fwd_strided(lib, q=A + 8) == 4
    assert _fwd_strided(lib, scale=float("nan")) == 5
    assert _fwd_strided(lib, o_dtype=7) == 8
    bad = sq + sk + sk + sq
    bad[4] = -128                                                # negative head stride of k
    assert _fwd_strided(lib, strides=bad) == 10
    bad = sq + sk + sk + sq
    bad[2] = 132                                                 # row stride not a multiple of 8
    assert _fwd_strided(lib, strides=bad) == 4
    bad = sq + sk + sk + sq
    bad[5] = 1 << 24                                             # row stride too large
    assert _fwd_strided(lib, strides=bad) == 6
    # order: dtype before strides, strides after the scale
    assert _fwd_strided(lib, o_dtype=7, strides=[-8] * 12) == 8
    assert _fwd_strided(lib, scale=float("inf"), strides=[-8] * 12) == 5


def _bwd_strided(lib, strides="dense", o_dtype=1, g_dtype=1, ws=A, wsb=1 << 40, dq=A, Nq=100, causal=1):
    if strides == "dense":
        sq, sk = _dense(2, Nq, 100, 128)
        strides = sq + sk + sk + sq + sq + sq + sk + sk
    return lib.mifa_bwd_strided_raw(A, A, A, A, A, A, dq, A, A, 1, 2, Nq, 100, 128, strides, o_dtype, g_dtype,
                                    causal, 0.1, ws, wsb, None)


def test_bwd_strided_validation(lib):
    sq, sk = _dense(2, 100, 100, 128)
    dense = sq + sk + sk + sq + sq + sq + sk + sk
    assert _bwd_strided(lib, strides=None) == 1
    assert _bwd_strided(lib, dq=0) == 1
    assert _bwd_strided(lib, Nq=101) == 2
    assert _bwd_strided(lib, o_dtype=5) == 8
    assert _bwd_strided(lib, g_dtype=-1) == 8
    bad = list(dense)
    bad[13] = -8                                                 # dO head stride
    assert _bwd_strided(lib, strides=bad) == 10
    bad = list(dense)
    bad[23] = 4                                                  # dv row stride
    assert _bwd_strided(lib, strides=bad) == 4
    assert _bwd_strided(lib, ws=0) == 9
    assert _bwd_strided(lib, ws=0, strides=bad) == 4             # strides before the workspace


def test_sdpa_argument_checks_need_no_gpu(lib):
    import torch
    from torch.nn.attention.bias import causal_upper_left

    from io_aware_softmax_mifa_amd.sdpa import scaled_dot_product_attention as sdpa

    x = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sdpa(x, x, x)                                   # CPU tensors
    with pytest.raises(ValueError):
        sdpa(x.float(), x, x)
    with pytest.raises(ValueError):
        sdpa(x[0], x, x)                                # not 4-D
    assert torch.ops.mifa.attention_fwd is not None and torch.ops.mifa.attention_bwd is not None
    assert causal_upper_left(8, 8) is not None
