"""GPU parity of the attention backward (mifa_bwd, through the C ABI) against the float64 CPU
oracle of the gradients.

Tolerance, from the arithmetic: q, k, v and dO are bf16 and every product is exact; sums are
float32 (relative error ~1e-6).  P and dS are rounded to bf16 before the products
dV = P^T dO, dQ = c dS K and dK = c dS^T Q; bf16 keeps 8 significant bits, so each rounding
is at most u = 2^-8 relative.  With rounding errors of random sign the RMS error of an output
is about u/sqrt(3) ~ 2.3e-3 of its terms' root-sum-square (measured: 1.5e-3 .. 1.8e-3 of the
output RMS); when every weight is equal (scale 0) the errors share one sign and reach u of
the output.  Hence: RMS error <= 5e-3 * RMS(ref) (u plus margin) and max-abs error
<= 1e-2 * max|ref| per gradient.  A gradient that is exactly zero in float64 (one key) must
come out below 1e-5 absolute: there the two float32 sums D = dO . O and dP = dO . v, equal in
exact arithmetic, differ by their rounding (~1e-7 for unit-size data).  Both the backward
alone (O and LSE from the oracle's forward, in float32) and the two passes end to end (O and
LSE from the GPU forward) are checked.
"""
import numpy as np
import pytest
import torch

from io_aware_softmax_mifa_amd import workloads as W
from oracle import attention_bwd_fp64, attention_fp64

pytestmark = pytest.mark.gpu

REL_MAX, REL_RMS = 1e-2, 5e-3


def say(msg):
    print(f"[parity-bwd] {msg}", flush=True)


def check_grads(got, ref, what):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.double().numpy()
        assert np.isfinite(g).all(), f"{what}: {name} non-finite"
        err = np.abs(g - r)
        ref_max = max(np.abs(r).max(), 1e-30)
        ref_rms = max(np.sqrt((r * r).mean()), 1e-30)
        rms = np.sqrt((err * err).mean())
        say(f"{what}: {name} max {err.max():.3e} (ref max {ref_max:.3e})  rms {rms:.3e} (ref rms {ref_rms:.3e})")
        if np.abs(r).max() == 0.0:
            assert err.max() <= 1e-5, f"{what}: {name} should be zero"
            continue
        assert err.max() <= REL_MAX * ref_max, f"{what}: {name} max-abs {err.max()} vs {ref_max}"
        assert rms <= REL_RMS * ref_rms, f"{what}: {name} rms {rms} vs {ref_rms}"


def gpu_bwd(q, k, v, o, lse, do, causal, scale):
    from io_aware_softmax_mifa_amd import binding

    args = [t.cuda().contiguous() for t in (q, k, v, o, lse, do)]
    dq, dk, dv = binding.attention_backward(*args, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def case(B, H, Nq, Nk, d, causal, seed, scale=None, dist="normal", end_to_end=False):
    from io_aware_softmax_mifa_amd import binding

    q, k, v = W.make_rect_inputs(B, H, Nq, Nk, d, seed, dist)
    do = W.make_grad_output(B, H, Nq, d, seed)
    scale = W.fp32_scale(d) if scale is None else float(np.float32(scale))  # as the library receives it
    what = f"B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} seed={seed} scale={scale:g} e2e={end_to_end}"
    say(what)
    rdq, rdk, rdv, rlse = attention_bwd_fp64(q, k, v, do, causal=causal, scale=scale)
    if end_to_end:
        o, lse = binding.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
        torch.cuda.synchronize()
        o, lse = o.cpu(), lse.cpu()
    else:
        ro, rl = attention_fp64(q, k, v, causal=causal, scale=scale)
        o, lse = torch.from_numpy(ro).float(), torch.from_numpy(rl).float()
    got = gpu_bwd(q, k, v, o, lse, do, causal, scale)
    check_grads(got, (rdq, rdk, rdv), what)


SHAPES = [
    # B, H, Nq, Nk, d, causal, seed
    (1, 2, 300, 300, 128, True, 1),     # several 128-row tiles and 64-row blocks, ragged tail
    (1, 2, 300, 300, 128, False, 2),
    (2, 3, 257, 257, 64, True, 3),
    (2, 3, 200, 200, 64, False, 4),
    (1, 1, 1, 1, 64, False, 5),          # one query, one key
    (1, 1, 1, 1, 128, True, 6),
    (1, 2, 65, 65, 128, True, 7),
    (1, 2, 128, 128, 64, True, 8),       # exactly one tile
    (1, 2, 100, 333, 128, True, 9),      # fewer queries than keys (bottom-right causal)
    (1, 2, 7, 500, 64, True, 10),
    (1, 2, 333, 100, 64, False, 11),     # more queries than keys
    (2, 4, 1024, 1024, 128, True, 12),
    (1, 4, 1024, 1024, 64, False, 13),
    (1, 2, 129, 129, 128, True, 14),     # last query block holds one row
    (1, 2, 192, 192, 128, False, 15),    # exactly three blocks: each buffer of the ring once
    (1, 2, 64, 64, 64, True, 16),        # exactly one block: the pipeline's prologue and epilogue only
    (1, 1, 4096, 4096, 64, True, 17),    # up to 64 blocks per key tile: the ring wraps many times
    (1, 16, 4160, 4160, 64, True, 18),   # 272 long dq tiles: the 8-wave dq kernel and its 4-buffer ring
    (1, 16, 4096, 4096, 64, False, 19),  # no mask, exactly 256 long dq tiles: the 8-wave dq kernel
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:5])) + ("c" if s[5] else "n"))
def test_backward_matches_oracle(shape):
    case(*shape)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_end_to_end(d, causal):
    case(1, 3, 700, 700, d, causal, 20 + d + causal, end_to_end=True)


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.3])
def test_backward_scales(scale):
    case(1, 2, 260, 260, 128, True, 30, scale=scale)
    case(1, 2, 190, 190, 64, False, 31, scale=scale)


def test_backward_stress_inputs():
    case(1, 2, 520, 520, 128, True, 40, dist="stress")


def test_backward_is_deterministic():
    from io_aware_softmax_mifa_amd import binding

    q, k, v = W.make_inputs(1, 4, 777, 128, 50)
    do = W.make_grad_output(1, 4, 777, 128, 50)
    q, k, v, do = (t.cuda() for t in (q, k, v, do))
    o, lse = binding.attention(q, k, v, causal=True)
    a = binding.attention_backward(q, k, v, o, lse, do, causal=True)
    b = binding.attention_backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_full_size_sampled():
    """B=1 H=32 N=16384 d=128 causal (the benchmarked backward workload, dense float32 entry
    point as the bench calls it): 64 sampled dq rows over all heads and 2 x 32 sampled dk, dv
    rows against the oracle's sampled-rows form."""
    from io_aware_softmax_mifa_amd import binding
    from oracle import attention_bwd_fp64_rows

    w = W.by_name("C4")
    q, k, v = W.make_workload_inputs(w)
    do = W.make_grad_output(w.B, w.H, w.N, w.d, w.seed)
    scale = W.fp32_scale(w.d)
    say(f"full size: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} seed={w.seed}")
    gq, gk, gv, gdo = (t.cuda() for t in (q, k, v, do))
    o, lse = binding.attention(gq, gk, gv, causal=w.causal, scale=scale)
    dq, dk, dv = binding.attention_backward(gq, gk, gv, o, lse, gdo, causal=w.causal, scale=scale)
    torch.cuda.synchronize()
    q_rows = W.sample_rows(w.B, w.H, w.N, 64, w.seed + 11)
    k_rows = W.sample_rows_in_heads(w.B, w.H, w.N, 2, 32, w.seed + 12)

    def pick(t, rows):
        r = rows.cuda()
        return t[r[:, 0], r[:, 1], r[:, 2]].cpu()

    got_q = pick(dq, q_rows)
    got_k, got_v = pick(dk, k_rows), pick(dv, k_rows)
    rdq, rdk, rdv = attention_bwd_fp64_rows(q, k, v, do, q_rows, k_rows, causal=w.causal, scale=scale)
    check_grads((got_q, got_k, got_v), (rdq, rdk, rdv), "C4 sampled rows")


# ---- the dq kernel's launch rule at its edges ------------------------------------------------
# 8-wave dq workgroups (256 query rows) when causal with Nq > 4096 and more than 256 of them, or
# without the mask with Nq >= 4096 and at least 256; 4-wave ones (128 rows) otherwise.  Each
# case checks every gradient row of two heads (first and last) against the oracle run on those
# heads alone (heads are independent).
DQ_EDGES = [
    # B, H, N, d, causal, shape
    (1, 16, 4097, 64, True, "causal, 272 tiles of 256 rows: 8-wave dq"),
    (1, 15, 4097, 64, True, "causal, 255 tiles of 256 rows: 4-wave dq"),
    (1, 16, 4096, 64, False, "non-causal, exactly 256 tiles: 8-wave dq"),
    (1, 15, 4096, 64, False, "non-causal, 240 tiles: 4-wave dq"),
]


@pytest.mark.parametrize("B,H,N,d,causal,shape", DQ_EDGES, ids=[c[5] for c in DQ_EDGES])
def test_dq_launch_rule_edges(B, H, N, d, causal, shape):
    from io_aware_softmax_mifa_amd import binding

    q, k, v = W.make_inputs(B, H, N, d, seed=7100 + H + N)
    do = W.make_grad_output(B, H, N, d, seed=7100 + H + N)
    scale = W.fp32_scale(d)
    say(f"B={B} H={H} N={N} d={d} causal={causal}: {shape}")
    o, lse = binding.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    got = gpu_bwd(q, k, v, o.cpu(), lse.cpu(), do, causal, scale)
    for h in (0, H - 1):
        sl = (slice(0, 1), slice(h, h + 1))
        rdq, rdk, rdv, _ = attention_bwd_fp64(q[sl], k[sl], v[sl], do[sl], causal=causal, scale=scale)
        check_grads(tuple(g[sl] for g in got), (rdq, rdk, rdv), f"{shape}, head {h}")

