"""Pins for the attention-gradient oracle, checked against facts that do not come from it.

Sources: central finite differences of the loss L = sum(dO * O) with O from the (separately
pinned) forward oracle, on tiny inputs; PyTorch's CPU float64 autograd through
scaled_dot_product_attention (the library call the Hacker News FlashAttention-3 thread names as
the user-facing entry to fused attention); closed forms: with one key the output is that key's
V row whatever q and k are (so dq = dk = 0 and dv = sum of dO); the key gradients sum to zero
(the softmax ignores a shift of every key by one vector); the value gradients sum to the sum
of dO (rows of P sum to one); rescaling q by a with the scale divided by a leaves P unchanged
and divides dq by a.  Every planted mistake in one step of the oracle must fail a pin.
"""
import numpy as np
import pytest
import torch

import oracle.attention as OA
import oracle.attention_bwd as OB


def _rand(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def bwd():
    return OB.attention_bwd_fp64


def _fd_grads(q, k, v, do, causal, scale, eps=1e-6):
    def loss(qq, kk, vv):
        o, _ = OA.attention_fp64(qq, kk, vv, causal=causal, scale=scale)
        return float((o * do).sum())

    out = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * eps)
        out.append(g)
    return out


# ---- pins ---------------------------------------------------------------------------------

def pin_finite_differences():
    for causal, nq, nk in ((False, 5, 5), (True, 5, 5), (True, 3, 6), (False, 4, 2)):
        q, k, v = _rand(1, 1, 2, nq, 3), _rand(2, 1, 2, nk, 3), _rand(3, 1, 2, nk, 2)
        do = _rand(4, 1, 2, nq, 2)
        dq, dk, dv, _ = bwd()(q, k, v, do, causal=causal, scale=0.7)
        fq, fk, fv = _fd_grads(q, k, v, do, causal, 0.7)
        np.testing.assert_allclose(dq, fq, atol=1e-7, err_msg=f"dq causal={causal} {nq}x{nk}")
        np.testing.assert_allclose(dk, fk, atol=1e-7, err_msg=f"dk causal={causal} {nq}x{nk}")
        np.testing.assert_allclose(dv, fv, atol=1e-7, err_msg=f"dv causal={causal} {nq}x{nk}")


def pin_torch_autograd():
    for causal, nq, nk in ((False, 9, 9), (True, 9, 9), (True, 4, 11), (False, 7, 3)):
        q, k, v = _rand(5, 2, 3, nq, 8), _rand(6, 2, 3, nk, 8), _rand(7, 2, 3, nk, 8)
        do = _rand(8, 2, 3, nq, 8)
        dq, dk, dv, lse = bwd()(q, k, v, do, causal=causal, scale=0.4)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        mask = None
        if causal:
            mask = torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=nk - nq)
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.4)
        o.backward(torch.tensor(do))
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-10)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-10)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-10)
        _, lse_f = OA.attention_fp64(q, k, v, causal=causal, scale=0.4)
        np.testing.assert_allclose(lse, lse_f, atol=1e-13)


def pin_single_key():
    q, k, v, do = _rand(9, 1, 2, 1, 4), _rand(10, 1, 2, 1, 4), _rand(11, 1, 2, 1, 4), _rand(12, 1, 2, 1, 4)
    dq, dk, dv, _ = bwd()(q, k, v, do, causal=False, scale=0.9)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv, do, atol=1e-15)
    # several queries, one key: dv sums dO over the queries
    q2, do2 = _rand(13, 1, 1, 5, 4), _rand(14, 1, 1, 5, 4)
    dq, dk, dv, _ = bwd()(q2, k[:, :1], v[:, :1], do2, causal=False, scale=0.9)
    np.testing.assert_allclose(dv[0, 0, 0], do2[0, 0].sum(axis=0), atol=1e-14)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)


def pin_key_gradients_sum_to_zero():
    for causal in (False, True):
        q, k, v, do = _rand(15, 2, 2, 12, 5), _rand(16, 2, 2, 12, 5), _rand(17, 2, 2, 12, 5), _rand(18, 2, 2, 12, 5)
        _, dk, dv, _ = bwd()(q, k, v, do, causal=causal, scale=0.6)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


def pin_query_rescaling():
    q, k, v, do = _rand(19, 1, 2, 8, 6), _rand(20, 1, 2, 8, 6), _rand(21, 1, 2, 8, 6), _rand(22, 1, 2, 8, 6)
    dq, dk, dv, _ = bwd()(q, k, v, do, causal=True, scale=0.5)
    dq2, dk2, dv2, _ = bwd()(3.0 * q, k, v, do, causal=True, scale=0.5 / 3.0)
    np.testing.assert_allclose(dq2, dq / 3.0, atol=1e-13)
    np.testing.assert_allclose(dk2, dk, atol=1e-12)
    np.testing.assert_allclose(dv2, dv, atol=1e-13)


def pin_rows_against_torch():
    for causal, nq, nk in ((True, 9, 9), (False, 6, 10), (True, 5, 12)):
        q, k, v = _rand(23, 1, 2, nq, 8), _rand(24, 1, 2, nk, 8), _rand(25, 1, 2, nk, 8)
        do = _rand(26, 1, 2, nq, 8)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        mask = torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=nk - nq) if causal else None
        torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.3).backward(
            torch.tensor(do))
        q_rows = [(0, h, i) for h in range(2) for i in range(nq)]
        k_rows = [(0, h, j) for h in range(2) for j in range(nk)]
        dq, dk, dv = OB.attention_bwd_fp64_rows(q, k, v, do, q_rows, k_rows, causal=causal, scale=0.3)
        np.testing.assert_allclose(dq, tq.grad.numpy()[0].reshape(-1, 8), atol=1e-10)
        np.testing.assert_allclose(dk, tk.grad.numpy()[0].reshape(-1, 8), atol=1e-10)
        np.testing.assert_allclose(dv, tv.grad.numpy()[0].reshape(-1, 8), atol=1e-10)


def pin_rows_match_full_in_chunks():
    saved = OB._CHUNK
    try:
        OB._CHUNK = 3   # several query chunks, the last one partial
        for causal, nq, nk in ((True, 11, 11), (True, 7, 13), (False, 10, 4)):
            q, k, v = _rand(27, 2, 2, nq, 4), _rand(28, 2, 2, nk, 4), _rand(29, 2, 2, nk, 4)
            do = _rand(30, 2, 2, nq, 4)
            fq, fk, fv, _ = OB.attention_bwd_fp64(q, k, v, do, causal=causal, scale=0.8)
            q_rows = [(1, 0, nq - 1), (0, 1, 0), (1, 1, nq // 2)]
            k_rows = [(0, 0, 0), (1, 1, nk - 1), (1, 0, nk // 2), (0, 1, 1)]
            dq, dk, dv = OB.attention_bwd_fp64_rows(q, k, v, do, q_rows, k_rows, causal=causal, scale=0.8)
            np.testing.assert_allclose(dq, [fq[b, h, i] for b, h, i in q_rows], atol=1e-12)
            np.testing.assert_allclose(dk, [fk[b, h, j] for b, h, j in k_rows], atol=1e-12)
            np.testing.assert_allclose(dv, [fv[b, h, j] for b, h, j in k_rows], atol=1e-12)
    finally:
        OB._CHUNK = saved


PINS = [pin_finite_differences, pin_torch_autograd, pin_single_key, pin_key_gradients_sum_to_zero,
        pin_query_rescaling, pin_rows_against_torch, pin_rows_match_full_in_chunks]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


MUTANTS = {
    "dv_not_transposed": ("_grad_v", lambda p, doh: p @ doh),
    "dp_not_transposed": ("_grad_p", lambda doh, vh: doh @ vh),
    "row_dot_wrong_axis": ("_row_dot", lambda p, dp: (p * dp).sum(axis=0, keepdims=True).T),
    "ds_without_row_dot": ("_grad_s", lambda p, dp, dd: p * dp),
    "ds_sign": ("_grad_s", lambda p, dp, dd: p * (dd - dp)),
    "dq_missing_scale": ("_grad_q", lambda ds, kh, c: ds @ kh),
    "dk_not_transposed": ("_grad_k", lambda ds, qh, c: c * (ds @ qh)),
    "dk_scale_squared": ("_grad_k", lambda ds, qh, c: c * c * (ds.T @ qh)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OB, attr, fn)
    caught = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1, f"planted mistake {name} passed every pin"
