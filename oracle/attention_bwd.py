"""CPU float64 oracle for the gradients of exact attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's CPU-baseline
leg may import this module.  The product path never calls it, and this module imports nothing
from the product package.

What is computed.  The forward is O = P V with P = softmax(S) row by row and S = c Q K^T (the
causal variant masks key j for query i iff j > i + Nk - Nq).  For an upstream gradient dO of
the loss with respect to O (the loss does not depend on LSE), the chain rule through the
matrix products and the row softmax gives, for one (b, h):

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij                 (equal to sum_t dO_it O_it)
    dS = P * (dP - D)                      (row softmax Jacobian applied to dP)
    dQ = c dS K
    dK = c dS^T Q

The pages stop at the forward pass (the ~100-line kernel's author leaves the "matrix
derivatives" out, "Show HN: Flash Attention in ~100 lines of CUDA"); the backward is the next
step the scope table lists.  This is the plain definition written out with the full P
materialised; the tiled kernels recompute P block by block from the saved LSE.

`attention_bwd_fp64_rows` applies the same step functions to slices, for long sequences: dQ
of selected query rows (each needs only its own row of P and dP), and dK, dV of selected keys
(each needs its column of P and dS over every query, so the rows' LSE and D are taken from the
full score rows, a chunk of queries at a time).
"""
from __future__ import annotations

import numpy as np

from .attention import _causal_mask, _lse, _row_max, _scale, _scores, _softmax_rows, _widen

_CHUNK = 1024  # query rows per slice of the key-side gradients

__all__ = ["attention_bwd_fp64", "attention_bwd_fp64_rows"]


def _probabilities(qh, kh, causal, c, pos):
    s = _scores(qh, kh, c)
    if causal:
        s = _causal_mask(s, pos)
    m = _row_max(s)
    p, l = _softmax_rows(s, m)
    return p, _lse(m, l)


def _grad_v(p, doh):
    return p.T @ doh


def _grad_p(doh, vh):
    return doh @ vh.T


def _row_dot(p, dp):
    return (p * dp).sum(axis=1, keepdims=True)


def _grad_s(p, dp, dd):
    return p * (dp - dd)


def _grad_q(ds, kh, c):
    return c * (ds @ kh)


def _grad_k(ds, qh, c):
    return c * (ds.T @ qh)


def attention_bwd_fp64(q, k, v, do, causal: bool = False, scale=None):
    """Gradients of O = attention(q, k, v) for the upstream gradient do, in float64.

    q, do: [B, H, Nq, d]; k, v: [B, H, Nk, d] (causal needs Nq <= Nk; query i sits at position
    i + Nk - Nq).  Returns (dq, dk, dv) shaped like q, k, v, and the forward's LSE [B, H, Nq]."""
    q, k, v, do = _widen(q), _widen(k), _widen(v), _widen(do)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if causal and Nk < Nq:
        raise ValueError("the causal variant needs Nq <= Nk")
    c = _scale(d, scale)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    lse = np.empty((B, H, Nq))
    pos = np.arange(Nq) + (Nk - Nq)
    for b in range(B):
        for h in range(H):
            p, lse[b, h] = _probabilities(q[b, h], k[b, h], causal, c, pos)
            dv[b, h] = _grad_v(p, do[b, h])
            dp = _grad_p(do[b, h], v[b, h])
            ds = _grad_s(p, dp, _row_dot(p, dp))
            dq[b, h] = _grad_q(ds, k[b, h], c)
            dk[b, h] = _grad_k(ds, q[b, h], c)
    return dq, dk, dv, lse


def _as_rows(rows) -> np.ndarray:
    rows = np.asarray(rows.cpu() if hasattr(rows, "cpu") else rows, dtype=np.int64)
    return rows.reshape(-1, 3)


def _group(rows: np.ndarray) -> dict:
    groups: dict[tuple[int, int], list[int]] = {}
    for r, (b, h, _) in enumerate(rows):
        groups.setdefault((int(b), int(h)), []).append(r)
    return groups


def attention_bwd_fp64_rows(q, k, v, do, q_rows, k_rows, causal: bool = False, scale=None):
    """Selected rows of the gradients of `attention_bwd_fp64`, in float64.

    q_rows: [R, 3] integer (b, h, i) query rows -> dq [R, d]; k_rows: [S, 3] integer (b, h, j)
    key rows -> dk [S, d], dv [S, dv].  Same shapes and readings as `attention_bwd_fp64`."""
    Nq, Nk, d = q.shape[2], k.shape[2], q.shape[3]
    if causal and Nk < Nq:
        raise ValueError("the causal variant needs Nq <= Nk")
    c = _scale(d, scale)
    shift = Nk - Nq
    q_rows, k_rows = _as_rows(q_rows), _as_rows(k_rows)
    dq = np.empty((q_rows.shape[0], d))
    dk = np.empty((k_rows.shape[0], d))
    dv = np.empty((k_rows.shape[0], v.shape[3]))
    for (b, h), idx in _group(q_rows).items():
        qi = q_rows[idx, 2]
        qh, kh, vh = _widen(q[b, h])[qi], _widen(k[b, h]), _widen(v[b, h])
        doh = _widen(do[b, h])[qi]
        p, _ = _probabilities(qh, kh, causal, c, qi + shift)
        dp = _grad_p(doh, vh)
        ds = _grad_s(p, dp, _row_dot(p, dp))
        dq[idx] = _grad_q(ds, kh, c)
    for (b, h), idx in _group(k_rows).items():
        kj = k_rows[idx, 2]
        qh, kh, vh, doh = _widen(q[b, h]), _widen(k[b, h]), _widen(v[b, h]), _widen(do[b, h])
        acc_k = np.zeros((len(idx), d))
        acc_v = np.zeros((len(idx), vh.shape[1]))
        for i0 in range(0, Nq, _CHUNK):
            i1 = min(Nq, i0 + _CHUNK)
            p, _ = _probabilities(qh[i0:i1], kh, causal, c, np.arange(i0, i1) + shift)
            dp = _grad_p(doh[i0:i1], vh)
            ds = _grad_s(p, dp, _row_dot(p, dp))
            acc_v += _grad_v(p[:, kj], doh[i0:i1])
            acc_k += _grad_k(ds[:, kj], qh[i0:i1], c)
        dk[idx], dv[idx] = acc_k, acc_v
    return dq, dk, dv
