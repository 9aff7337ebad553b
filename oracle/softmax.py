"""CPU float64 oracle for the stand-alone row softmax.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's CPU-baseline
leg may import this module.  The product path (the HIP library and its Python binding) never
calls it, and this module imports nothing from the product package.

What is computed.  The online-softmax trick that the interview "Tri Dao: prediction"
(transcript) names as the third ingredient of the method computes a row's softmax in one
pass over the row, keeping a running maximum and a running sum that is rescaled whenever the
maximum grows, and still reaches the exact softmax.  The plain, exact result is therefore the
reference; for every row r of X [R, C] and a scale c:

    s    = c * x_r
    m    = max_j s_j
    y_rj = exp(s_j - m) / sum_k exp(s_k - m)
    lse_r = m + log(sum_k exp(s_k - m))        (natural log, as for attention's LSE)

Readings where the pages are silent: rows are contiguous with the column index fastest; the
scale multiplies the inputs before the softmax and is used exactly as passed (callers pass
the float32 value the GPU receives); an entry of -inf takes no weight; a row must hold at
least one finite value.  Inputs may be bf16 or fp32 values in any wider float container and
are widened exactly to float64.

`softmax_online_fp64` is the one-pass recurrence itself, written out step by step (running
max, running sum rescaled by exp(m_old - m_new), then a normalising pass).  It serves as an
independent check of the plain definition, never as the reference.
"""
from __future__ import annotations

import numpy as np

__all__ = ["softmax_rows_fp64", "softmax_online_fp64"]


def _widen(x) -> np.ndarray:
    """bf16/fp32 values (numpy array or CPU torch tensor) -> float64 numpy, exactly."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


# ---- the steps of the plain definition -----------------------------------------------------

def _scaled(x: np.ndarray, c: float) -> np.ndarray:
    """c * x, with -inf entries kept at -inf (no weight) whatever the sign of c."""
    with np.errstate(invalid="ignore"):
        return np.where(np.isneginf(x), -np.inf, c * x)


def _row_max(s: np.ndarray) -> np.ndarray:
    return s.max(axis=-1, keepdims=True)


def _exp_shifted(s: np.ndarray, m: np.ndarray) -> np.ndarray:
    return np.exp(s - m)


def _row_sum(e: np.ndarray) -> np.ndarray:
    return e.sum(axis=-1, keepdims=True)


def _normalise(e: np.ndarray, l: np.ndarray) -> np.ndarray:
    return e / l


def _lse(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    return (m + np.log(l))[..., 0]


def softmax_rows_fp64(x, scale: float = 1.0):
    """Exact row softmax in float64.

    x: [..., C] (the last axis is the row).  Returns (y [..., C], lse [...]) in float64."""
    x = _widen(x)
    s = _scaled(x, float(scale))
    m = _row_max(s)
    e = _exp_shifted(s, m)
    l = _row_sum(e)
    return _normalise(e, l), _lse(m, l)


def softmax_online_fp64(x, scale: float = 1.0, block: int = 16):
    """The online normaliser: one pass for the max and the sum, one pass to normalise.

    Walking the row in blocks of `block` columns, it keeps a running max m (start -inf) and a
    running sum l of exp(s - m) (start 0); for each block it takes m_new = max(m, block max),
    rescales l by exp(m - m_new), adds the block's exp(s - m_new) and sets m = m_new.  Then
    y = exp(s - m) / l and lse = m + log l.  Returns (y, lse) like `softmax_rows_fp64`."""
    x = _widen(x)
    c = float(scale)
    lead, C = x.shape[:-1], x.shape[-1]
    rows = x.reshape(-1, C)
    y = np.empty_like(rows)
    lse = np.empty(rows.shape[0])
    for r in range(rows.shape[0]):
        s = np.array([-np.inf if v == -np.inf else c * v for v in rows[r]])
        m, l = -np.inf, 0.0
        for j0 in range(0, C, block):
            blk = s[j0:j0 + block]
            m_new = max(m, blk.max())
            if m_new == -np.inf:
                continue  # nothing visible yet
            l = l * np.exp(m - m_new) + np.exp(blk - m_new).sum()
            m = m_new
        y[r] = np.exp(s - m) / l
        lse[r] = m + np.log(l)
    return y.reshape(x.shape), lse.reshape(lead)
