"""CPU float64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's CPU-baseline
leg may import this module.  The product path (the HIP library and its Python binding)
never calls it, and this module imports nothing from the product package.

What is computed.  The interview "Tri Dao: prediction" (transcript) says that the online
softmax trick splits the row softmax of attention into pieces that are rescaled and still
give the right answer.  So the fused kernel must reach exactly (up to rounding order) the
plain, unfused result, and this oracle is that plain result written out: the full N x N
score matrix is materialised, masked, passed through a standard row softmax and multiplied
by V.  For each (b, h):

    S    = c * Q K^T                       (c = the softmax scale)
    S_ij = -inf  for j > i                 (causal variant: the lower-triangular score
                                            matrix of the FlashAttention-2 remark in the
                                            Hacker News FlashAttention-3 thread)
    m_i  = max_j S_ij
    P_ij = exp(S_ij - m_i) / sum_j exp(S_ij - m_i)
    O    = P V
    LSE_i = m_i + log(sum_j exp(S_ij - m_i))   (natural log of the row's partition sum)

Readings taken where the pages are silent: tensors are [B, H, N, d] with d fastest; the
causal mask keeps key j for query i iff j <= i (square N); with fewer queries than keys
(Nq < Nk, e.g. the newest Nq positions of a sequence whose keys are cached) the queries are
the last Nq positions, so query i keeps key j iff j <= i + (Nk - Nq), which is the square
mask restricted to those rows; Nq > Nk is not defined for the causal variant; LSE uses the
natural log of the scaled logits; the scale is used exactly as passed (callers pass the float32 value that the
GPU library receives).  Inputs may be bf16 values carried in any wider float type; they are
widened exactly to float64.

`attention_online_fp64` is the online-softmax recurrence itself (running max, running sum,
rescaled partial output per key block), taken in the order the interview describes it.  It
serves as an independent check of the plain definition, never as the reference.
`merge_partials` is the associative merge of two partial softmax states (the "algebraic
aggregate" view of the tiled softmax that the Hacker News thread mentions).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "attention_fp64",
    "attention_fp64_rows",
    "attention_online_fp64",
    "merge_partials",
]


def _widen(x) -> np.ndarray:
    """bf16/fp32 values (numpy array or CPU torch tensor) -> float64 numpy, exactly."""
    if hasattr(x, "detach"):  # a torch tensor; bf16 has no numpy dtype, fp32 holds it exactly
        x = x.detach().cpu()
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _scale(d: int, scale) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


# ---- the steps of the plain definition, one small function each --------------------------

def _scores(qh: np.ndarray, kh: np.ndarray, c: float) -> np.ndarray:
    """S = c * Q K^T for one head: [Nq, d] x [Nk, d] -> [Nq, Nk]."""
    return c * (qh @ kh.T)


def _causal_mask(s: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Set S[r, j] = -inf where key j lies after the position rows[r] of query r (j > pos)."""
    keys = np.arange(s.shape[1])
    out = s.copy()
    out[keys[None, :] > rows[:, None]] = -np.inf
    return out


def _row_max(s: np.ndarray) -> np.ndarray:
    return s.max(axis=1, keepdims=True)


def _softmax_rows(s: np.ndarray, m: np.ndarray):
    """Stable row softmax given the row max m: returns (P, row sum of exp(S - m))."""
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, l


def _combine(p: np.ndarray, vh: np.ndarray) -> np.ndarray:
    """O = P V."""
    return p @ vh


def _lse(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    return (m + np.log(l))[:, 0]


def _head(qh, kh, vh, causal: bool, c: float, rows: np.ndarray):
    s = _scores(qh, kh, c)
    if causal:
        s = _causal_mask(s, rows)
    m = _row_max(s)
    p, l = _softmax_rows(s, m)
    return _combine(p, vh), _lse(m, l)


# ---- public entry points ---------------------------------------------------------------

def attention_fp64(q, k, v, causal: bool = False, scale=None):
    """Exact attention in float64.

    q: [B, H, Nq, d], k: [B, H, Nk, d], v: [B, H, Nk, dv].  Causal requires Nq <= Nk; query i
    sits at position i + Nk - Nq.  Returns (O [B, H, Nq, dv] float64, LSE [B, H, Nq] float64)."""
    q, k, v = _widen(q), _widen(k), _widen(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, H, Nq, d = q.shape
    if k.shape[:2] != (B, H) or v.shape[:2] != (B, H) or k.shape[3] != d or k.shape[2] != v.shape[2]:
        raise ValueError("shape mismatch between q, k and v")
    if causal and k.shape[2] < Nq:
        raise ValueError("the causal variant needs Nq <= Nk")
    c = _scale(d, scale)
    o = np.empty((B, H, Nq, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    rows = np.arange(Nq) + (k.shape[2] - Nq)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = _head(q[b, h], k[b, h], v[b, h], causal, c, rows)
    return o, lse


def attention_fp64_rows(q, k, v, rows, causal: bool = False, scale=None):
    """The same definition for selected query rows only.

    rows: integer array [R, 3] of (b, h, i).  Each row still sees its full key range, so
    the result equals the matching rows of `attention_fp64`.  Only the needed head slices
    are widened, which keeps long-sequence checks cheap.
    Returns (O [R, dv] float64, LSE [R] float64)."""
    rows = np.asarray(rows.cpu() if hasattr(rows, "cpu") else rows, dtype=np.int64)
    d = q.shape[3]
    shift = k.shape[2] - q.shape[2]  # position of query i is i + Nk - Nq
    if causal and shift < 0:
        raise ValueError("the causal variant needs Nq <= Nk")
    c = _scale(d, scale)
    o = np.empty((rows.shape[0], v.shape[3]), dtype=np.float64)
    lse = np.empty(rows.shape[0], dtype=np.float64)
    groups: dict[tuple[int, int], list[int]] = {}
    for r, (b, h, _) in enumerate(rows):
        groups.setdefault((int(b), int(h)), []).append(r)
    for (b, h), idx in groups.items():
        kh, vh = _widen(k[b, h]), _widen(v[b, h])
        qi = rows[idx, 2]
        qh = _widen(q[b, h])[qi]
        o[idx], lse[idx] = _head(qh, kh, vh, causal, c, qi + shift)
    return o, lse


def attention_online_fp64(q, k, v, causal: bool = False, scale=None, block: int = 16):
    """The online-softmax recurrence in float64, one key block at a time.

    Per query row it keeps a running max m, a running sum l of exp(s - m) and an unnormalised
    output acc.  For every block of `block` keys it takes the new max, rescales l and acc by
    exp(m_old - m_new), adds the block's exp-weights and their weighted V rows, and after the
    last block divides acc by l.  Rows that have seen no visible key yet keep m = -inf and
    contribute nothing.  Returns (O, LSE) like `attention_fp64`."""
    q, k, v = _widen(q), _widen(k), _widen(v)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    c = _scale(d, scale)
    o = np.empty((B, H, N, v.shape[3]))
    lse = np.empty((B, H, N))
    qi = np.arange(N) + (Nk - N)  # query positions (bottom-right when N < Nk)
    for b in range(B):
        for h in range(H):
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, v.shape[3]))
            for j0 in range(0, Nk, block):
                j1 = min(j0 + block, Nk)
                s = c * (q[b, h] @ k[b, h, j0:j1].T)
                if causal:
                    s[np.arange(j0, j1)[None, :] > qi[:, None]] = -np.inf
                m_new = np.maximum(m, s.max(axis=1))
                live = np.isfinite(m_new)
                alpha = np.where(live, np.exp(np.where(live, m - m_new, 0.0)), 0.0)
                p = np.where(live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, h, j0:j1]
                m = m_new
            o[b, h] = acc / l[:, None]
            lse[b, h] = m + np.log(l)
    return o, lse


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Merge two partial attention results computed over disjoint key sets.

    With L = log(exp(LSE_a) + exp(LSE_b)), the merged output is
    exp(LSE_a - L) * O_a + exp(LSE_b - L) * O_b.  The merge is associative and commutative."""
    o_a, lse_a, o_b, lse_b = map(_widen, (o_a, lse_a, o_b, lse_b))
    lse = np.logaddexp(lse_a, lse_b)
    wa = np.exp(lse_a - lse)[..., None]
    wb = np.exp(lse_b - lse)[..., None]
    return wa * o_a + wb * o_b, lse
