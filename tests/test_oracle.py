"""Pins for the CPU float64 oracle, checked against facts that do not come from the oracle.

Each pin is a plain function of an attention callable so that the same pins can be run
against the oracle with a mistake planted in one of its steps (see
`test_pins_catch_planted_mistakes`): every plausible slip (a dropped scale, a transposed
operand, an off-by-one causal mask, a missing normaliser, a wrong log) must fail at least
one pin.

Sources of the pinned facts:
  * the hand-derived closed forms in tests/golden/closed_form_cases.json;
  * closed forms and invariants of the softmax: rows sum to one, one key returns its V row,
    constant V is returned unchanged, zero logits average V, shift and permutation
    invariance (the softmax over the attention row, "Tri Dao: prediction", transcript);
  * a pure-Python scalar loop on tiny inputs (brute force, no NumPy, no max shift);
  * the online-softmax recurrence itself: splitting the row into blocks, rescaling, still
    gives the same answer ("Tri Dao: prediction", transcript);
  * the associative merge of partial results (algebraic aggregates, Hacker News
    FlashAttention-3 thread);
  * PyTorch's CPU float64 scaled_dot_product_attention, the library call that the Hacker
    News thread names as the user-facing entry to fused attention;
  * causal prefix invariance (a row never reads keys after it).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.attention as OA

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")
TOL = 1e-12


def _num(s):
    s = str(s)
    if s.startswith("ln(") and s.endswith(")"):
        return math.log(float(Fraction(s[3:-1])))
    return float(Fraction(s))


def _arr(rows):
    return np.array([[_num(x) for x in r] for r in rows], dtype=np.float64)


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def attn():
    """The oracle entry point, looked up at call time so planted mistakes take effect."""
    return OA.attention_fp64


# ---- pins ---------------------------------------------------------------------------------

def pin_golden():
    cases = json.load(open(GOLDEN))["cases"]
    for case in cases:
        q, k, v = (_arr(case[x])[None, None] for x in ("q", "k", "v"))
        scale = _num(case["scale"])
        for causal, key in ((False, "noncausal"), (True, "causal")):
            exp = case[key]
            o, lse = attn()(q, k, v, causal=causal, scale=scale)
            np.testing.assert_allclose(o[0, 0], _arr(exp["o"]), rtol=TOL, atol=TOL, err_msg=case["name"])
            if "exp_lse" in exp:
                want = np.array([_num(x) for x in exp["exp_lse"]])
                np.testing.assert_allclose(np.exp(lse[0, 0]), want, rtol=TOL, err_msg=case["name"])
            else:
                want = np.array([_num(x) for x in exp["lse"]])
                np.testing.assert_allclose(lse[0, 0], want, rtol=TOL, atol=TOL, err_msg=case["name"])


def pin_rows_sum_to_one():
    """With V = identity, O is the probability matrix itself: rows sum to 1, entries are
    non-negative, and the causal variant is lower-triangular."""
    rng = _rng(1)
    for N, causal in ((7, False), (7, True), (20, True)):
        q, k = _rand(rng, 1, 2, N, 5), _rand(rng, 1, 2, N, 5)
        v = np.broadcast_to(np.eye(N), (1, 2, N, N)).copy()
        p, _ = attn()(q, k, v, causal=causal, scale=0.7)
        np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=TOL)
        assert (p >= 0).all()
        if causal:
            assert np.all(p[..., np.triu_indices(N, 1)[0], np.triu_indices(N, 1)[1]] == 0)


def pin_single_key():
    """N = 1: the only key gets weight 1, so O = V[0] and LSE = scale * q . k."""
    rng = _rng(2)
    for causal in (False, True):
        q, k, v = _rand(rng, 2, 3, 1, 8), _rand(rng, 2, 3, 1, 8), _rand(rng, 2, 3, 1, 8)
        o, lse = attn()(q, k, v, causal=causal, scale=0.3)
        np.testing.assert_allclose(o, v, rtol=TOL, atol=TOL)
        want = 0.3 * np.einsum("bhnd,bhnd->bhn", q, k)
        np.testing.assert_allclose(lse, want, rtol=TOL, atol=TOL)


def pin_causal_row0():
    """Causal row 0 sees key 0 only: O[0] = V[0], LSE[0] = scale * q0 . k0."""
    rng = _rng(3)
    q, k, v = _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 6)
    o, lse = attn()(q, k, v, causal=True, scale=0.9)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=TOL, atol=TOL)
    np.testing.assert_allclose(lse[:, :, 0], 0.9 * (q[:, :, 0] * k[:, :, 0]).sum(-1), rtol=TOL, atol=TOL)


def pin_constant_v():
    """Every V row equal to u: O is a convex combination of copies of u, so O_i = u."""
    rng = _rng(4)
    u = _rand(rng, 6)
    for causal in (False, True):
        q, k = _rand(rng, 1, 1, 11, 6, scale=3.0), _rand(rng, 1, 1, 11, 6, scale=3.0)
        v = np.broadcast_to(u, (1, 1, 11, 6)).copy()
        o, _ = attn()(q, k, v, causal=causal, scale=0.5)
        np.testing.assert_allclose(o, np.broadcast_to(u, o.shape), rtol=1e-12, atol=1e-12)


def pin_uniform_weights():
    """Q = 0 (or scale = 0) makes every visible logit 0: O_i is the mean of the visible V
    rows and LSE_i = ln(number of visible keys)."""
    rng = _rng(5)
    N = 10
    k, v = _rand(rng, 1, 1, N, 3), _rand(rng, 1, 1, N, 3)
    for q, scale in ((np.zeros((1, 1, N, 3)), 0.8), (_rand(rng, 1, 1, N, 3), 0.0)):
        o, lse = attn()(q, k, v, causal=False, scale=scale)
        np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(0), (N, 3)), rtol=TOL, atol=TOL)
        np.testing.assert_allclose(lse[0, 0], math.log(N), rtol=TOL, atol=TOL)
        o, lse = attn()(q, k, v, causal=True, scale=scale)
        counts = np.arange(1, N + 1)
        means = np.cumsum(v[0, 0], axis=0) / counts[:, None]
        np.testing.assert_allclose(o[0, 0], means, rtol=TOL, atol=TOL)
        np.testing.assert_allclose(lse[0, 0], np.log(counts), rtol=TOL, atol=TOL)


def _brute_force(q, k, v, causal, scale):
    """Scalar loops in pure Python with math.exp on the raw scores (no max shift)."""
    B, H, N, d = q.shape
    Nk, dv = k.shape[2], v.shape[3]
    o = [[[[0.0] * dv for _ in range(N)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(N):
                w = []
                for j in range(Nk):
                    if causal and j > i:
                        w.append(0.0)
                        continue
                    dot = 0.0
                    for t in range(d):
                        dot += float(q[b, h, i, t]) * float(k[b, h, j, t])
                    w.append(math.exp(scale * dot))
                z = sum(w)
                for e in range(dv):
                    o[b][h][i][e] = sum(w[j] * float(v[b, h, j, e]) for j in range(Nk)) / z
                lse[b][h][i] = math.log(z)
    return np.array(o), np.array(lse)


def pin_brute_force():
    rng = _rng(6)
    for (B, H, N, Nk, d, dv, causal) in ((1, 2, 5, 5, 3, 2, False), (2, 1, 12, 12, 4, 5, True),
                                         (1, 1, 4, 9, 2, 3, False), (1, 1, 1, 1, 1, 1, True)):
        q, k, v = _rand(rng, B, H, N, d), _rand(rng, B, H, Nk, d), _rand(rng, B, H, Nk, dv)
        o, lse = attn()(q, k, v, causal=causal, scale=0.45)
        bo, blse = _brute_force(q, k, v, causal, 0.45)
        np.testing.assert_allclose(o, bo, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, blse, rtol=1e-11, atol=1e-12)


def pin_online_blocked():
    """The block-by-block online-softmax recurrence reaches the plain result for any block
    size, including sizes that do not divide N."""
    rng = _rng(7)
    N = 37
    q, k, v = _rand(rng, 1, 2, N, 8, scale=2.0), _rand(rng, 1, 2, N, 8, scale=2.0), _rand(rng, 1, 2, N, 8)
    for causal in (False, True):
        o, lse = attn()(q, k, v, causal=causal, scale=0.6)
        for block in (1, 3, 16, N, 64):
            bo, blse = OA.attention_online_fp64(q, k, v, causal=causal, scale=0.6, block=block)
            np.testing.assert_allclose(o, bo, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(lse, blse, rtol=1e-11, atol=1e-12)


def pin_merge():
    """Attention over keys A u B equals the merge of attention over A and over B."""
    rng = _rng(8)
    q, k, v = _rand(rng, 1, 2, 6, 5), _rand(rng, 1, 2, 13, 5), _rand(rng, 1, 2, 13, 4)
    o, lse = attn()(q, k, v, scale=0.8)
    for cut in (1, 6, 12):
        oa, la = attn()(q, k[:, :, :cut], v[:, :, :cut], scale=0.8)
        ob, lb = attn()(q, k[:, :, cut:], v[:, :, cut:], scale=0.8)
        mo, ml = OA.merge_partials(oa, la, ob, lb)
        np.testing.assert_allclose(mo, o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(ml, lse, rtol=1e-11, atol=1e-12)
        mo2, ml2 = OA.merge_partials(ob, lb, oa, la)
        np.testing.assert_allclose(mo2, o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(ml2, lse, rtol=1e-11, atol=1e-12)


def pin_shift():
    """K' = K + 1 u^T adds scale * q_i . u to every logit of row i: O is unchanged and
    LSE_i moves by exactly that amount."""
    rng = _rng(9)
    q, k, v = _rand(rng, 1, 2, 8, 4), _rand(rng, 1, 2, 8, 4), _rand(rng, 1, 2, 8, 3)
    u = _rand(rng, 4)
    for causal in (False, True):
        o, lse = attn()(q, k, v, causal=causal, scale=0.5)
        o2, lse2 = attn()(q, k + u, v, causal=causal, scale=0.5)
        np.testing.assert_allclose(o2, o, rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(lse2, lse + 0.5 * (q @ u), rtol=1e-10, atol=1e-11)


def pin_permutation():
    """Non-causal attention is a function of the key/value set: a joint row permutation of
    K and V changes nothing."""
    rng = _rng(10)
    q, k, v = _rand(rng, 1, 1, 9, 4), _rand(rng, 1, 1, 9, 4), _rand(rng, 1, 1, 9, 5)
    perm = rng.permutation(9)
    o, lse = attn()(q, k, v, scale=0.7)
    o2, lse2 = attn()(q, k[:, :, perm], v[:, :, perm], scale=0.7)
    np.testing.assert_allclose(o2, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-11, atol=1e-12)


def pin_torch_sdpa():
    """PyTorch's CPU float64 scaled_dot_product_attention and logsumexp agree."""
    rng = _rng(11)
    for causal in (False, True):
        q, k, v = _rand(rng, 2, 3, 33, 16), _rand(rng, 2, 3, 33, 16), _rand(rng, 2, 3, 33, 8)
        o, lse = attn()(q, k, v, causal=causal, scale=0.25)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.25)
        s = 0.25 * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.ones(33, 33, dtype=torch.bool).triu(1), float("-inf"))
        tl = torch.logsumexp(s, dim=-1)
        np.testing.assert_allclose(o, to.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse, tl.numpy(), rtol=1e-10, atol=1e-12)


def pin_causal_prefix():
    """Causal: changing keys/values after row i leaves row i bitwise unchanged."""
    rng = _rng(12)
    N = 16
    q, k, v = _rand(rng, 1, 1, N, 4), _rand(rng, 1, 1, N, 4), _rand(rng, 1, 1, N, 3)
    o, lse = attn()(q, k, v, causal=True, scale=0.5)
    cut = 7
    k2, v2 = k.copy(), v.copy()
    k2[:, :, cut + 1:] = _rand(rng, 1, 1, N - cut - 1, 4) * 10
    v2[:, :, cut + 1:] = _rand(rng, 1, 1, N - cut - 1, 3) * 1e6
    o2, lse2 = attn()(q, k2, v2, causal=True, scale=0.5)
    assert np.array_equal(o2[:, :, : cut + 1], o[:, :, : cut + 1])
    assert np.array_equal(lse2[:, :, : cut + 1], lse[:, :, : cut + 1])


PINS = [pin_golden, pin_rows_sum_to_one, pin_single_key, pin_causal_row0, pin_constant_v,
        pin_uniform_weights, pin_brute_force, pin_online_blocked, pin_merge, pin_shift,
        pin_permutation, pin_torch_sdpa, pin_causal_prefix]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


# ---- planted mistakes: every one must trip at least one pin --------------------------------

def _mask_ge(s, rows):
    out = s.copy()
    out[np.arange(s.shape[1])[None, :] >= rows[:, None]] = -np.inf
    return out


def _mask_lt(s, rows):
    out = s.copy()
    out[np.arange(s.shape[1])[None, :] < rows[:, None]] = -np.inf
    return out


def _mask_zero(s, rows):
    out = s.copy()
    out[np.arange(s.shape[1])[None, :] > rows[:, None]] = 0.0
    return out


def _softmax_unnormalised(s, m):
    e = np.exp(s - m)
    return e, e.sum(axis=1, keepdims=True)


def _softmax_wrong_axis(s, m):
    e = np.exp(s - m)
    return e / e.sum(axis=0, keepdims=True), e.sum(axis=1, keepdims=True)


def _softmax_no_shift(s, m):
    e = np.exp(s)
    l = e.sum(axis=1, keepdims=True)
    return e / l, l * np.exp(-m)


MUTANTS = {
    "scores_transposed": ("_scores", lambda qh, kh, c: c * (kh @ qh.T)),
    "scale_dropped": ("_scores", lambda qh, kh, c: qh @ kh.T),
    "scale_squared": ("_scores", lambda qh, kh, c: c * c * (qh @ kh.T)),
    "mask_includes_diagonal": ("_causal_mask", _mask_ge),
    "mask_transposed": ("_causal_mask", _mask_lt),
    "mask_missing": ("_causal_mask", lambda s, rows: s),
    "mask_zero_not_neg_inf": ("_causal_mask", _mask_zero),
    "max_wrong_axis": ("_row_max", lambda s: s.max(axis=0, keepdims=True)),
    "softmax_unnormalised": ("_softmax_rows", _softmax_unnormalised),
    "softmax_wrong_axis": ("_softmax_rows", _softmax_wrong_axis),
    "softmax_unshifted_exp": ("_softmax_rows", _softmax_no_shift),
    "combine_transposed": ("_combine", lambda p, vh: p.T @ vh),
    "lse_without_max": ("_lse", lambda m, l: np.log(l)[:, 0]),
    "lse_log2": ("_lse", lambda m, l: (m + np.log2(l))[:, 0]),
    "lse_max_sign": ("_lse", lambda m, l: (-m + np.log(l))[:, 0]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OA, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except Exception:  # an assertion, or a shape error the mistake causes
                caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"


def test_rows_entry_matches_full():
    """The sampled-row entry point returns exactly the rows of the full computation."""
    rng = _rng(13)
    q, k, v = _rand(rng, 2, 3, 40, 8), _rand(rng, 2, 3, 40, 8), _rand(rng, 2, 3, 40, 8)
    rows = np.array([[0, 0, 0], [1, 2, 39], [0, 1, 17], [1, 0, 1], [1, 0, 38]])
    for causal in (False, True):
        o, lse = OA.attention_fp64(q, k, v, causal=causal, scale=0.4)
        ro, rl = OA.attention_fp64_rows(q, k, v, rows, causal=causal, scale=0.4)
        for r, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(ro[r], o[b, h, i], rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(rl[r], lse[b, h, i], rtol=1e-13, atol=1e-14)


def test_accepts_bf16_torch_tensors():
    """bf16 torch tensors are widened exactly (bf16 -> fp32 -> fp64 loses nothing)."""
    g = torch.Generator().manual_seed(0)
    q, k, v = (torch.randn(1, 1, 8, 4, generator=g).to(torch.bfloat16) for _ in range(3))
    o, lse = OA.attention_fp64(q, k, v, causal=True, scale=0.5)
    o2, lse2 = OA.attention_fp64(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal=True, scale=0.5)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


# ---- fewer queries than keys (the newest Nq positions of a longer sequence) -------------------

def test_rect_causal_is_the_square_mask_on_the_last_rows():
    """Nq < Nk causal equals the last Nq rows of the square causal problem over all Nk
    positions (queries are the newest positions): checked against the square definition."""
    rng = _rng(31)
    B, H, Nk, d = 1, 2, 23, 5
    qf = _rand(rng, B, H, Nk, d)
    k = _rand(rng, B, H, Nk, d)
    v = _rand(rng, B, H, Nk, 3)
    of, lf = OA.attention_fp64(qf, k, v, causal=True, scale=0.6)
    for nq in (1, 2, 7, 23):
        o, lse = OA.attention_fp64(qf[:, :, Nk - nq:], k, v, causal=True, scale=0.6)
        np.testing.assert_allclose(o, of[:, :, Nk - nq:], atol=1e-13)
        np.testing.assert_allclose(lse, lf[:, :, Nk - nq:], atol=1e-13)
        rows = np.array([[0, h, i] for h in range(H) for i in range(nq)])
        ro, rl = OA.attention_fp64_rows(qf[:, :, Nk - nq:], k, v, rows, causal=True, scale=0.6)
        np.testing.assert_allclose(ro, o.reshape(-1, 3), atol=1e-13)
        np.testing.assert_allclose(rl, lse.reshape(-1), atol=1e-13)
        oo, lo = OA.attention_online_fp64(qf[:, :, Nk - nq:], k, v, causal=True, scale=0.6, block=4)
        np.testing.assert_allclose(oo, o, atol=1e-12)
        np.testing.assert_allclose(lo, lse, atol=1e-12)


def test_rect_single_query_causal_sees_every_key():
    rng = _rng(32)
    q = _rand(rng, 2, 3, 1, 8)
    k = _rand(rng, 2, 3, 40, 8)
    v = _rand(rng, 2, 3, 40, 8)
    oc, lc = OA.attention_fp64(q, k, v, causal=True, scale=0.3)
    on, ln_ = OA.attention_fp64(q, k, v, causal=False, scale=0.3)
    np.testing.assert_allclose(oc, on, atol=1e-15)
    np.testing.assert_allclose(lc, ln_, atol=1e-15)


def test_rect_causal_brute_force():
    """Pure-Python loops: query i (of Nq) at position i + Nk - Nq sees keys j <= that position."""
    rng = _rng(33)
    Nq, Nk, d, dv = 3, 7, 4, 2
    q, k, v = _rand(rng, 1, 1, Nq, d), _rand(rng, 1, 1, Nk, d), _rand(rng, 1, 1, Nk, dv)
    o, lse = OA.attention_fp64(q, k, v, causal=True, scale=0.9)
    for i in range(Nq):
        pos = i + Nk - Nq
        w = [math.exp(0.9 * sum(float(q[0, 0, i, t]) * float(k[0, 0, j, t]) for t in range(d))) for j in range(pos + 1)]
        z = sum(w)
        for c in range(dv):
            ref = sum(w[j] * float(v[0, 0, j, c]) for j in range(pos + 1)) / z
            assert abs(o[0, 0, i, c] - ref) <= 1e-12
        assert abs(lse[0, 0, i] - math.log(z)) <= 1e-12


def test_rect_causal_more_queries_than_keys_is_rejected():
    rng = _rng(34)
    q, k = _rand(rng, 1, 1, 5, 4), _rand(rng, 1, 1, 4, 4)
    with pytest.raises(ValueError):
        OA.attention_fp64(q, k, k, causal=True)
    with pytest.raises(ValueError):
        OA.attention_fp64_rows(q, k, k, np.array([[0, 0, 0]]), causal=True)
