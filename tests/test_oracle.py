"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: the worked example
printed on the fusion/compiler notes page (section 3.1, example 5-6), closed
forms, invariants the method guarantees (the result does not depend on how
the keys are split into blocks), scalar brute force on tiny shapes, and
library routines (torch's CPU float64 scaled_dot_product_attention, scipy's
logsumexp).
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle.attention import _blocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sym(x):
    return {"0": 0.0, "ln2": math.log(2.0), "ln3": math.log(3.0)}[x] \
        if isinstance(x, str) else float(x)


@pytest.fixture(scope="module")
def example():
    with open(os.path.join(GOLDEN, "online_softmax_example_5_6.json")) as f:
        return json.load(f)


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Worked example 5-6
# ---------------------------------------------------------------------------

def test_worked_example_trace(example):
    scores = [_sym(s) for s in example["scores"]]
    values = np.array(example["values"]).reshape(-1, 1)
    res = oracle.online_softmax_ul(scores, values, boundaries=[1])
    assert len(res["trace"]) == len(example["after_block"])
    for (m, ell, u, r), want in zip(res["trace"], example["after_block"]):
        assert m == pytest.approx(_sym(want["m"]), abs=1e-15)
        assert ell == pytest.approx(want["l"], abs=1e-15)
        assert u[0] == pytest.approx(want["u"], abs=1e-15)
        if "r" in want:
            assert r == pytest.approx(want["r"], abs=1e-15)
    want_out = example["output_num"] / example["output_den"]
    assert res["out"][0] == pytest.approx(want_out, abs=1e-15)
    assert round(res["out"][0], 4) == example["output_printed"]
    assert res["lse"] == pytest.approx(_sym(example["lse"]), abs=1e-15)
    # the whole-row form printed beside it: (1 + 2*3) / (1 + 2)
    assert (1 + 2 * 3) / (1 + 2) == pytest.approx(want_out, abs=1e-15)


def test_worked_example_normalised_form(example):
    scores = [_sym(s) for s in example["scores"]]
    values = np.array(example["values"]).reshape(-1, 1)
    o, lse = oracle.online_softmax_normalised(scores, values, boundaries=[1])
    assert o[0] == pytest.approx(7.0 / 3.0, abs=1e-15)
    assert lse == pytest.approx(math.log(3.0), abs=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_worked_example_through_attention(causal):
    # q = e0, k0 = 0, k1 = e0, scale = ln 2 gives scores [0, ln 2].
    d = 4
    q = np.zeros((1, 1, 2 if causal else 1, d))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, 2, d))
    k[0, 0, 1, 0] = 1.0
    v = np.zeros((1, 1, 2, d))
    v[0, 0, 0, :] = 1.0
    v[0, 0, 1, :] = 3.0
    o, lse = oracle.attention(q, k, v, scale=math.log(2.0), causal=causal)
    last = o[0, 0, -1]
    assert np.allclose(last, 7.0 / 3.0, atol=1e-15, rtol=0)
    assert lse[0, 0, -1] == pytest.approx(math.log(3.0), abs=1e-15)
    if causal:   # row 0 sees key 0 only
        assert np.allclose(o[0, 0, 0], 1.0, atol=1e-15, rtol=0)
        assert lse[0, 0, 0] == pytest.approx(0.0, abs=1e-15)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lq,lk", [(5, 5), (3, 7), (7, 3), (1, 4), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_closed_form(lq, lk, causal):
    """Q = 0: every visible key gets the same weight.

    O_i = mean of the visible V rows and LSE_i = ln(#visible); with the
    bottom-right causal rule row i sees min(Lk, max(0, i + Lk - Lq + 1)) keys.
    """
    rng = _rng(1)
    d = 3
    q = np.zeros((1, 1, lq, d))
    k = rng.standard_normal((1, 1, lk, d))
    v = rng.standard_normal((1, 1, lk, d))
    o, lse = oracle.attention(q, k, v, scale=0.7, causal=causal)
    for i in range(lq):
        n = lk if not causal else min(lk, max(0, i + lk - lq + 1))
        if n == 0:
            assert lse[0, 0, i] == -math.inf
            assert np.all(o[0, 0, i] == 0.0)
        else:
            assert lse[0, 0, i] == pytest.approx(math.log(n), abs=1e-14)
            assert np.allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0),
                               atol=1e-14, rtol=0)


def test_uniform_scores_varlen():
    lens = [3, 1, 6, 2]
    cu = np.cumsum([0] + lens)
    rng = _rng(2)
    t, h, d = cu[-1], 2, 4
    q = np.zeros((t, h, d))
    k = rng.standard_normal((t, h, d))
    v = rng.standard_normal((t, h, d))
    o, lse = oracle.attention(q, k, v, scale=0.5, cu_seqlens_q=cu,
                              cu_seqlens_k=cu)
    for b, n in enumerate(lens):
        rows = slice(cu[b], cu[b + 1])
        assert np.allclose(lse[:, rows], math.log(n), atol=1e-14, rtol=0)
        mean = v[rows].mean(axis=0)                     # [h, d]
        assert np.allclose(o[rows], mean[None], atol=1e-14, rtol=0)


def test_single_key():
    rng = _rng(3)
    q = rng.standard_normal((2, 3, 1, 8))
    k = rng.standard_normal((2, 3, 1, 8))
    v = rng.standard_normal((2, 3, 1, 8))
    o, lse = oracle.attention(q, k, v, scale=0.3)
    assert np.allclose(o, v, atol=0, rtol=0)
    s0 = 0.3 * np.einsum("bhid,bhid->bhi", q, k)
    assert np.allclose(lse, s0, atol=1e-15, rtol=0)


def test_dominant_score_selects_value():
    """A key whose score exceeds the others by 60 takes all the weight."""
    d = 8
    q = np.zeros((1, 1, 1, d))
    q[..., 0] = 1.0
    rng = _rng(4)
    k = rng.standard_normal((1, 1, 6, d)) * 0.1
    k[0, 0, 4, 0] = 60.0
    v = rng.standard_normal((1, 1, 6, d))
    o, lse = oracle.attention(q, k, v, scale=1.0)
    assert np.allclose(o[0, 0, 0], v[0, 0, 4], atol=1e-20 + 1e-12, rtol=0)
    assert lse[0, 0, 0] == pytest.approx(60.0 + k[0, 0, 4, 1:] @ q[0, 0, 0, 1:],
                                         abs=1e-12)


def test_row_shift_moves_lse_only():
    """Adding delta to every score of one row: O unchanged, LSE + delta.

    K carries a column of ones, so adding x to that component of q_i adds
    scale * x to all of row i's scores.
    """
    rng = _rng(5)
    q = rng.standard_normal((1, 2, 6, 5))
    k = rng.standard_normal((1, 2, 9, 5))
    k[..., 0] = 1.0
    v = rng.standard_normal((1, 2, 9, 5))
    scale, x = 0.4, 2.5
    o0, l0 = oracle.attention(q, k, v, scale=scale)
    q2 = q.copy()
    q2[:, :, 3, 0] += x
    o1, l1 = oracle.attention(q2, k, v, scale=scale)
    assert np.allclose(o1, o0, atol=1e-13, rtol=0)
    want = l0.copy()
    want[:, :, 3] += scale * x
    assert np.allclose(l1, want, atol=1e-13, rtol=0)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    rng = _rng(6)
    qh = rng.standard_normal((17, 8))
    kh = rng.standard_normal((23, 8))
    p = oracle.row_probabilities(qh, kh, scale=0.9, causal=causal)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12, rtol=0)
    assert np.all(p >= 0)
    # and O = P V is what attention() returns
    vh = rng.standard_normal((23, 8))
    o, _ = oracle.attention(qh[None, None], kh[None, None], vh[None, None],
                            scale=0.9, causal=causal)
    assert np.allclose(o[0, 0], p @ vh, atol=1e-12, rtol=0)


SPLITS = [[1], list(range(1, 130)), [2], [3], [7], [16], [64], [128],
          [5, 6, 40, 41, 99], [129]]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("normalised", [False, True])
def test_block_split_invariance(causal, normalised):
    """The online recurrence over any key split equals the materialised result."""
    rng = _rng(7)
    q = rng.standard_normal((1, 2, 9, 16)) * 2.0
    k = rng.standard_normal((1, 1, 130, 16)) * 2.0
    v = rng.standard_normal((1, 1, 130, 16))
    o_ref, l_ref = oracle.attention(q, k, v, scale=0.35, causal=causal)
    for bnd in SPLITS + [sorted(rng.choice(np.arange(1, 130), 11,
                                           replace=False))]:
        o, lse = oracle.attention_blocked(q, k, v, scale=0.35, causal=causal,
                                          boundaries=bnd,
                                          normalised=normalised)
        assert np.allclose(o, o_ref, atol=1e-12, rtol=1e-12)
        fin = np.isfinite(l_ref)
        assert np.array_equal(fin, np.isfinite(lse))
        assert np.allclose(lse[fin], l_ref[fin], atol=1e-12, rtol=1e-12)


def test_blocks_helper_covers_range():
    assert _blocks(5, [0, 2, 2, 9, 4]) == [(0, 2), (2, 4), (4, 5)]
    assert _blocks(3, []) == [(0, 3)]


@pytest.mark.parametrize("lq", [1, 2, 3, 5, 7])
@pytest.mark.parametrize("lk", [1, 2, 3, 5, 7])
@pytest.mark.parametrize("d", [1, 2, 4])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(1, 1), (2, 1), (4, 2)])
def test_bruteforce_matches(lq, lk, d, causal, heads):
    hq, hkv = heads
    rng = _rng(lq * 100 + lk * 10 + d)
    q = rng.standard_normal((2, hq, lq, d))
    k = rng.standard_normal((2, hkv, lk, d))
    v = rng.standard_normal((2, hkv, lk, d))
    o, lse = oracle.attention(q, k, v, scale=0.6, causal=causal)
    ob, lb = oracle.attention_bruteforce(q, k, v, 0.6, causal=causal)
    assert np.allclose(o, ob, atol=1e-12, rtol=0)
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], lb[fin], atol=1e-12, rtol=0)


def test_permutation_invariance_noncausal():
    rng = _rng(8)
    q = rng.standard_normal((1, 2, 11, 8))
    k = rng.standard_normal((1, 2, 19, 8))
    v = rng.standard_normal((1, 2, 19, 8))
    perm = rng.permutation(19)
    o0, l0 = oracle.attention(q, k, v, scale=0.5)
    o1, l1 = oracle.attention(q, k[:, :, perm], v[:, :, perm], scale=0.5)
    assert np.allclose(o0, o1, atol=1e-13, rtol=0)
    assert np.allclose(l0, l1, atol=1e-13, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_heads(causal):
    rng = _rng(9)
    g = 4
    q = rng.standard_normal((2, 8, 13, 8))
    k = rng.standard_normal((2, 2, 13, 8))
    v = rng.standard_normal((2, 2, 13, 8))
    o, lse = oracle.attention(q, k, v, scale=0.4, causal=causal)
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    o2, l2 = oracle.attention(q, kr, vr, scale=0.4, causal=causal)
    assert np.allclose(o, o2, atol=0, rtol=0)
    assert np.allclose(l2, lse, atol=0, rtol=0)
    # a different grouping (h % Hkv) would give a different answer
    ko = np.tile(k, (1, g, 1, 1))
    vo = np.tile(v, (1, g, 1, 1))
    o3, _ = oracle.attention(q, ko, vo, scale=0.4, causal=causal)
    assert not np.allclose(o, o3, atol=1e-6)


# ---------------------------------------------------------------------------
# Library routines
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, scale, causal, mask=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else t(mask),
        is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 2, 33, 16), (1, 8, 8, 70, 64),
                                   (1, 2, 1, 129, 128)])
def test_matches_torch_sdpa_and_logsumexp(causal, shape):
    bsz, hq, hkv, n, d = shape
    rng = _rng(10 + n)
    q = rng.standard_normal((bsz, hq, n, d))
    k = rng.standard_normal((bsz, hkv, n, d))
    v = rng.standard_normal((bsz, hkv, n, d))
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, causal=causal)   # default scale
    g = hq // hkv
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    want = _sdpa(q, kr, vr, scale, causal)
    assert np.allclose(o, want, atol=1e-12, rtol=0)
    s = scale * np.einsum("bhid,bhjd->bhij", q, kr)
    if causal:
        s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    assert np.allclose(lse, logsumexp(s, axis=-1), atol=1e-12, rtol=0)


@pytest.mark.parametrize("lq,lk", [(5, 13), (17, 40), (13, 5), (40, 17), (1, 9), (9, 1)])
def test_bottom_right_causal_matches_torch_lower_right_bias(lq, lk):
    """Causal with Lq != Lk against torch's lower-right causal bias (the
    library's own definition of that alignment), CPU float64 SDPA: O on
    every row that sees a key, and the LSE from the library's probabilities
    (SDPA with V = identity returns P; LSE_i = s_ij - log P_ij for any visible
    j).  Rows that see no key (Lq > Lk): the library returns NaN or zeros
    there (depending on the version), the oracle O = 0 and LSE = -inf (its
    own reading)."""
    from torch.nn.attention.bias import causal_lower_right
    import warnings
    rng = _rng(100 + lq * 7 + lk)
    d, scale = 8, 0.35
    q = rng.standard_normal((1, 2, lq, d))
    k = rng.standard_normal((1, 2, lk, d))
    v = rng.standard_normal((1, 2, lk, d))
    o, lse = oracle.attention(q, k, v, scale=scale, causal=True)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")          # the bias warns about NaN rows
        bias = causal_lower_right(lq, lk)
        want = torch.nn.functional.scaled_dot_product_attention(
            t(q), t(k), t(v), attn_mask=bias, scale=scale).numpy()
        eye = np.broadcast_to(np.eye(lk), (1, 2, lk, lk))
        prob = torch.nn.functional.scaled_dot_product_attention(
            t(q), t(k), t(eye), attn_mask=bias, scale=scale).numpy()
    seen = np.nan_to_num(prob).sum(axis=-1) > 0.5   # rows whose probabilities sum to 1
    assert np.allclose(o[seen], want[seen], atol=1e-12, rtol=0)
    assert np.all(o[~seen] == 0.0) and np.all(lse[~seen] == -np.inf)
    assert seen.all() or lq > lk
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    for b, h, i in zip(*np.nonzero(seen)):
        j = int(np.argmax(prob[b, h, i]))
        assert abs(lse[b, h, i] - (s[b, h, i, j] - math.log(prob[b, h, i, j]))) < 1e-12
    # the visible keys are exactly where the library's probabilities are > 0
    rows, cols = np.nonzero(prob[0, 0] > 0)
    assert np.all(cols <= rows + lk - lq)
    assert len(rows) == sum(max(0, min(lk, i + lk - lq + 1)) for i in range(lq))


def test_varlen_equals_per_sequence_and_padded_mask():
    """Packed sequences == one dense call per sequence == padded batch with a
    key padding mask (True = keep), on the valid query rows."""
    lens = [5, 12, 1, 9]
    cu = np.cumsum([0] + lens)
    hq, hkv, d = 4, 2, 8
    rng = _rng(11)
    t = cu[-1]
    q = rng.standard_normal((t, hq, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    o, lse = oracle.attention(q, k, v, scale=0.3, cu_seqlens_q=cu,
                              cu_seqlens_k=cu)
    lmax = max(lens)
    qp = np.zeros((len(lens), hq, lmax, d))
    kp = np.zeros((len(lens), hkv, lmax, d))
    vp = np.zeros((len(lens), hkv, lmax, d))
    keep = np.zeros((len(lens), lmax), dtype=bool)
    for b, n in enumerate(lens):
        rows = slice(cu[b], cu[b + 1])
        ob, lb = oracle.attention(q[rows].transpose(1, 0, 2)[None],
                                  k[rows].transpose(1, 0, 2)[None],
                                  v[rows].transpose(1, 0, 2)[None], scale=0.3)
        assert np.allclose(o[rows], ob[0].transpose(1, 0, 2), atol=1e-14,
                           rtol=0)
        assert np.allclose(lse[:, rows], lb[0], atol=1e-14, rtol=0)
        qp[b, :, :n] = q[rows].transpose(1, 0, 2)
        kp[b, :, :n] = k[rows].transpose(1, 0, 2)
        vp[b, :, :n] = v[rows].transpose(1, 0, 2)
        keep[b, :n] = True
    g = hq // hkv
    mask = np.broadcast_to(keep[:, None, None, :], (len(lens), hq, lmax, lmax))
    want = _sdpa(qp, np.repeat(kp, g, 1), np.repeat(vp, g, 1), 0.3, False,
                 mask=mask)
    for b, n in enumerate(lens):
        got = o[cu[b]:cu[b + 1]].transpose(1, 0, 2)
        assert np.allclose(got, want[b, :, :n], atol=1e-12, rtol=0)


def test_empty_sequences_varlen():
    lens_q = [0, 3, 2]
    lens_k = [4, 0, 2]
    cq, ck = np.cumsum([0] + lens_q), np.cumsum([0] + lens_k)
    rng = _rng(12)
    q = rng.standard_normal((cq[-1], 2, 4))
    k = rng.standard_normal((ck[-1], 2, 4))
    v = rng.standard_normal((ck[-1], 2, 4))
    o, lse = oracle.attention(q, k, v, scale=1.0, cu_seqlens_q=cq,
                              cu_seqlens_k=ck)
    # sequence 1 has no keys: O = 0, LSE = -inf
    assert np.all(o[cq[1]:cq[2]] == 0)
    assert np.all(lse[:, cq[1]:cq[2]] == -math.inf)
    assert np.all(np.isfinite(lse[:, cq[2]:cq[3]]))
