"""Pins of the rotary-embedding oracle (CPU only).

Each test checks the oracle against something other than its own formula:
special angles whose rotations are exact, typed constants, the defining
properties of the rotary embedding (pair norms kept, scores depending only on
the position difference, angles adding up), and the two feature layouts
against each other through a permutation.
"""

import math

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(1234)


def test_position_zero_is_identity():
    x = RNG.standard_normal((3, 5, 64))
    for inter in (False, True):
        assert np.array_equal(oracle.rotate(x, np.zeros(5), 64, 10000.0, inter), x)


def test_inverse_frequencies_typed():
    # 10000 ** (-2k / 8) = 10 ** -k
    f = oracle.inverse_frequencies(8, 10000.0)
    assert np.allclose(f, [1.0, 0.1, 0.01, 0.001], rtol=1e-15, atol=0)
    # 10000 ** (-2k / 4) = 100 ** -k
    assert np.allclose(oracle.inverse_frequencies(4, 10000.0), [1.0, 0.01], rtol=1e-15)


@pytest.mark.parametrize("inter", [False, True])
def test_quarter_and_half_turns(inter):
    """base = 4 / pi^2 and rotary_dim 4: pair 1 turns by pi/2 per position,
    so one position maps (x, y) to (-y, x) and two positions to (-x, -y);
    pair 0 turns by one radian per position."""
    base = 4.0 / math.pi ** 2
    i0, i1 = oracle.pair_indices(4, inter)
    x = np.zeros((1, 4))
    x[0, i0[1]], x[0, i1[1]] = 0.75, -0.5
    x[0, i0[0]], x[0, i1[0]] = 1.0, 0.0
    r1 = oracle.rotate(x, [1], 4, base, inter)[0]
    assert abs(r1[i0[1]] - 0.5) < 1e-15 and abs(r1[i1[1]] - 0.75) < 1e-15
    r2 = oracle.rotate(x, [2], 4, base, inter)[0]
    assert abs(r2[i0[1]] + 0.75) < 1e-15 and abs(r2[i1[1]] - 0.5) < 1e-15
    # one radian: (cos 1, sin 1), typed
    assert abs(r1[i0[0]] - 0.5403023058681398) < 1e-15
    assert abs(r1[i1[0]] - 0.8414709848078965) < 1e-15


def test_pair_frequency_ratio():
    """Pair 1 of rotary_dim 8, base 10000, turns ten times slower than pair 0:
    position 10 on pair 1 equals position 1 on pair 0."""
    for inter in (False, True):
        i0, i1 = oracle.pair_indices(8, inter)
        x = np.zeros((1, 8))
        x[0, i0[0]], x[0, i1[0]] = 0.3, -1.7
        x[0, i0[1]], x[0, i1[1]] = 0.3, -1.7
        a = oracle.rotate(x, [1], 8, 10000.0, inter)[0]
        b = oracle.rotate(x, [10], 8, 10000.0, inter)[0]
        assert np.allclose([a[i0[0]], a[i1[0]]], [b[i0[1]], b[i1[1]]], atol=1e-14)


@pytest.mark.parametrize("inter", [False, True])
def test_pair_norms_are_kept(inter):
    x = RNG.standard_normal((4, 33, 128))
    pos = RNG.integers(0, 100000, size=33)
    y = oracle.rotate(x, pos, 96, 10000.0, inter)
    i0, i1 = oracle.pair_indices(96, inter)
    assert np.allclose(x[..., i0] ** 2 + x[..., i1] ** 2, y[..., i0] ** 2 + y[..., i1] ** 2,
                       rtol=1e-12, atol=1e-12)
    # features past the rotary dimension are untouched
    assert np.array_equal(y[..., 96:], x[..., 96:])


@pytest.mark.parametrize("inter", [False, True])
def test_scores_depend_on_position_difference_only(inter):
    q = RNG.standard_normal((1, 64))
    k = RNG.standard_normal((1, 64))
    def score(m, n):
        return float(oracle.rotate(q, [m], 64, 10000.0, inter)[0]
                     @ oracle.rotate(k, [n], 64, 10000.0, inter)[0])
    for m, n, s in [(5, 3, 1000), (0, 17, 4096), (123, 123, 77)]:
        assert abs(score(m, n) - score(m + s, n + s)) < 1e-10
    # and it does depend on the difference
    assert abs(score(5, 3) - score(5, 4)) > 1e-3


@pytest.mark.parametrize("inter", [False, True])
def test_angles_add(inter):
    x = RNG.standard_normal((2, 7, 64))
    a = RNG.integers(0, 5000, size=7)
    b = RNG.integers(0, 5000, size=7)
    twice = oracle.rotate(oracle.rotate(x, a, 64, 500.0, inter), b, 64, 500.0, inter)
    once = oracle.rotate(x, a + b, 64, 500.0, inter)
    assert np.allclose(twice, once, atol=1e-10)


def test_layouts_are_a_permutation_of_each_other():
    """GPT-J pairs (2k, 2k+1) are GPT-NeoX pairs (k, k + rd/2) after moving
    feature 2k to k and 2k+1 to k + rd/2."""
    rd, d = 32, 48
    x = RNG.standard_normal((3, 9, d))
    pos = RNG.integers(0, 9000, size=9)
    perm = np.arange(d)
    perm[:rd] = np.concatenate([np.arange(0, rd, 2), np.arange(1, rd, 2)])
    neox = oracle.rotate(x[..., perm], pos, rd, 10000.0, False)
    gptj = oracle.rotate(x, pos, rd, 10000.0, True)
    assert np.allclose(gptj[..., perm], neox, atol=1e-13)


def test_dense_and_packed_offsets():
    x = RNG.standard_normal((3, 2, 10, 32))
    offs = [0, 7, 1000]
    dense = oracle.rotate_dense(x, 32, 10000.0, False, offset=5, offsets=offs)
    for b in range(3):
        ref = oracle.rotate(x[b], 5 + offs[b] + np.arange(10), 32, 10000.0, False)
        assert np.array_equal(dense[b], ref)
    lens = [4, 0, 10, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    xp = RNG.standard_normal((int(cu[-1]), 2, 32))
    packed = oracle.rotate_packed(xp, cu, 16, 10000.0, True, offset=3, offsets=[1, 2, 3, 4])
    for b, n in enumerate(lens):
        if n == 0:
            continue
        rows = slice(cu[b], cu[b + 1])
        ref = oracle.rotate(xp[rows].transpose(1, 0, 2), 3 + (b + 1) + np.arange(n), 16,
                            10000.0, True).transpose(1, 0, 2)
        assert np.array_equal(packed[rows], ref)


def test_rejects_bad_dimensions():
    with pytest.raises(ValueError):
        oracle.inverse_frequencies(7, 10000.0)
    with pytest.raises(ValueError):
        oracle.rotate(np.zeros((2, 8)), [0, 1], 16)
