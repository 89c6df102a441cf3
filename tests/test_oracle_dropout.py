"""Pins of the dropout oracle (CPU only).

* Philox4x32-10 against the generator's published known-answer vectors (the
  Random123 distribution of Salmon, Moraes, Dror and Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC 2011).
* p = 0 reduces to the plain attention oracle (itself pinned elsewhere).
* The keep fraction of a large mask and the mean output over many seeds
  (dropout with the 1/(1-p) scale leaves the expected output unchanged),
  within bounds of a few standard deviations.
* The mask depends only on (seed, sequence, head, row, key).
"""

import math

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(77)


@pytest.mark.parametrize("ctr,key,want", [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
])
def test_philox_known_answers(ctr, key, want):
    got = oracle.philox4x32_10(np.array([ctr], dtype=np.uint64), key)[0]
    assert tuple(int(x) for x in got) == want


def test_threshold():
    assert oracle.drop_threshold(0.0) == 0
    assert oracle.drop_threshold(0.5) == 2 ** 15
    assert oracle.drop_threshold(0.25) == 2 ** 14
    assert oracle.drop_threshold(0.1) == 6553
    assert oracle.drop_threshold(1.0 - 2.0 ** -20) == 2 ** 16 - 1
    with pytest.raises(ValueError):
        oracle.drop_threshold(1.0)
    with pytest.raises(ValueError):
        oracle.drop_threshold(-0.1)


def test_p_zero_is_plain_attention():
    q = RNG.standard_normal((2, 4, 37, 16))
    k = RNG.standard_normal((2, 2, 41, 16))
    v = RNG.standard_normal((2, 2, 41, 16))
    for causal in (False, True):
        o, l = oracle.attention_dropout(q, k, v, p=0.0, seed=5, causal=causal)
        o2, l2 = oracle.attention(q, k, v, causal=causal)
        assert np.allclose(o, o2, atol=1e-14) and np.array_equal(l, l2)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_fraction(p):
    m = oracle.keep_mask(2 ** 40 + 3, 1, 2, np.arange(256), 1000, p)
    n = m.size
    sigma = math.sqrt(n * p * (1 - p))
    assert abs(m.sum() - n * (1 - p)) < 5 * sigma


def test_mean_over_seeds_is_plain_attention():
    """E[O] = attention: over 400 seeds the mean lands within 5 standard
    errors (estimated from the samples) of the plain output."""
    q = RNG.standard_normal((1, 1, 6, 8))
    k = RNG.standard_normal((1, 1, 9, 8))
    v = RNG.standard_normal((1, 1, 9, 8))
    ref, _ = oracle.attention(q, k, v)
    outs = np.stack([oracle.attention_dropout(q, k, v, p=0.3, seed=s)[0] for s in range(400)])
    mean, se = outs.mean(axis=0), outs.std(axis=0) / math.sqrt(len(outs))
    assert np.all(np.abs(mean - ref) <= 5 * se + 1e-12)
    # and a single draw differs from it
    assert np.max(np.abs(outs[0] - ref)) > 1e-3


def test_lse_is_that_of_the_softmax():
    q = RNG.standard_normal((1, 2, 10, 8))
    k = RNG.standard_normal((1, 2, 12, 8))
    v = RNG.standard_normal((1, 2, 12, 8))
    _, l = oracle.attention_dropout(q, k, v, p=0.4, seed=9, causal=True)
    _, l2 = oracle.attention(q, k, v, causal=True)
    assert np.allclose(l, l2, atol=1e-14)


def test_mask_depends_only_on_its_coordinates():
    full = oracle.keep_mask(99, 3, 5, np.arange(64), 130, 0.2)
    part = oracle.keep_mask(99, 3, 5, np.arange(20, 30), 130, 0.2)
    assert np.array_equal(full[20:30], part)
    # other head, sequence or seed: another mask
    assert not np.array_equal(full, oracle.keep_mask(99, 3, 6, np.arange(64), 130, 0.2))
    assert not np.array_equal(full, oracle.keep_mask(99, 4, 5, np.arange(64), 130, 0.2))
    assert not np.array_equal(full, oracle.keep_mask(98, 3, 5, np.arange(64), 130, 0.2))
    # keys 112..127 of row 7 (group 7): counter 14 decides offsets 0-3 and
    # 8-11 by its 8 halves in order, counter 15 offsets 4-7 and 12-15; each
    # half is the low then the high 16 bits of a word
    thr = oracle.drop_threshold(0.2)
    for c, offs in ((14, [0, 1, 2, 3, 8, 9, 10, 11]), (15, [4, 5, 6, 7, 12, 13, 14, 15])):
        w = oracle.philox4x32_10(np.array([[c, 7, 5, 3]], dtype=np.uint64), (99, 0))[0]
        halves = [int(x) >> s for x in w for s in (0, 16)]
        halves = [x & 0xFFFF for x in halves]
        assert [x >= thr for x in halves] == [bool(full[7, 112 + o]) for o in offs]


def test_every_key_has_its_own_half():
    """Within a row the (counter, half) pairs of distinct keys differ, and a
    16-key group uses exactly two counters: no two keys share a decision."""
    lk = 100
    j = np.arange(lk)
    cidx = 2 * (j // 16) + (j // 4) % 2
    half = 4 * ((j // 8) % 2) + j % 4
    pairs = set(zip(cidx.tolist(), half.tolist()))
    assert len(pairs) == lk
    for g in range(lk // 16):
        assert set(cidx[16 * g:16 * g + 16].tolist()) == {2 * g, 2 * g + 1}
    # the halves of one row are not all alike (a transposed or dropped
    # index would repeat them)
    hv = oracle.keep_halves(5, 0, 0, np.arange(3), lk)
    assert len(set(hv[0].tolist())) > 90 and not np.array_equal(hv[0], hv[1])


def test_packed_equals_dense_per_sequence():
    lens = [5, 0, 17]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = RNG.standard_normal((int(cu[-1]), 2, 8))
    k = RNG.standard_normal((int(cu[-1]), 1, 8))
    v = RNG.standard_normal((int(cu[-1]), 1, 8))
    o, l = oracle.attention_dropout(q, k, v, p=0.25, seed=11, causal=True,
                                    cu_seqlens_q=cu, cu_seqlens_k=cu)
    for b, n in enumerate(lens):
        if n == 0:
            continue
        sl = slice(cu[b], cu[b + 1])
        ob, lb = oracle.attention_dropout(q[None, sl].transpose(0, 2, 1, 3),
                                          k[None, sl].transpose(0, 2, 1, 3),
                                          v[None, sl].transpose(0, 2, 1, 3),
                                          p=0.25, seed=11, causal=True)
        # the dense call numbers its only sequence 0: compare with b = 0 masks
        if b == 0:
            assert np.allclose(ob[0].transpose(1, 0, 2), o[sl], atol=1e-14)
        assert np.allclose(lb[0], l[:, sl], atol=1e-14)
