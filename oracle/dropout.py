"""Plain fp64 CPU oracle for attention with dropout on the probabilities.

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's
CPU-baseline leg, never by the product path.  It shares no code with the HIP
library.

Source: the "Training integration" tutorial (inference.lei6393.com), sections
2.1 and 8.2: the attention module takes a dropout probability (0.1 in the
BERT-style example), used in training and set to 0 for inference.  The pages
fix no formula and no random-number contract, so this oracle takes the plain
reading of dropout on the attention probabilities and one counter-based
generator with a published definition:

* P = softmax(scale * Q K^T) over the visible keys as in the plain attention;
  each P[i, j] is kept with probability 1 - p and scaled by 1 / (1 - p), or
  set to 0: O = (P * M / (1 - p)) V.  The log-sum-exp is that of the softmax
  itself (dropout comes after the normalisation).
* M[i, j] comes from Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
  random numbers: as easy as 1, 2, 3", SC 2011): key = the 64-bit seed as
  (low word, high word); counter = (2 (j // 16) + (j // 4) % 2, i, h, b) for
  batch (sequence) b, query head h, query row i (within its sequence) and
  key j.  The four output words are read as eight 16-bit halves, half 2m
  the low and half 2m + 1 the high half of word m; key j takes half
  4 ((j // 8) % 2) + j % 4.  So one call decides 8 keys of a 16-key group
  (offsets 0-3 and 8-11, or 4-7 and 12-15), and every key of the group has
  its own half.  The key is kept iff its half is at least floor(p * 2^16)
  (an integer comparison, so both sides decide alike; p is resolved to
  2^-16).

Parity pinned by the generator's published known-answer vectors, by p = 0
reducing to the plain attention, and statistically (keep fraction, mean
over seeds).
"""

import math

import numpy as np

from .attention import _allowed_mask

PHILOX_M = (0xD2511F53, 0xCD9E8D57)
PHILOX_W = (0x9E3779B9, 0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counters, key):
    """Philox4x32 with 10 rounds.  counters: uint [N, 4]; key: (k0, k1).
    Returns uint32 [N, 4].  Each round multiplies words 0 and 2 by the two
    constants, takes high and low halves of the products and mixes in the
    other words and the key; the key gains the Weyl increments between
    rounds."""
    c = np.asarray(counters, dtype=np.uint64) & MASK32
    c0, c1, c2, c3 = (c[:, i].copy() for i in range(4))
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    m0, m1 = np.uint64(PHILOX_M[0]), np.uint64(PHILOX_M[1])
    for _ in range(10):
        p0 = c0 * m0                     # < 2^64: exact in uint64
        p1 = c2 * m1
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
        k0 = (k0 + PHILOX_W[0]) & 0xFFFFFFFF
        k1 = (k1 + PHILOX_W[1]) & 0xFFFFFFFF
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def drop_threshold(p):
    """floor(p * 2^16): a key is kept iff its 16-bit half is at least this."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return int(math.floor(float(p) * 65536.0))


def keep_halves(seed, b, h, rows, lk):
    """uint16 [len(rows), lk]: the Philox half that decides each key."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(lk, dtype=np.int64)
    cidx = 2 * (j // 16) + (j // 4) % 2                  # counter word 0 of key j
    half = 4 * ((j // 8) % 2) + j % 4                    # which of its 8 halves
    n_ctr = 2 * ((lk + 15) // 16)
    cc, ii = np.meshgrid(np.arange(n_ctr, dtype=np.int64), rows)   # [R, n_ctr]
    ctr = np.stack([cc.ravel(), ii.ravel(), np.full(cc.size, h), np.full(cc.size, b)], axis=1)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    words = philox4x32_10(ctr, key).reshape(len(rows), n_ctr, 4).astype(np.uint32)
    halves = np.empty((len(rows), n_ctr, 8), dtype=np.uint16)
    halves[..., 0::2] = (words & 0xFFFF).astype(np.uint16)
    halves[..., 1::2] = (words >> 16).astype(np.uint16)
    return halves[:, cidx, half]


def keep_mask(seed, b, h, rows, lk, p):
    """Boolean [len(rows), lk]: keys kept for query rows `rows` of (b, h)."""
    if lk == 0:
        return np.zeros((len(np.asarray(rows)), 0), bool)
    return keep_halves(seed, b, h, rows, lk) >= drop_threshold(p)


def _attend_one_head_dropout(qh, kh, vh, scale, causal, p, seed, b, h, row_chunk):
    """S, P, the kept mask M, O = (P * M / (1 - p)) V and LSE for one head."""
    lq, lk = qh.shape[0], kh.shape[0]
    o = np.zeros((lq, vh.shape[1]))
    lse = np.full(lq, -math.inf)
    if lq == 0 or lk == 0:
        return o, lse
    for r0 in range(0, lq, row_chunk):
        r1 = min(lq, r0 + row_chunk)
        s = scale * (qh[r0:r1] @ kh.T)
        s = np.where(_allowed_mask(r0, r1, lq, lk, causal), s, -math.inf)
        m = s.max(axis=1)
        live = np.isfinite(m)
        if not live.any():
            continue
        e = np.exp(s[live] - m[live, None])
        z = e.sum(axis=1)
        prob = e / z[:, None]                                 # softmax
        if p > 0.0:
            keep = keep_mask(seed, b, h, np.arange(r0, r1), lk, p)[live]
            prob = np.where(keep, prob / (1.0 - p), 0.0)      # dropout
        blk = o[r0:r1]
        blk[live] = prob @ vh
        lblk = lse[r0:r1]
        lblk[live] = m[live] + np.log(z)                      # LSE before dropout
    return o, lse


def attention_dropout(q, k, v, *, p, seed, scale=None, causal=False,
                      cu_seqlens_q=None, cu_seqlens_k=None, row_chunk=1024):
    """Attention with dropout on P; same layouts and LSE as attention().

    Returns (O, LSE) in float64.
    """
    drop_threshold(p)                    # checks the range of p
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if cu_seqlens_q is not None:
        cq = [int(x) for x in cu_seqlens_q]
        ck = [int(x) for x in cu_seqlens_k]
        hq, hkv = q.shape[1], k.shape[1]
        o = np.zeros(q.shape)
        lse = np.full((hq, q.shape[0]), -math.inf)
        for b in range(len(cq) - 1):
            for h in range(hq):
                g = h // (hq // hkv)
                ob, lb = _attend_one_head_dropout(q[cq[b]:cq[b + 1], h], k[ck[b]:ck[b + 1], g],
                                                  v[ck[b]:ck[b + 1], g], scale, causal, p,
                                                  seed, b, h, row_chunk)
                o[cq[b]:cq[b + 1], h] = ob
                lse[h, cq[b]:cq[b + 1]] = lb
        return o, lse
    bsz, hq = q.shape[0], q.shape[1]
    hkv = k.shape[1]
    o = np.zeros(q.shape)
    lse = np.full(q.shape[:3], -math.inf)
    for b in range(bsz):
        for h in range(hq):
            g = h // (hq // hkv)
            o[b, h], lse[b, h] = _attend_one_head_dropout(q[b, h], k[b, g], v[b, g], scale,
                                                          causal, p, seed, b, h, row_chunk)
    return o, lse
