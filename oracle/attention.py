"""Plain fp64 CPU oracle for the exact attention forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.

Sources (the pages this package restates, cited by title and section):

* "FlashAttention: turning the quadratic intermediate matrices into statistics"
  (clxhxhhr.top, post 5544, section 3): standard attention is S = QK^T/sqrt(d),
  P = softmax(S), O = PV, and the method does not change this result.
* Same page, section 3.1 and worked example 5-6: online softmax keeps m (max of
  the scores seen so far), l (sum of exponentials taken relative to m) and
  u (value sum with the same weights); when the max changes both l and u are
  multiplied by r = exp(m_old - m_new); the output is u / l.
* "Day 14" study notes (blog.ans20xx.com), online-softmax pseudocode: the same
  recurrence with a normalised accumulator o, rescaled by alpha * l / l_new.
* "Training integration" tutorial (inference.lei6393.com), sections 2.2-2.5 and
  8.5: causal masking, GQA (groups of query heads share one KV head), cross
  attention (Lq != Lk), padded batches turned into packed variable-length
  sequences, softmax scale defaulting to 1/sqrt(head_dim).

Readings where the pages are silent (each one is also listed in the design
notes of the repository):

* causal with Lq != Lk is bottom-right aligned: key j is visible to query i iff
  j <= i + Lk - Lq (new queries sit after the keys, as with a KV cache);
* a row with no visible key has O = 0 and LSE = -inf;
* LSE is the natural log of sum_j exp(scale * q_i . k_j) over visible keys;
* query head h uses KV head floor(h / G), G = Hq / Hkv (contiguous groups).

The bottom-right causal rule for Lq != Lk is pinned to a library: torch's
lower-right causal bias with its CPU float64 scaled-dot-product attention
(the pages fix no example of it).

Layouts: dense tensors are [B, H, L, d]; packed variable-length tensors are
[T, H, d] with cu_seqlens int arrays of length B + 1 (sequence b owns rows
cu[b] .. cu[b+1]-1).  LSE is [B, Hq, Lq] (dense) or [Hq, Tq] (packed).

Everything is computed in float64 on the exact input values.
"""

import math

import numpy as np

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# Materialised definition (section 3 of the fusion/compiler notes)
# ---------------------------------------------------------------------------

def _allowed_mask(r0, r1, lq, lk, causal):
    """Visible-key mask for query rows r0..r1-1 of one (batch, head).

    Keys beyond the sequence do not exist here (the caller slices them away);
    causal keeps key j for query i iff j <= i + lk - lq.
    """
    rows = np.arange(r0, r1)[:, None]
    cols = np.arange(lk)[None, :]
    if not causal:
        return np.ones((r1 - r0, lk), dtype=bool)
    return cols <= rows + (lk - lq)


def _attend_one_head(qh, kh, vh, scale, causal, row_chunk):
    """S, P materialised per chunk of query rows; returns (o [Lq, dv], lse [Lq])."""
    lq, lk = qh.shape[0], kh.shape[0]
    dv = vh.shape[1]
    o = np.zeros((lq, dv), dtype=np.float64)
    lse = np.full(lq, NEG_INF, dtype=np.float64)
    if lq == 0 or lk == 0:
        return o, lse
    for r0 in range(0, lq, row_chunk):
        r1 = min(lq, r0 + row_chunk)
        s = scale * (qh[r0:r1] @ kh.T)                      # S = scale * Q K^T
        s = np.where(_allowed_mask(r0, r1, lq, lk, causal), s, NEG_INF)
        m = s.max(axis=1)                                    # row max
        live = np.isfinite(m)
        if not live.any():
            continue
        e = np.exp(s[live] - m[live, None])                  # exp(S - m)
        z = e.sum(axis=1)                                    # row sum
        p = e / z[:, None]                                   # P = softmax(S)
        blk = o[r0:r1]
        blk[live] = p @ vh                                   # O = P V
        lblk = lse[r0:r1]
        lblk[live] = m[live] + np.log(z)                     # LSE = m + ln(sum)
    return o, lse


def _check_heads(hq, hkv):
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError(f"Hq={hq} must be a positive multiple of Hkv={hkv}")
    return hq // hkv


def attention(q, k, v, scale=None, causal=False, cu_seqlens_q=None,
              cu_seqlens_k=None, row_chunk=1024):
    """Exact attention forward in float64.

    Dense: q [B, Hq, Lq, d], k/v [B, Hkv, Lk, d] -> o [B, Hq, Lq, d],
    lse [B, Hq, Lq].  Packed: q [Tq, Hq, d], k/v [Tk, Hkv, d] plus
    cu_seqlens_q / cu_seqlens_k (length B + 1) -> o [Tq, Hq, d], lse [Hq, Tq].
    scale=None means 1/sqrt(d) (training tutorial, section 8.5).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    scale = float(scale)
    varlen = cu_seqlens_q is not None or cu_seqlens_k is not None
    if varlen:
        if cu_seqlens_q is None or cu_seqlens_k is None:
            raise ValueError("cu_seqlens_q and cu_seqlens_k go together")
        cq = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
        ck = [int(x) for x in np.asarray(cu_seqlens_k).reshape(-1)]
        if len(cq) != len(ck):
            raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
        hq, hkv = q.shape[1], k.shape[1]
        g = _check_heads(hq, hkv)
        o = np.zeros(q.shape[:2] + (v.shape[-1],), dtype=np.float64)
        lse = np.full((hq, q.shape[0]), NEG_INF, dtype=np.float64)
        for b in range(len(cq) - 1):
            qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
            for h in range(hq):
                hk = h // g
                ob, lb = _attend_one_head(q[qs:qe, h], k[ks:ke, hk],
                                          v[ks:ke, hk], scale, causal,
                                          row_chunk)
                o[qs:qe, h] = ob
                lse[h, qs:qe] = lb
        return o, lse
    bsz, hq, lq, _ = q.shape
    hkv = k.shape[1]
    g = _check_heads(hq, hkv)
    o = np.zeros((bsz, hq, lq, v.shape[-1]), dtype=np.float64)
    lse = np.full((bsz, hq, lq), NEG_INF, dtype=np.float64)
    for b in range(bsz):
        for h in range(hq):
            hk = h // g
            o[b, h], lse[b, h] = _attend_one_head(q[b, h], k[b, hk], v[b, hk],
                                                  scale, causal, row_chunk)
    return o, lse


def row_probabilities(qh, kh, scale, causal=False):
    """P = softmax(scale * Q K^T) with the causal rule, for one head [Lq, Lk].

    Rows with no visible key are all zero.
    """
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    lq, lk = qh.shape[0], kh.shape[0]
    s = float(scale) * (qh @ kh.T)
    s = np.where(_allowed_mask(0, lq, lq, lk, causal), s, NEG_INF)
    m = s.max(axis=1)
    p = np.zeros_like(s)
    live = np.isfinite(m)
    e = np.exp(s[live] - m[live, None])
    p[live] = e / e.sum(axis=1)[:, None]
    return p


# ---------------------------------------------------------------------------
# Online recurrences (section 3.1 of the fusion notes; the Day 14 pseudocode)
# ---------------------------------------------------------------------------

def _blocks(n, boundaries):
    """Split range(n) at the given interior boundaries (sorted, deduplicated)."""
    cuts = sorted({int(b) for b in boundaries if 0 < int(b) < n})
    edges = [0] + cuts + [n]
    return [(edges[i], edges[i + 1]) for i in range(len(edges) - 1)]


def online_softmax_ul(scores, values, boundaries):
    """The (m, l, u) recurrence over key blocks for ONE query row.

    scores: [L] already-scaled scores (may hold -inf for hidden keys);
    values: [L, dv].  Blocks end at the given boundaries.  Returns a dict with
    'out' (= u / l, zeros if no key is visible), 'lse' (= m + ln l) and
    'trace', a list of (m, l, u, r) after each block, where r is the factor
    exp(m_old - m_new) that was applied to the old l and u.
    """
    s = np.asarray(scores, dtype=np.float64).reshape(-1)
    val = np.asarray(values, dtype=np.float64).reshape(s.shape[0], -1)
    m, ell = NEG_INF, 0.0
    u = np.zeros(val.shape[1], dtype=np.float64)
    trace = []
    for a, b in _blocks(s.shape[0], boundaries):
        m_new = max(m, float(s[a:b].max()))
        if m_new == NEG_INF:                  # nothing visible yet: no change
            trace.append((m, ell, u.copy(), 1.0))
            continue
        r = math.exp(m - m_new)               # exp(-inf) = 0 on the first block
        w = np.exp(s[a:b] - m_new)            # weights relative to the new max
        ell = r * ell + float(w.sum())
        u = r * u + w @ val[a:b]
        m = m_new
        trace.append((m, ell, u.copy(), r))
    if m == NEG_INF:
        return {"out": np.zeros_like(u), "lse": NEG_INF, "trace": trace}
    return {"out": u / ell, "lse": m + math.log(ell), "trace": trace}


def _block_partial(s_blk, v_blk):
    """One key block on its own: (m_b, l_b, o_b) with m_b its max score,
    l_b = sum exp(s - m_b) and o_b the block's normalised output (its
    weighted value sum divided by l_b).  None if the block has no visible key.
    """
    m_b = float(s_blk.max())
    if m_b == NEG_INF:
        return None
    w = np.exp(s_blk - m_b)
    l_b = float(w.sum())
    return m_b, l_b, (w @ v_blk) / l_b


def _merge_normalised(a, b):
    """Combine two normalised partial results over disjoint key sets.

    Both are re-expressed relative to the larger max m: their exp-sums are
    scaled by exp(m_side - m) (the rescaling factor r of section 3.1) and the
    merged output is the exp-sum-weighted mean of the two outputs.
    """
    if a is None:
        return b
    if b is None:
        return a
    m = max(a[0], b[0])
    la = a[1] * math.exp(a[0] - m)
    lb = b[1] * math.exp(b[0] - m)
    ell = la + lb
    return m, ell, (la * a[2] + lb * b[2]) / ell


def online_softmax_normalised(scores, values, boundaries):
    """The normalised-output form of the recurrence for ONE query row.

    The state after each block is (m, l, o) with o already divided by l (the
    Day-14 notes keep o in this form).  Each key block is reduced to its own
    normalised partial result, which is merged into the running state by the
    combination rule above: the old state's weight is alpha * l with
    alpha = exp(m - m_new), the block's is its exp-sum relative to m_new.
    Returns (o, lse).
    """
    s = np.asarray(scores, dtype=np.float64).reshape(-1)
    val = np.asarray(values, dtype=np.float64).reshape(s.shape[0], -1)
    state = None
    for a, b in _blocks(s.shape[0], boundaries):
        state = _merge_normalised(state, _block_partial(s[a:b], val[a:b]))
    if state is None:
        return np.zeros(val.shape[1], dtype=np.float64), NEG_INF
    m, ell, o = state
    return o, m + math.log(ell)


def attention_blocked(q, k, v, scale=None, causal=False, boundaries=(64,),
                      normalised=False):
    """Dense attention through the online recurrence with arbitrary key blocks.

    Same layouts as attention() (dense only).  boundaries: interior key split
    points shared by every row.  normalised=True uses the (m, l, o) form.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, hq, lq, d = q.shape
    hkv, lk = k.shape[1], k.shape[2]
    g = _check_heads(hq, hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((bsz, hq, lq, v.shape[-1]), dtype=np.float64)
    lse = np.full((bsz, hq, lq), NEG_INF, dtype=np.float64)
    if lk == 0:
        return o, lse
    for b in range(bsz):
        for h in range(hq):
            hk = h // g
            s = float(scale) * (q[b, h] @ k[b, hk].T)
            s = np.where(_allowed_mask(0, lq, lq, lk, causal), s, NEG_INF)
            for i in range(lq):
                if normalised:
                    o[b, h, i], lse[b, h, i] = online_softmax_normalised(
                        s[i], v[b, hk], boundaries)
                else:
                    res = online_softmax_ul(s[i], v[b, hk], boundaries)
                    o[b, h, i], lse[b, h, i] = res["out"], res["lse"]
    return o, lse


# ---------------------------------------------------------------------------
# Scalar brute force for tiny shapes
# ---------------------------------------------------------------------------

def attention_bruteforce(q, k, v, scale, causal=False):
    """Scalar-loop attention (math.exp, math.fsum) for tiny dense shapes.

    Same layouts and conventions as attention(); deliberately written without
    numpy arithmetic so that it checks the vectorised path independently.
    """
    qn = np.asarray(q, dtype=np.float64).tolist()
    kn = np.asarray(k, dtype=np.float64).tolist()
    vn = np.asarray(v, dtype=np.float64).tolist()
    bsz, hq = len(qn), len(qn[0])
    hkv = len(kn[0])
    g = _check_heads(hq, hkv)
    lq = len(qn[0][0])
    lk = len(kn[0][0])
    d = len(qn[0][0][0]) if lq else 0
    dv = len(vn[0][0][0]) if lk else d
    o = [[[[0.0] * dv for _ in range(lq)] for _ in range(hq)] for _ in range(bsz)]
    lse = [[[NEG_INF] * lq for _ in range(hq)] for _ in range(bsz)]
    for b in range(bsz):
        for h in range(hq):
            hk = h // g
            for i in range(lq):
                vis = [j for j in range(lk)
                       if (not causal) or j <= i + lk - lq]
                if not vis:
                    continue
                sc = {j: scale * math.fsum(qn[b][h][i][c] * kn[b][hk][j][c]
                                           for c in range(d)) for j in vis}
                top = max(sc.values())
                w = {j: math.exp(sc[j] - top) for j in vis}
                z = math.fsum(w.values())
                for c in range(dv):
                    o[b][h][i][c] = math.fsum(w[j] * vn[b][hk][j][c]
                                              for j in vis) / z
                lse[b][h][i] = top + math.log(z)
    return np.array(o, dtype=np.float64), np.array(lse, dtype=np.float64)
