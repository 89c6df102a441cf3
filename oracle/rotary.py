"""Plain fp64 CPU oracle for the rotary position embedding.

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's
CPU-baseline leg, never by the product path.  It shares no code with the HIP
library.

Source: the "Training integration" tutorial (inference.lei6393.com), section
4: rotary embedding applied to Q and K before attention, with a rotary
dimension (even, usually the head dimension), a base frequency (10000), a
choice between the GPT-NeoX layout (interleaved = False) and the GPT-J layout
(interleaved = True), and, for generation with a KV cache (section 4.3), a
position offset: the new tokens' positions start at the cache length.

The pages give the interface, not the formula.  This oracle takes the plainest
reading, the rotary embedding as originally defined (each pair of features is
rotated by an angle proportional to the token position):

* pair k (k = 0 .. rd/2 - 1) turns at the inverse frequency
  base ** (-2k / rd), so at position p its angle is p * base ** (-2k / rd);
* GPT-NeoX layout: pair k is features (k, k + rd/2); GPT-J layout: pair k is
  features (2k, 2k + 1);
* a pair (x, y) becomes (x cos a - y sin a, x sin a + y cos a);
* features rd .. d-1 are left unchanged;
* the position of row t of sequence b is offset + offsets[b] + t.

The xPos variant of section 4.4 (scale_base) is not modelled: the pages do
not say how its scale depends on the position.

Everything is computed in float64 on the exact input values.
"""

import numpy as np


def inverse_frequencies(rotary_dim, base):
    """base ** (-2k / rotary_dim) for k = 0 .. rotary_dim/2 - 1, in fp64."""
    if rotary_dim <= 0 or rotary_dim % 2:
        raise ValueError("rotary_dim must be a positive even number")
    k = np.arange(rotary_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * k / rotary_dim)


def pair_indices(rotary_dim, interleaved):
    """(first, second) feature index of every rotated pair."""
    half = rotary_dim // 2
    k = np.arange(half)
    if interleaved:
        return 2 * k, 2 * k + 1
    return k, k + half


def rotate(x, positions, rotary_dim, base=10000.0, interleaved=False):
    """Rotary embedding of x [..., L, d] whose rows sit at positions [L].

    Returns a new float64 array; x is not modified.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if rotary_dim > d:
        raise ValueError("rotary_dim exceeds the feature dimension")
    pos = np.asarray(positions, dtype=np.float64)
    if pos.shape != (x.shape[-2],):
        raise ValueError("one position per row")
    angle = pos[:, None] * inverse_frequencies(rotary_dim, base)[None, :]
    c, s = np.cos(angle), np.sin(angle)
    i0, i1 = pair_indices(rotary_dim, interleaved)
    out = x.copy()
    a, b = x[..., i0], x[..., i1]
    out[..., i0] = a * c - b * s
    out[..., i1] = a * s + b * c
    return out


def rotate_dense(x, rotary_dim, base=10000.0, interleaved=False, offset=0,
                 offsets=None):
    """x [B, H, L, d]: row t of batch b at position offset + offsets[b] + t."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    bsz, _, seq, _ = x.shape
    for b in range(bsz):
        start = offset + (0 if offsets is None else int(offsets[b]))
        out[b] = rotate(x[b], start + np.arange(seq), rotary_dim, base, interleaved)
    return out


def rotate_packed(x, cu_seqlens, rotary_dim, base=10000.0, interleaved=False,
                  offset=0, offsets=None):
    """x [T, H, d] packed: row t of sequence b at offset + offsets[b] + t."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    cu = [int(c) for c in cu_seqlens]
    for b in range(len(cu) - 1):
        n = cu[b + 1] - cu[b]
        if n == 0:
            continue
        start = offset + (0 if offsets is None else int(offsets[b]))
        rows = x[cu[b]:cu[b + 1]].transpose(1, 0, 2)          # [H, n, d]
        out[cu[b]:cu[b + 1]] = rotate(rows, start + np.arange(n), rotary_dim, base,
                                      interleaved).transpose(1, 0, 2)
    return out
