"""GPU parity on tensors of 2^31 elements (4 GiB of bf16 each): the element
offsets of the last sequences pass 2^31 and their byte offsets 2^32, so a
32-bit index anywhere between the binding and the kernels would show here.
The inputs are drawn on the GPU; sampled (sequence, head) slices, among them
the last, are copied back and checked against the fp64 oracle at the usual
bars (O max-abs 1e-2, LSE max-abs 1e-3).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import compare, note

pytestmark = pytest.mark.gpu

B, H, L, D = 64, 32, 8192, 128           # B * H * L * D = 2^31
SAMPLES = [(B - 1, H - 1), (B - 1, 0), (B // 2, 7), (0, 0)]


def _randn(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, device="cuda", dtype=torch.bfloat16, generator=g)


def _f64(t):
    return workloads.to_f64(t.cpu())


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_forward_query_and_output_of_2_31_elements():
    """Q and O of [64, 32, 8192, 128]; 64 keys per sequence."""
    import exact_attention_61_amd as mi
    note(f"large forward: q/o [{B}, {H}, {L}, {D}] bf16, lk 64")
    q = _randn((B, H, L, D), 1)
    k = _randn((B, H, 64, D), 2)
    v = _randn((B, H, 64, D), 3)
    o, lse = mi.forward(q, k, v, causal=False)
    torch.cuda.synchronize()
    rows = slice(L - 160, L)             # the last rows of the sequence
    for b, h in SAMPLES:
        o_ref, l_ref = oracle.attention(_f64(q[b:b + 1, h:h + 1, rows]),
                                        _f64(k[b:b + 1, h:h + 1]), _f64(v[b:b + 1, h:h + 1]))
        eo, el = compare(_f64(o[b:b + 1, h:h + 1, rows]), _f64(lse[b:b + 1, h:h + 1, rows]),
                         o_ref, l_ref)
        note(f"  b {b} h {h}: err_O {eo:.3e}  err_LSE {el:.3e}")


def test_forward_keys_and_values_of_2_31_elements():
    """K and V of [64, 32, 8192, 128]; 64 causal query rows per sequence
    (bottom-right: the last query row sees every key)."""
    import exact_attention_61_amd as mi
    note(f"large forward: k/v [{B}, {H}, {L}, {D}] bf16, lq 64, causal")
    q = _randn((B, H, 64, D), 4)
    k = _randn((B, H, L, D), 5)
    v = _randn((B, H, L, D), 6)
    o, lse = mi.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    for b, h in SAMPLES:
        o_ref, l_ref = oracle.attention(_f64(q[b:b + 1, h:h + 1]), _f64(k[b:b + 1, h:h + 1]),
                                        _f64(v[b:b + 1, h:h + 1]), causal=True)
        eo, el = compare(_f64(o[b:b + 1, h:h + 1]), _f64(lse[b:b + 1, h:h + 1]), o_ref, l_ref)
        note(f"  b {b} h {h}: err_O {eo:.3e}  err_LSE {el:.3e}")


def test_decode_on_a_cache_of_2_31_elements():
    """One new query row per sequence and 2 query heads per kv head against
    a [64, 32, 8192, 128] cache; every head of the sampled sequences."""
    import exact_attention_61_amd as mi
    note(f"large decode: cache [{B}, {H}, {L}, {D}] bf16, hq {2 * H}, lq 1")
    q = _randn((B, 2 * H, 1, D), 7)
    k = _randn((B, H, L, D), 8)
    v = _randn((B, H, L, D), 9)
    o, lse = mi.decode(q, k, v, causal=True)
    torch.cuda.synchronize()
    for b in sorted({s[0] for s in SAMPLES}):
        o_ref, l_ref = oracle.attention(_f64(q[b:b + 1]), _f64(k[b:b + 1]), _f64(v[b:b + 1]),
                                        causal=True)
        eo, el = compare(_f64(o[b:b + 1]), _f64(lse[b:b + 1]), o_ref, l_ref)
        note(f"  b {b}: err_O {eo:.3e}  err_LSE {el:.3e}")
    assert np.isfinite(lse.float().cpu().numpy()).all()
