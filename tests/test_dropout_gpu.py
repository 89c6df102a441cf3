"""GPU parity of mi_attn_fwd_dropout against the fp64 dropout oracle.

Both sides draw the keep mask from Philox4x32-10 on the same counters and
decide it by the same integer comparison, so the masks are identical and the
outputs compare element by element.  Tolerances: the attention ones scaled
by the dropout's keep scale 1 / (1 - p) for O -- every kept probability, and
with it the output and its rounding to the working type, is multiplied by
that scale (a bf16 output of magnitude 4..8 already carries a rounding
error up to 2^-6) -- so max-abs 1e-2 / (1 - p) on O; 1e-3 on LSE, which is
that of the softmax before dropout; rows with no visible key exactly O = 0
and LSE = -inf.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import TOL_O, compare, note

pytestmark = pytest.mark.gpu

F16, BF16 = torch.float16, torch.bfloat16


def run_drop(q, k, v, p, seed, causal, **kw):
    import exact_attention_61_amd as mi
    o, lse = mi.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, dropout_p=p, seed=seed,
                        **kw)
    torch.cuda.synchronize()
    return o.to("cpu", torch.float64).numpy(), lse.to("cpu", torch.float64).numpy()


def dense_drop_case(b, hq, hkv, lq, lk, d, dtype, causal, p, seed, data_seed=0, **kw):
    q, k, v = workloads.make_dense(b, hq, hkv, lq, lk, d, dtype, data_seed)
    o, lse = run_drop(q, k, v, p, seed, causal, **kw)
    f64 = workloads.to_f64
    o_ref, l_ref = oracle.attention_dropout(f64(q), f64(k), f64(v), p=p, seed=seed,
                                            causal=causal, scale=kw.get("scale"))
    return compare(o, lse, o_ref, l_ref, tol_o=TOL_O / (1.0 - p))


@pytest.mark.parametrize("d,dtype", [(64, F16), (64, BF16), (128, F16), (128, BF16)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_dense(d, dtype, causal, p):
    note(f"dropout d {d} {dtype} causal {causal} p {p}")
    eo, el = dense_drop_case(2, 4, 2, 300, 300, d, dtype, causal, p, seed=0x1234_5678_9ABC)
    note(f"  err_O {eo:.3e}  err_LSE {el:.3e}")


@pytest.mark.parametrize("lq,lk", [(1, 700), (129, 65), (64, 1000), (200, 1)])
def test_dropout_cross_and_tails(lq, lk):
    note(f"dropout lq {lq} lk {lk}")
    dense_drop_case(1, 4, 1, lq, lk, 64, BF16, True, 0.2, seed=99)
    dense_drop_case(1, 4, 1, lq, lk, 128, F16, False, 0.2, seed=98)


def test_dropout_varlen():
    lens_q = [300, 1, 0, 129, 64]
    lens_k = [300, 5, 3, 0, 200]
    note(f"dropout varlen {lens_q} {lens_k}")
    q, k, v, cq, ck = workloads.make_packed(lens_q, lens_k, 4, 2, 64, BF16, seed=3)
    for causal in (False, True):
        o, lse = run_drop(q, k, v, 0.3, 42, causal, cu_seqlens_q=cq.cuda(),
                          cu_seqlens_k=ck.cuda(), max_seqlen_q=max(lens_q),
                          max_seqlen_k=max(lens_k))
        f64 = workloads.to_f64
        o_ref, l_ref = oracle.attention_dropout(f64(q), f64(k), f64(v), p=0.3, seed=42,
                                                causal=causal, cu_seqlens_q=cq.numpy(),
                                                cu_seqlens_k=ck.numpy())
        compare(o, lse, o_ref, l_ref, tol_o=TOL_O / 0.7)


def test_dropout_seed_and_repeatability():
    """Same seed: bit-identical outputs; another seed: another mask; LSE
    does not depend on the mask."""
    q, k, v = workloads.make_dense(1, 4, 4, 256, 256, 64, F16, 5)
    a = run_drop(q, k, v, 0.25, 7, False)
    b = run_drop(q, k, v, 0.25, 7, False)
    c = run_drop(q, k, v, 0.25, 8, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.max(np.abs(a[0] - c[0])) > 1e-2
    assert np.max(np.abs(a[1] - c[1])) <= 1e-6


def test_dropout_zero_is_the_forward():
    import exact_attention_61_amd as mi
    q, k, v = workloads.make_dense(1, 4, 2, 200, 200, 128, BF16, 6)
    o0, l0 = run_drop(q, k, v, 0.0, 1, True)
    o1, l1 = mi.forward(q.cuda(), k.cuda(), v.cuda(), causal=True)
    assert np.array_equal(o0, o1.to("cpu", torch.float64).numpy())
    assert np.array_equal(l0, l1.to("cpu", torch.float64).numpy())


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_dropout_with_safe_form_redo(dtype):
    """A late key far above the first tile's maximum sends the q-tile through
    the safe form; its mask must be the same as in the short form."""
    note(f"dropout redo {dtype}")
    q, k, v = workloads.make_dense(1, 2, 2, 128, 640, 64, dtype, 7)
    boost = 30.0 if dtype == F16 else 300.0
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    k[:, :, 600, 0] = boost               # score 2^boost-ish relative to the first tile
    o, lse = run_drop(q, k, v, 0.2, 11, False, scale=1.0)
    f64 = workloads.to_f64
    o_ref, l_ref = oracle.attention_dropout(f64(q), f64(k), f64(v), p=0.2, seed=11, scale=1.0)
    compare(o, lse, o_ref, l_ref, tol_o=TOL_O / 0.8)


@pytest.mark.parametrize("name", ["bert_varlen"])
def test_dropout_workload(name):
    """The packed BERT-style batch with the tutorial's dropout 0.1."""
    w = workloads.WORKLOADS[name]
    inp = workloads.make(name, seed=0)
    note(f"dropout workload {name}")
    o, lse = run_drop(inp["q"], inp["k"], inp["v"], 0.1, 2024, w.causal,
                      cu_seqlens_q=inp["cu_seqlens_q"].cuda(),
                      cu_seqlens_k=inp["cu_seqlens_k"].cuda(),
                      max_seqlen_q=inp["max_seqlen_q"], max_seqlen_k=inp["max_seqlen_k"],
                      scale=w.scale)
    f64 = workloads.to_f64
    o_ref, l_ref = oracle.attention_dropout(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), p=0.1,
                                            seed=2024, causal=w.causal, scale=w.scale,
                                            cu_seqlens_q=inp["cu_seqlens_q"].numpy(),
                                            cu_seqlens_k=inp["cu_seqlens_k"].numpy())
    eo, el = compare(o, lse, o_ref, l_ref, tol_o=TOL_O / 0.9)
    note(f"  err_O {eo:.3e}  err_LSE {el:.3e}")
