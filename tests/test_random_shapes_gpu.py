"""GPU parity over seeded random shapes: the forward (dense and packed, with
and without dropout) and the decode call against the fp64 oracle.

The named workloads and the hand-picked edge cases elsewhere fix particular
sizes; here one seeded generator draws batch, head counts (any GQA ratio),
lengths on both sides (1 to a few hundred, Lq != Lk, lengths 0 inside packed
batches), head size, input and output types, causal flag, dropout
probability and decode split count, so that tile edges, ragged tails and
their combinations are hit in mixes no one chose.  Same bars as the other
parity tests: O max-abs 1e-2 (scaled by 1 / (1 - p) with dropout), LSE
max-abs 1e-3, rows with no visible key exactly O = 0, LSE = -inf.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import TOL_O, compare, note, run_gpu

pytestmark = pytest.mark.gpu

DTYPES = [torch.float16, torch.bfloat16]
N_CASES = 24


def draw(i):
    """Case i of the sweep (a pure function of i)."""
    r = np.random.default_rng(9000 + i)
    d = int(r.choice([64, 128]))
    dtype = DTYPES[int(r.integers(2))]
    out = torch.float32 if r.random() < 0.3 else None     # the input type or fp32
    hkv = int(r.integers(1, 4))
    hq = hkv * int(r.choice([1, 1, 2, 3, 4, 7]))
    causal = bool(r.random() < 0.5)
    p = float(r.choice([0.0, 0.0, 0.0, 0.15, 0.4]))
    packed = bool(r.random() < 0.4)
    if packed:
        nb = int(r.integers(1, 6))
        lq = [int(x) for x in r.integers(0, 400, nb)]
        lk = [int(x) if r.random() < 0.5 else lq[j] for j, x in enumerate(r.integers(0, 400, nb))]
        if r.random() < 0.4:             # a sequence with no query rows
            lq[int(r.integers(nb))] = 0
        if r.random() < 0.3:             # a sequence with no keys (dead rows)
            lk[int(r.integers(nb))] = 0
        return dict(kind="packed", d=d, dtype=dtype, out=out, hq=hq, hkv=hkv, causal=causal,
                    p=p, lq=lq, lk=lk, seed=int(r.integers(1 << 40)))
    b = int(r.integers(1, 4))
    lq = int(r.integers(1, 420))
    lk = lq if r.random() < 0.4 else int(r.integers(1, 420))
    return dict(kind="dense", d=d, dtype=dtype, out=out, hq=hq, hkv=hkv, causal=causal, p=p,
                b=b, lq=lq, lk=lk, seed=int(r.integers(1 << 40)))


def tag(c):
    sizes = (f"lq {c['lq']} lk {c['lk']}" if c["kind"] == "packed"
             else f"b {c['b']} lq {c['lq']} lk {c['lk']}")
    return (f"{c['kind']} d {c['d']} {c['dtype']} out {c['out']} hq {c['hq']} hkv {c['hkv']} "
            f"causal {c['causal']} p {c['p']} {sizes}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_forward(i):
    c = draw(i)
    note(f"random case {i}: {tag(c)}")
    f64 = workloads.to_f64
    kw = dict(causal=c["causal"], out_dtype=c["out"])
    if c["p"]:
        kw.update(dropout_p=c["p"], seed=c["seed"])
    if c["kind"] == "packed":
        q, k, v, cq, ck = workloads.make_packed(c["lq"], c["lk"], c["hq"], c["hkv"], c["d"],
                                                c["dtype"], seed=i)
        o, lse = run_gpu(q, k, v, cu_seqlens_q=cq, cu_seqlens_k=ck,
                         max_seqlen_q=max(c["lq"]), max_seqlen_k=max(c["lk"]), **kw)
        ref_kw = dict(causal=c["causal"], cu_seqlens_q=cq.numpy(), cu_seqlens_k=ck.numpy())
    else:
        q, k, v = workloads.make_dense(c["b"], c["hq"], c["hkv"], c["lq"], c["lk"], c["d"],
                                       c["dtype"], seed=i)
        o, lse = run_gpu(q, k, v, **kw)
        ref_kw = dict(causal=c["causal"])
    if c["p"]:
        o_ref, l_ref = oracle.attention_dropout(f64(q), f64(k), f64(v), p=c["p"],
                                                seed=c["seed"], **ref_kw)
    else:
        o_ref, l_ref = oracle.attention(f64(q), f64(k), f64(v), **ref_kw)
    eo, el = compare(o, lse, o_ref, l_ref, tol_o=TOL_O / (1.0 - c["p"]))
    note(f"  err_O {eo:.3e}  err_LSE {el:.3e}")


def draw_decode(i):
    r = np.random.default_rng(7000 + i)
    d = int(r.choice([64, 128]))
    hkv = int(r.integers(1, 5))
    hq = hkv * int(r.choice([1, 2, 4, 8]))
    b = int(r.integers(1, 4))
    lq = int(r.integers(1, 9))
    lk = int(r.integers(1, 3000))
    seqlens = ([int(x) for x in r.integers(0, lk + 1, b)] if r.random() < 0.5 else None)
    return dict(d=d, dtype=DTYPES[int(r.integers(2))], hq=hq, hkv=hkv, b=b, lq=lq, lk=lk,
                seqlens=seqlens, causal=bool(r.random() < 0.7),
                splits=int(r.choice([0, 0, 1, 3, 7])))


@pytest.mark.parametrize("i", range(12))
def test_random_decode(i):
    import exact_attention_61_amd as mi
    c = draw_decode(i)
    note(f"random decode {i}: {c}")
    q, k, v = workloads.make_dense(c["b"], c["hq"], c["hkv"], c["lq"], c["lk"], c["d"],
                                   c["dtype"], seed=100 + i)
    dev = torch.device("cuda", 0)
    sl = (None if c["seqlens"] is None
          else torch.tensor(c["seqlens"], dtype=torch.int32, device=dev))
    o, lse = mi.decode(q.to(dev), k.to(dev), v.to(dev), seqlens_k=sl, causal=c["causal"],
                       num_splits=c["splits"])
    torch.cuda.synchronize()
    o = o.to("cpu", torch.float64).numpy()
    lse = lse.to("cpu", torch.float64).numpy()
    f64 = workloads.to_f64
    qd, kd, vd = f64(q), f64(k), f64(v)
    o_ref = np.zeros(qd.shape)
    l_ref = np.full(qd.shape[:3], -math.inf)
    for j in range(c["b"]):
        n = c["lk"] if c["seqlens"] is None else c["seqlens"][j]
        o_ref[j:j + 1], l_ref[j:j + 1] = oracle.attention(
            qd[j:j + 1], kd[j:j + 1, :, :n], vd[j:j + 1, :, :n], causal=c["causal"])
    eo, el = compare(o, lse, o_ref, l_ref)
    note(f"  err_O {eo:.3e}  err_LSE {el:.3e}")
