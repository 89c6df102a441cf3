"""mi_attn_decode_noalloc (static scratch, no allocation) against
mi_attn_decode (caller workspace) and the fp64 oracle, on two calls in a
row, the second with a smaller input."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import compare, note

pytestmark = pytest.mark.gpu


def _run(mi, noalloc, q, k, v, splits):
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if noalloc:
        mi.mi_attn_decode_noalloc(q, k, v, o, lse, causal=True, num_splits=splits)
    else:
        b, hq, lq, d = q.shape
        n = mi.mi_attn_decode_workspace_size(b, hq, k.shape[1], lq, k.shape[2], d, splits)
        ws = torch.zeros(max(n, 1), dtype=torch.uint8, device=q.device)
        mi.mi_attn_decode(q, k, v, o, lse, causal=True, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_decode(order):
    import exact_attention_61_amd as mi
    dev = torch.device("cuda", 0)
    cases = [(8, 32, 8, 1, 8192, 128, torch.bfloat16, 0),
             (2, 8, 2, 3, 1000, 64, torch.float16, 3)]
    for b, hq, hkv, lq, lk, d, dt, splits in cases:
        note(f"decode noalloc b{b} hq{hq} hkv{hkv} lq{lq} lk{lk} d{d} {dt} splits {splits}")
        q, k, v = workloads.make_dense(b, hq, hkv, lq, lk, d, dt, seed=11)
        qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
        o_ws, l_ws = _run(mi, False, qg, kg, vg, splits)
        o_na, l_na = _run(mi, True, qg, kg, vg, splits)
        # same kernels, same splits, same merge order: identical results
        assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na)
        o_ref, l_ref = oracle.attention(workloads.to_f64(q), workloads.to_f64(k),
                                        workloads.to_f64(v), causal=True)
        compare(o_na.double().cpu().numpy(), l_na.double().cpu().numpy(), o_ref, l_ref)
