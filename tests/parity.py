"""Helpers shared by the GPU parity tests: run the library, run the oracle on
the same CPU inputs, compare element by element."""

import math
import sys

import numpy as np
import torch

import oracle
import workloads

# Tolerances of the attention forward against the fp64 oracle: the output's
# max-abs error (any output dtype) and the log-sum-exp's max-abs error.
TOL_O = 1e-2
TOL_LSE = 1e-3


def note(msg):
    """Name the case before a GPU step, flushed, so a crash still shows it."""
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(q, k, v, **kw):
    import exact_attention_61_amd as mi
    dev = torch.device("cuda", 0)
    args = {}
    for name in ("cu_seqlens_q", "cu_seqlens_k"):
        if kw.get(name) is not None:
            args[name] = kw.pop(name).to(dev)
    o, lse = mi.forward(q.to(dev), k.to(dev), v.to(dev), **args, **kw)
    torch.cuda.synchronize()
    return (o.to("cpu", torch.float64).numpy(),
            None if lse is None else lse.to("cpu", torch.float64).numpy())


def compare(o_gpu, lse_gpu, o_ref, lse_ref, tol_o=TOL_O, tol_lse=TOL_LSE,
            row_mask=None):
    """Max-abs errors; rows whose oracle LSE is -inf must be exactly -inf / 0.

    o_* are [..., d] and lse_* the matching [...] (same leading shape after
    the caller arranges it).  row_mask selects the rows that exist.
    """
    o_gpu = np.asarray(o_gpu)
    o_ref = np.asarray(o_ref)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), "non-finite output"
    err_o = float(np.max(np.abs(o_gpu - o_ref))) if o_gpu.size else 0.0
    assert err_o <= tol_o, f"max|dO| = {err_o:.3e} > {tol_o}"
    err_l = 0.0
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu)
        lse_ref = np.asarray(lse_ref)
        assert lse_gpu.shape == lse_ref.shape
        dead = ~np.isfinite(lse_ref)
        assert np.all(lse_gpu[dead] == -math.inf), "dead row LSE must be -inf"
        assert np.all(np.isfinite(lse_gpu[~dead])), "live row LSE not finite"
        if (~dead).any():
            err_l = float(np.max(np.abs(lse_gpu[~dead] - lse_ref[~dead])))
        assert err_l <= tol_lse, f"max|dLSE| = {err_l:.3e} > {tol_lse}"
    return err_o, err_l


def dense_case(b, hq, hkv, lq, lk, d, dtype, causal, scale=None,
               out_dtype=None, seed=0, layout="bhsd", **select):
    """One dense case through the ABI against the oracle; select may hold
    kernel= / causal_order= for mi_attn_fwd_select."""
    q, k, v = workloads.make_dense(b, hq, hkv, lq, lk, d, dtype, seed)
    if layout == "bshd":
        qg, kg, vg = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    else:
        qg, kg, vg = q, k, v
    o, lse = run_gpu(qg, kg, vg, causal=causal, scale=scale,
                     out_dtype=out_dtype, layout=layout, **select)
    if layout == "bshd":
        o = o.transpose(0, 2, 1, 3)
    o_ref, l_ref = oracle.attention(workloads.to_f64(q), workloads.to_f64(k),
                                    workloads.to_f64(v), scale=scale,
                                    causal=causal)
    return compare(o, lse, o_ref, l_ref)
