"""Seeded synthetic inputs for the attention forward pass.

This module only draws numbers and lays them out: it holds none of the
attention arithmetic, so both the oracle side and the HIP side of every test
can take their inputs from it.

Every tensor is drawn on the CPU with torch.Generator().manual_seed(seed): Q
first, then K, then V, each as float32 N(0, 1) rounded to the working dtype
(round to nearest even).  Variable sequence lengths come from numpy's
default_rng(seed).integers(lo, hi + 1) (inclusive bounds).

The five named workloads follow the shapes the pages use:

* tiny:    one head, 128 x 128, d = 64, bf16 in, fp32 out (unit case).
* causal_b2h16: B=2, H=16, N=2048, d=64, causal, fp16 (the SDPA experiment of
           the "Day 14" notes, experiment 2).
* bert_varlen: B=8, 12 heads of d=64 (embed 768, training tutorial 2.1), each
           valid length uniform in [256, 1024], packed with cu_seqlens
           (tutorial 2.5: padding mask -> packed sequences).
* gqa_causal: B=1, L=4096, 32 query heads, 8 KV heads, d=128, causal, bf16
           (tutorial 2.3).
* long_8k: B=1, H=16, L=8192, d=128, non-causal, bf16 (the L=8192, d=128
           sizing table of the fusion notes, section 3).
* long_4k: long_8k at L=4096 (a check that HBM reads scale with L).
* bert_dropout: bert_varlen with the tutorial's attention dropout 0.1
           (sections 2.1 and 8.2), mask seed 2024.
* rotary_gqa: the rotary embedding (tutorial section 4, GPT-NeoX layout,
           rotary dimension = head dimension, base 10000) of the gqa_causal
           Q and K, in place.
* decode_gqa: one new token per sequence against an 8192-token key/value
           cache: B=8, 32 query heads over 8 KV heads, d=128, bf16, causal
           (bottom-right: the new token follows the cache, tutorial section
           4.3); the GQA grouping of tutorial section 2.3.
"""

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    hq: int
    hkv: int
    lq: int            # dense: sequence length; varlen: max length
    lk: int
    d: int
    causal: bool
    in_dtype: str      # "f16" | "bf16"
    out_dtype: str     # "f16" | "bf16" | "f32"
    scale: float
    varlen: bool = False
    len_range: tuple = field(default=(0, 0))   # varlen: inclusive [lo, hi]
    decode: bool = False   # a few query rows against a key/value cache
    rotary: bool = False   # the rotary embedding of Q and K, in place
    dropout: float = 0.0   # dropout probability on P (seed 2024)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 128, 128, 64, False, "bf16", "f32",
                     1.0 / 8.0),
    "causal_b2h16": Workload("causal_b2h16", 2, 16, 16, 2048, 2048, 64, True,
                             "f16", "f16", 1.0 / 8.0),
    "bert_varlen": Workload("bert_varlen", 8, 12, 12, 1024, 1024, 64, False,
                            "bf16", "bf16", 1.0 / 8.0, varlen=True,
                            len_range=(256, 1024)),
    "gqa_causal": Workload("gqa_causal", 1, 32, 8, 4096, 4096, 128, True,
                           "bf16", "bf16", 1.0 / math.sqrt(128.0)),
    "long_8k": Workload("long_8k", 1, 16, 16, 8192, 8192, 128, False,
                        "bf16", "bf16", 1.0 / math.sqrt(128.0)),
    "decode_gqa": Workload("decode_gqa", 8, 32, 8, 1, 8192, 128, True,
                           "bf16", "bf16", 1.0 / math.sqrt(128.0), decode=True),
    "bert_dropout": Workload("bert_dropout", 8, 12, 12, 1024, 1024, 64, False,
                             "bf16", "bf16", 1.0 / 8.0, varlen=True,
                             len_range=(256, 1024), dropout=0.1),
    "rotary_gqa": Workload("rotary_gqa", 1, 32, 8, 4096, 4096, 128, False,
                           "bf16", "bf16", 1.0, rotary=True),
    # long_8k at half the length: its HBM read bytes should halve with L
    "long_4k": Workload("long_4k", 1, 16, 16, 4096, 4096, 128, False,
                        "bf16", "bf16", 1.0 / math.sqrt(128.0)),
}

# The workload the benchmark headline is quoted on.
HEADLINE = "causal_b2h16"


def varlen_lengths(batch, lo, hi, seed=0):
    """Per-sequence lengths uniform on the integers lo..hi (both inclusive)."""
    return [int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1,
                                                                  size=batch)]


def cu_seqlens(lengths):
    """Prefix offsets [0, L0, L0+L1, ...] as an int32 tensor."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32)


def randn(shape, dtype, gen):
    """float32 N(0,1) draw rounded to dtype."""
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(dtype)


def make_dense(batch, hq, hkv, lq, lk, d, dtype, seed=0):
    """Q [B,Hq,Lq,d], K/V [B,Hkv,Lk,d] on the CPU, drawn Q, K, V in order."""
    gen = torch.Generator().manual_seed(seed)
    q = randn((batch, hq, lq, d), dtype, gen)
    k = randn((batch, hkv, lk, d), dtype, gen)
    v = randn((batch, hkv, lk, d), dtype, gen)
    return q, k, v


def make_packed(lengths_q, lengths_k, hq, hkv, d, dtype, seed=0):
    """Packed Q [Tq,Hq,d], K/V [Tk,Hkv,d] plus cu_seqlens for each side."""
    gen = torch.Generator().manual_seed(seed)
    tq, tk = sum(lengths_q), sum(lengths_k)
    q = randn((tq, hq, d), dtype, gen)
    k = randn((tk, hkv, d), dtype, gen)
    v = randn((tk, hkv, d), dtype, gen)
    return q, k, v, cu_seqlens(lengths_q), cu_seqlens(lengths_k)


def make(name, seed=0):
    """Inputs of a named workload: a dict with q, k, v (+ cu_seqlens)."""
    w = WORKLOADS[name]
    dt = DTYPES[w.in_dtype]
    if w.varlen:
        lens = varlen_lengths(w.batch, w.len_range[0], w.len_range[1], seed)
        q, k, v, cq, ck = make_packed(lens, lens, w.hq, w.hkv, w.d, dt, seed)
        return {"q": q, "k": k, "v": v, "cu_seqlens_q": cq,
                "cu_seqlens_k": ck, "max_seqlen_q": max(lens),
                "max_seqlen_k": max(lens), "lengths": lens}
    q, k, v = make_dense(w.batch, w.hq, w.hkv, w.lq, w.lk, w.d, dt, seed)
    return {"q": q, "k": k, "v": v}


def to_f64(t):
    """Exact widening of a CPU tensor to a numpy float64 array."""
    return t.detach().to("cpu", torch.float64).numpy()
