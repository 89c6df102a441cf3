"""GPU parity of mi_attn_rotary (in-place rotary embedding) against the fp64
oracle, and of rotary followed by attention against the oracle's rotation
followed by its attention.

Tolerance: the kernel rotates in fp32 and rounds each result to the
working type (nearest even), so each element may be off by one rounding of
its value plus the fp32 arithmetic before it: |gpu - oracle| <= 2^-7 |oracle|
+ 1e-5 for bf16 (8-bit significand) and 2^-10 |oracle| + 1e-5 for fp16 --
twice the half-ulp bound, since the fp32 value may sit on the other side of
a rounding boundary.  Features past the rotary dimension, and rows outside
every sequence of a packed tensor, must come back bit for bit.
"""


import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import compare, note

pytestmark = pytest.mark.gpu

F16, BF16 = torch.float16, torch.bfloat16
REL = {F16: 2.0 ** -10, BF16: 2.0 ** -7}


def check(gpu, ref, dtype):
    g = gpu.to("cpu", torch.float64).numpy()
    err = np.abs(g - ref)
    bound = REL[dtype] * np.abs(ref) + 1e-5
    worst = float(np.max(err - bound))
    assert worst <= 0.0, f"max excess {worst:.3e}, max err {float(np.max(err)):.3e}"
    return float(np.max(err))


def rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return workloads.randn(shape, dtype, g)


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("inter", [False, True])
@pytest.mark.parametrize("d,rd", [(128, 128), (128, 64), (64, 64), (64, 16), (96, 48)])
def test_rotary_dense(dtype, inter, d, rd):
    note(f"rotary dense {dtype} interleaved {inter} d {d} rd {rd}")
    x = rand((2, 3, 77, d), dtype, seed=d + rd)
    ref = oracle.rotate_dense(workloads.to_f64(x), rd, 10000.0, inter)
    import exact_attention_61_amd as mi
    xg = x.cuda()
    mi.mi_attn_rotary(xg, rd, interleaved=inter)
    torch.cuda.synchronize()
    check(xg, ref, dtype)
    assert torch.equal(xg[..., rd:].cpu(), x[..., rd:])


@pytest.mark.parametrize("inter", [False, True])
def test_rotary_bshd_offsets_and_large_positions(inter):
    """[B, L, H, d] layout; a common offset of a million positions plus one
    offset per sequence (a KV cache of different lengths, tutorial 4.3)."""
    import exact_attention_61_amd as mi
    note(f"rotary bshd offsets interleaved {inter}")
    x = rand((3, 40, 4, 128), BF16, seed=5)               # [B, L, H, d]
    offs = [0, 17, 4096]
    ref = oracle.rotate_dense(workloads.to_f64(x).transpose(0, 2, 1, 3), 128, 10000.0, inter,
                              offset=1_000_000, offsets=offs).transpose(0, 2, 1, 3)
    xg = x.cuda()
    mi.mi_attn_rotary(xg, 128, interleaved=inter, position_offset=1_000_000,
                      position_offsets=torch.tensor(offs, dtype=torch.int32, device="cuda"),
                      layout="bshd")
    torch.cuda.synchronize()
    check(xg, ref, BF16)


def test_rotary_base_and_strided_view():
    """Another base, and a strided view (the K half of a packed [B, L, 2, H, d]
    tensor) whose other half must stay as it was."""
    import exact_attention_61_amd as mi
    note("rotary base 500 strided view")
    kv = rand((2, 33, 2, 4, 64), F16, seed=6)
    ref = oracle.rotate_dense(workloads.to_f64(kv[:, :, 0]).transpose(0, 2, 1, 3), 64, 500.0,
                              False).transpose(0, 2, 1, 3)
    g = kv.cuda()
    mi.mi_attn_rotary(g[:, :, 0], 64, base=500.0, layout="bshd")
    torch.cuda.synchronize()
    check(g[:, :, 0], ref, F16)
    assert torch.equal(g[:, :, 1].cpu(), kv[:, :, 1])


@pytest.mark.parametrize("inter", [False, True])
def test_rotary_packed(inter):
    import exact_attention_61_amd as mi
    lens = [5, 0, 300, 1, 64]
    note(f"rotary packed {lens} interleaved {inter}")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    total = int(cu[-1])
    x = rand((total + 7, 8, 128), BF16, seed=7)          # 7 rows past every sequence
    offs = [3, 9, 0, 100000, 2]
    ref = oracle.rotate_packed(workloads.to_f64(x), cu.numpy(), 96, 10000.0, inter,
                               offset=11, offsets=offs)
    xg = x.cuda()
    mi.mi_attn_rotary(xg, 96, interleaved=inter, position_offset=11,
                      position_offsets=torch.tensor(offs, dtype=torch.int32, device="cuda"),
                      cu_seqlens=cu.cuda(), max_seqlen=max(lens))
    torch.cuda.synchronize()
    check(xg, ref, BF16)
    assert torch.equal(xg[total:].cpu(), x[total:])


@pytest.mark.parametrize("causal", [False, True])
def test_rotary_then_attention(causal):
    """The path of the tutorial's MHA with rotary_emb_dim = head_dim: Q and K
    rotated in place, then attention; against the oracle's rotation of the
    exact inputs followed by its attention (the attention tolerances).  In
    fp16: the in-place rotation stores Q and K rounded to the working type,
    which in fp16 (2^-11 relative) moves the output far less than the 1e-2
    bound; in bf16 that rounding alone is of the order of the bound, so bf16
    is covered by the element-wise rotary tests plus the attention tests."""
    import exact_attention_61_amd as mi
    note(f"rotary + attention causal {causal}")
    q, k, v = workloads.make_dense(1, 8, 2, 300, 300, 128, F16, seed=10)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    mi.mi_attn_rotary(qg, 128)
    mi.mi_attn_rotary(kg, 128)
    o, lse = mi.forward(qg, kg, vg, causal=causal)
    torch.cuda.synchronize()
    f64 = workloads.to_f64
    qr = oracle.rotate_dense(f64(q), 128)
    kr = oracle.rotate_dense(f64(k), 128)
    o_ref, l_ref = oracle.attention(qr, kr, f64(v), causal=causal)
    compare(o.to("cpu", torch.float64).numpy(), lse.to("cpu", torch.float64).numpy(),
            o_ref, l_ref)


# mi_attn_rotary_qk: Q and K in one launch, each against the oracle's
# rotation of that tensor (the same bound), with its own head count.
@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("inter", [False, True])
@pytest.mark.parametrize("hq,hkv,d,rd", [(8, 2, 128, 128), (5, 3, 64, 32), (32, 8, 128, 64),
                                         (1, 1, 64, 64)])
def test_rotary_qk_dense(dtype, inter, hq, hkv, d, rd):
    import exact_attention_61_amd as mi
    note(f"rotary qk {dtype} interleaved {inter} hq {hq} hkv {hkv} d {d} rd {rd}")
    q = rand((2, hq, 129, d), dtype, seed=20 + hq)
    k = rand((2, hkv, 129, d), dtype, seed=30 + hkv)
    qg, kg = q.cuda(), k.cuda()
    mi.mi_attn_rotary_qk(qg, kg, rd, interleaved=inter, position_offset=5)
    torch.cuda.synchronize()
    f64 = workloads.to_f64
    check(qg, oracle.rotate_dense(f64(q), rd, 10000.0, inter, offset=5), dtype)
    check(kg, oracle.rotate_dense(f64(k), rd, 10000.0, inter, offset=5), dtype)
    assert torch.equal(qg[..., rd:].cpu(), q[..., rd:])
    assert torch.equal(kg[..., rd:].cpu(), k[..., rd:])


def test_rotary_qk_matches_two_calls_bitwise():
    """One launch over Q and K gives exactly the results of mi_attn_rotary on
    each: the same arithmetic per element."""
    import exact_attention_61_amd as mi
    note("rotary qk against two single calls")
    q = rand((1, 32, 1000, 128), BF16, seed=40).cuda()
    k = rand((1, 8, 1000, 128), BF16, seed=41).cuda()
    q1, k1 = q.clone(), k.clone()
    mi.mi_attn_rotary_qk(q, k, 128, position_offset=123)
    mi.mi_attn_rotary(q1, 128, position_offset=123)
    mi.mi_attn_rotary(k1, 128, position_offset=123)
    torch.cuda.synchronize()
    assert torch.equal(q, q1) and torch.equal(k, k1)


@pytest.mark.parametrize("inter", [False, True])
def test_rotary_qk_packed_bshd_view(inter):
    """Packed Q and K that are views into one [T, 3, H, d] QKV tensor: Q and K
    rotated, V and the rows past every sequence untouched."""
    import exact_attention_61_amd as mi
    lens = [7, 0, 250, 1]
    note(f"rotary qk packed qkv view {lens} interleaved {inter}")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    total = int(cu[-1])
    qkv = rand((total + 3, 3, 4, 64), F16, seed=42)
    offs = [1, 2, 3, 70000]
    g = qkv.cuda()
    mi.mi_attn_rotary_qk(g[:, 0], g[:, 1], 64, interleaved=inter,
                         position_offsets=torch.tensor(offs, dtype=torch.int32, device="cuda"),
                         cu_seqlens=cu.cuda(), max_seqlen=max(lens))
    torch.cuda.synchronize()
    f64 = workloads.to_f64
    for i in (0, 1):
        ref = oracle.rotate_packed(f64(qkv[:, i]), cu.numpy(), 64, 10000.0, inter, offsets=offs)
        check(g[:, i], ref, F16)
        assert torch.equal(g[total:, i].cpu(), qkv[total:, i])
    assert torch.equal(g[:, 2].cpu(), qkv[:, 2])
