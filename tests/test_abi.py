"""libmi_attn C ABI, checked on the host (no GPU needed).

The library must load, export every function include/mi_attn.h declares, and
reject every invalid argument with its status code before any HIP call, so
these calls never reach a device.  Pointers here are fake aligned addresses:
no call in this file passes validation with rows to compute.
"""

import ctypes
import math
import os
import re

import pytest

import exact_attention_61_amd as mi
from exact_attention_61_amd import Strides

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include",
                      "mi_attn.h")


def _header():
    with open(HEADER) as f:
        return f.read()


def test_exports_every_declared_function():
    names = re.findall(r"MI_ATTN_API\s+[\w\s\*]+?\b(mi_attn_\w+)\s*\(",
                       _header())
    assert set(names) == {"mi_attn_fwd", "mi_attn_fwd_select", "mi_attn_decode",
                          "mi_attn_decode_noalloc", "mi_attn_decode_noalloc_max_bytes",
                          "mi_attn_decode_workspace_size", "mi_attn_decode_splits",
                          "mi_attn_rotary", "mi_attn_rotary_qk", "mi_attn_fwd_dropout",
                          "mi_attn_status_string",
                          "mi_attn_version",
                          "mi_attn_last_hip_error"}
    for n in names:
        assert hasattr(mi.lib(), n), n


def test_version_matches_header():
    m = re.search(r"#define MI_ATTN_ABI_VERSION (\d+)", _header())
    assert mi.mi_attn_version() == int(m.group(1))


def test_enum_values_match_header():
    h = _header()
    for code, name in mi.STATUS_NAMES.items():
        assert re.search(rf"\b{name}\s*=\s*{code}\b", h), name
    for name, code in (("MI_ATTN_F16", 0), ("MI_ATTN_BF16", 1),
                       ("MI_ATTN_F32", 2), ("MI_ATTN_KERNEL_MFMA", 0),
                       ("MI_ATTN_KERNEL_SCALAR", 1)):
        assert re.search(rf"\b{name}\s*=\s*{code}\b", h)


def test_status_strings():
    for code, name in mi.STATUS_NAMES.items():
        assert mi.mi_attn_status_string(code).startswith(name)
    assert "unknown" in mi.mi_attn_status_string(99)
    assert mi.mi_attn_last_hip_error() == 0


A = 0x10000          # fake 16-byte-aligned addresses (never dereferenced)


def call(q=A, k=A * 2, v=A * 3, o=A * 4, lse=A * 5, in_dt=0, out_dt=0,
         b=1, hq=2, hkv=1, lq=16, lk=16, d=64, qs=None, ks=None, vs=None,
         os_=None, cuq=None, cuk=None, scale=0.125, causal=0, select=None):
    ref = lambda s: None if s is None else ctypes.byref(s)
    args = (q, k, v, o, lse, in_dt, out_dt, b, hq, hkv, lq, lk, d, ref(qs),
            ref(ks), ref(vs), ref(os_), cuq, cuk, scale, causal, None)
    if select is None:
        return mi.lib().mi_attn_fwd(*args)
    return mi.lib().mi_attn_fwd_select(*args, *select)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(in_dt=2), 4), (dict(in_dt=3), 4), (dict(in_dt=-1), 4),
    (dict(in_dt=0, out_dt=1), 4), (dict(in_dt=1, out_dt=0), 4),
    (dict(b=-1), 2), (dict(lq=-1), 2), (dict(lk=-5), 2), (dict(hq=0), 2),
    (dict(hkv=0), 2), (dict(hq=6, hkv=4), 2), (dict(hq=70000, hkv=1), 2),
    (dict(b=70000), 2), (dict(lq=65535 * 128 + 1), 2),   # grid axes y and z
    (dict(d=32), 5), (dict(d=96), 5), (dict(d=256), 5), (dict(d=0), 5),
    (dict(scale=math.nan), 6), (dict(scale=math.inf), 6),
    (dict(scale=-math.inf), 6), (dict(causal=2), 6), (dict(causal=-1), 6),
    (dict(cuq=A * 6), 6), (dict(cuk=A * 6), 6),
    (dict(q=A + 8), 3), (dict(k=A + 2), 3), (dict(o=A + 4), 3),
    (dict(lse=A + 2), 3),
    (dict(qs=Strides(2048, 1024, 63)), 3),
    (dict(ks=Strides(2048, 1020, 64)), 3),
    (dict(vs=Strides(-2048, 1024, 64)), 3),
    (dict(os_=Strides(2048, 1024, -64)), 3),
    (dict(qs=Strides(0, 64, 1 << 24)), 3),
    (dict(ks=Strides(0, 64, 1 << 24)), 3),
    (dict(vs=Strides(0, 64, 1 << 25)), 3),
    # rows may not overlap: row stride 0 (an expanded view) or below head_dim
    (dict(qs=Strides(0, 0, 0)), 3), (dict(ks=Strides(0, 0, 0)), 3),
    (dict(vs=Strides(0, 0, 0)), 3), (dict(os_=Strides(0, 0, 0)), 3),
    (dict(qs=Strides(2048, 1024, 56)), 3), (dict(ks=Strides(2048, 1024, 32)), 3),
    (dict(vs=Strides(2048, 1024, 8)), 3), (dict(os_=Strides(2048, 1024, 48)), 3),
    (dict(d=128, ks=Strides(4096, 2048, 64)), 3),
    (dict(d=128, qs=Strides(4096, 2048, 120)), 3),
    (dict(cuq=A * 6, cuk=A * 7, qs=Strides(0, 64, 0)), 3),   # packed: always
    # mi_attn_fwd_select: unknown kernel or causal order
    (dict(select=(2, -1)), 6), (dict(select=(-1, -1)), 6),
    (dict(select=(0, 4)), 6), (dict(select=(0, -2)), 6),
    (dict(select=(1, 0), in_dt=3), 4),
])
def test_rejected_before_any_hip_call(kw, code):
    assert call(**kw) == code


@pytest.mark.parametrize("kw", [dict(b=0), dict(lq=0),
                                dict(b=0, q=None, k=None, v=None, o=None),
                                dict(lq=0, q=None, o=None, lse=None)])
def test_empty_work_is_a_noop(kw):
    assert call(**kw) == 0


def test_error_precedence_dtype_before_shape():
    # a call with several faults reports the dtype one first
    assert call(in_dt=3, hq=3, hkv=2) == 4


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(mi.MiAttnError) as e:
        mi.mi_attn_fwd(q, q, q, q.clone())
    assert e.value.status == 6


# ---------------------------------------------------------------------------
# mi_attn_decode: rejected before any HIP call
# ---------------------------------------------------------------------------

def dcall(q=A, k=A * 2, v=A * 3, o=A * 4, lse=A * 5, in_dt=1, out_dt=1, b=2, hq=8,
          hkv=2, lq=1, lk=4096, d=128, qs=None, ks=None, vs=None, os_=None, seq=None,
          scale=0.1, causal=1, splits=0, ws=A * 16, ws_bytes=1 << 30):
    ref = lambda s: None if s is None else ctypes.byref(s)
    return mi.lib().mi_attn_decode(q, k, v, o, lse, in_dt, out_dt, b, hq, hkv, lq, lk, d,
                                   ref(qs), ref(ks), ref(vs), ref(os_), seq, scale, causal,
                                   splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(o=None), 1),
    (dict(in_dt=2), 4), (dict(in_dt=0, out_dt=1), 4),
    (dict(lq=33), 2), (dict(lq=-1), 2), (dict(hq=6, hkv=4), 2), (dict(b=-1), 2),
    (dict(d=96), 5), (dict(scale=math.nan), 6), (dict(causal=3), 6),
    (dict(splits=-1), 6), (dict(splits=70000), 6),
    (dict(ws=None), 1),                    # several splits need a workspace
    (dict(ws=A * 16 + 64), 3),             # not 256-byte aligned
    (dict(ws_bytes=1000), 8),              # smaller than required
    (dict(ks=Strides(0, 4096 * 128, 64)), 3),   # rows overlap
    (dict(q=A + 8), 3),
])
def test_decode_rejected_before_any_hip_call(kw, code):
    assert dcall(**kw) == code


@pytest.mark.parametrize("pdrop", [-0.1, 1.0, 1.5, math.nan, math.inf])
def test_dropout_probability_rejected_before_any_hip_call(pdrop):
    args = (A, A * 2, A * 3, A * 4, A * 5, 0, 0, 1, 2, 1, 16, 16, 64, None, None, None, None,
            None, None, 0.125, 0)
    assert mi.lib().mi_attn_fwd_dropout(*args, pdrop, 1234, None) == 6


def test_dropout_other_rejections_match_the_forward():
    for kw, code in [(dict(q=None), 1), (dict(in_dt=2), 4), (dict(d=96), 5), (dict(causal=2), 6)]:
        base = dict(q=A, k=A * 2, v=A * 3, o=A * 4, lse=A * 5, in_dt=0, out_dt=0, b=1, hq=2,
                    hkv=1, lq=16, lk=16, d=64, causal=0)
        base.update(kw)
        args = (base["q"], base["k"], base["v"], base["o"], base["lse"], base["in_dt"],
                base["out_dt"], base["b"], base["hq"], base["hkv"], base["lq"], base["lk"],
                base["d"], None, None, None, None, None, None, 0.125, base["causal"])
        assert mi.lib().mi_attn_fwd_dropout(*args, 0.1, 7, None) == code


def rcall(x=A, dt=1, b=2, h=4, l=100, d=128, xs=None, cu=None, offs=None, off=0, rd=128,
          base=10000.0, inter=0):
    ref = lambda s: None if s is None else ctypes.byref(s)
    return mi.lib().mi_attn_rotary(x, dt, b, h, l, d, ref(xs), cu, offs, off, rd, base, inter,
                                   None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(dt=2), 4), (dict(dt=-1), 4),
    (dict(b=-1), 2), (dict(h=0), 2), (dict(l=-1), 2), (dict(d=0), 2), (dict(b=70000), 2),
    (dict(h=65535 * 4 + 1), 2),
    (dict(rd=0), 5), (dict(rd=8), 5), (dict(rd=24), 5), (dict(rd=144), 5),
    (dict(d=512, rd=272), 5),
    (dict(base=0.0), 6), (dict(base=-2.0), 6), (dict(base=math.nan), 6),
    (dict(base=math.inf), 6), (dict(inter=2), 6),
    (dict(x=A + 8), 3), (dict(xs=Strides(0, 128, 60)), 3),      # row stride not 8k
    (dict(xs=Strides(0, 64, 512)), 3),                            # heads overlap
    (dict(xs=Strides(0, 128 * 100, 64)), 3),                      # rows overlap
])
def test_rotary_rejected_before_any_hip_call(kw, code):
    assert rcall(**kw) == code


def test_rotary_empty_is_noop():
    assert rcall(x=None, b=0) == 0
    assert rcall(x=None, l=0) == 0


def qkcall(q=A, k=A * 2, dt=1, b=2, hq=8, hkv=2, l=100, d=128, qs=None, ks=None, cu=None,
           offs=None, off=0, rd=128, base=10000.0, inter=0):
    ref = lambda s: None if s is None else ctypes.byref(s)
    return mi.lib().mi_attn_rotary_qk(q, k, dt, b, hq, hkv, l, d, ref(qs), ref(ks), cu, offs, off,
                                      rd, base, inter, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(dt=2), 4), (dict(dt=2, hkv=0), 4),
    (dict(hkv=0), 2), (dict(hq=0), 2), (dict(b=70000), 2), (dict(l=-1), 2),
    (dict(hq=65535 * 4, hkv=8), 2),                              # grid z of both tensors
    (dict(rd=24), 5), (dict(base=0.0), 6), (dict(inter=3), 6),
    (dict(k=A), 3),                                              # the same tensor twice
    (dict(k=A * 2 + 8), 3), (dict(ks=Strides(0, 128, 60)), 3),
    (dict(ks=Strides(0, 64, 512)), 3), (dict(qs=Strides(0, 128 * 100, 64)), 3),
])
def test_rotary_qk_rejected_before_any_hip_call(kw, code):
    assert qkcall(**kw) == code


def test_rotary_qk_empty_is_noop():
    assert qkcall(q=None, k=None, b=0) == 0
    assert qkcall(q=None, k=None, l=0) == 0


def test_decode_workspace_plan():
    size = mi.mi_attn_decode_workspace_size
    splits = mi.mi_attn_decode_splits
    # one work-group per CU for 8 x 8 query groups, 4 heads x 1 row each
    assert splits(8, 32, 8, 1, 8192, 128) == 4
    assert size(8, 32, 8, 1, 8192, 128) >= 8 * 32 * 1 * 4 * (128 + 2) * 4
    # a single split needs no workspace, and a short cache gets one split
    assert size(1, 4, 1, 1, 100, 64) == 0 and splits(1, 4, 1, 1, 100, 64) == 1
    # the caller's split count is capped so every split has keys
    assert splits(1, 8, 8, 1, 1000, 64, 64) == 8
    assert splits(1, 8, 8, 1, 1000, 64, 3) == 3
    # invalid sizes give 0
    assert size(1, 8, 3, 1, 100, 64) == 0 and splits(1, 8, 8, 40, 100, 64) == 0
    # empty work is a no-op without any pointers
    assert dcall(b=0, q=None, k=None, v=None, o=None, ws=None) == 0


def test_decode_noalloc_rejects_sizes_beyond_its_scratch():
    """Rejected before any HIP call: partials past the static scratch."""
    cap = mi.lib().mi_attn_decode_noalloc_max_bytes()
    assert cap == 8 << 20

    def ncall(b, hq, hkv, lq, lk, d, splits):
        return mi.lib().mi_attn_decode_noalloc(A, A * 2, A * 3, A * 4, A * 5, 1, 1, b, hq, hkv,
                                               lq, lk, d, None, None, None, None, None,
                                               0.1, 1, splits, None)
    # 64 x 32 heads x 32 rows x 16 splits x 128 columns x 4 B = 64 MiB of partials
    assert mi.mi_attn_decode_workspace_size(64, 32, 8, 32, 8192, 128, 16) > cap
    assert ncall(64, 32, 8, 32, 8192, 128, 16) == 8
    # 20000 sequences x 2 splits x (64 + 2) floats: just past the scratch
    assert mi.mi_attn_decode_workspace_size(20000, 1, 1, 1, 4096, 64, 2) > cap
    assert ncall(20000, 1, 1, 1, 4096, 64, 2) == 8
    # and a size that fits is accepted by validation (only a null stream
    # and fake pointers here, so no launch is attempted: batch 0)
    assert ncall(0, 1, 1, 1, 4096, 64, 2) == 0
    # validation errors come first, as for mi_attn_decode
    assert ncall(1, 8, 3, 1, 100, 64, 0) == 2
