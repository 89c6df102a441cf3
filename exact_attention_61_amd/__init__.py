"""Python binding of libmi_attn (exact attention forward for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
library.  PyTorch supplies device memory and the current stream.  If the
shared library has not been built, importing this package raises.

Entry points mirror the C ABI of include/mi_attn.h:

* mi_attn_fwd(q, k, v, o, lse, ...)  -- writes into caller-provided tensors;
* mi_attn_fwd_select(..., kernel=, causal_order=) -- the same with the kernel
  and the causal tile order chosen explicitly (tests and diagnostics);
* mi_attn_decode(q, k, v, o, lse, ...) -- a few query rows against a long
  key/value cache, keys split across work-groups (needs a workspace);
* mi_attn_decode_noalloc(q, k, v, o, lse, ...) -- the same with its scratch
  in a static device array of the library (no allocation at all);
* mi_attn_decode_workspace_size(...), mi_attn_decode_splits(...);
* mi_attn_fwd_dropout(..., dropout_p=, seed=) -- dropout on the probabilities;
* mi_attn_rotary(x, ...), mi_attn_rotary_qk(q, k, ...) -- rotary position
  embedding in place (one tensor, or Q and K in one launch);
* mi_attn_status_string(code), mi_attn_version(), mi_attn_last_hip_error();

plus forward(q, k, v, ...) -> (out, lse) and decode(q, k, v, ...) ->
(out, lse), which allocate the outputs (and decode's workspace).
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmi_attn.so")

MI_ATTN_F16, MI_ATTN_BF16, MI_ATTN_F32 = 0, 1, 2
MI_ATTN_KERNEL_MFMA, MI_ATTN_KERNEL_SCALAR = 0, 1
_DTYPE_CODE = {torch.float16: MI_ATTN_F16, torch.bfloat16: MI_ATTN_BF16,
               torch.float32: MI_ATTN_F32}

STATUS_NAMES = {0: "MI_ATTN_OK", 1: "MI_ATTN_ERR_NULL", 2: "MI_ATTN_ERR_SHAPE",
                3: "MI_ATTN_ERR_LAYOUT", 4: "MI_ATTN_ERR_DTYPE",
                5: "MI_ATTN_ERR_UNSUPPORTED", 6: "MI_ATTN_ERR_ARG",
                7: "MI_ATTN_ERR_HIP", 8: "MI_ATTN_ERR_WORKSPACE"}


class Strides(ctypes.Structure):
    """mi_attn_strides_t: element strides of a [batch, head, row, col] view."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64),
                ("row", ctypes.c_int64)]


class MiAttnError(RuntimeError):
    def __init__(self, status, detail=""):
        self.status = status
        msg = mi_attn_status_string(status)
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmi_attn.so is not built ({LIB_PATH} missing); build it with "
            "`python exact_attention_61_amd/build.py` from the repository "
            "root (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    S = ctypes.POINTER(Strides)
    i32 = ctypes.c_int32
    lib.mi_attn_fwd.restype = ctypes.c_int
    lib.mi_attn_fwd.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                i32, i32, i32, i32, i32, i32, S, S, S, S, P, P,
                                ctypes.c_float, i32, P]
    lib.mi_attn_fwd_dropout.restype = ctypes.c_int
    lib.mi_attn_fwd_dropout.argtypes = lib.mi_attn_fwd.argtypes[:-1] + [
        ctypes.c_double, ctypes.c_uint64, P]
    lib.mi_attn_fwd_select.restype = ctypes.c_int
    lib.mi_attn_fwd_select.argtypes = lib.mi_attn_fwd.argtypes + [ctypes.c_int, i32]
    lib.mi_attn_decode.restype = ctypes.c_int
    lib.mi_attn_decode.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                   i32, i32, i32, i32, i32, i32, S, S, S, S, P,
                                   ctypes.c_float, i32, i32, P, ctypes.c_size_t, P]
    lib.mi_attn_decode_noalloc.restype = ctypes.c_int
    lib.mi_attn_decode_noalloc.argtypes = lib.mi_attn_decode.argtypes[:20] + [P]
    lib.mi_attn_decode_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.mi_attn_decode_noalloc_max_bytes.argtypes = []
    lib.mi_attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.mi_attn_decode_workspace_size.argtypes = [i32] * 7
    lib.mi_attn_decode_splits.restype = i32
    lib.mi_attn_decode_splits.argtypes = [i32] * 7
    lib.mi_attn_rotary.restype = ctypes.c_int
    lib.mi_attn_rotary.argtypes = [P, ctypes.c_int, i32, i32, i32, i32, S, P, P,
                                   ctypes.c_int64, i32, ctypes.c_double, i32, P]
    lib.mi_attn_rotary_qk.restype = ctypes.c_int
    lib.mi_attn_rotary_qk.argtypes = [P, P, ctypes.c_int, i32, i32, i32, i32, i32, S, S, P, P,
                                      ctypes.c_int64, i32, ctypes.c_double, i32, P]
    lib.mi_attn_status_string.restype = ctypes.c_char_p
    lib.mi_attn_status_string.argtypes = [ctypes.c_int]
    lib.mi_attn_version.restype = i32
    lib.mi_attn_version.argtypes = []
    lib.mi_attn_last_hip_error.restype = i32
    lib.mi_attn_last_hip_error.argtypes = []
    return lib


_lib = _load()


def lib():
    """The loaded ctypes library (raw C entry points)."""
    return _lib


def mi_attn_status_string(status):
    return _lib.mi_attn_status_string(int(status)).decode()


def mi_attn_version():
    return int(_lib.mi_attn_version())


def mi_attn_last_hip_error():
    return int(_lib.mi_attn_last_hip_error())


def _strides(t, layout, packed):
    """Element strides (batch, head, row) of q/k/v/o as the ABI wants them."""
    if t.stride(-1) != 1:
        raise MiAttnError(3, "last dimension must be contiguous")
    st = t.stride()
    if packed:                      # [T, H, d]
        return Strides(0, st[1], st[0])
    if layout == "bhsd":            # [B, H, L, d]
        return Strides(st[0], st[1], st[2])
    if layout == "bshd":            # [B, L, H, d]
        return Strides(st[0], st[2], st[1])
    raise ValueError(f"unknown layout {layout!r}")


def _dims(q, k, layout, packed):
    if packed:
        return 0, q.shape[1], k.shape[1], q.shape[0], k.shape[0]
    if layout == "bhsd":
        return q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2]
    return q.shape[0], q.shape[2], k.shape[2], q.shape[1], k.shape[1]


def _ptr(t):
    if t is None or t.numel() == 0:
        return None
    return ctypes.c_void_p(t.data_ptr())


def mi_attn_fwd(q, k, v, o, lse=None, *, causal=False, scale=None,
                cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                max_seqlen_k=None, layout="bhsd", stream=None):
    """Call the C entry point on caller-provided tensors (all on one device).

    Dense q is [B, Hq, Lq, d] ("bhsd") or [B, Lq, Hq, d] ("bshd"); packed q is
    [Tq, Hq, d] with int32 cu_seqlens_q / cu_seqlens_k of length B + 1 and
    max_seqlen_q / max_seqlen_k.  lse (float32) is [B, Hq, Lq] dense or
    [Hq, Tq] packed, or None.  scale=None means 1/sqrt(head_dim).
    """
    _call(q, k, v, o, lse, causal, scale, cu_seqlens_q, cu_seqlens_k,
          max_seqlen_q, max_seqlen_k, layout, stream, None)


def mi_attn_fwd_select(q, k, v, o, lse=None, *, kernel=MI_ATTN_KERNEL_MFMA,
                       causal_order=-1, causal=False, scale=None,
                       cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                       max_seqlen_k=None, layout="bhsd", stream=None):
    """mi_attn_fwd with the kernel (MI_ATTN_KERNEL_MFMA / _SCALAR) and the
    causal q-tile order (-1 default, 0, 1, 2) chosen explicitly."""
    _call(q, k, v, o, lse, causal, scale, cu_seqlens_q, cu_seqlens_k,
          max_seqlen_q, max_seqlen_k, layout, stream,
          (int(kernel), int(causal_order)))


def mi_attn_fwd_dropout(q, k, v, o, lse=None, *, dropout_p, seed, causal=False,
                        scale=None, cu_seqlens_q=None, cu_seqlens_k=None,
                        max_seqlen_q=None, max_seqlen_k=None, layout="bhsd",
                        stream=None):
    """mi_attn_fwd with dropout on the probabilities: each kept with
    probability 1 - dropout_p (then scaled by 1 / (1 - dropout_p)), the mask
    drawn from Philox4x32-10 keyed by the 64-bit seed."""
    _call(q, k, v, o, lse, causal, scale, cu_seqlens_q, cu_seqlens_k,
          max_seqlen_q, max_seqlen_k, layout, stream, None,
          dropout=(float(dropout_p), int(seed) & 0xFFFFFFFFFFFFFFFF))


def _call(q, k, v, o, lse, causal, scale, cu_seqlens_q, cu_seqlens_k,
          max_seqlen_q, max_seqlen_k, layout, stream, select, dropout=None):
    packed = cu_seqlens_q is not None or cu_seqlens_k is not None
    for t in (q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k):
        if t is not None and (not t.is_cuda or t.device != q.device):
            raise MiAttnError(6, "every tensor must be on q's GPU device")
    if q.dtype not in _DTYPE_CODE or o.dtype not in _DTYPE_CODE:
        raise MiAttnError(4, f"{q.dtype} -> {o.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise MiAttnError(4, "q, k and v must share one dtype")
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    bsz, hq, hkv, lq, lk = _dims(q, k, layout, packed)
    if packed:
        if cu_seqlens_q is None or cu_seqlens_k is None:
            raise MiAttnError(6, "give both cu_seqlens_q and cu_seqlens_k")
        bsz = cu_seqlens_q.numel() - 1
        lq = int(max_seqlen_q)
        lk = int(max_seqlen_k)
        for cu in (cu_seqlens_q, cu_seqlens_k):
            if cu.dtype != torch.int32 or not cu.is_contiguous():
                raise MiAttnError(3, "cu_seqlens must be contiguous int32")
        if os.environ.get("MI_ATTN_DEBUG") == "1":
            _check_cu(cu_seqlens_q, lq, q.shape[0])
            _check_cu(cu_seqlens_k, lk, k.shape[0])
    if lse is not None and (lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise MiAttnError(3, "lse must be contiguous float32")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    qs, ks, vs, os_ = (_strides(t, layout, packed) for t in (q, k, v, o))
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
            _DTYPE_CODE[q.dtype], _DTYPE_CODE[o.dtype],
            bsz, hq, hkv, lq, lk, d,
            ctypes.byref(qs), ctypes.byref(ks), ctypes.byref(vs),
            ctypes.byref(os_), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
            float(scale), int(bool(causal)), ctypes.c_void_p(stream))
    if dropout is not None:
        st = _lib.mi_attn_fwd_dropout(*args[:-1], dropout[0], dropout[1], args[-1])
    elif select is None:
        st = _lib.mi_attn_fwd(*args)
    else:
        st = _lib.mi_attn_fwd_select(*args, *select)
    if st != 0:
        detail = ""
        if st == 7:
            detail = f"hipError {mi_attn_last_hip_error()}"
        raise MiAttnError(st, detail)


def mi_attn_decode_workspace_size(batch, hq, hkv, lq, lk, head_dim, num_splits=0):
    """Bytes of workspace mi_attn_decode needs (0: a single split)."""
    return int(_lib.mi_attn_decode_workspace_size(batch, hq, hkv, lq, lk, head_dim,
                                                  num_splits))


def mi_attn_decode_splits(batch, hq, hkv, lq, lk, head_dim, num_splits=0):
    """The key splits mi_attn_decode uses for these sizes."""
    return int(_lib.mi_attn_decode_splits(batch, hq, hkv, lq, lk, head_dim, num_splits))


def mi_attn_decode_noalloc(q, k, v, o, lse=None, *, seqlens_k=None, causal=True,
                           scale=None, num_splits=0, stream=None):
    """mi_attn_decode with the library's static scratch instead of a
    workspace: nothing is allocated.  Calls that overlap in time on one GPU
    race (they share the scratch)."""
    _decode_call(q, k, v, o, lse, seqlens_k, causal, scale, num_splits, None, stream,
                 noalloc=True)


def mi_attn_decode(q, k, v, o, lse=None, *, seqlens_k=None, causal=True, scale=None,
                   num_splits=0, workspace=None, stream=None):
    """Call mi_attn_decode on caller-provided tensors (one device).

    q, o: [B, Hq, Lq, d] (Lq <= 32); k, v: the cache [B, Hkv, Lk, d]; lse
    [B, Hq, Lq] float32 or None; seqlens_k: int32 [B] keys per sequence or
    None (all Lk).  workspace: a uint8 tensor of at least
    mi_attn_decode_workspace_size(...) bytes (any contents), or None when
    that size is 0.
    """
    _decode_call(q, k, v, o, lse, seqlens_k, causal, scale, num_splits, workspace, stream,
                 noalloc=False)


def _decode_call(q, k, v, o, lse, seqlens_k, causal, scale, num_splits, workspace, stream,
                 noalloc):
    for t in (q, k, v, o, lse, seqlens_k, workspace):
        if t is not None and (not t.is_cuda or t.device != q.device):
            raise MiAttnError(6, "every tensor must be on q's GPU device")
    if q.dtype not in _DTYPE_CODE or o.dtype not in _DTYPE_CODE:
        raise MiAttnError(4, f"{q.dtype} -> {o.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise MiAttnError(4, "q, k and v must share one dtype")
    if seqlens_k is not None and (seqlens_k.dtype != torch.int32
                                  or not seqlens_k.is_contiguous()):
        raise MiAttnError(3, "seqlens_k must be contiguous int32")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise MiAttnError(3, "lse must be contiguous float32")
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    bsz, hq, hkv, lq, lk = _dims(q, k, "bhsd", False)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    qs, ks, vs, os_ = (_strides(t, "bhsd", False) for t in (q, k, v, o))
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
            _DTYPE_CODE[q.dtype], _DTYPE_CODE[o.dtype], bsz, hq, hkv, lq, lk, d,
            ctypes.byref(qs), ctypes.byref(ks), ctypes.byref(vs), ctypes.byref(os_),
            _ptr(seqlens_k), float(scale), int(bool(causal)), int(num_splits))
    if noalloc:
        st = _lib.mi_attn_decode_noalloc(*args, ctypes.c_void_p(stream))
    else:
        ws_ptr, ws_bytes = (None, 0) if workspace is None else (
            ctypes.c_void_p(workspace.data_ptr()),
            workspace.numel() * workspace.element_size())
        st = _lib.mi_attn_decode(*args, ws_ptr, ws_bytes, ctypes.c_void_p(stream))
    if st != 0:
        detail = f"hipError {mi_attn_last_hip_error()}" if st == 7 else ""
        raise MiAttnError(st, detail)


def decode(q, k, v, *, seqlens_k=None, causal=True, scale=None, num_splits=0,
           out_dtype=None, workspace=None, return_lse=True):
    """Allocate out (and lse, and a workspace unless given) and run
    mi_attn_decode; returns (out, lse)."""
    out_dtype = q.dtype if out_dtype is None else out_dtype
    out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    bsz, hq, hkv, lq, lk = _dims(q, k, "bhsd", False)
    lse = (torch.empty((bsz, hq, lq), dtype=torch.float32, device=q.device)
           if return_lse else None)
    if workspace is None:
        n = mi_attn_decode_workspace_size(bsz, hq, hkv, lq, lk, q.shape[-1], num_splits)
        if n > 0:
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        mi_attn_decode(q, k, v, out, lse, seqlens_k=seqlens_k, causal=causal, scale=scale,
                       num_splits=num_splits, workspace=workspace)
    return out, lse


def mi_attn_rotary(x, rotary_dim=None, *, base=10000.0, interleaved=False,
                   position_offset=0, position_offsets=None, cu_seqlens=None,
                   max_seqlen=None, layout="bhsd", stream=None):
    """Rotary embedding of x in place (Q or K; one call per tensor).

    Dense x is [B, H, L, d] ("bhsd") or [B, L, H, d] ("bshd"); packed x is
    [T, H, d] with int32 cu_seqlens of length B + 1 and max_seqlen.  Row t of
    sequence b sits at position position_offset + position_offsets[b] + t
    (position_offsets: int32 [B] on the device, or None).  rotary_dim
    defaults to d.  interleaved=False is the GPT-NeoX layout, True GPT-J.
    """
    packed = cu_seqlens is not None
    for t in (position_offsets, cu_seqlens):
        if t is not None and (not t.is_cuda or t.device != x.device):
            raise MiAttnError(6, "every tensor must be on x's GPU device")
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise MiAttnError(3, "position_offsets / cu_seqlens must be contiguous int32")
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise MiAttnError(4, f"{x.dtype}")
    d = x.shape[-1]
    rd = d if rotary_dim is None else int(rotary_dim)
    if packed:
        bsz, heads, seqlen = cu_seqlens.numel() - 1, x.shape[1], int(max_seqlen)
    elif layout == "bhsd":
        bsz, heads, seqlen = x.shape[0], x.shape[1], x.shape[2]
    else:
        bsz, heads, seqlen = x.shape[0], x.shape[2], x.shape[1]
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    xs = _strides(x, layout, packed)
    st = _lib.mi_attn_rotary(_ptr(x), _DTYPE_CODE[x.dtype], bsz, heads, seqlen, d,
                             ctypes.byref(xs), _ptr(cu_seqlens), _ptr(position_offsets),
                             int(position_offset), rd, float(base), int(bool(interleaved)),
                             ctypes.c_void_p(stream))
    if st != 0:
        detail = f"hipError {mi_attn_last_hip_error()}" if st == 7 else ""
        raise MiAttnError(st, detail)
    return x


def mi_attn_rotary_qk(q, k, rotary_dim=None, *, base=10000.0, interleaved=False,
                      position_offset=0, position_offsets=None, cu_seqlens=None,
                      max_seqlen=None, layout="bhsd", stream=None):
    """Rotary embedding of q and k in place, one launch (the result of
    mi_attn_rotary on each).  q and k share the layout, the rows and the
    positions; their head counts may differ."""
    packed = cu_seqlens is not None
    for t in (k, position_offsets, cu_seqlens):
        if t is not None and (not t.is_cuda or t.device != q.device):
            raise MiAttnError(6, "every tensor must be on q's GPU device")
    for t in (position_offsets, cu_seqlens):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise MiAttnError(3, "position_offsets / cu_seqlens must be contiguous int32")
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype:
        raise MiAttnError(4, f"{q.dtype} / {k.dtype}")
    d = q.shape[-1]
    if k.shape[-1] != d:
        raise MiAttnError(2, "q and k head dims differ")
    rd = d if rotary_dim is None else int(rotary_dim)
    if packed:
        bsz, hq, hkv, seqlen = cu_seqlens.numel() - 1, q.shape[1], k.shape[1], int(max_seqlen)
    elif layout == "bhsd":
        bsz, hq, hkv, seqlen = q.shape[0], q.shape[1], k.shape[1], q.shape[2]
    else:
        bsz, hq, hkv, seqlen = q.shape[0], q.shape[2], k.shape[2], q.shape[1]
    if not packed and (k.shape[0] != bsz or k.shape[2 if layout == "bhsd" else 1] != seqlen):
        raise MiAttnError(2, "q and k rows differ")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    qs = _strides(q, layout, packed)
    ks = _strides(k, layout, packed)
    st = _lib.mi_attn_rotary_qk(_ptr(q), _ptr(k), _DTYPE_CODE[q.dtype], bsz, hq, hkv, seqlen, d,
                                ctypes.byref(qs), ctypes.byref(ks), _ptr(cu_seqlens),
                                _ptr(position_offsets), int(position_offset), rd, float(base),
                                int(bool(interleaved)), ctypes.c_void_p(stream))
    if st != 0:
        detail = f"hipError {mi_attn_last_hip_error()}" if st == 7 else ""
        raise MiAttnError(st, detail)
    return q, k


def _check_cu(cu, max_len, rows):
    """Host-side check of a cu_seqlens array (only with MI_ATTN_DEBUG=1)."""
    c = cu.to("cpu").tolist()
    if c[0] != 0:
        raise MiAttnError(6, "cu_seqlens[0] must be 0")
    for a, b in zip(c, c[1:]):
        if b < a or b - a > max_len:
            raise MiAttnError(6, "cu_seqlens must be non-decreasing with "
                                 "lengths <= max_seqlen")
    if c[-1] > rows:
        raise MiAttnError(6, "cu_seqlens points past the tensor")


def forward(q, k, v, *, causal=False, scale=None, cu_seqlens_q=None,
            cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
            out_dtype=None, layout="bhsd", return_lse=True, kernel=None,
            causal_order=None, dropout_p=0.0, seed=0):
    """Allocate out (and lse) and run mi_attn_fwd; returns (out, lse).

    kernel / causal_order (optional) go through mi_attn_fwd_select instead;
    dropout_p > 0 goes through mi_attn_fwd_dropout with the given seed.
    """
    packed = cu_seqlens_q is not None or cu_seqlens_k is not None
    out_dtype = q.dtype if out_dtype is None else out_dtype
    out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    lse = None
    if return_lse:
        if packed:
            lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32,
                              device=q.device)
        else:
            bsz, hq, _, lq, _ = _dims(q, k, layout, packed)
            lse = torch.empty((bsz, hq, lq), dtype=torch.float32,
                              device=q.device)
    kw = dict(causal=causal, scale=scale, cu_seqlens_q=cu_seqlens_q,
              cu_seqlens_k=cu_seqlens_k, max_seqlen_q=max_seqlen_q,
              max_seqlen_k=max_seqlen_k, layout=layout)
    with torch.cuda.device(q.device):
        if dropout_p:
            if kernel is not None or causal_order is not None:
                raise MiAttnError(6, "dropout runs the default kernel and order")
            mi_attn_fwd_dropout(q, k, v, out, lse, dropout_p=dropout_p, seed=seed, **kw)
        elif kernel is None and causal_order is None:
            mi_attn_fwd(q, k, v, out, lse, **kw)
        else:
            mi_attn_fwd_select(
                q, k, v, out, lse,
                kernel=MI_ATTN_KERNEL_MFMA if kernel is None else kernel,
                causal_order=-1 if causal_order is None else causal_order,
                **kw)
    return out, lse
