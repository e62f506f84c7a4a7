"""Python binding of the C ABI in include/fa.h (ctypes; argument marshalling only).

The functions ``fa_fwd``, ``fa_fwd_workspace_bytes``, ``fa_set_workspace``,
``fa_status_string`` and ``fa_abi_version`` mirror the C entry points one to
one and take plain integers for device pointers and streams.  ``attention``
is the tensor-level convenience on top: it checks the torch tensors, takes
the current HIP stream, registers that stream's split-KV workspace when the
shape needs one (reserved once per stream, never released, never grown
during graph capture), allocates ``out``/``lse`` only when they are not
passed (the allocation-free form is the one with both passed), and raises
on any error code.  Every arithmetic step runs in the HIP kernels; there is no other
implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_mi355x.so")

FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_UNSUPPORTED = 3
FA_ERR_ALIGN = 4
FA_ERR_SCALE = 5
FA_ERR_WORKSPACE = 6
FA_ERR_LAUNCH = 7
FA_ERR_ALIAS = 8
FA_ERR_SCRATCH = 9
FA_STATIC_SCRATCH_BYTES = 8 << 20

FA_BF16 = 0
FA_FP16 = 1

EXPORTS = ("fa_fwd", "fa_fwd_static", "fa_fwd_strided", "fa_fwd_varlen", "fa_fwd_nvfp4", "fa_fwd_workspace_bytes", "fa_set_workspace",
           "fa_fwd_variant",
           "fa_fwd_variant_workspace_bytes", "fa_fwd_plan", "fa_status_string", "fa_abi_version")

_lib = None
_lib_lock = threading.Lock()


class FAError(RuntimeError):
    """An FA_ERR_* status returned by the library."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {fa_status_string(code)} (code {code})")


def load_library():
    """Load the built HIP library (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m attention_forward_amd.build` "
                "(there is no other implementation of the attention path)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.fa_fwd.restype = i32
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, f32, vp]
        lib.fa_fwd_static.restype = i32
        lib.fa_fwd_static.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, f32, vp]
        i64 = ctypes.c_int64
        lib.fa_fwd_strided.restype = i32
        lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp] + [i32] * 6 + [i64] * 12 + [i32, i32, vp, f32, vp]
        lib.fa_fwd_varlen.restype = i32
        lib.fa_fwd_varlen.argtypes = [vp] * 7 + [i32] * 10 + [f32, vp]
        lib.fa_fwd_nvfp4.restype = i32
        lib.fa_fwd_nvfp4.argtypes = [vp] * 6 + [i32] * 7 + [vp, f32, vp]
        lib.fa_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_workspace_bytes.argtypes = [i32] * 7
        lib.fa_set_workspace.restype = i32
        lib.fa_set_workspace.argtypes = [vp, ctypes.c_size_t]
        lib.fa_fwd_variant.restype = i32
        lib.fa_fwd_variant.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, f32,
                                       i32, i32, i32, i32, i32, i32, vp]
        lib.fa_fwd_variant_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_variant_workspace_bytes.argtypes = [i32] * 13
        lib.fa_fwd_plan.restype = i32
        lib.fa_fwd_plan.argtypes = [i32] * 7 + [ctypes.POINTER(i32)] * 6
        lib.fa_status_string.restype = ctypes.c_char_p
        lib.fa_status_string.argtypes = [i32]
        lib.fa_abi_version.restype = i32
        lib.fa_abi_version.argtypes = []
        _lib = lib
        return lib


# ------------------------------------------------------------ raw C entry points

def fa_fwd(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, causal, seqused_k, scale, stream) -> int:
    """C ``fa_fwd``; pointers and stream are integers (0 for NULL)."""
    return load_library().fa_fwd(q or None, k or None, v or None, out or None, lse or None,
                                 B, Sq, Sk, Hq, Hkv, D, int(causal), seqused_k or None,
                                 ctypes.c_float(scale), stream or None)


def fa_fwd_static(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, causal, seqused_k, scale, stream) -> int:
    """C ``fa_fwd_static`` (split-KV partials in the library's device scratch;
    no workspace registration); pointers and stream are integers (0 for NULL)."""
    return load_library().fa_fwd_static(q or None, k or None, v or None, out or None, lse or None,
                                        B, Sq, Sk, Hq, Hkv, D, int(causal), seqused_k or None,
                                        ctypes.c_float(scale), stream or None)


def fa_fwd_strided(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, q_strides, k_strides, v_strides, o_strides,
                   dtype, causal, seqused_k, scale, stream) -> int:
    """C ``fa_fwd_strided``; each ``*_strides`` is (batch, seq, head) in elements."""
    st = [int(x) for x in (*q_strides, *k_strides, *v_strides, *o_strides)]
    if len(st) != 12:
        raise ValueError("each stride triple needs three entries")
    return load_library().fa_fwd_strided(q or None, k or None, v or None, out or None, lse or None,
                                         B, Sq, Sk, Hq, Hkv, D, *st, int(dtype), int(causal),
                                         seqused_k or None, ctypes.c_float(scale), stream or None)


def fa_fwd_varlen(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, max_seqlen_k, total_q, total_k,
                  Hq, Hkv, D, dtype, causal, scale, stream) -> int:
    """C ``fa_fwd_varlen``; pointers and stream are integers (0 for NULL)."""
    return load_library().fa_fwd_varlen(q or None, k or None, v or None, out or None, lse or None,
                                        cu_seqlens_q or None, cu_seqlens_k or None, B, max_seqlen_q, max_seqlen_k,
                                        total_q, total_k, Hq, Hkv, D, int(dtype), int(causal),
                                        ctypes.c_float(scale), stream or None)


def fa_fwd_nvfp4(q, k, v, out_fp4, out_sf, lse, B, Sq, Sk, Hq, Hkv, D, causal, seqused_k, scale, stream) -> int:
    """C ``fa_fwd_nvfp4``; pointers and stream are integers (0 for NULL)."""
    return load_library().fa_fwd_nvfp4(q or None, k or None, v or None, out_fp4 or None, out_sf or None, lse or None,
                                       B, Sq, Sk, Hq, Hkv, D, int(causal), seqused_k or None,
                                       ctypes.c_float(scale), stream or None)


def fa_fwd_workspace_bytes(B, Sq, Sk, Hq, Hkv, D, causal) -> int:
    return int(load_library().fa_fwd_workspace_bytes(B, Sq, Sk, Hq, Hkv, D, int(causal)))


def fa_fwd_variant(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, causal, seqused_k, scale,
                   qt, nw, kw, bn, nst, kps, stream) -> int:
    """C ``fa_fwd_variant``: fa_fwd with an explicit kernel variant."""
    return load_library().fa_fwd_variant(q or None, k or None, v or None, out or None, lse or None,
                                         B, Sq, Sk, Hq, Hkv, D, int(causal), seqused_k or None,
                                         ctypes.c_float(scale), qt, nw, kw, bn, nst, kps, stream or None)


def fa_fwd_variant_workspace_bytes(B, Sq, Sk, Hq, Hkv, D, causal, qt, nw, kw, bn, nst, kps) -> int:
    return int(load_library().fa_fwd_variant_workspace_bytes(B, Sq, Sk, Hq, Hkv, D, int(causal),
                                                             qt, nw, kw, bn, nst, kps))


def fa_fwd_plan(B, Sq, Sk, Hq, Hkv, D, causal):
    """(qt, nw, kw, bn, nst, kps) that fa_fwd uses for this shape."""
    out = [ctypes.c_int() for _ in range(6)]
    rc = load_library().fa_fwd_plan(B, Sq, Sk, Hq, Hkv, D, int(causal), *[ctypes.byref(x) for x in out])
    if rc != FA_OK:
        raise FAError(rc, "fa_fwd_plan")
    return tuple(x.value for x in out)


def fa_set_workspace(dev_ptr, nbytes) -> int:
    return load_library().fa_set_workspace(dev_ptr or None, nbytes)


def fa_status_string(code: int) -> str:
    return load_library().fa_status_string(code).decode()


def fa_abi_version() -> int:
    return load_library().fa_abi_version()


# ------------------------------------------------------------- tensor interface

# Split-KV workspaces: one torch buffer per (device index, stream handle),
# so calls queued on different streams never share partial results.  A
# buffer that has ever been registered is never released: a HIP graph
# captured earlier keeps its address in the kernel arguments and writes
# there on every replay, so a superseded buffer moves to _retired and lives
# as long as the process.  Registration and the call that uses it happen
# under one lock, because the library keeps one registered workspace per
# device and reads it when the call is queued.
_ws_lock = threading.RLock()
_workspaces = {}  # (device index, stream handle) -> torch uint8 buffer
_retired = []     # superseded buffers, kept alive on purpose


class WorkspaceCaptureError(RuntimeError):
    """A split-KV call under graph capture needs more workspace than its
    stream holds (allocating then would give the graph memory that a later,
    larger call could replace)."""


def _stream_workspace(idx: int, stream_handle: int, nbytes: int):
    """The buffer of (device, stream), grown to at least ``nbytes``
    outside graph capture.  Call with _ws_lock held."""
    import torch

    key = (idx, int(stream_handle or 0))
    buf = _workspaces.get(key)
    if buf is not None and buf.numel() >= nbytes:
        return buf
    if torch.cuda.is_current_stream_capturing():
        have = 0 if buf is None else buf.numel()
        raise WorkspaceCaptureError(
            f"split-KV workspace of {nbytes} bytes needed while capturing a graph, but this stream holds "
            f"{have}: run the same shape once on the capture stream before capturing, or call "
            "reserve_workspace(device, nbytes, stream) first")
    new = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=torch.device("cuda", idx))
    if buf is not None:
        _retired.append(buf)
    _workspaces[key] = new
    return new


def _register(idx: int, buf) -> None:
    import torch

    with torch.cuda.device(idx):
        rc = fa_set_workspace(buf.data_ptr(), buf.numel())
    if rc != FA_OK:
        raise FAError(rc, "fa_set_workspace")


def reserve_workspace(device, nbytes: int, stream=None):
    """Reserve (never release) a split-KV workspace of at least ``nbytes``
    for ``stream`` (a torch.cuda.Stream or raw handle; default: the current
    stream of ``device``) and register it with the library, for callers of
    the raw C entry points.  Returns the buffer, or None when ``nbytes`` is 0."""
    import torch

    if nbytes <= 0:
        return None
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if stream is None:
        handle = torch.cuda.current_stream(idx).cuda_stream
    else:
        handle = getattr(stream, "cuda_stream", stream)
    with _ws_lock:
        buf = _stream_workspace(idx, handle, nbytes)
        _register(idx, buf)
    return buf


def _call_with_workspace(dev, stream_handle, nbytes, fn):
    """fn() with the workspace of (device, stream) registered, atomically
    with respect to other calls of this module."""
    import torch

    if nbytes <= 0:
        return fn()
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    with _ws_lock:
        _register(idx, _stream_workspace(idx, stream_handle, nbytes))
        return fn()


def attention(q, k, v, *, causal=False, seqused_k=None, scale=None, out=None, lse=None,
              return_lse=True, variant=None):
    """out, lse = softmax(scale * q k^T + mask) v for bf16 or fp16 cuda tensors.

    q [B, Sq, Hq, D]; k, v [B, Sk, Hkv, D], all of one dtype (bfloat16 or
    float16), each a (batch, seq, heads, head_dim) view whose head_dim is
    contiguous (e.g. slices of one fused QKV tensor); seqused_k int32 [B] on
    the same device or None.  ``scale`` defaults to 1/sqrt(D).  Returns
    (out, lse) with out like q (allocated contiguous when not passed; a
    passed ``out`` may be a strided view) and lse [B, Hq, Sq] float32 (None
    when ``return_lse`` is False and no ``lse`` tensor is passed).
    Contiguous bf16 tensors go through fa_fwd, everything else through
    fa_fwd_strided.  ``variant`` = (qt, nw, kw, bn, nst, kps) runs that kernel
    variant through fa_fwd_variant (contiguous bf16 only).
    """
    import torch

    dtypes = {torch.bfloat16: FA_BF16, torch.float16: FA_FP16}
    if not isinstance(q, torch.Tensor) or q.dtype not in dtypes:
        raise TypeError("q must be a bfloat16 or float16 cuda tensor")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != q.dtype or not t.is_cuda:
            raise TypeError(f"{name} must be a cuda tensor of q's dtype ({q.dtype})")
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{name} must be a 4-D (batch, seq, heads, head_dim) view with contiguous head_dim")
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Sk, Hkv, D] matching q")
    dev = q.device
    if k.device != dev or v.device != dev:
        raise ValueError("q, k, v must be on one device")
    if seqused_k is not None:
        if seqused_k.dtype != torch.int32 or seqused_k.device != dev or seqused_k.numel() != B \
                or not seqused_k.is_contiguous():
            raise ValueError("seqused_k must be a contiguous int32 tensor of B entries on q's device")
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=q.dtype, device=dev)
    elif tuple(out.shape) != (B, Sq, Hq, D) or out.dtype != q.dtype or out.device != dev or out.stride(3) != 1:
        raise ValueError("out must be a tensor shaped and typed like q with contiguous head_dim")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    elif lse is not None and (tuple(lse.shape) != (B, Hq, Sq) or lse.dtype != torch.float32
                              or lse.device != dev or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Sq] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    causal = bool(causal)
    dense = q.dtype == torch.bfloat16 and all(t.is_contiguous() for t in (q, k, v, out))
    if variant is not None and not dense:
        raise ValueError("variant is only available for contiguous bfloat16 tensors")
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), 0 if lse is None else lse.data_ptr())
    sq = 0 if seqused_k is None else seqused_k.data_ptr()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        if variant is not None:
            rc = _call_with_workspace(
                dev, stream, fa_fwd_variant_workspace_bytes(B, Sq, Sk, Hq, Hkv, D, causal, *variant),
                lambda: fa_fwd_variant(*ptrs, B, Sq, Sk, Hq, Hkv, D, causal, sq, float(scale), *variant, stream))
            where = "fa_fwd_variant"
        elif dense:
            rc = _call_with_workspace(
                dev, stream, fa_fwd_workspace_bytes(B, Sq, Sk, Hq, Hkv, D, causal),
                lambda: fa_fwd(*ptrs, B, Sq, Sk, Hq, Hkv, D, causal, sq, float(scale), stream))
            where = "fa_fwd"
        else:
            rc = _call_with_workspace(
                dev, stream, fa_fwd_workspace_bytes(B, Sq, Sk, Hq, Hkv, D, causal),
                lambda: fa_fwd_strided(*ptrs, B, Sq, Sk, Hq, Hkv, D, q.stride()[:3], k.stride()[:3],
                                       v.stride()[:3], out.stride()[:3], dtypes[q.dtype], causal, sq,
                                       float(scale), stream))
            where = "fa_fwd_strided"
    if rc != FA_OK:
        raise FAError(rc, where)
    return out, lse


def attention_nvfp4(q, k, v, *, causal=False, seqused_k=None, scale=None, out_fp4=None, out_sf=None, lse=None,
                    return_lse=True):
    """Attention with the output quantised to NVFP4 in the same launch
    (fa_fwd_nvfp4): contiguous bfloat16 q [B, Sq, Hq, D], k, v [B, Sk, Hkv, D]
    with D 64 or 256.  Returns (codes uint8 [B, Sq, Hq, D/2], scales uint8
    [B, Sq, Hq, D/16], lse [B, Hq, Sq] float32 or None)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bfloat16 cuda tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D (batch, seq, heads, head_dim)")
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Sk, Hkv, D] matching q")
    dev = q.device
    if k.device != dev or v.device != dev:
        raise ValueError("q, k, v must be on one device")
    if D % 16 != 0:
        raise ValueError("NVFP4 output needs a head dim that is a multiple of 16")
    if seqused_k is not None and (seqused_k.dtype != torch.int32 or seqused_k.device != dev
                                  or seqused_k.numel() != B or not seqused_k.is_contiguous()):
        raise ValueError("seqused_k must be a contiguous int32 tensor of B entries on q's device")
    shapes = {"out_fp4": (B, Sq, Hq, D // 2), "out_sf": (B, Sq, Hq, D // 16)}
    bufs = {"out_fp4": out_fp4, "out_sf": out_sf}
    for name, t in bufs.items():
        if t is None:
            bufs[name] = torch.empty(shapes[name], dtype=torch.uint8, device=dev)
        elif tuple(t.shape) != shapes[name] or t.dtype != torch.uint8 or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 tensor of shape {shapes[name]}")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    elif lse is not None and (tuple(lse.shape) != (B, Hq, Sq) or lse.dtype != torch.float32
                              or lse.device != dev or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Sq] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    causal = bool(causal)
    sq = 0 if seqused_k is None else seqused_k.data_ptr()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = _call_with_workspace(
            dev, stream, fa_fwd_workspace_bytes(B, Sq, Sk, Hq, Hkv, D, causal),
            lambda: fa_fwd_nvfp4(q.data_ptr(), k.data_ptr(), v.data_ptr(), bufs["out_fp4"].data_ptr(),
                                 bufs["out_sf"].data_ptr(), 0 if lse is None else lse.data_ptr(), B, Sq, Sk, Hq,
                                 Hkv, D, causal, sq, float(scale), stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_fwd_nvfp4")
    return bufs["out_fp4"], bufs["out_sf"], lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, causal=False,
                     scale=None, out=None, lse=None, return_lse=True):
    """Attention over packed variable-length sequences (fa_fwd_varlen).

    q [total_q, Hq, D], k and v [total_k, Hkv, D], contiguous, one dtype
    (bfloat16 or float16); cu_seqlens_q / cu_seqlens_k contiguous int32
    [B + 1] on q's device; max_seqlen_q / max_seqlen_k host ints bounding the
    sequence lengths.  Returns (out [total_q, Hq, D], lse [Hq, total_q]
    float32 or None).  A passed ``out`` keeps the values of rows that belong
    to no sequence.
    """
    import torch

    dtypes = {torch.bfloat16: FA_BF16, torch.float16: FA_FP16}
    if not isinstance(q, torch.Tensor) or q.dtype not in dtypes or not q.is_cuda:
        raise TypeError("q must be a bfloat16 or float16 cuda tensor")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != q.dtype or t.device != q.device:
            raise TypeError(f"{name} must be a tensor of q's dtype on q's device")
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 3-D (tokens, heads, head_dim) tensor")
    total_q, Hq, D = q.shape
    total_k, Hkv, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Dk != D:
        raise ValueError("k and v must be [total_k, Hkv, D] matching q")
    dev = q.device
    for name, c in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not isinstance(c, torch.Tensor) or c.dtype != torch.int32 or c.device != dev or c.dim() != 1 \
                or not c.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 vector on q's device")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same B + 1 >= 2 entries")
    B = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or out.device != dev or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev)
    elif lse is not None and (tuple(lse.shape) != (Hq, total_q) or lse.dtype != torch.float32
                              or lse.device != dev or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [Hq, total_q] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    causal = bool(causal)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = _call_with_workspace(
            dev, stream, fa_fwd_workspace_bytes(B, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D, causal),
            lambda: fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  0 if lse is None else lse.data_ptr(), cu_seqlens_q.data_ptr(),
                                  cu_seqlens_k.data_ptr(), B, int(max_seqlen_q), int(max_seqlen_k), total_q, total_k,
                                  Hq, Hkv, D, dtypes[q.dtype], causal, float(scale), stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_fwd_varlen")
    return out, lse
