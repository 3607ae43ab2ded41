"""MI355X (gfx950) SageAttention-style quantized attention forward.

A thin ctypes binding over libsage.so (include/sage.h). Every step of the
computation runs in the library's HIP kernels; this module only turns torch
tensors into pointers, sizes and strides, allocates outputs and workspace
with torch, passes torch's current HIP stream, and turns error codes into
exceptions. There is no fallback: if libsage.so is missing or the device is
not a gfx950, calls raise.

Entry points (the kernels-community issue "aiter-sage-attention", section
"What I have so far", names sageattn(q, k, v, tensor_layout, is_causal,
sm_scale, return_lse) and gfx1201_sage_attention(query, key, value,
softmax_scale, ...)):

  sageattn(q, k, v, tensor_layout="NHD", is_causal=False, sm_scale=None,
           return_lse=False, smooth_k=True)
  gfx950_sage_attention(query, key, value, softmax_scale=None, smooth_k=True)
  prepare(q, k, v, smooth_k, reuse=None) -> dict of quantized tensors
  attn(prepared, sm_scale, out=None, return_lse=False, is_causal=False)
                                        -> BF16 output (, lse)
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import struct
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsage.so")

SAGE_BF16 = 1
SAGE_OK, SAGE_ERR_INVALID_ARGUMENT, SAGE_ERR_UNSUPPORTED, SAGE_ERR_WORKSPACE_TOO_SMALL, SAGE_ERR_DEVICE = range(5)
HEAD_DIM = 128   # the pages' head dim; the library also takes 64


class SageTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("size", ctypes.c_int64 * 4),
                ("stride", ctypes.c_int64 * 4)]


# The same record as raw bytes (pointer, dtype, 4 bytes of padding, sizes,
# strides): the fused call fills a per-thread array of four in place, which
# costs less host time per call than building four SageTensor objects.
_DESC = struct.Struct("<Qi4x4q4q")
assert _DESC.size == ctypes.sizeof(SageTensor)
_TLS = threading.local()


class SageError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class SageUnsupported(SageError, NotImplementedError):
    pass


class SageInvalid(SageError, ValueError):
    pass


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int64
_T = ctypes.POINTER(SageTensor)


def lib():
    """Load libsage.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # Load torch's HIP runtime first: libsage.so then binds to that same
        # libamdhip64 (matched by soname) instead of mapping a second runtime
        # that would compete with torch's for the device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        L.sage_kv_tile.restype = ctypes.c_int
        L.sage_padded_len.argtypes = [_I]
        L.sage_padded_len.restype = _I
        L.sage_prepare_workspace_bytes.argtypes = [_I, _I, _I, _I, ctypes.c_int]
        L.sage_prepare_workspace_bytes.restype = ctypes.c_size_t
        L.sage_fused_workspace_bytes.argtypes = [_I, _I, _I, _I]
        L.sage_fused_workspace_bytes.restype = ctypes.c_size_t
        L.sage_prepare.argtypes = [_T, _T, _T, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.sage_prepare.restype = ctypes.c_int
        L.sage_prepare_noalloc.argtypes = [_T, _T, _T, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P]
        L.sage_prepare_noalloc.restype = ctypes.c_int
        L.sage_attn.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _T, _P]
        L.sage_attn.restype = ctypes.c_int
        L.sage_attn_lse.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _T, _P, _P]
        L.sage_attn_lse.restype = ctypes.c_int
        L.sage_attn_ex.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, ctypes.c_int, _T, _P,
                                   _P]
        L.sage_attn_ex.restype = ctypes.c_int
        L.sage_attn_fused.argtypes = [_T, _T, _T, _T, ctypes.c_int, ctypes.c_float, ctypes.c_int, _P, ctypes.c_int,
                                      _P, ctypes.c_size_t, _P]
        L.sage_attn_fused.restype = ctypes.c_int
        L.sage_status_string.argtypes = [ctypes.c_int]
        L.sage_status_string.restype = ctypes.c_char_p
        L.sage_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def check(status: int) -> None:
    if status == SAGE_OK:
        return
    L = lib()
    msg = f"{L.sage_status_string(status).decode()}: {L.sage_last_error().decode()}"
    if status == SAGE_ERR_UNSUPPORTED:
        raise SageUnsupported(status, msg)
    if status in (SAGE_ERR_INVALID_ARGUMENT, SAGE_ERR_WORKSPACE_TOO_SMALL):
        raise SageInvalid(status, msg)
    raise SageError(status, msg)


def kv_tile() -> int:
    return int(lib().sage_kv_tile())


def padded_len(S: int) -> int:
    return int(lib().sage_padded_len(S))


_DTYPE_CODES = {}
_I64x4 = ctypes.c_int64 * 4


def _dtype_code(t) -> int:
    if not _DTYPE_CODES:
        import torch
        _DTYPE_CODES.update({torch.bfloat16: 1, torch.float16: 2, torch.float32: 3})
    return _DTYPE_CODES.get(t.dtype, 0)


def describe(t, layout: str = "NHD") -> SageTensor:
    """sage_tensor for a 4-D torch tensor in NHD ([B,S,H,D]) or HND ([B,H,S,D]) order."""
    if t.dim() != 4:
        raise ValueError("expected a 4-D tensor")
    if layout == "NHD":
        size, stride = t.shape, t.stride()
    elif layout == "HND":
        B, H, S, D = t.shape
        sb, sh, ss, sd = t.stride()
        size, stride = (B, S, H, D), (sb, ss, sh, sd)
    else:
        raise ValueError(f"tensor_layout must be 'NHD' or 'HND', not {layout!r}")
    return SageTensor(t.data_ptr(), _dtype_code(t), _I64x4(*size), _I64x4(*stride))


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _gpu_of(*tensors, stream=None) -> int:
    """Index of the one GPU every given tensor (and the stream) lives on; the
    library takes device pointers, so a host tensor or a mix of devices is an
    error here rather than a fault on the device."""
    idx = None
    for t in tensors:
        if t is None:
            continue
        dev = t.get_device()   # -1 for a host tensor
        if dev < 0 or not t.is_cuda:
            raise ValueError("every tensor must be on a GPU: the library takes device pointers")
        if idx is None:
            idx = dev
        elif dev != idx:
            raise ValueError(f"tensors on different GPUs ({idx} and {dev})")
    if stream is not None and idx is not None and stream.device.index != idx:
        raise ValueError(f"the stream belongs to GPU {stream.device.index}, the tensors to GPU {idx}")
    return idx


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _fill(buf, i, t, layout):
    """Descriptor i of buf (a SageTensor array) for t, as describe() makes it;
    returns a reference to it for the library call."""
    if t.dim() != 4:
        raise ValueError("expected a 4-D tensor")
    if layout == "NHD":
        size, stride = t.shape, t.stride()
    elif layout == "HND":
        B, H, S, D = t.shape
        sb, sh, ss, sd = t.stride()
        size, stride = (B, S, H, D), (sb, ss, sh, sd)
    else:
        raise ValueError(f"tensor_layout must be 'NHD' or 'HND', not {layout!r}")
    _DESC.pack_into(buf[0], i * _DESC.size, t.data_ptr(), _dtype_code(t), *size, *stride)
    return buf[2][i]


def _on_device(idx):
    """torch.cuda.device(idx), entered only when idx is not already current."""
    import torch
    if idx is None or idx == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(idx)


def _alloc_on(stream):
    """Allocate on the stream the library will use: torch's caching allocator
    then reuses a freed block only behind that stream's pending work (a
    temporary allocated on the current stream but used on another could be
    handed out again while the other stream still reads it)."""
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def prepare(q, k, v, smooth_k: bool = True, layout: str = "NHD", stream=None, reuse: dict | None = None) -> dict:
    """Run the prologue; returns the quantized tensors in the library's layouts.

    reuse: the dict a previous prepare() returned for the same B, S, H, D; its
    tensors and workspace are written again instead of allocating new ones.
    """
    import torch
    reused = [reuse[key] for key in ("q8", "q_scale", "k8", "k_scale", "v8t", "v_scale", "k_mean", "_ws")] \
        if reuse is not None else []
    with _on_device(_gpu_of(q, k, v, *reused, stream=stream)):
        return _prepare(q, k, v, smooth_k, layout, stream, reuse)


def _prepare(q, k, v, smooth_k, layout, stream, reuse):
    import torch
    tq, tk, tv = describe(q, layout), describe(k, layout), describe(v, layout)
    B, S, H, D = tq.size
    Sp = padded_len(S)
    dev = q.device
    L = lib()
    nws = L.sage_prepare_workspace_bytes(B, S, H, D, int(bool(smooth_k)))
    if reuse is not None:
        if reuse["q8"].shape != (B, H, Sp, D) or reuse["S"] != S or reuse["_ws"].numel() < max(int(nws), 1):
            raise ValueError("prepare(reuse=...) needs the result of a call with the same B, S, H, D")
        out = reuse
        ws = reuse["_ws"]
    else:
        with _alloc_on(stream):
            out = _alloc_prepared(B, S, H, D, Sp, dev)
            ws = torch.empty(max(int(nws), 1), dtype=torch.uint8, device=dev)
    check(L.sage_prepare(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), int(bool(smooth_k)), _ptr(out["q8"]),
                         _ptr(out["q_scale"]), _ptr(out["k8"]), _ptr(out["k_scale"]), _ptr(out["v8t"]),
                         _ptr(out["v_scale"]), _ptr(out["k_mean"]), _ptr(ws), nws, _stream(stream)))
    out["S"] = S
    out["_ws"] = ws   # keep the workspace alive until the stream is done with it
    return out


def _alloc_prepared(B, S, H, D, Sp, dev):
    import torch
    return dict(q8=torch.empty((B, H, Sp, D), dtype=torch.int8, device=dev),
                q_scale=torch.empty((B, H, Sp // 32), dtype=torch.float32, device=dev),
                k8=torch.empty((B, H, Sp, D), dtype=torch.int8, device=dev),
                k_scale=torch.empty((B, H, Sp // 32), dtype=torch.float32, device=dev),
                v8t=torch.empty((B, H, D, Sp), dtype=torch.uint8, device=dev),
                v_scale=torch.empty((B, H, D), dtype=torch.float32, device=dev),
                k_mean=torch.empty((B, H, D), dtype=torch.float32, device=dev))


def attn(prep: dict, sm_scale: float, out=None, stream=None, return_lse: bool = False, lse=None,
         is_causal: bool = False):
    """Attention step on prepare()'s output; returns BF16 [B, S, H, D], and with
    return_lse also the rows' log-sum-exp, float32 [B, H, S] (sage_attn_lse).
    is_causal: query i sees keys 0 .. i (sage_attn_ex)."""
    import torch
    tensors = [prep[key] for key in ("q8", "q_scale", "k8", "k_scale", "v8t", "v_scale")]
    with _on_device(_gpu_of(*tensors, out, lse, stream=stream)):
        return _attn(prep, sm_scale, out, stream, return_lse, lse, is_causal)


def _attn(prep, sm_scale, out, stream, return_lse, lse, is_causal):
    import torch
    B, H, Sp, D = prep["q8"].shape
    S = prep["S"]
    with _alloc_on(stream):
        if out is None:
            out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=prep["q8"].device)
        if return_lse and lse is None:
            lse = torch.empty((B, H, S), dtype=torch.float32, device=prep["q8"].device)
    to = describe(out)
    args = (_ptr(prep["q8"]), _ptr(prep["q_scale"]), _ptr(prep["k8"]), _ptr(prep["k_scale"]), _ptr(prep["v8t"]),
            _ptr(prep["v_scale"]), B, S, H, D, float(sm_scale), ctypes.byref(to))
    if is_causal:
        check(lib().sage_attn_ex(*args[:11], 1, args[11], _ptr(lse) if return_lse else None, _stream(stream)))
    elif not return_lse:
        check(lib().sage_attn(*args, _stream(stream)))
    else:
        check(lib().sage_attn_lse(*args, _ptr(lse), _stream(stream)))
    return (out, lse) if return_lse else out


def fused_workspace_bytes(B: int, S: int, H: int, D: int = HEAD_DIM) -> int:
    return int(lib().sage_fused_workspace_bytes(B, S, H, D))


def sageattn(q, k, v, tensor_layout: str = "NHD", is_causal: bool = False, sm_scale=None, return_lse: bool = False,
             smooth_k: bool = True, out=None, workspace=None, stream=None):
    """Quantized attention forward (prologue + attention) on one stream.

    q, k, v: BF16 [B, S, H, D] ("NHD") or [B, H, S, D] ("HND"), equal shapes, D = 128
    (the pages' head dim) or 64.
    is_causal=True lets query i see keys 0 .. i only, and return_lse=True also
    returns the rows' log-sum-exp of the dequantized scores, float32 [B, H, S]
    (both extensions: the pages' sageattn rejects them).
    """
    with _on_device(_gpu_of(q, k, v, out, workspace, stream=stream)):
        return _sageattn(q, k, v, tensor_layout, is_causal, sm_scale, return_lse, smooth_k, out, workspace, stream)


def _sageattn(q, k, v, tensor_layout, is_causal, sm_scale, return_lse, smooth_k, out, workspace, stream):
    import torch
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    buf = getattr(_TLS, "desc", None)
    if buf is None:   # the array, its elements (aliasing it) and references to them
        arr = (SageTensor * 4)()
        elems = [arr[i] for i in range(4)]
        buf = _TLS.desc = (arr, elems, [ctypes.byref(e) for e in elems])
    tq, tk, tv = _fill(buf, 0, q, tensor_layout), _fill(buf, 1, k, tensor_layout), _fill(buf, 2, v, tensor_layout)
    B, S, H, D = buf[1][0].size
    L = lib()
    lse = None
    if out is None or workspace is None or return_lse:   # the library itself allocates nothing
        with _alloc_on(stream):
            if out is None:
                out = torch.empty_like(q)
            if workspace is None:
                nws = int(L.sage_fused_workspace_bytes(B, S, H, D))
                workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=q.device)
            if return_lse:
                lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    to = _fill(buf, 3, out, tensor_layout)
    check(L.sage_attn_fused(tq, tk, tv, to, int(bool(is_causal)),
                            float(sm_scale), int(bool(return_lse)), _ptr(lse), int(bool(smooth_k)), _ptr(workspace),
                            workspace.numel(), _stream(stream)))
    return (out, lse) if return_lse else out


def gfx950_sage_attention(query, key, value, softmax_scale=None, smooth_k: bool = True):
    """BF16 [B, S, H, D] attention with the quantized forward (NHD layout, D = 128 or 64)."""
    return sageattn(query, key, value, "NHD", False, softmax_scale, False, smooth_k)
