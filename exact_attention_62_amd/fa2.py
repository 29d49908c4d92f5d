"""Python binding of libfa2.so: argument marshalling only.

Every step of the forward pass runs in the library's HIP kernels; this module
checks tensor properties, passes raw device pointers, sizes and the current
HIP stream through ctypes, and turns status codes into exceptions.  PyTorch
supplies device memory and streams and nothing else.  There is no fallback:
if the library has not been built, or the tensors are not on a GPU, the call
raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

__all__ = ["FA2Error", "FlashAttention", "attention", "attention_backward", "attention_partial",
           "fa2_bwd", "fa2_bwd_workspace_size", "fa2_fwd", "fa2_fwd_cross", "fa2_fwd_partial",
           "fa2_fwd_splitkv", "fa2_fwd_splitkv_noalloc", "fa2_launch_shape", "fa2_merge", "fa2_num_splits",
           "fa2_splitkv_workspace_size", "fa2_strerror", "fa2_last_error", "library_path",
           "load_library", "merge_partials"]

FA2_OK, FA2_EINVAL, FA2_ENOTSUP, FA2_EHIP = 0, -1, -2, -3
FA2_BF16, FA2_FP32, FA2_FP16 = 0, 1, 2
_DTYPES = {torch.bfloat16: FA2_BF16, torch.float32: FA2_FP32, torch.float16: FA2_FP16}

_lib = None
_lock = threading.Lock()


class FA2Error(RuntimeError):
    """A non-zero status from libfa2.so; ``status`` holds the code."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{fa2_strerror(status)} ({status}): {detail}")


def library_path() -> str:
    return os.environ.get("FA2_LIBRARY",
                          os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa2.so"))


def load_library() -> ctypes.CDLL:
    """Load libfa2.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it first (python -m exact_attention_62_amd.build)")
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.fa2_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                ctypes.c_float, ctypes.c_int, vp]
        lib.fa2_fwd.restype = ctypes.c_int
        lib.fa2_fwd_cross.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int,
                                      ctypes.c_float, ctypes.c_int, vp]
        lib.fa2_fwd_cross.restype = ctypes.c_int
        lib.fa2_launch_shape.argtypes = [i64, i64, i64, i64, ctypes.c_int,
                                         ctypes.POINTER(i64), ctypes.POINTER(i64),
                                         ctypes.POINTER(i64)]
        lib.fa2_launch_shape.restype = ctypes.c_int
        lib.fa2_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                        ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                        vp, ctypes.c_size_t, vp]
        lib.fa2_fwd_splitkv.restype = ctypes.c_int
        lib.fa2_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                                ctypes.c_int, vp]
        lib.fa2_fwd_splitkv_noalloc.restype = ctypes.c_int
        lib.fa2_splitkv_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                                   ctypes.POINTER(ctypes.c_size_t)]
        lib.fa2_splitkv_workspace_size.restype = ctypes.c_int
        lib.fa2_num_splits.argtypes = [i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int)]
        lib.fa2_num_splits.restype = ctypes.c_int
        lib.fa2_fwd_partial.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int,
                                        ctypes.c_float, ctypes.c_int, vp]
        lib.fa2_fwd_partial.restype = ctypes.c_int
        lib.fa2_merge.argtypes = [vp, vp, ctypes.c_int, vp, vp, i64, i64, ctypes.c_int, vp]
        lib.fa2_merge.restype = ctypes.c_int
        lib.fa2_bwd.argtypes = [vp] * 9 + [i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                           ctypes.c_int, vp, ctypes.c_size_t, vp]
        lib.fa2_bwd.restype = ctypes.c_int
        lib.fa2_bwd_cross.argtypes = [vp] * 9 + [i64, i64, i64, i64, i64, ctypes.c_int,
                                                 ctypes.c_float, ctypes.c_int, vp, ctypes.c_size_t,
                                                 vp]
        lib.fa2_bwd_cross.restype = ctypes.c_int
        lib.fa2_bwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
        lib.fa2_bwd_workspace_size.restype = ctypes.c_int
        lib.fa2_strerror.argtypes = [ctypes.c_int]
        lib.fa2_strerror.restype = ctypes.c_char_p
        lib.fa2_last_error.argtypes = []
        lib.fa2_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def fa2_strerror(status: int) -> str:
    return load_library().fa2_strerror(int(status)).decode()


def fa2_last_error() -> str:
    return load_library().fa2_last_error().decode()


def _check(status: int) -> None:
    if status != FA2_OK:
        raise FA2Error(status, fa2_last_error())


def fa2_launch_shape(B: int, H: int, N: int, d: int, dtype: torch.dtype = torch.bfloat16):
    """(kBlockM, num_m_block, items): the work decomposition fa2_fwd uses (one item per query block of one (batch, head))."""
    lib = load_library()
    out = [ctypes.c_int64(0) for _ in range(3)]
    _check(lib.fa2_launch_shape(B, H, N, d, _DTYPES.get(dtype, -1), *(ctypes.byref(o) for o in out)))
    return tuple(o.value for o in out)


def _check_tensors(q, k, v, o, lse):
    """q, o [B, H, Nq, d]; k, v [B, H, Nk, d]; lse float32 [B, H, Nq].  Returns B, H, Nq, Nk, d."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError(f"q, k, v must be [B, H, N, d], got {tuple(q.shape)}, {tuple(k.shape)}")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for name, t, shape in (("k", k, (B, H, Nk, d)), ("v", v, (B, H, Nk, d)), ("o", o, q.shape)):
        if t is None:  # an output checked by the caller (a float32 partial result)
            continue
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError(f"lse must be float32 [{B}, {H}, {Nq}], got {lse.dtype} {tuple(lse.shape)}")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    tensors = tuple(t for t in (q, k, v, o, lse) if t is not None)
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("every tensor must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("every tensor must be contiguous")
    if any(t.device != q.device for t in tensors):
        raise ValueError("every tensor must be on the same device")
    return B, H, Nq, Nk, d


def _ptr(t: torch.Tensor):
    """Device address of t, or NULL for an empty tensor (the library does not read it)."""
    return t.data_ptr() if t.numel() else None


def fa2_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
            lse: torch.Tensor, causal: bool = False, scale: float | None = None,
            stream: torch.cuda.Stream | None = None) -> None:
    """Enqueue the forward pass on ``stream`` (default: the current stream).

    q, k, v, o: contiguous [B, H, N, d] tensors of one dtype (bfloat16,
    float16 or float32) on the current GPU; lse: contiguous float32 [B, H, N].
    Writes o and lse in place.
    """
    B, H, N, Nk, d = _check_tensors(q, k, v, o, lse)
    if Nk != N:
        raise ValueError(f"fa2_fwd needs equal query and key lengths ({N} != {Nk}): use fa2_fwd_cross")
    dev = q.device
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         B, H, N, d, 1 if causal else 0, float(scale), _DTYPES[q.dtype],
                         ctypes.c_void_p(stream.cuda_stream))
    _check(st)


def fa2_fwd_cross(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                  lse: torch.Tensor, causal: bool = False, scale: float | None = None,
                  stream: torch.cuda.Stream | None = None) -> None:
    """Enqueue the forward pass of Nq queries over Nk keys.

    q, o: [B, H, Nq, d]; k, v: [B, H, Nk, d]; lse: float32 [B, H, Nq].  With
    causal, key j is visible to query i iff j <= i + Nk - Nq; a query that sees
    no key gets o = 0 and lse = -inf.  Writes o and lse in place.
    """
    B, H, Nq, Nk, d = _check_tensors(q, k, v, o, lse)
    dev = q.device
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.fa2_fwd_cross(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                               1 if causal else 0, float(scale), _DTYPES[q.dtype],
                               ctypes.c_void_p(stream.cuda_stream))
    _check(st)


def fa2_splitkv_workspace_size(B: int, H: int, Nq: int, Nk: int, d: int, num_splits: int) -> int:
    """Bytes of workspace fa2_fwd_splitkv needs with ``num_splits`` splits (no GPU call)."""
    out = ctypes.c_size_t(0)
    _check(load_library().fa2_splitkv_workspace_size(B, H, Nq, Nk, d, int(num_splits),
                                                      ctypes.byref(out)))
    return out.value


def fa2_num_splits(B: int, H: int, Nq: int, Nk: int, d: int, device=None) -> int:
    """The pages' num_splits rule for this problem on ``device`` (default: the current GPU)."""
    out = ctypes.c_int(0)
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        _check(load_library().fa2_num_splits(B, H, Nq, Nk, d, ctypes.byref(out)))
    return out.value


def fa2_fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                    lse: torch.Tensor, workspace: torch.Tensor, num_splits: int = 0,
                    causal: bool = False, scale: float | None = None,
                    stream: torch.cuda.Stream | None = None) -> None:
    """Enqueue the split-KV forward pass (bfloat16 or float16; q [B, H, Nq, d] over k, v
    [B, H, Nk, d]).  ``workspace`` is a contiguous GPU tensor of at least
    fa2_splitkv_workspace_size(...) bytes; num_splits = 0 takes fa2_num_splits's choice.
    Writes o and lse in place."""
    B, H, Nq, Nk, d = _check_tensors(q, k, v, o, lse)
    dev = q.device
    if not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != dev:
        raise ValueError("workspace must be a contiguous tensor on the inputs' GPU")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.fa2_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                                 1 if causal else 0, float(scale), _DTYPES[q.dtype],
                                 int(num_splits), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(),
                                 ctypes.c_void_p(stream.cuda_stream))
    _check(st)


def fa2_fwd_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                            lse: torch.Tensor, num_splits: int = 0, causal: bool = False,
                            scale: float | None = None,
                            stream: torch.cuda.Stream | None = None) -> None:
    """fa2_fwd_splitkv with the partial results in the library's own device scratch
    (FA2_NOALLOC_SCRATCH_BYTES per GPU) instead of a workspace: the call allocates
    nothing.  Calls that overlap on one GPU share that scratch and race.  Writes o
    and lse in place."""
    B, H, Nq, Nk, d = _check_tensors(q, k, v, o, lse)
    dev = q.device
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.fa2_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H,
                                         Nq, Nk, d, 1 if causal else 0, float(scale),
                                         _DTYPES[q.dtype], int(num_splits),
                                         ctypes.c_void_p(stream.cuda_stream))
    _check(st)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
              scale: float | None = None, num_splits: int | None = None):
    """Allocate O and L and run the forward pass.  Returns (o, lse).

    q is [B, H, Nq, d] and k, v [B, H, Nk, d] (Nq != Nk runs fa2_fwd_cross, causal
    aligned bottom-right).  num_splits=None runs the plain pass; an integer runs
    fa2_fwd_splitkv with that many splits (0: the pages' rule), with a workspace
    allocated here."""
    o = torch.empty_like(q, memory_format=torch.contiguous_format)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if num_splits is None:
        if Nq == Nk:
            fa2_fwd(q, k, v, o, lse, causal=causal, scale=scale)
        else:
            fa2_fwd_cross(q, k, v, o, lse, causal=causal, scale=scale)
        return o, lse
    s = num_splits if num_splits > 0 else fa2_num_splits(B, H, Nq, Nk, d, q.device)
    ws = torch.empty(fa2_splitkv_workspace_size(B, H, Nq, Nk, d, s), dtype=torch.uint8,
                     device=q.device)
    fa2_fwd_splitkv(q, k, v, o, lse, ws, num_splits=s, causal=causal, scale=scale)
    return o, lse


def fa2_fwd_partial(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o_part: torch.Tensor,
                    l_part: torch.Tensor, causal: bool = False, scale: float | None = None,
                    stream: torch.cuda.Stream | None = None) -> None:
    """Enqueue attention of q [B, H, Nq, d] over one key/value shard k, v [B, H, Nk, d]
    (bfloat16 or float16), kept as a mergeable partial result: o_part float32
    [B, H, Nq, d] (normalised over this shard) and l_part float32 [B, H, Nq]
    (the shard's logsumexp, -inf for a row that sees none of its keys)."""
    if o_part.dtype != torch.float32 or tuple(o_part.shape) != tuple(q.shape):
        raise ValueError(f"o_part must be float32 {tuple(q.shape)}")
    B, H, Nq, Nk, d = _check_tensors(q, k, v, None, l_part)
    if not o_part.is_cuda or not o_part.is_contiguous() or o_part.device != q.device:
        raise ValueError("o_part must be a contiguous tensor on the inputs' GPU")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa2_fwd_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(l_part), B, H, Nq,
                                 Nk, d, 1 if causal else 0, float(scale), _DTYPES[q.dtype],
                                 ctypes.c_void_p(stream.cuda_stream))
    _check(st)


def fa2_merge(o_parts: torch.Tensor, l_parts: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
              stream: torch.cuda.Stream | None = None) -> None:
    """Enqueue the merge of S partial results: o_parts float32 [S, ..., d], l_parts float32
    [S, ...] -> o [..., d] (bfloat16, float16 or float32) and lse float32 [...]."""
    S = o_parts.shape[0]
    if (o_parts.dtype != torch.float32 or l_parts.dtype != torch.float32
            or lse.dtype != torch.float32):
        raise ValueError("o_parts, l_parts and lse must be float32")
    if tuple(o_parts.shape[1:]) != tuple(o.shape) or tuple(l_parts.shape) != (S, *o.shape[:-1]) \
            or tuple(lse.shape) != tuple(o.shape[:-1]):
        raise ValueError(f"shapes do not match: o_parts {tuple(o_parts.shape)}, l_parts "
                         f"{tuple(l_parts.shape)}, o {tuple(o.shape)}, lse {tuple(lse.shape)}")
    if o.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {o.dtype}")
    for t in (o_parts, l_parts, o, lse):
        if not t.is_cuda or not t.is_contiguous() or t.device != o.device:
            raise ValueError("every tensor must be contiguous and on the same GPU")
    rows = lse.numel()
    if stream is None:
        stream = torch.cuda.current_stream(o.device)
    with torch.cuda.device(o.device):
        st = load_library().fa2_merge(_ptr(o_parts), _ptr(l_parts), int(S), _ptr(o), _ptr(lse),
                                      rows, o.shape[-1], _DTYPES[o.dtype],
                                      ctypes.c_void_p(stream.cuda_stream))
    _check(st)


def attention_partial(q, k, v, causal: bool = False, scale: float | None = None):
    """Allocate and return (o_part float32, l_part float32) from fa2_fwd_partial."""
    o_part = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    l_part = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa2_fwd_partial(q, k, v, o_part, l_part, causal=causal, scale=scale)
    return o_part, l_part


def merge_partials(parts, dtype: torch.dtype = torch.bfloat16):
    """Merge a list of (o_part, l_part) pairs (as attention_partial returns) into (o, lse)."""
    o_parts = torch.stack([p[0] for p in parts])
    l_parts = torch.stack([p[1] for p in parts])
    o = torch.empty(o_parts.shape[1:], dtype=dtype, device=o_parts.device)
    lse = torch.empty(l_parts.shape[1:], dtype=torch.float32, device=o_parts.device)
    fa2_merge(o_parts, l_parts, o, lse)
    return o, lse


def fa2_bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    """Bytes of workspace fa2_bwd needs, N the query length (no GPU call)."""
    out = ctypes.c_size_t(0)
    _check(load_library().fa2_bwd_workspace_size(B, H, N, d, ctypes.byref(out)))
    return out.value


def fa2_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
            do: torch.Tensor, lse: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor,
            dv: torch.Tensor, workspace: torch.Tensor, causal: bool = False,
            scale: float | None = None, stream: torch.cuda.Stream | None = None) -> None:
    """Enqueue the backward pass (bfloat16 or float16): writes dq, dk, dv in place.  o and lse
    are the forward's outputs for q [B, H, Nq, d], k, v [B, H, Nk, d] (Nq != Nk runs
    fa2_bwd_cross, causal aligned bottom-right); workspace holds at least
    fa2_bwd_workspace_size(B, H, Nq, d) bytes."""
    B, H, N, Nk, d = _check_tensors(q, k, v, o, lse)
    for name, t, like in (("do", do, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if t.shape != like.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must be {q.dtype} {tuple(like.shape)}")
        if not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor on the inputs' GPU")
    if not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous tensor on the inputs' GPU")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lib = load_library()
    ptrs = [_ptr(t) for t in (q, k, v, o, do, lse, dq, dk, dv)]
    tail = (1 if causal else 0, float(scale), _DTYPES[q.dtype], _ptr(workspace),
            workspace.numel() * workspace.element_size(), ctypes.c_void_p(stream.cuda_stream))
    with torch.cuda.device(q.device):
        if Nk == N:
            st = lib.fa2_bwd(*ptrs, B, H, N, d, *tail)
        else:
            st = lib.fa2_bwd_cross(*ptrs, B, H, N, Nk, d, *tail)
    _check(st)


def attention_backward(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None):
    """Allocate dQ, dK, dV and a workspace, run fa2_bwd, return (dq, dk, dv)."""
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, H, N, d = q.shape
    ws = torch.empty(fa2_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=q.device)
    fa2_bwd(q, k, v, o, do.contiguous(), lse, dq, dk, dv, ws, causal=causal, scale=scale)
    return dq, dk, dv


class FlashAttention(torch.autograd.Function):
    """Autograd wrapper: forward through fa2_fwd / fa2_fwd_cross, backward through fa2_bwd /
    fa2_bwd_cross (bfloat16 or float16; every head dimension of the forward)."""

    @staticmethod
    def forward(ctx, q, k, v, causal=False, scale=None):
        o, lse = attention(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attention_backward(q, k, v, o, lse, do, causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None
