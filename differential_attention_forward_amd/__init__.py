"""Python binding of the gfx950 differential-attention library (libdiffattn.so).

Argument marshalling only: every function below forwards to the C entry point
of the same name (declared in ``include/diffattn.h``) with device pointers
taken from torch tensors and the current HIP stream.  All arithmetic of the
path runs in the HIP kernels.  Importing works without the library; the first
call raises ``RuntimeError`` if ``libdiffattn.so`` has not been built (there is
no CPU fallback).

The method (paperleet "Differential Transformer Attention", equation for A1,
A2 and O):  O = (softmax(Q1 K1^T/sqrt(D) + M) - lambda softmax(Q2 K2^T/sqrt(D) + M)) V
with Q/K [B, H, T, D] and V, O [B, H, T, 2D].
"""

from __future__ import annotations

import contextlib
import ctypes
import functools
import os
import re

import torch

__all__ = [
    "DIFFATTN_F32", "DIFFATTN_BF16", "library_path", "lib",
    "diffattn_status_string", "diffattn_lambda_init", "diffattn_lambda", "diffattn_fwd",
    "diffattn_fwd_reparam", "diffattn_fwd_window", "diffattn_fwd_strided", "diffattn_attention_fwd",
    "diffattn_decode_default_splits", "diffattn_decode_workspace_bytes", "diffattn_decode",
    "diffattn_decode_ragged", "diffattn_decode_noalloc", "DIFFATTN_NOALLOC_SCRATCH_BYTES",
    "diffattn_train_saved_bytes", "diffattn_fwd_train", "diffattn_bwd_workspace_bytes",
    "diffattn_bwd", "diffattn_v2_fwd", "diffattn_v2_decode_workspace_bytes", "diffattn_v2_decode",
]

DIFFATTN_F32 = 0
DIFFATTN_BF16 = 1
DIFFATTN_NOALLOC_SCRATCH_BYTES = 32 << 20  # the header's macro of the same name

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libdiffattn.so"
_lib = None

_VP = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_LLP = ctypes.POINTER(ctypes.c_longlong)
_SIGS = {
    "diffattn_status_string": (ctypes.c_char_p, [_I]),
    "diffattn_lambda_init": (_F, [_I]),
    "diffattn_lambda": (_I, [_VP, _VP, _VP, _VP, _I, _I, _F, _VP, _VP]),
    "diffattn_fwd": (_I, [_I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _F, _F,
                          _VP, _VP]),
    "diffattn_fwd_reparam": (_I, [_I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                  _I, _I, _I, _F, _F, _VP, _VP, _VP]),
    "diffattn_attention_fwd": (_I, [_I, _I, _I, _I, _I, _VP, _VP, _VP, _I, _VP, _VP]),
    "diffattn_fwd_window": (_I, [_I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _F, _F,
                                 _VP, _VP]),
    "diffattn_fwd_strided": (_I, [_I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _LLP, _VP, _I, _I, _F,
                                  _F, _VP, _VP]),
    "diffattn_decode_default_splits": (_I, [_I, _I, _I]),
    "diffattn_decode_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "diffattn_decode": (_I, [_I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _I, _F, _F, _I,
                             _VP, ctypes.c_size_t, _VP, _VP]),
    "diffattn_decode_ragged": (_I, [_I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _F, _F,
                                    _I, _VP, ctypes.c_size_t, _VP, _VP]),
    "diffattn_decode_noalloc": (_I, [_I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _I, _F, _F,
                                     _I, _VP, _VP]),
    "diffattn_train_saved_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "diffattn_fwd_train": (_I, [_I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _F, _F,
                                _VP, _VP, ctypes.c_size_t, _VP]),
    "diffattn_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "diffattn_v2_fwd": (_I, [_I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _I, _VP, _VP]),
    "diffattn_v2_decode_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I]),
    "diffattn_v2_decode": (_I, [_I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _I, _VP,
                                ctypes.c_size_t, _VP, _VP]),
    "diffattn_bwd": (_I, [_I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                          ctypes.c_size_t, _I, _I, _F, _F, _VP, _VP, _VP, _VP, _VP, _VP,
                          _VP, _VP, _VP, _VP, _I, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
}


def library_path() -> str:
    """The in-tree libdiffattn.so, or the file DIFFATTN_LIBRARY names (used to
    run the CPU ABI tests against a sanitizer-instrumented host build)."""
    return os.environ.get("DIFFATTN_LIBRARY") or os.path.join(_HERE, _LIB_NAME)


def lib() -> ctypes.CDLL:
    """The loaded C library (loaded on first use; raises if it was not built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m differential_attention_forward_amd.build`"
                " (there is no CPU fallback)")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions() -> list:
    """Names of the functions declared in include/diffattn.h (for symbol checks)."""
    hdr = os.path.join(os.path.dirname(_HERE), "include", "diffattn.h")
    with open(hdr) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(diffattn_\w+)\s*\(", text, re.M)))


def _check(status: int) -> None:
    if status != 0:
        raise RuntimeError(f"diffattn: {diffattn_status_string(status)} (status {status})")


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


@contextlib.contextmanager
def _on_stream(stream):
    """Makes ``stream`` (a torch stream or a raw HIP stream handle) current for
    the body: it first waits for the work queued so far on the caller's current
    stream (which produced the inputs), and every temporary the body allocates
    (contiguous copies, the lambda vector, a default output or workspace)
    belongs to it, so the caching allocator does not hand that memory out
    while the launch still reads it.  Tensors the caller passes in stay the
    caller's to keep alive until the stream has finished with them."""
    if stream is None:
        yield
        return
    target = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    current = torch.cuda.current_stream(target.device)
    if current.cuda_stream != target.cuda_stream:
        target.wait_stream(current)
    with torch.cuda.stream(target):
        yield


def _streamed(fn):
    """Runs ``fn`` with its ``stream`` argument made current (see _on_stream)."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        with _on_stream(stream):
            return fn(*args, **kwargs)
    return wrapper


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DIFFATTN_F32
    if t.dtype == torch.bfloat16:
        return DIFFATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on a HIP device")
    return t.contiguous()


def _lambda_vec(lam, h: int, device) -> torch.Tensor:
    """A per-head fp32 device vector [H] from a scalar, 0-d or [H] lambda."""
    if isinstance(lam, torch.Tensor):
        lam = lam.to(device=device, dtype=torch.float32)
        if lam.dim() == 0 or lam.numel() == 1:
            return lam.reshape(1).expand(h).contiguous()
        if lam.shape != (h,):
            raise ValueError(f"lambda must be a scalar or have shape [{h}]")
        return lam.contiguous()
    return torch.full((h,), float(lam), device=device, dtype=torch.float32)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def diffattn_status_string(status: int) -> str:
    return lib().diffattn_status_string(int(status)).decode()


def diffattn_lambda_init(layer: int) -> float:
    return float(lib().diffattn_lambda_init(int(layer)))


@_streamed
def diffattn_lambda(lq1, lk1, lq2, lk2, lambda_init: float, out=None, stream=None):
    """lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init, per head.

    Vectors of shape [Dl] give a 0-d tensor, [H, Dl] give [H] (fp32, device).
    """
    vecs = [_dev(t, n).float() for t, n in ((lq1, "lq1"), (lk1, "lk1"), (lq2, "lq2"), (lk2, "lk2"))]
    one_d = vecs[0].dim() == 1
    vecs = [v.reshape(1, -1) if one_d else v for v in vecs]
    h, dl = vecs[0].shape
    for v in vecs:
        if v.shape != (h, dl):
            raise ValueError("the four lambda vectors must have the same shape")
    if out is None:
        out = torch.empty((h,), device=vecs[0].device, dtype=torch.float32)
    _check(lib().diffattn_lambda(*map(_ptr, vecs), h, dl, float(lambda_init), _ptr(out),
                                 _stream(stream)))
    return out.reshape(()) if one_d else out


def _fwd_inputs(q1, k1, q2, k2, v):
    q1, k1, q2, k2, v = (_dev(t, n) for t, n in
                         ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2"), (v, "v")))
    if q1.dim() != 4:
        raise ValueError("q1 must be [B, H, T, D]")
    b, h, t, d = q1.shape
    for x, n in ((k1, "k1"), (q2, "q2"), (k2, "k2")):
        if x.shape != q1.shape or x.dtype != q1.dtype:
            raise ValueError(f"{n} must match q1 in shape and dtype")
    if v.shape != (b, h, t, 2 * d) or v.dtype != q1.dtype:
        raise ValueError("v must be [B, H, T, 2D] with the dtype of q1")
    return q1, k1, q2, k2, v


@_streamed
def diffattn_fwd(q1, k1, q2, k2, v, lam, causal: bool = True, headnorm: bool = False,
                 lambda_init: float = 0.8, eps: float = 1e-5, out=None, stream=None):
    """Prefill forward; q*, k* [B,H,T,D], v [B,H,T,2D] -> out [B,H,T,2D].

    ``lam``: a scalar, a 0-d tensor or an [H] tensor (lambda itself).
    """
    q1, k1, q2, k2, v = _fwd_inputs(q1, k1, q2, k2, v)
    b, h, t, d = q1.shape
    lamv = _lambda_vec(lam, h, q1.device)
    if out is None:
        out = torch.empty_like(v)
    _check(lib().diffattn_fwd(_dtype_code(q1), b, h, t, d, _ptr(q1), _ptr(k1), _ptr(q2),
                              _ptr(k2), _ptr(v), _ptr(lamv), int(bool(causal)),
                              int(bool(headnorm)), float(lambda_init), float(eps), _ptr(out),
                              _stream(stream)))
    return out


def _view4(t, name, width_of_last):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on a HIP device")
    if t.dim() != 4 or t.shape[-1] != width_of_last:
        raise ValueError(f"{name} must be 4-D with last dimension {width_of_last}")
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return t


@_streamed
def diffattn_fwd_strided(q1, k1, q2, k2, v, lam, causal: bool = True, headnorm: bool = False,
                         lambda_init: float = 0.8, eps: float = 1e-5, out=None, stream=None):
    """Prefill forward on strided views, without copies: q*, k* are [B,H,T,D]
    views, v a [B,H,T,2D] view (each with a contiguous last dimension, e.g.
    the halves of a fused projection); ``out`` may be a view too (default: a
    new dense [B,H,T,2D] tensor)."""
    if not isinstance(q1, torch.Tensor) or q1.dim() != 4:
        raise ValueError("q1 must be [B, H, T, D]")
    b, h, t, d = q1.shape
    q1, k1, q2, k2 = (_view4(x, n, d) for x, n in ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2")))
    v = _view4(v, "v", 2 * d)
    for x, n in ((k1, "k1"), (q2, "q2"), (k2, "k2")):
        if x.shape != q1.shape or x.dtype != q1.dtype:
            raise ValueError(f"{n} must match q1 in shape and dtype")
    if v.shape != (b, h, t, 2 * d) or v.dtype != q1.dtype:
        raise ValueError("v must be [B, H, T, 2D] with the dtype of q1")
    lamv = _lambda_vec(lam, h, q1.device)
    if out is None:
        out = torch.empty((b, h, t, 2 * d), device=q1.device, dtype=q1.dtype)
    out = _view4(out, "out", 2 * d)
    if out.shape != v.shape or out.dtype != v.dtype:
        raise ValueError("out must be [B, H, T, 2D] with the dtype of q1")
    st = (ctypes.c_longlong * 18)(*[s for x in (q1, k1, q2, k2, v, out) for s in x.stride()[:3]])
    _check(lib().diffattn_fwd_strided(_dtype_code(q1), b, h, t, d, _ptr(q1), _ptr(k1), _ptr(q2),
                                      _ptr(k2), _ptr(v), st, _ptr(lamv), int(bool(causal)),
                                      int(bool(headnorm)), float(lambda_init), float(eps), _ptr(out),
                                      _stream(stream)))
    return out


@_streamed
def diffattn_fwd_window(q1, k1, q2, k2, v, lam, window: int, headnorm: bool = False,
                        lambda_init: float = 0.8, eps: float = 1e-5, out=None, stream=None):
    """Causal prefill with a sliding window: row i sees keys i - window < j <= i."""
    q1, k1, q2, k2, v = _fwd_inputs(q1, k1, q2, k2, v)
    b, h, t, d = q1.shape
    lamv = _lambda_vec(lam, h, q1.device)
    if out is None:
        out = torch.empty_like(v)
    _check(lib().diffattn_fwd_window(_dtype_code(q1), b, h, t, d, _ptr(q1), _ptr(k1), _ptr(q2),
                                     _ptr(k2), _ptr(v), _ptr(lamv), int(window), int(bool(headnorm)),
                                     float(lambda_init), float(eps), _ptr(out), _stream(stream)))
    return out


@_streamed
def diffattn_fwd_reparam(q1, k1, q2, k2, v, lq1, lk1, lq2, lk2, lambda_init: float,
                         causal: bool = True, headnorm: bool = False, eps: float = 1e-5,
                         lambda_out=None, out=None, stream=None):
    """Prefill forward with lambda formed in the same launch from its four
    [H, Dl] vectors (diffattn_lambda then diffattn_fwd, as one kernel).
    ``lambda_out`` (optional [H] fp32 device tensor) receives lambda."""
    q1, k1, q2, k2, v = _fwd_inputs(q1, k1, q2, k2, v)
    b, h, t, d = q1.shape
    vecs = [_dev(x, n).float() for x, n in ((lq1, "lq1"), (lk1, "lk1"), (lq2, "lq2"), (lk2, "lk2"))]
    if vecs[0].dim() != 2 or vecs[0].shape[0] != h or any(x.shape != vecs[0].shape for x in vecs):
        raise ValueError(f"the four lambda vectors must all be [{h}, Dl]")
    dl = vecs[0].shape[1]
    if lambda_out is not None and (lambda_out.shape != (h,) or lambda_out.dtype != torch.float32
                                   or not lambda_out.is_cuda or not lambda_out.is_contiguous()):
        raise ValueError(f"lambda_out must be a contiguous float32 device tensor of shape [{h}]")
    if out is None:
        out = torch.empty_like(v)
    _check(lib().diffattn_fwd_reparam(_dtype_code(q1), b, h, t, d, _ptr(q1), _ptr(k1), _ptr(q2),
                                      _ptr(k2), _ptr(v), *map(_ptr, vecs), dl, int(bool(causal)),
                                      int(bool(headnorm)), float(lambda_init), float(eps),
                                      _ptr(lambda_out) if lambda_out is not None else None,
                                      _ptr(out), _stream(stream)))
    return out


@_streamed
def diffattn_attention_fwd(q, k, v, causal: bool = True, out=None, stream=None):
    """Standard softmax attention (bf16); q, k, v [B,H,T,D], D in {64, 128} ->
    out [B,H,T,D].  The comparison kernel for differential heads of width D/2."""
    q, k, v = (_dev(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v")))
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, T, D]")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must be bfloat16")
    b, h, t, d = q.shape
    if out is None:
        out = torch.empty_like(v)
    _check(lib().diffattn_attention_fwd(DIFFATTN_BF16, b, h, t, d, _ptr(q), _ptr(k), _ptr(v),
                                        int(bool(causal)), _ptr(out), _stream(stream)))
    return out


def diffattn_decode_default_splits(B: int, H: int, L: int) -> int:
    return int(lib().diffattn_decode_default_splits(B, H, L))


def diffattn_decode_workspace_bytes(B: int, H: int, L: int, D: int, num_splits: int = 0) -> int:
    return int(lib().diffattn_decode_workspace_bytes(B, H, L, D, num_splits))


@_streamed
def diffattn_decode(q1, k1, q2, k2, v, lam, headnorm: bool = False, lambda_init: float = 0.8,
                    eps: float = 1e-5, num_splits: int = 0, workspace=None, out=None,
                    stream=None):
    """Decode; q* [B,H,D], caches k* [B,H,L,D] and v [B,H,L,2D] -> out [B,H,2D]."""
    q1, k1, q2, k2, v = (_dev(t, n) for t, n in
                         ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2"), (v, "v")))
    if k1.dim() != 4:
        raise ValueError("k1 must be [B, H, L, D]")
    b, h, l, d = k1.shape
    if q1.shape != (b, h, d) or q2.shape != (b, h, d):
        raise ValueError("q1, q2 must be [B, H, D]")
    if k2.shape != k1.shape or v.shape != (b, h, l, 2 * d):
        raise ValueError("k2 must match k1 and v must be [B, H, L, 2D]")
    for x in (q2, k1, k2, v):
        if x.dtype != q1.dtype:
            raise ValueError("all inputs must share one dtype")
    lamv = _lambda_vec(lam, h, q1.device)
    need = diffattn_decode_workspace_bytes(b, h, l, d, num_splits)
    if workspace is None:
        workspace = torch.empty((max(need, 16) + 3) // 4, device=q1.device, dtype=torch.float32)
    if out is None:
        out = torch.empty((b, h, 2 * d), device=q1.device, dtype=q1.dtype)
    _check(lib().diffattn_decode(_dtype_code(q1), b, h, l, d, _ptr(q1), _ptr(k1), _ptr(q2),
                                 _ptr(k2), _ptr(v), _ptr(lamv), int(bool(headnorm)),
                                 float(lambda_init), float(eps), int(num_splits),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _ptr(out), _stream(stream)))
    return out


@_streamed
def diffattn_decode_noalloc(q1, k1, q2, k2, v, lam, headnorm: bool = False,
                            lambda_init: float = 0.8, eps: float = 1e-5, num_splits: int = 0,
                            out=None, stream=None):
    """diffattn_decode without a workspace: the library's per-GPU scratch
    array holds the partial states (calls that overlap on one GPU race).
    Pass `out` and a tensor `lam` [H] to keep this call free of allocations."""
    q1, k1, q2, k2, v = (_dev(t, n) for t, n in
                         ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2"), (v, "v")))
    if k1.dim() != 4:
        raise ValueError("k1 must be [B, H, L, D]")
    b, h, l, d = k1.shape
    if q1.shape != (b, h, d) or q2.shape != (b, h, d):
        raise ValueError("q1, q2 must be [B, H, D]")
    if k2.shape != k1.shape or v.shape != (b, h, l, 2 * d):
        raise ValueError("k2 must match k1 and v must be [B, H, L, 2D]")
    for x in (q2, k1, k2, v):
        if x.dtype != q1.dtype:
            raise ValueError("all inputs must share one dtype")
    lamv = _lambda_vec(lam, h, q1.device)
    if out is None:
        out = torch.empty((b, h, 2 * d), device=q1.device, dtype=q1.dtype)
    _check(lib().diffattn_decode_noalloc(_dtype_code(q1), b, h, l, d, _ptr(q1), _ptr(k1), _ptr(q2),
                                         _ptr(k2), _ptr(v), _ptr(lamv), int(bool(headnorm)),
                                         float(lambda_init), float(eps), int(num_splits),
                                         _ptr(out), _stream(stream)))
    return out


def _v2_inputs(q1, q2, k, v, tdim):
    q1, q2, k, v = (_dev(t, n) for t, n in ((q1, "q1"), (q2, "q2"), (k, "k"), (v, "v")))
    if q1.dim() != tdim or k.dim() != 4:
        raise ValueError("DIFF V2 shapes: q1, q2 [B, H, (T,) D], k, v [B, Hkv, T, D]")
    if q2.shape != q1.shape or v.shape != k.shape:
        raise ValueError("q2 must match q1 and v must match k")
    if k.shape[0] != q1.shape[0] or k.shape[-1] != q1.shape[-1]:
        raise ValueError("k, v must have the batch and head width of q1")
    for x in (q2, k, v):
        if x.dtype != q1.dtype:
            raise ValueError("all inputs must share one dtype")
    return q1, q2, k, v


@_streamed
def diffattn_v2_fwd(q1, q2, k, v, lam, causal: bool = True, out=None, stream=None):
    """DIFF V2 prefill; q1, q2 [B,H,T,D], k, v [B,Hkv,T,D] -> out [B,H,T,D]."""
    q1, q2, k, v = _v2_inputs(q1, q2, k, v, 4)
    b, h, t, d = q1.shape
    hkv = k.shape[1]
    if k.shape[2] != t:
        raise ValueError("k, v must have the sequence length of q1")
    lamv = _lambda_vec(lam, h, q1.device)
    if out is None:
        out = torch.empty_like(q1)
    _check(lib().diffattn_v2_fwd(_dtype_code(q1), b, h, hkv, t, d, _ptr(q1), _ptr(q2), _ptr(k),
                                 _ptr(v), _ptr(lamv), int(bool(causal)), _ptr(out), _stream(stream)))
    return out


def diffattn_v2_decode_workspace_bytes(B: int, H: int, Hkv: int, L: int, D: int, num_splits: int = 0) -> int:
    return int(lib().diffattn_v2_decode_workspace_bytes(B, H, Hkv, L, D, num_splits))


@_streamed
def diffattn_v2_decode(q1, q2, k, v, lam, num_splits: int = 0, workspace=None, out=None, stream=None):
    """DIFF V2 decode; q1, q2 [B,H,D], caches k, v [B,Hkv,L,D] -> out [B,H,D]."""
    q1, q2, k, v = _v2_inputs(q1, q2, k, v, 3)
    b, h, d = q1.shape
    hkv, l = k.shape[1], k.shape[2]
    lamv = _lambda_vec(lam, h, q1.device)
    need = diffattn_v2_decode_workspace_bytes(b, h, hkv, l, d, num_splits)
    if workspace is None:
        workspace = torch.empty((max(need, 16) + 3) // 4, device=q1.device, dtype=torch.float32)
    if out is None:
        out = torch.empty((b, h, d), device=q1.device, dtype=q1.dtype)
    _check(lib().diffattn_v2_decode(_dtype_code(q1), b, h, hkv, l, d, _ptr(q1), _ptr(q2), _ptr(k),
                                    _ptr(v), _ptr(lamv), int(num_splits), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _ptr(out),
                                    _stream(stream)))
    return out


@_streamed
def diffattn_decode_ragged(q1, k1, q2, k2, v, lam, lengths, headnorm: bool = False,
                           lambda_init: float = 0.8, eps: float = 1e-5, num_splits: int = 0,
                           workspace=None, out=None, stream=None):
    """Decode where sequence b sees only its first lengths[b] cache rows;
    ``lengths``: [B] int32 device tensor (values in [0, L])."""
    q1, k1, q2, k2, v = (_dev(t, n) for t, n in
                         ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2"), (v, "v")))
    b, h, l, d = k1.shape
    if q1.shape != (b, h, d) or q2.shape != (b, h, d) or k2.shape != k1.shape or v.shape != (b, h, l, 2 * d):
        raise ValueError("shapes: q* [B,H,D], k* [B,H,L,D], v [B,H,L,2D]")
    lens = _dev(lengths, "lengths")
    if lens.dtype != torch.int32 or lens.shape != (b,):
        raise ValueError("lengths must be an int32 tensor of shape [B]")
    lamv = _lambda_vec(lam, h, q1.device)
    need = diffattn_decode_workspace_bytes(b, h, l, d, num_splits)
    if workspace is None:
        workspace = torch.empty((max(need, 16) + 3) // 4, device=q1.device, dtype=torch.float32)
    if out is None:
        out = torch.empty((b, h, 2 * d), device=q1.device, dtype=q1.dtype)
    _check(lib().diffattn_decode_ragged(_dtype_code(q1), b, h, l, d, _ptr(q1), _ptr(k1), _ptr(q2),
                                        _ptr(k2), _ptr(v), _ptr(lamv), _ptr(lens), int(bool(headnorm)),
                                        float(lambda_init), float(eps), int(num_splits), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _ptr(out),
                                        _stream(stream)))
    return out


def diffattn_train_saved_bytes(B: int, H: int, T: int, D: int) -> int:
    return int(lib().diffattn_train_saved_bytes(B, H, T, D))


def diffattn_bwd_workspace_bytes(B: int, H: int, T: int, D: int) -> int:
    return int(lib().diffattn_bwd_workspace_bytes(B, H, T, D))


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


@_streamed
def diffattn_fwd_train(q1, k1, q2, k2, v, lam, causal: bool = True, headnorm: bool = False,
                       lambda_init: float = 0.8, eps: float = 1e-5, out=None, saved=None,
                       stream=None):
    """Training forward (bf16, D = 32, 64 or 128): the output of diffattn_fwd plus the
    saved state diffattn_bwd reads.  Returns (out, saved); ``saved`` is an
    opaque uint8 device tensor of diffattn_train_saved_bytes bytes."""
    q1, k1, q2, k2, v = _fwd_inputs(q1, k1, q2, k2, v)
    b, h, t, d = q1.shape
    lamv = _lambda_vec(lam, h, q1.device)
    if out is None:
        out = torch.empty_like(v)
    if saved is None:
        saved = torch.empty(max(diffattn_train_saved_bytes(b, h, t, d), 16), device=q1.device,
                            dtype=torch.uint8)
    _check(lib().diffattn_fwd_train(_dtype_code(q1), b, h, t, d, _ptr(q1), _ptr(k1), _ptr(q2),
                                    _ptr(k2), _ptr(v), _ptr(lamv), int(bool(causal)),
                                    int(bool(headnorm)), float(lambda_init), float(eps), _ptr(out),
                                    _ptr(saved), _nbytes(saved), _stream(stream)))
    return out, saved


@_streamed
def diffattn_bwd(q1, k1, q2, k2, v, lam, dout, saved, causal: bool = True,
                 headnorm: bool = False, lambda_init: float = 0.8, eps: float = 1e-5,
                 lvecs=None, workspace=None, stream=None):
    """Backward of diffattn_fwd_train.  Returns (dq1, dk1, dq2, dk2, dv, dlambda)
    and, when ``lvecs`` = (lq1, lk1, lq2, lk2) ([H, Dl] fp32) is given, a
    seventh item: the tuple of their four gradients."""
    q1, k1, q2, k2, v = _fwd_inputs(q1, k1, q2, k2, v)
    b, h, t, d = q1.shape
    dout = _dev(dout, "dout")
    if dout.shape != v.shape or dout.dtype != v.dtype:
        raise ValueError("dout must match v in shape and dtype")
    lamv = _lambda_vec(lam, h, q1.device)
    grads = [torch.empty_like(x) for x in (q1, k1, q2, k2, v)]
    dlam = torch.empty((h,), device=q1.device, dtype=torch.float32)
    vec_ptrs, dvec_ptrs, dl, dvecs = [None] * 4, [None] * 4, 0, None
    if lvecs is not None:
        vecs = [_dev(x, n).float() for x, n in zip(lvecs, ("lq1", "lk1", "lq2", "lk2"))]
        if vecs[0].dim() != 2 or vecs[0].shape[0] != h or any(x.shape != vecs[0].shape for x in vecs):
            raise ValueError(f"the four lambda vectors must all be [{h}, Dl]")
        dl = vecs[0].shape[1]
        dvecs = [torch.empty_like(x) for x in vecs]
        vec_ptrs, dvec_ptrs = [_ptr(x) for x in vecs], [_ptr(x) for x in dvecs]
    if workspace is None:
        workspace = torch.empty(max(diffattn_bwd_workspace_bytes(b, h, t, d), 16), device=q1.device,
                                dtype=torch.uint8)
    _check(lib().diffattn_bwd(_dtype_code(q1), b, h, t, d, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2),
                              _ptr(v), _ptr(lamv), _ptr(dout), _ptr(saved), _nbytes(saved),
                              int(bool(causal)), int(bool(headnorm)), float(lambda_init), float(eps),
                              *map(_ptr, grads), _ptr(dlam), *vec_ptrs, dl, *dvec_ptrs,
                              _ptr(workspace), _nbytes(workspace), _stream(stream)))
    res = (*grads, dlam)
    return res + (tuple(dvecs),) if dvecs is not None else res
