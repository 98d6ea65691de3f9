"""Python binding of libattn.so, the gfx950 causal attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/attn.h.  Torch tensors supply
device memory and the current stream.  There is no fallback: if the shared
library is missing, every call raises.

Entry points (same names as the C ABI):
    attn_prefill(Q, K, V, O, LSE, causal=1, window=0, scale=None, stream=None)
    attn_prefill_cache(Q, Kcache, Vcache, lens, O, LSE, window=0, scale=None, stream=None)
    attn_decode(q, Kcache, Vcache, lens, O, LSE=None, workspace=None, stream=None)
    attn_decode_window(q, Kcache, Vcache, lens, O, LSE=None, workspace=None,
                       window=0, scale=None, stream=None)
    attn_decode_workspace_bytes(B, Nq, Nkv, Dh, Tcap, dtype)
    attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, window, dtype)
    attn_kv_append(Knew, Vnew, Kcache, Vcache, pos, rolling=0, stream=None)
    attn_backward(Q, K, V, O, dO, LSE, dQ, dK, dV, causal=1, window=0, scale=None,
                  workspace=None, stream=None)
    attn_backward_workspace_bytes(B, Nq, Nkv, S, Dh, dtype)
    attn_strerror(status)
Conveniences that allocate outputs with torch:
    prefill(q, k, v, causal=True, window=0, scale=None) -> (O, LSE)
    prefill_cache(q, Kcache, Vcache, lens, window=0, scale=None) -> (O, LSE)
    decode(q, Kcache, Vcache, lens, window=0, scale=None) -> (O, LSE)
    backward(q, k, v, O, LSE, dO, causal=True, window=0, scale=None) -> (dQ, dK, dV)
"""

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK = 0
ATTN_EINVAL = -1
ATTN_EGQA = -2
ATTN_EUNSUPPORTED = -3
ATTN_EWORKSPACE = -4
ATTN_EHIP = -5
ATTN_BF16 = 0
ATTN_F32 = 1

EXPORTS = ("attn_prefill", "attn_prefill_cache", "attn_decode", "attn_decode_window",
           "attn_decode_workspace_bytes", "attn_decode_window_workspace_bytes",
           "attn_kv_append", "attn_backward", "attn_backward_workspace_bytes",
           "attn_strerror")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {attn_strerror(status)} (status {status})")


def lib():
    """The loaded library with argument types declared; raises if not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m transformer_causal_head_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.attn_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                   f32, i32, vp]
        L.attn_prefill.restype = i32
        L.attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.attn_decode_workspace_bytes.restype = ctypes.c_size_t
        L.attn_decode_window_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.attn_decode_window_workspace_bytes.restype = ctypes.c_size_t
        L.attn_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp,
                                  ctypes.c_size_t, i32, vp]
        L.attn_decode.restype = i32
        L.attn_prefill_cache.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                         i32, f32, i32, vp]
        L.attn_prefill_cache.restype = i32
        L.attn_decode_window.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                         vp, vp, ctypes.c_size_t, i32, vp]
        L.attn_decode_window.restype = i32
        L.attn_kv_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
        L.attn_kv_append.restype = i32
        L.attn_backward_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.attn_backward_workspace_bytes.restype = ctypes.c_size_t
        L.attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                    i32, i32, f32, vp, ctypes.c_size_t, i32, vp]
        L.attn_backward.restype = i32
        L.attn_strerror.argtypes = [i32]
        L.attn_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def attn_strerror(status):
    return lib().attn_strerror(int(status)).decode()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def attn_prefill(Q, K, V, O, LSE, causal=1, window=0, scale=None, stream=None):
    """Q [B,Nq,S,Dh], K/V [B,Nkv,S,Dh], O like Q, LSE fp32 [B,Nq,S] or None."""
    B, Nq, S, Dh = Q.shape
    Nkv = K.shape[1]
    if tuple(K.shape) != (B, Nkv, S, Dh) or K.shape != V.shape or O.shape != Q.shape:
        raise ValueError("shape mismatch between Q, K, V, O")
    if not (Q.dtype == K.dtype == V.dtype == O.dtype):
        raise ValueError("Q, K, V, O must share one dtype")
    if LSE is not None and (tuple(LSE.shape) != (B, Nq, S) or LSE.dtype.itemsize != 4):
        raise ValueError("LSE must be fp32 [B, Nq, S]")
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    st = lib().attn_prefill(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), B, Nq, Nkv, S, Dh,
                            int(causal), int(window), float(scale), _dtype_code(Q),
                            _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_prefill")


def attn_decode_workspace_bytes(B, Nq, Nkv, Dh, Tcap, dtype):
    return int(lib().attn_decode_workspace_bytes(B, Nq, Nkv, Dh, Tcap, dtype))


def attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, window, dtype):
    return int(lib().attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, int(window), dtype))


def _check_decode(q, Kcache, Vcache, lens, O, LSE):
    import torch
    B, Nq, Dh = q.shape
    Nkv, Tcap = Kcache.shape[1], Kcache.shape[2]
    if tuple(Kcache.shape) != (B, Nkv, Tcap, Dh) or Kcache.shape != Vcache.shape:
        raise ValueError("cache shapes must be [B, Nkv, Tcap, Dh]")
    if O.shape != q.shape or lens.dtype != torch.int32 or tuple(lens.shape) != (B,):
        raise ValueError("O must match q; lens must be int32 [B]")
    if LSE is not None and (tuple(LSE.shape) != (B, Nq) or LSE.dtype.itemsize != 4):
        raise ValueError("LSE must be fp32 [B, Nq]")
    return B, Nq, Nkv, Dh, Tcap


def attn_decode(q, Kcache, Vcache, lens, O, LSE=None, workspace=None, stream=None):
    """q [B,Nq,Dh], caches [B,Nkv,Tcap,Dh], lens int32 [B] on the GPU, O like q."""
    B, Nq, Nkv, Dh, Tcap = _check_decode(q, Kcache, Vcache, lens, O, LSE)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_decode(_ptr(q), _ptr(Kcache), _ptr(Vcache), _ptr(lens), _ptr(O), B, Nq,
                           Nkv, Dh, Tcap, _ptr(LSE), _ptr(workspace), ws_bytes,
                           _dtype_code(q), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode")


def attn_decode_window(q, Kcache, Vcache, lens, O, LSE=None, workspace=None, window=0,
                       scale=None, stream=None):
    """attn_decode with a sliding window (keys lens-window .. lens-1) and a scale."""
    B, Nq, Nkv, Dh, Tcap = _check_decode(q, Kcache, Vcache, lens, O, LSE)
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_decode_window(_ptr(q), _ptr(Kcache), _ptr(Vcache), _ptr(lens), _ptr(O), B,
                                  Nq, Nkv, Dh, Tcap, int(window), float(scale), _ptr(LSE),
                                  _ptr(workspace), ws_bytes, _dtype_code(q), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_window")


def attn_prefill_cache(Q, Kcache, Vcache, lens, O, LSE, window=0, scale=None, stream=None):
    """Q [B,Nq,Sq,Dh] against caches [B,Nkv,Tcap,Dh]; lens int32 [B] on the GPU."""
    import torch
    B, Nq, Sq, Dh = Q.shape
    Nkv, Tcap = Kcache.shape[1], Kcache.shape[2]
    if tuple(Kcache.shape) != (B, Nkv, Tcap, Dh) or Kcache.shape != Vcache.shape:
        raise ValueError("cache shapes must be [B, Nkv, Tcap, Dh]")
    if O.shape != Q.shape or lens.dtype != torch.int32 or tuple(lens.shape) != (B,):
        raise ValueError("O must match Q; lens must be int32 [B]")
    if not (Q.dtype == Kcache.dtype == Vcache.dtype == O.dtype):
        raise ValueError("Q, caches and O must share one dtype")
    if LSE is not None and (tuple(LSE.shape) != (B, Nq, Sq) or LSE.dtype.itemsize != 4):
        raise ValueError("LSE must be fp32 [B, Nq, Sq]")
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    st = lib().attn_prefill_cache(_ptr(Q), _ptr(Kcache), _ptr(Vcache), _ptr(lens), _ptr(O),
                                  _ptr(LSE), B, Nq, Nkv, Sq, Dh, Tcap, int(window), float(scale),
                                  _dtype_code(Q), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_prefill_cache")


def attn_kv_append(Knew, Vnew, Kcache, Vcache, pos, rolling=0, stream=None):
    """New rows [B,Nkv,Snew,Dh] into caches [B,Nkv,Tcap,Dh] at pos (int32 [B], GPU)."""
    import torch
    B, Nkv, Snew, Dh = Knew.shape
    Tcap = Kcache.shape[2]
    if Knew.shape != Vnew.shape or tuple(Kcache.shape) != (B, Nkv, Tcap, Dh) \
            or Kcache.shape != Vcache.shape:
        raise ValueError("new rows must be [B, Nkv, Snew, Dh] and caches [B, Nkv, Tcap, Dh]")
    if not (Knew.dtype == Vnew.dtype == Kcache.dtype == Vcache.dtype):
        raise ValueError("all four buffers must share one dtype")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (B,):
        raise ValueError("pos must be int32 [B]")
    st = lib().attn_kv_append(_ptr(Knew), _ptr(Vnew), _ptr(Kcache), _ptr(Vcache), _ptr(pos), B,
                              Nkv, Snew, Dh, Tcap, int(rolling), _dtype_code(Knew),
                              _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_kv_append")


def attn_backward_workspace_bytes(B, Nq, Nkv, S, Dh, dtype):
    return int(lib().attn_backward_workspace_bytes(B, Nq, Nkv, S, Dh, dtype))


def attn_backward(Q, K, V, O, dO, LSE, dQ, dK, dV, causal=1, window=0, scale=None,
                  workspace=None, stream=None):
    """Gradients of attn_prefill; shapes as attn_prefill, dQ like Q, dK/dV like K."""
    B, Nq, S, Dh = Q.shape
    Nkv = K.shape[1]
    if tuple(K.shape) != (B, Nkv, S, Dh) or K.shape != V.shape:
        raise ValueError("K and V must be [B, Nkv, S, Dh]")
    if O.shape != Q.shape or dO.shape != Q.shape or dQ.shape != Q.shape:
        raise ValueError("O, dO, dQ must have the shape of Q")
    if dK.shape != K.shape or dV.shape != K.shape:
        raise ValueError("dK, dV must have the shape of K")
    if len({t.dtype for t in (Q, K, V, O, dO, dQ, dK, dV)}) != 1:
        raise ValueError("all tensors but LSE must share one dtype")
    if tuple(LSE.shape) != (B, Nq, S) or LSE.dtype.itemsize != 4:
        raise ValueError("LSE must be fp32 [B, Nq, S]")
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(dQ),
                             _ptr(dK), _ptr(dV), B, Nq, Nkv, S, Dh, int(causal), int(window),
                             float(scale), _ptr(workspace), ws_bytes, _dtype_code(Q),
                             _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_backward")


def backward(q, k, v, O, LSE, dO, causal=True, window=0, scale=None):
    """Allocate dQ, dK, dV and the workspace with torch and run attn_backward."""
    import torch
    dQ, dK, dV = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, Nq, S, Dh = q.shape
    n = attn_backward_workspace_bytes(B, Nq, k.shape[1], S, Dh, _dtype_code(q))
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    attn_backward(q, k, v, O, dO, LSE, dQ, dK, dV, causal=int(causal), window=window, scale=scale,
                  workspace=ws)
    return dQ, dK, dV


def prefill(q, k, v, causal=True, window=0, scale=None):
    """Allocate O and LSE with torch and run attn_prefill on the current stream."""
    import torch
    O = torch.empty_like(q)
    LSE = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_prefill(q, k, v, O, LSE, causal=int(causal), window=window, scale=scale)
    return O, LSE


def prefill_cache(q, Kcache, Vcache, lens, window=0, scale=None):
    """Allocate O and LSE with torch and run attn_prefill_cache."""
    import torch
    O = torch.empty_like(q)
    LSE = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_prefill_cache(q, Kcache, Vcache, lens, O, LSE, window=window, scale=scale)
    return O, LSE


def decode(q, Kcache, Vcache, lens, window=0, scale=None):
    """Allocate O, LSE and the workspace with torch and run attn_decode (or, with a
    window or an explicit scale, attn_decode_window)."""
    import torch
    B, Nq, Dh = q.shape
    O = torch.empty_like(q)
    LSE = torch.empty((B, Nq), dtype=torch.float32, device=q.device)
    nbytes = attn_decode_window_workspace_bytes(B, Nq, Kcache.shape[1], Dh, Kcache.shape[2],
                                                window, _dtype_code(q))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device) if nbytes else None
    if window or scale is not None:
        attn_decode_window(q, Kcache, Vcache, lens, O, LSE, ws, window=window, scale=scale)
    else:
        attn_decode(q, Kcache, Vcache, lens, O, LSE, ws)
    return O, LSE
