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
    attn_decode_noalloc(q, Kcache, Vcache, lens, O, LSE=None, stream=None)
    attn_decode_workspace_bytes(B, Nq, Nkv, Dh, Tcap, dtype)
    attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, window, dtype)
    attn_kv_append(Knew, Vnew, Kcache, Vcache, pos, rolling=0, stream=None)
    attn_decode_append(q, knew, vnew, Kcache, Vcache, lens, slot, O, LSE=None, workspace=None,
                       window=0, scale=None, stream=None)
    attn_backward(Q, K, V, O, dO, LSE, dQ, dK, dV, causal=1, window=0, scale=None,
                  workspace=None, stream=None)
    attn_backward_padded(Q, K, V, key_bits, O, dO, LSE, dQ, dK, dV, causal=1, window=0,
                         scale=None, workspace=None, stream=None)
    attn_backward_workspace_bytes(B, Nq, Nkv, S, Dh, dtype)
    attn_pack_key_mask(mask, key_bits, stream=None)
    attn_prefill_padded(Q, K, V, key_bits, O, LSE, causal=1, window=0, scale=None, stream=None)
    attn_prefill_cache_padded(Q, Kcache, Vcache, lens, key_bits, O, LSE, window=0, scale=None,
                              stream=None)
    attn_decode_padded(q, Kcache, Vcache, lens, key_bits, O, LSE=None, workspace=None,
                       window=0, scale=None, stream=None)
    attn_rope_cos_sin(table, base=10000.0, stream=None)
    attn_rope(X, Y, table, positions=None, start=None, style=0, stream=None)
    attn_kv_append_rope(Knew, Vnew, Kcache, Vcache, pos, table, positions=None, rolling=0,
                        style=0, stream=None)
    attn_prefill_rope(Q, K, V, O, LSE, table, key_bits=None, positions=None, start=None,
                      style=0, causal=1, window=0, scale=None, stream=None)
    attn_prefill_cache_rope(Q, Kcache, Vcache, lens, O, LSE, table, key_bits=None,
                            positions=None, start=None, style=0, window=0, scale=None, stream=None)
    attn_decode_rope(q, Kcache, Vcache, lens, O, LSE, table, workspace=None, key_bits=None,
                     positions=None, style=0, window=0, scale=None, stream=None)
    attn_strerror(status)
Key bits are held in int64 tensors [B, ceil(T / 64)] (the C ABI's uint64 words).
Conveniences that allocate outputs with torch:
    prefill(q, k, v, causal=True, window=0, scale=None, key_mask=None) -> (O, LSE)
    prefill_cache(q, Kcache, Vcache, lens, window=0, scale=None, key_mask=None) -> (O, LSE)
    decode(q, Kcache, Vcache, lens, window=0, scale=None, key_mask=None) -> (O, LSE)
    backward(q, k, v, O, LSE, dO, causal=True, window=0, scale=None) -> (dQ, dK, dV)
    pack_key_mask(mask) -> key_bits          (mask: bool or uint8 [B, T])
    rope_table(P, Dh, base=10000.0, device=None) -> table [P, Dh] fp32
    rope(x, table, positions=None, start=None, style="pairs", out=None) -> rotated x
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
ATTN_ESCRATCH = -6
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20
ATTN_BF16 = 0
ATTN_F32 = 1

EXPORTS = ("attn_prefill", "attn_prefill_cache", "attn_decode", "attn_decode_window",
           "attn_decode_workspace_bytes", "attn_decode_window_workspace_bytes",
           "attn_kv_append", "attn_decode_append", "attn_backward", "attn_backward_padded",
           "attn_backward_workspace_bytes",
           "attn_pack_key_mask", "attn_prefill_padded", "attn_prefill_cache_padded",
           "attn_decode_padded", "attn_rope_cos_sin", "attn_rope", "attn_kv_append_rope",
           "attn_decode_noalloc", "attn_prefill_rope", "attn_prefill_cache_rope",
           "attn_decode_rope", "attn_strerror")
ROPE_STYLES = {"pairs": 0, "half": 1}

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
        L.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32,
                                          vp]
        L.attn_decode_noalloc.restype = i32
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
        L.attn_backward_padded.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                           i32, i32, i32, i32, f32, vp, ctypes.c_size_t, i32, vp]
        L.attn_backward_padded.restype = i32
        L.attn_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                         i32, f32, vp, vp, ctypes.c_size_t, i32, vp]
        L.attn_decode_append.restype = i32
        L.attn_pack_key_mask.argtypes = [vp, i32, i32, vp, vp]
        L.attn_pack_key_mask.restype = i32
        L.attn_prefill_padded.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                          i32, f32, i32, vp]
        L.attn_prefill_padded.restype = i32
        L.attn_prefill_cache_padded.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                i32, i32, i32, f32, i32, vp]
        L.attn_prefill_cache_padded.restype = i32
        L.attn_decode_padded.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                         vp, vp, ctypes.c_size_t, i32, vp]
        L.attn_decode_padded.restype = i32
        L.attn_rope_cos_sin.argtypes = [vp, i32, i32, ctypes.c_double, vp]
        L.attn_rope_cos_sin.restype = i32
        L.attn_rope.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
        L.attn_rope.restype = i32
        L.attn_kv_append_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                          i32, i32, i32, vp]
        L.attn_kv_append_rope.restype = i32
        L.attn_prefill_rope.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                        f32, vp, i32, vp, vp, i32, i32, vp]
        L.attn_prefill_rope.restype = i32
        L.attn_prefill_cache_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                              i32, i32, f32, vp, i32, vp, vp, i32, i32, vp]
        L.attn_prefill_cache_rope.restype = i32
        L.attn_decode_rope.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                       vp, i32, vp, i32, vp, vp, ctypes.c_size_t, i32, vp]
        L.attn_decode_rope.restype = i32
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


def _check_bits(key_bits, B, T):
    import torch
    if key_bits is None:
        return
    if key_bits.dtype != torch.int64 or tuple(key_bits.shape) != (B, (T + 63) // 64):
        raise ValueError(f"key_bits must be int64 [B, ceil({T} / 64)]")


def _check_lse(LSE, shape):
    import torch
    if LSE is not None and (tuple(LSE.shape) != tuple(shape) or LSE.dtype != torch.float32):
        raise ValueError(f"LSE must be float32 {list(shape)}")


def _check_prefill(Q, K, V, O, LSE):
    B, Nq, S, Dh = Q.shape
    Nkv = K.shape[1]
    if tuple(K.shape) != (B, Nkv, S, Dh) or K.shape != V.shape or O.shape != Q.shape:
        raise ValueError("shape mismatch between Q, K, V, O")
    if not (Q.dtype == K.dtype == V.dtype == O.dtype):
        raise ValueError("Q, K, V, O must share one dtype")
    _check_lse(LSE, (B, Nq, S))
    return B, Nq, Nkv, S, Dh


def attn_prefill(Q, K, V, O, LSE, causal=1, window=0, scale=None, stream=None):
    """Q [B,Nq,S,Dh], K/V [B,Nkv,S,Dh], O like Q, LSE fp32 [B,Nq,S] or None."""
    B, Nq, Nkv, S, Dh = _check_prefill(Q, K, V, O, LSE)
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    st = lib().attn_prefill(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), B, Nq, Nkv, S, Dh,
                            int(causal), int(window), float(scale), _dtype_code(Q),
                            _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_prefill")


def attn_prefill_padded(Q, K, V, key_bits, O, LSE, causal=1, window=0, scale=None, stream=None):
    """attn_prefill with a key-padding mask: key_bits int64 [B, ceil(S/64)] on the GPU."""
    B, Nq, Nkv, S, Dh = _check_prefill(Q, K, V, O, LSE)
    _check_bits(key_bits, B, S)
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    st = lib().attn_prefill_padded(_ptr(Q), _ptr(K), _ptr(V), _ptr(key_bits), _ptr(O), _ptr(LSE),
                                   B, Nq, Nkv, S, Dh, int(causal), int(window), float(scale),
                                   _dtype_code(Q), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_prefill_padded")


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
    # the C ABI takes one element type (q's): the caches and O must have it too
    if not (q.dtype == Kcache.dtype == Vcache.dtype == O.dtype):
        raise ValueError("q, Kcache, Vcache and O must share one dtype")
    _check_lse(LSE, (B, Nq))
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


def attn_decode_noalloc(q, Kcache, Vcache, lens, O, LSE=None, stream=None):
    """attn_decode without a workspace: the library's fixed device scratch holds the
    partials (at most ATTN_NOALLOC_SCRATCH_BYTES; calls on one device must not overlap)."""
    B, Nq, Nkv, Dh, Tcap = _check_decode(q, Kcache, Vcache, lens, O, LSE)
    st = lib().attn_decode_noalloc(_ptr(q), _ptr(Kcache), _ptr(Vcache), _ptr(lens), _ptr(O), B,
                                   Nq, Nkv, Dh, Tcap, _ptr(LSE), _dtype_code(q), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_noalloc")


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


def attn_prefill_cache(Q, Kcache, Vcache, lens, O, LSE, window=0, scale=None, stream=None,
                       key_bits=None):
    """Q [B,Nq,Sq,Dh] against caches [B,Nkv,Tcap,Dh]; lens int32 [B] on the GPU.
    With key_bits (int64 [B, ceil(Tcap/64)]) it calls attn_prefill_cache_padded."""
    import torch
    B, Nq, Sq, Dh = Q.shape
    Nkv, Tcap = Kcache.shape[1], Kcache.shape[2]
    if tuple(Kcache.shape) != (B, Nkv, Tcap, Dh) or Kcache.shape != Vcache.shape:
        raise ValueError("cache shapes must be [B, Nkv, Tcap, Dh]")
    if O.shape != Q.shape or lens.dtype != torch.int32 or tuple(lens.shape) != (B,):
        raise ValueError("O must match Q; lens must be int32 [B]")
    if not (Q.dtype == Kcache.dtype == Vcache.dtype == O.dtype):
        raise ValueError("Q, caches and O must share one dtype")
    _check_lse(LSE, (B, Nq, Sq))
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    if key_bits is None:
        st = lib().attn_prefill_cache(_ptr(Q), _ptr(Kcache), _ptr(Vcache), _ptr(lens), _ptr(O),
                                      _ptr(LSE), B, Nq, Nkv, Sq, Dh, Tcap, int(window),
                                      float(scale), _dtype_code(Q), _stream(stream))
        if st != ATTN_OK:
            raise AttnError(st, "attn_prefill_cache")
        return
    _check_bits(key_bits, B, Tcap)
    st = lib().attn_prefill_cache_padded(_ptr(Q), _ptr(Kcache), _ptr(Vcache), _ptr(lens),
                                         _ptr(key_bits), _ptr(O), _ptr(LSE), B, Nq, Nkv, Sq, Dh,
                                         Tcap, int(window), float(scale), _dtype_code(Q),
                                         _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_prefill_cache_padded")


def attn_prefill_cache_padded(Q, Kcache, Vcache, lens, key_bits, O, LSE, window=0, scale=None,
                              stream=None):
    """attn_prefill_cache with a key-padding mask over the cache rows."""
    attn_prefill_cache(Q, Kcache, Vcache, lens, O, LSE, window=window, scale=scale,
                       stream=stream, key_bits=key_bits)


def attn_decode_padded(q, Kcache, Vcache, lens, key_bits, O, LSE=None, workspace=None, window=0,
                       scale=None, stream=None):
    """attn_decode_window with a key-padding mask over the cache rows (key_bits int64
    [B, ceil(Tcap/64)] on the GPU); same workspace as attn_decode_window."""
    B, Nq, Nkv, Dh, Tcap = _check_decode(q, Kcache, Vcache, lens, O, LSE)
    _check_bits(key_bits, B, Tcap)
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_decode_padded(_ptr(q), _ptr(Kcache), _ptr(Vcache), _ptr(lens),
                                  _ptr(key_bits), _ptr(O), B, Nq, Nkv, Dh, Tcap, int(window),
                                  float(scale), _ptr(LSE), _ptr(workspace), ws_bytes,
                                  _dtype_code(q), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_padded")


def attn_decode_append(q, knew, vnew, Kcache, Vcache, lens, slot, O, LSE=None, workspace=None,
                       window=0, scale=None, stream=None):
    """One decode step that writes knew / vnew ([B, Nkv, Dh]) to cache row slot[b]
    (int32 [B] on the GPU) and attends over lens[b] keys, in one launch."""
    import torch
    B, Nq, Nkv, Dh, Tcap = _check_decode(q, Kcache, Vcache, lens, O, LSE)
    if tuple(knew.shape) != (B, Nkv, Dh) or knew.shape != vnew.shape:
        raise ValueError("knew and vnew must be [B, Nkv, Dh]")
    if not (q.dtype == knew.dtype == vnew.dtype == Kcache.dtype == Vcache.dtype == O.dtype):
        raise ValueError("q, new rows, caches and O must share one dtype")
    if slot.dtype != torch.int32 or tuple(slot.shape) != (B,):
        raise ValueError("slot must be int32 [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_decode_append(_ptr(q), _ptr(knew), _ptr(vnew), _ptr(Kcache), _ptr(Vcache),
                                  _ptr(lens), _ptr(slot), _ptr(O), B, Nq, Nkv, Dh, Tcap,
                                  int(window), float(scale), _ptr(LSE), _ptr(workspace), ws_bytes,
                                  _dtype_code(q), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_append")


def _check_rope(table, Dh, positions, start, shape, style):
    import torch
    _check_table(table, Dh)
    if positions is not None and (positions.dtype != torch.int32
                                  or tuple(positions.shape) != tuple(shape)):
        raise ValueError(f"positions must be int32 {list(shape)}")
    if start is not None and (start.dtype != torch.int32 or tuple(start.shape) != (shape[0],)):
        raise ValueError("start must be int32 [B]")
    return _rope_style(style)


def attn_prefill_rope(Q, K, V, O, LSE, table, key_bits=None, positions=None, start=None, style=0,
                      causal=1, window=0, scale=None, stream=None):
    """attn_prefill with Q rotated at load (K already rotated): table [P, Dh] fp32,
    positions int32 [B, S] or start int32 [B] or neither (row i at position i)."""
    B, Nq, Nkv, S, Dh = _check_prefill(Q, K, V, O, LSE)
    _check_bits(key_bits, B, S)
    st_code = _check_rope(table, Dh, positions, start, (B, S), style)
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    st = lib().attn_prefill_rope(_ptr(Q), _ptr(K), _ptr(V), _ptr(key_bits), _ptr(O), _ptr(LSE), B,
                                 Nq, Nkv, S, Dh, int(causal), int(window), float(scale),
                                 _ptr(table), table.shape[0], _ptr(positions), _ptr(start), st_code,
                                 _dtype_code(Q), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_prefill_rope")


def attn_prefill_cache_rope(Q, Kcache, Vcache, lens, O, LSE, table, key_bits=None, positions=None,
                            start=None, style=0, window=0, scale=None, stream=None):
    """attn_prefill_cache with the chunk's queries rotated at load (row i of sequence b
    at positions[b, i], start[b] + i, or lens[b] - Sq + i)."""
    import torch
    B, Nq, Sq, Dh = Q.shape
    Nkv, Tcap = Kcache.shape[1], Kcache.shape[2]
    if tuple(Kcache.shape) != (B, Nkv, Tcap, Dh) or Kcache.shape != Vcache.shape:
        raise ValueError("cache shapes must be [B, Nkv, Tcap, Dh]")
    if O.shape != Q.shape or lens.dtype != torch.int32 or tuple(lens.shape) != (B,):
        raise ValueError("O must match Q; lens must be int32 [B]")
    if not (Q.dtype == Kcache.dtype == Vcache.dtype == O.dtype):
        raise ValueError("Q, caches and O must share one dtype")
    _check_lse(LSE, (B, Nq, Sq))
    _check_bits(key_bits, B, Tcap)
    st_code = _check_rope(table, Dh, positions, start, (B, Sq), style)
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    st = lib().attn_prefill_cache_rope(_ptr(Q), _ptr(Kcache), _ptr(Vcache), _ptr(lens),
                                       _ptr(key_bits), _ptr(O), _ptr(LSE), B, Nq, Nkv, Sq, Dh, Tcap,
                                       int(window), float(scale), _ptr(table), table.shape[0],
                                       _ptr(positions), _ptr(start), st_code, _dtype_code(Q),
                                       _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_prefill_cache_rope")


def attn_decode_rope(q, Kcache, Vcache, lens, O, LSE, table, workspace=None, key_bits=None,
                     positions=None, style=0, window=0, scale=None, stream=None):
    """attn_decode_window with q rotated at load (at positions[b], or lens[b] - 1)."""
    B, Nq, Nkv, Dh, Tcap = _check_decode(q, Kcache, Vcache, lens, O, LSE)
    _check_bits(key_bits, B, Tcap)
    st_code = _check_rope(table, Dh, positions, None, (B,), style)
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_decode_rope(_ptr(q), _ptr(Kcache), _ptr(Vcache), _ptr(lens), _ptr(key_bits),
                                _ptr(O), B, Nq, Nkv, Dh, Tcap, int(window), float(scale),
                                _ptr(table), table.shape[0], _ptr(positions), st_code, _ptr(LSE),
                                _ptr(workspace), ws_bytes, _dtype_code(q), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_rope")


def attn_pack_key_mask(mask, key_bits, stream=None):
    """mask bool or uint8 [B, T] (nonzero = real token) -> key_bits int64 [B, ceil(T/64)]."""
    import torch
    if mask.dtype not in (torch.bool, torch.uint8) or mask.dim() != 2:
        raise ValueError("mask must be bool or uint8 [B, T]")
    B, T = mask.shape
    _check_bits(key_bits, B, T)
    st = lib().attn_pack_key_mask(_ptr(mask), B, T, _ptr(key_bits), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_pack_key_mask")


def attn_rope_cos_sin(table, base=10000.0, stream=None):
    """Fill table fp32 [P, Dh]: cos(p theta_m) in column m, sin in column Dh/2 + m."""
    import torch
    if table.dtype != torch.float32 or table.dim() != 2:
        raise ValueError("table must be fp32 [P, Dh]")
    P, Dh = table.shape
    st = lib().attn_rope_cos_sin(_ptr(table), P, Dh, float(base), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_rope_cos_sin")


def _rope_style(style):
    return ROPE_STYLES[style] if isinstance(style, str) else int(style)


def _check_table(table, Dh):
    import torch
    if table.dtype != torch.float32 or table.dim() != 2 or table.shape[1] != Dh:
        raise ValueError(f"table must be fp32 [P, {Dh}]")


def attn_rope(X, Y, table, positions=None, start=None, style=0, stream=None):
    """Rotate X [B,H,S,Dh] into Y (may be X) at positions (int32 [B,S]) or start (int32 [B])."""
    import torch
    B, H, S, Dh = X.shape
    if Y.shape != X.shape or Y.dtype != X.dtype:
        raise ValueError("Y must match X")
    _check_table(table, Dh)
    if positions is not None and (positions.dtype != torch.int32 or tuple(positions.shape) != (B, S)):
        raise ValueError("positions must be int32 [B, S]")
    if start is not None and (start.dtype != torch.int32 or tuple(start.shape) != (B,)):
        raise ValueError("start must be int32 [B]")
    st = lib().attn_rope(_ptr(X), _ptr(Y), _ptr(positions), _ptr(start), _ptr(table),
                         table.shape[0], B, H, S, Dh, _rope_style(style), _dtype_code(X),
                         _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_rope")


def attn_kv_append_rope(Knew, Vnew, Kcache, Vcache, pos, table, positions=None, rolling=0,
                        style=0, stream=None):
    """attn_kv_append with the new keys rotated at positions (int32 [B,Snew]) or pos[b] + i."""
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
    if positions is not None and (positions.dtype != torch.int32
                                  or tuple(positions.shape) != (B, Snew)):
        raise ValueError("positions must be int32 [B, Snew]")
    _check_table(table, Dh)
    st = lib().attn_kv_append_rope(_ptr(Knew), _ptr(Vnew), _ptr(Kcache), _ptr(Vcache), _ptr(pos),
                                   _ptr(positions), _ptr(table), table.shape[0], B, Nkv, Snew,
                                   Dh, Tcap, int(rolling), _rope_style(style), _dtype_code(Knew),
                                   _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_kv_append_rope")


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


def _check_backward(Q, K, V, O, dO, LSE, dQ, dK, dV):
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
    if LSE is None:
        raise ValueError("LSE is required")
    _check_lse(LSE, (B, Nq, S))
    return B, Nq, Nkv, S, Dh


def attn_backward(Q, K, V, O, dO, LSE, dQ, dK, dV, causal=1, window=0, scale=None,
                  workspace=None, stream=None):
    """Gradients of attn_prefill; shapes as attn_prefill, dQ like Q, dK/dV like K."""
    B, Nq, Nkv, S, Dh = _check_backward(Q, K, V, O, dO, LSE, dQ, dK, dV)
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(dQ),
                             _ptr(dK), _ptr(dV), B, Nq, Nkv, S, Dh, int(causal), int(window),
                             float(scale), _ptr(workspace), ws_bytes, _dtype_code(Q),
                             _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_backward")


def attn_backward_padded(Q, K, V, key_bits, O, dO, LSE, dQ, dK, dV, causal=1, window=0,
                         scale=None, workspace=None, stream=None):
    """attn_backward for a forward pass with a key-padding mask: key_bits int64
    [B, ceil(S/64)] on the GPU, as attn_prefill_padded took."""
    B, Nq, Nkv, S, Dh = _check_backward(Q, K, V, O, dO, LSE, dQ, dK, dV)
    if key_bits is not None:
        _check_bits(key_bits, B, S)
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_backward_padded(_ptr(Q), _ptr(K), _ptr(V), _ptr(key_bits), _ptr(O), _ptr(dO),
                                    _ptr(LSE), _ptr(dQ), _ptr(dK), _ptr(dV), B, Nq, Nkv, S, Dh,
                                    int(causal), int(window), float(scale), _ptr(workspace),
                                    ws_bytes, _dtype_code(Q), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_backward_padded")


def backward(q, k, v, O, LSE, dO, causal=True, window=0, scale=None, key_mask=None):
    """Allocate dQ, dK, dV and the workspace with torch and run attn_backward (with a
    key_mask, bool / uint8 [B, S], attn_backward_padded)."""
    import torch
    dQ, dK, dV = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, Nq, S, Dh = q.shape
    n = attn_backward_workspace_bytes(B, Nq, k.shape[1], S, Dh, _dtype_code(q))
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    if key_mask is not None:
        attn_backward_padded(q, k, v, pack_key_mask(key_mask), O, dO, LSE, dQ, dK, dV,
                             causal=int(causal), window=window, scale=scale, workspace=ws)
    else:
        attn_backward(q, k, v, O, dO, LSE, dQ, dK, dV, causal=int(causal), window=window,
                      scale=scale, workspace=ws)
    return dQ, dK, dV


def pack_key_mask(mask):
    """Key bits (int64 [B, ceil(T/64)]) of a bool / uint8 mask [B, T] on the GPU."""
    import torch
    B, T = mask.shape
    bits = torch.empty((B, (T + 63) // 64), dtype=torch.int64, device=mask.device)
    attn_pack_key_mask(mask.contiguous(), bits)
    return bits


def rope_table(P, Dh, base=10000.0, device=None):
    """cos/sin table fp32 [P, Dh] for positions 0 .. P-1, built on the GPU."""
    import torch
    table = torch.empty((P, Dh), dtype=torch.float32, device=device or "cuda")
    attn_rope_cos_sin(table, base)
    return table


def rope(x, table, positions=None, start=None, style="pairs", out=None):
    """Rotated copy of x [B,H,S,Dh] (or rotate into `out`, which may be x itself)."""
    import torch
    y = torch.empty_like(x) if out is None else out
    attn_rope(x, y, table, positions=positions, start=start, style=style)
    return y


def prefill(q, k, v, causal=True, window=0, scale=None, key_mask=None):
    """Allocate O and LSE with torch and run attn_prefill (attn_prefill_padded with a
    key_mask, bool / uint8 [B, S]) on the current stream."""
    import torch
    O = torch.empty_like(q)
    LSE = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if key_mask is None:
        attn_prefill(q, k, v, O, LSE, causal=int(causal), window=window, scale=scale)
    else:
        attn_prefill_padded(q, k, v, pack_key_mask(key_mask), O, LSE, causal=int(causal),
                            window=window, scale=scale)
    return O, LSE


def prefill_cache(q, Kcache, Vcache, lens, window=0, scale=None, key_mask=None):
    """Allocate O and LSE with torch and run attn_prefill_cache (key_mask: bool / uint8
    [B, Tcap] over the cache rows, or None)."""
    import torch
    O = torch.empty_like(q)
    LSE = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    bits = None if key_mask is None else pack_key_mask(key_mask)
    attn_prefill_cache(q, Kcache, Vcache, lens, O, LSE, window=window, scale=scale,
                       key_bits=bits)
    return O, LSE


def decode(q, Kcache, Vcache, lens, window=0, scale=None, key_mask=None):
    """Allocate O, LSE and the workspace with torch and run attn_decode (or, with a
    window or an explicit scale, attn_decode_window; with a key_mask, bool / uint8
    [B, Tcap], attn_decode_padded)."""
    import torch
    B, Nq, Dh = q.shape
    O = torch.empty_like(q)
    LSE = torch.empty((B, Nq), dtype=torch.float32, device=q.device)
    nbytes = attn_decode_window_workspace_bytes(B, Nq, Kcache.shape[1], Dh, Kcache.shape[2],
                                                window, _dtype_code(q))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device) if nbytes else None
    if key_mask is not None:
        attn_decode_padded(q, Kcache, Vcache, lens, pack_key_mask(key_mask), O, LSE, ws,
                           window=window, scale=scale)
    elif window or scale is not None:
        attn_decode_window(q, Kcache, Vcache, lens, O, LSE, ws, window=window, scale=scale)
    else:
        attn_decode(q, Kcache, Vcache, lens, O, LSE, ws)
    return O, LSE
