"""ctypes binding of libcca.so (argument marshalling only).

Every computation runs in the HIP library; this module checks tensor shapes,
dtypes and devices (the C ABI receives raw pointers and cannot), allocates
outputs with torch when the caller does not pass them, and forwards the
current torch stream.  If the library is missing it raises; there is no
fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcca.so")

CCA_F32, CCA_BF16, CCA_F16 = 0, 1, 2
_DT = {torch.float32: CCA_F32, torch.bfloat16: CCA_BF16, torch.float16: CCA_F16}
_TORCH_DT = {CCA_F32: torch.float32, CCA_BF16: torch.bfloat16, CCA_F16: torch.float16}

_lib = None


class CCAError(RuntimeError):
    pass


class CacheDesc(ctypes.Structure):
    """Mirror of cca_cache_t (include/cca.h)."""

    _fields_ = [
        ("core_k", ctypes.c_void_p),
        ("core_v", ctypes.c_void_p),
        ("ring_k", ctypes.c_void_p),
        ("ring_v", ctypes.c_void_p),
        ("B", ctypes.c_int),
        ("H", ctypes.c_int),
        ("d", ctypes.c_int),
        ("g", ctypes.c_int),
        ("k_local", ctypes.c_int),
        ("dt", ctypes.c_int),
        ("max_groups", ctypes.c_int64),
        ("n_tokens", ctypes.c_int64),
        ("n_pooled", ctypes.c_int64),
    ]


EXPORTS = {
    # name: (restype, argtypes)
    "cca_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "cca_pool_kv": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                                          ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "cca_prefill": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                                          ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                                          ctypes.c_int, ctypes.c_void_p]),
    "cca_attention": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                                            ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                                            ctypes.c_int, ctypes.c_void_p]),
    "cca_pool_kv_gqa": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                              ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                              ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "cca_prefill_gqa": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                              ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                              ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                                              ctypes.c_int, ctypes.c_void_p]),
    "cca_attention_gqa": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                                ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                                ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                                                ctypes.c_int, ctypes.c_void_p]),
    "cca_prefill_lse": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                              ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                                              ctypes.c_void_p]),
    "cca_backward_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                                       ctypes.c_int]),
    "cca_backward": (ctypes.c_int, [ctypes.c_void_p] * 12 + [ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                                             ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                             ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "cca_prefill_lse_gqa": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                                  ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                                  ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                                                  ctypes.c_int, ctypes.c_void_p]),
    "cca_backward_gqa_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                                           ctypes.c_int, ctypes.c_int]),
    "cca_backward_gqa": (ctypes.c_int, [ctypes.c_void_p] * 12 + [ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                                                 ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                                                 ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                                                 ctypes.c_int, ctypes.c_void_p]),
    "cca_pool_kv_lca": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                              ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "cca_prefill_lca": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                                              ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                              ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                                              ctypes.c_void_p]),
    "cca_pool_kv_lca_gqa": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                                  ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                                  ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                                                  ctypes.c_void_p]),
    "cca_prefill_lca_gqa": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                                  ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                                  ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "cca_cache_load_prefill_lca": (ctypes.c_int, [ctypes.POINTER(CacheDesc)] + [ctypes.c_void_p] * 6 +
                                   [ctypes.c_int64, ctypes.c_void_p]),
    "cca_cache_append_decode_lca": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p, ctypes.c_int] +
                                    [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                                             ctypes.c_float, ctypes.c_void_p]),
    "cca_cache_ring_slots": (ctypes.c_int64, [ctypes.POINTER(CacheDesc)]),
    "cca_cache_load_prefill": (ctypes.c_int, [ctypes.POINTER(CacheDesc)] + [ctypes.c_void_p] * 4
                               + [ctypes.c_int64, ctypes.c_void_p]),
    "cca_cache_append": (ctypes.c_int, [ctypes.POINTER(CacheDesc)] + [ctypes.c_void_p] * 3
                         + [ctypes.c_float, ctypes.c_void_p]),
    "cca_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(CacheDesc)]),
    "cca_decode_step": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p]),
    "cca_cache_append_decode": (ctypes.c_int, [ctypes.POINTER(CacheDesc)] + [ctypes.c_void_p] * 4
                                + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p]),
    "cca_cache_append_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(CacheDesc)] + [ctypes.c_void_p] * 4
                                        + [ctypes.c_int, ctypes.c_float, ctypes.c_void_p]),
    "cca_serve_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(CacheDesc), ctypes.c_int]),
    "cca_cache_append_decode_varlen": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p, ctypes.c_int64,
                                                      ctypes.c_int] + [ctypes.c_void_p] * 4
                                       + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float,
                                          ctypes.c_void_p]),
    "cca_cache_append_decode_varlen_lca": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p, ctypes.c_int,
                                                          ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
                                           + [ctypes.c_void_p] * 4
                                           + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float,
                                              ctypes.c_void_p]),
    "cca_cache_load_prefill_lca_gqa": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p, ctypes.c_int]
                                       + [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_void_p]),
    "cca_cache_extend_lca": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
                             + [ctypes.c_void_p] * 4
                             + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p]),
    "cca_extend_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(CacheDesc), ctypes.c_int]),
    "cca_cache_extend": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_int] + [ctypes.c_void_p] * 4
                         + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p]),
    "cca_kv_cache_bytes": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int64)]),
}


def load_library(path: str = LIB_PATH):
    """Load libcca.so (once).  Raises CCAError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise CCAError(f"{path} not found: build it with `python -m long_context_sparse_cca_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        msg = _lib.cca_status_string(status).decode()
        raise CCAError(f"{what}: {msg} (status {status})")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, shape, dtype, name: str):
    if not isinstance(t, torch.Tensor):
        raise CCAError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise CCAError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise CCAError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise CCAError(f"{name} must be a contiguous device tensor")


def _dtype_code(dtype) -> int:
    if dtype not in _DT:
        raise CCAError(f"unsupported dtype {dtype}")
    return _DT[dtype]


def _core_buffer(B, H, m, d, like):
    # a zero-length result still needs a real (non-null, aligned) base address
    return torch.empty((B, H, max(m, 1), d), dtype=like.dtype, device=like.device)[:, :, :m]


def _heads(q, k, v):
    """(B, H, H_kv, L, d) of q [B,H,L,d] and k, v [B,H_kv,L,d] (H a multiple of H_kv)."""
    B, H, L, d = q.shape
    if k.dim() != 4:
        raise CCAError("k must be [B, H_kv, L, d]")
    Hkv = k.shape[1]
    if Hkv < 1 or H % Hkv != 0:
        raise CCAError(f"query heads {H} must be a multiple of key/value heads {Hkv}")
    _need(q, (B, H, L, d), q.dtype, "q")
    _need(k, (B, Hkv, L, d), q.dtype, "k")
    _need(v, (B, Hkv, L, d), q.dtype, "v")
    return B, H, Hkv, L, d


def pool_kv(q, k, v, g: int, scale: float | None = None, kc=None, vc=None):
    """Core keys/values [B,H_kv,L//g,d] of q [B,H,L,d], k, v [B,H_kv,L,d].

    cca_pool_kv when H == H_kv, else cca_pool_kv_gqa (each key/value head
    pooled once with the mean of its query heads' last-token queries).
    """
    lib = load_library()
    B, H, Hkv, L, d = _heads(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    m = L // g if g >= 1 else 0
    if kc is None:
        kc = _core_buffer(B, Hkv, m, d, q)
    if vc is None:
        vc = _core_buffer(B, Hkv, m, d, q)
    _need(kc, (B, Hkv, m, d), q.dtype, "kc")
    _need(vc, (B, Hkv, m, d), q.dtype, "vc")
    if Hkv == H:
        st = lib.cca_pool_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), B, H, L, d, g, scale,
                             _dtype_code(q.dtype), _stream())
    else:
        st = lib.cca_pool_kv_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), B, H, Hkv, L, d, g, scale,
                                 _dtype_code(q.dtype), _stream())
    _check(st, "cca_pool_kv")
    return kc, vc


def prefill(q, k, v, g: int, k_local: int, scale: float | None = None, out_dtype=None, out=None,
            kc=None, vc=None, return_core: bool = False):
    """CCA prefill output [B,H,L,d] (pooling + fused attention): cca_prefill / cca_prefill_gqa."""
    lib = load_library()
    B, H, Hkv, L, d = _heads(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    m = L // g if g >= 1 else 0
    if kc is None:
        kc = _core_buffer(B, Hkv, m, d, q)
    if vc is None:
        vc = _core_buffer(B, Hkv, m, d, q)
    if out is None:
        out = torch.empty((B, H, L, d), dtype=out_dtype, device=q.device)
    _need(kc, (B, Hkv, m, d), q.dtype, "kc")
    _need(vc, (B, Hkv, m, d), q.dtype, "vc")
    _need(out, (B, H, L, d), out_dtype, "out")
    if Hkv == H:
        st = lib.cca_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(out), B, H, L, d, g, k_local,
                             scale, _dtype_code(q.dtype), _dtype_code(out_dtype), _stream())
    else:
        st = lib.cca_prefill_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(out), B, H, Hkv, L, d, g,
                                 k_local, scale, _dtype_code(q.dtype), _dtype_code(out_dtype), _stream())
    _check(st, "cca_prefill")
    if return_core:
        return out, kc, vc
    return out


def attention(q, k, v, kc, vc, g: int, k_local: int, scale: float | None = None, out_dtype=None, out=None):
    """Attention step only, given the pooled core tokens kc, vc: cca_attention / cca_attention_gqa."""
    lib = load_library()
    B, H, Hkv, L, d = _heads(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    m = L // g if g >= 1 else 0
    _need(kc, (B, Hkv, m, d), q.dtype, "kc")
    _need(vc, (B, Hkv, m, d), q.dtype, "vc")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, H, L, d), dtype=out_dtype, device=q.device)
    _need(out, (B, H, L, d), out_dtype, "out")
    if Hkv == H:
        st = lib.cca_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(out), B, H, L, d, g, k_local,
                               scale, _dtype_code(q.dtype), _dtype_code(out_dtype), _stream())
    else:
        st = lib.cca_attention_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(out), B, H, Hkv, L, d, g,
                                   k_local, scale, _dtype_code(q.dtype), _dtype_code(out_dtype), _stream())
    _check(st, "cca_attention")
    return out


def pool_kv_lca(q, k, v, g: int, d_rope: int, scale: float | None = None):
    """LCA-style condensed keys/values and anchors of q [B,H,L,d], k, v [B,H_kv,L,d]:
    (kc, vc [B,H_kv,L//g,d], anchors int32 [B,H_kv,L//g]); cca_pool_kv_lca_gqa."""
    lib = load_library()
    B, H, Hkv, L, d = _heads(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    m = L // g if g >= 1 else 0
    kc = _core_buffer(B, Hkv, m, d, q)
    vc = _core_buffer(B, Hkv, m, d, q)
    anchors = torch.empty((B, Hkv, max(m, 1)), dtype=torch.int32, device=q.device)[:, :, :m]
    _check(lib.cca_pool_kv_lca_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(anchors), B, H, Hkv, L, d, g,
                                   d_rope, scale, _dtype_code(q.dtype), _stream()), "cca_pool_kv_lca")
    return kc, vc, anchors


def prefill_lca(q, k, v, g: int, k_local: int, d_rope: int, scale: float | None = None, out_dtype=None):
    """LCA-style prefill of q [B,H,L,d], k, v [B,H_kv,L,d]: (out [B,H,L,d], kc, vc [B,H_kv,L//g,d],
    anchors int32 [B,H_kv,L//g]); cca_prefill_lca_gqa."""
    lib = load_library()
    B, H, Hkv, L, d = _heads(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    m = L // g if g >= 1 else 0
    kc = _core_buffer(B, Hkv, m, d, q)
    vc = _core_buffer(B, Hkv, m, d, q)
    anchors = torch.empty((B, Hkv, max(m, 1)), dtype=torch.int32, device=q.device)[:, :, :m]
    out = torch.empty((B, H, L, d), dtype=out_dtype, device=q.device)
    _check(lib.cca_prefill_lca_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(out), _ptr(anchors), B, H, Hkv,
                                   L, d, g, k_local, d_rope, scale, _dtype_code(q.dtype), _dtype_code(out_dtype),
                                   _stream()), "cca_prefill_lca")
    return out, kc, vc, anchors


def prefill_lse(q, k, v, g: int, k_local: int, scale: float | None = None, out_dtype=None):
    """Forward for training: (out [B,H,L,d], lse [B,H,L] float32, kc, vc [B,H_kv,L//g,d]).

    q [B,H,L,d], k, v [B,H_kv,L,d]: cca_prefill_lse, or cca_prefill_lse_gqa when H_kv < H.
    """
    lib = load_library()
    B, H, Hkv, L, d = _heads(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    m = L // g if g >= 1 else 0
    kc = _core_buffer(B, Hkv, m, d, q)
    vc = _core_buffer(B, Hkv, m, d, q)
    out = torch.empty((B, H, L, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, max(L, 1)), dtype=torch.float32, device=q.device)[:, :, :L]
    if Hkv == H:
        st = lib.cca_prefill_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(out), _ptr(lse), B, H, L, d, g,
                                 k_local, scale, _dtype_code(q.dtype), _dtype_code(out_dtype), _stream())
    else:
        st = lib.cca_prefill_lse_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(out), _ptr(lse), B, H, Hkv,
                                     L, d, g, k_local, scale, _dtype_code(q.dtype), _dtype_code(out_dtype),
                                     _stream())
    _check(st, "cca_prefill_lse")
    return out, lse, kc, vc


def backward(q, k, v, kc, vc, out, lse, dout, g: int, k_local: int, scale: float | None = None):
    """Gradients of sum(out * dout): dq float32 [B,H,L,d], dk, dv float32 [B,H_kv,L,d].

    cca_backward, or cca_backward_gqa when k, v have fewer heads than q.
    """
    lib = load_library()
    B, H, Hkv, L, d = _heads(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    m = L // g if g >= 1 else 0
    _need(kc, (B, Hkv, m, d), q.dtype, "kc")
    _need(vc, (B, Hkv, m, d), q.dtype, "vc")
    _need(out, (B, H, L, d), q.dtype, "out")
    _need(dout, (B, H, L, d), q.dtype, "dout")
    if tuple(lse.shape) != (B, H, L) or lse.dtype != torch.float32 or not lse.is_cuda:
        raise CCAError("lse must be a float32 device tensor [B, H, L]")
    dq = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    dk, dv = (torch.empty((B, Hkv, L, d), dtype=torch.float32, device=q.device) for _ in range(2))
    ws_bytes = lib.cca_backward_gqa_workspace_bytes(B, H, Hkv, L, d, g)
    ws = torch.empty((max(ws_bytes, 16) + 15) // 16 * 4, dtype=torch.float32, device=q.device)
    if Hkv == H:
        st = lib.cca_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(out), _ptr(lse), _ptr(dout),
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel() * 4, B, H, L, d, g, k_local, scale,
                              _dtype_code(q.dtype), _stream())
    else:
        st = lib.cca_backward_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(out), _ptr(lse), _ptr(dout),
                                  _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel() * 4, B, H, Hkv, L, d, g,
                                  k_local, scale, _dtype_code(q.dtype), _stream())
    _check(st, "cca_backward")
    return dq, dk, dv


class CCAAttention(torch.autograd.Function):
    """CCA prefill attention as an autograd function (bf16, binary16 or float32, d = 64 or 128; k, v may
    have fewer heads than q): forward cca_prefill_lse, backward cca_backward.
    apply(q, k, v, g, k_local, scale=None) -> out [B,H,L,d]."""

    @staticmethod
    def forward(ctx, q, k, v, g, k_local, scale=None):
        out, lse, kc, vc = prefill_lse(q, k, v, g, k_local, scale)
        ctx.save_for_backward(q, k, v, kc, vc, out, lse)
        ctx.cfg = (g, k_local, scale)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, kc, vc, out, lse = ctx.saved_tensors
        g, k_local, scale = ctx.cfg
        dq, dk, dv = backward(q, k, v, kc, vc, out, lse, dout.to(q.dtype).contiguous(), g, k_local, scale)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None, None


class KVCache:
    """Compressed CCA KV cache: core-token array + raw ring (tensors owned here)."""

    def __init__(self, B: int, H: int, d: int, g: int, k_local: int, max_tokens: int, dtype=torch.bfloat16,
                 device="cuda"):
        lib = load_library()
        self.max_groups = max(1, max_tokens // g)
        self.R = (k_local + 1) * g
        self.dtype = dtype
        self.core_k = torch.zeros((B, H, self.max_groups, d), dtype=dtype, device=device)
        self.core_v = torch.zeros_like(self.core_k)
        self.ring_k = torch.zeros((B, H, self.R, d), dtype=dtype, device=device)
        self.ring_v = torch.zeros_like(self.ring_k)
        self.desc = CacheDesc(_ptr(self.core_k), _ptr(self.core_v), _ptr(self.ring_k), _ptr(self.ring_v),
                              B, H, d, g, k_local, _dtype_code(dtype), self.max_groups, 0, 0)
        ws_bytes = lib.cca_decode_workspace_bytes(ctypes.byref(self.desc))
        self.workspace = torch.empty((ws_bytes + 15) // 16 * 4, dtype=torch.float32, device=device)
        self.ws_bytes = ws_bytes

    @property
    def n_tokens(self) -> int:
        return int(self.desc.n_tokens)

    @property
    def shape_bhd(self):
        return (self.desc.B, self.desc.H, self.desc.d)

    def load_prefill(self, k, v, kc, vc):
        """Seed the empty cache with the state after a prefill of L = k.shape[2] tokens."""
        B, H, d = self.shape_bhd
        L = k.shape[2]
        m = L // self.desc.g
        _need(k, (B, H, L, d), self.dtype, "k")
        _need(v, (B, H, L, d), self.dtype, "v")
        _need(kc, (B, H, m, d), self.dtype, "kc")
        _need(vc, (B, H, m, d), self.dtype, "vc")
        _check(_lib.cca_cache_load_prefill(ctypes.byref(self.desc), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), L,
                                           _stream()), "cca_cache_load_prefill")

    def append(self, q, k, v, scale: float | None = None):
        """Append one token per sequence (q, k, v: [B,H,d])."""
        B, H, d = self.shape_bhd
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        for name, t in (("q", q), ("k", k), ("v", v)):
            _need(t, (B, H, d), self.dtype, name)
        _check(_lib.cca_cache_append(ctypes.byref(self.desc), _ptr(q), _ptr(k), _ptr(v), scale, _stream()),
               "cca_cache_append")

    def append_decode(self, q, k, v, out_dtype=None, out=None, scale: float | None = None):
        """Append one token and return its attention output [B,H,d] (one launch)."""
        B, H, d = self.shape_bhd
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        out_dtype = self.dtype if out_dtype is None else out_dtype
        for name, t in (("q", q), ("k", k), ("v", v)):
            _need(t, (B, H, d), self.dtype, name)
        if out is None:
            out = torch.empty((B, H, d), dtype=out_dtype, device=q.device)
        _need(out, (B, H, d), out_dtype, "out")
        _check(_lib.cca_cache_append_decode(ctypes.byref(self.desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                            _dtype_code(out_dtype), _ptr(self.workspace), self.ws_bytes, scale,
                                            _stream()), "cca_cache_append_decode")
        return out

    def append_decode_noalloc(self, q, k, v, out, out_dtype=None, scale: float | None = None):
        """append_decode with the chunk partial states in the library's own per-GPU device
        array instead of this cache's workspace (cca_cache_append_decode_noalloc); `out`
        is caller-provided, so the call allocates nothing."""
        B, H, d = self.shape_bhd
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        out_dtype = self.dtype if out_dtype is None else out_dtype
        for name, t in (("q", q), ("k", k), ("v", v)):
            _need(t, (B, H, d), self.dtype, name)
        _need(out, (B, H, d), out_dtype, "out")
        _check(_lib.cca_cache_append_decode_noalloc(ctypes.byref(self.desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                                    _dtype_code(out_dtype), scale, _stream()),
               "cca_cache_append_decode_noalloc")
        return out

    def decode(self, q, out_dtype=None, out=None, scale: float | None = None):
        """Attention output [B,H,d] of the newest token (q: its query)."""
        B, H, d = self.shape_bhd
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        out_dtype = self.dtype if out_dtype is None else out_dtype
        _need(q, (B, H, d), self.dtype, "q")
        if out is None:
            out = torch.empty((B, H, d), dtype=out_dtype, device=q.device)
        _need(out, (B, H, d), out_dtype, "out")
        _check(_lib.cca_decode_step(ctypes.byref(self.desc), _ptr(q), _ptr(out), _dtype_code(out_dtype),
                                    _ptr(self.workspace), self.ws_bytes, scale, _stream()), "cca_decode_step")
        return out


class LCACache(KVCache):
    """LCA-style decode cache: condensed tokens (mean-query importance, positional dims from
    the top-scored token) plus the raw ring, and `qsum` (float32 [B,H,d]), the running sum
    of the current group's queries."""

    def __init__(self, B: int, H: int, d: int, g: int, k_local: int, max_tokens: int, d_rope: int,
                 dtype=torch.bfloat16, device="cuda"):
        super().__init__(B, H, d, g, k_local, max_tokens, dtype, device)
        self.d_rope = int(d_rope)
        self.qsum = torch.zeros((B, H, d), dtype=torch.float32, device=device)

    def load_prefill(self, q, k, v, kc, vc):
        """Seed the empty cache after an LCA-style prefill of L = k.shape[2] tokens (kc, vc from prefill_lca)."""
        B, H, d = self.shape_bhd
        L = k.shape[2]
        m = L // self.desc.g
        for name, t in (("q", q), ("k", k), ("v", v)):
            _need(t, (B, H, L, d), self.dtype, name)
        _need(kc, (B, H, m, d), self.dtype, "kc")
        _need(vc, (B, H, m, d), self.dtype, "vc")
        _check(_lib.cca_cache_load_prefill_lca(ctypes.byref(self.desc), _ptr(self.qsum), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(kc), _ptr(vc), L, _stream()), "cca_cache_load_prefill_lca")

    def append(self, q, k, v, scale: float | None = None):
        raise CCAError("an LCA-style cache appends with append_decode")

    def append_decode(self, q, k, v, out_dtype=None, out=None, scale: float | None = None):
        """Append one token (condensing a completed group) and return its attention output [B,H,d]."""
        B, H, d = self.shape_bhd
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        out_dtype = self.dtype if out_dtype is None else out_dtype
        for name, t in (("q", q), ("k", k), ("v", v)):
            _need(t, (B, H, d), self.dtype, name)
        if out is None:
            out = torch.empty((B, H, d), dtype=out_dtype, device=q.device)
        _need(out, (B, H, d), out_dtype, "out")
        _check(_lib.cca_cache_append_decode_lca(ctypes.byref(self.desc), _ptr(self.qsum), self.d_rope, _ptr(q), _ptr(k),
                                                _ptr(v), _ptr(out), _dtype_code(out_dtype), _ptr(self.workspace),
                                                self.ws_bytes, scale, _stream()), "cca_cache_append_decode_lca")
        return out


class ServeCache(KVCache):
    """Compressed cache for serving: per-sequence lengths on the device, grouped-query heads.

    H_kv key/value heads are cached; steps take H_q = r * H_kv query heads.
    `lens` (int32 [B], device) holds each sequence's token count; `step`
    appends one token to every sequence (the library advances `lens` by one).
    """

    def __init__(self, B: int, H_q: int, H_kv: int, d: int, g: int, k_local: int, max_tokens: int,
                 dtype=torch.bfloat16, device="cuda"):
        super().__init__(B, H_kv, d, g, k_local, max_tokens, dtype, device)
        if H_q % H_kv != 0:
            raise CCAError("H_q must be a multiple of H_kv")
        self.H_q = H_q
        self.lens = torch.zeros((B,), dtype=torch.int32, device=device)
        self.lens_host = [0] * B
        ws_bytes = _lib.cca_serve_workspace_bytes(ctypes.byref(self.desc), H_q)
        self.serve_ws = torch.empty((ws_bytes + 15) // 16 * 4, dtype=torch.float32, device=device)
        self.serve_ws_bytes = ws_bytes
        self._ext_ws = None   # staging workspace of `extend`, sized on first use

    def _seq_desc(self, b: int):
        B, H, d = self.shape_bhd
        esz = self.core_k.element_size()
        per_core = H * self.max_groups * d * esz
        per_ring = H * self.R * d * esz
        return CacheDesc(self.desc.core_k + b * per_core, self.desc.core_v + b * per_core,
                         self.desc.ring_k + b * per_ring, self.desc.ring_v + b * per_ring,
                         1, H, d, self.desc.g, self.desc.k_local, self.desc.dt, self.max_groups, 0, 0)

    def load_sequence(self, b: int, k, v, kc, vc):
        """Seed sequence b (empty) with the state after a prefill of L_b = k.shape[2] tokens.

        k, v: [1, H_kv, L_b, d]; kc, vc: [1, H_kv, L_b // g, d] (from `prefill(..., return_core=True)`).
        Uses cca_cache_load_prefill on a one-sequence view of the cache.
        """
        _, H, d = self.shape_bhd
        L = k.shape[2]
        m = L // self.desc.g
        _need(k, (1, H, L, d), self.dtype, "k")
        _need(v, (1, H, L, d), self.dtype, "v")
        _need(kc, (1, H, m, d), self.dtype, "kc")
        _need(vc, (1, H, m, d), self.dtype, "vc")
        if self.lens_host[b] != 0:
            raise CCAError(f"sequence {b} is not empty")
        desc = self._seq_desc(b)
        _check(_lib.cca_cache_load_prefill(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), L, _stream()),
               "cca_cache_load_prefill")
        self.lens_host[b] = L
        self.lens[b] = L

    def _step_call(self, q, k, v, out, out_dtype, max_len, scale):
        _check(_lib.cca_cache_append_decode_varlen(ctypes.byref(self.desc), _ptr(self.lens), max_len, self.H_q,
                                                   _ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(out_dtype),
                                                   _ptr(self.serve_ws), self.serve_ws_bytes, scale, _stream()),
               "cca_cache_append_decode_varlen")

    def step(self, q, k, v, out_dtype=None, out=None, scale: float | None = None, max_len: int | None = None):
        """Append one token to every sequence and return its outputs [B, H_q, d].

        q: [B, H_q, d]; k, v: [B, H_kv, d].  cca_cache_append_decode_varlen (which also advances `lens`).
        `max_len` (default: the longest sequence) bounds every length (capacity check, streaming loads).
        """
        B, H, d = self.shape_bhd
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        out_dtype = self.dtype if out_dtype is None else out_dtype
        _need(q, (B, self.H_q, d), self.dtype, "q")
        _need(k, (B, H, d), self.dtype, "k")
        _need(v, (B, H, d), self.dtype, "v")
        if out is None:
            out = torch.empty((B, self.H_q, d), dtype=out_dtype, device=q.device)
        _need(out, (B, self.H_q, d), out_dtype, "out")
        bound = max(self.lens_host)
        max_len = bound if max_len is None else int(max_len)
        if max_len < bound:
            raise CCAError("max_len is below a sequence length")
        self._step_call(q, k, v, out, out_dtype, max_len, scale)
        self.lens_host = [x + 1 for x in self.lens_host]   # the call advanced `lens` on the device
        return out

    def graph(self, max_len: int, out_dtype=None, scale: float | None = None):
        """A serving step captured in a HIP graph (see ServeGraph)."""
        return ServeGraph(self, max_len, out_dtype, scale)

    def _extend_call(self, m, qs, ks, vs, os_, out_dtype, scale):
        _check(_lib.cca_cache_extend(ctypes.byref(self.desc), _ptr(self.lens), max(self.lens_host), self.H_q, m,
                                     _ptr(qs), _ptr(ks), _ptr(vs), _ptr(os_), _dtype_code(out_dtype),
                                     _ptr(self._ext_ws), self._ext_ws.numel() * 4, scale, _stream()),
               "cca_cache_extend")

    def extend(self, q, k, v, out_dtype=None, scale: float | None = None):
        """Append n tokens to every sequence and return their outputs [B, H_q, n, d].

        q: [B, H_q, n, d]; k, v: [B, H_kv, n, d].  Chunks longer than k_local*g + 1 (rounded
        down to a multiple of 256 when that is at least 256) are split into consecutive
        cca_cache_extend calls (each advances `lens`).
        """
        B, H, d = self.shape_bhd
        n = q.shape[2]
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        out_dtype = self.dtype if out_dtype is None else out_dtype
        _need(q, (B, self.H_q, n, d), self.dtype, "q")
        _need(k, (B, H, n, d), self.dtype, "k")
        _need(v, (B, H, n, d), self.dtype, "v")
        out = torch.empty((B, self.H_q, n, d), dtype=out_dtype, device=q.device)
        # at most k*g+1 tokens per call; above 256, whole 256-query tiles of the attention kernel
        piece = self.desc.k_local * self.desc.g + 1
        if piece >= 256:
            piece -= piece % 256
        for a in range(0, n, piece):
            e = min(n, a + piece)
            m = e - a
            qs, ks, vs = (x[:, :, a:e].contiguous() for x in (q, k, v))
            os_ = out if m == n else torch.empty((B, self.H_q, m, d), dtype=out_dtype, device=q.device)
            ws_bytes = _lib.cca_extend_workspace_bytes(ctypes.byref(self.desc), m)
            if self._ext_ws is None or self._ext_ws.numel() * 4 < ws_bytes:
                self._ext_ws = torch.empty(((ws_bytes + 15) // 16) * 4, dtype=torch.float32, device=q.device)
            self._extend_call(m, qs, ks, vs, os_, out_dtype, scale)
            self.lens_host = [x + m for x in self.lens_host]   # the call advanced `lens` on the device
            if m != n:
                out[:, :, a:e] = os_
        return out


class LCAServeCache(ServeCache):
    """Serving cache with the LCA-style condensation: per-sequence lengths, grouped-query heads,
    groups condensed with the mean of their queries over positions and the query heads that
    share a key/value head, positional dims (the last d_rope) from the top-scored token.
    `qsum` (float32 [B, H_kv, d]) holds each sequence's running sum of its current group's
    queries.  `step` and `extend` (cca_cache_append_decode_varlen_lca, cca_cache_extend_lca)
    work as for ServeCache."""

    def __init__(self, B: int, H_q: int, H_kv: int, d: int, g: int, k_local: int, max_tokens: int, d_rope: int,
                 dtype=torch.bfloat16, device="cuda"):
        super().__init__(B, H_q, H_kv, d, g, k_local, max_tokens, dtype, device)
        self.d_rope = int(d_rope)
        self.qsum = torch.zeros((B, H_kv, d), dtype=torch.float32, device=device)

    def load_sequence(self, b: int, q, k, v, kc, vc):
        """Seed sequence b (empty) after an LCA-style prefill of L_b = k.shape[2] tokens.

        q: [1, H_q, L_b, d]; k, v: [1, H_kv, L_b, d]; kc, vc: [1, H_kv, L_b // g, d] (from
        `prefill_lca`).  cca_cache_load_prefill_lca_gqa on a one-sequence view of the cache.
        """
        _, H, d = self.shape_bhd
        L = k.shape[2]
        m = L // self.desc.g
        _need(q, (1, self.H_q, L, d), self.dtype, "q")
        _need(k, (1, H, L, d), self.dtype, "k")
        _need(v, (1, H, L, d), self.dtype, "v")
        _need(kc, (1, H, m, d), self.dtype, "kc")
        _need(vc, (1, H, m, d), self.dtype, "vc")
        if self.lens_host[b] != 0:
            raise CCAError(f"sequence {b} is not empty")
        desc = self._seq_desc(b)
        qsum_b = self.qsum[b]
        _check(_lib.cca_cache_load_prefill_lca_gqa(ctypes.byref(desc), _ptr(qsum_b), self.H_q, _ptr(q), _ptr(k),
                                                   _ptr(v), _ptr(kc), _ptr(vc), L, _stream()),
               "cca_cache_load_prefill_lca_gqa")
        self.lens_host[b] = L
        self.lens[b] = L

    def _step_call(self, q, k, v, out, out_dtype, max_len, scale):
        _check(_lib.cca_cache_append_decode_varlen_lca(ctypes.byref(self.desc), _ptr(self.qsum), self.d_rope,
                                                       _ptr(self.lens), max_len, self.H_q, _ptr(q), _ptr(k), _ptr(v),
                                                       _ptr(out), _dtype_code(out_dtype), _ptr(self.serve_ws),
                                                       self.serve_ws_bytes, scale, _stream()),
               "cca_cache_append_decode_varlen_lca")

    def _extend_call(self, m, qs, ks, vs, os_, out_dtype, scale):
        _check(_lib.cca_cache_extend_lca(ctypes.byref(self.desc), _ptr(self.qsum), self.d_rope, _ptr(self.lens),
                                         max(self.lens_host), self.H_q, m, _ptr(qs), _ptr(ks), _ptr(vs), _ptr(os_),
                                         _dtype_code(out_dtype), _ptr(self._ext_ws), self._ext_ws.numel() * 4, scale,
                                         _stream()),
               "cca_cache_extend_lca")


class ServeGraph:
    """One serving decode step of a ServeCache (or LCAServeCache) captured in a HIP graph.

    The step keeps every length on the device and allocates nothing, so it can be captured
    once and replayed per token.  The capture fixes the host-side length bound `max_len`:
    every replay must leave each sequence at most that long.  A sequence that has outgrown
    it gets NaN outputs and is not advanced, as in the plain call.  Write the token's q, k, v
    into `self.q`, `self.k`, `self.v` (or pass them to `step`), replay, and read `self.out`.
    """

    def __init__(self, cache: ServeCache, max_len: int, out_dtype=None, scale: float | None = None):
        B, H, d = cache.shape_bhd
        if max(cache.lens_host) > max_len:
            raise CCAError("max_len is below a sequence length")
        self.cache = cache
        self.max_len = int(max_len)
        self.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        self.out_dtype = cache.dtype if out_dtype is None else out_dtype
        dev = cache.core_k.device
        self.q = torch.zeros((B, cache.H_q, d), dtype=cache.dtype, device=dev)
        self.k = torch.zeros((B, H, d), dtype=cache.dtype, device=dev)
        self.v = torch.zeros((B, H, d), dtype=cache.dtype, device=dev)
        self.out = torch.empty((B, cache.H_q, d), dtype=self.out_dtype, device=dev)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            # capture only: nothing runs, so the cache and the lengths are untouched here
            cache._step_call(self.q, self.k, self.v, self.out, self.out_dtype, self.max_len, self.scale)

    def step(self, q=None, k=None, v=None):
        """Copy the token's inputs in (if given), replay the step and return `self.out`."""
        for dst, src in ((self.q, q), (self.k, k), (self.v, v)):
            if src is not None:
                dst.copy_(src)
        self.graph.replay()
        self.cache.lens_host = [x + 1 if x <= self.max_len else x for x in self.cache.lens_host]
        return self.out


def cache_append(cache: KVCache, q, k, v, scale=None):
    cache.append(q, k, v, scale)


def decode_step(cache: KVCache, q, out_dtype=None, out=None, scale=None):
    return cache.decode(q, out_dtype, out, scale)


def kv_cache_bytes(n_tokens: int, g: int, k_local: int, B: int, H: int, d: int, dtype=torch.bfloat16):
    """(resident compressed bytes, full KV bytes): cca_kv_cache_bytes (host arithmetic)."""
    lib = load_library()
    res = ctypes.c_int64()
    full = ctypes.c_int64()
    _check(lib.cca_kv_cache_bytes(n_tokens, g, k_local, B, H, d, _dtype_code(dtype), ctypes.byref(res),
                                  ctypes.byref(full)), "cca_kv_cache_bytes")
    return res.value, full.value
