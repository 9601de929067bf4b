"""Thin ctypes binding over libswa.so (include/swa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libswa.so.  torch supplies device memory and the stream (the
current torch stream of the tensors' device).  There is no CPU fallback: if
the library is missing, or a call returns a non-OK status, a RuntimeError is
raised with the library's message.
"""
from __future__ import annotations

import ctypes
import os

import torch  # must be imported before libswa.so is loaded: the two share torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswa.so")

SWA_OK, SWA_ERR_INVALID, SWA_ERR_UNSUPPORTED, SWA_ERR_HIP = 0, 1, 2, 3
SWA_F32, SWA_BF16 = 0, 1

EXPORTS = ("swa_last_error", "swa_version", "swa_prefill_workspace_size", "swa_attn_prefill", "swa_debug_visibility", "swa_rope_table",
           "swa_rope_table_host",
           "kv_pool_compress_rope", "swa_kv_quantize", "swa_decode_workspace_size", "swa_attn_decode",
           "swa_attn_decode_noalloc", "swa_attn_decode_compressed", "swa_chunk_prefill_workspace_size",
           "swa_attn_chunk_prefill", "swa_prefill_backward_workspace_size", "swa_attn_prefill_backward",
           "swa_nsa_select_workspace_size", "swa_nsa_select_attn",
           "swa_kv_budget_window", "swa_effective_kv_window")


class ChunkParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("D", ctypes.c_int),
                ("W", ctypes.c_int), ("S", ctypes.c_int), ("Tc", ctypes.c_int), ("scale", ctypes.c_float)]


class PrefillParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("T", ctypes.c_int),
                ("D", ctypes.c_int), ("window", ctypes.c_int), ("compress_block", ctypes.c_int),
                ("rope_len", ctypes.c_int), ("scale", ctypes.c_float), ("dtype", ctypes.c_int)]


class DecodeParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("D", ctypes.c_int),
                ("W", ctypes.c_int), ("S", ctypes.c_int), ("scale", ctypes.c_float), ("num_splits", ctypes.c_int)]


class SwaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libswa status {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libswa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m compressed_kv_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I, LL, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_size_t
    L.swa_last_error.restype = ctypes.c_char_p
    L.swa_last_error.argtypes = []
    L.swa_version.restype = I
    L.swa_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillParams)]
    L.swa_prefill_workspace_size.restype = Z
    L.swa_attn_prefill.argtypes = [ctypes.POINTER(PrefillParams)] + [P] * 11 + [P, Z, P]
    L.swa_attn_prefill.restype = I
    L.swa_debug_visibility.argtypes = [ctypes.POINTER(PrefillParams), P, P, P, P, P, Z, P]
    L.swa_debug_visibility.restype = I
    L.swa_rope_table.argtypes = [ctypes.c_double, I, I, P, P, P]
    L.swa_rope_table.restype = I
    L.swa_rope_table_host.argtypes = [ctypes.c_double, I, I, P, P]
    L.swa_rope_table_host.restype = I
    L.kv_pool_compress_rope.argtypes = [I, I, I, I, I, I, P, P, P, P, I, P, P, P]
    L.kv_pool_compress_rope.restype = I
    L.swa_kv_quantize.argtypes = [LL, I, P, P, P, P]
    L.swa_kv_quantize.restype = I
    L.swa_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeParams)]
    L.swa_decode_workspace_size.restype = Z
    L.swa_attn_decode.argtypes = [ctypes.POINTER(DecodeParams)] + [P] * 14 + [P, Z, P]
    L.swa_attn_decode.restype = I
    L.swa_attn_decode_noalloc.argtypes = [ctypes.POINTER(DecodeParams)] + [P] * 14 + [P]
    L.swa_attn_decode_noalloc.restype = I
    L.swa_attn_decode_compressed.argtypes = [ctypes.POINTER(DecodeParams), I, P, P, I] + [P] * 16 + [P, Z, P]
    L.swa_attn_decode_compressed.restype = I
    L.swa_nsa_select_workspace_size.argtypes = [ctypes.POINTER(PrefillParams)]
    L.swa_nsa_select_workspace_size.restype = Z
    L.swa_nsa_select_attn.argtypes = [ctypes.POINTER(PrefillParams), I] + [P] * 8 + [P, Z, P]
    L.swa_nsa_select_attn.restype = I
    L.swa_prefill_backward_workspace_size.argtypes = [ctypes.POINTER(PrefillParams)]
    L.swa_prefill_backward_workspace_size.restype = Z
    L.swa_attn_prefill_backward.argtypes = [ctypes.POINTER(PrefillParams)] + [P] * 13 + [P, Z, P]
    L.swa_attn_prefill_backward.restype = I
    L.swa_chunk_prefill_workspace_size.argtypes = [ctypes.POINTER(ChunkParams)]
    L.swa_chunk_prefill_workspace_size.restype = Z
    L.swa_attn_chunk_prefill.argtypes = [ctypes.POINTER(ChunkParams)] + [P] * 14 + [P, Z, P]
    L.swa_attn_chunk_prefill.restype = I
    L.swa_kv_budget_window.argtypes = [LL] * 7
    L.swa_kv_budget_window.restype = LL
    L.swa_effective_kv_window.argtypes = [LL] * 8
    L.swa_effective_kv_window.restype = LL
    _lib = L
    return L


def _check(rc):
    if rc != SWA_OK:
        raise SwaError(rc, lib().swa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _shape(t, name, shape):
    """Raise ValueError unless tensor t (if given) has exactly this shape.  The C ABI receives raw pointers and
    cannot see shapes, so every extent the kernels index with is checked here, before any launch."""
    if t is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    return t


def _same_device(ref, *tensors):
    for name, t in tensors:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _swa_dtype(t):
    if t.dtype == torch.bfloat16:
        return SWA_BF16
    if t.dtype == torch.float32:
        return SWA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def rope_table(theta: float, rope_len: int, D: int, device="cuda"):
    """cos/sin tables [rope_len, D/2] fp32 (angle pos * theta^(-2i/D), fp64 on device)."""
    c = torch.empty((rope_len, D // 2), dtype=torch.float32, device=device)
    s = torch.empty_like(c)
    _check(lib().swa_rope_table(float(theta), int(rope_len), int(D), _ptr(c), _ptr(s), _stream(c)))
    return c, s


def rope_table_host(theta: float, rope_len: int, D: int):
    """cos/sin tables [rope_len, D/2] as host numpy fp32 arrays, computed by the library on the host
    (angle pos * theta^(-2i/D) in fp64, rounded once)."""
    import numpy as np
    c = np.empty((int(rope_len), int(D) // 2), dtype=np.float32)
    s = np.empty_like(c)
    _check(lib().swa_rope_table_host(float(theta), int(rope_len), int(D), c.ctypes.data_as(ctypes.c_void_p),
                                     s.ctypes.data_as(ctypes.c_void_p)))
    return c, s


def prefill_params(q, k, window, compress_block=0, rope_len=0, scale=0.0):
    B, Hq, T, D = q.shape
    return PrefillParams(B, Hq, k.shape[1], T, D, int(window), int(compress_block), int(rope_len), float(scale),
                         _swa_dtype(q))


def prefill_workspace(q, k, window=0, rope=None, compress_block=0):
    """Allocate the workspace a prefill call with these arguments needs (None if none)."""
    rope_len = rope[0].shape[0] if rope is not None else 0
    p = prefill_params(q, k, window, compress_block, rope_len)
    n = lib().swa_prefill_workspace_size(ctypes.byref(p))
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def prefill(q, k, v, seg_ids=None, prefix=None, window=0, rope=None, pooled_k=None, pooled_v=None,
            compress_block=0, scale=0.0, return_lse=False, out=None, workspace=None):
    """Windowed+sink (or compressed) prefill attention.  q [B,Hq,T,D], k/v [B,Hkv,T,D].

    workspace: optional preallocated buffer (see prefill_workspace); allocated here if needed.
    Shapes are checked first, then devices and dtypes; nothing is launched unless all pass."""
    cos, sin = rope if rope is not None else (None, None)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D: [B, Hq, T, D] and [B, Hkv, T, D]")
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    _shape(k, "k", (B, Hkv, T, D))
    _shape(v, "v", (B, Hkv, T, D))
    _shape(seg_ids, "seg_ids", (B, T))
    _shape(prefix, "prefix", (B, T))
    if compress_block:
        _shape(pooled_k, "pooled_k", (B, Hkv, T // int(compress_block), D))
        _shape(pooled_v, "pooled_v", (B, Hkv, T // int(compress_block), D))
    elif pooled_k is not None or pooled_v is not None:
        raise ValueError("pooled_k / pooled_v are only used with compress_block > 0")
    if (cos is None) != (sin is None):
        raise ValueError("rope must be a (cos, sin) pair")
    rope_len = cos.shape[0] if cos is not None else 0
    _shape(cos, "rope_cos", (rope_len, D // 2))
    _shape(sin, "rope_sin", (rope_len, D // 2))
    _shape(out, "out", (B, Hq, T, D))
    _dev(q, "q")
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    _dev(seg_ids, "seg_ids", torch.int32)
    _dev(prefix, "prefix", torch.uint8)
    _dev(pooled_k, "pooled_k", q.dtype)
    _dev(pooled_v, "pooled_v", q.dtype)
    _dev(cos, "rope_cos", torch.float32)
    _dev(sin, "rope_sin", torch.float32)
    _dev(out, "out", q.dtype)
    _same_device(q, ("k", k), ("v", v), ("seg_ids", seg_ids), ("prefix", prefix), ("pooled_k", pooled_k),
                 ("pooled_v", pooled_v), ("rope_cos", cos), ("rope_sin", sin), ("out", out))
    p = prefill_params(q, k, window, compress_block, rope_len, scale)
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    ws_bytes = lib().swa_prefill_workspace_size(ctypes.byref(p))
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().swa_attn_prefill(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(pooled_k), _ptr(pooled_v),
                                  _ptr(seg_ids), _ptr(prefix), _ptr(cos), _ptr(sin), _ptr(out), _ptr(lse),
                                  _ptr(workspace), ws_len, _stream(q)))
    return (out, lse) if return_lse else out


def debug_visibility(B, Hq, Hkv, T, D, window, dtype=torch.bfloat16, seg_ids=None, prefix=None, compress_block=0,
                     want_mask=True, device="cuda"):
    """Mask [B,T,Tk] (uint8) and visible counts [B,T] exactly as the prefill kernel for `dtype` applies them."""
    p = PrefillParams(B, Hq, Hkv, T, D, int(window), int(compress_block), 0, 0.0,
                      SWA_BF16 if dtype == torch.bfloat16 else SWA_F32)
    _dev(seg_ids, "seg_ids", torch.int32)
    _dev(prefix, "prefix", torch.uint8)
    _shape(seg_ids, "seg_ids", (B, T))
    _shape(prefix, "prefix", (B, T))
    Tk = T + (T // compress_block if compress_block else 0)
    mask = torch.empty((B, T, Tk), dtype=torch.uint8, device=device) if want_mask else None
    count = torch.empty((B, T), dtype=torch.int32, device=device)
    ws_bytes = lib().swa_prefill_workspace_size(ctypes.byref(p))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device) if ws_bytes else None
    _check(lib().swa_debug_visibility(ctypes.byref(p), _ptr(seg_ids), _ptr(prefix), _ptr(mask), _ptr(count),
                                      _ptr(ws), ws_bytes, _stream(count)))
    return mask, count


def pool_compress_rope(k_pre, v, block, rope=None, out=None):
    """Mean-pool b-row blocks of k_pre and v ([B,H,T,D]); rotate pooled keys at block midpoints.

    out: optional (pooled_k, pooled_v) tensors [B,H,T//block,D] to write into."""
    if k_pre.dim() != 4:
        raise ValueError("k_pre must be 4-D: [B, H, T, D]")
    B, H, T, D = k_pre.shape
    _shape(v, "v", (B, H, T, D))
    cos, sin = rope if rope is not None else (None, None)
    if (cos is None) != (sin is None):
        raise ValueError("rope must be a (cos, sin) pair")
    rope_len = cos.shape[0] if cos is not None else 0
    _shape(cos, "rope_cos", (rope_len, D // 2))
    _shape(sin, "rope_sin", (rope_len, D // 2))
    _dev(cos, "rope_cos", torch.float32)
    _dev(sin, "rope_sin", torch.float32)
    _dev(k_pre, "k_pre")
    _dev(v, "v", k_pre.dtype)
    _same_device(k_pre, ("v", v), ("rope_cos", cos), ("rope_sin", sin))
    if out is None:
        pk = torch.empty((B, H, T // block, D), dtype=k_pre.dtype, device=k_pre.device)
        pv = torch.empty_like(pk)
    else:
        pk, pv = _dev(out[0], "pooled_k", k_pre.dtype), _dev(out[1], "pooled_v", k_pre.dtype)
        if tuple(pk.shape) != (B, H, T // block, D) or tuple(pv.shape) != (B, H, T // block, D):
            raise ValueError("pooled outputs must be [B, H, T // block, D]")
    _check(lib().kv_pool_compress_rope(B, H, T, D, int(block), _swa_dtype(k_pre), _ptr(k_pre), _ptr(v), _ptr(cos),
                                       _ptr(sin), int(rope_len), _ptr(pk), _ptr(pv), _stream(k_pre)))
    return pk, pv


def kv_quantize(x):
    """bf16 [..., D] -> (int8 codes [..., D], fp32 scales [..., D/32])."""
    _dev(x, "x", torch.bfloat16)
    D = x.shape[-1]
    N = x.numel() // D
    xq = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    xs = torch.empty(x.shape[:-1] + (D // 32,), dtype=torch.float32, device=x.device)
    _check(lib().swa_kv_quantize(N, D, _ptr(x), _ptr(xq), _ptr(xs), _stream(x)))
    return xq, xs


def decode_params(q, ring_k, sink_k, scale=0.0, num_splits=0):
    B, Hq, D = q.shape
    Hkv, W = ring_k.shape[1], ring_k.shape[2]
    S = sink_k.shape[2] if sink_k is not None else 0
    return DecodeParams(B, Hq, Hkv, D, W, S, float(scale), int(num_splits))


def decode_workspace(q, ring_k, sink_k, num_splits=0):
    """A zero-filled workspace for decode calls of this shape and split count (None when none is needed).
    The library leaves its counter words zero after every completed call, so it can be reused."""
    p = decode_params(q, ring_k, sink_k, 0.0, num_splits)
    n = lib().swa_decode_workspace_size(ctypes.byref(p))
    return torch.zeros(n, dtype=torch.uint8, device=q.device) if n else None


def _cache_shapes(B, Hkv, W, D, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos, sink_len):
    """Shapes of the ring and sink caches and the per-row position arrays."""
    _shape(ring_k, "ring_k", (B, Hkv, W, D))
    _shape(ring_v, "ring_v", (B, Hkv, W, D))
    _shape(ring_ks, "ring_ks", (B, Hkv, W, D // 32))
    _shape(ring_vs, "ring_vs", (B, Hkv, W, D // 32))
    if (sink_k is None) != (sink_v is None) or (sink_k is None) != (sink_ks is None) or \
            (sink_k is None) != (sink_vs is None):
        raise ValueError("sink_k, sink_v, sink_ks and sink_vs must all be given or all be None")
    S = sink_k.shape[2] if sink_k is not None else 0
    _shape(sink_k, "sink_k", (B, Hkv, S, D))
    _shape(sink_v, "sink_v", (B, Hkv, S, D))
    _shape(sink_ks, "sink_ks", (B, Hkv, S, D // 32))
    _shape(sink_vs, "sink_vs", (B, Hkv, S, D // 32))
    _shape(pos, "pos", (B,))
    _shape(sink_len, "sink_len", (B,))


def _cache_devices(ref, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos, sink_len):
    for name, t, dt in (("ring_k", ring_k, torch.int8), ("ring_v", ring_v, torch.int8),
                        ("ring_ks", ring_ks, torch.float32), ("ring_vs", ring_vs, torch.float32),
                        ("sink_k", sink_k, torch.int8), ("sink_v", sink_v, torch.int8),
                        ("sink_ks", sink_ks, torch.float32), ("sink_vs", sink_vs, torch.float32),
                        ("pos", pos, torch.int32), ("sink_len", sink_len, torch.int32)):
        _dev(t, name, dt)
    _same_device(ref, ("ring_k", ring_k), ("ring_v", ring_v), ("ring_ks", ring_ks), ("ring_vs", ring_vs),
                 ("sink_k", sink_k), ("sink_v", sink_v), ("sink_ks", sink_ks), ("sink_vs", sink_vs), ("pos", pos),
                 ("sink_len", sink_len))


def _decode_checks(q, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos, sink_len, k_new,
                   v_new, out):
    if q.dim() != 3 or ring_k.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and ring_k [B, Hkv, W, D]")
    B, Hq, D = q.shape
    Hkv, W = ring_k.shape[1], ring_k.shape[2]
    if D % 32:
        raise ValueError(f"head dim {D} must be a multiple of 32")
    _shape(ring_k, "ring_k", (B, Hkv, W, D))
    _shape(ring_v, "ring_v", (B, Hkv, W, D))
    _shape(ring_ks, "ring_ks", (B, Hkv, W, D // 32))
    _shape(ring_vs, "ring_vs", (B, Hkv, W, D // 32))
    if (sink_k is None) != (sink_v is None) or (sink_k is None) != (sink_ks is None) or \
            (sink_k is None) != (sink_vs is None):
        raise ValueError("sink_k, sink_v, sink_ks and sink_vs must all be given or all be None")
    S = sink_k.shape[2] if sink_k is not None else 0
    _shape(sink_k, "sink_k", (B, Hkv, S, D))
    _shape(sink_v, "sink_v", (B, Hkv, S, D))
    _shape(sink_ks, "sink_ks", (B, Hkv, S, D // 32))
    _shape(sink_vs, "sink_vs", (B, Hkv, S, D // 32))
    _shape(pos, "pos", (B,))
    _shape(sink_len, "sink_len", (B,))
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    _shape(k_new, "k_new", (B, Hkv, D))
    _shape(v_new, "v_new", (B, Hkv, D))
    _shape(out, "out", (B, Hq, D))
    _dev(q, "q", torch.bfloat16)
    for name, t, dt in (("ring_k", ring_k, torch.int8), ("ring_v", ring_v, torch.int8),
                        ("ring_ks", ring_ks, torch.float32), ("ring_vs", ring_vs, torch.float32),
                        ("sink_k", sink_k, torch.int8), ("sink_v", sink_v, torch.int8),
                        ("sink_ks", sink_ks, torch.float32), ("sink_vs", sink_vs, torch.float32),
                        ("pos", pos, torch.int32), ("sink_len", sink_len, torch.int32),
                        ("k_new", k_new, torch.bfloat16), ("v_new", v_new, torch.bfloat16),
                        ("out", out, torch.bfloat16)):
        _dev(t, name, dt)
    _same_device(q, ("ring_k", ring_k), ("ring_v", ring_v), ("ring_ks", ring_ks), ("ring_vs", ring_vs),
                 ("sink_k", sink_k), ("sink_v", sink_v), ("sink_ks", sink_ks), ("sink_vs", sink_vs), ("pos", pos),
                 ("sink_len", sink_len), ("k_new", k_new), ("v_new", v_new), ("out", out))


def decode(q, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos, sink_len=None, k_new=None,
           v_new=None, scale=0.0, num_splits=0, out=None, workspace=None):
    """One decode step; appends k_new/v_new into the ring (in place) first.  Returns out [B,Hq,D] bf16.

    num_splits: 0 lets the library choose; k > 0 cuts every (sequence, kv head) walk into k parts.
    workspace: optional zero-filled buffer from decode_workspace(); allocated (zeroed) here if needed."""
    _decode_checks(q, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos, sink_len, k_new,
                   v_new, out)
    p = decode_params(q, ring_k, sink_k, scale, num_splits)
    ws_bytes = lib().swa_decode_workspace_size(ctypes.byref(p))
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_len = workspace.numel() * workspace.element_size() if (ws_bytes and workspace is not None) else 0
    if out is None:
        out = torch.empty_like(q)
    _check(lib().swa_attn_decode(ctypes.byref(p), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(ring_k), _ptr(ring_v),
                                 _ptr(ring_ks), _ptr(ring_vs), _ptr(sink_k), _ptr(sink_v), _ptr(sink_ks),
                                 _ptr(sink_vs), _ptr(pos), _ptr(sink_len), _ptr(out),
                                 _ptr(workspace) if ws_len else None, ws_len, _stream(q)))
    return out


def decode_noalloc(q, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos, sink_len=None,
                   k_new=None, v_new=None, scale=0.0, num_splits=0, out=None):
    """decode() without a workspace: the split-K state lives in the library's own device array (for callers
    that cannot allocate; `out` should then be passed in).  Calls overlapping in time on one GPU race."""
    _decode_checks(q, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos, sink_len, k_new,
                   v_new, out)
    p = decode_params(q, ring_k, sink_k, scale, num_splits)
    if out is None:
        out = torch.empty_like(q)
    _check(lib().swa_attn_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(ring_k),
                                         _ptr(ring_v), _ptr(ring_ks), _ptr(ring_vs), _ptr(sink_k), _ptr(sink_v),
                                         _ptr(sink_ks), _ptr(sink_vs), _ptr(pos), _ptr(sink_len), _ptr(out),
                                         _stream(q)))
    return out


def decode_compressed(q, k_new, k_new_pre, v_new, ring_k, ring_v, ring_ks, ring_vs, pool_k, pool_v, pool_ks, pool_vs,
                      front_k, front_v, pos, block, rope=None, scale=0.0, num_splits=0, out=None, workspace=None):
    """One compressed decode step (swa_attn_decode_compressed).  q [B,Hq,D] and k_new [B,Hkv,D] are rotated
    at pos, k_new_pre is the same key before rotation, v_new [B,Hkv,D]; all bf16.  ring_* as in decode();
    pool_k/pool_v [B,Hkv,P,D] int8 and pool_ks/pool_vs [B,Hkv,P,D/32] fp32 (P may be 0: pass None);
    front_k/front_v [B,Hkv,D] fp32.  rope: (cos, sin) from rope_table(), or None for no rotation of the
    pooled keys.  The caches and the frontier are updated in place.  Returns out [B,Hq,D] bf16."""
    if q.dim() != 3 or ring_k.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and ring_k [B, Hkv, W, D]")
    B, Hq, D = q.shape
    Hkv = ring_k.shape[1]
    if int(block) < 1:
        raise ValueError(f"block must be >= 1 (got {block})")
    if k_new is None or v_new is None or k_new_pre is None:
        raise ValueError("k_new, k_new_pre and v_new are required")
    _shape(k_new_pre, "k_new_pre", (B, Hkv, D))
    _shape(front_k, "front_k", (B, Hkv, D))
    _shape(front_v, "front_v", (B, Hkv, D))
    _decode_checks(q, ring_k, ring_v, ring_ks, ring_vs, pool_k, pool_v, pool_ks, pool_vs, pos, None, k_new, v_new,
                   out)
    _dev(k_new_pre, "k_new_pre", torch.bfloat16)
    _dev(front_k, "front_k", torch.float32)
    _dev(front_v, "front_v", torch.float32)
    cos, sin = rope if rope is not None else (None, None)
    rope_len = 0
    if cos is not None:
        _shape(cos, "rope cos", (cos.shape[0], D // 2))
        _shape(sin, "rope sin", (cos.shape[0], D // 2))
        _dev(cos, "rope cos", torch.float32)
        _dev(sin, "rope sin", torch.float32)
        rope_len = cos.shape[0]
    _same_device(q, ("k_new_pre", k_new_pre), ("front_k", front_k), ("front_v", front_v), ("rope cos", cos),
                 ("rope sin", sin))
    p = decode_params(q, ring_k, pool_k, scale, num_splits)
    ws_bytes = lib().swa_decode_workspace_size(ctypes.byref(p))
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_len = workspace.numel() * workspace.element_size() if (ws_bytes and workspace is not None) else 0
    if out is None:
        out = torch.empty_like(q)
    _check(lib().swa_attn_decode_compressed(ctypes.byref(p), int(block), _ptr(cos), _ptr(sin), int(rope_len),
                                            _ptr(q), _ptr(k_new), _ptr(k_new_pre), _ptr(v_new), _ptr(ring_k),
                                            _ptr(ring_v), _ptr(ring_ks), _ptr(ring_vs), _ptr(pool_k), _ptr(pool_v),
                                            _ptr(pool_ks), _ptr(pool_vs), _ptr(front_k), _ptr(front_v), _ptr(pos),
                                            _ptr(out), _ptr(workspace) if ws_len else None, ws_len, _stream(q)))
    return out


def prefill_backward(q, k, v, out, lse, dout, seg_ids=None, prefix=None, window=0, rope=None, scale=0.0,
                     workspace=None):
    """Gradients (dq, dk, dv) of prefill() in plain mode, fp32, from the forward's out and lse (prefill(...,
    return_lse=True)).  q, k, v, out, dout share the forward's dtype; with rope (the forward's table) q and k
    are the unrotated inputs and so are dq and dk."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, T, D] and k [B, Hkv, T, D]")
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    _shape(k, "k", (B, Hkv, T, D))
    _shape(v, "v", (B, Hkv, T, D))
    _shape(out, "out", (B, Hq, T, D))
    _shape(dout, "dout", (B, Hq, T, D))
    _shape(lse, "lse", (B, Hq, T))
    _shape(seg_ids, "seg_ids", (B, T))
    _shape(prefix, "prefix", (B, T))
    cos, sin = rope if rope is not None else (None, None)
    if cos is not None:
        _shape(cos, "rope cos", (cos.shape[0], D // 2))
        _shape(sin, "rope sin", (cos.shape[0], D // 2))
    _dev(q, "q")
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        _dev(t, name, q.dtype)
    _dev(lse, "lse", torch.float32)
    _dev(seg_ids, "seg_ids", torch.int32)
    _dev(prefix, "prefix", torch.uint8)
    _dev(cos, "rope cos", torch.float32)
    _dev(sin, "rope sin", torch.float32)
    _same_device(q, ("k", k), ("v", v), ("out", out), ("dout", dout), ("lse", lse), ("seg_ids", seg_ids),
                 ("prefix", prefix), ("rope cos", cos), ("rope sin", sin))
    p = prefill_params(q, k, window, 0, cos.shape[0] if cos is not None else 0, scale)
    n = lib().swa_prefill_backward_workspace_size(ctypes.byref(p))
    if n and (workspace is None or workspace.numel() * workspace.element_size() < n):
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    _check(lib().swa_attn_prefill_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                           _ptr(dout), _ptr(seg_ids), _ptr(prefix), _ptr(cos), _ptr(sin), _ptr(dq),
                                           _ptr(dk), _ptr(dv), _ptr(workspace) if n else None, n, _stream(q)))
    return dq, dk, dv


def nsa_select(q, k, v, window, block, n_select, rope=None, scale=0.0, workspace=None):
    """The NSA selection branch without its gate (swa_nsa_select_attn).  q [B,Hq,T,D], k/v [B,Hkv,T,D] before
    RoPE (fp32 or bf16); rope: (cos, sin) from rope_table() or None.  Returns (out [B,Hq,T,D] in q's dtype,
    lse [B,Hq,T] fp32, sel [B,Hq,T,n_select] int32: the chosen blocks in score order, -1 after the last)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, T, D] and k [B, Hkv, T, D]")
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    _shape(k, "k", (B, Hkv, T, D))
    _shape(v, "v", (B, Hkv, T, D))
    if not 1 <= int(n_select) <= 32:
        raise ValueError(f"n_select must be in [1, 32] (got {n_select})")
    if int(block) < 1 or int(window) < 1:
        raise ValueError("block and window must be >= 1")
    cos, sin = rope if rope is not None else (None, None)
    if cos is not None:
        _shape(cos, "rope cos", (cos.shape[0], D // 2))
        _shape(sin, "rope sin", (cos.shape[0], D // 2))
    _dev(q, "q")
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    _dev(cos, "rope cos", torch.float32)
    _dev(sin, "rope sin", torch.float32)
    _same_device(q, ("k", k), ("v", v), ("rope cos", cos), ("rope sin", sin))
    p = prefill_params(q, k, window, block, cos.shape[0] if cos is not None else 0, scale)
    n = lib().swa_nsa_select_workspace_size(ctypes.byref(p))
    if n and (workspace is None or workspace.numel() * workspace.element_size() < n):
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    sel = torch.empty((B, Hq, T, int(n_select)), dtype=torch.int32, device=q.device)
    _check(lib().swa_nsa_select_attn(ctypes.byref(p), int(n_select), _ptr(q), _ptr(k), _ptr(v), _ptr(cos), _ptr(sin),
                                     _ptr(out), _ptr(lse), _ptr(sel), _ptr(workspace) if n else None, n, _stream(q)))
    return out, lse, sel


def chunk_params(q, ring_k, sink_k, scale=0.0):
    B, Hq, Tc, D = q.shape
    Hkv, W = ring_k.shape[1], ring_k.shape[2]
    S = sink_k.shape[2] if sink_k is not None else 0
    return ChunkParams(B, Hq, Hkv, D, W, S, Tc, float(scale))


def chunk_prefill_workspace(q, ring_k, sink_k):
    """The workspace swa_attn_chunk_prefill needs for these shapes (None when none is needed)."""
    n = lib().swa_chunk_prefill_workspace_size(ctypes.byref(chunk_params(q, ring_k, sink_k)))
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def chunk_prefill(q, k, v, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos0, sink_len=None,
                  scale=0.0, out=None, workspace=None):
    """Chunked prefill into existing caches (swa_attn_chunk_prefill).  q [B,Hq,Tc,D], k/v [B,Hkv,Tc,D] bf16
    (q and k rotated); ring/sink caches as in decode(); pos0 [B] int32 (first position of the chunk).  The
    ring takes the chunk's last min(W, Tc) tokens.  Returns out [B,Hq,Tc,D] bf16."""
    if q.dim() != 4 or ring_k.dim() != 4:
        raise ValueError("q must be [B, Hq, Tc, D] and ring_k [B, Hkv, W, D]")
    B, Hq, Tc, D = q.shape
    Hkv, W = ring_k.shape[1], ring_k.shape[2]
    if D % 32:
        raise ValueError(f"head dim {D} must be a multiple of 32")
    _shape(k, "k", (B, Hkv, Tc, D))
    _shape(v, "v", (B, Hkv, Tc, D))
    _shape(out, "out", (B, Hq, Tc, D))
    _cache_shapes(B, Hkv, W, D, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos0, sink_len)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _dev(t, name, torch.bfloat16)
    _same_device(q, ("k", k), ("v", v), ("out", out))
    _cache_devices(q, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos0, sink_len)
    p = chunk_params(q, ring_k, sink_k, scale)
    ws_bytes = lib().swa_chunk_prefill_workspace_size(ctypes.byref(p))
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_len = workspace.numel() * workspace.element_size() if (ws_bytes and workspace is not None) else 0
    if out is None:
        out = torch.empty_like(q)
    _check(lib().swa_attn_chunk_prefill(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(ring_k), _ptr(ring_v),
                                        _ptr(ring_ks), _ptr(ring_vs), _ptr(sink_k), _ptr(sink_v), _ptr(sink_ks),
                                        _ptr(sink_vs), _ptr(pos0), _ptr(sink_len), _ptr(out),
                                        _ptr(workspace) if ws_len else None, ws_len, _stream(q)))
    return out


def kv_budget_window(d_model, num_heads, num_kv_heads, num_layers, max_seq_len, sites=2, attn_dim=0):
    return int(lib().swa_kv_budget_window(d_model, attn_dim, num_heads, num_kv_heads, num_layers, sites,
                                          max_seq_len))


def effective_kv_window(d_model, num_heads, num_kv_heads, num_layers, max_seq_len, kv_window, sites=2, attn_dim=0):
    return int(lib().swa_effective_kv_window(d_model, attn_dim, num_heads, num_kv_heads, num_layers, sites,
                                             max_seq_len, kv_window or 0))
