"""CPU oracle for windowed+sink GQA attention and compressed-KV attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``compressed_kv_attention_amd``) never imports, loads or calls it, and
the two share no code: the oracle is plain fp64 loops in ``oracle.cpp``
(built with g++, no fast-math), wrapped here with ctypes over numpy arrays.

Each function restates what one passage of the pages defines; the C source
names the page and section for each.  Parity-unpinned parts: the RoPE pairing
convention (rotate-half, reading R-A7), the quantizer's rounding convention
(reading R-A13) and the empty-row constant (reading R-A4).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.cpp with g++ into oracle/liboracle.so (fp64, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    LL = ctypes.c_longlong
    D = ctypes.c_double
    lib.oracle_mask.argtypes = [I, I, P, P, I, P]
    lib.oracle_compressed_mask.argtypes = [I, I, I, P]
    lib.oracle_rope.argtypes = [I, I, D, P, P, P]
    lib.oracle_prefill.argtypes = [I, I, I, I, I, P, P, P, P, P, I, D, D, LL, P, P, P]
    lib.oracle_pool_rope.argtypes = [LL, I, I, I, D, I, P, P, P, P]
    lib.oracle_compressed_prefill.argtypes = [I, I, I, I, I, P, P, P, I, I, D, D, I, LL, P, P, P]
    lib.oracle_kv_budget_per_pos.argtypes = [LL] * 6
    lib.oracle_kv_budget_per_pos.restype = LL
    lib.oracle_kv_budget_window.argtypes = [LL] * 7
    lib.oracle_kv_budget_window.restype = LL
    lib.oracle_effective_kv_window.argtypes = [LL] * 8
    lib.oracle_effective_kv_window.restype = LL
    lib.oracle_quantize.argtypes = [LL, I, P, P, P]
    lib.oracle_decode.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, D, P, P]
    lib.oracle_nsa_select.argtypes = [I, I, I, I, I, P, P, P, I, I, I, D, D, I, P, P, P, P]
    lib.oracle_prefill_backward.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I, D, D, P, P, P]
    lib.oracle_chunk_prefill.argtypes = [I, I, I, I, I, I, I] + [P] * 13 + [D, P, P]
    lib.oracle_compressed_decode.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, D, I, D, I,
                                             P, P]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _opt(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def mask(seg_ids, prefix=None, window=0, T=None):
    """O1: prefill visibility [B, T, T] (uint8).  seg_ids [B,T] int32 or None (all 1)."""
    lib = _load()
    seg = _opt(seg_ids, np.int32)
    pre = _opt(prefix, np.uint8)
    if seg is not None:
        B, T = seg.shape
    elif pre is not None:
        B, T = pre.shape
    else:
        B = 1
    out = np.zeros((B, T, T), dtype=np.uint8)
    lib.oracle_mask(B, T, _ptr(seg), _ptr(pre), int(window), _ptr(out))
    return out


def compressed_mask(T, window, block):
    """O4 mask [T, T//block + T] (uint8), columns [pooled blocks, exact keys]."""
    lib = _load()
    out = np.zeros((T, T // block + T), dtype=np.uint8)
    lib.oracle_compressed_mask(int(T), int(window), int(block), _ptr(out))
    return out


def rope(x, pos, theta=10000.0):
    """O2: rotate-half RoPE of x[N, D] at integer positions pos[N] (fp64)."""
    lib = _load()
    x = _f64(x)
    N, Dm = x.shape
    p = np.ascontiguousarray(pos, dtype=np.int64)
    y = np.empty_like(x)
    lib.oracle_rope(N, Dm, float(theta), _ptr(p), _ptr(x), _ptr(y))
    return y


def _rows_arg(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, r.shape[0]


def prefill(q, k, v, seg_ids=None, prefix=None, window=0, scale=None, theta=0.0, rows=None):
    """O1+O2+O3.  q [B,Hq,T,D], k/v [B,Hkv,T,D].  Returns (out, lse).

    rows: optional flat row indices ((b*Hq + h)*T + t); then out is [n, D].
    Otherwise out is [B,Hq,T,D] and lse [B,Hq,T].  theta > 0 applies RoPE.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, T, Dm = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(Dm)
    seg = _opt(seg_ids, np.int32)
    pre = _opt(prefix, np.uint8)
    r, n = _rows_arg(rows)
    nout = n if r is not None else B * Hq * T
    out = np.empty((nout, Dm), dtype=np.float64)
    lse = np.empty((nout,), dtype=np.float64)
    lib.oracle_prefill(B, Hq, Hkv, T, Dm, _ptr(q), _ptr(k), _ptr(v), _ptr(seg), _ptr(pre),
                       int(window), float(scale), float(theta), n, _ptr(r), _ptr(out), _ptr(lse))
    if r is None:
        return out.reshape(B, Hq, T, Dm), lse.reshape(B, Hq, T)
    return out, lse


def pool_rope(k_pre, v, block, theta=0.0, rope_len=None):
    """O4 pooling: (pooled_k rotated at block midpoints, pooled_v). Inputs [..., T, D]."""
    lib = _load()
    k_pre, v = _f64(k_pre), _f64(v)
    lead = k_pre.shape[:-2]
    T, Dm = k_pre.shape[-2:]
    N = int(np.prod(lead)) if lead else 1
    nblk = T // block
    if rope_len is None:
        rope_len = T
    pk = np.empty(lead + (nblk, Dm), dtype=np.float64)
    pv = np.empty(lead + (nblk, Dm), dtype=np.float64)
    lib.oracle_pool_rope(N, T, Dm, int(block), float(theta), int(rope_len), _ptr(k_pre), _ptr(v),
                         _ptr(pk), _ptr(pv))
    return pk, pv


def compressed_prefill(q, k_pre, v, window, block, scale=None, theta=10000.0, rope_len=None, rows=None):
    """O4: attention over [pooled blocks, exact keys].  Returns (out, lse) like prefill()."""
    lib = _load()
    q, k_pre, v = _f64(q), _f64(k_pre), _f64(v)
    B, Hq, T, Dm = q.shape
    Hkv = k_pre.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(Dm)
    if rope_len is None:
        rope_len = T
    r, n = _rows_arg(rows)
    nout = n if r is not None else B * Hq * T
    out = np.empty((nout, Dm), dtype=np.float64)
    lse = np.empty((nout,), dtype=np.float64)
    lib.oracle_compressed_prefill(B, Hq, Hkv, T, Dm, _ptr(q), _ptr(k_pre), _ptr(v), int(window),
                                  int(block), float(scale), float(theta), int(rope_len), n, _ptr(r),
                                  _ptr(out), _ptr(lse))
    if r is None:
        return out.reshape(B, Hq, T, Dm), lse.reshape(B, Hq, T)
    return out, lse


def kv_budget_per_pos(d_model, num_heads, num_kv_heads, num_layers, sites=2, attn_dim=0):
    return int(_load().oracle_kv_budget_per_pos(d_model, attn_dim, num_heads, num_kv_heads,
                                                num_layers, sites))


def kv_budget_window(d_model, num_heads, num_kv_heads, num_layers, max_seq_len, sites=2, attn_dim=0):
    """O5 budget window (tokens)."""
    return int(_load().oracle_kv_budget_window(d_model, attn_dim, num_heads, num_kv_heads,
                                               num_layers, sites, max_seq_len))


def effective_kv_window(d_model, num_heads, num_kv_heads, num_layers, max_seq_len, kv_window,
                        sites=2, attn_dim=0):
    """O5 effective window (tokens); kv_window 0/None = unset."""
    return int(_load().oracle_effective_kv_window(d_model, attn_dim, num_heads, num_kv_heads,
                                                  num_layers, sites, max_seq_len, kv_window or 0))


def quantize(x):
    """O6: x [N, D] float32 -> (codes int8 [N, D], scales float32 [N, D/32])."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    N, Dm = x.shape
    xq = np.empty((N, Dm), dtype=np.int8)
    xs = np.empty((N, Dm // 32), dtype=np.float32)
    lib.oracle_quantize(N, Dm, _ptr(x), _ptr(xq), _ptr(xs))
    return xq, xs


def decode(q, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos,
           sink_len=None, k_new=None, v_new=None, scale=None):
    """O7: one decode step.  Ring arrays are copied, appended to, and returned.

    Returns (out [B,Hq,D] fp64, lse [B,Hq], ring_k, ring_v, ring_ks, ring_vs) after the append.
    """
    lib = _load()
    q = _f64(q)
    B, Hq, Dm = q.shape
    Hkv, W = ring_k.shape[1], ring_k.shape[2]
    S = sink_k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(Dm)
    rk = np.array(ring_k, dtype=np.int8, copy=True, order="C")
    rv = np.array(ring_v, dtype=np.int8, copy=True, order="C")
    rks = np.array(ring_ks, dtype=np.float32, copy=True, order="C")
    rvs = np.array(ring_vs, dtype=np.float32, copy=True, order="C")
    sk = np.ascontiguousarray(sink_k, dtype=np.int8)
    sv = np.ascontiguousarray(sink_v, dtype=np.int8)
    sks = np.ascontiguousarray(sink_ks, dtype=np.float32)
    svs = np.ascontiguousarray(sink_vs, dtype=np.float32)
    p = np.ascontiguousarray(pos, dtype=np.int32)
    sl = _opt(sink_len, np.int32)
    kn = _opt(k_new, np.float32)
    vn = _opt(v_new, np.float32)
    out = np.empty((B, Hq, Dm), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    lib.oracle_decode(B, Hq, Hkv, Dm, W, S, _ptr(q), _ptr(kn), _ptr(vn), _ptr(rk), _ptr(rv),
                      _ptr(rks), _ptr(rvs), _ptr(sk), _ptr(sv), _ptr(sks), _ptr(svs), _ptr(p),
                      _ptr(sl), float(scale), _ptr(out), _ptr(lse))
    return out, lse, rk, rv, rks, rvs


COMPRESSED_STATE = ("ring_k", "ring_v", "pool_k", "pool_v", "front_k", "front_v")


def compressed_decode_state(B, Hkv, D, W, P):
    """An empty compressed decode state (fp64 row values; see compressed_decode)."""
    return {"ring_k": np.zeros((B, Hkv, W, D)), "ring_v": np.zeros((B, Hkv, W, D)),
            "pool_k": np.zeros((B, Hkv, P, D)), "pool_v": np.zeros((B, Hkv, P, D)),
            "front_k": np.zeros((B, Hkv, D)), "front_v": np.zeros((B, Hkv, D))}


def compressed_decode(q, k_new, k_pre, v_new, state, pos, block, theta=10000.0, rope_len=None, scale=None,
                      quantize=True):
    """O8: one compressed decode step.  q [B,Hq,D] and k_new [B,Hkv,D] rotated at pos, k_pre the same key
    before rotation, v_new [B,Hkv,D].  state: dict of fp64 arrays ring_k/ring_v [B,Hkv,W,D], pool_k/pool_v
    [B,Hkv,P,D], front_k/front_v [B,Hkv,D] (row values: dequantized codes, or exact values with
    quantize=False).  Returns (out [B,Hq,D], lse [B,Hq], new state); the given state is not modified."""
    lib = _load()
    q = _f64(q)
    B, Hq, Dm = q.shape
    st = {k: np.array(state[k], dtype=np.float64, copy=True, order="C") for k in COMPRESSED_STATE}
    Hkv, W = st["ring_k"].shape[1], st["ring_k"].shape[2]
    P = st["pool_k"].shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(Dm)
    if rope_len is None:
        rope_len = 1 << 30
    kn, kp, vn = _f64(k_new), _f64(k_pre), _f64(v_new)
    p = np.ascontiguousarray(pos, dtype=np.int32)
    out = np.empty((B, Hq, Dm), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    lib.oracle_compressed_decode(B, Hq, Hkv, Dm, W, P, int(block), _ptr(q), _ptr(kn), _ptr(kp), _ptr(vn),
                                 _ptr(st["ring_k"]), _ptr(st["ring_v"]), _ptr(st["pool_k"]), _ptr(st["pool_v"]),
                                 _ptr(st["front_k"]), _ptr(st["front_v"]), _ptr(p), float(theta), int(rope_len),
                                 float(scale), int(bool(quantize)), _ptr(out), _ptr(lse))
    return out, lse, st


def chunk_prefill(q, k, v, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks, sink_vs, pos0, sink_len=None,
                  scale=None):
    """O9: a chunk q [B,Hq,Tc,D], k/v [B,Hkv,Tc,D] (float32 values) at positions pos0[b] .. + Tc - 1 over the
    sink cache, the ring and itself; then the ring takes the chunk's last W tokens.  The ring arrays are
    copied, updated and returned: (out [B,Hq,Tc,D], lse [B,Hq,Tc], ring_k, ring_v, ring_ks, ring_vs)."""
    lib = _load()
    q = _f64(q)
    B, Hq, Tc, Dm = q.shape
    Hkv, W = ring_k.shape[1], ring_k.shape[2]
    S = sink_k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(Dm)
    rk = np.array(ring_k, dtype=np.int8, copy=True, order="C")
    rv = np.array(ring_v, dtype=np.int8, copy=True, order="C")
    rks = np.array(ring_ks, dtype=np.float32, copy=True, order="C")
    rvs = np.array(ring_vs, dtype=np.float32, copy=True, order="C")
    kk = np.ascontiguousarray(k, dtype=np.float32)
    vv = np.ascontiguousarray(v, dtype=np.float32)
    sk = np.ascontiguousarray(sink_k, dtype=np.int8)
    sv = np.ascontiguousarray(sink_v, dtype=np.int8)
    sks = np.ascontiguousarray(sink_ks, dtype=np.float32)
    svs = np.ascontiguousarray(sink_vs, dtype=np.float32)
    p0 = np.ascontiguousarray(pos0, dtype=np.int32)
    sl = _opt(sink_len, np.int32)
    out = np.empty((B, Hq, Tc, Dm), dtype=np.float64)
    lse = np.empty((B, Hq, Tc), dtype=np.float64)
    lib.oracle_chunk_prefill(B, Hq, Hkv, Dm, W, S, Tc, _ptr(q), _ptr(kk), _ptr(vv), _ptr(rk), _ptr(rv), _ptr(rks),
                             _ptr(rvs), _ptr(sk), _ptr(sv), _ptr(sks), _ptr(svs), _ptr(p0), _ptr(sl), float(scale),
                             _ptr(out), _ptr(lse))
    return out, lse, rk, rv, rks, rvs


def prefill_backward(q, k, v, dout, seg_ids=None, prefix=None, window=0, scale=None, theta=0.0):
    """O10: gradients (dq, dk, dv) of the O1-O3 prefill for the output gradient dout [B,Hq,T,D].  With theta > 0
    q and k are the values before rotation and so are their gradients."""
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, T, Dm = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(Dm)
    seg = _opt(seg_ids, np.int32)
    pre = _opt(prefix, np.uint8)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    lib.oracle_prefill_backward(B, Hq, Hkv, T, Dm, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(seg), _ptr(pre),
                                int(window), float(scale), float(theta), _ptr(dq), _ptr(dk), _ptr(dv))
    return dq, dk, dv


def nsa_select(q, k_pre, v, window, block, n_select, scale=None, theta=10000.0, rope_len=None, sel=None):
    """O11: the NSA selection branch (no gate).  q/k_pre/v [B,Hq|Hkv,T,D] before RoPE.  Returns (out [B,Hq,T,D],
    lse [B,Hq,T], sel [B,Hq,T,n_select] int32 in score order, -1 = none).  `sel` replaces the selection."""
    lib = _load()
    q, k_pre, v = _f64(q), _f64(k_pre), _f64(v)
    B, Hq, T, Dm = q.shape
    Hkv = k_pre.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(Dm)
    if rope_len is None:
        rope_len = T
    sel_in = _opt(sel, np.int32)
    sel_out = np.empty((B, Hq, T, n_select), dtype=np.int32)
    out = np.empty((B, Hq, T, Dm), dtype=np.float64)
    lse = np.empty((B, Hq, T), dtype=np.float64)
    lib.oracle_nsa_select(B, Hq, Hkv, T, Dm, _ptr(q), _ptr(k_pre), _ptr(v), int(window), int(block), int(n_select),
                          float(scale), float(theta), int(rope_len), _ptr(sel_in), _ptr(sel_out), _ptr(out),
                          _ptr(lse))
    return out, lse, sel_out
