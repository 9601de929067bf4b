"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays out segment/sink structure; it
holds none of the method's arithmetic (no masks, no RoPE, no softmax, no
quantization), so both the HIP path and the CPU oracle may take their inputs
from it.

Recipe (numpy PCG64 via ``default_rng(seed)``): q, k, v are drawn in that order
as float32 standard normals, then the structure.  bf16 inputs are the float32
draws rounded to nearest-even; the float32 arrays returned alongside hold the
exact values of those bf16 numbers, which the oracle widens to fp64.

Workloads (the pages' own workloads are tool-calling conversations with tool
tokens as segment 1 and chat as segment 2, packed training rows, and text
blocks; none ships with the pages, so these stand in for them):

  tiny       fp32  B1  1q/1kv  D32 T64   W16  seg 8x1 then 56x2, prefix = seg==1
  tiny_sink  fp32  B1  1q/1kv  D32 T64   W16  one segment, first 8 positions sinks
  needle     bf16  B8  8q/2kv  D64 T2048 W256 per-row sink prefix S_b ~ U{64..384}
                                              (seg 1), rest seg 2; RoPE theta 1e4
  packed     bf16  B16 16q/4kv D64 T4096 W256 per row 3..6 segments with random
                                              cuts, seg-0 padding tail U{0..511},
                                              prefix on the first 128 tokens
  compressed f32/bf16 B4 8q/8kv D64 T4096 W256 block 4 or 16, RoPE theta 1e4
  decode     bf16 q, int8 KV  B256 16q/4kv D64, ring W256 + 256 sinks,
                                              positions U{512..32767}, 12 layers
"""
from __future__ import annotations

import numpy as np


def bf16_round(x: np.ndarray):
    """Round float32 to bf16 (nearest-even).  Returns (bits uint16, values float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    r = ((u + bias) >> 16).astype(np.uint16)
    vals = (r.astype(np.uint32) << 16).view(np.float32)
    return r, vals


def _normals(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _pack(arr32, dtype):
    """Return dict entries for an input: exact values (float32) and bf16 bits if needed."""
    if dtype == "bf16":
        bits, vals = bf16_round(arr32)
        return vals, bits
    return np.ascontiguousarray(arr32, dtype=np.float32), None


def _qkv(rng, B, Hq, Hkv, T, D, dtype):
    q = _normals(rng, (B, Hq, T, D))
    k = _normals(rng, (B, Hkv, T, D))
    v = _normals(rng, (B, Hkv, T, D))
    out = {}
    for name, a in (("q", q), ("k", k), ("v", v)):
        vals, bits = _pack(a, dtype)
        out[name] = vals
        if bits is not None:
            out[name + "_bits"] = bits
    return out


def prefill_case(B, Hq, Hkv, T, D, window, dtype="bf16", seed=0, seg_ids=None, prefix=None,
                 rope_theta=0.0, compress_block=0):
    """Generic prefill workload with explicit structure (tests use this for sweeps)."""
    rng = np.random.default_rng(seed)
    w = _qkv(rng, B, Hq, Hkv, T, D, dtype)
    w.update(dict(B=B, Hq=Hq, Hkv=Hkv, T=T, D=D, window=window, dtype=dtype,
                  seg_ids=None if seg_ids is None else np.ascontiguousarray(seg_ids, dtype=np.int32),
                  prefix=None if prefix is None else np.ascontiguousarray(prefix, dtype=np.uint8),
                  rope_theta=rope_theta, compress_block=compress_block, seed=seed))
    return w


def tiny(seed=1):
    seg = np.array([[1] * 8 + [2] * 56], dtype=np.int32)
    return prefill_case(1, 1, 1, 64, 32, 16, "f32", seed, seg, (seg == 1).astype(np.uint8))


def tiny_sink(seed=11):
    seg = np.ones((1, 64), dtype=np.int32)
    prefix = np.zeros((1, 64), dtype=np.uint8)
    prefix[0, :8] = 1
    return prefill_case(1, 1, 1, 64, 32, 16, "f32", seed, seg, prefix)


def needle(seed=2, B=8, Hq=8, Hkv=2, T=2048, D=64, window=256):
    rng = np.random.default_rng(seed)
    w = _qkv(rng, B, Hq, Hkv, T, D, "bf16")
    sink_lens = rng.integers(64, 385, size=B)
    seg = np.full((B, T), 2, dtype=np.int32)
    for b in range(B):
        seg[b, : sink_lens[b]] = 1
    w.update(dict(B=B, Hq=Hq, Hkv=Hkv, T=T, D=D, window=window, dtype="bf16", seg_ids=seg,
                  prefix=(seg == 1).astype(np.uint8), rope_theta=10000.0, compress_block=0,
                  sink_lens=sink_lens, seed=seed))
    return w


def packed_structure(rng, B, T, prefix_len=128, min_seg=3, max_seg=6, max_pad=511):
    """Per row: k ~ U{min_seg..max_seg} segments, seg-0 padding tail ~ U{0..max_pad},
    cut points drawn without replacement from 1..T-pad-1 and sorted."""
    seg = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        k = int(rng.integers(min_seg, max_seg + 1))
        pad = int(rng.integers(0, max_pad + 1))
        used = T - pad
        cuts = np.sort(rng.choice(np.arange(1, used), size=k - 1, replace=False))
        bounds = [0] + list(cuts) + [used]
        for i in range(k):
            seg[b, bounds[i]:bounds[i + 1]] = i + 1
    prefix = np.zeros((B, T), dtype=np.uint8)
    prefix[:, :prefix_len] = 1
    return seg, prefix


def packed(seed=3, B=16, Hq=16, Hkv=4, T=4096, D=64, window=256):
    rng = np.random.default_rng(seed)
    w = _qkv(rng, B, Hq, Hkv, T, D, "bf16")
    seg, prefix = packed_structure(rng, B, T, prefix_len=min(128, T))
    w.update(dict(B=B, Hq=Hq, Hkv=Hkv, T=T, D=D, window=window, dtype="bf16", seg_ids=seg,
                  prefix=prefix, rope_theta=0.0, compress_block=0, seed=seed))
    return w


def causal(seed=8, B=4, Hq=16, Hkv=4, T=4096, D=64, window=0):
    """Plain causal GQA prefill (one segment, no sinks, no RoPE; window 0 = none): the kernel on long
    fully visible spans, for measurement beside the windowed workloads."""
    rng = np.random.default_rng(seed)
    w = _qkv(rng, B, Hq, Hkv, T, D, "bf16")
    w.update(dict(B=B, Hq=Hq, Hkv=Hkv, T=T, D=D, window=window, dtype="bf16", seg_ids=None,
                  prefix=None, rope_theta=0.0, compress_block=0, seed=seed))
    return w


def compressed(block=4, dtype="bf16", seed=4, B=4, H=8, T=4096, D=64, window=256):
    rng = np.random.default_rng(seed)
    w = _qkv(rng, B, H, H, T, D, dtype)
    w.update(dict(B=B, Hq=H, Hkv=H, T=T, D=D, window=window, dtype=dtype, seg_ids=None,
                  prefix=None, rope_theta=10000.0, compress_block=block, seed=seed))
    return w


def decode_case(seed=5, B=256, Hq=16, Hkv=4, D=64, W=256, S=256, pos_lo=512, pos_hi=32767,
                sink_len=None):
    """One layer of decode inputs as bf16 values (float32 exact + bits).

    Returns the pre-quantization caches (ring_k/ring_v/sink_k/sink_v [B,Hkv,W|S,D]),
    q [B,Hq,D], k_new/v_new [B,Hkv,D], pos [B] and sink_len [B].  Each side
    quantizes the caches with its own quantizer.
    """
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in (("q", (B, Hq, D)), ("k_new", (B, Hkv, D)), ("v_new", (B, Hkv, D)),
                        ("ring_k", (B, Hkv, W, D)), ("ring_v", (B, Hkv, W, D)),
                        ("sink_k", (B, Hkv, S, D)), ("sink_v", (B, Hkv, S, D))):
        bits, vals = bf16_round(_normals(rng, shape))
        out[name] = vals
        out[name + "_bits"] = bits
    out["pos"] = rng.integers(pos_lo, pos_hi + 1, size=B).astype(np.int32)
    if sink_len is None:
        out["sink_len"] = np.full(B, S, dtype=np.int32)
    else:
        out["sink_len"] = np.ascontiguousarray(sink_len, dtype=np.int32)
    out.update(dict(B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, S=S, seed=seed))
    return out


def compressed_decode_case(seed=6, B=256, Hq=16, Hkv=4, D=64, W=256, P=1024, block=4, pos_lo=0, pos_hi=4095):
    """One layer of compressed-decode inputs: q [B,Hq,D] and k_new [B,Hkv,D] (standing for rotated values),
    k_pre [B,Hkv,D] (standing for the key before rotation), v_new [B,Hkv,D], the pre-quantization ring and
    pooled caches [B,Hkv,W|P,D] (bf16 values), frontier sums front_k/front_v [B,Hkv,D] (float32, the sum of
    pos % block standard-normal rows' worth of spread) and pos [B]."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in (("q", (B, Hq, D)), ("k_new", (B, Hkv, D)), ("k_pre", (B, Hkv, D)), ("v_new", (B, Hkv, D)),
                        ("ring_k", (B, Hkv, W, D)), ("ring_v", (B, Hkv, W, D)),
                        ("pool_k", (B, Hkv, P, D)), ("pool_v", (B, Hkv, P, D))):
        bits, vals = bf16_round(_normals(rng, shape))
        out[name] = vals
        out[name + "_bits"] = bits
    pos = rng.integers(pos_lo, pos_hi + 1, size=B).astype(np.int32)
    spread = np.sqrt(np.maximum(pos % block, 1)).astype(np.float32)[:, None, None]
    out["front_k"] = (_normals(rng, (B, Hkv, D)) * spread).astype(np.float32)
    out["front_v"] = (_normals(rng, (B, Hkv, D)) * spread).astype(np.float32)
    out["pos"] = pos
    out.update(dict(B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, P=P, block=block, seed=seed))
    return out


def compressed_decode_sequence(seed=7, B=3, Hq=4, Hkv=2, D=64, T=150):
    """Per-step inputs of a decode run from an empty cache: q [T,B,Hq,D], k_new/k_pre/v_new [T,B,Hkv,D]
    (bf16 values and bits)."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in (("q", (T, B, Hq, D)), ("k_new", (T, B, Hkv, D)), ("k_pre", (T, B, Hkv, D)),
                        ("v_new", (T, B, Hkv, D))):
        bits, vals = bf16_round(_normals(rng, shape))
        out[name] = vals
        out[name + "_bits"] = bits
    out.update(dict(B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, seed=seed))
    return out


def chunk_case(seed=8, B=8, Hq=16, Hkv=4, D=64, W=256, S=256, Tc=4096, pos_lo=256, pos_hi=32767, sink_len=None):
    """Inputs of one chunked-prefill call: q [B,Hq,Tc,D], k/v [B,Hkv,Tc,D] (standing for rotated q and k), the
    pre-quantization ring and sink caches [B,Hkv,W|S,D] (bf16 values), pos0 [B] and sink_len [B]."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in (("q", (B, Hq, Tc, D)), ("k", (B, Hkv, Tc, D)), ("v", (B, Hkv, Tc, D)),
                        ("ring_k", (B, Hkv, W, D)), ("ring_v", (B, Hkv, W, D)),
                        ("sink_k", (B, Hkv, S, D)), ("sink_v", (B, Hkv, S, D))):
        bits, vals = bf16_round(_normals(rng, shape))
        out[name] = vals
        out[name + "_bits"] = bits
    out["pos0"] = rng.integers(pos_lo, pos_hi + 1, size=B).astype(np.int32)
    out["sink_len"] = (np.full(B, S, dtype=np.int32) if sink_len is None
                       else np.ascontiguousarray(sink_len, dtype=np.int32))
    out.update(dict(B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, S=S, Tc=Tc, seed=seed))
    return out
