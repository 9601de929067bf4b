"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks an oracle function against a library routine, a closed form,
a value worked out by hand from the pages, an invariant, or brute force on tiny
inputs, chosen so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.

Sources: [NW] "How the 256-Token Sliding Window Works with Tools as KV Sinks in
Needle"; [NS] "256-token滑动窗口+KV sink：Needle 2工具钉住机制源码分析"; [CA]
"Compressed attention and the copy probe".
"""
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from compressed_kv_attention_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa(q, k, v, mask=None, causal=False, scale=None):
    """Reference attention from torch (fp64, CPU).  q [..., T, D], k/v [..., S, D]."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)) for a in (q, k, v))
    m = None if mask is None else torch.from_numpy(np.asarray(mask, dtype=bool))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal,
                                                         scale=scale)
    return o.numpy()


def band(T, W):
    """Lower band of width W built from library routines: tril(ones) - tril(ones, -W)."""
    ones = np.ones((T, T), dtype=np.int64)
    return (np.tril(ones) - np.tril(ones, -W)).astype(bool)


# --------------------------------------------------------------------------
# O1 mask  [NW §"KV Sinks for Tools: Pinning Critical Context"]
# --------------------------------------------------------------------------

def test_mask_worked_example_golden():
    lines = [l for l in open(os.path.join(GOLDEN, "needle_example_mask.txt")) if not l.startswith("#")]
    shape = tuple(int(x) for x in lines[0].split()[1:])
    seg = np.array([[int(x) for x in lines[1].split()[1:]]], dtype=np.int32)
    prefix = np.array([[int(x) for x in lines[2].split()[1:]]], dtype=np.uint8)
    window = int(lines[3].split()[1])
    expect = np.array([[int(x) for x in l.split()] for l in lines[4:4 + 8]], dtype=np.uint8)
    got = oracle.mask(seg, prefix, window)
    assert (1, 1) + got.shape[1:] == shape            # the page prints (1, 1, 8, 8)
    np.testing.assert_array_equal(got[0], expect)


@pytest.mark.parametrize("T", [1, 7, 33])
def test_mask_full_window_one_segment_is_tril(T):
    seg = np.ones((1, T), dtype=np.int32)
    for W in (0, T, T + 5):
        np.testing.assert_array_equal(oracle.mask(seg, None, W)[0], np.tril(np.ones((T, T), np.uint8)))


@pytest.mark.parametrize("T,W", [(16, 1), (16, 3), (40, 7), (40, 39)])
def test_mask_window_band(T, W):
    seg = np.ones((1, T), dtype=np.int32)
    got = oracle.mask(seg, None, W)[0].astype(bool)
    np.testing.assert_array_equal(got, band(T, W))
    if W == 1:
        np.testing.assert_array_equal(got, np.eye(T, dtype=bool))


def test_mask_segments_block_diagonal():
    lens = [5, 1, 9, 3]
    seg = np.concatenate([np.full(n, i + 1) for i, n in enumerate(lens)])[None].astype(np.int32)
    T = seg.shape[1]
    expect = scipy.linalg.block_diag(*[np.tril(np.ones((n, n))) for n in lens]).astype(np.uint8)
    np.testing.assert_array_equal(oracle.mask(seg, None, 0)[0], expect)
    # windowed: each diagonal block becomes a band
    W = 2
    expect_w = scipy.linalg.block_diag(*[band(n, W).astype(float) for n in lens]).astype(np.uint8)
    np.testing.assert_array_equal(oracle.mask(seg, None, W)[0], expect_w)
    # padding (segment 0) rows and columns are empty
    seg0 = seg.copy()
    seg0[0, -3:] = 0
    m = oracle.mask(seg0, None, 0)[0]
    assert m[-3:, :].sum() == 0 and m[:, -3:].sum() == 0
    assert T == m.shape[0]


def test_mask_sinks_within_one_segment():
    T, W, P = 30, 4, 5
    seg = np.ones((1, T), dtype=np.int32)
    prefix = np.zeros((1, T), dtype=np.uint8)
    prefix[0, :P] = 1
    got = oracle.mask(seg, prefix, W)[0].astype(bool)
    sink_cols = np.zeros((T, T), dtype=bool)
    sink_cols[:, :P] = True
    expect = band(T, W) | (np.tril(np.ones((T, T), dtype=bool)) & sink_cols)
    np.testing.assert_array_equal(got, expect)
    # window 0 switches windowing (and therefore the sinks) off: plain causal
    np.testing.assert_array_equal(oracle.mask(seg, prefix, 0)[0], np.tril(np.ones((T, T), np.uint8)))


def test_mask_sinks_do_not_cross_segments():
    # tools (segment 1, sinks) then chat (segment 2): chat rows never see the tools
    T, S, W = 24, 6, 4
    seg = np.array([[1] * S + [2] * (T - S)], dtype=np.int32)
    m = oracle.mask(seg, (seg == 1).astype(np.uint8), W)[0]
    assert m[S:, :S].sum() == 0
    np.testing.assert_array_equal(m[:S, :S], np.tril(np.ones((S, S), np.uint8)))


def test_mask_needle_counts_closed_form():
    # needle structure: row t sees t+1 keys inside the sink prefix, then
    # min(t - S + 1, W) keys of its own segment.
    T, W = 700, 256
    for S in (64, 200, 384):
        seg = np.array([[1] * S + [2] * (T - S)], dtype=np.int32)
        n = oracle.mask(seg, (seg == 1).astype(np.uint8), W)[0].sum(axis=1)
        t = np.arange(T)
        expect = np.where(t < S, t + 1, np.minimum(t - S + 1, W))
        np.testing.assert_array_equal(n, expect)


def test_mask_brute_force_random_small():
    # brute force: visible iff key is in the row's segment (equality, also for
    # repeated non-contiguous ids), not in the future, and inside the window
    # or a sink; rows of segment 0 see nothing.
    rng = np.random.default_rng(123)
    for _ in range(200):
        T = int(rng.integers(1, 20))
        seg = rng.integers(0, 4, size=(1, T)).astype(np.int32)
        prefix = (rng.random((1, T)) < 0.3).astype(np.uint8)
        W = int(rng.choice([0, 1, 2, 3, 5, T, T + 1]))
        got = oracle.mask(seg, prefix, W)[0]
        for q in range(T):
            for k in range(T):
                ok = seg[0, q] > 0 and seg[0, k] == seg[0, q] and k <= q
                if W:
                    ok = ok and (q - k < W or prefix[0, k] > 0)
                assert got[q, k] == int(ok), (T, W, q, k)


# --------------------------------------------------------------------------
# O2 RoPE (rotate-half; the pairing convention itself is parity-unpinned)
# --------------------------------------------------------------------------

def test_rope_invariants():
    rng = np.random.default_rng(7)
    D = 64
    x = rng.standard_normal((50, D))
    np.testing.assert_allclose(oracle.rope(x, np.zeros(50), 10000.0), x, atol=0, rtol=0)
    pos = rng.integers(0, 5000, 50)
    y = oracle.rope(x, pos, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # relative position: <R_m q, R_n k> = <R_{m-n} q, k>
    q, k = rng.standard_normal((2, 20, D))
    m, n = rng.integers(0, 4000, 20), rng.integers(0, 4000, 20)
    lhs = np.sum(oracle.rope(q, m, 1e4) * oracle.rope(k, n, 1e4), axis=1)
    rhs = np.sum(oracle.rope(q, m - n, 1e4) * k, axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-9)
    # composition: R_a R_b = R_{a+b}
    a, b = rng.integers(0, 2000, 20), rng.integers(0, 2000, 20)
    np.testing.assert_allclose(oracle.rope(oracle.rope(q, a, 1e4), b, 1e4), oracle.rope(q, a + b, 1e4),
                               rtol=1e-9, atol=1e-9)


def test_rope_frequencies():
    # pair i (channels i and i + D/2) turns by pos * theta^(-2i/D) radians
    D, theta = 16, 10000.0
    for i in range(D // 2):
        e = np.zeros((1, D))
        e[0, i] = 1.0
        for p in (1, 3, 17):
            y = oracle.rope(e, [p], theta)[0]
            ang = math.atan2(y[i + D // 2], y[i])
            expect = math.remainder(p * theta ** (-2.0 * i / D), 2 * math.pi)
            assert abs(math.remainder(ang - expect, 2 * math.pi)) < 1e-12
            others = np.delete(y, [i, i + D // 2])
            assert np.all(others == 0)


# --------------------------------------------------------------------------
# O3 attention
# --------------------------------------------------------------------------

def _case(B, Hq, Hkv, T, D, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, T, D)), rng.standard_normal((B, Hkv, T, D)),
            rng.standard_normal((B, Hkv, T, D)))


def test_prefill_full_causal_matches_sdpa():
    q, k, v = _case(2, 2, 2, 37, 16, seed=1)
    out, lse = oracle.prefill(q, k, v, None, None, 0)
    np.testing.assert_allclose(out, sdpa(q, k, v, causal=True), rtol=1e-12, atol=1e-12)
    out2, _ = oracle.prefill(q, k, v, np.ones((2, 37), np.int32), None, 37)
    np.testing.assert_allclose(out2, out, rtol=0, atol=0)
    # lse against a direct log-sum-exp
    s = np.einsum("bhtd,bhsd->bhts", q, k) / 4.0
    s = np.where(np.tril(np.ones((37, 37), bool)), s, -np.inf)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=1e-12)


def test_prefill_gqa_matches_repeated_heads():
    q, k, v = _case(1, 6, 2, 29, 8, seed=2)
    out, _ = oracle.prefill(q, k, v, None, None, 5)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)   # head h reads kv head h // 3
    np.testing.assert_allclose(out, sdpa(q, kr, vr, mask=band(29, 5)), rtol=1e-12, atol=1e-12)


def test_prefill_segments_and_sinks_match_sdpa_with_explicit_mask():
    T, W, P = 48, 6, 4
    lens = [20, 28]
    seg = np.concatenate([np.full(n, i + 1) for i, n in enumerate(lens)])[None].astype(np.int32)
    prefix = np.zeros((1, T), np.uint8)
    prefix[0, :P] = 1
    prefix[0, 20:20 + P] = 1
    q, k, v = _case(1, 2, 1, T, 16, seed=3)
    blocks = []
    for n in lens:
        sink_cols = np.zeros((n, n), bool)
        sink_cols[:, :P] = True
        blocks.append((band(n, W) | (np.tril(np.ones((n, n), bool)) & sink_cols)).astype(float))
    m = scipy.linalg.block_diag(*blocks).astype(bool)
    out, _ = oracle.prefill(q, k, v, seg, prefix, W)
    np.testing.assert_allclose(out, sdpa(q, np.repeat(k, 2, 1), np.repeat(v, 2, 1), mask=m),
                               rtol=1e-12, atol=1e-12)


def test_prefill_special_cases():
    T = 25
    q, k, v = _case(1, 1, 1, T, 8, seed=4)
    seg = np.ones((1, T), np.int32)
    # W = 1: each row sees only itself
    out, lse = oracle.prefill(q, k, v, seg, None, 1)
    np.testing.assert_allclose(out[0, 0], v[0, 0], rtol=0, atol=1e-15)
    # q = 0: uniform weights, output = mean of the visible values, lse = ln(n_vis)
    W = 7
    out, lse = oracle.prefill(np.zeros_like(q), k, v, seg, None, W)
    for t in range(T):
        lo = max(0, t - W + 1)
        np.testing.assert_allclose(out[0, 0, t], v[0, 0, lo:t + 1].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert abs(lse[0, 0, t] - math.log(t + 1 - lo)) < 1e-13
    # padding rows: output 0 and lse -inf
    seg0 = seg.copy()
    seg0[0, -4:] = 0
    out, lse = oracle.prefill(q, k, v, seg0, None, W)
    assert np.all(out[0, 0, -4:] == 0) and np.all(np.isneginf(lse[0, 0, -4:]))


def test_prefill_rope_matches_sdpa_on_rotated_inputs():
    B, H, T, D = 1, 2, 33, 16
    q, k, v = _case(B, H, H, T, D, seed=5)
    pos = np.arange(T)
    qr = np.stack([[oracle.rope(q[b, h], pos, 1e4) for h in range(H)] for b in range(B)])
    kr = np.stack([[oracle.rope(k[b, h], pos, 1e4) for h in range(H)] for b in range(B)])
    out, _ = oracle.prefill(q, k, v, None, None, 9, theta=1e4)
    np.testing.assert_allclose(out, sdpa(qr, kr, v, mask=band(T, 9)), rtol=1e-12, atol=1e-12)


def test_prefill_row_sampling_matches_full():
    q, k, v = _case(2, 4, 2, 40, 8, seed=6)
    seg = np.array([[1] * 10 + [2] * 30, [3] * 40], np.int32)
    pre = np.zeros((2, 40), np.uint8)
    pre[:, :3] = 1
    full, lse = oracle.prefill(q, k, v, seg, pre, 5, theta=1e4)
    rows = np.array([0, 17, 39, 40 * 4 + 3, 2 * 4 * 40 - 1])
    part, lse_p = oracle.prefill(q, k, v, seg, pre, 5, theta=1e4, rows=rows)
    np.testing.assert_array_equal(part, full.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(lse_p, lse.reshape(-1)[rows])


# --------------------------------------------------------------------------
# O4 compressed attention  [CA]
# --------------------------------------------------------------------------

def test_compressed_mask_invariants():
    for T, W, b in ((64, 8, 4), (100, 16, 3), (4096, 256, 4), (4096, 256, 16)):
        m = oracle.compressed_mask(T, W, b).astype(bool)
        nblk = T // b
        pooled, exact = m[:, :nblk], m[:, nblk:]
        np.testing.assert_array_equal(exact, band(T, W))
        nv = pooled.sum(axis=1)
        # staircase: each row's visible blocks are a prefix, growing by at most one per row
        for q in range(T):
            assert pooled[q, :nv[q]].all() and not pooled[q, nv[q]:].any()
        assert set(np.diff(nv).tolist()) <= {0, 1}
        # early rows see only exact keys
        assert nv[: W + b - 1].sum() == 0
        for q in range(T):
            covered_pooled = set(range(nv[q] * b))
            covered_exact = set(range(max(0, q - W + 1), q + 1))
            assert not (covered_pooled & covered_exact)          # no token counted twice
            if q >= W - 1:
                gap = (q - W + 1) - nv[q] * b
                assert gap == (q - W + 1) % b if nv[q] < nblk else gap >= 0


def test_compressed_cache_size_figure():
    # [CA §"So what happened ?"]: at 4K positions, window 256, block 4 the cache
    # drops from 4 MiB to about 1.2 MiB: the last row reads 960 pooled + 256 exact columns.
    m = oracle.compressed_mask(4096, 256, 4)
    cols = int(m[-1].sum())
    assert cols == 960 + 256
    mib = 4.0 * cols / 4096
    assert mib == 1.1875 and round(mib, 1) == 1.2
    assert int(oracle.compressed_mask(4096, 256, 16)[-1].sum()) == 240 + 256


def test_pool_means_match_reshape_mean():
    rng = np.random.default_rng(8)
    k, v = rng.standard_normal((2, 3, 2, 23, 8))
    for b in (1, 2, 4, 5):
        pk, pv = oracle.pool_rope(k, v, b, theta=0.0)
        n = (23 // b) * b
        np.testing.assert_allclose(pk, k[..., :n, :].reshape(3, 2, 23 // b, b, 8).mean(axis=3), rtol=1e-14)
        np.testing.assert_allclose(pv, v[..., :n, :].reshape(3, 2, 23 // b, b, 8).mean(axis=3), rtol=1e-14)


def test_pool_then_rotate_at_midpoint():
    rng = np.random.default_rng(9)
    T, D, b = 32, 16, 4
    k, v = rng.standard_normal((2, 1, T, D))
    pk, pv = oracle.pool_rope(k, v, b, theta=1e4, rope_len=T)
    mean = k[0].reshape(T // b, b, D).mean(axis=1)
    mids = np.arange(T // b) * b + b // 2
    np.testing.assert_allclose(pk[0], oracle.rope(mean, mids, 1e4), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(pv[0], v[0].reshape(T // b, b, D).mean(axis=1), rtol=1e-14)
    # linearity: rotating every key of a block at the midpoint angle, then pooling, is the same
    rot_all = oracle.rope(k[0], np.repeat(mids, b), 1e4).reshape(T // b, b, D).mean(axis=1)
    np.testing.assert_allclose(pk[0], rot_all, rtol=1e-12, atol=1e-13)
    # midpoints past the table are clamped to rope_len - 1
    pk2, _ = oracle.pool_rope(k, v, b, theta=1e4, rope_len=10)
    np.testing.assert_allclose(pk2[0], oracle.rope(mean, np.minimum(mids, 9), 1e4), rtol=1e-13, atol=1e-14)


def test_pool_before_rotate_keeps_norm():
    # [CA §"Pool before rotating, not after"]: averaging keys that were already
    # rotated at different positions shortens the average; pooling first does not.
    rng = np.random.default_rng(10)
    D, b = 64, 16
    key = np.tile(rng.standard_normal((1, D)), (b, 1))   # the same key at b positions
    pk, _ = oracle.pool_rope(key[None], key[None], b, theta=1e4, rope_len=b)
    after = oracle.rope(key, np.arange(b), 1e4).mean(axis=0)
    assert abs(np.linalg.norm(pk[0, 0]) - np.linalg.norm(key[0])) < 1e-12
    assert np.linalg.norm(after) < 0.95 * np.linalg.norm(key[0])


def test_compressed_block1_reduces_to_full_causal_rope_attention():
    # with b = 1 every pooled column is one key rotated at its own position and
    # visible exactly when it has left the window, so pooled + exact columns
    # cover [0, t] once each.
    B, H, T, D = 1, 2, 40, 16
    q, k, v = _case(B, H, H, T, D, seed=11)
    out, lse = oracle.compressed_prefill(q, k, v, window=6, block=1, theta=1e4)
    pos = np.arange(T)
    qr = np.stack([oracle.rope(q[0, h], pos, 1e4) for h in range(H)])[None]
    kr = np.stack([oracle.rope(k[0, h], pos, 1e4) for h in range(H)])[None]
    np.testing.assert_allclose(out, sdpa(qr, kr, v, causal=True), rtol=1e-12, atol=1e-12)
    full, lse_full = oracle.prefill(q, k, v, None, None, 0, theta=1e4)
    np.testing.assert_allclose(lse, lse_full, rtol=1e-12)


def test_compressed_window_covers_all_means_no_pooled_columns():
    B, H, T, D = 1, 1, 30, 8
    q, k, v = _case(B, H, H, T, D, seed=12)
    out, _ = oracle.compressed_prefill(q, k, v, window=T, block=4, theta=1e4)
    ref, _ = oracle.prefill(q, k, v, None, None, T, theta=1e4)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)


def test_compressed_q0_counts_and_means():
    B, H, T, D, W, b = 1, 1, 50, 8, 8, 4
    _, k, v = _case(B, H, H, T, D, seed=13)
    out, lse = oracle.compressed_prefill(np.zeros((B, H, T, D)), k, v, window=W, block=b, theta=1e4)
    pv = v[0, 0, :(T // b) * b].reshape(T // b, b, D).mean(axis=1)
    for t in range(T):
        nb = max(0, (t - W + 1) // b)
        lo = max(0, t - W + 1)
        cols = np.concatenate([pv[:nb], v[0, 0, lo:t + 1]])
        np.testing.assert_allclose(out[0, 0, t], cols.mean(axis=0), rtol=1e-12, atol=1e-14)
        assert abs(lse[0, 0, t] - math.log(len(cols))) < 1e-12


# --------------------------------------------------------------------------
# O5 budget window  [NW §"Effective KV Window"], [NS §"256 这个窗口宽度从哪来"]
# --------------------------------------------------------------------------

def test_budget_constants_and_cases():
    assert 11 * 1024 * 1024 + 512 * 1024 == 12058624
    rows = [l.split() for l in open(os.path.join(GOLDEN, "budget_window.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) >= 8
    for r in rows:
        d, ad, nh, nkv, L, sites, msl, kvw, per_pos, bw, eff = (int(x) for x in r)
        assert oracle.kv_budget_per_pos(d, nh, nkv, L, sites, ad) == per_pos, r
        assert oracle.kv_budget_window(d, nh, nkv, L, msl, sites, ad) == bw, r
        assert oracle.effective_kv_window(d, nh, nkv, L, msl, kvw, sites, ad) == eff, r


def test_budget_window_is_256_band():
    # the budget window alone is 256 exactly when per_pos lies in [41871, 47104]
    budget = 12058624
    for per_pos in (41870, 41871, 45000, 47104, 47105):
        raw = (budget // per_pos) // 32 * 32
        assert (raw == 256) == (41871 <= per_pos <= 47104)


# --------------------------------------------------------------------------
# O6 int8 quantizer (scheme is reading R-A13)
# --------------------------------------------------------------------------

def test_quantizer_properties():
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((300, 64)) * rng.uniform(0.01, 10, (300, 1))).astype(np.float32)
    x[5, :32] = 0.0                                   # an all-zero group
    q, s = oracle.quantize(x)
    assert q.dtype == np.int8 and s.shape == (300, 2)
    assert q.min() >= -127 and q.max() <= 127
    assert np.all(q[5, :32] == 0) and s[5, 0] == 0
    xg = x.reshape(300, 2, 32)
    qg = q.reshape(300, 2, 32).astype(np.float64)
    amax = np.abs(xg).max(axis=2)
    np.testing.assert_array_equal(s, (amax / np.float32(127)).astype(np.float32))
    err = np.abs(xg - qg * s[..., None])
    assert np.all(err <= s[..., None] * (0.5 + 1e-5) + 1e-30)
    # the largest element of each group maps to +-127
    idx = np.abs(xg).argmax(axis=2)
    top = np.take_along_axis(qg, idx[..., None], 2)[..., 0]
    nz = amax > 0
    np.testing.assert_array_equal(np.abs(top[nz]), 127)


def test_quantizer_rounds_half_to_even():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0                                   # scale becomes exactly 1
    x[0, 1:7] = [2.5, 3.5, -2.5, -3.5, 0.5, 1.5]
    q, s = oracle.quantize(x)
    assert s[0, 0] == 1.0
    assert q[0, :7].tolist() == [127, 2, 4, -2, -4, 0, 2]


# --------------------------------------------------------------------------
# O7 decode  [NS §"256-token 滑动窗口：源码走读"]
# --------------------------------------------------------------------------

def _decode_inputs(B=3, Hq=4, Hkv=2, D=64, W=8, S=5, seed=15, pos=None, sink_len=None):
    w = workloads.decode_case(seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, S=S, pos_lo=0, pos_hi=40,
                              sink_len=sink_len)
    if pos is not None:
        w["pos"] = np.asarray(pos, np.int32)
    rk, rks = oracle.quantize(w["ring_k"].reshape(-1, D))
    rv, rvs = oracle.quantize(w["ring_v"].reshape(-1, D))
    sk, sks = oracle.quantize(w["sink_k"].reshape(-1, D))
    sv, svs = oracle.quantize(w["sink_v"].reshape(-1, D))
    g = D // 32
    caches = dict(ring_k=rk.reshape(B, Hkv, W, D), ring_v=rv.reshape(B, Hkv, W, D),
                  ring_ks=rks.reshape(B, Hkv, W, g), ring_vs=rvs.reshape(B, Hkv, W, g),
                  sink_k=sk.reshape(B, Hkv, S, D), sink_v=sv.reshape(B, Hkv, S, D),
                  sink_ks=sks.reshape(B, Hkv, S, g), sink_vs=svs.reshape(B, Hkv, S, g))
    return w, caches


def test_decode_matches_sdpa_over_visible_rows():
    B, Hq, Hkv, D, W, S = 4, 4, 2, 64, 8, 5
    pos = [5, 7, 12, 33]                      # partial ring, exactly full, wrapped twice
    sink_len = [5, 3, 5, 0]
    w, c = _decode_inputs(B, Hq, Hkv, D, W, S, pos=pos, sink_len=sink_len)
    out, lse, rk, rv, rks, rvs = oracle.decode(w["q"], c["ring_k"], c["ring_v"], c["ring_ks"],
                                               c["ring_vs"], c["sink_k"], c["sink_v"], c["sink_ks"],
                                               c["sink_vs"], w["pos"], w["sink_len"], w["k_new"],
                                               w["v_new"])
    G = Hq // Hkv
    for b in range(B):
        p, sl = pos[b], sink_len[b]
        # the append wrote the quantized new token into slot p % W and nothing else
        kq, ks = oracle.quantize(w["k_new"][b])
        np.testing.assert_array_equal(rk[b, :, p % W], kq)
        np.testing.assert_array_equal(rks[b, :, p % W], ks)
        others = [s for s in range(W) if s != p % W]
        np.testing.assert_array_equal(rk[b][:, others], c["ring_k"][b][:, others])
        ring_pos = list(range(max(sl, p - W + 1), p + 1))
        assert len(ring_pos) + sl == sl + min(W, p - sl + 1)
        for h in range(Hq):
            hk = h // G
            kd = np.concatenate([c["sink_k"][b, hk, :sl].astype(np.float64) * np.repeat(c["sink_ks"][b, hk, :sl], 32, 1),
                                 np.stack([rk[b, hk, x % W].astype(np.float64) * np.repeat(rks[b, hk, x % W], 32) for x in ring_pos])])
            vd = np.concatenate([c["sink_v"][b, hk, :sl].astype(np.float64) * np.repeat(c["sink_vs"][b, hk, :sl], 32, 1),
                                 np.stack([rv[b, hk, x % W].astype(np.float64) * np.repeat(rvs[b, hk, x % W], 32) for x in ring_pos])])
            ref = sdpa(w["q"][b, h][None].astype(np.float64), kd.astype(np.float64), vd.astype(np.float64))
            np.testing.assert_allclose(out[b, h], ref[0], rtol=1e-12, atol=1e-12)


def test_decode_q0_is_mean_and_counts():
    B, Hq, Hkv, D, W, S = 2, 2, 1, 32, 6, 4
    w, c = _decode_inputs(B, Hq, Hkv, D, W, S, seed=16, pos=[4, 30], sink_len=[4, 2])
    out, lse, *_ = oracle.decode(np.zeros((B, Hq, D)), c["ring_k"], c["ring_v"], c["ring_ks"],
                                 c["ring_vs"], c["sink_k"], c["sink_v"], c["sink_ks"], c["sink_vs"],
                                 w["pos"], w["sink_len"], w["k_new"], w["v_new"])
    for b, (p, sl) in enumerate(zip([4, 30], [4, 2])):
        n = sl + min(W, p - sl + 1)
        np.testing.assert_allclose(np.exp(lse[b]), n, rtol=1e-12)


def test_decode_equals_prefill_row_with_sink_prefix():
    # decode of the token at position p equals row p of the prefill mask with one
    # segment and sinks on [0, sink_len), over the same dequantized keys/values.
    D, W, S, p, sl = 32, 6, 4, 17, 4
    w, c = _decode_inputs(1, 1, 1, D, W, S, seed=17, pos=[p], sink_len=[sl])
    out, _, rk, rv, rks, rvs = oracle.decode(w["q"], c["ring_k"], c["ring_v"], c["ring_ks"],
                                             c["ring_vs"], c["sink_k"], c["sink_v"], c["sink_ks"],
                                             c["sink_vs"], w["pos"], w["sink_len"], w["k_new"],
                                             w["v_new"])
    T = p + 1
    K = np.zeros((1, 1, T, D))
    V = np.zeros((1, 1, T, D))
    for t in range(sl):
        K[0, 0, t] = c["sink_k"][0, 0, t].astype(np.float64) * np.repeat(c["sink_ks"][0, 0, t], 32)
        V[0, 0, t] = c["sink_v"][0, 0, t].astype(np.float64) * np.repeat(c["sink_vs"][0, 0, t], 32)
    for t in range(max(sl, p - W + 1), p + 1):
        K[0, 0, t] = rk[0, 0, t % W].astype(np.float64) * np.repeat(rks[0, 0, t % W], 32)
        V[0, 0, t] = rv[0, 0, t % W].astype(np.float64) * np.repeat(rvs[0, 0, t % W], 32)
    Q = np.zeros((1, 1, T, D))
    Q[0, 0, p] = w["q"][0, 0]
    prefix = np.zeros((1, T), np.uint8)
    prefix[0, :sl] = 1
    ref, _ = oracle.prefill(Q, K, V, np.ones((1, T), np.int32), prefix, W, rows=[p])
    np.testing.assert_allclose(out[0, 0], ref[0], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# O8 compressed decode  [CA §"Two kinds of columns, pooled blocks and exact
# recent keys", §"Pool before rotating, not after", §"So what happened ?"]
# --------------------------------------------------------------------------

def _compressed_sequence(q, k, v, W, b, P, theta, rope_len, quantize, t_end=None):
    """Run O8 from an empty state over positions 0 .. t_end-1 of q/k/v [B,H,T,D] (pre-RoPE); q and k are
    rotated at their position with O2 before each step.  Returns the outputs [B,Hq,T,D], lse and the state."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    t_end = T if t_end is None else t_end
    st = oracle.compressed_decode_state(B, Hkv, D, W, P)
    outs, lses = [], []
    for t in range(t_end):
        pos = np.full(B, t, np.int32)
        qr = np.stack([oracle.rope(q[bb, :, t], np.full(Hq, t), theta) for bb in range(B)])
        kr = np.stack([oracle.rope(k[bb, :, t], np.full(Hkv, t), theta) for bb in range(B)])
        o, l, st = oracle.compressed_decode(qr, kr, k[:, :, t], v[:, :, t], st, pos, b, theta=theta,
                                            rope_len=rope_len, quantize=quantize)
        outs.append(o)
        lses.append(l)
    return np.stack(outs, axis=2), np.stack(lses, axis=2), st


@pytest.mark.parametrize("W,b,rope_len", [(5, 3, 41), (8, 4, 41), (8, 4, 20), (3, 1, 41), (50, 4, 41)])
def test_compressed_decode_sequence_equals_compressed_prefill(W, b, rope_len):
    # Decoding a sequence token by token from an empty cache reproduces every row
    # of the compressed prefill over the same pre-RoPE keys: the frontier, the
    # pooling at block completion, the midpoint rotation, the visibility and
    # the ring slots all have to agree with the pooled-then-attend definition.
    B, Hq, Hkv, T, D = 2, 4, 2, 41, 16
    q, k, v = _case(B, Hq, Hkv, T, D, seed=40 + W + b)
    P = (T + b - 1) // b
    out, lse, _ = _compressed_sequence(q, k, v, W, b, P, 1e4, rope_len, quantize=False)
    ref, ref_lse = oracle.compressed_prefill(q, k, v, window=W, block=b, theta=1e4, rope_len=rope_len)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


def test_compressed_decode_block1_is_full_causal_attention():
    # b = 1: each pooled block is one key rotated at its own position, so the
    # columns cover [0, t] once each: causal attention from the library.
    B, H, T, D = 1, 2, 30, 8
    q, k, v = _case(B, H, H, T, D, seed=47)
    out, _, _ = _compressed_sequence(q, k, v, 4, 1, T, 1e4, T, quantize=False)
    pos = np.arange(T)
    qr = np.stack([oracle.rope(q[0, h], pos, 1e4) for h in range(H)])[None]
    kr = np.stack([oracle.rope(k[0, h], pos, 1e4) for h in range(H)])[None]
    np.testing.assert_allclose(out, sdpa(qr, kr, v, causal=True), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("b,pooled", [(4, 960), (16, 240)])
def test_compressed_decode_column_count_figure(b, pooled):
    # [CA §"So what happened ?"]: at 4K positions with a 256 window the last
    # token reads 960 pooled blocks (block 4) + 256 exact keys = 1216 columns,
    # 1216 / 4096 of the 4 MiB cache, about 1.2 MiB.  With q = 0 the output is
    # the plain mean of the visible values and exp(lse) counts the columns.
    T, W, D = 4096, 256, 4
    rng = np.random.default_rng(48)
    k, v = rng.standard_normal((2, 1, 1, T, D))
    q = np.zeros((1, 1, T, D))
    st = oracle.compressed_decode_state(1, 1, D, W, T // b)
    for t in range(T):
        pos = np.array([t], np.int32)
        o, lse, st = oracle.compressed_decode(q[:, :, t], oracle.rope(k[0, :, t], [t], 1e4)[None], k[:, :, t],
                                              v[:, :, t], st, pos, b, theta=1e4, quantize=False)
    assert round(math.exp(lse[0, 0])) == pooled + W
    cols = np.concatenate([v[0, 0].reshape(T // b, b, D).mean(axis=1)[:pooled], v[0, 0, T - W:]])
    np.testing.assert_allclose(o[0, 0], cols.mean(axis=0), rtol=1e-12, atol=1e-14)
    assert 4.0 * (pooled + W) / T == (1.1875 if b == 4 else 0.484375)


def test_compressed_decode_quantized_state_and_edges():
    B, Hq, Hkv, T, D, W, b = 2, 2, 1, 37, 32, 6, 4
    q, k, v = _case(B, Hq, Hkv, T, D, seed=49)
    P = T // b                                          # the last, partial block has no slot
    _, _, st_exact = _compressed_sequence(q, k, v, W, b, P, 1e4, T, quantize=False)
    out_q, _, st_q = _compressed_sequence(q, k, v, W, b, P, 1e4, T, quantize=True)
    out_x, _, _ = _compressed_sequence(q, k, v, W, b, P, 1e4, T, quantize=False)
    # every stored row of the int8 cache is the O6 quantization of the exact row
    for name in ("ring_k", "ring_v", "pool_k", "pool_v"):
        x = st_exact[name].reshape(-1, D)
        xq, xs = oracle.quantize(x.astype(np.float32))
        np.testing.assert_array_equal(st_q[name].reshape(-1, D), xq.astype(np.float64) * np.repeat(xs, 32, 1))
    # the frontier holds the sum of the partial block's pre-RoPE keys and values
    lo = (T - 1) // b * b
    np.testing.assert_allclose(st_exact["front_k"], k[:, :, lo:T].sum(axis=2), rtol=1e-14)
    np.testing.assert_allclose(st_exact["front_v"], v[:, :, lo:T].sum(axis=2), rtol=1e-14)
    # int8 caches change the output by no more than the quantization noise
    assert np.abs(out_q - out_x).max() < 0.05
    # pos < 0: nothing appended, no column visible
    qr = np.ones((B, Hq, D))
    o, lse, st2 = oracle.compressed_decode(qr, k[:, :, 0], k[:, :, 0], v[:, :, 0], st_q,
                                           np.array([-1, -5], np.int32), b, theta=1e4, quantize=True)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    for name in oracle.COMPRESSED_STATE:
        np.testing.assert_array_equal(st2[name], st_q[name])


def test_compressed_decode_pool_capacity_drops_later_blocks():
    # blocks past the pooled cache's capacity P are dropped: at most P pooled columns
    T, W, b, D, P = 60, 4, 4, 8, 5
    rng = np.random.default_rng(50)
    k, v = rng.standard_normal((2, 1, 1, T, D))
    st = oracle.compressed_decode_state(1, 1, D, W, P)
    for t in range(T):
        o, lse, st = oracle.compressed_decode(np.zeros((1, 1, D)), k[:, :, t], k[:, :, t], v[:, :, t], st,
                                              np.array([t], np.int32), b, theta=0.0, quantize=False)
        n_pool = min(P, max(0, (t - W + 1) // b))
        assert round(math.exp(lse[0, 0])) == n_pool + min(W, t + 1)
    np.testing.assert_allclose(st["pool_v"][0, 0], v[0, 0, :P * b].reshape(P, b, D).mean(axis=1), rtol=1e-14)


# --------------------------------------------------------------------------
# O9 chunked prefill into existing caches (reading A20; decode mask of
# [NS §"256-token 滑动窗口：源码走读"])
# --------------------------------------------------------------------------

def _dequant(codes, scales):
    return codes.astype(np.float64) * np.repeat(scales.astype(np.float64), 32, axis=-1)


@pytest.mark.parametrize("W,S,Tc,pos0,sink_len", [
    (8, 5, 13, [5, 20, 40], [5, 3, 0]),      # empty ring after the sinks, a wrapped ring, no sinks
    (8, 5, 3, [9, 30, 2], [5, 5, 5]),        # a chunk shorter than the window; sink_len > pos0 (clamped)
    (64, 0, 20, [0, 7, 100], None),          # no sink cache; an empty cache at position 0
])
def test_chunk_prefill_equals_prefill_over_the_cached_sequence(W, S, Tc, pos0, sink_len):
    # The chunk's queries see exactly what a prefill over the whole sequence
    # would show them, given the cached rows as the keys of their positions:
    # sinks (prefix), the ring's window rows, and the chunk itself.  Positions
    # the ring no longer holds get random junk, which must stay invisible.
    B, Hq, Hkv, D = 3, 4, 2, 32
    rng = np.random.default_rng(60 + W + Tc)
    q = rng.standard_normal((B, Hq, Tc, D))
    k, v = rng.standard_normal((2, B, Hkv, Tc, D)).astype(np.float32)
    caches = {}
    for name, rows in (("ring_k", W), ("ring_v", W), ("sink_k", S), ("sink_v", S)):
        x = rng.standard_normal((B * Hkv * rows, D)).astype(np.float32) * 2
        c, sc = oracle.quantize(x)
        caches[name] = c.reshape(B, Hkv, rows, D)
        caches[name + "s"] = sc.reshape(B, Hkv, rows, D // 32)
    out, lse, rk, rv, rks, rvs = oracle.chunk_prefill(
        q, k, v, caches["ring_k"], caches["ring_v"], caches["ring_ks"], caches["ring_vs"], caches["sink_k"],
        caches["sink_v"], caches["sink_ks"], caches["sink_vs"], pos0, sink_len)
    G = Hq // Hkv
    for b in range(B):
        p0 = pos0[b]
        sl = min(S if sink_len is None else sink_len[b], p0, S)
        L = p0 + Tc
        Kf = rng.standard_normal((1, Hkv, L, D)) * 30          # junk where the cache holds nothing
        Vf = rng.standard_normal((1, Hkv, L, D)) * 30
        for h in range(Hkv):
            Kf[0, h, :sl] = _dequant(caches["sink_k"][b, h, :sl], caches["sink_ks"][b, h, :sl])
            Vf[0, h, :sl] = _dequant(caches["sink_v"][b, h, :sl], caches["sink_vs"][b, h, :sl])
            for p in range(max(sl, p0 - W + 1), p0):
                Kf[0, h, p] = _dequant(caches["ring_k"][b, h, p % W], caches["ring_ks"][b, h, p % W])
                Vf[0, h, p] = _dequant(caches["ring_v"][b, h, p % W], caches["ring_vs"][b, h, p % W])
            Kf[0, h, p0:] = k[b, h]
            Vf[0, h, p0:] = v[b, h]
        Qf = np.zeros((1, Hq, L, D))
        Qf[0, :, p0:] = q[b]
        prefix = np.zeros((1, L), np.uint8)
        prefix[0, :sl] = 1
        rows = [(h * L + t) for h in range(Hq) for t in range(p0, L)]
        ref, ref_lse = oracle.prefill(Qf, Kf, Vf, np.ones((1, L), np.int32), prefix, W, rows=rows)
        np.testing.assert_allclose(out[b].reshape(-1, D), ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b].reshape(-1), ref_lse, rtol=1e-12, atol=1e-12)
        # the ring: the chunk's last min(W, Tc) tokens, quantized into their slots; other slots untouched
        written = {(p0 + i) % W: i for i in range(max(0, Tc - W), Tc)}
        for h in range(Hkv):
            kq, ks = oracle.quantize(k[b, h])
            for slot in range(W):
                if slot in written:
                    np.testing.assert_array_equal(rk[b, h, slot], kq[written[slot]])
                    np.testing.assert_array_equal(rks[b, h, slot], ks[written[slot]])
                else:
                    np.testing.assert_array_equal(rk[b, h, slot], caches["ring_k"][b, h, slot])
    assert G == 2


def test_chunk_prefill_from_an_empty_cache_is_causal_window_attention():
    # pos0 = 0, no sinks: the chunk alone, causal with window W (SDPA with a band mask)
    B, H, Tc, D, W = 2, 2, 24, 32, 5
    rng = np.random.default_rng(70)
    q = rng.standard_normal((B, H, Tc, D))
    k, v = rng.standard_normal((2, B, H, Tc, D)).astype(np.float32)
    z8 = np.zeros((B, H, W, D), np.int8)
    z32 = np.zeros((B, H, W, 1), np.float32)
    s8 = np.zeros((B, H, 0, D), np.int8)
    s32 = np.zeros((B, H, 0, 1), np.float32)
    out, *_ = oracle.chunk_prefill(q, k, v, z8, z8, z32, z32, s8, s8, s32, s32, [0, 0])
    np.testing.assert_allclose(out, sdpa(q, k.astype(np.float64), v.astype(np.float64), mask=band(Tc, W)),
                               rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# O10 backward of the prefill  (the training-side mask of [NS §"KV sink 如何
# 「钉住」工具"] and [NW §"KV Sinks for Tools"]; reading A21)
# --------------------------------------------------------------------------

def _autograd_reference(q, k, v, dout, mask, scale):
    """dq, dk, dv of torch SDPA (fp64, CPU) under an explicit boolean mask [B, T, T]; GQA by repeated heads."""
    G = q.shape[1] // k.shape[1]
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    m = torch.from_numpy(np.asarray(mask, dtype=bool))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt.repeat_interleave(G, 1), vt.repeat_interleave(G, 1),
                                                         attn_mask=m, scale=scale)
    o.backward(torch.from_numpy(np.ascontiguousarray(dout, dtype=np.float64)))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("case", ["causal", "window_sinks", "segments", "gqa"])
def test_prefill_backward_matches_autograd(case):
    rng = np.random.default_rng({"causal": 80, "window_sinks": 81, "segments": 82, "gqa": 83}[case])
    B, T, D = 2, 40, 16
    Hq, Hkv = (4, 2) if case == "gqa" else (2, 2)
    seg = np.ones((B, T), np.int32)
    prefix = None
    W = 0
    if case == "window_sinks":
        W = 6
        prefix = np.zeros((B, T), np.uint8)
        prefix[:, :5] = 1
        seg[:, :5] = 1
    if case in ("segments", "gqa"):
        W = 9
        seg[0, 13:] = 2
        seg[0, 30:] = 3
        seg[1, 20:] = 2
        prefix = np.zeros((B, T), np.uint8)
        prefix[0, 13:16] = 1
        prefix[1, 0:4] = 1
    q = rng.standard_normal((B, Hq, T, D))
    k, v = rng.standard_normal((2, B, Hkv, T, D))
    dout = rng.standard_normal((B, Hq, T, D))
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = oracle.prefill_backward(q, k, v, dout, seg, prefix, W)
    mask = oracle.mask(seg, prefix, W).astype(bool)
    rq, rk, rv = _autograd_reference(q, k, v, dout, mask, scale)
    np.testing.assert_allclose(dq, rq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, rk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, rv, rtol=1e-10, atol=1e-12)


def test_prefill_backward_rope_is_the_rotated_problem_rotated_back():
    # with RoPE the gradients w.r.t. the unrotated q, k are those of the rotated
    # problem rotated back (the rotation at -pos is the transpose of the one at pos)
    rng = np.random.default_rng(84)
    B, H, T, D = 1, 2, 30, 16
    q, k, v, dout = rng.standard_normal((4, B, H, T, D))
    pos = np.arange(T)
    qr = np.stack([oracle.rope(q[0, h], pos, 1e4) for h in range(H)])[None]
    kr = np.stack([oracle.rope(k[0, h], pos, 1e4) for h in range(H)])[None]
    dq, dk, dv = oracle.prefill_backward(q, k, v, dout, None, None, 7, theta=1e4)
    dq0, dk0, dv0 = oracle.prefill_backward(qr, kr, v, dout, None, None, 7)
    np.testing.assert_allclose(dq[0], np.stack([oracle.rope(dq0[0, h], -pos, 1e4) for h in range(H)]),
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk[0], np.stack([oracle.rope(dk0[0, h], -pos, 1e4) for h in range(H)]),
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, dv0, rtol=1e-12, atol=1e-13)


def test_prefill_backward_finite_differences_and_padding():
    # central differences of L = <dout, out> on a tiny problem with sinks, a
    # window and a padding row (segment 0: no output, no gradient, no effect)
    rng = np.random.default_rng(85)
    B, Hq, Hkv, T, D, W = 1, 2, 1, 9, 4, 3
    seg = np.array([[1, 1, 1, 1, 2, 2, 2, 2, 0]], np.int32)
    prefix = np.array([[1, 0, 0, 0, 1, 0, 0, 0, 0]], np.uint8)
    q = rng.standard_normal((B, Hq, T, D))
    k, v = rng.standard_normal((2, B, Hkv, T, D))
    dout = rng.standard_normal((B, Hq, T, D))
    dq, dk, dv = oracle.prefill_backward(q, k, v, dout, seg, prefix, W, theta=1e4)

    def loss(qq, kk, vv):
        out, _ = oracle.prefill(qq, kk, vv, seg, prefix, W, theta=1e4)
        return float((out * dout).sum())
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            a_p = [xp if n == name else a for n, a in zip("qkv", args)]
            a_m = [xm if n == name else a for n, a in zip("qkv", args)]
            num[idx] = (loss(*a_p) - loss(*a_m)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg=name)
    assert np.all(dq[:, :, 8] == 0) and np.all(dk[:, :, 8] == 0) and np.all(dv[:, :, 8] == 0)


# --------------------------------------------------------------------------
# O11 NSA selection branch without the gate  ([CA §"Two kinds of columns,
# pooled blocks and exact recent keys", §"What we didn't build, and why"];
# reading A22)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("W,b,n_sel,Hq,Hkv", [(8, 4, 3, 2, 2), (5, 3, 5, 4, 2), (16, 8, 2, 2, 1)])
def test_nsa_select_is_top_k_of_numpy_scores_then_sdpa(W, b, n_sel, Hq, Hkv):
    # the selection is the stable argsort of the compressed scores (numpy
    # matmul of the O2-rotated q and the O4 pooled keys) over the visible
    # blocks; the output is SDPA over the chosen blocks' rotated exact keys
    B, T, D = 2, 64, 16
    q, k, v = _case(B, Hq, Hkv, T, D, seed=90 + W + b)
    out, lse, sel = oracle.nsa_select(q, k, v, W, b, n_sel, theta=1e4)
    pk, _ = oracle.pool_rope(k, v, b, theta=1e4, rope_len=T)
    pos = np.arange(T)
    scale = 1.0 / math.sqrt(D)
    G = Hq // Hkv
    for bb in range(B):
        for h in range(Hq):
            qr = oracle.rope(q[bb, h], pos, 1e4)
            kr = oracle.rope(k[bb, h // G], pos, 1e4)
            scores = scale * qr @ pk[bb, h // G].T
            for t in range(T):
                nv = max(0, (t - W + 1) // b)
                order = np.argsort(-scores[t, :nv], kind="stable")[:n_sel]
                want = np.full(n_sel, -1)
                want[:len(order)] = order
                np.testing.assert_array_equal(sel[bb, h, t], want)
                if len(order) == 0:
                    assert np.all(out[bb, h, t] == 0) and np.isneginf(lse[bb, h, t])
                    continue
                cols = np.concatenate([np.arange(j * b, (j + 1) * b) for j in order])
                ref = sdpa(qr[t][None], kr[cols], v[bb, h // G][cols])
                np.testing.assert_allclose(out[bb, h, t], ref[0], rtol=1e-12, atol=1e-12)


def test_nsa_select_all_blocks_is_attention_over_every_cleared_block():
    # n_select >= the number of candidates: every token of every block that
    # cleared the window, i.e. positions [0, floor((t - W + 1) / b) * b)
    B, H, T, D, W, b = 1, 2, 50, 8, 6, 4
    q, k, v = _case(B, H, H, T, D, seed=95)
    out, lse, sel = oracle.nsa_select(q, k, v, W, b, T, theta=1e4)
    pos = np.arange(T)
    qr = np.stack([oracle.rope(q[0, h], pos, 1e4) for h in range(H)])[None]
    kr = np.stack([oracle.rope(k[0, h], pos, 1e4) for h in range(H)])[None]
    nv = np.maximum(0, (pos - W + 1) // b)
    mask = np.arange(T)[None, :] < (nv * b)[:, None]
    ok = nv > 0
    ref = sdpa(qr[:, :, ok], kr, v, mask=mask[ok])
    np.testing.assert_allclose(out[:, :, ok], ref, rtol=1e-12, atol=1e-12)
    assert np.all(out[:, :, ~ok] == 0) and np.all(sel[:, :, ~ok] == -1)
    # the override replaces the selection
    out2, _, sel2 = oracle.nsa_select(q, k, v, W, b, T, theta=1e4, sel=sel)
    np.testing.assert_array_equal(out2, out)
