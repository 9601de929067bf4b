"""GPU parity of the windowed+sink prefill kernels against the CPU oracle.

Sources: [NW] "How the 256-Token Sliding Window Works with Tools as KV Sinks in
Needle" (section "KV Sinks for Tools: Pinning Critical Context") for the mask;
[CA] "Compressed attention and the copy probe" for RoPE placement.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_attention_amd import swa, workloads
from gpu_util import (assert_close, assert_lse_close, dev_input, dev_opt, sample_rows, say, to_np)

pytestmark = pytest.mark.gpu


def run_prefill(w, return_lse=True, q_override=None):
    q = dev_input(w, "q") if q_override is None else q_override
    k, v = dev_input(w, "k"), dev_input(w, "v")
    seg = dev_opt(w["seg_ids"], np.int32)
    pre = dev_opt(w["prefix"], np.uint8)
    rope = swa.rope_table(w["rope_theta"], w["T"], w["D"]) if w["rope_theta"] else None
    out, lse = swa.prefill(q, k, v, seg, pre, w["window"], rope=rope, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def oracle_rows(w, rows=None):
    return oracle.prefill(w["q"], w["k"], w["v"], w["seg_ids"], w["prefix"], w["window"],
                          theta=w["rope_theta"], rows=rows)


def random_structure(rng, B, T, kind):
    if kind == "one":
        seg = np.ones((B, T), np.int32)
    elif kind == "packed":
        # (at most T // 2 segments, so that very short rows can be cut)
        seg, _ = workloads.packed_structure(rng, B, T, prefix_len=0, min_seg=1, max_seg=min(4, max(1, T // 2)),
                                            max_pad=T // 4)
    else:  # repeated, non-contiguous ids with padding
        seg = rng.integers(0, 3, size=(B, T)).astype(np.int32)
    prefix = (rng.random((B, T)) < 0.08).astype(np.uint8)
    prefix[:, : int(rng.integers(0, 9))] = 1
    return seg, prefix


def test_rope_table_matches_fp64_angles():
    T, D, theta = 4096, 64, 10000.0
    c, s = swa.rope_table(theta, T, D)
    torch.cuda.synchronize()
    pos = np.arange(T)[:, None].astype(np.float64)
    inv = theta ** (-2.0 * np.arange(D // 2) / D)
    ang = pos * inv
    np.testing.assert_allclose(c.cpu().numpy(), np.cos(ang).astype(np.float32), rtol=0, atol=1.2e-7)
    np.testing.assert_allclose(s.cpu().numpy(), np.sin(ang).astype(np.float32), rtol=0, atol=1.2e-7)


@pytest.mark.parametrize("make", [workloads.tiny, workloads.tiny_sink], ids=["tiny", "tiny_sink"])
def test_tiny_fp32_full(make):
    w = make()
    out, lse = run_prefill(w)
    ref, ref_lse = oracle_rows(w)
    assert_close(to_np(out)[0, 0], ref[0, 0], "f32", make.__name__)
    assert_lse_close(to_np(lse), ref_lse, "f32", make.__name__)


CASES = []
for dtype in ("f32", "bf16"):
    for i, (B, Hq, Hkv, T, D, W, kind, rope) in enumerate([
        (1, 1, 1, 64, 32, 16, "one", False),
        (2, 4, 2, 77, 64, 0, "packed", False),
        (1, 2, 2, 130, 64, 1, "one", True),
        (2, 8, 2, 200, 64, 37, "packed", True),
        (1, 4, 1, 256, 64, 256, "ids", False),
        (2, 2, 1, 191, 32, 64, "packed", False),
        (1, 8, 8, 300, 64, 3, "ids", True),
        (1, 16, 2, 97, 64, 500, "one", False),
        (2, 4, 4, 160, 32, 48, "packed", True),
        # RoPE with every GQA geometry: groups of 8 and 4 (the workgroup's waves share
        # their rows' table entries; ragged last block), 2 (two row blocks per workgroup)
        (2, 8, 1, 150, 32, 40, "packed", True),
        (1, 4, 1, 99, 32, 0, "one", True),
        (1, 4, 2, 100, 64, 20, "ids", True),
    ]):
        CASES.append(pytest.param(dtype, B, Hq, Hkv, T, D, W, kind, rope, i, id=f"{dtype}-{i}"))


# A seeded sweep over shapes the fixed cases do not reach: every GQA group size
# 1..8 (3, 5, 6 and 7 included: 3 and 6 leave a wave of the workgroup idle, 5
# and 7 run one head per wave), T from 1, windows 0, 1 and up to past T.
SWEEP = []
_srng = np.random.default_rng(2024)
for _i in range(32):
    _G = int(_srng.integers(1, 9))
    _Hkv = int(_srng.integers(1, 3))
    _T = int(_srng.choice([1, 2, 31, 33, 63, 65]) if _i % 4 == 0 else _srng.integers(1, 400))
    _W = int(_srng.choice([0, 1, int(_srng.integers(2, 320))]))
    SWEEP.append(pytest.param(("f32", "bf16")[_i % 2], int(_srng.integers(1, 3)), _G * _Hkv, _Hkv, _T,
                              (32, 64)[int(_srng.integers(0, 2))], _W, ("one", "packed", "ids")[_i % 3],
                              bool(_srng.integers(0, 2)), 500 + _i, id=f"sweep{_i}"))


@pytest.mark.parametrize("dtype,B,Hq,Hkv,T,D,W,kind,rope,seed", SWEEP)
def test_prefill_random_sweep(dtype, B, Hq, Hkv, T, D, W, kind, rope, seed):
    test_prefill_random_small(dtype, B, Hq, Hkv, T, D, W, kind, rope, seed)


@pytest.mark.parametrize("dtype,B,Hq,Hkv,T,D,W,kind,rope,seed", CASES)
def test_prefill_random_small(dtype, B, Hq, Hkv, T, D, W, kind, rope, seed):
    rng = np.random.default_rng(100 + seed)
    seg, prefix = random_structure(rng, B, T, kind)
    w = workloads.prefill_case(B, Hq, Hkv, T, D, W, dtype, seed=200 + seed, seg_ids=seg, prefix=prefix,
                               rope_theta=10000.0 if rope else 0.0)
    say(f"case {dtype} B{B} {Hq}/{Hkv} T{T} D{D} W{W} {kind} rope={rope}")
    out, lse = run_prefill(w)
    ref, ref_lse = oracle_rows(w)
    assert_close(to_np(out), ref, dtype, "out")
    assert_lse_close(to_np(lse), ref_lse, dtype, "out")
    # padding rows are exactly zero
    pad = np.broadcast_to((seg == 0)[:, None, :], (B, Hq, T))
    assert np.all(to_np(out)[pad] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,W,kind,Hq,Hkv", [(64, 16, "one", 1, 1), (150, 7, "packed", 4, 2),
                                             (333, 0, "ids", 8, 2), (257, 64, "packed", 2, 2),
                                             (513, 256, "packed", 16, 4), (96, 1, "ids", 4, 1)])
def test_debug_visibility_bit_exact(dtype, T, W, kind, Hq, Hkv):
    rng = np.random.default_rng(T * 7 + W)
    B = 2
    seg, prefix = random_structure(rng, B, T, kind)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    mask, count = swa.debug_visibility(B, Hq, Hkv, T, 64, W, tdt, dev_opt(seg, np.int32), dev_opt(prefix, np.uint8))
    torch.cuda.synchronize()
    ref = oracle.mask(seg, prefix, W)
    np.testing.assert_array_equal(mask.cpu().numpy(), ref)
    np.testing.assert_array_equal(count.cpu().numpy(), ref.sum(axis=2))


@pytest.mark.parametrize("make", [workloads.needle, workloads.packed], ids=["needle", "packed"])
def test_full_size_visibility_and_counts(make):
    """The bf16 kernel's own mask (its DUMP instantiation) bit for bit against
    the oracle mask: every batch row of the needle config, the first two rows of
    the packed config (2 x 4096 x 4096), and every row's count of both."""
    w = make()
    B, T = w["B"], w["T"]
    seg = dev_opt(w["seg_ids"], np.int32)
    pre = dev_opt(w["prefix"], np.uint8)
    _, count = swa.debug_visibility(B, w["Hq"], w["Hkv"], T, w["D"], w["window"], torch.bfloat16, seg, pre,
                                    want_mask=False)
    nm = B if make is workloads.needle else 2
    mask, _ = swa.debug_visibility(nm, w["Hq"], w["Hkv"], T, w["D"], w["window"], torch.bfloat16,
                                   seg[:nm].contiguous(), pre[:nm].contiguous())
    torch.cuda.synchronize()
    ref = oracle.mask(w["seg_ids"][:nm], w["prefix"][:nm], w["window"])
    np.testing.assert_array_equal(mask.cpu().numpy(), ref)
    say(f"  {make.__name__}: mask of {nm} x {T} x {T} pairs bit-exact ({int(ref.sum())} visible)")
    del mask, ref
    ref_counts = np.stack([oracle.mask(w["seg_ids"][b:b + 1], w["prefix"][b:b + 1], w["window"])[0].sum(axis=1)
                           for b in range(B)])
    np.testing.assert_array_equal(count.cpu().numpy(), ref_counts)
    # the real kernel with q = 0 weights every visible key equally: exp(lse) = n_vis
    q0 = torch.zeros((B, w["Hq"], T, w["D"]), dtype=torch.bfloat16, device="cuda")
    _, lse = run_prefill(w, q_override=q0)
    lse = lse.cpu().numpy().astype(np.float64)
    n = np.broadcast_to(ref_counts[:, None, :], lse.shape)
    vis = n > 0
    assert np.all(np.isneginf(lse[~vis]))
    np.testing.assert_array_equal(np.rint(np.exp(lse[vis])).astype(np.int64), n[vis])


@pytest.mark.parametrize("make", [workloads.needle, workloads.packed], ids=["needle", "packed"])
def test_full_size_every_row(make):
    """Every output row and lse of the full-size needle (131 072 rows) and packed
    (1 048 576 rows) configs against the oracle; max-abs and mean-abs are taken
    over the whole tensors."""
    w = make()
    B, Hq, T = w["B"], w["Hq"], w["T"]
    say(f"{make.__name__}: B{B} Hq{Hq} Hkv{w['Hkv']} T{T} W{w['window']}, every row")
    out, lse = run_prefill(w)
    got = to_np(out)
    got_lse = lse.cpu().numpy()
    del out, lse
    ref, ref_lse = oracle_rows(w)
    assert_close(got, ref, "bf16", make.__name__)
    assert_lse_close(got_lse, ref_lse, "bf16", make.__name__)


def test_longest_sequence_sampled_rows():
    """T at the kernels' limit (131072 keys: 2048 key tiles, so the sink scan
    walks all 32 of its 64-tile words), with sinks in three places of two
    segments: every row sees its window band plus the sinks of its own
    segment that lie before it, up to 130 000 positions back."""
    T, W = 131072, 256
    seg = np.ones((1, T), np.int32)
    seg[0, 70000:] = 2
    prefix = np.zeros((1, T), np.uint8)
    prefix[0, :300] = 1            # sinks of segment 1 at its start
    prefix[0, 40000:40064] = 1     # and in its middle
    prefix[0, 70000:70500] = 1     # sinks of segment 2 at its start
    prefix[0, 131000:131010] = 1   # and near the end
    w = workloads.prefill_case(1, 2, 1, T, 64, W, "bf16", seed=21, seg_ids=seg, prefix=prefix, rope_theta=10000.0)
    say(f"longest: T{T} W{W} sinks {int(prefix.sum())}")
    out, lse = run_prefill(w)
    rng = np.random.default_rng(8)
    extra = [0, 299, 300, 555, 39999, 40000, 40063, 40064, 40300, 69999, 70000, 70255, 70499, 70500, 70756,
             100000, 130999, 131000, 131009, 131010, T - 1]
    rows = sample_rows(rng, 1, 2, T, 400, extra)
    ref, ref_lse = oracle_rows(w, rows)
    got = to_np(out).reshape(-1, 64)[rows]
    assert_close(got, ref, "bf16", "longest")
    assert_lse_close(lse.cpu().numpy().reshape(-1)[rows], ref_lse, "bf16", "longest")


def test_bitwise_deterministic():
    w = workloads.packed(B=4, T=1024)
    a, _ = run_prefill(w)
    b, _ = run_prefill(w)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_single_row_and_empty():
    w = workloads.prefill_case(1, 2, 1, 1, 64, 16, "bf16", seed=9)
    out, lse = run_prefill(w)
    np.testing.assert_allclose(to_np(out)[0, :, 0], w["v"][0, 0, 0][None].repeat(2, 0), atol=0)
    q = torch.zeros((0, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((0, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    assert swa.prefill(q, k, k, window=4).shape == (0, 2, 8, 64)
