"""GPU parity of the compressed-KV path (block pooling + midpoint RoPE, then one
softmax over [pooled blocks, exact keys]) against the CPU oracle.

Source: [CA] "Compressed attention and the copy probe", sections "Two kinds of
columns, pooled blocks and exact recent keys" and "Pool before rotating, not
after".
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_attention_amd import swa, workloads
from gpu_util import assert_close, assert_lse_close, dev_input, say, to_np

pytestmark = pytest.mark.gpu


def run_compressed(w, q_override=None):
    q = dev_input(w, "q") if q_override is None else q_override
    k, v = dev_input(w, "k"), dev_input(w, "v")
    rope = swa.rope_table(w["rope_theta"], w["T"], w["D"]) if w["rope_theta"] else None
    pk, pv = swa.pool_compress_rope(k, v, w["compress_block"], rope)
    out, lse = swa.prefill(q, k, v, window=w["window"], rope=rope, pooled_k=pk, pooled_v=pv,
                           compress_block=w["compress_block"], return_lse=True)
    torch.cuda.synchronize()
    return out, lse, pk, pv


def run_pool_in_call(w):
    """The compressed prefill with no pooled inputs: the call pools k and v itself."""
    q, k, v = dev_input(w, "q"), dev_input(w, "k"), dev_input(w, "v")
    rope = swa.rope_table(w["rope_theta"], w["T"], w["D"]) if w["rope_theta"] else None
    out, lse = swa.prefill(q, k, v, window=w["window"], rope=rope, compress_block=w["compress_block"],
                           return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def oracle_compressed(w, rows=None):
    return oracle.compressed_prefill(w["q"], w["k"], w["v"], w["window"], w["compress_block"],
                                     theta=w["rope_theta"], rope_len=w["T"], rows=rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("block,rope_len_short", [(1, False), (3, False), (4, False), (12, False), (16, False),
                                                  (4, True)])
def test_pool_kernel(dtype, block, rope_len_short):
    w = workloads.prefill_case(2, 3, 3, 101, 64, 8, dtype, seed=block)
    k, v = dev_input(w, "k"), dev_input(w, "v")
    rl = 20 if rope_len_short else w["T"]
    rope = swa.rope_table(10000.0, rl, 64)
    pk, pv = swa.pool_compress_rope(k, v, block, rope)
    torch.cuda.synchronize()
    rk, rv = oracle.pool_rope(w["k"], w["v"], block, theta=10000.0, rope_len=rl)
    # each pooled value is rounded once to the storage dtype
    # (fp32 sums and rotation with fp32 tables, then one rounding to the storage dtype)
    rtol = 1e-6 if dtype == "f32" else 2.0 ** -8
    atol = 1e-6
    for name, got, ref in (("pooled_k", pk, rk), ("pooled_v", pv, rv)):
        g = to_np(got)
        excess = np.abs(g - ref) - (rtol * np.abs(ref) + atol)
        say(f"  {name} b={block}: max abs err {np.abs(g - ref).max():.2e}")
        assert excess.max() <= 0


@pytest.mark.parametrize("block", [4, 8])
def test_pool_kernel_many_row_groups(block):
    """More row groups (B * H = 66000) than one grid dimension holds (65535):
    the pooling kernels loop over the rest.  Short rows keep it small."""
    w = workloads.prefill_case(1, 66000, 66000, 16, 32, 8, "bf16", seed=40 + block)
    k, v = dev_input(w, "k"), dev_input(w, "v")
    rope = swa.rope_table(10000.0, w["T"], 32)
    pk, pv = swa.pool_compress_rope(k, v, block, rope)
    torch.cuda.synchronize()
    rk, rv = oracle.pool_rope(w["k"], w["v"], block, theta=10000.0, rope_len=w["T"])
    for name, got, ref in (("pooled_k", pk, rk), ("pooled_v", pv, rv)):
        g = to_np(got)
        excess = np.abs(g - ref) - (2.0 ** -8 * np.abs(ref) + 1e-6)
        say(f"  {name} b={block}: max abs err {np.abs(g - ref).max():.2e} (last row group {np.abs(g - ref)[0, -1].max():.2e})")
        assert excess.max() <= 0



@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pool_kernel_narrow_rows(dtype):
    """A head dim whose half is not a whole number of 16-byte pieces (D = 36)
    takes the element-wise pooling kernel."""
    w = workloads.prefill_case(1, 2, 2, 64, 36, 8, dtype, seed=9)
    k, v = dev_input(w, "k"), dev_input(w, "v")
    rope = swa.rope_table(10000.0, w["T"], 36)
    pk, pv = swa.pool_compress_rope(k, v, 4, rope)
    torch.cuda.synchronize()
    rk, rv = oracle.pool_rope(w["k"], w["v"], 4, theta=10000.0, rope_len=w["T"])
    rtol = 1e-6 if dtype == "f32" else 2.0 ** -8
    for got, ref in ((pk, rk), (pv, rv)):
        g = to_np(got)
        assert (np.abs(g - ref) - (rtol * np.abs(ref) + 1e-6)).max() <= 0

CASES = []
for dtype in ("f32", "bf16"):
    for i, (B, H, Hkv, T, W, b) in enumerate([(1, 1, 1, 64, 8, 4), (2, 2, 2, 150, 16, 3), (1, 4, 2, 300, 32, 16),
                                              (1, 2, 2, 257, 64, 1), (2, 2, 1, 129, 5, 7), (1, 1, 1, 100, 200, 4)]):
        CASES.append(pytest.param(dtype, B, H, Hkv, T, W, b, i, id=f"{dtype}-{i}"))


# A seeded sweep: GQA groups 1..4, both head dims, T from 1, windows 1 to past
# T, blocks 1..20 (vector and wave pooling kernels, remainders T mod b).
SWEEP = []
_crng = np.random.default_rng(777)
for _i in range(16):
    _Hkv = int(_crng.integers(1, 3))
    _T = int(_crng.integers(1, 400))
    SWEEP.append(pytest.param(("f32", "bf16")[_i % 2], int(_crng.integers(1, 3)), int(_crng.integers(1, 5)) * _Hkv,
                              _Hkv, _T, int(_crng.integers(1, 300)), int(_crng.integers(1, 21)), 600 + _i,
                              (32, 64)[(_i // 2) % 2], id=f"sweep{_i}"))


@pytest.mark.parametrize("dtype,B,H,Hkv,T,W,b,seed,D", SWEEP)
def test_compressed_sweep(dtype, B, H, Hkv, T, W, b, seed, D):
    test_compressed_random_small(dtype, B, H, Hkv, T, W, b, seed, D)


@pytest.mark.parametrize("dtype,B,H,Hkv,T,W,b,seed", CASES)
def test_compressed_random_small(dtype, B, H, Hkv, T, W, b, seed, D=64):
    w = workloads.prefill_case(B, H, Hkv, T, D, W, dtype, seed=300 + seed, rope_theta=10000.0, compress_block=b)
    say(f"case {dtype} B{B} {H}/{Hkv} T{T} W{W} b{b}")
    out, lse, _, _ = run_compressed(w)
    ref, ref_lse = oracle_compressed(w)
    assert_close(to_np(out), ref, dtype, "out")
    assert_lse_close(to_np(lse), ref_lse, dtype, "out")


# dtype, B, Hq, Hkv, T, W, b, D: blocks that fit the fused pool-and-rotate pass
# (b <= 64 at D = 64, b <= 128 at D = 32) and blocks that do not (separate
# pooling pass), no RoPE, remainders T mod b, fp32 (separate passes).
POOL_IN_CALL = [("bf16", 1, 4, 2, 300, 32, 4, 64, True), ("bf16", 2, 2, 2, 150, 16, 3, 64, True),
                ("bf16", 1, 4, 2, 300, 32, 16, 64, True), ("bf16", 1, 2, 2, 257, 64, 1, 64, True),
                ("bf16", 1, 2, 1, 333, 40, 7, 32, True), ("bf16", 1, 2, 2, 500, 64, 64, 64, True),
                ("bf16", 1, 2, 2, 500, 64, 80, 64, True), ("bf16", 1, 2, 2, 600, 64, 128, 32, True),
                ("bf16", 1, 2, 2, 203, 30, 5, 64, False), ("f32", 1, 2, 2, 150, 16, 4, 64, True),
                ("bf16", 2, 8, 8, 1000, 256, 4, 64, True)]


@pytest.mark.parametrize("dtype,B,H,Hkv,T,W,b,D,rope", POOL_IN_CALL,
                         ids=[f"{c[0]}-T{c[4]}-b{c[6]}-D{c[7]}{'' if c[8] else '-norope'}" for c in POOL_IN_CALL])
def test_compressed_pools_in_call(dtype, B, H, Hkv, T, W, b, D, rope):
    """pooled_k = pooled_v = NULL: the call pools k and v itself.  Against the
    oracle, and against the call with pooled inputs from kv_pool_compress_rope:
    the same bits wherever both pool with the same summation order (fp32, or
    blocks below 8, whose pooling kernel adds rows one after another like the
    fused pass; blocks too long for the fused pass use that very kernel)."""
    w = workloads.prefill_case(B, H, Hkv, T, D, W, dtype, seed=900 + b, rope_theta=10000.0 if rope else 0.0,
                               compress_block=b)
    out, lse = run_pool_in_call(w)
    ref, ref_lse = oracle_compressed(w)
    assert_close(to_np(out), ref, dtype, "out (pooled in the call)")
    assert_lse_close(to_np(lse), ref_lse, dtype, "lse (pooled in the call)")
    out2, lse2, _, _ = run_compressed(w)
    fused = dtype == "bf16" and rope and b <= 256 // (D // 16)
    if dtype == "f32" or not fused or b < 8:
        assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("T,W,b", [(200, 16, 4), (333, 64, 16), (129, 8, 3), (4096, 256, 4), (4096, 256, 16)])
def test_compressed_visibility_bit_exact(T, W, b):
    """Both kernels' masks bit for bit against the oracle's compressed mask; the
    last two are the full-size compressed configs (4096 rows x [T/b pooled, T
    exact] columns; the mask has no batch dependence)."""
    for dt in (torch.bfloat16, torch.float32):
        mask, count = swa.debug_visibility(1, 4, 4, T, 64, W, dt, compress_block=b)
        torch.cuda.synchronize()
        ref = oracle.compressed_mask(T, W, b)
        np.testing.assert_array_equal(mask.cpu().numpy()[0], ref)
        np.testing.assert_array_equal(count.cpu().numpy()[0], ref.sum(axis=1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("block", [4, 16])
def test_compressed_full_size(dtype, block):
    w = workloads.compressed(block=block, dtype=dtype)
    B, H, T = w["B"], w["Hq"], w["T"]
    say(f"compressed {dtype} b={block}: B{B} H{H} T{T} W{w['window']}")
    out, lse, _, _ = run_compressed(w)
    # every row (131 072 of them) and its lse against the oracle
    ref, ref_lse = oracle_compressed(w)
    assert_close(to_np(out), ref, dtype, f"b={block}, every row")
    assert_lse_close(lse.cpu().numpy(), ref_lse, dtype, f"b={block}, every row")
    # the same call pooling k and v itself (the fused pre-pass for bf16)
    out_h, lse_h = run_pool_in_call(w)
    assert_close(to_np(out_h), ref, dtype, f"b={block}, pooled in the call, every row")
    assert_lse_close(lse_h.cpu().numpy(), ref_lse, dtype, f"b={block}, pooled in the call, every row")
    # the last row reads the pooled blocks that cleared the window plus W exact keys
    q0 = torch.zeros_like(dev_input(w, "q"))
    _, lse0, _, _ = run_compressed(w, q_override=q0)
    n_last = np.rint(np.exp(lse0[0, 0, T - 1].item()))
    assert n_last == (T - w["window"] + 1) // block + w["window"]


def test_compressed_bitwise_repeatable():
    """Thirty launches of the full-size compressed prefill (b = 4) give the same bits."""
    w = workloads.compressed(block=4, dtype="bf16")
    first = run_compressed(w)[0].view(torch.int16).clone()
    for i in range(30):
        out = run_compressed(w)[0].view(torch.int16)
        assert torch.equal(out, first), f"launch {i} differs"
