"""GPU parity of the compressed decode step (swa_attn_decode_compressed).

Source: [CA] "Compressed attention and the copy probe", sections "Two kinds of
columns, pooled blocks and exact recent keys" (columns = [pooled blocks that
cleared the window, exact window]), "Pool before rotating, not after" (mean of
pre-RoPE keys, rotated at the clamped block midpoint) and "So what happened ?"
(blocks join one at a time); the frontier state is the one [DS] names for
compressed layers ("磁盘 KV 缓存").  The oracle is O8 (oracle.compressed_decode).

What is compared:
  * outputs: every row, int8-KV tolerance (max-abs 2e-2, mean-abs 2e-3);
  * ring rows: bit-exact (the appended key and value are bf16, quantized in
    fp32 on both sides);
  * frontier sums: within one fp32 rounding of the exact sum;
  * pooled rows written by the step: the kernel forms the mean and the
    rotation in fp32, the oracle in fp64, so the codes are checked as a valid
    quantization of the exact row: each group scale within 1e-5 (relative) of
    amax/127 of the exact row and each code within half a step (plus that
    slack) of the exact value; every other pooled row is unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_attention_amd import swa, workloads
from gpu_util import assert_close, bf16_dev, say, to_np

pytestmark = pytest.mark.gpu


def deq(codes, scales):
    """int8 codes [..., D] and group scales [..., D/32] -> fp64 row values (exact products)."""
    return codes.astype(np.float64) * np.repeat(scales.astype(np.float64), 32, axis=-1)


def device_state(w):
    """GPU caches quantized by the library from the case's bf16 caches, the oracle's fp64 state from the same
    codes (exact products), and a check that the two quantizers agree bit for bit."""
    dev, ref = {}, {}
    for name in ("ring_k", "ring_v", "pool_k", "pool_v"):
        if w[name].shape[2] == 0:
            dev[name], dev[name + "s"] = None, None
            ref[name] = np.zeros(w[name].shape)
            continue
        q, s = swa.kv_quantize(bf16_dev(w[name + "_bits"]))
        dev[name], dev[name + "s"] = q, s
        shp = w[name].shape
        rq, rs = oracle.quantize(w[name].reshape(-1, shp[-1]))
        np.testing.assert_array_equal(q.cpu().numpy().reshape(-1, shp[-1]), rq)
        ref[name] = deq(rq, rs).reshape(shp)
    dev["front_k"] = torch.from_numpy(w["front_k"]).cuda()
    dev["front_v"] = torch.from_numpy(w["front_v"]).cuda()
    ref["front_k"] = w["front_k"].astype(np.float64)
    ref["front_v"] = w["front_v"].astype(np.float64)
    torch.cuda.synchronize()
    return dev, ref


def run_step(dev, q_bits, kn_bits, kp_bits, vn_bits, pos, block, rope, num_splits=0, workspace=None):
    out = swa.decode_compressed(bf16_dev(q_bits), bf16_dev(kn_bits), bf16_dev(kp_bits), bf16_dev(vn_bits),
                                dev["ring_k"], dev["ring_v"], dev["ring_ks"], dev["ring_vs"],
                                dev["pool_k"], dev["pool_v"], dev["pool_ks"], dev["pool_vs"],
                                dev["front_k"], dev["front_v"], torch.from_numpy(np.asarray(pos, np.int32)).cuda(),
                                block, rope=rope, num_splits=num_splits, workspace=workspace)
    torch.cuda.synchronize()
    return out


def check_pooled_rows(got_codes, got_scales, exact, what):
    """got_codes [N, D] int8, got_scales [N, D/32], exact [N, D] fp64: a valid quantization of the exact rows."""
    N, D = exact.shape
    amax = np.abs(exact).reshape(N, D // 32, 32).max(axis=2)
    s_ref = amax / 127.0
    s = got_scales.astype(np.float64)
    assert np.all(np.abs(s - s_ref) <= 1e-5 * s_ref + 1e-30), f"{what}: group scales off"
    step = np.repeat(s, 32, axis=1)
    err = np.abs(got_codes.astype(np.float64) * step - exact)
    bound = 0.5 * step * (1 + 1e-5) + 1e-5 * np.repeat(amax, 32, axis=1)
    assert np.all(err <= bound), f"{what}: codes off by {np.max(err / np.maximum(step, 1e-30)):.3f} steps"


def check_step(w, dev, ref, out, rope_np, theta, rope_len, what):
    """Compare one step's output and state updates with O8, starting from the state `ref` (updated in place
    to the oracle's quantized state)."""
    B, D, W, P, b = w["B"], w["D"], w["W"], w["P"], w["block"]
    pos = w["pos"]
    r_out, _, st_q = oracle.compressed_decode(w["q"], w["k_new"], w["k_pre"], w["v_new"], ref, pos, b,
                                              theta=theta, rope_len=rope_len, quantize=True)
    _, _, st_x = oracle.compressed_decode(w["q"], w["k_new"], w["k_pre"], w["v_new"], ref, pos, b,
                                          theta=theta, rope_len=rope_len, quantize=False)
    assert_close(to_np(out), r_out, "bf16", what)
    # ring: bit-exact
    np.testing.assert_array_equal(deq(dev["ring_k"].cpu().numpy(), dev["ring_ks"].cpu().numpy()), st_q["ring_k"])
    np.testing.assert_array_equal(deq(dev["ring_v"].cpu().numpy(), dev["ring_vs"].cpu().numpy()), st_q["ring_v"])
    # frontier: one fp32 rounding of the exact sums
    for name in ("front_k", "front_v"):
        got = dev[name].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - st_x[name]) <= 2.0 ** -23 * np.abs(st_x[name]) + 1e-30), f"{what}: {name}"
    # pooled rows: the completed blocks are valid quantizations of the exact rows, the rest unchanged
    if P:
        pk, pks = dev["pool_k"].cpu().numpy(), dev["pool_ks"].cpu().numpy()
        pv, pvs = dev["pool_v"].cpu().numpy(), dev["pool_vs"].cpu().numpy()
        done = [(bb, int(pos[bb]) // b) for bb in range(B)
                if pos[bb] >= 0 and pos[bb] % b == b - 1 and pos[bb] // b < P]
        say(f"  {what}: {len(done)} of {B} sequences completed a block")
        for bb, j in done:
            check_pooled_rows(pk[bb, :, j], pks[bb, :, j], st_x["pool_k"][bb, :, j], f"{what} pooled k")
            check_pooled_rows(pv[bb, :, j], pvs[bb, :, j], st_x["pool_v"][bb, :, j], f"{what} pooled v")
            st_q["pool_k"][bb, :, j] = deq(pk[bb, :, j], pks[bb, :, j])   # follow the kernel's codes
            st_q["pool_v"][bb, :, j] = deq(pv[bb, :, j], pvs[bb, :, j])
        np.testing.assert_array_equal(deq(pk, pks), st_q["pool_k"])
        np.testing.assert_array_equal(deq(pv, pvs), st_q["pool_v"])
    st_q["front_k"] = dev["front_k"].cpu().numpy().astype(np.float64)
    st_q["front_v"] = dev["front_v"].cpu().numpy().astype(np.float64)
    return st_q


@pytest.mark.parametrize("block,P,pos_hi", [(4, 1024, 4095), (16, 256, 4095)])
def test_compressed_decode_full_shape(block, P, pos_hi):
    """B256, 16q/4kv heads, D64, window 256 (the decode shape), positions 0..4095 (the page's 4K context)."""
    w = workloads.compressed_decode_case(seed=60 + block, block=block, P=P, pos_hi=pos_hi)
    say(f"compressed decode B{w['B']} {w['Hq']}/{w['Hkv']} D{w['D']} W{w['W']} b{block} P{P}")
    dev, ref = device_state(w)
    theta, rope_len = 10000.0, pos_hi + 1
    rope = swa.rope_table(theta, rope_len, w["D"])
    out = run_step(dev, w["q_bits"], w["k_new_bits"], w["k_pre_bits"], w["v_new_bits"], w["pos"], block, rope)
    check_step(w, dev, ref, out, rope, theta, rope_len, f"b{block} full shape")


def test_compressed_decode_long_positions_and_splits():
    """Positions up to 32767 (pooled walks of up to 8128 rows, split across workgroups by the automatic
    choice), and explicit split counts giving the same result."""
    w = workloads.compressed_decode_case(seed=70, B=3, P=8192, block=4, pos_lo=20000, pos_hi=32767)
    w["pos"][0] = 32767
    theta, rope_len = 10000.0, 32768
    rope = swa.rope_table(theta, rope_len, w["D"])
    outs = []
    for splits in (0, 1, 3, 8):
        dev, ref = device_state(w)
        out = run_step(dev, w["q_bits"], w["k_new_bits"], w["k_pre_bits"], w["v_new_bits"], w["pos"], 4, rope,
                       num_splits=splits)
        check_step(w, dev, ref, out, rope, theta, rope_len, f"long splits={splits}")
        outs.append(to_np(out))
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2e-2


@pytest.mark.parametrize("D,block,W,rope_mode", [(64, 4, 16, "table"), (32, 3, 8, "table"), (64, 16, 5, "none"),
                                                 (64, 4, 16, "short")])
def test_compressed_decode_sequence_from_empty(D, block, W, rope_mode):
    """A run of T steps from an empty cache: every step's output against O8 run side by side (its own
    state), so the frontier restarts, block completion, the growth of the visible pooled columns and ring
    wrap-around are all exercised."""
    T = 150
    s = workloads.compressed_decode_sequence(seed=80 + block + D, D=D, T=T)
    B, Hq, Hkv = s["B"], s["Hq"], s["Hkv"]
    P = (T + block - 1) // block
    theta = 10000.0
    rope_len = {"table": T, "short": 37, "none": 0}[rope_mode]
    rope = swa.rope_table(theta, rope_len, D) if rope_len else None
    dev = {"ring_k": torch.zeros((B, Hkv, W, D), dtype=torch.int8, device="cuda"),
           "ring_v": torch.zeros((B, Hkv, W, D), dtype=torch.int8, device="cuda"),
           "ring_ks": torch.zeros((B, Hkv, W, D // 32), device="cuda"),
           "ring_vs": torch.zeros((B, Hkv, W, D // 32), device="cuda"),
           "pool_k": torch.zeros((B, Hkv, P, D), dtype=torch.int8, device="cuda"),
           "pool_v": torch.zeros((B, Hkv, P, D), dtype=torch.int8, device="cuda"),
           "pool_ks": torch.zeros((B, Hkv, P, D // 32), device="cuda"),
           "pool_vs": torch.zeros((B, Hkv, P, D // 32), device="cuda"),
           "front_k": torch.zeros((B, Hkv, D), device="cuda"), "front_v": torch.zeros((B, Hkv, D), device="cuda")}
    st = oracle.compressed_decode_state(B, Hkv, D, W, P)
    st_x = oracle.compressed_decode_state(B, Hkv, D, W, P)
    worst = 0.0
    for t in range(T):
        pos = np.full(B, t, np.int32)
        out = run_step(dev, s["q_bits"][t], s["k_new_bits"][t], s["k_pre_bits"][t], s["v_new_bits"][t], pos,
                       block, rope)
        r_out, _, st = oracle.compressed_decode(s["q"][t], s["k_new"][t], s["k_pre"][t], s["v_new"][t], st, pos,
                                                block, theta=theta if rope_len else 0.0, rope_len=rope_len or 1,
                                                quantize=True)
        _, _, st_x = oracle.compressed_decode(s["q"][t], s["k_new"][t], s["k_pre"][t], s["v_new"][t], st_x, pos,
                                              block, theta=theta if rope_len else 0.0, rope_len=rope_len or 1,
                                              quantize=False)
        err = np.abs(to_np(out) - r_out)
        worst = max(worst, float(err.max()))
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, f"step {t}: max-abs {err.max():.3e}"
    say(f"  sequence D{D} b{block} W{W} rope {rope_mode}: worst max-abs over {T} steps {worst:.3e}")
    np.testing.assert_array_equal(deq(dev["ring_k"].cpu().numpy(), dev["ring_ks"].cpu().numpy()), st["ring_k"])
    np.testing.assert_array_equal(deq(dev["ring_v"].cpu().numpy(), dev["ring_vs"].cpu().numpy()), st["ring_v"])
    nfull = T // block
    pk, pks = dev["pool_k"].cpu().numpy(), dev["pool_ks"].cpu().numpy()
    pv, pvs = dev["pool_v"].cpu().numpy(), dev["pool_vs"].cpu().numpy()
    for bb in range(B):
        for h in range(Hkv):
            check_pooled_rows(pk[bb, h, :nfull], pks[bb, h, :nfull], st_x["pool_k"][bb, h, :nfull], "pooled k")
            check_pooled_rows(pv[bb, h, :nfull], pvs[bb, h, :nfull], st_x["pool_v"][bb, h, :nfull], "pooled v")
    assert np.all(pk[:, :, nfull:] == 0)                 # the block in progress has no row yet
    got = dev["front_k"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - st_x["front_k"]) <= 2.0 ** -21 * np.abs(st_x["front_k"]) + 1e-30)


def test_compressed_decode_edges():
    """No pooled capacity (window only), a capacity smaller than the blocks (later blocks dropped), positions
    below the window, and a negative position (nothing appended, output 0)."""
    theta = 10000.0
    for P, pos in ((0, [5, 300, 4000]), (3, [11, 41, 4095]), (64, [-1, 0, 255])):
        w = workloads.compressed_decode_case(seed=90 + P, B=3, Hq=8, Hkv=2, W=16, P=P, block=4, pos_lo=0,
                                             pos_hi=10)
        w["pos"] = np.asarray(pos, np.int32)
        say(f"edges P={P} pos={pos}")
        dev, ref = device_state(w)
        rope = swa.rope_table(theta, 4096, w["D"])
        out = run_step(dev, w["q_bits"], w["k_new_bits"], w["k_pre_bits"], w["v_new_bits"], w["pos"], 4, rope)
        check_step(w, dev, ref, out, rope, theta, 4096, f"edges P={P}")
        if pos[0] < 0:
            assert np.all(to_np(out)[0] == 0)


def test_compressed_decode_q0_counts_columns():
    """q = 0 weighs every visible column equally: the output is the plain mean of the visible dequantized
    values, which pins the number of pooled and exact columns (the oracle's lse count)."""
    w = workloads.compressed_decode_case(seed=95, B=4, Hq=4, Hkv=1, W=256, P=1024, block=4)
    w["pos"] = np.array([4095, 255, 256, 1000], np.int32)
    w["q"] = np.zeros_like(w["q"])
    w["q_bits"] = np.zeros_like(w["q_bits"])
    dev, ref = device_state(w)
    rope = swa.rope_table(10000.0, 4096, w["D"])
    out = run_step(dev, w["q_bits"], w["k_new_bits"], w["k_pre_bits"], w["v_new_bits"], w["pos"], 4, rope)
    r_out, lse, _ = oracle.compressed_decode(w["q"], w["k_new"], w["k_pre"], w["v_new"], ref, w["pos"], 4,
                                             rope_len=4096)
    assert [round(float(np.exp(x))) for x in lse[:, 0]] == [960 + 256, 256, 256, 186 + 256]
    assert_close(to_np(out), r_out, "bf16", "q=0")
