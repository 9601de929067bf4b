"""GPU parity of the prefill backward (swa_attn_prefill_backward) against O10.

The packing mask is the training-side mask ([NS] "256-token滑动窗口+KV sink：
Needle 2工具钉住机制源码分析", section "KV sink 如何「钉住」工具"; [NW] "How the
256-Token Sliding Window Works with Tools as KV Sinks in Needle", section "KV
Sinks for Tools"); the backward is the derivative of the forward (reading A21).

The GPU takes the forward's own out and lse; the oracle recomputes the exact
softmax.  Tolerances, relative to the largest gradient magnitude g of each
tensor: fp32 inputs, max-abs <= 1e-5 g (fp32 sums over at most a few
thousand terms); bf16 inputs, max-abs <= 2e-2 g and mean-abs <= 2e-3 g (the
forward's bf16 rounding of q * scale, P and out moves every weight by up to
2^-8 relative, the int8-KV / bf16 output bound scaled to the gradient).
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_attention_amd import swa, workloads
from gpu_util import dev_input, dev_opt, say, to_np

pytestmark = pytest.mark.gpu


def compare(got, ref, dtype, what):
    got = np.asarray(got, np.float64)
    g = float(np.abs(ref).max()) or 1.0
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} (max |grad| {g:.3e})")
    assert np.all(np.isfinite(got)), what
    if dtype == "f32":
        assert mx <= 1e-5 * g, what
    else:
        assert mx <= 2e-2 * g and mean <= 2e-3 * g, what


def run_case(w, theta=0.0, what=""):
    q, k, v = dev_input(w, "q"), dev_input(w, "k"), dev_input(w, "v")
    seg = dev_opt(w["seg_ids"], np.int32)
    pre = dev_opt(w["prefix"], np.uint8)
    rope = swa.rope_table(theta, w["T"], w["D"]) if theta else None
    out, lse = swa.prefill(q, k, v, seg, pre, w["window"], rope=rope, return_lse=True)
    rng = np.random.default_rng(w.get("seed", 0) + 1000)
    g32 = rng.standard_normal(out.shape).astype(np.float32)
    if w["dtype"] == "bf16":
        bits, gvals = workloads.bf16_round(g32)
        dout = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        gvals = g32
        dout = torch.from_numpy(g32).cuda()
    dq, dk, dv = swa.prefill_backward(q, k, v, out, lse, dout, seg, pre, w["window"], rope=rope)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.prefill_backward(w["q"], w["k"], w["v"], gvals, w["seg_ids"], w["prefix"], w["window"],
                                         theta=theta)
    say(f"backward {what}: B{w['B']} {w['Hq']}/{w['Hkv']} T{w['T']} D{w['D']} W{w['window']} {w['dtype']} "
        f"rope {bool(theta)}")
    compare(to_np(dq), rq, w["dtype"], "dq")
    compare(to_np(dk), rk, w["dtype"], "dk")
    compare(to_np(dv), rv, w["dtype"], "dv")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_tiny_config(dtype):
    w = workloads.prefill_case(1, 1, 1, 64, 32, 16, dtype=dtype, seed=1,
                               seg_ids=np.array([[1] * 8 + [2] * 56], np.int32),
                               prefix=np.array([[1] * 8 + [0] * 56], np.uint8))
    run_case(w, what="tiny")


CASES = [
    # B, Hq, Hkv, T, D, window, segments, rope
    (2, 8, 2, 256, 64, 32, "needle", True),
    (2, 4, 4, 200, 32, 0, "one", False),
    (3, 6, 2, 150, 64, 17, "packed", False),
    (1, 3, 1, 97, 32, 1, "needle", True),
    (2, 4, 2, 300, 64, 500, "packed", True),
]


def structure(kind, B, T, rng):
    if kind == "one":
        return None, None
    seg = np.ones((B, T), np.int32)
    pre = np.zeros((B, T), np.uint8)
    for b in range(B):
        if kind == "needle":
            n = int(rng.integers(4, T // 3))
            seg[b, n:] = 2
            pre[b, :n] = 1
        else:
            cuts = np.sort(rng.choice(np.arange(5, T - 5), size=3, replace=False))
            s = 1
            for i in range(T):
                if s <= 3 and i >= cuts[s - 1]:
                    s += 1
                seg[b, i] = s
            seg[b, T - int(rng.integers(0, 9)):] = 0
            pre[b, : int(rng.integers(1, 9))] = 1
    return seg, pre


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_small(case, dtype):
    B, Hq, Hkv, T, D, W, kind, rope = CASES[case]
    rng = np.random.default_rng(500 + case)
    seg, pre = structure(kind, B, T, rng)
    w = workloads.prefill_case(B, Hq, Hkv, T, D, W, dtype=dtype, seed=600 + case, seg_ids=seg, prefix=pre)
    run_case(w, theta=10000.0 if rope else 0.0, what=f"case {case}")


def test_backward_needle_full_size():
    """The needle configuration (B8, 8q/2kv, D64, T2048, window 256, sink prefixes 64..384, RoPE), bf16."""
    w = workloads.needle()
    run_case(w, theta=w["rope_theta"], what="needle full size")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_sinks_in_later_segments(dtype):
    """Sinks at the start of three segments of a 2500-token row (79 key tiles, a ragged tail of padding) and a
    short window: a key tile of sinks is seen by every later row of its segment, far past the band, so the dk/dv
    pass walks query tiles marked across several words of its tile set."""
    B, Hq, Hkv, T, D, W = 2, 4, 1, 2500, 64, 64
    seg = np.zeros((B, T), np.int32)
    pre = np.zeros((B, T), np.uint8)
    for b in range(B):
        seg[b, :800] = 1
        seg[b, 800:1900] = 2
        seg[b, 1900:T - 7 - b] = 3
        pre[b, :41] = 1
        pre[b, 800:831 + 3 * b] = 1
        pre[b, 1900:1906] = 1
    w = workloads.prefill_case(B, Hq, Hkv, T, D, W, dtype=dtype, seed=777, seg_ids=seg, prefix=pre)
    run_case(w, what="sinks in later segments")
