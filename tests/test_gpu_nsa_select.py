"""GPU parity of the NSA selection branch (swa_nsa_select_attn) against O11.

[CA] "Compressed attention and the copy probe": section "Two kinds of
columns, pooled blocks and exact recent keys" names the selected branch (the
top-k blocks by their compressed scores), section "What we didn't build, and
why" leaves it and the gate out; reading A22 fixes the rest.

The selection is an integer decision taken from fp32 scores on the GPU and
fp64 scores in the oracle, so, as for any result with several correct
answers, it is checked for validity: the kernel's blocks are candidates,
there are min(n_select, candidates) of them, in score order, and no block
left out scores above a chosen one by more than the fp32 error bound of the
score (1e-4 (1 + |s|)).  The attention is then compared exactly where it is
unique: the oracle attends over the kernel's own selection (fp32: max-abs
1e-5; bf16 inputs: 2e-2 / 2e-3).
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_attention_amd import swa, workloads
from gpu_util import assert_close, dev_input, say, to_np

pytestmark = pytest.mark.gpu


def check_selection(w, sel, n_sel, theta):
    """Validity of the GPU selection against fp64 scores; returns the number of rows whose selection differs
    from the oracle's own."""
    B, Hq, Hkv, T, D, W, b = w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["window"], w["compress_block"]
    G = Hq // Hkv
    pk, _ = oracle.pool_rope(w["k"], w["v"], b, theta=theta, rope_len=T)
    pos = np.arange(T)
    scale = 1.0 / np.sqrt(D)
    nv = np.maximum(0, (pos - W + 1) // b)
    nv = np.minimum(nv, T // b)
    for bb in range(B):
        for h in range(Hq):
            qr = oracle.rope(w["q"][bb, h], pos, theta) if theta else w["q"][bb, h].astype(np.float64)
            sc = scale * qr @ pk[bb, h // G].T
            s = sel[bb, h]
            for t in range(T):
                n = min(n_sel, nv[t])
                chosen = s[t][s[t] >= 0]
                assert len(chosen) == n and np.all(s[t][n:] == -1), (bb, h, t)
                if n == 0:
                    continue
                assert np.all(chosen < nv[t]) and len(set(chosen.tolist())) == n
                cs = sc[t, chosen]
                eps = 1e-4 * (1 + np.abs(cs).max())
                assert np.all(np.diff(cs) <= eps), (bb, h, t, "order")
                rest = np.setdiff1d(np.arange(nv[t]), chosen)
                if len(rest):
                    assert sc[t, rest].max() <= cs.min() + eps, (bb, h, t, "top-k")


def run(w, n_sel, theta, what):
    q, k, v = dev_input(w, "q"), dev_input(w, "k"), dev_input(w, "v")
    rope = swa.rope_table(theta, w["T"], w["D"]) if theta else None
    out, lse, sel = swa.nsa_select(q, k, v, w["window"], w["compress_block"], n_sel, rope=rope)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    say(f"nsa {what}: B{w['B']} {w['Hq']}/{w['Hkv']} T{w['T']} D{w['D']} W{w['window']} b{w['compress_block']} "
        f"n{n_sel} {w['dtype']} rope {bool(theta)}")
    check_selection(w, sel, n_sel, theta)
    r_out, r_lse, r_sel = oracle.nsa_select(w["q"], w["k"], w["v"], w["window"], w["compress_block"], n_sel,
                                            theta=theta, sel=sel)
    _, _, own = oracle.nsa_select(w["q"], w["k"], w["v"], w["window"], w["compress_block"], n_sel, theta=theta)
    differ = int(np.any(own != sel, axis=-1).sum())
    say(f"  rows whose selection differs from the oracle's own: {differ} of {sel.shape[0] * sel.shape[1] * sel.shape[2]}")
    assert_close(to_np(out), r_out, w["dtype"], "out over the kernel's selection")
    fin = np.isfinite(r_lse)
    assert np.array_equal(np.isfinite(lse.cpu().numpy()), fin)
    assert np.abs(lse.cpu().numpy()[fin] - r_lse[fin]).max(initial=0.0) <= (1e-5 if w["dtype"] == "f32" else 2e-2)


@pytest.mark.parametrize("block,dtype", [(4, "f32"), (16, "f32"), (4, "bf16")])
def test_nsa_select_compressed_config(block, dtype):
    """The compressed-attention config (B4, 8/8 heads, D64, T4096, window 256) with 16 selected blocks."""
    w = workloads.compressed(block=block, dtype=dtype)
    run(w, 16, w["rope_theta"], f"C4 b{block}")


@pytest.mark.parametrize("B,Hq,Hkv,T,D,W,b,n,dtype,theta", [
    (2, 4, 2, 300, 32, 20, 5, 3, "f32", 10000.0),
    (1, 6, 2, 257, 64, 1, 1, 32, "f32", 0.0),
    (3, 2, 2, 130, 64, 64, 8, 1, "bf16", 10000.0),
    (1, 2, 1, 100, 64, 200, 4, 8, "f32", 10000.0),   # window past T: no candidate anywhere
    (2, 4, 2, 400, 32, 48, 16, 8, "bf16", 10000.0),  # bf16 at D = 32, long blocks
    (1, 8, 4, 333, 64, 30, 3, 16, "bf16", 0.0),      # bf16, a block of 3, no RoPE
])
def test_nsa_select_small(B, Hq, Hkv, T, D, W, b, n, dtype, theta):
    w = workloads.prefill_case(B, Hq, Hkv, T, D, W, dtype=dtype, seed=B * 7 + T, compress_block=b)
    run(w, n, theta, "small")
