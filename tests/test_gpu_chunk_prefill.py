"""GPU parity of chunked prefill into existing caches (swa_attn_chunk_prefill).

Reading of the pages (oracle O9): a chunk at positions pos0 .. pos0+Tc-1
attends, with the decode mask of [NS] "256-token滑动窗口+KV sink：Needle 2工具钉住机制源码分析"
(section "256-token 滑动窗口：源码走读": recent | sink, no packing term), over
the sink rows, the ring as it was before the chunk and its own unquantized
keys; then the ring takes the chunk's last min(W, Tc) tokens.  Chunked prefill
itself is named by the DwarfStar README (4096-token chunks).

Compared: every output row at the int8-KV tolerance (cached rows are
dequantized and rounded to bf16 for the MFMA kernel); the ring bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_attention_amd import swa, workloads
from gpu_util import assert_close, bf16_dev, say, to_np

pytestmark = pytest.mark.gpu


def caches(w):
    """The ring and sink caches quantized by the library and by the oracle (checked equal)."""
    dev, ref = {}, {}
    for name in ("ring_k", "ring_v", "sink_k", "sink_v"):
        scal = name[:-2] + ("_ks" if name.endswith("k") else "_vs")
        shp = w[name].shape
        if shp[2] == 0:
            dev[name] = dev[scal] = None
            ref[name] = np.zeros(shp, np.int8)
            ref[scal] = np.zeros(shp[:-1] + (shp[-1] // 32,), np.float32)
            continue
        q, s = swa.kv_quantize(bf16_dev(w[name + "_bits"]))
        dev[name], dev[scal] = q, s
        rq, rs = oracle.quantize(w[name].reshape(-1, shp[-1]))
        ref[name] = rq.reshape(shp)
        ref[scal] = rs.reshape(shp[:-1] + (shp[-1] // 32,))
    torch.cuda.synchronize()
    for k in ref:
        if dev[k] is not None:
            np.testing.assert_array_equal(dev[k].cpu().numpy(), ref[k])
    return dev, ref


def run(w, dev):
    out = swa.chunk_prefill(bf16_dev(w["q_bits"]), bf16_dev(w["k_bits"]), bf16_dev(w["v_bits"]), dev["ring_k"],
                            dev["ring_v"], dev["ring_ks"], dev["ring_vs"], dev["sink_k"], dev["sink_v"],
                            dev["sink_ks"], dev["sink_vs"], torch.from_numpy(w["pos0"]).cuda(),
                            torch.from_numpy(w["sink_len"]).cuda())
    torch.cuda.synchronize()
    return out


def check(w, what):
    say(f"{what}: B{w['B']} {w['Hq']}/{w['Hkv']} D{w['D']} W{w['W']} S{w['S']} Tc{w['Tc']} "
        f"pos0 {list(w['pos0'][:4])} sink_len {list(w['sink_len'][:4])}")
    dev, ref = caches(w)
    out = run(w, dev)
    r_out, _, rk, rv, rks, rvs = oracle.chunk_prefill(w["q"], w["k"], w["v"], ref["ring_k"], ref["ring_v"],
                                                      ref["ring_ks"], ref["ring_vs"], ref["sink_k"], ref["sink_v"],
                                                      ref["sink_ks"], ref["sink_vs"], w["pos0"], w["sink_len"])
    assert_close(to_np(out), r_out, "bf16", what)
    for name, r in (("ring_k", rk), ("ring_v", rv), ("ring_ks", rks), ("ring_vs", rvs)):
        np.testing.assert_array_equal(dev[name].cpu().numpy(), r)


@pytest.mark.parametrize("D,W,S,Tc,pos0,sink_len", [
    (64, 8, 5, 13, [5, 20, 40], [5, 3, 0]),        # empty ring after the sinks, wrapped ring, no sinks
    (64, 8, 5, 3, [9, 30, 2], [5, 5, 5]),          # chunk shorter than the window; sink_len > pos0
    (32, 64, 0, 70, [0, 7, 100], [0, 0, 0]),       # no sink cache; an empty cache at position 0
    (64, 1, 4, 40, [4, 50, 77], [4, 2, 4]),        # window 1: every token sees sinks and itself
    (32, 37, 11, 129, [11, 300, 48], [11, 11, 6]), # odd sizes, several 64-key tiles, ragged tail
    (64, 256, 256, 1, [256, 5000, 40000], [256, 100, 256]),  # one token
    (64, 1, 0, 70, [0, 5, 130], [0, 0, 0]),        # no cached rows at all: the chunk alone
    (32, 65, 0, 100, [0, 64, 1000], [0, 0, 0]),    # cached part exactly 64 rows (no padding)
    (64, 33, 32, 65, [32, 40, 700], [32, 17, 32]), # sinks + ring exactly 64 rows
])
def test_chunk_prefill_small(D, W, S, Tc, pos0, sink_len):
    w = workloads.chunk_case(seed=D + W + Tc, B=3, Hq=4, Hkv=2, D=D, W=W, S=S, Tc=Tc, sink_len=sink_len)
    w["pos0"] = np.asarray(pos0, np.int32)
    check(w, "chunk small")


def test_chunk_prefill_gqa_groups():
    for G in (1, 3, 8):
        w = workloads.chunk_case(seed=100 + G, B=2, Hq=2 * G, Hkv=2, D=64, W=48, S=16, Tc=150, pos_lo=16,
                                 pos_hi=400)
        check(w, f"chunk G={G}")


def test_chunk_prefill_full_size():
    """B8, 16q/4kv heads, D64, ring 256 + 256 sinks (the decode caches), a 4096-token chunk at positions
    256..32767: every output row and the whole ring."""
    w = workloads.chunk_case(seed=9)
    check(w, "chunk full size")


def test_chunk_then_decode_sees_the_written_ring():
    """After a chunk, a decode step at the next position reads the ring the chunk wrote: the same result as
    the oracle's decode over the oracle's ring."""
    w = workloads.chunk_case(seed=11, B=2, Hq=4, Hkv=2, D=64, W=32, S=8, Tc=50, pos_lo=8, pos_hi=200)
    dev, ref = caches(w)
    run(w, dev)
    _, _, rk, rv, rks, rvs = oracle.chunk_prefill(w["q"], w["k"], w["v"], ref["ring_k"], ref["ring_v"],
                                                  ref["ring_ks"], ref["ring_vs"], ref["sink_k"], ref["sink_v"],
                                                  ref["sink_ks"], ref["sink_vs"], w["pos0"], w["sink_len"])
    d = workloads.decode_case(seed=12, B=2, Hq=4, Hkv=2, D=64, W=32, S=8)
    pos = (w["pos0"] + w["Tc"]).astype(np.int32)
    out = swa.decode(bf16_dev(d["q_bits"]), dev["ring_k"], dev["ring_v"], dev["ring_ks"], dev["ring_vs"],
                     dev["sink_k"], dev["sink_v"], dev["sink_ks"], dev["sink_vs"], torch.from_numpy(pos).cuda(),
                     torch.from_numpy(w["sink_len"]).cuda(), bf16_dev(d["k_new_bits"]), bf16_dev(d["v_new_bits"]))
    torch.cuda.synchronize()
    r_out, *_ = oracle.decode(d["q"], rk, rv, rks, rvs, ref["sink_k"], ref["sink_v"], ref["sink_ks"],
                              ref["sink_vs"], pos, w["sink_len"], d["k_new"], d["v_new"])
    assert_close(to_np(out), r_out, "bf16", "decode after chunk")
