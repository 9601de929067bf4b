"""swa_attn_decode_noalloc: the decode entry point for callers that cannot
allocate keeps its split-K state in the library's own device array.  Its
output must equal swa_attn_decode's (same kernels, same split count) and the
oracle's, on two calls in a row, the second smaller than the first."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from compressed_kv_attention_amd import swa, workloads
from gpu_util import assert_close, bf16_dev, say, to_np

pytestmark = pytest.mark.gpu


def _caches(w):
    dev, ref = {}, {}
    for name in ("ring_k", "ring_v", "sink_k", "sink_v"):
        q, s = swa.kv_quantize(bf16_dev(w[name + "_bits"]))
        sname = name[:-2] + ("_ks" if name.endswith("k") else "_vs")
        dev[name], dev[sname] = q, s
        shp = w[name].shape
        rq, rs = oracle.quantize(w[name].reshape(-1, shp[-1]))
        ref[name], ref[sname] = rq.reshape(shp), rs.reshape(shp[:-1] + (shp[-1] // 32,))
    return dev, ref


def _call(entry, w, dev, splits, out, workspace=None):
    """One call through the C ABI (ctypes on libswa.so)."""
    L = swa.lib()
    q = bf16_dev(w["q_bits"])
    kn, vn = bf16_dev(w["k_new_bits"]), bf16_dev(w["v_new_bits"])
    pos, sl = torch.from_numpy(w["pos"]).cuda(), torch.from_numpy(w["sink_len"]).cuda()
    p = swa.DecodeParams(w["B"], w["Hq"], w["Hkv"], w["D"], w["W"], w["S"], 0.0, splits)
    ptrs = [swa._ptr(t) for t in (q, kn, vn, dev["ring_k"], dev["ring_v"], dev["ring_ks"], dev["ring_vs"],
                                  dev["sink_k"], dev["sink_v"], dev["sink_ks"], dev["sink_vs"], pos, sl, out)]
    stream = swa._stream(q)
    if entry == "noalloc":
        rc = L.swa_attn_decode_noalloc(ctypes.byref(p), *ptrs, stream)
    else:
        nbytes = workspace.numel() if workspace is not None else 0
        rc = L.swa_attn_decode(ctypes.byref(p), *ptrs, swa._ptr(workspace), nbytes, stream)
    assert rc == swa.SWA_OK, L.swa_last_error().decode()
    torch.cuda.synchronize()
    return out


def _case(seed, B, W, S, sink_len, pos, splits):
    w = workloads.decode_case(seed=seed, B=B, Hq=16, Hkv=4, D=64, W=W, S=S, sink_len=sink_len)
    w["pos"] = np.asarray(pos, np.int32)
    dev, ref = _caches(w)
    ws = swa.decode_workspace(bf16_dev(w["q_bits"]), dev["ring_k"], dev["sink_k"], splits)
    say(f"no-alloc decode B{B} W{W} S{S} splits {splits}: workspace of the allocating call "
        f"{0 if ws is None else ws.numel()} bytes")
    want = _call("alloc", w, dev, splits, torch.empty((B, 16, 64), dtype=torch.bfloat16, device="cuda"), ws)
    got = _call("noalloc", w, dev, splits, torch.empty((B, 16, 64), dtype=torch.bfloat16, device="cuda"))
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "no-alloc output differs from swa_attn_decode"
    r_out, *_ = oracle.decode(w["q"], ref["ring_k"], ref["ring_v"], ref["ring_ks"], ref["ring_vs"], ref["sink_k"],
                              ref["sink_v"], ref["sink_ks"], ref["sink_vs"], w["pos"], w["sink_len"], w["k_new"],
                              w["v_new"])
    assert_close(to_np(got), r_out, "bf16", f"no-alloc B{B} splits {splits}")


def test_noalloc_matches_allocating_decode_twice_second_smaller():
    # first call: 6 sequences, automatic split count (8 parts: 192 workgroups of state)
    _case(seed=61, B=6, W=256, S=256, sink_len=[256, 200, 0, 256, 17, 256], pos=[9000, 300, 40, 256, 17, 700],
          splits=0)
    # second call, smaller: 2 sequences, shorter caches, 3 parts; the array keeps the first call's
    # partials, which this call must neither read nor depend on
    _case(seed=62, B=2, W=64, S=32, sink_len=[32, 5], pos=[100, 5], splits=3)


def test_noalloc_rejects_state_beyond_its_array_without_launching():
    L = swa.lib()
    p = swa.DecodeParams(256, 16, 4, 64, 256, 256, 0.0, 64)   # 1024 units x 64 splits: far beyond 4 MiB
    fake = 0x10000
    rc = L.swa_attn_decode_noalloc(ctypes.byref(p), *([fake] * 14), None)
    assert rc == swa.SWA_ERR_UNSUPPORTED and "exceeds" in L.swa_last_error().decode()
