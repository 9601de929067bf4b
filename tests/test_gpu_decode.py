"""GPU parity of the int8 quantizer and the ring + sink decode step.

Source: [NS] "256-token滑动窗口+KV sink：Needle 2工具钉住机制源码分析", section
"256-token 滑动窗口：源码走读" (decode keeps recent | sink, no packing term);
cache layout priced by [NW] "How the 256-Token Sliding Window Works with Tools
as KV Sinks in Needle", section "Effective KV Window: Bounding the Cache Size".
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_attention_amd import swa, workloads
from gpu_util import assert_close, bf16_dev, say, to_np

pytestmark = pytest.mark.gpu


def test_quantizer_bit_exact():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((4096, 64)) * rng.uniform(1e-3, 30, (4096, 1))).astype(np.float32)
    x[3, :32] = 0.0
    x[7, 32:] = 0.0
    x[11, 0] = 127.0
    x[11, 1:33] = np.arange(-16, 16) + 0.5          # ties with scale 1 (rows mix groups)
    bits, vals = workloads.bf16_round(x)
    q, s = swa.kv_quantize(bf16_dev(bits))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize(vals)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def make_caches(w):
    """Quantize the caches on the GPU (for the kernel) and in the oracle (for the
    reference), and check the two agree bit for bit."""
    dev, ref = {}, {}
    for name in ("ring_k", "ring_v", "sink_k", "sink_v"):
        q, s = swa.kv_quantize(bf16_dev(w[name + "_bits"]))
        dev[name], dev[name[:-2] + ("_ks" if name.endswith("k") else "_vs")] = q, s
        shp = w[name].shape
        rq, rs = oracle.quantize(w[name].reshape(-1, shp[-1]))
        ref[name] = rq.reshape(shp)
        ref[name[:-2] + ("_ks" if name.endswith("k") else "_vs")] = rs.reshape(shp[:-1] + (shp[-1] // 32,))
    torch.cuda.synchronize()
    for k in ref:
        np.testing.assert_array_equal(dev[k].cpu().numpy(), ref[k])
    return dev, ref


def run_decode(w, dev, append=True, num_splits=0):
    out = swa.decode(bf16_dev(w["q_bits"]), dev["ring_k"], dev["ring_v"], dev["ring_ks"], dev["ring_vs"],
                     dev["sink_k"], dev["sink_v"], dev["sink_ks"], dev["sink_vs"],
                     torch.from_numpy(w["pos"]).cuda(), torch.from_numpy(w["sink_len"]).cuda(),
                     bf16_dev(w["k_new_bits"]) if append else None, bf16_dev(w["v_new_bits"]) if append else None,
                     num_splits=num_splits)
    torch.cuda.synchronize()
    return out


def oracle_decode(w, ref, append=True):
    return oracle.decode(w["q"], ref["ring_k"], ref["ring_v"], ref["ring_ks"], ref["ring_vs"], ref["sink_k"],
                         ref["sink_v"], ref["sink_ks"], ref["sink_vs"], w["pos"], w["sink_len"],
                         w["k_new"] if append else None, w["v_new"] if append else None)


@pytest.mark.parametrize("B,Hq,Hkv,D,W,S,pos,sink_len", [
    (4, 4, 2, 64, 8, 5, [5, 7, 12, 33], [5, 3, 5, 0]),            # partial ring, full, wrapped
    (3, 8, 1, 64, 16, 4, [4, 19, 100], [4, 4, 1]),                # G = 8
    (2, 2, 2, 32, 6, 3, [3, 50], [3, 2]),                         # D = 32, G = 1
    (5, 16, 4, 64, 256, 256, [256, 300, 511, 512, 20000], [256, 256, 100, 0, 256]),
    (2, 4, 2, 64, 1, 0, [0, 9], [0, 0]),                          # W = 1, no sinks
    (3, 4, 2, 64, 37, 11, [11, 47, 48], [11, 11, 11]),            # odd sizes
    (2, 8, 2, 64, 2048, 448, [700, 90000], [448, 300]),          # long walks: 39 and 37 chunks
    (2, 4, 1, 32, 1000, 100, [1099, 5000], [100, 77]),          # D = 32, ring wrapping mid-chunk
])
def test_decode_small(B, Hq, Hkv, D, W, S, pos, sink_len):
    w = workloads.decode_case(seed=B * 100 + W, B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, S=S, sink_len=sink_len)
    w["pos"] = np.asarray(pos, np.int32)
    say(f"decode B{B} {Hq}/{Hkv} D{D} W{W} S{S} pos {pos} sink_len {sink_len}")
    dev, ref = make_caches(w)
    out = run_decode(w, dev)
    r_out, _, rk, rv, rks, rvs = oracle_decode(w, ref)
    assert_close(to_np(out), r_out, "bf16", "decode")
    for name, r in (("ring_k", rk), ("ring_v", rv), ("ring_ks", rks), ("ring_vs", rvs)):
        np.testing.assert_array_equal(dev[name].cpu().numpy(), r)


# A seeded sweep: GQA groups 1, 2, 4, 8, both head dims, rings of 1..400 rows,
# sink caches of 0..300 rows partly filled, positions from an empty ring (pos =
# sink_len) to many wraps.
DEC_SWEEP = []
_drng = np.random.default_rng(4242)
for _i in range(20):
    _B = int(_drng.integers(1, 7))
    _Hkv = int(_drng.integers(1, 3))
    _G = int(_drng.choice([1, 2, 4, 8]))
    _W = int(_drng.integers(1, 401))
    _S = int(_drng.integers(0, 301))
    _sl = [int(_drng.integers(0, _S + 1)) for _ in range(_B)]
    _pos = [sl if _drng.random() < 0.2 else sl + int(_drng.integers(0, 4 * _W + 2)) for sl in _sl]
    DEC_SWEEP.append(pytest.param(_B, _G * _Hkv, _Hkv, (32, 64)[_i % 2], _W, _S, _pos, _sl, id=f"sweep{_i}"))


@pytest.mark.parametrize("B,Hq,Hkv,D,W,S,pos,sink_len", DEC_SWEEP)
def test_decode_sweep(B, Hq, Hkv, D, W, S, pos, sink_len):
    test_decode_small(B, Hq, Hkv, D, W, S, pos, sink_len)


def test_decode_without_append_and_q0_counts():
    B, Hq, Hkv, D, W, S = 3, 4, 2, 64, 16, 8
    w = workloads.decode_case(seed=77, B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, S=S, sink_len=[8, 2, 0])
    w["pos"] = np.array([8, 30, 5], np.int32)
    dev, ref = make_caches(w)
    out = run_decode(w, dev, append=False)
    r_out, *_ = oracle_decode(w, ref, append=False)
    assert_close(to_np(out), r_out, "bf16", "no-append")
    # q = 0: uniform weights -> output is the mean of the visible dequantized values
    w0 = dict(w)
    w0["q_bits"] = np.zeros_like(w["q_bits"])
    w0["q"] = np.zeros_like(w["q"])
    out0 = run_decode(w0, dev, append=False)
    r0, lse0, *_ = oracle_decode(w0, ref, append=False)
    n = np.rint(np.exp(lse0)).astype(int)
    for b, (p, sl) in enumerate(zip(w["pos"], w["sink_len"])):
        assert np.all(n[b] == sl + min(W, p - sl + 1))
    assert_close(to_np(out0), r0, "bf16", "q0")


def test_decode_full_size_one_layer():
    w = workloads.decode_case(seed=5)
    say(f"decode full: B{w['B']} {w['Hq']}/{w['Hkv']} D{w['D']} W{w['W']} S{w['S']}")
    dev, ref = make_caches(w)
    out = run_decode(w, dev)
    r_out, _, rk, rv, rks, rvs = oracle_decode(w, ref)
    assert_close(to_np(out), r_out, "bf16", "decode full")
    np.testing.assert_array_equal(dev["ring_k"].cpu().numpy(), rk)
    np.testing.assert_array_equal(dev["ring_vs"].cpu().numpy(), rvs)


def test_decode_bitwise_repeatable():
    """Thirty launches of a full-size decode layer give the same output bits:
    the two waves' merge through LDS and the appended row follow one order.
    (Each launch appends the same token at the same ring slot, so every launch
    sees the same cache.)"""
    w = workloads.decode_case(seed=9)
    dev, _ = make_caches(w)
    first = run_decode(w, dev).view(torch.int16).clone()
    for i in range(30):
        out = run_decode(w, dev).view(torch.int16)
        assert torch.equal(out, first), f"launch {i} differs"


def vmax_per_head(w, ref):
    """max |dequantized V| over each (sequence, kv head)'s caches, broadcast to [B, Hq, 1]."""
    G = w["Hq"] // w["Hkv"]
    m = np.zeros((w["B"], w["Hkv"]))
    for codes, scales in (("ring_v", "ring_vs"), ("sink_v", "sink_vs")):
        c = ref[codes].astype(np.float64)
        if c.size:
            deq = c * np.repeat(ref[scales].astype(np.float64), 32, axis=-1)
            m = np.maximum(m, np.abs(deq).max(axis=(2, 3)))
    vn = np.abs(w["v_new"]).max(axis=-1)
    return np.repeat(np.maximum(m, vn), G, axis=1)[:, :, None]


def split_invariant(a, b, vmax, what):
    """Outputs of two split counts agree within the rounding both carry: each
    weight operand p * s_v is one f16 number (relative error <= 2^-11 each way),
    so the two fp32 results differ by at most 2 * 2^-11 * max|v| before their
    bf16 rounding (half a step each, 2^-9 relative)."""
    a = a.float().cpu().numpy().astype(np.float64)
    b = b.float().cpu().numpy().astype(np.float64)
    tol = 2.0 ** -10 * vmax + 2.0 ** -8 * np.maximum(np.abs(a), np.abs(b))
    d = np.abs(a - b)
    say(f"  {what}: max |diff| {d.max():.3e} (max of diff / bound {float((d / tol).max()):.3f})")
    assert np.all(d <= tol), what


# Split-K: every (sequence, kv head) walk cut into num_splits parts, combined by
# the last workgroup to finish.  Oracle parity for each split count, and the
# same output whatever the count (the pin "output invariant to num_splits").
@pytest.mark.parametrize("B,Hq,Hkv,D,W,S,pos,sink_len", [
    (1, 16, 4, 64, 256, 256, [20000], [256]),                  # one conversation: the small-batch case
    (3, 8, 2, 32, 100, 60, [59, 130, 4000], [60, 10, 0]),      # empty ring, partial ring, no sinks
    (2, 12, 4, 64, 64, 200, [300, 263], [200, 150]),           # G = 3
    (4, 40, 4, 64, 48, 16, [16, 17, 70, 5000], [16, 16, 0, 7]),  # G = 10: 3 head groups
])
def test_decode_split_k(B, Hq, Hkv, D, W, S, pos, sink_len):
    w = workloads.decode_case(seed=300 + B * 7 + W, B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, S=S, sink_len=sink_len)
    w["pos"] = np.asarray(pos, np.int32)
    dev, ref = make_caches(w)
    r_out, _, rk, rv, rks, rvs = oracle_decode(w, ref)
    vmax = vmax_per_head(w, ref)
    base = None
    for splits in (1, 2, 3, 4, 8, 16, 33, 0):
        say(f"decode split-K B{B} {Hq}/{Hkv} D{D} W{W} S{S} splits {splits}")
        out = run_decode(w, dev, num_splits=splits)
        assert_close(to_np(out), r_out, "bf16", f"splits={splits}")
        for name, r in (("ring_k", rk), ("ring_v", rv), ("ring_ks", rks), ("ring_vs", rvs)):
            np.testing.assert_array_equal(dev[name].cpu().numpy(), r)
        if base is None:
            base = out.clone()
        else:
            split_invariant(out, base, vmax, f"splits={splits} vs 1")


def test_decode_split_k_full_size_and_repeatable():
    """The full decode layer (B256, 16/4 heads, ring 256 + 256 sinks) with 2 and
    4 splits (2048 and 4096 workgroups) against the oracle and against one
    split; ten launches of 4 splits give the same bits (the combine reads the
    partials in split order whichever workgroup finishes last)."""
    w = workloads.decode_case(seed=15)
    dev, ref = make_caches(w)
    r_out, *_ = oracle_decode(w, ref)
    vmax = vmax_per_head(w, ref)
    one = run_decode(w, dev, num_splits=1)
    for splits in (2, 4):
        out = run_decode(w, dev, num_splits=splits)
        assert_close(to_np(out), r_out, "bf16", f"full size, splits={splits}")
        split_invariant(out, one, vmax, f"full size splits={splits} vs 1")
    first = run_decode(w, dev, num_splits=4).view(torch.int16).clone()
    for i in range(10):
        assert torch.equal(run_decode(w, dev, num_splits=4).view(torch.int16), first), f"launch {i} differs"


def _rescaled(w, name, factor):
    """Replace input `name` by its values times `factor` (broadcast), rounded to bf16."""
    bits, vals = workloads.bf16_round((w[name].astype(np.float64) * factor).astype(np.float32))
    w[name], w[name + "_bits"] = vals, bits


def assert_close_scaled(got, ref, mag, what):
    """The int8-KV tolerance on outputs measured in units of the values' magnitude
    (the bounds are absolute for N(0,1) data; scaling V by c scales the output by c)."""
    assert_close(got / mag, ref / mag, "bf16", what)


@pytest.mark.parametrize("qmag,vmag", [(1e-6, 1.0), (1e5, 1.0), (1.0, 1e-4), (1.0, 1e5), (3e4, 3e4)])
@pytest.mark.parametrize("splits", [1, 4])
def test_decode_input_ranges(qmag, vmag, splits):
    """q and V far from unit scale: q is scaled by a power of two before its f16
    conversion and the f16 weight operand p * s_v is formed relative to the
    largest V scale seen, so neither overflows nor loses its low bits."""
    B, Hq, Hkv, D, W, S = 3, 8, 2, 64, 64, 32
    w = workloads.decode_case(seed=41, B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, S=S, sink_len=[32, 10, 0])
    w["pos"] = np.array([40, 300, 2000], np.int32)
    _rescaled(w, "q", qmag)
    for name in ("ring_v", "sink_v", "v_new"):
        _rescaled(w, name, vmag)
    say(f"decode ranges |q|~{qmag:g} |v|~{vmag:g} splits {splits}")
    dev, ref = make_caches(w)
    out = run_decode(w, dev, num_splits=splits)
    r_out, *_ = oracle_decode(w, ref)
    assert_close_scaled(to_np(out), r_out, vmag, f"|q|~{qmag:g} |v|~{vmag:g}")


def test_decode_mixed_v_magnitudes():
    """Rows of very different V magnitude in one walk (1e-4 .. 1e4, by row): the
    exponent bookkeeping rescales the accumulators as larger scales arrive."""
    B, Hq, Hkv, D, W, S = 2, 4, 1, 64, 128, 128
    w = workloads.decode_case(seed=43, B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, S=S)
    w["pos"] = np.array([700, 300], np.int32)
    rng = np.random.default_rng(44)
    for name, rows in (("ring_v", W), ("sink_v", S)):
        _rescaled(w, name, 10.0 ** rng.uniform(-4, 4, size=(B, Hkv, rows, 1)))
    dev, ref = make_caches(w)
    r_out, *_ = oracle_decode(w, ref)
    for splits in (1, 3):
        out = run_decode(w, dev, num_splits=splits)
        assert_close_scaled(to_np(out), r_out, 1e4, f"mixed V magnitudes, splits={splits}")


def test_decode_ignores_unwritten_ring_slots():
    """Early in a sequence most ring slots were never written.  Their codes and
    scales (here NaN and +inf scales, arbitrary codes) must not reach the output:
    the rows padding a partial chunk carry zero weight and their scales are not
    used."""
    B, Hq, Hkv, D, W, S = 2, 8, 2, 64, 256, 256
    w = workloads.decode_case(seed=45, B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, S=S, sink_len=[256, 100])
    w["pos"] = np.array([259, 120], np.int32)          # ring holds positions 256..259 and 100..120
    dev, ref = make_caches(w)
    poison = torch.tensor([float("nan"), float("inf")], device="cuda")
    for b, (p, sl) in enumerate(zip(w["pos"], w["sink_len"])):
        live = set(x % W for x in range(max(sl, p - W + 1), p + 1))
        dead = torch.tensor([t for t in range(W) if t not in live], device="cuda")
        vals = poison[torch.arange(dead.numel(), device="cuda") % 2]          # NaN, +inf, NaN, ...
        for name in ("ring_ks", "ring_vs"):
            dev[name][b, :, dead, :] = vals[None, :, None].expand(Hkv, -1, D // 32)
        dev["ring_k"][b, :, dead, :] = 127
        dev["ring_v"][b, :, dead, :] = -127
    for splits in (1, 2, 8):
        out = run_decode(w, dev, num_splits=splits)
        r_out, *_ = oracle_decode(w, ref)
        assert_close(to_np(out), r_out, "bf16", f"poisoned unwritten slots, splits={splits}")
