"""The C ABI without a GPU: the library loads, exports every symbol include/swa.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from compressed_kv_attention_amd import swa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

pytestmark = pytest.mark.skipif(not os.path.exists(swa.LIB_PATH), reason="libswa.so not built")

FAKE = 0x10000  # an aligned address that validation must reject before it is ever dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("swa_attn_prefill", "swa_attn_decode", "kv_pool_compress_rope", "swa_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = swa.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    assert set(swa.EXPORTS) <= set(declared_functions())
    assert L.swa_version() >= 100


def _p(**kw):
    d = dict(B=1, Hq=4, Hkv=2, T=64, D=64, window=16, compress_block=0, rope_len=0, scale=0.0, dtype=swa.SWA_BF16)
    d.update(kw)
    return swa.PrefillParams(**d)


def _prefill(p, ptrs=None, seg=None, prefix=None, pk=None, pv=None, cos=None, sin=None, lse=None, ws=None,
             ws_bytes=0):
    L = swa.lib()
    q = k = v = out = ptrs
    rc = L.swa_attn_prefill(ctypes.byref(p), q, k, v, pk, pv, seg, prefix, cos, sin, out, lse, ws, ws_bytes, None)
    return rc, L.swa_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(Hq=3, Hkv=2), swa.SWA_ERR_INVALID, "multiple of Hkv"),
    (dict(window=-1), swa.SWA_ERR_INVALID, "window"),
    (dict(D=48), swa.SWA_ERR_UNSUPPORTED, "head dim"),
    (dict(dtype=7), swa.SWA_ERR_INVALID, "dtype"),
    (dict(compress_block=-2), swa.SWA_ERR_INVALID, "compress_block"),
    (dict(compress_block=4, window=0), swa.SWA_ERR_INVALID, "window >= 1"),
    (dict(rope_len=10), swa.SWA_ERR_INVALID, "rope_len"),
    (dict(T=200000), swa.SWA_ERR_UNSUPPORTED, "exceeds"),
    (dict(scale=float("inf")), swa.SWA_ERR_INVALID, "scale"),
])
def test_prefill_rejects_bad_params(kw, code, text):
    rc, msg = _prefill(_p(**kw), ptrs=FAKE)
    assert rc == code and text in msg, (rc, msg)


def test_prefill_rejects_null_and_misaligned_pointers():
    rc, msg = _prefill(_p(), ptrs=None)
    assert rc == swa.SWA_ERR_INVALID and "must not be NULL" in msg
    rc, msg = _prefill(_p(), ptrs=FAKE + 2)
    assert rc == swa.SWA_ERR_INVALID and "aligned" in msg
    rc, msg = _prefill(_p(compress_block=4), ptrs=FAKE, pk=FAKE)  # one pooled tensor only
    assert rc == swa.SWA_ERR_INVALID and "pooled_v" in msg
    rc, msg = _prefill(_p(compress_block=4), ptrs=FAKE, pv=FAKE)
    assert rc == swa.SWA_ERR_INVALID and "pooled_k" in msg
    rc, msg = _prefill(_p(compress_block=4), ptrs=FAKE)           # none: pooled in the call, into the workspace
    assert rc == swa.SWA_ERR_INVALID and "workspace" in msg
    rc, msg = _prefill(_p(compress_block=4), ptrs=FAKE, seg=FAKE)
    assert rc == swa.SWA_ERR_UNSUPPORTED and "seg_ids" in msg
    rc, msg = _prefill(_p(rope_len=64), ptrs=FAKE)                # tables missing
    assert rc == swa.SWA_ERR_INVALID and "rope_cos" in msg
    rc, msg = _prefill(_p(rope_len=64), ptrs=FAKE, cos=FAKE, sin=FAKE)   # workspace missing
    assert rc == swa.SWA_ERR_INVALID and "workspace" in msg
    size = lambda p: swa.lib().swa_prefill_workspace_size(ctypes.byref(p))
    need = size(_p(rope_len=64))
    # key metadata (B*T packed key info, 2 sub-tile summaries and 1 sink range per
    # 64-key tile; each part 256-rounded) + rotated keys
    assert need == 3 * 256 + 1 * 2 * 64 * 64 * 2
    rc, msg = _prefill(_p(rope_len=64), ptrs=FAKE, cos=FAKE, sin=FAKE, ws=FAKE, ws_bytes=need - 1)
    assert rc == swa.SWA_ERR_INVALID and "too small" in msg
    assert size(_p()) == 3 * 256                               # bf16 plain: key metadata only
    assert size(_p(T=65)) == 512 + 256 + 256
    assert size(_p(dtype=swa.SWA_F32)) == 0                    # the fp32 kernel reads seg/prefix itself
    # compressed mode: no key metadata; room for pooled keys and values [B,Hkv,T/b,D]
    pooled = 2 * 1 * 2 * (64 // 4) * 64 * 2
    assert size(_p(compress_block=4)) == pooled
    assert size(_p(compress_block=4, rope_len=64)) == 1 * 2 * 64 * 64 * 2 + pooled
    assert size(_p(compress_block=4, dtype=swa.SWA_F32)) == 2 * 1 * 2 * 16 * 64 * 4
    assert size(_p(compress_block=100)) == 0                   # T/b = 0 pooled rows
    rc, msg = _prefill(_p(), ptrs=FAKE)                        # bf16 plain without workspace
    assert rc == swa.SWA_ERR_INVALID and "workspace" in msg


def test_empty_problems_are_ok_without_pointers():
    assert _prefill(_p(B=0))[0] == swa.SWA_OK
    assert _prefill(_p(T=0))[0] == swa.SWA_OK
    L = swa.lib()
    assert L.swa_kv_quantize(0, 64, None, None, None, None) == swa.SWA_OK
    assert L.kv_pool_compress_rope(0, 1, 16, 64, 4, swa.SWA_BF16, None, None, None, None, 0, None, None, None) == 0
    assert L.kv_pool_compress_rope(1, 1, 3, 64, 4, swa.SWA_BF16, None, None, None, None, 0, None, None, None) == 0
    dp = swa.DecodeParams(0, 4, 2, 64, 8, 4, 0.0, 0)
    assert L.swa_attn_decode(ctypes.byref(dp), *([None] * 14), None, 0, None) == swa.SWA_OK


def test_debug_visibility_limits():
    L = swa.lib()
    p = _p(T=20000)
    assert L.swa_debug_visibility(ctypes.byref(p), None, None, FAKE, FAKE, None, 0, None) == swa.SWA_ERR_UNSUPPORTED
    p = _p(T=20000, dtype=swa.SWA_F32)
    assert L.swa_debug_visibility(ctypes.byref(p), None, None, None, FAKE, None, 0, None) == swa.SWA_ERR_UNSUPPORTED
    p = _p()
    assert L.swa_debug_visibility(ctypes.byref(p), None, None, None, None, None, 0, None) == swa.SWA_ERR_INVALID
    assert "count_out" in L.swa_last_error().decode()
    # bf16 with segment ids: the key-metadata pre-pass needs the workspace
    assert L.swa_debug_visibility(ctypes.byref(p), FAKE, None, None, FAKE, None, 0, None) == swa.SWA_ERR_INVALID
    assert "workspace" in L.swa_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(W=0), swa.SWA_ERR_INVALID, "W must be"),
    (dict(S=-1), swa.SWA_ERR_INVALID, "S must be"),
    (dict(D=128), swa.SWA_ERR_UNSUPPORTED, "head dim"),
    (dict(num_splits=257), swa.SWA_ERR_INVALID, "num_splits"),
    (dict(num_splits=-1), swa.SWA_ERR_INVALID, "num_splits"),
    (dict(Hq=5, Hkv=2), swa.SWA_ERR_INVALID, "multiple"),
])
def test_decode_rejects_bad_params(kw, code, text):
    d = dict(B=2, Hq=4, Hkv=2, D=64, W=8, S=4, scale=0.0, num_splits=0)
    d.update(kw)
    dp = swa.DecodeParams(**d)
    L = swa.lib()
    rc = L.swa_attn_decode(ctypes.byref(dp), *([FAKE] * 14), None, 0, None)
    assert rc == code and text in L.swa_last_error().decode()


def test_decode_workspace_sizes():
    """Split-K workspace: one counter per (batch row, kv head, group of 4 query
    heads), then (m, l) and o[D] per split and query head of the group, each
    part 256-byte aligned; nothing with one split."""
    L = swa.lib()
    size = lambda **kw: L.swa_decode_workspace_size(ctypes.byref(swa.DecodeParams(**dict(
        dict(B=256, Hq=16, Hkv=4, D=64, W=256, S=256, scale=0.0, num_splits=0), **kw))))
    assert size() == 0                                   # 1024 units: the automatic choice is one split
    assert size(num_splits=1) == 0
    units = 1 * 4 * 1
    r = lambda x: (x + 255) // 256 * 256
    assert size(B=1, num_splits=8) == r(units * 4) + r(units * 8 * 4 * 2 * 4) + r(units * 8 * 4 * 64 * 4)
    assert size(B=1, Hq=24, Hkv=4, num_splits=2) == r(8 * 4) + r(8 * 2 * 4 * 2 * 4) + r(8 * 2 * 4 * 64 * 4)
    # automatic: one split while the eight waves of a small batch's workgroup walk at most two 64-row chunks
    # each (S + W <= 1024), else one split per 1024 rows, within 1024 workgroups
    assert size(B=1) == 0
    assert size(B=1, W=1024, S=0) == 0
    assert size(B=1, W=1024, S=64) == r(units * 4) + r(units * 2 * 4 * 2 * 4) + r(units * 2 * 4 * 64 * 4)
    assert size(B=1, W=8192, S=256) == r(units * 4) + r(units * 9 * 4 * 2 * 4) + r(units * 9 * 4 * 64 * 4)
    big = 64 * 4                                          # 64 rows x 4 kv heads: 256 units, at most 4 splits
    assert size(B=64, W=8192, S=256) == r(big * 4) + r(big * 4 * 4 * 2 * 4) + r(big * 4 * 4 * 64 * 4)
    assert size(B=128, W=8192, S=256) == 0                 # 512 units: two-wave workgroups, one split
    dp = swa.DecodeParams(1, 16, 4, 64, 256, 256, 0.0, 8)
    args = [FAKE] * 14
    assert L.swa_attn_decode(ctypes.byref(dp), *args, None, 0, None) == swa.SWA_ERR_INVALID
    assert "workspace" in L.swa_last_error().decode()
    assert L.swa_attn_decode(ctypes.byref(dp), *args, FAKE, size(B=1, num_splits=8) - 1, None) == \
        swa.SWA_ERR_INVALID
    assert "too small" in L.swa_last_error().decode()


def test_decode_rejects_half_given_new_token():
    dp = swa.DecodeParams(2, 4, 2, 64, 8, 4, 0.0, 0)
    L = swa.lib()
    args = [FAKE] * 14
    args[2] = None                                             # v_new missing, k_new given
    assert L.swa_attn_decode(ctypes.byref(dp), *args, None, 0, None) == swa.SWA_ERR_INVALID
    assert "k_new and v_new" in L.swa_last_error().decode()


def test_rope_and_quantize_validation():
    L = swa.lib()
    assert L.swa_rope_table(0.0, 4, 64, FAKE, FAKE, None) == swa.SWA_ERR_INVALID
    assert L.swa_rope_table(1e4, 4, 63, FAKE, FAKE, None) == swa.SWA_ERR_INVALID
    assert L.swa_kv_quantize(4, 48, FAKE, FAKE, FAKE, None) == swa.SWA_ERR_INVALID
    assert L.kv_pool_compress_rope(1, 1, 16, 64, 0, 1, FAKE, FAKE, None, None, 0, FAKE, FAKE, None) == 1


def test_budget_window_host_functions_match_golden_cases():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "budget_window.txt")) if l.strip() and not l.startswith("#")]
    for r in rows:
        d, ad, nh, nkv, L_, sites, msl, kvw, per_pos, bw, eff = (int(x) for x in r)
        assert swa.kv_budget_window(d, nh, nkv, L_, msl, sites, ad) == bw, r
        assert swa.effective_kv_window(d, nh, nkv, L_, msl, kvw, sites, ad) == eff, r
    assert swa.kv_budget_window(0, 16, 4, 12, 100) == -1


def _device_asm(src):
    import subprocess
    import tempfile
    from compressed_kv_attention_amd import build
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "k.s")
        cmd = [build._hipcc()] + [f for f in build.compile_flags() if f != "-fPIC"] + [
            "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def _vgprs(tok):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", tok):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def test_kernels_leave_m0_to_direct_loads():
    """The direct global->LDS loads set M0 inside their inline asm; that is
    only sound while no compiler-generated instruction of the kernels reads M0
    (the compiler reserves it and would not expect the asm to change it)."""
    for src in ("prefill_bf16.hip", "decode.hip"):
        text = _device_asm(src)
        outside = re.sub(r";;#ASMSTART.*?;;#ASMEND", "", text, flags=re.S)
        code = [l for l in outside.splitlines() if l.strip() and not l.strip().startswith((";", "."))]
        users = [l for l in code if re.search(r"\bm0\b", l)]
        assert not users, f"{src}: compiler-generated code uses M0: {users[:5]}"


def test_untracked_loads_are_left_alone_until_waited_for():
    """q and the appended token reach the decode kernel through global loads
    issued from inline asm, whose registers fill in later than the compiler
    believes; no instruction may read or write those registers before a
    vmcnt wait (checked on the generated assembly, in program order)."""
    text = _device_asm("decode.hip")
    pending, inasm, bad = {}, False, []
    for i, line in enumerate(text.splitlines()):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if s.startswith(";;#ASMEND"):
            inasm = False
            continue
        if not s or s.startswith((";", ".")):
            continue
        if s.startswith("s_endpgm") or re.match(r"s_waitcnt vmcnt\(", s):
            pending.clear()
            continue
        m = re.match(r"(global_load_\w+)\s+(v\[\d+:\d+\]|v\d+),", s)
        if m and inasm and "lds" not in m.group(1):
            for r in _vgprs(m.group(2)):
                pending[r] = i
            continue
        if pending and s[0].isalpha() and _vgprs(s) & set(pending):
            bad.append(s)
    assert not bad, f"instructions touch untracked-load registers before their wait: {bad[:5]}"


def test_rope_table_host_matches_fp64_angles():
    """Host table = cos/sin of pos * theta^(-2i/D) evaluated in fp64 and rounded
    once to fp32 (within one fp32 ulp: numpy's fp64 cos/sin and the C library's
    may round the last bit differently)."""
    import numpy as np
    for theta, T, D in ((10000.0, 4096, 64), (500.0, 300, 32), (1e6, 17, 36)):
        c, s = swa.rope_table_host(theta, T, D)
        i = np.arange(D // 2, dtype=np.float64)
        ang = np.arange(T, dtype=np.float64)[:, None] * theta ** (-2.0 * i / D)[None, :]
        for got, ref in ((c, np.cos(ang)), (s, np.sin(ang))):
            ref32 = ref.astype(np.float32)
            ulp = np.spacing(np.abs(ref32)).astype(np.float64)
            assert np.all(np.abs(got.astype(np.float64) - ref32.astype(np.float64)) <= ulp)
        assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)      # position 0 is the identity


def test_rope_table_host_validation():
    L = swa.lib()
    assert L.swa_rope_table_host(0.0, 4, 64, FAKE, FAKE) == swa.SWA_ERR_INVALID
    assert L.swa_rope_table_host(1e4, 4, 63, FAKE, FAKE) == swa.SWA_ERR_INVALID
    assert L.swa_rope_table_host(1e4, -1, 64, FAKE, FAKE) == swa.SWA_ERR_INVALID
    assert L.swa_rope_table_host(1e4, 4, 64, None, FAKE) == swa.SWA_ERR_INVALID
    assert L.swa_rope_table_host(1e4, 0, 64, None, None) == swa.SWA_OK


# The binding checks every tensor's full shape before any launch (the C ABI
# sees raw pointers only); CPU tensors suffice: shape errors come first, then
# the device check, so nothing here reaches the library's kernels.
def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def _prefill_kw(**over):
    import torch
    kw = dict(q=_t(2, 4, 64, 64), k=_t(2, 2, 64, 64), v=_t(2, 2, 64, 64),
              seg_ids=_t(2, 64, dtype=torch.int32), prefix=_t(2, 64, dtype=torch.uint8), window=16)
    kw.update(over)
    return kw


@pytest.mark.parametrize("over,what", [
    (dict(v=_t(2, 2, 63, 64)), "v"),
    (dict(k=_t(2, 2, 64, 32)), "k"),
    (dict(seg_ids=_t(2, 65, dtype=__import__("torch").int32)), "seg_ids"),
    (dict(prefix=_t(1, 64, dtype=__import__("torch").uint8)), "prefix"),
    (dict(out=_t(2, 4, 64, 32)), "out"),
    (dict(rope=(_t(64, 16, dtype=__import__("torch").float32), _t(64, 32, dtype=__import__("torch").float32))),
     "rope_cos"),
    (dict(compress_block=4, seg_ids=None, prefix=None, pooled_k=_t(2, 2, 16, 64), pooled_v=_t(2, 2, 15, 64)),
     "pooled_v"),
])
def test_prefill_wrapper_rejects_bad_shapes(over, what):
    with pytest.raises(ValueError, match=what):
        swa.prefill(**_prefill_kw(**over))


def test_prefill_wrapper_rejects_host_tensors_after_shapes():
    with pytest.raises(ValueError, match="device tensor"):
        swa.prefill(**_prefill_kw())


def _decode_args(**over):
    import torch
    B, Hq, Hkv, D, W, S = 3, 8, 2, 64, 16, 8
    a = dict(q=_t(B, Hq, D), ring_k=_t(B, Hkv, W, D, dtype=torch.int8), ring_v=_t(B, Hkv, W, D, dtype=torch.int8),
             ring_ks=_t(B, Hkv, W, 2, dtype=torch.float32), ring_vs=_t(B, Hkv, W, 2, dtype=torch.float32),
             sink_k=_t(B, Hkv, S, D, dtype=torch.int8), sink_v=_t(B, Hkv, S, D, dtype=torch.int8),
             sink_ks=_t(B, Hkv, S, 2, dtype=torch.float32), sink_vs=_t(B, Hkv, S, 2, dtype=torch.float32),
             pos=_t(B, dtype=torch.int32), sink_len=_t(B, dtype=torch.int32), k_new=_t(B, Hkv, D),
             v_new=_t(B, Hkv, D))
    a.update(over)
    return a


@pytest.mark.parametrize("over,what", [
    (dict(ring_v=_t(3, 2, 15, 64, dtype=__import__("torch").int8)), "ring_v"),
    (dict(ring_ks=_t(3, 2, 16, 1, dtype=__import__("torch").float32)), "ring_ks"),
    (dict(sink_vs=_t(3, 2, 9, 2, dtype=__import__("torch").float32)), "sink_vs"),
    (dict(sink_k=_t(3, 2, 8, 32, dtype=__import__("torch").int8)), "sink_k"),
    (dict(pos=_t(4, dtype=__import__("torch").int32)), "pos"),
    (dict(sink_len=_t(2, dtype=__import__("torch").int32)), "sink_len"),
    (dict(k_new=_t(3, 1, 64)), "k_new"),
    (dict(v_new=None), "k_new and v_new"),
    (dict(sink_v=None), "sink_k, sink_v"),
    (dict(out=_t(3, 8, 32)), "out"),
])
def test_decode_wrapper_rejects_bad_shapes(over, what):
    with pytest.raises(ValueError, match=what):
        swa.decode(**_decode_args(**over))


def test_decode_wrapper_rejects_host_tensors_after_shapes():
    with pytest.raises(ValueError, match="device tensor"):
        swa.decode(**_decode_args())


def test_pool_wrapper_rejects_bad_shapes():
    import torch
    with pytest.raises(ValueError, match="v must have shape"):
        swa.pool_compress_rope(_t(1, 2, 32, 64), _t(1, 2, 31, 64), 4)
    with pytest.raises(ValueError, match="rope_cos"):
        swa.pool_compress_rope(_t(1, 2, 32, 64), _t(1, 2, 32, 64), 4,
                               rope=(_t(32, 16, dtype=torch.float32), _t(32, 32, dtype=torch.float32)))


def test_compressed_decode_validation():
    L = swa.lib()
    dp = swa.DecodeParams(2, 4, 2, 64, 8, 16, 0.0, 0)
    P = [FAKE] * 16          # q, k_new, k_pre, v_new, ring x4, pool x4, front x2, pos, out

    def call(block=4, cos=None, sin=None, rope_len=0, ptrs=None, params=dp):
        rc = L.swa_attn_decode_compressed(ctypes.byref(params), block, cos, sin, rope_len, *(ptrs or P), None, 0,
                                          None)
        return rc, L.swa_last_error().decode()

    assert call(block=0) == (swa.SWA_ERR_INVALID, call(block=0)[1]) and "block" in call(block=0)[1]
    rc, msg = call(cos=FAKE)
    assert rc == swa.SWA_ERR_INVALID and "rope_cos and rope_sin" in msg
    rc, msg = call(cos=FAKE, sin=FAKE, rope_len=0)
    assert rc == swa.SWA_ERR_INVALID and "rope_len" in msg
    for i, name in ((2, "k_new_pre"), (12, "front_k"), (13, "front_v"), (1, "k_new")):
        ptrs = list(P)
        ptrs[i] = None
        rc, msg = call(ptrs=ptrs)
        assert rc == swa.SWA_ERR_INVALID and name.split("_pre")[0] in msg, (name, msg)
    ptrs = list(P)
    ptrs[8] = None                                    # pooled cache missing while P > 0
    rc, msg = call(ptrs=ptrs)
    assert rc == swa.SWA_ERR_INVALID and "sink_k" in msg
    rc, msg = call(params=swa.DecodeParams(2, 4, 2, 48, 8, 16, 0.0, 0))
    assert rc == swa.SWA_ERR_UNSUPPORTED


def test_compressed_decode_wrapper_rejects_bad_shapes():
    import torch
    a = _decode_args()
    kw = dict(q=a["q"], k_new=a["k_new"], k_new_pre=_t(3, 2, 64), v_new=a["v_new"], ring_k=a["ring_k"],
              ring_v=a["ring_v"], ring_ks=a["ring_ks"], ring_vs=a["ring_vs"], pool_k=a["sink_k"],
              pool_v=a["sink_v"], pool_ks=a["sink_ks"], pool_vs=a["sink_vs"],
              front_k=_t(3, 2, 64, dtype=torch.float32), front_v=_t(3, 2, 64, dtype=torch.float32), pos=a["pos"],
              block=4)
    for over, what in ((dict(k_new_pre=_t(3, 2, 32)), "k_new_pre"), (dict(front_v=_t(3, 1, 64)), "front_v"),
                       (dict(pool_vs=_t(3, 2, 7, 2, dtype=torch.float32)), "sink_vs"),
                       (dict(block=0), "block"), (dict(k_new_pre=None), "k_new_pre")):
        with pytest.raises(ValueError, match=what):
            swa.decode_compressed(**dict(kw, **over))
    with pytest.raises(ValueError, match="device tensor"):
        swa.decode_compressed(**kw)


def test_chunk_prefill_validation_and_workspace():
    L = swa.lib()
    size = lambda **kw: L.swa_chunk_prefill_workspace_size(ctypes.byref(swa.ChunkParams(**dict(
        dict(B=2, Hq=4, Hkv=2, D=64, W=8, S=5, Tc=13, scale=0.0), **kw))))
    C = 64                     # S + W - 1 = 12 cached rows, rounded up to 64
    Tv = C + 13
    r = lambda x: (x + 255) // 256 * 256
    pf = L.swa_prefill_workspace_size(ctypes.byref(swa.PrefillParams(2, 4, 2, Tv, 64, 8, 0, 0, 0.0, swa.SWA_BF16)))
    assert size() == 2 * r(2 * 2 * C * 64 * 2) + r(2 * Tv * 4) + r(2 * Tv) + r(pf)
    assert size(S=52, W=13) == size(S=64, W=1) < size(S=65, W=1)   # C = 64, 64, 128
    assert size(Tc=0) == 0 and size(W=0) == 0
    args = [FAKE] * 14        # q, k, v, ring x4, sink x4, pos0, sink_len, out
    p = swa.ChunkParams(2, 4, 2, 64, 8, 5, 13, 0.0)
    assert L.swa_attn_chunk_prefill(ctypes.byref(p), *args, None, 0, None) == swa.SWA_ERR_INVALID
    assert "workspace" in L.swa_last_error().decode()
    for i, name in ((0, "q"), (3, "ring_k"), (11, "pos0"), (7, "sink_k")):
        a2 = list(args)
        a2[i] = None
        assert L.swa_attn_chunk_prefill(ctypes.byref(p), *a2, FAKE, size(), None) == swa.SWA_ERR_INVALID
        assert name in L.swa_last_error().decode()
    bad = swa.ChunkParams(2, 4, 2, 64, 0, 5, 13, 0.0)
    assert L.swa_attn_chunk_prefill(ctypes.byref(bad), *args, FAKE, 1 << 30, None) == swa.SWA_ERR_INVALID
    big = swa.ChunkParams(2, 4, 2, 64, 8, 5, 131072, 0.0)
    assert L.swa_attn_chunk_prefill(ctypes.byref(big), *args, FAKE, 1 << 30, None) == swa.SWA_ERR_UNSUPPORTED
    empty = swa.ChunkParams(2, 4, 2, 64, 8, 5, 0, 0.0)
    assert L.swa_attn_chunk_prefill(ctypes.byref(empty), *([None] * 14), None, 0, None) == swa.SWA_OK


def test_chunk_prefill_wrapper_rejects_bad_shapes():
    import torch
    a = _decode_args()
    kw = dict(q=_t(3, 8, 10, 64), k=_t(3, 2, 10, 64), v=_t(3, 2, 10, 64), ring_k=a["ring_k"], ring_v=a["ring_v"],
              ring_ks=a["ring_ks"], ring_vs=a["ring_vs"], sink_k=a["sink_k"], sink_v=a["sink_v"],
              sink_ks=a["sink_ks"], sink_vs=a["sink_vs"], pos0=a["pos"], sink_len=a["sink_len"])
    for over, what in ((dict(k=_t(3, 2, 9, 64)), "k must"), (dict(v=_t(3, 1, 10, 64)), "v must"),
                       (dict(ring_vs=_t(3, 2, 16, 1, dtype=torch.float32)), "ring_vs"),
                       (dict(pos0=_t(2, dtype=torch.int32)), "pos"), (dict(out=_t(3, 8, 10, 32)), "out")):
        with pytest.raises(ValueError, match=what):
            swa.chunk_prefill(**dict(kw, **over))
    with pytest.raises(ValueError, match="device tensor"):
        swa.chunk_prefill(**kw)


def test_prefill_backward_validation():
    L = swa.lib()
    p = _p(T=64, D=64, window=16)
    n = L.swa_prefill_backward_workspace_size(ctypes.byref(p))
    r = lambda x: (x + 255) // 256 * 256
    nq, nk = 1 * 4 * 64 * 64 * 4, 1 * 2 * 64 * 64 * 4
    assert n == 2 * r(nq) + 2 * r(nk) + r(1 * 4 * 64 * 4) + 2 * r(nq)   # GQA 2: per-head dk/dv shares
    ptrs = [FAKE] * 13       # q, k, v, out, lse, dout, seg, prefix, cos, sin, dq, dk, dv
    call = lambda pp, pt, ws=FAKE, nb=n: L.swa_attn_prefill_backward(ctypes.byref(pp), *pt, ws, nb, None)
    assert call(_p(T=64, compress_block=4), ptrs) == swa.SWA_ERR_UNSUPPORTED
    assert call(p, ptrs, None, 0) == swa.SWA_ERR_INVALID and "workspace" in L.swa_last_error().decode()
    for i, name in ((0, "q"), (4, "lse"), (5, "dout"), (12, "dv")):
        pt = list(ptrs)
        pt[i] = None
        assert call(p, pt) == swa.SWA_ERR_INVALID and name in L.swa_last_error().decode()
    assert call(_p(T=64, D=48), ptrs) == swa.SWA_ERR_UNSUPPORTED
    assert call(_p(T=0), [None] * 13, None, 0) == swa.SWA_OK


def test_nsa_select_validation():
    L = swa.lib()
    p = _p(T=64, D=64, window=16, compress_block=4)
    n = L.swa_nsa_select_workspace_size(ctypes.byref(p))
    r = lambda x: (x + 255) // 256 * 256
    assert n == r(1 * 2 * 16 * 64 * 4)                            # fp32 pooled keys
    pr = _p(T=64, D=64, window=16, compress_block=4, rope_len=64)
    assert L.swa_nsa_select_workspace_size(ctypes.byref(pr)) == r(1 * 2 * 64 * 64 * 2) + r(1 * 2 * 16 * 64 * 4)
    pr = _p(T=64, D=64, window=16, compress_block=4, rope_len=64, dtype=swa.SWA_F32)
    assert L.swa_nsa_select_workspace_size(ctypes.byref(pr)) == r(1 * 2 * 64 * 64 * 4) + r(1 * 2 * 16 * 64 * 4)
    assert L.swa_nsa_select_workspace_size(ctypes.byref(_p(T=64, compress_block=0))) == 0
    ptrs = [FAKE] * 8           # q, k, v, cos, sin, out, lse, sel
    call = lambda pp, ns, pt, ws=FAKE, nb=n: L.swa_nsa_select_attn(ctypes.byref(pp), ns, *pt, ws, nb, None)
    assert call(p, 0, ptrs) == swa.SWA_ERR_INVALID and "n_select" in L.swa_last_error().decode()
    assert call(p, 33, ptrs) == swa.SWA_ERR_INVALID
    assert call(_p(T=64, compress_block=0), 4, ptrs) == swa.SWA_ERR_INVALID
    assert call(_p(T=64, window=0, compress_block=4), 4, ptrs) == swa.SWA_ERR_INVALID
    assert call(p, 4, ptrs, None, 0) == swa.SWA_ERR_INVALID and "workspace" in L.swa_last_error().decode()
    pt = list(ptrs)
    pt[1] = None
    assert call(p, 4, pt) == swa.SWA_ERR_INVALID and "k" in L.swa_last_error().decode()
