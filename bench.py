"""Benchmark of the hot path on one MI355X.

One step = one pass of every hot-path row over one batch of synthetic input:
  * needle-shaped windowed+sink GQA prefill, bf16 (B8, 8q/2kv heads, D64,
    T2048, window 256, per-row sink prefix of 64..384 tool tokens, RoPE);
  * compressed-column prefill, bf16 (B4, 8/8 heads, D64, T4096, window 256,
    block 4): pooling + midpoint RoPE, then attention over [pooled, exact];
  * one decode step over 12 layers of int8 ring (256) + sink (256) caches
    (B256, 16q/4kv heads, D64, positions up to 32768).
Each part is captured in a HIP graph and replayed, input copies rotate so that
the working set exceeds the 256 MB Infinity Cache, and HIP events on the
launch stream time the region.  `value` is the prefill throughput in TFLOP/s
counted on visible (query, key) pairs only: 4 * D * Hq * sum(n_vis).

The JSON line also carries the decode HBM rate, the other prefill workloads
(packed multi-segment rows, compressed block 16), a `roofline` object for the
dominant kernel and a `cpu_baseline` object (the CPU oracle on a bounded
sample of the same workload).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CUs x 4096 FLOP/clk x 2.4 GHz, dense
HBM_PEAK_GBS = 8000.0
FP32_PEAK_TFLOPS = 157.3          # vector fp32 (the backward's arithmetic)
ROTATE_BYTES = 600 << 20          # > 2 x the 256 MB MALL


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=20, help="iterations per timed graph when timing one kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--parts", default="needle,compressed4,decode,packed,compressed16,decode_b1,decode_b8,decode_b32,decode_c4,chunk,backward,nsa")
    ap.add_argument("--decode-splits", type=int, default=0,
                    help="num_splits of the batch-256 decode part (0: the library's choice)")
    ap.add_argument("--eager", action="store_true",
                    help="launch kernels directly instead of replaying HIP graphs (for counter collection)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times) and exit; its HBM counters "
                         "give the scale factor of FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


def kernel_source_hash(names):
    """sha256 (first 16 hex digits) of the HIP sources a kernel is built from (concatenated in the given
    order); a counter summary taken on other source no longer describes the kernel."""
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "compressed_kv_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# the files the decode kernel is compiled from (its own source and the device helpers it includes)
DECODE_SOURCES = ("decode.hip", "swa_common.h", "swa_internal.h")
# the files the kernels of a bf16 prefill call (pre-pass and attention) are compiled from
PREFILL_SOURCES = ("prefill_bf16.hip", "pool_rope.hip", "swa_common.h", "swa_internal.h", "swa_tiles.h")


def measured_traffic(kernel, sources):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib):
    import torch
    dev = torch.device("cuda:0")
    n = mib << 20
    x = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 3}))


class Part:
    """One workload: device inputs (several rotating copies), a launch function and its work counts."""

    def __init__(self, name, launch, ncopies, flops=0.0, bytes_=0.0, kernel=None):
        self.name, self.launch, self.ncopies = name, launch, ncopies
        self.flops, self.bytes, self.kernel = flops, bytes_, kernel


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    import torch

    from compressed_kv_attention_amd import swa, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    parts_wanted = args.parts.split(",")

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    def copies(n, *tensors):
        return [tuple(t.clone() for t in tensors) for _ in range(n)]

    parts = {}

    # ---- needle-shaped prefill -------------------------------------------------
    def make_prefill(name, w, step_bytes_extra=0):
        q, k, v = bf16(w["q_bits"]), bf16(w["k_bits"]), bf16(w["v_bits"])
        seg = torch.from_numpy(w["seg_ids"]).to(dev) if w["seg_ids"] is not None else None
        pre = torch.from_numpy(w["prefix"]).to(dev) if w["prefix"] is not None else None
        rope = swa.rope_table(w["rope_theta"], w["T"], w["D"]) if w["rope_theta"] else None
        per_copy = (q.numel() * 2 + k.numel() * 4) * 2
        n = max(2, min(16, ROTATE_BYTES // per_copy + 1))
        bufs = [(q.clone(), k.clone(), v.clone(), torch.empty_like(q)) for _ in range(n)]
        ws = swa.prefill_workspace(q, k, w["window"], rope)
        _, count = swa.debug_visibility(w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["window"], torch.bfloat16,
                                        seg, pre, want_mask=False)
        nvis = int(count.to(torch.int64).sum().item())
        flops = 4.0 * w["D"] * w["Hq"] * nvis
        bytes_ = q.numel() * 2 * 2 + k.numel() * 2 * 2

        def launch(i):
            qq, kk, vv, oo = bufs[i % n]
            swa.prefill(qq, kk, vv, seg, pre, w["window"], rope=rope, out=oo, workspace=ws)
        p = Part(name, launch, n, flops, bytes_, kernel="prefill_bf16_kernel")
        p.extra = dict(B=w["B"], Hq=w["Hq"], Hkv=w["Hkv"], T=w["T"], D=w["D"], window=w["window"],
                       visible_pairs_per_head=nvis)
        p.w = w
        p.count = count.cpu().numpy()
        return p

    def make_compressed(name, block):
        w = workloads.compressed(block=block, dtype="bf16")
        q, k, v = bf16(w["q_bits"]), bf16(w["k_bits"]), bf16(w["v_bits"])
        rope = swa.rope_table(w["rope_theta"], w["T"], w["D"])
        per_copy = q.numel() * 2 * 4
        n = max(2, min(16, ROTATE_BYTES // per_copy + 1))
        bufs = []
        for _ in range(n):
            bufs.append((q.clone(), k.clone(), v.clone(), torch.empty_like(q)))
        ws = swa.prefill_workspace(q, k, w["window"], rope, block)
        _, count = swa.debug_visibility(w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["window"], torch.bfloat16,
                                        compress_block=block, want_mask=False)
        nvis = int(count.to(torch.int64).sum().item())
        flops = 4.0 * w["D"] * w["Hq"] * nvis
        nb = w["T"] // block
        bytes_ = q.numel() * 2 * 2 + k.numel() * 2 * 2 + 2 * (w["B"] * w["Hkv"] * nb * w["D"] * 2) * 2

        # the step pools k and v and attends: one call, given no pooled inputs (its pre-pass rotates the exact
        # keys and forms the rotated pooled keys and the pooled values in one read of k and v)
        def launch_step(i):
            qq, kk, vv, oo = bufs[i % n]
            swa.prefill(qq, kk, vv, window=w["window"], rope=rope, compress_block=block, out=oo, workspace=ws)
        p = Part(name, launch_step, n, flops, bytes_, kernel="prefill_bf16_kernel")
        p.extra = dict(B=w["B"], Hq=w["Hq"], Hkv=w["Hkv"], T=w["T"], D=w["D"], window=w["window"], block=block,
                       visible_pairs_per_head=nvis)
        p.w = w
        return p

    decode_ws = {}

    def make_decode(name, B=256, min_layers=12, num_splits=0):
        """One decode launch per layer over distinct caches.  The batch-256 part is the step's 12 layers
        (0.92 GB of cache); smaller batches use as many cache sets as it takes to exceed the 256 MB
        Infinity Cache, so every rate is an HBM rate."""
        Hq, Hkv, D, W, S = 16, 4, 64, 256, 256
        cache_bytes = 2 * (B * Hkv * (W + S) * D) + 2 * (B * Hkv * (W + S) * (D // 32) * 4)
        io_bytes = 2 * B * Hq * D * 2 + 2 * B * Hkv * D * 2 + 2 * B * Hkv * (D + (D // 32) * 4)
        per_layer = cache_bytes + io_bytes
        layers = max(min_layers, min(2048, -(-ROTATE_BYTES // per_layer)))
        g = torch.Generator(device=dev)
        g.manual_seed(5)
        caches = []
        for _ in range(layers):
            c = {}
            for nm, rows in (("ring_k", W), ("ring_v", W), ("sink_k", S), ("sink_v", S)):
                x = torch.randn((B, Hkv, rows, D), generator=g, device=dev).to(torch.bfloat16)
                c[nm], c[nm + "s"] = swa.kv_quantize(x)
            c["q"] = torch.randn((B, Hq, D), generator=g, device=dev).to(torch.bfloat16)
            c["k_new"] = torch.randn((B, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
            c["v_new"] = torch.randn((B, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
            c["out"] = torch.empty_like(c["q"])
            caches.append(c)
        rng = np.random.default_rng(5)
        pos = torch.from_numpy(rng.integers(512, 32768, size=B).astype(np.int32)).to(dev)
        sink_len = torch.full((B,), S, dtype=torch.int32, device=dev)
        # one zero-filled split-K workspace serves every layer: launches on one stream run one after
        # another and each leaves its counters at zero
        c0 = caches[0]
        ws = swa.decode_workspace(c0["q"], c0["ring_k"], c0["sink_k"], num_splits)
        decode_ws[name] = ws

        def launch(i):
            for c in caches:
                swa.decode(c["q"], c["ring_k"], c["ring_v"], c["ring_ks"], c["ring_vs"], c["sink_k"], c["sink_v"],
                           c["sink_ks"], c["sink_vs"], pos, sink_len, c["k_new"], c["v_new"],
                           num_splits=num_splits, out=c["out"], workspace=ws)
        p = Part(name, launch, 1, 0.0, per_layer * layers, kernel="decode_kernel")
        p.extra = dict(B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, S=S, layers=layers, bytes_per_layer=per_layer,
                       num_splits=num_splits or "auto",
                       workspace_bytes=0 if ws is None else ws.numel())
        p.tokens = B
        p.launches = layers
        # iterations per timed graph: about as many launches as 20 passes over 12 layers
        p.reps = max(1, (args.reps * 12) // layers)
        return p

    def make_compressed_decode(name, block=4, layers=12, B=256):
        """The compressed decode step: B256 16q/4kv D64, window 256, pooled blocks of `block` (capacity for
        4096 positions), positions 512..4095 (the 4K context of the compressed-cache figure); 12 layers of
        caches.  Bytes counted: the rows each query walks (visible pooled blocks + window, codes and scales),
        q, out, the appended token, the frontier read and write, and the pooled rows written."""
        Hq, Hkv, D, W = 16, 4, 64, 256
        P = 4096 // block
        g = torch.Generator(device=dev)
        g.manual_seed(6)
        rng = np.random.default_rng(6)
        pos_np = rng.integers(512, 4096, size=B).astype(np.int64)
        pos = torch.from_numpy(pos_np.astype(np.int32)).to(dev)
        rope = swa.rope_table(10000.0, 4096, D)
        caches = []
        for _ in range(layers):
            c = {}
            for nm, rows in (("ring_k", W), ("ring_v", W), ("pool_k", P), ("pool_v", P)):
                x = torch.randn((B, Hkv, rows, D), generator=g, device=dev).to(torch.bfloat16)
                c[nm], c[nm + "s"] = swa.kv_quantize(x)
            for nm, shape in (("q", (B, Hq, D)), ("k_new", (B, Hkv, D)), ("k_pre", (B, Hkv, D)),
                              ("v_new", (B, Hkv, D))):
                c[nm] = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
            c["front_k"] = torch.randn((B, Hkv, D), generator=g, device=dev)
            c["front_v"] = torch.randn((B, Hkv, D), generator=g, device=dev)
            c["out"] = torch.empty_like(c["q"])
            caches.append(c)
        row = D + (D // 32) * 4                                   # int8 codes + fp32 scales of one row
        n_vis = np.maximum(pos_np - W + 1, 0) // block
        walked = (n_vis + np.minimum(W, pos_np + 1) - 1).sum()    # cached rows (the new token is in registers)
        done = int((pos_np % block == block - 1).sum())
        # per (b, kv head): the walked K and V rows; k_new, k_pre, v_new read (bf16), the ring rows written,
        # the frontier sums read and written (fp32), and the pooled K and V rows of a completed block
        per_layer = int(Hkv * (2 * row * walked + B * (3 * 2 * D + 2 * row + 2 * 2 * D * 4) + done * 2 * row)
                        + 2 * B * Hq * D * 2)

        def launch(i):
            for c in caches:
                swa.decode_compressed(c["q"], c["k_new"], c["k_pre"], c["v_new"], c["ring_k"], c["ring_v"],
                                      c["ring_ks"], c["ring_vs"], c["pool_k"], c["pool_v"], c["pool_ks"],
                                      c["pool_vs"], c["front_k"], c["front_v"], pos, block, rope=rope,
                                      out=c["out"])
        p = Part(name, launch, 1, 0.0, per_layer * layers, kernel="decode_kernel<64, 2, true>")
        p.extra = dict(B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, P=P, block=block, layers=layers, bytes_per_layer=per_layer,
                       mean_walked_rows=round(float(walked) / B, 1))
        p.tokens = B
        p.launches = layers
        return p

    def make_chunk(name, B=8, Tc=4096):
        """Chunked prefill into the decode caches: B8, 16q/4kv D64, ring 256 + 256 sinks, a 4096-token chunk
        at positions 256..32767.  FLOPs are counted on visible (query, key) pairs: sinks + the ring rows in
        the window + the chunk's own causal window."""
        Hq, Hkv, D, W, S = 16, 4, 64, 256, 256
        g = torch.Generator(device=dev)
        g.manual_seed(8)
        rng = np.random.default_rng(8)
        pos0_np = rng.integers(256, 32768 - Tc, size=B).astype(np.int64)
        pos0 = torch.from_numpy(pos0_np.astype(np.int32)).to(dev)
        sink_len = torch.full((B,), S, dtype=torch.int32, device=dev)
        c = {}
        for nm, rows in (("ring_k", W), ("ring_v", W), ("sink_k", S), ("sink_v", S)):
            x = torch.randn((B, Hkv, rows, D), generator=g, device=dev).to(torch.bfloat16)
            c[nm], c[nm + "s"] = swa.kv_quantize(x)
        per_copy = (B * Hq * Tc * D * 2) * 2 + (B * Hkv * Tc * D * 2) * 2
        n = max(2, min(8, ROTATE_BYTES // per_copy + 1))
        bufs = []
        for _ in range(n):
            q = torch.randn((B, Hq, Tc, D), generator=g, device=dev).to(torch.bfloat16)
            k = torch.randn((B, Hkv, Tc, D), generator=g, device=dev).to(torch.bfloat16)
            v = torch.randn((B, Hkv, Tc, D), generator=g, device=dev).to(torch.bfloat16)
            bufs.append((q, k, v, torch.empty_like(q)))
        ws = swa.chunk_prefill_workspace(bufs[0][0], c["ring_k"], c["sink_k"])
        i = np.arange(Tc)
        vis = 0
        for p0 in pos0_np:
            t = p0 + i
            ring = np.maximum(0, p0 - np.maximum(S, t - W + 1))
            vis += int((S + ring + np.minimum(i + 1, W)).sum())
        flops = 4.0 * D * Hq * vis
        bytes_ = per_copy + 2 * (B * Hkv * (W + S) * (D + (D // 32) * 4))

        def launch(it):
            q, k, v, o = bufs[it % n]
            swa.chunk_prefill(q, k, v, c["ring_k"], c["ring_v"], c["ring_ks"], c["ring_vs"], c["sink_k"],
                              c["sink_v"], c["sink_ks"], c["sink_vs"], pos0, sink_len, out=o, workspace=ws)
        p = Part(name, launch, n, flops, bytes_, kernel="prefill_bf16_kernel")
        p.extra = dict(B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, S=S, Tc=Tc, visible_pairs_per_head=vis)
        return p

    def make_backward(name):
        """The backward of the needle prefill (bf16 inputs, fp32 gradients): the forward's out and lse are made
        once; a call is the whole backward (preparation, dq pass, dk/dv pass).  FLOPs counted as 2.5x the
        forward's visible-pair FLOPs (five products per visible pair instead of two)."""
        w = workloads.needle()
        q, k, v = bf16(w["q_bits"]), bf16(w["k_bits"]), bf16(w["v_bits"])
        seg = torch.from_numpy(w["seg_ids"]).to(dev)
        pre = torch.from_numpy(w["prefix"]).to(dev)
        rope = swa.rope_table(w["rope_theta"], w["T"], w["D"])
        out, lse = swa.prefill(q, k, v, seg, pre, w["window"], rope=rope, return_lse=True)
        dout = torch.randn(out.shape, device=dev).to(torch.bfloat16)
        _, count = swa.debug_visibility(w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["window"], torch.bfloat16,
                                        seg, pre, want_mask=False)
        nvis = int(count.to(torch.int64).sum().item())
        flops = 2.5 * 4.0 * w["D"] * w["Hq"] * nvis
        ws = [None]

        def launch(i):
            swa.prefill_backward(q, k, v, out, lse, dout, seg, pre, w["window"], rope=rope, workspace=ws[0])
        # the workspace, allocated once outside the timed graphs
        p_ = swa.prefill_params(q, k, w["window"], 0, w["T"], 0.0)
        import ctypes as _ct
        ws[0] = torch.empty(swa.lib().swa_prefill_backward_workspace_size(_ct.byref(p_)), dtype=torch.uint8,
                            device=dev)
        p = Part(name, launch, 1, flops, 0.0, kernel="bwd_dq_kernel + bwd_dkv_kernel")
        p.extra = dict(B=w["B"], Hq=w["Hq"], Hkv=w["Hkv"], T=w["T"], D=w["D"], window=w["window"],
                       visible_pairs_per_head=nvis)
        return p

    def make_nsa(name, block=4, n_select=16):
        """The NSA selection branch on the compressed config (B4, 8/8 heads, D64, T4096, window 256, bf16
        inputs), 16 blocks of 4 per row.  FLOPs: the compressed scores of every candidate block (2 D each) and
        attention over the chosen tokens (4 D per token)."""
        w = workloads.compressed(block=block, dtype="bf16")
        q, k, v = bf16(w["q_bits"]), bf16(w["k_bits"]), bf16(w["v_bits"])
        rope = swa.rope_table(w["rope_theta"], w["T"], w["D"])
        T, W, D = w["T"], w["window"], w["D"]
        nv = np.minimum(np.maximum(0, (np.arange(T) - W + 1) // block), T // block)
        per_row = 2.0 * D * nv + 4.0 * D * block * np.minimum(nv, n_select)
        flops = float(per_row.sum()) * w["B"] * w["Hq"]
        p_ = swa.prefill_params(q, k, W, block, T, 0.0)
        import ctypes as _ct
        ws = torch.empty(swa.lib().swa_nsa_select_workspace_size(_ct.byref(p_)), dtype=torch.uint8, device=dev)

        def launch(i):
            swa.nsa_select(q, k, v, W, block, n_select, rope=rope, workspace=ws)
        p = Part(name, launch, 1, flops, 0.0, kernel="nsa_select_kernel")
        p.extra = dict(B=w["B"], Hq=w["Hq"], Hkv=w["Hkv"], T=T, D=D, window=W, block=block, n_select=n_select)
        return p

    t_setup = time.time()
    if "needle" in parts_wanted:
        parts["needle"] = make_prefill("needle", workloads.needle())
    if "compressed4" in parts_wanted:
        parts["compressed4"] = make_compressed("compressed4", 4)
    if "decode" in parts_wanted:
        parts["decode"] = make_decode("decode", num_splits=args.decode_splits)
    for b in (1, 8, 32):
        if f"decode_b{b}" in parts_wanted:
            parts[f"decode_b{b}"] = make_decode(f"decode_b{b}", B=b)
    if "nsa" in parts_wanted:
        parts["nsa"] = make_nsa("nsa")
    if "backward" in parts_wanted:
        parts["backward"] = make_backward("backward")
    if "chunk" in parts_wanted:
        parts["chunk"] = make_chunk("chunk")
    if "decode_c4" in parts_wanted:
        parts["decode_c4"] = make_compressed_decode("decode_c4", 4)
    if "packed" in parts_wanted:
        parts["packed"] = make_prefill("packed", workloads.packed())
    if "compressed16" in parts_wanted:
        parts["compressed16"] = make_compressed("compressed16", 16)
    if "causal" in parts_wanted:  # (not in the default set) plain causal B4 16q/4kv T4096, no window
        parts["causal"] = make_prefill("causal", workloads.causal())
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s")

    stream = torch.cuda.Stream(device=dev)

    class Eager:
        """Stands in for a captured graph: replay() launches the same work directly."""

        def __init__(self, fn, iters, offset=0):
            self.fn, self.iters, self.offset = fn, iters, offset

        def replay(self):
            for i in range(self.iters):
                self.fn(self.offset + i)

    def capture(fn, iters, offset=0, prewarm=True):
        if args.eager:
            if prewarm:
                with torch.cuda.stream(stream):
                    fn(offset)
                torch.cuda.synchronize()
            return Eager(fn, iters, offset)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            if prewarm:
                fn(offset)  # warm the code path on the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for i in range(iters):
                    fn(offset + i)
        torch.cuda.synchronize()
        return g

    def time_graph(g, replays):
        # HIP events recorded on the stream the kernels run on
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(replays):
                g.replay()
            e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1)

    def warm(g, n):
        with torch.cuda.stream(stream):
            for _ in range(n):
                g.replay()
        torch.cuda.synchronize()

    # ---- per-part timing (one graph of `reps` iterations each) -----------------
    results = {}
    for name, p in parts.items():
        reps = getattr(p, "reps", max(p.ncopies, args.reps))
        g = capture(p.launch, reps)
        warm(g, args.warmup)
        ms = time_graph(g, max(1, args.steps // 4)) / (max(1, args.steps // 4) * reps)
        r = dict(ms=ms)
        if p.flops:
            r["tflops"] = p.flops / (ms * 1e-3) / 1e12
            r["frac_mfma_peak"] = r["tflops"] / MFMA_BF16_PEAK_TFLOPS
        if p.bytes:
            r["gbs"] = p.bytes / (ms * 1e-3) / 1e9
            r["frac_hbm_peak"] = r["gbs"] / HBM_PEAK_GBS
        if hasattr(p, "tokens"):
            r["tokens_per_s"] = p.tokens / (ms * 1e-3)
            r["ms_per_launch"] = ms / p.launches
        r.update(p.extra)
        results[name] = r
        log(f"{name}: {json.dumps(r)}")
        del g

    # ---- the step: needle + compressed4 + decode, K timed steps ----------------
    # W warmup steps launched directly, then one graph of exactly K steps (input copies cycle with the
    # step index) replayed once inside the timed region.
    step_names = [n for n in ("needle", "compressed4", "decode") if n in parts]

    def step(i):
        for n in step_names:
            parts[n].launch(i)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()
    step_graph = capture(step, args.steps, offset=args.warmup, prewarm=False)
    steps_timed = args.steps
    ms_total = time_graph(step_graph, 1)
    ms_per_step = ms_total / steps_timed

    head = results.get("needle", {})
    dec = results.get("decode", {})
    out = {
        "metric": "prefill TFLOP/s (unmasked) + decode GB/s, % of MI355X roofline",
        "value": round(head.get("tflops", 0.0), 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "needle-shaped windowed+sink GQA prefill, B8 8q/2kv D64 T2048 window 256, "
                               "sink prefix 64..384, RoPE (value); the step also runs compressed b=4 (B4 8/8 "
                               "T4096) and a 12-layer int8 decode step (B256 16q/4kv ring 256 + 256 sinks); the "
                               "largest prefill, packed multi-segment B16 16q/4kv T4096 (3-6 segments per row, "
                               "128-token prefix), is timed on its own under packed",
                   "global_batch": 8, "seq_len": 2048, "parallelism": "none (1 GPU)"},
        "decode": {"value": round(dec.get("gbs", 0.0), 1), "unit": "GB/s",
                   "frac_hbm_peak": round(dec.get("frac_hbm_peak", 0.0), 4),
                   "tokens_per_s": round(dec.get("tokens_per_s", 0.0), 1),
                   "us_per_layer": round(dec.get("ms_per_launch", 0.0) * 1e3, 2)},
        "decode_by_batch": {str(r["B"]): {"us_per_layer": round(r["ms_per_launch"] * 1e3, 2),
                                          "gbs": round(r["gbs"], 1), "frac_hbm_peak": round(r["frac_hbm_peak"], 4),
                                          "tokens_per_s": round(r["tokens_per_s"], 1)}
                            for n, r in sorted(results.items(), key=lambda kv: kv[1].get("B", 0))
                            if n.startswith("decode") and n != "decode_c4"},
        "compressed_decode": {k: (round(v, 5) if isinstance(v, float) else v)
                              for k, v in results.get("decode_c4", {}).items()},
        "backward": {"value": round(results.get("backward", {}).get("tflops", 0.0), 3), "unit": "TFLOP/s",
                     "frac_mfma_peak": round(results.get("backward", {}).get("tflops", 0.0) / MFMA_BF16_PEAK_TFLOPS, 5),
                     "us_per_call": round(results.get("backward", {}).get("ms", 0.0) * 1e3, 2),
                     "config": "needle prefill backward, bf16 inputs on bf16 matrix instructions (fp32 accumulation)"},
        "nsa_selection": {"value": round(results.get("nsa", {}).get("tflops", 0.0), 3), "unit": "TFLOP/s",
                          "frac_fp32_peak": round(results.get("nsa", {}).get("tflops", 0.0) / FP32_PEAK_TFLOPS, 5),
                          "us_per_call": round(results.get("nsa", {}).get("ms", 0.0) * 1e3, 2),
                          "config": "compressed config, b=4, 16 selected blocks; scores on fp32 matrix instructions, the rest fp32 vector"},
        "chunked_prefill": {"value": round(results.get("chunk", {}).get("tflops", 0.0), 3), "unit": "TFLOP/s",
                            "frac_mfma_peak": round(results.get("chunk", {}).get("frac_mfma_peak", 0.0), 5),
                            "us_per_call": round(results.get("chunk", {}).get("ms", 0.0) * 1e3, 2)},
        "packed": {"value": round(results.get("packed", {}).get("tflops", 0.0), 3), "unit": "TFLOP/s",
                   "frac_mfma_peak": round(results.get("packed", {}).get("frac_mfma_peak", 0.0), 5),
                   "us_per_call": round(results.get("packed", {}).get("ms", 0.0) * 1e3, 2),
                   "traffic": measured_traffic("prefill_packed_call", PREFILL_SOURCES)},
        "compressed4": {"value": round(results.get("compressed4", {}).get("tflops", 0.0), 3), "unit": "TFLOP/s",
                        "frac_mfma_peak": round(results.get("compressed4", {}).get("frac_mfma_peak", 0.0), 5),
                        "us_per_call": round(results.get("compressed4", {}).get("ms", 0.0) * 1e3, 2),
                        "traffic": measured_traffic("prefill_compressed4_call", PREFILL_SOURCES)},
        "parts": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                  for k, v in results.items()},
        # The dominant kernel of the step by GPU time is the decode kernel (12 launches per step); one
        # swa_attn_decode call is exactly one launch of it.  achieved = algorithmic bytes per launch / the
        # HIP-event average launch duration.
        "roofline": roofline_decode(dec),
        # The prefill call on the needle workload: key-info pre-pass + key rotation pre-pass + attention
        # kernel; the time is that of the whole call.
        "roofline_prefill": {"bound": "mfma", "achieved": round(head.get("tflops", 0.0), 3),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(head.get("frac_mfma_peak", 0.0), 5),
                             "hbm_ceiling_tflops": round(hbm_ceiling(head), 1),
                             "traffic": measured_traffic("prefill_needle_call", PREFILL_SOURCES),
                             "kernel": "prefill_prep_kernel + prefill_bf16_kernel "
                                       "(one swa_attn_prefill call, needle workload)"},
    }

    # ---- CPU baseline: the oracle on a bounded sample of the needle workload ----
    if not args.no_cpu_baseline and "needle" in parts:
        out["cpu_baseline"] = cpu_baseline(parts["needle"], args.cpu_seconds)
    print(json.dumps(out), flush=True)


def hbm_ceiling(r):
    """MFMA-equivalent ceiling the HBM roof puts on a prefill: 8 TB/s x (visible-pair FLOPs / compulsory
    bytes)."""
    if not r.get("gbs"):
        return 0.0
    ai = r["tflops"] * 1e12 / (r["gbs"] * 1e9)
    return HBM_PEAK_GBS * 1e9 * ai / 1e12


def roofline_decode(dec):
    if not dec:
        return None
    per_launch = dec["bytes_per_layer"]
    traffic = measured_traffic("decode_kernel", DECODE_SOURCES)
    return {"bound": "hbm", "achieved": round(dec["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dec["gbs"] / HBM_PEAK_GBS, 5), "traffic": traffic,
            "kernel": "decode_kernel", "bytes_per_launch": per_launch,
            "ms_per_launch": round(dec["ms_per_launch"], 5)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(part, seconds):
    """Time the CPU oracle on the needle workload (visible-pair TFLOP/s).  The oracle evaluates whole
    passes over every (b, head, row) of the workload, repeated until about `seconds` have elapsed."""
    import oracle
    w = part.w
    B, Hq, T, D = w["B"], w["Hq"], w["T"], w["D"]
    rows = np.arange(B * Hq * T, dtype=np.int64)
    passes, elapsed = 0, 0.0
    t0 = time.perf_counter()
    while passes == 0 or elapsed < seconds:
        oracle.prefill(w["q"], w["k"], w["v"], w["seg_ids"], w["prefix"], w["window"], theta=w["rope_theta"],
                       rows=rows)
        passes += 1
        elapsed = time.perf_counter() - t0
    nvis = float(part.count.astype(np.float64).sum())
    flops = 4.0 * D * Hq * nvis * passes
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{passes} full passes of the oracle over the needle workload ({B * Hq * T} query rows, "
                      f"RoPE of all keys included); {elapsed:.1f} s", "seconds": round(elapsed, 2)}


if __name__ == "__main__":
    main()
