"""Windowed+sink GQA attention and compressed-KV attention for MI355X (gfx950).

The compute lives in ``libswa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/swa.h``).  ``compressed_kv_attention_amd.swa`` is a thin
ctypes binding over it that takes torch tensors for device memory and streams.
``workloads`` draws the seeded synthetic inputs.
"""
__all__ = ["swa", "workloads"]
