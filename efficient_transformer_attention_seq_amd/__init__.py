"""Linformer low-rank self-attention for AMD Instinct MI355X (gfx950).

The computation lives in liblinformer.so (hand-written HIP kernels behind a C ABI declared in
include/linformer.h); ``linformer`` is its ctypes binding with the same function names, and
``synth`` draws the seeded synthetic workloads.
"""
from . import synth  # noqa: F401
