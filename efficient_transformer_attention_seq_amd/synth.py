"""Seeded synthetic inputs for Linformer attention (shared by the oracle side and the GPU side).

This module only draws and stores inputs: random normal tensors, the bf16 rounding of those
inputs, padding lengths and zeroed padding rows.  It holds none of the attention arithmetic, so
the oracle and the HIP path can both consume its arrays without sharing any of the method.

Workloads follow the shapes the Linformer pages use: head dim d = 64, projected length k of 128
or 256, sequence lengths from 512 to 65536 (Linformer summary card, section 证据 "evidence";
Linformer 요약 설명, section "Inference-time Efficiency Results"), and the RoBERTa-base layer
shape (12 heads, d_model 768).  The pages time randomly generated inputs, so seeded normal draws
are the workload itself, not a stand-in for a dataset.

Draw order (one ``numpy.random.default_rng(seed)`` stream per workload):
  Q, K, V (each ``standard_normal([B, H, n, d])``), then E, then F when it is a separate matrix,
  then the padding lengths.  E and F entries are ``standard_normal / sqrt(k)`` (variance 1/k).
Values are drawn in float64, rounded to float32 (round to nearest even) and, for bf16 workloads,
rounded again to bf16 with round-to-nearest-even.  The rounded values are kept as float32 arrays
whose every element is exactly representable in the workload dtype.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SHARE_NONE = 0
SHARE_HEADWISE = 1
SHARE_KV = 2
SHARE_LAYERWISE = 3
SHARE_NAMES = {SHARE_NONE: "none", SHARE_HEADWISE: "headwise", SHARE_KV: "kv",
               SHARE_LAYERWISE: "layerwise"}

DT_F32 = 0
DT_BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, dtype, projection sharing and padding recipe."""
    name: str
    batch: int
    heads: int
    n: int
    d: int
    k: int
    dtype: int
    share: int
    padded: bool = False      # draw lengths in [n/2, n] and zero rows >= length
    seed: int = 0

    @property
    def e_heads(self) -> int:
        """Number of distinct E matrices stored: one per head unless shared across heads."""
        return self.heads if self.share == SHARE_NONE else 1

    @property
    def separate_f(self) -> bool:
        """Whether F is its own matrix (unshared or headwise) or aliases E (key-value, layerwise)."""
        return self.share in (SHARE_NONE, SHARE_HEADWISE)

    @property
    def tokens(self) -> int:
        return self.batch * self.n

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: single-head fp32; RoBERTa-base shape with one key-value matrix; long
# sequences with unshared per-head projections and padding; extreme length with layerwise
# sharing; and the attention part of a 12-layer RoBERTa-base-shaped stack.
C1 = Workload("single_head_n512_k128_f32", 1, 1, 512, 64, 128, DT_F32, SHARE_NONE)
C2 = Workload("roberta_base_b32_n512_k256_kv", 32, 12, 512, 64, 256, DT_BF16, SHARE_KV)
C3 = Workload("long_b8_h12_n4096_k256_unshared_padded", 8, 12, 4096, 64, 256, DT_BF16,
              SHARE_NONE, padded=True)
C4 = Workload("extreme_b1_h12_n65536_k128_layerwise", 1, 12, 65536, 64, 128, DT_BF16,
              SHARE_LAYERWISE)
C5A = Workload("stack_layer_b16_h12_n1024_k256_layerwise", 16, 12, 1024, 64, 256, DT_BF16,
               SHARE_LAYERWISE)
WORKLOADS = {w.name: w for w in (C1, C2, C3, C4, C5A)}


def round_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> float32, round to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32.

    Inputs are finite (normal draws), so no NaN handling is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    out = ((bits + bias) >> np.uint64(16)) << np.uint64(16)
    return out.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are exactly bf16 (the bf16 storage encoding)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def to_dtype(x: np.ndarray, dtype: int) -> np.ndarray:
    x32 = round_f32(x)
    return round_bf16(x32) if dtype == DT_BF16 else x32


@dataclasses.dataclass
class Inputs:
    """Host copies of one workload's inputs; all float arrays are float32 holding dtype values."""
    wl: Workload
    Q: np.ndarray                   # [B, H, n, d]
    K: np.ndarray                   # [B, H, n, d]
    V: np.ndarray                   # [B, H, n, d]
    E: np.ndarray                   # [H_E, k, n]
    F: Optional[np.ndarray]         # [H_E, k, n] or None when F aliases E
    lengths: Optional[np.ndarray]   # int32 [B] or None


def make_inputs(wl: Workload, seed: Optional[int] = None, batch_limit: Optional[int] = None,
                ) -> Inputs:
    """Draw the workload's inputs in the fixed order Q, K, V, E, [F], [lengths].

    ``batch_limit`` draws every tensor at full size (so the values match the full workload) and
    then keeps only the first ``batch_limit`` batch items.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    shp = (wl.batch, wl.heads, wl.n, wl.d)
    Q = to_dtype(rng.standard_normal(shp), wl.dtype)
    K = to_dtype(rng.standard_normal(shp), wl.dtype)
    V = to_dtype(rng.standard_normal(shp), wl.dtype)
    eshape = (wl.e_heads, wl.k, wl.n)
    E = to_dtype(rng.standard_normal(eshape) / np.sqrt(wl.k), wl.dtype)
    F = to_dtype(rng.standard_normal(eshape) / np.sqrt(wl.k), wl.dtype) if wl.separate_f else None
    lengths = None
    if wl.padded:
        lengths = rng.integers(wl.n // 2, wl.n, endpoint=True, size=wl.batch).astype(np.int32)
        for b, L in enumerate(lengths):
            Q[b, :, L:, :] = 0.0
            K[b, :, L:, :] = 0.0
            V[b, :, L:, :] = 0.0
    if batch_limit is not None and batch_limit < wl.batch:
        Q, K, V = Q[:batch_limit].copy(), K[:batch_limit].copy(), V[:batch_limit].copy()
        if lengths is not None:
            lengths = lengths[:batch_limit].copy()
        wl = wl.with_(batch=batch_limit)
    return Inputs(wl, Q, K, V, E, F, lengths)


def random_inputs(batch: int, heads: int, n: int, d: int, k: int, dtype: int, share: int,
                  seed: int, lengths: Optional[list] = None, e_scale: Optional[float] = None,
                  ) -> Inputs:
    """Small seeded inputs of any shape (parity and edge-case tests), same recipe as above.

    ``lengths`` (if given) are used as-is; rows past them are filled with fresh normal draws
    instead of zeros, so that a kernel which reads padding would be caught.
    """
    wl = Workload(f"rand_b{batch}h{heads}n{n}d{d}k{k}", batch, heads, n, d, k, dtype, share,
                  seed=seed)
    rng = np.random.default_rng(seed)
    shp = (batch, heads, n, d)
    Q = to_dtype(rng.standard_normal(shp), dtype)
    K = to_dtype(rng.standard_normal(shp), dtype)
    V = to_dtype(rng.standard_normal(shp), dtype)
    es = (1.0 / np.sqrt(k)) if e_scale is None else e_scale
    eshape = (wl.e_heads, k, n)
    E = to_dtype(rng.standard_normal(eshape) * es, dtype)
    F = to_dtype(rng.standard_normal(eshape) * es, dtype) if wl.separate_f else None
    lens = None if lengths is None else np.asarray(lengths, dtype=np.int32)
    return Inputs(wl, Q, K, V, E, F, lens)


@dataclasses.dataclass
class Projected:
    """Seeded stand-ins for projected keys/values, to drive the attention half on its own.

    Kbar holds the values the stand-in stands for (float32); putting them into the attention
    kernel's storage format is the caller's business.  Vbar is rounded to the workload dtype.
    """
    Q: np.ndarray       # [B, H, n, d]
    Kbar: np.ndarray    # [B, H, k, d]
    Vbar: np.ndarray    # [B, H, k, d]


def random_projected(batch: int, heads: int, n: int, d: int, k: int, dtype: int, seed: int,
                     kbar_std: float = 4.0, vbar_std: float = 4.0) -> Projected:
    """Q ~ N(0,1); Kbar ~ N(0, kbar_std^2); Vbar ~ N(0, vbar_std^2).

    The default standard deviation 4 matches sqrt(n/k) at n = 4096, k = 256 (the spread of
    E . K with E ~ N(0, 1/k) and K ~ N(0, 1)).
    """
    rng = np.random.default_rng(seed)
    Q = to_dtype(rng.standard_normal((batch, heads, n, d)), dtype)
    kb = rng.standard_normal((batch, heads, k, d)) * kbar_std
    vb = rng.standard_normal((batch, heads, k, d)) * vbar_std
    return Projected(Q, round_f32(kb), to_dtype(vb, dtype))


# ---------------------------------------------------------------------------------------------
# Encoder attention stack inputs: the 12-layer RoBERTa-base-shaped stack (d_model 768, 12 heads,
# n = 1024, k = 256, batch 16, bf16) whose per-layer attention part is the stack-layer workload
# above.  Draw order: X, then for each layer l = 0 .. L-1 its Wqkv[l] and then its Wo[l], then E.
# X ~ N(0, 1); weights ~ 0.02 N(0, 1); E ~ N(0, 1/k), one matrix for every layer.
# ---------------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class StackWorkload:
    name: str
    batch: int
    n: int
    d_model: int
    heads: int
    k: int
    layers: int
    w_std: float = 0.02
    padded: bool = False
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.batch * self.n

    def with_(self, **kw) -> "StackWorkload":
        return dataclasses.replace(self, **kw)


C5 = StackWorkload("encoder_stack_l12_b16_n1024_d768_k256_layerwise", 16, 1024, 768, 12, 256, 12)
STACK_WORKLOADS = {C5.name: C5}


@dataclasses.dataclass
class StackInputs:
    """Host copies (float32 arrays holding bf16 values)."""
    wl: StackWorkload
    X: np.ndarray                   # [B, n, d_model]
    Wqkv: np.ndarray                # [L, 3 d_model, d_model]
    Wo: np.ndarray                  # [L, d_model, d_model]
    E: np.ndarray                   # [1, k, n]
    lengths: Optional[np.ndarray]   # int32 [B] or None


def make_stack_inputs(wl: StackWorkload, seed: Optional[int] = None,
                      lengths: Optional[list] = None) -> StackInputs:
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    dm, L = wl.d_model, wl.layers
    X = to_dtype(rng.standard_normal((wl.batch, wl.n, dm)), DT_BF16)
    Wqkv = np.empty((L, 3 * dm, dm), dtype=np.float32)
    Wo = np.empty((L, dm, dm), dtype=np.float32)
    for l in range(L):
        Wqkv[l] = to_dtype(rng.standard_normal((3 * dm, dm)) * wl.w_std, DT_BF16)
        Wo[l] = to_dtype(rng.standard_normal((dm, dm)) * wl.w_std, DT_BF16)
    E = to_dtype(rng.standard_normal((1, wl.k, wl.n)) / np.sqrt(wl.k), DT_BF16)
    lens = None if lengths is None else np.asarray(lengths, dtype=np.int32)
    return StackInputs(wl, X, Wqkv, Wo, E, lens)


def conv_weights(e_heads: int, s: int, seed: int, dtype: int = DT_BF16) -> np.ndarray:
    """Window weights [e_heads, s] of the convolution compression, N(0, 1/s) (so a window of
    N(0, 1) keys projects to unit variance, as a dense E ~ N(0, 1/k) over n = k s positions
    does), from their own seeded stream."""
    rng = np.random.default_rng(seed)
    return to_dtype(rng.standard_normal((e_heads, s)) / np.sqrt(s), dtype)
