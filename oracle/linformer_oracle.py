"""Plain float64 CPU oracle for Linformer low-rank self-attention (one non-causal encoder layer).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this module: only the
tests, the package's smoke check and the benchmark's CPU-baseline leg use it.  It shares no code
with the HIP path; its only inputs are plain numpy arrays.

What it computes (per batch item b and head h), written out as the definition, in float64, on the
exact input values:

  * sequence projection (Linformer 요약 설명, section "Model"; Linformer summary card, section
    方法适配 "method"; efficient-Transformer survey, section on the low-rank improvement):
    the keys and values are mixed along the sequence axis by E, F of shape k x n,
        Kbar = E . K,   Vbar = F . V,   giving k x d matrices.
    Each row of E holds the weights that combine the n positions into one projected key.
  * compressed scaled dot-product attention (Linformer 요약 설명, sections "Model" and
    "Transformer and Self-Attention"; survey, section 2.1): an n x k score matrix, softmax over
    the k projected slots for each query, then the weighted sum of Vbar; the queries are not
    compressed, so the output is n x d.  Scale = 1/sqrt(d) unless given.
  * projection sharing (Linformer summary card, section 方法适配; Linformer 요약 설명, section
    "Additional Efficiency Techniques"): unshared per-head E_h, F_h; headwise (one E and one F
    for all heads); key-value (one matrix, E = F, for all heads); layerwise (one matrix for
    every head, both K and V, and every layer -- within one layer it computes what key-value
    sharing computes).
  * padding to a fixed maximum length (Linformer 요약 설명, section "Model": E, F are sized for the
    maximum length, so shorter inputs are padded).  Reading: positions t >= L_b contribute
    nothing to Kbar, Vbar (exactly what zero padding gives), the softmax still runs over all k
    slots, and output rows i >= L_b are zero.

Library primitives used as single steps: ``numpy.matmul`` (dense products) and ``numpy.exp``.
No blocking, fusion or reordering beyond the definition.

Every function here is pinned by the "not gpu" tests (hand-derived fixtures under
tests/golden/, a separately written brute-force textbook attention, closed forms and
invariants); none is "parity unpinned".
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

SHARE_NONE = 0
SHARE_HEADWISE = 1
SHARE_KV = 2
SHARE_LAYERWISE = 3


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def head_projections(E: np.ndarray, F: Optional[np.ndarray], share: int, heads: int
                     ) -> Tuple[list, list]:
    """The (E_h, F_h) pair each head uses, per the sharing mode.

    Linformer summary card, section 方法适配: headwise, key-value and layerwise sharing; the
    layerwise mode uses a single projection matrix for the whole model.  E and F are stored as
    [H_E, k, n] with H_E = heads for unshared projections and 1 otherwise.  For key-value and
    layerwise sharing F must be None or equal to E.  Unshared mode also accepts F = None, which
    means E_h = F_h per head.
    """
    E = _f64(E)
    if share == SHARE_NONE:
        if E.shape[0] != heads:
            raise ValueError("unshared projections need one E per head")
        Fm = E if F is None else _f64(F)
        if Fm.shape != E.shape:
            raise ValueError("E and F shapes differ")
        return [E[h] for h in range(heads)], [Fm[h] for h in range(heads)]
    if E.shape[0] != 1:
        raise ValueError("shared projections store a single E")
    if share == SHARE_HEADWISE:
        if F is None:
            raise ValueError("headwise sharing keeps a separate F")
        Fm = _f64(F)
        return [E[0]] * heads, [Fm[0]] * heads
    if share in (SHARE_KV, SHARE_LAYERWISE):
        if F is not None and not np.array_equal(_f64(F), E):
            raise ValueError("key-value / layerwise sharing uses E = F")
        return [E[0]] * heads, [E[0]] * heads
    raise ValueError(f"unknown sharing mode {share}")


def project(P: np.ndarray, X: np.ndarray, length: Optional[int] = None) -> np.ndarray:
    """Sequence projection Pbar = P . X over the valid positions.

    Linformer 요약 설명, section "Model": P (E or F) is k x n, X (K or V) is n x d, the product is
    k x d.  Positions t >= length contribute nothing (the padding reading), which is the same as
    multiplying by X with those rows set to zero.
    """
    P = _f64(P)
    X = _f64(X)
    n = X.shape[0]
    L = n if length is None else max(0, min(int(length), n))
    return np.matmul(P[:, :L], X[:L, :])


def scores(Q: np.ndarray, Kbar: np.ndarray, scale: float) -> np.ndarray:
    """n x k context scores scale * Q . Kbar^T (scaled dot product against the projected keys)."""
    return float(scale) * np.matmul(_f64(Q), _f64(Kbar).T)


def softmax_rows(S: np.ndarray) -> np.ndarray:
    """Softmax of each row (one query) over its k entries: exp(s - max) / sum exp(s - max).

    Linformer 요약 설명, section "Transformer and Self-Attention": the softmax runs per query along
    the key axis.  Subtracting the row maximum changes nothing mathematically and keeps exp finite.
    """
    S = _f64(S)
    m = S.max(axis=1, keepdims=True)
    w = np.exp(S - m)
    return w / w.sum(axis=1, keepdims=True)


def attention_weights(Q: np.ndarray, Kbar: np.ndarray, scale: float) -> np.ndarray:
    """P-bar = softmax(scale * Q . Kbar^T), the n x k context matrix of one head."""
    return softmax_rows(scores(Q, Kbar, scale))


def attend(Q: np.ndarray, Kbar: np.ndarray, Vbar: np.ndarray, scale: Optional[float] = None,
           length: Optional[int] = None) -> np.ndarray:
    """O = softmax(scale * Q . Kbar^T) . Vbar for one head, rows >= length set to zero.

    Linformer 요약 설명, section "Model": queries are not compressed, so there is one output row
    per input position (n x d).  ``length`` None computes every row.
    """
    Q = _f64(Q)
    d = Q.shape[1]
    s = (1.0 / np.sqrt(d)) if (scale is None or scale == 0.0) else float(scale)
    O = np.matmul(attention_weights(Q, Kbar, s), _f64(Vbar))
    if length is not None:
        L = max(0, min(int(length), Q.shape[0]))
        O[L:, :] = 0.0
    return O


def forward(Q, K, V, E, F, share: int, lengths: Optional[Sequence[int]] = None,
            scale: Optional[float] = None, pairs: Optional[Sequence[Tuple[int, int]]] = None,
            return_intermediates: bool = False):
    """Linformer attention for a [B, H, n, d] batch: project K and V, then attend.

    ``pairs`` restricts the work to the listed (b, h) slices (the others stay zero), for bounded
    checks of large workloads.  With ``return_intermediates`` it also returns Kbar, Vbar
    ([B, H, k, d]) so each half of the path can be checked on its own.
    """
    Q = _f64(Q)
    B, H, n, d = Q.shape
    Es, Fs = head_projections(E, F, share, H)
    k = Es[0].shape[0]
    O = np.zeros((B, H, n, d))
    Kb = np.zeros((B, H, k, d))
    Vb = np.zeros((B, H, k, d))
    todo = [(b, h) for b in range(B) for h in range(H)] if pairs is None else list(pairs)
    for b, h in todo:
        L = None if lengths is None else int(lengths[b])
        Kb[b, h] = project(Es[h], K[b, h], L)
        Vb[b, h] = project(Fs[h], V[b, h], L)
        O[b, h] = attend(Q[b, h], Kb[b, h], Vb[b, h], scale, L)
    if return_intermediates:
        return O, Kb, Vb
    return O


def dense_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: Optional[float] = None,
                    length: Optional[int] = None) -> np.ndarray:
    """Standard softmax attention of one head: softmax(scale * Q . K^T) . V with an n x n matrix.

    Linformer 요약 설명, section "Transformer and Self-Attention"; survey, section 2.1 (scaled dot
    product).  With a ``length``, keys at positions >= length are left out of each softmax (the
    same padding reading as for the projection: padded positions contribute nothing) and output
    rows >= length are zero.  This is the comparison baseline's definition.
    """
    Q = _f64(Q)
    n, d = Q.shape
    s = (1.0 / np.sqrt(d)) if (scale is None or scale == 0.0) else float(scale)
    L = n if length is None else max(0, min(int(length), n))
    O = np.zeros((n, _f64(V).shape[1]))
    if L == 0:
        return O
    Sm = s * np.matmul(Q[:L], _f64(K)[:L].T)
    O[:L] = np.matmul(softmax_rows(Sm), _f64(V)[:L])
    return O


def dense_forward(Q, K, V, lengths: Optional[Sequence[int]] = None,
                  scale: Optional[float] = None,
                  pairs: Optional[Sequence[Tuple[int, int]]] = None) -> np.ndarray:
    """Dense attention over a [B, H, n, d] batch (optionally only some (b, h) slices)."""
    Q = _f64(Q)
    B, H, n, d = Q.shape
    O = np.zeros((B, H, n, d))
    todo = [(b, h) for b in range(B) for h in range(H)] if pairs is None else list(pairs)
    for b, h in todo:
        L = None if lengths is None else int(lengths[b])
        O[b, h] = dense_attention(Q[b, h], K[b, h], V[b, h], scale, L)
    return O


def slice_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """Largest per-(b, h) slice value of max|out - ref| / max|ref| (0/0 counts as 0).

    The accuracy metric the tolerances are stated in: elementwise relative error is unbounded
    where an output crosses zero, so each slice is normalised by its own largest magnitude.
    """
    out = _f64(out)
    ref = _f64(ref)
    lead = ref.shape[:-2]
    worst = 0.0
    for idx in np.ndindex(*lead) if lead else [()]:
        r = ref[idx]
        o = out[idx]
        den = np.abs(r).max() if r.size else 0.0
        num = np.abs(o - r).max() if r.size else 0.0
        if den == 0.0:
            e = 0.0 if num == 0.0 else np.inf
        else:
            e = num / den
        worst = max(worst, float(e))
    return worst


# ---------------------------------------------------------------------------------------------
# Encoder attention stack: per layer, the input projection to per-head queries, keys and values,
# Linformer attention of every head with one layerwise-shared projection, the concatenation of the
# heads and the output projection; the layer's output is the next layer's input.
#
# Linformer 요약 설명, section "Transformer and Self-Attention": with model width d_m, h heads of
# width d, each head's query, key and value are X W^Q, X W^K, X W^V with W of size d_m x d, and
# the heads' outputs are concatenated and mapped by an output projection as in ordinary
# multi-head attention.  Linformer summary card, section 方法适配: layerwise sharing uses a single
# projection matrix for the whole model (every layer, head, key and value).
#
# Weight layout (a reading; the pages fix only the shapes): Wqkv[l] is [3 d_m, d_m] and Wo[l] is
# [d_m, d_m], applied as y = x . W^T (row f of a weight holds output feature f); rows 0..d_m-1 of
# Wqkv[l] give the queries, d_m..2 d_m-1 the keys, 2 d_m..3 d_m-1 the values, and feature f of
# each belongs to head f // d, column f % d.  Concatenation puts head h's column c at feature
# h d + c.  The stack has no other step (no bias, residual or normalisation): the configuration
# names only these.
# ---------------------------------------------------------------------------------------------
def split_heads(Y: np.ndarray, heads: int) -> np.ndarray:
    """[B, n, heads * d] -> [B, heads, n, d]: feature f goes to head f // d, column f % d."""
    Y = _f64(Y)
    B, n, w = Y.shape
    return Y.reshape(B, n, heads, w // heads).transpose(0, 2, 1, 3)


def concat_heads(O: np.ndarray) -> np.ndarray:
    """[B, heads, n, d] -> [B, n, heads * d]: head h's column c becomes feature h d + c."""
    O = _f64(O)
    B, H, n, d = O.shape
    return O.transpose(0, 2, 1, 3).reshape(B, n, H * d)


def stack_layer(X: np.ndarray, Wqkv: np.ndarray, Wo: np.ndarray, E: np.ndarray, heads: int,
                lengths: Optional[Sequence[int]] = None, scale: Optional[float] = None
                ) -> np.ndarray:
    """One layer: X [B, n, d_m] -> concat_h(Linformer attention of head h) . Wo^T."""
    X = _f64(X)
    dm = X.shape[2]
    Y = np.matmul(X, _f64(Wqkv).T)                     # [B, n, 3 d_m]
    Q = split_heads(Y[:, :, 0:dm], heads)
    K = split_heads(Y[:, :, dm:2 * dm], heads)
    V = split_heads(Y[:, :, 2 * dm:3 * dm], heads)
    O = forward(Q, K, V, E, None, SHARE_LAYERWISE, lengths, scale)
    return np.matmul(concat_heads(O), _f64(Wo).T)


def stack_forward(X: np.ndarray, Wqkv: np.ndarray, Wo: np.ndarray, E: np.ndarray, heads: int,
                  lengths: Optional[Sequence[int]] = None, scale: Optional[float] = None,
                  return_layers: bool = False):
    """The whole stack: Wqkv [L, 3 d_m, d_m], Wo [L, d_m, d_m], one E [1, k, n] for every layer.

    Returns the last layer's output [B, n, d_m], or the list of every layer's output.
    """
    outs = []
    Y = _f64(X)
    for l in range(np.shape(Wqkv)[0]):
        Y = stack_layer(Y, Wqkv[l], Wo[l], E, heads, lengths, scale)
        outs.append(Y)
    return outs if return_layers else Y


# ---------------------------------------------------------------------------------------------
# Convolution / pooling compression (Linformer 요약 설명, section "Additional Efficiency
# Techniques": besides shared linear projections, the sequence can be compressed by pooling or a
# convolution).  Reading: a 1-D convolution along the sequence with window s = n / k and stride
# s, so projected row r combines positions r s .. r s + s - 1 with weights w[0 .. s-1]; mean
# pooling is w = 1/s.  As a projection this is the banded E with E[r][r s + j] = w[j] and zeros
# elsewhere, so the method's definition applies unchanged: the oracle builds that E and calls
# the same projection and attention.
# ---------------------------------------------------------------------------------------------
def conv_projection_matrix(w: np.ndarray, n: int) -> np.ndarray:
    """The k x n banded E of a stride-s, window-s convolution with weights w (s = len(w))."""
    w = _f64(w)
    s = w.shape[0]
    if n % s:
        raise ValueError("the window must divide n")
    k = n // s
    E = np.zeros((k, n))
    for r in range(k):
        E[r, r * s:(r + 1) * s] = w
    return E


def conv_forward(Q, K, V, wE, wF, share: int, lengths=None, scale=None, pairs=None,
                 return_intermediates: bool = False):
    """Linformer attention with convolution compression: wE, wF are [H_E, s] window weights
    (H_E per the sharing mode, as for E and F); F = None as in ``forward``."""
    n = np.shape(Q)[2]
    E = np.stack([conv_projection_matrix(w, n) for w in _f64(wE)])
    F = None if wF is None else np.stack([conv_projection_matrix(w, n) for w in _f64(wF)])
    return forward(Q, K, V, E, F, share, lengths, scale, pairs=pairs,
                   return_intermediates=return_intermediates)


# ---------------------------------------------------------------------------------------------
# Backward pass for learned projections (Linformer card, 方法适配: E and F are learned, so training
# needs the gradients of the layer with respect to Q, K, V, E and F).  For a loss whose gradient
# with respect to O is dO, per (b, h) with valid length L (rows i >= L of O are fixed at zero, so
# dO there has no effect):
#   Kbar = E[:, :L] K[:L],  Vbar = F[:, :L] V[:L],  P = softmax(s Q Kbar^T),  O = P Vbar
#   dVbar = P^T dO          dP = dO Vbar^T          dS = P o (dP - rowsum(P o dP))
#   dQ = s dS Kbar          dKbar = s dS^T Q
#   dE[:, :L] += dKbar K[:L]^T,   dK[:L] = E[:, :L]^T dKbar
#   dF[:, :L] += dVbar V[:L]^T,   dV[:L] = F[:, :L]^T dVbar
# (the softmax Jacobian written out: d s_r = P_r (dP_r - sum_q P_q dP_q)).  Shared matrices
# collect the gradients of every head (and of both K and V when E = F) that uses them.
# ---------------------------------------------------------------------------------------------
def backward(Q, K, V, E, F, share: int, dO, lengths: Optional[Sequence[int]] = None,
             scale: Optional[float] = None):
    """Returns dQ, dK, dV ([B, H, n, d]), dE ([H_E, k, n]) and dF (same shape, or None when F
    aliases E, in which case dE holds both contributions)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    B, H, n, d = Q.shape
    s = (1.0 / np.sqrt(d)) if (scale is None or scale == 0.0) else float(scale)
    Es, Fs = head_projections(E, F, share, H)
    E = _f64(E)
    separate = share in (SHARE_NONE, SHARE_HEADWISE) and F is not None
    dE = np.zeros_like(E)
    dF = np.zeros_like(E) if separate else None
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)

    def e_index(h):
        return h if share == SHARE_NONE else 0

    for b in range(B):
        L = n if lengths is None else max(0, min(int(lengths[b]), n))
        for h in range(H):
            Eh, Fh = Es[h], Fs[h]
            Kb = project(Eh, K[b, h], L)
            Vb = project(Fh, V[b, h], L)
            P = attention_weights(Q[b, h], Kb, s)
            g = dO[b, h].copy()
            g[L:] = 0.0
            dVb = np.matmul(P.T, g)
            dP = np.matmul(g, Vb.T)
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
            dQ[b, h] = s * np.matmul(dS, Kb)
            dKb = s * np.matmul(dS.T, Q[b, h])
            dK[b, h, :L] = np.matmul(Eh[:, :L].T, dKb)
            dV[b, h, :L] = np.matmul(Fh[:, :L].T, dVb)
            dE[e_index(h), :, :L] += np.matmul(dKb, K[b, h, :L].T)
            if separate:
                dF[e_index(h), :, :L] += np.matmul(dVb, V[b, h, :L].T)
            else:
                dE[e_index(h), :, :L] += np.matmul(dVb, V[b, h, :L].T)
    return dQ, dK, dV, dE, dF
