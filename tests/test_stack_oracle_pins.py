"""Pins for the oracle of the encoder attention stack (per layer: input projection, head split,
Linformer attention with one layerwise-shared projection, head concatenation, output projection).

* With k = n and E = I a layer is ordinary multi-head attention, so the stack must equal PyTorch's
  own multi-head attention routine (float64, no biases) applied layer after layer: a library
  routine that fixes the input-projection layout, the head split, the scale, the concatenation
  and the output projection.
* A separately written brute force in pure Python loops (k < n, random E) for a tiny stack.
* Invariants: a consistent permutation of the heads changes nothing; padded rows are zero at
  every layer and the valid rows do not depend on what the padded rows hold.
"""
import math

import numpy as np
import pytest

from oracle import linformer_oracle as orc


def _weights(rng, L, dm, scale=0.4):
    return (rng.standard_normal((L, 3 * dm, dm)) * scale, rng.standard_normal((L, dm, dm)) * scale)


def test_stack_reduces_to_library_mha():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as Fn
    rng = np.random.default_rng(11)
    B, n, heads, d, L = 2, 5, 3, 4, 2
    dm = heads * d
    X = rng.standard_normal((B, n, dm))
    Wqkv, Wo = _weights(rng, L, dm)
    E = np.eye(n)[None]                      # k = n, identity projection
    ours = orc.stack_forward(X, Wqkv, Wo, E, heads)
    y = torch.from_numpy(X).transpose(0, 1).contiguous()   # [n, B, dm] (sequence first)
    for l in range(L):
        y, _ = Fn.multi_head_attention_forward(
            y, y, y, dm, heads, torch.from_numpy(Wqkv[l]), None, None, None, False, 0.0,
            torch.from_numpy(Wo[l]), None, training=False, need_weights=False)
    ref = y.transpose(0, 1).numpy()
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-12)


def _brute_layer(x, Wqkv, Wo, E, heads):
    """Textbook loops: projections, per-head Linformer attention, concatenation, output map."""
    n, dm = len(x), len(x[0])
    d = dm // heads
    k = len(E)
    proj = [[sum(x[i][c] * Wqkv[f][c] for c in range(dm)) for f in range(3 * dm)]
            for i in range(n)]
    cat = [[0.0] * dm for _ in range(n)]
    for h in range(heads):
        q = [[proj[i][h * d + c] for c in range(d)] for i in range(n)]
        kk = [[proj[i][dm + h * d + c] for c in range(d)] for i in range(n)]
        vv = [[proj[i][2 * dm + h * d + c] for c in range(d)] for i in range(n)]
        kbar = [[sum(E[r][t] * kk[t][c] for t in range(n)) for c in range(d)] for r in range(k)]
        vbar = [[sum(E[r][t] * vv[t][c] for t in range(n)) for c in range(d)] for r in range(k)]
        for i in range(n):
            logits = [sum(q[i][c] * kbar[r][c] for c in range(d)) / math.sqrt(d)
                      for r in range(k)]
            top = max(logits)
            wts = [math.exp(s - top) for s in logits]
            tot = sum(wts)
            for c in range(d):
                cat[i][h * d + c] = sum(wts[r] * vbar[r][c] for r in range(k)) / tot
    return [[sum(cat[i][f] * Wo[g][f] for f in range(dm)) for g in range(dm)] for i in range(n)]


def test_stack_brute_force_tiny():
    rng = np.random.default_rng(5)
    n, heads, d, k, L = 6, 2, 2, 3, 2
    dm = heads * d
    X = rng.standard_normal((1, n, dm))
    Wqkv, Wo = _weights(rng, L, dm, scale=0.8)
    E = rng.standard_normal((1, k, n)) * 0.5
    y = X[0].tolist()
    for l in range(L):
        y = _brute_layer(y, Wqkv[l].tolist(), Wo[l].tolist(), E[0].tolist(), heads)
    ours = orc.stack_forward(X, Wqkv, Wo, E, heads)
    assert np.allclose(ours[0], np.array(y), rtol=1e-11, atol=1e-12)


def test_stack_head_permutation_invariance():
    rng = np.random.default_rng(7)
    B, n, heads, d, k, L = 2, 8, 4, 3, 5, 2
    dm = heads * d
    X = rng.standard_normal((B, n, dm))
    Wqkv, Wo = _weights(rng, L, dm)
    E = rng.standard_normal((1, k, n)) * 0.4
    perm = [2, 0, 3, 1]
    feat = np.concatenate([np.arange(p * d, (p + 1) * d) for p in perm])
    Wqkv_p = Wqkv.copy()
    for part in range(3):
        Wqkv_p[:, part * dm:(part + 1) * dm, :] = Wqkv[:, part * dm + feat, :]
    Wo_p = Wo[:, :, feat]
    a = orc.stack_forward(X, Wqkv, Wo, E, heads)
    b = orc.stack_forward(X, Wqkv_p, Wo_p, E, heads)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    # a permutation of only the query block mixes heads up and must change the result
    Wqkv_q = Wqkv.copy()
    Wqkv_q[:, 0:dm, :] = Wqkv[:, feat, :]
    c = orc.stack_forward(X, Wqkv_q, Wo, E, heads)
    assert not np.allclose(a, c, rtol=1e-6, atol=1e-6)


def test_stack_padding():
    rng = np.random.default_rng(9)
    B, n, heads, d, k, L = 2, 10, 2, 3, 4, 3
    dm = heads * d
    X = rng.standard_normal((B, n, dm))
    Wqkv, Wo = _weights(rng, L, dm)
    E = rng.standard_normal((1, k, n)) * 0.4
    lengths = [7, 10]
    outs = orc.stack_forward(X, Wqkv, Wo, E, heads, lengths, return_layers=True)
    for Y in outs:
        assert np.all(Y[0, 7:] == 0.0)
    X2 = X.copy()
    X2[0, 7:] = rng.standard_normal((3, dm)) * 5.0
    Y2 = orc.stack_forward(X2, Wqkv, Wo, E, heads, lengths)
    assert np.allclose(Y2, outs[-1], rtol=1e-12, atol=1e-12)
