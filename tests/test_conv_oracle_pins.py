"""Pins for the convolution / pooling compression in the oracle.

* Mean pooling (w = 1/s): each projected key is the mean of its window of s keys -- checked
  against numpy's reshape-and-mean, written independently of the banded matrix.
* A general window against a pure-Python loop over windows.
* With s = 1 (k = n) and w = [1] the banded E is the identity, so the result is textbook softmax
  attention (the existing brute force).
"""
import numpy as np

from oracle import linformer_oracle as orc
from tests import test_oracle_pins as pins


def test_mean_pooling_closed_form():
    rng = np.random.default_rng(2)
    B, H, n, d, s = 2, 3, 32, 4, 4
    Q, K, V = (rng.standard_normal((B, H, n, d)) for _ in range(3))
    w = np.full((1, s), 1.0 / s)
    O, Kb, Vb = orc.conv_forward(Q, K, V, w, None, orc.SHARE_LAYERWISE,
                                 return_intermediates=True)
    assert np.allclose(Kb, K.reshape(B, H, n // s, s, d).mean(axis=3), rtol=1e-13, atol=1e-14)
    assert np.allclose(Vb, V.reshape(B, H, n // s, s, d).mean(axis=3), rtol=1e-13, atol=1e-14)


def test_window_weights_against_loops():
    rng = np.random.default_rng(4)
    H, n, d, s = 2, 12, 3, 3
    Q, K, V = (rng.standard_normal((1, H, n, d)) for _ in range(3))
    wE, wF = rng.standard_normal((H, s)), rng.standard_normal((H, s))
    _, Kb, Vb = orc.conv_forward(Q, K, V, wE, wF, orc.SHARE_NONE, return_intermediates=True)
    for h in range(H):
        for r in range(n // s):
            for c in range(d):
                kk = sum(wE[h][j] * K[0, h, r * s + j, c] for j in range(s))
                vv = sum(wF[h][j] * V[0, h, r * s + j, c] for j in range(s))
                assert abs(Kb[0, h, r, c] - kk) < 1e-12 and abs(Vb[0, h, r, c] - vv) < 1e-12


def test_unit_window_is_textbook_attention():
    rng = np.random.default_rng(6)
    n, d = 7, 3
    Q, K, V = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    O = orc.conv_forward(Q, K, V, np.ones((1, 1)), None, orc.SHARE_LAYERWISE)
    ref = pins.brute_attention(Q[0, 0].tolist(), K[0, 0].tolist(), V[0, 0].tolist(),
                               1.0 / np.sqrt(d))
    assert np.allclose(O[0, 0], ref, rtol=1e-12, atol=1e-12)


def test_padding_inside_a_window():
    rng = np.random.default_rng(8)
    n, d, s = 16, 2, 4
    Q, K, V = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    w = rng.standard_normal((1, s))
    _, Kb, _ = orc.conv_forward(Q, K, V, w, None, orc.SHARE_LAYERWISE, lengths=[6],
                                return_intermediates=True)
    # window 0 complete, window 1 holds positions 4, 5 only, windows 2 and 3 empty
    assert np.allclose(Kb[0, 0, 0], w[0] @ K[0, 0, 0:4])
    assert np.allclose(Kb[0, 0, 1], w[0, :2] @ K[0, 0, 4:6])
    assert np.all(Kb[0, 0, 2:] == 0.0)
