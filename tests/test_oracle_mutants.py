"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutant replaces one oracle function with a plausible wrong version; the listed pin tests are
then run against the mutated oracle and must raise.  This shows the pins are sharp enough to
catch a transposed operand, a dropped scale, a wrong softmax axis, a wrong padding reading and a
wrong sharing map.
"""
import numpy as np
import pytest

from oracle import linformer_oracle as orc
from tests import test_oracle_pins as pins


def _proj_transposed(P, X, length=None):
    P = np.asarray(P, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    L = X.shape[0] if length is None else int(length)
    return np.matmul(P.T[:, :L], X[:L])


def _scores_unscaled(Q, Kbar, scale):
    return np.matmul(np.asarray(Q, float), np.asarray(Kbar, float).T)


def _softmax_cols(S):
    S = np.asarray(S, dtype=np.float64)
    w = np.exp(S - S.max(axis=0, keepdims=True))
    return w / w.sum(axis=0, keepdims=True)


def _proj_ignores_length(P, X, length=None):
    return np.matmul(np.asarray(P, float), np.asarray(X, float))


_orig_heads = orc.head_projections


def _headwise_uses_E_for_V(E, F, share, heads):
    Es, Fs = _orig_heads(E, F, share, heads)
    return Es, list(Es)


def _sign_flip_scores(Q, Kbar, scale):
    return -float(scale) * np.matmul(np.asarray(Q, float), np.asarray(Kbar, float).T)


MUTANTS = [
    ("project", _proj_transposed, [pins.test_golden_orientation]),
    ("scores", _scores_unscaled, [pins.test_golden_scale]),
    ("scores", _sign_flip_scores, [pins.test_golden_orientation, pins.test_golden_scale]),
    ("softmax_rows", _softmax_cols, [pins.test_golden_orientation,
                                     pins.test_softmax_rows_sum_to_one]),
    ("project", _proj_ignores_length, [pins.test_golden_padding,
                                       pins.test_padding_ignores_positions_past_length]),
    ("head_projections", _headwise_uses_E_for_V, [pins.test_golden_orientation,
                                                   pins.test_golden_orientation_sharing_modes]),
]


@pytest.mark.parametrize("idx", range(len(MUTANTS)))
def test_mutant_is_caught(idx, monkeypatch):
    name, fn, checks = MUTANTS[idx]
    monkeypatch.setattr(orc, name, fn)
    for check in checks:
        with pytest.raises((AssertionError, ValueError)):
            if check is pins.test_golden_orientation_sharing_modes:
                check(orc.SHARE_HEADWISE)
            else:
                check()


# ---- encoder-stack oracle: planted mistakes in the head split, the concatenation and the layer
from tests import test_stack_oracle_pins as spins


def _split_heads_interleaved(Y, heads):
    Y = np.asarray(Y, dtype=np.float64)
    B, n, w = Y.shape
    return Y.reshape(B, n, w // heads, heads).transpose(0, 3, 1, 2)   # feature f -> head f % H


def _concat_heads_transposed(O):
    O = np.asarray(O, dtype=np.float64)
    B, H, n, d = O.shape
    return O.transpose(0, 2, 3, 1).reshape(B, n, H * d)               # column-major over heads


_orig_layer = orc.stack_layer


def _layer_swaps_k_and_v(X, Wqkv, Wo, E, heads, lengths=None, scale=None):
    W = np.asarray(Wqkv, dtype=np.float64).copy()
    dm = W.shape[1]
    W[dm:2 * dm], W[2 * dm:] = W[2 * dm:].copy(), W[dm:2 * dm].copy()
    return _orig_layer(X, W, Wo, E, heads, lengths, scale)


STACK_MUTANTS = [
    ("split_heads", _split_heads_interleaved, [spins.test_stack_reduces_to_library_mha,
                                               spins.test_stack_brute_force_tiny]),
    ("concat_heads", _concat_heads_transposed, [spins.test_stack_reduces_to_library_mha,
                                                spins.test_stack_brute_force_tiny]),
    ("stack_layer", _layer_swaps_k_and_v, [spins.test_stack_reduces_to_library_mha,
                                           spins.test_stack_brute_force_tiny]),
]


@pytest.mark.parametrize("idx", range(len(STACK_MUTANTS)))
def test_stack_mutant_is_caught(idx, monkeypatch):
    name, fn, checks = STACK_MUTANTS[idx]
    monkeypatch.setattr(orc, name, fn)
    for check in checks:
        with pytest.raises((AssertionError, ValueError)):
            check()


# ---- batched entries: the per-item length and the (b, h) slice a result is written to
def _dense_forward_lengths_by_head(Q, K, V, lengths=None, scale=None, pairs=None):
    Q = np.asarray(Q, dtype=np.float64)
    B, H, n, d = Q.shape
    O = np.zeros((B, H, n, d))
    todo = [(b, h) for b in range(B) for h in range(H)] if pairs is None else list(pairs)
    for b, h in todo:
        L = None if lengths is None else int(lengths[h])           # slip: indexed by head
        O[b, h] = orc.dense_attention(Q[b, h], K[b, h], V[b, h], scale, L)
    return O


def _dense_forward_swapped(Q, K, V, lengths=None, scale=None, pairs=None):
    Q = np.asarray(Q, dtype=np.float64)
    B, H, n, d = Q.shape
    O = np.zeros((B, H, n, d))
    todo = [(b, h) for b in range(B) for h in range(H)] if pairs is None else list(pairs)
    for b, h in todo:
        L = None if lengths is None else int(lengths[b])
        O[h, b] = orc.dense_attention(Q[b, h], K[b, h], V[b, h], scale, L)   # slip: O[h, b]
    return O


def _forward_variant(slip):
    def fwd(Q, K, V, E, F, share, lengths=None, scale=None, pairs=None,
            return_intermediates=False):
        Q = np.asarray(Q, dtype=np.float64)
        B, H, n, d = Q.shape
        Es, Fs = orc.head_projections(E, F, share, H)
        k = Es[0].shape[0]
        O = np.zeros((B, H, n, d))
        Kb = np.zeros((B, H, k, d))
        Vb = np.zeros((B, H, k, d))
        every = [(b, h) for b in range(B) for h in range(H)]
        todo = every if (pairs is None or slip == "pairs_ignored") else list(pairs)
        for b, h in todo:
            L = None if lengths is None else int(lengths[h if slip == "lengths_by_head" else b])
            ib, ih = (h, b) if slip == "swapped" else (b, h)
            Kb[b, h] = orc.project(Es[h], K[ib, ih], L)
            Vb[b, h] = orc.project(Fs[h], V[ib, ih], L)
            O[b, h] = orc.attend(Q[ib, ih], Kb[b, h], Vb[b, h], scale, L)
        if return_intermediates:
            return O, Kb, Vb
        return O
    return fwd


def _run_all(test, params):
    for args in params:
        test(*args)


_DENSE_CASES = [(3, 3, 5, [0, 5, 3]), (4, 2, 6, [2, 6, 0, 5])]
_FWD_CASES = [(3, 3, 7, [0, 7, 4]), (4, 2, 6, [3, 6, 0, 1])]

BATCH_MUTANTS = [
    ("dense_forward", _dense_forward_lengths_by_head,
     lambda: _run_all(pins.test_dense_forward_batch_matches_brute_per_item, _DENSE_CASES)),
    ("dense_forward", _dense_forward_swapped,
     lambda: _run_all(pins.test_dense_forward_batch_matches_brute_per_item, _DENSE_CASES)),
    ("forward", _forward_variant("lengths_by_head"),
     lambda: _run_all(pins.test_forward_batch_matches_brute_per_item, _FWD_CASES)),
    ("forward", _forward_variant("swapped"),
     lambda: _run_all(pins.test_forward_batch_matches_brute_per_item, _FWD_CASES)),
    ("forward", _forward_variant("pairs_ignored"),
     lambda: pins.test_forward_pairs_subset_equals_full(orc.SHARE_NONE)),
]


@pytest.mark.parametrize("idx", range(len(BATCH_MUTANTS)))
def test_batch_mutant_is_caught(idx, monkeypatch):
    name, fn, check = BATCH_MUTANTS[idx]
    monkeypatch.setattr(orc, name, fn)
    with pytest.raises((AssertionError, ValueError)):
        check()


def test_batch_mutant_harness_passes_unmutated():
    # the same checks pass on the oracle as written, so a caught mutant is the slip's doing
    for _, _, check in BATCH_MUTANTS:
        check()
