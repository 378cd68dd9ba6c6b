"""Pins for the float64 oracle, checked against things other than the oracle itself.

* hand-derived fixtures under tests/golden/ (each cites its passage);
* a separately written brute-force textbook attention (pure Python loops, log-sum-exp);
* closed forms (identical rows of E, k = 1, Q = 0) and invariants (row sums, linearity,
  permutations, padding, sharing modes).

Each pin is chosen so a plausible slip in the oracle fails at least one of them: a transposed E
or F (hand_orientation), a missing or wrong scale (hand_scale), softmax over the wrong axis
(brute force with k = n), padding handled as a softmax mask or ignored (hand_padding, V8), a
sharing mode mapped to the wrong matrix (V9).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import linformer_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------------------------
# Independent brute force (pure Python loops), written from the textbook definition of softmax
# attention (Linformer 요약 설명, section "Transformer and Self-Attention"), not from the oracle.
# ----------------------------------------------------------------------------------------------
def brute_attention(Q, K, V, scale, valid=None):
    n, d = len(Q), len(Q[0])
    nk = len(K)
    keys = range(nk) if valid is None else range(valid)
    out = []
    for i in range(n):
        if valid is not None and i >= valid:
            out.append([0.0] * len(V[0]))
            continue
        logit = {}
        for j in keys:
            acc = 0.0
            for c in range(d):
                acc += Q[i][c] * K[j][c]
            logit[j] = acc * scale
        top = max(logit.values())
        lse = top + math.log(sum(math.exp(v - top) for v in logit.values()))
        row = []
        for c in range(len(V[0])):
            row.append(sum(math.exp(logit[j] - lse) * V[j][c] for j in keys))
        out.append(row)
    return np.array(out)


def brute_matmul(A, B):
    return np.array([[sum(A[i][t] * B[t][j] for t in range(len(B))) for j in range(len(B[0]))]
                     for i in range(len(A))])


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------- golden fixtures
def test_golden_orientation():
    g = _golden("hand_orientation.json")
    Kb = orc.project(g["E"], g["K"])
    Vb = orc.project(g["F"], g["V"])
    np.testing.assert_allclose(Kb, g["Kbar"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(Vb, g["Vbar"], rtol=0, atol=1e-15)
    P = orc.attention_weights(g["Q"], Kb, g["scale"])
    np.testing.assert_allclose(P, g["P"], rtol=0, atol=1e-14)
    O = orc.attend(g["Q"], Kb, Vb, g["scale"])
    np.testing.assert_allclose(O, g["O"], rtol=0, atol=1e-13)
    # the same through the batched entry, unshared mode with one head
    O4 = orc.forward(np.array(g["Q"])[None, None], np.array(g["K"])[None, None],
                     np.array(g["V"])[None, None], np.array(g["E"])[None],
                     np.array(g["F"])[None], orc.SHARE_NONE, scale=g["scale"])
    np.testing.assert_allclose(O4[0, 0], g["O"], rtol=0, atol=1e-13)


def test_golden_padding():
    g = _golden("hand_padding.json")
    L = g["length"]
    Kb = orc.project(g["E"], g["K"], L)
    Vb = orc.project(g["F"], g["V"], L)
    np.testing.assert_allclose(Kb, g["Kbar"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(Vb, g["Vbar"], rtol=0, atol=1e-15)
    O = orc.attend(g["Q"], Kb, Vb, g["scale"], L)
    np.testing.assert_allclose(O, g["O"], rtol=0, atol=1e-14)
    O4 = orc.forward(np.array(g["Q"])[None, None], np.array(g["K"])[None, None],
                     np.array(g["V"])[None, None], np.array(g["E"])[None],
                     np.array(g["F"])[None], orc.SHARE_NONE, lengths=[L], scale=g["scale"])
    np.testing.assert_allclose(O4[0, 0], g["O"], rtol=0, atol=1e-14)


def test_golden_scale():
    g = _golden("hand_scale.json")
    O = orc.forward(np.array(g["Q"])[None, None], np.array(g["K"])[None, None],
                    np.array(g["V"])[None, None], np.array(g["E"])[None],
                    np.array(g["F"])[None], orc.SHARE_NONE, scale=g["scale"])
    np.testing.assert_allclose(O[0, 0], g["O"], rtol=0, atol=1e-13)


def test_golden_model_section_shapes():
    g = _golden("model_section_shapes.json")
    rng = np.random.default_rng(0)
    n, d, k = g["n"], g["d"], g["k"]
    Q, K, V = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    E, F = _rand(rng, k, n) / math.sqrt(k), _rand(rng, k, n) / math.sqrt(k)
    Kb, Vb = orc.project(E, K), orc.project(F, V)
    assert list(Kb.shape) == g["Kbar_shape"]
    assert list(Vb.shape) == g["Vbar_shape"]
    assert list(orc.attention_weights(Q, Kb, 1 / math.sqrt(d)).shape) == g["attention_shape"]
    assert list(orc.attend(Q, Kb, Vb).shape) == g["output_shape"]


# ------------------------------------------------------------- V1: k = n, E = F = I is textbook
@pytest.mark.parametrize("n,d", [(1, 1), (2, 4), (3, 1), (8, 8), (17, 4)])
@pytest.mark.parametrize("share", [orc.SHARE_NONE, orc.SHARE_KV, orc.SHARE_LAYERWISE])
def test_identity_projection_is_textbook_attention(n, d, share):
    rng = np.random.default_rng(100 + n * 10 + d)
    H = 2
    Q, K, V = _rand(rng, 1, H, n, d), _rand(rng, 1, H, n, d), _rand(rng, 1, H, n, d)
    I = np.eye(n)
    E = np.stack([I] * H) if share == orc.SHARE_NONE else I[None]
    F = E.copy() if share == orc.SHARE_NONE else None
    scale = 1 / math.sqrt(d)
    O = orc.forward(Q, K, V, E, F, share)
    for h in range(H):
        ref = brute_attention(Q[0, h].tolist(), K[0, h].tolist(), V[0, h].tolist(), scale)
        np.testing.assert_allclose(O[0, h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n,d,L", [(5, 3, 2), (8, 4, 8), (9, 2, 1), (6, 4, 0)])
def test_dense_oracle_is_textbook_attention(n, d, L):
    rng = np.random.default_rng(7 + n + L)
    Q, K, V = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    scale = 1 / math.sqrt(d)
    ref = brute_attention(Q.tolist(), K.tolist(), V.tolist(), scale, valid=L)
    np.testing.assert_allclose(orc.dense_attention(Q, K, V, None, L), ref, rtol=1e-12,
                               atol=1e-12)
    ref_full = brute_attention(Q.tolist(), K.tolist(), V.tolist(), scale)
    np.testing.assert_allclose(orc.dense_attention(Q, K, V), ref_full, rtol=1e-12, atol=1e-12)


def test_projection_matches_brute_matmul():
    rng = np.random.default_rng(3)
    E, K = _rand(rng, 5, 7), _rand(rng, 7, 3)
    np.testing.assert_allclose(orc.project(E, K), brute_matmul(E.tolist(), K.tolist()),
                               rtol=1e-13, atol=1e-13)
    # length 4: only the first 4 positions count
    np.testing.assert_allclose(orc.project(E, K, 4),
                               brute_matmul(E[:, :4].tolist(), K[:4].tolist()),
                               rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------- V2: softmax rows sum to 1
def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(11)
    Q, Kb = _rand(rng, 40, 16) * 5, _rand(rng, 24, 16) * 5
    P = orc.attention_weights(Q, Kb, 0.25)
    assert P.shape == (40, 24)
    assert np.all(P > 0) and np.all(P <= 1)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    # shift invariance of each row, and the argmax stays the argmax of the scores
    S = orc.scores(Q, Kb, 0.25)
    np.testing.assert_allclose(orc.softmax_rows(S + 123.0), P, rtol=1e-12, atol=1e-14)
    assert np.array_equal(P.argmax(axis=1), S.argmax(axis=1))


# ---------------------------------------- V3, V4, V5: closed forms where the softmax is uniform
def _mean_vbar(F, V, L=None):
    """(1/k) sum_r sum_t F[r][t] V[t][c] by explicit loops."""
    k, n = len(F), len(F[0])
    L = n if L is None else L
    return [sum(F[r][t] * V[t][c] for r in range(k) for t in range(L)) / k
            for c in range(len(V[0]))]


@pytest.mark.parametrize("share", [orc.SHARE_NONE, orc.SHARE_HEADWISE])
def test_identical_rows_of_E_give_mean_of_vbar(share):
    rng = np.random.default_rng(21)
    B, H, n, d, k = 2, 3, 12, 4, 5
    Q, K, V = _rand(rng, B, H, n, d), _rand(rng, B, H, n, d), _rand(rng, B, H, n, d)
    HE = H if share == orc.SHARE_NONE else 1
    row = _rand(rng, HE, 1, n)
    E = np.repeat(row, k, axis=1)
    F = _rand(rng, HE, k, n)
    O = orc.forward(Q, K, V, E, F, share)
    for b in range(B):
        for h in range(H):
            Fh = F[h if share == orc.SHARE_NONE else 0]
            want = _mean_vbar(Fh.tolist(), V[b, h].tolist())
            np.testing.assert_allclose(O[b, h], np.tile(want, (n, 1)), rtol=1e-12, atol=1e-12)


def test_k_equals_one_gives_projected_value_row():
    rng = np.random.default_rng(22)
    n, d = 9, 3
    Q, K, V = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    E, F = _rand(rng, 1, 1, n), _rand(rng, 1, 1, n)
    O = orc.forward(Q, K, V, E, F, orc.SHARE_NONE)
    want = brute_matmul(F[0].tolist(), V[0, 0].tolist())[0]
    np.testing.assert_allclose(O[0, 0], np.tile(want, (n, 1)), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("share", [orc.SHARE_NONE, orc.SHARE_KV])
def test_one_token_item_closed_form(share):
    """An item of one valid position: every projected key is E[r, 0] K_0 and every projected value
    F[r, 0] V_0, so row 0 of the output is (sum_r w_r F[r, 0]) V_0 with w the softmax over r of
    scale (q_0 . K_0) E[r, 0], written here with plain loops (a weighted mean of one column of
    F times one value row), and rows past the length are zero."""
    rng = np.random.default_rng(31)
    n, d, k = 6, 4, 5
    Q, K, V = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    E = _rand(rng, 1, k, n)
    F = _rand(rng, 1, k, n) if share == orc.SHARE_NONE else None
    Fm = (F if F is not None else E)[0]
    O = orc.forward(Q, K, V, E, F, share, lengths=[1])
    scale = 1.0 / math.sqrt(d)
    qk = sum(Q[0, 0, 0, c] * K[0, 0, 0, c] for c in range(d))
    logits = [scale * qk * E[0, r, 0] for r in range(k)]
    top = max(logits)
    z = sum(math.exp(x - top) for x in logits)
    coef = sum(math.exp(logits[r] - top) / z * Fm[r, 0] for r in range(k))
    want = np.zeros((n, d))
    want[0] = [coef * V[0, 0, 0, c] for c in range(d)]
    np.testing.assert_allclose(O[0, 0], want, rtol=1e-12, atol=1e-14)


def test_zero_queries_give_mean_of_vbar():
    rng = np.random.default_rng(23)
    n, d, k = 10, 4, 6
    K, V = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    Q = np.zeros((1, 1, n, d))
    E, F = _rand(rng, 1, k, n), _rand(rng, 1, k, n)
    O = orc.forward(Q, K, V, E, F, orc.SHARE_NONE)
    want = _mean_vbar(F[0].tolist(), V[0, 0].tolist())
    np.testing.assert_allclose(O[0, 0], np.tile(want, (n, 1)), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------- V6: linear in V at fixed K
def test_linear_in_values():
    rng = np.random.default_rng(31)
    n, d, k = 16, 4, 6
    Q, K = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    V1, V2 = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    E, F = _rand(rng, 1, k, n), _rand(rng, 1, k, n)
    f = lambda V: orc.forward(Q, K, V, E, F, orc.SHARE_NONE)
    np.testing.assert_allclose(f(V1 - 2.5 * V2), f(V1) - 2.5 * f(V2), rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------------- V7: permutations
def test_position_permutation_invariance():
    rng = np.random.default_rng(41)
    n, d, k = 13, 4, 5
    Q, K, V = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    E, F = _rand(rng, 1, k, n), _rand(rng, 1, k, n)
    perm = rng.permutation(n)
    O = orc.forward(Q, K, V, E, F, orc.SHARE_NONE)
    # permuting the key/value positions together with E, F columns changes nothing
    Ok = orc.forward(Q, K[:, :, perm], V[:, :, perm], E[:, :, perm], F[:, :, perm],
                     orc.SHARE_NONE)
    np.testing.assert_allclose(Ok, O, rtol=1e-12, atol=1e-12)
    # permuting the queries permutes the output rows
    Oq = orc.forward(Q[:, :, perm], K, V, E, F, orc.SHARE_NONE)
    np.testing.assert_allclose(Oq, O[:, :, perm], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- V8: padding
def test_padding_ignores_positions_past_length():
    rng = np.random.default_rng(51)
    B, H, n, d, k = 3, 2, 20, 4, 6
    lengths = [20, 7, 0]
    Q, K, V = _rand(rng, B, H, n, d), _rand(rng, B, H, n, d), _rand(rng, B, H, n, d)
    E, F = _rand(rng, H, k, n), _rand(rng, H, k, n)
    O = orc.forward(Q, K, V, E, F, orc.SHARE_NONE, lengths=lengths)
    # garbage past each length changes nothing
    Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
    for b, L in enumerate(lengths):
        Q2[b, :, L:] = 1e3 * _rand(rng, H, n - L, d)
        K2[b, :, L:] = 1e3 * _rand(rng, H, n - L, d)
        V2[b, :, L:] = 1e3 * _rand(rng, H, n - L, d)
    np.testing.assert_array_equal(orc.forward(Q2, K2, V2, E, F, orc.SHARE_NONE,
                                              lengths=lengths), O)
    # equal to a run at n' = L on the truncated inputs (and E, F truncated to L columns)
    for b, L in enumerate(lengths):
        assert np.all(O[b, :, L:] == 0.0)
        if L == 0:
            continue
        Ot = orc.forward(Q[b:b + 1, :, :L], K[b:b + 1, :, :L], V[b:b + 1, :, :L],
                         E[:, :, :L], F[:, :, :L], orc.SHARE_NONE)
        np.testing.assert_allclose(O[b, :, :L], Ot[0], rtol=1e-12, atol=1e-13)
    # the same as zero padding with no lengths, on the valid rows
    Kz, Vz = K.copy(), V.copy()
    for b, L in enumerate(lengths):
        Kz[b, :, L:] = 0.0
        Vz[b, :, L:] = 0.0
    Oz = orc.forward(Q, Kz, Vz, E, F, orc.SHARE_NONE)
    for b, L in enumerate(lengths):
        np.testing.assert_allclose(O[b, :, :L], Oz[b, :, :L], rtol=1e-12, atol=1e-13)


def test_length_zero_gives_uniform_zero_projection():
    # with L = 0, Kbar = Vbar = 0 and every output row is zero
    rng = np.random.default_rng(52)
    Q, K, V = _rand(rng, 1, 1, 4, 2), _rand(rng, 1, 1, 4, 2), _rand(rng, 1, 1, 4, 2)
    E = _rand(rng, 1, 3, 4)
    O, Kb, Vb = orc.forward(Q, K, V, E, None, orc.SHARE_NONE, lengths=[0],
                            return_intermediates=True)
    assert np.all(Kb == 0) and np.all(Vb == 0) and np.all(O == 0)


# ------------------------------------------------------------------------ V9: sharing modes
@pytest.mark.parametrize("share", [orc.SHARE_HEADWISE, orc.SHARE_KV, orc.SHARE_LAYERWISE])
def test_sharing_modes_equal_expanded_unshared(share):
    rng = np.random.default_rng(61)
    B, H, n, d, k = 2, 3, 11, 4, 5
    Q, K, V = _rand(rng, B, H, n, d), _rand(rng, B, H, n, d), _rand(rng, B, H, n, d)
    E = _rand(rng, 1, k, n)
    F = _rand(rng, 1, k, n) if share == orc.SHARE_HEADWISE else None
    O = orc.forward(Q, K, V, E, F, share, lengths=[11, 6])
    Ex = np.repeat(E, H, axis=0)
    Fx = np.repeat(F if F is not None else E, H, axis=0)
    Ox = orc.forward(Q, K, V, Ex, Fx, orc.SHARE_NONE, lengths=[11, 6])
    np.testing.assert_array_equal(O, Ox)


def test_sharing_mode_errors():
    E = np.zeros((2, 3, 4))
    with pytest.raises(ValueError):
        orc.head_projections(E, None, orc.SHARE_KV, 2)          # shared needs a single E
    with pytest.raises(ValueError):
        orc.head_projections(E[:1], None, orc.SHARE_HEADWISE, 2)  # headwise needs F
    with pytest.raises(ValueError):
        orc.head_projections(E[:1], E[:1] + 1, orc.SHARE_KV, 2)   # key-value needs E = F


def test_slice_rel_err_metric():
    ref = np.zeros((2, 1, 3, 2))
    ref[0, 0] = [[1, -2], [0.5, 0], [0, 0]]
    ref[1, 0] = [[10, 0], [0, 0], [0, 0]]
    out = ref.copy()
    out[0, 0, 1, 1] += 0.02      # 0.02 / 2 = 1e-2 on slice 0
    out[1, 0, 0, 0] += 0.05      # 0.05 / 10 = 5e-3 on slice 1
    assert abs(orc.slice_rel_err(out, ref) - 1e-2) < 1e-15


@pytest.mark.parametrize("share", [orc.SHARE_NONE, orc.SHARE_HEADWISE, orc.SHARE_KV,
                                   orc.SHARE_LAYERWISE])
def test_golden_orientation_sharing_modes(share):
    """Two heads on the hand example: headwise keeps E and F apart, key-value/layerwise use E."""
    g = _golden("hand_orientation.json")
    Q = np.array([g["Q"], g["Q"]])[None]
    K = np.array([g["K"], g["K"]])[None]
    V = np.array([g["V"], g["V"]])[None]
    E1, F1 = np.array(g["E"])[None], np.array(g["F"])[None]
    if share == orc.SHARE_NONE:
        O = orc.forward(Q, K, V, np.concatenate([E1, E1]), np.concatenate([F1, F1]), share,
                        scale=g["scale"])
        want = g["O"]
    elif share == orc.SHARE_HEADWISE:
        O = orc.forward(Q, K, V, E1, F1, share, scale=g["scale"])
        want = g["O"]
    else:
        O = orc.forward(Q, K, V, E1, None, share, scale=g["scale"])
        want = g["O_kv_shared"]
    for h in range(2):
        np.testing.assert_allclose(O[0, h], want, rtol=0, atol=1e-13)


# ------------------------------------------ batched entries: each (b, h) on its own item's length
# The batched entry points look up one length per batch item and write slice (b, h) from the
# inputs of slice (b, h).  Checked per slice against the separately written brute force, on
# batches whose items all have different lengths (0 and n included), with as many heads as
# batch items so that a slip between the two indices gives a wrong value rather than an
# index error.
def _per_item_lengths_batch(seed, B, H, n, d):
    rng = np.random.default_rng(seed)
    Q, K, V = _rand(rng, B, H, n, d), _rand(rng, B, H, n, d), _rand(rng, B, H, n, d)
    return rng, Q, K, V


@pytest.mark.parametrize("B,H,n,lengths", [(3, 3, 5, [0, 5, 3]), (4, 2, 6, [2, 6, 0, 5])])
def test_dense_forward_batch_matches_brute_per_item(B, H, n, lengths):
    d = 3
    _, Q, K, V = _per_item_lengths_batch(81 + B, B, H, n, d)
    scale = 1 / math.sqrt(d)
    O = orc.dense_forward(Q, K, V, lengths)
    for b in range(B):
        for h in range(H):
            ref = brute_attention(Q[b, h].tolist(), K[b, h].tolist(), V[b, h].tolist(), scale,
                                  valid=lengths[b])
            np.testing.assert_allclose(O[b, h], ref, rtol=1e-12, atol=1e-12)
    # no lengths: every key and every row of every slice
    O = orc.dense_forward(Q, K, V)
    for b in range(B):
        for h in range(H):
            ref = brute_attention(Q[b, h].tolist(), K[b, h].tolist(), V[b, h].tolist(), scale)
            np.testing.assert_allclose(O[b, h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("B,H,n,lengths", [(3, 3, 7, [0, 7, 4]), (4, 2, 6, [3, 6, 0, 1])])
def test_forward_batch_matches_brute_per_item(B, H, n, lengths):
    # Kbar = E_h[:, :L] K[:L] and Vbar = F_h[:, :L] V[:L] by explicit loops, then the textbook
    # attention over all k projected slots, then rows past the item's length set to zero
    d, k = 3, 4
    rng, Q, K, V = _per_item_lengths_batch(91 + B, B, H, n, d)
    E, F = _rand(rng, H, k, n), _rand(rng, H, k, n)
    scale = 0.7
    O = orc.forward(Q, K, V, E, F, orc.SHARE_NONE, lengths=lengths, scale=scale)
    for b in range(B):
        L = lengths[b]
        for h in range(H):
            Kb = brute_matmul(E[h][:, :L].tolist(), K[b, h][:L].tolist()) if L else np.zeros((k, d))
            Vb = brute_matmul(F[h][:, :L].tolist(), V[b, h][:L].tolist()) if L else np.zeros((k, d))
            ref = brute_attention(Q[b, h].tolist(), Kb.tolist(), Vb.tolist(), scale)
            ref[L:] = 0.0
            np.testing.assert_allclose(O[b, h], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------ the (b, h) subset mode used by bounded checks
PAIRS = [(0, 3), (2, 1), (1, 0), (2, 2)]


def _subset_inputs():
    rng = np.random.default_rng(101)
    B, H, n, d, k = 3, 4, 8, 3, 5
    Q, K, V = _rand(rng, B, H, n, d), _rand(rng, B, H, n, d), _rand(rng, B, H, n, d)
    return rng, Q, K, V, [8, 3, 0], k


def _check_subset(sub, full):
    assert sub.shape == full.shape
    for b in range(full.shape[0]):
        for h in range(full.shape[1]):
            if (b, h) in PAIRS:
                np.testing.assert_array_equal(sub[b, h], full[b, h])
            else:
                assert np.all(sub[b, h] == 0.0)


@pytest.mark.parametrize("share", [orc.SHARE_NONE, orc.SHARE_HEADWISE, orc.SHARE_KV])
def test_forward_pairs_subset_equals_full(share):
    rng, Q, K, V, lengths, k = _subset_inputs()
    H, n = Q.shape[1], Q.shape[2]
    HE = H if share == orc.SHARE_NONE else 1
    E = _rand(rng, HE, k, n)
    F = None if share == orc.SHARE_KV else _rand(rng, HE, k, n)
    full = orc.forward(Q, K, V, E, F, share, lengths=lengths)
    fullO, fullK, fullV = orc.forward(Q, K, V, E, F, share, lengths=lengths,
                                      return_intermediates=True)
    np.testing.assert_array_equal(full, fullO)
    # the slices the subset touches are not all zero, so "equal" is not vacuous
    assert all(np.abs(fullO[b, h]).max() > 0 for b, h in PAIRS if lengths[b] > 0)
    _check_subset(orc.forward(Q, K, V, E, F, share, lengths=lengths, pairs=PAIRS), full)
    subO, subK, subV = orc.forward(Q, K, V, E, F, share, lengths=lengths, pairs=PAIRS,
                                   return_intermediates=True)
    _check_subset(subO, fullO)
    _check_subset(subK, fullK)
    _check_subset(subV, fullV)


def test_conv_and_dense_pairs_subset_equal_full():
    rng, Q, K, V, lengths, _ = _subset_inputs()
    H, n = Q.shape[1], Q.shape[2]
    wE, wF = _rand(rng, H, 2), _rand(rng, H, 2)   # window 2: k = n / 2
    full = orc.conv_forward(Q, K, V, wE, wF, orc.SHARE_NONE, lengths=lengths)
    _check_subset(orc.conv_forward(Q, K, V, wE, wF, orc.SHARE_NONE, lengths=lengths,
                                   pairs=PAIRS), full)
    full = orc.dense_forward(Q, K, V, lengths)
    _check_subset(orc.dense_forward(Q, K, V, lengths, pairs=PAIRS), full)
