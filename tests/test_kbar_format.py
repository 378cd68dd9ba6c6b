"""CPU checks of the test-side codec for the bf16 Kbar storage format (the GPU tests use it to
feed stand-ins to the attention kernel and to read the projection's output): the e4m3 encoder
against brute-force nearest rounding, the residual byte order, and the accuracy the format
promises (each value within 2^-12 of its block's largest magnitude)."""
import numpy as np

from tests import gpu_util as G


def _all_e4m3():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    return codes, G.e4m3_decode(codes)


def test_e4m3_encoder_is_nearest_even():
    codes, vals = _all_e4m3()
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-0.05, 0.05, 4000),
                        vals, (vals[1:] + vals[:-1]) / 2])
    x = x[np.abs(x) <= 448]
    got = G.e4m3_decode(G.e4m3_encode(x))
    # brute force: nearest representable value; on a tie, the one with an even code
    d = np.abs(x[:, None] - vals[None, :])
    best = d.min(axis=1)
    for i in np.flatnonzero(np.abs(got - x) != best):
        raise AssertionError(f"{x[i]} -> {got[i]}, nearest distance {best[i]}")
    ties = np.isclose(d, best[:, None], rtol=0, atol=0).sum(axis=1) > 1
    for i in np.flatnonzero(ties):
        cand = codes[d[i] == best[i]]
        assert int(G.e4m3_encode(np.array([x[i]]))[0]) in cand
        mags = cand & 0x7F
        assert int(G.e4m3_encode(np.array([x[i]]))[0]) & 1 == 0 or np.all(mags & 1)


def test_residual_order_is_a_permutation():
    assert sorted(G.LO_PERM.tolist()) == list(range(64))
    # columns 16 ks + 8 h + j sit at byte 32 h + 8 ks + j
    for ks in range(4):
        for h in range(2):
            for j in range(8):
                assert G.LO_PERM[16 * ks + 8 * h + j] == 32 * h + 8 * ks + j


def test_kbar_codec_accuracy():
    rng = np.random.default_rng(3)
    B, H, k = 2, 3, 64
    kbar = (rng.standard_normal((B, H, k, 64)) * np.exp(rng.uniform(-6, 6, (B, H, k, 1)))).astype(np.float32)
    kbar[0, 0, 5, :32] = 0.0                     # an all-zero block
    c = 0.125 * G.LOG2E
    raw = G.encode_kbar_bf16(kbar, c)
    assert raw.size == 3 * B * H * k * 64 + 2 * B * H * k
    hi, res, x = G.decode_kbar_bf16(raw, kbar.shape)
    ref = np.float32(c) * kbar.astype(np.float32)
    blocks = np.abs(ref.astype(np.float64)).reshape(-1, 2, 32).max(axis=2)
    err = np.abs(x - ref).reshape(-1, 2, 32).max(axis=2)
    assert np.all(err <= blocks * 2.0 ** -12 + 1e-30)
    assert np.all(x.reshape(-1, 2, 32)[0 * 0 + 5, 0] == 0.0)
    # without the residual the error would be up to 2^-9 relative: the residual matters
    assert np.abs(hi - ref).max() > 4 * np.abs(x - ref).max()
