"""Pins for the oracle's backward pass.

* Central finite differences of f = sum(O * dO) in float64 along random directions, for every
  input (Q, K, V, E, F) and every sharing mode, with padding.
* PyTorch autograd (float64) through a separately written forward: torch matmul, softmax and
  masking, not the oracle's functions.
* Padding: gradients of K, V rows past the length and of the E, F columns past every length are
  exactly zero.
"""
import numpy as np
import pytest

from oracle import linformer_oracle as orc


def _inputs(rng, B, H, n, d, k, share, separate):
    Q, K, V, dO = (rng.standard_normal((B, H, n, d)) for _ in range(4))
    he = H if share == orc.SHARE_NONE else 1
    E = rng.standard_normal((he, k, n)) / np.sqrt(k)
    F = rng.standard_normal((he, k, n)) / np.sqrt(k) if separate else None
    return Q, K, V, dO, E, F


CASES = [(orc.SHARE_NONE, True), (orc.SHARE_NONE, False), (orc.SHARE_HEADWISE, True),
         (orc.SHARE_KV, False), (orc.SHARE_LAYERWISE, False)]


@pytest.mark.parametrize("share,separate", CASES)
def test_backward_finite_differences(share, separate):
    rng = np.random.default_rng(3 + share)
    B, H, n, d, k = 2, 2, 6, 3, 4
    Q, K, V, dO, E, F = _inputs(rng, B, H, n, d, k, share, separate)
    lengths = [6, 4]
    grads = orc.backward(Q, K, V, E, F, share, dO, lengths)
    # with F aliasing E (F = None) a step along E moves both projections, and dE holds both parts
    names = ["Q", "K", "V", "E"] + (["F"] if separate else [])
    base = {"Q": Q, "K": K, "V": V, "E": E, "F": F}
    gmap = {"Q": grads[0], "K": grads[1], "V": grads[2], "E": grads[3], "F": grads[4]}

    def f(args):
        O = orc.forward(args["Q"], args["K"], args["V"], args["E"], args["F"], share, lengths)
        return float(np.sum(O * dO))

    eps = 1e-6
    for name in names:
        for trial in range(3):
            delta = rng.standard_normal(base[name].shape)
            plus, minus = dict(base), dict(base)
            plus[name] = base[name] + eps * delta
            minus[name] = base[name] - eps * delta
            fd = (f(plus) - f(minus)) / (2 * eps)
            an = float(np.sum(gmap[name] * delta))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_backward_matches_autograd():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    B, H, n, d, k = 2, 3, 8, 4, 5
    Q, K, V, dO, E, F = _inputs(rng, B, H, n, d, k, orc.SHARE_NONE, True)
    lengths = [8, 5]
    t = {name: torch.tensor(x, requires_grad=True) for name, x in
         (("Q", Q), ("K", K), ("V", V), ("E", E), ("F", F))}
    mask = torch.zeros(B, 1, n, 1, dtype=torch.float64)
    for b, L in enumerate(lengths):
        mask[b, :, :L] = 1.0
    Kb = torch.einsum("hrt,bhtc->bhrc", t["E"], t["K"] * mask)
    Vb = torch.einsum("hrt,bhtc->bhrc", t["F"], t["V"] * mask)
    P = torch.softmax(torch.matmul(t["Q"], Kb.transpose(-1, -2)) / np.sqrt(d), dim=-1)
    O = torch.matmul(P, Vb) * mask
    (O * torch.tensor(dO)).sum().backward()
    ours = orc.backward(Q, K, V, E, F, orc.SHARE_NONE, dO, lengths)
    for name, g in zip(("Q", "K", "V", "E", "F"), ours):
        assert np.allclose(g, t[name].grad.numpy(), rtol=1e-10, atol=1e-12), name


def test_backward_padding_zeros():
    rng = np.random.default_rng(12)
    B, H, n, d, k = 2, 2, 10, 3, 4
    Q, K, V, dO, E, F = _inputs(rng, B, H, n, d, k, orc.SHARE_HEADWISE, True)
    dQ, dK, dV, dE, dF = orc.backward(Q, K, V, E, F, orc.SHARE_HEADWISE, dO, [7, 5])
    assert np.all(dK[0, :, 7:] == 0) and np.all(dK[1, :, 5:] == 0)
    assert np.all(dV[0, :, 7:] == 0) and np.all(dV[1, :, 5:] == 0)
    assert np.all(dQ[0, :, 7:] == 0) and np.all(dQ[1, :, 5:] == 0)
    assert np.all(dE[:, :, 7:] == 0) and np.all(dF[:, :, 7:] == 0)
