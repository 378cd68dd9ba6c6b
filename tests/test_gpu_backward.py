"""GPU parity of the backward pass (linformer_backward) against the oracle's backward on the same
inputs (bf16 values for bf16 workloads, exactly as the kernels see them).  All of the backward's
arithmetic is fp32, so it is held to the fp32 bar, 1e-4 of each gradient slice's largest
magnitude (per (b, h) for dQ, dK, dV; per matrix for dE, dF), for both input dtypes."""
import numpy as np
import pytest

from efficient_transformer_attention_seq_amd import linformer as L
from efficient_transformer_attention_seq_amd import synth
from oracle import linformer_oracle as orc
from tests import gpu_util as G

pytestmark = pytest.mark.gpu
TOL = 1e-4
BF, F32 = synth.DT_BF16, synth.DT_F32
NONE, HEAD, KV, LAYER = (synth.SHARE_NONE, synth.SHARE_HEADWISE, synth.SHARE_KV,
                         synth.SHARE_LAYERWISE)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if G.torch_mod().cuda.device_count() < 1:
        pytest.skip("no GPU")
    yield


def _mat_err(out, ref):
    return float(np.abs(out - ref).max() / max(np.abs(ref).max(), 1e-300))


@pytest.mark.parametrize("B,H,n,k,dtype,share,lengths", [
    (2, 3, 128, 64, BF, NONE, [128, 77]),
    (1, 2, 256, 128, F32, NONE, None),
    (2, 2, 192, 96, BF, HEAD, [150, 192]),
    (3, 2, 128, 32, BF, KV, [128, 1, 64]),
    (2, 1, 320, 256, BF, LAYER, [300, 320]),
    (1, 4, 512, 160, F32, LAYER, [511]),
    (1, 2, 2112, 96, BF, NONE, [2000]),   # reduction split 8 ways, ragged last chunk and row block
    (2, 4, 256, 64, BF, KV, [256, 100]),  # dE's reduction split, second part added with beta
    (1, 3, 384, 192, BF, HEAD, [333]),
    (3, 2, 256, 64, BF, NONE, [0, 256, 17]),   # an empty item
    (2, 1, 256, 224, F32, NONE, [256, 129]),
    # 512 slot tiles of 64: one slot-block workgroup per tile over all queries (smaller problems
    # split each tile's queries between two workgroups whose sums are paired)
    (4, 32, 128, 256, BF, NONE, [128, 70, 33, 128]),
    (8, 16, 64, 256, F32, LAYER, None),
])
def test_backward_parity(B, H, n, k, dtype, share, lengths):
    inp = synth.random_inputs(B, H, n, 64, k, dtype, share, seed=B * 100 + n + k, lengths=lengths)
    rng = np.random.default_rng(n + k)
    dO = synth.to_dtype(rng.standard_normal((B, H, n, 64)), dtype)
    G.log(f"backward B{B} H{H} n{n} k{k} dtype {dtype} share {share} lengths {lengths}")
    got = G.run_backward(inp, dO)
    ref = orc.backward(inp.Q, inp.K, inp.V, inp.E, inp.F, share, dO, inp.lengths)
    errs = []
    for name, g, r in zip(("dQ", "dK", "dV", "dE", "dF"), got, ref):
        if r is None:
            assert g is None
            continue
        assert np.all(np.isfinite(g)), name
        e = orc.slice_rel_err(g, r) if name in ("dQ", "dK", "dV") else _mat_err(g, r)
        errs.append((name, e))
    G.log("  " + "  ".join(f"{n_} {e:.2e}" for n_, e in errs))
    for name, e in errs:
        assert e <= TOL, (name, e)
    if lengths is not None:   # gradients of padded positions are exactly zero
        for b, L in enumerate(lengths):
            assert np.all(got[1][b, :, L:] == 0) and np.all(got[2][b, :, L:] == 0)


def _random_case(seed):
    """A seeded shape over the supported space: batch and heads 1-4, n a multiple of 64 up to
    1024, k a multiple of 32 up to 256, any sharing mode and input dtype, lengths of at least a
    quarter of n (or 0 for one item of a multi-item batch).  Items of one or a few tokens are
    left to the normwise test below: their gradient slices cancel to far below the terms they
    sum."""
    rng = np.random.default_rng(8100 + seed)
    B, H = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    n = 64 * int(rng.integers(1, 17))
    k = 32 * int(rng.integers(1, 9))
    share = [NONE, HEAD, KV, LAYER][int(rng.integers(0, 4))]
    dtype = F32 if rng.random() < 0.4 else BF
    lens = [int(rng.integers(max(2, n // 4), n + 1)) for _ in range(B)]
    if B > 1:
        lens[int(rng.integers(0, B))] = 0
    return B, H, n, k, dtype, share, lens


@pytest.mark.parametrize("seed", range(8))
def test_backward_random_shapes(seed):
    B, H, n, k, dtype, share, lengths = _random_case(seed)
    test_backward_parity(B, H, n, k, dtype, share, lengths)


def test_backward_one_token_item_is_normwise_accurate():
    """A one-token item's gradients are covariances under the softmax weights over the k slots
    (dS sums to zero), so a head's dQ, dK, dV slice can come out orders of magnitude below the
    terms it sums.  The products carry their operands to within 2^-16, so such a slice meets the
    1e-4 bar against the gradient tensor's largest magnitude (normwise), not against its own;
    every slice of the other items meets it against its own."""
    B, H, n, k, lengths = 4, 32, 128, 256, [128, 70, 1, 128]
    inp = synth.random_inputs(B, H, n, 64, k, BF, NONE, seed=B * 100 + n + k, lengths=lengths)
    dO = synth.to_dtype(np.random.default_rng(n + k).standard_normal((B, H, n, 64)), BF)
    got = G.run_backward(inp, dO)
    ref = orc.backward(inp.Q, inp.K, inp.V, inp.E, inp.F, NONE, dO, inp.lengths)
    for name, g, r in zip(("dQ", "dK", "dV"), got[:3], ref[:3]):
        scale = np.abs(r).max()
        for b in range(B):
            for h in range(H):
                d = np.abs(g[b, h] - r[b, h]).max()
                if lengths[b] > 1:
                    assert d <= TOL * np.abs(r[b, h]).max(), (name, b, h)
                else:
                    assert d <= TOL * scale, (name, b, h, d / scale)
    for name, g, r in zip(("dE",), got[3:4], ref[3:4]):
        assert _mat_err(g, r) <= TOL, name


def test_backward_unshared_same_f_as_e():
    """Unshared with F omitted (F = E per head): dF is not written, dE holds both parts."""
    inp = synth.random_inputs(2, 2, 128, 64, 64, BF, NONE, seed=5, lengths=[128, 90])
    inp = synth.Inputs(inp.wl, inp.Q, inp.K, inp.V, inp.E, None, inp.lengths)
    dO = synth.to_dtype(np.random.default_rng(6).standard_normal((2, 2, 128, 64)), BF)
    got = G.run_backward(inp, dO)
    ref = orc.backward(inp.Q, inp.K, inp.V, inp.E, None, NONE, dO, inp.lengths)
    assert got[4] is None and ref[4] is None
    assert _mat_err(got[3], ref[3]) <= TOL and orc.slice_rel_err(got[1], ref[1]) <= TOL


@pytest.mark.parametrize("dtype,share", [(BF, NONE), (F32, LAYER)])
def test_backward_ignores_padded_rows(dtype, share):
    """Rows of K, V and dO at or past an item's length are not part of the problem: filled with
    other values they change nothing (the oracle ignores them by construction)."""
    B, H, n, k, lengths = 2, 2, 320, 64, [200, 77]
    inp = synth.random_inputs(B, H, n, 64, k, dtype, share, seed=11, lengths=lengths)
    rng = np.random.default_rng(12)
    dO = rng.standard_normal((B, H, n, 64))
    Q, K, V = inp.Q.copy(), inp.K.copy(), inp.V.copy()
    for b, L in enumerate(lengths):
        for x in (Q, K, V, dO):
            x[b, :, L:] = 3.0 * rng.standard_normal(x[b, :, L:].shape)
    Q, K, V, dO = (synth.to_dtype(x, dtype) for x in (Q, K, V, dO))
    inp = synth.Inputs(inp.wl, Q, K, V, inp.E, inp.F, inp.lengths)
    got = G.run_backward(inp, dO)
    ref = orc.backward(Q, K, V, inp.E, inp.F, share, dO, inp.lengths)
    for name, g, r in zip(("dQ", "dK", "dV", "dE", "dF"), got, ref):
        if r is None:
            continue
        e = orc.slice_rel_err(g, r) if name in ("dQ", "dK", "dV") else _mat_err(g, r)
        assert e <= TOL, (name, e)
    for b, L in enumerate(lengths):
        assert np.all(got[0][b, :, L:] == 0) and np.all(got[1][b, :, L:] == 0)


def test_backward_long_padded_sampled():
    """The benchmarked shape (B8 H12 n4096 k256, per-head E, F, padded lengths), one launch over
    the whole batch; checked on one head against the oracle run on that head alone (dE, dF of a
    head collect only that head's items, so the slice is exact), every item of it."""
    wl = synth.WORKLOADS["long_b8_h12_n4096_k256_unshared_padded"]
    inp = synth.make_inputs(wl)
    dO = synth.to_dtype(np.random.default_rng(1).standard_normal((wl.batch, wl.heads, wl.n, wl.d)),
                        wl.dtype)
    G.log(f"backward {wl.name} full launch")
    got = G.run_backward(inp, dO)
    h = 5
    ref = orc.backward(inp.Q[:, h:h + 1], inp.K[:, h:h + 1], inp.V[:, h:h + 1], inp.E[h:h + 1],
                       inp.F[h:h + 1], wl.share, dO[:, h:h + 1], inp.lengths)
    errs = [("dQ", orc.slice_rel_err(got[0][:, h:h + 1], ref[0])),
            ("dK", orc.slice_rel_err(got[1][:, h:h + 1], ref[1])),
            ("dV", orc.slice_rel_err(got[2][:, h:h + 1], ref[2])),
            ("dE", _mat_err(got[3][h:h + 1], ref[3])), ("dF", _mat_err(got[4][h:h + 1], ref[4]))]
    G.log("  " + "  ".join(f"{n_} {e:.2e}" for n_, e in errs))
    for name, e in errs:
        assert e <= TOL, (name, e)
    for b, L in enumerate(inp.lengths):   # padded positions: zero gradients, every head
        assert np.all(got[1][b, :, L:] == 0) and np.all(got[2][b, :, L:] == 0)
    Lmax = int(max(inp.lengths))   # no item reaches these positions
    assert np.all(got[3][:, :, Lmax:] == 0) and np.all(got[4][:, :, Lmax:] == 0)
    assert all(np.all(np.isfinite(g)) for g in got)


def test_backward_in_hip_graph():
    """linformer_backward captured once into a HIP graph (split reductions included) and
    replayed for new upstream gradients: every replay equals the eager call bitwise."""
    torch = G.torch_mod()
    B, H, n, k = 2, 2, 1024, 128
    inp = synth.random_inputs(B, H, n, 64, k, BF, NONE, seed=61, lengths=[1024, 640])
    wl = inp.wl
    p = G.prob(wl)
    Q, K, V, E, F = (G.dev(x, wl.dtype) for x in (inp.Q, inp.K, inp.V, inp.E, inp.F))
    lens = G.lengths_dev(inp.lengths)
    dO = G.empty((B, H, n, 64), wl.dtype)
    f32 = lambda shape: torch.empty(shape, dtype=torch.float32, device="cuda")
    outs = [f32((B, H, n, 64)) for _ in range(3)] + [f32(inp.E.shape), f32(inp.F.shape)]
    wsb = L.linformer_backward_workspace_size(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    call = lambda o: L.linformer_backward(p, Q, K, V, E, F, lens, dO, *o, ws, wsb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(outs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(62)
    for _ in range(3):
        dO.copy_(G.dev(synth.to_dtype(rng.standard_normal((B, H, n, 64)), BF), BF))
        ref = [torch.empty_like(o) for o in outs]
        call(ref)
        torch.cuda.synchronize()
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(o, r) for o, r in zip(outs, ref))
