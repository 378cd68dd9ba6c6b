"""GPU parity of the encoder attention stack (linformer_stack_forward) against the float64
oracle: per layer (the oracle's layer applied to the exact bf16 input the GPU layer read) and end
to end.  Metric: per batch item, max|gpu - ref| / max|ref| over the [n, d_model] output.

Both bars are the bf16 accuracy bar, 2e-2.  Per layer the error comes from that layer's own bf16
roundings (queries, keys, values, Vbar, weights, attention output, layer output: about 2^-9
relative each).  End to end it also carries every earlier layer's error through the later
layers, whose amplification grows with the logit spread (it depends on the weights' scale, not
on the implementation): the synthetic cases use weights of standard deviation 0.5 / sqrt(d_model),
the 12-layer workload its own 0.02.
"""
import numpy as np
import pytest

from efficient_transformer_attention_seq_amd import linformer as L
from efficient_transformer_attention_seq_amd import synth
from oracle import linformer_oracle as orc
from tests import gpu_util as G

pytestmark = pytest.mark.gpu
LAYER_TOL = 2e-2


END_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _device():
    torch = G.torch_mod()
    if torch.cuda.device_count() < 1:
        pytest.skip("no GPU")
    yield


def _check_layers(si, Y, items=None):
    """Per-layer parity on the listed batch items (all by default); returns the worst error."""
    wl = si.wl
    items = list(range(wl.batch)) if items is None else list(items)
    lens = None if si.lengths is None else [int(si.lengths[b]) for b in items]
    worst = 0.0
    x = si.X[items].astype(np.float64)
    for l in range(wl.layers):
        ref = orc.stack_layer(x, si.Wqkv[l], si.Wo[l], si.E, wl.heads, lens)
        err = orc.slice_rel_err(Y[l][items], ref)
        G.log(f"  layer {l}: err {err:.3e}")
        assert err <= LAYER_TOL, (l, err)
        worst = max(worst, err)
        x = Y[l][items]
    return worst


def _stack_wl(batch, n, d_model, k, layers, w_std=None, seed=1):
    heads = d_model // 64
    ws = (0.5 / np.sqrt(d_model)) if w_std is None else w_std
    return synth.StackWorkload(f"stack_b{batch}n{n}d{d_model}k{k}l{layers}", batch, n, d_model,
                               heads, k, layers, w_std=ws, seed=seed)


@pytest.mark.parametrize("batch,n,d_model,k,layers", [
    (2, 256, 384, 64, 2),     # 6 heads, two feature tiles of the output map
    (1, 512, 768, 128, 1),    # 12 feature tiles (queries | keys | values), 2 token tiles
    (4, 128, 192, 32, 3),     # token tiles spanning batch items, three layers
])
def test_stack_parity(batch, n, d_model, k, layers):
    wl = _stack_wl(batch, n, d_model, k, layers)
    G.log(f"stack {wl.name}")
    si = synth.make_stack_inputs(wl)
    Y, ok = G.run_stack(si, keep_layers=True, guard=True)
    assert ok, "stray writes outside Y"
    assert np.all(np.isfinite(Y))
    _check_layers(si, Y)
    ref = orc.stack_forward(si.X, si.Wqkv, si.Wo, si.E, wl.heads)
    err = orc.slice_rel_err(Y[-1], ref)
    G.log(f"  end to end: err {err:.3e}")
    assert err <= END_TOL


# The stack form of the fused kernel (projected keys and values of each (b, h) computed into LDS
# from the layer's projected input and W_K, W_V, then the attention, in one launch) serves k of 128
# or 256; forced here on small shapes, with padding, and compared with the two-launch path (the
# projected-key GEMM, then the attention kernel).
@pytest.mark.parametrize("batch,n,d_model,k,layers,lens", [
    (2, 256, 384, 128, 2, None),
    (1, 512, 768, 256, 2, None),
    (3, 320, 192, 128, 2, [320, 77, 1]),
])
def test_stack_fused_parity(batch, n, d_model, k, layers, lens):
    wl = _stack_wl(batch, n, d_model, k, layers, seed=5)
    G.log(f"stack fused {wl.name} lengths {lens}")
    si = synth.make_stack_inputs(wl, lengths=lens)
    with G.env(LINFORMER_FUSED="force"):
        Y, ok = G.run_stack(si, keep_layers=True, guard=True)
    assert ok, "stray writes outside Y"
    assert np.all(np.isfinite(Y))
    _check_layers(si, Y)
    if lens is not None:
        for l in range(wl.layers):
            for b, Lb in enumerate(lens):
                assert np.all(Y[l][b, Lb:] == 0.0)
    with G.env(LINFORMER_FUSED=0):
        Y2, _ = G.run_stack(si, keep_layers=True)
    diff = orc.slice_rel_err(Y[-1], Y2[-1])
    G.log(f"  fused vs two-launch, last layer: {diff:.3e}")
    assert diff <= 1e-2


def _random_stack_case(seed):
    """A seeded shape: batch 1-3, n a multiple of 64 up to 512, d_model of 192 or 384 (whole
    192-feature tiles of the output map), k a multiple of 32 up to 256, one to three layers, and
    lengths from 1 to n (or none)."""
    rng = np.random.default_rng(9300 + seed)
    batch = int(rng.integers(1, 4))
    n = 64 * int(rng.integers(1, 9))
    d_model = int(rng.choice([192, 384]))
    k = 32 * int(rng.integers(1, 9))
    layers = int(rng.integers(1, 4))
    lens = None if rng.random() < 0.3 else [int(x) for x in rng.integers(1, n + 1, size=batch)]
    return batch, n, d_model, k, layers, lens


@pytest.mark.parametrize("seed", range(6))
def test_stack_random_shapes(seed):
    batch, n, d_model, k, layers, lens = _random_stack_case(seed)
    wl = _stack_wl(batch, n, d_model, k, layers, seed=20 + seed)
    G.log(f"stack random {wl.name} lengths {lens}")
    si = synth.make_stack_inputs(wl, lengths=lens)
    Y, ok = G.run_stack(si, keep_layers=True, guard=True)
    assert ok, "stray writes outside Y"
    assert np.all(np.isfinite(Y))
    _check_layers(si, Y)
    if lens is not None:
        for l in range(layers):
            for b, Lb in enumerate(lens):
                assert np.all(Y[l][b, Lb:] == 0.0)


def test_stack_last_layer_only_matches_kept():
    wl = _stack_wl(2, 256, 384, 64, 3)
    si = synth.make_stack_inputs(wl)
    Yk, _ = G.run_stack(si, keep_layers=True)
    Y1, ok = G.run_stack(si, keep_layers=False, guard=True)
    assert ok
    assert np.array_equal(Y1, Yk[-1])


def test_stack_padding():
    wl = _stack_wl(2, 256, 384, 64, 2, seed=3)
    si = synth.make_stack_inputs(wl, lengths=[200, 77])
    Y, ok = G.run_stack(si, keep_layers=True, guard=True)
    assert ok
    for l in range(wl.layers):
        assert np.all(Y[l][0, 200:] == 0.0) and np.all(Y[l][1, 77:] == 0.0)
    _check_layers(si, Y)


def test_stack_full_size_sampled():
    """The 12-layer d_model 768 stack at batch 16, n 1024, k 256 (the workload the benchmark
    times), checked per layer and end to end on two batch items."""
    wl = synth.C5
    G.log(f"stack {wl.name}")
    si = synth.make_stack_inputs(wl)
    Y, _ = G.run_stack(si, keep_layers=True)
    assert np.all(np.isfinite(Y))
    items = [0, wl.batch - 1]
    _check_layers(si, Y, items)
    ref = orc.stack_forward(si.X[items], si.Wqkv, si.Wo, si.E, wl.heads)
    err = orc.slice_rel_err(Y[-1][items], ref)
    G.log(f"  end to end: err {err:.3e}")
    assert err <= END_TOL


def test_stack_in_hip_graph():
    """linformer_stack_forward captured once into a HIP graph and replayed for new inputs:
    every replay equals the eager call bitwise."""
    torch = G.torch_mod()
    wl = synth.StackWorkload("graph_stack", 2, 512, 384, 6, 128, 2, 0.5 / np.sqrt(384), False, 7)
    si = synth.make_stack_inputs(wl)
    s = L.stack(wl.batch, wl.n, wl.d_model, wl.heads, wl.k, wl.layers)
    BF = synth.DT_BF16
    X = G.empty((wl.batch, wl.n, wl.d_model), BF)
    Wq, Wo, E = G.dev(si.Wqkv, BF), G.dev(si.Wo, BF), G.dev(si.E, BF)
    Y = G.empty((wl.batch, wl.n, wl.d_model), BF)
    wsb = L.linformer_stack_workspace_size(s)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    call = lambda out: L.linformer_stack_forward(s, X, Wq, Wo, E, None, out, ws, wsb)
    X.copy_(G.dev(si.X, BF))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(Y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(Y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    for _ in range(3):
        X.copy_(G.dev(synth.to_dtype(rng.standard_normal(X.shape), BF), BF))
        ref = torch.empty_like(Y)
        call(ref)
        torch.cuda.synchronize()
        Y.fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref)
