"""GPU parity: liblinformer (through its C ABI) against the float64 oracle on the same seeded
inputs.  Tolerances (per (b, h) slice, max|gpu - ref| / max|ref|): 1e-4 for the fp32 path and
2e-2 for bf16 in / fp32 accumulate, the accuracy bars set for this path.  The bf16 Kbar planes
(bf16 hi plus an e4m3 residual with per-block power-of-two scales) hold Kbar to at most 2^-12 of
each block's largest magnitude (half an e4m3 step of a residual below 2^-8 of it), so Kbar is
held to KBAR_TOL = 3e-4; the bf16 Vbar to its rounding (4e-3).
"""
import numpy as np
import pytest

from efficient_transformer_attention_seq_amd import linformer as L
from efficient_transformer_attention_seq_amd import synth
from oracle import linformer_oracle as orc
from tests import gpu_util as G

pytestmark = pytest.mark.gpu
KBAR_TOL = 3e-4

BF, F32 = synth.DT_BF16, synth.DT_F32
NONE, HEAD, KV, LAYER = (synth.SHARE_NONE, synth.SHARE_HEADWISE, synth.SHARE_KV,
                         synth.SHARE_LAYERWISE)


@pytest.fixture(scope="module", autouse=True)
def _device():
    torch = G.torch_mod()
    if torch.cuda.device_count() < 1:
        pytest.skip("no GPU")
    G.log(f"device: {torch.cuda.get_device_name(0)}")
    yield


def _ref_forward(inp, scale=None, pairs=None):
    return orc.forward(inp.Q, inp.K, inp.V, inp.E, inp.F, inp.wl.share, inp.lengths, scale,
                       pairs=pairs)


def _ref_project(inp):
    _, Kb, Vb = orc.forward(inp.Q, inp.K, inp.V, inp.E, inp.F, inp.wl.share, inp.lengths,
                            return_intermediates=True)
    return Kb, Vb


def _lengths(rng, B, n):
    out = [n] + [int(x) for x in rng.integers(1, n, size=B - 1)] if B > 1 else [n - 17]
    return out


# --------------------------------------------------------------------------- projection
PROJ_CASES = [
    # B, H, n, k, share
    (2, 3, 192, 64, NONE),
    (1, 2, 320, 96, HEAD),
    (2, 2, 256, 256, KV),
    (3, 1, 128, 32, LAYER),
    (1, 3, 512, 128, NONE),
    (2, 2, 448, 160, HEAD),
]


@pytest.mark.parametrize("dtype", [BF, F32])
@pytest.mark.parametrize("case", PROJ_CASES)
def test_project_parity(case, dtype):
    B, H, n, k, share = case
    rng = np.random.default_rng(1000 + n + k)
    lens = _lengths(rng, B, n)
    inp = synth.random_inputs(B, H, n, 64, k, dtype, share, seed=n * 7 + k, lengths=lens)
    G.log(f"project case={case} dtype={dtype} lengths={lens}")
    kb, vb = G.run_project(inp)
    rk, rv = _ref_project(inp)
    ek, ev = orc.slice_rel_err(kb, rk), orc.slice_rel_err(vb, rv)
    G.log(f"  Kbar err {ek:.3e}  Vbar err {ev:.3e}")
    assert ek <= (1e-5 if dtype == F32 else KBAR_TOL)
    assert ev <= (1e-5 if dtype == F32 else 4e-3)


@pytest.mark.parametrize("k,cfg,split", [
    (256, "256x128", 1), (256, "256x256", 2), (256, "128x256w4", 3), (256, "128x256", 5),
    (256, "64x512", 2), (256, "32x512", 1), (128, "128x256", 8), (128, "128x256w4", 2),
    (128, "64x512", 3), (96, "32x512", 2), (192, "64x512", 4), (64, "64x512", 1),
    (128, "128x256", 10), (64, "64x512", 10), (256, "128x128w4", 1), (128, "128x128w4", 3)])
def test_project_tile_configs_and_splits(k, cfg, split):
    """Every tile configuration and split count computes the same thing (fixed-order split
    sums), including tiles whose later steps lie entirely past every length."""
    B, H, n = 3, 2, 640
    lens = [640, 333, 64]
    inp = synth.random_inputs(B, H, n, 64, k, BF, NONE, seed=5 + k, lengths=lens)
    G.log(f"project k={k} cfg={cfg} split={split}")
    with G.env(LINFORMER_PROJ_SPLIT=split, LINFORMER_PROJ_CFG=cfg):
        kb, vb = G.run_project(inp)
    rk, rv = _ref_project(inp)
    ek, ev = orc.slice_rel_err(kb, rk), orc.slice_rel_err(vb, rv)
    G.log(f"  Kbar err {ek:.3e}  Vbar err {ev:.3e}")
    assert ek <= KBAR_TOL
    assert ev <= 4e-3


@pytest.mark.parametrize("split", [2, 5])
def test_project_split_workspace_contents_do_not_matter(split):
    """With a split, the partial sums pass through the workspace; whatever it holds on entry
    (zeros, ones, random bytes, a previous call's partials) the output is bitwise the same, call
    after call."""
    torch = G.torch_mod()
    inp = synth.random_inputs(3, 4, 1024, 64, 128, BF, NONE, seed=21, lengths=[1024, 700, 65])
    wl = inp.wl
    p = G.prob(wl)
    K, V, E, F = (G.dev(x, wl.dtype) for x in (inp.K, inp.V, inp.E, inp.F))
    lens = G.lengths_dev(inp.lengths)
    kbytes, _ = L.linformer_kv_sizes(p)
    outs = []
    with G.env(LINFORMER_PROJ_SPLIT=split):
        wsb = L.linformer_workspace_size(p)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        gen = torch.Generator(device="cuda").manual_seed(3)
        for fill in ("zero", "ones", "random", "again", "again"):
            if fill == "zero":
                ws.zero_()
            elif fill == "ones":
                ws.fill_(255)
            elif fill == "random":
                ws.copy_(torch.randint(0, 256, (wsb,), dtype=torch.uint8, device="cuda",
                                       generator=gen))
            Kbar = torch.empty(kbytes, dtype=torch.uint8, device="cuda")
            Vbar = G.empty((wl.batch, wl.heads, wl.k, wl.d), wl.dtype)
            L.linformer_project_kv(p, K, V, E, F, lens, Kbar, Vbar, ws, wsb)
            torch.cuda.synchronize()
            outs.append((Kbar.cpu().numpy(), G.host(Vbar)))
    G.log(f"split {split}: {len(outs)} calls")
    for kb, vb in outs[1:]:
        assert np.array_equal(kb, outs[0][0]) and np.array_equal(vb, outs[0][1])
    rk, rv = _ref_project(inp)
    _, _, x = G.decode_kbar_bf16(outs[0][0], (wl.batch, wl.heads, wl.k, wl.d))
    assert orc.slice_rel_err(x / G.log2e_scale(wl), rk) <= KBAR_TOL
    assert orc.slice_rel_err(outs[0][1], rv) <= 4e-3


@pytest.mark.parametrize("split", [2, 5])
def test_project_split_other_inputs_on_one_workspace(split):
    """Calls with different inputs, one after another on one workspace, each give bitwise the
    output of a call on a fresh workspace: no call reads partial sums (or, with two splits, the
    in-kernel pairing state) that an earlier call left behind.  Two splits are paired inside the
    projection kernel; five go through the fixup pass."""
    torch = G.torch_mod()
    ins = [synth.random_inputs(3, 4, 1024, 64, 128, BF, NONE, seed=s, lengths=L_)
           for s, L_ in ((31, [1024, 700, 65]), (32, [999, 1024, 300]))]
    wl = ins[0].wl
    p = G.prob(wl)
    kbytes, _ = L.linformer_kv_sizes(p)

    def call(inp, ws, wsb):
        K, V, E, F = (G.dev(x, wl.dtype) for x in (inp.K, inp.V, inp.E, inp.F))
        Kbar = torch.empty(kbytes, dtype=torch.uint8, device="cuda")
        Vbar = G.empty((wl.batch, wl.heads, wl.k, wl.d), wl.dtype)
        L.linformer_project_kv(p, K, V, E, F, G.lengths_dev(inp.lengths), Kbar, Vbar, ws, wsb)
        torch.cuda.synchronize()
        return Kbar.cpu().numpy(), G.host(Vbar)

    with G.env(LINFORMER_PROJ_SPLIT=split):
        wsb = L.linformer_workspace_size(p)
        fresh = []
        for inp in ins:
            ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
            fresh.append(call(inp, ws, wsb))
        shared = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        order = [0, 1, 0, 1, 1, 0]
        G.log(f"split {split}: calls in the order {order} on one workspace")
        for i in order:
            kb, vb = call(ins[i], shared, wsb)
            assert np.array_equal(kb, fresh[i][0]) and np.array_equal(vb, fresh[i][1])
    rk, rv = _ref_project(ins[1])
    _, _, x = G.decode_kbar_bf16(fresh[1][0], (wl.batch, wl.heads, wl.k, wl.d))
    assert orc.slice_rel_err(x / G.log2e_scale(wl), rk) <= KBAR_TOL
    assert orc.slice_rel_err(fresh[1][1], rv) <= 4e-3


@pytest.mark.parametrize("split", [1, 3])
def test_kbar_storage_format(split):
    """The bf16 Kbar bytes follow the documented format, from both the single-split epilogue and
    the split fixup: hi is the bf16 rounding of x = hi + residual (|residual| <= half an ulp of hi,
    plus the e4m3 step), every block's largest residual lies in [128, 256) before its e4m3
    rounding, so its code decodes to [128, 256] (or the block is all zero), and x / c matches the
    oracle's Kbar."""
    inp = synth.random_inputs(2, 2, 256, 64, 128, BF, KV, seed=9, lengths=[256, 200])
    with G.env(LINFORMER_PROJ_SPLIT=split):
        raw, (hi, res, x) = G.run_project_planes(inp)
    ulp = np.abs(hi) * 2.0 ** -7
    assert np.all(np.abs(res) <= 0.5 * ulp * (1 + 2.0 ** -3) + 1e-30)
    B, H, k = 2, 2, 128
    e = B * H * k * 64
    codes = G.e4m3_decode(raw[2 * e:3 * e].reshape(-1, 64)[:, G.LO_PERM]).reshape(-1, 2, 32)
    top = np.abs(codes).max(axis=2)
    assert np.all((top == 0) | ((top >= 128) & (top <= 256)))
    rk, _ = _ref_project(inp)
    c = G.log2e_scale(inp.wl)
    assert orc.slice_rel_err(x / c, rk) <= KBAR_TOL


# ------------------------------------------------------------------------------- attend
ATT_CASES = [
    # B, H, n, k, lengths
    (2, 2, 256, 256, [256, 100]),
    (1, 3, 192, 128, None),
    (1, 1, 64, 32, [1]),
    (2, 1, 320, 96, [0, 319]),
    (1, 2, 576, 160, [500]),
    (1, 1, 1088, 224, [1088]),
]


@pytest.mark.parametrize("dtype", [BF, F32])
@pytest.mark.parametrize("case", ATT_CASES)
def test_attend_parity(case, dtype):
    B, H, n, k, lens = case
    pr = synth.random_projected(B, H, n, 64, k, dtype, seed=n + k)
    wl = synth.Workload("attend", B, H, n, 64, k, dtype, NONE)
    G.log(f"attend case={case} dtype={dtype}")
    out = G.run_attend(pr, wl, lens)
    ref = np.zeros_like(out)
    for b in range(B):
        for h in range(H):
            ref[b, h] = orc.attend(pr.Q[b, h], pr.Kbar[b, h], pr.Vbar[b, h], None,
                                   None if lens is None else lens[b])
    err = orc.slice_rel_err(out, ref)
    G.log(f"  err {err:.3e}")
    assert err <= G.TOL[dtype]


@pytest.mark.parametrize("grid", [8, 16, 64, 256])
def test_attend_persistent_grid_sizes(grid):
    """Work ranges of the persistent attention kernel that start and end inside a head, span
    several heads, or hold no tiles at all, all give the same result."""
    B, H, n, k = 3, 2, 1024, 256
    lens = [700, 1024, 33]
    pr = synth.random_projected(B, H, n, 64, k, BF, seed=3)
    wl = synth.Workload("attend", B, H, n, 64, k, BF, NONE)
    G.log(f"attend grid={grid}")
    with G.env(LINFORMER_ATTEND_GRID=grid):
        out = G.run_attend(pr, wl, lens)
    ref = np.zeros_like(out)
    for b in range(B):
        for h in range(H):
            ref[b, h] = orc.attend(pr.Q[b, h], pr.Kbar[b, h], pr.Vbar[b, h], None, lens[b])
    assert orc.slice_rel_err(out, ref) <= 2e-2
    for b, Lb in enumerate(lens):
        assert np.all(out[b, :, Lb:] == 0.0)


def test_attend_many_batch_items():
    """More than 64 batch items (the length tables are built by the block-wide scan), with empty,
    one-tile and ragged sequences."""
    B, H, n, k = 70, 2, 128, 32
    rng = np.random.default_rng(12)
    lens = [int(x) for x in rng.integers(0, n + 1, size=B)]
    lens[0], lens[1], lens[2] = 0, n, 1
    pr = synth.random_projected(B, H, n, 64, k, BF, seed=13)
    wl = synth.Workload("attend", B, H, n, 64, k, BF, NONE)
    G.log(f"attend B={B}")
    out = G.run_attend(pr, wl, lens)
    ref = np.zeros_like(out)
    for b in range(B):
        for h in range(H):
            ref[b, h] = orc.attend(pr.Q[b, h], pr.Kbar[b, h], pr.Vbar[b, h], None, lens[b])
    assert orc.slice_rel_err(out, ref) <= 2e-2
    for b, Lb in enumerate(lens):
        assert np.all(out[b, :, Lb:] == 0.0)


@pytest.mark.parametrize("kind", ["all_low", "all_high", "late_jump"])
def test_attend_extreme_logits(kind):
    """Logits far outside the reference's starting window: every slot 100+ below it (the first
    block's weights underflow and the reference must move down), 100+ above it (overflow), and a
    later block 60 above the first (the partial sums must be rescaled mid-row)."""
    B, H, n, k = 1, 2, 128, 256
    rng = np.random.default_rng(21)
    Q = synth.to_dtype(np.abs(rng.standard_normal((B, H, n, 64))) + 0.5, BF)
    base = rng.standard_normal((B, H, k, 64))
    if kind == "all_low":
        kbar = base - 12.0
    elif kind == "all_high":
        kbar = base + 12.0
    else:
        kbar = base * 0.5
        kbar[:, :, 128:192] += 9.0
    pr = synth.Projected(Q, synth.round_f32(kbar), synth.to_dtype(rng.standard_normal((B, H, k, 64)), BF))
    wl = synth.Workload("attend", B, H, n, 64, k, BF, NONE)
    out = G.run_attend(pr, wl, None)
    ref = np.zeros_like(out)
    for h in range(H):
        ref[0, h] = orc.attend(pr.Q[0, h], pr.Kbar[0, h], pr.Vbar[0, h])
    err = orc.slice_rel_err(out, ref)
    G.log(f"  extreme logits {kind}: err {err:.3e}")
    assert np.all(np.isfinite(out)) and err <= 2e-2


@pytest.mark.parametrize("kind", ["large", "mixed_blocks", "mixed_queries"])
def test_forward_query_magnitudes_beyond_e4m3(kind):
    """Queries far outside e4m3's range (largest finite value 448), where the residual product
    takes Q: every element scaled up to |q| of 1e3-1e4 (keys scaled down by the same factor so
    the logits stay moderate); the two 32-column blocks of every query at 4000x and 1/512x (each
    block of the keys scaled inversely, so both blocks carry the logits); alternate queries of
    every tile at 8000x and 1e-3x (keys at 1/8000x, so the small queries' softmax is near
    uniform).  Every result must be finite and within the bf16 bar."""
    B, H, n, k = 2, 2, 256, 128
    inp = synth.random_inputs(B, H, n, 64, k, BF, NONE, seed=77, lengths=[256, 161])
    Q, K = inp.Q.astype(np.float64), inp.K.astype(np.float64)
    if kind == "large":
        Q, K = Q * 3000.0, K / 3000.0
    elif kind == "mixed_blocks":
        Q[..., :32] *= 4000.0
        Q[..., 32:] /= 512.0
        K[..., :32] /= 4000.0
        K[..., 32:] *= 512.0
    else:
        Q[:, :, 0::2] *= 8000.0
        Q[:, :, 1::2] *= 1e-3
        K = K / 8000.0
    inp = synth.Inputs(inp.wl, synth.to_dtype(Q, BF), synth.to_dtype(K, BF), inp.V, inp.E,
                       inp.F, inp.lengths)
    G.log(f"forward query magnitudes {kind}: max|q| {np.abs(inp.Q).max():.3e}")
    out, ok = G.run_forward(inp, guard=True)
    err = orc.slice_rel_err(out, _ref_forward(inp))
    G.log(f"  err {err:.3e}")
    assert ok and np.all(np.isfinite(out))
    assert err <= G.TOL[BF]


def test_attend_explicit_scale():
    B, H, n, k = 1, 1, 128, 64
    pr = synth.random_projected(B, H, n, 64, k, BF, seed=4, kbar_std=1.0)
    wl = synth.Workload("attend", B, H, n, 64, k, BF, NONE)
    out = G.run_attend(pr, wl, None, scale=0.3)
    ref = orc.attend(pr.Q[0, 0], pr.Kbar[0, 0], pr.Vbar[0, 0], 0.3)
    assert orc.slice_rel_err(out[0, 0][None, None], ref[None, None]) <= 2e-2


# ------------------------------------------------------------------------------ forward
FWD_CASES = [
    (2, 3, 384, 128, NONE),
    (2, 2, 256, 256, HEAD),
    (3, 2, 320, 64, KV),
    (1, 4, 640, 96, LAYER),
]


@pytest.mark.parametrize("dtype", [BF, F32])
@pytest.mark.parametrize("case", FWD_CASES)
def test_forward_parity_small(case, dtype):
    B, H, n, k, share = case
    rng = np.random.default_rng(n + B)
    lens = _lengths(rng, B, n)
    inp = synth.random_inputs(B, H, n, 64, k, dtype, share, seed=11 + n, lengths=lens)
    G.log(f"forward case={case} dtype={dtype} lengths={lens}")
    out, ok = G.run_forward(inp, guard=True)
    err = orc.slice_rel_err(out, _ref_forward(inp))
    G.log(f"  err {err:.3e}")
    assert ok, "write outside the output tensor"
    assert err <= G.TOL[dtype]


def _random_case(seed):
    """A seeded shape drawn over the supported space: batch and heads 1-4, n a multiple of 64 up
    to 1536, k a multiple of 32 up to 256 (128 or 256, the one-launch kernel's, drawn more
    often), any sharing mode, bf16 (three in four) or fp32, lengths drawn from 1, n - 1, n and
    random values, with one item of every multi-item batch empty."""
    rng = np.random.default_rng(7000 + seed)
    B, H = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    n = 64 * int(rng.integers(1, 25))
    k = 32 * int(rng.integers(1, 9)) if rng.random() < 0.6 else int(rng.choice([128, 256]))
    share = [NONE, HEAD, KV, LAYER][int(rng.integers(0, 4))]
    dtype = F32 if rng.random() < 0.25 else BF
    pool = [1, n, n - 1, int(rng.integers(1, n + 1)), int(rng.integers(1, n + 1))]
    lens = [pool[int(rng.integers(0, len(pool)))] for _ in range(B)]
    if B > 1:
        lens[int(rng.integers(0, B))] = 0
    return B, H, n, k, share, dtype, lens


@pytest.mark.parametrize("seed", range(16))
def test_forward_random_shapes(seed):
    """Seeded shapes across the whole supported space (both paths: the one-launch short-sequence
    kernel where it applies, projection + attention elsewhere), in full against the oracle, with
    guard bands around the output."""
    B, H, n, k, share, dtype, lens = _random_case(seed)
    inp = synth.random_inputs(B, H, n, 64, k, dtype, share, seed=900 + seed, lengths=lens)
    G.log(f"random forward seed={seed} B={B} H={H} n={n} k={k} share={share} dtype={dtype} "
          f"lengths={lens}")
    out, ok = G.run_forward(inp, guard=True)
    err = _sampled_err_one_token_aware(out, inp, [(b, h) for b in range(B) for h in range(H)])
    G.log(f"  err {err:.3e}")
    assert ok, "write outside the output tensor"
    assert err <= G.TOL[dtype]


def test_forward_single_head_f32_full():
    """Single-head fp32 workload: B1 H1 n512 k128, separate E, F, seed 0 (full comparison)."""
    inp = synth.make_inputs(synth.C1)
    G.log("forward C1 full")
    out, ok = G.run_forward(inp, guard=True)
    err = orc.slice_rel_err(out, _ref_forward(inp))
    G.log(f"  err {err:.3e}")
    assert ok and err <= 1e-4


def test_forward_roberta_kv_full():
    """RoBERTa-base shape, one key-value matrix: B32 H12 n512 k256 bf16 (full comparison)."""
    inp = synth.make_inputs(synth.C2)
    G.log("forward C2 full")
    out, ok = G.run_forward(inp, guard=True)
    err = orc.slice_rel_err(out, _ref_forward(inp))
    G.log(f"  err {err:.3e}")
    assert ok and err <= 2e-2


def _sampled(inp, pairs, guard=False):
    out, ok = G.run_forward(inp, guard=guard)
    ref = _ref_forward(inp, pairs=pairs)
    idx = tuple(np.array(pairs).T)
    return orc.slice_rel_err(out[idx], ref[idx]), ok, out


def test_forward_long_padded_sampled():
    """B8 H12 n4096 k256 unshared, padded lengths in [2048, 4096]: the benchmarked launch,
    checked on sampled (b, h) slices plus zero rows past every length."""
    inp = synth.make_inputs(synth.C3)
    G.log(f"forward C3 lengths={inp.lengths.tolist()}")
    pairs = [(0, 0), (1, 5), (3, 11), (5, 2), (7, 7), (int(np.argmin(inp.lengths)), 4)]
    err, ok, out = _sampled(inp, pairs, guard=True)
    G.log(f"  err {err:.3e}")
    assert ok and err <= 2e-2
    for b, Lb in enumerate(inp.lengths):
        assert np.all(out[b, :, Lb:] == 0.0)
    assert np.all(np.isfinite(out))


def test_forward_extreme_length_sampled():
    """B1 H12 n65536 k128 layerwise E = F: sampled heads."""
    inp = synth.make_inputs(synth.C4)
    G.log("forward C4")
    err, ok, out = _sampled(inp, [(0, 0), (0, 6), (0, 11)])
    G.log(f"  err {err:.3e}")
    assert err <= 2e-2 and np.all(np.isfinite(out))


def test_forward_stack_layer_sampled():
    """Attention part of the 12-layer stack: B16 H12 n1024 k256 layerwise E = F."""
    inp = synth.make_inputs(synth.C5A)
    G.log("forward C5A")
    err, ok, _ = _sampled(inp, [(0, 0), (7, 3), (15, 11)])
    G.log(f"  err {err:.3e}")
    assert err <= 2e-2


# --------------------------------------------------------------------------- edge cases
@pytest.mark.parametrize("lens", [[0, 0], [1, 64], [64, 63], [33, 0]])
def test_forward_edge_lengths(lens):
    inp = synth.random_inputs(2, 2, 64, 64, 32, BF, NONE, seed=21, lengths=lens)
    G.log(f"edge lengths {lens}")
    out, ok = G.run_forward(inp, guard=True)
    ref = _ref_forward(inp)
    assert ok
    assert orc.slice_rel_err(out, ref) <= 2e-2
    for b, Lb in enumerate(lens):
        assert np.all(out[b, :, Lb:] == 0.0)


@pytest.mark.parametrize("k", [128, 256])
def test_forward_tile_edge_lengths_with_guard(k):
    """Lengths one below, at and one above a 32-query tile edge and inside a later tile, at the
    production tile shapes: the attention moves Q and O as whole 32-row tiles, so rows past a
    length inside the last tile must come out zero and nothing outside O may be written."""
    lens = [31, 32, 33, 95]
    inp = synth.random_inputs(4, 3, 256, 64, k, BF, NONE, seed=41 + k, lengths=lens)
    G.log(f"tile-edge lengths {lens}, k {k}")
    out, ok = G.run_forward(inp, guard=True)
    ref = _ref_forward(inp)
    assert ok
    assert orc.slice_rel_err(out, ref) <= 2e-2
    for b, Lb in enumerate(lens):
        assert np.all(out[b, :, Lb:] == 0.0)


# The fused short-sequence path (one launch: projection into LDS, then attention) serves bf16
# forwards with n <= 1024, k of 128 or 256 and one matrix for keys and values (key-value and
# layerwise sharing, per-head E_h with F omitted).  Lengths of one valid position are left out:
# with k >= 128 such a row's output is a near-uniform average of k rank-one Vbar rows that
# cancels to a small value, and the bf16 weights alone put it near the bar (a float64 emulation
# of the rounding gives 2.0e-2 at k = 128 and 0.26 at k = 256); lengths of 7 and 17 take the
# same single-step, single-tile branches.
FUSED_CASES = [
    # B, H, n, k, share, lengths
    (3, 2, 512, 256, KV, [512, 0, 257]),
    (2, 3, 1024, 128, LAYER, [1024, 95]),
    (2, 2, 64, 128, NONE, [64, 17]),
    (1, 5, 960, 256, KV, None),
    (4, 2, 128, 256, LAYER, [7, 33, 0, 128]),
    (2, 2, 768, 128, NONE, [31, 700]),
]


@pytest.mark.parametrize("case", FUSED_CASES)
def test_forward_fused_parity(case):
    B, H, n, k, share, lens = case
    inp = synth.random_inputs(B, H, n, 64, k, BF, share, seed=13 + n + k, lengths=lens)
    if share == NONE:   # one matrix per head for keys and values: F omitted
        inp = synth.Inputs(inp.wl, inp.Q, inp.K, inp.V, inp.E, None, inp.lengths)
    G.log(f"fused forward case={case}")
    out, ok = G.run_forward(inp, guard=True)
    err = orc.slice_rel_err(out, _ref_forward(inp))
    G.log(f"  err {err:.3e}")
    assert ok, "write outside the output tensor"
    assert err <= G.TOL[BF]
    if lens is not None:
        for b, Lb in enumerate(lens):
            assert np.all(out[b, :, Lb:] == 0.0)
    # the two-launch path (projection to HBM, then attention) on the same inputs
    with G.env(LINFORMER_FUSED=0):
        out2, _ = G.run_forward(inp)
    G.log(f"  fused vs two-launch: bitwise equal {np.array_equal(out, out2)}, "
          f"max slice diff {orc.slice_rel_err(out, out2):.3e}")
    assert orc.slice_rel_err(out, out2) <= 1e-2


@pytest.mark.parametrize("case", [FUSED_CASES[0], FUSED_CASES[1], FUSED_CASES[4],
                                  (3, 3, 1024, 256, LAYER, [1024, 40, 990])])
def test_forward_fused_work_split_is_bitwise_the_same(case):
    """The fused kernel's work split (the units of a last, partial round taken by several
    workgroups, each projecting the unit and attending a share of its tiles; the small problems
    here are all one partial round) writes bitwise what one workgroup per unit writes,
    including rows past the lengths and units whose shares hold no tile."""
    B, H, n, k, share, lens = case
    inp = synth.random_inputs(B, H, n, 64, k, BF, share, seed=17 + n + k, lengths=lens)
    G.log(f"fused work split case={case}")
    out, ok = G.run_forward(inp, guard=True)
    assert ok, "write outside the output tensor"
    with G.env(LINFORMER_FUSED_SPLIT=0):
        ref, _ = G.run_forward(inp)
    assert np.array_equal(out, ref)
    assert orc.slice_rel_err(out, _ref_forward(inp)) <= G.TOL[BF]


def _sampled_err_one_token_aware(out, inp, pairs):
    """Per-slice error against the oracle on the listed (b, h) slices; the slices of one-token
    items are measured against the weighted magnitude of the projected values their outputs
    average (max of P |Vbar|), not against their own largest value: with one token every
    projected key and value is a multiple of that token's, so each output row is one weighted sum
    of the E (F) entries times the token's value row, which can cancel far below its terms while
    the bf16 weights and values carry 2^-9 of the terms."""
    ref, Kb, Vb = orc.forward(inp.Q, inp.K, inp.V, inp.E, inp.F, inp.wl.share, inp.lengths,
                              pairs=pairs, return_intermediates=True)
    worst = 0.0
    for b, h in pairs:
        Lb = int(inp.lengths[b])
        if Lb != 1:
            worst = max(worst, orc.slice_rel_err(out[b, h], ref[b, h]))
            continue
        W = orc.attention_weights(inp.Q[b, h][:1], Kb[b, h], 1.0 / np.sqrt(inp.wl.d))
        terms = float(np.max(W @ np.abs(Vb[b, h])))
        worst = max(worst, float(np.abs(out[b, h] - ref[b, h]).max()) / max(terms, 1e-300))
    return worst


@pytest.mark.parametrize("B,H,n,k,share,seed", [
    (24, 12, 256, 256, KV, 1),      # 288 (b, h) units: 32 extra units handed off
    (32, 12, 512, 128, LAYER, 2),   # 384: the most the hand-off takes, 128 extra units
])
def test_forward_fused_handoff_is_bitwise_the_same(B, H, n, k, share, seed):
    """With more (b, h) units than compute units (up to one and a half times as many), each extra
    unit is projected by one workgroup, published in the workspace and attended by its
    neighbour.  The output equals bitwise the one without the hand-off, on a fresh workspace and
    on one an earlier call with other inputs left its planes and flags in (the flags carry a
    per-call tag), and the oracle on sampled slices (items of every length class, every head)."""
    torch = G.torch_mod()
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(0, n + 1, size=B)]
    lens[0], lens[1], lens[2] = n, 0, 1
    ins = [synth.random_inputs(B, H, n, 64, k, BF, share, seed=40 + seed + i, lengths=lens)
           for i in range(2)]
    G.log(f"fused hand-off B={B} H={H} n={n} k={k} share={share}")
    wl = ins[0].wl
    p = G.prob(wl)
    wsb = L.linformer_workspace_size(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    outs = []
    for inp in ins:   # one workspace, two calls
        Q, K, V, E = (G.dev(x, BF) for x in (inp.Q, inp.K, inp.V, inp.E))
        buf, O = G.guarded((B, H, n, 64), BF)
        L.linformer_forward(p, Q, K, V, E, None, G.lengths_dev(inp.lengths), O, ws, wsb)
        torch.cuda.synchronize()
        assert G.guards_intact(buf), "write outside the output tensor"
        outs.append(G.host(O))
    for inp, out in zip(ins, outs):
        with G.env(LINFORMER_FUSED_HANDOFF=0):
            ref, _ = G.run_forward(inp)
        assert np.array_equal(out, ref)
    pairs = [(b, h) for b in (0, 1, 2, B - 1) for h in range(H)]
    err = _sampled_err_one_token_aware(outs[1], ins[1], pairs)
    G.log(f"  sampled err {err:.3e}")
    assert err <= G.TOL[BF]


def test_forward_without_lengths_equals_full_lengths():
    inp = synth.random_inputs(2, 2, 256, 64, 128, BF, KV, seed=22)
    a, _ = G.run_forward(inp)
    inp2 = synth.random_inputs(2, 2, 256, 64, 128, BF, KV, seed=22, lengths=[256, 256])
    b, _ = G.run_forward(inp2)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("split,k", [(1, 128), (2, 256), (3, 128), (6, 96)])
def test_forward_equals_project_then_attend(split, k):
    """linformer_forward gives bitwise the output of linformer_project_kv followed by
    linformer_attend, with and without a split projection."""
    torch = G.torch_mod()
    inp = synth.random_inputs(2, 3, 768, 64, k, BF, NONE, seed=31 + k, lengths=[768, 301])
    wl = inp.wl
    p = G.prob(wl)
    Q, K, V, E, F = (G.dev(x, wl.dtype) for x in (inp.Q, inp.K, inp.V, inp.E, inp.F))
    lens = G.lengths_dev(inp.lengths)
    with G.env(LINFORMER_PROJ_SPLIT=split):
        wsb = L.linformer_workspace_size(p)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        O1 = G.empty((wl.batch, wl.heads, wl.n, wl.d), wl.dtype)
        L.linformer_forward(p, Q, K, V, E, F, lens, O1, ws, wsb)
        kbytes, _ = L.linformer_kv_sizes(p)
        Kbar = torch.empty(kbytes, dtype=torch.uint8, device="cuda")
        Vbar = G.empty((wl.batch, wl.heads, wl.k, wl.d), wl.dtype)
        O2 = G.empty((wl.batch, wl.heads, wl.n, wl.d), wl.dtype)
        L.linformer_project_kv(p, K, V, E, F, lens, Kbar, Vbar, ws, wsb)
        L.linformer_attend(p, Q, Kbar, Vbar, lens, O2)
    torch.cuda.synchronize()
    G.log(f"forward vs project + attend, split {split} k {k}")
    assert torch.equal(O1, O2)


def test_forward_is_deterministic():
    inp = synth.random_inputs(2, 3, 1024, 64, 256, BF, NONE, seed=23, lengths=[1000, 517])
    a, _ = G.run_forward(inp)
    b, _ = G.run_forward(inp)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- pins checked on the GPU
@pytest.mark.parametrize("n", [64, 128, 256])
def test_identity_projection_equals_dense(n):
    """k = n, E = F = I: Linformer is standard softmax attention (both GPU paths, vs oracle)."""
    rng = np.random.default_rng(n)
    B, H = 1, 2
    Q = synth.to_dtype(rng.standard_normal((B, H, n, 64)), BF)
    K = synth.to_dtype(rng.standard_normal((B, H, n, 64)), BF)
    V = synth.to_dtype(rng.standard_normal((B, H, n, 64)), BF)
    E = np.eye(n, dtype=np.float32)[None]
    wl = synth.Workload("identity", B, H, n, 64, n, BF, KV)
    inp = synth.Inputs(wl, Q, K, V, E, None, None)
    out, _ = G.run_forward(inp)
    dense = G.run_dense(inp)
    ref = orc.dense_forward(Q, K, V)
    assert orc.slice_rel_err(out, ref) <= 2e-2
    assert orc.slice_rel_err(dense, ref) <= 2e-2


def test_identical_rows_closed_form():
    """All rows of E equal: every output row is the mean of the projected values."""
    rng = np.random.default_rng(5)
    B, H, n, k = 1, 2, 256, 128
    Q = synth.to_dtype(rng.standard_normal((B, H, n, 64)), BF)
    K = synth.to_dtype(rng.standard_normal((B, H, n, 64)), BF)
    V = synth.to_dtype(rng.standard_normal((B, H, n, 64)), BF)
    row = synth.to_dtype(rng.standard_normal((1, 1, n)) / np.sqrt(k), BF)
    E = np.repeat(row, k, axis=1)
    F = synth.to_dtype(rng.standard_normal((1, k, n)) / np.sqrt(k), BF)
    wl = synth.Workload("rows", B, H, n, 64, k, BF, HEAD)
    out, _ = G.run_forward(synth.Inputs(wl, Q, K, V, E, F, None))
    for h in range(H):
        want = (F[0].astype(np.float64).sum(axis=0) @ V[0, h].astype(np.float64)) / k
        got = out[0, h]
        assert np.max(np.abs(got - want[None, :])) <= 2e-2 * np.max(np.abs(want))


# ------------------------------------------------------------------ dense comparator
@pytest.mark.parametrize("case", [(1, 2, 256, None), (2, 1, 1024, [1024, 333]),
                                  (1, 1, 64, [1])])
def test_dense_parity(case):
    B, H, n, lens = case
    inp = synth.random_inputs(B, H, n, 64, 32, BF, NONE, seed=n, lengths=lens)
    G.log(f"dense case={case}")
    out = G.run_dense(inp)
    ref = orc.dense_forward(inp.Q, inp.K, inp.V, lens)
    err = orc.slice_rel_err(out, ref)
    G.log(f"  err {err:.3e}")
    assert err <= 2e-2


# ------------------------------------------------------------------- error paths on GPU
def test_error_paths_on_device():
    torch = G.torch_mod()
    wl = synth.Workload("err", 1, 1, 128, 64, 64, BF, NONE)
    p = G.prob(wl)
    x = torch.zeros(2 * 128 * 64 + 64, dtype=torch.bfloat16, device="cuda")
    Q = x[:128 * 64]
    O = torch.zeros(128 * 64, dtype=torch.bfloat16, device="cuda")
    K = torch.zeros(128 * 64, dtype=torch.bfloat16, device="cuda")
    E = torch.zeros(64 * 128, dtype=torch.bfloat16, device="cuda")
    wsb = L.linformer_workspace_size(p)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    # misaligned output
    assert L.linformer_forward(p, Q, K, K, E, None, None, x[1:].data_ptr(), ws, wsb,
                               check=False) == 6
    # output aliases an input
    assert L.linformer_forward(p, Q, K, K, E, None, None, Q, ws, wsb, check=False) == 7
    # workspace too small
    assert L.linformer_forward(p, Q, K, K, E, None, None, O, ws, wsb - 1,
                               check=False) == 5
    # key-value sharing with a distinct F
    p2 = G.prob(wl.with_(share=KV))
    assert L.linformer_forward(p2, Q, K, K, E, O, None, O, ws, wsb, check=False) == 4
    # valid call succeeds
    assert L.linformer_forward(p, Q, K, K, E, None, None, O, ws, wsb, check=False) == 0
    torch.cuda.synchronize()


def test_forward_fused_handoff_in_hip_graph():
    """The hand-off captured in a HIP graph: replays carry the tag of the captured call, so each
    consumer clears its flag once it has read the planes.  Replays back to back on one workspace,
    each with new inputs copied into the captured buffers, equal the eager results bitwise."""
    torch = G.torch_mod()
    B, H, n, k = 24, 12, 256, 256   # 288 (b, h) units: 32 of them handed off
    lens = [256, 200, 77, 256] * 6
    inputs = [synth.random_inputs(B, H, n, 64, k, BF, KV, seed=60 + i, lengths=lens)
              for i in range(3)]
    wl = inputs[0].wl
    p = G.prob(wl)
    shp = (B, H, n, 64)
    Q, K, V = (G.empty(shp, BF) for _ in range(3))
    E = G.dev(inputs[0].E, BF)
    lensd = G.lengths_dev(lens)
    O = G.empty(shp, BF)
    wsb = L.linformer_workspace_size(p)
    ws, ws2 = (torch.empty(wsb, dtype=torch.uint8, device="cuda") for _ in range(2))

    def load(inp):
        Q.copy_(G.dev(inp.Q, BF))
        K.copy_(G.dev(inp.K, BF))
        V.copy_(G.dev(inp.V, BF))

    refs = []
    for inp in inputs:   # eager results, on another workspace
        load(inp)
        ref = G.empty(shp, BF)
        L.linformer_forward(p, Q, K, V, E, None, lensd, ref, ws2, wsb)
        torch.cuda.synchronize()
        refs.append(ref)
    load(inputs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm up on the capture stream
        L.linformer_forward(p, Q, K, V, E, None, lensd, O, ws, wsb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.linformer_forward(p, Q, K, V, E, None, lensd, O, ws, wsb)
    torch.cuda.synchronize()
    for rep in range(2):
        for inp, ref in zip(inputs, refs):
            load(inp)
            O.fill_(7.0)
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(O, ref), rep
    G.log("hand-off graph replays equal the eager calls")


def test_forward_in_hip_graph():
    """linformer_forward captured once into a HIP graph and replayed: every replay, with new
    inputs copied into the captured buffers and eager work between replays, equals the eager
    call bitwise (the library enqueues kernels only: no allocation, no memset, no host sync)."""
    torch = G.torch_mod()
    wl0 = synth.random_inputs(2, 3, 1024, 64, 128, BF, NONE, seed=41, lengths=[1024, 555])
    wl = wl0.wl
    p = G.prob(wl)
    shp = (wl.batch, wl.heads, wl.n, wl.d)
    Q, K, V = (G.empty(shp, wl.dtype) for _ in range(3))
    E, F = G.dev(wl0.E, wl.dtype), G.dev(wl0.F, wl.dtype)
    lens = G.lengths_dev(wl0.lengths)
    O = G.empty(shp, wl.dtype)
    wsb = L.linformer_workspace_size(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    inputs = [synth.random_inputs(2, 3, 1024, 64, 128, BF, NONE, seed=50 + i, lengths=[1024, 555])
              for i in range(3)]

    def load(inp):
        Q.copy_(G.dev(inp.Q, wl.dtype))
        K.copy_(G.dev(inp.K, wl.dtype))
        V.copy_(G.dev(inp.V, wl.dtype))

    load(inputs[0])
    torch.cuda.synchronize()
    with G.env(LINFORMER_PROJ_SPLIT=2):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):   # warm up on the capture stream
            L.linformer_forward(p, Q, K, V, E, F, lens, O, ws, wsb)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            L.linformer_forward(p, Q, K, V, E, F, lens, O, ws, wsb)
        torch.cuda.synchronize()
        for inp in inputs:
            load(inp)
            ref = G.empty(shp, wl.dtype)
            L.linformer_forward(p, Q, K, V, E, F, lens, ref, ws, wsb)   # eager
            torch.cuda.synchronize()
            O.fill_(7.0)
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(O, ref)
    G.log("graph replays equal the eager calls")
