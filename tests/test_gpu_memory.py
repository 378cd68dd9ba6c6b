"""The library allocates no device memory of its own: every buffer is the caller's (inputs,
outputs, workspace), so warmed-up calls leave the device's free memory (hipMemGetInfo, through
torch.cuda.mem_get_info) unchanged, for the forward, the no-allocation forward (whose fixed
scratch array is part of the loaded library, present from the first call on), the backward, the
encoder stack and the dense comparator.  This is the measured half of the memory comparison with
standard attention (Linformer 요약 설명, section "Inference-time Efficiency Results": the largest
batch that fits)."""
import numpy as np
import pytest

from efficient_transformer_attention_seq_amd import linformer as L
from efficient_transformer_attention_seq_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _delta(torch, fn, warm=2, calls=3):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    f0, _ = torch.cuda.mem_get_info()
    for _ in range(calls):
        fn()
    torch.cuda.synchronize()
    f1, _ = torch.cuda.mem_get_info()
    return int(f0 - f1)


def test_library_allocates_no_device_memory():
    torch = G.torch_mod()
    if torch.cuda.device_count() < 1:
        pytest.skip("no GPU")
    B, H, n, k = 2, 3, 1024, 128
    inp = synth.random_inputs(B, H, n, 64, k, synth.DT_BF16, synth.SHARE_NONE, seed=5,
                              lengths=[1024, 700])
    wl = inp.wl
    p = G.prob(wl)
    Q, K, V, E, F = (G.dev(x, wl.dtype) for x in (inp.Q, inp.K, inp.V, inp.E, inp.F))
    lens = G.lengths_dev(inp.lengths)
    O = G.empty((B, H, n, 64), wl.dtype)
    wsb = L.linformer_workspace_size(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    f32 = lambda *s: torch.empty(*s, dtype=torch.float32, device="cuda")
    dQ, dK, dV = f32(B, H, n, 64), f32(B, H, n, 64), f32(B, H, n, 64)
    dE, dF = f32(*inp.E.shape), f32(*inp.F.shape)
    bwb = L.linformer_backward_workspace_size(p)
    bws = torch.empty(bwb, dtype=torch.uint8, device="cuda")
    si = synth.make_stack_inputs(synth.StackWorkload("mem", 2, 256, 384, 6, 128, 2), seed=3)
    s = L.stack(2, 256, 384, 6, 128, 2, False, 0.0)
    X, Wq, Wo, Es = (G.dev(x, synth.DT_BF16) for x in (si.X, si.Wqkv, si.Wo, si.E))
    Y = G.empty((2, 256, 384), synth.DT_BF16)
    swb = L.linformer_stack_workspace_size(s)
    sws = torch.empty(swb, dtype=torch.uint8, device="cuda")
    calls = {
        "forward": lambda: L.linformer_forward(p, Q, K, V, E, F, lens, O, ws, wsb),
        "forward_noalloc": lambda: L.linformer_forward_noalloc(p, Q, K, V, E, F, lens, O),
        "backward": lambda: L.linformer_backward(p, Q, K, V, E, F, lens, O, dQ, dK, dV, dE, dF,
                                                 bws, bwb),
        "stack": lambda: L.linformer_stack_forward(s, X, Wq, Wo, Es, None, Y, sws, swb),
        "dense_comparator": lambda: L.attention_dense_forward(p, Q, K, V, lens, O),
    }
    for name, fn in calls.items():
        d = _delta(torch, fn)
        G.log(f"{name}: free device memory changed by {d} bytes over 3 warmed-up calls")
        assert d == 0, (name, d)
