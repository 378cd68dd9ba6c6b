"""Host-side checks of liblinformer (no GPU needed): the library loads, exports every function
include/linformer.h declares, sizes its buffers as documented, and rejects bad arguments before
touching a device.  No compute call is made here."""
import ctypes
import os
import re

import pytest

from efficient_transformer_attention_seq_amd import linformer as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linformer.h")

# Fake, 16-byte aligned, non-overlapping "device" addresses: every call below fails validation
# on the host before any device work, so they are never dereferenced.
A = 1 << 40


def fake(i):
    return A + i * (1 << 34)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:linformer|attention)_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = L.lib()
    declared = header_functions()
    assert set(declared) == set(L.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code, name in L.STATUS.items():
        assert L.status_string(code).startswith(name)
    assert "unknown" in L.status_string(99)


def test_sizes_match_layout():
    B, H, n, k = 8, 12, 4096, 256
    p = L.problem(B, H, n, 64, k, L.LF_BF16, L.LF_SHARE_NONE)
    kb, vb = L.linformer_kv_sizes(p)
    assert kb == 3 * B * H * k * 64 + 2 * B * H * k   # bf16 hi, e4m3 residual, block scales
    assert vb == B * H * k * 64 * 2
    ws = L.linformer_workspace_size(p)
    assert ws >= kb + vb
    p32 = L.problem(1, 1, 512, 64, 128, L.LF_F32, L.LF_SHARE_NONE)
    kb, vb = L.linformer_kv_sizes(p32)
    assert kb == vb == 128 * 64 * 4
    assert L.linformer_workspace_size(p32) >= kb + vb


def _r256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("B,H,n,k,share,splits", [
    (8, 12, 4096, 256, L.LF_SHARE_NONE, 2),       # bench shape: 96 tiles x 2 position splits
    (1, 12, 1024, 128, L.LF_SHARE_LAYERWISE, 4),  # 6 tiles, at least 256 positions per split
    (1, 12, 512, 128, L.LF_SHARE_LAYERWISE, 1),   # at most 512 positions: never split
    (32, 12, 512, 256, L.LF_SHARE_KV, 1),         # short reduction over many tiles: unsplit
])
def test_workspace_holds_partials_only_for_split_projections(B, H, n, k, share, splits):
    """The forward workspace is Kbar | Vbar | fp32 partial sums of the position splits | the
    one-launch kernel's hand-off flags, each region 256-byte aligned; an unsplit projection needs
    no partials.  Three or more splits keep [splits, 2, B, H, k, 64] for the fixup pass; two
    splits are paired inside the projection kernel, which needs one block of sums per workgroup
    tile (128 slots x 4 units x 64 columns at the bench shape: 2 (keys, values) x 12 heads x 2
    slot tiles x 2 unit tiles) and one 8-byte counter per tile.  Shapes the one-launch
    short-sequence kernel takes (bf16, n <= 1024, k of 128 or 256) add one 8-byte flag per
    (b, h).  Pins the host's split plan for a few shapes."""
    p = L.problem(B, H, n, 64, k, L.LF_BF16, share)
    kb, vb = L.linformer_kv_sizes(p)
    if splits == 2:
        tiles = 2 * H * (k // 128) * ((B + 3) // 4)
        part = _r256(tiles * 128 * 4 * 64 * 4) + 8 * tiles
    else:
        part = splits * 2 * B * H * k * 64 * 4 if splits > 1 else 0
    flags = 8 * B * H if n <= 1024 and k in (128, 256) else 0
    assert L.linformer_workspace_size(p) == _r256(kb) + _r256(vb) + _r256(part) + _r256(flags)


@pytest.mark.parametrize("field,value,code", [
    ("d", 32, 2), ("n", 100, 2), ("n", 0, 2), ("k", 48, 2), ("k", 288, 2), ("k", 0, 2),
    ("batch", 0, 2), ("batch", 4097, 2), ("heads", 0, 2), ("dtype", 5, 3), ("share", 9, 4),
    ("scale", -1.0, 2),
    ("scale", float("nan"), 2),
])
def test_problem_validation(field, value, code):
    p = L.problem(2, 2, 256, 64, 64, L.LF_BF16, L.LF_SHARE_NONE)
    setattr(p, field, value)
    out = ctypes.c_size_t(0)
    assert L.lib().linformer_workspace_size(ctypes.byref(p), ctypes.byref(out)) == code
    assert L.linformer_forward(p, fake(0), fake(1), fake(2), fake(3), None, None, fake(4),
                               fake(5), 1 << 30, check=False) == code


def test_size_overflow_rejected():
    p = L.problem(64, 64, 65536, 64, 64, L.LF_BF16, L.LF_SHARE_NONE)   # 2^34 elements
    out = ctypes.c_size_t(0)
    assert L.lib().linformer_workspace_size(ctypes.byref(p), ctypes.byref(out)) == 2


def test_argument_errors_before_any_device_work():
    p = L.problem(2, 2, 256, 64, 64, L.LF_BF16, L.LF_SHARE_NONE)
    big = 1 << 32
    f = lambda *a, **kw: L.linformer_forward(p, *a, check=False, **kw)
    # null inputs / outputs
    assert f(None, fake(1), fake(2), fake(3), None, None, fake(4), fake(5), big) == 1
    assert f(fake(0), fake(1), None, fake(3), None, None, fake(4), fake(5), big) == 1
    assert f(fake(0), fake(1), fake(2), fake(3), None, None, None, fake(5), big) == 1
    # misaligned pointer
    assert f(fake(0) + 2, fake(1), fake(2), fake(3), None, None, fake(4), fake(5), big) == 6
    assert f(fake(0), fake(1), fake(2), fake(3), None, fake(6) + 2, fake(4), fake(5), big) == 6
    # workspace missing or too small
    assert f(fake(0), fake(1), fake(2), fake(3), None, None, fake(4), None, big) == 5
    need = L.linformer_workspace_size(p)
    assert f(fake(0), fake(1), fake(2), fake(3), None, None, fake(4), fake(5), need - 1) == 5
    # output overlapping an input, or the workspace overlapping the output
    assert f(fake(0), fake(1), fake(2), fake(3), None, None, fake(0) + 64, fake(5), big) == 7
    assert f(fake(0), fake(1), fake(2), fake(3), None, None, fake(4), fake(4) + 256, big) == 7
    # sharing rules: headwise needs F; key-value / layerwise need F = E or NULL
    ph = L.problem(2, 2, 256, 64, 64, L.LF_BF16, L.LF_SHARE_HEADWISE)
    assert L.linformer_forward(ph, fake(0), fake(1), fake(2), fake(3), None, None, fake(4),
                               fake(5), big, check=False) == 1
    for mode in (L.LF_SHARE_KV, L.LF_SHARE_LAYERWISE):
        pk = L.problem(2, 2, 256, 64, 64, L.LF_BF16, mode)
        assert L.linformer_forward(pk, fake(0), fake(1), fake(2), fake(3), fake(7), None,
                                   fake(4), fake(5), big, check=False) == 4
    # attend and project halves validate too
    assert L.linformer_attend(p, fake(0), fake(1), fake(2), None, fake(1), check=False) == 7
    assert L.linformer_attend(p, None, fake(1), fake(2), None, fake(3), check=False) == 1
    assert L.linformer_project_kv(p, fake(0), fake(1), fake(2), None, None, fake(3), fake(3),
                                  fake(5), big, check=False) == 7
    # dense comparator: bf16 only
    p32 = L.problem(2, 2, 256, 64, 64, L.LF_F32, L.LF_SHARE_NONE)
    assert L.attention_dense_forward(p32, fake(0), fake(1), fake(2), None, fake(3),
                                     check=False) == 3


def test_no_device_reported_when_absent():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is present; this checks the host-only path")
    p = L.problem(2, 2, 256, 64, 64, L.LF_BF16, L.LF_SHARE_NONE)
    code = L.linformer_forward(p, fake(0), fake(1), fake(2), fake(3), None, None, fake(4),
                               fake(5), 1 << 32, check=False)
    assert code == 8


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        L.lib()


# ---- encoder attention stack
def _stack(**kw):
    s = L.stack(2, 256, 384, 6, 64, 2)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def test_stack_workspace_and_validation():
    out = ctypes.c_size_t(0)
    s = _stack()
    assert L.lib().linformer_stack_workspace_size(ctypes.byref(s), ctypes.byref(out)) == 0
    act = 2 * 256 * 384 * 2
    assert out.value >= 2 * act    # the query plane and the attention output at least
    for field, value, code in [("d_model", 320, 2), ("heads", 5, 2), ("layers", 0, 2),
                               ("n", 100, 2), ("batch", 0, 2), ("k", 48, 2), ("dtype", 0, 3),
                               ("keep_layers", 2, 2), ("scale", -1.0, 2)]:
        bad = _stack(**{field: value})
        assert L.lib().linformer_stack_workspace_size(ctypes.byref(bad), ctypes.byref(out)) == code, field
    # any batch * n (a last token tile may be partial); d_model whole 192-feature tiles
    assert L.lib().linformer_stack_workspace_size(
        ctypes.byref(L.stack(1, 192, 384, 6, 64, 1)), ctypes.byref(out)) == 0
    assert L.lib().linformer_stack_workspace_size(
        ctypes.byref(L.stack(2, 256, 256, 4, 64, 1)), ctypes.byref(out)) == 2


def test_stack_argument_errors_before_any_device_work():
    s = _stack()
    big = 1 << 32
    f = lambda *a: L.linformer_stack_forward(s, *a, check=False)
    assert f(None, fake(1), fake(2), fake(3), None, fake(4), fake(5), big) == 1
    assert f(fake(0), fake(1), fake(2), fake(3), None, None, fake(5), big) == 1
    assert f(fake(0) + 2, fake(1), fake(2), fake(3), None, fake(4), fake(5), big) == 6
    need = L.linformer_stack_workspace_size(s)
    assert f(fake(0), fake(1), fake(2), fake(3), None, fake(4), fake(5), need - 1) == 5
    assert f(fake(0), fake(1), fake(2), fake(3), None, fake(0) + 64, fake(5), big) == 7
    assert f(fake(0), fake(1), fake(2), fake(3), None, fake(4), fake(4) + 256, big) == 7


def test_backward_workspace_and_argument_errors():
    p = L.problem(2, 2, 256, 64, 64, L.LF_BF16, L.LF_SHARE_NONE)
    need = L.linformer_backward_workspace_size(p)
    # at least Kbar, Vbar, their gradients (fp32 [B, H, k, 64]) and the per-query softmax
    # statistics (fp32 [B, H, n, 4])
    assert need >= 4 * (2 * 2 * 64 * 64 * 4) + 2 * 2 * 256 * 4 * 4
    big = 1 << 33
    f = lambda *a, **kw: L.linformer_backward(p, *a, check=False, **kw)
    ok = [fake(0), fake(1), fake(2), fake(3), fake(4), None, fake(5),
          fake(6), fake(7), fake(8), fake(9), fake(10), fake(11), big]
    def args(i, v):
        a = list(ok)
        a[i] = v
        return a
    assert f(*args(0, None)) == 1                # Q missing
    assert f(*args(11, None)) == 1               # dF missing while F is separate
    assert f(*args(4, fake(3))) == 4             # F = E: dF must be NULL
    assert f(*args(7, fake(7) + 4)) == 6         # misaligned dQ
    assert f(*args(13, need - 1)) == 5           # workspace too small
    assert f(*args(8, fake(1) + 64)) == 7        # dK overlaps K
    pk = L.problem(2, 2, 256, 64, 64, L.LF_BF16, L.LF_SHARE_KV)
    assert L.linformer_backward(pk, fake(0), fake(1), fake(2), fake(3), None, None, fake(5),
                                fake(6), fake(7), fake(8), fake(9), fake(10), fake(11), big,
                                check=False) == 4       # shared F: no dF
    assert L.linformer_backward(pk, fake(0), fake(1), fake(2), fake(3), None, None, fake(5),
                                fake(6), fake(7), fake(8), fake(9), None, fake(11), big,
                                check=False) in (0, 8)  # valid up to the device check


def test_conv_argument_errors():
    p = L.problem(2, 2, 256, 64, 64, L.LF_BF16, L.LF_SHARE_NONE)
    f = lambda *a: L.linformer_project_kv_conv(p, *a, check=False)
    assert f(None, fake(1), fake(2), fake(3), None, fake(4), fake(5)) == 1
    assert f(fake(0) + 2, fake(1), fake(2), fake(3), None, fake(4), fake(5)) == 6
    assert f(fake(0), fake(1), fake(2), fake(3), None, fake(0), fake(5)) == 7   # Kbar over K
    p3 = L.problem(2, 2, 256, 64, 96, L.LF_BF16, L.LF_SHARE_NONE)                # n % k != 0
    assert L.linformer_project_kv_conv(p3, fake(0), fake(1), fake(2), fake(3), None, fake(4),
                                       fake(5), check=False) == 2
    p32 = L.problem(2, 2, 256, 64, 64, L.LF_F32, L.LF_SHARE_NONE)
    assert L.linformer_project_kv_conv(p32, fake(0), fake(1), fake(2), fake(3), None, fake(4),
                                       fake(5), check=False) == 3


def test_noalloc_forward_validates_on_the_host():
    # a workload whose workspace exceeds the fixed scratch buffer is refused before any device work
    big_p = L.problem(256, 12, 512, 64, 256, L.LF_BF16, L.LF_SHARE_KV)
    assert L.linformer_workspace_size(big_p) > L.NOALLOC_SCRATCH_BYTES
    f = lambda p, *a: L.linformer_forward_noalloc(p, *a, check=False)
    assert f(big_p, fake(0), fake(1), fake(2), fake(3), None, None, fake(4)) == 11
    assert "scratch" in L.status_string(11)
    # the benchmarked workloads fit
    for B, H, n, k, share in ((8, 12, 4096, 256, L.LF_SHARE_NONE), (32, 12, 512, 256, L.LF_SHARE_KV),
                              (1, 12, 65536, 128, L.LF_SHARE_LAYERWISE),
                              (16, 12, 1024, 256, L.LF_SHARE_LAYERWISE)):
        p = L.problem(B, H, n, 64, k, L.LF_BF16, share)
        assert L.linformer_workspace_size(p) <= L.NOALLOC_SCRATCH_BYTES
    # argument errors as for linformer_forward
    p = L.problem(2, 2, 256, 64, 64, L.LF_BF16, L.LF_SHARE_NONE)
    assert f(p, None, fake(1), fake(2), fake(3), None, None, fake(4)) == 1
    assert f(p, fake(0), fake(1), fake(2), fake(3), None, None, None) == 1
    assert f(p, fake(0) + 2, fake(1), fake(2), fake(3), None, None, fake(4)) == 6
    assert f(p, fake(0), fake(1), fake(2), fake(3), None, None, fake(1) + 64) == 7
    bad = L.problem(2, 2, 200, 64, 64, L.LF_BF16, L.LF_SHARE_NONE)
    assert f(bad, fake(0), fake(1), fake(2), fake(3), None, None, fake(4)) == 2
    import torch
    if torch.cuda.device_count() == 0:
        assert f(p, fake(0), fake(1), fake(2), fake(3), None, None, fake(4)) == 8
