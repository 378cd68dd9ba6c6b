"""ctypes binding for liblinformer (include/linformer.h), same names as the C ABI.

Argument marshalling only: tensors become device pointers, None becomes NULL, the stream defaults
to torch's current stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback -- if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinformer.so")

LF_OK = 0
STATUS = {0: "LF_OK", 1: "LF_ERR_NULL", 2: "LF_ERR_SHAPE", 3: "LF_ERR_DTYPE", 4: "LF_ERR_SHARE",
          5: "LF_ERR_WORKSPACE", 6: "LF_ERR_ALIGN", 7: "LF_ERR_ALIAS", 8: "LF_ERR_NO_DEVICE",
          9: "LF_ERR_ARCH", 10: "LF_ERR_LAUNCH", 11: "LF_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20   # LINFORMER_NOALLOC_SCRATCH_BYTES
LF_F32, LF_BF16 = 0, 1
LF_SHARE_NONE, LF_SHARE_HEADWISE, LF_SHARE_KV, LF_SHARE_LAYERWISE = 0, 1, 2, 3

# every symbol include/linformer.h declares
EXPORTS = ("linformer_status_string", "linformer_workspace_size", "linformer_kv_sizes",
           "linformer_project_kv", "linformer_attend", "linformer_forward",
           "attention_dense_forward", "linformer_stack_workspace_size",
           "linformer_stack_forward", "linformer_project_kv_conv", "linformer_forward_conv",
           "linformer_backward_workspace_size", "linformer_backward",
           "linformer_forward_noalloc")


class lf_problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("n", ctypes.c_int32),
                ("d", ctypes.c_int32), ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("share", ctypes.c_int32), ("scale", ctypes.c_float)]


def problem(batch: int, heads: int, n: int, d: int, k: int, dtype: int, share: int,
            scale: float = 0.0) -> lf_problem:
    return lf_problem(batch, heads, n, d, k, dtype, share, scale)


class lf_stack(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("k", ctypes.c_int32), ("layers", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("keep_layers", ctypes.c_int32),
                ("scale", ctypes.c_float)]


def stack(batch: int, n: int, d_model: int, heads: int, k: int, layers: int,
          keep_layers: bool = False, scale: float = 0.0, dtype: int = LF_BF16) -> lf_stack:
    return lf_stack(batch, n, d_model, heads, k, layers, dtype, int(bool(keep_layers)), scale)


class LinformerError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblinformer.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"liblinformer.so not found at {LIB_PATH}; build it with "
                           "`python -m efficient_transformer_attention_seq_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(lf_problem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.linformer_status_string.restype = ctypes.c_char_p
    L.linformer_status_string.argtypes = [ctypes.c_int]
    L.linformer_workspace_size.restype = ctypes.c_int
    L.linformer_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    L.linformer_kv_sizes.restype = ctypes.c_int
    L.linformer_kv_sizes.argtypes = [P, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.linformer_project_kv.restype = ctypes.c_int
    L.linformer_project_kv.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.linformer_attend.restype = ctypes.c_int
    L.linformer_attend.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.linformer_forward.restype = ctypes.c_int
    L.linformer_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.linformer_forward_noalloc.restype = ctypes.c_int
    L.linformer_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    L.attention_dense_forward.restype = ctypes.c_int
    L.attention_dense_forward.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.linformer_project_kv_conv.restype = ctypes.c_int
    L.linformer_project_kv_conv.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    L.linformer_forward_conv.restype = ctypes.c_int
    L.linformer_forward_conv.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.linformer_backward_workspace_size.restype = ctypes.c_int
    L.linformer_backward_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    L.linformer_backward.restype = ctypes.c_int
    L.linformer_backward.argtypes = [P] + [vp] * 12 + [vp, sz, vp]
    S = ctypes.POINTER(lf_stack)
    L.linformer_stack_workspace_size.restype = ctypes.c_int
    L.linformer_stack_workspace_size.argtypes = [S, ctypes.POINTER(sz)]
    L.linformer_stack_forward.restype = ctypes.c_int
    L.linformer_stack_forward.argtypes = [S, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    _lib = L
    return L


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(code: int, where: str, check: bool) -> int:
    if check and code != LF_OK:
        raise LinformerError(code, where)
    return code


def status_string(code: int) -> str:
    return lib().linformer_status_string(code).decode()


def linformer_status_string(code: int) -> str:
    return status_string(code)


def linformer_workspace_size(p: lf_problem) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().linformer_workspace_size(ctypes.byref(p), ctypes.byref(out)),
           "linformer_workspace_size", True)
    return out.value


def linformer_kv_sizes(p: lf_problem) -> Tuple[int, int]:
    kb, vb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().linformer_kv_sizes(ctypes.byref(p), ctypes.byref(kb), ctypes.byref(vb)),
           "linformer_kv_sizes", True)
    return kb.value, vb.value


def linformer_project_kv(p: lf_problem, K, V, E, F, lengths, Kbar, Vbar, ws, ws_bytes=None,
                         stream=None, check: bool = True) -> int:
    wsb = ws_bytes if ws_bytes is not None else (
        0 if ws is None or isinstance(ws, int) else ws.numel() * ws.element_size())
    code = lib().linformer_project_kv(ctypes.byref(p), _ptr(K), _ptr(V), _ptr(E), _ptr(F),
                                      _ptr(lengths), _ptr(Kbar), _ptr(Vbar), _ptr(ws), wsb,
                                      _stream(stream))
    return _check(code, "linformer_project_kv", check)


def linformer_attend(p: lf_problem, Q, Kbar, Vbar, lengths, O, stream=None,
                     check: bool = True) -> int:
    code = lib().linformer_attend(ctypes.byref(p), _ptr(Q), _ptr(Kbar), _ptr(Vbar),
                                  _ptr(lengths), _ptr(O), _stream(stream))
    return _check(code, "linformer_attend", check)


def linformer_forward(p: lf_problem, Q, K, V, E, F, lengths, O, ws, ws_bytes=None, stream=None,
                      check: bool = True) -> int:
    wsb = ws_bytes if ws_bytes is not None else (
        0 if ws is None or isinstance(ws, int) else ws.numel() * ws.element_size())
    code = lib().linformer_forward(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(E), _ptr(F),
                                   _ptr(lengths), _ptr(O), _ptr(ws), wsb, _stream(stream))
    return _check(code, "linformer_forward", check)


def linformer_forward_noalloc(p: lf_problem, Q, K, V, E, F, lengths, O, stream=None,
                              check: bool = True) -> int:
    code = lib().linformer_forward_noalloc(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(E),
                                           _ptr(F), _ptr(lengths), _ptr(O), _stream(stream))
    return _check(code, "linformer_forward_noalloc", check)


def attention_dense_forward(p: lf_problem, Q, K, V, lengths, O, stream=None,
                            check: bool = True) -> int:
    code = lib().attention_dense_forward(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V),
                                         _ptr(lengths), _ptr(O), _stream(stream))
    return _check(code, "attention_dense_forward", check)


def linformer_stack_workspace_size(s: lf_stack) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().linformer_stack_workspace_size(ctypes.byref(s), ctypes.byref(out)),
           "linformer_stack_workspace_size", True)
    return out.value


def linformer_stack_forward(s: lf_stack, X, Wqkv, Wo, E, lengths, Y, ws, ws_bytes=None,
                            stream=None, check: bool = True) -> int:
    wsb = ws_bytes if ws_bytes is not None else (
        0 if ws is None or isinstance(ws, int) else ws.numel() * ws.element_size())
    code = lib().linformer_stack_forward(ctypes.byref(s), _ptr(X), _ptr(Wqkv), _ptr(Wo), _ptr(E),
                                         _ptr(lengths), _ptr(Y), _ptr(ws), wsb, _stream(stream))
    return _check(code, "linformer_stack_forward", check)


def linformer_project_kv_conv(p: lf_problem, K, V, wE, wF, lengths, Kbar, Vbar, stream=None,
                              check: bool = True) -> int:
    code = lib().linformer_project_kv_conv(ctypes.byref(p), _ptr(K), _ptr(V), _ptr(wE), _ptr(wF),
                                           _ptr(lengths), _ptr(Kbar), _ptr(Vbar), _stream(stream))
    return _check(code, "linformer_project_kv_conv", check)


def linformer_forward_conv(p: lf_problem, Q, K, V, wE, wF, lengths, O, ws, ws_bytes=None,
                           stream=None, check: bool = True) -> int:
    wsb = ws_bytes if ws_bytes is not None else (
        0 if ws is None or isinstance(ws, int) else ws.numel() * ws.element_size())
    code = lib().linformer_forward_conv(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(wE),
                                        _ptr(wF), _ptr(lengths), _ptr(O), _ptr(ws), wsb,
                                        _stream(stream))
    return _check(code, "linformer_forward_conv", check)


def linformer_backward_workspace_size(p: lf_problem) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().linformer_backward_workspace_size(ctypes.byref(p), ctypes.byref(out)),
           "linformer_backward_workspace_size", True)
    return out.value


def linformer_backward(p: lf_problem, Q, K, V, E, F, lengths, dO, dQ, dK, dV, dE, dF, ws,
                       ws_bytes=None, stream=None, check: bool = True) -> int:
    wsb = ws_bytes if ws_bytes is not None else (
        0 if ws is None or isinstance(ws, int) else ws.numel() * ws.element_size())
    code = lib().linformer_backward(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(E), _ptr(F),
                                    _ptr(lengths), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV),
                                    _ptr(dE), _ptr(dF), _ptr(ws), wsb, _stream(stream))
    return _check(code, "linformer_backward", check)
