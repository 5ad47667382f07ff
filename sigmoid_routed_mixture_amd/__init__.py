"""Python binding of libmoe.so, the MI355X (gfx950) sigmoid-routed mixture-of-experts layer.

Argument marshalling only: every step of the layer runs in the HIP kernels behind the C ABI of
include/moe.h. PyTorch supplies device memory and streams. The functions keep the C names:

    moe_workspace_bytes(T, H, E, k, I, Is)
    moe_permute_workspace_bytes(T, E)
    moe_route(x, w_router, bias, k, scale, topk_ids, topk_gates, logits=None, stream=None)
    moe_permute(topk_ids, E, counts, offsets, row_token, slot_row, workspace, x=None, x_perm=None, stream=None)
    moe_forward(x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, k, scale, out, workspace, topk_ids=None,
                topk_gates=None, expert_counts=None, stream=None, stream_shared=None)
    moe_forward_noalloc_max_bytes()
    moe_forward_noalloc(x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, k, scale, out, topk_ids=None,
                        topk_gates=None, expert_counts=None, stream=None)

the knobs of include/moe_tuning.h (tests and benchmarks only):

    moe_set_tuning(knob, value), moe_get_tuning(knob), and the context manager tuned(MOE_TUNE_...=value)

and those of include/moe_block.h:

    moe_forward_routed(x, topk_ids, topk_gates, w1, w3, w2, ws1, ws3, ws2, out, workspace, expert_counts=None,
                       stream=None, stream_shared=None)
    moe_block_workspace_bytes(T, H, E, k, I, Is)
    moe_block_forward(resid, gamma, eps, w_router, bias, w1, w3, w2, ws1, ws3, ws2, k, scale, out, workspace,
                      x_norm=None, topk_ids=None, topk_gates=None, expert_counts=None, stream=None,
                      stream_shared=None)
    moe_dense_mlp_workspace_bytes(T, H, I)
    moe_dense_mlp(x, w1, w3, w2, out, workspace, stream=None)

bf16 tensors are torch.bfloat16; ids and counts int32; gates, bias, logits and out float32. All tensors
must be contiguous and on the same HIP device. A non-OK status raises MoEError with the library's text.
If libmoe.so is missing this module raises at import: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libmoe.so is not built; run `python sigmoid_routed_mixture_amd/_build.py` "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)
_p, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_lib.moe_workspace_bytes.argtypes = [_i] * 6
_lib.moe_workspace_bytes.restype = _sz
_lib.moe_permute_workspace_bytes.argtypes = [_i, _i]
_lib.moe_permute_workspace_bytes.restype = _sz
_lib.moe_route.argtypes = [_p, _p, _p, _i, _i, _i, _i, _f, _p, _p, _p, _p]
_lib.moe_route.restype = _i
_lib.moe_permute.argtypes = [_p, _p, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p]
_lib.moe_permute.restype = _i
_lib.moe_forward.argtypes = [_p] * 9 + [_i] * 6 + [_f] + [_p] * 5 + [_sz, _p, _p]
_lib.moe_forward.restype = _i
_lib.moe_forward_profiled.argtypes = [_p] * 9 + [_i] * 6 + [_f] + [_p] * 5 + [_sz, _p, _p, _p]
_lib.moe_forward_profiled.restype = _i
_d = ctypes.c_double
_lib.moe_forward_routed.argtypes = [_p] * 9 + [_i] * 6 + [_p, _p, _p, _sz, _p, _p]
_lib.moe_forward_routed.restype = _i
_lib.moe_block_workspace_bytes.argtypes = [_i] * 6
_lib.moe_block_workspace_bytes.restype = _sz
_lib.moe_block_forward.argtypes = [_p, _p, _d] + [_p] * 8 + [_i] * 6 + [_f] + [_p] * 6 + [_sz, _p, _p]
_lib.moe_block_forward.restype = _i
_lib.moe_dense_mlp_workspace_bytes.argtypes = [_i] * 3
_lib.moe_dense_mlp_workspace_bytes.restype = _sz
_lib.moe_dense_mlp.argtypes = [_p] * 4 + [_i] * 3 + [_p, _p, _sz, _p]
_lib.moe_dense_mlp.restype = _i
_lib.moe_forward_noalloc_max_bytes.argtypes = []
_lib.moe_forward_noalloc_max_bytes.restype = _sz
_lib.moe_forward_noalloc.argtypes = [_p] * 9 + [_i] * 6 + [_f] + [_p] * 4 + [_p]
_lib.moe_forward_noalloc.restype = _i
_lib.moe_set_tuning.argtypes = [_i, _i]
_lib.moe_set_tuning.restype = _i
_lib.moe_get_tuning.argtypes = [_i]
_lib.moe_get_tuning.restype = _i
_lib.moe_status_string.argtypes = [_i]
_lib.moe_status_string.restype = ctypes.c_char_p
_lib.moe_last_error.argtypes = []
_lib.moe_last_error.restype = ctypes.c_char_p

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_MISALIGNED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(6)
EXPORTED_SYMBOLS = ("moe_workspace_bytes", "moe_permute_workspace_bytes", "moe_route", "moe_permute",
                    "moe_forward", "moe_forward_profiled", "moe_status_string", "moe_last_error",
                    "moe_forward_routed", "moe_block_workspace_bytes", "moe_block_forward",
                    "moe_dense_mlp_workspace_bytes", "moe_dense_mlp", "moe_set_tuning", "moe_get_tuning",
                    "moe_forward_noalloc", "moe_forward_noalloc_max_bytes")
# Knobs of include/moe_tuning.h (tests and benchmarks only; 0 = the size rules).
(MOE_TUNE_GEMM_PATH, MOE_TUNE_XCD_SPLIT, MOE_TUNE_PERSIST, MOE_TUNE_KSPLIT, MOE_TUNE_ORDER, MOE_TUNE_SHARED,
 MOE_TUNE_RING, MOE_TUNE_ROUTE_PERMUTE, MOE_TUNE_STREAMK) = range(9)
MOE_TUNE_KNOBS = 9
GEMM_PATHS = {"auto": 0, "wide": 1, "tall": 2, "dma": 3, "skinny": 4}


class MoEError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = _lib.moe_status_string(status).decode()
        detail = _lib.moe_last_error().decode()
        super().__init__("%s (status %d)%s" % (msg, status, ": " + detail if detail else ""))


def library() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoEError(status)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    return t.data_ptr()


def _stream(s, device):
    if s is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def moe_set_tuning(knob: int, value: int) -> None:
    _check(_lib.moe_set_tuning(knob, value))


def moe_get_tuning(knob: int) -> int:
    return _lib.moe_get_tuning(knob)


class tuned:
    """Context manager that sets tuning knobs (include/moe_tuning.h) and restores them on exit:
    `with tuned(MOE_TUNE_GEMM_PATH=3): ...`."""

    _names = {"MOE_TUNE_GEMM_PATH": 0, "MOE_TUNE_XCD_SPLIT": 1, "MOE_TUNE_PERSIST": 2, "MOE_TUNE_KSPLIT": 3,
              "MOE_TUNE_ORDER": 4, "MOE_TUNE_SHARED": 5, "MOE_TUNE_RING": 6,
              "MOE_TUNE_ROUTE_PERMUTE": 7, "MOE_TUNE_STREAMK": 8}

    def __init__(self, **knobs):
        self.knobs = {self._names[k]: v for k, v in knobs.items()}
        self.saved = {}

    def __enter__(self):
        for k, v in self.knobs.items():
            self.saved[k] = moe_get_tuning(k)
            moe_set_tuning(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            moe_set_tuning(k, v)
        return False


def moe_workspace_bytes(T: int, H: int, E: int, k: int, I: int, Is: int) -> int:
    return _lib.moe_workspace_bytes(T, H, E, k, I, Is)


def moe_permute_workspace_bytes(T: int, E: int) -> int:
    return _lib.moe_permute_workspace_bytes(T, E)


def moe_route(x, w_router, bias, k, scale, topk_ids, topk_gates, logits=None, stream=None):
    T, H = x.shape
    E = w_router.shape[0]
    _check(_lib.moe_route(_ptr(x, torch.bfloat16, "x"), _ptr(w_router, torch.bfloat16, "w_router"),
                          _ptr(bias, torch.float32, "bias"), T, H, E, k, float(scale),
                          _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_gates, torch.float32, "topk_gates"),
                          _ptr(logits, torch.float32, "logits"), _stream(stream, x.device)))


def moe_permute(topk_ids, E, counts, offsets, row_token, slot_row, workspace, x=None, x_perm=None, stream=None):
    T, k = topk_ids.shape
    H = x.shape[1] if x is not None else (x_perm.shape[1] if x_perm is not None else 64)
    _check(_lib.moe_permute(_ptr(x, torch.bfloat16, "x"), _ptr(topk_ids, torch.int32, "topk_ids"), T, H, E, k,
                            _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
                            _ptr(row_token, torch.int32, "row_token"), _ptr(slot_row, torch.int32, "slot_row"),
                            _ptr(x_perm, torch.bfloat16, "x_perm"), _ptr(workspace, None, "workspace"),
                            workspace.numel() * workspace.element_size(), _stream(stream, topk_ids.device)))


def _forward(fn, extra, x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, k, scale, out, workspace, topk_ids,
             topk_gates, expert_counts, stream, stream_shared):
    T, H = x.shape
    E, I, _ = w1.shape
    Is = 0 if ws1 is None else ws1.shape[0]
    bf = torch.bfloat16
    s1 = None if stream_shared is None else _stream(stream_shared, x.device)
    _check(fn(
        _ptr(x, bf, "x"), _ptr(w_router, bf, "w_router"), _ptr(bias, torch.float32, "bias"), _ptr(w1, bf, "w1"),
        _ptr(w3, bf, "w3"), _ptr(w2, bf, "w2"), _ptr(ws1, bf, "ws1"), _ptr(ws3, bf, "ws3"), _ptr(ws2, bf, "ws2"),
        T, H, E, k, I, Is, float(scale), _ptr(out, torch.float32, "out"), _ptr(topk_ids, torch.int32, "topk_ids"),
        _ptr(topk_gates, torch.float32, "topk_gates"), _ptr(expert_counts, torch.int32, "expert_counts"),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream, x.device), s1, *extra))


def moe_forward(x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, k, scale, out, workspace, topk_ids=None,
                topk_gates=None, expert_counts=None, stream=None, stream_shared=None):
    _forward(_lib.moe_forward, (), x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, k, scale, out, workspace, topk_ids,
             topk_gates, expert_counts, stream, stream_shared)


def moe_forward_noalloc_max_bytes() -> int:
    return _lib.moe_forward_noalloc_max_bytes()


def moe_forward_noalloc(x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, k, scale, out, topk_ids=None,
                        topk_gates=None, expert_counts=None, stream=None):
    """moe_forward on the library's own per-device scratch (include/moe.h): no workspace argument, nothing
    allocated; sizes whose workspace exceeds moe_forward_noalloc_max_bytes() raise MoEError."""
    T, H = x.shape
    E, I, _ = w1.shape
    Is = 0 if ws1 is None else ws1.shape[0]
    bf = torch.bfloat16
    _check(_lib.moe_forward_noalloc(
        _ptr(x, bf, "x"), _ptr(w_router, bf, "w_router"), _ptr(bias, torch.float32, "bias"), _ptr(w1, bf, "w1"),
        _ptr(w3, bf, "w3"), _ptr(w2, bf, "w2"), _ptr(ws1, bf, "ws1"), _ptr(ws3, bf, "ws3"), _ptr(ws2, bf, "ws2"),
        T, H, E, k, I, Is, float(scale), _ptr(out, torch.float32, "out"), _ptr(topk_ids, torch.int32, "topk_ids"),
        _ptr(topk_gates, torch.float32, "topk_gates"), _ptr(expert_counts, torch.int32, "expert_counts"),
        _stream(stream, x.device)))


def moe_forward_profiled(x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, k, scale, out, workspace, events,
                         topk_ids=None, topk_gates=None, expert_counts=None, stream=None, stream_shared=None):
    """moe_forward that also records seven torch.cuda.Event objects (timing enabled, already recorded once so
    their HIP events exist) at the stage boundaries; see include/moe_profile.h. An entry may be None: that
    boundary is not recorded."""
    if len(events) != 7:
        raise ValueError("moe_forward_profiled takes 7 events")
    handles = (ctypes.c_void_p * 7)(*[None if e is None else e.cuda_event for e in events])
    _forward(_lib.moe_forward_profiled, (handles,), x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, k, scale, out,
             workspace, topk_ids, topk_gates, expert_counts, stream, stream_shared)


def _nbytes(t):
    return t.numel() * t.element_size()


def moe_forward_routed(x, topk_ids, topk_gates, w1, w3, w2, ws1, ws3, ws2, out, workspace, expert_counts=None,
                       stream=None, stream_shared=None):
    T, H = x.shape
    E, I, _ = w1.shape
    k = topk_ids.shape[1]
    Is = 0 if ws1 is None else ws1.shape[0]
    bf = torch.bfloat16
    s1 = None if stream_shared is None else _stream(stream_shared, x.device)
    _check(_lib.moe_forward_routed(
        _ptr(x, bf, "x"), _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_gates, torch.float32, "topk_gates"),
        _ptr(w1, bf, "w1"), _ptr(w3, bf, "w3"), _ptr(w2, bf, "w2"), _ptr(ws1, bf, "ws1"), _ptr(ws3, bf, "ws3"),
        _ptr(ws2, bf, "ws2"), T, H, E, k, I, Is, _ptr(out, torch.float32, "out"),
        _ptr(expert_counts, torch.int32, "expert_counts"), _ptr(workspace, None, "workspace"), _nbytes(workspace),
        _stream(stream, x.device), s1))


def moe_block_workspace_bytes(T: int, H: int, E: int, k: int, I: int, Is: int) -> int:
    return _lib.moe_block_workspace_bytes(T, H, E, k, I, Is)


def moe_block_forward(resid, gamma, eps, w_router, bias, w1, w3, w2, ws1, ws3, ws2, k, scale, out, workspace,
                      x_norm=None, topk_ids=None, topk_gates=None, expert_counts=None, stream=None,
                      stream_shared=None):
    T, H = resid.shape
    E, I, _ = w1.shape
    Is = 0 if ws1 is None else ws1.shape[0]
    bf = torch.bfloat16
    s1 = None if stream_shared is None else _stream(stream_shared, resid.device)
    _check(_lib.moe_block_forward(
        _ptr(resid, bf, "resid"), _ptr(gamma, bf, "gamma"), float(eps), _ptr(w_router, bf, "w_router"),
        _ptr(bias, torch.float32, "bias"), _ptr(w1, bf, "w1"), _ptr(w3, bf, "w3"), _ptr(w2, bf, "w2"),
        _ptr(ws1, bf, "ws1"), _ptr(ws3, bf, "ws3"), _ptr(ws2, bf, "ws2"), T, H, E, k, I, Is, float(scale),
        _ptr(out, torch.float32, "out"), _ptr(x_norm, bf, "x_norm"), _ptr(topk_ids, torch.int32, "topk_ids"),
        _ptr(topk_gates, torch.float32, "topk_gates"), _ptr(expert_counts, torch.int32, "expert_counts"),
        _ptr(workspace, None, "workspace"), _nbytes(workspace), _stream(stream, resid.device), s1))


def moe_dense_mlp_workspace_bytes(T: int, H: int, I: int) -> int:
    return _lib.moe_dense_mlp_workspace_bytes(T, H, I)


def moe_dense_mlp(x, w1, w3, w2, out, workspace, stream=None):
    T, H = x.shape
    I = w1.shape[0]
    bf = torch.bfloat16
    _check(_lib.moe_dense_mlp(_ptr(x, bf, "x"), _ptr(w1, bf, "w1"), _ptr(w3, bf, "w3"), _ptr(w2, bf, "w2"), T, H, I,
                              _ptr(out, torch.float32, "out"), _ptr(workspace, None, "workspace"),
                              _nbytes(workspace), _stream(stream, x.device)))


class MoELayer:
    """Convenience holder: weights plus a workspace sized for up to T_max tokens."""

    def __init__(self, w_router, bias, w1, w3, w2, ws1, ws3, ws2, k: int, scale: float, T_max: int):
        self.w_router, self.bias = w_router, bias
        self.w1, self.w3, self.w2 = w1, w3, w2
        self.ws1, self.ws3, self.ws2 = ws1, ws3, ws2
        self.k, self.scale = k, scale
        E, I, H = w1.shape
        Is = 0 if ws1 is None else ws1.shape[0]
        nbytes = moe_workspace_bytes(T_max, H, E, k, I, Is)
        if nbytes == 0:
            raise ValueError("unsupported sizes")
        self.T_max = T_max
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=w1.device)

    def __call__(self, x, out=None, topk_ids=None, topk_gates=None, expert_counts=None, stream=None,
                 stream_shared=None):
        T, H = x.shape
        if T > self.T_max:
            raise ValueError("T exceeds the workspace's T_max")
        if out is None:
            out = torch.empty(T, H, dtype=torch.float32, device=x.device)
        moe_forward(x, self.w_router, self.bias, self.w1, self.w3, self.w2, self.ws1, self.ws3, self.ws2, self.k,
                    self.scale, out, self.workspace, topk_ids, topk_gates, expert_counts, stream, stream_shared)
        return out
