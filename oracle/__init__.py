"""CPU oracle of the sigmoid-routed MoE layer: ctypes bindings to `oracle.c`.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the benchmark's CPU-baseline leg may
import this module. The product path never does; it shares no code with it.

Each call is plain single-threaded C. `run_sharded` splits a list of tokens over host threads (the C code
releases the GIL through ctypes), each thread running the same single-threaded code on its own tokens;
tokens are independent, so the result is the same bytes whatever the split.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (plain -O2: no fast-math, so every sum keeps its written order)."""
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()  # no-op unless the source is newer than the built library
            L = ctypes.CDLL(_LIB_PATH)
            p, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
            L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
            L.oracle_bf16_to_double.restype = ctypes.c_double
            L.oracle_sigmoid.argtypes = [f32]
            L.oracle_sigmoid.restype = f32
            L.oracle_route.argtypes = [i32, i32, i32, f32, p, p, p, p, i32, p, p, p, p]
            L.oracle_route.restype = i32
            L.oracle_forward.argtypes = [i32, i32, i32, i32, i32, f32] + [p] * 10 + [i32] + [p] * 6
            L.oracle_forward.restype = i32
            L.oracle_forward_routed.argtypes = [i32, i32, i32, i32, i32] + [p] * 10 + [i32, p]
            L.oracle_forward_routed.restype = i32
            L.oracle_permute.argtypes = [i32, i32, i32, p, p, p, p, p]
            L.oracle_permute.restype = i32
            L.oracle_param_count.argtypes = [ctypes.c_uint64] * 4
            L.oracle_param_count.restype = ctypes.c_uint64
            dbl = ctypes.c_double
            L.oracle_round_bf16.argtypes = [dbl]
            L.oracle_round_bf16.restype = ctypes.c_uint16
            L.oracle_rmsnorm.argtypes = [i32, dbl, p, p, p, i32, p]
            L.oracle_rmsnorm.restype = i32
            L.oracle_block_forward.argtypes = [i32, i32, i32, i32, i32, f32, dbl] + [p] * 11 + [i32] + [p] * 5
            L.oracle_block_forward.restype = i32
            L.oracle_dense_mlp.argtypes = [i32, i32, p, p, p, p, p, i32, p]
            L.oracle_dense_mlp.restype = i32
            _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous numpy"
    return a.ctypes.data


def _bf16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, "bf16 tensors are passed as uint16 bit patterns"
    return a


def bf16_to_double(v: int) -> float:
    return lib().oracle_bf16_to_double(v)


def sigmoid(z: float) -> float:
    return lib().oracle_sigmoid(z)


def param_count(H: int, E: int, I: int, Is: int) -> int:
    return lib().oracle_param_count(H, E, I, Is)


def _rows_arg(rows, T):
    if rows is None:
        return None, T
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    return rows, rows.size


def route(x, wr, b, k, scale, rows=None, want_logits=False):
    """Routing of the listed tokens (all if rows is None). Returns dict ids, gates, gap[, logits]."""
    x, wr = _bf16(x), _bf16(wr)
    b = np.ascontiguousarray(b, dtype=np.float32)
    H = x.shape[1]
    E = wr.shape[0]
    rows, n = _rows_arg(rows, x.shape[0])
    ids = np.empty((n, k), np.int32)
    gates = np.empty((n, k), np.float32)
    gap = np.empty(n, np.float64)
    logits = np.empty((n, E), np.float32) if want_logits else None
    rc = lib().oracle_route(H, E, k, scale, _p(x), _p(wr), _p(b), _p(rows), n, _p(ids), _p(gates),
                            _p(logits), _p(gap))
    if rc != 0:
        raise ValueError("oracle_route rejected its arguments")
    d = {"ids": ids, "gates": gates, "gap": gap}
    if want_logits:
        d["logits"] = logits
    return d


def forward(inp, k, scale, rows=None, parts=False):
    """The whole layer for the listed tokens. inp holds x, wr, b, w1, w3, w2, ws1, ws3, ws2 (bf16 as uint16;
    ws* may be None with Is = 0). Returns dict out, ids, gates, gap[, routed, shared]."""
    x, wr = _bf16(inp["x"]), _bf16(inp["wr"])
    b = np.ascontiguousarray(inp["b"], dtype=np.float32)
    w1, w3, w2 = _bf16(inp["w1"]), _bf16(inp["w3"]), _bf16(inp["w2"])
    H, E, I = x.shape[1], wr.shape[0], w1.shape[1]
    ws1 = inp.get("ws1")
    Is = 0 if ws1 is None or ws1.size == 0 else ws1.shape[0]
    ws1 = _bf16(ws1) if Is else None
    ws3 = _bf16(inp["ws3"]) if Is else None
    ws2 = _bf16(inp["ws2"]) if Is else None
    rows, n = _rows_arg(rows, x.shape[0])
    out = np.empty((n, H), np.float32)
    ids = np.empty((n, k), np.int32)
    gates = np.empty((n, k), np.float32)
    gap = np.empty(n, np.float64)
    routed = np.empty((n, H), np.float32) if parts else None
    shared = np.empty((n, H), np.float32) if parts else None
    rc = lib().oracle_forward(H, E, k, I, Is, scale, _p(x), _p(wr), _p(b), _p(w1), _p(w3), _p(w2), _p(ws1),
                              _p(ws3), _p(ws2), _p(rows), n, _p(out), _p(ids), _p(gates), _p(gap), _p(routed),
                              _p(shared))
    if rc != 0:
        raise ValueError("oracle_forward rejected its arguments")
    d = {"out": out, "ids": ids, "gates": gates, "gap": gap}
    if parts:
        d["routed"], d["shared"] = routed, shared
    return d


def forward_routed(inp, ids, gates, rows=None):
    """The layer with given routing: ids [T, k] int32, gates [T, k] fp32, used as written."""
    x = _bf16(inp["x"])
    w1, w3, w2 = _bf16(inp["w1"]), _bf16(inp["w3"]), _bf16(inp["w2"])
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    gates = np.ascontiguousarray(gates, dtype=np.float32)
    H, E, I = x.shape[1], w1.shape[0], w1.shape[1]
    k = ids.shape[1]
    ws1 = inp.get("ws1")
    Is = 0 if ws1 is None or ws1.size == 0 else ws1.shape[0]
    ws1 = _bf16(ws1) if Is else None
    ws3 = _bf16(inp["ws3"]) if Is else None
    ws2 = _bf16(inp["ws2"]) if Is else None
    rows, n = _rows_arg(rows, x.shape[0])
    out = np.empty((n, H), np.float32)
    rc = lib().oracle_forward_routed(H, E, k, I, Is, _p(x), _p(ids), _p(gates), _p(w1), _p(w3), _p(w2),
                                     _p(ws1), _p(ws3), _p(ws2), _p(rows), n, _p(out))
    if rc != 0:
        raise ValueError("oracle_forward_routed rejected its arguments")
    return out


def round_bf16(v: float) -> int:
    """bf16 bits of the double v, rounded to nearest, ties to even, in one step."""
    return lib().oracle_round_bf16(v)


def rmsnorm(x, gamma, eps, rows=None):
    """RMSNorm of the listed rows: bf16 bits [n, H] of (x * rstd) * gamma, rstd = 1 / sqrt(mean x^2 + eps)."""
    x, gamma = _bf16(x), _bf16(gamma)
    H = x.shape[1]
    rows, n = _rows_arg(rows, x.shape[0])
    out = np.empty((n, H), np.uint16)
    if lib().oracle_rmsnorm(H, eps, _p(x), _p(gamma), _p(rows), n, _p(out)) != 0:
        raise ValueError("oracle_rmsnorm rejected its arguments")
    return out


def _shared(inp):
    ws1 = inp.get("ws1")
    Is = 0 if ws1 is None or ws1.size == 0 else ws1.shape[0]
    if not Is:
        return 0, None, None, None
    return Is, _bf16(ws1), _bf16(inp["ws3"]), _bf16(inp["ws2"])


def block_forward(inp, gamma, eps, k, scale, rows=None):
    """The mixture half of a block on the residual stream inp["x"]: out = x' + mixture(RMSNorm(x')).
    Returns dict out, x_norm, ids, gates, gap for the listed tokens."""
    x, wr = _bf16(inp["x"]), _bf16(inp["wr"])
    gamma = _bf16(gamma)
    b = np.ascontiguousarray(inp["b"], dtype=np.float32)
    w1, w3, w2 = _bf16(inp["w1"]), _bf16(inp["w3"]), _bf16(inp["w2"])
    H, E, I = x.shape[1], wr.shape[0], w1.shape[1]
    Is, ws1, ws3, ws2 = _shared(inp)
    rows, n = _rows_arg(rows, x.shape[0])
    out = np.empty((n, H), np.float32)
    xn = np.empty((n, H), np.uint16)
    ids = np.empty((n, k), np.int32)
    gates = np.empty((n, k), np.float32)
    gap = np.empty(n, np.float64)
    rc = lib().oracle_block_forward(H, E, k, I, Is, scale, eps, _p(x), _p(gamma), _p(wr), _p(b), _p(w1), _p(w3),
                                    _p(w2), _p(ws1), _p(ws3), _p(ws2), _p(rows), n, _p(out), _p(xn), _p(ids),
                                    _p(gates), _p(gap))
    if rc != 0:
        raise ValueError("oracle_block_forward rejected its arguments")
    return {"out": out, "x_norm": xn, "ids": ids, "gates": gates, "gap": gap}


def dense_mlp(x, w1, w3, w2, rows=None):
    """Dense SwiGLU MLP of the listed rows: fp32 [n, H] of (silu(x W1) * (x W3)) W2, W1/W3 [Id, H], W2 [H, Id]."""
    x, w1, w3, w2 = _bf16(x), _bf16(w1), _bf16(w3), _bf16(w2)
    H, Id = x.shape[1], w1.shape[0]
    rows, n = _rows_arg(rows, x.shape[0])
    out = np.empty((n, H), np.float32)
    if lib().oracle_dense_mlp(H, Id, _p(x), _p(w1), _p(w3), _p(w2), _p(rows), n, _p(out)) != 0:
        raise ValueError("oracle_dense_mlp rejected its arguments")
    return out


def permute(ids, E):
    """Stable counting sort of the T*k slots by expert. Returns counts, offsets, row_token, slot_row."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_token = np.empty(T * k, np.int32)
    slot_row = np.empty(T * k, np.int32)
    rc = lib().oracle_permute(T, E, k, _p(ids), _p(counts), _p(offsets), _p(row_token), _p(slot_row))
    if rc != 0:
        raise ValueError("oracle_permute: expert id out of range")
    return {"counts": counts, "offsets": offsets, "row_token": row_token, "slot_row": slot_row}


def host_threads() -> int:
    """Host threads the oracle runs on: the job's granted CPU share when OMP_NUM_THREADS states one, else
    every core this process may run on (its CPU affinity)."""
    try:
        n = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        n = 0
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(n, avail) if n > 0 else avail)


def host_description() -> dict:
    """What the oracle's host is: the threads it uses, the logical CPUs of the machine and of this process's
    affinity, and the CPU model from /proc/cpuinfo."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"threads": host_threads(), "nproc": os.cpu_count(), "affinity": affinity, "cpu_model": model}


def run_sharded(fn, rows, nthreads=None, **kw):
    """Run fn(rows=chunk, **kw) over contiguous chunks of `rows` on host threads and concatenate the dict
    results along axis 0. The per-chunk code is the plain single-threaded oracle."""
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    nthreads = nthreads or host_threads()
    nthreads = max(1, min(nthreads, rows.size))
    chunks = [c for c in np.array_split(rows, nthreads) if c.size]
    with ThreadPoolExecutor(max_workers=len(chunks)) as ex:
        parts = list(ex.map(lambda c: fn(rows=c, **kw), chunks))
    if isinstance(parts[0], dict):
        return {key: np.concatenate([p[key] for p in parts], axis=0) for key in parts[0]}
    return np.concatenate(parts, axis=0)
