"""The C ABI on the host: libmoe.so loads, exports every function include/moe.h declares, and its argument
checks return the documented status before anything touches a GPU (CPU only)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]
LIB = os.path.join(ROOT, "sigmoid_routed_mixture_amd", "libmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe.so not built")

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, HIP = range(6)


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"moe_route", "moe_permute", "moe_forward", "moe_workspace_bytes"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_[a-z_]+)\b", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n)


def test_binding_names_match_header():
    import sigmoid_routed_mixture_amd as m

    for n in declared_functions():
        assert n in m.EXPORTED_SYMBOLS
        if n not in ("moe_status_string", "moe_last_error"):
            assert callable(getattr(m, n))


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(LIB)
    p, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.moe_workspace_bytes.argtypes = [i] * 6
    L.moe_workspace_bytes.restype = sz
    L.moe_permute_workspace_bytes.argtypes = [i, i]
    L.moe_permute_workspace_bytes.restype = sz
    L.moe_route.argtypes = [p, p, p, i, i, i, i, f, p, p, p, p]
    L.moe_permute.argtypes = [p, p, i, i, i, i, p, p, p, p, p, p, sz, p]
    L.moe_forward.argtypes = [p] * 9 + [i] * 6 + [f] + [p] * 5 + [sz, p, p]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.restype = ctypes.c_char_p
    d = ctypes.c_double
    L.moe_forward_routed.argtypes = [p] * 9 + [i] * 6 + [p, p, p, sz, p, p]
    L.moe_block_workspace_bytes.argtypes = [i] * 6
    L.moe_block_workspace_bytes.restype = sz
    L.moe_block_forward.argtypes = [p, p, d] + [p] * 8 + [i] * 6 + [f] + [p] * 6 + [sz, p, p]
    L.moe_dense_mlp_workspace_bytes.argtypes = [i] * 3
    L.moe_dense_mlp_workspace_bytes.restype = sz
    L.moe_dense_mlp.argtypes = [p] * 4 + [i] * 3 + [p, p, sz, p]
    return L


A = 0x10000  # aligned fake device address: never dereferenced by a call that fails its checks


def route(L, T=64, H=256, E=16, k=4, x=A, wr=A, b=A, ids=A, gates=A, logits=None):
    return L.moe_route(x, wr, b, T, H, E, k, 2.5, ids, gates, logits, None)


def forward(L, T=64, H=256, E=16, k=4, I=128, Is=128, ws_bytes=None, **ptrs):
    P = dict(x=A, wr=A, b=A, w1=A, w3=A, w2=A, ws1=A, ws3=A, ws2=A, out=A, ids=None, gates=None, counts=None,
             ws=0x100000)
    P.update(ptrs)
    if ws_bytes is None:
        ws_bytes = L.moe_workspace_bytes(max(T, 0), H, E, k, I, Is)
    return L.moe_forward(P["x"], P["wr"], P["b"], P["w1"], P["w3"], P["w2"], P["ws1"], P["ws3"], P["ws2"], T, H,
                         E, k, I, Is, 2.5, P["out"], P["ids"], P["gates"], P["counts"], P["ws"], ws_bytes, None, None)


def test_status_strings(lib):
    assert lib.moe_status_string(OK) == b"ok"
    assert lib.moe_status_string(WORKSPACE) == b"workspace too small"
    assert lib.moe_status_string(99) == b"unknown status"


def test_workspace_bytes(lib):
    small = lib.moe_workspace_bytes(64, 256, 16, 4, 128, 128)
    big = lib.moe_workspace_bytes(8192, 6144, 256, 8, 2048, 2048)
    assert 0 < small < big
    # at least the per-slot activations and outputs it must hold
    assert big >= 8192 * 8 * (2048 + 6144) * 2
    assert lib.moe_workspace_bytes(64, 256, 16, 4, 128, 0) < small
    assert lib.moe_workspace_bytes(64, 250, 16, 4, 128, 128) == 0  # H not a multiple of 64
    assert lib.moe_workspace_bytes(64, 256, 300, 4, 128, 128) == 0  # E > 256
    assert lib.moe_permute_workspace_bytes(1000, 64) >= 4 * 64 * 4


@pytest.mark.parametrize("shape", [(6144, 256, 8, 2048, 2048), (2048, 64, 4, 1536, 1536), (256, 16, 4, 128, 128)])
def test_workspace_queries_never_shrink_with_T(lib, shape):
    # a workspace sized for the largest batch must serve every smaller one: the layout loses regions as T
    # grows (the decode K split past 64 tokens, the folded shared expert), so the queries take the largest
    H, E, k, I, Is = shape
    for q, args in ((lib.moe_workspace_bytes, (H, E, k, I, Is)), (lib.moe_block_workspace_bytes, (H, E, k, I, Is)),
                    (lib.moe_dense_mlp_workspace_bytes, (H, I))):
        sizes = [q(T, *args) for T in range(0, 1200)]
        assert all(b >= a for a, b in zip(sizes, sizes[1:])), q.__name__


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), INVALID), (dict(H=0), INVALID), (dict(E=0), INVALID), (dict(k=0), INVALID),
    (dict(k=17), INVALID), (dict(E=300, k=4), UNSUPPORTED), (dict(E=64, k=33), UNSUPPORTED),
    (dict(H=100), UNSUPPORTED), (dict(x=None), INVALID), (dict(b=None), INVALID), (dict(ids=None), INVALID),
    (dict(x=A + 2), MISALIGNED), (dict(gates=A + 8), MISALIGNED), (dict(logits=A + 4), MISALIGNED),
    (dict(T=0), OK),
])
def test_route_argument_checks(lib, kw, status):
    assert route(lib, **kw) == status
    if status != OK:
        assert lib.moe_last_error() != b""


@pytest.mark.parametrize("kw,status", [
    (dict(I=0), INVALID), (dict(Is=-64), INVALID), (dict(I=100), UNSUPPORTED), (dict(Is=96), UNSUPPORTED),
    (dict(w2=None), INVALID), (dict(out=None), INVALID), (dict(ws=None), INVALID), (dict(ws1=None), INVALID),
    (dict(w1=A + 8), MISALIGNED), (dict(ws=0x100000 + 16), MISALIGNED), (dict(counts=A + 4), MISALIGNED),
    (dict(ws_bytes=1024), WORKSPACE), (dict(T=0), OK), (dict(T=0, ws1=None, ws3=None, ws2=None, Is=0), OK),
    (dict(T=1 << 28, k=8), UNSUPPORTED),
])
def test_forward_argument_checks(lib, kw, status):
    assert forward(lib, **kw) == status


def test_permute_argument_checks(lib):
    L = lib
    ws = 0x100000
    nb = L.moe_permute_workspace_bytes(64, 16)
    assert L.moe_permute(None, A, 0, 256, 16, 4, A, A, A, A, None, ws, nb, None) == OK
    assert L.moe_permute(None, None, 64, 256, 16, 4, A, A, A, A, None, ws, nb, None) == INVALID
    assert L.moe_permute(None, A, 64, 256, 16, 4, A, A, A, A, A, ws, nb, None) == INVALID  # x_perm needs x
    assert L.moe_permute(None, A, 64, 256, 16, 4, A, A, A, A, None, ws, 4, None) == WORKSPACE
    assert L.moe_permute(None, A, 64, 256, 16, 4, A, A, A, A, None, ws + 64, nb, None) == MISALIGNED


def routed(L, T=64, H=256, E=16, k=4, I=128, Is=128, ws_bytes=None, **ptrs):
    P = dict(x=A, ids=A, gates=A, w1=A, w3=A, w2=A, ws1=A, ws3=A, ws2=A, out=A, counts=None, ws=0x100000)
    P.update(ptrs)
    if ws_bytes is None:
        ws_bytes = L.moe_workspace_bytes(max(T, 0), H, E, k, I, Is)
    return L.moe_forward_routed(P["x"], P["ids"], P["gates"], P["w1"], P["w3"], P["w2"], P["ws1"], P["ws3"],
                                P["ws2"], T, H, E, k, I, Is, P["out"], P["counts"], P["ws"], ws_bytes, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ids=None), INVALID), (dict(gates=None), INVALID), (dict(x=None), INVALID), (dict(w3=None), INVALID),
    (dict(gates=A + 4), MISALIGNED), (dict(I=96), UNSUPPORTED), (dict(ws_bytes=4096), WORKSPACE),
    (dict(T=0), OK), (dict(T=0, ids=None, gates=None), OK), (dict(k=17), INVALID),
])
def test_forward_routed_argument_checks(lib, kw, status):
    assert routed(lib, **kw) == status


def block(L, T=64, H=256, E=16, k=4, I=128, Is=128, eps=1e-5, ws_bytes=None, **ptrs):
    P = dict(resid=A, gamma=A, wr=A, b=A, w1=A, w3=A, w2=A, ws1=A, ws3=A, ws2=A, out=A, xn=None, ids=None,
             gates=None, counts=None, ws=0x100000)
    P.update(ptrs)
    if ws_bytes is None:
        ws_bytes = L.moe_block_workspace_bytes(max(T, 0), H, E, k, I, Is)
    return L.moe_block_forward(P["resid"], P["gamma"], eps, P["wr"], P["b"], P["w1"], P["w3"], P["w2"], P["ws1"],
                               P["ws3"], P["ws2"], T, H, E, k, I, Is, 2.5, P["out"], P["xn"], P["ids"], P["gates"],
                               P["counts"], P["ws"], ws_bytes, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(resid=None), INVALID), (dict(gamma=None), INVALID), (dict(eps=-1.0), INVALID),
    (dict(eps=float("nan")), INVALID), (dict(eps=float("inf")), INVALID), (dict(xn=A + 2), MISALIGNED),
    (dict(wr=None), INVALID), (dict(H=100), UNSUPPORTED), (dict(T=0), OK), (dict(T=0, eps=-1.0), INVALID),
])
def test_block_forward_argument_checks(lib, kw, status):
    assert block(lib, **kw) == status


def test_block_workspace_holds_the_normalised_stream(lib):
    for T, H, E, k, I, Is in ((64, 256, 16, 4, 128, 128), (8192, 6144, 256, 8, 2048, 2048)):
        plain = lib.moe_workspace_bytes(T, H, E, k, I, Is)
        assert lib.moe_block_workspace_bytes(T, H, E, k, I, Is) >= plain + T * H * 2
        # the plain workspace is too small for the block entry point
        assert block(lib, T=T, H=H, E=E, k=k, I=I, Is=Is, ws_bytes=plain) == WORKSPACE


def test_dense_mlp_argument_checks(lib):
    L = lib
    ws = 0x100000
    nb = L.moe_dense_mlp_workspace_bytes(64, 256, 384)
    assert nb >= 64 * 384 * 2
    assert L.moe_dense_mlp_workspace_bytes(64, 250, 384) == 0
    assert L.moe_dense_mlp_workspace_bytes(64, 256, 100) == 0
    assert L.moe_dense_mlp(None, A, A, A, 64, 256, 384, A, ws, nb, None) == INVALID
    assert L.moe_dense_mlp(A, A, None, A, 64, 256, 384, A, ws, nb, None) == INVALID
    assert L.moe_dense_mlp(A, A, A, A, 64, 256, 384, None, ws, nb, None) == INVALID
    assert L.moe_dense_mlp(A, A, A, A, 64, 256, 384, A, ws, 16, None) == WORKSPACE
    assert L.moe_dense_mlp(A, A, A, A, 64, 256, 384, A, ws + 16, nb, None) == MISALIGNED
    assert L.moe_dense_mlp(A + 2, A, A, A, 64, 256, 384, A, ws, nb, None) == MISALIGNED
    assert L.moe_dense_mlp(A, A, A, A, -1, 256, 384, A, ws, nb, None) == INVALID
    assert L.moe_dense_mlp(A, A, A, A, 64, 256, 96, A, ws, nb, None) == UNSUPPORTED
    assert L.moe_dense_mlp(None, None, None, None, 0, 256, 384, None, None, 0, None) == OK


def test_tuning_knobs_set_get_and_reject_out_of_range(lib):
    # include/moe_tuning.h: process-wide knobs, 0 = the size rules; bad knobs or values change nothing
    lib.moe_set_tuning.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.moe_get_tuning.argtypes = [ctypes.c_int]
    maxima = {0: 4, 1: 1, 2: 1, 3: 3, 4: 4, 5: 1, 6: 3, 7: 1, 8: 2}
    for knob, top in maxima.items():
        assert lib.moe_get_tuning(knob) == 0
        for v in range(top + 1):
            assert lib.moe_set_tuning(knob, v) == OK
            assert lib.moe_get_tuning(knob) == v
        assert lib.moe_set_tuning(knob, top + 1) == INVALID
        assert lib.moe_set_tuning(knob, -1) == INVALID
        assert lib.moe_get_tuning(knob) == top
        assert lib.moe_set_tuning(knob, 0) == OK
    assert lib.moe_set_tuning(9, 0) == INVALID
    assert lib.moe_get_tuning(9) == -1 and lib.moe_get_tuning(-1) == -1


def test_library_reads_no_environment():
    # every kernel choice comes from the sizes and the tuning knobs, never from the process environment
    out = subprocess.run(["nm", "-D", "--undefined-only", LIB], capture_output=True, text=True, check=True).stdout
    assert not re.search(r"\b(secure_)?getenv\b", out)
