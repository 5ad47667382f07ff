"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the five workloads and edge shapes.

The five workloads run at their full sizes in the launch configuration the benchmark times. Routing is
compared on every token; outputs on every token where the oracle is quick (tiny, mid sample, decode) and
on a seeded sample that covers every active expert elsewhere (tokens are independent, so a sample is a
faithful check of the rows it covers).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import (NEAR_TIE, case, compare_out, compare_routing, config_host, dev, dev_bf16,
                    oracle_forward_rows, oracle_route_all, route_ref, sample_rows, say, to_device)

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def moe():
    import sigmoid_routed_mixture_amd as m

    return m


def run_forward(m, cfg, d, stream_shared=None, T=None):
    T = cfg.T if T is None else T
    out = torch.empty(T, cfg.H, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, cfg.k, dtype=torch.float32, device="cuda")
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    nbytes = m.moe_workspace_bytes(T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.Is)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    x = d["x"][:T]
    m.moe_forward(x, d["wr"], d["b"], d["w1"], d["w3"], d["w2"], d.get("ws1"), d.get("ws3"), d.get("ws2"), cfg.k,
                  cfg.scale, out, ws, ids, gates, counts, stream_shared=stream_shared)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), gates.cpu().numpy(), counts.cpu().numpy()


ALL = [c.name for c in wl.CONFIGS]


@pytest.mark.parametrize("name", ALL)
def test_route_parity(moe, name):
    say("[route] %s" % name)
    cfg, h, d = case(name)
    ref = route_ref(name)
    ids = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device="cuda")
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda")
    moe.moe_route(d["x"], d["wr"], d["b"], cfg.k, cfg.scale, ids, gates, logits)
    torch.cuda.synchronize()
    same, nnear, ndiff = compare_routing(ids.cpu().numpy(), gates.cpu().numpy(), ref, name)
    say("  near-tie tokens: %d (of %d), %d of them chose differently" % (nnear, cfg.T, ndiff))
    # logits: fp32 accumulation against the exact value rounded once
    rows = np.arange(0, cfg.T, max(1, cfg.T // 256), dtype=np.int32)
    zref = oracle.route(h["x"], h["wr"], h["b"], cfg.k, cfg.scale, rows=rows, want_logits=True)["logits"]
    dz = np.abs(logits.cpu().numpy()[rows] - zref)
    say("  max |z_gpu - z_oracle| = %.3e" % dz.max())
    assert dz.max() <= 1e-4 * max(1.0, np.abs(zref).max())


@pytest.mark.parametrize("name", ALL)
def test_permute_parity(moe, name):
    say("[permute] %s" % name)
    cfg, h, d = case(name)
    ids = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device="cuda")
    moe.moe_route(d["x"], d["wr"], d["b"], cfg.k, cfg.scale, ids, gates)
    Tk = cfg.T * cfg.k
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda")
    row_token = torch.empty(Tk, dtype=torch.int32, device="cuda")
    slot_row = torch.empty(Tk, dtype=torch.int32, device="cuda")
    x_perm = torch.empty(Tk, cfg.H, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_permute_workspace_bytes(cfg.T, cfg.E), dtype=torch.uint8, device="cuda")
    moe.moe_permute(ids, cfg.E, counts, offsets, row_token, slot_row, ws, x=d["x"], x_perm=x_perm)
    torch.cuda.synchronize()
    ref = oracle.permute(ids.cpu().numpy(), cfg.E)
    for key, t in (("counts", counts), ("offsets", offsets), ("row_token", row_token), ("slot_row", slot_row)):
        assert np.array_equal(t.cpu().numpy(), ref[key]), "%s differs" % key
    assert torch.equal(x_perm, d["x"][row_token.long()])
    say("  active experts: %d, largest %d rows, empty %d" % (
        (ref["counts"] > 0).sum(), ref["counts"].max(), (ref["counts"] == 0).sum()))


SAMPLE = {"tiny": None, "mid": 512, "glm5_decode": None, "glm5_prefill": 96, "glm5_skewed": 64,
          "glm47_decode": None, "glm47_prefill": 256}


@pytest.mark.parametrize("name", ALL)
def test_forward_parity(moe, name):
    say("[forward] %s" % name)
    cfg, h, d = case(name)
    ref = route_ref(name)
    out, ids, gates, counts = run_forward(moe, cfg, d)
    same, nnear, ndiff = compare_routing(ids, gates, ref, name)
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=cfg.E))
    if ndiff == 0:
        assert np.array_equal(counts, np.bincount(ref["ids"].ravel(), minlength=cfg.E))
    n = SAMPLE[name]
    rows = np.arange(cfg.T, dtype=np.int32) if n is None else sample_rows(ref["ids"], n, seed=cfg.index)
    rows = rows[same[rows]]
    say("  oracle forward on %d tokens (near-tie %d, differing %d)" % (rows.size, nnear, ndiff))
    orc = oracle_forward_rows(h, cfg.k, cfg.scale, rows)
    compare_out(out[rows], orc["out"], name)
    if name == "glm5_skewed":
        assert counts[0] == cfg.T and np.all(counts[59:] == 0)


@pytest.mark.parametrize("name", ["tiny", "glm5_decode", "glm47_decode"])
@pytest.mark.parametrize("ks", ["1", "2"])
def test_decode_k_split(moe, monkeypatch, name, ks):
    # decode-sized grouped GEMMs (gate/up with its reduction, down with the combine adding the halves) with
    # the K split forced off and on, against the oracle on every token
    say("[K split %s] %s" % (ks, name))
    monkeypatch.setenv("MOE_KSPLIT", ks)
    cfg, h, d = case(name)
    ref = route_ref(name)
    out, ids, gates, counts = run_forward(moe, cfg, d)
    same, nnear, ndiff = compare_routing(ids, gates, ref, name)
    rows = np.arange(cfg.T, dtype=np.int32)[same]
    orc = oracle_forward_rows(h, cfg.k, cfg.scale, rows)
    compare_out(out[rows], orc["out"], "%s/ks%s" % (name, ks))


@pytest.mark.parametrize("name,T", [("tiny", 64), ("glm5_decode", 16), ("mid", 384)])
@pytest.mark.parametrize("path", ["wide", "tall", "dma", "skinny"])
def test_both_gemm_kernels(moe, monkeypatch, name, T, path):
    say("[gemm path %s] %s T=%d" % (path, name, T))
    monkeypatch.setenv("MOE_GEMM_PATH", path)
    cfg, h, d = case(name)
    out, ids, gates, counts = run_forward(moe, cfg, d, T=T)
    ref = oracle_forward_rows(h, cfg.k, cfg.scale, np.arange(T))
    same, _, _ = compare_routing(ids, gates, ref, name)
    compare_out(out[same], ref["out"][same], "%s/%s" % (name, path))


@pytest.mark.parametrize("name,T", [("mid", 700), ("glm47_prefill", 2048)])
def test_dma_kernel_matches_register_kernel_bitwise(moe, monkeypatch, name, T):
    # the LDS-copy kernel sums every accumulator in the register-streaming kernel's order
    say("[dma vs tall] %s T=%d" % (name, T))
    cfg, h, d = case(name)
    monkeypatch.setenv("MOE_GEMM_PATH", "tall")
    a = run_forward(moe, cfg, d, T=T)
    monkeypatch.setenv("MOE_GEMM_PATH", "dma")
    b = run_forward(moe, cfg, d, T=T)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_xcd_split_does_not_change_results(moe, monkeypatch):
    # the work-balanced and the block-count XCD split only reorder the same blocks
    say("[xcd split] mid")
    cfg, h, d = case("mid")
    a = run_forward(moe, cfg, d)
    monkeypatch.setenv("MOE_XCD_SPLIT", "count")
    b = run_forward(moe, cfg, d)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("name", ["mid", "glm47_prefill"])
def test_persistent_grid_does_not_change_results(moe, monkeypatch, name):
    # one workgroup per CU claiming blocks from the XCD counters (and from the back of other XCDs' ranges
    # once its own is used up) computes every block exactly as one workgroup per block does
    say("[persistent] %s" % name)
    cfg, h, d = case(name)
    a = run_forward(moe, cfg, d)
    monkeypatch.setenv("MOE_PERSIST", "0")
    b = run_forward(moe, cfg, d)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("name", ["tiny", "glm5_decode", "mid"])
def test_second_stream_and_determinism(moe, name):
    say("[streams] %s" % name)
    cfg, h, d = case(name)
    a = run_forward(moe, cfg, d)
    s1 = torch.cuda.Stream()
    b = run_forward(moe, cfg, d, stream_shared=s1)
    c = run_forward(moe, cfg, d)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    for x, y in zip(a, c):
        assert np.array_equal(x, y)


def test_second_stream_with_dense_shared_expert(moe):
    # Is != I: the shared expert runs as a dense MLP of its own, on the second stream when one is given
    say("[streams] Is != I")
    cfg = wl.MoEConfig(52, "dense_shared", T=1000, H=256, E=32, k=2, I=128, Is=320, scale=2.5)
    h = config_host(cfg)
    d = to_device(h)
    a = run_forward(moe, cfg, d)
    b = run_forward(moe, cfg, d, stream_shared=torch.cuda.Stream())
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    ref = oracle_forward_rows(h, cfg.k, cfg.scale, np.arange(0, cfg.T, 5))
    same, _, _ = compare_routing(a[1][::5], a[2][::5], ref, "dense_shared")
    compare_out(a[0][::5][same], ref["out"][same], "dense_shared")


def test_crafted_ties_on_gpu(moe):
    path = os.path.join(os.path.dirname(__file__), "golden", "tie_cases.json")
    cases = json.load(open(path))["cases"]
    for c in cases:
        say("[ties] E=%d k=%d" % (c["E"], c["k"]))
        T, H = 40, 64
        x = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
        wr = dev_bf16(wl.normal_bf16(11, 1, 0.02, 0, c["E"] * H).reshape(c["E"], H))
        b = dev(np.array(c["b"], np.float32))
        ids = torch.empty(T, c["k"], dtype=torch.int32, device="cuda")
        gates = torch.empty(T, c["k"], dtype=torch.float32, device="cuda")
        moe.moe_route(x, wr, b, c["k"], c["scale"], ids, gates)
        torch.cuda.synchronize()
        assert np.all(ids.cpu().numpy() == np.array(c["ids"])[None, :])
        assert np.allclose(gates.cpu().numpy(), c["gate"], rtol=1e-6)


EDGE = [
    # T, H, E, k, I, Is, what
    (1, 256, 16, 4, 128, 128, "one token"),
    (129, 192, 8, 8, 64, 0, "k = E, H % 128 = 64, no shared expert"),
    (300, 128, 1, 1, 64, 64, "one expert"),
    (1000, 256, 32, 1, 128, 192, "k = 1, Is != I, ragged T"),
    (257, 320, 24, 6, 192, 64, "E not a multiple of 16"),
]


@pytest.mark.parametrize("path", ["wide", "tall", "dma", "skinny"])
@pytest.mark.parametrize("shape", EDGE, ids=[e[-1] for e in EDGE])
def test_edge_shapes(moe, monkeypatch, shape, path):
    T, H, E, k, I, Is, what = shape
    say("[edge %s] %s T=%d H=%d E=%d k=%d I=%d Is=%d" % (path, what, T, H, E, k, I, Is))
    monkeypatch.setenv("MOE_GEMM_PATH", path)
    cfg = wl.MoEConfig(50, "edge", T=T, H=H, E=E, k=k, I=I, Is=Is, scale=2.5)
    h = config_host(cfg)
    if Is == 0:
        for n in ("ws1", "ws3", "ws2"):
            h[n] = None
    d = to_device(h)
    out, ids, gates, counts = run_forward(moe, cfg, d)
    ref = oracle_forward_rows(h, k, cfg.scale, np.arange(T))
    same, _, _ = compare_routing(ids, gates, ref, what)
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    compare_out(out[same], ref["out"][same], what)


@pytest.mark.parametrize("path", ["wide", "tall", "dma", "skinny"])
def test_identical_tokens_one_giant_group(moe, monkeypatch, path):
    say("[giant group %s]" % path)
    monkeypatch.setenv("MOE_GEMM_PATH", path)
    cfg = wl.MoEConfig(51, "same", T=700, H=256, E=16, k=4, I=128, Is=128, scale=1.8)
    h = config_host(cfg)
    h["x"] = np.ascontiguousarray(np.repeat(h["x"][:1], cfg.T, axis=0))
    d = to_device(h)
    out, ids, gates, counts = run_forward(moe, cfg, d)
    assert np.sort(counts)[-cfg.k:].tolist() == [cfg.T] * cfg.k
    ref = oracle_forward_rows(h, cfg.k, cfg.scale, np.array([0]))
    compare_routing(ids[:1], gates[:1], ref, "same")
    compare_out(out, np.repeat(ref["out"], cfg.T, axis=0), "same")


@pytest.mark.parametrize("name", ["tiny", "glm5_decode", "mid"])
def test_graph_capture_replays_match_eager(moe, name):
    """The library neither allocates nor synchronises, so a forward pass can be captured in a HIP graph:
    every replay, with eager work and synchronisations between them, gives the eager bytes."""
    say("[graph capture] %s" % name)
    cfg, h, d = case(name)
    T = cfg.T
    out = torch.empty(T, cfg.H, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, cfg.k, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.Is), dtype=torch.uint8, device="cuda")
    args = (d["x"], d["wr"], d["b"], d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"], d["ws2"], cfg.k, cfg.scale, out, ws,
            ids, gates)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(2):
            moe.moe_forward(*args, stream=s)
    torch.cuda.synchronize()
    eager, eager_ids = out.clone(), ids.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_forward(*args, stream=s)
    torch.cuda.synchronize()
    other = run_forward(moe, cfg, d, T=max(1, T // 2))[0]
    for i in range(3):
        out.fill_(float("nan"))
        ids.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs" % i
        assert torch.equal(ids, eager_ids), "replay %d routed differently" % i
        assert np.array_equal(run_forward(moe, cfg, d, T=max(1, T // 2))[0], other)  # eager work in between


def test_zero_tokens_and_errors(moe):
    say("[zero tokens / errors]")
    cfg, h, d = case("tiny")
    out = torch.full((4, cfg.H), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    moe.moe_forward(d["x"][:0], d["wr"], d["b"], d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"], d["ws2"], cfg.k,
                    cfg.scale, out[:0], ws)  # zero-row views may carry a null data pointer
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    with pytest.raises(moe.MoEError) as e:
        ids = torch.empty(cfg.T * cfg.k + 1, dtype=torch.int32, device="cuda")[1:].view(cfg.T, cfg.k)
        gates = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device="cuda")
        moe.moe_route(d["x"], d["wr"], d["b"], cfg.k, cfg.scale, ids, gates)
    assert e.value.status == moe.MOE_ERR_MISALIGNED
    with pytest.raises(moe.MoEError) as e:
        moe.moe_forward(d["x"], d["wr"], d["b"], d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"], d["ws2"], cfg.k,
                        cfg.scale, torch.empty(cfg.T, cfg.H, device="cuda"), ws[:1024])
    assert e.value.status == moe.MOE_ERR_WORKSPACE
