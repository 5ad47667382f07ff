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
                    host_line, oracle_forward_rows, oracle_route_all, output_rows, route_ref, sample_rows, say,
                    to_device)

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def moe():
    import sigmoid_routed_mixture_amd as m

    return m


@pytest.fixture
def tune(moe):
    """Sets tuning knobs of include/moe_tuning.h by name; every knob is back at 0 after the test."""

    def set_knobs(**knobs):
        for name, value in knobs.items():
            moe.moe_set_tuning(getattr(moe, name), value)

    yield set_knobs
    for knob in range(moe.MOE_TUNE_KNOBS):
        moe.moe_set_tuning(knob, 0)


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


# Outputs on every token where the oracle takes well under a minute on the host's threads; on the two
# largest GLM-5 batches a seeded sample of parity.SAMPLE_FLOOR tokens plus every expert's first and last
# token and the tokens on both sides of each of its tile boundaries.
FULL_OUTPUT = {"tiny": True, "mid": True, "glm5_decode": True, "glm5_prefill": False, "glm5_skewed": False,
               "glm47_decode": True, "glm47_prefill": True}


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
    rows = output_rows(cfg.T, ref["ids"], cfg.index, FULL_OUTPUT[name])
    rows = rows[same[rows]]
    say("  %s; oracle forward on %d of %d tokens (near-tie %d, differing %d)" % (
        host_line(), rows.size, cfg.T, nnear, ndiff))
    orc = oracle_forward_rows(h, cfg.k, cfg.scale, rows)
    compare_out(out[rows], orc["out"], name)
    if name == "glm5_skewed":
        assert counts[0] == cfg.T and np.all(counts[59:] == 0)


@pytest.mark.parametrize("name", ["tiny", "glm5_decode", "glm47_decode"])
@pytest.mark.parametrize("ks", ["1", "2", "3"])
def test_decode_k_split(moe, tune, name, ks):
    # decode-sized grouped GEMMs (gate/up with its reduction, down with the combine adding the ranges) with
    # the K split forced off, in two, and to the largest split allowed (down: up to four ranges at these
    # batch sizes), against the oracle on every token
    say("[K split %s] %s" % (ks, name))
    tune(MOE_TUNE_KSPLIT=int(ks))
    cfg, h, d = case(name)
    ref = route_ref(name)
    out, ids, gates, counts = run_forward(moe, cfg, d)
    same, nnear, ndiff = compare_routing(ids, gates, ref, name)
    rows = np.arange(cfg.T, dtype=np.int32)[same]
    orc = oracle_forward_rows(h, cfg.k, cfg.scale, rows)
    compare_out(out[rows], orc["out"], "%s/ks%s" % (name, ks))


@pytest.mark.parametrize("name,T", [("tiny", 64), ("glm5_decode", 16), ("mid", 384)])
@pytest.mark.parametrize("path", ["wide", "tall", "dma", "skinny"])
def test_both_gemm_kernels(moe, tune, name, T, path):
    say("[gemm path %s] %s T=%d" % (path, name, T))
    tune(MOE_TUNE_GEMM_PATH=moe.GEMM_PATHS[path])
    cfg, h, d = case(name)
    out, ids, gates, counts = run_forward(moe, cfg, d, T=T)
    ref = oracle_forward_rows(h, cfg.k, cfg.scale, np.arange(T))
    same, _, _ = compare_routing(ids, gates, ref, name)
    compare_out(out[same], ref["out"][same], "%s/%s" % (name, path))


@pytest.mark.parametrize("name,T", [("mid", 700), ("glm47_prefill", 2048)])
def test_dma_kernel_matches_register_kernel_bitwise(moe, tune, name, T):
    # the LDS-copy kernel sums every accumulator in the register-streaming kernel's order
    say("[dma vs tall] %s T=%d" % (name, T))
    cfg, h, d = case(name)
    tune(MOE_TUNE_GEMM_PATH=moe.GEMM_PATHS["tall"])
    a = run_forward(moe, cfg, d, T=T)
    tune(MOE_TUNE_GEMM_PATH=moe.GEMM_PATHS["dma"])
    b = run_forward(moe, cfg, d, T=T)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_xcd_split_does_not_change_results(moe, tune):
    # the work-balanced and the block-count XCD split only reorder the same blocks
    say("[xcd split] mid")
    cfg, h, d = case("mid")
    a = run_forward(moe, cfg, d)
    tune(MOE_TUNE_XCD_SPLIT=1)
    b = run_forward(moe, cfg, d)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("name", ["mid", "glm47_prefill", "glm5_prefill", "glm5_skewed"])
def test_block_order_does_not_change_results(moe, tune, name):
    # every block order of the persistent GEMMs (index order in long or short chunks, the dealt orders) runs
    # the same blocks, each computing exactly what it computes in the others
    say("[block order] %s" % name)
    cfg, h, d = case(name)
    a = run_forward(moe, cfg, d)
    for order in range(1, 5):
        tune(MOE_TUNE_ORDER=order)
        b = run_forward(moe, cfg, d)
        for x, y in zip(a, b):
            assert np.array_equal(x, y), "order %d" % order


@pytest.mark.parametrize("name", ["mid", "glm47_prefill", "glm5_prefill"])
def test_prefill_shared_fold_matches_dense_mlp_bitwise(moe, tune, name):
    # above the decode sizes the shared expert runs as one more group of the persistent routed GEMMs (its
    # tiles spread over the XCDs, fp32 rows of its own); its tiles compute exactly what the dense MLP's do
    say("[shared fold] %s" % name)
    cfg, h, d = case(name)
    a = run_forward(moe, cfg, d)
    tune(MOE_TUNE_SHARED=1)
    b = run_forward(moe, cfg, d)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("name,T", [("tiny", 32), ("glm5_decode", 16), ("glm47_decode", 16), ("glm5_decode", 3)])
def test_decode_copy_ring_does_not_change_results(moe, tune, name, T):
    # up to 32 tokens the grouped GEMMs copy three K steps ahead, streamed (one workgroup per CU running its
    # blocks back to back) where the launch allows it; every tile computes what the two-step ring computes, bit
    # for bit, and so does the three-step ring with one workgroup per block
    say("[copy ring] %s T=%d" % (name, T))
    cfg, h, d = case(name)
    tune(MOE_TUNE_STREAMK=1)  # whole blocks in every ring (stream-K cuts blocks where the ring streams)
    a = run_forward(moe, cfg, d, T=T)
    for ring in (1, 2, 3):
        tune(MOE_TUNE_RING=ring)
        b = run_forward(moe, cfg, d, T=T)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("name,T,ks", [("glm5_decode", 16, 1), ("glm5_decode", 16, 2), ("glm5_decode", 16, 3),
                                       ("glm5_decode", 1, 0), ("glm47_decode", 16, 1), ("glm47_decode", 16, 2),
                                       ("glm47_decode", 16, 3), ("glm47_decode", 5, 0)])
def test_streamed_decode_gemms(moe, tune, name, T, ks):
    # the streamed GEMMs with the K split forced off and on (the gate/up halves then go through the reduction,
    # the down halves through the combine), one token (fewer blocks than CUs) and the batch sizes of decode:
    # bit for bit what one workgroup per block computes, and within the bar of the oracle
    say("[streamed] %s T=%d ksplit knob %d" % (name, T, ks))
    cfg, h, d = case(name)
    tune(MOE_TUNE_KSPLIT=ks, MOE_TUNE_RING=3, MOE_TUNE_STREAMK=1)
    a = run_forward(moe, cfg, d, T=T)
    tune(MOE_TUNE_RING=2)
    b = run_forward(moe, cfg, d, T=T)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    ref = oracle_forward_rows(h, cfg.k, cfg.scale, np.arange(T))
    same, _, _ = compare_routing(a[1], a[2], ref, name)
    compare_out(a[0][same], ref["out"][same], "%s streamed T=%d" % (name, T))


STREAMK = [
    # workload or shape, batch, what
    ("glm47_decode", 16, "GLM-4.7-Flash decode (its default: both GEMMs streamed with stream-K)"),
    ("glm5_decode", 16, "GLM-5 decode, streamed by the ring knob (about 5 blocks per CU)"),
    ((24, 2048, 96, 6, 1024), 24, "E 96, k 6, I 1024: gate/up K of 32 steps, down K of 16"),
    ((16, 2048, 64, 8, 1536), 16, "E 64, k 8, I 1536: down K of 24 steps (6 ring periods)"),
]


@pytest.mark.parametrize("knob", [0, 2])
@pytest.mark.parametrize("case_", STREAMK, ids=[c[-1].split(":")[0] for c in STREAMK])
def test_streamk_decode_gemms(moe, tune, case_, knob):
    # streamed decode GEMMs with stream-K (each workgroup one contiguous share of all blocks' K steps, the
    # blocks cut between two workgroups summed from two fp32 planes by the combine, and with knob value 2 the
    # gate/up GEMM's too, by its reduction): deterministic, within the bar of the oracle on every token, and
    # not bitwise the whole-block result (so the cut blocks really ran)
    name, T, what = case_
    say("[stream-K, knob %d] %s T=%d" % (knob, what, T))
    if isinstance(name, str):
        cfg, h, d = case(name)
    else:
        Tc, H, E, k, I = name
        cfg = wl.MoEConfig(54, "streamk", T=Tc, H=H, E=E, k=k, I=I, Is=I, scale=2.5)
        h = config_host(cfg)
        d = to_device(h)
    tune(MOE_TUNE_RING=3, MOE_TUNE_STREAMK=knob)
    a = run_forward(moe, cfg, d, T=T)
    b = run_forward(moe, cfg, d, T=T)
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "stream-K is not deterministic"
    tune(MOE_TUNE_STREAMK=1)
    c = run_forward(moe, cfg, d, T=T)
    assert np.array_equal(a[1], c[1]) and np.array_equal(a[3], c[3])  # routing untouched
    # both GEMMs have at least as many blocks as CUs (the folded shared expert is one more group), so both
    # take stream-K
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    groups = int((a[3] > 0).sum()) + 1
    blocks = (groups * 2 * cfg.I // 256, groups * ((cfg.H + 255) // 256))
    say("  %d groups: %d gate/up and %d down blocks on %d CUs" % (groups, blocks[0], blocks[1], cus))
    assert min(blocks) >= cus, "the shape has too few blocks for stream-K"
    assert not np.array_equal(a[0], c[0]), "stream-K did not run (outputs bitwise the whole-block ones)"
    ref = oracle_forward_rows(h, cfg.k, cfg.scale, np.arange(T))
    same, _, _ = compare_routing(a[1], a[2], ref, what)
    compare_out(a[0][same], ref["out"][same], "%s stream-K" % what)
    compare_out(c[0][same], ref["out"][same], "%s whole blocks" % what)


@pytest.mark.parametrize("name", ["tiny", "glm47_decode"])
def test_profiled_entry_matches_forward(moe, name):
    # moe_forward_profiled computes what moe_forward computes, with events at every stage boundary or only
    # around the gate/up launch (null entries record nothing), and its stage intervals add up to the pass
    say("[profiled] %s" % name)
    cfg, h, d = case(name)
    a = run_forward(moe, cfg, d)
    for pick in (range(7), (0, 3, 4)):
        ev = [torch.cuda.Event(enable_timing=True) if i in pick else None for i in range(7)]
        for e in ev:
            if e is not None:
                e.record()
        torch.cuda.synchronize()
        out = torch.empty(cfg.T, cfg.H, dtype=torch.float32, device="cuda")
        ws = torch.empty(moe.moe_workspace_bytes(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.Is), dtype=torch.uint8,
                         device="cuda")
        moe.moe_forward_profiled(d["x"], d["wr"], d["b"], d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"], d["ws2"],
                                 cfg.k, cfg.scale, out, ws, ev)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), a[0])
        marks = [e for e in ev if e is not None]
        spans = [marks[i].elapsed_time(marks[i + 1]) for i in range(len(marks) - 1)]
        assert min(spans) >= 0.0


@pytest.mark.parametrize("name", ["mid", "glm47_prefill"])
def test_persistent_grid_does_not_change_results(moe, tune, name):
    # one workgroup per CU claiming blocks from the XCD counters (and from the back of other XCDs' ranges
    # once its own is used up) computes every block exactly as one workgroup per block does
    say("[persistent] %s" % name)
    cfg, h, d = case(name)
    a = run_forward(moe, cfg, d)
    tune(MOE_TUNE_PERSIST=1)
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
def test_edge_shapes(moe, tune, shape, path):
    T, H, E, k, I, Is, what = shape
    say("[edge %s] %s T=%d H=%d E=%d k=%d I=%d Is=%d" % (path, what, T, H, E, k, I, Is))
    tune(MOE_TUNE_GEMM_PATH=moe.GEMM_PATHS[path])
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


SMALL_ROUTER = [
    # T, H, E, k: decode-sized router shapes of moe_forward (K-split logits of few experts, then the top-k)
    (1, 64, 1, 1),      # one expert, one K range
    (5, 2048, 24, 3),   # E not a multiple of 16
    (16, 6144, 64, 8),  # the longest K ranges
    (16, 2048, 64, 4),  # the GLM-4.7-Flash decode shape
]


@pytest.mark.parametrize("shape", SMALL_ROUTER, ids=["T%d_H%d_E%d_k%d" % s for s in SMALL_ROUTER])
def test_small_router_shapes(moe, shape):
    # ids and gates of moe_forward at decode sizes against the oracle (exact apart from counted near-ties), and
    # the layer's outputs within the bar
    T, H, E, k = shape
    say("[small router] T=%d H=%d E=%d k=%d" % shape)
    cfg = wl.MoEConfig(53, "small_router", T=T, H=H, E=E, k=k, I=64, Is=64, scale=1.8)
    h = config_host(cfg)
    d = to_device(h)
    out, ids, gates, counts = run_forward(moe, cfg, d)
    ref = oracle_forward_rows(h, k, cfg.scale, np.arange(T))
    same, _, _ = compare_routing(ids, gates, ref, "small router")
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    compare_out(out[same], ref["out"][same], "small router")


def forward_into(m, cfg, d, T, ws):
    """moe_forward of the first T tokens on the caller's workspace `ws` (sized for any T up to its own)."""
    out = torch.empty(T, cfg.H, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, cfg.k, dtype=torch.float32, device="cuda")
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    m.moe_forward(d["x"][:T], d["wr"], d["b"], d["w1"], d["w3"], d["w2"], d.get("ws1"), d.get("ws3"), d.get("ws2"),
                  cfg.k, cfg.scale, out, ws, ids, gates, counts)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), gates.cpu().numpy(), counts.cpu().numpy()


ROUTE_PERMUTE = ["glm5_decode", "glm47_decode"] + ["T%d_H%d_E%d_k%d" % s for s in SMALL_ROUTER]


@pytest.mark.parametrize("name", ROUTE_PERMUTE)
def test_route_permute_one_launch_matches_two(moe, tune, name):
    # up to 16 tokens the router's top-k and the permutation run as one launch whose last workgroup permutes
    # every token: bit for bit the two launches, over several batch sizes in a row on one workspace (each
    # call's logits kernel zeroes the ticket the last workgroup is found by; the first call finds whatever
    # the fresh workspace held), and within the bar of the oracle
    if name in wl.BY_NAME:
        cfg, h, d = case(name)
    else:
        T, H, E, k = next(s for s in SMALL_ROUTER if "T%d_H%d_E%d_k%d" % s == name)
        cfg = wl.MoEConfig(53, "small_router", T=T, H=H, E=E, k=k, I=64, Is=64, scale=1.8)
        h = config_host(cfg)
        d = to_device(h)
    sizes = [cfg.T, 1, max(1, cfg.T // 2), 3, cfg.T]
    say("[route+permute] %s, batches %s" % (name, sizes))
    nbytes = moe.moe_workspace_bytes(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.Is)
    ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
    for T in sizes:
        tune(MOE_TUNE_ROUTE_PERMUTE=0)
        a = forward_into(moe, cfg, d, T, ws)
        tune(MOE_TUNE_ROUTE_PERMUTE=1)
        b = forward_into(moe, cfg, d, T, ws)
        for x, y, what in zip(a, b, ("out", "ids", "gates", "counts")):
            assert np.array_equal(x, y), "%s, T=%d: %s differs between one launch and two" % (name, T, what)
    out, ids, gates, counts = a
    ref = oracle_forward_rows(h, cfg.k, cfg.scale, np.arange(cfg.T))
    same, _, _ = compare_routing(ids, gates, ref, name)
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=cfg.E))
    compare_out(out[same], ref["out"][same], name)


STREAM_EDGE = [
    # T, H, E, k, I, what: decode-sized shapes whose K steps make whole ring periods (the streamed GEMMs run)
    (29, 1024, 24, 3, 512, "29 tokens, E 24, k 3"),
    (7, 512, 72, 2, 1024, "7 tokens, E 72, k 2"),
    (32, 1024, 40, 5, 512, "32 tokens, E 40, k 5"),
]


@pytest.mark.parametrize("ks", [0, 3])
@pytest.mark.parametrize("shape", STREAM_EDGE, ids=[e[-1] for e in STREAM_EDGE])
def test_streamed_edge_shapes(moe, tune, shape, ks):
    # the streamed decode GEMMs away from the GLM shapes (tiles of every height up to 32 rows, the folded shared
    # expert, the K split by size and the largest one): bit for bit the one-workgroup-per-block kernel, and
    # within the bar of the oracle
    T, H, E, k, I, what = shape
    say("[streamed edge] %s ksplit knob %d" % (what, ks))
    cfg = wl.MoEConfig(52, "stream_edge", T=T, H=H, E=E, k=k, I=I, Is=I, scale=2.5)
    h = config_host(cfg)
    d = to_device(h)
    tune(MOE_TUNE_KSPLIT=ks, MOE_TUNE_RING=3, MOE_TUNE_STREAMK=1)
    a = run_forward(moe, cfg, d)
    tune(MOE_TUNE_RING=2)
    b = run_forward(moe, cfg, d)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    out, ids, gates, counts = a
    ref = oracle_forward_rows(h, k, cfg.scale, np.arange(T))
    same, _, _ = compare_routing(ids, gates, ref, what)
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    compare_out(out[same], ref["out"][same], what)


@pytest.mark.parametrize("path", ["wide", "tall", "dma", "skinny"])
def test_identical_tokens_one_giant_group(moe, tune, path):
    say("[giant group %s]" % path)
    tune(MOE_TUNE_GEMM_PATH=moe.GEMM_PATHS[path])
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
