"""Parity of the entry points around the mixture (include/moe_block.h) with the CPU oracle, through the C ABI:
the mixture with caller-given routing (the pages' ablation and gate editing), the mixture half of a block
(RMSNorm before it, the residual add after it), the dense SwiGLU MLP of the dense-first blocks, and the
GLM-4.7-Flash workloads' block pass. Same acceptance rules as the mixture's own tests (tests/parity.py).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import (SAMPLE_FLOOR, case, compare_out, compare_routing, dense_case, dev, dev_bf16, host_line,
                    oracle_forward_rows, output_rows, route_ref, sample_rows, say)

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


def forward(m, cfg, d, x=None, b=None):
    x = d["x"] if x is None else x
    T = x.shape[0]
    out = torch.empty(T, cfg.H, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, cfg.k, dtype=torch.float32, device="cuda")
    ws = torch.empty(m.moe_workspace_bytes(T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.Is), dtype=torch.uint8, device="cuda")
    m.moe_forward(x, d["wr"], d["b"] if b is None else b, d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"], d["ws2"],
                  cfg.k, cfg.scale, out, ws, ids, gates)
    torch.cuda.synchronize()
    return out, ids, gates


def forward_routed(m, cfg, d, ids, gates, x=None, stream_shared=None):
    x = d["x"] if x is None else x
    T = x.shape[0]
    out = torch.empty(T, cfg.H, dtype=torch.float32, device="cuda")
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    k = ids.shape[1]
    ws = torch.empty(m.moe_workspace_bytes(T, cfg.H, cfg.E, k, cfg.I, cfg.Is), dtype=torch.uint8, device="cuda")
    m.moe_forward_routed(x, ids, gates, d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"], d["ws2"], out, ws,
                         expert_counts=counts, stream_shared=stream_shared)
    torch.cuda.synchronize()
    return out.cpu().numpy(), counts.cpu().numpy()


# ---------------------------------------------------------------------------------------------------
# routing given by the caller

def test_layer_sized_for_a_larger_batch(moe):
    """One workspace sized for T_max serves every smaller batch. At the GLM-5 shape the layout of 64 tokens
    (decode K split, shared expert folded in) is larger than that of 100: MoELayer(T_max = 100) runs 16, 64
    and 100 tokens, each equal bit for bit to moe_forward with a workspace of its own size."""
    say("[layer sized for 100 tokens]")
    cfg, h, d = case("glm5_prefill")
    layer = moe.MoELayer(d["wr"], d["b"], d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"], d["ws2"], cfg.k,
                         cfg.scale, 100)
    for T in (16, 64, 100):
        x = d["x"][:T]
        out = layer(x)
        torch.cuda.synchronize()
        ref, _, _ = forward(moe, cfg, d, x=x)
        assert torch.equal(out, ref), T


@pytest.mark.parametrize("name", ["tiny", "mid", "glm5_decode", "glm47_decode", "glm5_prefill"])
def test_routed_with_own_routing_is_forward_bitwise(moe, name):
    """moe_forward_routed fed moe_forward's own ids and gates runs the same kernels on the same bytes."""
    say("[routed = forward] %s" % name)
    cfg, h, d = case(name)
    out, ids, gates = forward(moe, cfg, d)
    out_r, counts = forward_routed(moe, cfg, d, ids, gates)
    assert np.array_equal(out_r, out.cpu().numpy())
    assert np.array_equal(counts, np.bincount(ids.cpu().numpy().ravel(), minlength=cfg.E))


@pytest.mark.parametrize("name", ["tiny", "mid", "glm5_decode", "glm47_prefill"])
def test_routed_ablation_matches_oracle(moe, name):
    """The pages' ablation: zero the gate of every slot that chose one expert, leave the rest as they are."""
    say("[ablation] %s" % name)
    cfg, h, d = case(name)
    ref = route_ref(name)
    ids, gates = ref["ids"].copy(), ref["gates"].copy()
    victim = int(np.bincount(ids.ravel(), minlength=cfg.E).argmax())
    gates[ids == victim] = 0.0
    rows = np.arange(cfg.T, dtype=np.int32) if cfg.T <= 256 else sample_rows(ids, 128, seed=cfg.index)
    out, counts = forward_routed(moe, cfg, d, dev(ids), dev(gates))
    ref_out = oracle.run_sharded(lambda rows: {"o": oracle.forward_routed(h, ids, gates, rows=rows)}, rows)["o"]
    compare_out(out[rows], ref_out, "%s ablate expert %d" % (name, victim))
    # the ablated expert still counts its tokens (its slots are routed, with weight 0)
    assert counts[victim] == int((ids == victim).any(axis=1).sum())
    # and the tokens that chose it now differ from the unablated layer
    full = oracle_forward_rows(h, cfg.k, cfg.scale, rows)["out"]
    chose = (ids[rows] == victim).any(axis=1)
    assert chose.any() and np.abs(out[rows][chose] - full[chose]).max() > 0


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_routed_arbitrary_ids_and_gates(moe, name):
    """Random distinct experts with arbitrary (negative, > 1) weights, repeated experts within a token, and
    ids outside [0, E) (such a slot adds nothing: the oracle gets the same slot with weight 0)."""
    say("[routed arbitrary] %s" % name)
    cfg, h, d = case(name)
    rng = np.random.default_rng(cfg.index + 100)
    T, k, E = cfg.T, cfg.k, cfg.E
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    gates = rng.uniform(-1.0, 2.0, size=(T, k)).astype(np.float32)
    dup = rng.random(T) < 0.2
    ids[dup, 1] = ids[dup, 0]
    bad = rng.random(T) < 0.1
    ids[bad, k - 1] = np.where(rng.random(bad.sum()) < 0.5, -1, E + 3)
    out, counts = forward_routed(moe, cfg, d, dev(ids), dev(gates))
    ids_o, gates_o = ids.copy(), gates.copy()
    outside = (ids_o < 0) | (ids_o >= E)
    ids_o[outside] = 0
    gates_o[outside] = 0.0
    rows = np.arange(T, dtype=np.int32) if T <= 256 else np.sort(rng.choice(T, 256, replace=False)).astype(np.int32)
    ref_out = oracle.run_sharded(lambda rows: {"o": oracle.forward_routed(h, ids_o, gates_o, rows=rows)}, rows)["o"]
    compare_out(out[rows], ref_out, "%s arbitrary routing" % name)
    want = np.zeros(E, np.int64)
    for t in range(T):
        for e in set(int(v) for v in ids[t] if 0 <= v < E):
            want[e] += 1
    assert np.array_equal(counts, want)


def test_bias_moves_only_the_choice_on_gpu(moe):
    """A bias change that leaves every choice unchanged leaves the layer's output bit for bit unchanged
    (the bias is added to the sigmoids only to choose)."""
    cfg, h, d = case("tiny")
    ref = route_ref("tiny")
    b2 = h["b"].copy()
    b2[::2] += np.float32(1e-3)
    ref2 = oracle.route(h["x"], h["wr"], b2, cfg.k, cfg.scale)
    same = np.all(np.sort(ref2["ids"], 1) == np.sort(ref["ids"], 1), axis=1)
    out1, ids1, _ = forward(moe, cfg, d)
    out2, ids2, _ = forward(moe, cfg, d, b=dev(b2))
    # same experts in the same slot order (the combine adds the slots in that order)
    keep = same & np.all(ids1.cpu().numpy() == ids2.cpu().numpy(), axis=1)
    assert keep.sum() > cfg.T // 2
    assert np.array_equal(out1.cpu().numpy()[keep], out2.cpu().numpy()[keep])


# ---------------------------------------------------------------------------------------------------
# the block: RMSNorm before the mixture, residual add after it

def block(m, cfg, d, gamma, T=None, stream_shared=None):
    T = cfg.T if T is None else T
    resid = d["x"][:T]
    out = torch.empty(T, cfg.H, dtype=torch.float32, device="cuda")
    xn = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
    ids = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, cfg.k, dtype=torch.float32, device="cuda")
    nb = m.moe_block_workspace_bytes(T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.Is)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    m.moe_block_forward(resid, gamma, wl.NORM_EPS, d["wr"], d["b"], d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"],
                        d["ws2"], cfg.k, cfg.scale, out, ws, x_norm=xn, topk_ids=ids, topk_gates=gates,
                        stream_shared=stream_shared)
    torch.cuda.synchronize()
    return out, xn, ids, gates


# the block's output on every token, but at GLM-5 prefill on parity.sample_rows' sample (parity.SAMPLE_FLOOR
# seeded tokens plus every expert's first, last and tile-boundary tokens)
BLOCK_FULL = {"tiny": True, "mid": True, "glm5_decode": True, "glm47_decode": True, "glm5_prefill": False,
              "glm47_prefill": True}


@pytest.mark.parametrize("name", list(BLOCK_FULL))
def test_block_forward_parity(moe, name):
    say("[block] %s" % name)
    cfg, h, d = case(name)
    gamma_h = wl.norm_weight(cfg.H, cfg.seed)
    gamma = dev_bf16(gamma_h)
    out, xn, ids, gates = block(moe, cfg, d, gamma)
    xn_h = xn.cpu().view(torch.int16).numpy().view(np.uint16)
    # 1. the normalised stream, bit for bit (fp64 on both sides; a sum-order difference could only flip a
    #    value lying within ~1e-16 of a bf16 rounding boundary)
    xn_ref = oracle.run_sharded(lambda rows: {"x": oracle.rmsnorm(h["x"], gamma_h, wl.NORM_EPS, rows=rows)},
                                np.arange(cfg.T))["x"]
    nbad = int((xn_h != xn_ref).sum())
    say("  x_norm: %d of %d values differ from the oracle" % (nbad, xn_h.size))
    assert nbad <= xn_h.size // 1000000
    # 2. the residual is added last, in fp32, to exactly what moe_forward computes on x_norm
    out_f, ids_f, gates_f = forward(moe, cfg, d, x=xn)
    resid = (h["x"].astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(out.cpu().numpy(), out_f.cpu().numpy() + resid)
    assert torch.equal(ids, ids_f) and torch.equal(gates, gates_f)
    # 3. routing on the normalised stream against the oracle's
    hn = dict(h)
    hn["x"] = xn_ref
    ref = oracle.run_sharded(lambda rows: oracle.route(xn_ref, h["wr"], h["b"], cfg.k, cfg.scale, rows=rows),
                             np.arange(cfg.T))
    same, nnear, ndiff = compare_routing(ids.cpu().numpy(), gates.cpu().numpy(), ref, name)
    # 4. the block output against the oracle's block on (a sample of) the tokens that chose alike
    rows = output_rows(cfg.T, ref["ids"], cfg.index, BLOCK_FULL[name])
    rows = rows[same[rows]]
    say("  %s; oracle block on %d of %d tokens (near-tie %d, differing %d)" % (
        host_line(), rows.size, cfg.T, nnear, ndiff))
    orc = oracle.run_sharded(lambda rows: oracle.block_forward(h, gamma_h, wl.NORM_EPS, cfg.k, cfg.scale, rows=rows),
                             rows)
    assert np.array_equal(orc["x_norm"], xn_ref[rows])
    compare_out(out.cpu().numpy()[rows] - resid[rows], orc["out"].astype(np.float64) - resid[rows],
                "%s block delta" % name)
    compare_out(out.cpu().numpy()[rows], orc["out"], "%s block out" % name)


def test_block_second_stream_and_no_shared_expert(moe):
    cfg, h, d = case("mid")
    gamma = dev_bf16(wl.norm_weight(cfg.H, cfg.seed))
    a = block(moe, cfg, d, gamma, T=700)
    b = block(moe, cfg, d, gamma, T=700, stream_shared=torch.cuda.Stream())
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # without a shared expert: x' + routed only
    c0 = cfg.with_(Is=0)
    d0 = dict(d)
    d0["ws1"] = d0["ws3"] = d0["ws2"] = None
    out, xn, ids, gates = block(moe, c0, d0, gamma, T=300)
    h0 = dict(h)
    h0["ws1"] = h0["ws3"] = h0["ws2"] = None
    rows = np.arange(0, 300, 7, dtype=np.int32)
    orc = oracle.block_forward(h0, wl.norm_weight(cfg.H, cfg.seed), wl.NORM_EPS, cfg.k, cfg.scale, rows=rows)
    same, _, _ = compare_routing(ids.cpu().numpy()[rows], gates.cpu().numpy()[rows], orc, "mid Is=0")
    resid = (h["x"][rows].astype(np.uint32) << 16).view(np.float32)
    compare_out(out.cpu().numpy()[rows][same] - resid[same], orc["out"][same] - resid[same], "mid Is=0 delta")


def test_block_zero_tokens(moe):
    cfg, h, d = case("tiny")
    empty = d["x"][:0]
    out = torch.empty(0, cfg.H, dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    moe.moe_block_forward(empty, dev_bf16(wl.norm_weight(cfg.H, 1)), 1e-5, d["wr"], d["b"], d["w1"], d["w3"],
                          d["w2"], d["ws1"], d["ws3"], d["ws2"], cfg.k, cfg.scale, out, ws)
    moe.moe_forward_routed(empty, torch.empty(0, cfg.k, dtype=torch.int32, device="cuda"),
                           torch.empty(0, cfg.k, dtype=torch.float32, device="cuda"), d["w1"], d["w3"], d["w2"],
                           d["ws1"], d["ws3"], d["ws2"], out, ws)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------------------------------
# dense SwiGLU MLP of the dense-first blocks

def dense(m, cfg, d, T=None):
    T = cfg.T if T is None else T
    x = d["x"][:T]
    out = torch.empty(T, cfg.H, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, m.moe_dense_mlp_workspace_bytes(T, cfg.H, cfg.Id)), dtype=torch.uint8, device="cuda")
    m.moe_dense_mlp(x, d["w1"], d["w3"], d["w2"], out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# dense MLP outputs on every token up to parity.SAMPLE_FLOOR tokens, else on that many seeded tokens plus
# the first and the last
DENSE_FULL = {"dense_tiny": True, "glm5_dense_decode": True, "glm5_dense_prefill": False,
              "glm47_dense_prefill": False}


@pytest.mark.parametrize("name", list(DENSE_FULL))
def test_dense_mlp_parity(moe, name):
    say("[dense mlp] %s" % name)
    cfg, h, d = dense_case(name)
    out = dense(moe, cfg, d)
    rng = np.random.default_rng(cfg.index)
    n = SAMPLE_FLOOR
    rows = np.arange(cfg.T, dtype=np.int32) if DENSE_FULL[name] or cfg.T <= n else np.sort(
        np.concatenate([[0, cfg.T - 1], rng.choice(np.arange(1, cfg.T - 1), n, replace=False)])).astype(np.int32)
    say("  %s; oracle dense MLP on %d of %d tokens" % (host_line(), rows.size, cfg.T))
    ref = oracle.run_sharded(lambda rows: {"o": oracle.dense_mlp(h["x"], h["w1"], h["w3"], h["w2"], rows=rows)},
                             rows)["o"]
    compare_out(out[rows], ref, name)


@pytest.mark.parametrize("T", [1, 7, 16])
def test_dense_decode_copy_ring_bitwise(moe, tune, T):
    # the GLM-5 dense MLP at decode sizes: the K-split LDS-copy GEMMs with the three-step copy ring and one
    # workgroup per block against the two-step ring, bit for bit; the streamed form (its own K splits, so its
    # own summation order) and both against the oracle
    cfg, h, d = dense_case("glm5_dense_decode")
    rows = np.arange(T, dtype=np.int32)
    ref = oracle.dense_mlp(h["x"], h["w1"], h["w3"], h["w2"], rows=rows)
    s = dense(moe, cfg, d, T=T)
    compare_out(s, ref, "glm5_dense_decode streamed T=%d" % T)
    tune(MOE_TUNE_RING=2)
    a = dense(moe, cfg, d, T=T)
    tune(MOE_TUNE_RING=1)
    b = dense(moe, cfg, d, T=T)
    assert np.array_equal(a, b)
    compare_out(a, ref, "glm5_dense_decode ring T=%d" % T)


@pytest.mark.parametrize("path", ["wide", "tall", "dma", "skinny"])
@pytest.mark.parametrize("T", [1, 16, 100])
def test_dense_mlp_both_kernels_and_ragged(moe, tune, path, T):
    tune(MOE_TUNE_GEMM_PATH=moe.GEMM_PATHS[path])
    cfg, h, d = dense_case("dense_tiny")
    out = dense(moe, cfg, d, T=min(T, cfg.T))
    rows = np.arange(min(T, cfg.T), dtype=np.int32)
    ref = oracle.dense_mlp(h["x"], h["w1"], h["w3"], h["w2"], rows=rows)
    compare_out(out, ref, "dense_tiny %s T=%d" % (path, T))
