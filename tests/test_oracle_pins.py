"""Pins of the CPU oracle to facts the pages and the mathematics fix (CPU only).

Each test checks the oracle against something other than itself: values the pages print (parameter
counts, gate sums, config shapes), closed forms (the logistic function's special values), brute force
over every k-subset, crafted exact ties derived by hand, special cases that reduce to a dense SwiGLU MLP
computed independently with numpy, invariants (bias moves only the choice, token independence,
linearity), the stable sort a library routine gives, and the skewed workload's closed forms.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------------------------------
# independent numpy helpers (test code: decode bf16 bits and run a dense SwiGLU MLP with matmuls)

def dec(a):
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def enc_exact(v):
    """bf16 bits of float32 values that are exactly representable in bf16."""
    f = np.asarray(v, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def np_swiglu(x, w1, w3, w2):
    g = x @ w1.T
    u = x @ w3.T
    return ((g / (1.0 + np.exp(-g))) * u) @ w2.T


def small_inputs(T, H, E, I, Is, seed=7, skewed=False):
    cfg = wl.MoEConfig(99, "pin", T=T, H=H, E=E, k=1, I=I, Is=Is, scale=2.5, skewed=skewed)
    d = wl.host_inputs(cfg, seed=seed)
    if Is == 0:
        d["ws1"] = d["ws3"] = d["ws2"] = None
    return d


# ---------------------------------------------------------------------------------------------------
# pages' printed numbers

def test_param_count_matches_pages():
    g = load("glm5_moe_params.json")
    s = g["shape"]
    H, E, I = s["hidden_size"], s["n_routed_experts"], s["moe_intermediate_size"]
    Is = s["n_shared_experts"] * I
    assert oracle.param_count(H, E, I, Is) == g["mixture_of_experts_parameters_per_block"]
    # the block total adds the attention and the two norms; the 75 MoE blocks are the 78 less 3 dense
    assert (g["mixture_of_experts_parameters_per_block"] + g["mla_parameters_per_block"]
            + g["moe_rmsnorm_parameters"] + g["attention_rmsnorm_parameters"]) == g["moe_block_total"]
    assert s["num_hidden_layers"] - s["first_k_dense_replace"] == g["moe_blocks"]
    assert g["moe_block_total"] * g["moe_blocks"] == g["all_moe_blocks_total"]
    # one fp selection-bias value per routed expert per MoE block
    assert E * g["moe_blocks"] == g["router_correction_bias_values_all_blocks"]


def test_workload_shapes_follow_pages():
    g5 = load("glm5_moe_params.json")["shape"]
    for name in ("glm5_decode", "glm5_prefill", "glm5_skewed"):
        c = wl.BY_NAME[name]
        assert (c.H, c.E, c.k, c.I, c.Is, c.scale) == (
            g5["hidden_size"], g5["n_routed_experts"], g5["num_experts_per_tok"], g5["moe_intermediate_size"],
            g5["n_shared_experts"] * g5["moe_intermediate_size"], g5["routed_scaling_factor"])
    f = load("glm47_flash_moe_shape.json")
    c = wl.BY_NAME["mid"]
    assert (c.H, c.E, c.k, c.I) == (f["hidden_size"], f["n_routed_experts"], f["num_experts_per_tok"],
                                    f["moe_intermediate_size"])
    for name in ("glm47_decode", "glm47_prefill"):
        c = wl.BY_NAME[name]
        assert (c.H, c.E, c.k, c.I, c.Is, c.scale) == (
            f["hidden_size"], f["n_routed_experts"], f["num_experts_per_tok"], f["moe_intermediate_size"],
            f["n_shared_experts"] * f["moe_intermediate_size"], f["routed_scaling_factor"])
    dn = load("dense_mlp_and_norm_shapes.json")
    for name, model in (("glm5_dense_decode", "glm5"), ("glm5_dense_prefill", "glm5"),
                        ("glm47_dense_prefill", "glm47_flash")):
        c = wl.DENSE_BY_NAME[name]
        assert (c.H, c.Id) == (dn[model]["hidden_size"], dn[model]["intermediate_size"])
    assert wl.NORM_EPS == dn["glm5"]["rms_norm_eps"] == dn["glm47_flash"]["rms_norm_eps"]


# ---------------------------------------------------------------------------------------------------
# sigmoid and bf16 decode: closed forms

def test_bf16_decode_known_patterns():
    assert oracle.bf16_to_double(0x3F80) == 1.0
    assert oracle.bf16_to_double(0xC000) == -2.0
    assert oracle.bf16_to_double(0x3E80) == 0.25
    assert oracle.bf16_to_double(0x0000) == 0.0
    assert oracle.bf16_to_double(0x3FC0) == 1.5
    assert oracle.bf16_to_double(0x0001) == 2.0 ** -133  # smallest subnormal


def test_sigmoid_closed_forms():
    assert oracle.sigmoid(0.0) == 0.5
    ln3 = float(np.float32(math.log(3.0)))
    # sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4; fp32 rounding of ln 3 moves them by < 1e-7
    assert abs(oracle.sigmoid(ln3) - 0.75) < 1e-7
    assert abs(oracle.sigmoid(-ln3) - 0.25) < 1e-7
    # sigma(1) = e / (1 + e)
    assert abs(oracle.sigmoid(1.0) - math.e / (1.0 + math.e)) < 6e-8
    zs = np.linspace(-30, 30, 6001, dtype=np.float32)
    s = np.array([oracle.sigmoid(float(z)) for z in zs])
    assert np.all(np.diff(s) >= 0) and s.min() >= 0.0 and s.max() <= 1.0
    sm = np.array([oracle.sigmoid(float(-z)) for z in zs])
    assert np.all(np.abs(s + sm - 1.0) <= 2.0 ** -23)


# ---------------------------------------------------------------------------------------------------
# routing

def test_router_hand_case():
    # x = [1, 2]; W_r rows [0.5, 0.25], [-1, 0], [0, 0] give z = [1, -1, 0] exactly
    x = enc_exact([[1.0, 2.0]])
    wr = enc_exact([[0.5, 0.25], [-1.0, 0.0], [0.0, 0.0]])
    b = np.zeros(3, np.float32)
    r = oracle.route(x, wr, b, k=2, scale=2.5, want_logits=True)
    assert r["logits"].tolist() == [[1.0, -1.0, 0.0]]
    assert r["ids"].tolist() == [[0, 2]]  # sigma(1) > sigma(0) = 0.5 > sigma(-1)
    g = r["gates"][0].astype(np.float64)
    assert abs(g.sum() - 2.5) <= 2 * 2.0 ** -22
    # G0 / G1 = sigma(1) / sigma(0) = 2e / (1 + e)
    assert abs(g[0] / g[1] - 2 * math.e / (1 + math.e)) < 1e-6
    # gap between the 2nd and 3rd biased scores: 0.5 - sigma(-1) = 0.5 - 1/(1+e)
    assert abs(r["gap"][0] - (0.5 - 1.0 / (1.0 + math.e))) < 1e-7


@pytest.mark.parametrize("case", load("tie_cases.json")["cases"])
def test_crafted_exact_ties(case):
    E, k = case["E"], case["k"]
    x = np.zeros((3, 16), np.uint16)  # three identical zero tokens
    wr = wl.normal_bf16(11, 1, 0.02, 0, E * 16).reshape(E, 16)
    b = np.array(case["b"], np.float32)
    r = oracle.route(x, wr, b, k=k, scale=case["scale"])
    for t in range(3):
        assert r["ids"][t].tolist() == case["ids"]
        assert np.all(np.abs(r["gates"][t] - case["gate"]) <= 2.0 ** -22)
        if case["gap"] is None:
            assert math.isinf(r["gap"][t])
        else:
            assert r["gap"][t] == case["gap"]


def _biased_scores(x, wr, b):
    z = oracle.route(x, wr, b, k=1, scale=1.0, want_logits=True)["logits"]
    s = np.vectorize(lambda v: oracle.sigmoid(float(v)), otypes=[np.float32])(z)
    return (s.astype(np.float32) + b.astype(np.float32)).astype(np.float32), s


@pytest.mark.parametrize("E,k", [(5, 1), (6, 2), (8, 3), (10, 4), (7, 7), (9, 4)])
def test_topk_brute_force(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T, H = 40, 24
    x = wl.normal_bf16(E, 0, 1.0, 0, T * H).reshape(T, H)
    x[:8] = 0  # rows with every score exactly 0.5: ties decided by the bias grid alone
    wr = wl.normal_bf16(E, 1, 0.3, 0, E * H).reshape(E, H)
    b = (rng.integers(-2, 3, size=E) / 8.0).astype(np.float32)  # coarse grid: many equal biases
    c, _ = _biased_scores(x, wr, b)
    r = oracle.route(x, wr, b, k=k, scale=2.5)
    for t in range(T):
        key = [(float(c[t, e]), -e) for e in range(E)]
        winners = [S for S in itertools.combinations(range(E), k)
                   if min(key[e] for e in S) > max((key[e] for e in range(E) if e not in S),
                                                   default=(-math.inf, 0))]
        assert len(winners) == 1
        assert sorted(r["ids"][t].tolist()) == list(winners[0])
        # slot order: descending (c, -index)
        ks = [key[e] for e in r["ids"][t]]
        assert ks == sorted(ks, reverse=True)


def test_gates_sum_to_scale_and_k1():
    d = small_inputs(T=64, H=128, E=16, I=32, Is=0)
    for k, scale in [(4, 2.5), (8, 1.8), (3, 1.0)]:
        r = oracle.route(d["x"], d["wr"], d["b"], k=k, scale=scale)
        sums = r["gates"].astype(np.float64).sum(axis=1)
        ulp = np.spacing(np.float32(scale)).astype(np.float64)
        assert np.all(np.abs(sums - scale) <= k * ulp)
    r = oracle.route(d["x"], d["wr"], d["b"], k=1, scale=2.5)
    assert np.all(r["gates"] == np.float32(2.5))


def test_bias_moves_only_the_choice():
    d = small_inputs(T=6, H=64, E=12, I=32, Is=32)
    k, scale = 3, 2.5
    for t in range(6):
        one = dict(d)
        one["x"] = np.ascontiguousarray(d["x"][t:t + 1])
        base = oracle.forward(one, k, scale)
        sel = set(base["ids"][0].tolist())
        b2 = np.array([d["b"][e] + (0.25 if e in sel else -0.25) for e in range(12)], np.float32)
        moved = dict(one, b=b2)
        r2 = oracle.forward(moved, k, scale)
        assert r2["ids"][0].tolist() == base["ids"][0].tolist()
        assert np.array_equal(r2["gates"], base["gates"])
        assert np.array_equal(r2["out"], base["out"])
        # a bias that does change the choice does change the output
        b3 = d["b"].copy()
        drop = base["ids"][0][0]
        b3[drop] -= 10.0
        r3 = oracle.forward(dict(one, b=b3), k, scale)
        assert drop not in r3["ids"][0].tolist()
        assert not np.array_equal(r3["out"], base["out"])


def test_k_equals_E_is_dense_mixture():
    T, H, E, I, Is = 8, 64, 5, 48, 40
    d = small_inputs(T, H, E, I, Is, seed=3)
    scale = 2.5
    r = oracle.forward(d, k=E, scale=scale)
    x = dec(d["x"])
    z = x @ dec(d["wr"]).T
    s = 1.0 / (1.0 + np.exp(-z))
    G = scale * s / s.sum(axis=1, keepdims=True)
    want = np_swiglu(x, dec(d["ws1"]), dec(d["ws3"]), dec(d["ws2"]))
    for e in range(E):
        want += G[:, e:e + 1] * np_swiglu(x, dec(d["w1"][e]), dec(d["w3"][e]), dec(d["w2"][e]))
    rms = np.sqrt(np.mean(want ** 2))
    assert np.max(np.abs(r["out"] - want)) <= 1e-6 * rms
    # with every expert chosen, the bias cannot matter
    r2 = oracle.forward(dict(d, b=(d["b"] * -7.0).astype(np.float32)), k=E, scale=scale)
    assert np.max(np.abs(r2["out"] - r["out"])) <= 1e-6 * rms


def test_single_expert_is_dense_swiglu():
    T, H, I, Is = 6, 96, 40, 56
    d = small_inputs(T, H, 1, I, Is, seed=5)
    scale = 1.8
    r = oracle.forward(d, k=1, scale=scale, parts=True)
    x = dec(d["x"])
    routed = scale * np_swiglu(x, dec(d["w1"][0]), dec(d["w3"][0]), dec(d["w2"][0]))
    shared = np_swiglu(x, dec(d["ws1"]), dec(d["ws3"]), dec(d["ws2"]))
    rms = np.sqrt(np.mean((routed + shared) ** 2))
    assert np.max(np.abs(r["out"] - (routed + shared))) <= 1e-6 * rms
    assert np.max(np.abs(r["routed"] - routed)) <= 1e-6 * rms
    assert np.max(np.abs(r["shared"] - shared)) <= 1e-6 * rms
    # the pages' identity: routed + shared == out (each side rounded to fp32 once)
    assert np.max(np.abs(r["routed"].astype(np.float64) + r["shared"] - r["out"])) <= 2e-6 * rms


def test_linearity_in_W2_and_scale():
    d = small_inputs(T=10, H=64, E=6, I=32, Is=0, seed=9)
    base = oracle.forward(d, k=2, scale=2.5)["out"]
    w2x2 = (d["w2"].astype(np.uint32) + np.where((d["w2"] & 0x7F80) != 0, 0x80, 0)).astype(np.uint16)
    assert np.array_equal(dec(w2x2), 2 * dec(d["w2"]))  # exponent + 1: exact doubling
    assert np.array_equal(oracle.forward(dict(d, w2=w2x2), k=2, scale=2.5)["out"], 2 * base)
    assert np.array_equal(oracle.forward(d, k=2, scale=5.0)["out"], 2 * base)


def test_token_independence():
    d = small_inputs(T=12, H=64, E=8, I=32, Is=32, seed=13)
    full = oracle.forward(d, k=3, scale=2.5)
    for t in range(12):
        one = oracle.forward(d, k=3, scale=2.5, rows=[t])
        assert np.array_equal(one["out"][0], full["out"][t])
        assert np.array_equal(one["ids"][0], full["ids"][t])
    shards = oracle.run_sharded(lambda rows: oracle.forward(d, 3, 2.5, rows=rows), np.arange(12), nthreads=4)
    assert np.array_equal(shards["out"], full["out"])


def test_forward_routed_matches_and_ablates():
    d = small_inputs(T=8, H=64, E=6, I=32, Is=24, seed=21)
    k = 3
    f = oracle.forward(d, k=k, scale=2.5)
    out = oracle.forward_routed(d, f["ids"], f["gates"])
    rms = np.sqrt(np.mean(f["out"].astype(np.float64) ** 2))
    assert np.max(np.abs(out - f["out"])) <= 1e-6 * rms
    # ablation: zero the gate of every slot that chose expert e; the other gates stay as they were, so the
    # output drops by exactly those slots' gated expert outputs (checked with the dense numpy MLP)
    e = int(f["ids"][0, 0])
    g = f["gates"].copy()
    g[f["ids"] == e] = 0
    abl = oracle.forward_routed(d, f["ids"], g)
    x = dec(d["x"])
    ye = np_swiglu(x, dec(d["w1"][e]), dec(d["w3"][e]), dec(d["w2"][e]))
    ge = np.where(f["ids"] == e, f["gates"], 0).sum(axis=1).astype(np.float64)
    assert np.max(np.abs((out.astype(np.float64) - abl) - ge[:, None] * ye)) <= 1e-5 * rms
    assert np.all(g.sum(axis=1)[ge > 0] < 2.5)


# ---------------------------------------------------------------------------------------------------
# permutation

def test_permute_is_stable_counting_sort():
    rng = np.random.default_rng(1)
    T, E, k = 300, 20, 4
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[:30] = [0, 1, 2, 3]  # one crowded expert set
    p = oracle.permute(ids, E)
    flat = ids.ravel()
    order = np.argsort(flat, kind="stable")  # library stable sort of slots by expert
    assert np.array_equal(p["counts"], np.bincount(flat, minlength=E))
    assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(p["row_token"], order // k)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    assert np.array_equal(p["slot_row"], inv)
    assert p["counts"].sum() == T * k


def test_permute_empty_experts_and_rejects_bad_ids():
    ids = np.array([[3, 1], [1, 3], [3, 0]], np.int32)
    p = oracle.permute(ids, 6)
    assert p["counts"].tolist() == [1, 2, 0, 3, 0, 0]
    assert p["offsets"].tolist() == [0, 1, 3, 3, 6, 6, 6]
    assert p["row_token"].tolist() == [2, 0, 1, 0, 1, 2]
    assert p["slot_row"].tolist() == [3, 1, 2, 4, 5, 0]
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 6]], np.int32), 6)


# ---------------------------------------------------------------------------------------------------
# skewed workload: closed forms that hold for any router weights and tokens, since 0 < s < 1

def test_skewed_routing_closed_forms():
    cfg = wl.BY_NAME["glm5_skewed"].with_(T=512, H=256)
    b = wl.selection_bias(cfg)
    assert b[0] == 0.0
    exact = -0.5 * np.log(np.arange(1, 257))
    assert np.all(np.abs(b - exact) <= np.spacing(np.abs(b).astype(np.float32)) / 2)  # one fp32 rounding
    x = wl.tokens(cfg)
    wr = wl.router_weight(cfg)
    r = oracle.route(x, wr, b, k=cfg.k, scale=cfg.scale)
    counts = np.bincount(r["ids"].ravel(), minlength=cfg.E)
    # experts 1..6 are the only ones that can outrank expert 0 (b_0 - b_j < 1 iff j + 1 < e^2), fewer than
    # k = 8, so expert 0 is always chosen
    assert counts[0] == cfg.T
    # experts 0..7 outrank every i >= 59: b_j - b_i >= 0.5 ln(60 / 8) > 1 >= s_i - s_j
    assert np.all(counts[59:] == 0)
    assert counts.sum() == cfg.T * cfg.k


# ---------------------------------------------------------------------------------------------------
# bf16 rounding, RMSNorm, the block's residual wiring and the dense MLP

def f32_to_bf16_rne(f):
    """Textbook fp32 -> bf16 round-to-nearest-even with integer operations (finite inputs)."""
    b = np.asarray(f, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def test_round_bf16_against_fp32_rounding_and_ties():
    rng = np.random.default_rng(5)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    got = np.array([oracle.round_bf16(float(v)) for v in f], np.uint16)
    assert np.array_equal(got, f32_to_bf16_rne(f))
    # halfway cases go to the even neighbour; a bit below fp32's precision breaks the tie upward (a detour
    # through fp32 would lose it and round down)
    assert oracle.round_bf16(1 + 2 ** -8) == 0x3F80
    assert oracle.round_bf16(1 + 3 * 2 ** -8) == 0x3F82
    assert oracle.round_bf16(1 + 2 ** -8 + 2 ** -40) == 0x3F81
    assert oracle.round_bf16(-(1 + 2 ** -8 + 2 ** -40)) == 0xBF81
    # subnormals step by 2^-133; the largest finite bf16 is 0x7F7F
    assert oracle.round_bf16(2.0 ** -133) == 0x0001
    assert oracle.round_bf16(1.5 * 2.0 ** -133) == 0x0002
    assert oracle.round_bf16(2.0 ** -126) == 0x0080
    assert oracle.round_bf16(0.0) == 0x0000 and oracle.round_bf16(-0.0) == 0x8000
    assert oracle.round_bf16(3.3895313892515355e38) == 0x7F7F
    assert oracle.round_bf16(3.4e38) == 0x7F80


def test_rmsnorm_scale_invariance_and_closed_forms():
    H = 256
    gamma = wl.norm_weight(H, 11)
    x = wl.normal_bf16(3, 0, 1.0, 0, 8 * H).reshape(8, H)
    assert np.all((x & 0x7F80) > 0x0080) and np.all((x & 0x7F80) < 0x7E00)  # normal, room to double
    # eps = 0: doubling x (exponent + 1, exact) leaves x / rms unchanged bit for bit
    x2 = (x + 0x0080).astype(np.uint16)
    assert np.array_equal(dec(x2), 2 * dec(x))
    assert np.array_equal(oracle.rmsnorm(x2, gamma, 0.0), oracle.rmsnorm(x, gamma, 0.0))
    # a constant row c: x / rms = sign(c), so the row is gamma or -gamma exactly
    xc = np.stack([np.full(H, enc_exact([0.75])[0]), np.full(H, enc_exact([-3.0])[0])])
    out = oracle.rmsnorm(xc, gamma, 0.0)
    assert np.array_equal(out[0], gamma) and np.array_equal(out[1], gamma ^ 0x8000)
    # eps = 3 c^2 halves it: x / sqrt(c^2 + 3 c^2) = sign(c) / 2
    for c in (2.0, -0.5):
        row = np.full((1, H), enc_exact([c])[0])
        half = oracle.rmsnorm(row, gamma, 3 * c * c)[0]
        assert np.array_equal(dec(half), np.sign(c) * dec(gamma) / 2)
    # a one-hot row a e_j (H = 256): rms = |a| / 16, so position j holds 16 sign(a) gamma_j, the rest 0
    for a, j in ((4.0, 5), (-0.25, 200)):
        row = np.zeros((1, H), np.uint16)
        row[0, j] = enc_exact([a])[0]
        out = oracle.rmsnorm(row, gamma, 0.0)[0]
        want = np.zeros(H)
        want[j] = 16 * np.sign(a) * dec(gamma[j])
        assert np.array_equal(dec(out), want)
    # a zero row stays zero with eps > 0; mean((out / gamma)^2) = m / (m + eps) for mean square m
    assert np.all(dec(oracle.rmsnorm(np.zeros((1, H), np.uint16), gamma, 1e-5)) == 0)
    out = dec(oracle.rmsnorm(x, gamma, 0.5))
    m = np.mean(dec(x) ** 2, axis=1)
    assert np.allclose(np.mean((out / dec(gamma)) ** 2, axis=1), m / (m + 0.5), rtol=1e-2)
    # rows are independent and the listed-rows form picks the same bytes
    assert np.array_equal(oracle.rmsnorm(x, gamma, 1e-5, rows=[6, 1]), oracle.rmsnorm(x, gamma, 1e-5)[[6, 1]])


def test_block_forward_wires_norm_and_residual():
    d = small_inputs(T=6, H=128, E=8, I=64, Is=64, seed=21)
    gamma = wl.norm_weight(128, 21)
    k, scale, eps = 2, 2.5, 1e-5
    blk = oracle.block_forward(d, gamma, eps, k, scale)
    xn = oracle.rmsnorm(d["x"], gamma, eps)
    assert np.array_equal(blk["x_norm"], xn)
    dn = dict(d)
    dn["x"] = xn
    f = oracle.forward(dn, k, scale, parts=True)
    assert np.array_equal(blk["ids"], f["ids"]) and np.array_equal(blk["gates"], f["gates"])
    # out = x' + routed + shared, rounded once: within an ulp of the sum of the separately rounded parts
    want = dec(d["x"]) + f["routed"].astype(np.float64) + f["shared"].astype(np.float64)
    assert np.allclose(blk["out"], want, rtol=0, atol=2 * np.spacing(np.float32(np.abs(want).max())))
    # with eps = 0 the norm ignores the stream's scale, so doubling x' doubles only the residual term
    d2 = dict(d)
    d2["x"] = (d["x"] + 0x0080).astype(np.uint16)
    b1 = oracle.block_forward(d, gamma, 0.0, k, scale)
    b2 = oracle.block_forward(d2, gamma, 0.0, k, scale)
    assert np.array_equal(b1["x_norm"], b2["x_norm"])
    delta1 = b1["out"].astype(np.float64) - dec(d["x"])
    delta2 = b2["out"].astype(np.float64) - dec(d2["x"])
    assert np.allclose(delta1, delta2, rtol=0, atol=4 * np.spacing(np.float32(np.abs(dec(d2["x"])).max())))


def test_dense_mlp_against_numpy_matmuls():
    H, Id, T = 96, 160, 5
    x = wl.normal_bf16(31, 0, 1.0, 0, T * H).reshape(T, H)
    w1 = wl.normal_bf16(31, 10, 0.02, 0, Id * H).reshape(Id, H)
    w3 = wl.normal_bf16(31, 11, 0.02, 0, Id * H).reshape(Id, H)
    w2 = wl.normal_bf16(31, 12, 0.02, 0, H * Id).reshape(H, Id)
    got = oracle.dense_mlp(x, w1, w3, w2)
    ref = np_swiglu(dec(x), dec(w1), dec(w3), dec(w2))
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-12)
    assert np.array_equal(oracle.dense_mlp(x, w1, w3, w2, rows=[4, 0]), got[[4, 0]])
    # the mixture with one expert, k = 1, scale 1 and no shared expert is exactly this MLP
    d = {"x": x, "wr": wl.normal_bf16(31, 1, 0.02, 0, H).reshape(1, H), "b": np.zeros(1, np.float32),
         "w1": w1[None], "w3": w3[None], "w2": w2[None], "ws1": None, "ws3": None, "ws2": None}
    assert np.array_equal(oracle.forward(d, 1, 1.0)["out"], got)
