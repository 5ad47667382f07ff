"""moe_forward_noalloc (include/moe.h): the layer on the library's own per-device scratch, for callers that
cannot allocate. Through the C ABI, against moe_forward with a caller workspace (bit for bit: same kernels,
same layout) and against the oracle (the layer's acceptance bar), on two calls in a row, the second with a
smaller batch, so nothing the first call leaves in the scratch may leak into the second."""
import numpy as np
import pytest
import torch

from parity import case, compare_out, compare_routing, oracle_forward_rows, route_ref, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import sigmoid_routed_mixture_amd as m

    return m


def outputs(cfg, T):
    return (torch.empty(T, cfg.H, dtype=torch.float32, device="cuda"),
            torch.empty(T, cfg.k, dtype=torch.int32, device="cuda"),
            torch.empty(T, cfg.k, dtype=torch.float32, device="cuda"),
            torch.empty(cfg.E, dtype=torch.int32, device="cuda"))


def with_workspace(m, cfg, d, T):
    out, ids, gates, counts = outputs(cfg, T)
    ws = torch.empty(m.moe_workspace_bytes(T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.Is), dtype=torch.uint8, device="cuda")
    m.moe_forward(d["x"][:T], d["wr"], d["b"], d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"], d["ws2"], cfg.k,
                  cfg.scale, out, ws, ids, gates, counts)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (out, ids, gates, counts)]


def no_alloc(m, cfg, d, T):
    out, ids, gates, counts = outputs(cfg, T)
    m.moe_forward_noalloc(d["x"][:T], d["wr"], d["b"], d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"], d["ws2"],
                          cfg.k, cfg.scale, out, ids, gates, counts)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (out, ids, gates, counts)]


# (workload, first batch, second smaller batch): GLM-4.7-Flash at 512 tokens runs the persistent routed GEMMs
# (their block counters live in the scratch) and at 100 the decode path; GLM-5 decode at 16, then 3.
CASES = [("glm47_prefill", 512, 100), ("glm5_decode", 16, 3)]


@pytest.mark.parametrize("name,T1,T2", CASES)
def test_noalloc_matches_workspace_entry_two_calls(moe, name, T1, T2):
    cfg, h, d = case(name)
    assert moe.moe_forward_noalloc_max_bytes() == 64 << 20
    ref = route_ref(name)
    for T in (T1, T2):
        say("[no-alloc] %s T=%d" % (name, T))
        a = no_alloc(moe, cfg, d, T)
        b = with_workspace(moe, cfg, d, T)
        for x, y in zip(a, b):
            assert np.array_equal(x, y), "%s T=%d: no-alloc differs from moe_forward" % (name, T)
        sub = {key: v[:T] for key, v in ref.items()}
        same, _, _ = compare_routing(a[1], a[2], sub, name)
        rows = np.arange(T, dtype=np.int32)[same]
        orc = oracle_forward_rows(h, cfg.k, cfg.scale, rows)
        compare_out(a[0][rows], orc["out"], "%s no-alloc T=%d" % (name, T))


def test_noalloc_rejects_sizes_beyond_its_scratch(moe):
    cfg, h, d = case("glm47_prefill")
    T = 4096  # needs about 240 MB of workspace
    out, ids, gates, counts = outputs(cfg, T)
    out.fill_(7.0)
    with pytest.raises(moe.MoEError) as err:
        moe.moe_forward_noalloc(d["x"][:T], d["wr"], d["b"], d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"],
                                d["ws2"], cfg.k, cfg.scale, out, ids, gates, counts)
    assert err.value.status == moe.MOE_ERR_WORKSPACE and "maximum" in str(err.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call must enqueue nothing"
