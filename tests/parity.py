"""Helpers of the GPU parity tests: host inputs -> device tensors, the oracle on host threads, and the
comparison rules.

Rules (from the layer's acceptance bar):
* expert selection is compared as id sets per token, bit-exact, except tokens whose oracle k-th and
  (k+1)-th biased scores differ by less than NEAR_TIE (counted and reported);
* per-expert counts are bit-exact wherever no near-tie token changed its set;
* outputs: max |gpu - oracle| <= OUT_TOL * RMS(oracle output) over every token whose id set matches.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads as wl

NEAR_TIE = 1e-5
OUT_TOL = 2e-2
GATE_RTOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(host: dict, device="cuda") -> dict:
    out = {}
    for key, v in host.items():
        if v is None:
            out[key] = None
        elif v.dtype == np.uint16:
            out[key] = dev_bf16(v, device)
        else:
            out[key] = dev(v, device)
    return out


def oracle_route_all(h: dict, k: int, scale: float):
    T = h["x"].shape[0]
    return oracle.run_sharded(lambda rows: oracle.route(h["x"], h["wr"], h["b"], k, scale, rows=rows), np.arange(T))


def oracle_forward_rows(h: dict, k: int, scale: float, rows):
    return oracle.run_sharded(lambda rows: oracle.forward(h, k, scale, rows=rows), np.asarray(rows))


def compare_routing(ids_gpu, gates_gpu, ref, label=""):
    """Returns (mask of tokens whose sets agree, number of near-tie tokens, number of those that differ)."""
    ids_gpu = np.asarray(ids_gpu)
    gates_gpu = np.asarray(gates_gpu)
    near = ref["gap"] < NEAR_TIE
    sg = np.sort(ids_gpu, axis=1)
    so = np.sort(ref["ids"], axis=1)
    same = np.all(sg == so, axis=1)
    bad = ~same & ~near
    assert not bad.any(), "%s: %d tokens chose other experts outside the near-tie band (first %s)" % (
        label, bad.sum(), np.nonzero(bad)[0][:8])
    # every gpu id is a valid, distinct expert
    assert ids_gpu.min() >= 0
    assert np.all(np.diff(sg, axis=1) > 0), "%s: repeated expert within a token" % label
    # gates per expert id, on agreeing tokens
    og = np.argsort(ids_gpu, axis=1)
    oo = np.argsort(ref["ids"], axis=1)
    gg = np.take_along_axis(gates_gpu, og, axis=1)[same]
    go = np.take_along_axis(ref["gates"], oo, axis=1)[same]
    assert np.allclose(gg, go, rtol=GATE_RTOL, atol=1e-7), "%s: gates differ (max %g)" % (
        label, np.abs(gg - go).max())
    return same, int(near.sum()), int((near & ~same).sum())


def compare_out(out_gpu, out_ref, label=""):
    out_gpu = np.asarray(out_gpu, dtype=np.float64)
    out_ref = np.asarray(out_ref, dtype=np.float64)
    assert np.all(np.isfinite(out_gpu)), "%s: non-finite output" % label
    rms = float(np.sqrt(np.mean(out_ref ** 2)))
    err = float(np.max(np.abs(out_gpu - out_ref))) if out_ref.size else 0.0
    ratio = err / rms if rms > 0 else err
    say("  %s: %d tokens compared, max|err| = %.3e, RMS = %.3e, ratio = %.4f (limit %.3f)"
        % (label, out_ref.shape[0] if out_ref.ndim > 1 else 1, err, rms, ratio, OUT_TOL))
    assert ratio <= OUT_TOL, "%s: max|err|/RMS = %.4f > %.3f" % (label, ratio, OUT_TOL)
    return ratio


# Output comparisons on a sample take at least this many seeded random tokens (plus the boundary tokens of
# sample_rows); smaller batches are compared on every token.
SAMPLE_FLOOR = 1024


def tile_height(n: int, BM: int = 256) -> int:
    """Height of the GPU's token tiles of an expert with n rows: n split evenly over ceil(n / BM) tiles,
    rounded up to 32 rows (the LDS-copy GEMM's tiles of up to 256 tokens). Used only to pick which tokens
    a sample must contain."""
    if n <= 0:
        return BM
    nt = (n + BM - 1) // BM
    h = ((n + nt - 1) // nt + 31) // 32 * 32
    return min(h, BM)


def sample_rows(ids_ref, n_random: int, seed: int = 0):
    """A seeded sample of n_random tokens plus, for every expert that got any token, the first and the last
    token routed to it and the two tokens on each side of every boundary between its GPU token tiles (the
    rows of an expert are its tokens in ascending order; the last tile is the shortest, where the row masks
    apply)."""
    ids_ref = np.asarray(ids_ref)
    T, k = ids_ref.shape
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=min(n_random, T), replace=False).tolist())
    flat = ids_ref.ravel()
    order = np.argsort(flat, kind="stable")  # slots by expert, ascending token within an expert
    experts, starts, counts = np.unique(flat[order], return_index=True, return_counts=True)
    for e, s0, n in zip(experts, starts, counts):
        if e < 0:
            continue
        toks = order[s0:s0 + n] // k
        pick.add(int(toks[0]))
        pick.add(int(toks[-1]))
        ht = tile_height(int(n))
        for b in range(ht, int(n), ht):
            pick.add(int(toks[b - 1]))
            pick.add(int(toks[b]))
    return np.array(sorted(pick), dtype=np.int32)


def output_rows(T: int, ids_ref, seed: int, full: bool):
    """Tokens whose outputs a test compares: all of them when `full` or T <= SAMPLE_FLOOR, else
    sample_rows with SAMPLE_FLOOR random tokens."""
    if full or T <= SAMPLE_FLOOR:
        return np.arange(T, dtype=np.int32)
    return sample_rows(ids_ref, SAMPLE_FLOOR, seed=seed)


def host_line() -> str:
    d = oracle.host_description()
    return "oracle host: %d threads (nproc %s, affinity %s, %s)" % (d["threads"], d["nproc"], d["affinity"],
                                                                     d["cpu_model"])


def config_host(cfg: wl.MoEConfig, weights: dict | None = None) -> dict:
    h = {"x": wl.tokens(cfg), "wr": wl.router_weight(cfg), "b": wl.selection_bias(cfg)}
    if weights is None:
        weights = {n: wl.weight(cfg, n) for n in ("w1", "w3", "w2", "ws1", "ws3", "ws2")}
    h.update(weights)
    return h


# ---------------------------------------------------------------------------------------------------
# workload cache shared by the GPU test modules (one host and one device copy of each layer's weights)

WEIGHT_NAMES = ("w1", "w3", "w2", "ws1", "ws3", "ws2")
_CACHE = {}


def layer_weights(cfg: wl.MoEConfig):
    key = ("weights", cfg.weight_seed, cfg.E, cfg.H, cfg.I, cfg.Is)
    if key not in _CACHE:
        gb = (3 * cfg.E * cfg.H * cfg.I + 3 * cfg.H * cfg.Is) * 2 / 1e9
        say("generating the expert weights of %s (%.1f GB) on host and device" % (cfg.name, gb))
        host = {n: wl.weight(cfg, n) for n in WEIGHT_NAMES}
        _CACHE[key] = (host, to_device(host))
    return _CACHE[key]


def case(name):
    """(cfg, host inputs, device inputs) of a mixture workload."""
    if name not in _CACHE:
        cfg = wl.BY_NAME[name]
        wh, wd = layer_weights(cfg)
        h = config_host(cfg, wh)
        d = to_device({"x": h["x"], "wr": h["wr"], "b": h["b"]})
        d.update(wd)
        _CACHE[name] = (cfg, h, d)
    return _CACHE[name]


def route_ref(name):
    key = ("route", name)
    if key not in _CACHE:
        cfg, h, _ = case(name)
        say("oracle routing of %s (T=%d) on host threads" % (name, cfg.T))
        _CACHE[key] = oracle_route_all(h, cfg.k, cfg.scale)
    return _CACHE[key]


def dense_case(name):
    """(cfg, host inputs, device inputs) of a dense-MLP workload."""
    key = ("dense", name)
    if key not in _CACHE:
        cfg = wl.DENSE_BY_NAME[name]
        wkey = ("dense_weights", cfg.weight_seed, cfg.H, cfg.Id)
        if wkey not in _CACHE:
            say("generating the dense MLP weights of %s (%.2f GB)" % (name, 3 * cfg.H * cfg.Id * 2 / 1e9))
            host = {n: wl.dense_weight(cfg, n) for n in ("w1", "w3", "w2")}
            _CACHE[wkey] = (host, to_device(host))
        wh, wd = _CACHE[wkey]
        h = dict(wh)
        h["x"] = wl.dense_tokens(cfg)
        d = dict(wd)
        d["x"] = dev_bf16(h["x"])
        _CACHE[key] = (cfg, h, d)
    return _CACHE[key]
