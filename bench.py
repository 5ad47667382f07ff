#!/usr/bin/env python3
"""Benchmark of the MI355X sigmoid-routed MoE layer at the GLM-5 shape (one GPU).

A step is one pass of the whole layer (router, top-k and gates, permutation, SwiGLU routed experts, shared
expert, combine) over one batch of seeded synthetic tokens already resident in HBM. The default workload
is the GLM-5-shape prefill (T = 8192 tokens, H 6144, 256 experts top-8, I = Is = 2048, scale 2.5); the
GLM-5 decode step (T = 16) is measured in the same run and reported under "decode". At decode the shared expert
(Is = I) runs as one more group of the routed experts' grouped GEMMs; at prefill as a dense MLP on the main
stream unless --two-streams is given.

Prints one JSON line. `value` is prefill tokens/s. `next` holds the entry points around the mixture, each
timed on its own workload after the main measurement: the GLM-4.7-Flash layer, the block pass (RMSNorm +
mixture + residual) and the routing override at the GLM-5 shapes, and the dense SwiGLU MLP. `roofline` is the dominant kernel (the routed gate/up
SwiGLU grouped GEMM): algorithmic FLOPs per launch / its mean launch time from HIP events recorded on the
kernel's stream inside the timed region. `cpu_baseline` is the CPU oracle timed on a bounded sample of the
same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at GLM-5 shape (prefill & decode); % peak MFMA / HBM BW"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
WEIGHT_NAMES = ("w1", "w3", "w2", "ws1", "ws3", "ws2")
STAGES = ("router", "permute", "shared", "gate_up", "down", "combine")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev_bf16(a, device):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


class Runner:
    def __init__(self, m, cfg, dev_weights, host_tokens, device, two_streams):
        import torch

        self.m, self.cfg, self.w = m, cfg, dev_weights
        self.x = to_dev_bf16(host_tokens["x"], device)
        self.wr = to_dev_bf16(host_tokens["wr"], device)
        self.b = torch.from_numpy(host_tokens["b"]).to(device)
        T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
        self.out = torch.empty(T, H, dtype=torch.float32, device=device)
        self.ids = torch.empty(T, k, dtype=torch.int32, device=device)
        self.gates = torch.empty(T, k, dtype=torch.float32, device=device)
        self.counts = torch.empty(E, dtype=torch.int32, device=device)
        nbytes = m.moe_workspace_bytes(T, H, E, k, cfg.I, cfg.Is)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.s1 = torch.cuda.Stream(device) if two_streams else None

    def step(self, events=None):
        w = self.w
        args = (self.x, self.wr, self.b, w["w1"], w["w3"], w["w2"], w["ws1"], w["ws3"], w["ws2"], self.cfg.k,
                self.cfg.scale, self.out, self.ws)
        kw = dict(topk_ids=self.ids, topk_gates=self.gates, expert_counts=self.counts, stream_shared=self.s1)
        if events is None:
            self.m.moe_forward(*args, **kw)
        else:
            self.m.moe_forward_profiled(*args, events, **kw)

    def time(self, steps, warmup):
        """Mean ms per pass over `steps` timed passes, and the stages of a pass. The timed window records HIP
        events only around the gate/up launch (self.gate_up_ms, the roofline kernel's launch time, and
        self.step_ms from each pass's start): every recorded event costs the stream a few microseconds. The
        split into all six stages comes from a second window of as many passes, after the timed one, with
        an event at every stage boundary."""
        import torch

        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
        gu = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for row in ev + gu:  # materialise the HIP events before the timed region
            for e in row:
                e.record()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            self.step(events=[gu[i][0], None, None, gu[i][1], gu[i][2], None, None])
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        self.gate_up_ms = float(np.mean([gu[i][1].elapsed_time(gu[i][2]) for i in range(steps)]))
        # pass i: from its start to the next pass's start (the last one to the window's end)
        marks = [gu[i][0] for i in range(steps)] + [end]
        self.step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
        for i in range(steps):
            self.step(events=ev[i])
        torch.cuda.synchronize()
        stages = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)]))
                  for j, name in enumerate(STAGES)}
        return ms, stages


# Sources that fix the routed gate/up kernel's memory traffic at a given workload: the kernel, its tile list
# and block order, and the seeded workload generator. Counter figures stored under profiles/ carry this
# digest; bench.py reports them as `traffic` only while it still matches the tree.
TRAFFIC_SOURCES = ("sigmoid_routed_mixture_amd/csrc/gemm.hip", "sigmoid_routed_mixture_amd/csrc/common.h",
                   "sigmoid_routed_mixture_amd/csrc/kernels.h", "sigmoid_routed_mixture_amd/csrc/plan.h",
                   "sigmoid_routed_mixture_amd/csrc/permute.hip", "workloads/gen.c")
TRAFFIC_PROFILE = "profiles/gate_up_glm5_prefill_traffic.txt"


def kernel_sources_digest():
    import hashlib

    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per routed gate/up launch from the stored counter summary (FETCH_SIZE and WRITE_SIZE, each
    scaled by the plain-copy calibration), or None when the summary is missing or the kernel changed since."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    if fields.get("kernel_sources_sha256") != kernel_sources_digest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def shared_folded(cfg, m=None, two_streams=False):
    """Whether the shared expert runs as one more group of the routed grouped GEMMs, so that their launches
    hold its work too. It needs the routed width (Is = I); at decode sizes (at most 16 routed rows per expert
    on average) it is always folded in; above them when it has no stream of its own and the persistent
    launches run with the library's default placement (the knobs of moe_tuning.h read through `m`)."""
    if not (cfg.Is > 0 and cfg.Is == cfg.I):
        return False
    if cfg.T * cfg.k <= 16 * cfg.E:
        return True
    if two_streams:
        return False
    if m is None:
        return True
    get = lambda n: m.moe_get_tuning(getattr(m, n))
    return (get("MOE_TUNE_SHARED") == 0 and get("MOE_TUNE_PERSIST") == 0 and get("MOE_TUNE_XCD_SPLIT") == 0
            and get("MOE_TUNE_GEMM_PATH") in (0, 3))


def gate_up_rows(cfg, folded):
    return cfg.T * cfg.k + (cfg.T if folded else 0)


def gate_up_flops(cfg, folded):
    return 4 * gate_up_rows(cfg, folded) * cfg.H * cfg.I


def layer_bytes(cfg, active):
    """Algorithmic bytes of one layer pass: weights of the experts that got tokens, the shared expert, router
    weight and bias, x once, out (fp32), ids and gates."""
    return (active * 3 * cfg.H * cfg.I * 2 + 3 * cfg.H * cfg.Is * 2 + cfg.E * cfg.H * 2 + 4 * cfg.E
            + 2 * cfg.T * cfg.H + 4 * cfg.T * cfg.H + 8 * cfg.T * cfg.k)


def gate_up_bytes(cfg, active, folded):
    """Algorithmic bytes of one grouped gate/up launch: W1 and W3 of the active experts (and Ws1, Ws3 when
    the shared expert is folded in), x once, h written."""
    groups = active + (1 if folded else 0)
    return groups * 2 * cfg.H * cfg.I * 2 + 2 * cfg.T * cfg.H + 2 * gate_up_rows(cfg, folded) * cfg.I


def time_call(fn, steps, warmup, min_warm_s=0.2, reps=3):
    """Mean ms of fn() over `steps` calls after `warmup` untimed calls, and at least `min_warm_s` seconds of
    them (a workload timed right after the host generated its weights finds the GPU's clocks idle: a few
    warmup calls of a 0.1 ms decode pass do not bring them up), HIP events on the current stream; the median
    of `reps` such timed windows, back to back (one slow window, 30 ms at decode sizes, does not decide it)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    means = []
    for _ in range(reps):
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(steps):
            fn()
        s1.record()
        torch.cuda.synchronize()
        means.append(s0.elapsed_time(s1) / steps)
    return float(np.median(means))


def tp8_share(wl):
    """One GPU's share of expert tensor parallelism over 8 GPUs at GLM-5 decode: every GPU holds all 256
    experts at I / 8 = 256, and runs the whole layer at that width, router included."""
    return wl.MoEConfig(61, "tp8_decode_share", T=16, H=6144, E=256, k=8, I=256, Is=256, scale=2.5)


def bench_next(m, wl, dev_w, host_w, early, device, steps, decode_steps, warmup):
    """The other workloads and the entry points around the mixture, each timed on its own: tiny, mid and
    skewed, the GLM-4.7-Flash layer (decode and prefill), the block (RMSNorm + mixture + residual) and the
    routing override at the GLM-5 shapes, and the dense SwiGLU MLP of the dense-first blocks. Every mixture
    entry reports both the MFMA and the HBM fraction."""
    import torch

    res = {}
    s1 = None  # shared expert on the main stream, as in the main measurement
    cfg_glm5_H = wl.BY_NAME["glm5_decode"].H

    def layer_inputs(cfg, w):
        host_t = {"x": wl.tokens(cfg), "wr": wl.router_weight(cfg), "b": wl.selection_bias(cfg)}
        d = {k: to_dev_bf16(v, device) for k, v in host_t.items() if k != "b"}
        d["b"] = torch.from_numpy(host_t["b"]).to(device)
        d.update(w)
        return d

    def mixture(cfg, d, nsteps):
        T = cfg.T
        out = torch.empty(T, cfg.H, dtype=torch.float32, device=device)
        ids = torch.empty(T, cfg.k, dtype=torch.int32, device=device)
        gates = torch.empty(T, cfg.k, dtype=torch.float32, device=device)
        counts = torch.empty(cfg.E, dtype=torch.int32, device=device)
        ws = torch.empty(m.moe_block_workspace_bytes(T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.Is), dtype=torch.uint8,
                         device=device)
        w = (d["w1"], d["w3"], d["w2"], d["ws1"], d["ws3"], d["ws2"])

        def fwd():
            m.moe_forward(d["x"], d["wr"], d["b"], *w, cfg.k, cfg.scale, out, ws, ids, gates, counts,
                          stream_shared=s1)

        ms = time_call(fwd, nsteps, warmup)
        active = int((counts.cpu().numpy() > 0).sum())
        r = {"T": T, "ms": ms, "tokens_per_s": T / (ms * 1e-3), "active_experts": active}
        gbs = layer_bytes(cfg, active) / (ms * 1e-3) / 1e9
        tf = cfg.flops() / (ms * 1e-3) / 1e12
        r.update(gbs=gbs, hbm_frac=gbs / PEAK_HBM_GBS, tflops=tf, mfma_frac=tf / PEAK_BF16_TFLOPS)
        return r, fwd, (out, ids, gates, ws, w)

    # the other workloads of the measurement table: tiny (latency), mid (GLM-4.7-Flash shape at scale 1.0,
    # near the ridge: both fractions), skewed (32768 tokens, expert 0 takes every token)
    for name, n in (("tiny", decode_steps), ("mid", steps), ("glm5_skewed", max(2, steps // 2))):
        cfg = wl.BY_NAME[name]
        if cfg.H == cfg_glm5_H and cfg.E == 256:
            w = dev_w
        else:
            w = {k: to_dev_bf16(wl.weight(cfg, k), device) for k in WEIGHT_NAMES}
        res[name], _, _ = mixture(cfg, layer_inputs(cfg, w), n)
        log("%s: %s" % (name, res[name]))
        del w
    torch.cuda.empty_cache()

    # GLM-4.7-Flash layer (H 2048, 64 experts top-4, I = Is = 1536, scale 1.8)
    c47d, c47p = wl.BY_NAME["glm47_decode"], wl.BY_NAME["glm47_prefill"]
    w47 = early["glm47"]  # allocated at start
    for cfg, n in ((c47d, decode_steps), (c47p, steps)):
        res[cfg.name], _, _ = mixture(cfg, layer_inputs(cfg, w47), n)
        log("%s: %s" % (cfg.name, res[cfg.name]))

    # block pass and routing override at the GLM-5 shapes, against the plain mixture on the same tokens
    for name, n in (("glm5_prefill", steps), ("glm5_decode", decode_steps)):
        cfg = wl.BY_NAME[name]
        d = layer_inputs(cfg, dev_w)
        base, fwd, (out, ids, gates, ws, w) = mixture(cfg, d, n)
        gamma = to_dev_bf16(wl.norm_weight(cfg.H, cfg.seed), device)
        xn = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device=device)

        def blk():
            m.moe_block_forward(d["x"], gamma, wl.NORM_EPS, d["wr"], d["b"], *w, cfg.k, cfg.scale, out, ws,
                                x_norm=xn, stream_shared=s1)

        ms_b = time_call(blk, n, warmup)
        fwd()
        g2 = gates.clone()
        g2[ids == 0] = 0.0  # the pages' ablation of one expert

        def rtd():
            m.moe_forward_routed(d["x"], ids, g2, *w, out, ws, stream_shared=s1)

        ms_r = time_call(rtd, n, warmup)
        res["block_" + name] = {"ms": ms_b, "tokens_per_s": cfg.T / (ms_b * 1e-3), "mixture_ms": base["ms"],
                                "norm_and_residual_ms": ms_b - base["ms"]}
        res["routed_" + name] = {"ms": ms_r, "tokens_per_s": cfg.T / (ms_r * 1e-3), "mixture_ms": base["ms"]}
        log("block/routed %s: %s %s" % (name, res["block_" + name], res["routed_" + name]))

    # dense SwiGLU MLP of the dense-first blocks
    for name, n in (("glm5_dense_prefill", steps), ("glm5_dense_decode", decode_steps),
                    ("glm47_dense_prefill", steps)):
        cfg = wl.DENSE_BY_NAME[name]
        w = {k: to_dev_bf16(wl.dense_weight(cfg, k), device) for k in ("w1", "w3", "w2")}
        x = to_dev_bf16(wl.dense_tokens(cfg), device)
        out = torch.empty(cfg.T, cfg.H, dtype=torch.float32, device=device)
        ws = torch.empty(m.moe_dense_mlp_workspace_bytes(cfg.T, cfg.H, cfg.Id), dtype=torch.uint8, device=device)
        ms = time_call(lambda: m.moe_dense_mlp(x, w["w1"], w["w3"], w["w2"], out, ws), n, warmup)
        r = {"T": cfg.T, "H": cfg.H, "I": cfg.Id, "ms": ms, "tokens_per_s": cfg.T / (ms * 1e-3)}
        if cfg.T <= 64:
            gbs = (3 * cfg.H * cfg.Id * 2 + 2 * cfg.T * cfg.H + 4 * cfg.T * cfg.H) / (ms * 1e-3) / 1e9
            r.update(gbs=gbs, hbm_frac=gbs / PEAK_HBM_GBS)
        else:
            tf = cfg.flops() / (ms * 1e-3) / 1e12
            r.update(tflops=tf, mfma_frac=tf / PEAK_BF16_TFLOPS)
        res[name] = r
        log("%s: %s" % (name, r))
        del w
    torch.cuda.empty_cache()

    # One GPU's share of the two multi-GPU layouts of the GLM-5 layer (nothing here uses a second GPU):
    # expert parallelism over 8 GPUs at prefill, where a GPU holds 32 experts and receives the slots routed to
    # them from 8 batches of 8192 tokens (65,536 rows, here uniformly spread: one slot per row, gate 1, through
    # the routed entry point; the shared expert runs data-parallel elsewhere), and expert tensor parallelism
    # over 8 GPUs at decode, where every GPU holds all 256 experts with I / 8 = 256 (the whole layer at that
    # width, router included).
    ep = wl.MoEConfig(60, "ep8_prefill_share", T=65536, H=6144, E=32, k=1, I=2048, Is=0, scale=1.0)
    w = {n: to_dev_bf16(wl.weight(ep, n), device) for n in ("w1", "w3", "w2")}
    x = to_dev_bf16(wl.tokens(ep), device)
    ids = torch.from_numpy(np.random.default_rng(ep.seed).integers(0, ep.E, size=(ep.T, 1), dtype=np.int32)).to(device)
    gates = torch.ones(ep.T, 1, dtype=torch.float32, device=device)
    out = torch.empty(ep.T, ep.H, dtype=torch.float32, device=device)
    ws = torch.empty(m.moe_workspace_bytes(ep.T, ep.H, ep.E, ep.k, ep.I, 0), dtype=torch.uint8, device=device)
    ms = time_call(lambda: m.moe_forward_routed(x, ids, gates, w["w1"], w["w3"], w["w2"], None, None, None, out, ws),
                   steps, warmup)
    tf = 6 * ep.T * ep.k * ep.H * ep.I / (ms * 1e-3) / 1e12
    res[ep.name] = {"rows": ep.T, "E": ep.E, "ms": ms, "tflops": tf, "mfma_frac": tf / PEAK_BF16_TFLOPS}
    log("%s: %s" % (ep.name, res[ep.name]))
    del w, x, out, ws
    torch.cuda.empty_cache()
    tp = tp8_share(wl)
    res[tp.name], _, _ = mixture(tp, layer_inputs(tp, early["tp8"]), decode_steps)
    log("%s: %s" % (tp.name, res[tp.name]))
    torch.cuda.empty_cache()
    return res


def profile_workload(m, wl, name, args, device):
    """Only the timed steps of one workload, for profiler runs: a mixture workload (prefill and decode name
    the GLM-5 ones) through moe_forward_profiled, or a dense-MLP workload through moe_dense_mlp."""
    import torch

    name = {"prefill": "glm5_prefill", "decode": "glm5_decode"}.get(name, name)
    if name in wl.DENSE_BY_NAME:
        cfg = wl.DENSE_BY_NAME[name]
        w = {k: to_dev_bf16(wl.dense_weight(cfg, k), device) for k in ("w1", "w3", "w2")}
        x = to_dev_bf16(wl.dense_tokens(cfg), device)
        out = torch.empty(cfg.T, cfg.H, dtype=torch.float32, device=device)
        ws = torch.empty(m.moe_dense_mlp_workspace_bytes(cfg.T, cfg.H, cfg.Id), dtype=torch.uint8, device=device)
        steps = args.steps if cfg.T > 64 else args.decode_steps
        ms = time_call(lambda: m.moe_dense_mlp(x, w["w1"], w["w3"], w["w2"], out, ws), steps, args.warmup, reps=1)
        log("%s: %.4f ms/step" % (name, ms))
        return
    if name not in wl.BY_NAME:
        raise SystemExit("unknown workload %r" % name)
    cfg = wl.BY_NAME[name]
    log("generating the expert weights of %s" % name)
    w = {n: to_dev_bf16(wl.weight(cfg, n), device) for n in WEIGHT_NAMES}
    host_t = {"x": wl.tokens(cfg), "wr": wl.router_weight(cfg), "b": wl.selection_bias(cfg)}
    r = Runner(m, cfg, w, host_t, device, args.two_streams)
    ms, stages = r.time(args.steps if cfg.T > 64 else args.decode_steps, args.warmup)
    active = int((r.counts.cpu().numpy() > 0).sum())
    log("%s: %.4f ms/step, stages %s, active experts %d" % (name, ms, stages, active))


ROUTINGS = ("one_tile", "two_tiles", "workload")


def profile_routing(m, wl, kind, args, device):
    """The GLM-5 prefill routed experts alone (no shared expert) through moe_forward_routed under a chosen
    routing, for profiler runs: one_tile gives each of the 256 experts 256 rows (token t takes experts 8t ..
    8t + 7 mod 256: one full tile each), two_tiles gives 128 experts 512 rows (mod 128: two full tiles each),
    workload is the workload's own top-8 (216 experts, 1 to 963 rows). Gates are 1/8."""
    import torch

    cfg = wl.BY_NAME["glm5_prefill"]
    log("generating the expert weights of %s" % cfg.name)
    w = {n: to_dev_bf16(wl.weight(cfg, n), device) for n in ("w1", "w3", "w2")}
    x = to_dev_bf16(wl.tokens(cfg), device)
    t = torch.arange(cfg.T, device=device)[:, None]
    j = torch.arange(cfg.k, device=device)[None, :]
    if kind == "one_tile":
        ids = ((cfg.k * t + j) % cfg.E).to(torch.int32).contiguous()
    elif kind == "two_tiles":
        ids = ((cfg.k * t + j) % (cfg.E // 2)).to(torch.int32).contiguous()
    else:
        wr = to_dev_bf16(wl.router_weight(cfg), device)
        b = torch.from_numpy(wl.selection_bias(cfg)).to(device)
        ids = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=device)
        g = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=device)
        m.moe_route(x, wr, b, cfg.k, cfg.scale, ids, g)
    gates = torch.full((cfg.T, cfg.k), 1.0 / cfg.k, dtype=torch.float32, device=device)
    out = torch.empty(cfg.T, cfg.H, dtype=torch.float32, device=device)
    ws = torch.empty(m.moe_workspace_bytes(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, 0), dtype=torch.uint8, device=device)
    counts = torch.bincount(ids.flatten().long(), minlength=cfg.E)
    ms = time_call(lambda: m.moe_forward_routed(x, ids, gates, w["w1"], w["w3"], w["w2"], None, None, None, out, ws),
                   args.steps, args.warmup, reps=1)
    log("routing %s: %d experts active, at most %d rows; %.4f ms/step (routed experts and combine)"
        % (kind, int((counts > 0).sum()), int(counts.max()), ms))


def cpu_baseline(cfg, host, budget_s, rounds=5):
    """The CPU oracle as it stands, token-sharded over the host's threads, on `rounds` equal slices of one
    seeded sample of the workload's tokens (about budget_s seconds in all); the value is the median rate of
    the slices."""
    import oracle

    desc = oracle.host_description()
    threads = desc["threads"]
    rng = np.random.default_rng(0)
    t0 = time.perf_counter()
    oracle.forward(host, cfg.k, cfg.scale, rows=np.array([0], dtype=np.int32))
    t1 = time.perf_counter() - t0  # one token on one thread
    per_round = max(threads, int(budget_s / rounds / max(t1, 1e-3)) * threads)
    per_round = min(per_round, cfg.T // rounds)
    sample = rng.choice(cfg.T, size=per_round * rounds, replace=False).astype(np.int32)
    rates, total = [], 0.0
    for r in range(rounds):
        rows = np.sort(sample[r * per_round:(r + 1) * per_round])
        t0 = time.perf_counter()
        oracle.run_sharded(lambda rows: oracle.forward(host, cfg.k, cfg.scale, rows=rows), rows, nthreads=threads)
        dt = time.perf_counter() - t0
        total += dt
        rates.append(per_round / dt)
    return {"value": float(np.median(rates)), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d seeded random tokens of the %s workload (T=%d) in %d slices of %d, fp64 plain C, %d threads "
                      "(host: nproc %s, affinity %s, %s), %.1f s in all; value = median slice rate"
                      % (per_round * rounds, cfg.name, cfg.T, rounds, per_round, threads, desc["nproc"],
                         desc["affinity"], desc["cpu_model"], total),
            "threads": threads, "nproc": desc["nproc"], "affinity": desc["affinity"], "cpu_model": desc["cpu_model"],
            "slice_rates": rates}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--two-streams", action="store_true",
                    help="run the shared expert on a second stream, overlapping the routed experts, where it is a "
                         "dense MLP of its own (prefill; by default it runs on the main stream: at the GLM-5 shapes "
                         "the overlap slows the routed GEMMs as much as it hides)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the GLM-4.7-Flash, block, routing-override and dense-MLP measurements")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--copy-calibration", type=float, default=None, metavar="GIB",
                    help="time a plain device-to-device copy of this many GiB (HBM ceiling, and the known-size "
                         "reference for profiler byte counters) and exit")
    ap.add_argument("--profile-only", default=None, metavar="WORKLOAD",
                    help="run only this workload's timed steps and print its timings (for profiler runs): prefill, "
                         "decode, or any mixture or dense-MLP workload name (mid, glm5_skewed, glm47_prefill, "
                         "glm5_dense_decode, ...)")
    ap.add_argument("--profile-routing", default=None, choices=ROUTINGS,
                    help="profiler runs: only the GLM-5 prefill routed experts under the given routing")
    ap.add_argument("--tune", action="append", default=[], metavar="KNOB=VALUE",
                    help="set a knob of include/moe_tuning.h before measuring (e.g. MOE_TUNE_ORDER=1); the default "
                         "run sets none")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this layer's hot path has no multi-GPU mode (see the sharding "
              "design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = int(args.copy_calibration * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        s0.record()
        for _ in range(reps):
            dst.copy_(src)
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / reps
        print(json.dumps({"copy_bytes_each_way": n, "ms": ms, "read_plus_write_GBs": 2 * n / ms / 1e6}), flush=True)
        return

    import sigmoid_routed_mixture_amd as m
    import workloads as wl

    for item in args.tune:
        knob, _, value = item.partition("=")
        m.moe_set_tuning(getattr(m, knob), int(value))
        log("tuning %s = %s" % (knob, value))
    device = torch.device("cuda", 0)
    if args.profile_routing:
        profile_routing(m, wl, args.profile_routing, args, device)
        return
    if args.profile_only:
        profile_workload(m, wl, args.profile_only, args, device)
        return
    cfg_p = wl.BY_NAME["glm5_prefill"]
    cfg_d = wl.BY_NAME["glm5_decode"]
    # The decode-sized secondary workloads stream every weight once per pass, so where their weights sit
    # in device memory shows: the same GLM-4.7-Flash decode pass took 0.1453 ms with its weights allocated
    # first in the process and 0.159-0.172 ms with weights allocated after other workloads' large buffers had
    # come and gone. A serving process allocates its layers' weights at load time, so these are allocated
    # here, before anything else, and kept.
    early = None
    if not args.no_next:
        early = {"glm47": {n: to_dev_bf16(wl.weight(wl.BY_NAME["glm47_decode"], n), device) for n in WEIGHT_NAMES},
                 "tp8": {n: to_dev_bf16(wl.weight(tp8_share(wl), n), device) for n in WEIGHT_NAMES}}
    log("generating GLM-5 expert weights on the host (%d threads)" % wl.host_threads())
    t0 = time.perf_counter()
    host_w = {n: wl.weight(cfg_p, n) for n in WEIGHT_NAMES}
    dev_w = {n: to_dev_bf16(a, device) for n, a in host_w.items()}
    torch.cuda.synchronize()
    log("weights ready in %.1f s" % (time.perf_counter() - t0))
    two = args.two_streams

    results = {}
    plan = ((cfg_p, args.steps), (cfg_d, args.decode_steps))
    for cfg, steps in plan:
        host_t = {"x": wl.tokens(cfg), "wr": wl.router_weight(cfg), "b": wl.selection_bias(cfg)}
        r = Runner(m, cfg, dev_w, host_t, device, two)
        ms, stages = r.time(steps, args.warmup)
        active = int((r.counts.cpu().numpy() > 0).sum())
        results[cfg.name] = (ms, stages, active, host_t, float(np.median(r.step_ms)), r.gate_up_ms)
        log("%s: %.4f ms/step, gate/up launch %.4f ms, stages %s, active experts %d" % (cfg.name, ms, r.gate_up_ms,
                                                                                       stages, active))
        del r
        torch.cuda.empty_cache()

    ms_p, st_p, act_p, host_tp, med_p, gu_p = results[cfg_p.name]
    ms_d, st_d, act_d, _, med_d, gu_d = results[cfg_d.name]
    gu_ms = gu_p
    fold_p, fold_d = shared_folded(cfg_p, m, two), shared_folded(cfg_d, m, two)
    achieved = gate_up_flops(cfg_p, fold_p) / (gu_ms * 1e-3) / 1e12
    layer_tflops = cfg_p.flops() / (ms_p * 1e-3) / 1e12
    dec_gbs = layer_bytes(cfg_d, act_d) / (ms_d * 1e-3) / 1e9
    dec_gu_gbs = gate_up_bytes(cfg_d, act_d, fold_d) / (gu_d * 1e-3) / 1e9

    line = {
        "metric": METRIC,
        "value": cfg_p.T / (ms_p * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_p,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg_p.name, "T": cfg_p.T, "H": cfg_p.H, "E": cfg_p.E, "k": cfg_p.k, "I": cfg_p.I,
                   "Is": cfg_p.Is, "scale": cfg_p.scale, "shared_expert_stream": two, "parallelism": "none",
                   "tuning": args.tune},
        "roofline": {"bound": "mfma", "kernel": "gate/up SwiGLU grouped GEMM (routed experts%s)"
                     % (" + shared expert" if fold_p else ""), "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(), "launch_ms": gu_ms,
                     "algorithmic_bytes": gate_up_bytes(cfg_p, act_p, fold_p),
                     "algorithmic_flops": gate_up_flops(cfg_p, fold_p)},
        "layer": {"tflops": layer_tflops, "mfma_frac": layer_tflops / PEAK_BF16_TFLOPS, "median_step_ms": med_p,
                  "gbs": layer_bytes(cfg_p, act_p) / (ms_p * 1e-3) / 1e9, "active_experts": act_p,
                  "stages_ms": st_p},
        "decode": {"workload": cfg_d.name, "T": cfg_d.T, "steps": args.decode_steps, "ms_per_step": ms_d,
                   "tokens_per_s": cfg_d.T / (ms_d * 1e-3), "median_step_ms": med_d, "gbs": dec_gbs,
                   "hbm_frac": dec_gbs / PEAK_HBM_GBS,
                   "active_experts": act_d, "stages_ms": st_d,
                   "gate_up_roofline": {"bound": "hbm", "achieved": dec_gu_gbs, "peak": PEAK_HBM_GBS,
                                        "unit": "GB/s", "frac": dec_gu_gbs / PEAK_HBM_GBS}},
        "next": None,
        "cpu_baseline": None,
    }
    if not args.no_next:
        line["next"] = bench_next(m, wl, dev_w, host_w, early, device, max(3, args.steps // 2), args.decode_steps,
                                  args.warmup)
    if not args.no_cpu_baseline:
        host = dict(host_tp)
        host.update(host_w)
        log("timing the CPU oracle on a sample of %s" % cfg_p.name)
        line["cpu_baseline"] = cpu_baseline(cfg_p, host, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
