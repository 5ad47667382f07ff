"""Seeded synthetic workloads for the sigmoid-routed MoE layer.

This module is shared by both sides of every parity check (the HIP path's harness and the CPU oracle's
harness) and holds none of the layer's arithmetic: it only describes the five workload shapes and makes
their input tensors, byte-identical wherever they are made, from `gen.c`'s counter-based generator.

Shapes follow the pages:
* GLM-5 (GlmMoeDsa) MoE block: hidden 6144, 256 routed experts, top-8, expert width 2048, one shared
  expert of the same width, routed scaling factor 2.5 (nnterp encyclopedia "glm_moe_dsa", Config table;
  atlas.klimoza.dev GLM-5 "Vocabulary projection", config.json).
* GLM-4.7-Flash (Glm4MoeLite): hidden 2048, 64 experts, top-4, width 1536, one shared expert, routed
  scaling factor 1.8 (nnterp encyclopedia "glm4_moe_lite", Config table); the mid workload keeps those
  shapes at scale 1.0, the glm47 workloads use the model's own scale.
* Dense-first blocks: the dense SwiGLU MLP of GLM-5 (intermediate 12288) and GLM-4.7-Flash (10240)
  (the module trees' GlmMoeDsaMLP / Glm4MoeLiteMLP gate_proj, up_proj, down_proj).
* The RMSNorm before the mixture has eps 1e-5 on both models (post_attention_layernorm in the module
  trees); its weight gamma ~ 1 + N(0, 0.1) stands in for a trained one.

Value distributions: x ~ N(0, 1) stands in for the RMS-normalised stream that enters the mixture (the
GLM-5 block's equations on open-model-atlas apply RMSNorm before the router); weights ~ N(0, 0.02), the
config's initializer range; selection bias ~ U(-0.1, 0.1). The skewed workload replaces the bias with
b_i = 0.5 ln(1 / (i + 1)) and adds a Zipf(1.2)-ordered offset alpha (e + 1)^-1.2 to every router-weight
entry of expert e (alpha = 0.02). Trained weights and real activations are not available; these stand in.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgen.so")
_lib = None
_lib_lock = threading.Lock()

# Tensor ids of the counter-based generator.
T_X, T_WR, T_B, T_W1, T_W3, T_W2, T_WS1, T_WS3, T_WS2, T_GAMMA, T_WD1, T_WD3, T_WD2 = range(13)

SIGMA_W = 0.02
BIAS_LO, BIAS_HI = -0.1, 0.1
SKEW_ALPHA, SKEW_POWER, SKEW_BIAS_COEF = 0.02, 1.2, 0.5
NORM_EPS = 1e-5
GAMMA_SIGMA = 0.1


def build(force: bool = False) -> str:
    """Compile gen.c into libgen.so with gcc (host code only)."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, src, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lib_lock:
        if _lib is None:
            build()  # no-op unless the source is newer than the built library
            L = ctypes.CDLL(_LIB_PATH)
            u64, u32, i32, dbl = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_double
            p = ctypes.c_void_p
            L.gen_normal_bf16.argtypes = [u64, u32, dbl, u64, u64, p, i32]
            L.gen_uniform_f32.argtypes = [u64, u32, dbl, dbl, u64, u64, p, i32]
            L.gen_skew_router_bf16.argtypes = [u64, u32, i32, i32, dbl, dbl, dbl, p]
            L.gen_log_bias_f32.argtypes = [i32, dbl, p]
            L.gen_bf16_from_double.argtypes = [dbl]
            L.gen_bf16_from_double.restype = ctypes.c_uint16
            L.gen_normal_quantile.argtypes = [i32]
            L.gen_normal_quantile.restype = dbl
            _lib = L
    return _lib


def host_threads() -> int:
    """Generator threads: the job's granted CPU share when OMP_NUM_THREADS states one, else every core this
    process may run on."""
    try:
        n = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        n = 0
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(n, avail) if n > 0 else avail)


@dataclass(frozen=True)
class MoEConfig:
    index: int
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    Is: int
    scale: float
    skewed: bool = False
    weights_of: int = -1  # index of the workload whose expert weights this one shares (-1: its own)

    @property
    def seed(self) -> int:
        """Seed of the tokens, router weight and bias."""
        return 0x5EED0000 + self.index

    @property
    def weight_seed(self) -> int:
        """Seed of the routed and shared expert weights."""
        return 0x5EED0000 + (self.index if self.weights_of < 0 else self.weights_of)

    def with_(self, **kw) -> "MoEConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return MoEConfig(**d)

    def flops(self) -> int:
        """Algorithmic FLOPs of one layer pass: router 2TEH, routed 6TkHI, shared 6THIs."""
        return 2 * self.T * self.E * self.H + 6 * self.T * self.k * self.H * self.I + 6 * self.T * self.H * self.Is


CONFIGS = [
    MoEConfig(0, "tiny", T=64, H=256, E=16, k=4, I=128, Is=128, scale=2.5),
    MoEConfig(1, "mid", T=4096, H=2048, E=64, k=4, I=1536, Is=1536, scale=1.0),
    MoEConfig(2, "glm5_decode", T=16, H=6144, E=256, k=8, I=2048, Is=2048, scale=2.5),
    MoEConfig(3, "glm5_prefill", T=8192, H=6144, E=256, k=8, I=2048, Is=2048, scale=2.5, weights_of=2),
    MoEConfig(4, "glm5_skewed", T=32768, H=6144, E=256, k=8, I=2048, Is=2048, scale=2.5, skewed=True,
              weights_of=2),
    MoEConfig(5, "glm47_decode", T=16, H=2048, E=64, k=4, I=1536, Is=1536, scale=1.8),
    MoEConfig(6, "glm47_prefill", T=8192, H=2048, E=64, k=4, I=1536, Is=1536, scale=1.8, weights_of=5),
]
# The three GLM-5 workloads are one layer (one set of expert weights, 19.3 GB of routed experts) run on
# three token batches; each has its own tokens, router weight and bias. The two GLM-4.7-Flash workloads
# likewise share one layer.
BY_NAME = {c.name: c for c in CONFIGS}


@dataclass(frozen=True)
class DenseConfig:
    """The dense SwiGLU MLP of a dense-first block: x [T, H] -> (silu(x W1) * (x W3)) W2, width Id."""
    index: int
    name: str
    T: int
    H: int
    Id: int
    weights_of: int = -1

    @property
    def seed(self) -> int:
        return 0x5EED0000 + self.index

    @property
    def weight_seed(self) -> int:
        return 0x5EED0000 + (self.index if self.weights_of < 0 else self.weights_of)

    def flops(self) -> int:
        return 6 * self.T * self.H * self.Id


DENSE_CONFIGS = [
    DenseConfig(7, "dense_tiny", T=64, H=256, Id=384),
    DenseConfig(8, "glm5_dense_decode", T=16, H=6144, Id=12288),
    DenseConfig(9, "glm5_dense_prefill", T=8192, H=6144, Id=12288, weights_of=8),
    DenseConfig(10, "glm47_dense_prefill", T=8192, H=2048, Id=10240),
]
DENSE_BY_NAME = {c.name: c for c in DENSE_CONFIGS}


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal_bf16(seed: int, tensor: int, sigma: float, start: int, count: int, out: np.ndarray | None = None,
                nthreads: int | None = None) -> np.ndarray:
    """bf16 bits (uint16) of sigma * N for elements [start, start + count) of one tensor."""
    if out is None:
        out = np.empty(count, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == count
    lib().gen_normal_bf16(seed, tensor, sigma, start, count, _ptr(out), nthreads or host_threads())
    return out


def uniform_f32(seed: int, tensor: int, lo: float, hi: float, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    lib().gen_uniform_f32(seed, tensor, lo, hi, start, count, _ptr(out), host_threads())
    return out


def router_weight(cfg: MoEConfig, seed: int | None = None) -> np.ndarray:
    seed = cfg.seed if seed is None else seed
    if cfg.skewed:
        out = np.empty(cfg.E * cfg.H, dtype=np.uint16)
        lib().gen_skew_router_bf16(seed, T_WR, cfg.E, cfg.H, SIGMA_W, SKEW_ALPHA, SKEW_POWER, _ptr(out))
        return out.reshape(cfg.E, cfg.H)
    return normal_bf16(seed, T_WR, SIGMA_W, 0, cfg.E * cfg.H).reshape(cfg.E, cfg.H)


def selection_bias(cfg: MoEConfig, seed: int | None = None) -> np.ndarray:
    seed = cfg.seed if seed is None else seed
    if cfg.skewed:
        out = np.empty(cfg.E, dtype=np.float32)
        lib().gen_log_bias_f32(cfg.E, SKEW_BIAS_COEF, _ptr(out))
        return out
    return uniform_f32(seed, T_B, BIAS_LO, BIAS_HI, 0, cfg.E)


def tokens(cfg: MoEConfig, seed: int | None = None, start_row: int = 0, rows: int | None = None) -> np.ndarray:
    seed = cfg.seed if seed is None else seed
    rows = cfg.T - start_row if rows is None else rows
    return normal_bf16(seed, T_X, 1.0, start_row * cfg.H, rows * cfg.H).reshape(rows, cfg.H)


def weight_shapes(cfg: MoEConfig) -> dict:
    return {
        "w1": (T_W1, (cfg.E, cfg.I, cfg.H)),
        "w3": (T_W3, (cfg.E, cfg.I, cfg.H)),
        "w2": (T_W2, (cfg.E, cfg.H, cfg.I)),
        "ws1": (T_WS1, (cfg.Is, cfg.H)),
        "ws3": (T_WS3, (cfg.Is, cfg.H)),
        "ws2": (T_WS2, (cfg.H, cfg.Is)),
    }


def weight(cfg: MoEConfig, name: str, seed: int | None = None) -> np.ndarray:
    seed = cfg.weight_seed if seed is None else seed
    tid, shape = weight_shapes(cfg)[name]
    n = int(np.prod(shape))
    return normal_bf16(seed, tid, SIGMA_W, 0, n).reshape(shape)


def norm_weight(H: int, seed: int) -> np.ndarray:
    """RMSNorm weight gamma [H] as bf16 bits: bf16(1 + bf16(0.1 N))."""
    dev = normal_bf16(seed, T_GAMMA, GAMMA_SIGMA, 0, H)
    vals = (dev.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.array([lib().gen_bf16_from_double(1.0 + v) for v in vals], dtype=np.uint16)


def dense_tokens(cfg: DenseConfig) -> np.ndarray:
    return normal_bf16(cfg.seed, T_X, 1.0, 0, cfg.T * cfg.H).reshape(cfg.T, cfg.H)


def dense_weight(cfg: DenseConfig, name: str) -> np.ndarray:
    tid, shape = {"w1": (T_WD1, (cfg.Id, cfg.H)), "w3": (T_WD3, (cfg.Id, cfg.H)),
                  "w2": (T_WD2, (cfg.H, cfg.Id))}[name]
    return normal_bf16(cfg.weight_seed, tid, SIGMA_W, 0, int(np.prod(shape))).reshape(shape)


def host_inputs(cfg: MoEConfig, seed: int | None = None, with_weights: bool = True) -> dict:
    """Every input of one layer pass as host arrays (bf16 as uint16 bits)."""
    d = {"x": tokens(cfg, seed), "wr": router_weight(cfg, seed), "b": selection_bias(cfg, seed)}
    if with_weights:
        for name in ("w1", "w3", "w2", "ws1", "ws3", "ws2"):
            d[name] = weight(cfg, name, None if seed is None else seed)
    return d


def device_inputs(cfg: MoEConfig, device, seed: int | None = None, chunk_elems: int = 1 << 27) -> dict:
    """Every input of one layer pass as torch tensors on `device` (bf16 tensors as torch.bfloat16).

    Large tensors are generated on the host in chunks into one pinned staging buffer and copied up, so
    host memory stays at one chunk whatever the layer's size.
    """
    import torch

    wseed = cfg.weight_seed if seed is None else seed
    seed = cfg.seed if seed is None else seed
    out = {}
    small = {"x": tokens(cfg, seed) if cfg.T * cfg.H <= chunk_elems else None,
             "wr": router_weight(cfg, seed)}
    b = selection_bias(cfg, seed)
    out["b"] = torch.from_numpy(b).to(device)
    out["wr"] = torch.from_numpy(small["wr"].view(np.int16)).view(torch.bfloat16).to(device)
    stage = torch.empty(chunk_elems, dtype=torch.int16, pin_memory=True)
    stage_np = stage.numpy().view(np.uint16)

    def fill(tid, sigma, shape, fseed=seed):
        n = int(np.prod(shape))
        dst = torch.empty(n, dtype=torch.bfloat16, device=device)
        for s in range(0, n, chunk_elems):
            c = min(chunk_elems, n - s)
            normal_bf16(fseed, tid, sigma, s, c, out=stage_np[:c])
            dst[s:s + c].copy_(stage[:c].view(torch.bfloat16), non_blocking=True)
            torch.cuda.current_stream(device).synchronize()
        return dst.view(shape)

    if small["x"] is not None:
        out["x"] = torch.from_numpy(small["x"].view(np.int16)).view(torch.bfloat16).to(device)
    else:
        out["x"] = fill(T_X, 1.0, (cfg.T, cfg.H))
    for name, (tid, shape) in weight_shapes(cfg).items():
        out[name] = fill(tid, SIGMA_W, shape, wseed)
    torch.cuda.synchronize(device)
    return out

