"""Seeded synthetic inputs for the DeepSeekMoE layer forward.

This module is shared by the oracle-side tests and by the HIP-side tests and
benchmark.  It draws random numbers and nothing else: no routing, no
quantisation, no GEMM.  Every tensor comes from its own NumPy PCG64 child
stream ``default_rng([seed, tensor_id, index])`` so that tensors can be drawn
in any order, in parallel, or one expert at a time.

Workload shapes follow the DeepSeek-V3 model-shape table (hidden 7168; one
shared plus 256 routed experts, 8 active per token) printed in the aliyun
study note "DeepSeek-V3：671B 巨兽" (developer.aliyun.com/article/1776647),
section 一 (规模), and the news.qq.com article on how V3 was built
(news.qq.com/rain/a/20241229A05OQF00), section 架构 › DeepSeekMoE 架构.
The expert intermediate width (2048), the 8-group / keep-4 group rule and the
distributions define the measured workloads (the pages give them only in part).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids of the child streams
TID_X = 1
TID_CENTROIDS = 2
TID_BIAS = 3
TID_W_GU = 4
TID_W_DN = 5
TID_GEMM_A = 6
TID_GEMM_COUNTS = 7
TID_ZIPF_SCALE = 8
TID_DY = 9


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens
    H: int            # hidden size
    E: int            # routed experts
    n_group: int      # expert groups (contiguous blocks of E/n_group experts)
    topk_group: int   # groups kept per token
    k: int            # routed experts per token
    I: int            # expert intermediate size (SwiGLU)
    n_shared: int = 1
    x_std: float = 1.0
    c_std: float = 0.02
    w_std: float = 0.02
    bias_lim: float = 0.01
    seed: int = 0

    @property
    def R(self) -> int:
        """Rows of the grouped GEMMs: routed assignments plus shared rows."""
        return self.T * self.k + self.n_shared * self.T

    @property
    def G(self) -> int:
        """GEMM groups: routed experts plus the shared expert(s)."""
        return self.E + self.n_shared

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# Tiny layer: hidden 256, 16 experts in 4 groups, keep 2, top-4, I=128.
TINY = MoEConfig("tiny", T=64, H=256, E=16, n_group=4, topk_group=2, k=4, I=128,
                 w_std=0.02)
# V3 shapes at decode batch (T=128) and at a prefill batch (T=16384).
DECODE = MoEConfig("decode", T=128, H=7168, E=256, n_group=8, topk_group=4, k=8,
                   I=2048, w_std=0.006)
PREFILL = DECODE.with_(name="prefill", T=16384)
# Skewed-load layer (Zipf-scaled centroids, fresh batch per step).
SKEWED = DECODE.with_(name="skewed", T=8192, bias_lim=0.0)
# Mid-size case: several tiles of every kernel plus ragged tails, yet the
# FP64 oracle finishes in seconds.
MID = MoEConfig("mid", T=200, H=1024, E=64, n_group=8, topk_group=4, k=8, I=384,
                w_std=0.02)

CONFIGS = {c.name: c for c in (TINY, DECODE, PREFILL, SKEWED, MID)}


def _rng(seed: int, tid: int, idx: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tid, idx])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 draws to bf16 (round to nearest even) and return the bits.

    Uses torch's CPU cast, which rounds to nearest even; this only defines the
    input tensor x, it is not a step of the method.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def gen_x(cfg: MoEConfig, seed: int | None = None, T: int | None = None) -> np.ndarray:
    """Activations x [T, H] as bf16 bit patterns (uint16), N(0, x_std) then RNE."""
    seed = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    x = _rng(seed, TID_X).standard_normal((T, cfg.H), dtype=np.float32)
    if cfg.x_std != 1.0:
        x *= np.float32(cfg.x_std)
    return f32_to_bf16_bits(x)


def gen_dy(cfg: MoEConfig, seed: int | None = None, T: int | None = None) -> np.ndarray:
    """Gradient of the layer output dy [T, H] as bf16 bit patterns, N(0, 1) then RNE."""
    seed = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    return f32_to_bf16_bits(_rng(seed, TID_DY).standard_normal((T, cfg.H), dtype=np.float32))


def gen_centroids(cfg: MoEConfig, seed: int | None = None) -> np.ndarray:
    """Router centroids C [E, H] fp32, N(0, c_std)."""
    seed = cfg.seed if seed is None else seed
    c = _rng(seed, TID_CENTROIDS).standard_normal((cfg.E, cfg.H), dtype=np.float32)
    return (c * np.float32(cfg.c_std)).astype(np.float32)


def gen_bias(cfg: MoEConfig, seed: int | None = None) -> np.ndarray:
    """Per-expert selection bias b [E] fp32, U(-bias_lim, bias_lim)."""
    seed = cfg.seed if seed is None else seed
    if cfg.bias_lim == 0.0:
        return np.zeros(cfg.E, np.float32)
    b = _rng(seed, TID_BIAS).uniform(-cfg.bias_lim, cfg.bias_lim, cfg.E)
    return b.astype(np.float32)


def gen_expert_weight(cfg: MoEConfig, which: str, e: int,
                      seed: int | None = None) -> np.ndarray:
    """fp32 weights of expert e (e == E is the shared expert) before quantisation.

    which='gu': fused gate+up [2I, H] (rows [0, I) gate, [I, 2I) up).
    which='dn': down projection [H, I].
    Both are stored [N, K] (K contiguous), N(0, w_std).
    """
    seed = cfg.seed if seed is None else seed
    if which == "gu":
        shape, tid = (2 * cfg.I, cfg.H), TID_W_GU
    elif which == "dn":
        shape, tid = (cfg.H, cfg.I), TID_W_DN
    else:
        raise ValueError(which)
    w = _rng(seed, tid, e).standard_normal(shape, dtype=np.float32)
    w *= np.float32(cfg.w_std)
    return w


def gen_all_expert_weights(cfg: MoEConfig, which: str, experts=None,
                           threads: int | None = None, seed: int | None = None):
    """Yield (e, fp32 weight) for the given experts, drawn on a thread pool."""
    if experts is None:
        experts = range(cfg.G)
    experts = list(experts)
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(threads) as ex:
        futs = [(e, ex.submit(gen_expert_weight, cfg, which, e, seed)) for e in experts]
        for e, f in futs:
            yield e, f.result()


def gen_group_counts(n_rows: int, G: int, seed: int = 0) -> np.ndarray:
    """Rows per group, Multinomial(n_rows, uniform over G groups)."""
    return _rng(seed, TID_GEMM_COUNTS).multinomial(n_rows, np.full(G, 1.0 / G)).astype(np.int64)


def gen_gemm_activations(rows: int, K: int, seed: int = 0) -> np.ndarray:
    """Dense activations [rows, K] as bf16 bits, N(0, 1) then RNE."""
    a = _rng(seed, TID_GEMM_A).standard_normal((rows, K), dtype=np.float32)
    return f32_to_bf16_bits(a)


def int_fp8_operand(shape, seed: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Integer values in [lo, hi] as float32 (for exact-arithmetic GEMM cases)."""
    r = np.random.default_rng([seed, 99])
    return r.integers(lo, hi + 1, size=shape).astype(np.float32)


def pow2_scales(shape, seed: int, lo: int = -3, hi: int = 3) -> np.ndarray:
    """Power-of-two fp32 scales 2^[lo, hi] (exact-arithmetic GEMM cases)."""
    r = np.random.default_rng([seed, 98])
    return np.ldexp(np.float32(1.0), r.integers(lo, hi + 1, size=shape)).astype(np.float32)


# ---------------------------------------------------------------------------
# Skewed-load workload: router centroids N(0, c_std) whose expert rows are
# scaled by per-expert factors, so that expert popularity follows a Zipf(1.1)
# curve over a random ranking of the experts.  The factors are fitted once, on
# a calibration batch, by tests/golden/make_zipf_scale.py and stored in
# tests/golden/zipf_scale.txt; this module only reads them.
ZIPF_S = 1.1
ZIPF_CAL_SEED = 7          # calibration batch of the fit
ZIPF_STEP_SEED0 = 1000     # batch of run step i: seed 1000 + i
ZIPF_SCALE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                               "tests", "golden", "zipf_scale.txt")


def zipf_ranks(E: int, seed: int = 0) -> np.ndarray:
    """Popularity rank (1 = most popular) of each expert: a random permutation."""
    return _rng(seed, TID_ZIPF_SCALE).permutation(E).astype(np.int64) + 1


def load_zipf_scale(path: str = ZIPF_SCALE_FILE) -> np.ndarray:
    """Per-expert centroid scale factors [E] (fp32) from the stored fit."""
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    return np.array([float(r[1]) for r in rows], dtype=np.float32)


def gen_zipf_centroids(cfg: MoEConfig, scale: np.ndarray | None = None) -> np.ndarray:
    """Skewed-load centroids: gen_centroids(cfg) with row e multiplied by scale[e]."""
    scale = load_zipf_scale() if scale is None else np.asarray(scale, np.float32)
    return (gen_centroids(cfg) * scale[:, None]).astype(np.float32)
