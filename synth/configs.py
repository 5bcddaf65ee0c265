"""The synthetic layer workloads and their seeded generators.

Every draw comes from numpy PCG64 streams keyed by (base seed, stream id, ...),
so any expert can be regenerated on its own, in any order:
  stream (0,)        router weight Wr [E, H], fp32 N(0, 0.02)
  stream (1,)        router bias rank permutation (Zipf-skewed workload only)
  stream (2,)        hidden states x [T, H], N(0, 1); the first rows do not
                     depend on T
  stream (3,)        outlier mask (Bernoulli, multiplies x by the outlier scale)
  stream (4, e, j)   expert e, matrix j (0 gate, 1 up, 2 down)
"""
from dataclasses import dataclass, replace
from typing import Optional, Tuple

import numpy as np

from .formats import (FMT_ASYM, FMT_E2M1, QMat, quantize_asym, quantize_e2m1,
                      random_qmat, f32_to_bf16_bits)

ACT_NONE = 0
ACT_I8_X = 1
ACT_I8_XH = 2


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    x_dtype: str                 # "f32" or "bf16"
    fmt: Tuple[int, int, int]    # (fmt, bits, group) of every expert ...
    cold_fmt: Optional[Tuple[int, int, int]] = None  # ... or of the cold ones
    n_hot: int = 0               # hot experts = the n_hot largest router biases
    expert_fmts: Optional[Tuple[Tuple[int, int, int], ...]] = None  # per-expert override
    zipf_alpha: float = 0.0      # router bias b_e = -alpha * ln(rank_e)
    act: int = ACT_NONE          # per-token int8 expert inputs
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    weight_mode: str = "codes"   # "quantize" (N(0,0.02) then quantise) or "codes"
    seed: int = 0
    decode_T: Tuple[int, ...] = ()
    # share of each expert matrix kept as an fp16 outlier side list
    weight_outlier_frac: float = 0.0
    # per-expert (gate, up, down) formats, overriding the ones above
    matrix_fmts: Optional[Tuple[Tuple[Tuple[int, int, int], ...], ...]] = None


A4G32 = (FMT_ASYM, 4, 32)
A2G16 = (FMT_ASYM, 2, 16)
A4G128 = (FMT_ASYM, 4, 128)
A1G16 = (FMT_ASYM, 1, 16)
A1G32 = (FMT_ASYM, 1, 32)
A3G32 = (FMT_ASYM, 3, 32)
A3G64 = (FMT_ASYM, 3, 64)
E2M1G16 = (FMT_E2M1, 4, 16)

# Router bias strength for the hot/cold workload: with alpha = 0.375 the 32
# most-routed of 256 experts take about half of the top-8 assignments at
# T = 4096 (checked against the oracle's routing in the tests).
HOTCOLD_ALPHA = 0.375

CONFIGS = {
    # 64 tokens, hidden 256, 8 experts, top-2, intermediate 512; 4-bit g32.
    "tiny": LayerConfig("tiny", 64, 256, 512, 8, 2, "f32", A4G32,
                        weight_mode="quantize", seed=1001),
    # Mixtral-8x7B-shaped layer (decode 1/8/32 tokens, prefill 2048).
    "mixtral": LayerConfig("mixtral", 2048, 4096, 14336, 8, 2, "bf16", A4G32,
                           seed=1002, decode_T=(1, 8, 32)),
    # 256 fine-grained experts, top-6, e2m1 weights with an fp16 scale per 16.
    "fine_e2m1": LayerConfig("fine_e2m1", 4096, 2048, 512, 256, 6, "bf16", E2M1G16,
                             seed=1003, decode_T=(1, 64)),
    # 64 hot experts at 4-bit g32, 192 cold at 2-bit g16, Zipf-skewed routing.
    "hotcold": LayerConfig("hotcold", 4096, 2048, 512, 256, 8, "bf16", A4G32,
                           cold_fmt=A2G16, n_hot=64, zipf_alpha=HOTCOLD_ALPHA,
                           seed=1004),
    # Large experts, 4-bit g128 weights, per-token int8 x and h.
    "w4a8": LayerConfig("w4a8", 8192, 8192, 16384, 64, 2, "bf16", A4G128,
                        act=ACT_I8_XH, outlier_frac=0.001, outlier_scale=20.0,
                        seed=1005, decode_T=(16,)),
}


def get_config(name: str, T: Optional[int] = None) -> LayerConfig:
    cfg = CONFIGS[name]
    return cfg if T is None else replace(cfg, T=T)


def scaled_config(name: str, T: int, H: int, I: int, E: Optional[int] = None,
                  k: Optional[int] = None, weight_mode: Optional[str] = None,
                  n_hot: Optional[int] = None) -> LayerConfig:
    """The same workload (formats, dtypes, skew, activation mode, seed) at
    reduced sizes, for parity runs the oracle finishes in seconds."""
    cfg = CONFIGS[name]
    kw = dict(T=T, H=H, I=I)
    if E is not None:
        kw["E"] = E
    if k is not None:
        kw["k"] = k
    if weight_mode is not None:
        kw["weight_mode"] = weight_mode
    if n_hot is not None:
        kw["n_hot"] = n_hot
    return replace(cfg, **kw)


def _rng(cfg: LayerConfig, *key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(entropy=cfg.seed, spawn_key=tuple(key))))


def _bias_ranks(cfg: LayerConfig) -> np.ndarray:
    """rank_e in 1..E (1 = largest bias), a seeded permutation of experts."""
    perm = _rng(cfg, 1).permutation(cfg.E)
    ranks = np.empty(cfg.E, dtype=np.int64)
    ranks[perm] = np.arange(1, cfg.E + 1)
    return ranks


def gen_router(cfg: LayerConfig):
    """Wr [E, H] fp32 N(0, 0.02); b [E] fp32 (zeros unless Zipf-skewed)."""
    Wr = (_rng(cfg, 0).standard_normal((cfg.E, cfg.H), dtype=np.float32)
          * np.float32(0.02))
    if cfg.zipf_alpha > 0:
        b = (-cfg.zipf_alpha * np.log(_bias_ranks(cfg).astype(np.float64))).astype(np.float32)
    else:
        b = np.zeros(cfg.E, dtype=np.float32)
    return Wr, b


def gen_x(cfg: LayerConfig, T: Optional[int] = None) -> np.ndarray:
    """Hidden states [T, H]: fp32 array, or uint16 bf16 bit patterns."""
    T = cfg.T if T is None else T
    x = _rng(cfg, 2).standard_normal((T, cfg.H), dtype=np.float32)
    if cfg.outlier_frac > 0:
        mask = _rng(cfg, 3).random((T, cfg.H)) < cfg.outlier_frac
        x = np.where(mask, x * np.float32(cfg.outlier_scale), x).astype(np.float32)
    if cfg.x_dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def expert_format(cfg: LayerConfig, e: int) -> Tuple[int, int, int]:
    if cfg.expert_fmts is not None:
        return cfg.expert_fmts[e]
    if cfg.cold_fmt is None:
        return cfg.fmt
    return cfg.fmt if _bias_ranks(cfg)[e] <= cfg.n_hot else cfg.cold_fmt


def matrix_formats(cfg: LayerConfig, e: int):
    """(gate, up, down) formats of expert e."""
    if cfg.matrix_fmts is not None:
        return tuple(cfg.matrix_fmts[e])
    f = expert_format(cfg, e)
    return (f, f, f)


def gen_expert(cfg: LayerConfig, e: int):
    """Expert e as a dict of canonical QMats: gate [I,H], up [I,H], down [H,I]."""
    shapes = {"gate": (cfg.I, cfg.H), "up": (cfg.I, cfg.H), "down": (cfg.H, cfg.I)}
    fr = cfg.weight_outlier_frac
    out = {}
    for j, (role, (fmt, bits, group)) in enumerate(zip(("gate", "up", "down"),
                                                       matrix_formats(cfg, e))):
        rows, cols = shapes[role]
        rng = _rng(cfg, 4, e, j)
        if cfg.weight_mode == "quantize":
            W = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02)
            if fr > 0:
                # heavy tail: a few weights well beyond the Gaussian bulk
                n = int(np.ceil(fr * rows * cols))
                pos = rng.choice(rows * cols, size=n, replace=False)
                W.reshape(-1)[pos] *= np.float32(8.0)
            if fmt == FMT_ASYM:
                out[role] = quantize_asym(W, bits, group, fr)
            else:
                out[role] = quantize_e2m1(W, group, fr)
        else:
            out[role] = random_qmat(rng, rows, cols, fmt, bits, group, outlier_frac=fr)
    return out
