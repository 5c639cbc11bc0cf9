"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module draws random numbers and rounds them to bf16; it holds none of the
projection's arithmetic.  Neither the oracle nor the HIP library imports it;
both receive the tensors it makes.

Recipe (stands in for model weights, which the blog series "On descend d'un
cran" loads from Qwen3.5 safetensors files and which are not available here):

* generator: numpy ``PCG64`` seeded with
  ``SeedSequence(entropy=config_no, spawn_key=(tensor_id, stream))``;
  ``stream`` 0 draws the values, ``stream`` 1 draws the outlier mask;
* values: ``standard_normal(float32) * sigma`` (sigma is the standard
  deviation), then optional outliers: each element independently, with
  probability ``outlier_frac``, is multiplied by ``outlier_scale``;
* rounding to bf16: IEEE round-to-nearest-even, done by torch's CPU cast
  ``float32 -> bfloat16`` (a library routine);
* integer probes: uniform integers in ``[-lim, lim]`` stored as bf16 (exact).

bf16 tensors are returned as numpy ``uint16`` bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE, via torch) -> uint16 bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def rng(config_no: int, tensor_id: int, stream: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=config_no, spawn_key=(tensor_id, stream))
    return np.random.Generator(np.random.PCG64(ss))


def normal_bf16(config_no: int, tensor_id: int, shape, sigma: float,
                outlier_frac: float = 0.0, outlier_scale: float = 10.0) -> np.ndarray:
    g = rng(config_no, tensor_id, 0)
    v = g.standard_normal(size=shape, dtype=np.float32)
    v *= np.float32(sigma)
    if outlier_frac > 0:
        mask = rng(config_no, tensor_id, 1).random(size=shape) < outlier_frac
        v[mask] *= np.float32(outlier_scale)
    return bf16_from_f32(v)


def int_bf16(seed: int, shape, lim: int = 4) -> np.ndarray:
    """Integer-valued bf16 tensor, entries uniform in [-lim, lim] (exact in bf16)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(7777,))))
    v = g.integers(-lim, lim + 1, size=shape).astype(np.float32)
    return bf16_from_f32(v)


def norm_boundary_case(K: int, seed: int = 0):
    """Rows and norm weights whose normalised values sit next to bf16 rounding
    boundaries (for tests that must tell the divisor of the mean and the place
    of epsilon apart, which a one-ulp comparison on random rows cannot).

    Returns (X, gamma, lo, hi):
      X      bf16 bits [2, K]: row 0 all ones, row 1 all 2^-10;
      gamma  f32 [K]: gamma[j] = f32(m_j * (1 + 1/(4K))), where m_j is the
             midpoint between a random bf16 value v_j (|v_j| in [0.5, 2), random
             sign) and its neighbour one ulp further from zero;
      lo, hi the bf16 bits of v_j and of that neighbour."""
    g = rng(90000 + K, seed, 0)
    mag = g.uniform(0.5, 2.0, size=K).astype(np.float32)
    lo = bf16_from_f32(mag)
    lo = np.where(lo >= 0x4000, np.uint16(0x3FFF), lo).astype(np.uint16)   # keep |v| < 2 after the step up
    hi = (lo + 1).astype(np.uint16)
    sign = (g.random(size=K) < 0.5).astype(np.uint16) << 15
    lo, hi = lo | sign, hi | sign
    wide = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mid = (wide(lo) + wide(hi)) / 2.0
    gamma = (mid * (1.0 + 1.0 / (4.0 * K))).astype(np.float32)
    X = np.empty((2, K), dtype=np.uint16)
    X[0] = 0x3F80                     # 1.0
    X[1] = 0x3A80                     # 2^-10
    return X, gamma, lo, hi


@dataclass(frozen=True)
class Projection:
    name: str
    N: int          # output features (rows of W)
    K: int          # input features


@dataclass(frozen=True)
class Config:
    no: int
    name: str
    projections: tuple
    Ms: tuple
    w_sigma: float
    x_sigma: float = 1.0
    outlier_frac: float = 0.0
    notes: str = ""
    extra: dict = field(default_factory=dict)


_L08 = (Projection("qkv", 2048, 1024), Projection("out", 1024, 1024),
        Projection("gate_up", 6144, 1024), Projection("down", 1024, 3072))
_L4B = (Projection("qkv", 5120, 2560), Projection("out", 2560, 4096),
        Projection("gate_up", 18432, 2560), Projection("down", 2560, 9216))
_L27 = (Projection("qkv", 10240, 5120), Projection("out", 5120, 8192),
        Projection("gate_up", 34816, 5120), Projection("down", 5120, 17408))

CONFIGS = (
    Config(0, "single_1024x1024", (Projection("proj", 1024, 1024),), (1, 16), 0.02,
           notes="single projection, Y fp32"),
    Config(1, "decode_0.8b_layer_m1", _L08 + (Projection("head", 151936, 1024),), (1,), 0.02,
           notes="0.8B-like decoder layer plus output head at M=1"),
    Config(2, "prefill_4b_layer", _L4B, (128, 512, 2048), 0.02,
           notes="4B-like decoder layer"),
    Config(3, "long_prompt_4b_8192x1024", _L4B + (Projection("head", 151936, 2560),), (1024,), 0.02,
           notes="8192 prompt rows as 8 blocks of 1024; head on the last row only",
           extra={"prompt_rows": 8192, "block": 1024}),
    Config(4, "layer_27b", _L27, (1, 8192), 0.01, outlier_frac=0.01,
           notes="27B-like layer, weights with 1% outliers x10"),
)

_BY_NAME = {c.name: c for c in CONFIGS}


def workload(name: str) -> Config:
    """The workload of that name (single_1024x1024, decode_0.8b_layer_m1,
    prefill_4b_layer, long_prompt_4b_8192x1024, layer_27b)."""
    return _BY_NAME[name]


# Extra shape printed by the pages: the 0.8B gate/up projection 1024 -> 7168
# ("#002 le meme compilateur sur un GPU", section "Emettre pour un GPU").
PAGES_GATE_UP_08B = Projection("gate_up_pages", 7168, 1024)


def tensor_ids(cfg: Config, proj_index: int):
    """(W tensor id, X tensor id) for a projection: W and X of each projection
    are drawn from their own streams, in the listed order."""
    return 2 * proj_index, 2 * proj_index + 1


def weights(cfg: Config, proj_index: int) -> np.ndarray:
    p = cfg.projections[proj_index]
    wid, _ = tensor_ids(cfg, proj_index)
    return normal_bf16(cfg.no, wid, (p.N, p.K), cfg.w_sigma, cfg.outlier_frac)


def activations(cfg: Config, proj_index: int, M: int) -> np.ndarray:
    p = cfg.projections[proj_index]
    _, xid = tensor_ids(cfg, proj_index)
    # Seed by (config, tensor, M) through the stream index so every M gets its own X.
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        entropy=cfg.no, spawn_key=(xid, 100 + M))))
    v = g.standard_normal(size=(M, p.K), dtype=np.float32) * np.float32(cfg.x_sigma)
    return bf16_from_f32(v)

