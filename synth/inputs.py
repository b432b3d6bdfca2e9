"""Seeded synthetic inputs for the fused linear + cross-entropy (log-prob) path.

This module only draws random numbers and rounds them to bf16 bit patterns.  It
holds none of the method's arithmetic, so both the fp64 oracle's tests and the
HIP path's tests can use it without sharing any computation.

Workloads follow the pages' synthetic, "random BF16" shape sweeps (Liger-Kernel
FSLCE commit message, section "Model-shape campaign"; SkyRL PR 2141, section
"H100 benchmark": a synthetic kernel-shape sweep that consumes no dataset).

Every stream is ``default_rng(SeedSequence([2026, case_id, k]))`` with

  k = 0 X, 1 W, 2 targets, 3 ignored rows, 4 large-magnitude rows,
      5 grad_logprob, 6 grad_entropy.

Normals are drawn as float32, multiplied by the standard deviation in float32
and rounded to bf16 with round-to-nearest-even on the bit pattern.  Large draws
are made in row chunks; numpy's generator yields the same sequence either way.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SEED_ROOT = 2026
IGNORE_INDEX = -100

_STREAM_X, _STREAM_W, _STREAM_T, _STREAM_IGN, _STREAM_BIG, _STREAM_GLP, _STREAM_GENT = range(7)


def _rng(case_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, int(case_id), int(stream)]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, rows: int, cols: int, std: float,
                 chunk_elems: int = 1 << 26) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint16)
    std32 = np.float32(std)
    rows_per = max(1, chunk_elems // max(cols, 1))
    for r0 in range(0, rows, rows_per):
        r1 = min(rows, r0 + rows_per)
        x = rng.standard_normal((r1 - r0) * cols, dtype=np.float32)
        x *= std32
        out[r0:r1] = f32_to_bf16_bits(x).reshape(r1 - r0, cols)
    return out


@dataclasses.dataclass
class Case:
    """One synthetic problem: bf16 bit arrays, targets, grads and scalars."""
    name: str
    M: int
    H: int
    V: int
    X: np.ndarray            # uint16 [M, H] bf16 bits
    W: np.ndarray            # uint16 [V, H] bf16 bits
    targets: np.ndarray      # int64 [M]
    ignore_index: int
    scale: float             # the float32 value handed to the kernel
    compute_entropy: bool
    grad_logprob: Optional[np.ndarray]   # float32 [M] or None
    grad_entropy: Optional[np.ndarray]   # float32 [M] or None


def make_case(name: str, case_id: int, M: int, H: int, V: int, *,
              scale: float = 1.0, compute_entropy: bool = True,
              ignore_frac: float = 0.0, big_rows_frac: float = 0.0, big_factor: float = 64.0,
              grad_mode: str = "inv_m", ignore_index: int = IGNORE_INDEX,
              x_std: float = 1.0, w_std: Optional[float] = None) -> Case:
    """Draw one case.

    grad_mode: "inv_m" -> grad_logprob = 1/M, no grad_entropy;
               "normal" -> grad_logprob and grad_entropy both N(0,1) float32;
               "normal_lp" -> grad_logprob N(0,1), no grad_entropy;
               "none" -> neither.
    """
    if w_std is None:
        w_std = 1.0 / math.sqrt(H)
    X = _normal_bf16(_rng(case_id, _STREAM_X), M, H, x_std)
    W = _normal_bf16(_rng(case_id, _STREAM_W), V, H, w_std)
    t = _rng(case_id, _STREAM_T).integers(0, V, size=M, dtype=np.int64)
    n_ign = int(round(ignore_frac * M))
    if n_ign:
        rows = _rng(case_id, _STREAM_IGN).permutation(M)[:n_ign]
        t[rows] = ignore_index
    n_big = int(round(big_rows_frac * M))
    if n_big:
        rows = np.sort(_rng(case_id, _STREAM_BIG).permutation(M)[:n_big])
        # big_factor is a power of two, so scaling the bf16 values is exact.
        xb = (X[rows].astype(np.uint32) << np.uint32(16)).view(np.float32) * np.float32(big_factor)
        X[rows] = f32_to_bf16_bits(xb)
    glp = gent = None
    if grad_mode == "inv_m":
        glp = np.full(M, np.float32(1.0) / np.float32(M), dtype=np.float32)
    elif grad_mode == "normal":
        glp = _rng(case_id, _STREAM_GLP).standard_normal(M, dtype=np.float32)
        gent = _rng(case_id, _STREAM_GENT).standard_normal(M, dtype=np.float32)
    elif grad_mode == "normal_lp":
        glp = _rng(case_id, _STREAM_GLP).standard_normal(M, dtype=np.float32)
    elif grad_mode != "none":
        raise ValueError(grad_mode)
    return Case(name, M, H, V, X, W, t, ignore_index, float(np.float32(scale)),
                compute_entropy, glp, gent)


# The five workloads the measurements are quoted on (sizes and distributions as
# stated for them; ignore fractions rounded to whole rows).
CONFIGS = {
    1: dict(M=64, H=128, V=1000, scale=1.0, compute_entropy=True, ignore_frac=0.05,
            grad_mode="inv_m"),
    2: dict(M=4096, H=4096, V=32768, scale=1.0, compute_entropy=True, ignore_frac=0.02,
            grad_mode="inv_m"),
    3: dict(M=4096, H=4096, V=128256, scale=float(np.float32(1.0 / 0.7)), compute_entropy=False,
            ignore_frac=0.0, grad_mode="inv_m"),
    4: dict(M=8192, H=8192, V=131072, scale=1.0, compute_entropy=True, ignore_frac=0.0,
            grad_mode="inv_m"),
    5: dict(M=32767, H=2048, V=151936, scale=1.0, compute_entropy=True, ignore_frac=0.10,
            big_rows_frac=0.10, big_factor=64.0, grad_mode="normal"),
}

CONFIG_NAMES = {
    1: "tiny M=64 H=128 V=1000",
    2: "M=4096 H=4096 V=32768",
    3: "ragged-vocab logprob-only M=4096 H=4096 V=128256 T=0.7",
    4: "large M=8192 H=8192 V=131072",
    5: "stress M=32767 H=2048 V=151936 x64 rows",
}


def config_case(cfg: int, **overrides) -> Case:
    kw = dict(CONFIGS[cfg])
    kw.update(overrides)
    return make_case(f"config{cfg}", cfg, **kw)


def decode_bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> float32 values (exact).  Used for building crafted inputs."""
    return (np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)
