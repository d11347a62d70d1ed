"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds input recipes only: random draws, the fp32 -> BF16 rounding
of those draws, and the placement of special entries.  It computes nothing
of the coding method itself (no symbols, counts, dictionaries, codes or
escapes), so the oracle and the GPU path both receive the same bytes from it
without sharing any of the method's arithmetic.

The pages measured the method on a real checkpoint that is not available
here; these tensors stand in for it, with the shapes, value distributions
and special structure of the five workloads below.  Every array is BF16 bit
patterns (``uint16``), row-major.

Workloads (``rows x cols``):
  small     1024 x 1024, N(0, 0.02), 0.05% of entries scaled x1000; x ~ N(0,1)
  square    4096 x 4096, N(0, 0.02), 1% exact +0, 0.1% outliers ~ N(0, 2)
  mlp       14336 x 4096 and 4096 x 14336, row std 10^U(-4,-1)
  layerset  48 x (6144 x 24576) and 24 x (24576 x 6144) ~ N(0, 0.015),
            24 norm vectors [6144] ~ N(1, 0.05)
  banded    6144 x 24576, N(0, 0.02) with 5 of the 96 64-row bands filled
            (96% of their entries) with rare sign+exponent patterns;
            X [16, 24576] ~ N(0, 1) (batch 1 and 4 use its first rows)
"""
from __future__ import annotations

import numpy as np

SEEDS = {"small": 1, "square": 2, "mlp": 3, "layerset": 4, "banded": 5}


def bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to the nearest BF16, ties to even.

    A BF16 value is the upper 16 bits of an fp32.  Rounding adds half of the
    dropped range (0x7FFF) plus the kept part's lowest bit, so a tie moves
    to the even neighbour, then truncates.  Inputs must be finite."""
    a = np.ascontiguousarray(f32, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("bf16_bits expects finite inputs")
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, sigma, mean=0.0):
    z = rng.standard_normal(shape, dtype=np.float32)
    return (np.float32(mean) + np.float32(sigma) * z).astype(np.float32)


def _vectors(cfg: int, batch: int, cols: int) -> np.ndarray:
    rng = np.random.default_rng([cfg, 1000])
    return bf16_bits(_normal(rng, (batch, cols), 1.0))


def small(seed: int = SEEDS["small"]):
    """1024x1024 N(0, 0.02); round(0.0005 n) entries scaled x1000; x ~ N(0,1)."""
    rows = cols = 1024
    n = rows * cols
    rng = np.random.default_rng(seed)
    w = _normal(rng, n, 0.02)
    k = int(round(0.0005 * n))
    pos = rng.permutation(n)[:k]
    w[pos] *= np.float32(1000.0)
    return {"W": bf16_bits(w).reshape(rows, cols), "x": _vectors(seed, 1, cols),
            "scaled_positions": np.sort(pos)}


def square(seed: int = SEEDS["square"]):
    """4096x4096 N(0, 0.02); 1% exact +0; 0.1% outliers ~ N(0, 2); x ~ N(0,1)."""
    rows = cols = 4096
    n = rows * cols
    rng = np.random.default_rng(seed)
    w = _normal(rng, n, 0.02)
    nz = int(round(0.01 * n))
    no = int(round(0.001 * n))
    perm = rng.permutation(n)
    zpos, opos = perm[:nz], perm[nz:nz + no]
    w[opos] = _normal(rng, no, 2.0)
    bits = bf16_bits(w)
    bits[zpos] = 0x0000  # +0.0
    return {"W": bits.reshape(rows, cols), "x": _vectors(seed, 1, cols),
            "zero_positions": np.sort(zpos), "outlier_positions": np.sort(opos)}


def mlp(seed: int = SEEDS["mlp"]):
    """W1 14336x4096 and W2 4096x14336; row r scaled by 10^U(-4,-1)."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, (rows, cols) in (("W1", (14336, 4096)), ("W2", (4096, 14336))):
        sig = np.power(10.0, rng.uniform(-4.0, -1.0, rows)).astype(np.float32)
        z = rng.standard_normal((rows, cols), dtype=np.float32)
        out[name] = bf16_bits(sig[:, None] * z)
    xr = np.random.default_rng([seed, 1000])
    out["x1"] = bf16_bits(_normal(xr, (1, 4096), 1.0))
    out["x2"] = bf16_bits(_normal(xr, (1, 14336), 1.0))
    return out


LAYERSET_TENSORS = 96


def layerset_spec(t: int):
    """(name, shape, mean, sigma) of tensor t of the 96-tensor layer set."""
    if t < 48:
        return f"up.{t}", (6144, 24576), 0.0, 0.015
    if t < 72:
        return f"down.{t - 48}", (24576, 6144), 0.0, 0.015
    if t < 96:
        return f"norm.{t - 72}", (6144,), 1.0, 0.05
    raise IndexError(t)


def layerset_tensor(t: int, scale_rows: int | None = None):
    """Tensor t of the layer set (seeded by [4, t]).  ``scale_rows`` keeps only
    that many leading rows (for tests that need a smaller slice)."""
    name, shape, mean, sigma = layerset_spec(t)
    rng = np.random.default_rng([SEEDS["layerset"], t])
    if scale_rows is not None and len(shape) == 2:
        shape = (min(scale_rows, shape[0]), shape[1])
    return name, bf16_bits(_normal(rng, shape, sigma, mean))


# Sign+exponent patterns for the dense escape bands: high bytes h (sign bit
# and the top 7 exponent bits) whose magnitude lies outside the range N(0,
# 0.02) weights occupy (|w| in [2^-21, 2^-1), i.e. h & 0x7F in 53..62), and
# whose exponent stays normal and finite (h & 0x7F in 1..71 gives
# 2^-125 <= |w| < 2^17).
BAND_HIGH_BYTES = np.array(
    [s | m for s in (0x00, 0x80) for m in list(range(1, 53)) + list(range(63, 72))],
    dtype=np.uint16)


def banded(seed: int = SEEDS["banded"], rows: int = 6144, cols: int = 24576,
           bands: int = 5, band_rows: int = 64, fill: float = 0.96, batch: int = 16):
    """N(0, 0.02) with `bands` of the 64-row bands filled (Bernoulli `fill`)
    with (h << 8) | lo, h cycling over a shuffled BAND_HIGH_BYTES and lo
    uniform in 0..255.  X [batch, cols] ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    w = bf16_bits(_normal(rng, (rows, cols), 0.02))
    nb = rows // band_rows
    chosen = np.sort(rng.choice(nb, size=bands, replace=False))
    order = rng.permutation(BAND_HIGH_BYTES)
    k = 0
    for b in chosen:
        blk = w[b * band_rows:(b + 1) * band_rows]
        mask = rng.random(blk.shape) < fill
        m = int(mask.sum())
        hi = order[(k + np.arange(m)) % len(order)]
        lo = rng.integers(0, 256, size=m, dtype=np.uint16)
        blk[mask] = (hi << 8) | lo
        k += m
    return {"W": w, "X": _vectors(seed, batch, cols), "bands": chosen}


def random_bits(n: int, seed: int, kind: str = "normal", sigma: float = 0.02) -> np.ndarray:
    """Generic test tensors: 'normal' N(0, sigma) rounded to BF16, 'uniform'
    16-bit patterns (NaN payloads, infinities, subnormals included),
    'few' values drawn from at most 7 patterns."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return bf16_bits(_normal(rng, n, sigma))
    if kind == "uniform":
        return rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
    if kind == "few":
        vals = rng.integers(0, 1 << 16, size=7, dtype=np.uint16)
        return vals[rng.integers(0, 7, size=n)]
    raise ValueError(kind)


def all_patterns(shuffle_seed: int | None = None) -> np.ndarray:
    """Every one of the 65,536 BF16 bit patterns, in order or shuffled."""
    a = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if shuffle_seed is not None:
        a = np.random.default_rng(shuffle_seed).permutation(a)
    return a


def vectors(cfg_seed: int, batch: int, cols: int) -> np.ndarray:
    """x [batch, cols] ~ N(0, 1) rounded to BF16 (seeded by [cfg_seed, 1000])."""
    return _vectors(cfg_seed, batch, cols)


def layerset_tensor_device(t: int, device):
    """Tensor t of the layer set drawn on a GPU (torch's seeded device
    generator, seed 4000 + t), as int16 BF16 bit patterns: the same shapes and
    distributions as ``layerset_tensor``, without drawing 20 GiB on the host.
    The values differ from the host draw; both stand in for the same recipe."""
    import torch
    name, shape, mean, sigma = layerset_spec(t)
    n = int(np.prod(shape))
    g = torch.Generator(device=device)
    g.manual_seed(4000 + t)
    z = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    z.mul_(sigma).add_(mean)
    return name, shape, z.to(torch.bfloat16).view(torch.int16)
