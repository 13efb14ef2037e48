"""Seeded synthetic inputs for the GEMM workloads (shared by tests, oracle and bench).

This module only draws random numbers and turns them into 16-bit bit patterns; it
holds none of the GEMM's arithmetic.  Values are drawn in fp64 with numpy's PCG64
``default_rng(seed)``, converted to fp32 (round to nearest even) and then to the
16-bit type (fp16 through numpy's own conversion, bf16 by round-to-nearest-even on
the fp32 bit pattern).  The same bits are handed to the GPU and to the oracle, so
the exact rounding used here does not matter for parity.

Distributions follow the workloads: U[-1,1] for square/Strassen problems, N(0,1)
for activations and C_in, N(0, 0.02) (standard deviation 0.02) for weights.
"""
from __future__ import annotations

import numpy as np

F16, BF16 = 0, 1


def fp32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return uint16 bits."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x32, dtype=np.float32))
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    r = np.where(nan, np.uint64(0x7FC0), r)
    return r.astype(np.uint16)


def to_bits(x64: np.ndarray, dtype: int) -> np.ndarray:
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == F16:
        return x32.astype(np.float16).view(np.uint16)
    return fp32_to_bf16_bits(x32)


def uniform(shape, seed: int, dtype: int, lo=-1.0, hi=1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return to_bits(rng.uniform(lo, hi, size=shape), dtype)


def normal(shape, seed: int, dtype: int, std=1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return to_bits(rng.standard_normal(size=shape) * std, dtype)


def integers(shape, seed: int, dtype: int, lo: int, hi: int) -> np.ndarray:
    """Small integers in [lo, hi] (exact in both 16-bit types)."""
    rng = np.random.default_rng(seed)
    return to_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float64), dtype)


def bits_to_float32(bits: np.ndarray, dtype: int) -> np.ndarray:
    """View 16-bit bit patterns as fp32 values (for convenience in reports)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def sample_rows(M: int, n: int, seed: int) -> np.ndarray:
    """A sorted seeded sample of n distinct row indices of an M-row output,
    always including the first and last rows (ragged tiles live there)."""
    rng = np.random.default_rng(seed)
    n = min(n, M)
    pick = set(rng.choice(M, size=n, replace=False).tolist())
    pick.update({0, M - 1})
    return np.array(sorted(pick), dtype=np.int64)


# ---------------------------------------------------------------- 8-bit inputs
E4M3, E5M2 = 0, 1
F8_MAX = {E4M3: 448.0, E5M2: 57344.0}   # largest finite values of the two formats


def _to_f8_codes(x32: np.ndarray, fmt: int) -> np.ndarray:
    """fp32 values -> 8-bit codes through torch's float8 conversion (RNE, values
    already inside the format's range)."""
    import torch
    tdt = torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(tdt)
    return t.view(torch.uint8).numpy().copy()


def f8_integers(shape, seed: int, fmt: int, lo: int, hi: int) -> np.ndarray:
    """Small integers in [lo, hi] as 8-bit codes (exact in both formats for |v| <= 8)."""
    rng = np.random.default_rng(seed)
    return _to_f8_codes(rng.integers(lo, hi + 1, size=shape).astype(np.float32), fmt)


def f8_normal(shape, seed: int, fmt: int, std=1.0):
    """N(0, std) values stored per-tensor-scaled as 8-bit codes: the scale is a
    power of two that puts the largest magnitude just inside the format's range.
    Returns (codes, scale)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape) * std
    amax = float(np.max(np.abs(x))) if x.size else 1.0
    scale = 2.0 ** np.ceil(np.log2(amax / F8_MAX[fmt])) if amax > 0 else 1.0
    return _to_f8_codes((x / scale).astype(np.float32), fmt), float(scale)
