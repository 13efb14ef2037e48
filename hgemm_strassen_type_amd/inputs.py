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


def mx_scale_cols(K: int) -> int:
    """Columns of an E8M0 block-scale array for K values per row: K/32 blocks,
    rounded up to whole 16-byte groups."""
    return max(16, (K // 32 + 15) // 16 * 16)


def mx_normal(shape, seed: int, fmt: int, std=1.0):
    """N(0, std) values stored MX-style: every block of 32 values along a row gets
    the power-of-two scale that puts its largest magnitude just inside the 8-bit
    format's range, stored as E8M0 (2^(e-127)).  Returns (codes, scales) with
    scales of shape [rows][mx_scale_cols(K)] (unused tail bytes are 127)."""
    rows, K = shape
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape) * std
    blocks = x.reshape(rows, K // 32, 32)
    amax = np.max(np.abs(blocks), axis=2)
    e = np.where(amax > 0, np.ceil(np.log2(np.maximum(amax, 1e-300) / F8_MAX[fmt])), 0.0)
    e = np.clip(e, -127, 127).astype(np.int64)
    scales = np.full((rows, mx_scale_cols(K)), 127, dtype=np.uint8)
    scales[:, :K // 32] = (e + 127).astype(np.uint8)
    q = (blocks / np.ldexp(1.0, e)[:, :, None]).reshape(rows, K)
    return _to_f8_codes(q.astype(np.float32), fmt), scales


def mx_integers(shape, seed: int, fmt: int, lo: int, hi: int, e_lo=124, e_hi=130):
    """Small integer codes with random E8M0 block scales in [e_lo, e_hi] (2^-3..2^3)."""
    rows, K = shape
    codes = f8_integers(shape, seed, fmt, lo, hi)
    rng = np.random.default_rng(seed + 1)
    scales = np.full((rows, mx_scale_cols(K)), 127, dtype=np.uint8)
    scales[:, :K // 32] = rng.integers(e_lo, e_hi + 1, size=(rows, K // 32)).astype(np.uint8)
    return codes, scales


# 4-bit E2M1 codes: bit 3 the sign, bits 2-0 the magnitude index into these values
# (the OCP E2M1 encoding).  Rows are stored two codes a byte, code 2i in the low
# nibble of byte i.
F4_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def pack_f4_codes(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8) & 15
    return np.ascontiguousarray((codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8))


def mxf4_small(shape, seed: int, max_index=4, e_lo=125, e_hi=129):
    """Random E2M1 codes of magnitude index <= max_index (4: |v| <= 2) with random
    signs, packed, and random E8M0 block scales in [e_lo, e_hi] (2^-2..2^2 by
    default).  Returns (packed [rows][K/2], scales [rows][mx_scale_cols(K)])."""
    rows, K = shape
    rng = np.random.default_rng(seed)
    codes = (rng.integers(0, max_index + 1, size=shape) |
             (rng.integers(0, 2, size=shape) << 3)).astype(np.uint8)
    scales = np.full((rows, mx_scale_cols(K)), 127, dtype=np.uint8)
    scales[:, :K // 32] = rng.integers(e_lo, e_hi + 1, size=(rows, K // 32)).astype(np.uint8)
    return pack_f4_codes(codes), scales


def mxf4_normal(shape, seed: int, std=1.0):
    """N(0, std) values stored MXFP4-style: every block of 32 values along a row gets
    the power-of-two scale that puts its largest magnitude at or below 6 (the largest
    E2M1 value), stored as E8M0, and each scaled value becomes the code of the
    nearest E2M1 magnitude (the smaller one on a tie).  Returns (packed, scales)."""
    rows, K = shape
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape) * std
    blocks = x.reshape(rows, K // 32, 32)
    amax = np.max(np.abs(blocks), axis=2)
    e = np.where(amax > 0, np.ceil(np.log2(np.maximum(amax, 1e-300) / 6.0)), 0.0)
    e = np.clip(e, -127, 127).astype(np.int64)
    q = (blocks / np.ldexp(1.0, e)[:, :, None]).reshape(rows, K)
    # nearest magnitude: count the midpoints between neighbours strictly below |q|
    mids = (F4_MAGNITUDES[1:] + F4_MAGNITUDES[:-1]) / 2
    idx = np.searchsorted(mids, np.abs(q), side="left").astype(np.uint8)
    codes = idx | ((q < 0).astype(np.uint8) << 3)
    scales = np.full((rows, mx_scale_cols(K)), 127, dtype=np.uint8)
    scales[:, :K // 32] = (e + 127).astype(np.uint8)
    return pack_f4_codes(codes), scales
