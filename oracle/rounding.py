"""Rounding of exact (fp64) values to the buffer dtype: fp32 and bf16.

TEST INFRASTRUCTURE ONLY: part of the CPU oracle. Only the tests, the smoke
check and the CPU-baseline leg of the benchmark may import this module.

The ring all-reduce moves every partial sum across a link in the buffer's own
dtype, so each hop ends with one rounding to that dtype (the per-hop rounding
of the reduce-scatter phase, page "DDP 与 Ring-AllReduce" (xuesongtap.github.io),
§1.3.2.1). The pages fix neither the rounding mode nor the handling of
subnormals; the reading taken here is IEEE round-to-nearest, ties to even, with
subnormals kept.

Representation: fp32 buffers are numpy float32 arrays; bf16 buffers are numpy
uint16 arrays holding the bf16 bit patterns (the upper half of an fp32 word).

Why one fp64 add followed by one rounding is the correctly rounded sum of two
values of the buffer dtype: the fp64 sum is either exact or itself a correct
rounding to 53 bits, and rounding twice (first to p' = 53 bits, then to p
bits) gives the same result as rounding once whenever p' >= 2p + 2
(S. A. Figueroa, "When is double rounding innocuous?", SIGNUM Newsletter
30(3), 1995). fp32 has p = 24 (2p+2 = 50) and bf16 has p = 8 (2p+2 = 18).
The same argument covers the product of two fp32 values, which fp64 holds
exactly.
"""

import numpy as np

FP32 = "fp32"
BF16 = "bf16"
DTYPES = (FP32, BF16)

BF16_MAX_EXP = 127      # largest unbiased exponent of a finite bf16
BF16_MIN_EXP = -126     # exponent of the smallest normal bf16
BF16_FRAC_BITS = 7      # stored fraction bits of bf16 (8 significant bits)
BF16_QNAN = 0x7FC0


def storage_dtype(dtype):
    """numpy storage type of a buffer of the given dtype."""
    if dtype == FP32:
        return np.float32
    if dtype == BF16:
        return np.uint16
    raise ValueError(f"unknown dtype {dtype!r}")


def bf16_bits_to_f64(bits):
    """Exact value of bf16 bit patterns, as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f64(x, dtype):
    """Exact value of a buffer of the given dtype, as float64."""
    if dtype == FP32:
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f64(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to_fp32(x64):
    """Round float64 values to the nearest fp32, ties to even.

    numpy's float64 -> float32 conversion is the C conversion under the default
    IEEE rounding mode (nearest, ties to even); it keeps subnormals and turns
    values at or beyond 2^128 - 2^103 into infinities.
    """
    with np.errstate(over="ignore", invalid="ignore"):
        return np.asarray(x64, dtype=np.float64).astype(np.float32)


def round_to_bf16(x64):
    """Round float64 values to the nearest bf16, ties to even; returns uint16 bits.

    Written from the definition of rounding to a binary format with 8
    significant bits and the exponent range of fp32:
      * the spacing of bf16 values around |x| is 2^(max(E, -126) - 7), where
        E = floor(log2 |x|) (the max() gives the fixed subnormal spacing);
      * |x| / spacing is rounded to an integer, halfway cases to the even
        integer (numpy.rint), which is the even last significand bit;
      * a result of 2^128 or more is an overflow and becomes infinity;
      * the sign is kept, including the sign of zero;
      * NaN becomes the quiet NaN 0x7FC0 with the input's sign.
    """
    x = np.asarray(x64, dtype=np.float64)
    ax = np.abs(x)
    nan = np.isnan(x)
    finite = np.isfinite(x)
    safe = np.where(finite, ax, 0.0)
    _, e = np.frexp(safe)                      # safe = m * 2^e, m in [0.5, 1)
    exp = np.maximum(e - 1, BF16_MIN_EXP)      # floor(log2 |x|), clamped
    spacing = np.ldexp(1.0, exp - BF16_FRAC_BITS)
    q = np.rint(safe / spacing)                # exact division by a power of two
    r = q * spacing                            # exact
    r = np.where(r >= 2.0 ** (BF16_MAX_EXP + 1), np.inf, r)
    r = np.where(finite, r, np.inf)            # +-inf stays infinite
    r = np.copysign(r, x)
    with np.errstate(invalid="ignore"):
        bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    sign = (np.signbit(x).astype(np.uint16) << np.uint16(15))
    bits = np.where(nan, np.uint16(BF16_QNAN) | sign, bits).astype(np.uint16)
    return bits


def round_to(x64, dtype):
    """Round float64 values to the buffer dtype (see the two functions above)."""
    if dtype == FP32:
        return round_to_fp32(x64)
    if dtype == BF16:
        return round_to_bf16(x64)
    raise ValueError(f"unknown dtype {dtype!r}")


def f32_to_bf16(x32):
    """Round fp32 values (e.g. freshly drawn inputs) to bf16 bits, RNE."""
    with np.errstate(invalid="ignore"):
        return round_to_bf16(np.asarray(x32, dtype=np.float32).astype(np.float64))


def unit_roundoff(dtype):
    """u = 2^-p for the dtype's p significant bits (fp32: 24, bf16: 8)."""
    if dtype == FP32:
        return 2.0 ** -24
    if dtype == BF16:
        return 2.0 ** -8
    raise ValueError(f"unknown dtype {dtype!r}")
