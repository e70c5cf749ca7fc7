"""The oracle's rounding against hand-derived halfway cases and against
library conversions (torch's float32 -> bfloat16 and numpy's float32 add,
both IEEE round-to-nearest-even)."""

import os

import numpy as np
import pytest
import torch

from oracle import ring, rounding


def parse_cases(path):
    out = []
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            dtype, rest = line.split(None, 1)
            expr, bits = rest.rsplit(None, 1)
            out.append((dtype, float(eval(expr, {"__builtins__": {}})), int(bits, 16)))
    return out


def test_hand_derived_cases(golden_dir):
    cases = parse_cases(os.path.join(golden_dir, "rounding_cases.txt"))
    assert len(cases) == 21
    for dtype, value, bits in cases:
        got = rounding.round_to(np.array([value]), dtype)
        got_bits = int(got.view(np.uint32)[0]) if dtype == "fp32" else int(got[0])
        assert got_bits == bits, (dtype, value, hex(got_bits), hex(bits))


def spread_f32(n, seed):
    """float32 values with random bit patterns (all exponents, subnormals,
    infinities and NaNs included)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)


def test_bf16_matches_torch_conversion():
    x = spread_f32(1_000_000, 1)
    x = np.concatenate([x, np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45,
                                     3.3895314e38, 3.3961776e38], np.float32)])
    ours = rounding.f32_to_bf16(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], theirs[~nan])
    # NaN stays NaN: exponent all ones, non-zero fraction
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)


def test_fp32_hop_matches_ieee_single_add():
    """hop_add in fp32 (fp64 add + one rounding) equals the hardware float32
    add for pairs spread over the whole exponent range."""
    a = spread_f32(500_000, 2)
    b = spread_f32(500_000, 3)
    # also pairs of close exponents, where cancellation and carries happen
    rng = np.random.default_rng(4)
    c = rng.normal(0, 1, 200_000).astype(np.float32)
    d = (c * rng.uniform(-2, 2, 200_000)).astype(np.float32)
    a, b = np.concatenate([a, c]), np.concatenate([b, d])
    with np.errstate(all="ignore"):
        ieee = a + b
        ours = ring.hop_add(a, b, "fp32")
    fin = np.isfinite(ieee) | np.isinf(ieee)
    nan = np.isnan(ieee)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[fin & ~nan].view(np.uint32), ieee[fin & ~nan].view(np.uint32))


def test_bf16_hop_matches_torch_bf16_add():
    """hop_add in bf16 equals torch's CPU bfloat16 add (float32 add, then
    round to nearest even) on random bf16 pairs."""
    rng = np.random.default_rng(5)
    x = (rng.normal(0, 1, 400_000) * np.exp2(rng.integers(-30, 30, 400_000))).astype(np.float32)
    y = (rng.normal(0, 1, 400_000) * np.exp2(rng.integers(-30, 30, 400_000))).astype(np.float32)
    xb, yb = rounding.f32_to_bf16(x), rounding.f32_to_bf16(y)
    ours = ring.hop_add(xb, yb, "bf16")
    tx = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16)
    ty = torch.from_numpy(yb.view(np.int16)).view(torch.bfloat16)
    theirs = (tx + ty).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_signed_zero(dtype):
    """(+0) + (-0) = +0 and (-0) + (-0) = -0 under round-to-nearest."""
    pz = rounding.round_to(np.array([0.0]), dtype)
    nz = rounding.round_to(np.array([-0.0]), dtype)
    assert np.signbit(rounding.to_f64(ring.hop_add(pz, nz, dtype), dtype))[0] == False  # noqa: E712
    assert np.signbit(rounding.to_f64(ring.hop_add(nz, nz, dtype), dtype))[0] == True  # noqa: E712
