"""Pins of the FP8 (E4M3, one power-of-two scale per vector) quantizer of the oracle (CPU)."""
import math

import numpy as np
import pytest
import torch

from oracle import fp8

# (code, value) pairs fixed by the E4M3 definition: bias 7, 3 mantissa bits, subnormals 2^-6 * m/8
DECODE_TABLE = [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x0F, 1.875 * 2.0 ** -6),
    (0x30, 0.5), (0x38, 1.0), (0x39, 1.125), (0x3A, 1.25), (0x40, 2.0), (0x58, 16.0), (0x77, 240.0),
    (0x78, 256.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
]


def test_e4m3_decode_table():
    for code, value in DECODE_TABLE:
        assert fp8.e4m3_decode(np.uint8(code)) == value, hex(code)
    assert np.isnan(fp8.e4m3_decode(np.uint8(0x7F))) and np.isnan(fp8.e4m3_decode(np.uint8(0xFF)))


def test_e4m3_encode_exhaustive_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)
    assert fp8.e4m3_encode(np.array([-0.0]))[0] == 0  # -0 folds onto +0


@pytest.mark.parametrize("value,code", [
    (1.0625, 0x38),            # halfway 1 .. 1.125: even mantissa 0
    (1.1875, 0x3A),            # halfway 1.125 .. 1.25: even mantissa 2
    (17.0, 0x58),              # halfway 16 .. 18: 16
    (2.0 ** -10, 0x00),        # halfway 0 .. 2^-9: 0
    (3 * 2.0 ** -10, 0x02),    # halfway 2^-9 .. 2^-8: even 2 * 2^-9
    (0.99 * 2.0 ** -6, 0x08),  # rounds up into the smallest normal
    (1.97, 0x40),              # mantissa carry into the next binade
    (440.0, 0x7E), (-300.0, 0xF9), (100.0, 0x6C), (-0.3, 0xAA),
])
def test_e4m3_encode_cases(value, code):
    assert fp8.e4m3_encode(np.array([value]))[0] == code


def test_e4m3_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-0.02, 0.02, 3000),
                        np.ldexp(rng.uniform(-1, 1, 2000), rng.integers(-12, 9, 2000))])
    grid_codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], np.uint8)
    grid = fp8.e4m3_decode(grid_codes)
    got = fp8.e4m3_encode(y)
    d = np.abs(grid[None, :] - y[:, None])
    best = d.min(axis=1)
    assert np.array_equal(np.abs(fp8.e4m3_decode(got) - y), best)
    # among equally near codes the chosen one has an even mantissa (ties to even)
    ties = (d == best[:, None]).sum(axis=1) > 1
    assert np.all((got[ties] & 1) == 0)


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(2)
    y = np.concatenate([rng.uniform(-448, 448, 5000), rng.normal(0, 0.05, 5000)]).astype(np.float32)
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(fp8.e4m3_decode(fp8.e4m3_encode(y.astype(np.float64))), want)


def test_vector_exponent_closed_form():
    rng = np.random.default_rng(3)
    amax = np.ldexp(rng.uniform(0.5, 1.0, 4000), rng.integers(-30, 20, 4000))
    amax = np.concatenate([amax, [448.0, 449.0, 224.0, 224.00001, 1.0]])
    e = fp8.vector_exponent(amax)
    assert np.all(amax <= 448.0 * np.ldexp(1.0, e))
    assert np.all(amax > 448.0 * np.ldexp(1.0, e - 1))
    assert list(fp8.vector_exponent(np.array([448.0, 449.0, 224.0, 0.0]))) == [0, 1, -1, 0]


def test_quantize_bounds_and_scale():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 1 / math.sqrt(128), (300, 128))
    x[7] = 0.0
    codes, scale = fp8.quantize(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    deq = fp8.dequantize(codes, scale).astype(np.float64)
    s = scale.astype(np.float64)[:, None]
    # every element within half a quantum of the E4M3 grid at its magnitude (in units of the scale)
    a = np.abs(x) / s
    _, ex = np.frexp(a)
    quantum = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    assert np.all(np.abs(deq - x) <= quantum * s / 2)
    # the largest element of each vector is in (224, 448] before rounding, so in [224, 448] after it
    top = np.max(np.abs(fp8.e4m3_decode(codes)), axis=1)
    assert np.all(top[np.arange(300) != 7] >= 224) and np.all(top <= 448)
    assert scale[7] == 1.0 and not codes[7].any()
    # scales are powers of two, so dequantization is exact in float32
    assert np.all(np.frexp(scale)[0] == 0.5)
    assert np.array_equal(deq, fp8.e4m3_decode(codes) * s)
