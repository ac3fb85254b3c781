"""FP8 form of the Lightning Indexer's inputs (TEST INFRASTRUCTURE ONLY: the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the HIP library never does).

The page "LongCat Sparse Attention: Taming the Lightning via Streaming-aware Hierarchical Cross-Layer
Indexing" (§2.2, the Lightning Indexer) states only that the indexer supports FP8 computation; the
format and the scaling are a reading:

* elements: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; subnormals; the
  largest finite magnitude is 448; no infinities; codes 0x7f / 0xff are NaN and never produced);
* one power-of-two scale per vector -- per key over its d_I dims, per (query row, indexer head) --
  2^e with e the smallest integer such that max|x| <= 448 * 2^e (e = 0 for an all-zero vector), so
  that x / 2^e is exact and never needs saturation;
* elements rounded to the nearest E4M3 value, ties to the even code.

The indexer then computes Eq. 1 on the dequantized values 2^e * decode(code).  Those values have at
most 4 significant bits and are exact in float32, so the Eq. 1 oracle (``oracle.index_score``, fp64
accumulation) applies to them unchanged.
"""
import numpy as np

E4M3_MAX = 448.0
_EMIN = -6          # exponent of the smallest normal (2^-6)
_MBITS = 3


def e4m3_decode(codes):
    """Exact value (float64) of E4M3 codes (uint8); NaN codes decode to NaN."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, _EMIN), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return s * mag


def e4m3_encode(y):
    """Nearest E4M3 code to each finite y with |y| <= 448 (ties to the even code)."""
    y = np.asarray(y, np.float64)
    if not np.all(np.isfinite(y)) or np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("e4m3_encode: inputs must be finite with |y| <= 448")
    a = np.abs(y)
    # quantum of the E4M3 grid at |y|: 2^(E - 3) for a normal |y| in [2^E, 2^(E+1)), 2^-9 below 2^-6
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1): E = ex - 1
    E = np.maximum(ex - 1, _EMIN)
    quantum = np.ldexp(1.0, E - _MBITS)
    n = np.rint(a / quantum)                  # exact division by a power of two; rint = ties to even
    # n in [0, 16]; n == 16 carries into the next binade (representable, since |y| <= 448)
    E = np.where(n >= 16, E + 1, E)
    n = np.where(n >= 16, n / 2, n)
    normal = n >= 8
    efield = np.where(normal, E + 7, 0).astype(np.int64)
    mfield = np.where(normal, n - 8, n).astype(np.int64)
    code = (efield << 3) | mfield
    code = np.where(np.signbit(y) & (code != 0), code | 0x80, code)
    return code.astype(np.uint8)


def vector_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e (0 where amax == 0)."""
    amax = np.asarray(amax, np.float64)
    f, ex = np.frexp(amax)                    # amax = f * 2^ex; 448 = 0.875 * 2^9
    e = ex - 9 + (f > 0.875)
    return np.where(amax == 0, 0, e).astype(np.int64)


def quantize(x):
    """x [..., d] (float64 values of bf16 / fp32 inputs) -> (codes uint8 [..., d], scale float32 [...]).

    One power-of-two scale per vector (the last axis)."""
    x = np.asarray(x, np.float64)
    e = vector_exponent(np.max(np.abs(x), axis=-1))
    codes = e4m3_encode(np.ldexp(x, -e[..., None]))
    return codes, np.ldexp(np.ones_like(e, dtype=np.float64), e).astype(np.float32)


def dequantize(codes, scale):
    """float32 [..., d] = scale * decode(codes) (exact)."""
    return (e4m3_decode(codes) * np.asarray(scale, np.float64)[..., None]).astype(np.float32)
