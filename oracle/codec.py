"""Storage codecs of the oracle (test infrastructure only).

The oracle is a plain, slow CPU model of the CSA/HCA hot path.  Only the test
suite, the smoke check and the CPU-baseline leg of the benchmark use it; the
product path never imports anything under ``oracle/``.

Formats, as the pages name them:
* KV rows: RoPE dims kept in BF16, all other dims in FP8 (llm-tech overview,
  "other architecture details"; kenelite analysis section 8.2).
* Indexer: FP4 (MXFP4, E2M1 elements with a shared power-of-two scale per 32
  values; llm-tech overview, infrastructure section on FP4 QAT; kenelite
  analysis section 8.3), or FP8 for the Flash/Pro-like workloads.

Definitions used (public format specs, restated):
* FP8 E4M3FN (OCP 8-bit floating point spec): 1 sign, 4 exponent (bias 7),
  3 mantissa bits, no infinities, S.1111.111 is NaN, max finite 448.
* BF16: the top 16 bits of an IEEE binary32.
* E2M1 (OCP MX v1.0): 1 sign, 2 exponent (bias 1), 1 mantissa bit; values
  0, 0.5, 1, 1.5, 2, 3, 4, 6.  E8M0: a biased power of two, 2^(code-127).
Encoders round to nearest, ties to even, and saturate to the largest finite
magnitude.  Sign is kept on values that round to zero.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


# ----------------------------------------------------------------- FP8 E4M3FN
def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    mt = (c & 7).astype(np.float64)
    val = np.where(e == 0, mt * 2.0 ** -9, (8.0 + mt) * np.ldexp(1.0, (e - 10).astype(np.int64)))
    val = np.where((e == 15) & (mt == 7), np.nan, val)
    return np.where(s == 1, -val, val)


def e4m3_encode(x) -> np.ndarray:
    """Round-to-nearest-even E4M3FN codes of float64 values, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    fl = np.maximum(ex - 1, -6)              # binade of a; below 2^-6 the spacing is 2^-9
    quantum = np.ldexp(1.0, fl - 3)
    q = np.minimum(np.rint(a / quantum) * quantum, E4M3_MAX)
    _, ex2 = np.frexp(q)
    fl2 = ex2 - 1
    is_norm = q >= 2.0 ** -6
    e_field = np.where(is_norm, fl2 + 7, 0)
    mant = np.where(is_norm, q / np.ldexp(1.0, fl2) * 8.0 - 8.0, q / 2.0 ** -9)
    code = (e_field.astype(np.int64) << 3) | mant.astype(np.int64)
    code = code | (neg.astype(np.int64) << 7)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


# ----------------------------------------------------------------------- BF16
def bf16_encode(x) -> np.ndarray:
    """BF16 bit patterns of values rounded first to binary32 (the kernels' working
    precision), then to BF16 with round-to-nearest-even."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    r = np.where(np.isnan(f), 0x7FC0, r)
    return r.astype(np.uint16)


def bf16_decode(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------- E2M1
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    v = E2M1_VALUES[c & 7]
    return np.where((c >> 3) & 1, -v, v)


def e2m1_encode(x) -> np.ndarray:
    """Round-to-nearest-even E2M1 codes (4 bits), saturating at 6."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    quantum = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = np.minimum(np.rint(a / quantum) * quantum, E2M1_MAX)
    # q is one of E2M1_VALUES: map value -> magnitude code
    code = np.searchsorted(E2M1_VALUES, q)
    return (code | (neg.astype(np.int64) << 3)).astype(np.uint8)


# ------------------------------------------------------- per-row FP8 scaling
def fp8_row_scale(amax) -> np.ndarray:
    """Per-row power-of-two scale s = 2^e, e the smallest integer with
    amax <= 448 * 2^e (so every x/s lies in the E4M3 range and x/s is exact).
    e is clamped to [-126, 127]; an all-zero row gets s = 1."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    # fix any off-by-one of the floating log with exact comparisons
    e = np.where(safe > E4M3_MAX * np.ldexp(1.0, e), e + 1, e)
    e = np.where(safe <= E4M3_MAX * np.ldexp(1.0, e - 1), e - 1, e)
    e = np.clip(e, -126, 127)
    e = np.where(amax > 0, e, 0)
    return np.ldexp(1.0, e)


# ----------------------------------------------------------------- MXFP4 block
def mxfp4_block_exponent(amax) -> np.ndarray:
    """OCP MX v1.0 shared exponent: floor(log2 amax) - 2 (2 = emax of E2M1),
    clamped to the E8M0 range [-127, 127]; an all-zero block gets -127."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    _, ex = np.frexp(safe)
    e = np.clip(ex - 1 - 2, -127, 127)
    return np.where(amax > 0, e, -127).astype(np.int64)


def mxfp4_encode(x):
    """x [..., D] (D % 32 == 0) -> (codes uint8 [..., D] in 0..15, e8m0 uint8 [..., D/32])."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    D = x.shape[-1]
    xb = x.reshape(x.shape[:-1] + (D // 32, 32))
    e = mxfp4_block_exponent(np.max(np.abs(xb), axis=-1))
    codes = e2m1_encode(xb / np.ldexp(1.0, e)[..., None])
    return codes.reshape(x.shape), (e + 127).astype(np.uint8)


def mxfp4_decode(codes, e8m0) -> np.ndarray:
    codes = np.asarray(codes)
    D = codes.shape[-1]
    v = e2m1_decode(codes).reshape(codes.shape[:-1] + (D // 32, 32))
    s = np.ldexp(1.0, np.asarray(e8m0).astype(np.int64) - 127)
    return (v * s[..., None]).reshape(codes.shape)
