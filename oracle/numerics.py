"""Number formats used by the oracle (test infrastructure).

bf16: a bfloat16 value is the float32 whose upper 16 bits are the stored bits
and whose lower 16 bits are zero, so widening is exact.

MXFP4 (the OCP microscaling format: blocks of 32 FP4 E2M1 elements sharing one
E8M0 power-of-two scale, about 4.25 bits per weight): the expert weights of
the gpt-oss models ("MoE: what it costs to train and serve", "Memory: sparsity
only helps once it fits").  Decoding is exact in float64.

fp8 e4m3fn (the OCP 8-bit float with 4 exponent bits, bias 7, 3 mantissa bits,
no infinities, a single NaN mantissa pattern per sign, largest finite 448): the
pages quantise activations to FP8 before dispatch ("MoE: what it costs to train
and serve", worked example "how many bytes does one token send?", where FP8
halves the payload).  The encoder rounds to nearest with ties to even.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen a stored tensor ("f32" values or "bf16" bits) to float64."""
    if dtype == "bf16":
        return bf16_to_f64(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of e4m3fn codes (uint8) as float64; the NaN codes 0x7F/0xFF give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    sub = man / 8.0 * 2.0 ** -6                       # exponent field 0: subnormal
    nor = (1.0 + man / 8.0) * np.exp2(ex - 7.0)
    v = np.where(ex == 0, sub, nor)
    v = np.where((ex == 15) & (man == 7), np.nan, v)
    return sign * v


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round float32 values with |v| < 464 to e4m3fn codes, nearest, ties to even.

    Values in [448, 464) round to 448 (464 is the midpoint to 480, which the
    format does not have); the per-token scaling can land a hair above 448.

    The quantum in the binade [2^e, 2^(e+1)) is 2^(e-3); below 2^-6 the format
    is subnormal with quantum 2^-9.  |v| / quantum is exact in float64, so
    ``np.rint`` (ties to even) gives the rounded significand; a carry into the
    next binade is handled by re-deriving the code from the rounded value.
    A negative zero keeps its sign (code 0x80)."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) >= 464.0):
        raise ValueError("e4m3_encode: input outside the finite e4m3fn range")
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # guard against log2 rounding at exact powers of two
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    e = np.maximum(e, -6.0)
    q = np.exp2(e - 3.0)
    r = np.rint(a / q) * q                              # rounded magnitude
    # encode the rounded magnitude
    with np.errstate(divide="ignore"):
        er = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    er = np.where(np.exp2(er) > r, er - 1, er)
    er = np.where(np.exp2(er + 1) <= r, er + 1, er)
    normal = r >= 2.0 ** -6
    ex_field = np.where(normal, er + 7.0, 0.0)
    man = np.where(normal, r / np.exp2(er) * 8.0 - 8.0, r / 2.0 ** -9)
    code = (ex_field.astype(np.int64) << 3) | np.rint(man).astype(np.int64)
    code = np.where(r == 0, 0, code)
    sign = np.signbit(v)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def f32(a) -> np.ndarray:
    """Round to float32 (IEEE, nearest even)."""
    return np.asarray(a, dtype=np.float32)


# ------------------------------------------------------------------- MXFP4 --

MX_BLOCK = 32


def fp4_e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Value of FP4 E2M1 codes (0..15) as float64: bit 3 the sign, bits 2-1 the
    exponent (bias 1), bit 0 the mantissa; exponent field 0 is subnormal
    (0 or 0.5).  The magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6; code 8 is -0."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    ex = (c >> 1) & 0x3
    man = (c & 0x1).astype(np.float64)
    mag = np.where(ex == 0, 0.5 * man, (1.0 + 0.5 * man) * np.exp2(ex - 1.0))
    return sign * mag


def e8m0_decode(e: np.ndarray) -> np.ndarray:
    """Value of E8M0 scales (unsigned 8-bit exponents, bias 127, no mantissa):
    2^(e - 127); 255 is NaN."""
    e = np.asarray(e).astype(np.int64)
    return np.where(e == 255, np.nan, np.exp2(e - 127.0))


def mxfp4_split(buf: np.ndarray, rows: int, K: int) -> tuple:
    """The two planes of an MXFP4 matrix [rows][K] stored as the library takes
    it: rows * K / 2 bytes of codes (row-major; element 2i in the low nibble of
    byte i, element 2i + 1 in the high nibble), then rows * K / 32 E8M0 scales
    (row-major; scale b of a row covers its elements 32b .. 32b + 31)."""
    buf = np.asarray(buf, np.uint8).ravel()
    nc, ns = rows * K // 2, rows * K // MX_BLOCK
    if buf.size != nc + ns:
        raise ValueError(f"mxfp4 buffer of {buf.size} bytes for a [{rows}][{K}] matrix")
    return buf[:nc].reshape(rows, K // 2), buf[nc:].reshape(rows, K // MX_BLOCK)


def mxfp4_decode(buf: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Exact float64 values of an MXFP4 matrix [rows][K]: code value times its
    block's scale (each code byte looked up as its two values)."""
    codes, scales = mxfp4_split(buf, rows, K)
    pairs = np.stack([fp4_e2m1_decode(np.arange(256) & 0xF), fp4_e2m1_decode(np.arange(256) >> 4)], axis=1)
    vals = pairs[codes].reshape(rows, K // MX_BLOCK, MX_BLOCK)
    return (vals * e8m0_decode(scales)[:, :, None]).reshape(rows, K)


def as_weights(a: np.ndarray, wfmt: str, dtype: str, rows: int, K: int) -> np.ndarray:
    """One stored weight matrix [rows][K] widened to float64: MXFP4 buffers
    decoded, else the layer's storage type widened."""
    if wfmt == "mxfp4":
        return mxfp4_decode(a, rows, K)
    return as_f64(a, dtype)
