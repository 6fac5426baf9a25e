"""O4 — the MXFP8 codec, step by step (test infrastructure only).

The pages fix that MXFP8 is a low-precision weight format whose weights are
quantized before the kernel runs ("Mixture-of-Kittens (MoK)" project summary,
Key-concepts table; "Cursor Open-Sources Mixture-of-Kittens (MoK)" digest,
English abstract: BF16 and MXFP8 precision modes). The block format itself is
the OCP Microscaling (MX) v1.0 definition of MXFP8: 32 consecutive values
along the contraction axis share one E8M0 scale; elements are E4M3.

Steps for one block v[0..31] (values are bf16, exact in fp64):
  amax = max |v|
  e    = floor(log2 amax) - 8   (8 = exponent of E4M3's largest normal, 448),
         clamped to [-127, 127]; e = 0 when amax == 0 (reading: the pages and
         the rule leave the zero block open)
  scale byte = e + 127
  element    = E4M3FN(v * 2^-e): round to nearest even, saturate to +-448,
               sign kept (so -0 encodes as 0x80)
E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
0x7F / 0xFF are NaN; largest normal 448; subnormals m * 2^-9.
NaN and infinite inputs are outside the format's use here.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """floor(log2 amax) - 8 clamped to [-127, 127]; 0 for amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)            # amax = m * 2^ex, m in [0.5, 1)
    e = (ex.astype(np.int64) - 1) - E4M3_EMAX
    e = np.clip(e, -127, 127)
    return np.where(amax == 0, 0, e)


def e4m3fn_encode(u: np.ndarray) -> np.ndarray:
    """Encode fp64 values as E4M3FN bytes, nearest-even, saturating."""
    u = np.asarray(u, dtype=np.float64)
    sign = np.signbit(u).astype(np.uint8)
    a = np.minimum(np.abs(u), E4M3_MAX)
    _, ex = np.frexp(a)
    E = np.maximum(ex.astype(np.int64) - 1, -6)        # binade; subnormals share 2^-6's quantum
    quantum = np.ldexp(1.0, E - 3)
    r = np.round(a / quantum) * quantum                # numpy rounds halves to even
    r = np.minimum(r, E4M3_MAX)
    code = np.zeros(u.shape, dtype=np.int64)
    sub = (r > 0) & (r < 2.0 ** -6)
    code[sub] = np.round(r[sub] / 2.0 ** -9).astype(np.int64)
    nrm = r >= 2.0 ** -6
    _, ex2 = np.frexp(r[nrm])
    E2 = ex2.astype(np.int64) - 1
    mant = np.round((r[nrm] / np.ldexp(1.0, E2) - 1.0) * 8).astype(np.int64)
    code[nrm] = ((E2 + 7) << 3) | mant
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def e4m3fn_decode(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    ef = (b >> 3) & 0xF
    m = b & 7
    val = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))
    val = np.where((ef == 15) & (m == 7), np.nan, val)
    return s * val


def quantize(v: np.ndarray):
    """Quantize along the last axis (length a multiple of 32).
    Returns (elements uint8 [..., K], scales uint8 [..., K/32])."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % BLOCK == 0
    blk = v.reshape(v.shape[:-1] + (K // BLOCK, BLOCK))
    e = scale_exponent(np.max(np.abs(blk), axis=-1))
    elems = e4m3fn_encode(blk * np.ldexp(1.0, -e)[..., None])
    return elems.reshape(v.shape), (e + 127).astype(np.uint8)


def dequantize(elems: np.ndarray, scales: np.ndarray) -> np.ndarray:
    K = elems.shape[-1]
    val = e4m3fn_decode(elems).reshape(elems.shape[:-1] + (K // BLOCK, BLOCK))
    val = val * np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]
    return val.reshape(elems.shape)


def fake_quant(v: np.ndarray, axis: int) -> np.ndarray:
    """dequantize(quantize(v)) with blocks along ``axis``."""
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    return np.moveaxis(dequantize(*quantize(v)), -1, axis)
