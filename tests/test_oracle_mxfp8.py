"""Pins for the MXFP8 codec oracle (O4): hand-worked blocks, the closed-form
scale rule, and element encoding against torch's float8_e4m3fn cast over every
finite bf16 input."""
import os

import numpy as np
import pytest
import torch

from oracle import mxfp8 as M
from oracle.layer import bf16_bits_to_f64


def _golden(path):
    blocks = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, kind, *rest = line.split()
        b = blocks.setdefault(name, {"in": {}, "out": {}})
        if kind == "scale":
            b["scale"] = int(rest[0])
        else:
            for item in rest:
                i, v = item.split(":")
                b[kind][int(i)] = int(v, 16) if kind == "out" else float(v)
    return blocks


def test_hand_worked_blocks(golden_dir):
    for name, b in _golden(os.path.join(golden_dir, "mxfp8_hand_worked.txt")).items():
        v = np.zeros(32)
        for i, x in b["in"].items():
            v[i] = x
        el, sc = M.quantize(v[None])
        assert int(sc[0, 0]) == b["scale"], name
        exp = np.zeros(32, np.uint8)
        for i, x in b["out"].items():
            exp[i] = x
        assert el[0].tolist() == exp.tolist(), name


def _finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        v = bf16_bits_to_f64(bits)
    return v[np.isfinite(v)]


def test_scale_closed_form():
    # e is the largest integer with 2^(e+8) <= amax, clamped to [-127, 127]
    v = np.abs(_finite_bf16())
    v = v[v > 0]
    e = M.scale_exponent(v)
    for n in range(-150, 130):
        lo = 2.0 ** (n + 8)
        sel = (v >= lo) & (v < 2 * lo)
        assert np.all(e[sel] == np.clip(n, -127, 127))
    assert M.scale_exponent(np.array([0.0]))[0] == 0


@pytest.mark.parametrize("e", [-127, -20, -3, 0, 1, 7, 119])
def test_elements_match_library_cast_exhaustive(e):
    v = _finite_bf16()
    u = v * 2.0 ** -e
    mine = M.e4m3fn_encode(u)
    ref = torch.from_numpy(np.clip(u, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_decode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    v = M.e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(v, ref)
    assert np.array_equal(M.e4m3fn_encode(v), codes)


def test_quantize_bounds_and_error():
    rng = np.random.default_rng(0)
    v = bf16_bits_to_f64(((rng.standard_normal((64, 256)).astype(np.float32).view(np.uint32)
                           + 0x8000) >> 16).astype(np.uint16))
    el, sc = M.quantize(v)
    dq = M.dequantize(el, sc)
    scale = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    u = np.abs(v) / scale
    # before rounding the block maximum lies in [256, 512)
    umax = u.reshape(64, 8, 32).max(-1)
    assert np.all((umax >= 256) & (umax < 512))
    # below 448: nearest-even error <= half an ulp (2^-4 relative, 2^-10 absolute
    # in the subnormal range); at or above 448: saturation to 448
    err = np.abs(dq - v) / scale
    inside = u < 448
    assert np.all(err[inside] <= np.maximum(2.0 ** -4 * u[inside], 2.0 ** -10))
    assert np.all(np.abs(dq[~inside]) / scale[~inside] == 448)
    assert np.array_equal(M.fake_quant(v.T, 0), dq.T)


def test_torch_e8m0_agrees_on_powers_of_two():
    if not hasattr(torch, "float8_e8m0fnu"):
        pytest.skip("torch lacks float8_e8m0fnu")
    # a power of two 2^n is encoded by E8M0 as byte n + 127 under any rounding mode
    e = np.arange(-127, 128)
    t = torch.from_numpy(np.ldexp(1.0, e).astype(np.float32)).to(torch.float8_e8m0fnu)
    assert np.array_equal(t.view(torch.uint8).numpy(), (e + 127).astype(np.uint8))
