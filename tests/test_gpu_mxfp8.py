"""mok_mxfp8_quantize on the GPU equals the oracle's codec bit for bit."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_table_amd as mok
import synth
from oracle import mxfp8 as M
from oracle.layer import bf16_bits_to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def _check(bits_bkr, transposed):
    """bits_bkr: uint16 [B, rows, K] logical source (quantized along K)."""
    src = np.ascontiguousarray(bits_bkr.transpose(0, 2, 1)) if transposed else bits_bkr
    el, sc = mok.mxfp8_quantize(_dev(src), transposed)
    torch.cuda.synchronize()
    ref_el, ref_sc = M.quantize(bf16_bits_to_f64(bits_bkr))
    assert np.array_equal(sc.cpu().numpy(), ref_sc)
    assert np.array_equal(el.cpu().numpy(), ref_el)


def test_every_finite_bf16_pattern_at_many_scales():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = bits[(bits & 0x7F80) != 0x7F80]                      # drop Inf / NaN
    rng = np.random.default_rng(0)
    rows = []
    # each block: the tested pattern among values that fix the block maximum
    for amax_bits in (0x0000, 0x0001, 0x0080, 0x3F80, 0x4380, 0x43E0, 0x7F7F, 0x2000, 0x5000):
        vals = rng.permutation(fin)
        blocks = np.zeros((vals.size // 31 + 1) * 32, np.uint16)
        blocks[:] = amax_bits
        v = np.full(((vals.size + 30) // 31) * 31, 0, np.uint16)
        v[:vals.size] = vals
        blk = blocks.reshape(-1, 32)[: v.size // 31]
        blk[:, 1:] = v.reshape(-1, 31)
        rows.append(blk)
    data = np.concatenate(rows).reshape(1, -1, 32)
    _check(data, False)


@pytest.mark.parametrize("transposed", [False, True])
def test_weight_shapes(transposed):
    cfg = synth.CONFIGS["tiny"]
    w = synth.expert_weights(cfg, "gate")          # [E, H, I]
    if transposed:
        _check(np.ascontiguousarray(w.transpose(0, 2, 1)), True)   # quantize W^T along H
    else:
        _check(w, False)                                            # along I


def test_special_blocks():
    vals = np.zeros((4, 32), np.float32)
    vals[0, :3] = [448, -1, 2 ** -9]
    vals[1, :3] = [1000, 464, -2]
    vals[3, 7] = 2.0 ** -130
    bits = synth.f32_to_bf16_bits(vals).reshape(1, 4, 32)
    bits[0, 2, 5] = 0x8000                                          # -0 in a zero block
    _check(bits, False)


def test_every_finite_bf16_pattern_at_every_scale_exponent():
    """Each block holds one element 2^(e+8) that fixes the scale exponent e
    (-127 .. 119, every exponent a block can have) and patterns no larger in
    magnitude: every finite bf16 pattern meets every scale it can meet."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = bits[(bits & 0x7F80) != 0x7F80]
    blocks = []
    for e in range(-127, 120):
        top = np.uint16(max(0, min(254, e + 135)) << 7)          # 2^(e+8) as bf16 (e = -127: the smallest normal binade)
        vals = fin[(fin & 0x7FFF) <= top]
        n = -(-vals.size // 31)
        blk = np.zeros((n, 32), np.uint16)
        blk[:, 0] = top
        v = np.zeros(n * 31, np.uint16)
        v[:vals.size] = vals
        blk[:, 1:] = v.reshape(n, 31)
        blocks.append(blk)
    data = np.concatenate(blocks).reshape(1, -1, 32)
    _check(data, False)
