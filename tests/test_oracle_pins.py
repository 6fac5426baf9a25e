"""Pins for the oracle's parity measures and for its MXFP8 mode against its
BF16 mode on inputs that quantize losslessly.

* rel_frobenius and rel_rows are checked against values worked out by hand,
  including two tensors of equal norm that differ (the measure must see the
  difference, not the norms) and the all-zero reference.
* MXFP8 ("Mixture-of-Kittens (MoK)" project summary, Key-concepts table: the
  MXFP8 mode): when every operand the mode quantizes holds values n * 2^p with
  a small integer n, E4M3 elements with an E8M0 block scale represent them
  exactly, so the fake-quant is the identity at every quantization point and
  the MXFP8 layer must equal the BF16 layer.
"""
import numpy as np
import pytest

import synth
from oracle import layer as L
from oracle import mxfp8 as M


# ----------------------------------------------------------------------------- parity measures

def test_rel_frobenius_by_hand():
    ref = np.array([3.0, 4.0])                                      # ||ref|| = 5
    assert L.rel_frobenius(ref, ref) == 0.0
    assert L.rel_frobenius([3.0, 4.05], ref) == pytest.approx(0.01, rel=1e-12)    # 0.05 / 5
    assert L.rel_frobenius([4.0, 3.0], ref) == pytest.approx(np.sqrt(2) / 5, rel=1e-12)   # equal norms, differ
    assert L.rel_frobenius([-3.0, -4.0], ref) == pytest.approx(2.0, rel=1e-12)
    assert L.rel_frobenius([0.0, 0.0], ref) == pytest.approx(1.0, rel=1e-12)
    m = np.array([[1.0, 2.0], [2.0, 4.0]])                         # ||m||_F = 5
    assert L.rel_frobenius(m + np.array([[0, 0], [0, 3.0]]), m) == pytest.approx(0.6, rel=1e-12)
    assert L.rel_frobenius(np.zeros(3), np.zeros(3)) == 0.0
    assert L.rel_frobenius([0.0, 1e-3, 0.0], np.zeros(3)) == np.inf


def test_rel_frobenius_not_a_difference_of_norms():
    # a permuted tensor has the same norm as the reference and must still fail
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((64, 32))
    got = ref[::-1].copy()
    assert abs(np.linalg.norm(got) - np.linalg.norm(ref)) < 1e-9
    assert L.rel_frobenius(got, ref) > 1.0


def test_rel_rows_by_hand():
    ref = np.array([[3.0, 4.0], [0.0, 0.0], [1.0, 0.0], [0.0, 0.0]])
    got = np.array([[3.0, 4.05], [0.0, 0.0], [0.0, 1.0], [0.0, 2.0]])
    r = L.rel_rows(got, ref)
    assert r[0] == pytest.approx(0.01, rel=1e-12)
    assert r[1] == 0.0
    assert r[2] == pytest.approx(np.sqrt(2), rel=1e-12)   # same norm, wrong row
    assert r[3] == np.inf
    # trailing axes form the row: [2, 2, 2] -> two rows of 4
    t = np.arange(8.0).reshape(2, 2, 2) + 1
    u = t.copy()
    u[1, 1, 1] += 1.0
    rr = L.rel_rows(u, t)
    assert rr[0] == 0.0 and rr[1] == pytest.approx(1.0 / np.linalg.norm(t[1]), rel=1e-12)


def test_rel_rows_sees_one_wrong_row_that_the_norm_hides():
    # one wholly wrong row of 16,384 moves the Frobenius measure by < 1%: the
    # per-row measure must still flag it
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((16384, 64))
    got = ref.copy()
    got[777] = rng.standard_normal(64)
    assert L.rel_frobenius(got, ref) < 1.2e-2
    r = L.rel_rows(got, ref)
    assert r[777] > 1.0 and np.count_nonzero(r) == 1


# ----------------------------------------------------------------------------- MXFP8 lossless inputs

LOSSLESS = [synth.small_config("ll_k1", T=160, H=256, I=128, E=3, k=1, routing="zipf", precision="mxfp8"),
            synth.small_config("ll_k2", T=96, H=256, I=128, E=4, k=2, precision="mxfp8")]


def _f64(inp):
    f = L.bf16_bits_to_f64
    return f(inp.x), f(inp.dy), f(inp.w_gate), f(inp.w_up), f(inp.w_down)


@pytest.mark.parametrize("cfg", LOSSLESS, ids=lambda c: c.name)
def test_fake_quant_is_identity_on_lossless_operands(cfg):
    inp = synth.lossless_mxfp8_inputs(cfg)
    x, dy, Wg, Wu, Wd = _f64(inp)
    assert np.array_equal(M.fake_quant(x, 1), x) and np.array_equal(M.fake_quant(dy, 1), dy)
    for W in (Wg, Wu, Wd):                    # both orientations of every weight
        assert np.array_equal(M.fake_quant(W, 1), W) and np.array_equal(M.fake_quant(W, 2), W)
    # the derived activations of every expert: a along I, dh along I, and (for
    # the MXFP8 weight gradients) x, dh, g*a, dy along the expert's rows
    flat = inp.topk_ids.reshape(-1)
    wflat = inp.topk_w.reshape(-1).astype(np.float64)
    for e in range(cfg.E):
        rows = np.nonzero(flat == e)[0]
        if rows.size == 0:
            continue
        tok = rows // cfg.k
        r = L.expert_backward(x[tok], dy[tok], wflat[rows][:, None], Wg[e], Wu[e], Wd[e])
        _, _, a, _ = L.expert_forward(x[tok], Wg[e], Wu[e], Wd[e])
        for v in (a, r["dhg"], r["dhu"], wflat[rows][:, None] * a):
            # silu(h) = h to within exp(-32) here, so a and dh sit that close
            # to values the codec holds exactly
            np.testing.assert_allclose(M.fake_quant(v, 1), v, rtol=1e-12, atol=0)
            np.testing.assert_allclose(L.rows_fq(M.fake_quant, v), v, rtol=1e-12, atol=0)
        assert np.array_equal(L.rows_fq(M.fake_quant, x[tok]), x[tok])
        assert np.array_equal(L.rows_fq(M.fake_quant, dy[tok]), dy[tok])


@pytest.mark.parametrize("cfg", LOSSLESS, ids=lambda c: c.name)
def test_mxfp8_layer_equals_bf16_layer_on_lossless_inputs(cfg):
    inp = synth.lossless_mxfp8_inputs(cfg)
    x, dy, Wg, Wu, Wd = _f64(inp)
    ids, w = inp.topk_ids, inp.topk_w
    out, _ = L.forward(x, ids, w, Wg, Wu, Wd)
    out_q, _ = L.forward(x, ids, w, Wg, Wu, Wd, M.fake_quant)
    g = L.backward(x, ids, w, Wg, Wu, Wd, dy)
    gq = L.backward(x, ids, w, Wg, Wu, Wd, dy, M.fake_quant)
    gqw = L.backward(x, ids, w, Wg, Wu, Wd, dy, M.fake_quant, M.fake_quant)
    assert np.linalg.norm(out) > 0
    assert L.rel_frobenius(out_q, out) <= 1e-12
    for k in ("dx", "dWg", "dWu", "dWd", "dw"):
        assert np.linalg.norm(g[k]) > 0, k
        assert L.rel_frobenius(gq[k], g[k]) <= 1e-12, k
        assert L.rel_frobenius(gqw[k], g[k]) <= 1e-12, k


def test_mxfp8_layer_differs_from_bf16_on_ordinary_inputs():
    # control for the pin above: on normal draws the fake-quant does change results
    cfg = synth.small_config("ctl", T=64, H=256, I=128, E=3, k=2, precision="mxfp8")
    inp = synth.make_inputs(cfg)
    x, dy, Wg, Wu, Wd = _f64(inp)
    out, _ = L.forward(x, inp.topk_ids, inp.topk_w, Wg, Wu, Wd)
    out_q, _ = L.forward(x, inp.topk_ids, inp.topk_w, Wg, Wu, Wd, M.fake_quant)
    assert L.rel_frobenius(out_q, out) > 1e-2
