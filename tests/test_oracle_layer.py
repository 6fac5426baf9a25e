"""Pins for the fp64 layer oracle (O2/O3): reductions to a dense SwiGLU FFN,
central finite differences, an independent autograd formulation, and the fused
router-weight-gradient identity."""
import numpy as np
import pytest
import torch

import synth
from oracle import layer as L
from oracle import mxfp8 as M


def _tiny(T=5, H=8, I=4, E=3, k=2, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    w = rng.random((T, k)) + 0.1
    Wg = rng.standard_normal((E, H, I)) / np.sqrt(H)
    Wu = rng.standard_normal((E, H, I)) / np.sqrt(H)
    Wd = rng.standard_normal((E, I, H)) / np.sqrt(I)
    dy = rng.standard_normal((T, H))
    return x, ids, w, Wg, Wu, Wd, dy


def _dense_swiglu_torch(x, Wg, Wu, Wd):
    x, Wg, Wu, Wd = (torch.from_numpy(np.ascontiguousarray(a)) for a in (x, Wg, Wu, Wd))
    return (torch.nn.functional.silu(x @ Wg) * (x @ Wu) @ Wd).numpy()


def test_single_expert_is_dense_ffn():
    x, _, _, Wg, Wu, Wd, _ = _tiny(T=7, E=1, k=1)
    ids = np.zeros((7, 1), np.int64)
    w = np.ones((7, 1))
    out, _ = L.forward(x, ids, w, Wg, Wu, Wd)
    ref = _dense_swiglu_torch(x, Wg[0], Wu[0], Wd[0])
    assert np.max(np.abs(out - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_identical_experts_reduce_to_dense_ffn():
    # renormalised top-k weights sum to one, so identical experts give the dense FFN
    cfg = synth.CONFIGS["tiny"]
    ids, w, _ = synth.make_routing(cfg)
    _, _, _, Wg, Wu, Wd, _ = _tiny(H=16, I=8, E=1, k=1)
    Wg, Wu, Wd = (np.repeat(a, cfg.E, axis=0) for a in (Wg, Wu, Wd))
    x = np.random.default_rng(1).standard_normal((cfg.T, 16))
    out, _ = L.forward(x, ids, w, Wg, Wu, Wd)
    ref = _dense_swiglu_torch(x, Wg[0], Wu[0], Wd[0]) * w.astype(np.float64).sum(1, keepdims=True)
    assert np.max(np.abs(out - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    # and the fp32-rounded weights sum to one within fp32 rounding
    assert np.max(np.abs(w.astype(np.float64).sum(1) - 1)) < 1e-6


def _loss(x, ids, w, Wg, Wu, Wd, dy):
    return float(np.sum(dy * L.forward(x, ids, w, Wg, Wu, Wd)[0]))


@pytest.mark.parametrize("seed", [0, 1])
def test_finite_differences(seed):
    x, ids, w, Wg, Wu, Wd, dy = _tiny(seed=seed)
    g = L.backward(x, ids, w, Wg, Wu, Wd, dy)
    params = dict(x=x, w=w, Wg=Wg, Wu=Wu, Wd=Wd)
    analytic = dict(x=g["dx"], w=g["dw"], Wg=g["dWg"], Wu=g["dWu"], Wd=g["dWd"])
    for name, p in params.items():
        fd = np.zeros_like(p)
        for idx in np.ndindex(p.shape):
            old = p[idx]
            h = 1e-5 * max(1.0, abs(old))
            p[idx] = old + h
            lp = _loss(x, ids, w, Wg, Wu, Wd, dy)
            p[idx] = old - h
            lm = _loss(x, ids, w, Wg, Wu, Wd, dy)
            p[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = L.rel_frobenius(analytic[name], fd)
        assert err <= 1e-6, (name, err)


def test_router_logit_chain_finite_differences():
    # The harness chains softmax -> top-k -> renormalise in front of the layer;
    # the layer's router-weight gradient must give the logits' gradient by the
    # chain rule through that map (top-k set held fixed).
    x, _, _, Wg, Wu, Wd, dy = _tiny(T=4, E=4, k=2, seed=3)
    logits = np.random.default_rng(5).standard_normal((4, 4)).astype(np.float32).astype(np.float64)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :2]

    def weights(z):
        p = np.exp(z - z.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        s = np.take_along_axis(p, ids, 1)
        return s / s.sum(1, keepdims=True)

    dw = L.backward(x, ids, weights(logits), Wg, Wu, Wd, dy)["dw"]
    # analytic chain: w_j = exp(z_j)/sum_{sel} exp(z) -> dL/dz_j = w_j (dw_j - sum_i w_i dw_i)
    w = weights(logits)
    dz = np.zeros_like(logits)
    np.put_along_axis(dz, ids, w * (dw - np.sum(w * dw, 1, keepdims=True)), 1)
    fd = np.zeros_like(logits)
    for idx in np.ndindex(logits.shape):
        zp, zm = logits.copy(), logits.copy()
        zp[idx] += 1e-6
        zm[idx] -= 1e-6
        fd[idx] = (_loss(x, ids, weights(zp), Wg, Wu, Wd, dy) -
                   _loss(x, ids, weights(zm), Wg, Wu, Wd, dy)) / 2e-6
    assert L.rel_frobenius(dz, fd) <= 1e-6


def test_autograd_independent_formulation():
    # per-slot gather of each token's expert weights, torch autograd in fp64
    x, ids, w, Wg, Wu, Wd, dy = _tiny(T=6, H=12, I=8, E=4, k=3, seed=7)
    tx, tw = torch.tensor(x, requires_grad=True), torch.tensor(w, requires_grad=True)
    tg, tu, td = (torch.tensor(a, requires_grad=True) for a in (Wg, Wu, Wd))
    tid = torch.tensor(ids)
    out = torch.zeros_like(tx)
    for j in range(ids.shape[1]):
        e = tid[:, j]
        hg = torch.bmm(tx[:, None, :], tg[e])[:, 0]
        hu = torch.bmm(tx[:, None, :], tu[e])[:, 0]
        y = torch.bmm((torch.nn.functional.silu(hg) * hu)[:, None, :], td[e])[:, 0]
        out = out + tw[:, j:j + 1] * y
    (out * torch.tensor(dy)).sum().backward()
    g = L.backward(x, ids, w, Wg, Wu, Wd, dy)
    ref_out, _ = L.forward(x, ids, w, Wg, Wu, Wd)
    assert L.rel_frobenius(ref_out, out.detach().numpy()) <= 1e-12
    for mine, theirs in ((g["dx"], tx.grad), (g["dw"], tw.grad), (g["dWg"], tg.grad),
                         (g["dWu"], tu.grad), (g["dWd"], td.grad)):
        assert L.rel_frobenius(mine, theirs.numpy()) <= 1e-12


def test_fused_router_grad_identity():
    x, ids, w, Wg, Wu, Wd, dy = _tiny(T=9, H=16, I=8, E=4, k=2, seed=11)
    g = L.backward(x, ids, w, Wg, Wu, Wd, dy)
    assert np.max(np.abs(g["dw"] - g["dw_direct"])) <= 1e-12 * max(1.0, np.max(np.abs(g["dw"])))


@pytest.mark.parametrize("fq,wfq", [(None, None), (M.fake_quant, None), (M.fake_quant, M.fake_quant)],
                         ids=["bf16", "mxfp8", "mxfp8_wgrad"])
def test_sampled_forms_match_full(fq, wfq):
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_inputs(cfg)
    f = L.bf16_bits_to_f64
    x, dy, Wg, Wu, Wd = f(inp.x), f(inp.dy), f(inp.w_gate), f(inp.w_up), f(inp.w_down)
    out, _ = L.forward(x, inp.topk_ids, inp.topk_w, Wg, Wu, Wd, fq)
    g = L.backward(x, inp.topk_ids, inp.topk_w, Wg, Wu, Wd, dy, fq, wfq)
    toks = np.array([0, 5, 17, 63])
    ew = lambda e: (Wg[e], Wu[e], Wd[e])
    o = L.token_forward(x[toks], inp.topk_ids[toks], inp.topk_w[toks], ew, fq)
    assert np.max(np.abs(o - out[toks])) < 1e-12
    dx, dw = L.token_backward(x[toks], dy[toks], inp.topk_ids[toks], inp.topk_w[toks], ew, fq)
    assert np.max(np.abs(dx - g["dx"][toks])) < 1e-12
    assert np.max(np.abs(dw - g["dw"][toks])) < 1e-12
    e = 3
    rows = np.nonzero(inp.topk_ids.reshape(-1) == e)[0]
    cols = np.array([0, 7, 63])
    gw = inp.topk_w.reshape(-1)[rows][:, None].astype(np.float64)
    a, b, c = L.expert_wgrad_columns(x[rows // cfg.k], dy[rows // cfg.k], gw, Wg[e], Wu[e], Wd[e], cols, fq, wfq)
    assert np.max(np.abs(a - g["dWg"][e][:, cols])) < 1e-12
    assert np.max(np.abs(b - g["dWu"][e][:, cols])) < 1e-12
    assert np.max(np.abs(c - g["dWd"][e][cols, :])) < 1e-12


def test_bf16_decode():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], np.uint16)
    v = L.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 0.0 and np.signbit(v[3])
    assert v[4] == (2 - 2 ** -7) * 2.0 ** 127 and v[5] == 2.0 ** -133 and v[6] == 3.140625


def test_mxfp8_quantization_points():
    """The fake-quant hook is applied to exactly the operands the MXFP8 reading
    names, each along its contraction axis: forward gate/up (x, W_gate, W_up
    along H), forward down (a, W_down along I), backward dA (dy, W_down along
    H), backward dX (dh_g, dh_u, W_gate, W_up along I); nothing else."""
    n, H, I = 3, 64, 32                      # H != I tells the axes apart
    rng = np.random.default_rng(5)
    xe, dye = rng.standard_normal((n, H)), rng.standard_normal((n, H))
    Wg, Wu = rng.standard_normal((H, I)), rng.standard_normal((H, I))
    Wd = rng.standard_normal((I, H))
    calls = []

    def spy(a, axis):
        calls.append((a.shape, a.shape[axis]))
        return a

    L.expert_forward(xe, Wg, Wu, Wd, spy)
    fwd = sorted(calls)
    assert fwd == sorted([((n, H), H), ((H, I), H), ((H, I), H), ((n, I), I), ((I, H), I)])
    calls.clear()
    L.expert_backward(xe, dye, np.ones((n, 1)), Wg, Wu, Wd, spy)
    bwd_only = list(calls)
    for c in fwd:                            # the recomputed forward quantizes as above
        bwd_only.remove(c)
    assert sorted(bwd_only) == sorted([((n, H), H), ((I, H), H),            # dA: dy, W_down along H
                                       ((n, I), I), ((H, I), I),            # dX: dh_g, W_gate along I
                                       ((n, I), I), ((H, I), I)])           # dX: dh_u, W_up along I


def test_mxfp8_wgrad_quantization_points():
    """The weight-gradient hook quantizes exactly x, dh_g, dh_u, g*a and dy,
    each along the row (token) axis, zero-padded to whole 32-row blocks."""
    n, H, I = 37, 64, 32
    rng = np.random.default_rng(6)
    xe, dye = rng.standard_normal((n, H)), rng.standard_normal((n, H))
    Wg, Wu, Wd = rng.standard_normal((H, I)), rng.standard_normal((H, I)), rng.standard_normal((I, H))
    calls = []

    def spy(a, axis):
        calls.append((a.shape, axis))
        return a

    plain = L.expert_backward(xe, dye, np.full((n, 1), 0.5), Wg, Wu, Wd)
    r = L.expert_backward(xe, dye, np.full((n, 1), 0.5), Wg, Wu, Wd, wgrad_fq=spy)
    assert sorted(calls) == sorted([((64, H), 0), ((64, I), 0), ((64, H), 0), ((64, I), 0),
                                    ((64, I), 0), ((64, H), 0)])
    for k in ("dWg", "dWu", "dWd"):          # the identity hook reduces to the unquantized products
        np.testing.assert_allclose(r[k], plain[k], rtol=1e-13, atol=1e-12)


def test_mxfp8_wgrad_blocks_by_hand():
    """rows_fq on 40 rows: rows 0-31 form one block per column, rows 32-39 a
    block of their own (its scale from those 8 rows alone), checked against the
    codec applied to each column's blocks one by one."""
    rng = np.random.default_rng(7)
    a = rng.standard_normal((40, 3)) * np.array([1.0, 300.0, 1e-3])
    a[35:, 1] *= 1000.0                       # the tail block's amax differs from the first block's
    got = L.rows_fq(M.fake_quant, a)
    want = np.zeros_like(a)
    for c in range(3):
        for r0, r1 in ((0, 32), (32, 40)):
            blk = np.zeros(32)
            blk[:r1 - r0] = a[r0:r1, c]
            el, sc = M.quantize(blk[None, :])
            want[r0:r1, c] = M.dequantize(el, sc)[0, :r1 - r0]
    np.testing.assert_array_equal(got, want)


def test_mxfp8_wgrad_error_bound():
    """Each quantized operand is within 2^-4 relative of its value (E4M3 keeps 3
    mantissa bits, so half an ulp is 2^-4 of the value's binade), so every
    product term, and the sum, moves by at most (2*2^-4 + 2^-8) sum |x||dh|."""
    n, H, I = 70, 64, 32
    rng = np.random.default_rng(8)
    xe, dye = rng.standard_normal((n, H)), rng.standard_normal((n, H))
    Wg, Wu, Wd = rng.standard_normal((H, I)), rng.standard_normal((H, I)), rng.standard_normal((I, H))
    g = rng.uniform(0.1, 1.0, (n, 1))
    plain = L.expert_backward(xe, dye, g, Wg, Wu, Wd)
    q = L.expert_backward(xe, dye, g, Wg, Wu, Wd, wgrad_fq=M.fake_quant)
    eps = 2 * 2.0 ** -4 + 2.0 ** -8
    bounds = dict(dWg=np.abs(xe).T @ np.abs(plain["dhg"]), dWu=np.abs(xe).T @ np.abs(plain["dhu"]))
    _, _, a, _ = L.expert_forward(xe, Wg, Wu, Wd)
    bounds["dWd"] = np.abs(g * a).T @ np.abs(dye)
    for k, b in bounds.items():
        assert np.all(np.abs(q[k] - plain[k]) <= eps * b + 1e-12), k
        assert not np.allclose(q[k], plain[k], rtol=1e-6), k   # the hook did quantize
