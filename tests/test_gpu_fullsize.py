"""Full-size workloads, in the launch configuration the benchmark times,
checked against the oracle at sampled outputs it can compute one by one:
whole output rows of sampled tokens (out, dx, router-weight gradient) and
whole columns of each expert's weight gradients."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_table_amd as mok
import synth
from gpu_support import TOL_BF16, TOL_MXFP8, DeviceInputs, host_f64, knobs, run_layer, status_word
from oracle import layer as L
from oracle import mxfp8 as M

pytestmark = pytest.mark.gpu


def _sample_tokens(cfg, ids, rng, n=48):
    flat = ids.reshape(-1)
    picks = set(rng.choice(cfg.T, size=min(n, cfg.T), replace=False).tolist())
    picks |= {0, cfg.T - 1}
    for e in range(min(cfg.E, 8)):               # first and last row of the first experts
        rows = np.nonzero(flat == e)[0]
        if rows.size:
            picks |= {int(rows[0] // cfg.k), int(rows[-1] // cfg.k)}
    return np.array(sorted(picks))


def _check(cfg, experts_for_wgrad=2, n_tokens=48, mx_wgrad=False):
    mx = cfg.precision == "mxfp8"
    fq, tol = (M.fake_quant, TOL_MXFP8) if mx else (None, TOL_BF16)
    wfq = M.fake_quant if mx_wgrad else None
    print(f"[fullsize] {cfg.name}: generating inputs", flush=True)
    inp = synth.make_inputs(cfg)
    d = DeviceInputs(inp)
    print(f"[fullsize] {cfg.name}: running layer", flush=True)
    res = run_layer(d, knobs(cfg, precision=mok.MOK_MXFP8_WGRAD) if mx_wgrad else knobs(cfg))
    assert status_word(res["schedule"]) == 0
    rng = np.random.default_rng(1)
    f = L.bf16_bits_to_f64
    toks = _sample_tokens(cfg, inp.topk_ids, rng, n_tokens)
    cache = {}

    def ew(e):
        if e not in cache:
            cache[e] = (f(inp.w_gate[e]), f(inp.w_up[e]), f(inp.w_down[e]))
        return cache[e]

    x, dy = f(inp.x[toks]), f(inp.dy[toks])
    ref_out = L.token_forward(x, inp.topk_ids[toks], inp.topk_w[toks], ew, fq)
    ref_dx, ref_dw = L.token_backward(x, dy, inp.topk_ids[toks], inp.topk_w[toks], ew, fq)
    it = torch.from_numpy(toks).to(res["out"].device)
    errs = dict(out=L.rel_frobenius(host_f64(res["out"][it]), ref_out),
                dx=L.rel_frobenius(host_f64(res["dx"][it]), ref_dx),
                dtopk_w=L.rel_frobenius(host_f64(res["dtopk_w"][it]), ref_dw))
    # weight gradients: whole columns (rows of dW_down) for the largest and smallest experts
    counts = np.bincount(inp.topk_ids.reshape(-1), minlength=cfg.E)
    nz = [e for e in np.argsort(-counts, kind="stable") if counts[e] > 0]
    for e in [nz[0], nz[-1]][:experts_for_wgrad]:
        rows = np.nonzero(inp.topk_ids.reshape(-1) == e)[0]
        cols = np.unique(np.concatenate([[0, cfg.I - 1], rng.choice(cfg.I, 6, replace=False)]))
        tok = rows // cfg.k
        gw = inp.topk_w.reshape(-1)[rows][:, None].astype(np.float64)
        Wg, Wu, Wd = ew(int(e))
        a, b, c = L.expert_wgrad_columns(f(inp.x[tok]), f(inp.dy[tok]), gw, Wg, Wu, Wd, cols, fq, wfq)
        ic = torch.from_numpy(cols).to(res["out"].device)
        errs[f"dw_gate[{e}]"] = L.rel_frobenius(host_f64(res["dw_gate"][int(e)][:, ic]), a)
        errs[f"dw_up[{e}]"] = L.rel_frobenius(host_f64(res["dw_up"][int(e)][:, ic]), b)
        errs[f"dw_down[{e}]"] = L.rel_frobenius(host_f64(res["dw_down"][int(e)][ic, :]), c)
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


def test_ep64_share():
    _check(synth.CONFIGS["ep64_share"])


def test_stream_macro_batches():
    _check(synth.CONFIGS["stream"])


def test_full_layer():
    # 256 experts: few sampled tokens keep the oracle's weight decoding short
    _check(synth.CONFIGS["full_layer"], n_tokens=6)


def test_ep64_share_mxfp8_zipf():
    _check(synth.CONFIGS["ep64_share_mxfp8"])


def test_ep64_share_mxfp8_uniform():
    _check(synth.CONFIGS["ep64_share_mxfp8_uniform"])


def test_ep64_share_mxfp8_wgrad():
    _check(synth.CONFIGS["ep64_share_mxfp8"], mx_wgrad=True)
