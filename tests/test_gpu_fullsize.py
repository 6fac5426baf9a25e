"""Full-size workloads, in the launch configuration the benchmark times,
checked against the oracle at sampled outputs it can compute one by one, and
for bitwise reproducibility over ten runs.

Sampling reaches every tile of every GEMM:
* tokens: one routed row from every 128-row chunk of every (mini-batch,
  expert) segment of the schedule, whose whole output rows (out, dx) and
  router-weight gradients are checked. An m-tile of the segment GEMMs is 128
  or 256 consecutive rows of one segment, so every m-tile holds a sampled row,
  and a whole output row crosses every n-tile;
* weight gradients: for every expert that received rows, one column of
  dW_gate and dW_up (one row of dW_down) in every 128-wide block of I; the
  weight-gradient GEMMs tile I in 128 or 256 wide blocks, and each sampled
  column (dW_down row) crosses every tile along H.
Every sampled row and column passes the per-row gate beside the Frobenius
gate (gpu_support)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_table_amd as mok
import synth
from gpu_support import (ROW_FACTOR, TOL_BF16, TOL_MXFP8, DeviceInputs, host_f64, knobs, row_gate, run_layer,
                         same_bits, scalar_gate, status_word)
from oracle import layer as L
from oracle import mxfp8 as M
from oracle import schedule as S

pytestmark = pytest.mark.gpu

CHUNK = 128   # the smaller of the two m-tile heights


def tokens_covering_mtiles(cfg, ids, rng):
    """Tokens such that every CHUNK-row piece of every schedule segment holds
    one of their routed rows (greedy: each pick covers the k pieces its rows
    fall in), plus the first and last token."""
    s = S.build(ids, cfg.E, cfg.minibatch_rows, cfg.macrobatch_tokens)
    assert s.status == 0
    R = cfg.R
    piece_of_q = np.empty(R, dtype=np.int64)
    pieces = []
    for (_, _, q0, n) in s.segments:
        for c0 in range(q0, q0 + n, CHUNK):
            piece_of_q[c0: min(c0 + CHUNK, q0 + n)] = len(pieces)
            pieces.append((c0, min(c0 + CHUNK, q0 + n)))
    covered = np.zeros(len(pieces), dtype=bool)
    toks = {0, cfg.T - 1}
    for t in toks:
        covered[piece_of_q[s.inv[t * cfg.k: (t + 1) * cfg.k]]] = True
    for p in rng.permutation(len(pieces)):
        if covered[p]:
            continue
        lo, hi = pieces[p]
        t = int(s.perm[rng.integers(lo, hi)]) // cfg.k
        toks.add(t)
        covered[piece_of_q[s.inv[t * cfg.k: (t + 1) * cfg.k]]] = True
    assert covered.all()
    return np.array(sorted(toks)), len(pieces)


def wgrad_columns(I, rng):
    """One column in every CHUNK-wide block of I."""
    return np.array([b + int(rng.integers(0, min(CHUNK, I - b))) for b in range(0, I, CHUNK)])


def _check(cfg, mx_wgrad=False):
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
    k = cfg.k
    toks, n_pieces = tokens_covering_mtiles(cfg, inp.topk_ids, rng)
    cols = wgrad_columns(cfg.I, rng)
    print(f"[fullsize] {cfg.name}: {toks.size} tokens cover {n_pieces} row pieces; "
          f"{cols.size} weight-gradient columns per expert", flush=True)
    dev = res["out"].device
    it = torch.from_numpy(toks).to(dev)
    ic = torch.from_numpy(cols).to(dev)
    got_out, got_dx, got_dw = host_f64(res["out"][it]), host_f64(res["dx"][it]), host_f64(res["dtopk_w"][it])
    dwg = host_f64(res["dw_gate"][:, :, ic])           # [E, H, cols]
    dwu = host_f64(res["dw_up"][:, :, ic])
    dwd = host_f64(res["dw_down"][:, ic, :])           # [E, cols, H]

    x_s, dy_s = f(inp.x[toks]), f(inp.dy[toks])
    ids_s, w_s = inp.topk_ids[toks], inp.topk_w[toks].astype(np.float64)
    ref_out, ref_dx, ref_dw = np.zeros_like(x_s), np.zeros_like(x_s), np.zeros((toks.size, k))
    flat = inp.topk_ids.reshape(-1)
    counts = np.bincount(flat, minlength=cfg.E)
    errs, bad = {}, {}
    experts = [e for e in range(cfg.E) if counts[e] > 0]
    for n, e in enumerate(experts):                      # one expert's weights decoded at a time
        if n % 32 == 0:
            print(f"[fullsize] {cfg.name}: oracle expert {n + 1}/{len(experts)}", flush=True)
        Wg, Wu, Wd = f(inp.w_gate[e]), f(inp.w_up[e]), f(inp.w_down[e])
        ti, tj = np.nonzero(ids_s == e)
        if ti.size:
            g = w_s[ti, tj][:, None]
            y = L.expert_forward(x_s[ti], Wg, Wu, Wd, fq)[3]
            np.add.at(ref_out, ti, g * y)
            r = L.expert_backward(x_s[ti], dy_s[ti], g, Wg, Wu, Wd, fq)
            np.add.at(ref_dx, ti, r["dxr"])
            ref_dw[ti, tj] = r["dw"]
        rows = np.nonzero(flat == e)[0]
        tok = rows // k
        ga = inp.topk_w.reshape(-1)[rows][:, None].astype(np.float64)
        a, b, c = L.expert_wgrad_columns(f(inp.x[tok]), f(inp.dy[tok]), ga, Wg, Wu, Wd, cols, fq, wfq)
        for name, got, ref in ((f"dw_gate[{e}]", dwg[e].T, a.T), (f"dw_up[{e}]", dwu[e].T, b.T),
                               (f"dw_down[{e}]", dwd[e], c)):
            errs[name] = L.rel_frobenius(got, ref)
            row_gate(got, ref, name, tol, bad)           # rows here: sampled columns of dW_gate / dW_up
    for e in range(cfg.E):
        if counts[e] == 0:                               # experts without rows: zero gradients
            assert not (np.any(dwg[e]) or np.any(dwu[e]) or np.any(dwd[e])), e
    for name, got, ref in (("out", got_out, ref_out), ("dx", got_dx, ref_dx)):
        errs[name] = L.rel_frobenius(got, ref)
        errs[name + " worst row"] = row_gate(got, ref, name, tol, bad)
    errs["dtopk_w"] = L.rel_frobenius(got_dw, ref_dw)
    errs["dtopk_w worst elem"] = scalar_gate(got_dw, ref_dw, "dtopk_w", tol, bad)
    shown = {k2: f"{v:.2e}" for k2, v in errs.items() if not k2.startswith("dw_") or k2.endswith("[0]")}
    print(shown, flush=True)
    bad.update({k2: v for k2, v in errs.items() if "worst" not in k2 and not v <= tol})
    assert not bad, f"over tolerance {tol} (rows {ROW_FACTOR * tol}): {bad}"


def test_ep64_share():
    _check(synth.CONFIGS["ep64_share"])


def test_stream_macro_batches():
    _check(synth.CONFIGS["stream"])


def test_full_layer():
    _check(synth.CONFIGS["full_layer"])


def test_ep64_share_mxfp8_zipf():
    _check(synth.CONFIGS["ep64_share_mxfp8"])


def test_ep64_share_mxfp8_uniform():
    _check(synth.CONFIGS["ep64_share_mxfp8_uniform"])


def test_ep64_share_mxfp8_wgrad():
    _check(synth.CONFIGS["ep64_share_mxfp8"], mx_wgrad=True)


@pytest.mark.timeout(400)
def test_largest_activation_under_the_byte_bound():
    """x, dy, out and dx of (2^17 - 1) x 8192 bf16 each, 16 KiB short of 2 GiB:
    the largest [T, H] the layer's 32-bit byte offsets take at H = 8192 (one
    token more is refused). Eight ring rounds of 16,384 rows."""
    _check(synth.small_config("x_byte_bound", T=(1 << 17) - 1, H=8192, I=64, E=8, k=1, minibatch_rows=512,
                              ring_bytes=256 << 20))


@pytest.mark.parametrize("name", ["ep64_share", "ep64_share_mxfp8"])
def test_ten_runs_bitwise_at_full_size(name):
    """Ten runs of the benchmark's configuration (default knobs, the persistent
    kernels) give the same bits in every output."""
    cfg = synth.CONFIGS[name]
    d = DeviceInputs(synth.make_inputs(cfg))
    first = run_layer(d, knobs(cfg))
    assert status_word(first["schedule"]) == 0
    for i in range(9):
        print(f"[fullsize] {name}: run {i + 2}/10", flush=True)
        same_bits(first, run_layer(d, knobs(cfg)))
