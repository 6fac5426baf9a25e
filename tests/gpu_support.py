"""Helpers for the GPU tests: upload seeded inputs, run the layer through the
C ABI, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_layer_table_amd as mok
import synth
from oracle import layer as L

DEV = "cuda:0"
TOL_BF16 = 1e-2      # relative Frobenius error, per output tensor (per expert for dW)
TOL_MXFP8 = 6e-2     # same measure, MXFP8 mode against the fake-quant oracle
# Per-row gates beside each Frobenius gate: rel_rows of every output row (token
# rows of out / dx, rows of each expert's dW), and for the router-weight
# gradient (one value per routed row) |got - ref| <= tol * (|ref| + rms(ref)).
# Twice the tensor tolerance: a row averages the same per-element rounding
# errors over >= 64 elements, so its error sits near the tensor's; a wrong row
# (another row's values, zeros, the wrong expert) scores about 1 or more.
ROW_FACTOR = 2.0


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    """bf16 / fp32 device tensor -> fp64 numpy (exact)."""
    if t.dtype == torch.bfloat16:
        return L.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def knobs(cfg: synth.LayerConfig, **over) -> mok.MoKConfig:
    k = dict(minibatch_rows=cfg.minibatch_rows, macrobatch_tokens=cfg.macrobatch_tokens,
             ring_bytes=cfg.ring_bytes, capacity_multiplier=1.0,
             precision=mok.MOK_BF16 if cfg.precision == "bf16" else mok.MOK_MXFP8)
    k.update(over)
    return mok.MoKConfig(**k)


class DeviceInputs:
    def __init__(self, inp: synth.LayerInputs):
        self.cfg = inp.cfg
        self.ids = torch.from_numpy(inp.topk_ids.astype(np.int32)).to(DEV)
        self.w = torch.from_numpy(inp.topk_w.astype(np.float32)).to(DEV)
        self.x = dev_bf16(inp.x)
        self.dy = dev_bf16(inp.dy)
        self.wg = dev_bf16(inp.w_gate)
        self.wu = dev_bf16(inp.w_up)
        self.wd = dev_bf16(inp.w_down)


def run_layer(d: DeviceInputs, config: mok.MoKConfig, backward: bool = True):
    """Schedule + forward (+ backward) on the device. Returns dict of device tensors."""
    c = d.cfg
    ws = mok.get_workspace(config, device=DEV, num_local_tokens=c.T, hidden_size=c.H,
                           intermediate_size=c.I, num_experts=c.E, topk=c.k)
    sched = mok.build_schedule(ws, d.ids)
    if config.precision in (mok.MOK_MXFP8, mok.MOK_MXFP8_WGRAD):
        q = mok.MXFP8Weights(d.wg, d.wu, d.wd)
        wf, wb = q.fwd, q.bwd
    else:
        wf = wb = mok.weights_bf16(d.wg, d.wu, d.wd)
    out, ctx = mok.forward(ws, sched, d.x, d.w, wf)
    res = dict(out=out, schedule=sched)
    if backward:
        res.update(mok.backward(ws, sched, ctx, d.x, d.w, wb, d.dy))
    torch.cuda.synchronize()
    return res


def status_word(sched: torch.Tensor) -> int:
    return int(sched[:4].cpu().numpy().view(np.uint32)[0])


def oracle_full(inp: synth.LayerInputs, fq=None, wgrad_fq=None):
    """fp64 oracle of the whole layer; fq = the MXFP8 fake-quant for MXFP8 mode,
    wgrad_fq the same for the MXFP8 weight gradients."""
    f = L.bf16_bits_to_f64
    x, dy = f(inp.x), f(inp.dy)
    Wg, Wu, Wd = f(inp.w_gate), f(inp.w_up), f(inp.w_down)
    out, _ = L.forward(x, inp.topk_ids, inp.topk_w, Wg, Wu, Wd, fq)
    g = L.backward(x, inp.topk_ids, inp.topk_w, Wg, Wu, Wd, dy, fq, wgrad_fq)
    return dict(out=out, dx=g["dx"], dw_gate=g["dWg"], dw_up=g["dWu"], dw_down=g["dWd"], dtopk_w=g["dw"])


def row_gate(got, ref, name, tol, bad):
    """Per-row check (ROW_FACTOR * tol): records the worst row of `name` in
    `bad` when it is over; returns the worst row error."""
    r = L.rel_rows(got, ref)
    worst = float(np.max(r)) if r.size else 0.0
    if not worst <= ROW_FACTOR * tol:
        bad[f"{name} row {int(np.argmax(r))}"] = worst
    return worst


def scalar_gate(got, ref, name, tol, bad):
    """Per-element check of a vector of scalars (the router-weight gradient):
    |got - ref| <= ROW_FACTOR * tol * (|ref| + rms(ref))."""
    got, ref = np.asarray(got, np.float64).reshape(-1), np.asarray(ref, np.float64).reshape(-1)
    if ref.size == 0:
        return 0.0
    scale = np.abs(ref) + np.sqrt(np.mean(ref * ref))
    r = np.abs(got - ref) / np.where(scale > 0, scale, 1.0)
    r[(scale == 0) & (got != ref)] = np.inf
    worst = float(np.max(r))
    if not worst <= ROW_FACTOR * tol:
        bad[f"{name} element {int(np.argmax(r))}"] = worst
    return worst


def compare_full(res, ref, E, tol=TOL_BF16):
    """Frobenius gate per tensor (per expert for dW) plus the per-row gates."""
    errs, bad = {}, {}
    for name in ("out", "dx", "dtopk_w"):
        if name in res:
            got = host_f64(res[name])
            errs[name] = L.rel_frobenius(got, ref[name])
            if name == "dtopk_w":
                errs[name + " worst elem"] = scalar_gate(got, ref[name], name, tol, bad)
            else:
                errs[name + " worst row"] = row_gate(got, ref[name], name, tol, bad)
    for name in ("dw_gate", "dw_up", "dw_down"):
        if name in res:
            got = host_f64(res[name])
            for e in range(E):
                errs[f"{name}[{e}]"] = L.rel_frobenius(got[e], ref[name][e])
                errs[f"{name}[{e}] worst row"] = row_gate(got[e], ref[name][e], f"{name}[{e}]", tol, bad)
    bad.update({k: v for k, v in errs.items() if "worst" not in k and not v <= tol})
    assert not bad, f"over tolerance {tol} (rows: {ROW_FACTOR * tol}): {bad}"
    return errs


def same_bits(a: dict, b: dict, names=("out", "dx", "dw_gate", "dw_up", "dw_down", "dtopk_w")):
    for n in names:
        if n in a:
            assert torch.equal(a[n].view(torch.uint8) if a[n].dtype != torch.float32 else a[n].view(torch.int32),
                               b[n].view(torch.uint8) if b[n].dtype != torch.float32 else b[n].view(torch.int32)), n
