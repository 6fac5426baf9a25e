"""MXFP8 mode of the layer on the GPU: forward + backward against the fp64
oracle with the MXFP8 fake-quant at the reading's quantization points
(relative Frobenius error <= 6e-2), and bitwise reproducibility across runs and
knob settings."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_table_amd as mok
import synth
from gpu_support import (DEV, TOL_MXFP8, DeviceInputs, compare_full, host_f64, knobs, oracle_full, run_layer,
                         same_bits, status_word)
from oracle import layer as L
from oracle import mxfp8 as M

pytestmark = pytest.mark.gpu


def _mx(name, **kw):
    return synth.small_config(name, precision="mxfp8", **kw)


# MXFP8 needs H and I to be multiples of 128; the ring rows are H + H/32 bytes
SMALL = {
    "mx_k2_ragged": _mx("mx_k2_ragged", T=300, H=256, I=128, E=5, k=2, minibatch_rows=48, macrobatch_tokens=100,
                        ring_bytes=3 * 48 * 264),
    "mx_k1_macro": _mx("mx_k1_macro", T=1000, H=384, I=256, E=3, k=1, minibatch_rows=64, macrobatch_tokens=300,
                       ring_bytes=4 * 64 * 396, routing="dirichlet"),
    "mx_wide": _mx("mx_wide", T=520, H=640, I=384, E=2, k=1, minibatch_rows=160, ring_bytes=1 << 22,
                   routing="zipf"),
    "mx_k_eq_E": _mx("mx_k_eq_E", T=70, H=128, I=128, E=4, k=4, minibatch_rows=16, ring_bytes=2 * 16 * 132),
    # one token: two m-tiles of one row each, every other expert empty
    "mx_single_token": _mx("mx_single_token", T=1, H=128, I=128, E=4, k=2, minibatch_rows=16,
                           ring_bytes=2 * 16 * 132),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_parity_small(name):
    cfg = SMALL[name]
    print(f"[mxfp8 layer] parity {name}", flush=True)
    inp = synth.make_inputs(cfg)
    res = run_layer(DeviceInputs(inp), knobs(cfg))
    assert status_word(res["schedule"]) == 0
    errs = compare_full(res, oracle_full(inp, M.fake_quant), cfg.E, tol=TOL_MXFP8)
    print("vs fake-quant oracle", {k: f"{v:.2e}" for k, v in errs.items() if not k.startswith("dw_")}, flush=True)
    plain = oracle_full(inp)                    # reported, not gated: the quantization error itself
    print("vs unquantized oracle", {n: f"{L.rel_frobenius(host_f64(res[n]), plain[n]):.2e}"
                                    for n in ("out", "dx", "dtopk_w")}, flush=True)


# The k == 1 case hung once (no output for minutes) in a run whose MXFP8 code
# still had a whole-pass mode; that mode is removed (the flag is ignored in
# MXFP8 mode) but the hang's cause was not shown, so the case does not run.
HUNG = "hung once with the MXFP8 whole-pass mode present; cause not shown, kept off the GPU"


@pytest.mark.parametrize("name", ["mx_k2_ragged", pytest.param("mx_k1_macro", marks=pytest.mark.skip(reason=HUNG))])
def test_bitwise_deterministic_and_knob_invariant(name):
    cfg = SMALL[name]
    row = cfg.H + cfg.H // 32                  # MXFP8 ring row bytes
    d = DeviceInputs(synth.make_inputs(cfg))
    first = run_layer(d, knobs(cfg))
    for _ in range(2):
        same_bits(first, run_layer(d, knobs(cfg)))
    for over in (dict(minibatch_rows=16), dict(minibatch_rows=96, ring_bytes=2 * 96 * row),
                 dict(macrobatch_tokens=0), dict(ring_bytes=1 << 22), dict(capacity_multiplier=2.0),
                 dict(debug_flags=mok.MOK_DEBUG_SEPARATE_LAUNCHES)):
        print(f"[mxfp8 layer] knobs {name} {over}", flush=True)
        same_bits(first, run_layer(d, knobs(cfg, **over)))


@pytest.mark.parametrize("name", ["mx_k2_ragged", "mx_wide"])
def test_persistent_grid_size_does_not_change_bits(name):
    # the forward's two GEMMs run in the persistent pair kernel: one workgroup
    # runs every tile in claim order, a few contend for them, more than the
    # compute units queue behind the resident ones; every grid gives the same bits
    cfg = SMALL[name]
    d = DeviceInputs(synth.make_inputs(cfg))
    first = run_layer(d, knobs(cfg))
    for n in (1, 3, 64, 300):
        print(f"[mxfp8 layer] grid {name} {n}", flush=True)
        same_bits(first, run_layer(d, knobs(cfg, persistent_workgroups=n)))


def test_item_trace_records_every_forward_tile_without_changing_bits():
    # the measurement aid on the block-scaled pair: one record per gate/up and
    # down tile of each forward launch, times ordered, outputs unchanged
    cfg = SMALL["mx_k2_ragged"]
    d = DeviceInputs(synth.make_inputs(cfg))
    base = run_layer(d, knobs(cfg))
    assert mok.mok_item_trace_enable(1) == mok.MOK_OK
    try:
        traced = run_layer(d, knobs(cfg))
        rec, n = mok.item_trace_read()
    finally:
        mok.mok_item_trace_enable(0)
    same_bits(base, traced)
    f = rec[rec["kernel"] == mok.MOK_TRACE_FWD_GEMMS]
    assert len(f) > 0
    assert np.all(f["t_claim"] <= f["t_start"]) and np.all(f["t_start"] <= f["t_kloop"])
    assert np.all(f["t_kloop"] <= f["t_end"])
    for launch in set(f["launch"].tolist()):
        r = f[f["launch"] == launch]
        for cls in (1, 2):
            items = r["item"][r["item_class"] == cls]
            assert len(items) == len(set(items.tolist())) > 0


def test_forced_stall_ends_the_forward():
    # the forward's down tiles wait for their m-tiles' gate/up tiles; with every
    # wait giving up at once the launch must end, flag the stall and leave the
    # output unwritten (the backward's GEMMs are separate launches: no waits)
    cfg = SMALL["mx_k2_ragged"]
    d = DeviceInputs(synth.make_inputs(cfg))
    q = mok.MXFP8Weights(d.wg, d.wu, d.wd)
    c = knobs(cfg, debug_flags=mok.MOK_DEBUG_FORCE_STALL)
    ws = mok.get_workspace(c, device=DEV, num_local_tokens=cfg.T, hidden_size=cfg.H, intermediate_size=cfg.I,
                           num_experts=cfg.E, topk=cfg.k)
    sched = mok.build_schedule(ws, d.ids)
    out = torch.full((cfg.T, cfg.H), 7.0, dtype=torch.bfloat16, device=DEV)
    mok.forward(ws, sched, d.x, d.w, q.fwd, out=out)
    torch.cuda.synchronize()
    assert status_word(sched) == mok.MOK_SCHEDULER_STALLED
    assert torch.all(out == 7.0)


@pytest.mark.skip(reason="the whole-pass mode is switched off (MOK_ERROR_UNSUPPORTED): it was present in two "
                         "hangs whose cause was not shown")
@pytest.mark.parametrize("name", ["mx_k2_ragged", "mx_k1_macro"])
def test_whole_pass_flag_in_mxfp8_mode(name):
    cfg = SMALL[name]
    row = cfg.H + cfg.H // 32
    d = DeviceInputs(synth.make_inputs(cfg))
    first = run_layer(d, knobs(cfg))
    for over in (dict(debug_flags=mok.MOK_DEBUG_WHOLE_PASS),
                 dict(debug_flags=mok.MOK_DEBUG_WHOLE_PASS, ring_bytes=2 * cfg.minibatch_rows * row)):
        same_bits(first, run_layer(d, knobs(cfg, **over)))



# ----------------------------------------------------------------------------- MXFP8 weight gradients

@pytest.mark.parametrize("name", ["mx_k2_ragged", "mx_k1_macro", "mx_wide", "mx_k_eq_E", "mx_single_token"])
def test_wgrad_parity_small(name):
    """MOK_MXFP8_WGRAD: weight gradients from operands quantized along the
    expert's rows (zero-padded tails) against the oracle with the same
    quantization; every other output is bit-identical to MXFP8 mode."""
    cfg = SMALL[name]
    print(f"[mxfp8 wgrad] parity {name}", flush=True)
    inp = synth.make_inputs(cfg)
    d = DeviceInputs(inp)
    res = run_layer(d, knobs(cfg, precision=mok.MOK_MXFP8_WGRAD))
    assert status_word(res["schedule"]) == 0
    errs = compare_full(res, oracle_full(inp, M.fake_quant, M.fake_quant), cfg.E, tol=TOL_MXFP8)
    print("vs fake-quant oracle", {k: f"{v:.2e}" for k, v in errs.items() if k.startswith("dw_")}, flush=True)
    same_bits(res, run_layer(d, knobs(cfg)), names=("out", "dx", "dtopk_w"))


def test_wgrad_deterministic_knob_invariant_and_empty_experts():
    cfg = _mx("mx_sparse", T=260, H=256, I=128, E=6, k=1, minibatch_rows=32, ring_bytes=1 << 20,
              routing="zipf")
    inp = synth.make_inputs(cfg)
    inp.topk_ids[:] = np.where(inp.topk_ids < 3, inp.topk_ids, 0)   # experts 3..5 receive nothing
    d = DeviceInputs(inp)
    first = run_layer(d, knobs(cfg, precision=mok.MOK_MXFP8_WGRAD))
    compare_full(first, oracle_full(inp, M.fake_quant, M.fake_quant), cfg.E, tol=TOL_MXFP8)
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert not first[n][3:].float().abs().sum().item()
    row = cfg.H + cfg.H // 32
    for over in ({}, dict(minibatch_rows=16), dict(macrobatch_tokens=50), dict(ring_bytes=2 * 32 * row),
                 dict(debug_flags=mok.MOK_DEBUG_SEPARATE_LAUNCHES)):
        print(f"[mxfp8 wgrad] knobs {over}", flush=True)
        same_bits(first, run_layer(d, knobs(cfg, precision=mok.MOK_MXFP8_WGRAD, **over)))


def test_wgrad_empty_call():
    # T = 0: every expert is empty, so the weight gradients are zeros
    cfg = _mx("mx_empty", T=0, H=128, I=128, E=4, k=2, minibatch_rows=16, ring_bytes=1 << 20)
    d = DeviceInputs(synth.make_inputs(cfg))
    res = run_layer(d, knobs(cfg, precision=mok.MOK_MXFP8_WGRAD))
    assert res["out"].numel() == 0 and res["dx"].numel() == 0
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert not res[n].float().abs().sum().item()



# ----------------------------------------------------------------------------- lossless inputs

LOSSLESS = [_mx("ll_k1", T=160, H=256, I=128, E=3, k=1, routing="zipf", minibatch_rows=32),
            _mx("ll_k2", T=96, H=384, I=128, E=4, k=2, minibatch_rows=48, macrobatch_tokens=40)]


@pytest.mark.parametrize("cfg", LOSSLESS, ids=lambda c: c.name)
def test_lossless_inputs_mxfp8_matches_bf16(cfg):
    """On inputs whose every quantization point is exact (integers times powers
    of two; synth.lossless_mxfp8_inputs), the MXFP8 path must give the BF16
    path's results (BF16 tolerance), in both MXFP8 modes, and the BF16 path
    must match the oracle."""
    inp = synth.lossless_mxfp8_inputs(cfg)
    d = DeviceInputs(inp)
    bf = run_layer(d, knobs(cfg, precision=mok.MOK_BF16))
    assert status_word(bf["schedule"]) == 0
    compare_full(bf, oracle_full(inp), cfg.E)
    ref = {n: host_f64(bf[n]) for n in ("out", "dx", "dw_gate", "dw_up", "dw_down", "dtopk_w")}
    for prec in (mok.MOK_MXFP8, mok.MOK_MXFP8_WGRAD):
        mx = run_layer(d, knobs(cfg, precision=prec))
        assert status_word(mx["schedule"]) == 0
        errs = compare_full(mx, ref, cfg.E)             # against the BF16 path, at the BF16 tolerance
        exact = [n for n in ref if torch.equal(mx[n].view(torch.uint8), bf[n].view(torch.uint8))]
        print(f"[mxfp8 lossless] {cfg.name} precision {prec}: worst {max(errs.values()):.2e}; "
              f"bit-identical to BF16: {exact}", flush=True)
        # every value on the path is exact in both modes, so the bits agree too
        assert sorted(exact) == sorted(ref), f"not bit-identical: {sorted(set(ref) - set(exact))}"
