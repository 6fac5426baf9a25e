"""Forward + backward on the GPU against the fp64 oracle at sizes the oracle
finishes in seconds, plus the method's invariants: permute then unpermute is
the identity, runs and knob settings are bitwise identical, data-dependent
errors raise the status word."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_table_amd as mok
import synth
from gpu_support import (DEV, DeviceInputs, compare_full, knobs, oracle_full, run_layer, same_bits,
                         status_word)

pytestmark = pytest.mark.gpu

# several tiles in every GEMM dimension, ragged tails, rings smaller than the data
SMALL = {
    "tiny": synth.CONFIGS["tiny"],
    "ragged_k2": synth.small_config("ragged_k2", T=300, H=256, I=192, E=5, k=2, minibatch_rows=48,
                                    macrobatch_tokens=100, ring_bytes=3 * 48 * 512),
    "k1_macro": synth.small_config("k1_macro", T=1000, H=384, I=128, E=3, k=1, minibatch_rows=64,
                                   macrobatch_tokens=300, ring_bytes=4 * 64 * 768, routing="dirichlet"),
    "k_eq_E": synth.small_config("k_eq_E", T=70, H=128, I=64, E=4, k=4, minibatch_rows=16,
                                 ring_bytes=2 * 16 * 256),
    "wide": synth.small_config("wide", T=520, H=640, I=320, E=2, k=1, minibatch_rows=160,
                               ring_bytes=1 << 22, routing="zipf"),
    # one token: two m-tiles of one row each, every other expert empty
    "single_token": synth.small_config("single_token", T=1, H=128, I=64, E=4, k=2, minibatch_rows=16,
                                       ring_bytes=2 * 16 * 256),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_parity_small(name):
    cfg = SMALL[name]
    print(f"[layer] parity {name}", flush=True)
    inp = synth.make_inputs(cfg)
    res = run_layer(DeviceInputs(inp), knobs(cfg))
    assert status_word(res["schedule"]) == 0          # includes: the persistent queues never stalled
    errs = compare_full(res, oracle_full(inp), cfg.E)
    print({k: f"{v:.2e}" for k, v in errs.items() if not k.startswith("dw_")}, flush=True)


def test_empty_experts_get_zero_weight_grads():
    cfg = synth.small_config("sparse", T=200, H=128, I=64, E=6, k=1, minibatch_rows=32, ring_bytes=1 << 20,
                             routing="zipf")
    inp = synth.make_inputs(cfg)
    inp.topk_ids[:] = np.where(inp.topk_ids < 3, inp.topk_ids, 0)   # experts 3..5 receive nothing
    res = run_layer(DeviceInputs(inp), knobs(cfg))
    compare_full(res, oracle_full(inp), cfg.E)
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert not res[n][3:].float().abs().sum().item()


def test_empty_call():
    cfg = synth.small_config("empty", T=0, H=128, I=64, E=4, k=2, minibatch_rows=16, ring_bytes=1 << 20)
    inp = synth.make_inputs(cfg)
    d = DeviceInputs(inp)
    res = run_layer(d, knobs(cfg))
    assert res["out"].numel() == 0 and res["dx"].numel() == 0
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert not res[n].float().abs().sum().item()


def test_permute_unpermute_identity():
    # identity experts, k = 1, unit gates: out must equal x bit for bit
    cfg = synth.small_config("perm", T=777, H=256, I=64, E=7, k=1, minibatch_rows=32, macrobatch_tokens=200,
                             ring_bytes=3 * 32 * 512, routing="dirichlet")
    inp = synth.make_inputs(cfg)
    inp.topk_w[:] = 1.0
    d = DeviceInputs(inp)
    res = run_layer(d, knobs(cfg, debug_flags=mok.MOK_DEBUG_IDENTITY_EXPERT), backward=False)
    assert torch.equal(res["out"].view(torch.int16), d.x.view(torch.int16))


def test_weighted_identity_rounds_to_nearest_even():
    # identity experts, k = 1, gates in (0, 1): out = bf16(fp32(g) * fp32(x)), one
    # fp32 product rounded to bf16 to nearest even; torch's CPU cast gives the
    # expected bits, so any other rounding of the kernels' bf16 stores shows
    cfg = synth.small_config("perm_w", T=517, H=256, I=64, E=5, k=1, minibatch_rows=32, ring_bytes=3 * 32 * 512,
                             routing="zipf")
    inp = synth.make_inputs(cfg)
    d = DeviceInputs(inp)
    res = run_layer(d, knobs(cfg, debug_flags=mok.MOK_DEBUG_IDENTITY_EXPERT), backward=False)
    g = torch.from_numpy(np.ascontiguousarray(inp.topk_w, dtype=np.float32)).reshape(-1, 1)
    want = (g * d.x.cpu().float()).to(torch.bfloat16)
    got = res["out"].cpu()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    assert not torch.equal(got.view(torch.int16), (g * d.x.cpu().float()).view(torch.int32).bitwise_right_shift(16)
                           .to(torch.int16))   # the products do need rounding (truncation differs)


def test_bitwise_deterministic_ten_runs():
    cfg = SMALL["ragged_k2"]
    d = DeviceInputs(synth.make_inputs(cfg))
    first = run_layer(d, knobs(cfg))
    for _ in range(9):
        same_bits(first, run_layer(d, knobs(cfg)))


# The whole-pass mode was present in both runs that hung without a shown
# cause; the library now rejects it (MOK_ERROR_UNSUPPORTED) and its cases stay
# off the GPU until a cause is shown and fixed.
WHOLE_PASS_OFF = "whole-pass mode switched off: it was present in two hangs whose cause was not shown"


def _knob_sweep(name, overrides):
    cfg = SMALL[name]
    d = DeviceInputs(synth.make_inputs(cfg))
    base = run_layer(d, knobs(cfg))
    row = 2 * cfg.H
    for over in overrides(cfg, row):
        print(f"[layer] knobs {name} {over}", flush=True)
        same_bits(base, run_layer(d, knobs(cfg, **over)))


@pytest.mark.parametrize("name", ["ragged_k2", "k1_macro"])
def test_knobs_do_not_change_bits(name):
    _knob_sweep(name, lambda cfg, row: (
        dict(minibatch_rows=16), dict(minibatch_rows=512, ring_bytes=2 * 512 * row),
        dict(macrobatch_tokens=0), dict(macrobatch_tokens=7), dict(ring_bytes=2 * cfg.minibatch_rows * row),
        dict(ring_bytes=1 << 24), dict(capacity_multiplier=4.0),
        dict(debug_flags=mok.MOK_DEBUG_SEPARATE_LAUNCHES)))


@pytest.mark.parametrize("name", ["ragged_k2", "k1_macro"])
def test_persistent_grid_size_does_not_change_bits(name):
    # race check of the persistent work queues: one workgroup runs every tile
    # in claim order, a few contend for them, more than the compute units
    # queue behind the resident ones; every grid gives the same bits
    _knob_sweep(name, lambda cfg, row: tuple(dict(persistent_workgroups=n) for n in (1, 2, 3, 7, 64, 300, 1024)) +
                (dict(persistent_workgroups=5, ring_bytes=2 * cfg.minibatch_rows * row),))


@pytest.mark.skip(reason=WHOLE_PASS_OFF)
@pytest.mark.parametrize("name", ["ragged_k2", "k1_macro"])
def test_whole_pass_mode_gives_the_same_bits(name):
    _knob_sweep(name, lambda cfg, row: (
        dict(debug_flags=mok.MOK_DEBUG_WHOLE_PASS),
        dict(debug_flags=mok.MOK_DEBUG_WHOLE_PASS, ring_bytes=2 * cfg.minibatch_rows * row)))


@pytest.mark.parametrize("name", ["ragged_k2", "k1_macro"])
def test_autosized_config_gives_the_same_bits(name):
    # the two-wave mini-batch changes no output bit (at these sizes it is one
    # macro-batch's rows; the full-size step compares every point of a sweep)
    cfg = SMALL[name]
    d = DeviceInputs(synth.make_inputs(cfg))
    base = run_layer(d, knobs(cfg))
    for n_cu in (0, 1):
        c = mok.autosize_config(knobs(cfg), cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, n_cu)
        print(f"[layer] autosize {name} n_cu={n_cu} mb={c.minibatch_rows} ring={c.ring_bytes}", flush=True)
        same_bits(base, run_layer(d, c))


def test_status_flags_stop_the_layer():
    cfg = SMALL["tiny"]
    inp = synth.make_inputs(cfg)
    d = DeviceInputs(inp)
    c = knobs(cfg)
    ws = mok.get_workspace(c, device=DEV, num_local_tokens=cfg.T, hidden_size=cfg.H, intermediate_size=cfg.I,
                           num_experts=cfg.E, topk=cfg.k)
    bad = d.ids.clone()
    bad[5, 1] = cfg.E
    sched = mok.build_schedule(ws, bad)
    out = torch.full((cfg.T, cfg.H), 7.0, dtype=torch.bfloat16, device=DEV)
    w = mok.weights_bf16(d.wg, d.wu, d.wd)
    mok.forward(ws, sched, d.x, d.w, w, out=out)
    torch.cuda.synchronize()
    assert status_word(sched) == mok.MOK_BAD_EXPERT_ID
    assert torch.all(out == 7.0)   # no work was done
    # capacity overflow
    ws2 = mok.get_workspace(knobs(cfg, capacity_multiplier=0.05), device=DEV, num_local_tokens=cfg.T,
                            hidden_size=cfg.H, intermediate_size=cfg.I, num_experts=cfg.E, topk=cfg.k)
    sched2 = mok.build_schedule(ws2, d.ids)
    mok.forward(ws2, sched2, d.x, d.w, w, out=out)
    torch.cuda.synchronize()
    assert status_word(sched2) == mok.MOK_SCHEDULE_OVERFLOW
    assert torch.all(out == 7.0)


def test_schedule_built_for_other_knobs_is_refused():
    # a table built under another capacity multiplier (or mini-batch size) has
    # another layout: the readers' fingerprint check flags it before any work
    cfg = SMALL["tiny"]
    d = DeviceInputs(synth.make_inputs(cfg))
    w = mok.weights_bf16(d.wg, d.wu, d.wd)
    big = mok.get_workspace(knobs(cfg, capacity_multiplier=4.0), device=DEV, num_local_tokens=cfg.T,
                            hidden_size=cfg.H, intermediate_size=cfg.I, num_experts=cfg.E, topk=cfg.k)
    sched = mok.build_schedule(big, d.ids)
    torch.cuda.synchronize()
    assert status_word(sched) == 0
    ws = mok.get_workspace(knobs(cfg), device=DEV, num_local_tokens=cfg.T, hidden_size=cfg.H,
                           intermediate_size=cfg.I, num_experts=cfg.E, topk=cfg.k)
    assert ws.schedule_bytes <= sched.numel()
    out = torch.full((cfg.T, cfg.H), 7.0, dtype=torch.bfloat16, device=DEV)
    mok.forward(ws, sched, d.x, d.w, w, out=out)
    torch.cuda.synchronize()
    assert status_word(sched) == mok.MOK_SCHEDULE_MISMATCH
    assert torch.all(out == 7.0)
    # the matching reader runs normally on a fresh table
    sched2 = mok.build_schedule(big, d.ids)
    mok.forward(big, sched2, d.x, d.w, w, out=out)
    torch.cuda.synchronize()
    assert status_word(sched2) == 0 and not torch.all(out == 7.0)


@pytest.mark.parametrize("flags", [0, pytest.param(mok.MOK_DEBUG_WHOLE_PASS, marks=pytest.mark.skip(reason=WHOLE_PASS_OFF))])
def test_forced_stall_ends_the_call(flags):
    # every in-kernel wait gives up at once: the launch must end, flag the
    # stall, and leave the outputs that depend on the waits unwritten
    cfg = SMALL["k1_macro"]
    d = DeviceInputs(synth.make_inputs(cfg))
    w = mok.weights_bf16(d.wg, d.wu, d.wd)
    c = knobs(cfg, debug_flags=flags | mok.MOK_DEBUG_FORCE_STALL)
    ws = mok.get_workspace(c, device=DEV, num_local_tokens=cfg.T, hidden_size=cfg.H, intermediate_size=cfg.I,
                           num_experts=cfg.E, topk=cfg.k)
    sched = mok.build_schedule(ws, d.ids)
    out = torch.full((cfg.T, cfg.H), 7.0, dtype=torch.bfloat16, device=DEV)
    mok.forward(ws, sched, d.x, d.w, w, out=out)
    torch.cuda.synchronize()
    assert status_word(sched) == mok.MOK_SCHEDULER_STALLED
    assert torch.all(out == 7.0)
    # backward after a normal forward: the dgrad waits give up
    ok = knobs(cfg, debug_flags=flags)
    ws2 = mok.get_workspace(ok, device=DEV, num_local_tokens=cfg.T, hidden_size=cfg.H, intermediate_size=cfg.I,
                            num_experts=cfg.E, topk=cfg.k)
    sched2 = mok.build_schedule(ws2, d.ids)
    _, ctx = mok.forward(ws2, sched2, d.x, d.w, w)
    torch.cuda.synchronize()
    assert status_word(sched2) == 0
    ws2.config = c
    grads = mok.backward(ws2, sched2, ctx, d.x, d.w, w, d.dy)
    torch.cuda.synchronize()
    assert status_word(sched2) == mok.MOK_SCHEDULER_STALLED
    del grads


def test_item_trace_records_every_tile_without_changing_bits():
    # the measurement aid: one record per tile of the pair kernels and the
    # weight-gradient kernels, times ordered, outputs unchanged
    cfg = SMALL["k1_macro"]
    d = DeviceInputs(synth.make_inputs(cfg))
    base = run_layer(d, knobs(cfg))
    assert mok.mok_item_trace_enable(1) == mok.MOK_OK
    try:
        traced = run_layer(d, knobs(cfg))
        rec, n = mok.item_trace_read()
    finally:
        mok.mok_item_trace_enable(0)
    same_bits(base, traced)
    assert n == len(rec) > 0
    assert np.all(rec["t_claim"] <= rec["t_start"]) and np.all(rec["t_start"] <= rec["t_kloop"])
    assert np.all(rec["t_kloop"] <= rec["t_end"])
    kinds = set(rec["kernel"].tolist())
    assert {mok.MOK_TRACE_FWD_GEMMS, mok.MOK_TRACE_BWD_GEMMS, mok.MOK_TRACE_WGRAD_GATE_UP,
            mok.MOK_TRACE_WGRAD_DOWN} <= kinds
    # every producer and consumer tile of each pair launch appears exactly once
    for launch in set(rec["launch"][rec["kernel"] <= 1].tolist()):
        r = rec[rec["launch"] == launch]
        for cls in (1, 2):
            items = r["item"][r["item_class"] == cls]
            assert len(items) == len(set(items.tolist())) > 0
    # tracing off again: nothing more is recorded
    run_layer(d, knobs(cfg))
    _, n2 = mok.item_trace_read()
    assert n2 == n
