"""mok_forward_noalloc, the forward pass with the library's static scratch
instead of a workspace argument, against mok_forward on the same inputs: two
calls in a row (the second with a smaller input, so that it runs over what the
first left in the shared scratch), then an MXFP8 call; every output bit equal."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_table_amd as mok
import synth
from gpu_support import DEV, DeviceInputs, knobs, status_word

pytestmark = pytest.mark.gpu

CASES = [
    synth.small_config("noalloc_k2", T=300, H=256, I=192, E=5, k=2, minibatch_rows=48, macrobatch_tokens=100,
                       ring_bytes=3 * 48 * 512),
    synth.small_config("noalloc_k1_smaller", T=130, H=256, I=192, E=3, k=1, minibatch_rows=32,
                       ring_bytes=2 * 32 * 512, routing="zipf", seed=3),
    synth.small_config("noalloc_mxfp8", T=200, H=256, I=128, E=4, k=2, minibatch_rows=32,
                       ring_bytes=1 << 20, precision="mxfp8", seed=5),
]


def _forward_both(cfg):
    print(f"[noalloc] {cfg.name}", flush=True)
    d = DeviceInputs(synth.make_inputs(cfg))
    c = knobs(cfg)
    ws = mok.get_workspace(c, device=DEV, num_local_tokens=cfg.T, hidden_size=cfg.H, intermediate_size=cfg.I,
                           num_experts=cfg.E, topk=cfg.k)
    sched = mok.build_schedule(ws, d.ids)
    if cfg.precision == "mxfp8":
        w = mok.MXFP8Weights(d.wg, d.wu, d.wd).fwd
    else:
        w = mok.weights_bf16(d.wg, d.wu, d.wd)
    ref_out, ref_ctx = mok.forward(ws, sched, d.x, d.w, w)
    out = torch.full_like(ref_out, 7.0)
    ctx = torch.zeros_like(ref_ctx)
    mok.forward_noalloc(ws, sched, d.x, d.w, w, out, ctx)
    torch.cuda.synchronize()
    assert status_word(sched) == 0
    h_bytes = cfg.R * 2 * cfg.I * 2
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(ctx[:h_bytes], ref_ctx[:h_bytes])
    assert out.float().abs().sum().item() > 0


def test_noalloc_forward_matches_forward_call_after_call():
    for cfg in CASES:
        _forward_both(cfg)


def test_noalloc_rejects_a_forward_beyond_its_scratch():
    # the EP-64 share with its 256 MiB ring needs more scratch than the array
    cfg = synth.CONFIGS["ep64_share"]
    c = knobs(cfg).c()
    sh = mok.mok_shape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    p = torch.zeros(256, dtype=torch.uint8, device=DEV)
    w = mok.mok_weights(p.data_ptr(), p.data_ptr(), p.data_ptr())
    st = mok.mok_forward_noalloc(c, sh, p.data_ptr(), 1 << 40, p.data_ptr(), p.data_ptr(), w, p.data_ptr(),
                                 p.data_ptr(), 1 << 40, None)
    assert st == mok.MOK_ERROR_BUFFER_TOO_SMALL
    assert "scratch" in mok.mok_last_error()
    # a 4-slot ring of the same layer fits, and gives mok_forward's bits
    small = dict(ring_bytes=4 * cfg.minibatch_rows * 2 * cfg.H)
    print("[noalloc] ep64_share, 4-slot ring", flush=True)
    inp = synth.make_inputs(cfg)
    d = DeviceInputs(inp)
    ws = mok.get_workspace(knobs(cfg, **small), device=DEV, num_local_tokens=cfg.T, hidden_size=cfg.H,
                           intermediate_size=cfg.I, num_experts=cfg.E, topk=cfg.k)
    sched = mok.build_schedule(ws, d.ids)
    wts = mok.weights_bf16(d.wg, d.wu, d.wd)
    ref_out, ref_ctx = mok.forward(ws, sched, d.x, d.w, wts)
    out, ctx = torch.empty_like(ref_out), torch.empty_like(ref_ctx)
    mok.forward_noalloc(ws, sched, d.x, d.w, wts, out, ctx)
    torch.cuda.synchronize()
    assert status_word(sched) == 0
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(ctx, ref_ctx)
