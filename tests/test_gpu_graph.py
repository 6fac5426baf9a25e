"""The layer under HIP graph capture.

Schedule build, forward and backward are captured once into a graph and
replayed several times, with eager layer calls and synchronizations between
the replays; every replay must give the eager outputs bit for bit. The
backward forks the library's side stream for dW_down (one macro-batch that
fits the ring: the dy rows stay in the ring, which dW_down then reads beside
the dgrad GEMMs); the fork and the join are captured with it. No kernel of
the path records a memset."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_table_amd as mok
import synth
from gpu_support import DEV, DeviceInputs, knobs

pytestmark = pytest.mark.gpu

CASES = {
    # k = 1, 4 mini-batches in a 20-slot ring: dy rows read by dW_down from the ring
    "k1_ring": (synth.small_config("k1_ring", T=520, H=640, I=320, E=2, k=1, minibatch_rows=160,
                                   ring_bytes=1 << 22, routing="zipf"), {}),
    # k = 2, macro-batches and a 3-slot ring: several rounds, staged combines
    "k2_rounds": (synth.small_config("k2_rounds", T=300, H=256, I=192, E=5, k=2, minibatch_rows=48,
                                     macrobatch_tokens=100, ring_bytes=3 * 48 * 512), {}),
    "mx_k1": (synth.small_config("mx_k1", T=520, H=640, I=384, E=2, k=1, minibatch_rows=160,
                                 ring_bytes=1 << 22, routing="zipf", precision="mxfp8"), {}),
    "mx_k2_rounds": (synth.small_config("mx_k2_rounds", T=300, H=256, I=128, E=5, k=2, minibatch_rows=48,
                                        macrobatch_tokens=100, ring_bytes=3 * 48 * 264, precision="mxfp8"), {}),
    # MXFP8 weight gradients: the x and dy quantizers run on the side stream
    "mx_wgrad": (synth.small_config("mx_wgrad", T=520, H=640, I=384, E=2, k=1, minibatch_rows=160,
                                    ring_bytes=1 << 22, routing="zipf", precision="mxfp8"),
                 dict(precision=mok.MOK_MXFP8_WGRAD)),
}


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_give_the_eager_bits(name):
    cfg, over = CASES[name]
    print(f"[graph] {name}", flush=True)
    d = DeviceInputs(synth.make_inputs(cfg))
    config = knobs(cfg, **over)
    ws = mok.get_workspace(config, device=DEV, num_local_tokens=cfg.T, hidden_size=cfg.H,
                           intermediate_size=cfg.I, num_experts=cfg.E, topk=cfg.k)
    if config.precision in (mok.MOK_MXFP8, mok.MOK_MXFP8_WGRAD):
        q = mok.MXFP8Weights(d.wg, d.wu, d.wd)
        wf, wb = q.fwd, q.bwd
    else:
        wf = wb = mok.weights_bf16(d.wg, d.wu, d.wd)

    def layer(sched=None, out=None, ctx=None, grads=None):
        sched = mok.build_schedule(ws, d.ids, sched)
        out, ctx = mok.forward(ws, sched, d.x, d.w, wf, out, ctx)
        grads = mok.backward(ws, sched, ctx, d.x, d.w, wb, d.dy, grads)
        return sched, out, ctx, grads

    # eager reference (also makes the side stream and sets kernel attributes before capture)
    _, out, ctx, grads = layer()
    torch.cuda.synchronize()
    ref = dict(out=out.clone(), **{n: t.clone() for n, t in grads.items()})

    g_sched = torch.empty(max(ws.schedule_bytes, 256), dtype=torch.uint8, device=DEV)
    g_ctx = torch.empty_like(ctx)
    got = {n: torch.empty_like(t) for n, t in ref.items()}
    g_grads = {n: got[n] for n in grads}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(g_sched, got["out"], g_ctx, g_grads)

    for rep in range(3):
        for t in got.values():
            t.zero_()
        g_ctx.zero_()
        torch.cuda.synchronize()
        layer()   # eager work through the same workspace between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(g_sched[:4].cpu().numpy().view(np.uint32)[0]) == 0, (name, rep)
        for n, t in ref.items():
            assert torch.equal(_bits(got[n]), _bits(t)), (name, rep, n)
