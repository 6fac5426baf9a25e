"""Router front-end on the GPU against the router oracle: ids bit-exact, weights
and logit gradients within the fp32 bound, ties, edge shapes, determinism, and
the route -> schedule hand-off."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_table_amd as mok
import synth
from gpu_support import DEV
from oracle import router as R
from oracle import schedule as S

pytestmark = pytest.mark.gpu

# fp32 exp, sum and divide: at most k + 3 roundings of relative size 2^-24 on
# values in (0, 1], so |w_gpu - w| <= (64 + 3) * 2^-24 < 4e-6 for k <= 64
TOL_W = 4e-6


def _logits(T, E, seed):
    return synth.draw_logits(np.random.default_rng(seed), T, E)   # N(0,1) fp32, no ties


SHAPES = [(64, 8, 2), (2048, 256, 8), (1000, 512, 10), (300, 1000, 64), (5, 3, 3), (17, 64, 1), (9, 1, 1),
          (130, 65, 7)]


@pytest.mark.parametrize("T,E,k", SHAPES)
def test_route_matches_oracle(T, E, k):
    print(f"[router] forward T={T} E={E} k={k}", flush=True)
    l = _logits(T, E, T + 31 * E + k)
    ids, w = mok.route(torch.from_numpy(l).to(DEV), k)
    torch.cuda.synchronize()
    rid, rw = R.route(l, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy().astype(np.float64) - rw).max() <= TOL_W


def test_route_ties_take_the_lower_index():
    l = np.array([[1, 3, 3, 0, 2, 3, 3, 3],
                  [0, 0, 0, 0, 0, 0, 0, 0],
                  [5, -1, 5, -1, 5, -1, 5, -1]], np.float32)
    ids, w = mok.route(torch.from_numpy(l).to(DEV), 4)
    rid, rw = R.route(l, 4)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy() - rw).max() <= TOL_W


@pytest.mark.parametrize("T,E,k", SHAPES)
def test_route_backward_matches_oracle(T, E, k):
    print(f"[router] backward T={T} E={E} k={k}", flush=True)
    l = _logits(T, E, 7 * T + E + k)
    dw = np.random.default_rng(T + k).standard_normal((T, k)).astype(np.float32)
    ids, w = mok.route(torch.from_numpy(l).to(DEV), k)
    dl = mok.route_backward(ids, w, torch.from_numpy(dw).to(DEV), E)
    torch.cuda.synchronize()
    ref = R.route_backward(l, ids.cpu().numpy(), dw)
    # w within TOL_W and fp32 sums of k products: about (k + 3) * 2^-24 * |dw| more
    tol = 2 * TOL_W * max(1.0, float(np.abs(dw).max()))
    got = dl.cpu().numpy()
    assert np.abs(got - ref).max() <= tol
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, ids.cpu().numpy().astype(np.int64), True, axis=1)
    assert np.all(got[~mask] == 0)          # written exactly, every entry


def test_route_is_bitwise_deterministic():
    l = torch.from_numpy(_logits(4096, 256, 5)).to(DEV)
    ids0, w0 = mok.route(l, 8)
    dw = torch.randn(4096, 8, device=DEV, generator=torch.Generator(DEV).manual_seed(3))
    g0 = mok.route_backward(ids0, w0, dw, 256)
    for _ in range(3):
        ids, w = mok.route(l, 8)
        assert torch.equal(ids, ids0) and torch.equal(w.view(torch.int32), w0.view(torch.int32))
        assert torch.equal(mok.route_backward(ids, w, dw, 256).view(torch.int32), g0.view(torch.int32))


def test_route_feeds_the_schedule():
    # the device route's ids drive the device schedule builder to the oracle's schedule
    T, E, k = 2048, 256, 8
    l = _logits(T, E, 11)
    ids, _ = mok.route(torch.from_numpy(l).to(DEV), k)
    cfg = mok.MoKConfig(minibatch_rows=512, macrobatch_tokens=0, ring_bytes=1 << 28, capacity_multiplier=1.0,
                        precision=mok.MOK_BF16)
    ws = mok.get_workspace(cfg, device=DEV, num_local_tokens=T, hidden_size=128, intermediate_size=64,
                           num_experts=E, topk=k)
    sched = mok.build_schedule(ws, ids)
    got = mok.read_schedule(sched, mok.schedule_layout(cfg, T, 128, 64, E, k), E)
    ref = S.build(R.route(l, k)[0], E, 512, 0)
    assert got["status"] == 0
    assert np.array_equal(got["counts"], ref.counts) and np.array_equal(got["perm"], ref.perm)


def test_route_time_at_the_full_layer_shape():
    # measurement: 2,048 tokens x 256 experts, top-8 (one GPU before routing), and 8x that
    for T in (2048, 16384):
        l = torch.from_numpy(_logits(T, 256, 13)).to(DEV)
        mok.route(l, 8)
        torch.cuda.synchronize()
        mok._check(mok.mok_kernel_timing_enable(1), "timing")
        for _ in range(20):
            ids, w = mok.route(l, 8)
            mok.route_backward(ids, w, w, 256)
        t = mok.kernel_times()
        f = t["route"][1] / t["route"][0]
        b = t["route_backward"][1] / t["route_backward"][0]
        fwd_bytes, bwd_bytes = T * 256 * 4 + T * 8 * 8, T * 8 * 12 + T * 256 * 4
        print(f"[router] T={T}: route {1e3 * f:.1f} us ({fwd_bytes / (f * 1e6):.0f} GB/s), "
              f"backward {1e3 * b:.1f} us ({bwd_bytes / (b * 1e6):.0f} GB/s)", flush=True)
