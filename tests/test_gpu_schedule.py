"""Schedule table on the GPU equals the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_table_amd as mok
import synth
from oracle import schedule as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(ids: np.ndarray, E, MB, MT, cm=1.0, H=128, I=64, ring_bytes=1 << 22):
    T, k = ids.shape
    c = mok.MoKConfig(minibatch_rows=MB, macrobatch_tokens=MT, ring_bytes=ring_bytes, capacity_multiplier=cm)
    ws = mok.get_workspace(c, device=DEV, num_local_tokens=T, hidden_size=H, intermediate_size=I,
                           num_experts=E, topk=k)
    d_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(DEV)
    sched = mok.build_schedule(ws, d_ids)
    lay = mok.schedule_layout(c, T, H, I, E, k)
    return mok.read_schedule(sched, lay, E)


def _check(ids, E, MB, MT, cm=1.0, **kw):
    got = _run(ids, E, MB, MT, cm, **kw)
    ref = S.build(ids, E, MB, MT, cm)
    assert got["status"] == ref.status
    if ref.status & S.BAD_EXPERT_ID:
        return got, ref
    assert got["n_seg"] == ref.n_seg
    assert np.array_equal(got["segments"], ref.segments)
    if ref.status:
        return got, ref
    for f in ("counts", "offsets", "mcounts", "moffsets", "perm", "inv", "canon", "mb_start"):
        assert np.array_equal(got[f], getattr(ref, f)), f
    return got, ref


@pytest.mark.parametrize("name", ["tiny", "full_layer", "ep64_share", "stream"])
def test_named_workloads(name):
    cfg = synth.CONFIGS[name]
    ids, _, _ = synth.make_routing(cfg)
    print(f"[schedule] {name} T={cfg.T} k={cfg.k} E={cfg.E}", flush=True)
    _check(ids, cfg.E, cfg.minibatch_rows, cfg.macrobatch_tokens, H=cfg.H, I=cfg.I, ring_bytes=cfg.ring_bytes)


@pytest.mark.parametrize("seed", range(12))
def test_random_small(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 3000))
    E = int(rng.integers(1, 40))
    k = int(rng.integers(1, min(E, 8) + 1))
    MB = 16 * int(rng.integers(1, 20))
    MT = int(rng.choice([0, int(rng.integers(1, T + 1))]))
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    print(f"[schedule] random seed={seed} T={T} E={E} k={k} MB={MB} MT={MT}", flush=True)
    _check(ids, E, MB, MT)


def test_skewed_and_empty_experts():
    rng = np.random.default_rng(7)
    ids = rng.choice([0, 3], size=(2500, 1), p=[0.9, 0.1]).astype(np.int32)   # experts 1, 2, 4.. empty
    _check(ids, 9, 64, 700)


def test_empty_call():
    got = _run(np.zeros((0, 2), np.int32), 8, 32, 0)
    assert got["status"] == 0 and got["n_seg"] == 0
    assert not got["counts"].any() and not got["offsets"].any()


def test_capacity_overflow_flag():
    ids = np.repeat(np.arange(8, dtype=np.int32), 40).reshape(-1, 1)   # 8 experts, 40 rows each
    got, ref = _check(ids, 8, 48, 0, cm=0.25)
    assert ref.status == S.SCHEDULE_OVERFLOW and got["status"] == mok.MOK_SCHEDULE_OVERFLOW


def test_bad_expert_id_flag():
    ids = np.array([[0, 1], [2, 8], [3, 4]], np.int32)
    got, _ = _check(ids, 8, 16, 0)
    assert got["status"] == mok.MOK_BAD_EXPERT_ID
    got, _ = _check(np.array([[-1]], np.int32), 8, 16, 0)
    assert got["status"] == mok.MOK_BAD_EXPERT_ID
