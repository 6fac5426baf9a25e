"""Pins for the schedule oracle (O1): a hand-worked table, brute force on random
tiny routings, and invariants on the named workloads."""
import itertools
import os

import numpy as np
import pytest

import synth
from oracle import schedule as S


def _read_golden(path):
    d = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        d[key] = [int(v) for v in vals]
    return d


def test_hand_worked_table(golden_dir):
    g = _read_golden(os.path.join(golden_dir, "schedule_hand_worked.txt"))
    T, k, E, MB, MT = g["T"][0], g["k"][0], g["E"][0], g["MB"][0], g["MT"][0]
    ids = np.array(g["ids"]).reshape(T, k)
    s = S.build(ids, E, MB, MT, 1.0)
    assert s.status == 0
    assert s.counts.tolist() == g["counts"]
    assert s.offsets.tolist() == g["offsets"]
    assert s.mcounts.ravel().tolist() == g["mcounts"]
    assert s.moffsets.ravel().tolist() == g["moffsets"]
    assert s.perm.tolist() == g["perm"]
    assert s.inv.tolist() == g["inv"]
    assert s.canon.tolist() == g["canon"]
    assert s.mb_start.tolist() == g["mb_start"]
    assert s.segments.ravel().tolist() == g["segments"]
    assert s.n_seg == g["n_seg"][0]
    assert s.cap == g["cap_at_1.0"][0]
    s2 = S.build(ids, E, MB, MT, 0.5)
    assert s2.cap == g["cap_at_0.5"][0]
    assert s2.status == S.SCHEDULE_OVERFLOW
    assert s2.n_seg == g["n_seg"][0]
    assert s2.segments.ravel().tolist() == g["segments"][:4 * 4]


def _brute(ids, E, MB, MT):
    """Pure-Python restatement: sort routed rows with a key tuple, walk the order."""
    T, k = ids.shape
    mt = T if MT <= 0 else MT
    rows = [(t * k + j) for t in range(T) for j in range(k)]
    key = lambda f: ((f // k) // mt, int(ids[f // k, f % k]), f)
    order = sorted(rows, key=key)
    # mini-batches: restart at each macro-batch, MB positions each
    segs, g = [], -1
    pos_in_macro, cur_macro = 0, -1
    prev = None
    for q, f in enumerate(order):
        m, e, _ = key(f)
        if m != cur_macro:
            cur_macro, pos_in_macro = m, 0
        if pos_in_macro % MB == 0:
            g += 1
        pos_in_macro += 1
        if prev == (g, e):
            segs[-1][3] += 1
        else:
            segs.append([g, e, q, 1])
            prev = (g, e)
    return order, segs


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_random(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(0, 40))
    E = int(rng.integers(1, 9))
    k = int(rng.integers(1, E + 1))
    MB = int(rng.integers(1, 12))
    MT = int(rng.integers(0, 12))
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).reshape(T, k) \
        if T else np.zeros((0, k), np.int64)
    s = S.build(ids, E, MB, MT, 4.0)
    order, segs = _brute(ids, E, MB, MT)
    R = T * k
    assert s.perm.tolist() == order
    assert s.inv[s.perm].tolist() == list(range(R))
    assert s.segments.tolist() == segs
    assert s.n_seg == len(segs) <= S.worst_case_segments(T, k, E, MB, MT)
    assert s.status == 0
    # drop-free and exact tiling of [0, R)
    assert int(s.counts.sum()) == R
    if segs:
        assert segs[0][2] == 0 and sum(x[3] for x in segs) == R
        for a, b in zip(segs, segs[1:]):
            assert b[2] == a[2] + a[3]
    # canonical order lists each expert's rows by routed-row index
    f_of_c = s.perm[s.canon]
    flat = ids.reshape(-1)
    assert sorted(f_of_c.tolist(), key=lambda f: (flat[f], f)) == f_of_c.tolist()


def test_worst_case_is_reached():
    # Every mini-batch boundary and every expert boundary cut apart: W is attained.
    T, k, E, MB = 12, 1, 4, 5
    ids = np.repeat(np.arange(E), 3).reshape(T, 1)
    s = S.build(ids, E, MB, 0, 1.0)
    assert s.n_seg == S.worst_case_segments(T, k, E, MB, 0) == 3 + 4 - 1


def test_bad_expert_id_flag():
    ids = np.array([[0, 1], [2, 5]])
    assert S.build(ids, 4, 2, 0, 1.0).status == S.BAD_EXPERT_ID
    assert S.build(np.array([[-1]]), 4, 2, 0, 1.0).status == S.BAD_EXPERT_ID


@pytest.mark.parametrize("name", ["tiny", "full_layer", "ep64_share", "stream"])
def test_named_workloads_invariants(name):
    cfg = synth.CONFIGS[name]
    ids, _, _ = synth.make_routing(cfg)
    s = S.build(ids, cfg.E, cfg.minibatch_rows, cfg.macrobatch_tokens, 1.0)
    R = cfg.R
    assert s.status == 0
    assert int(s.counts.sum()) == R
    assert np.array_equal(np.sort(s.perm), np.arange(R))
    assert np.array_equal(s.inv[s.perm], np.arange(R))
    flat = ids.reshape(-1)
    # within processing order: macro-batch, then expert, then f ascending
    f = s.perm
    key = ((f // cfg.k) // (cfg.macrobatch_tokens or cfg.T)) * (cfg.E * R) + flat[f] * R + f
    assert np.all(np.diff(key) > 0)
    assert int(s.segments[:, 3].sum()) == R
    assert s.n_seg <= s.cap
    if name == "ep64_share":
        assert s.counts.tolist() == [8658, 3769, 2317, 1640]
        assert s.G == 32 and s.n_seg <= 35
    if name == "stream":
        assert s.NM == 8 and s.G == 320


def _read_two_wave(path):
    rows = []
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(tuple(int(v) for v in line.split()))
    return rows


def test_two_wave_rule_worked_example(golden_dir):
    for units, tm, tn, I, rows in _read_two_wave(os.path.join(golden_dir, "two_wave_rule.txt")):
        assert S.two_wave_min_rows(units, tm, tn, I) == rows


@pytest.mark.parametrize("units,tm,tn,I", [(1, 16, 16, 64), (3, 32, 64, 96), (7, 128, 256, 320),
                                           (256, 256, 256, 1024), (5, 48, 80, 2048)])
def test_two_wave_rule_is_the_least_row_count(units, tm, tn, I):
    # brute force: the fewest rows r with r*2I/(tm*tn) >= 2*units output tiles
    r = 0
    while r * 2 * I < 2 * units * tm * tn:
        r += 1
    assert S.two_wave_min_rows(units, tm, tn, I) == r


@pytest.mark.parametrize("T,k,I,MT,units,tm", [(16384, 1, 2048, 0, 256, 256), (2048, 8, 2048, 0, 256, 128),
                                                (163840, 1, 1024, 20480, 256, 256), (64, 2, 64, 0, 256, 128),
                                                (1000, 3, 512, 100, 8, 256), (0, 1, 64, 0, 256, 256)])
def test_autosize_minibatch_by_enumeration(T, k, I, MT, units, tm):
    mb = S.autosize_minibatch(T, k, I, MT, units, tm, 256)
    mt = T if (MT == 0 or MT >= T) else MT
    macro_rows = k * max(mt, 1)
    # the smallest whole number of m-tiles that reaches two waves, unless one macro-batch is smaller
    n = 1
    while n * tm * 2 * I < 2 * units * tm * 256:
        n += 1
    want = n * tm if n * tm <= macro_rows else -(-macro_rows // 16) * 16
    assert mb == max(16, want) and mb % 16 == 0


@pytest.mark.parametrize("T,k,E,I,units,tm", [(16384, 1, 1, 2048, 256, 256), (16384, 1, 4, 2048, 256, 256),
                                              (4096, 8, 1, 2048, 256, 128), (20480, 1, 8, 1024, 256, 256),
                                              (2000, 2, 3, 512, 8, 128)])
def test_autosize_minibatch_fills_two_waves_of_the_schedules_own_tiles(T, k, E, I, units, tm):
    """The auto-sized mini-batch, counted through the schedule oracle's own
    segments (not the closed form): every full mini-batch's gate/up GEMM has at
    least two waves of output tiles (explainer 4 ②); with one expert, one m-tile
    fewer would not (the size is the least such whole number of m-tiles)."""
    tn = 256
    rng = np.random.default_rng(T + k + E)
    ids = np.stack([rng.permutation(E)[:k] if k <= E else rng.integers(0, E, k) for _ in range(T)]) \
        if E > 1 else np.zeros((T, k), np.int64)
    mb = S.autosize_minibatch(T, k, I, 0, units, tm, tn)
    s = S.build(ids, E, mb, 0)
    n_tiles_n = -(-2 * I // tn)
    full = [g for g in range(s.G) if s.mb_start[g + 1] - s.mb_start[g] == mb]
    assert full, "no full mini-batch"
    for g in full:
        segs = s.segments[s.segments[:, 0] == g]
        tiles = sum(-(-int(length) // tm) for length in segs[:, 3]) * n_tiles_n
        assert tiles >= 2 * units, (g, tiles)
    if E == 1 and mb > tm:
        fewer = S.build(ids, E, mb - tm, 0)
        segs = fewer.segments[fewer.segments[:, 0] == 0]
        assert sum(-(-int(length) // tm) for length in segs[:, 3]) * n_tiles_n < 2 * units
