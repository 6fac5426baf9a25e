"""O1 — the schedule table, written from its definition (test infrastructure only).

What the pages fix:
* "Mixture-of-Kittens (MoK)" project summary, Functional API: schedule building
  takes the caller's top-k expert ids; Key-concepts table: the config carries a
  mini-batch granularity, a macro-batch size and a schedule capacity multiplier.
* "Mixture-of-Kittens(MoK)란?" explainer, section 4 ①: a single schedule table
  drives dispatch and combine, forward and backward.
* same page, section 4 ③: no token is ever dropped; rows move through a fixed
  ring buffer in mini-batches; macro-batches bound dispatch/combine.

Readings where the pages are silent (each listed in the design notes):
* processing order q sorts routed rows f = t*k + j by (macro-batch, expert, f);
* macro-batch m covers tokens [m*MT, min(T, (m+1)*MT)); MT = 0 means one;
* mini-batch (m, b) covers processing positions [base_m + b*MB, base_m + min(R_m, (b+1)*MB));
  its global index g counts mini-batches of earlier macro-batches first;
* segments are the non-empty intersections of a mini-batch with an expert's
  rows, listed by g then expert;
* capacity = ceil(multiplier * W) with W = sum_m (ceil(R_m/MB) + min(E, R_m) - 1),
  the largest number of segments any routing can produce; more segments than
  capacity sets SCHEDULE_OVERFLOW (nothing is dropped silently);
* an expert id outside [0, E) sets BAD_EXPERT_ID and nothing else is defined.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SCHEDULE_OVERFLOW = 1
BAD_EXPERT_ID = 2


@dataclasses.dataclass
class Schedule:
    status: int
    counts: np.ndarray      # [E] rows per expert
    offsets: np.ndarray     # [E+1] exclusive scan of counts
    mcounts: np.ndarray     # [NM, E] rows per (macro-batch, expert)
    moffsets: np.ndarray    # [NM, E+1] first processing position of (m, e)
    perm: np.ndarray        # [R] processing position -> routed row f
    inv: np.ndarray         # [R] routed row f -> processing position
    canon: np.ndarray       # [R] canonical position (sorted by (e, f)) -> processing position
    mb_start: np.ndarray    # [G+1] first processing position of each mini-batch
    mb_macro: np.ndarray    # [G] macro-batch of each mini-batch
    segments: np.ndarray    # [min(n_seg, cap), 4] (g, e, q0, len)
    n_seg: int
    cap: int
    G: int
    NM: int


def macro_batches(T: int, k: int, MT: int):
    """(token_start, token_end, row_base) for each macro-batch."""
    if T == 0:
        return []
    mt = T if MT <= 0 else MT
    return [(t0, min(T, t0 + mt), k * t0) for t0 in range(0, T, mt)]


def worst_case_segments(T: int, k: int, E: int, MB: int, MT: int) -> int:
    W = 0
    for t0, t1, _ in macro_batches(T, k, MT):
        Rm = k * (t1 - t0)
        W += -(-Rm // MB) + min(E, Rm) - 1
    return W


def capacity(T: int, k: int, E: int, MB: int, MT: int, multiplier: float) -> int:
    W = worst_case_segments(T, k, E, MB, MT)
    # the multiplier is an fp32 knob; the product is taken in fp64
    return int(math.ceil(float(np.float32(multiplier)) * W))


def build(topk_ids: np.ndarray, E: int, MB: int, MT: int = 0,
          capacity_multiplier: float = 1.0) -> Schedule:
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    R = T * k
    flat = ids.reshape(R)
    macros = macro_batches(T, k, MT)
    NM = len(macros)
    cap = capacity(T, k, E, MB, MT, capacity_multiplier)
    if R and (flat.min() < 0 or flat.max() >= E):
        z = np.zeros(0, np.int64)
        return Schedule(BAD_EXPERT_ID, z, z, z, z, z, z, z, z, z, np.zeros((0, 4), np.int64),
                        0, cap, 0, NM)

    counts = np.bincount(flat, minlength=E).astype(np.int64)
    assert counts.sum() == R  # drop-free: every routed row is scheduled
    offsets = np.concatenate([[0], np.cumsum(counts)])

    f = np.arange(R, dtype=np.int64)
    mt = T if MT <= 0 else MT
    macro_of_f = (f // k) // mt if R else f
    # processing order: stable sort by (macro-batch, expert, f)
    perm = np.lexsort((f, flat, macro_of_f)) if R else f
    inv = np.empty(R, dtype=np.int64)
    inv[perm] = f
    canon_f = np.lexsort((f, flat)) if R else f   # canonical order: (expert, f)
    canon = inv[canon_f]

    mcounts = np.zeros((NM, E), dtype=np.int64)
    moffsets = np.zeros((NM, E + 1), dtype=np.int64)
    mb_start, mb_macro = [], []
    for m, (t0, t1, base) in enumerate(macros):
        rows = flat[base: k * t1]
        mcounts[m] = np.bincount(rows, minlength=E)
        moffsets[m] = base + np.concatenate([[0], np.cumsum(mcounts[m])])
        Rm = k * (t1 - t0)
        for b in range(-(-Rm // MB)):
            mb_start.append(base + b * MB)
            mb_macro.append(m)
    G = len(mb_start)
    mb_start.append(R)
    mb_start = np.asarray(mb_start, dtype=np.int64)
    mb_macro = np.asarray(mb_macro, dtype=np.int64)

    segs = []
    for g in range(G):
        m = mb_macro[g]
        lo, hi = mb_start[g], mb_start[g + 1]
        for e in range(E):
            a = max(lo, moffsets[m, e])
            b = min(hi, moffsets[m, e + 1])
            if b > a:
                segs.append((g, e, a, b - a))
    n_seg = len(segs)
    status = SCHEDULE_OVERFLOW if n_seg > cap else 0
    segments = np.asarray(segs[:cap], dtype=np.int64).reshape(-1, 4)
    return Schedule(status, counts, offsets, mcounts, moffsets, perm, inv, canon, mb_start,
                    mb_macro, segments, n_seg, cap, G, NM)


def ring_slots(ring_bytes: int, MB: int, row_bytes: int) -> int:
    """Number of whole mini-batch slots a ring of ``ring_bytes`` holds."""
    return ring_bytes // (MB * row_bytes)


def two_wave_min_rows(n_units: int, tile_m: int, tile_n: int, I: int) -> int:
    """Fewest routed rows whose gate/up grouped GEMM fills two full waves.

    "Mixture-of-Kittens(MoK)란?" explainer, section 4 ②: the overlap unit is
    sized so that each expert-grouped GEMM runs at least two full waves of the
    GPU's compute units. The gate/up GEMM of r rows has N = 2I output columns,
    so it holds r*2I / (tile_m*tile_n) output tiles counted fractionally; two
    waves over n_units units need r >= 2*n_units*tile_m*tile_n / (2I).
    Reading: tiles are counted fractionally (the pages' worked example, 2,368
    tokens for the Kimi 2.5 shape, is 2 * 148 * 128*256 / 4096 exactly).
    """
    return -(-(2 * n_units * tile_m * tile_n) // (2 * I))


def autosize_minibatch(T: int, k: int, I: int, MT: int, n_units: int, tile_m: int,
                       tile_n: int) -> int:
    """Mini-batch rows under the two-wave rule, in whole m-tiles.

    Reading (the pages give the minimum, not the rounding): m-tiles are cut at
    mini-batch boundaries, so the two-wave minimum is rounded up to a whole
    number of tile_m-row tiles; a mini-batch never holds more rows than one
    macro-batch routes (k * MT, MT = 0 meaning all T tokens), rounded up to the
    16-row granule of the mini-batch size, and is at least 16 rows.
    """
    rows = two_wave_min_rows(n_units, tile_m, tile_n, I)
    mb = -(-rows // tile_m) * tile_m
    mt = T if (MT == 0 or MT >= T) else MT
    cap = -(-(k * max(mt, 1)) // 16) * 16
    return max(16, min(mb, cap))
