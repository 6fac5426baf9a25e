"""bench.py's item-trace summary on hand-made records: each workgroup's span
splits into claim/wait, K loop, epilogue and idle time, as worked out here."""
import numpy as np
import pytest

import bench
import synth

DT = np.dtype([("t_claim", "<u8"), ("t_start", "<u8"), ("t_kloop", "<u8"), ("t_end", "<u8"), ("launch", "<u4"),
               ("kernel", "u1"), ("item_class", "u1"), ("xcd", "<u2"), ("item", "<u4"), ("workgroup", "<u4")])


def test_shares_and_per_item_times_by_hand():
    # one launch of the forward pair kernel, two workgroups, times in 10 ns ticks
    rec = np.array([
        (0, 10, 60, 70, 0, 0, 1, 0, 0, 0),      # wg 0: claim 10, K loop 50, epilogue 10
        (70, 80, 90, 100, 0, 0, 2, 0, 0, 0),    # wg 0: claim 10, K loop 10, epilogue 10
        (20, 20, 80, 90, 0, 0, 1, 1, 1, 1),     # wg 1 starts at 20: idle 20; ends at 90: idle 10
    ], dtype=DT)
    cfg = synth.small_config("t", T=64, H=128, I=64, E=2, k=1)
    s = bench.item_trace_summary(rec, cfg)["fwd_gemms"]
    sh = s["shares"]
    span = 100 * 2                                # launch span 0..100 ticks, two workgroups
    assert sh["claim"] == pytest.approx((10 + 10 + 0) / span)
    assert sh["kloop"] == pytest.approx((50 + 10 + 60) / span)
    assert sh["epilogue"] == pytest.approx((10 + 10 + 10) / span)
    assert sh["idle_start"] == pytest.approx(20 / span)
    assert sh["idle_end"] == pytest.approx(10 / span)
    assert sum(sh[k] for k in ("claim", "kloop", "epilogue", "idle_start", "idle_end")) == pytest.approx(1.0)
    assert sh["span_us"] == pytest.approx(1.0) and sh["workgroups"] == 2
    c1 = s["classes"][1]                          # producer tiles: K loops of 50 and 60 ticks
    assert c1["items_per_launch"] == 2 and c1["kloop_us"] == pytest.approx(0.55)
    assert c1["us_per_kstep"] == pytest.approx(0.55 / (128 // 32), abs=1e-3)
    assert s["classes"][2]["us_per_kstep"] == pytest.approx(0.10 / (64 // 32), abs=1e-3)


def test_ticket_taken_during_the_previous_epilogue_counts_from_its_end():
    # wg 0 takes its second item's ticket at 65, inside its first item's
    # epilogue (60..70); the claim time of that item counts from 70
    rec = np.array([
        (0, 10, 60, 70, 0, 0, 1, 0, 0, 0),
        (65, 80, 90, 100, 0, 0, 2, 0, 0, 0),
    ], dtype=DT)
    cfg = synth.small_config("t", T=64, H=128, I=64, E=2, k=1)
    s = bench.item_trace_summary(rec, cfg)["fwd_gemms"]
    sh = s["shares"]
    assert sh["claim"] == pytest.approx((10 + 10) / 100)
    assert sum(sh[k] for k in ("claim", "kloop", "epilogue", "idle_start", "idle_end")) == pytest.approx(1.0)
    assert s["classes"][2]["claim_us"] == pytest.approx(0.10)
