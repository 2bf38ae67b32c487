"""bench.py's timeline summary on hand-made rows (CPU only): units, first
steps, step intervals, restarts, ends and dispatch slots come out as the
rows say."""

import numpy as np

import bench

W = 64


def _row(events, end):
    r = np.zeros(W, dtype=np.int64)
    for i, (typ, t) in enumerate(events):
        r[i] = (t << 4) | typ
    r[W - 1] = (end << 4) | 7
    return r


def test_timeline_stats_tile_units():
    # 3 workgroups of 2 waves on 1 compute unit (dispatch slots 0, 1, 2);
    # a counter of 1000 kHz: one tick per us
    info = {"wallclock_khz": 1000, "waves_per_group": 2, "packed": 0, "compute_units": 1}
    rows = [
        _row([(1, 100), (2, 101), (3, 102), (4, 105), (4, 107), (4, 109), (5, 110), (3, 111), (4, 115),
              (4, 116), (5, 118)], 120),
        _row([(1, 100), (2, 101)], 121),  # wave 1 of workgroup 0: not a unit of its own
        _row([(1, 103), (2, 104), (3, 104), (4, 110), (4, 113), (5, 114)], 130),
        np.zeros(W, dtype=np.int64),  # a wave that never ran
        _row([(1, 105), (2, 106), (3, 107), (4, 120), (4, 124), (5, 125)], 140),
        np.zeros(W, dtype=np.int64),
    ]
    st = bench.timeline_stats(np.stack(rows), info)
    assert st["units"] == 3 and st["units_with_chunks"] == 3
    assert st["span_us"] == 40.0
    assert st["first_step_us"]["median"] == 10.0  # first steps at 5, 10, 20
    # step gaps: unit 0 pieces (2, 2) and (1) -> median 2; unit 1 (3) -> 3; unit 2 (4) -> 4
    assert st["step_interval_us"]["median"] == 3.0
    assert st["restart_us"]["count"] == 1 and st["restart_us"]["median"] == 115 - 110
    assert st["end_us"]["min"] == 20.0 and st["end_us"]["max"] == 40.0
    assert [st["by_slot"][k]["units"] for k in ("0", "1", "2")] == [1, 1, 1]
    # start split, medians over the three units: entries 0, 3, 5; schedule 1, 1, 1;
    # set-up 1, 0, 1; first data 3, 6, 13
    assert st["start_split_us"]["entry"] == 3.0 and st["start_split_us"]["setup"] == 1.0
    assert st["start_split_us"]["first_data"] == 6.0
    assert abs(st["end_corr"]["dispatch_slot"] - 1.0) < 1e-12


def test_timeline_stats_packed_waves_are_units():
    info = {"wallclock_khz": 1000, "waves_per_group": 4, "packed": 2, "compute_units": 256}
    rows = [_row([(1, 0), (2, 1), (3, 1), (4, 3 + i), (5, 9)], 10 + i) for i in range(4)]
    st = bench.timeline_stats(np.stack(rows), info)
    assert st["units"] == 4
    assert st["first_step_us"]["p10"] >= 3 and st["first_step_us"]["p90"] <= 6
    assert abs(st["end_corr"]["first_step"] - 1.0) < 1e-12
