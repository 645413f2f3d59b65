"""Pins for oracle O1-O4 (packing plans and packed-row metadata); CPU only."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import packing as P

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- O1

def test_worked_example_metadata_matches_page():
    g = _gold("worked_5_3_4.json")
    md = P.packed_row_metadata(g["lengths"])
    assert md["cu"].tolist() == g["cu_seqlens"]
    assert md["pos"].tolist() == g["position_ids"]
    assert md["max_seqlen"] == g["max_seqlen"]
    assert md["seg"].tolist() == [0] * 5 + [1] * 3 + [2] * 4


def test_metadata_loop_equals_per_token_definition():
    rng = np.random.default_rng(7)
    for _ in range(50):
        B = int(rng.integers(0, 9))
        lengths = rng.integers(0, 7, size=B).tolist()
        cap = sum(lengths) + int(rng.integers(0, 4))
        base = int(rng.integers(0, 5))
        a = P.packed_row_metadata(lengths, cap, base)
        b = P.packed_row_metadata_by_search(lengths, cap, base)
        for key in ("cu", "pos", "seg"):
            assert np.array_equal(a[key], b[key]), key


def test_metadata_zero_length_segments_consume_ids():
    md = P.packed_row_metadata([2, 0, 0, 3, 0], capacity=7, segment_base=10)
    assert md["cu"].tolist() == [0, 2, 2, 2, 5, 5]
    assert md["seg"].tolist() == [10, 10, 13, 13, 13, -1, -1]
    assert md["pos"].tolist() == [0, 1, 0, 1, 2, 0, 0]
    assert md["max_seqlen"] == 3


def test_metadata_token_axis_invariants():
    lengths = [4, 1, 7, 3]
    md = P.packed_row_metadata(lengths)
    T = sum(lengths)
    assert md["cu"][0] == 0 and md["cu"][-1] == T and len(md["cu"]) == len(lengths) + 1
    assert len(md["pos"]) == T and len(md["seg"]) == T
    # positions reset exactly at the boundaries
    assert sorted(np.flatnonzero(md["pos"] == 0).tolist()) == md["cu"][:-1].tolist()


def test_metadata_errors():
    with pytest.raises(P.PackingError):
        P.packed_row_metadata([3, -1])
    with pytest.raises(P.PackingError):
        P.packed_row_metadata([3, 4], capacity=6)
    with pytest.raises(P.PackingError):
        P.cu_seqlens_from_lengths([2**31 - 1, 1])


# ---------------------------------------------------------------- O2 + O4

def test_fixture_rows_match_page():
    g = _gold("nextfit_capacity6.json")
    rows = P.packed_rows(g["documents"], g["capacity"])
    assert rows["lengths"] == g["prediction_lengths"]
    for key in ("inputs", "targets", "segments", "positions"):
        assert rows[key].tolist() == g[key], key
    assert rows["valid"].tolist() == g["valid"]
    assert rows["inputs"].size == g["cells"]
    assert int(rows["valid"].sum()) == g["real_targets"]


def test_fixture_pairs_do_not_cross_documents():
    g = _gold("nextfit_capacity6.json")
    for doc in g["documents"]:
        pairs = P.form_pairs(doc)
        assert len(pairs) == len(doc) - 1
        assert pairs[-1][1] == 1          # each document's last input predicts its own EOS
    # a global shift of the concatenation would add EOS->BOS targets
    cat = sum(g["documents"], [])
    assert (1, 0) in P.form_pairs(cat)
    assert all((1, 0) not in P.form_pairs(doc) for doc in g["documents"])


def test_next_fit_edge_cases():
    assert P.next_fit([], 5) == ([], [], 0)
    # exact fill opens no extra row
    assert P.next_fit([2, 3], 5) == ([0, 0], [0, 2], 1)
    # zero length goes into the current row at its fill level
    assert P.next_fit([5, 0, 1], 5) == ([0, 0, 1], [0, 5, 0], 2)
    # capacity 1
    assert P.next_fit([1, 1, 0, 1], 1) == ([0, 1, 1, 2], [0, 0, 1, 0], 3)
    # order preserved, rows never revisited (the 1 would fit row 0)
    assert P.next_fit([4, 5, 1], 6) == ([0, 1, 1], [0, 0, 5], 2)
    with pytest.raises(P.PackingError):
        P.next_fit([3, 7], 6)
    with pytest.raises(P.PackingError):
        P.next_fit([1], 0)


def test_next_fit_definition_brute_force():
    """Every row's fill <= capacity; a new row opens only when the item did not fit."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        cap = int(rng.integers(1, 12))
        lengths = rng.integers(0, cap + 1, size=int(rng.integers(0, 12))).tolist()
        row_of, start_of, n_rows = P.next_fit(lengths, cap)
        fill = {}
        for i, L in enumerate(lengths):
            r = row_of[i]
            assert start_of[i] == fill.get(r, 0)
            if i > 0 and r != row_of[i - 1]:
                assert r == row_of[i - 1] + 1
                assert L > cap - fill[row_of[i - 1]]
            fill[r] = fill.get(r, 0) + L
            assert fill[r] <= cap
        assert n_rows == (row_of[-1] + 1 if lengths else 0)


# ---------------------------------------------------------------- O3

def test_bfd_hand_worked_cases():
    for case in _gold("bfd_hand_worked.json")["cases"]:
        bin_of, start_of, n_bins, order, offs = P.best_fit_decreasing(case["lengths"], case["capacity"])
        bins = [order[offs[j]:offs[j + 1]] for j in range(n_bins)]
        assert bins == case["bins"], case


def test_bfd_replay_random():
    rng = np.random.default_rng(11)
    for _ in range(200):
        cap = int(rng.integers(1, 20))
        lengths = rng.integers(0, cap + 1, size=int(rng.integers(0, 25))).tolist()
        bin_of, start_of, n_bins, order, offs = P.best_fit_decreasing(lengths, cap)
        P.replay_best_fit(lengths, cap, bin_of, start_of, n_bins)
        assert sorted(order) == list(range(len(lengths)))
        for j in range(n_bins):
            members = order[offs[j]:offs[j + 1]]
            assert all(bin_of[i] == j for i in members)
            # starts are consecutive in insertion order
            s = 0
            for i in members:
                assert start_of[i] == s
                s += lengths[i]
            assert s <= cap


def _all_best_fit_runs(lengths, cap):
    """Enumerate, for tiny inputs, the bin choices of every greedy run that
    always picks a feasible bin of least room (any tie) or a new bin when none
    fits; the pinned tie-break must be one of them and the lowest-numbered one."""
    ids = sorted(range(len(lengths)), key=lambda i: (-lengths[i], i))
    runs = [([], [])]                       # (choices, fills)
    for i in ids:
        nxt = []
        for choices, fills in runs:
            feas = [j for j, f in enumerate(fills) if cap - f >= lengths[i]]
            if feas:
                best = min(cap - fills[j] for j in feas)
                opts = [j for j in feas if cap - fills[j] == best]
            else:
                opts = [len(fills)]
            for j in opts:
                f2 = list(fills) + ([0] if j == len(fills) else [])
                f2[j] += lengths[i]
                nxt.append((choices + [j], f2))
        runs = nxt
    return ids, runs


def test_bfd_brute_force_tiny():
    for cap in (1, 2, 3, 5):
        for n in range(0, 5):
            for lengths in itertools.product(range(0, cap + 1), repeat=n):
                lengths = list(lengths)
                bin_of, _, n_bins, _, _ = P.best_fit_decreasing(lengths, cap)
                ids, runs = _all_best_fit_runs(lengths, cap)
                mine = [bin_of[i] for i in ids]
                assert mine in [c for c, _ in runs]
                assert mine == min(c for c, _ in runs)   # lowest bin on every tie


def test_bfd_cfg3_first_pack_is_one_full_sample():
    from workloads import raw_lengths_cfg3
    L = raw_lengths_cfg3(0)
    bin_of, start_of, n_bins, order, offs = P.best_fit_decreasing(L.tolist(), 8192)
    first = [int(L[i]) for i in order[offs[0]:offs[1]]]
    assert first == [8192]
    assert sum(int(x) for x in L) <= n_bins * 8192


def test_bfd_errors():
    with pytest.raises(P.PackingError):
        P.best_fit_decreasing([9], 8)
    with pytest.raises(P.PackingError):
        P.best_fit_decreasing([1], 0)


# ---------------------------------------------------------------- O9

def test_boundaries_from_positions_worked_example():
    """Section 3's table: resets at 0, 5, 8; the total 12 appended."""
    g = _gold("worked_5_3_4.json")
    cu, mx = P.boundaries_from_positions(g["position_ids"])
    assert cu.tolist() == g["cu_seqlens"] and mx == g["max_seqlen"]
    cu2, mx2 = P.boundaries_from_positions(g["position_ids"], "min")
    assert cu2.tolist() == g["cu_seqlens"] and mx2 == g["max_seqlen"]


def test_boundaries_round_trip_and_zero_length_loss():
    """lengths -> positions (O1) -> boundaries gives the lengths back, except
    that zero-length segments vanish."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        B = int(rng.integers(1, 12))
        lengths = rng.integers(0, 9, size=B).tolist()
        if sum(lengths) == 0:
            continue
        md = P.packed_row_metadata(lengths)
        cu, mx = P.boundaries_from_positions(md["pos"])
        kept = [L for L in lengths if L > 0]
        assert cu.tolist() == P.cu_seqlens_from_lengths(kept)
        assert mx == max(kept)


def test_boundaries_min_sentinel_offset_positions():
    """Positions that start at 1 (or any c): the min path still finds the
    starts; the zero path has no start at token 0 and is an error."""
    md = P.packed_row_metadata([4, 2, 5])
    for c in (1, 7, -3):
        cu, mx = P.boundaries_from_positions(md["pos"] + c, "min")
        assert cu.tolist() == [0, 4, 6, 11] and mx == 5
    with pytest.raises(P.PackingError):
        P.boundaries_from_positions(md["pos"] + 1, "zero")


def test_boundaries_from_text_plane_not_rotary_planes():
    """Section 6: rotary coordinates repeat inside a sample (several tokens of
    an image grid share a temporal, height or width coordinate, and several
    of them are 0), so reset points read from those planes over-split a
    sample; the text plane (0, 1, 2, ... per sample) gives the true
    boundaries."""
    # sample A: a 2x3 image grid whose coordinates start at 0, then 2 text
    # tokens continuing after the grid; sample B: 3 text tokens
    temporal = np.array([0, 0, 0, 0, 0, 0, 3, 4] + [0, 1, 2])
    height = np.array([0, 0, 0, 1, 1, 1, 3, 4] + [0, 1, 2])
    width = np.array([0, 1, 2, 0, 1, 2, 3, 4] + [0, 1, 2])
    text = np.array(list(range(8)) + list(range(3)))
    cu, mx = P.boundaries_from_positions(text)
    assert cu.tolist() == [0, 8, 11] and mx == 8
    for plane in (temporal, height, width):
        assert len(P.boundaries_from_positions(plane)[0]) > len(cu)   # over-split


def test_boundaries_edge_cases():
    cu, mx = P.boundaries_from_positions([])
    assert cu.tolist() == [0] and mx == 0
    cu, mx = P.boundaries_from_positions([0])
    assert cu.tolist() == [0, 1] and mx == 1
    cu, mx = P.boundaries_from_positions([0, 0, 0])
    assert cu.tolist() == [0, 1, 2, 3] and mx == 1
    with pytest.raises(P.PackingError):
        P.boundaries_from_positions([1, 0, 1])
