"""Pins for oracle O8 (the constructed loss probe); CPU only."""
import json
import math
import os

import numpy as np
import pytest

from oracle import loss_probe as LP
from oracle import packing as P

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _setup():
    g = json.load(open(os.path.join(GOLD, "nextfit_capacity6.json")))
    lp = json.load(open(os.path.join(GOLD, "loss_probe.json")))
    rows = P.packed_rows(g["documents"], g["capacity"])
    z = LP.constructed_logits(rows, lp["vocab"])
    return rows, z, lp


def test_probe_matches_printed_values():
    rows, z, lp = _setup()
    s, m = LP.token_weighted_nll(z, rows["targets"], rows["valid"])
    assert round(s, 6) == lp["loss_sum_printed"]
    assert round(m, 6) == lp["loss_mean_printed"]
    assert math.isclose(m, 11 / 9 * math.log(2), rel_tol=1e-12)
    assert math.isclose(s, 11 * math.log(2), rel_tol=1e-12)


def test_other_weightings_do_not_come_out():
    rows, z, lp = _setup()
    rm = LP.row_mean_nll(z, rows["targets"], rows["valid"])
    dm = LP.document_mean_nll(z, rows["targets"], rows["valid"], rows["segments"])
    assert round(rm, 6) == lp["row_mean_printed"]
    assert round(dm, 6) == lp["document_mean_printed"]
    _, m = LP.token_weighted_nll(z, rows["targets"], rows["valid"])
    assert round(m, 6) not in (lp["row_mean_printed"], lp["document_mean_printed"])


def test_gold_probability_is_q():
    rows, z, lp = _setup()
    for r in range(2):
        for c in range(6):
            if rows["valid"][r, c]:
                p = np.exp(z[r, c] - z[r, c].max())
                p /= p.sum()
                want = 0.25 if rows["segments"][r, c] == 1 else 0.5
                assert math.isclose(p[rows["targets"][r, c]], want, rel_tol=1e-12)


def test_zero_eligible_is_an_error():
    rows, z, _ = _setup()
    with pytest.raises(ValueError):
        LP.token_weighted_nll(z, rows["targets"], np.zeros_like(rows["valid"]))


# ---------------------------------------------------------------- O10

def test_packed_nll_matches_probe_on_flat_cells():
    """The probe's twelve cells laid flat: the same sum, count and mean."""
    rows, z, lp = _setup()
    C = z.shape[0] * z.shape[1]
    flat = z.reshape(C, -1)
    tg = np.where(rows["valid"].reshape(-1), rows["targets"].reshape(-1), -1)
    row, s, n, m = LP.packed_nll(flat, tg)
    assert n == 9
    assert round(s, 6) == lp["loss_sum_printed"] and round(m, 6) == lp["loss_mean_printed"]
    assert np.all(row[tg < 0] == 0.0)


def test_packed_nll_grad_by_finite_differences():
    rng = np.random.default_rng(5)
    C, V = 7, 11
    z = rng.normal(size=(C, V)) * 2
    tg = rng.integers(0, V, size=C)
    tg[[1, 4]] = -1                          # two cells without a target
    mask = np.ones(C, dtype=np.uint8)
    mask[5] = 0                              # one target not supervised
    g = LP.packed_nll_grad(z, tg, mask)
    h = 1e-6
    for c in range(C):
        for v in range(V):
            zp, zm = z.copy(), z.copy()
            zp[c, v] += h
            zm[c, v] -= h
            fd = (LP.packed_nll(zp, tg, mask)[3] - LP.packed_nll(zm, tg, mask)[3]) / (2 * h)
            assert abs(fd - g[c, v]) < 1e-8, (c, v)
    assert np.all(g[[1, 4, 5]] == 0.0)
    assert np.allclose(g.sum(axis=1), 0.0, atol=1e-15)


def test_excluded_cells_are_skipped_not_multiplied():
    """NaN/Inf logits in excluded cells change nothing (x0 would give NaN)."""
    rng = np.random.default_rng(6)
    z = rng.normal(size=(5, 9))
    tg = np.array([3, -1, 2, -100, 8])
    base = LP.packed_nll(z, tg)
    gb = LP.packed_nll_grad(z, tg)
    z[1, :] = np.nan
    z[3, 2] = np.inf
    after = LP.packed_nll(z, tg)
    assert after[1] == base[1] and after[2] == base[2]
    ga = LP.packed_nll_grad(z, tg)
    assert np.array_equal(ga, gb)


def test_zero_eligible_and_bad_target_are_errors():
    z = np.zeros((3, 4))
    with pytest.raises(ValueError):
        LP.packed_nll(z, np.array([-1, -100, -1]))
    with pytest.raises(ValueError):
        LP.packed_nll(z, np.array([0, 1, 2]), mask=np.zeros(3))
    with pytest.raises(ValueError):
        LP.packed_nll(z, np.array([0, 4, 1]))


def test_shifted_targets_page_figure():
    """Section 2's figure: A0 A1 A2 | B0 B1 -> A1 A2 -1 | B1 -1; A's last
    logit never supervises B's first token."""
    ids = np.array([10, 11, 12, 20, 21])
    t = LP.shifted_targets(ids, [0, 3, 5])
    assert t.tolist() == [11, 12, -100, 21, -100]
    t2 = LP.shifted_targets(ids, [0, 5])             # one sample: a plain shift
    assert t2.tolist() == [11, 12, 20, 21, -100]
