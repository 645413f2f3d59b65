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
