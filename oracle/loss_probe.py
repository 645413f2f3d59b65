"""Oracle O8: the constructed loss probe on the packed capacity-6 rows.

"Pack sequences without joining their contexts", "Keep the same nine-target
objective": with vocabulary V, every non-gold logit is 0 and the gold logit is
ln((V-1) q / (1-q)), so softmax gives the gold class probability q.  Targets
in occurrence segment 1 get q = 1/4, all others q = 1/2.  The loss is the sum
of -ln p(target) over eligible cells divided once by their count (token
weighting); zero eligible targets is an error.
"""
from __future__ import annotations

import math

import numpy as np


def constructed_logits(rows, vocab: int):
    """[n_rows, C, V] logits of the probe, zero on cells that are not valid."""
    n_rows, C = rows["inputs"].shape
    z = np.zeros((n_rows, C, vocab))
    for r in range(n_rows):
        for c in range(C):
            if rows["valid"][r, c]:
                q = 0.25 if rows["segments"][r, c] == 1 else 0.5
                z[r, c, rows["targets"][r, c]] = math.log((vocab - 1) * q / (1.0 - q))
    return z


def token_weighted_nll(logits, targets, eligible):
    """Return (loss_sum, loss_mean) over eligible cells only.

    Ineligible cells are skipped before any arithmetic.
    """
    total = 0.0
    count = 0
    n_rows, C, _ = logits.shape
    for r in range(n_rows):
        for c in range(C):
            if not eligible[r, c]:
                continue
            row = logits[r, c]
            m = row.max()
            log_z = m + math.log(np.exp(row - m).sum())
            total += log_z - row[targets[r, c]]
            count += 1
    if count == 0:
        raise ValueError("no eligible targets: the mean has no denominator")
    return total, total / count


def row_mean_nll(logits, targets, eligible):
    """Mean of per-row means (a different weighting, for contrast only)."""
    means = []
    for r in range(logits.shape[0]):
        s, m = token_weighted_nll(logits[r:r + 1], targets[r:r + 1], eligible[r:r + 1])
        means.append(m)
    return sum(means) / len(means)


def document_mean_nll(logits, targets, eligible, segments):
    """Mean of per-document means (a different weighting, for contrast only)."""
    per = {}
    n_rows, C, _ = logits.shape
    for r in range(n_rows):
        for c in range(C):
            if eligible[r, c]:
                row = logits[r, c]
                m = row.max()
                nll = m + math.log(np.exp(row - m).sum()) - row[targets[r, c]]
                per.setdefault(int(segments[r, c]), []).append(nll)
    means = [sum(v) / len(v) for v in per.values()]
    return sum(means) / len(means)
