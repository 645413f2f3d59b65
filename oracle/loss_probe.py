"""Oracle O8: the constructed loss probe on the packed capacity-6 rows.

"Pack sequences without joining their contexts", "Keep the same nine-target
objective": with vocabulary V, every non-gold logit is 0 and the gold logit is
ln((V-1) q / (1-q)), so softmax gives the gold class probability q.  Targets
in occurrence segment 1 get q = 1/4, all others q = 1/2.  The loss is the sum
of -ln p(target) over eligible cells divided once by their count (token
weighting); zero eligible targets is an error.

O10 the packed-row loss and its logit gradient, on flat cells [C, V]
    Same page and section: the token-weighted mean over eligible targets, and
    the mean-loss logit derivative (p_ic - 1[c = y_i]) / N for eligible
    target i (N = eligible count over all rows); excluded cells contribute
    exactly zero and are skipped before any arithmetic.  "Packing与
    FlashAttention Varlen" section 2: labels are made sample-local before
    packing (the first label of every sample is ignored), so after the
    one-step shift the last cell of a sample targets nothing and never the
    next sample's first token.
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


# ---------------------------------------------------------------------------
# O10
# ---------------------------------------------------------------------------

IGNORE = -100


def eligible_cells(targets, mask=None):
    """A cell is eligible when it has a target (>= 0) and, if a mask is given,
    the mask marks it supervised."""
    t = np.asarray(targets)
    e = t >= 0
    if mask is not None:
        e = e & (np.asarray(mask) != 0)
    return e


def packed_nll(logits, targets, mask=None):
    """O10.  logits [C, V] (any float), targets [C] int.  Returns
    (row_nll [C] with 0 on excluded cells, loss_sum, count, loss_mean)."""
    z = np.asarray(logits, dtype=np.float64)
    C, V = z.shape
    e = eligible_cells(targets, mask)
    row = np.zeros(C)
    for c in range(C):
        if not e[c]:
            continue                       # excluded before any arithmetic
        y = int(targets[c])
        if not 0 <= y < V:
            raise ValueError("a supervised target is not a class of the vocabulary")
        m = z[c].max()
        log_z = m + math.log(np.exp(z[c] - m).sum())
        row[c] = log_z - z[c, y]
    n = int(e.sum())
    if n == 0:
        raise ValueError("no eligible targets: the mean has no denominator")
    total = float(row.sum())
    return row, total, n, total / n


def packed_nll_grad(logits, targets, mask=None):
    """O10.  d(mean loss)/d logits [C, V]: (softmax - onehot) / N on eligible
    rows, exactly 0 elsewhere (never computed from those logits)."""
    z = np.asarray(logits, dtype=np.float64)
    C, V = z.shape
    e = eligible_cells(targets, mask)
    n = int(e.sum())
    if n == 0:
        raise ValueError("no eligible targets: the mean has no denominator")
    g = np.zeros((C, V))
    for c in range(C):
        if not e[c]:
            continue
        m = z[c].max()
        p = np.exp(z[c] - m)
        p /= p.sum()
        p[int(targets[c])] -= 1.0
        g[c] = p / n
    return g


def shifted_targets(input_ids, cu, ignore: int = IGNORE):
    """One-step shift inside each sample [cu[b], cu[b+1]): cell t targets
    input t+1 of the same sample; a sample's last cell gets `ignore`."""
    ids = np.asarray(input_ids)
    out = np.full(len(ids), ignore, dtype=np.int64)
    for b in range(len(cu) - 1):
        for t in range(int(cu[b]), int(cu[b + 1]) - 1):
            out[t] = ids[t + 1]
    return out
