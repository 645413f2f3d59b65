"""Oracle O1-O4: packing plans and packed-row metadata (plain Python).

O1  packed-row metadata from segment lengths
    "Packing与 FlashAttention Varlen" section 1 (the 5/3/4 figure) and
    section 3 (cu_seqlens = reset indices plus the total; max_seqlen = largest
    difference); "Pack sequences without joining their contexts", "Fill only
    the current row" (segment rows, local position rows, PAD_CELL, NO_SEGMENT).
O2  order-preserving next-fit
    "Pack sequences without joining their contexts", "Fill only the current
    row" and "Extend the existing storage and decoder" (whole examples only, an
    oversized example is an error, an exact fill opens no extra row);
    "Packing与 FlashAttention Varlen" section 2 (the sequential strategy).
O3  best-fit-decreasing
    "Packing与 FlashAttention Varlen" section 2 names it as the default packing
    strategy; the page gives no body.  Reading: stable sort by decreasing
    length (ties by input index); each item goes to the open bin with the least
    remaining room that still fits it (room >= length), ties to the lowest bin
    number; otherwise a new bin.  Bins are numbered in creation order and keep
    their items in insertion order.  A length above the capacity is an error.
O4  next-token pair forming inside each document
    "Pack sequences without joining their contexts", "Form pairs inside each
    source range".
O9  boundaries compiled back from position_ids
    "Packing与 FlashAttention Varlen" section 3: the reset points of the
    sample-local positions (position == 0, or position == the smallest
    position for the general path), followed by the total token count, are
    cu_seqlens; max_seqlen is the largest difference.  Section 6: when the
    positions are multimodal rotary coordinates that repeat inside a sample,
    the boundary is read from a separate strictly increasing text-position
    plane instead.  Readings: the first token must be a reset point (else
    cu[0] would not be 0 and the contract of section 3 fails: an error); an
    empty stream gives cu = [0] and max_seqlen = 0; zero-length segments
    cannot be represented and vanish.
"""
from __future__ import annotations

import numpy as np

PAD_CELL = -1
NO_SEGMENT = -1
INT32_MAX = 2**31 - 1


class PackingError(ValueError):
    pass


# ---------------------------------------------------------------------------
# O1
# ---------------------------------------------------------------------------

def cu_seqlens_from_lengths(lengths) -> list[int]:
    """cu[0] = 0, cu[b+1] = cu[b] + L_b; every value must fit int32."""
    cu = [0]
    for L in lengths:
        L = int(L)
        if L < 0:
            raise PackingError("negative segment length")
        nxt = cu[-1] + L
        if nxt > INT32_MAX:
            raise PackingError("cu_seqlens overflows int32")
        cu.append(nxt)
    return cu


def segment_of_token(cu, t: int) -> int:
    """s(t) = max{b : cu[b] <= t} over segments b (zero-length ones own no token)."""
    best = -1
    for b in range(len(cu) - 1):
        if cu[b] <= t:
            best = b
    return best


def packed_row_metadata(lengths, capacity: int | None = None, segment_base: int = 0):
    """O1.  Returns dict(cu, pos, seg, max_seqlen) for one packed row.

    Cells t < sum(L) are real: seg = segment_base + s(t), pos = t - cu[s(t)].
    Cells sum(L) <= t < capacity are padding: seg = NO_SEGMENT, pos = 0.
    """
    cu = cu_seqlens_from_lengths(lengths)
    total = cu[-1]
    C = total if capacity is None else int(capacity)
    if C < total:
        raise PackingError("segments do not fit the row capacity")
    pos = np.zeros(C, dtype=np.int32)
    seg = np.full(C, NO_SEGMENT, dtype=np.int32)
    # walk the segments; each owns the half-open token range [cu[b], cu[b+1])
    for b in range(len(cu) - 1):
        for t in range(cu[b], cu[b + 1]):
            pos[t] = t - cu[b]
            seg[t] = segment_base + b
    max_seqlen = 0
    for b in range(len(cu) - 1):
        max_seqlen = max(max_seqlen, cu[b + 1] - cu[b])
    return {"cu": np.asarray(cu, dtype=np.int32), "pos": pos, "seg": seg,
            "max_seqlen": max_seqlen}


def packed_row_metadata_by_search(lengths, capacity: int | None = None, segment_base: int = 0):
    """O1 written as its per-token definition (tiny inputs): s(t) by search."""
    cu = cu_seqlens_from_lengths(lengths)
    total = cu[-1]
    C = total if capacity is None else int(capacity)
    pos = np.zeros(C, dtype=np.int32)
    seg = np.full(C, NO_SEGMENT, dtype=np.int32)
    for t in range(total):
        s = segment_of_token(cu, t)
        pos[t] = t - cu[s]
        seg[t] = segment_base + s
    return {"cu": np.asarray(cu, dtype=np.int32), "pos": pos, "seg": seg}


# ---------------------------------------------------------------------------
# O2
# ---------------------------------------------------------------------------

def _validate(lengths, capacity):
    if int(capacity) <= 0:
        raise PackingError("capacity must be positive")
    if len(lengths) > INT32_MAX:
        raise PackingError("occurrence ids must fit int32")
    for L in lengths:
        if int(L) < 0:
            raise PackingError("negative length")
        if int(L) > int(capacity):
            raise PackingError("example longer than the capacity")


def next_fit(lengths, capacity: int):
    """O2.  Returns (row_of, start_of, n_rows).

    Reads items in their given order.  An item that does not fit the room left
    in the current row opens a new row; rows are never revisited and items are
    never split.  Zero-length items go into the current row at its fill level.
    n = 0 gives 0 rows.
    """
    _validate(lengths, capacity)
    n = len(lengths)
    row_of = [0] * n
    start_of = [0] * n
    if n == 0:
        return row_of, start_of, 0
    row, used = 0, 0
    for i, L in enumerate(lengths):
        L = int(L)
        if L > capacity - used:
            row += 1
            used = 0
        row_of[i] = row
        start_of[i] = used
        used += L
    return row_of, start_of, row + 1


# ---------------------------------------------------------------------------
# O3
# ---------------------------------------------------------------------------

def best_fit_decreasing(lengths, capacity: int):
    """O3.  Returns (bin_of, start_of, n_bins, order, bin_offsets).

    ``order`` lists item ids bin by bin, each bin in insertion order;
    ``bin_offsets[j]:bin_offsets[j+1]`` is bin j's slice of ``order``.
    """
    _validate(lengths, capacity)
    n = len(lengths)
    ids = sorted(range(n), key=lambda i: (-int(lengths[i]), i))
    room = np.zeros(0, dtype=np.int64)      # remaining room per bin, bin-number order
    members: list[list[int]] = []
    bin_of = [0] * n
    start_of = [0] * n
    for i in ids:
        L = int(lengths[i])
        fits = np.flatnonzero(room >= L)
        if fits.size:
            # least remaining room; np.argmin returns the first (lowest bin) of ties
            j = int(fits[np.argmin(room[fits])])
        else:
            j = len(members)
            room = np.append(room, capacity)
            members.append([])
        bin_of[i] = j
        start_of[i] = int(capacity - room[j])
        room[j] -= L
        members[j].append(i)
    order = [i for m in members for i in m]
    offsets = [0]
    for m in members:
        offsets.append(offsets[-1] + len(m))
    return bin_of, start_of, len(members), order, offsets


def replay_best_fit(lengths, capacity, bin_of, start_of, n_bins):
    """Check a plan against the best-fit-decreasing definition step by step.

    Independent of ``best_fit_decreasing``'s code: it recomputes each bin's
    fill from the plan, in the decreasing order, and asserts that each step put
    the item in the tightest bin that fit (lowest number on ties) or in a new
    bin when none fit.  Returns None or raises AssertionError.
    """
    n = len(lengths)
    ids = sorted(range(n), key=lambda i: (-int(lengths[i]), i))
    fill: list[int] = []
    for i in ids:
        L = int(lengths[i])
        cands = [(capacity - f, j) for j, f in enumerate(fill) if capacity - f >= L]
        if cands:
            want = min(cands)[1]
        else:
            want = len(fill)
            fill.append(0)
        assert bin_of[i] == want, (i, bin_of[i], want)
        assert start_of[i] == fill[want], (i, start_of[i], fill[want])
        fill[want] += L
    assert len(fill) == n_bins
    assert all(f <= capacity for f in fill)


# ---------------------------------------------------------------------------
# O4 and the fixture rows
# ---------------------------------------------------------------------------

def form_pairs(document):
    """O4.  A document of n tokens gives n-1 (input, target) pairs inside it."""
    return [(document[j], document[j + 1]) for j in range(len(document) - 1)]


def packed_rows(documents, capacity: int):
    """Next-fit rows of pair-formed documents, with their per-cell metadata.

    Returns a dict of [n_rows, capacity] int arrays: inputs, targets, segments,
    positions and a bool ``valid`` (input validity).  Occurrence ordinal b is
    the segment id of document b.  Padding: inputs/targets PAD_CELL, segment
    NO_SEGMENT, position 0, valid False.
    """
    pairs = [form_pairs(doc) for doc in documents]
    lengths = [len(p) for p in pairs]
    row_of, start_of, n_rows = next_fit(lengths, capacity)
    inputs = np.full((n_rows, capacity), PAD_CELL, dtype=np.int64)
    targets = np.full((n_rows, capacity), PAD_CELL, dtype=np.int64)
    segments = np.full((n_rows, capacity), NO_SEGMENT, dtype=np.int64)
    positions = np.zeros((n_rows, capacity), dtype=np.int64)
    valid = np.zeros((n_rows, capacity), dtype=bool)
    for b, p in enumerate(pairs):
        r, s = row_of[b], start_of[b]
        for j, (x, y) in enumerate(p):
            inputs[r, s + j] = x
            targets[r, s + j] = y
            segments[r, s + j] = b
            positions[r, s + j] = j
            valid[r, s + j] = True
    return {"inputs": inputs, "targets": targets, "segments": segments,
            "positions": positions, "valid": valid, "lengths": lengths,
            "row_of": row_of, "start_of": start_of}


# ---------------------------------------------------------------------------
# O9
# ---------------------------------------------------------------------------

def boundaries_from_positions(position_ids, sentinel: str = "zero"):
    """O9.  Returns (cu, max_seqlen) for a flat position stream.

    sentinel "zero": a token starts a segment when its position is 0;
    sentinel "min": when its position equals the smallest position.
    """
    pos = [int(x) for x in np.asarray(position_ids).reshape(-1)]
    T = len(pos)
    if T == 0:
        return np.zeros(1, dtype=np.int32), 0
    if sentinel == "zero":
        s = 0
    elif sentinel == "min":
        s = min(pos)
    else:
        raise ValueError("sentinel must be 'zero' or 'min'")
    starts = [t for t in range(T) if pos[t] == s]
    if not starts or starts[0] != 0:
        raise PackingError("the first token is not a segment start")
    if T > INT32_MAX:
        raise PackingError("token count overflows int32")
    cu = starts + [T]
    max_seqlen = max(cu[b + 1] - cu[b] for b in range(len(cu) - 1))
    return np.asarray(cu, dtype=np.int32), max_seqlen
