"""Oracle O5-O7: block-causal attention over a flat packed token stream (fp64).

O5 forward -- "Packing与 FlashAttention Varlen" section 1 (each cu_seqlens
   slice is an independent causal attention, written back in flat order;
   merging boundaries changes the problem) and section 5 (per-slice base and
   extent, causal only inside the slice, output at Q's offsets);
   "Pack sequences without joining their contexts", "Permission depends on the
   example" (a key is permitted when it is in the query's segment and not later
   than the query).  Softmax scale 1/sqrt(d) is a reading (the pages leave it
   open); it is passed in.
O6 backward -- the textbook gradient of softmax attention, restricted to the
   same per-segment ranges ("the same boundary" drives forward and backward
   calculation: "Pack sequences without joining their contexts", "Extend the
   existing storage and decoder").
O7 brute force -- the dense [T, T] permission matrix of "Permission depends on
   the example" built from segment ids, local positions and validity, with a
   masked softmax over whole rows; rows with no permitted key give a zero
   mixture.  Tiny inputs only.

Grouped key/value heads ("Packing与 FlashAttention Varlen" section 5: the
key/value view has h_k heads beside the query view's h): K and V may carry
H_k heads with H a multiple of H_k; query head h reads key/value head
h // (H / H_k) (consecutive query heads share a group -- a reading, the page
gives only the shapes), and the gradient of a key/value head is the sum over
its group's query heads.

Separate query and key boundaries and local windows (first page, section 5:
cu_seqlens_q and cu_seqlens_k give each slice its own query and key extents,
L_q and L_k; the causal clamp is aligned to the bottom right by L_k - L_q and
widened by a right window; a local window also bounds it on the left).
Reading, with delta = L_k - L_q: query i (local) may use key j (local) when
0 <= j < L_k, j <= i + delta + window_right (window_right >= 0; -1 = no
bound) and j >= i + delta - window_left (window_left >= 0; -1 = no bound).
Causal self-attention is window (-1, 0) with cu_k = cu_q.  A query with no
permitted key gets a zero output and LSE = -inf, and passes no gradient.

All arrays are float64 numpy; inputs are [T, H, d] (K, V: [T, H_k, d]).  LSE is natural-log,
layout [H, T].  No blocking beyond a plain split of query rows into chunks
(which changes no arithmetic inside a row).
"""
from __future__ import annotations

import math

import numpy as np

ROW_CHUNK = 512


def _segments(cu):
    cu = [int(x) for x in cu]
    return [(cu[b], cu[b + 1]) for b in range(len(cu) - 1)]


def segment_head_forward(q, k, v, scale):
    """Causal softmax attention inside one segment, one head.

    q, k, v: [L, d].  Query i sees keys j <= i (local indices).
    Returns (O [L, d], LSE [L]).
    """
    L = q.shape[0]
    out = np.zeros_like(q)
    lse = np.zeros(L)
    for r0 in range(0, L, ROW_CHUNK):
        r1 = min(L, r0 + ROW_CHUNK)
        s = scale * (q[r0:r1] @ k[:r1].T)                    # [rows, keys 0..r1-1]
        i = np.arange(r0, r1)[:, None]
        j = np.arange(r1)[None, :]
        s = np.where(j <= i, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        p = e / z
        out[r0:r1] = p @ v[:r1]
        lse[r0:r1] = (m + np.log(z))[:, 0]
    return out, lse


def segment_head_backward(q, k, v, do, scale):
    """Gradients of sum(O * dO) for one segment and head; returns (dq, dk, dv).

    P_ij = softmax_j(scale * q_i . k_j) over j <= i;  O_i = sum_j P_ij v_j.
    dV_j = sum_i P_ij dO_i;  dP_ij = dO_i . v_j;
    dS_ij = P_ij (dP_ij - sum_l P_il dP_il)   (softmax Jacobian);
    dQ_i = scale sum_j dS_ij k_j;  dK_j = scale sum_i dS_ij q_i.
    """
    L = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, L, ROW_CHUNK):
        r1 = min(L, r0 + ROW_CHUNK)
        s = scale * (q[r0:r1] @ k[:r1].T)
        i = np.arange(r0, r1)[:, None]
        j = np.arange(r1)[None, :]
        s = np.where(j <= i, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        dv[:r1] += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v[:r1].T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[r0:r1] = scale * (ds @ k[:r1])
        dk[:r1] += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


def _group(q, k):
    H, Hk = q.shape[1], k.shape[1]
    if Hk <= 0 or H % Hk != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    return H // Hk


def varlen_forward(q, k, v, cu, scale=None, heads=None):
    """O5 over the whole packed stream.  Returns (O [T,H,d], LSE [H,T]).

    ``heads`` restricts the computation to a subset of heads (the others are
    left zero) so that large workloads can be checked on a sample.
    """
    T, H, d = q.shape
    G = _group(q, k)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if int(cu[0]) != 0 or int(cu[-1]) != T:
        raise ValueError("cu_seqlens must start at 0 and end at T")
    out = np.zeros((T, H, d))
    lse = np.zeros((H, T))
    hs = range(H) if heads is None else heads
    for s, e in _segments(cu):
        if e == s:
            continue
        for h in hs:
            o, l = segment_head_forward(q[s:e, h], k[s:e, h // G], v[s:e, h // G], scale)
            out[s:e, h] = o
            lse[h, s:e] = l
    return out, lse


def varlen_backward(q, k, v, do, cu, scale=None, heads=None):
    """O6 over the whole packed stream.  Returns (dQ [T,H,d], dK, dV [T,H_k,d]).

    With ``heads``, dK and dV hold only those query heads' contributions."""
    T, H, d = q.shape
    G = _group(q, k)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros((T, H, d))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    hs = range(H) if heads is None else heads
    for s, e in _segments(cu):
        if e == s:
            continue
        for h in hs:
            a, b, c = segment_head_backward(q[s:e, h], k[s:e, h // G], v[s:e, h // G], do[s:e, h], scale)
            dq[s:e, h] = a
            dk[s:e, h // G] += b
            dv[s:e, h // G] += c
    return dq, dk, dv


def forward_rows(q, k, v, cu, rows, heads, scale=None):
    """O5 for chosen (row, head) pairs only: each output row is computed alone.

    rows, heads: equal-length integer sequences of flat token index and query
    head; K and V may carry fewer heads (query head h reads key/value head
    h // (H / H_k), as in varlen_forward).  Returns (O [n, d], LSE [n]).
    """
    T, H, d = q.shape
    G = _group(q, k)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cu = [int(x) for x in cu]
    out = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for n, (t, h) in enumerate(zip(rows, heads)):
        t, h = int(t), int(h)
        if not 0 <= t < cu[-1]:
            raise ValueError("row outside the token axis")
        # t's segment starts at the last boundary at or below t
        start = max(c for c in cu[:-1] if c <= t)
        hk = h // G                       # the key/value head query head h reads
        sc = scale * (k[start:t + 1, hk] @ q[t, h])
        m = sc.max()
        e = np.exp(sc - m)
        z = e.sum()
        out[n] = (e / z) @ v[start:t + 1, hk]
        lse[n] = m + math.log(z)
    return out, lse


def allowed_matrix(seg, pos, valid):
    """Dense permission: valid(q) & valid(k) & seg(q)==seg(k) & pos(k) <= pos(q)."""
    seg = np.asarray(seg)
    pos = np.asarray(pos)
    valid = np.asarray(valid, dtype=bool)
    return (valid[:, None] & valid[None, :] & (seg[:, None] == seg[None, :])
            & (pos[None, :] <= pos[:, None]))


def dense_masked_forward(q, k, v, seg, pos, valid, scale=None):
    """O7: masked softmax over full rows of the [T, T] score matrix.

    Rows with no permitted key (inactive queries) produce zeros.
    """
    T, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    allow = allowed_matrix(seg, pos, valid)
    out = np.zeros((T, H, d))
    for h in range(H):
        s = scale * (q[:, h] @ k[:, h].T)
        for i in range(T):
            if not allow[i].any():
                continue
            row = np.where(allow[i], s[i], -np.inf)
            m = row.max()
            e = np.exp(row - m)
            out[i, h] = (e / e.sum()) @ v[:, h]
    return out


# ---------------------------------------------------------------------------
# separate query/key extents and local windows
# ---------------------------------------------------------------------------

def band_allowed(Lq, Lk, window_left=-1, window_right=0):
    """[Lq, Lk] permission of query i to key j (local indices)."""
    delta = Lk - Lq
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    ok = np.ones((Lq, Lk), dtype=bool)
    if window_right >= 0:
        ok &= j <= i + delta + window_right
    if window_left >= 0:
        ok &= j >= i + delta - window_left
    return ok


def segment_head_forward_band(q, k, v, scale, window_left=-1, window_right=0):
    """One segment and head with extents L_q = len(q), L_k = len(k).
    Returns (O [L_q, d], LSE [L_q])."""
    Lq, Lk = q.shape[0], k.shape[0]
    out = np.zeros((Lq, v.shape[1]))
    lse = np.full(Lq, -np.inf)
    if Lq == 0 or Lk == 0:
        return out, lse
    ok = band_allowed(Lq, Lk, window_left, window_right)
    for r0 in range(0, Lq, ROW_CHUNK):
        r1 = min(Lq, r0 + ROW_CHUNK)
        s = np.where(ok[r0:r1], scale * (q[r0:r1] @ k.T), -np.inf)
        for r in range(r1 - r0):
            row = s[r]
            if not ok[r0 + r].any():
                continue                                   # no permitted key
            m = row.max()
            e = np.exp(row - m)
            z = e.sum()
            out[r0 + r] = (e / z) @ v
            lse[r0 + r] = m + math.log(z)
    return out, lse


def segment_head_backward_band(q, k, v, do, scale, window_left=-1, window_right=0):
    """Gradients of sum(O * dO) for one segment and head; returns (dq, dk, dv)."""
    Lq, Lk = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if Lq == 0 or Lk == 0:
        return dq, dk, dv
    ok = band_allowed(Lq, Lk, window_left, window_right)
    for i in range(Lq):
        if not ok[i].any():
            continue
        s = np.where(ok[i], scale * (k @ q[i]), -np.inf)
        m = s.max()
        e = np.exp(s - m)
        p = e / e.sum()
        dp = v @ do[i]
        ds = p * (dp - (p * dp).sum())
        dv += np.outer(p, do[i])
        dq[i] = scale * (ds @ k)
        dk += scale * np.outer(ds, q[i])
    return dq, dk, dv


def _check_cu(cu, T, what):
    if int(cu[0]) != 0 or int(cu[-1]) != T:
        raise ValueError(f"{what} must start at 0 and end at the token count")


def varlen_cross_forward(q, k, v, cu_q, cu_k, scale=None, window=(-1, 0), heads=None):
    """Forward over a packed stream with separate query/key boundaries (same
    number of slices).  Returns (O [T_q,H,d], LSE [H,T_q])."""
    Tq, H, d = q.shape
    G = _group(q, k)
    if len(cu_q) != len(cu_k):
        raise ValueError("query and key boundaries must have the same number of slices")
    _check_cu(cu_q, Tq, "cu_q")
    _check_cu(cu_k, k.shape[0], "cu_k")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((Tq, H, d))
    lse = np.full((H, Tq), -np.inf)
    hs = range(H) if heads is None else heads
    for (qs, qe), (ks, ke) in zip(_segments(cu_q), _segments(cu_k)):
        for h in hs:
            o, l = segment_head_forward_band(q[qs:qe, h], k[ks:ke, h // G], v[ks:ke, h // G], scale, *window)
            out[qs:qe, h] = o
            lse[h, qs:qe] = l
    return out, lse


def varlen_cross_backward(q, k, v, do, cu_q, cu_k, scale=None, window=(-1, 0), heads=None):
    """Backward of varlen_cross_forward: (dQ [T_q,H,d], dK, dV [T_k,H_k,d])."""
    Tq, H, d = q.shape
    G = _group(q, k)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros((Tq, H, d))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    hs = range(H) if heads is None else heads
    for (qs, qe), (ks, ke) in zip(_segments(cu_q), _segments(cu_k)):
        for h in hs:
            a, b, c = segment_head_backward_band(q[qs:qe, h], k[ks:ke, h // G], v[ks:ke, h // G],
                                                 do[qs:qe, h], scale, *window)
            dq[qs:qe, h] = a
            dk[ks:ke, h // G] += b
            dv[ks:ke, h // G] += c
    return dq, dk, dv
