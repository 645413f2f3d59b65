"""Pins for oracle O5-O7 (packed block-causal attention, fp64); CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import packing as P

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(T, H, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d)),
            rng.standard_normal((T, H, d)))


def _close(a, b, abs_tol=1e-10, rel=1e-9):
    """The pages' equivalence tolerance: abs 1e-10 + rel 1e-9 * max|x|."""
    scale = max(np.abs(a).max(initial=0.0), np.abs(b).max(initial=0.0))
    return np.abs(a - b).max(initial=0.0) <= abs_tol + rel * scale


# ----------------------------------------------------------- O5 vs O7

def test_forward_equals_brute_force_dense_mask():
    rng = np.random.default_rng(0)
    for trial in range(20):
        lengths = rng.integers(0, 7, size=int(rng.integers(1, 6))).tolist()
        if sum(lengths) == 0:
            lengths.append(1)
        T, H, d = sum(lengths), 2, 8
        q, k, v = _rand(T, H, d, trial)
        md = P.packed_row_metadata(lengths)
        o, _ = A.varlen_forward(q, k, v, md["cu"])
        od = A.dense_masked_forward(q, k, v, md["seg"], md["pos"], np.ones(T, bool))
        assert _close(o, od), lengths


def test_three_representations_agree():
    """separate per-segment calls == padded rows with validity == packed flat stream."""
    lengths = [5, 3, 4]
    T, H, d = 12, 2, 16
    q, k, v = _rand(T, H, d, 1)
    cu = P.packed_row_metadata(lengths)["cu"]
    packed, _ = A.varlen_forward(q, k, v, cu)
    sep = np.zeros_like(packed)
    pad = np.zeros_like(packed)
    W = max(lengths)
    for b in range(3):
        s, e = int(cu[b]), int(cu[b + 1])
        for h in range(H):
            sep[s:e, h], _ = A.segment_head_forward(q[s:e, h], k[s:e, h], v[s:e, h], 1 / math.sqrt(d))
        # one right-padded row of width W, junk in the padding
        qq = np.full((W, H, d), 7.0); kk = np.full((W, H, d), -3.0); vv = np.full((W, H, d), 1e3)
        qq[:e - s], kk[:e - s], vv[:e - s] = q[s:e], k[s:e], v[s:e]
        valid = np.arange(W) < (e - s)
        o_row = A.dense_masked_forward(qq, kk, vv, np.where(valid, 0, -1), np.where(valid, np.arange(W), 0), valid)
        assert np.all(o_row[~valid] == 0.0)          # inactive queries: zero mixture
        pad[s:e] = o_row[:e - s]
    assert _close(packed, sep)
    assert _close(packed, pad)


def test_merged_boundary_changes_only_the_merged_slice():
    g = json.load(open(os.path.join(GOLD, "worked_5_3_4.json")))
    q, k, v = _rand(12, 2, 64, 2)
    o3, _ = A.varlen_forward(q, k, v, g["cu_seqlens"])
    o2, _ = A.varlen_forward(q, k, v, g["merged_cu_seqlens"])
    # A is untouched; B's queries come first in B+C, so causality hides C from them
    assert _close(o3[:8], o2[:8])
    # C's queries now see B's keys
    assert np.abs(o3[8:] - o2[8:]).min() > 1e-6
    # and the three slices are independent attentions
    for s, e in [(0, 5), (5, 8), (8, 12)]:
        o_alone, _ = A.varlen_forward(q[s:e], k[s:e], v[s:e], [0, e - s])
        assert _close(o_alone, o3[s:e])


def test_closed_forms():
    d = 16
    scale = 1 / math.sqrt(d)
    q, k, v = _rand(1, 1, d, 3)
    o, lse = A.varlen_forward(q, k, v, [0, 1])
    assert np.allclose(o, v, rtol=0, atol=1e-15)                 # L = 1: O = v
    assert math.isclose(lse[0, 0], scale * float(q[0, 0] @ k[0, 0]), rel_tol=1e-14)
    # all keys equal: uniform softmax, O_i = prefix mean of v, LSE_i = s + ln(i+1)
    L = 9
    qq, _, vv = _rand(L, 1, d, 4)
    kk = np.repeat(np.random.default_rng(5).standard_normal((1, 1, d)), L, axis=0)
    o, lse = A.varlen_forward(qq, kk, vv, [0, L])
    pref = np.cumsum(vv[:, 0], axis=0) / np.arange(1, L + 1)[:, None]
    assert np.allclose(o[:, 0], pref, rtol=0, atol=1e-13)
    s = scale * (qq[:, 0] @ kk[0, 0])
    assert np.allclose(lse[0], s + np.log(np.arange(1, L + 1)), rtol=0, atol=1e-12)


def test_matches_torch_sdpa_with_explicit_mask():
    lengths = [37, 1, 0, 64, 15]
    T, H, d = sum(lengths), 3, 32
    q, k, v = _rand(T, H, d, 6)
    md = P.packed_row_metadata(lengths)
    o, _ = A.varlen_forward(q, k, v, md["cu"])
    seg = torch.tensor(md["seg"]); pos = torch.tensor(md["pos"])
    mask = (seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None])
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).contiguous() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    assert np.abs(o - ref.permute(1, 0, 2).numpy()).max() < 1e-12


def test_isolation_and_lse_bounds():
    lengths = [6, 9]
    q, k, v = _rand(15, 2, 8, 7)
    o, lse = A.varlen_forward(q, k, v, [0, 6, 15])
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:6] += 5.0; k2[:6] *= -3.0; v2[:6] = 1e6         # perturb segment A only
    o2, lse2 = A.varlen_forward(q2, k2, v2, [0, 6, 15])
    assert np.array_equal(o[6:], o2[6:]) and np.array_equal(lse[:, 6:], lse2[:, 6:])
    # LSE >= max permitted score, and <= max + ln(count)
    for h in range(2):
        for t in range(15):
            s0 = 0 if t < 6 else 6
            sc = (k[s0:t + 1, h] @ q[t, h]) / math.sqrt(8)
            assert sc.max() - 1e-12 <= lse[h, t] <= sc.max() + math.log(t - s0 + 1) + 1e-12


def test_forward_rows_equals_full_forward():
    lengths = [13, 0, 40, 7]
    T = sum(lengths)
    q, k, v = _rand(T, 2, 16, 8)
    cu = P.packed_row_metadata(lengths)["cu"]
    o, lse = A.varlen_forward(q, k, v, cu)
    rows = [0, 12, 13, 30, 52, 59]
    heads = [0, 1, 1, 0, 1, 0]
    orow, lrow = A.forward_rows(q, k, v, cu, rows, heads)
    for n, (t, h) in enumerate(zip(rows, heads)):
        assert np.allclose(orow[n], o[t, h], rtol=0, atol=1e-13)
        assert math.isclose(lrow[n], lse[h, t], rel_tol=0, abs_tol=1e-12)


def test_forward_rows_grouped_heads():
    """Grouped key/value heads (first page, section 5: the key view carries
    h_k heads): query head h of forward_rows reads key/value head h // (H / H_k),
    as varlen_forward does; a planted mutant that reads the query head's own
    index fails."""
    lengths = [9, 0, 17, 5]
    T, H, Hk, d = sum(lengths), 6, 2, 8
    rng = np.random.default_rng(7)
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, Hk, d))
    v = rng.standard_normal((T, Hk, d))
    cu = P.packed_row_metadata(lengths)["cu"]
    o, lse = A.varlen_forward(q, k, v, cu)
    rows = [0, 8, 9, 20, 25, 30, 26, 3]
    heads = [0, 5, 1, 2, 3, 4, 5, 2]
    orow, lrow = A.forward_rows(q, k, v, cu, rows, heads)
    for n, (t, h) in enumerate(zip(rows, heads)):
        assert np.allclose(orow[n], o[t, h], rtol=0, atol=1e-13)
        assert math.isclose(lrow[n], lse[h, t], rel_tol=0, abs_tol=1e-12)

    # mutant: K/V indexed by the query head modulo H_k (a plausible slip)
    def wrong(t, h):
        start = max(c for c in [int(x) for x in cu[:-1]] if c <= t)
        sc = (k[start:t + 1, h % Hk] @ q[t, h]) / math.sqrt(d)
        e = np.exp(sc - sc.max())
        return (e / e.sum()) @ v[start:t + 1, h % Hk]
    assert any(not np.allclose(wrong(t, h), o[t, h], rtol=0, atol=1e-6) for t, h in zip(rows, heads))


# ----------------------------------------------------------- O6

def _loss(q, k, v, do, cu):
    o, _ = A.varlen_forward(q, k, v, cu)
    return float((o * do).sum())


def test_backward_finite_differences():
    lengths = [3, 0, 5, 1]
    T, H, d = sum(lengths), 2, 4
    q, k, v = _rand(T, H, d, 9)
    do = np.random.default_rng(10).standard_normal((T, H, d))
    cu = P.packed_row_metadata(lengths)["cu"]
    dq, dk, dv = A.varlen_backward(q, k, v, do, cu)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, cu)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, cu)
            assert abs((lp - lm) / (2 * eps) - g[idx]) < 1e-7, (name, idx)


def test_backward_closed_forms_and_isolation():
    d = 8
    q, k, v = _rand(1, 1, d, 11)
    do = np.random.default_rng(12).standard_normal((1, 1, d))
    dq, dk, dv = A.varlen_backward(q, k, v, do, [0, 1])
    assert np.all(dq == 0) and np.all(dk == 0) and np.array_equal(dv, do)
    # cross-segment derivatives are exactly zero: B's loss does not reach A
    q, k, v = _rand(10, 2, d, 13)
    do = np.zeros((10, 2, d)); do[4:] = 1.0
    dq, dk, dv = A.varlen_backward(q, k, v, do, [0, 4, 10])
    assert np.all(dq[:4] == 0) and np.all(dk[:4] == 0) and np.all(dv[:4] == 0)


def test_backward_matches_torch_autograd():
    lengths = [20, 1, 33, 0, 9]
    T, H, d = sum(lengths), 2, 16
    q, k, v = _rand(T, H, d, 14)
    do = np.random.default_rng(15).standard_normal((T, H, d))
    md = P.packed_row_metadata(lengths)
    dq, dk, dv = A.varlen_backward(q, k, v, do, md["cu"])
    seg = torch.tensor(md["seg"]); pos = torch.tensor(md["pos"])
    mask = (seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None])
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).contiguous().requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    out.backward(torch.from_numpy(do).permute(1, 0, 2))
    for mine, ref in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(mine - ref.grad.permute(1, 0, 2).numpy()).max() < 1e-11


# ----------------------------------------------------------- pin sensitivity

def test_pins_catch_planted_mistakes(monkeypatch):
    """A plausible slip in O5 (strict causality, a dropped boundary, a wrong
    scale) must fail the brute-force and library pins above."""
    lengths = [5, 3, 4]
    T, H, d = 12, 2, 8
    q, k, v = _rand(T, H, d, 16)
    md = P.packed_row_metadata(lengths)
    ref = A.dense_masked_forward(q, k, v, md["seg"], md["pos"], np.ones(T, bool))

    def strict(qs, ks, vs, scale):       # key j < i instead of j <= i
        L = qs.shape[0]
        out = np.zeros_like(qs)
        for i in range(L):
            if i == 0:
                continue
            sc = scale * (ks[:i] @ qs[i])
            e = np.exp(sc - sc.max())
            out[i] = (e / e.sum()) @ vs[:i]
        return out, np.zeros(L)

    monkeypatch.setattr(A, "segment_head_forward", strict)
    o, _ = A.varlen_forward(q, k, v, md["cu"])
    assert not _close(o, ref)
    monkeypatch.undo()
    o, _ = A.varlen_forward(q, k, v, [0, 12])          # boundary dropped
    assert not _close(o, ref)
    o, _ = A.varlen_forward(q, k, v, md["cu"], scale=1.0)  # scale forgotten
    assert not _close(o, ref)


# ------------------------------------------------ grouped key/value heads

def _gqa_inputs(lengths, H, Hk, d, seed):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, Hk, d))
    v = rng.standard_normal((T, Hk, d))
    do = rng.standard_normal((T, H, d))
    return q, k, v, do


def test_grouped_heads_match_torch_with_repeated_kv():
    """H = 6 query heads over H_k = 2 key/value heads: torch fp64 SDPA on K/V
    repeated per query head (repeat_interleave), with autograd summing the
    key/value gradients over each group."""
    lengths = [17, 0, 30, 1, 12]
    H, Hk, d = 6, 2, 16
    q, k, v, do = _gqa_inputs(lengths, H, Hk, d, 41)
    md = P.packed_row_metadata(lengths)
    o, _ = A.varlen_forward(q, k, v, md["cu"])
    dq, dk, dv = A.varlen_backward(q, k, v, do, md["cu"])
    assert dk.shape == k.shape and dv.shape == v.shape
    seg = torch.tensor(md["seg"]); pos = torch.tensor(md["pos"])
    mask = (seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None])
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).contiguous().requires_grad_() for x in (q, k, v))
    G = H // Hk
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=0), tv.repeat_interleave(G, dim=0), attn_mask=mask)
    assert np.abs(o - out.detach().permute(1, 0, 2).numpy()).max() < 1e-12
    out.backward(torch.from_numpy(do).permute(1, 0, 2))
    for mine, ref in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(mine - ref.grad.permute(1, 0, 2).numpy()).max() < 1e-11


def test_grouped_heads_finite_differences_on_shared_kv():
    """dK of a shared head by central differences of sum(O * dO) (tiny case)."""
    lengths = [4, 3]
    H, Hk, d = 4, 2, 3
    q, k, v, do = _gqa_inputs(lengths, H, Hk, d, 42)
    cu = P.cu_seqlens_from_lengths(lengths)
    _, dk, dv = A.varlen_backward(q, k, v, do, cu)
    f = lambda kk, vv: float((A.varlen_forward(q, kk, vv, cu)[0] * do).sum())
    h = 1e-6
    for idx in [(0, 0, 0), (2, 1, 2), (5, 0, 1), (6, 1, 0)]:
        kp, km = k.copy(), k.copy()
        kp[idx] += h
        km[idx] -= h
        assert abs((f(kp, v) - f(km, v)) / (2 * h) - dk[idx]) < 1e-7
        vp, vm = v.copy(), v.copy()
        vp[idx] += h
        vm[idx] -= h
        assert abs((f(k, vp) - f(k, vm)) / (2 * h) - dv[idx]) < 1e-7


def test_grouped_heads_reject_uneven_groups():
    q, k, v, _ = _gqa_inputs([5], 3, 2, 4, 43)
    with pytest.raises(ValueError):
        A.varlen_forward(q, k, v, [0, 5])


# ------------------------------------- separate query/key extents, windows

def _cross_inputs(lq, lk, H, Hk, d, seed):
    rng = np.random.default_rng(seed)
    Tq, Tk = sum(lq), sum(lk)
    return (rng.standard_normal((Tq, H, d)), rng.standard_normal((Tk, Hk, d)),
            rng.standard_normal((Tk, Hk, d)), rng.standard_normal((Tq, H, d)))


def test_band_self_causal_equals_causal_oracle():
    lengths = [37, 1, 0, 64, 15]
    q, k, v, do = _cross_inputs(lengths, lengths, 3, 3, 16, 51)
    cu = P.cu_seqlens_from_lengths(lengths)
    o1, l1 = A.varlen_forward(q, k, v, cu)
    o2, l2 = A.varlen_cross_forward(q, k, v, cu, cu)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12
    g1 = A.varlen_backward(q, k, v, do, cu)
    g2 = A.varlen_cross_backward(q, k, v, do, cu, cu)
    for a, b in zip(g1, g2):
        assert np.abs(a - b).max() < 1e-11


def _torch_band_mask(lq, lk, wl, wr):
    """The permission written with torch index ops, per slice, as a dense
    block-diagonal [T_q, T_k] mask."""
    Tq, Tk = sum(lq), sum(lk)
    mask = torch.zeros((Tq, Tk), dtype=torch.bool)
    q0 = k0 = 0
    for a, b in zip(lq, lk):
        i = torch.arange(a)[:, None]
        j = torch.arange(b)[None, :]
        m = torch.ones((a, b), dtype=torch.bool)
        if wr >= 0:
            m &= j - i <= (b - a) + wr
        if wl >= 0:
            m &= j - i >= (b - a) - wl
        mask[q0:q0 + a, k0:k0 + b] = m
        q0 += a
        k0 += b
    return mask


@pytest.mark.parametrize("lq,lk,window", [
    ([9, 20, 5, 0], [20, 9, 5, 3], (-1, 0)),      # cross, causal aligned bottom-right
    ([9, 20, 5], [20, 9, 5], (-1, -1)),           # cross, no clamp
    ([30, 17], [30, 17], (4, 0)),                 # self, sliding window of 4 back
    ([12, 25], [25, 12], (3, 2)),                 # cross, two-sided local window
])
def test_band_matches_torch_sdpa_and_autograd(lq, lk, window):
    H, Hk, d = 4, 2, 8
    q, k, v, do = _cross_inputs(lq, lk, H, Hk, d, 52)
    cq, ck = P.cu_seqlens_from_lengths(lq), P.cu_seqlens_from_lengths(lk)
    o, lse = A.varlen_cross_forward(q, k, v, cq, ck, window=window)
    dq, dk, dv = A.varlen_cross_backward(q, k, v, do, cq, ck, window=window)
    mask = _torch_band_mask(lq, lk, *window)
    rows = mask.any(dim=1)                          # queries with a permitted key
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).contiguous().requires_grad_() for x in (q, k, v))
    G = H // Hk
    kk, vv = tk.repeat_interleave(G, dim=0), tv.repeat_interleave(G, dim=0)
    out = torch.nn.functional.scaled_dot_product_attention(tq[:, rows], kk, vv, attn_mask=mask[rows])
    ref = out.detach().permute(1, 0, 2).numpy()
    assert np.abs(o[rows.numpy()] - ref).max() < 1e-12
    assert np.all(o[~rows.numpy()] == 0) and np.all(np.isneginf(lse[:, ~rows.numpy()]))
    out.backward(torch.from_numpy(do[rows.numpy()]).permute(1, 0, 2))
    for mine, ref_t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(mine - ref_t.grad.permute(1, 0, 2).numpy()).max() < 1e-11


def test_band_closed_form_single_key_window():
    """window (0, 0): query i sees exactly key i + L_k - L_q, so O_i = v of that
    key and LSE_i = scale q_i . k; queries with no such key get zeros."""
    lq, lk = [6, 4], [4, 7]
    q, k, v, _ = _cross_inputs(lq, lk, 2, 2, 5, 53)
    cq, ck = P.cu_seqlens_from_lengths(lq), P.cu_seqlens_from_lengths(lk)
    o, lse = A.varlen_cross_forward(q, k, v, cq, ck, window=(0, 0))
    s = 1 / math.sqrt(5)
    for b in range(2):
        for i in range(lq[b]):
            j = i + lk[b] - lq[b]
            t = cq[b] + i
            if 0 <= j < lk[b]:
                assert np.allclose(o[t], v[ck[b] + j]) and np.allclose(lse[:, t], s * (q[t] * k[ck[b] + j]).sum(-1))
            else:
                assert np.all(o[t] == 0) and np.all(np.isneginf(lse[:, t]))


def test_band_finite_differences():
    lq, lk = [5, 3], [3, 6]
    q, k, v, do = _cross_inputs(lq, lk, 2, 1, 3, 54)
    cq, ck = P.cu_seqlens_from_lengths(lq), P.cu_seqlens_from_lengths(lk)
    w = (2, 1)
    dq, dk, dv = A.varlen_cross_backward(q, k, v, do, cq, ck, window=w)
    f = lambda qq, kk, vv: float((A.varlen_cross_forward(qq, kk, vv, cq, ck, window=w)[0] * do).sum())
    h = 1e-6
    for arr, grad, idx in ((q, dq, (1, 1, 2)), (q, dq, (6, 0, 0)), (k, dk, (4, 0, 1)), (v, dv, (7, 0, 2))):
        ap, am = arr.copy(), arr.copy()
        ap[idx] += h
        am[idx] -= h
        args_p = [ap if x is arr else x for x in (q, k, v)]
        args_m = [am if x is arr else x for x in (q, k, v)]
        assert abs((f(*args_p) - f(*args_m)) / (2 * h) - grad[idx]) < 1e-7
