"""Pins for oracle O11 (gated delta rule with the state reset at every boundary).

Each pin checks the oracle against something other than its own formula: a
one-token closed form, the pure-decay closed form, an associative memory
simulated as a table of slots (one-hot keys), exact retrieval and overwrite
with orthonormal keys, an independent chunked (UT-transform) evaluation of the
same recurrence, and isolation between slices.  Planted mistakes (decay after
the write, S k instead of S^T k, reading before the write, no reset at a
boundary) must each fail one of them.
"""
import numpy as np
import pytest

from oracle import linear_attention as LA


def _rand(seed, T, H, dk, dv, gmin=-0.3):
    r = np.random.default_rng(seed)
    q = r.normal(size=(T, H, dk))
    k = r.normal(size=(T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = r.normal(size=(T, H, dv))
    g = r.uniform(gmin, 0.0, size=(T, H))
    beta = r.uniform(0.05, 1.0, size=(T, H))
    return q, k, v, g, beta


def test_one_token_closed_form():
    q, k, v, g, beta = _rand(1, 1, 1, 5, 3)
    o, s = LA.gated_delta_segment(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], 0.7)
    b = beta[0, 0]
    assert np.allclose(s, b * np.outer(k[0, 0], v[0, 0]), rtol=0, atol=1e-14)
    assert np.allclose(o[0], 0.7 * b * (k[0, 0] @ q[0, 0]) * v[0, 0], rtol=0, atol=1e-14)
    # with an initial state the decay applies to it before the write
    s0 = np.random.default_rng(2).normal(size=(5, 3))
    o, s = LA.gated_delta_segment(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], 0.7, s0)
    a = np.exp(g[0, 0])
    want = a * s0 + b * np.outer(k[0, 0], v[0, 0] - a * s0.T @ k[0, 0])
    assert np.allclose(s, want, rtol=0, atol=1e-13)


def test_pure_decay_closed_form():
    """beta = 0: nothing is written; the initial state only decays."""
    q, k, v, g, _ = _rand(3, 9, 1, 4, 6)
    s0 = np.random.default_rng(4).normal(size=(4, 6))
    o, s = LA.gated_delta_segment(q[:, 0], k[:, 0], v[:, 0], g[:, 0], np.zeros(9), 0.5, s0)
    cg = np.cumsum(g[:, 0])
    for t in range(9):
        assert np.allclose(o[t], 0.5 * np.exp(cg[t]) * s0.T @ q[t, 0], rtol=1e-12, atol=1e-14)
    assert np.allclose(s, np.exp(cg[-1]) * s0, rtol=1e-12)
    o, s = LA.gated_delta_segment(q[:, 0], k[:, 0], v[:, 0], g[:, 0], np.zeros(9), 0.5)
    assert not o.any() and not s.any()


def _table_memory(slots, vals, g, q, scale, dk):
    """One-hot keys with beta = 1: an associative table.  A write stores the
    value in its slot exactly; every stored value then decays by exp(g) per
    later token; a read mixes the slots with the query's weights."""
    table = {}
    out = []
    for t, (i, val) in enumerate(zip(slots, vals)):
        for j in table:
            table[j] = table[j] * np.exp(g[t])
        table[i] = val.copy()
        mix = sum(q[t][j] * table[j] for j in table)
        out.append(scale * mix)
    return np.array(out)


def test_one_hot_keys_are_a_decaying_table():
    r = np.random.default_rng(5)
    dk, dv, L = 6, 4, 40
    slots = r.integers(0, dk, size=L)
    k = np.eye(dk)[slots]
    v = r.normal(size=(L, dv))
    q = r.normal(size=(L, dk))
    g = r.uniform(-0.4, 0.0, size=L)
    o, s = LA.gated_delta_segment(q, k, v, g, np.ones(L), 0.9)
    want = _table_memory(slots, v, g, q, 0.9, dk)
    assert np.allclose(o, want, rtol=1e-12, atol=1e-13)


def test_orthonormal_keys_retrieve_and_overwrite(dv=5):
    """g = 0, beta = 1, orthonormal keys: reading with a stored key returns its
    value; writing the key again replaces the value."""
    r = np.random.default_rng(6)
    dk = 8
    basis, _ = np.linalg.qr(r.normal(size=(dk, dk)))
    keys = basis.T[:3]                      # three orthonormal keys
    vals = r.normal(size=(4, dv))
    k = np.stack([keys[0], keys[1], keys[2], keys[0]])   # key 0 written twice
    v = vals
    q = np.stack([keys[1], keys[0], keys[2], keys[0]])
    o, s = LA.gated_delta_segment(q, k, v, np.zeros(4), np.ones(4), 1.0)
    assert np.allclose(o[1], vals[0], atol=1e-12)          # key 0 before its overwrite
    assert np.allclose(o[2], vals[2], atol=1e-12)
    assert np.allclose(o[3], vals[3], atol=1e-12)          # overwritten value
    assert np.allclose(s.T @ keys[1], vals[1], atol=1e-12)


def test_orthonormal_keys_square_state():
    test_orthonormal_keys_retrieve_and_overwrite(dv=8)


def _chunked(q, k, v, g, beta, scale, C, s0=None):
    """The same recurrence evaluated chunk by chunk (the UT transform of the
    delta rule, with gates): inside a chunk of positions 0..c-1 with
    G_i = exp(sum_{j<=i} g_j) (the gate since the chunk start),
      (I + A) U = diag(beta) (V - diag(G) K S0),  A_ij = beta_i (G_i/G_j) k_i.k_j  (j < i),
      O = scale (diag(G) Q S0 + (Q K^T * D) U),   D_ij = G_i/G_j (j <= i), 0 otherwise,
      S_end = G_c S0 + (diag(G_c/G) K)^T U."""
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else s0.copy()
    out = np.zeros((L, dv))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        Q, K, V, gg, bb = q[sl], k[sl], v[sl], g[sl], beta[sl]
        n = K.shape[0]
        lg = np.cumsum(gg)
        Dm = np.exp(lg[:, None] - lg[None, :])
        A = np.tril(bb[:, None] * Dm * (K @ K.T), -1)
        rhs = bb[:, None] * (V - np.exp(lg)[:, None] * (K @ S))
        U = np.linalg.solve(np.eye(n) + A, rhs)
        out[sl] = scale * (np.exp(lg)[:, None] * (Q @ S) + (np.tril(Q @ K.T * Dm)) @ U)
        S = np.exp(lg[-1]) * S + (np.exp(lg[-1] - lg)[:, None] * K).T @ U
    return out, S


@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunked_form_agrees(C):
    q, k, v, g, beta = _rand(7, 150, 1, 16, 12, gmin=-0.2)
    s0 = np.random.default_rng(8).normal(size=(16, 12)) * 0.3
    o, s = LA.gated_delta_segment(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], 0.25, s0)
    oc, sc = _chunked(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], 0.25, C, s0)
    assert np.allclose(o, oc, rtol=1e-10, atol=1e-12)
    assert np.allclose(s, sc, rtol=1e-10, atol=1e-12)


def test_slices_are_isolated_and_reset():
    lengths = [7, 0, 13, 1, 20]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, dk, dv = int(cu[-1]), 2, 6, 5
    q, k, v, g, beta = _rand(9, T, H, dk, dv)
    s0 = np.random.default_rng(10).normal(size=(len(lengths), H, dk, dv))
    o, fin = LA.gated_delta_varlen(q, k, v, g, beta, cu, 0.5, s0)
    for b in range(len(lengths)):
        a, e = cu[b], cu[b + 1]
        for h in range(H):
            ob, sb = LA.gated_delta_segment(q[a:e, h], k[a:e, h], v[a:e, h], g[a:e, h], beta[a:e, h], 0.5,
                                            s0[b, h])
            assert np.array_equal(o[a:e, h], ob) and np.array_equal(fin[b, h], sb)
    assert np.array_equal(fin[1], s0[1])                    # empty slice keeps its initial state
    # NaN in one slice's inputs reaches no other slice
    v2 = v.copy()
    v2[cu[2]:cu[3]] = np.nan
    o2, fin2 = LA.gated_delta_varlen(q, k, v2, g, beta, cu, 0.5, s0)
    keep = np.ones(T, bool)
    keep[cu[2]:cu[3]] = False
    assert np.array_equal(o2[keep], o[keep])
    assert np.isnan(o2[~keep]).all()
    assert np.array_equal(np.delete(fin2, 2, axis=0), np.delete(fin, 2, axis=0))


def test_errors():
    q, k, v, g, beta = _rand(11, 5, 1, 3, 3)
    with pytest.raises(ValueError):
        LA.gated_delta_varlen(q, k, v, g, beta, [0, 3], 1.0)
    with pytest.raises(ValueError):
        LA.gated_delta_varlen(q, k, v, g, beta, [0, 4, 3, 5], 1.0)
    o, fin = LA.gated_delta_varlen(q[:0], k[:0], v[:0], g[:0], beta[:0], [0], 1.0)
    assert o.shape == (0, 1, 3) and fin.shape == (0, 1, 3, 3)


# ------------------------------------------------------------ planted mistakes

def _decay_after_write(q, k, v, g, beta, scale, s0=None):
    S = np.zeros((k.shape[1], v.shape[1])) if s0 is None else s0.copy()
    o = np.zeros((len(k), v.shape[1]))
    for t in range(len(k)):
        u = beta[t] * (v[t] - S.T @ k[t])
        S = np.exp(g[t]) * (S + np.outer(k[t], u))
        o[t] = scale * S.T @ q[t]
    return o, S


def _no_transpose(q, k, v, g, beta, scale, s0=None):
    # on square states this runs; on the others it is a shape error
    S = np.zeros((k.shape[1], v.shape[1])) if s0 is None else s0.copy()
    o = np.zeros((len(k), v.shape[1]))
    for t in range(len(k)):
        S = np.exp(g[t]) * S
        u = beta[t] * (v[t] - S @ k[t])
        S = S + np.outer(k[t], u)
        o[t] = scale * S.T @ q[t]
    return o, S


def _read_before_write(q, k, v, g, beta, scale, s0=None):
    S = np.zeros((k.shape[1], v.shape[1])) if s0 is None else s0.copy()
    o = np.zeros((len(k), v.shape[1]))
    for t in range(len(k)):
        S = np.exp(g[t]) * S
        o[t] = scale * S.T @ q[t]
        u = beta[t] * (v[t] - S.T @ k[t])
        S = S + np.outer(k[t], u)
    return o, S


@pytest.mark.parametrize("mutant", [_decay_after_write, _no_transpose, _read_before_write])
def test_planted_mistakes_fail_a_pin(mutant, monkeypatch):
    monkeypatch.setattr(LA, "gated_delta_segment", mutant)
    failed = 0
    for pin in (test_one_token_closed_form, test_one_hot_keys_are_a_decaying_table,
                test_orthonormal_keys_retrieve_and_overwrite, test_orthonormal_keys_square_state):
        try:
            pin()
        except (AssertionError, ValueError):    # a shape error also exposes the mistake
            failed += 1
    assert failed >= 1


def test_planted_missing_reset_fails_isolation(monkeypatch):
    real = LA.gated_delta_segment
    carry = {}

    def leaky(q, k, v, g, beta, scale, s0=None):
        o, s = real(q, k, v, g, beta, scale, carry.get("s", s0))
        carry["s"] = s
        return o, s
    monkeypatch.setattr(LA, "gated_delta_segment", leaky)
    with pytest.raises(AssertionError):
        test_slices_are_isolated_and_reset()


def test_grouped_heads_equal_repeated_heads():
    """H value heads over H_k query/key heads: the same as repeating each
    query/key head for its group (consecutive value heads share one)."""
    lengths = [9, 0, 14]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, Hk, G, dk, dv = int(cu[-1]), 2, 3, 5, 4
    q, k, _, _, _ = _rand(12, T, Hk, dk, dv)
    _, _, v, g, beta = _rand(13, T, Hk * G, dk, dv)
    o, fin = LA.gated_delta_varlen(q, k, v, g, beta, cu, 0.4)
    o2, fin2 = LA.gated_delta_varlen(np.repeat(q, G, axis=1), np.repeat(k, G, axis=1), v, g, beta, cu, 0.4)
    assert np.array_equal(o, o2) and np.array_equal(fin, fin2)
    with pytest.raises(ValueError):
        LA.gated_delta_varlen(q, k, v[:, :5], g[:, :5], beta[:, :5], cu, 0.4)


# ----------------------------------------------------------- O12 (backward)

def _loss_seg(q, k, v, g, beta, scale, do, s0, dsf):
    o, s = LA.gated_delta_segment(q, k, v, g, beta, scale, s0)
    return float(np.sum(o * do) + np.sum(s * dsf))


def _bwd_case(seed, L=6, dk=4, dv=3, gmin=-0.5):
    r = np.random.default_rng(seed)
    q = r.normal(size=(L, dk))
    k = r.normal(size=(L, dk)) / np.sqrt(dk)
    v = r.normal(size=(L, dv))
    g = r.uniform(gmin, 0.0, size=L)
    beta = r.uniform(0.1, 1.0, size=L)
    s0 = r.normal(size=(dk, dv)) * 0.5
    do = r.normal(size=(L, dv))
    dsf = r.normal(size=(dk, dv))
    return q, k, v, g, beta, s0, do, dsf


def _finite_differences(args, scale, h=1e-6):
    """Central differences of the loss for every entry of q, k, v, g, beta, s0."""
    q, k, v, g, beta, s0, do, dsf = args
    out = []
    for idx in range(6):
        base = [q, k, v, g, beta, s0]
        x = base[idx]
        grad = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            bp, bm = list(base), list(base)
            bp[idx], bm[idx] = xp, xm
            lp = _loss_seg(bp[0], bp[1], bp[2], bp[3], bp[4], scale, do, bp[5], dsf)
            lm = _loss_seg(bm[0], bm[1], bm[2], bm[3], bm[4], scale, do, bm[5], dsf)
            grad[pos] = (lp - lm) / (2 * h)
        out.append(grad)
    return out


def _order(r):
    """(dq, dk, dv, dg, dbeta, ds0) -> the input order q, k, v, g, beta, s0."""
    return [r[0], r[1], r[2], r[3], r[4], r[5]]


def test_backward_matches_finite_differences():
    for seed in range(3):
        args = _bwd_case(10 + seed)
        q, k, v, g, beta, s0, do, dsf = args
        got = _order(LA.gated_delta_segment_backward(q, k, v, g, beta, 0.6, do, s0, dsf))
        fd = _finite_differences(args, 0.6)
        for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "ds0"), got, fd):
            assert np.abs(a - b).max() <= 1e-7 * max(1.0, np.abs(b).max()), name


def test_backward_matches_torch_autograd():
    """torch fp64 autograd through the token loop (a library differentiation
    of the forward, not of the backward's formulas)."""
    torch = pytest.importorskip("torch")
    args = _bwd_case(20, L=17, dk=8, dv=5)
    q, k, v, g, beta, s0, do, dsf = args
    T = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, g, beta, s0)]
    tq, tk, tv, tg, tb, ts0 = T
    S = ts0
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(q.shape[0]):
        S = torch.exp(tg[t]) * S
        u = tb[t] * (tv[t] - S.T @ tk[t])
        S = S + torch.outer(tk[t], u)
        loss = loss + (0.3 * (S.T @ tq[t])) @ torch.tensor(do[t])
    loss = loss + (S * torch.tensor(dsf)).sum()
    loss.backward()
    got = _order(LA.gated_delta_segment_backward(q, k, v, g, beta, 0.3, do, s0, dsf))
    for name, a, t in zip(("dq", "dk", "dv", "dg", "dbeta", "ds0"), got, T):
        assert np.allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-12), name


def test_backward_pure_decay_closed_forms():
    """beta = 0: o_t = scale e^{c_t} S0^T q_t with c_t = g_0 + .. + g_t and the
    final state e^{c_L} S0, so dq_t = scale e^{c_t} S0 do_t, dv = 0, dk = 0,
    dS0 = sum_t scale e^{c_t} q_t do_t^T + e^{c_L} dS_final and
    dg_t = sum_{t' >= t} scale e^{c_t'} (S0^T q_t').do_t' + e^{c_L} <S0, dS_final>."""
    q, k, v, g, _, s0, do, dsf = _bwd_case(30, L=7)
    L = q.shape[0]
    dq, dk, dv, dg, dbeta, ds0 = LA.gated_delta_segment_backward(q, k, v, g, np.zeros(L), 0.5, do, s0, dsf)
    c = np.cumsum(g)
    for t in range(L):
        assert np.allclose(dq[t], 0.5 * np.exp(c[t]) * s0 @ do[t], rtol=1e-12, atol=1e-14)
    assert not dv.any() and np.abs(dk).max() == 0.0
    want_ds0 = sum(0.5 * np.exp(c[t]) * np.outer(q[t], do[t]) for t in range(L)) + np.exp(c[-1]) * dsf
    assert np.allclose(ds0, want_ds0, rtol=1e-12, atol=1e-14)
    term = [0.5 * np.exp(c[t]) * (s0.T @ q[t]) @ do[t] for t in range(L)]
    for t in range(L):
        want = sum(term[t:]) + np.exp(c[-1]) * np.sum(s0 * dsf)
        assert np.isclose(dg[t], want, rtol=1e-12, atol=1e-13)
    # dbeta_t = (dS_t^T k_t) . (v_t - e^{c_t} S0^T k_t), dS_t the gradient of S_t
    for t in range(L):
        dSt = sum(0.5 * np.exp(c[u] - c[t]) * np.outer(q[u], do[u]) for u in range(t, L)) \
            + np.exp(c[-1] - c[t]) * dsf
        assert np.isclose(dbeta[t], (dSt.T @ k[t]) @ (v[t] - np.exp(c[t]) * s0.T @ k[t]), rtol=1e-11, atol=1e-13)


def test_backward_planted_mistakes_fail():
    """Three plausible slips in the backward, each caught by finite differences."""
    args = _bwd_case(40)
    q, k, v, g, beta, s0, do, dsf = args
    fd = _finite_differences(args, 0.6)

    def mutant(kind):
        L, dk_ = k.shape
        S = s0.copy()
        keep = []
        for t in range(L):
            Sd = np.exp(g[t]) * S
            pred = Sd.T @ k[t]
            u = beta[t] * (v[t] - pred)
            keep.append((S, Sd, pred, u, Sd + np.outer(k[t], u)))
            S = keep[-1][4]
        dq, dk = np.zeros_like(q), np.zeros_like(k)
        dS = dsf.copy()
        for t in range(L - 1, -1, -1):
            Sp, Sd, pred, u, St = keep[t]
            dS = dS + 0.6 * np.outer(q[t], do[t])
            dq[t] = 0.6 * ((Sp if kind == "read_before_write" else St) @ do[t])
            du = dS.T @ k[t]
            dk[t] = dS @ u
            dpred = -beta[t] * du
            dSd = dS + np.outer(k[t], dpred)
            if kind != "no_pred_term":
                dk[t] += Sd @ dpred
            dS = dSd if kind == "no_decay" else np.exp(g[t]) * dSd
        return dq, dk
    for kind in ("read_before_write", "no_pred_term", "no_decay"):
        mq, mk = mutant(kind)
        bad = np.abs(mq - fd[0]).max() > 1e-5 or np.abs(mk - fd[1]).max() > 1e-5
        assert bad, kind


def test_backward_varlen_isolation_empty_slices_and_grouped_heads():
    """Slices are independent (NaN in one slice leaves the others' gradients
    exact), an empty slice passes its final-state gradient through to its
    initial state, and grouped heads equal the call with repeated query/key
    heads, summed over each group."""
    r = np.random.default_rng(50)
    lengths = [5, 0, 7, 3]
    T, H, Hk, dk, dv = sum(lengths), 4, 2, 4, 3
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q = r.normal(size=(T, Hk, dk))
    k = r.normal(size=(T, Hk, dk)) / 2
    v = r.normal(size=(T, H, dv))
    g = r.uniform(-0.4, 0, size=(T, H))
    beta = r.uniform(0.1, 1, size=(T, H))
    h0 = r.normal(size=(4, H, dk, dv))
    do = r.normal(size=(T, H, dv))
    dht = r.normal(size=(4, H, dk, dv))
    dq, dk_, dv_, dg, db, dh0 = LA.gated_delta_varlen_backward(q, k, v, g, beta, cu, 0.5, do, h0, dht)
    assert np.array_equal(dh0[1], dht[1])                       # the empty slice
    # repeated heads, summed per group
    G = H // Hk
    qr, kr = np.repeat(q, G, axis=1), np.repeat(k, G, axis=1)
    rq, rk, rv, rg, rb, rh = LA.gated_delta_varlen_backward(qr, kr, v, g, beta, cu, 0.5, do, h0, dht)
    assert np.allclose(dq, rq.reshape(T, Hk, G, dk).sum(2), rtol=1e-13, atol=1e-13)
    assert np.allclose(dk_, rk.reshape(T, Hk, G, dk).sum(2), rtol=1e-13, atol=1e-13)
    assert np.array_equal(dv_, rv) and np.array_equal(dg, rg) and np.array_equal(dh0, rh)
    # NaN in slice 2 (tokens 5..11) changes nothing in slices 0 and 3
    v2 = v.copy()
    v2[6, :, 0] = np.nan
    n = LA.gated_delta_varlen_backward(q, k, v2, g, beta, cu, 0.5, do, h0, dht)
    for a, b in zip(n, (dq, dk_, dv_, dg, db)):
        assert np.array_equal(a[:5], b[:5]) and np.array_equal(a[12:], b[12:])
    assert np.array_equal(n[5][[0, 1, 3]], dh0[[0, 1, 3]])
