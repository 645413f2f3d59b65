"""GPU parity of the next-row readings at the sizes and in the launch
configurations the benchmark times, on outputs the oracle can afford: whole
sampled heads (attention), sampled rows (the loss); the properties that hold
at any size check the rest."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import loss_probe as LP
from tests.parity import check, dev_bf16, host_cu, say, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import packed_varlen_block_amd  # noqa: F401  (fails loudly if libpvb.so is missing)


def _dev_cu(h):
    import torch
    return torch.tensor(np.asarray(h, dtype=np.int32)).cuda()


def test_grouped_heads_bench_config():
    """T=8192 single slice, 32 query heads over 8 key/value heads, d=128, O bf16,
    fp32 gradients; query heads 0 and 13 (O, LSE, dQ) and key/value head 3
    (dK, dV: the sum over query heads 12-15) compared in full."""
    import packed_varlen_block_amd as pvb
    import torch
    say("gqa T=8192 H=32 H_kv=8 d=128 (query heads 0, 13; key/value head 3)")
    qb, kb, vb, db = W.random_cross(1001, [8192], [8192], 32, 8, 128, scale=0.5)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(db)
    cu = _dev_cu([0, 8192])
    o, lse, st = pvb.varlen_attn_fwd(q, k, v, cu)
    pvb.check_status(st)
    dq, dk, dv, st = pvb.varlen_attn_bwd(q, k, v, o, do, lse, cu, grad_dtype=torch.float32)
    pvb.check_status(st)
    qo, ko, vo, doo = (W.bf16_bits_to_f64(x) for x in (qb, kb, vb, db))
    ro, rl = A.varlen_forward(qo, ko, vo, [0, 8192], heads=[0, 13])
    check("O", to64(o)[:, [0, 13]], ro[:, [0, 13]])
    check("LSE", lse.double().cpu().numpy()[[0, 13]], rl[[0, 13]], max_abs=1e-3, mean_abs=1e-4)
    rq, rk, rv = A.varlen_backward(qo, ko, vo, doo, [0, 8192], heads=[0, 12, 13, 14, 15])
    check("dQ", to64(dq)[:, [0, 13]], rq[:, [0, 13]])
    check("dK", to64(dk)[:, 3], rk[:, 3])
    check("dV", to64(dv)[:, 3], rv[:, 3])


@pytest.mark.parametrize("case", ["window1024_T8192", "prefill_q2048_k8192_x4"])
def test_cross_and_window_bench_config_forward(case):
    """The two band readings (H=32, d=128, O bf16), forward, heads 0 and 31 in full."""
    import packed_varlen_block_amd as pvb
    lq, lk, win = {"window1024_T8192": ([8192], [8192], (1023, 0)),
                   "prefill_q2048_k8192_x4": ([2048] * 4, [8192] * 4, (-1, 0))}[case]
    say(f"band reading {case}: heads 0, 31")
    qb, kb, vb, _ = W.random_cross(1002, lq, lk, 32, 32, 128, scale=0.5, backward=False)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    hq, hk = host_cu(lq), host_cu(lk)
    o, lse, st = pvb.varlen_cross_attn_fwd(q, k, v, _dev_cu(hq), _dev_cu(hk), hq, hk, window=win)
    pvb.check_status(st)
    heads = [0, 31]
    qo, ko, vo = (W.bf16_bits_to_f64(x)[:, heads] for x in (qb, kb, vb))
    ro, rl = A.varlen_cross_forward(qo, ko, vo, hq, hk, window=win)
    check("O", to64(o)[:, heads], ro)
    check("LSE", lse.double().cpu().numpy()[heads], rl, max_abs=1e-3, mean_abs=1e-4)


def _band_reading_backward(case):
    """The band reading's inputs and its GPU forward and backward (H=32,
    d=128, O bf16, fp32 gradients, dO ~ N(0,1)), launched as the benchmark
    launches them."""
    import packed_varlen_block_amd as pvb
    import torch
    lq, lk, win = {"window1024_T8192": ([8192], [8192], (1023, 0)),
                   "prefill_q2048_k8192_x4": ([2048] * 4, [8192] * 4, (-1, 0))}[case]
    qb, kb, vb, db = W.random_cross(1004, lq, lk, 32, 32, 128, scale=0.5)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(db)
    hq, hk = host_cu(lq), host_cu(lk)
    cq, ck = _dev_cu(hq), _dev_cu(hk)
    o, lse, st = pvb.varlen_cross_attn_fwd(q, k, v, cq, ck, hq, hk, window=win)
    pvb.check_status(st)
    dq, dk, dv, st = pvb.varlen_cross_attn_bwd(q, k, v, o, do, lse, cq, ck, hq, hk, window=win,
                                               grad_dtype=torch.float32)
    pvb.check_status(st)
    f = W.bf16_bits_to_f64
    return (f(qb), f(kb), f(vb), f(db)), (to64(dq), to64(dk), to64(dv))


def test_window_bench_config_backward():
    """The 1024-key causal window over the T=8192 slice, backward, heads 0 and
    31.  Every row's keys lie within the 1023 before it, so the band oracle
    runs on two sub-streams that reproduce those bands exactly: queries
    [a, b) over keys [max(0, a - 1023), b) with the same window, aligned to
    the bottom right (for a >= 1023 the offset L_k - L_q = 1023 puts local
    row r' on local keys r' .. r' + 1023, i.e. global r - 1023 .. r).  There
    dQ of every row in [a, b) is exact, and dK, dV of every key whose rows
    (its own through 1023 after it) all lie in [a, b)."""
    say("band reading window1024_T8192: backward, heads 0 and 31, two sub-streams")
    (qo, ko, vo, doo), (dq, dk, dv) = _band_reading_backward("window1024_T8192")
    for a, b in ((0, 1280), (6912, 8192)):
        ka = max(0, a - 1023)
        keys_exact = slice(a, b) if b == 8192 else slice(a, b - 1023)
        for h in (0, 31):
            sub = lambda x: x[:, [h]]
            rq, rk, rv = A.varlen_cross_backward(sub(qo[a:b]), sub(ko[ka:b]), sub(vo[ka:b]), sub(doo[a:b]),
                                                 [0, b - a], [0, b - ka], window=(1023, 0))
            check(f"rows {a}-{b} h{h} dQ", dq[a:b, [h]], rq)
            ks = slice(keys_exact.start - ka, keys_exact.stop - ka)
            check(f"keys {keys_exact.start}-{keys_exact.stop} h{h} dK", dk[keys_exact, [h]], rk[ks])
            check(f"keys {keys_exact.start}-{keys_exact.stop} h{h} dV", dv[keys_exact, [h]], rv[ks])


def test_prefill_bench_config_backward():
    """Four slices of 2048 queries over 8192 keys with the causal clamp aligned
    to the bottom right, backward: slice 0 on head 0 and slice 3 on head 31, in
    full.  A slice's query r sees keys 0 .. r + 6144, which is row r + 6144 of
    causal self-attention over its 8192 keys; so the causal self oracle runs on
    the slice with its queries placed at rows 6144-8191 and zero queries and dO
    above them (whose rows then add nothing to dK and dV: dS = 0 where dO = 0)."""
    say("band reading prefill_q2048_k8192_x4: backward, slice 0 head 0, slice 3 head 31")
    (qo, ko, vo, doo), (dq, dk, dv) = _band_reading_backward("prefill_q2048_k8192_x4")
    for sl, h in ((0, 0), (3, 31)):
        qs, ks = slice(2048 * sl, 2048 * (sl + 1)), slice(8192 * sl, 8192 * (sl + 1))
        qf = np.zeros((8192, 1, 128))
        gf = np.zeros((8192, 1, 128))
        qf[6144:, 0] = qo[qs, h]
        gf[6144:, 0] = doo[qs, h]
        rq, rk, rv = A.varlen_backward(qf, ko[ks, [h]], vo[ks, [h]], gf, [0, 8192])
        check(f"slice {sl} h{h} dQ", dq[qs, [h]], rq[6144:])
        check(f"slice {sl} h{h} dK", dk[ks, [h]], rk)
        check(f"slice {sl} h{h} dV", dv[ks, [h]], rv)


def test_packed_loss_bench_config_sampled_rows():
    """C=8192 cells over a 32768 vocabulary, bf16 logits N(0,1)*2 with about 1%
    of the cells ignored, bf16 gradient (the reading's configuration): 96
    sampled rows against O10; the count exactly; the sum and mean against the
    fp64 sum of the row values."""
    import packed_varlen_block_amd as pvb
    import torch
    C, V = 8192, 32768
    say(f"loss C={C} V={V} bf16: 96 sampled rows")
    r = np.random.default_rng(1003)
    z = W.f32_to_bf16_bits(r.standard_normal((C, V), dtype=np.float32) * np.float32(2.0))
    tg = r.integers(0, V, size=C).astype(np.int32)
    tg[r.random(C) < 0.01] = -100
    zt = dev_bf16(z)
    out = pvb.packed_nll(zt, torch.tensor(tg).cuda())
    pvb.check_status(out["status"])
    elig = LP.eligible_cells(tg, None)
    n = int(elig.sum())
    assert out["count"].item() == n
    rows = np.sort(r.choice(C, size=96, replace=False))
    zs = W.bf16_bits_to_f64(z[rows])
    rrow, _, ns, _ = LP.packed_nll(zs, tg[rows], None)
    got_row = out["row_nll"].double().cpu().numpy()
    assert np.abs(got_row[rows] - rrow).max() <= 2e-5 * max(1.0, np.abs(rrow).max())
    # the sampled rows' gradient: O10 divides by the sample's own count
    rg = LP.packed_nll_grad(zs, tg[rows], None) * (ns / n)
    gg = out["grad"][torch.tensor(rows).cuda()].double().cpu().numpy()
    assert np.all(gg[~elig[rows]] == 0.0)
    # bf16 gradient: one rounding of values below 1/N
    assert np.abs(gg - rg).max() <= 4e-3 / n
    loss = out["loss"].cpu().numpy()
    total = float(np.sum(got_row.astype(np.float64)))
    assert abs(loss[0] - total) <= 1e-6 * abs(total)
    assert abs(loss[1] - total / n) <= 1e-6 * abs(total / n)
