"""GPU parity of the cross-attention / local-window entry points against the
fp64 band oracle (separate query and key boundaries, the causal clamp aligned
to the bottom right of each slice, windows on either side)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
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


def _run(seed, lq, lk, H, Hk, d, window, grad_dtype="f32", precision="bf16", backward=True):
    import packed_varlen_block_amd as pvb
    import torch
    qb, kb, vb, db = W.random_cross(seed, lq, lk, H, Hk, d, backward=backward)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    hq, hk = host_cu(lq), host_cu(lk)
    cq, ck = _dev_cu(hq), _dev_cu(hk)
    o, lse, st = pvb.varlen_cross_attn_fwd(q, k, v, cq, ck, hq, hk, window=window,
                                           o_dtype=torch.float32 if precision == "split" else torch.bfloat16,
                                           precision=precision)
    pvb.check_status(st)
    qo, ko, vo = (W.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    ro, rl = A.varlen_cross_forward(qo, ko, vo, hq, hk, window=window)
    check("O", to64(o), ro)
    gl = lse.double().cpu().numpy()
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty), "rows without keys must have LSE = -inf"
    check("LSE", np.where(empty, 0.0, gl), np.where(empty, 0.0, rl), max_abs=1e-3, mean_abs=1e-4)
    if not backward:
        return
    do = dev_bf16(db)
    gd = torch.float32 if grad_dtype == "f32" else torch.bfloat16
    dq, dk, dv, st = pvb.varlen_cross_attn_bwd(q, k, v, o, do, lse, cq, ck, hq, hk, window=window,
                                               grad_dtype=gd, precision=precision)
    pvb.check_status(st)
    rq, rk, rv = A.varlen_cross_backward(qo, ko, vo, W.bf16_bits_to_f64(db), hq, hk, window=window)
    # bf16 gradients: the bar also admits the format's own rounding of the
    # largest values (half an ulp of max|ref|)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check(name, to64(got), ref, bf16_out=grad_dtype == "bf16")


# (query lengths, key lengths): longer and shorter key extents than query
# extents, empty slices on either side, ragged tile ends, several tiles
CROSS_LENGTHS = [
    ([5, 3, 4], [5, 3, 4]),
    ([5, 3, 4], [9, 1, 6]),
    ([64, 1, 130], [200, 7, 0]),
    ([300], [129]),
    ([0, 77, 0, 3], [12, 0, 0, 150]),
    ([129, 256, 1], [513, 64, 65]),
]
WINDOWS = [(-1, 0), (-1, -1), (16, 0), (0, 0), (40, 7), (-1, 5), (3, -1)]


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("d", [64, 128])
def test_cross_forward_backward(window, d):
    for i, (lq, lk) in enumerate(CROSS_LENGTHS):
        say(f"cross d={d} window={window} lq={lq} lk={lk}")
        _run(700 + i, lq, lk, 4, 2, d, window)


@pytest.mark.parametrize("grad_dtype,precision", [("bf16", "bf16"), ("f32", "split")])
def test_cross_dtypes(grad_dtype, precision):
    for i, (lq, lk) in enumerate(CROSS_LENGTHS[2:4]):
        for window in ((-1, 0), (33, 0)):
            say(f"cross g={grad_dtype} prec={precision} window={window} lq={lq} lk={lk}")
            _run(760 + i, lq, lk, 2, 2, 128, window, grad_dtype, precision)


LONG_CASES = [([1030], [2100], (-1, 0)), ([2048, 5], [700, 900], (-1, -1)), ([1800], [1800], (255, 0)),
              ([900], [3000], (100, 100))]


@pytest.mark.parametrize("case", range(len(LONG_CASES)))
def test_cross_long_segments(case):
    """Many key tiles per query tile and many query tiles per key tile."""
    lq, lk, window = LONG_CASES[case]
    say(f"cross long lq={lq} lk={lk} window={window}")
    _run(780 + case, lq, lk, 4, 1, 128, window)


def test_self_window_equals_cross_with_same_boundaries():
    """cu_k = cu_q and (-1, 0) is the causal self-attention call, bit for bit."""
    import packed_varlen_block_amd as pvb
    lengths = [200, 1, 0, 130, 64, 65]
    qb, kb, vb, db = W.random_cross(790, lengths, lengths, 4, 2, 128)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(db)
    h = host_cu(lengths)
    c = _dev_cu(h)
    o1, l1, s1 = pvb.varlen_attn_fwd(q, k, v, c)
    o2, l2, s2 = pvb.varlen_cross_attn_fwd(q, k, v, c, c, h, h)
    pvb.check_status(s1)
    pvb.check_status(s2)
    assert (o1 == o2).all() and (l1 == l2).all()
    g1 = pvb.varlen_attn_bwd(q, k, v, o1, do, l1, c)
    g2 = pvb.varlen_cross_attn_bwd(q, k, v, o2, do, l2, c, c, h, h)
    for a, b in zip(g1[:3], g2[:3]):
        assert (a == b).all()


def test_cross_no_keys_or_no_queries():
    """T_k = 0: every row is empty (O = 0, LSE = -inf, dQ = 0); T_q = 0: dK = dV = 0."""
    import packed_varlen_block_amd as pvb
    import torch
    say("cross T_k = 0")
    q = torch.randn((10, 2, 64), device="cuda").bfloat16()
    k = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    hq, hk = np.array([0, 4, 10], np.int32), np.array([0, 0, 0], np.int32)
    o, lse, st = pvb.varlen_cross_attn_fwd(q, k, k, _dev_cu(hq), _dev_cu(hk), hq, hk)
    pvb.check_status(st)
    assert (o == 0).all() and torch.isneginf(lse).all()
    do = torch.randn_like(q)
    dq, dk, dv, st = pvb.varlen_cross_attn_bwd(q, k, k, o, do, lse, _dev_cu(hq), _dev_cu(hk), hq, hk)
    pvb.check_status(st)
    assert (dq == 0).all() and dk.numel() == 0
    # T_q = 0: no queries at all; the key-side kernel writes zero gradients
    say("cross T_q = 0")
    q0 = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    k2 = torch.randn((20, 2, 64), device="cuda").bfloat16()
    hq, hk = np.array([0, 0, 0], np.int32), np.array([0, 12, 20], np.int32)
    o, lse, st = pvb.varlen_cross_attn_fwd(q0, k2, k2, _dev_cu(hq), _dev_cu(hk), hq, hk)
    pvb.check_status(st)
    assert o.numel() == 0 and lse.numel() == 0
    dq, dk, dv, st = pvb.varlen_cross_attn_bwd(q0, k2, k2, o, q0, lse, _dev_cu(hq), _dev_cu(hk), hq, hk)
    pvb.check_status(st)
    assert dq.numel() == 0 and (dk == 0).all() and (dv == 0).all()


def test_cross_planner_path():
    """Enough work items that both lists come from the planner kernel."""
    lq = [300] * 12
    lk = [520] * 6 + [90] * 6
    say("cross planner path")
    _run(795, lq, lk, 8, 2, 128, (-1, 0))
    _run(796, lq, lk, 8, 2, 128, (64, 64))


def test_cross_bad_device_cu_k_reported_by_the_key_list():
    """A device cu_k that differs from its (valid) host mirror: the key list
    reports PVB_E_BAD_CU_SEQLENS and cannot be overwritten by the query list."""
    import packed_varlen_block_amd as pvb
    import torch
    lq, lk = [40, 24], [50, 30]
    qb, kb, vb, db = W.random_cross(797, lq, lk, 2, 2, 64)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(db)
    hq, hk = host_cu(lq), host_cu(lk)
    o, lse, st = pvb.varlen_cross_attn_fwd(q, k, v, _dev_cu(hq), _dev_cu(hk), hq, hk)
    pvb.check_status(st)
    bad_k = _dev_cu([0, 60, 50])                       # decreasing on the device only
    st = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    pvb.varlen_cross_attn_bwd(q, k, v, o, do, lse, _dev_cu(hq), bad_k, hq, hk, status=st)
    torch.cuda.synchronize()
    assert st.item() == 4


# seeded random draws: per-segment query and key lengths (on and next to the
# tile edges, anywhere below 300, or zero on either side), a window from
# unbounded to tight on both sides, grouped heads, both head sizes
EDGES = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129]


@pytest.mark.parametrize("case", range(16))
def test_cross_random(case):
    r = np.random.default_rng(4000 + case)
    n = int(r.integers(1, 7))

    def length():
        u = r.random()
        return 0 if u < 0.12 else int(r.choice(EDGES)) if u < 0.5 else int(r.integers(1, 300))

    lq = [length() for _ in range(n)]
    lk = [length() for _ in range(n)]
    window = (int(r.choice([-1, 0, 3, 16, 40, 100])), int(r.choice([-1, 0, 0, 5])))
    Hk = int(r.integers(1, 4))
    H = Hk * int(r.choice([1, 2, 4]))
    d = int(r.choice([64, 128]))
    grad_dtype = "bf16" if r.random() < 0.4 else "f32"
    precision = "split" if r.random() < 0.25 else "bf16"
    say(f"cross random {case}: lq={lq} lk={lk} window={window} H={H} H_kv={Hk} d={d} "
        f"grad={grad_dtype} precision={precision}")
    _run(4100 + case, lq, lk, H, Hk, d, window, grad_dtype, precision)
