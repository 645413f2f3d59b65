"""GPU parity of the varlen attention kernels against the fp64 oracle.

Small cases are compared element by element in full; the full-size workloads
are launched exactly as the benchmark launches them and compared on sampled
heads, each sampled head in full (every segment, every row).
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from tests.parity import (check, compare_bwd, compare_fwd, dev_bf16, dev_cu, gpu_bwd, gpu_fwd,
                          host_cu, oracle_inputs, say, to64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import packed_varlen_block_amd  # noqa: F401  (fails loudly if libpvb.so is missing)


SMALL_LENGTHS = [
    [1], [2], [63], [64], [65], [127], [128], [129],
    [5, 3, 4], [0, 0, 7, 0], [200, 1, 0, 130, 64, 65], [300], [17, 129, 0, 1, 256],
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("o_dtype,precision", [("bf16", "bf16"), ("f32", "bf16"), ("f32", "split")])
def test_forward_small_sweep(d, o_dtype, precision):
    for i, lengths in enumerate(SMALL_LENGTHS):
        say(f"fwd small d={d} o={o_dtype} prec={precision} lengths={lengths}")
        w = W.random_small(100 + i, lengths, H=3, d=d, backward=False)
        _, o, lse = gpu_fwd(w, o_dtype, precision)
        compare_fwd(w, o, lse)


# long segments (many key tiles per query tile, ragged ends) at d = 128
LONG_LENGTHS = [[512], [513], [700], [1030], [1300, 1], [255, 1800], [2048], [0, 1111, 0]]


@pytest.mark.parametrize("o_dtype", ["bf16", "f32"])
def test_forward_long_segments(o_dtype):
    for i, lengths in enumerate(LONG_LENGTHS):
        say(f"fwd long d=128 o={o_dtype} lengths={lengths}")
        w = W.random_small(300 + i, lengths, H=2, d=128, backward=False)
        _, o, lse = gpu_fwd(w, o_dtype, "bf16")
        compare_fwd(w, o, lse)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("grad_dtype,precision", [("f32", "bf16"), ("bf16", "bf16"), ("f32", "split")])
def test_backward_small_sweep(d, grad_dtype, precision):
    for i, lengths in enumerate(SMALL_LENGTHS):
        say(f"bwd small d={d} g={grad_dtype} prec={precision} lengths={lengths}")
        w = W.random_small(200 + i, lengths, H=3, d=d, backward=True)
        dev, o, lse = gpu_fwd(w, "f32" if precision == "split" else "bf16", precision)
        dq, dk, dv = gpu_bwd(dev, o, lse, w, grad_dtype, precision)
        compare_bwd(w, dq, dk, dv)


# long segments through the backward: many query steps per key tile in the
# dK/dV kernel, many key tiles per query tile in the dQ kernel, ragged ends
LONG_BWD_LENGTHS = [[513], [1030], [1300, 1], [255, 1800], [0, 1111, 0]]


@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
def test_backward_long_segments(grad_dtype):
    for i, lengths in enumerate(LONG_BWD_LENGTHS):
        say(f"bwd long d=128 g={grad_dtype} lengths={lengths}")
        w = W.random_small(400 + i, lengths, H=2, d=128, backward=True)
        dev, o, lse = gpu_fwd(w, "bf16", "bf16")
        dq, dk, dv = gpu_bwd(dev, o, lse, w, grad_dtype, "bf16")
        compare_bwd(w, dq, dk, dv)


def test_empty_pack():
    """T = 0 (no segments, or only empty ones): every call succeeds and
    returns empty outputs."""
    import torch
    import packed_varlen_block_amd as pvb
    H, d = 2, 128
    for lengths in ([], [0], [0, 0, 0]):
        say(f"empty pack lengths={lengths}")
        cu = torch.tensor(host_cu(lengths), dtype=torch.int32).cuda()
        z = torch.empty((0, H, d), dtype=torch.bfloat16, device="cuda")
        o, lse, st = pvb.varlen_attn_fwd(z, z, z, cu)
        pvb.check_status(st)
        assert tuple(o.shape) == (0, H, d) and tuple(lse.shape) == (H, 0)
        dq, dk, dv, st = pvb.varlen_attn_bwd(z, z, z, o, z, lse, cu)
        pvb.check_status(st)
        assert all(tuple(g.shape) == (0, H, d) for g in (dq, dk, dv))


def test_worked_example_and_merged_boundary():
    say("cfg1: worked example, forward, and the merged boundary [0,5,12]")
    import packed_varlen_block_amd as pvb
    import torch
    w = W.make(1)
    for od in ("bf16", "f32"):
        dev, o, lse = gpu_fwd(w, od)
        compare_fwd(w, o, lse, tag=f"cfg1 {od} ")
    q, k, v, _ = dev
    merged = torch.tensor([0, 5, 12], dtype=torch.int32).cuda()
    om, lm, st = pvb.varlen_attn_fwd(q, k, v, merged, o_dtype=torch.float32)
    pvb.check_status(st)
    o3, _, st = pvb.varlen_attn_fwd(q, k, v, dev[3], o_dtype=torch.float32)
    pvb.check_status(st)
    qo, ko, vo, _ = oracle_inputs(w)
    ref_m, _ = A.varlen_forward(qo, ko, vo, [0, 5, 12])
    check("cfg1 merged O", to64(om), ref_m)
    # rows of A and B do not change when B and C merge; C's rows do
    assert torch.allclose(om[:8], o3[:8], atol=1e-6)
    assert (om[8:] - o3[8:]).abs().max().item() > 1e-3


def test_cfg2_forward_full():
    say("cfg2: T=4096, 16 segments, H=16, d=128, forward, every head")
    w = W.make(2)
    _, o, lse = gpu_fwd(w, "bf16")
    compare_fwd(w, o, lse, tag="cfg2 ")


def _cfg3():
    import packed_varlen_block_amd as pvb
    raw = W.raw_lengths_cfg3(0)
    _, _, _, order, offs = pvb.pack_plan_bfd(raw, 8192)
    return W.make(3, first_pack_lengths=raw[order[offs[0]:offs[1]]])


def test_cfg3_forward_backward_sampled_heads():
    say("cfg3: BFD first pack T=8192, H=32, d=128, fwd+bwd; heads 0, 13, 31 compared")
    w = _cfg3()
    assert w.T == 8192 and len(w.lengths) == 1
    dev, o, lse = gpu_fwd(w, "bf16")
    dq, dk, dv = gpu_bwd(dev, o, lse, w, "f32")
    compare_fwd(w, o, lse, heads=[0, 13, 31], tag="cfg3 ")
    compare_bwd(w, dq, dk, dv, heads=[0, 31], tag="cfg3 ")


def test_cfg4_forward_backward_sampled_heads():
    say("cfg4: T=32768 with a 16384 segment, H=32, d=128, fwd+bwd; head 7 compared")
    w = W.make(4)
    dev, o, lse = gpu_fwd(w, "bf16")
    dq, dk, dv = gpu_bwd(dev, o, lse, w, "f32")
    compare_fwd(w, o, lse, heads=[7], tag="cfg4 ")
    compare_bwd(w, dq, dk, dv, heads=[7], tag="cfg4 ")


def test_cfg5_forward_backward_split_precision():
    say("cfg5: T=16384 edge lengths incl. 0, outliers x30, H=16, fwd+bwd split/fp32; heads 0, 9")
    w = W.make(5)
    assert (w.lengths == 0).any()
    dev, o, lse = gpu_fwd(w, "f32", "split")
    dq, dk, dv = gpu_bwd(dev, o, lse, w, "f32", "split")
    compare_fwd(w, o, lse, heads=[0, 9], tag="cfg5 ")
    compare_bwd(w, dq, dk, dv, heads=[0, 9], tag="cfg5 ")


def test_isolation_nan_in_other_segment():
    say("isolation: NaN/Inf in segment A leaves segment B bit-identical and finite")
    import torch
    w = W.random_small(7, [70, 150], H=2, d=128, backward=True)
    dev, o, lse = gpu_fwd(w, "f32")
    dq, dk, dv = gpu_bwd(dev, o, lse, w, "f32")
    w2 = W.random_small(7, [70, 150], H=2, d=128, backward=True)
    for arr in (w2.q, w2.k, w2.v, w2.do):
        arr[:70] = 0x7FC0            # bf16 NaN
        arr[3] = 0x7F80              # bf16 +Inf
    dev2, o2, lse2 = gpu_fwd(w2, "f32")
    dq2, dk2, dv2 = gpu_bwd(dev2, o2, lse2, w2, "f32")
    for a, b in ((o, o2), (dk, dk2), (dv, dv2)):
        assert torch.isfinite(b[70:]).all()
        assert torch.equal(a[70:], b[70:])
    assert torch.isfinite(dq2[70:]).all()
    assert torch.allclose(dq[70:], dq2[70:], atol=1e-6)
    assert torch.equal(lse[:, 70:], lse2[:, 70:])


def test_bad_device_cu_sets_status_and_writes_nothing():
    say("device-detected bad cu_seqlens")
    import packed_varlen_block_amd as pvb
    import torch
    w = W.random_small(9, [40, 24], H=2, d=64, backward=False)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    for bad in ([0, 40, 30], [1, 40, 64], [0, 40, 63]):
        cu = torch.tensor(bad, dtype=torch.int32).cuda()
        o = torch.full((64, 2, 64), 7.0, dtype=torch.float32).cuda()
        _, _, st = pvb.varlen_attn_fwd(q, k, v, cu, out=o)
        with pytest.raises(pvb.PvbError) as e:
            pvb.check_status(st)
        assert e.value.status == 4
        assert (o == 7.0).all()
    with pytest.raises(pvb.PvbError) as e:
        pvb.varlen_attn_fwd(q, k, v, torch.tensor([0, 40, 30], dtype=torch.int32).cuda(),
                            h_cu=[0, 40, 30])
    assert e.value.status == 4


def test_backward_dk_dv_deterministic():
    say("determinism: dK/dV bitwise repeatable")
    import torch
    w = W.random_small(11, [300, 77], H=2, d=128, backward=True)
    dev, o, lse = gpu_fwd(w, "bf16")
    a = gpu_bwd(dev, o, lse, w, "f32")
    b = gpu_bwd(dev, o, lse, w, "f32")
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert torch.allclose(a[0], b[0], atol=1e-5)


@pytest.mark.parametrize("d", [64, 128])
def test_planner_path_many_segments(d):
    # More than 1024 segments: the work list comes from the one-workgroup
    # planner instead of the in-kernel decode used for smaller packs.
    rng = np.random.default_rng(1234 + d)
    lengths = rng.integers(0, 25, size=1100).tolist()
    lengths[5] = 300                      # one segment spanning several tiles
    say(f"planner path: {len(lengths)} segments, T={sum(lengths)}, d={d}")
    w = W.random_small(13, lengths, H=2, d=d, backward=True)
    dev, o, lse = gpu_fwd(w, "bf16")
    compare_fwd(w, o, lse, tag="planner path ")
    dq, dk, dv = gpu_bwd(dev, o, lse, w, "f32")
    compare_bwd(w, dq, dk, dv, tag="planner path ")


def test_bad_device_cu_backward_and_planner_path():
    say("device-detected bad cu_seqlens: backward, and the planner path")
    import packed_varlen_block_amd as pvb
    import torch
    w = W.random_small(9, [40, 24], H=2, d=64, backward=True)
    dev, o, lse = gpu_fwd(w, "bf16")
    q, k, v, _ = dev
    do = dev_bf16(w.do)
    bad = torch.tensor([0, 40, 30], dtype=torch.int32).cuda()
    grads = [torch.full((64, 2, 64), 7.0, dtype=torch.float32).cuda() for _ in range(3)]
    st = pvb.varlen_attn_bwd(q, k, v, o, do, lse, bad, dq=grads[0], dk=grads[1], dv=grads[2])[3]
    with pytest.raises(pvb.PvbError) as e:
        pvb.check_status(st)
    assert e.value.status == 4
    assert all((g == 7.0).all() for g in grads)
    # 1100 segments (planner path), one decreasing entry
    cu = np.arange(1101, dtype=np.int32)
    cu[500] = 700
    T = 1100
    qq = torch.zeros((T, 2, 64), dtype=torch.bfloat16).cuda()
    out = torch.full((T, 2, 64), 7.0, dtype=torch.float32).cuda()
    _, _, st = pvb.varlen_attn_fwd(qq, qq, qq, torch.from_numpy(cu).cuda(), out=out)
    with pytest.raises(pvb.PvbError) as e:
        pvb.check_status(st)
    assert e.value.status == 4
    assert (out == 7.0).all()


# ------------------------------------------------ grouped key/value heads

GQA_CASES = [([5, 3, 4], 4, 2, 64), ([200, 1, 0, 130, 64, 65], 6, 1, 128), ([1030], 8, 2, 128),
             ([255, 1800], 4, 1, 128), ([300, 77], 8, 8, 128)]


@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
def test_grouped_heads_forward_backward(grad_dtype):
    import packed_varlen_block_amd as pvb
    for i, (lengths, H, Hk, d) in enumerate(GQA_CASES):
        say(f"gqa lengths={lengths} H={H} H_kv={Hk} d={d} g={grad_dtype}")
        w = W.random_small(500 + i, lengths, H=H, d=d, backward=True)
        kb = np.ascontiguousarray(w.k[:, :Hk])
        vb = np.ascontiguousarray(w.v[:, :Hk])
        q, k, v, do = dev_bf16(w.q), dev_bf16(kb), dev_bf16(vb), dev_bf16(w.do)
        cu = dev_cu(w.lengths)
        o, lse, st = pvb.varlen_attn_fwd(q, k, v, cu)
        pvb.check_status(st)
        gd = __import__("torch").float32 if grad_dtype == "f32" else __import__("torch").bfloat16
        dq, dk, dv, st = pvb.varlen_attn_bwd(q, k, v, o, do, lse, cu, grad_dtype=gd)
        pvb.check_status(st)
        assert tuple(dk.shape) == tuple(dv.shape) == (w.T, Hk, d)
        qo, ko, vo, doo = (W.bf16_bits_to_f64(x) for x in (w.q, kb, vb, w.do))
        cuh = host_cu(w.lengths)
        ro, rl = A.varlen_forward(qo, ko, vo, cuh)
        check("O", to64(o), ro)
        check("LSE", lse.double().cpu().numpy(), rl, max_abs=1e-3, mean_abs=1e-4)
        rq, rk, rv = A.varlen_backward(qo, ko, vo, doo, cuh)
        check("dQ", to64(dq), rq)
        # dK, dV sum H / H_kv query heads, so they grow with the group; stored
        # in bf16 they carry one rounding of up to 2^-9 of their magnitude on
        # top of the bar
        for name, got, ref in (("dK", dk, rk), ("dV", dv, rv)):
            extra = 2.0 ** -9 * float(np.abs(ref).max()) if grad_dtype == "bf16" else 0.0
            check(name, to64(got), ref, max_abs=2e-2 + extra)


def test_grouped_heads_rejects_uneven_groups():
    import packed_varlen_block_amd as pvb
    import torch
    q = torch.zeros((8, 3, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((8, 2, 64), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 8], dtype=torch.int32, device="cuda")
    with pytest.raises(pvb.PvbError):
        pvb.varlen_attn_fwd(q, k, k, cu)


@pytest.mark.parametrize("lengths", [
    [5, 3, 4],                              # host-listed items
    [84, 0, 99, 460, 487, 1, 129],          # host-listed, zeros and tile edges
    [130] * 240,                            # 480 tiles: more than the host list holds, device plan
    [40000, 100],                           # a segment past 32768 tokens: device plan
])
def test_host_mirror_gives_the_same_forward(lengths):
    """With the host mirror of cu_seqlens a small self-attention forward lists
    its items on the host and passes them with the launch; O and LSE equal the
    device-planned call bit for bit, and the oracle on one head."""
    import torch

    import packed_varlen_block_amd as pvb
    say(f"fwd with/without the host mirror: {len(lengths)} segments, T {sum(lengths)}")
    H, d = 2, 128
    w = W.random_small(777, lengths, H=H, d=d, backward=False)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    hc = host_cu(lengths)
    cu = torch.tensor(hc).cuda()
    o1, l1, s1 = pvb.varlen_attn_fwd(q, k, v, cu, h_cu=hc)
    o2, l2, s2 = pvb.varlen_attn_fwd(q, k, v, cu)
    pvb.check_status(s1)
    pvb.check_status(s2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    if sum(lengths) <= 20000:
        compare_fwd(w, o1, l1, heads=[1])
