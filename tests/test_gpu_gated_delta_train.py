"""GPU parity of the gated delta rule's training pair (pvb_gated_delta_fwd_train,
then pvb_gated_delta_bwd_after_fwd on the workspace it leaves) against the fp64
oracles O11 (O, final states) and O12 (the gradients), and against the plain
forward and backward on the same inputs."""
import numpy as np
import pytest

import workloads as W
from oracle import linear_attention as LA
from tests.parity import host_cu, say

pytestmark = pytest.mark.gpu

# Bars as for the plain calls (same kernels, same arithmetic): 1e-3 of a
# tensor's largest magnitude against fp64, plus half a bf16 ulp of it for a
# bf16 output.  Against the plain calls the pair computes every value with the
# same operations in the same order (the checkpoints it leaves are the ones
# the plain backward recomputes), so the results are equal bit for bit; only
# dq and dk of a query/key head shared by several value heads, summed with
# atomics in no fixed order, may differ in rounding (bar 1e-6 of the largest
# magnitude).
TOL = 1e-3
SAME = 1e-6
BF16_ULP = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import packed_varlen_block_amd  # noqa: F401  (fails loudly if libpvb.so is missing)


def _dev(x):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _check(name, got, ref, extra=0.0, rel=TOL):
    tol = 0.0 if rel == 0.0 else rel * max(1.0, float(np.abs(ref).max(initial=0.0))) + extra
    err = np.abs(got - ref)
    mx = float(err.max(initial=0.0))
    say(f"  {name}: max-abs {mx:.3e}  (bar {tol:.2e})")
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert mx <= tol, f"{name}: max-abs {mx:.3e} > {tol:.3e}"


def _pair(w, do, dsf, hc, mirror, h0, scale, o_dtype, grad_dtype):
    """The training pair and the plain calls on the same device inputs."""
    import torch

    import packed_varlen_block_amd as pvb
    T, H, d = w["v"].shape
    args = [_dev(w[x]) for x in ("q", "k", "v", "g", "beta")] + [_dev(hc)]
    hm = hc if mirror else None
    s0 = _dev(w["h0"]) if h0 else None
    dht = _dev(dsf) if dsf is not None else None
    n_seg = len(hc) - 1
    ws = torch.empty(pvb.gated_delta_bwd_workspace_bytes(T, H, n_seg), dtype=torch.uint8, device="cuda")
    o, ht, st = pvb.gated_delta_fwd(*args, h_cu=hm, scale=scale, initial_state=s0, o_dtype=o_dtype, workspace=ws,
                                    train=True)
    pvb.check_status(st)
    grads = pvb.gated_delta_bwd(*args, _dev(do), h_cu=hm, scale=scale, initial_state=s0, dht=dht,
                                grad_dtype=grad_dtype, workspace=ws, after_fwd=True)
    pvb.check_status(grads[-1])
    po, pht, st = pvb.gated_delta_fwd(*args, h_cu=hm, scale=scale, initial_state=s0, o_dtype=o_dtype)
    pvb.check_status(st)
    plain = pvb.gated_delta_bwd(*args, _dev(do), h_cu=hm, scale=scale, initial_state=s0, dht=dht,
                                grad_dtype=grad_dtype)
    pvb.check_status(plain[-1])
    torch.cuda.synchronize()
    return (o, ht), grads[:6], (po, pht), plain[:6]


def _case(seed, lengths, H, Hk=None, g_range=(-0.1, 0.0), beta_range=(0.05, 1.0), h0=False, dht=False,
          grad_dtype="f32", o_dtype="f32", scale=None, mirror=True):
    import torch
    w = W.random_gated_delta(seed, lengths, H, g_range=g_range, beta_range=beta_range, initial_state=h0, Hk=Hk)
    T, d = int(np.sum(lengths)), 128
    r = np.random.default_rng(seed + 1)
    do = W.f32_to_bf16_bits(r.standard_normal((T, H, d)).astype(np.float32))
    dsf = (r.standard_normal((len(lengths), H, d, d)) * 0.1).astype(np.float32) if dht else None
    hc = host_cu(lengths)
    od = torch.float32 if o_dtype == "f32" else torch.bfloat16
    gd = torch.float32 if grad_dtype == "f32" else torch.bfloat16
    (o, ht), grads, (po, pht), plain = _pair(w, do, dsf, hc, mirror, h0, scale, od, gd)
    f = W.bf16_bits_to_f64
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    s0 = w["h0"].astype(np.float64) if h0 else None
    ro, rs = LA.gated_delta_varlen(f(w["q"]), f(w["k"]), f(w["v"]), w["g"].astype(np.float64),
                                   w["beta"].astype(np.float64), hc, sc, s0)
    obf = BF16_ULP * float(np.abs(ro).max(initial=0.0)) if o_dtype == "bf16" else 0.0
    _check("O", o.double().cpu().numpy(), ro, obf)
    _check("final state", ht.double().cpu().numpy(), rs)
    _check("O against the plain forward", o.double().cpu().numpy(), po.double().cpu().numpy(), rel=0.0)
    _check("final state against the plain forward", ht.double().cpu().numpy(), pht.double().cpu().numpy(),
           rel=0.0)
    ref = LA.gated_delta_varlen_backward(f(w["q"]), f(w["k"]), f(w["v"]), w["g"].astype(np.float64),
                                         w["beta"].astype(np.float64), hc, sc, f(do), s0,
                                         dsf.astype(np.float64) if dht else None)
    names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
    shared = H != w["q"].shape[1]
    for name, a, p, b in zip(names, grads, plain, ref):
        a, p = a.double().cpu().numpy(), p.double().cpu().numpy()
        extra = BF16_ULP * float(np.abs(b).max(initial=0.0)) if (name == "dv" and grad_dtype == "bf16") else 0.0
        _check(name, a, b, extra)
        same = SAME if (shared and name in ("dq", "dk")) else 0.0
        _check(f"{name} against the plain backward", a, p, rel=same)


@pytest.mark.parametrize("lengths", [[1], [65], [130, 0, 64, 7]])
def test_train_pair_small(lengths):
    say(f"gated delta training pair: lengths {lengths}")
    _case(700 + sum(lengths), lengths, H=2)


def test_train_pair_states_grouped_heads_bf16():
    say("gated delta training pair: states, 4 value heads over 2, bf16 O and dv, scale 0.3")
    _case(711, [70, 0, 129, 3], H=4, Hk=2, h0=True, dht=True, o_dtype="bf16", grad_dtype="bf16", scale=0.3)


@pytest.mark.parametrize("with_mirror", [True, False])
def test_train_pair_group_edges(with_mirror):
    """Slices of one group, one token more, and 2.05 groups beside an empty
    one: the forward's group maps (every group's, the last one's too) feed the
    backward's transposed scan."""
    say(f"gated delta training pair: group edges, host mirror {with_mirror}")
    _case(712, [1024, 1025, 0, 2100], H=2, h0=True, dht=True, mirror=with_mirror)


def test_train_pair_long_slice_grouped_heads():
    say("gated delta training pair: a 2100-token slice beside short ones, 4 value heads over 2, states")
    _case(713, [2100, 300, 0, 65], H=4, Hk=2, h0=True, dht=True, mirror=False)


def test_train_pair_zero_length_slices_and_empty_stream():
    """Zero-length slices pass their initial state to their final state and
    their final-state gradient to their initial-state gradient; an empty stream
    (no token, no slice) runs both calls and writes nothing."""
    import torch

    import packed_varlen_block_amd as pvb
    say("gated delta training pair: zero-length slices, an all-empty pack, an empty stream")
    _case(720, [0, 5, 0], H=2, h0=True, dht=True)
    _case(721, [0, 0], H=2, h0=True, dht=True)
    z = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    zf = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0], dtype=torch.int32, device="cuda")
    ws = torch.empty(pvb.gated_delta_bwd_workspace_bytes(0, 2, 0), dtype=torch.uint8, device="cuda")
    o, ht, st = pvb.gated_delta_fwd(z, z, z, zf, zf, cu, workspace=ws, train=True)
    pvb.check_status(st)
    assert o.numel() == 0 and ht.numel() == 0
    grads = pvb.gated_delta_bwd(z, z, z, zf, zf, cu, z, workspace=ws, after_fwd=True)
    pvb.check_status(grads[-1])
    assert all(x.numel() == 0 for x in grads[:5])


def test_train_pair_bad_cu_writes_nothing():
    import torch

    import packed_varlen_block_amd as pvb
    say("gated delta training pair: a bad device cu_seqlens sets the status in both calls")
    w = W.random_gated_delta(714, [10, 6], 2)
    bad = torch.tensor([0, 12, 9], dtype=torch.int32).cuda()      # decreasing
    args = [_dev(w[x]) for x in ("q", "k", "v", "g", "beta")] + [bad]
    ws = torch.empty(pvb.gated_delta_bwd_workspace_bytes(16, 2, 2), dtype=torch.uint8, device="cuda")
    o = torch.full((16, 2, 128), 7.0, dtype=torch.float32, device="cuda")
    _, _, st = pvb.gated_delta_fwd(*args, out=o, workspace=ws, train=True)
    assert int(st.item()) == 4                                     # PVB_E_BAD_CU_SEQLENS
    assert bool((o == 7.0).all())
    do = _dev(W.f32_to_bf16_bits(np.ones((16, 2, 128), np.float32)))
    out = pvb.gated_delta_bwd(*args, do, workspace=ws, after_fwd=True)
    assert int(out[-1].item()) == 4


def test_train_pair_long_mixed_pack_against_plain():
    """The long mixed pack (T=32768, 32 heads) as the bench runs it: the
    training pair's O, final states and every gradient against the plain
    forward and backward, all heads and tokens."""
    import torch
    lengths = W.lengths_cfg4(0)
    H, d = 32, 128
    T = int(lengths.sum())
    say(f"gated delta training pair: long mixed pack T={T}, H={H}, against the plain calls")
    w = W.random_gated_delta(715, lengths, H)
    r = np.random.default_rng(716)
    do = W.f32_to_bf16_bits(r.standard_normal((T, H, d), dtype=np.float32))
    dsf = (r.standard_normal((len(lengths), H, d, d), dtype=np.float32) * np.float32(0.1))
    hc = host_cu(lengths)
    (o, ht), grads, (po, pht), plain = _pair(w, do, dsf, hc, False, False, None, torch.bfloat16, torch.float32)
    _check("O against the plain forward", o.float().cpu().numpy(), po.float().cpu().numpy(), rel=0.0)
    _check("final state against the plain forward", ht.cpu().numpy(), pht.cpu().numpy(), rel=0.0)
    for name, a, p in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), grads, plain):
        _check(f"{name} against the plain backward", a.cpu().numpy(), p.cpu().numpy(), rel=0.0)
