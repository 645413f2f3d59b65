"""GPU parity of the gated delta rule's backward (pvb_gated_delta_bwd) against
the fp64 oracle O12: dq, dk, dv, dg, dbeta and the initial-state gradient."""
import numpy as np
import pytest

import workloads as W
from oracle import linear_attention as LA
from tests.parity import host_cu, say

pytestmark = pytest.mark.gpu

# Bar (per tensor, absolute, against fp64): the kernels work in fp32 with
# matrix-core products of two-part bf16 operands (about 16 significant bits),
# as the forward does, so the bar is the forward's: 1e-3 of the tensor's
# largest magnitude (at least 1e-3).  A bf16 dv also carries its own rounding,
# half an ulp of its largest value.
TOL = 1e-3
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


def _check(name, got, ref, extra=0.0):
    tol = TOL * max(1.0, float(np.abs(ref).max(initial=0.0))) + extra
    err = np.abs(got - ref)
    mx = float(err.max(initial=0.0))
    say(f"  {name}: max-abs {mx:.3e}  (bar {tol:.2e}, max|ref| {float(np.abs(ref).max(initial=0.0)):.2e})")
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert mx <= tol, f"{name}: max-abs {mx:.3e} > {tol:.3e}"


def _case(seed, lengths, H, Hk=None, g_range=(-0.1, 0.0), beta_range=(0.05, 1.0), h0=False, dht=False,
          grad_dtype="f32", scale=None, mirror=True):
    import torch

    import packed_varlen_block_amd as pvb
    w = W.random_gated_delta(seed, lengths, H, g_range=g_range, beta_range=beta_range, initial_state=h0, Hk=Hk)
    T, d = int(np.sum(lengths)), 128
    Hk = H if Hk is None else Hk
    r = np.random.default_rng(seed + 1)
    do = W.f32_to_bf16_bits(r.standard_normal((T, H, d)).astype(np.float32))
    dsf = (r.standard_normal((len(lengths), H, d, d)) * 0.1).astype(np.float32) if dht else None
    hc = host_cu(lengths)
    gd = torch.float32 if grad_dtype == "f32" else torch.bfloat16
    dq, dk, dv, dg, db, dh0, st = pvb.gated_delta_bwd(
        _dev(w["q"]), _dev(w["k"]), _dev(w["v"]), _dev(w["g"]), _dev(w["beta"]), _dev(hc), _dev(do),
        h_cu=hc if mirror else None,
        scale=scale, initial_state=_dev(w["h0"]) if h0 else None, dht=_dev(dsf) if dht else None, grad_dtype=gd)
    pvb.check_status(st)
    f = W.bf16_bits_to_f64
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    ref = LA.gated_delta_varlen_backward(f(w["q"]), f(w["k"]), f(w["v"]), w["g"].astype(np.float64),
                                         w["beta"].astype(np.float64), hc, sc, f(do),
                                         w["h0"].astype(np.float64) if h0 else None,
                                         dsf.astype(np.float64) if dht else None)
    got = [x.double().cpu().numpy() for x in (dq, dk, dv, dg, db)]
    for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta"), got, ref[:5]):
        extra = BF16_ULP * float(np.abs(b).max(initial=0.0)) if (name == "dv" and grad_dtype == "bf16") else 0.0
        _check(name, a, b, extra)
    _check("dh0", dh0.double().cpu().numpy(), ref[5])


@pytest.mark.parametrize("lengths", [[1], [5], [63], [64], [65], [130, 0, 64, 7], [200]])
def test_backward_small(lengths):
    say(f"gated delta bwd: lengths {lengths}")
    _case(400 + len(lengths) + sum(lengths), lengths, H=2)


def test_backward_states_and_grouped_heads():
    say("gated delta bwd: initial states, final-state gradient, 4 value heads over 2 query/key heads")
    _case(501, [70, 0, 129, 3], H=4, Hk=2, h0=True, dht=True)


@pytest.mark.parametrize("g_range,beta_range", [((0.0, 0.0), (0.05, 1.0)), ((-1.0, 0.0), (0.9, 1.0)),
                                                ((-8.0, -4.0), (0.05, 0.2))])
def test_backward_gate_ranges(g_range, beta_range):
    say(f"gated delta bwd: gates {g_range}, beta {beta_range}")
    _case(502, [150, 40], H=2, g_range=g_range, beta_range=beta_range, h0=True, dht=True)


def test_backward_bf16_dv_and_scale():
    say("gated delta bwd: bf16 dv, scale 0.3")
    _case(503, [100, 28], H=2, grad_dtype="bf16", scale=0.3, dht=True)


def test_backward_long_slice_grouped():
    say("gated delta bwd: a 2100-token slice beside short ones, 4 value heads over 2, states")
    _case(504, [2100, 300, 0, 65], H=4, Hk=2, h0=True, dht=True)


@pytest.mark.parametrize("with_mirror", [True, False])
def test_backward_group_edges(with_mirror):
    """Slices of exactly one group (1024 tokens), one token more, and 2.05
    groups with a partial last chunk, beside an empty one: the walks in
    groups of 1024 tokens (the recomputation's maps and the state-gradient
    walk's offsets and transposed maps) against O12, with and without the
    host mirror of cu_seqlens."""
    say(f"gated delta bwd: group edges, host mirror {with_mirror}")
    _case(508, [1024, 1025, 0, 2100], H=2, h0=True, dht=True, mirror=with_mirror)


def test_backward_bad_cu_writes_nothing():
    import torch

    import packed_varlen_block_amd as pvb
    say("gated delta bwd: a bad device cu_seqlens sets the status and writes no gradient")
    w = W.random_gated_delta(505, [10, 6], 2)
    bad = torch.tensor([0, 12, 9], dtype=torch.int32).cuda()      # decreasing
    do = _dev(W.f32_to_bf16_bits(np.ones((16, 2, 128), np.float32)))
    dq, dk, dv, dg, db, dh0, st = pvb.gated_delta_bwd(_dev(w["q"]), _dev(w["k"]), _dev(w["v"]), _dev(w["g"]),
                                                      _dev(w["beta"]), bad, do)
    assert int(st.item()) == 4                                     # PVB_E_BAD_CU_SEQLENS


def test_backward_long_mixed_pack_sampled_head():
    """The long mixed pack (T=32768: a 16384-token slice, then slices of
    16-1024) at 32 heads, launched as the bench launches it (fp32 gradients,
    a final-state gradient); value head 5 compared in full, every slice, with
    the oracle run slice by slice on that head."""
    import torch

    import packed_varlen_block_amd as pvb
    lengths = W.lengths_cfg4(0)
    H, d = 32, 128
    say(f"gated delta bwd: long mixed pack T={int(lengths.sum())}, H={H}, head 5 against the oracle")
    w = W.random_gated_delta(506, lengths, H)
    T = int(lengths.sum())
    r = np.random.default_rng(507)
    do = W.f32_to_bf16_bits(r.standard_normal((T, H, d), dtype=np.float32))
    dsf = (r.standard_normal((len(lengths), H, d, d), dtype=np.float32) * np.float32(0.1))
    hc = host_cu(lengths)
    dq, dk, dv, dg, db, dh0, st = pvb.gated_delta_bwd(_dev(w["q"]), _dev(w["k"]), _dev(w["v"]), _dev(w["g"]),
                                                      _dev(w["beta"]), _dev(hc), _dev(do), dht=_dev(dsf))
    pvb.check_status(st)
    h = 5
    f = W.bf16_bits_to_f64
    q, k, v, dof = f(w["q"][:, h]), f(w["k"][:, h]), f(w["v"][:, h]), f(do[:, h])
    g, b = w["g"][:, h].astype(np.float64), w["beta"][:, h].astype(np.float64)
    ref = [np.zeros((T, d)), np.zeros((T, d)), np.zeros((T, d)), np.zeros(T), np.zeros(T)]
    ref_h0 = np.zeros((len(lengths), d, d))
    for s in range(len(lengths)):
        a, e = int(hc[s]), int(hc[s + 1])
        out = LA.gated_delta_segment_backward(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], d ** -0.5, dof[a:e],
                                              None, dsf[s, h].astype(np.float64))
        for i in range(5):
            ref[i][a:e] = out[i]
        ref_h0[s] = out[5]
    got = [dq[:, h], dk[:, h], dv[:, h], dg[:, h], db[:, h]]
    for name, a, bref in zip(("dq", "dk", "dv", "dg", "dbeta"), got, ref):
        _check(name, a.double().cpu().numpy(), bref)
    _check("dh0", dh0[:, h].double().cpu().numpy(), ref_h0)


# Seeded random draws: chunk-edge and arbitrary slice lengths with zeros mixed
# in, grouped heads, the gate and write-strength ranges, initial states and
# final-state gradients, fp32 or bf16 dv, two scales.
CHUNK_EDGES = [1, 63, 64, 65, 127, 128, 129, 192]


@pytest.mark.parametrize("case", range(12))
def test_backward_random_draws(case):
    r = np.random.default_rng(6000 + case)
    n = int(r.integers(1, 7))
    lengths = [0 if (u := r.random()) < 0.12 else int(r.choice(CHUNK_EDGES)) if u < 0.5 else int(r.integers(1, 300))
               for _ in range(n)]
    if sum(lengths) == 0:
        lengths[-1] = int(r.choice(CHUNK_EDGES))
    Hk = int(r.integers(1, 4))
    H = Hk * int(r.choice([1, 2, 4]))
    g_range = [(0.0, 0.0), (-0.1, 0.0), (-1.0, 0.0), (-6.0, -2.0)][int(r.integers(0, 4))]
    beta_range = [(0.05, 1.0), (0.9, 1.0), (0.0, 0.3)][int(r.integers(0, 3))]
    h0, dht = bool(r.random() < 0.5), bool(r.random() < 0.5)
    grad_dtype = "bf16" if r.random() < 0.3 else "f32"
    scale = None if r.random() < 0.6 else 0.3
    # odd cases go without the host mirror (the walks in groups, on the device's
    # decision); the last two add a slice longer than one group of 1024 tokens
    mirror = case % 2 == 0
    if case >= 10:
        lengths.append(int(r.integers(1025, 2200)))
    say(f"gated delta bwd random {case}: lengths={lengths} H={H} H_k={Hk} g={g_range} beta={beta_range} "
        f"h0={h0} dht={dht} dv={grad_dtype} scale={scale} mirror={mirror}")
    _case(6100 + case, lengths, H, Hk=Hk, g_range=g_range, beta_range=beta_range, h0=h0, dht=dht,
          grad_dtype=grad_dtype, scale=scale, mirror=mirror)
