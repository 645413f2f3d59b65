"""GPU parity of the gated delta rule over a packed stream (state reset at every
boundary) against the fp64 oracle O11."""
import numpy as np
import pytest

import workloads as W
from oracle import linear_attention as LA
from tests.parity import host_cu, say

pytestmark = pytest.mark.gpu

# Bars (per tensor, absolute, against fp64): the kernel works in fp32 with
# matrix-core products of two-part bf16 operands (about 16 significant bits),
# so its own error is a few 1e-5 of the values' scale; 1e-3 leaves margin for
# long slices.  A bf16 output also carries its own rounding: half an ulp, up
# to 2^-9 of the largest |O|.
TOL_F32 = 1e-3
BF16_ULP = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import packed_varlen_block_amd  # noqa: F401  (fails loudly if libpvb.so is missing)


def _dev(x, dtype=None):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _check(name, got, ref, tol):
    err = np.abs(got - ref)
    mx = float(err.max(initial=0.0))
    say(f"  {name}: max-abs {mx:.3e}  mean-abs {float(err.mean()) if err.size else 0.0:.3e}  (bar {tol:.2e})")
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert mx <= tol, f"{name}: max-abs {mx:.3e} > {tol:.3e}"


def _run(w, o_dtype="f32", heads=None, scale=None, check=True):
    import packed_varlen_block_amd as pvb
    import torch
    T, H, d = w["v"].shape
    hc = host_cu(w["lengths"])
    cu = _dev(hc)
    h0 = _dev(w["h0"]) if "h0" in w else None
    od = torch.float32 if o_dtype == "f32" else torch.bfloat16
    o, ht, st = pvb.gated_delta_fwd(_dev(w["q"]), _dev(w["k"]), _dev(w["v"]), _dev(w["g"]), _dev(w["beta"]), cu,
                                    h_cu=hc, scale=scale, initial_state=h0, o_dtype=od)
    pvb.check_status(st)
    if not check:
        return o, ht
    hs = list(range(H)) if heads is None else list(heads)
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    G = H // w["q"].shape[1]
    hq = sorted({h // G for h in hs})               # the query/key heads the sampled heads read
    q, k = (W.bf16_bits_to_f64(w[x])[:, hq] for x in ("q", "k"))
    if G > 1:                                       # one query/key head per sampled value head
        q, k = (np.ascontiguousarray(x[:, [hq.index(h // G) for h in hs]]) for x in (q, k))
    else:
        q, k = (W.bf16_bits_to_f64(w[x])[:, hs] for x in ("q", "k"))
    v = W.bf16_bits_to_f64(w["v"])[:, hs]
    g, b = w["g"].astype(np.float64)[:, hs], w["beta"].astype(np.float64)[:, hs]
    s0 = w["h0"].astype(np.float64)[:, hs] if "h0" in w else None
    ro, rs = LA.gated_delta_varlen(q, k, v, g, b, hc, sc, s0)
    go = o.double().cpu().numpy()[:, hs]
    tol = TOL_F32 * max(1.0, float(np.abs(ro).max(initial=0.0)))
    if o_dtype == "bf16":
        tol += BF16_ULP * float(np.abs(ro).max(initial=0.0))
    _check("O", go, ro, tol)
    if ht is not None:
        _check("final state", ht.double().cpu().numpy()[:, hs], rs,
               TOL_F32 * max(1.0, float(np.abs(rs).max(initial=0.0))))
    return o, ht


SMALL = [[1], [2], [63], [64], [65], [127], [128], [129], [5, 3, 4], [0, 0, 7, 0],
         [200, 1, 0, 130, 64, 65], [300]]


@pytest.mark.parametrize("o_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("init", [False, True])
def test_small_sweep(o_dtype, init):
    for i, lengths in enumerate(SMALL):
        say(f"gated delta lengths={lengths} o={o_dtype} init={init}")
        w = W.random_gated_delta(900 + i, lengths, H=2, initial_state=init)
        _run(w, o_dtype)


@pytest.mark.parametrize("g_range,beta_range", [((0.0, 0.0), (0.05, 1.0)), ((-1.0, 0.0), (0.05, 1.0)),
                                                ((-0.02, 0.0), (0.9, 1.0)), ((-8.0, -4.0), (0.0, 0.3))])
def test_gate_ranges(g_range, beta_range):
    lengths = [130, 64, 1, 257]
    say(f"gated delta gates g={g_range} beta={beta_range}")
    w = W.random_gated_delta(930, lengths, H=2, g_range=g_range, beta_range=beta_range, initial_state=True)
    _run(w, "f32")


def test_many_short_slices():
    """600 slices of 0-20 tokens (the cu_seqlens check strides over them)."""
    lengths = np.random.default_rng(985).integers(0, 21, size=600)
    say(f"gated delta {len(lengths)} slices, T={int(lengths.sum())}")
    w = W.random_gated_delta(986, lengths, H=2, initial_state=True)
    _run(w, "f32")


def test_long_slices():
    for i, lengths in enumerate(([1030], [2100, 5], [700, 0, 1500])):
        say(f"gated delta long lengths={lengths}")
        w = W.random_gated_delta(940 + i, lengths, H=2, g_range=(-0.05, 0.0), initial_state=i == 1)
        _run(w, "f32")


def test_long_mixed_pack_sampled_heads():
    """The T=32768 long mixed pack at 32 heads, launched as the bench launches
    it (bf16 O, final states), two heads compared in full."""
    lengths = W.lengths_cfg4(0)
    say(f"gated delta T={int(lengths.sum())} segments={len(lengths)} H=32 (heads 0 and 21)")
    w = W.random_gated_delta(950, lengths, H=32, g_range=(-0.1, 0.0))
    _run(w, "bf16", heads=[0, 21])


@pytest.mark.parametrize("H,Hk", [(4, 2), (6, 1), (8, 8)])
def test_grouped_query_key_heads(H, Hk):
    say(f"gated delta grouped heads H={H} H_k={Hk}")
    w = W.random_gated_delta(990, [130, 0, 64, 257], H=H, Hk=Hk, initial_state=True)
    _run(w, "f32")


def test_grouped_heads_long_mixed_pack():
    """The long mixed pack with 32 value heads over 16 query/key heads."""
    lengths = W.lengths_cfg4(0)
    say("gated delta long mixed pack H=32 H_k=16 (heads 1 and 30)")
    w = W.random_gated_delta(995, lengths, H=32, Hk=16, g_range=(-0.1, 0.0))
    _run(w, "bf16", heads=[1, 30])


def test_scale_argument_and_isolation():
    import torch
    lengths = [40, 70, 33]
    w = W.random_gated_delta(960, lengths, H=3, initial_state=True)
    say("gated delta scale 0.3")
    o1, h1 = _run(w, "f32", scale=0.3)
    # NaN in the middle slice's values reaches no other slice
    w2 = dict(w)
    v = w["v"].copy()
    v[40:110] = 0x7FC0                                   # bf16 NaN
    w2["v"] = v
    o2, h2 = _run(w2, "f32", scale=0.3, check=False)
    keep = np.r_[0:40, 110:143]
    assert torch.equal(o1[keep], o2[keep])
    assert torch.isnan(o2[40:110]).all()
    assert torch.equal(h1[[0, 2]], h2[[0, 2]])


def test_empty_and_zero_length_slices():
    import packed_varlen_block_amd as pvb
    import torch
    say("gated delta: zero-length slices keep their initial state; empty stream")
    w = W.random_gated_delta(970, [0, 5, 0], H=2, initial_state=True)
    o, ht = _run(w, "f32")
    assert torch.equal(ht[0], _dev(w["h0"])[0]) and torch.equal(ht[2], _dev(w["h0"])[2])
    z = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    zf = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0], dtype=torch.int32, device="cuda")
    o, ht, st = pvb.gated_delta_fwd(z, z, z, zf, zf, cu)
    pvb.check_status(st)
    assert o.numel() == 0 and ht.numel() == 0


def test_bad_device_cu_writes_nothing():
    import packed_varlen_block_amd as pvb
    import torch
    say("gated delta: bad device cu_seqlens")
    w = W.random_gated_delta(980, [30, 34], H=2)
    bad = torch.tensor([0, 50, 40], dtype=torch.int32, device="cuda")     # decreasing, and not ending at T
    o = torch.full((64, 2, 128), 7.0, device="cuda")
    ht = torch.full((2, 2, 128, 128), 7.0, device="cuda")
    st = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    pvb.gated_delta_fwd(_dev(w["q"]), _dev(w["k"]), _dev(w["v"]), _dev(w["g"]), _dev(w["beta"]), bad,
                        o_dtype=torch.float32, out=o, state_out=ht, status=st)
    torch.cuda.synchronize()
    assert st.item() == 4
    assert (o == 7.0).all() and (ht == 7.0).all()


# seeded random draws: slice lengths on and next to the 64-token chunk edges,
# anywhere below 300, or zero; grouped query/key heads; gate and write-strength
# ranges; with or without initial states; fp32 or bf16 O; two scales
CHUNK_EDGES = [1, 63, 64, 65, 127, 128, 129, 192]


@pytest.mark.parametrize("case", range(12))
def test_random_draws(case):
    r = np.random.default_rng(5000 + case)
    n = int(r.integers(1, 7))
    lengths = [0 if (u := r.random()) < 0.12 else int(r.choice(CHUNK_EDGES)) if u < 0.5 else int(r.integers(1, 300))
               for _ in range(n)]
    Hk = int(r.integers(1, 4))
    H = Hk * int(r.choice([1, 2, 4]))
    g_range = [(0.0, 0.0), (-0.1, 0.0), (-1.0, 0.0), (-6.0, -2.0)][int(r.integers(0, 4))]
    beta_range = [(0.05, 1.0), (0.9, 1.0), (0.0, 0.3)][int(r.integers(0, 3))]
    init = bool(r.random() < 0.5)
    o_dtype = "bf16" if r.random() < 0.4 else "f32"
    scale = None if r.random() < 0.6 else 0.3
    say(f"gated delta random {case}: lengths={lengths} H={H} H_k={Hk} g={g_range} beta={beta_range} "
        f"init={init} o={o_dtype} scale={scale}")
    w = W.random_gated_delta(5100 + case, lengths, H=H, Hk=Hk, g_range=g_range, beta_range=beta_range,
                             initial_state=init)
    _run(w, o_dtype, scale=scale)


@pytest.mark.parametrize("Hk", [4, 2])
def test_grouped_evaluation_equals_one_chain(Hk):
    """Slices longer than one group of 1024 tokens (2.9 groups, exactly one and
    two groups, one token more than a group, and short ones): the grouped
    evaluation (the default, with a workspace) matches O11 on two heads, and
    one chain per (slice, head) (no workspace) agrees with it within rounding."""
    import torch

    import packed_varlen_block_amd as pvb
    lengths = [3000, 1024, 0, 2048, 1025, 100, 64]
    H = 4
    say(f"gated delta grouped vs chain: lengths {lengths}, H {H}, H_k {Hk}")
    w = W.random_gated_delta(5300 + Hk, lengths, H=H, Hk=Hk, initial_state=True)
    og, hg_ = _run(w, "f32", heads=[0, 3])
    oc, hc_, sc = pvb.gated_delta_fwd(_dev(w["q"]), _dev(w["k"]), _dev(w["v"]), _dev(w["g"]), _dev(w["beta"]),
                                      _dev(host_cu(lengths)), initial_state=_dev(w["h0"]), o_dtype=torch.float32,
                                      chain=True)
    pvb.check_status(sc)
    d_o = float((og - oc).abs().max())
    d_s = float((hg_ - hc_).abs().max())
    say(f"  grouped vs chain: O {d_o:.3e}, final states {d_s:.3e}")
    assert d_o <= 1e-3 * max(1.0, float(oc.abs().max())) and d_s <= 1e-3 * max(1.0, float(hc_.abs().max()))
