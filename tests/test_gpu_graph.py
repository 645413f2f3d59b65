"""The hot path under HIP graph capture.

One step -- the device packed-row build from segment lengths, the forward and
the backward -- is recorded once into a graph and replayed.  Nothing in the
library allocates, frees, synchronises or clears memory with a memset, and the
forward and backward plan their work lists on the device from the device
cu_seqlens, so one recorded graph serves every pack with the same token count
and number of segments.  Each replay must equal the eager calls on the same
inputs bit for bit (every kernel of the path writes each output element once,
in a fixed order), also after the token values and the segment lengths change
in place between replays; eager work and synchronisations run between the
replays, and one head of each input set is checked against the oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import linear_attention as LA
from tests.parity import check, host_cu, say, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import packed_varlen_block_amd  # noqa: F401  (fails loudly if libpvb.so is missing)


def _bits(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)


def _step(L, q, k, v, do, T):
    import packed_varlen_block_amd as pvb
    row = pvb.build_packed_row(L, capacity=T)
    o, lse, st = pvb.varlen_attn_fwd(q, k, v, row["cu"])
    dq, dk, dv, st2 = pvb.varlen_attn_bwd(q, k, v, o, do, lse, row["cu"])
    return {"cu": row["cu"], "pos": row["pos"], "seg": row["seg"], "o": o, "lse": lse, "dq": dq, "dk": dk,
            "dv": dv, "status": (row["status"], st, st2)}


def _statuses_ok(out):
    import packed_varlen_block_amd as pvb
    for s in out["status"]:
        pvb.check_status(s)


def _same(name, a, b):
    import torch
    assert torch.equal(a, b), f"{name}: graph replay differs from the eager call"


def test_attention_step_graph_replays():
    import torch
    T, H, d = 2048, 8, 128
    packs = [[700, 1, 0, 300, 1047], [300, 1047, 0, 700, 1], [1, 1, 2046, 0, 0]]
    sets = [W.random_small(2100 + i, p, H=H, d=d, scale=0.5) for i, p in enumerate(packs)]
    dev = torch.device("cuda:0")
    # static inputs of the graph, first holding set 0
    sL = torch.tensor(np.asarray(packs[0], np.int32), device=dev)
    sq, sk, sv, sdo = (_bits(getattr(sets[0], n)).to(dev) for n in ("q", "k", "v", "do"))

    eager0 = _step(sL, sq, sk, sv, sdo, T)        # also warms the library up before capture
    _statuses_ok(eager0)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        static = _step(sL, sq, sk, sv, sdo, T)
    torch.cuda.synchronize()

    names = ("cu", "pos", "seg", "o", "lse", "dq", "dk", "dv")
    for rep, i in enumerate([0, 1, 2, 1, 0]):
        w = sets[i]
        say(f"graph replay {rep}: pack {packs[i]}")
        sL.copy_(torch.tensor(np.asarray(packs[i], np.int32)))
        for t, n in ((sq, "q"), (sk, "k"), (sv, "v"), (sdo, "do")):
            t.copy_(_bits(getattr(w, n)))
        # eager calls on fresh tensors with the same inputs, then the replay
        ref = _step(torch.tensor(np.asarray(packs[i], np.int32), device=dev), sq.clone(), sk.clone(),
                    sv.clone(), sdo.clone(), T)
        _statuses_ok(ref)
        graph.replay()
        torch.cuda.synchronize()
        _statuses_ok(static)
        for n in names:
            _same(n, static[n], ref[n])
        if rep < 3:
            # one head against the oracle
            hc = host_cu(w.lengths)
            assert np.array_equal(static["cu"].cpu().numpy(), hc)
            qo, ko, vo, doo = (W.bf16_bits_to_f64(x) for x in (w.q, w.k, w.v, w.do))
            h = 5
            ro, rl = A.varlen_forward(qo, ko, vo, hc, heads=[h])
            check("O", to64(static["o"])[:, h], ro[:, h])
            check("LSE", static["lse"].double().cpu().numpy()[h], rl[h], max_abs=1e-3, mean_abs=1e-4)
            rq, rk, rv = A.varlen_backward(qo, ko, vo, doo, hc, heads=[h])
            check("dQ", to64(static["dq"])[:, h], rq[:, h])
            check("dK", to64(static["dk"])[:, h], rk[:, h])
            check("dV", to64(static["dv"])[:, h], rv[:, h])


def test_gated_delta_graph_replays():
    import packed_varlen_block_amd as pvb
    import torch
    packs = [[130, 0, 64, 257], [257, 64, 0, 130]]
    sets = [W.random_gated_delta(2200 + i, p, H=4, Hk=2, initial_state=True) for i, p in enumerate(packs)]
    dev = torch.device("cuda:0")

    def upload(w):
        return {n: (_bits(w[n]) if w[n].dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(w[n])))
                for n in ("q", "k", "v", "g", "beta", "h0")}

    st_in = {n: t.to(dev) for n, t in upload(sets[0]).items()}
    sL = torch.tensor(np.asarray(packs[0], np.int32), device=dev)
    T = int(np.sum(packs[0]))

    def step(L, x):
        row = pvb.build_packed_row(L, capacity=T)
        o, ht, st = pvb.gated_delta_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], row["cu"],
                                        initial_state=x["h0"], o_dtype=torch.float32)
        return o, ht, (row["status"], st)

    o0, h0, s0 = step(sL, st_in)
    for s in s0:
        pvb.check_status(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        so, sh, ss = step(sL, st_in)
    torch.cuda.synchronize()
    for rep, i in enumerate([1, 0, 1]):
        w = sets[i]
        say(f"gated delta graph replay {rep}: pack {packs[i]}")
        sL.copy_(torch.tensor(np.asarray(packs[i], np.int32)))
        for n, t in upload(w).items():
            st_in[n].copy_(t)
        ro_, rh_, rs_ = step(torch.tensor(np.asarray(packs[i], np.int32), device=dev),
                             {n: t.clone() for n, t in st_in.items()})
        for s in rs_:
            pvb.check_status(s)
        graph.replay()
        torch.cuda.synchronize()
        for s in ss:
            pvb.check_status(s)
        _same("O", so, ro_)
        _same("final state", sh, rh_)
        if rep < 2:
            q, k = (W.bf16_bits_to_f64(w[n]) for n in ("q", "k"))
            v = W.bf16_bits_to_f64(w["v"])
            ref_o, ref_s = LA.gated_delta_varlen(q, k, v, w["g"].astype(np.float64), w["beta"].astype(np.float64),
                                                 host_cu(w["lengths"]), 1.0 / np.sqrt(128),
                                                 w["h0"].astype(np.float64))
            err_o = float(np.abs(so.double().cpu().numpy() - ref_o).max())
            err_s = float(np.abs(sh.double().cpu().numpy() - ref_s).max())
            say(f"  O max-abs {err_o:.3e}  state max-abs {err_s:.3e}")
            assert err_o <= 1e-3 * max(1.0, float(np.abs(ref_o).max()))
            assert err_s <= 1e-3 * max(1.0, float(np.abs(ref_s).max()))


def test_gated_delta_backward_graph_replays():
    """The gated delta backward recorded once into a HIP graph (its workspace
    allocated before the capture; value and query/key heads one to one, so no
    atomics and replays are bitwise repeatable) and replayed over two packs of
    the same size, each with a slice longer than one group of 1024 tokens (so
    the group maps, both walks and the group walks are recorded); every replay
    equals an eager call bit for bit, and the first two replays match O12."""
    import packed_varlen_block_amd as pvb
    import torch
    packs = [[1100, 0, 64, 257], [257, 64, 0, 1100]]
    H, d = 4, 128
    T = int(np.sum(packs[0]))
    sets = [W.random_gated_delta(2300 + i, p, H=H, initial_state=True) for i, p in enumerate(packs)]
    r = np.random.default_rng(2310)
    dos = [W.f32_to_bf16_bits(r.standard_normal((T, H, d)).astype(np.float32)) for _ in packs]
    dev = torch.device("cuda:0")

    def upload(w, do):
        x = {n: (_bits(w[n]) if w[n].dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(w[n])))
             for n in ("q", "k", "v", "g", "beta", "h0")}
        x["do"] = _bits(do)
        return x

    st_in = {n: t.to(dev) for n, t in upload(sets[0], dos[0]).items()}
    cu = torch.tensor(host_cu(packs[0]), dtype=torch.int32, device=dev)
    ws = torch.empty(pvb.gated_delta_bwd_workspace_bytes(T, H, len(packs[0])), dtype=torch.uint8, device=dev)

    def step(c, x):
        return pvb.gated_delta_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], c, x["do"], initial_state=x["h0"],
                                   workspace=ws)

    out0 = step(cu, st_in)
    pvb.check_status(out0[-1])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sout = step(cu, st_in)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
    for rep, i in enumerate([1, 0, 1]):
        w = sets[i]
        say(f"gated delta backward graph replay {rep}: pack {packs[i]}")
        cu.copy_(torch.tensor(host_cu(packs[i]), dtype=torch.int32))
        for n, t in upload(w, dos[i]).items():
            st_in[n].copy_(t)
        eager = step(cu.clone(), {n: t.clone() for n, t in st_in.items()})
        pvb.check_status(eager[-1])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        pvb.check_status(sout[-1])
        for n, a, b in zip(names, sout[:6], eager[:6]):
            _same(n, a, b)
        if rep < 2:
            f = W.bf16_bits_to_f64
            ref = LA.gated_delta_varlen_backward(f(w["q"]), f(w["k"]), f(w["v"]), w["g"].astype(np.float64),
                                                 w["beta"].astype(np.float64), host_cu(packs[i]),
                                                 1.0 / np.sqrt(d), f(dos[i]), w["h0"].astype(np.float64))
            for n, a, b in zip(names, sout[:6], ref):
                err = float(np.abs(a.double().cpu().numpy() - b).max())
                say(f"  {n} max-abs {err:.3e}")
                assert err <= 1e-3 * max(1.0, float(np.abs(b).max()))


def test_gated_delta_training_pair_graph_replays():
    """The training pair (the forward that leaves the backward's checkpoints,
    then the backward that reads them) recorded once into a HIP graph on one
    workspace and replayed over two packs of the same size, each with a slice
    longer than one group; every replay equals the plain forward and backward,
    called eagerly on their own workspaces, bit for bit."""
    import packed_varlen_block_amd as pvb
    import torch
    packs = [[1100, 0, 64, 257], [257, 64, 0, 1100]]
    H, d = 4, 128
    T, B = int(np.sum(packs[0])), len(packs[0])
    sets = [W.random_gated_delta(2400 + i, p, H=H, initial_state=True) for i, p in enumerate(packs)]
    r = np.random.default_rng(2410)
    dos = [W.f32_to_bf16_bits(r.standard_normal((T, H, d)).astype(np.float32)) for _ in packs]
    dev = torch.device("cuda:0")

    def upload(w, do):
        x = {n: (_bits(w[n]) if w[n].dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(w[n])))
             for n in ("q", "k", "v", "g", "beta", "h0")}
        x["do"] = _bits(do)
        return x

    st_in = {n: t.to(dev) for n, t in upload(sets[0], dos[0]).items()}
    cu = torch.tensor(host_cu(packs[0]), dtype=torch.int32, device=dev)
    ws = torch.empty(pvb.gated_delta_bwd_workspace_bytes(T, H, B), dtype=torch.uint8, device=dev)
    ws_e = torch.empty_like(ws)

    def pair(c, x):
        a = (x["q"], x["k"], x["v"], x["g"], x["beta"], c)
        o, ht, st = pvb.gated_delta_fwd(*a, initial_state=x["h0"], o_dtype=torch.float32, workspace=ws, train=True)
        grads = pvb.gated_delta_bwd(*a, x["do"], initial_state=x["h0"], workspace=ws, after_fwd=True)
        return (o, ht) + tuple(grads[:6]), (st, grads[-1])

    def plain(c, x):
        a = (x["q"], x["k"], x["v"], x["g"], x["beta"], c)
        o, ht, st = pvb.gated_delta_fwd(*a, initial_state=x["h0"], o_dtype=torch.float32)
        grads = pvb.gated_delta_bwd(*a, x["do"], initial_state=x["h0"], workspace=ws_e)
        return (o, ht) + tuple(grads[:6]), (st, grads[-1])

    out0, s0 = pair(cu, st_in)
    for s in s0:
        pvb.check_status(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sout, ss = pair(cu, st_in)
    torch.cuda.synchronize()
    names = ("O", "final state", "dq", "dk", "dv", "dg", "dbeta", "dh0")
    for rep, i in enumerate([1, 0, 1]):
        say(f"gated delta training pair graph replay {rep}: pack {packs[i]}")
        cu.copy_(torch.tensor(host_cu(packs[i]), dtype=torch.int32))
        for n, t in upload(sets[i], dos[i]).items():
            st_in[n].copy_(t)
        eager, es = plain(cu.clone(), {n: t.clone() for n, t in st_in.items()})
        for s in es:
            pvb.check_status(s)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for s in ss:
            pvb.check_status(s)
        for n, a, b in zip(names, sout, eager):
            _same(n, a, b)
