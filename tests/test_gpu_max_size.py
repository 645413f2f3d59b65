"""Forward and backward at the largest size the entry points accept: T·H·d
one token row short of 2^31 elements per tensor (T = 262143, H = 64, d = 128),
so byte offsets into Q, K, V, O, dO and the gradients pass 4 GB.  2047
segments of 128 tokens and a ragged last one of 127 keep the products cheap;
the segments at the start, in the middle and at the very end of the stream are
compared with the oracle on three heads.  O and the gradients are bf16 (about
35 GB of device memory in all)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from tests.parity import check, host_cu, say, to64

pytestmark = pytest.mark.gpu


def test_forward_backward_at_the_element_limit():
    import packed_varlen_block_amd as pvb
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    T, H, d = 262143, 64, 128
    assert T * H * d < 2 ** 31 <= (T + 1) * H * d
    lengths = [128] * 2047 + [127]
    hc = host_cu(lengths)
    dev = torch.device("cuda:0")
    say(f"max size: T={T} H={H} d={d} ({T * H * d} elements per tensor), {len(lengths)} segments")
    q, k, v, do = (W.device_normal_bf16((T, H, d), 7001 + i, 0.5, dev) for i in range(4))
    cu = torch.tensor(hc).to(dev)
    o, lse, st = pvb.varlen_attn_fwd(q, k, v, cu)
    pvb.check_status(st)
    dq, dk, dv, st = pvb.varlen_attn_bwd(q, k, v, o, do, lse, cu, grad_dtype=torch.bfloat16)
    pvb.check_status(st)
    heads = [0, 37, 63]
    for b in (0, 1023, len(lengths) - 1):
        a, e = int(hc[b]), int(hc[b + 1])
        say(f"  segment {b}: rows [{a}, {e})")
        take = lambda t: t[a:e][:, heads].double().cpu().numpy()
        qo, ko, vo, doo = take(q), take(k), take(v), take(do)
        ro, rl = A.varlen_forward(qo, ko, vo, [0, e - a])
        check("O", take(o), ro, bf16_out=True)
        check("LSE", lse[heads][:, a:e].double().cpu().numpy(), rl, max_abs=1e-3, mean_abs=1e-4)
        rq, rk, rv = A.varlen_backward(qo, ko, vo, doo, [0, e - a])
        for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            check(name, take(got), ref, bf16_out=True)
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_packed_loss_past_2_to_the_32_elements():
    """C = 140000 cells over a 32768 vocabulary: 4.6e9 logits (9.2 GB of bf16,
    the same again for the gradient), so row offsets pass 2^32 elements.  Rows
    at the start and the end of the matrix are compared with O10."""
    import packed_varlen_block_amd as pvb
    import torch
    from oracle import loss_probe as LP
    C, V = 140000, 32768
    assert C * V > 2 ** 32
    dev = torch.device("cuda:0")
    say(f"loss C={C} V={V} ({C * V} logits)")
    z = W.device_normal_bf16((C, V), 7101, 2.0, dev)
    r = np.random.default_rng(7102)
    tg = r.integers(0, V, size=C).astype(np.int32)
    tg[r.random(C) < 0.01] = -100
    out = pvb.packed_nll(z, torch.tensor(tg).to(dev))
    pvb.check_status(out["status"])
    n = int(LP.eligible_cells(tg, None).sum())
    assert out["count"].item() == n
    rows = np.r_[0:8, C // 2:C // 2 + 8, C - 16:C]
    zs = z[torch.tensor(rows).to(dev)].double().cpu().numpy()
    rrow, _, ns, _ = LP.packed_nll(zs, tg[rows], None)
    got_row = out["row_nll"].double().cpu().numpy()
    assert np.abs(got_row[rows] - rrow).max() <= 2e-5 * max(1.0, np.abs(rrow).max())
    rg = LP.packed_nll_grad(zs, tg[rows], None) * (ns / n)
    gg = out["grad"][torch.tensor(rows).to(dev)].double().cpu().numpy()
    assert np.abs(gg - rg).max() <= 4e-3 / n
    total = float(np.sum(got_row))
    assert abs(float(out["loss"][0].item()) - total) <= 1e-6 * abs(total)
    del z, out
    torch.cuda.empty_cache()


def test_gated_delta_forward_backward_at_the_element_limit():
    """The gated delta rule, forward and backward, with T·H·d one token row short
    of 2^31 elements in v, O, dO and dv (T = 262143, H = 64 value heads over 32
    query/key heads, d = 128): byte offsets pass 4 GB, dq and dk are summed over
    value-head pairs with atomics, and the backward's workspace is about 58 GB.
    255 slices of 1024 tokens and a ragged last one of 1023, with initial states
    and final-state gradients; slices at the start, in the middle and at the end
    are compared with O11 and O12 on three value heads (and their query/key
    heads, summed over both value heads that share each)."""
    import packed_varlen_block_amd as pvb
    import torch
    from oracle import linear_attention as LA
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    T, H, Hk, d = 262143, 64, 32, 128
    assert T * H * d < 2 ** 31 <= (T + 1) * H * d
    lengths = [1024] * 255 + [1023]
    B = len(lengths)
    hc = host_cu(lengths)
    dev = torch.device("cuda:0")
    say(f"gated delta max size: T={T} H={H} H_k={Hk} d={d}, {B} slices")
    q = W.device_unit_rows_bf16((T, Hk, d), 7101, dev)
    k = W.device_unit_rows_bf16((T, Hk, d), 7102, dev)
    v = W.device_normal_bf16((T, H, d), 7103, 1.0, dev)
    do = W.device_normal_bf16((T, H, d), 7104, 1.0, dev)
    g = W.device_uniform_f32((T, H), 7105, -0.1, 0.0, dev)
    beta = W.device_uniform_f32((T, H), 7106, 0.05, 1.0, dev)
    h0 = W.device_normal_bf16((B, H, d, d), 7107, 0.125, dev).float()
    dht = W.device_normal_bf16((B, H, d, d), 7108, 0.125, dev).float()
    cu = torch.tensor(hc).to(dev)
    o, ht, st = pvb.gated_delta_fwd(q, k, v, g, beta, cu, h_cu=hc, initial_state=h0)
    pvb.check_status(st)
    dq, dk, dv, dg, db, dh0, st = pvb.gated_delta_bwd(q, k, v, g, beta, cu, do, h_cu=hc, initial_state=h0,
                                                      dht=dht, grad_dtype=torch.bfloat16)
    pvb.check_status(st)
    sc = 1.0 / np.sqrt(d)

    def bar(ref):
        return 1e-3 * max(1.0, float(np.abs(ref).max()))
    for b, heads in ((0, (0, 1)), (127, (36, 37)), (B - 1, (62, 63))):
        a, e = int(hc[b]), int(hc[b + 1])
        hk = heads[0] // 2
        say(f"  slice {b}: rows [{a}, {e}), value heads {heads}, query/key head {hk}")
        qo = q[a:e, hk].double().cpu().numpy()
        ko = k[a:e, hk].double().cpu().numpy()
        rdq, rdk = np.zeros((e - a, d)), np.zeros((e - a, d))
        for h in heads:
            vo = v[a:e, h].double().cpu().numpy()
            go, bo = g[a:e, h].double().cpu().numpy(), beta[a:e, h].double().cpu().numpy()
            s0 = h0[b, h].double().cpu().numpy()
            ro, rs = LA.gated_delta_segment(qo, ko, vo, go, bo, sc, s0)
            got = {"O": o[a:e, h].double().cpu().numpy(), "final state": ht[b, h].double().cpu().numpy()}
            for name, ref in (("O", ro), ("final state", rs)):
                err = float(np.abs(got[name] - ref).max())
                extra = 2.0 ** -8 * float(np.abs(ref).max()) if name == "O" else 0.0
                say(f"    h{h} {name}: max-abs {err:.3e}")
                assert err <= bar(ref) + extra, name
            r = LA.gated_delta_segment_backward(qo, ko, vo, go, bo, sc, do[a:e, h].double().cpu().numpy(), s0,
                                                dht[b, h].double().cpu().numpy())
            rdq += r[0]
            rdk += r[1]
            got = {"dv": dv[a:e, h], "dg": dg[a:e, h], "dbeta": db[a:e, h], "dh0": dh0[b, h]}
            for name, ref in zip(("dv", "dg", "dbeta", "dh0"), r[2:]):
                err = float(np.abs(got[name].double().cpu().numpy() - ref).max())
                extra = 2.0 ** -8 * float(np.abs(ref).max()) if name == "dv" else 0.0
                say(f"    h{h} {name}: max-abs {err:.3e}")
                assert err <= bar(ref) + extra, name
        for name, got, ref in (("dq", dq[a:e, hk], rdq), ("dk", dk[a:e, hk], rdk)):
            err = float(np.abs(got.double().cpu().numpy() - ref).max())
            say(f"    hk{hk} {name}: max-abs {err:.3e}")
            assert err <= bar(ref), name
    # the training pair on the same inputs: the same results as the plain calls,
    # bit for bit (dq and dk, summed over the value-head pairs with atomics in
    # no fixed order, to 1e-6 of their largest magnitude)
    say("  the training pair at the same size, against the plain calls")
    ws = torch.empty(pvb.gated_delta_bwd_workspace_bytes(T, H, B), dtype=torch.uint8, device=dev)
    o2, ht2, st = pvb.gated_delta_fwd(q, k, v, g, beta, cu, h_cu=hc, initial_state=h0, workspace=ws, train=True)
    pvb.check_status(st)
    grads = pvb.gated_delta_bwd(q, k, v, g, beta, cu, do, h_cu=hc, initial_state=h0, dht=dht,
                                grad_dtype=torch.bfloat16, workspace=ws, after_fwd=True)
    pvb.check_status(grads[-1])
    del ws
    for name, a2, a1 in (("O", o2, o), ("final state", ht2, ht), ("dv", grads[2], dv), ("dg", grads[3], dg),
                         ("dbeta", grads[4], db), ("dh0", grads[5], dh0)):
        assert torch.equal(a2, a1), f"training pair {name} differs from the plain call"
    for name, a2, a1 in (("dq", grads[0], dq), ("dk", grads[1], dk)):
        err = float((a2 - a1).abs().max())
        say(f"    training pair {name}: max-abs difference {err:.3e}")
        assert err <= 1e-6 * max(1.0, float(a1.abs().max())), name
    del o2, ht2, grads
    del q, k, v, do, o, ht, dq, dk, dv, dg, db, dh0
    torch.cuda.empty_cache()
