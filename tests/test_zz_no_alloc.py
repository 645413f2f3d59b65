"""GPU: the backward without a workspace (pvb_varlen_attn_bwd_noalloc, for
callers that cannot allocate) equals the workspace entry point bit for bit,
on two calls in a row whose second input is smaller (the fixed scratch keeps
the first call's contents), and stays within the attention bar of the oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from tests.parity import check, dev_bf16, host_cu, say, to64

pytestmark = pytest.mark.gpu


def _case(seed, lengths, H, Hk, d, gdtype):
    import torch

    import packed_varlen_block_amd as pvb
    qb, kb, vb, db = W.random_cross(seed, lengths, lengths, H, Hk, d, scale=0.5)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(db)
    hc = host_cu(lengths)
    cu = torch.tensor(hc).cuda()
    o, lse, st = pvb.varlen_attn_fwd(q, k, v, cu)
    pvb.check_status(st)
    ref = pvb.varlen_attn_bwd(q, k, v, o, do, lse, cu, grad_dtype=gdtype)
    pvb.check_status(ref[3])
    T = int(hc[-1])
    out = [torch.full(s, float("nan"), dtype=gdtype, device="cuda") for s in ((T, H, d), (T, Hk, d), (T, Hk, d))]
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    pvb.varlen_attn_bwd_noalloc(q, k, v, o, do, lse, cu, *out, status)
    pvb.check_status(status)
    for name, a, b in zip(("dQ", "dK", "dV"), out, ref[:3]):
        assert torch.equal(a, b), f"{name} differs from the workspace entry point"
    # one query head and its key/value head against the oracle
    f = W.bf16_bits_to_f64
    qo, ko, vo, doo = f(qb), f(kb), f(vb), f(db)
    G = H // Hk
    rq, rk, rv = A.varlen_backward(qo, ko, vo, doo, hc, heads=list(range(G)))
    check("dQ", to64(out[0])[:, :G], rq[:, :G], bf16_out=gdtype == torch.bfloat16)
    check("dK", to64(out[1])[:, :1], rk[:, :1], bf16_out=gdtype == torch.bfloat16)
    check("dV", to64(out[2])[:, :1], rv[:, :1], bf16_out=gdtype == torch.bfloat16)


def test_noalloc_backward_equals_workspace_call_twice_then_smaller():
    import torch
    say("noalloc backward: T=8192 pack (planner path), then a smaller pack (in-kernel decode)")
    # 4 segments over 8192 tokens at 16 heads: 1072 workgroups, the planner's list
    _case(41, [3000, 0, 4000, 1192], 16, 8, 128, torch.float32)
    # smaller, grouped heads, bf16 gradients, d = 64: decoded in the kernels
    _case(42, [100, 37, 0, 255], 4, 2, 64, torch.bfloat16)


def test_noalloc_backward_refuses_sizes_beyond_its_scratch():
    import torch

    import packed_varlen_block_amd as pvb
    say("noalloc backward: a size beyond the scratch is refused before any launch")
    T, H, d = 262144, 32, 64
    x = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, T), device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    g = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(pvb.PvbError) as e:
        pvb.varlen_attn_bwd_noalloc(x, x, x, x, x, lse, cu, g, g, g, st)
    assert e.value.status == 5
