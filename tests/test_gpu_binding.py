"""GPU: the binding refuses mistyped or misplaced device arguments before any
launch (a host tensor or an int32 offset array read as int64 would become a
wild device address), and the calls still work with correct arguments."""
import pytest

from tests.parity import say

pytestmark = pytest.mark.gpu


def _refused(fn, *a, **kw):
    import packed_varlen_block_amd as pvb
    with pytest.raises(pvb.PvbError) as e:
        fn(*a, **kw)
    assert e.value.status == 1, str(e.value)


def test_each_bad_device_argument_is_refused():
    say("binding: bad device arguments")
    import torch

    import packed_varlen_block_amd as pvb
    dev = torch.device("cuda:0")
    i32 = dict(dtype=torch.int32, device=dev)
    L = torch.tensor([3, 2], **i32)
    toks = torch.arange(10, **i32)
    off = torch.tensor([0, 4], dtype=torch.int64, device=dev)
    _refused(pvb.build_packed_row, L.cpu(), capacity=5)
    _refused(pvb.build_packed_row, L, capacity=5, tokens=toks, tok_off=off.int())      # int32 offsets
    _refused(pvb.build_packed_row, L, capacity=5, tokens=toks, tok_off=off.cpu())      # host offsets
    _refused(pvb.build_packed_row, L, capacity=5, tokens=toks.cpu(), tok_off=off)      # host tokens
    _refused(pvb.build_packed_row, L, capacity=5, tokens=toks.long(), tok_off=off)     # int64 tokens
    _refused(pvb.build_packed_row, L, capacity=5, tokens=toks, tok_off=off[:1])        # one offset short
    _refused(pvb.build_packed_row, L, capacity=5, status=torch.zeros(1, dtype=torch.int64, device=dev))
    out = pvb.build_packed_row(L, capacity=5, tokens=toks, tok_off=off)
    pvb.check_status(out["status"])
    assert out["inputs"].cpu().tolist() == [0, 1, 2, 4, 5]

    pos = torch.tensor([0, 1, 2, 0, 1], **i32)
    _refused(pvb.boundaries_from_positions, pos.cpu())
    _refused(pvb.boundaries_from_positions, pos.long())
    _refused(pvb.boundaries_from_positions, pos, status=torch.zeros(1, device=dev))
    b = pvb.boundaries_from_positions(pos)
    pvb.check_status(b["status"])
    assert b["cu"][:3].cpu().tolist() == [0, 3, 5]

    logits = torch.zeros(4, 16, dtype=torch.bfloat16, device=dev)
    tg = torch.tensor([1, -100, 3, 2], **i32)
    _refused(pvb.packed_nll, logits.cpu(), tg)
    _refused(pvb.packed_nll, logits, tg.cpu())
    _refused(pvb.packed_nll, logits, tg.long())
    _refused(pvb.packed_nll, logits, tg, mask=torch.ones(4, dtype=torch.uint8))
    _refused(pvb.packed_nll, logits, tg, mask=torch.ones(4, dtype=torch.bool, device=dev))
    r = pvb.packed_nll(logits, tg)
    pvb.check_status(r["status"])
    assert r["count"].item() == 3

    q = torch.zeros(8, 2, 64, dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, 8], **i32)
    _refused(pvb.varlen_attn_fwd, q, q, q, cu.cpu())
    _refused(pvb.varlen_attn_fwd, q, q.cpu(), q, cu)
    _refused(pvb.varlen_attn_fwd, q, q, q, cu, out=torch.zeros(8, 2, 64, device=dev, dtype=torch.float16))
    _refused(pvb.varlen_attn_fwd, q, q, q, cu, lse=torch.zeros(8, 2, device=dev))
    _refused(pvb.varlen_attn_fwd, q, q, q, cu, workspace=torch.zeros(1 << 16, dtype=torch.uint8))
    o, lse, st = pvb.varlen_attn_fwd(q, q, q, cu)
    _refused(pvb.varlen_attn_bwd, q, q, q, o, q, lse.cpu(), cu)
    _refused(pvb.varlen_attn_bwd, q, q, q, o, q, lse, cu, dq=torch.zeros(8, 2, 64, dtype=torch.bfloat16, device=dev))
    pvb.varlen_attn_bwd(q, q, q, o, q, lse, cu)
    pvb.check_status(st)

    qg = torch.zeros(8, 2, 128, dtype=torch.bfloat16, device=dev)
    g = torch.zeros(8, 2, device=dev)
    _refused(pvb.gated_delta_fwd, qg, qg, qg, g.cpu(), g, cu)
    _refused(pvb.gated_delta_fwd, qg, qg, qg, g, g, cu, initial_state=torch.zeros(1, 2, 128, 128))
    _refused(pvb.gated_delta_fwd, qg, qg, qg, g, g, cu, state_out=torch.zeros(1, 2, 128, 128, device=dev).half())
    _, _, st = pvb.gated_delta_fwd(qg, qg, qg, g, g, cu)
    pvb.check_status(st)
