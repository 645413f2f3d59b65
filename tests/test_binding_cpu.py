"""The Python binding refuses bad device arguments before any library call.

A host tensor, an int32 offset array read as int64, or a wrong shape would hand
the kernels a wild address; the binding raises PvbError(PVB_E_INVALID_ARG)
first.  On the CPU every tensor is a host tensor, so each call below must fail
in the binding, and the library stand-in proves that nothing reached the C ABI.
"""
import numpy as np
import pytest
import torch

import packed_varlen_block_amd as pvb


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"the binding called {name} with arguments it should have refused")


@pytest.fixture
def no_lib(monkeypatch):
    monkeypatch.setattr(pvb, "_lib", _NoCalls())
    yield


def _raises_invalid(fn, *a, **kw):
    with pytest.raises(pvb.PvbError) as e:
        fn(*a, **kw)
    assert e.value.status == 1, str(e.value)
    return str(e.value)


def test_need_checks_each_property(no_lib):
    t = torch.zeros(4, 3, dtype=torch.int32)
    assert "must be torch.int64" in _raises_invalid(pvb._need, t, "x", torch.int64)
    assert "shape (4, 4)" in _raises_invalid(pvb._need, t, "x", torch.int32, (4, 4))
    assert "2-d" not in _raises_invalid(pvb._need, t, "x", dim=1)
    assert "contiguous" in _raises_invalid(pvb._need, t.t(), "x", torch.int32, (3, 4))
    assert "CUDA" in _raises_invalid(pvb._need, t, "x", torch.int32, (4, 3))
    assert "torch tensor" in _raises_invalid(pvb._need, np.zeros(3), "x")


def test_packed_row_and_positions_refuse_host_and_mistyped_tensors(no_lib):
    L = torch.tensor([3, 2], dtype=torch.int32)
    _raises_invalid(pvb.build_packed_row, L, capacity=5)                       # host lengths
    _raises_invalid(pvb.build_packed_row, L.long(), capacity=5)                # int64 lengths
    _raises_invalid(pvb.build_packed_row, L, capacity=5, tokens=torch.zeros(8, dtype=torch.int32))  # no tok_off
    _raises_invalid(pvb.build_packed_row, L, capacity=5, tok_off=torch.zeros(2, dtype=torch.int64))  # no tokens
    _raises_invalid(pvb.boundaries_from_positions, torch.zeros(6, dtype=torch.int32))   # host positions
    _raises_invalid(pvb.boundaries_from_positions, torch.zeros(6, dtype=torch.int64))   # int64 positions
    _raises_invalid(pvb.boundaries_from_positions, torch.zeros(2, 3, dtype=torch.int32))


def test_loss_refuses_host_and_mistyped_tensors(no_lib):
    logits = torch.zeros(4, 10, dtype=torch.bfloat16)
    tg = torch.zeros(4, dtype=torch.int32)
    _raises_invalid(pvb.packed_nll, logits, tg)                                # host logits
    _raises_invalid(pvb.packed_nll, logits.half(), tg)                         # unsupported dtype
    _raises_invalid(pvb.packed_nll, logits.t(), tg)                            # not contiguous
    _raises_invalid(pvb.packed_nll, torch.zeros(40, dtype=torch.bfloat16), tg)  # 1-d logits


def test_attention_refuses_host_and_mistyped_tensors(no_lib):
    q = torch.zeros(8, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    _raises_invalid(pvb.varlen_attn_fwd, q, q, q, cu)                          # host tensors
    _raises_invalid(pvb.varlen_attn_fwd, q.float(), q, q, cu)                  # fp32 q
    _raises_invalid(pvb.varlen_attn_fwd, q, q[:, :1].expand(8, 2, 64), q, cu)  # non-contiguous k
    lse = torch.zeros(2, 8)
    _raises_invalid(pvb.varlen_attn_bwd, q, q, q, q, q, lse, cu)
    _raises_invalid(pvb.varlen_cross_attn_fwd, q, q, q, cu, cu, [0, 8], [0, 8])
    _raises_invalid(pvb.varlen_cross_attn_bwd, q, q, q, q, q, lse, cu, cu, [0, 8], [0, 8])


def test_gated_delta_refuses_host_and_mistyped_tensors(no_lib):
    q = torch.zeros(8, 2, 128, dtype=torch.bfloat16)
    g = torch.zeros(8, 2)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    _raises_invalid(pvb.gated_delta_fwd, q, q, q, g, g, cu)
    _raises_invalid(pvb.gated_delta_fwd, q.float(), q, q, g, g, cu)
