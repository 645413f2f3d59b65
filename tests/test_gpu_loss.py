"""GPU: the packed-row loss and its logit gradient against oracle O10."""
import json
import math
import os

import numpy as np
import pytest

from oracle import loss_probe as LP
from oracle import packing as P
from tests.parity import say

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _run(z, tg, mask=None, dtype="f32", grad_dtype=None):
    import packed_varlen_block_amd as pvb
    torch = _torch()
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    zt = torch.tensor(np.asarray(z, dtype=np.float32)).to(dt).cuda()
    tt = torch.tensor(np.asarray(tg, dtype=np.int32)).cuda()
    mt = None if mask is None else torch.tensor(np.asarray(mask, dtype=np.uint8)).cuda()
    gdt = None if grad_dtype is None else (torch.float32 if grad_dtype == "f32" else torch.bfloat16)
    out = pvb.packed_nll(zt, tt, mt, grad=True, grad_dtype=gdt)
    return zt, out


def _check(z_used, tg, out, mask=None, grad_tol=1e-6):
    """Compare against O10 evaluated on the exact values the kernel saw."""
    import packed_varlen_block_amd as pvb
    pvb.check_status(out["status"])
    z64 = z_used.double().cpu().numpy()
    row, s, n, m = LP.packed_nll(z64, tg, mask)
    g = LP.packed_nll_grad(z64, tg, mask)
    assert out["count"].item() == n
    got_row = out["row_nll"].double().cpu().numpy()
    assert np.abs(got_row - row).max() <= 2e-5 * max(1.0, np.abs(row).max())
    loss = out["loss"].cpu().numpy()
    assert abs(loss[0] - s) <= 2e-5 * max(1.0, abs(s))
    assert abs(loss[1] - m) <= 2e-5 * max(1.0, abs(m))
    gg = out["grad"].double().cpu().numpy()
    e = LP.eligible_cells(tg, mask)
    assert np.all(gg[~e] == 0.0)
    assert np.abs(gg - g).max() <= grad_tol


def test_loss_probe_on_device():
    """The capacity-6 rows of the probe, laid flat (12 cells, 9 targets)."""
    say("loss: probe rows")
    g = json.load(open(os.path.join(GOLD, "nextfit_capacity6.json")))
    lp = json.load(open(os.path.join(GOLD, "loss_probe.json")))
    rows = P.packed_rows(g["documents"], g["capacity"])
    z = LP.constructed_logits(rows, lp["vocab"]).reshape(12, -1)
    tg = np.where(rows["valid"].reshape(-1), rows["targets"].reshape(-1), -1)
    zt, out = _run(z, tg)
    _check(zt, tg, out)
    loss = out["loss"].cpu().numpy()
    assert abs(loss[1] - 11 / 9 * math.log(2)) < 1e-6
    assert abs(loss[0] - 11 * math.log(2)) < 1e-5


def test_loss_probe_targets_from_device_gather():
    """Targets produced by the device packed-row gather of the same documents."""
    import packed_varlen_block_amd as pvb
    torch = _torch()
    say("loss: probe with device-gathered targets")
    g = json.load(open(os.path.join(GOLD, "nextfit_capacity6.json")))
    lp = json.load(open(os.path.join(GOLD, "loss_probe.json")))
    rows = P.packed_rows(g["documents"], g["capacity"])
    z = LP.constructed_logits(rows, lp["vocab"]).reshape(12, -1)
    targets = []
    for r in range(2):
        docs = [g["documents"][i] for i in range(len(g["documents"])) if rows["row_of"][i] == r]
        lens = [len(d) - 1 for d in docs]
        toks = np.concatenate([np.asarray(d, dtype=np.int32) for d in docs])
        offs = np.concatenate([[0], np.cumsum([len(d) for d in docs])[:-1]]).astype(np.int64)
        out = pvb.build_packed_row(torch.tensor(lens, dtype=torch.int32).cuda(), capacity=6,
                                   tokens=torch.tensor(toks).cuda(), tok_off=torch.tensor(offs).cuda())
        pvb.check_status(out["status"])
        targets.append(out["targets"].cpu().numpy())
    tg = np.concatenate(targets)
    zt, res = _run(z, tg)
    _check(zt, tg, res)
    assert abs(res["loss"][1].item() - 11 / 9 * math.log(2)) < 1e-6


@pytest.mark.parametrize("dtype,grad_dtype", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
def test_loss_random_sweep(dtype, grad_dtype):
    rng = np.random.default_rng(31)
    for C, V in ((1, 1), (7, 5), (300, 266), (129, 4096), (64, 32768), (33, 50257)):
        say(f"loss: C={C} V={V} logits={dtype} grad={grad_dtype}")
        z = rng.normal(size=(C, V)) * 3
        tg = rng.integers(0, V, size=C)
        tg[rng.random(C) < 0.2] = -100
        tg[rng.random(C) < 0.1] = -1
        tg[0] = 0 if V == 1 else tg[0] % V     # at least one eligible cell
        mask = (rng.random(C) > 0.1).astype(np.uint8)
        mask[0] = 1
        zt, out = _run(z, tg, mask, dtype, grad_dtype)
        # bf16 gradients carry a 2^-9 relative rounding of each entry
        tol = 1e-6 if grad_dtype == "f32" else 4e-3 / max(1, int(LP.eligible_cells(tg, mask).sum()))
        _check(zt, tg, out, mask, grad_tol=tol)


def test_loss_excluded_cells_with_nan_and_inf():
    """NaN/Inf logits in excluded cells leave every output unchanged."""
    torch = _torch()
    say("loss: excluded NaN/Inf cells")
    rng = np.random.default_rng(32)
    C, V = 40, 1000
    z = rng.normal(size=(C, V))
    tg = rng.integers(0, V, size=C)
    tg[[3, 17, 30]] = -100
    mask = np.ones(C, dtype=np.uint8)
    mask[[5, 6]] = 0
    _, a = _run(z, tg, mask)
    z2 = z.copy()
    z2[3, :] = np.nan
    z2[17, 10] = np.inf
    z2[5, :] = -np.inf
    z2[6, 0] = np.nan
    _, b = _run(z2, tg, mask)
    for k in ("row_nll", "loss", "count", "grad"):
        assert torch.equal(a[k], b[k]), k


def test_loss_device_detected_errors():
    import packed_varlen_block_amd as pvb
    torch = _torch()
    say("loss: zero eligible targets, target out of range")
    for tg, mask, code in (([-1, -100, -1], None, 8), ([0, 1, 2], [0, 0, 0], 8), ([0, 12, 1], None, 1)):
        zt = torch.zeros((3, 12), dtype=torch.float32, device="cuda")
        tt = torch.tensor(tg, dtype=torch.int32, device="cuda")
        mt = None if mask is None else torch.tensor(mask, dtype=torch.uint8, device="cuda")
        row = torch.full((3,), 7.0, device="cuda")
        loss = torch.full((2,), 7.0, dtype=torch.float64, device="cuda")
        grad = torch.full((3, 12), 7.0, device="cuda")
        cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
        st = torch.empty(1, dtype=torch.int32, device="cuda")
        rc = pvb.lib().pvb_packed_nll(zt.data_ptr(), pvb.PVB_F32, 3, 12, tt.data_ptr(),
                                      mt.data_ptr() if mt is not None else None, row.data_ptr(),
                                      loss.data_ptr(), cnt.data_ptr(), grad.data_ptr(), pvb.PVB_F32,
                                      st.data_ptr(), None)
        assert rc == 0
        torch.cuda.synchronize()
        assert st.item() == code
        assert (row == 7.0).all() and (loss == 7.0).all() and (grad == 7.0).all()
