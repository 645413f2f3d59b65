"""GPU: the device packed-row scan is bit-exact against oracle O1/O2/O4."""
import json
import os

import numpy as np
import pytest

from oracle import packing as P
from tests.parity import say

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _row(lengths, capacity=None, base=0, **kw):
    import packed_varlen_block_amd as pvb
    torch = _torch()
    L = torch.tensor(np.asarray(lengths, dtype=np.int32), dtype=torch.int32).cuda()
    return pvb.build_packed_row(L, capacity=capacity, segment_base=base, **kw)


def test_worked_example():
    say("packed_row: worked example 5/3/4")
    g = json.load(open(os.path.join(GOLD, "worked_5_3_4.json")))
    out = _row(g["lengths"])
    import packed_varlen_block_amd as pvb
    pvb.check_status(out["status"])
    assert out["cu"].cpu().tolist() == g["cu_seqlens"]
    assert out["pos"].cpu().tolist() == g["position_ids"]
    assert out["max_seqlen"].item() == g["max_seqlen"]
    assert out["seg"].cpu().tolist() == [0] * 5 + [1] * 3 + [2] * 4


def test_fixture_rows_with_token_gather():
    say("packed_row: capacity-6 fixture with token gather")
    import packed_varlen_block_amd as pvb
    torch = _torch()
    g = json.load(open(os.path.join(GOLD, "nextfit_capacity6.json")))
    docs = g["documents"]
    lengths = [len(d) - 1 for d in docs]
    row_of, start_of, n_rows = pvb.pack_plan_nextfit(lengths, g["capacity"])
    toks = torch.tensor(sum(docs, []), dtype=torch.int32).cuda()
    doc_off = np.concatenate([[0], np.cumsum([len(d) for d in docs])[:-1]])
    for r in range(n_rows):
        members = [i for i in range(len(docs)) if row_of[i] == r]
        L = [lengths[i] for i in members]
        off = torch.tensor(doc_off[members].astype(np.int64)).cuda()
        out = _row(L, capacity=g["capacity"], base=members[0], tokens=toks, tok_off=off)
        pvb.check_status(out["status"])
        assert out["inputs"].cpu().tolist() == g["inputs"][r]
        assert out["targets"].cpu().tolist() == g["targets"][r]
        assert out["seg"].cpu().tolist() == g["segments"][r]
        assert out["pos"].cpu().tolist() == g["positions"][r]
        assert [bool(x) for x in out["valid"].cpu().tolist()] == g["valid"][r]


def test_random_rows_bit_exact():
    say("packed_row: random rows incl. zero lengths, padding, 5000 segments")
    import packed_varlen_block_amd as pvb
    from workloads import lengths_cfg5
    rng = np.random.default_rng(1)
    cases = [([], 0, 0), ([], 7, 3), (lengths_cfg5(0)[0].tolist(), 16384 + 37, 5),
             (rng.integers(0, 9, size=5000).tolist(), None, 11)]
    for _ in range(20):
        lengths = rng.integers(0, 300, size=int(rng.integers(1, 40))).tolist()
        cases.append((lengths, sum(lengths) + int(rng.integers(0, 50)), int(rng.integers(0, 100))))
    for lengths, cap, base in cases:
        C = sum(lengths) if cap is None else cap
        out = _row(lengths, capacity=C, base=base)
        pvb.check_status(out["status"])
        ref = P.packed_row_metadata(lengths, C, base)
        assert np.array_equal(out["cu"].cpu().numpy(), ref["cu"])
        assert np.array_equal(out["pos"].cpu().numpy(), ref["pos"])
        assert np.array_equal(out["seg"].cpu().numpy(), ref["seg"])
        assert out["max_seqlen"].item() == ref["max_seqlen"]


def test_device_detected_errors():
    say("packed_row: device-detected errors")
    import packed_varlen_block_amd as pvb
    for lengths, cap, code in (([3, 4], 6, 2), ([3, -1], 8, 1), ([2**31 - 1, 1], 8, 3)):
        out = _row(lengths, capacity=cap)
        with pytest.raises(pvb.PvbError) as e:
            pvb.check_status(out["status"])
        assert e.value.status == code


# ------------------------------------------------ boundaries from positions (O9)

def _bounds(pos, sentinel="zero", capacity=None):
    import packed_varlen_block_amd as pvb
    torch = _torch()
    p = torch.tensor(np.asarray(pos, dtype=np.int32), dtype=torch.int32).cuda()
    out = pvb.boundaries_from_positions(p, sentinel, capacity)
    return out


def _check_bounds(pos, sentinel="zero"):
    import packed_varlen_block_amd as pvb
    out = _bounds(pos, sentinel)
    pvb.check_status(out["status"])
    cu, mx = P.boundaries_from_positions(pos, sentinel)
    n = out["n_seg"].item()
    assert n == len(cu) - 1
    assert np.array_equal(out["cu"].cpu().numpy()[:n + 1], cu)
    assert out["max_seqlen"].item() == mx


def test_boundaries_worked_example():
    say("boundaries: worked example table")
    g = json.load(open(os.path.join(GOLD, "worked_5_3_4.json")))
    for sentinel in ("zero", "min"):
        out = _bounds(g["position_ids"], sentinel)
        import packed_varlen_block_amd as pvb
        pvb.check_status(out["status"])
        assert out["n_seg"].item() == 3
        assert out["cu"].cpu().tolist()[:4] == g["cu_seqlens"]
        assert out["max_seqlen"].item() == g["max_seqlen"]


def test_boundaries_round_trip_device_rows():
    """lengths -> device packed row -> its positions -> device boundaries,
    compared with oracle O9 on the same positions (bit-exact); streams span
    several 1024-token chunks of the scan."""
    rng = np.random.default_rng(21)
    cases = [[8192], [16384] + [int(x) for x in rng.integers(16, 1025, size=40)], [1] * 3000,
             [0, 5, 0, 0, 7], [1023, 1, 1024, 1025]]
    for _ in range(12):
        B = int(rng.integers(1, 60))
        cases.append([int(x) for x in rng.integers(0, 300, size=B)])
    for lengths in cases:
        if sum(lengths) == 0:
            continue
        say(f"boundaries: round trip B={len(lengths)} T={sum(lengths)}")
        row = _row(lengths)
        import packed_varlen_block_amd as pvb
        pvb.check_status(row["status"])
        pos = row["pos"].cpu().numpy()
        _check_bounds(pos, "zero")
        _check_bounds(pos + 3, "min")
        kept = [L for L in lengths if L > 0]
        out = _bounds(pos)
        n = out["n_seg"].item()
        assert out["cu"].cpu().tolist()[:n + 1] == P.cu_seqlens_from_lengths(kept)


def test_boundaries_edge_cases_and_errors():
    import packed_varlen_block_amd as pvb
    torch = _torch()
    say("boundaries: empty stream, all starts, errors")
    _check_bounds([], "zero")
    _check_bounds([], "min")
    _check_bounds([0] * 2500, "zero")
    _check_bounds([5] * 1500, "min")
    for pos, sentinel, cap, code in (([1, 0, 1], "zero", None, 4), ([0, 1, 0, 1], "zero", 2, 2),
                                     ([3, 2, 2], "min", None, 4)):
        p = torch.tensor(pos, dtype=torch.int32).cuda()
        cu = torch.full((max(cap or len(pos) + 1, 1),), 7, dtype=torch.int32, device="cuda")
        out = {"n_seg": torch.full((1,), 7, dtype=torch.int32, device="cuda")}
        st = torch.empty(1, dtype=torch.int32, device="cuda")
        rc = pvb.lib().pvb_boundaries_from_positions(
            p.data_ptr(), len(pos), 1 if sentinel == "min" else 0, cu.data_ptr(), cu.numel(),
            out["n_seg"].data_ptr(), None, st.data_ptr(), None)
        assert rc == 0
        torch.cuda.synchronize()
        assert st.item() == code
        assert (cu == 7).all() and out["n_seg"].item() == 7
