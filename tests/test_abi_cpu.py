"""C-ABI library on the CPU: symbols, host planners vs the oracle, host-side errors.

No GPU is touched: the device entry points are only called with arguments
that their host-side validation rejects before any HIP call.
"""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import packed_varlen_block_amd as pvb
from oracle import packing as P
from workloads import raw_lengths_cfg3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = os.path.join(ROOT, "tests", "golden")


def _header_symbols():
    text = open(os.path.join(ROOT, "include", "pvb.h")).read()
    return sorted(set(re.findall(r"\b(pvb_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = pvb.lib()
    syms = _header_symbols()
    assert len(syms) >= 8
    for s in syms:
        assert hasattr(L, s), s
    assert sorted(pvb.EXPORTS) == syms
    assert "gfx950" in pvb.version()


def test_status_strings():
    for code in range(9):
        assert pvb.status_string(code) and pvb.status_string(code) != "unknown status"
    assert pvb.status_string(99) == "unknown status"


def test_nextfit_fixture_matches_oracle():
    g = json.load(open(os.path.join(GOLD, "nextfit_capacity6.json")))
    row_of, start_of, n_rows = pvb.pack_plan_nextfit(g["prediction_lengths"], g["capacity"])
    o_row, o_start, o_n = P.next_fit(g["prediction_lengths"], g["capacity"])
    assert row_of.tolist() == o_row == [0, 0, 1]
    assert start_of.tolist() == o_start == [0, 3, 0]
    assert n_rows == o_n == 2


def test_planners_bit_exact_random():
    rng = np.random.default_rng(5)
    for _ in range(300):
        cap = int(rng.integers(1, 40))
        n = int(rng.integers(0, 60))
        lengths = rng.integers(0, cap + 1, size=n)
        a = pvb.pack_plan_nextfit(lengths, cap)
        b = P.next_fit(lengths.tolist(), cap)
        assert a[0].tolist() == b[0] and a[1].tolist() == b[1] and a[2] == b[2]
        a = pvb.pack_plan_bfd(lengths, cap)
        b = P.best_fit_decreasing(lengths.tolist(), cap)
        assert a[0].tolist() == b[0] and a[1].tolist() == b[1] and a[2] == b[2]
        assert a[3].tolist() == b[3] and a[4].tolist() == b[4]


def test_bfd_cfg3_20000_lengths_bit_exact():
    L = raw_lengths_cfg3(0)
    a = pvb.pack_plan_bfd(L, 8192)
    b = P.best_fit_decreasing(L.tolist(), 8192)
    assert a[2] == b[2]
    assert np.array_equal(a[0], np.asarray(b[0])) and np.array_equal(a[1], np.asarray(b[1]))
    assert np.array_equal(a[3], np.asarray(b[3])) and np.array_equal(a[4], np.asarray(b[4]))
    first = L[a[3][a[4][0]:a[4][1]]]
    assert first.tolist() == [8192]


def test_planners_large_n_and_capacity_one():
    L = np.ones(100000, np.int32)
    row_of, start_of, n_rows = pvb.pack_plan_nextfit(L, 1)
    assert n_rows == 100000 and row_of[-1] == 99999 and start_of.max() == 0
    bin_of, start_of, n_bins, order, offs = pvb.pack_plan_bfd(L, 7)
    assert n_bins == (100000 + 6) // 7 and offs[-1] == 100000
    assert pvb.pack_plan_nextfit([], 5)[2] == 0
    assert pvb.pack_plan_bfd([], 5)[2] == 0


def test_planner_errors():
    with pytest.raises(pvb.PvbError) as e:
        pvb.pack_plan_nextfit([3, 9], 8)
    assert e.value.status == 2
    with pytest.raises(pvb.PvbError) as e:
        pvb.pack_plan_bfd([3, -1], 8)
    assert e.value.status == 1
    with pytest.raises(pvb.PvbError) as e:
        pvb.pack_plan_bfd([1], 0)
    assert e.value.status == 1
    # null output pointer
    L = pvb.lib()
    a = np.array([1, 2], np.int32)
    n = ctypes.c_int64(0)
    assert L.pvb_pack_plan_nextfit(a.ctypes.data, 2, 4, None, None, ctypes.addressof(n)) == 1


def test_workspace_sizes():
    assert pvb.workspace_bytes(8192, 32, 128, 1, False) >= 256 + 64 * 8
    fwd = pvb.workspace_bytes(4096, 16, 128, 16, False)
    bwd32 = pvb.workspace_bytes(4096, 16, 128, 16, True, pvb.PVB_F32)
    bwd16 = pvb.workspace_bytes(4096, 16, 128, 16, True, pvb.PVB_BF16)
    # the backward keeps only the tile list and D = rowsum(dO * O) in fp32 [H, T]
    assert bwd32 >= 16 * 4096 * 4 and bwd16 == bwd32
    assert fwd > 0
    assert pvb.workspace_bytes(10, 2, 96, 1, False) == 0


FAKE = 0x1000   # a non-null address that host validation never dereferences


def _fwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, h_cu=None, n_seg=1, T=8, H=2, d=64, scale=0.125,
                o=FAKE, o_dtype=0, lse=FAKE, prec=0, ws=FAKE, ws_bytes=1 << 20, status=FAKE)
    args.update(kw)
    return pvb.lib().pvb_varlen_attn_fwd(*args.values(), None)


def _bwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, o_dtype=0, do=FAKE, lse=FAKE, cu=FAKE, h_cu=None,
                n_seg=1, T=8, H=2, d=64, scale=0.125, dq=FAKE, dk=FAKE, dv=FAKE, g=1, prec=0,
                ws=FAKE, ws_bytes=1 << 24, status=FAKE)
    args.update(kw)
    return pvb.lib().pvb_varlen_attn_bwd(*args.values(), None)


def test_device_entry_points_reject_bad_arguments_on_host():
    assert _fwd(d=96) == 6
    assert _fwd(H=0) == 1
    assert _fwd(q=None) == 1
    assert _fwd(status=None) == 1
    assert _fwd(o_dtype=5) == 1
    assert _fwd(prec=7) == 1
    assert _fwd(scale=0.0) == 1
    assert _fwd(scale=float("nan")) == 1
    assert _fwd(ws=None) == 5
    assert _fwd(ws_bytes=16) == 5
    bad = np.array([0, 9], np.int32)                  # cu[B] != T
    assert _fwd(h_cu=bad.ctypes.data) == 4
    dec = np.array([0, 6, 5, 8], np.int32)            # decreasing
    assert _fwd(h_cu=dec.ctypes.data, n_seg=3) == 4
    first = np.array([1, 8], np.int32)
    assert _fwd(h_cu=first.ctypes.data) == 4
    # the element limit: T·H·d = 2^31 is refused; one row less passes that check
    # (and stops at the too-small workspace, before any launch)
    assert _fwd(T=2 ** 24, H=1, d=128) == 6
    assert _fwd(T=2 ** 24 - 1, H=1, d=128, ws_bytes=16) == 5
    assert _bwd(T=2 ** 24, H=1, d=128) == 6
    assert _bwd(T=2 ** 24 - 1, H=1, d=128, ws_bytes=8) == 5
    assert _bwd(d=32) == 6
    assert _bwd(dv=None) == 1
    assert _bwd(g=3) == 1
    assert _bwd(ws_bytes=8) == 5
    assert _bwd(h_cu=bad.ctypes.data) == 4
    L = pvb.lib()
    assert L.pvb_build_packed_row(None, 2, 8, 0, FAKE, FAKE, FAKE, None, None, None, None, None, None,
                                  FAKE, None) == 1
    assert L.pvb_build_packed_row(FAKE, 2, 8, -1, FAKE, FAKE, FAKE, None, None, None, None, None, None,
                                  FAKE, None) == 1
    assert L.pvb_build_packed_row(FAKE, 2, 8, 2**31 - 1, FAKE, FAKE, FAKE, None, None, None, None,
                                  None, None, FAKE, None) == 3
    # token outputs without a token source
    assert L.pvb_build_packed_row(FAKE, 2, 8, 0, FAKE, FAKE, FAKE, None, None, None, FAKE, None, None,
                                  FAKE, None) == 1


def test_boundaries_host_side_errors():
    L = pvb.lib()
    FAKE = 1 << 40
    Z, M = pvb.PVB_SENTINEL_ZERO, pvb.PVB_SENTINEL_MIN
    assert L.pvb_boundaries_from_positions(None, 4, Z, FAKE, 5, FAKE, None, FAKE, None) == 1   # null positions
    assert L.pvb_boundaries_from_positions(FAKE, -1, Z, FAKE, 5, FAKE, None, FAKE, None) == 1  # negative T
    assert L.pvb_boundaries_from_positions(FAKE, 4, 2, FAKE, 5, FAKE, None, FAKE, None) == 1   # bad sentinel
    assert L.pvb_boundaries_from_positions(FAKE, 4, M, FAKE, 0, FAKE, None, FAKE, None) == 1   # no room for cu
    assert L.pvb_boundaries_from_positions(FAKE, 4, M, None, 5, FAKE, None, FAKE, None) == 1   # null cu
    assert L.pvb_boundaries_from_positions(FAKE, 4, M, FAKE, 5, None, None, FAKE, None) == 1   # null n_seg
    assert L.pvb_boundaries_from_positions(FAKE, 4, M, FAKE, 5, FAKE, None, None, None) == 1   # null status
    assert L.pvb_boundaries_from_positions(FAKE, 2**31 - 1, Z, FAKE, 5, FAKE, None, FAKE, None) == 3


def test_packed_nll_host_side_errors():
    L = pvb.lib()
    FAKE = 1 << 40
    B, F32 = pvb.PVB_BF16, pvb.PVB_F32
    ok = dict(l=FAKE, ld=B, C=4, V=10, t=FAKE, m=None, r=FAKE, loss=FAKE, n=FAKE, g=None, gd=F32, st=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return L.pvb_packed_nll(a["l"], a["ld"], a["C"], a["V"], a["t"], a["m"], a["r"], a["loss"], a["n"],
                                a["g"], a["gd"], a["st"], None)
    assert call(C=-1) == 1
    assert call(V=0) == 1
    assert call(l=None) == 1
    assert call(t=None) == 1
    assert call(r=None) == 1
    assert call(loss=None) == 1
    assert call(n=None) == 1
    assert call(st=None) == 1
    assert call(ld=2) == 1
    assert call(g=FAKE, gd=3) == 1
    assert call(C=2**31) == 6


def _xfwd(**kw):
    cq = np.array([0, 8], np.int32)
    ck = np.array([0, 12], np.int32)
    args = dict(q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, h_cu_q=cq.ctypes.data, cu_k=FAKE, h_cu_k=ck.ctypes.data,
                n_seg=1, T_q=8, T_k=12, H=4, H_kv=2, d=64, wl=-1, wr=0, scale=0.125, o=FAKE, o_dtype=0,
                lse=FAKE, prec=0, ws=FAKE, ws_bytes=16, status=FAKE)
    args.update(kw)
    return pvb.lib().pvb_varlen_cross_attn_fwd(*args.values(), None)


def _xbwd(**kw):
    cq = np.array([0, 8], np.int32)
    ck = np.array([0, 12], np.int32)
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, o_dtype=0, do=FAKE, lse=FAKE, cu_q=FAKE,
                h_cu_q=cq.ctypes.data, cu_k=FAKE, h_cu_k=ck.ctypes.data, n_seg=1, T_q=8, T_k=12, H=4, H_kv=2,
                d=64, wl=-1, wr=0, scale=0.125, dq=FAKE, dk=FAKE, dv=FAKE, g=1, prec=0, ws=FAKE, ws_bytes=16,
                status=FAKE)
    args.update(kw)
    return pvb.lib().pvb_varlen_cross_attn_bwd(*args.values(), None)


def test_cross_entry_points_reject_bad_arguments_on_host():
    """Every case fails host validation; the valid ones stop at the (too small) workspace."""
    assert _xfwd() == 5 and _xbwd() == 5
    for call in (_xfwd, _xbwd):
        assert call(h_cu_q=None) == 1                 # the host mirrors are required
        assert call(h_cu_k=None) == 1
        assert call(cu_k=None) == 1
        assert call(wl=-2) == 1
        assert call(wr=-5) == 1
        assert call(T_k=-1) == 1
        assert call(H_kv=3) == 1                      # 4 query heads over 3 key/value heads
        assert call(d=96) == 6
        assert call(k=None) == 1
        assert call(T_k=13) == 4                      # h_cu_k[B] != T_k
        assert call(T_q=9) == 4                       # h_cu_q[B] != T_q
        dec = np.array([0, 9, 8, 12], np.int32)
        ok3 = np.array([0, 2, 4, 8], np.int32)
        assert call(n_seg=3, h_cu_k=dec.ctypes.data, h_cu_q=ok3.ctypes.data) == 4
        assert call(scale=0.0) == 1
    assert _xbwd(g=5) == 1
    assert _xbwd(dk=None) == 1
    # no keys at all: k, v (and dK, dV) may be null
    assert _xfwd(k=None, v=None, T_k=0, h_cu_k=np.array([0, 0], np.int32).ctypes.data) == 5


def test_cross_workspace_sizes():
    W = pvb.cross_workspace_bytes
    # the forward needs only the query tile list: the self-attention size for T_q
    assert W(4096, 9000, 16, 128, 16, False) == pvb.workspace_bytes(4096, 16, 128, 16, False)
    # the backward adds the key tile list to the self-attention size for T_q
    assert W(4096, 4096, 16, 128, 16, True) > pvb.workspace_bytes(4096, 16, 128, 16, True)
    assert W(4096, 64000, 16, 128, 16, True) >= 16 * 4096 * 8 + 64000 // 128 * 8
    assert W(10, 10, 2, 96, 1, False) == 0 and W(10, -1, 2, 64, 1, True) == 0


def test_gated_delta_host_side_errors():
    L = pvb.lib()
    ok = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, cu=FAKE, h_cu=None, n_seg=1, T=8, H=2, d=128,
              scale=0.125, h0=None, o=FAKE, o_dtype=0, ht=None, ws=None, ws_bytes=0, status=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return L.pvb_gated_delta_fwd(*a.values(), None)
    assert call(d=64) == 6                            # only d = 128 is built
    assert call(H=0) == 1
    assert call(T=-1) == 1
    assert call(n_seg=-1) == 1
    assert call(cu=None) == 1
    assert call(status=None) == 1
    for name in ("q", "k", "v", "g", "b", "o"):
        assert call(**{name: None}) == 1, name
    assert call(o_dtype=3) == 1
    assert call(scale=0.0) == 1
    assert call(scale=float("inf")) == 1
    assert call(T=2**24, H=2**7) == 6                 # T H d reaches 2^31
    bad = np.array([0, 9], np.int32)                  # h_cu[B] != T
    assert call(h_cu=bad.ctypes.data) == 4
    dec = np.array([0, 6, 5, 8], np.int32)
    assert call(h_cu=dec.ctypes.data, n_seg=3) == 4
    # the grouped evaluation's workspace: too small, or missing with a size
    need = L.pvb_gated_delta_fwd_workspace_bytes(8, 2, 1)
    assert call(ws=FAKE, ws_bytes=need - 1) == 5
    assert call(ws=None, ws_bytes=need) == 5


def test_gated_delta_forward_workspace_size():
    """T's six split fragments for every 64-token chunk slot (12 KB per head)
    and, per 1024-token group slot and head, the group map A_g, the state Z_g
    and the starting state (64 KB each); slots: T/64 + B + 1 and
    T/1024 + B + 1."""
    W = pvb.gated_delta_fwd_workspace_bytes
    up = lambda x: (x + 255) // 256 * 256
    for T, H, B in ((8, 2, 1), (32768, 32, 32), (4096, 3, 600)):
        slots, gslots = T // 64 + B + 1, T // 1024 + B + 1
        assert W(T, H, B) == up(slots * H * 12288) + 3 * up(gslots * H * 128 * 128 * 4)
    assert W(-1, 2, 1) == 0 and W(8, 0, 1) == 0


def test_gated_delta_training_forward_host_side_errors():
    """The training forward checks the forward's arguments and needs the
    backward's workspace (PVB_E_WORKSPACE, 5, below it, or without one)."""
    L = pvb.lib()
    need = L.pvb_gated_delta_bwd_workspace_bytes(8, 2, 1)
    ok = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, cu=FAKE, h_cu=None, n_seg=1, T=8, H=2, H_k=2, d=128,
              scale=0.125, h0=None, o=FAKE, o_dtype=0, ht=None, ws=FAKE, ws_bytes=need, status=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return L.pvb_gated_delta_fwd_train(*a.values(), None)
    assert call(ws=None, ws_bytes=0) == 5
    assert call(ws_bytes=need - 1) == 5
    assert call(ws_bytes=L.pvb_gated_delta_fwd_workspace_bytes(8, 2, 1)) == 5
    assert call(d=64) == 6
    assert call(H=0) == 1
    assert call(H_k=3) == 1
    assert call(o_dtype=3) == 1
    assert call(scale=0.0) == 1
    for name in ("q", "k", "v", "g", "b", "o", "cu", "status"):
        assert call(**{name: None}) == 1, name
    assert call(n_seg=pvb.PVB_MAX_COUNT + 1) == 3
    assert call(T=2 ** 24, H=2 ** 7, H_k=2 ** 7, ws_bytes=1 << 40) == 6
    bad = np.array([0, 9], np.int32)
    assert call(h_cu=bad.ctypes.data) == 4


def test_gated_delta_grouped_heads_host_side_errors():
    L = pvb.lib()
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, cu=FAKE, h_cu=None, n_seg=1, T=8, H=6, H_k=4, d=128,
                scale=0.125, h0=None, o=FAKE, o_dtype=0, ht=None, ws=None, ws_bytes=0, status=FAKE)
    assert L.pvb_gated_delta_fwd_gqa(*args.values(), None) == 1          # 6 value heads over 4
    args.update(H_k=0)
    assert L.pvb_gated_delta_fwd_gqa(*args.values(), None) == 1
    args.update(H_k=3, d=64)
    assert L.pvb_gated_delta_fwd_gqa(*args.values(), None) == 6


def test_counts_above_the_documented_maximum_are_refused_on_host():
    """PVB_MAX_COUNT (2^31 - 65536) bounds every count a device entry point
    takes, so that no kernel's stride loop can step past INT32_MAX; one more
    returns PVB_E_OVERFLOW (3) before anything is enqueued."""
    big = pvb.PVB_MAX_COUNT + 1
    L = pvb.lib()
    assert _fwd(n_seg=big) == 3
    assert _bwd(n_seg=big) == 3
    assert L.pvb_build_packed_row(FAKE, big, 8, 0, FAKE, FAKE, FAKE, None, None, None, None, None, None,
                                  FAKE, None) == 3
    assert L.pvb_build_packed_row(FAKE, 2, big, 0, FAKE, FAKE, FAKE, None, None, None, None, None, None,
                                  FAKE, None) == 3
    assert L.pvb_boundaries_from_positions(FAKE, big, 0, FAKE, 8, FAKE, None, FAKE, None) == 3
    assert L.pvb_packed_nll(FAKE, 0, 4, big, FAKE, None, FAKE, FAKE, FAKE, None, 0, FAKE, None) == 3
    assert L.pvb_gated_delta_fwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, big, 8, 1, 1, 128, 0.1, None,
                                     FAKE, 1, None, None, 0, FAKE, None) == 3


def test_grids_of_2_to_the_32_work_items_are_refused_on_host():
    """A dispatch carries its grid size in work-items as a 32-bit count; a call
    whose launch would need 2^32 or more is refused with PVB_E_UNSUPPORTED (6)
    before anything is enqueued, and one workgroup fewer passes that check
    (stopping at the too-small workspace, 5)."""
    L = pvb.lib()
    # 2^16 tokens in 2^16 one-token segments: 2^16 tiles per head
    assert _fwd(T=2 ** 16, n_seg=2 ** 16, H=256, d=64) == 6
    assert _fwd(T=2 ** 16, n_seg=2 ** 16, H=255, d=64, ws_bytes=16) == 5
    # the dK/dV launch has two workgroups per tile and key/value head
    assert _bwd(T=2 ** 16, n_seg=2 ** 16, H=128, d=64) == 6
    assert _bwd(T=2 ** 16, n_seg=2 ** 16, H=127, d=64, ws_bytes=8) == 5
    # zero-length segments add no tiles: 2^16 empty segments and T = 128
    assert _fwd(T=128, n_seg=2 ** 16, H=256, d=64, ws_bytes=16) == 5
    assert L.pvb_packed_nll(FAKE, 0, 2 ** 24, 8, FAKE, None, FAKE, FAKE, FAKE, None, 0, FAKE, None) == 6
    assert L.pvb_gated_delta_fwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 2 ** 16, 8, 256, 256, 128, 0.1,
                                     None, FAKE, 1, None, None, 0, FAKE, None) == 6


def test_gated_delta_grid_limits_on_host():
    """The gated delta group walks launch four workgroups of 256 per slice and
    head (the backward's two walks together eight), so a forward with
    B * H >= 2^22 or a backward with B * H >= 2^21 returns PVB_E_UNSUPPORTED
    (6); one head fewer passes the grid checks and stops at the too-small
    workspace (5)."""
    L = pvb.lib()

    def fwd(n_seg, H):
        return L.pvb_gated_delta_fwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, n_seg, 8, H, H, 128, 0.1,
                                         None, FAKE, 1, None, FAKE, 16, FAKE, None)

    def bwd(n_seg, H):
        return L.pvb_gated_delta_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, n_seg, 8, H, H, 128, 0.1, None,
                                     FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, FAKE, 16, FAKE, None)
    assert fwd(2 ** 16, 64) == 6 and fwd(2 ** 16, 63) == 5
    assert bwd(2 ** 16, 32) == 6 and bwd(2 ** 16, 31) == 5
    assert L.pvb_gated_delta_fwd_train(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 2 ** 16, 8, 64, 64, 128, 0.1,
                                       None, FAKE, 1, None, FAKE, 16, FAKE, None) == 6


def test_noalloc_backward_refuses_sizes_beyond_its_scratch_on_host():
    """pvb_varlen_attn_bwd_noalloc serves sizes whose workspace fits its fixed
    scratch (PVB_STATIC_SCRATCH_BYTES); larger ones return PVB_E_WORKSPACE (5)
    before any HIP call, bad sizes PVB_E_INVALID_ARG (1) or PVB_E_OVERFLOW (3)."""
    L = pvb.lib()
    cap = pvb.PVB_STATIC_SCRATCH_BYTES

    def call(T, H, n_seg=1):
        return L.pvb_varlen_attn_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, n_seg, T, H, H,
                                             128, 0.088, FAKE, FAKE, FAKE, 1, 0, FAKE, None)
    assert pvb.workspace_bytes(262144, 33, 128, 1, True) > cap
    assert call(262144, 33) == 5
    assert pvb.workspace_bytes(2 ** 20, 32, 128, 1, True) > cap
    assert call(2 ** 20, 32) == 5
    assert call(-1, 4) == 1
    assert call(8, 0) == 1
    assert call(8, 4, n_seg=-1) == 1
    assert call(8, 4, n_seg=pvb.PVB_MAX_COUNT + 1) == 3
    assert call(262144, 32) == 5                                       # the documented examples
    assert pvb.workspace_bytes(131072, 32, 128, 1, True) <= cap


@pytest.mark.parametrize("entry", ["pvb_gated_delta_bwd", "pvb_gated_delta_bwd_after_fwd"])
def test_gated_delta_backward_host_side_errors(entry):
    L = pvb.lib()
    ok = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, cu=FAKE, h_cu=None, n_seg=1, T=8, H=2, H_k=2, d=128,
              scale=0.125, h0=None, do=FAKE, dht=None, dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, db=FAKE, dh0=None,
              gd=1, ws=FAKE, ws_bytes=16, status=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return getattr(L, entry)(*a.values(), None)
    assert call() == 5                                # the workspace is too small
    assert call(d=64) == 6
    assert call(H=0) == 1
    assert call(H_k=3) == 1
    assert call(gd=4) == 1
    assert call(scale=0.0) == 1
    for name in ("q", "k", "v", "g", "b", "do", "dq", "dk", "dv", "dg", "db", "cu", "status"):
        assert call(**{name: None}) == 1, name
    assert call(n_seg=pvb.PVB_MAX_COUNT + 1) == 3
    assert call(T=2 ** 24, H=2 ** 7, H_k=2 ** 7) == 6
    bad = np.array([0, 9], np.int32)
    assert call(h_cu=bad.ctypes.data, ws_bytes=1 << 40) == 4
    assert pvb.gated_delta_bwd_workspace_bytes(8, 2, 1) > 0 and pvb.gated_delta_bwd_workspace_bytes(-1, 2, 1) == 0
