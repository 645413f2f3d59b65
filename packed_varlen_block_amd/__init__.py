"""Python binding of libpvb (packed block-causal varlen attention, gfx950).

Argument marshalling only: every step runs in the C-ABI library's host code or
HIP kernels.  torch supplies device memory (outputs, workspace) and the
current HIP stream.  There is no fallback: if libpvb.so is missing or a call
fails, an exception is raised.

Functions (same names as the C entry points without the ``pvb_`` prefix):
  pack_plan_nextfit, pack_plan_bfd       host planners (numpy in / numpy out)
  build_packed_row                       device prefix scan -> cu, pos, seg, ...
  varlen_attn_fwd, varlen_attn_bwd       bf16 MFMA attention kernels
  workspace_bytes, status_string, check_status
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PVB_LIB_PATH selects another build of the same library (the CPU sanitizer
# build, libpvb_san.so); there is no other implementation to fall back to.
LIB_PATH = os.environ.get("PVB_LIB_PATH") or os.path.join(_HERE, "libpvb.so")

PVB_OK = 0
PVB_MAX_COUNT = 2 ** 31 - 65536   # largest T, capacity, B, n_seg or V a device entry point accepts
PVB_BF16, PVB_F32 = 0, 1
PVB_PREC_BF16, PVB_PREC_SPLIT = 0, 1
PVB_SENTINEL_ZERO, PVB_SENTINEL_MIN = 0, 1
STATUS_NAMES = {0: "PVB_OK", 1: "PVB_E_INVALID_ARG", 2: "PVB_E_OVERSIZED", 3: "PVB_E_OVERFLOW",
                4: "PVB_E_BAD_CU_SEQLENS", 5: "PVB_E_WORKSPACE", 6: "PVB_E_UNSUPPORTED", 7: "PVB_E_HIP",
                8: "PVB_E_NO_TARGETS"}

# every symbol include/pvb.h declares
EXPORTS = ("pvb_pack_plan_nextfit", "pvb_pack_plan_bfd", "pvb_build_packed_row", "pvb_boundaries_from_positions",
           "pvb_packed_nll", "pvb_varlen_attn_fwd_gqa", "pvb_varlen_attn_bwd_gqa",
           "pvb_varlen_cross_attn_workspace_bytes", "pvb_varlen_cross_attn_fwd", "pvb_varlen_cross_attn_bwd",
           "pvb_gated_delta_fwd", "pvb_gated_delta_fwd_gqa", "pvb_gated_delta_fwd_workspace_bytes",
           "pvb_gated_delta_bwd", "pvb_gated_delta_bwd_workspace_bytes", "pvb_gated_delta_fwd_train",
           "pvb_gated_delta_bwd_after_fwd",
           "pvb_varlen_attn_workspace_bytes", "pvb_varlen_attn_fwd", "pvb_varlen_attn_bwd",
           "pvb_varlen_attn_bwd_noalloc", "pvb_status_string", "pvb_version")
PVB_STATIC_SCRATCH_BYTES = 64 << 20   # the fixed scratch array of pvb_varlen_attn_bwd_noalloc


class PvbError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: {STATUS_NAMES.get(self.status, self.status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libpvb.so (built in-tree by packed_varlen_block_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m packed_varlen_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        L.pvb_pack_plan_nextfit.argtypes = [P, I64, I32, P, P, P]
        L.pvb_pack_plan_bfd.argtypes = [P, I64, I32, P, P, P, P, P]
        L.pvb_build_packed_row.argtypes = [P, I32, I32, I32, P, P, P, P, P, P, P, P, P, P, P]
        L.pvb_boundaries_from_positions.argtypes = [P, I32, I32, P, I32, P, P, P, P]
        L.pvb_packed_nll.argtypes = [P, I32, I64, I32, P, P, P, P, P, P, I32, P, P]
        L.pvb_varlen_attn_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
        L.pvb_varlen_attn_workspace_bytes.restype = SZ
        L.pvb_varlen_attn_fwd.argtypes = [P, P, P, P, P, I32, I32, I32, I32, F, P, I32, P, I32, P, SZ, P, P]
        L.pvb_varlen_attn_bwd.argtypes = [P, P, P, P, I32, P, P, P, P, I32, I32, I32, I32, F,
                                          P, P, P, I32, I32, P, SZ, P, P]
        L.pvb_varlen_attn_fwd_gqa.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, F, P, I32, P, I32, P, SZ,
                                              P, P]
        L.pvb_varlen_attn_bwd_gqa.argtypes = [P, P, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, F,
                                              P, P, P, I32, I32, P, SZ, P, P]
        L.pvb_varlen_attn_bwd_noalloc.argtypes = [P, P, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, F,
                                                  P, P, P, I32, I32, P, P]
        L.pvb_gated_delta_bwd.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, F, P, P, P, P, P, P, P,
                                          P, P, I32, P, SZ, P, P]
        L.pvb_gated_delta_bwd_after_fwd.argtypes = L.pvb_gated_delta_bwd.argtypes
        L.pvb_gated_delta_bwd_workspace_bytes.argtypes = [I32, I32, I32]
        L.pvb_gated_delta_bwd_workspace_bytes.restype = SZ
        L.pvb_gated_delta_fwd.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, F, P, P, I32, P, P, SZ, P, P]
        L.pvb_gated_delta_fwd_gqa.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, F, P, P, I32, P, P, SZ,
                                              P, P]
        L.pvb_gated_delta_fwd_train.argtypes = L.pvb_gated_delta_fwd_gqa.argtypes
        L.pvb_gated_delta_fwd_workspace_bytes.argtypes = [I32, I32, I32]
        L.pvb_gated_delta_fwd_workspace_bytes.restype = SZ
        L.pvb_varlen_cross_attn_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32]
        L.pvb_varlen_cross_attn_workspace_bytes.restype = SZ
        L.pvb_varlen_cross_attn_fwd.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, F,
                                                P, I32, P, I32, P, SZ, P, P]
        L.pvb_varlen_cross_attn_bwd.argtypes = [P, P, P, P, I32, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                                I32, I32, F, P, P, P, I32, I32, P, SZ, P, P]
        for name in ("pvb_pack_plan_nextfit", "pvb_pack_plan_bfd", "pvb_build_packed_row",
                     "pvb_boundaries_from_positions", "pvb_packed_nll", "pvb_varlen_attn_fwd",
                     "pvb_varlen_attn_bwd", "pvb_varlen_attn_fwd_gqa", "pvb_varlen_attn_bwd_gqa",
                     "pvb_varlen_attn_bwd_noalloc",
                     "pvb_varlen_cross_attn_fwd", "pvb_varlen_cross_attn_bwd", "pvb_gated_delta_fwd",
                     "pvb_gated_delta_bwd", "pvb_gated_delta_bwd_after_fwd", "pvb_gated_delta_fwd_train",
                     "pvb_gated_delta_fwd_gqa"):
            getattr(L, name).restype = ctypes.c_int
        L.pvb_status_string.argtypes = [I32]
        L.pvb_status_string.restype = ctypes.c_char_p
        L.pvb_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pvb_status_string(int(status)).decode()


def version() -> str:
    return lib().pvb_version().decode()


def _check(rc: int, where: str):
    if rc != PVB_OK:
        raise PvbError(rc, where)


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()


# ---------------------------------------------------------------- host planners

def _lengths_array(lengths) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(lengths, dtype=np.int64))
    if a.size and (a.min() < -2**31 or a.max() > 2**31 - 1):
        raise PvbError(3, "lengths")
    return np.ascontiguousarray(a.astype(np.int32))


def pack_plan_nextfit(lengths, capacity: int):
    """Order-preserving next-fit.  Returns (row_of, start_of, n_rows)."""
    a = _lengths_array(lengths)
    n = a.size
    row_of = np.zeros(max(n, 1), np.int32)
    start_of = np.zeros(max(n, 1), np.int32)
    n_rows = ctypes.c_int64(0)
    _check(lib().pvb_pack_plan_nextfit(_ptr(a), n, int(capacity), _ptr(row_of), _ptr(start_of),
                                       ctypes.addressof(n_rows)), "pack_plan_nextfit")
    return row_of[:n], start_of[:n], int(n_rows.value)


def pack_plan_bfd(lengths, capacity: int):
    """Best-fit-decreasing.  Returns (bin_of, start_of, n_bins, order, bin_offsets)."""
    a = _lengths_array(lengths)
    n = a.size
    bin_of = np.zeros(max(n, 1), np.int32)
    start_of = np.zeros(max(n, 1), np.int32)
    order = np.zeros(max(n, 1), np.int32)
    offs = np.zeros(n + 1, np.int64)
    n_bins = ctypes.c_int64(0)
    _check(lib().pvb_pack_plan_bfd(_ptr(a), n, int(capacity), _ptr(bin_of), _ptr(start_of),
                                   ctypes.addressof(n_bins), _ptr(order), _ptr(offs)), "pack_plan_bfd")
    nb = int(n_bins.value)
    return bin_of[:n], start_of[:n], nb, order[:n], offs[:nb + 1]


# ---------------------------------------------------------------- device calls

def _torch():
    import torch
    return torch


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype=None, shape=None, dev=None, dim=None):
    """Check one device argument before anything is enqueued: a torch tensor of
    the given dtype and shape, contiguous, on a CUDA device (the same one as
    the call's other tensors when ``dev`` is given).  A host tensor, or a
    mismatched dtype or shape, would hand the kernels a wrong address or
    reinterpret its bytes; it raises PvbError(PVB_E_INVALID_ARG) instead."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise PvbError(1, f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise PvbError(1, f"{name} must be {dtype}, not {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise PvbError(1, f"{name} must be {dim}-d, not of shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise PvbError(1, f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if not t.is_contiguous():
        raise PvbError(1, f"{name} must be contiguous")
    if not t.is_cuda:
        raise PvbError(1, f"{name} must be a CUDA tensor")
    if dev is not None and t.device != dev:
        raise PvbError(1, f"{name} is on {t.device}, the call's other tensors on {dev}")
    return t


def _status_arg(status, dev):
    torch = _torch()
    if status is None:
        return torch.empty(1, dtype=torch.int32, device=dev)
    return _need(status, "status", torch.int32, (1,), dev)


def _workspace_arg(workspace, nbytes, dev):
    torch = _torch()
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    return _need(workspace, "workspace", dev=dev)


def check_status(status) -> None:
    """Synchronise on a device status word and raise if it holds an error."""
    st = int(status.item())
    if st != PVB_OK:
        raise PvbError(st, "device status")


def build_packed_row(lengths, capacity: int | None = None, segment_base: int = 0,
                     tokens=None, tok_off=None, status=None):
    """Device packed-row metadata.  ``lengths`` is an int32 CUDA tensor [B].

    Returns a dict of CUDA tensors: cu [B+1], pos [C], seg [C], max_seqlen [1],
    status [1]; with ``tokens``/``tok_off`` also inputs, targets [C] and valid [C].
    Enqueued on the current stream; call check_status(out["status"]) to
    synchronise and raise on a device-detected error.
    """
    torch = _torch()
    _need(lengths, "build_packed_row: lengths", torch.int32, dim=1)
    dev = lengths.device
    B = lengths.numel()
    gather = tokens is not None
    if gather or tok_off is not None:
        if tokens is None or tok_off is None:
            raise PvbError(1, "build_packed_row: tokens and tok_off go together")
        _need(tokens, "build_packed_row: tokens", torch.int32, dim=1, dev=dev)
        _need(tok_off, "build_packed_row: tok_off", torch.int64, (B,), dev)
    if capacity is None:
        capacity = int(lengths.sum().item())
    C = int(capacity)
    out = {"cu": torch.empty(B + 1, dtype=torch.int32, device=dev),
           "pos": torch.empty(max(C, 1), dtype=torch.int32, device=dev)[:C],
           "seg": torch.empty(max(C, 1), dtype=torch.int32, device=dev)[:C],
           "max_seqlen": torch.zeros(1, dtype=torch.int32, device=dev),
           "status": _status_arg(status, dev)}
    if gather:
        out["inputs"] = torch.empty(max(C, 1), dtype=torch.int32, device=dev)[:C]
        out["targets"] = torch.empty(max(C, 1), dtype=torch.int32, device=dev)[:C]
        out["valid"] = torch.empty(max(C, 1), dtype=torch.uint8, device=dev)[:C]
    rc = lib().pvb_build_packed_row(
        _ptr(lengths), B, C, int(segment_base), _ptr(out["cu"]), _ptr(out["pos"]), _ptr(out["seg"]),
        _ptr(out["max_seqlen"]), _ptr(tokens) if gather else None, _ptr(tok_off) if gather else None,
        _ptr(out["inputs"]) if gather else None, _ptr(out["targets"]) if gather else None,
        _ptr(out["valid"]) if gather else None, _ptr(out["status"]), _stream(dev))
    _check(rc, "build_packed_row")
    return out


def _reuse(out, name, shape, dtype, dev):
    """An output tensor taken from a caller's dict (no allocation), checked."""
    return _need(out[name], f"out[{name!r}]", dtype, shape, dev)


def boundaries_from_positions(pos, sentinel: str = "zero", capacity: int | None = None, status=None,
                              out=None):
    """cu_seqlens compiled back from a flat int32 CUDA position stream [T].

    ``sentinel`` "zero" (a segment starts where the position is 0) or "min"
    (where it equals the smallest position).  Returns a dict of CUDA tensors:
    cu [capacity] (entries 0..n_seg valid), n_seg [1], max_seqlen [1],
    status [1].  ``capacity`` defaults to T + 1.  ``out``: a dict returned by an
    earlier call, whose tensors are written again (nothing is allocated; its
    values are those of the last call until the kernel writes them).  Enqueued
    on the current stream; call check_status(out["status"]) to synchronise and
    raise.
    """
    torch = _torch()
    _need(pos, "boundaries_from_positions: pos", torch.int32, dim=1)
    dev = pos.device
    if sentinel not in ("zero", "min"):
        raise PvbError(1, "boundaries_from_positions: sentinel must be 'zero' or 'min'")
    T = pos.numel()
    cap = T + 1 if capacity is None else int(capacity)
    if out is not None:
        out = {"cu": _reuse(out, "cu", (max(cap, 1),), torch.int32, dev),
               "n_seg": _reuse(out, "n_seg", (1,), torch.int32, dev),
               "max_seqlen": _reuse(out, "max_seqlen", (1,), torch.int32, dev),
               "status": _status_arg(status, dev) if status is not None
               else _reuse(out, "status", (1,), torch.int32, dev)}
    else:
        out = {"cu": torch.empty(max(cap, 1), dtype=torch.int32, device=dev),
               "n_seg": torch.zeros(1, dtype=torch.int32, device=dev),
               "max_seqlen": torch.zeros(1, dtype=torch.int32, device=dev),
               "status": _status_arg(status, dev)}
    rc = lib().pvb_boundaries_from_positions(
        _ptr(pos) if T > 0 else None, T, PVB_SENTINEL_MIN if sentinel == "min" else PVB_SENTINEL_ZERO,
        _ptr(out["cu"]), cap, _ptr(out["n_seg"]), _ptr(out["max_seqlen"]), _ptr(out["status"]),
        _stream(dev))
    _check(rc, "boundaries_from_positions")
    return out


def packed_nll(logits, targets, mask=None, grad=True, grad_dtype=None, status=None, out=None):
    """Token-weighted NLL over packed cells.  ``logits`` is a CUDA [C, V]
    bf16/fp32 tensor, ``targets`` int32 [C] (cells with a negative target are
    excluded), ``mask`` optional uint8 [C] loss eligibility.  Returns a dict of
    CUDA tensors: row_nll [C], loss [2] (float64 sum, mean), count [1],
    status [1], and grad [C, V] (logits' dtype unless ``grad_dtype``) when
    ``grad``.  ``out``: a dict returned by an earlier call of the same shapes,
    whose tensors are written again (nothing is allocated).  Enqueued on the
    current stream; call check_status(out["status"]) to synchronise and raise
    on a device-detected error."""
    torch = _torch()
    _need(logits, "packed_nll: logits", dim=2)
    _dtype_code(logits.dtype)
    dev = logits.device
    C, V = logits.shape
    _need(targets, "packed_nll: targets", torch.int32, (C,), dev)
    if mask is not None:
        _need(mask, "packed_nll: mask", torch.uint8, (C,), dev)
    gdt = logits.dtype if grad_dtype is None else grad_dtype
    _dtype_code(gdt)
    if out is not None:
        prev = out
        out = {"row_nll": _reuse(prev, "row_nll", (C,), torch.float32, dev),
               "loss": _reuse(prev, "loss", (2,), torch.float64, dev),
               "count": _reuse(prev, "count", (1,), torch.int32, dev),
               "status": _status_arg(status, dev) if status is not None
               else _reuse(prev, "status", (1,), torch.int32, dev)}
        if grad:
            out["grad"] = _reuse(prev, "grad", (C, V), gdt, dev)
    else:
        out = {"row_nll": torch.empty(max(C, 1), dtype=torch.float32, device=dev)[:C],
               "loss": torch.zeros(2, dtype=torch.float64, device=dev),
               "count": torch.zeros(1, dtype=torch.int32, device=dev),
               "status": _status_arg(status, dev)}
        if grad:
            out["grad"] = torch.empty((C, V), dtype=gdt, device=dev)
    rc = lib().pvb_packed_nll(
        _ptr(logits) if C > 0 else None, _dtype_code(logits.dtype), C, V, _ptr(targets) if C > 0 else None,
        _ptr(mask) if mask is not None else None, _ptr(out["row_nll"]) if C > 0 else None, _ptr(out["loss"]),
        _ptr(out["count"]), _ptr(out["grad"]) if grad and C > 0 else None, _dtype_code(gdt),
        _ptr(out["status"]), _stream(dev))
    _check(rc, "packed_nll")
    return out


def workspace_bytes(T: int, H: int, d: int, n_seg: int, backward: bool, grad_dtype=PVB_F32) -> int:
    return int(lib().pvb_varlen_attn_workspace_bytes(T, H, d, n_seg, int(bool(backward)), int(grad_dtype)))


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.bfloat16:
        return PVB_BF16
    if dt == torch.float32:
        return PVB_F32
    raise PvbError(1, f"unsupported dtype {dt}")


def _prec_code(p):
    return {"bf16": PVB_PREC_BF16, "split": PVB_PREC_SPLIT, PVB_PREC_BF16: PVB_PREC_BF16,
            PVB_PREC_SPLIT: PVB_PREC_SPLIT}[p]


def _check_qkv(q, k, v, *rest):
    """q (and dO) [T, H, d]; k, v [T, H_kv, d] with H a multiple of H_kv."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, dim=3)
    _need(k, "k", torch.bfloat16, dim=3)
    T, H, d = q.shape
    Hk = k.shape[1]
    dev = q.device
    _need(k, "k", shape=(T, Hk, d), dev=dev)
    _need(v, "v", torch.bfloat16, (T, Hk, d), dev)
    for t in rest:
        _need(t, "dO", torch.bfloat16, (T, H, d), dev)
    if Hk <= 0 or H % Hk != 0:
        raise PvbError(1, "the query heads must be a multiple of the key/value heads")
    return T, H, Hk, d


def _cu_arg(cu, name, dev):
    torch = _torch()
    _need(cu, name, torch.int32, dim=1, dev=dev)
    if cu.numel() < 1:
        raise PvbError(1, f"{name} needs at least one entry")
    return cu.numel() - 1


def varlen_attn_fwd(q, k, v, cu, h_cu=None, softmax_scale=None, o_dtype=None, precision="bf16",
                    out=None, lse=None, workspace=None, status=None):
    """Forward packed block-causal attention.  Returns (O [T,H,d], LSE [H,T] fp32, status).

    q: contiguous bf16 CUDA [T, H, d]; k, v: [T, H_kv, d] (grouped heads when
    H_kv < H: query head h reads key/value head h // (H / H_kv)); cu: int32
    CUDA [B+1]; h_cu: optional host (numpy/list) mirror of cu, validated on the host.
    """
    torch = _torch()
    T, H, Hk, d = _check_qkv(q, k, v)
    dev = q.device
    n_seg = _cu_arg(cu, "cu", dev)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if o_dtype is None:
        o_dtype = out.dtype if out is not None else torch.bfloat16
    _dtype_code(o_dtype)
    if out is None:
        out = torch.empty((T, H, d), dtype=o_dtype, device=dev)
    _need(out, "out", o_dtype, (T, H, d), dev)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    _need(lse, "lse", torch.float32, (H, T), dev)
    nbytes = workspace_bytes(T, H, d, n_seg, False)
    workspace = _workspace_arg(workspace, nbytes, dev)
    status = _status_arg(status, dev)
    hc = None
    if h_cu is not None:
        hc = np.ascontiguousarray(np.asarray(h_cu, dtype=np.int32))
        if hc.size != n_seg + 1:
            raise PvbError(1, "h_cu must have B+1 entries")
    rc = lib().pvb_varlen_attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(cu), _ptr(hc), n_seg, T, H, Hk, d,
                                       scale, _ptr(out), _dtype_code(out.dtype), _ptr(lse),
                                       _prec_code(precision), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _ptr(status),
                                       _stream(dev))
    _check(rc, "varlen_attn_fwd")
    return out, lse, status


def varlen_attn_bwd(q, k, v, o, do, lse, cu, h_cu=None, softmax_scale=None, grad_dtype=None,
                    precision="bf16", dq=None, dk=None, dv=None, workspace=None, status=None):
    """Backward.  Returns (dQ, dK, dV, status) in grad_dtype: dQ [T, H, d],
    dK and dV [T, H_kv, d] (summed over each group's query heads)."""
    torch = _torch()
    T, H, Hk, d = _check_qkv(q, k, v, do)
    dev = q.device
    _need(o, "o", shape=(T, H, d), dev=dev)
    _dtype_code(o.dtype)
    _need(lse, "lse", torch.float32, (H, T), dev)
    n_seg = _cu_arg(cu, "cu", dev)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    grad_dtype = torch.float32 if grad_dtype is None else grad_dtype
    gcode = _dtype_code(grad_dtype)
    dq = torch.empty((T, H, d), dtype=grad_dtype, device=dev) if dq is None else dq
    dk = torch.empty((T, Hk, d), dtype=grad_dtype, device=dev) if dk is None else dk
    dv = torch.empty((T, Hk, d), dtype=grad_dtype, device=dev) if dv is None else dv
    _need(dq, "dq", grad_dtype, (T, H, d), dev)
    _need(dk, "dk", grad_dtype, (T, Hk, d), dev)
    _need(dv, "dv", grad_dtype, (T, Hk, d), dev)
    nbytes = workspace_bytes(T, H, d, n_seg, True, gcode)
    workspace = _workspace_arg(workspace, nbytes, dev)
    status = _status_arg(status, dev)
    hc = None
    if h_cu is not None:
        hc = np.ascontiguousarray(np.asarray(h_cu, dtype=np.int32))
        if hc.size != n_seg + 1:
            raise PvbError(1, "h_cu must have B+1 entries")
    rc = lib().pvb_varlen_attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(o.dtype), _ptr(do),
                                       _ptr(lse), _ptr(cu), _ptr(hc), n_seg, T, H, Hk, d, scale,
                                       _ptr(dq), _ptr(dk), _ptr(dv), gcode, _prec_code(precision),
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _ptr(status), _stream(dev))
    _check(rc, "varlen_attn_bwd")
    return dq, dk, dv, status


def varlen_attn_bwd_noalloc(q, k, v, o, do, lse, cu, dq, dk, dv, status, h_cu=None, softmax_scale=None,
                            precision="bf16"):
    """The backward through pvb_varlen_attn_bwd_noalloc: no workspace argument
    (the library's fixed scratch array serves), and every output passed in,
    so that neither the binding nor the library allocates device memory.
    dQ [T, H, d], dK and dV [T, H_kv, d] share one dtype (bf16 or fp32),
    status int32 [1].  Calls that overlap on one GPU share the scratch and
    race.  Returns (dq, dk, dv, status)."""
    torch = _torch()
    T, H, Hk, d = _check_qkv(q, k, v, do)
    dev = q.device
    _need(o, "o", shape=(T, H, d), dev=dev)
    _dtype_code(o.dtype)
    _need(lse, "lse", torch.float32, (H, T), dev)
    n_seg = _cu_arg(cu, "cu", dev)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    _need(dq, "dq", None, (T, H, d), dev)
    gcode = _dtype_code(dq.dtype)
    _need(dk, "dk", dq.dtype, (T, Hk, d), dev)
    _need(dv, "dv", dq.dtype, (T, Hk, d), dev)
    _need(status, "status", torch.int32, (1,), dev)
    hc = None
    if h_cu is not None:
        hc = np.ascontiguousarray(np.asarray(h_cu, dtype=np.int32))
        if hc.size != n_seg + 1:
            raise PvbError(1, "h_cu must have B+1 entries")
    rc = lib().pvb_varlen_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(o.dtype), _ptr(do),
                                           _ptr(lse), _ptr(cu), _ptr(hc), n_seg, T, H, Hk, d, scale,
                                           _ptr(dq), _ptr(dk), _ptr(dv), gcode, _prec_code(precision),
                                           _ptr(status), _stream(dev))
    _check(rc, "varlen_attn_bwd_noalloc")
    return dq, dk, dv, status


def cross_workspace_bytes(T_q: int, T_k: int, H: int, d: int, n_seg: int, backward: bool,
                          grad_dtype=PVB_F32) -> int:
    return int(lib().pvb_varlen_cross_attn_workspace_bytes(T_q, T_k, H, d, n_seg, int(bool(backward)),
                                                           int(grad_dtype)))


def _check_cross(q, k, v, cu_q, cu_k, h_cu_q, h_cu_k, *rest):
    """q (and dO) [T_q, H, d]; k, v [T_k, H_kv, d]; device cu_q, cu_k int32 [B+1]
    with their host mirrors (both required)."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, dim=3)
    _need(k, "k", torch.bfloat16, dim=3)
    T_q, H, d = q.shape
    T_k, Hk = k.shape[0], k.shape[1]
    dev = q.device
    _need(k, "k", shape=(T_k, Hk, d), dev=dev)
    _need(v, "v", torch.bfloat16, (T_k, Hk, d), dev)
    for t in rest:
        _need(t, "dO", torch.bfloat16, (T_q, H, d), dev)
    if Hk <= 0 or H % Hk != 0:
        raise PvbError(1, "the query heads must be a multiple of the key/value heads")
    n_seg = _cu_arg(cu_q, "cu_q", dev)
    _cu_arg(cu_k, "cu_k", dev)
    if cu_k.numel() != n_seg + 1:
        raise PvbError(1, "cu_q and cu_k must have the same number of segments")
    if h_cu_q is None or h_cu_k is None:
        raise PvbError(1, "the cross form needs the host mirrors h_cu_q and h_cu_k")
    hq = np.ascontiguousarray(np.asarray(h_cu_q, dtype=np.int32))
    hk = np.ascontiguousarray(np.asarray(h_cu_k, dtype=np.int32))
    if hq.size != n_seg + 1 or hk.size != n_seg + 1:
        raise PvbError(1, "h_cu_q and h_cu_k must have B+1 entries")
    return T_q, T_k, H, Hk, d, n_seg, hq, hk


def varlen_cross_attn_fwd(q, k, v, cu_q, cu_k, h_cu_q, h_cu_k, window=(-1, 0), softmax_scale=None,
                          o_dtype=None, precision="bf16", out=None, lse=None, workspace=None, status=None):
    """Forward attention with separate query and key boundaries and a local
    window (window_left, window_right; -1 leaves a side unbounded; (-1, 0) is
    causal aligned to the bottom right).  Returns (O [T_q,H,d], LSE [H,T_q], status);
    rows with no key get O = 0 and LSE = -inf."""
    torch = _torch()
    T_q, T_k, H, Hk, d, n_seg, hq, hk = _check_cross(q, k, v, cu_q, cu_k, h_cu_q, h_cu_k)
    wl, wr = int(window[0]), int(window[1])
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dev = q.device
    if o_dtype is None:
        o_dtype = out.dtype if out is not None else torch.bfloat16
    _dtype_code(o_dtype)
    if out is None:
        out = torch.empty((T_q, H, d), dtype=o_dtype, device=dev)
    _need(out, "out", o_dtype, (T_q, H, d), dev)
    if lse is None:
        lse = torch.empty((H, T_q), dtype=torch.float32, device=dev)
    _need(lse, "lse", torch.float32, (H, T_q), dev)
    nbytes = cross_workspace_bytes(T_q, T_k, H, d, n_seg, False)
    workspace = _workspace_arg(workspace, nbytes, dev)
    status = _status_arg(status, dev)
    rc = lib().pvb_varlen_cross_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_q), _ptr(hq), _ptr(cu_k), _ptr(hk),
                                         n_seg, T_q, T_k, H, Hk, d, wl, wr, scale, _ptr(out),
                                         _dtype_code(out.dtype), _ptr(lse), _prec_code(precision),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _ptr(status), _stream(dev))
    _check(rc, "varlen_cross_attn_fwd")
    return out, lse, status


def varlen_cross_attn_bwd(q, k, v, o, do, lse, cu_q, cu_k, h_cu_q, h_cu_k, window=(-1, 0),
                          softmax_scale=None, grad_dtype=None, precision="bf16", dq=None, dk=None, dv=None,
                          workspace=None, status=None):
    """Backward of varlen_cross_attn_fwd.  Returns (dQ [T_q,H,d], dK, dV [T_k,H_kv,d], status)."""
    torch = _torch()
    T_q, T_k, H, Hk, d, n_seg, hq, hk = _check_cross(q, k, v, cu_q, cu_k, h_cu_q, h_cu_k, do)
    dev = q.device
    _need(o, "o", shape=(T_q, H, d), dev=dev)
    _dtype_code(o.dtype)
    _need(lse, "lse", torch.float32, (H, T_q), dev)
    wl, wr = int(window[0]), int(window[1])
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    grad_dtype = torch.float32 if grad_dtype is None else grad_dtype
    gcode = _dtype_code(grad_dtype)
    dq = torch.empty((T_q, H, d), dtype=grad_dtype, device=dev) if dq is None else dq
    dk = torch.empty((T_k, Hk, d), dtype=grad_dtype, device=dev) if dk is None else dk
    dv = torch.empty((T_k, Hk, d), dtype=grad_dtype, device=dev) if dv is None else dv
    _need(dq, "dq", grad_dtype, (T_q, H, d), dev)
    _need(dk, "dk", grad_dtype, (T_k, Hk, d), dev)
    _need(dv, "dv", grad_dtype, (T_k, Hk, d), dev)
    nbytes = cross_workspace_bytes(T_q, T_k, H, d, n_seg, True, gcode)
    workspace = _workspace_arg(workspace, nbytes, dev)
    status = _status_arg(status, dev)
    rc = lib().pvb_varlen_cross_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(o.dtype), _ptr(do),
                                         _ptr(lse), _ptr(cu_q), _ptr(hq), _ptr(cu_k), _ptr(hk), n_seg, T_q, T_k,
                                         H, Hk, d, wl, wr, scale, _ptr(dq), _ptr(dk), _ptr(dv), gcode,
                                         _prec_code(precision), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _ptr(status),
                                         _stream(dev))
    _check(rc, "varlen_cross_attn_bwd")
    return dq, dk, dv, status


def gated_delta_fwd_workspace_bytes(T: int, H: int, n_seg: int) -> int:
    return int(lib().pvb_gated_delta_fwd_workspace_bytes(T, H, n_seg))


def gated_delta_fwd(q, k, v, g, beta, cu, h_cu=None, scale=None, initial_state=None, final_state=True,
                    o_dtype=None, out=None, state_out=None, workspace=None, chain=False, status=None,
                    train=False):
    """Gated delta rule over the packed stream, the state reset at every
    boundary of ``cu``.  q, k: contiguous bf16 CUDA [T, H_k, 128]; v: [T, H, 128]
    with H a multiple of H_k (value head h reads query/key head h // (H / H_k));
    g, beta: fp32 [T, H]; initial_state: optional fp32 [B, H, 128, 128].  The
    grouped evaluation takes a workspace (allocated when not given); chain=True
    walks each slice's chunks in one chain without one.  train=True runs the
    training forward: the workspace is the backward's
    (gated_delta_bwd_workspace_bytes) and is left holding what
    gated_delta_bwd(..., after_fwd=True) reads.
    Returns (O [T, H, 128], final states [B, H, 128, 128] fp32 or None, status)."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, dim=3)
    _need(v, "v", torch.bfloat16, dim=3)
    T, Hk, d = q.shape
    H = v.shape[1]
    dev = q.device
    _need(k, "k", torch.bfloat16, (T, Hk, d), dev)
    _need(v, "v", shape=(T, H, d), dev=dev)
    if Hk <= 0 or H % Hk != 0:
        raise PvbError(1, "the value heads must be a multiple of the query/key heads")
    _need(g, "g", torch.float32, (T, H), dev)
    _need(beta, "beta", torch.float32, (T, H), dev)
    n_seg = _cu_arg(cu, "cu", dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (n_seg, H, d, d), dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if o_dtype is None:
        o_dtype = out.dtype if out is not None else torch.bfloat16
    _dtype_code(o_dtype)
    if out is None:
        out = torch.empty((T, H, d), dtype=o_dtype, device=dev)
    _need(out, "out", o_dtype, (T, H, d), dev)
    ht = None
    if final_state:
        ht = state_out if state_out is not None else torch.empty((max(n_seg, 0), H, d, d), dtype=torch.float32,
                                                                   device=dev)
        _need(ht, "state_out", torch.float32, (n_seg, H, d, d), dev)
    status = _status_arg(status, dev)
    hc = None
    if h_cu is not None:
        hc = np.ascontiguousarray(np.asarray(h_cu, dtype=np.int32))
        if hc.size != n_seg + 1:
            raise PvbError(1, "h_cu must have B+1 entries")
    if train and (chain or workspace is None):
        raise PvbError(1, "the training forward takes the grouped evaluation and the backward's workspace")
    if chain:
        wp, wb = None, 0
    else:
        nbytes = (gated_delta_bwd_workspace_bytes if train else gated_delta_fwd_workspace_bytes)(T, H, n_seg)
        workspace = _workspace_arg(workspace, nbytes, dev)
        wp, wb = _ptr(workspace), workspace.numel() * workspace.element_size()
    fn = lib().pvb_gated_delta_fwd_train if train else lib().pvb_gated_delta_fwd_gqa
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu), _ptr(hc), n_seg, T, H, Hk, d, scale,
            _ptr(initial_state), _ptr(out), _dtype_code(out.dtype),
            _ptr(ht) if ht is not None and ht.numel() > 0 else None, wp, wb, _ptr(status), _stream(dev))
    _check(rc, "gated_delta_fwd")
    return out, ht, status


def gated_delta_bwd_workspace_bytes(T: int, H: int, n_seg: int) -> int:
    return int(lib().pvb_gated_delta_bwd_workspace_bytes(T, H, n_seg))


def gated_delta_bwd(q, k, v, g, beta, cu, do, h_cu=None, scale=None, initial_state=None, dht=None,
                    grad_dtype=None, dh0=True, workspace=None, status=None, after_fwd=False):
    """Backward of gated_delta_fwd: the gradients of sum(O * do) + sum(ht * dht)
    (dht: gradient of the final states, optional).  after_fwd=True: the
    workspace holds what gated_delta_fwd(..., train=True) left for the same
    inputs, and the recomputation is skipped.  Returns (dq, dk [T, H_k, 128]
    fp32, dv [T, H, 128] in grad_dtype (fp32 by default), dg, dbeta [T, H] fp32,
    dh0 [B, H, 128, 128] fp32 or None, status)."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, dim=3)
    _need(v, "v", torch.bfloat16, dim=3)
    T, Hk, d = q.shape
    H = v.shape[1]
    dev = q.device
    _need(k, "k", torch.bfloat16, (T, Hk, d), dev)
    _need(v, "v", shape=(T, H, d), dev=dev)
    _need(do, "do", torch.bfloat16, (T, H, d), dev)
    if Hk <= 0 or H % Hk != 0:
        raise PvbError(1, "the value heads must be a multiple of the query/key heads")
    _need(g, "g", torch.float32, (T, H), dev)
    _need(beta, "beta", torch.float32, (T, H), dev)
    n_seg = _cu_arg(cu, "cu", dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (n_seg, H, d, d), dev)
    if dht is not None:
        _need(dht, "dht", torch.float32, (n_seg, H, d, d), dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    grad_dtype = torch.float32 if grad_dtype is None else grad_dtype
    gcode = _dtype_code(grad_dtype)
    dq = torch.empty((T, Hk, d), dtype=torch.float32, device=dev)
    dk = torch.empty((T, Hk, d), dtype=torch.float32, device=dev)
    dv = torch.empty((T, H, d), dtype=grad_dtype, device=dev)
    dg = torch.empty((T, H), dtype=torch.float32, device=dev)
    db = torch.empty((T, H), dtype=torch.float32, device=dev)
    dh = torch.empty((max(n_seg, 0), H, d, d), dtype=torch.float32, device=dev) if dh0 else None
    nbytes = gated_delta_bwd_workspace_bytes(T, H, n_seg)
    if after_fwd and workspace is None:
        raise PvbError(5, "gated_delta_bwd(after_fwd=True) needs the training forward's workspace")
    workspace = _workspace_arg(workspace, nbytes, dev)
    status = _status_arg(status, dev)
    hc = None
    if h_cu is not None:
        hc = np.ascontiguousarray(np.asarray(h_cu, dtype=np.int32))
        if hc.size != n_seg + 1:
            raise PvbError(1, "h_cu must have B+1 entries")
    fn = lib().pvb_gated_delta_bwd_after_fwd if after_fwd else lib().pvb_gated_delta_bwd
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu), _ptr(hc), n_seg, T, H, Hk, d, scale,
            _ptr(initial_state), _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db),
            _ptr(dh) if dh is not None and dh.numel() else None, gcode, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(status), _stream(dev))
    _check(rc, "gated_delta_bwd")
    return dq, dk, dv, dg, db, dh, status
