"""Helpers for the GPU parity tests: device upload, the library call chain and
the oracle comparison at the stated tolerance."""
from __future__ import annotations

import sys

import numpy as np

import workloads as W
from oracle import attention as A

# The parity bar for attention outputs and gradients, per tensor, against the
# fp64 oracle, for bf16 inputs with fp32 accumulation.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def torch():
    import torch as t
    return t


def dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).cuda()


def dev_cu(lengths):
    """cu_seqlens built on the device by the library's prefix scan."""
    import packed_varlen_block_amd as pvb
    t = torch()
    L = t.tensor(np.asarray(lengths, dtype=np.int32), dtype=t.int32).cuda()
    out = pvb.build_packed_row(L, capacity=int(np.sum(lengths)))
    pvb.check_status(out["status"])
    return out["cu"]


def host_cu(lengths):
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def gpu_fwd(w: W.Workload, o_dtype="bf16", precision="bf16"):
    import packed_varlen_block_amd as pvb
    t = torch()
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    cu = dev_cu(w.lengths)
    od = t.bfloat16 if o_dtype == "bf16" else t.float32
    o, lse, st = pvb.varlen_attn_fwd(q, k, v, cu, o_dtype=od, precision=precision)
    pvb.check_status(st)
    return (q, k, v, cu), o, lse


def gpu_bwd(dev, o, lse, w: W.Workload, grad_dtype="f32", precision="bf16"):
    import packed_varlen_block_amd as pvb
    t = torch()
    q, k, v, cu = dev
    do = dev_bf16(w.do)
    gd = t.bfloat16 if grad_dtype == "bf16" else t.float32
    dq, dk, dv, st = pvb.varlen_attn_bwd(q, k, v, o, do, lse, cu, grad_dtype=gd, precision=precision)
    pvb.check_status(st)
    return dq, dk, dv


def to64(x):
    return x.double().cpu().numpy()


def errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref)
    return float(d.max(initial=0.0)), float(d.mean()) if d.size else 0.0


def bf16_half_ulp(ref: np.ndarray) -> float:
    """Half a bf16 ulp at the largest magnitude of ``ref``: how far rounding to
    the bf16 output format alone can move a value of that size (8 significant
    bits, so the ulp on [2^e, 2^(e+1)) is 2^(e-7))."""
    m = float(np.abs(ref).max(initial=0.0))
    return 0.0 if m == 0.0 else float(2.0 ** (np.floor(np.log2(m)) - 8))


def check(name: str, got: np.ndarray, ref: np.ndarray, max_abs=MAX_ABS, mean_abs=MEAN_ABS, bf16_out=False):
    """Per-tensor max-abs / mean-abs comparison.  With ``bf16_out`` the output
    tensor is stored in bf16 and the max-abs bar also admits that format's own
    rounding of the largest values (half an ulp of max|ref|)."""
    if bf16_out:
        max_abs = max_abs + bf16_half_ulp(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    mx, mn = errors(got, ref)
    say(f"  {name}: max-abs {mx:.3e}  mean-abs {mn:.3e}")
    assert mx <= max_abs and mn <= mean_abs, f"{name}: max-abs {mx:.3e} mean-abs {mn:.3e}"
    return mx, mn


def oracle_inputs(w: W.Workload):
    q = W.bf16_bits_to_f64(w.q)
    k = W.bf16_bits_to_f64(w.k)
    v = W.bf16_bits_to_f64(w.v)
    do = W.bf16_bits_to_f64(w.do) if w.do is not None else None
    return q, k, v, do


def compare_fwd(w: W.Workload, o, lse, heads=None, tag=""):
    q, k, v, _ = oracle_inputs(w)
    cu = host_cu(w.lengths)
    hs = list(range(w.H)) if heads is None else list(heads)
    ro, rl = A.varlen_forward(q, k, v, cu, heads=hs)
    go = to64(o)[:, hs]
    check(f"{tag}O", go, ro[:, hs])
    gl = lse.double().cpu().numpy()[hs]
    # LSE is a diagnostic: tight absolute check on real rows
    check(f"{tag}LSE", gl, rl[hs], max_abs=1e-3, mean_abs=1e-4)


def compare_bwd(w: W.Workload, dq, dk, dv, heads=None, tag=""):
    q, k, v, do = oracle_inputs(w)
    cu = host_cu(w.lengths)
    hs = list(range(w.H)) if heads is None else list(heads)
    rq, rk, rv = A.varlen_backward(q, k, v, do, cu, heads=hs)
    check(f"{tag}dQ", to64(dq)[:, hs], rq[:, hs])
    check(f"{tag}dK", to64(dk)[:, hs], rk[:, hs])
    check(f"{tag}dV", to64(dv)[:, hs], rv[:, hs])
