"""Seeded synthetic inputs for the five packed-attention workloads.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark. It holds no attention, packing or metadata arithmetic: it only
draws sample lengths and bf16 tensors from fixed seeds, so that both sides of
every comparison see the same bits.

Random streams: ``numpy.random.default_rng([seed, cfg, stream])`` with
stream 0 = lengths, 1 = Q, 2 = K, 3 = V, 4 = dO, 5 = outlier mask.

Tensors are drawn as float32 standard normals, scaled in float32, and rounded
once to bfloat16 (round to nearest, ties to even).  They are returned as raw
``uint16`` bit patterns of shape ``[T, H, d]``; ``bf16_bits_to_f64`` gives the
exact values as float64.

The lengths for the best-fit-decreasing workload are the 20,000 raw sample
lengths; choosing the first pack is the packer's job, not this module's.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

STREAM_LENGTHS, STREAM_Q, STREAM_K, STREAM_V, STREAM_DO, STREAM_OUTLIER = range(6)

# The capacity-6 next-fit example of "Pack sequences without joining their
# contexts" ("Form pairs inside each source range"): BOS=0, EOS=1, three
# documents of 4, 3 and 5 tokens in a 266-entry vocabulary.  The page lost the
# arrays themselves; these are the only documents consistent with the printed
# packed rows and targets ("Fill only the current row").
FIXTURE_DOCUMENTS = ([0, 99, 100, 1], [0, 101, 1], [0, 102, 103, 104, 1])
FIXTURE_CAPACITY = 6
FIXTURE_VOCAB = 266

# The 5/3/4 example of "Packing与 FlashAttention Varlen", section 1.
WORKED_LENGTHS = (5, 3, 4)

CONFIG_NAMES = {
    1: "worked_5_3_4_T12_H2_d64",
    2: "pack_T4096_16seg_H16_d128",
    3: "bfd_first_pack_T8192_H32_d128",
    4: "long_mixed_T32768_H32_d128",
    5: "edge_case_T16384_H16_d128",
}

EDGE_VALUES = (0, 1, 2, 63, 64, 65, 127, 128, 129)


def _rng(seed: int, cfg: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, cfg, stream])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, cfg: int, stream: int, shape, scale: float = 1.0,
                outlier_frac: float = 0.0, outlier_scale: float = 1.0) -> np.ndarray:
    """float32 N(0,1) * scale, optional Bernoulli outliers * outlier_scale, to bf16 bits."""
    x = _rng(seed, cfg, stream).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if outlier_frac > 0.0:
        # one mask stream per tensor: offset the stream id by the tensor's stream
        m = _rng(seed, cfg, STREAM_OUTLIER * 16 + stream).random(shape, dtype=np.float32)
        x[m < np.float32(outlier_frac)] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(x)


# ---------------------------------------------------------------------------
# sample-length recipes
# ---------------------------------------------------------------------------

def lengths_cfg2(seed: int = 0) -> np.ndarray:
    """16 lengths uniform in [64,512], rescaled to sum exactly to 4096.

    floor(raw * 4096 / sum(raw)), then +1 to the entries with the largest
    fractional part (ties to the lower index) until the sum is 4096.
    """
    raw = _rng(seed, 2, STREAM_LENGTHS).integers(64, 512, size=16, endpoint=True)
    total = int(raw.sum())
    scaled = [r * 4096 for r in raw.tolist()]
    base = [s // total for s in scaled]
    frac = [s % total for s in scaled]
    short = 4096 - sum(base)
    order = sorted(range(16), key=lambda i: (-frac[i], i))
    for i in order[:short]:
        base[i] += 1
    return np.asarray(base, dtype=np.int32)


def raw_lengths_cfg3(seed: int = 0, n: int = 20000) -> np.ndarray:
    """20,000 log-normal sample lengths: median 600, sigma 1, clipped to [8, 8192]."""
    z = _rng(seed, 3, STREAM_LENGTHS).standard_normal(n)
    return np.clip(np.rint(600.0 * np.exp(z)), 8, 8192).astype(np.int32)


def lengths_cfg4(seed: int = 0) -> np.ndarray:
    """One 16384-token segment, then uniform [16,1024] lengths filling 32768."""
    rng = _rng(seed, 4, STREAM_LENGTHS)
    out = [16384]
    used = 16384
    while used < 32768:
        x = int(rng.integers(16, 1024, endpoint=True))
        x = min(x, 32768 - used)
        out.append(x)
        used += x
    return np.asarray(out, dtype=np.int32)


def lengths_cfg5(seed: int = 0):
    """Edge-case lengths summing to 16384; returns (lengths, seed_used).

    Each draw picks c in [0,10); c < 9 selects EDGE_VALUES[c], c == 9 a uniform
    length in [1,4096].  The last draw is truncated to the remainder.  If some
    listed value never occurs the seed is stepped until every one does.
    """
    s = seed
    while True:
        rng = _rng(s, 5, STREAM_LENGTHS)
        out = []
        used = 0
        while used < 16384:
            c = int(rng.integers(0, 10))
            x = EDGE_VALUES[c] if c < 9 else int(rng.integers(1, 4096, endpoint=True))
            x = min(x, 16384 - used)
            out.append(x)
            used += x
        if all(v in out for v in EDGE_VALUES):
            return np.asarray(out, dtype=np.int32), s
        s += 1000


# ---------------------------------------------------------------------------
# full workloads
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    cfg: int
    name: str
    lengths: np.ndarray            # int32 [B] segment lengths of the attention pack
    H: int
    d: int
    q: np.ndarray                  # uint16 bf16 bits [T, H, d]
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray | None          # uint16 bf16 bits [T, H, d] or None (forward only)
    backward: bool
    seed: int
    extra: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.q.shape[0])


def tensors(seed: int, cfg: int, T: int, H: int, d: int, scale: float,
            backward: bool, outlier_frac: float = 0.0, outlier_scale: float = 1.0):
    shp = (T, H, d)
    q = normal_bf16(seed, cfg, STREAM_Q, shp, scale, outlier_frac, outlier_scale)
    k = normal_bf16(seed, cfg, STREAM_K, shp, scale, outlier_frac, outlier_scale)
    v = normal_bf16(seed, cfg, STREAM_V, shp, scale, outlier_frac, outlier_scale)
    do = normal_bf16(seed, cfg, STREAM_DO, shp, 1.0) if backward else None
    return q, k, v, do


# head counts of the five workloads
HEADS = {1: 2, 2: 16, 3: 32, 4: 32, 5: 16}


def make(cfg: int, seed: int = 0, first_pack_lengths=None, H=None, backward=None) -> Workload:
    """Build workload ``cfg`` (1..5).

    ``cfg == 3`` needs ``first_pack_lengths``: the lengths of the first pack that a
    best-fit-decreasing packer makes from ``raw_lengths_cfg3(seed)`` at budget 8192.
    ``H`` overrides the head count (used to cut a bounded sample of a workload).
    """
    extra = {}
    if cfg not in HEADS:
        raise ValueError(f"unknown workload {cfg}")
    h = HEADS[cfg]
    if cfg == 1:
        lengths = np.asarray(WORKED_LENGTHS, dtype=np.int32)
        d, scale, bwd = 64, 1.0, False
    elif cfg == 2:
        lengths = lengths_cfg2(seed)
        d, scale, bwd = 128, 0.5, False
    elif cfg == 3:
        if first_pack_lengths is None:
            raise ValueError("cfg 3 needs the first pack's lengths from a BFD packer")
        lengths = np.asarray(first_pack_lengths, dtype=np.int32)
        d, scale, bwd = 128, 0.5, True
    elif cfg == 4:
        lengths = lengths_cfg4(seed)
        d, scale, bwd = 128, 0.5, True
    else:
        lengths, used = lengths_cfg5(seed)
        extra["seed_used"] = used
        d, scale, bwd = 128, 1.0, True
    if H is not None:
        h = int(H)
    if backward is not None:
        bwd = bool(backward)
    T = int(lengths.sum())
    if cfg == 5:
        q, k, v, do = tensors(seed, cfg, T, h, d, 1.0, bwd, 0.01, 30.0)
    else:
        q, k, v, do = tensors(seed, cfg, T, h, d, scale, bwd)
    return Workload(cfg, CONFIG_NAMES[cfg], lengths, h, d, q, k, v, do, bwd, seed, extra)


def random_small(seed: int, lengths, H: int, d: int, scale: float = 1.0,
                 backward: bool = True, outlier_frac: float = 0.0,
                 outlier_scale: float = 1.0, cfg_tag: int = 99) -> Workload:
    """A small ad-hoc workload with the given segment lengths (parity sweeps)."""
    lengths = np.asarray(lengths, dtype=np.int32)
    T = int(lengths.sum())
    q, k, v, do = tensors(seed, cfg_tag, T, H, d, scale, backward, outlier_frac, outlier_scale)
    return Workload(cfg_tag, f"small_{cfg_tag}", lengths, H, d, q, k, v, do, backward, seed)


def random_cross(seed: int, lengths_q, lengths_k, H: int, Hk: int, d: int, scale: float = 1.0,
                 backward: bool = True, cfg_tag: int = 98):
    """Inputs with separate query and key segment lengths (cross attention,
    local windows): q, dO bf16 bits [T_q, H, d]; k, v [T_k, Hk, d]."""
    Tq = int(np.sum(np.asarray(lengths_q, dtype=np.int64)))
    Tk = int(np.sum(np.asarray(lengths_k, dtype=np.int64)))
    q = normal_bf16(seed, cfg_tag, STREAM_Q, (Tq, H, d), scale)
    k = normal_bf16(seed, cfg_tag, STREAM_K, (Tk, Hk, d), scale)
    v = normal_bf16(seed, cfg_tag, STREAM_V, (Tk, Hk, d), scale)
    do = normal_bf16(seed, cfg_tag, STREAM_DO, (Tq, H, d), 1.0) if backward else None
    return q, k, v, do


def random_gated_delta(seed: int, lengths, H: int, d: int = 128, g_range=(-0.1, 0.0),
                       beta_range=(0.05, 1.0), initial_state: bool = False, cfg_tag: int = 97,
                       Hk: int | None = None):
    """Inputs of the gated delta rule over a packed stream: q, k bf16 bits of
    unit-norm rows (normalised in float32, then rounded) with Hk heads (H when
    None), v bf16 bits of N(0,1) with H heads, log gates g ~ U(g_range) and
    write strengths beta ~ U(beta_range) as float32 [T, H], and optionally
    float32 initial states N(0,1)*0.1 [B, H, d, d].  Returned as a dict."""
    lengths = np.asarray(lengths, dtype=np.int32)
    T = int(lengths.sum())
    Hk = H if Hk is None else Hk
    r = _rng(seed, cfg_tag, STREAM_Q)
    qf = r.standard_normal((T, Hk, d), dtype=np.float32)
    kf = _rng(seed, cfg_tag, STREAM_K).standard_normal((T, Hk, d), dtype=np.float32)
    qf /= np.maximum(np.linalg.norm(qf, axis=-1, keepdims=True), np.float32(1e-6))
    kf /= np.maximum(np.linalg.norm(kf, axis=-1, keepdims=True), np.float32(1e-6))
    out = {"lengths": lengths, "q": f32_to_bf16_bits(qf), "k": f32_to_bf16_bits(kf),
           "v": normal_bf16(seed, cfg_tag, STREAM_V, (T, H, d), 1.0)}
    rg = _rng(seed, cfg_tag, STREAM_DO)
    out["g"] = rg.uniform(g_range[0], g_range[1], size=(T, H)).astype(np.float32)
    out["beta"] = rg.uniform(beta_range[0], beta_range[1], size=(T, H)).astype(np.float32)
    if initial_state:
        out["h0"] = (_rng(seed, cfg_tag, STREAM_OUTLIER).standard_normal((len(lengths), H, d, d), dtype=np.float32)
                     * np.float32(0.1))
    return out


def device_normal_bf16(shape, seed: int, scale: float, device):
    """N(0,1)·scale rounded to bf16, drawn on the device by torch's seeded
    generator: for tensors too large to draw on the host.  The same values
    feed the kernels and, copied back in samples, the oracle.  ``scale`` should
    be a power of two, so that scaling in bf16 is exact."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.bfloat16).mul_(scale)


def device_unit_rows_bf16(shape, seed: int, device):
    """Rows of unit norm (N(0,1) draws normalised over the last axis in float32,
    then rounded to bf16), drawn on the device by torch's seeded generator, for
    the gated delta rule's q and k at sizes too large for the host."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    x /= x.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    return x.to(torch.bfloat16)


def device_uniform_f32(shape, seed: int, lo: float, hi: float, device):
    """U(lo, hi) float32, drawn on the device by torch's seeded generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32).mul_(hi - lo).add_(lo)
