"""Oracle O11: the gated delta rule over a flat packed token stream, with its
recurrent state reset at every boundary (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages ("Packing与 FlashAttention Varlen", section 6) say that the layers
of a hybrid model that carry a linear-attention recurrence (Gated DeltaNet)
take the same cumulative boundaries as the attention layers, and that the
boundary stops the recurrent state from flowing from one sample into the
next.  The pages do not write the recurrence out; the plainest reading is the
published gated delta rule (Yang, Kautz and Hatamizadeh, "Gated Delta
Networks: Improving Mamba2 with Delta Rule", 2024), applied to each slice of
the stream independently:

    for each slice b and head h, with S a [d_k, d_v] state starting at S0[b, h]
    (zero when no initial state is given), for each token t of the slice:
        S   <- exp(g_t) * S                         (gate: decay, g_t <= 0)
        u_t  = beta_t * (v_t - S^T k_t)             (delta: what the memory misses)
        S   <- S + k_t u_t^T                        (write)
        o_t  = scale * S^T q_t                      (read, after the write)
    the slice's final state is S.

This is the same as S_t = S_{t-1} exp(g_t) (I - beta_t k_t k_t^T) + beta_t k_t v_t^T
in the [d_k, d_v] orientation.  Nothing crosses a slice: the state of slice b
starts from S0[b] whatever the previous slice ended with.  Zero-length slices
return their initial state.  Any l2 normalisation of q and k is the caller's
(the pages do not say); the scale is an argument.

Arrays: q, k [T, H_k, d_k]; v [T, H, d_v]; g, beta [T, H]; S0 and the final
states [B, H, d_k, d_v].  H is a multiple of H_k: value head h reads query/key
head h // (H / H_k) (consecutive value heads share one, a reading: the pages
give no head layout for these layers).  A token loop per slice and head,
nothing else.
"""
from __future__ import annotations

import numpy as np


def _check_cu(cu, T):
    cu = [int(x) for x in cu]
    if len(cu) < 1 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0, never decrease and end at T")
    return cu


def gated_delta_segment(q, k, v, g, beta, scale, s0=None):
    """One slice, one head: q, k [L, d_k], v [L, d_v], g, beta [L].
    Returns (O [L, d_v], final state [d_k, d_v])."""
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, dtype=np.float64, copy=True)
    o = np.zeros((L, dv))
    for t in range(L):
        S = np.exp(g[t]) * S
        u = beta[t] * (v[t] - S.T @ k[t])
        S = S + np.outer(k[t], u)
        o[t] = scale * (S.T @ q[t])
    return o, S


def gated_delta_varlen(q, k, v, g, beta, cu, scale, initial_state=None):
    """The packed stream: every slice [cu[b], cu[b+1]) and head runs the
    recurrence from its own initial state.  Returns (O [T, H, d_v],
    final states [B, H, d_k, d_v])."""
    T, Hk, dk = q.shape
    H, dv = v.shape[1], v.shape[2]
    if k.shape != q.shape or H % Hk != 0:
        raise ValueError("q and k share a shape [T, H_k, d_k], and H is a multiple of H_k")
    G = H // Hk
    cu = _check_cu(cu, T)
    B = len(cu) - 1
    o = np.zeros((T, H, dv))
    fin = np.zeros((B, H, dk, dv))
    for b in range(B):
        a, e = cu[b], cu[b + 1]
        for h in range(H):
            s0 = None if initial_state is None else initial_state[b, h]
            ob, sb = gated_delta_segment(q[a:e, h // G], k[a:e, h // G], v[a:e, h], g[a:e, h], beta[a:e, h],
                                         scale, s0)
            o[a:e, h] = ob
            fin[b, h] = sb
    return o, fin
