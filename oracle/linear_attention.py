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

O12, the backward: the gradients of  sum_t o_t . dO_t + <S_final, dS_final>
(the loss whose output gradient is dO and whose final-state gradient is
dS_final) with respect to q, k, v, g, beta and the initial state, by
reverse-mode differentiation of the same token loop, step by step (the
forward states are kept and the loop is walked backwards).  The pages say
nothing about training these layers beyond their taking the boundaries; the
plainest reading is the exact gradient of the forward above, slice by slice,
with nothing crossing a boundary.

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


def gated_delta_segment_backward(q, k, v, g, beta, scale, do, s0=None, ds_final=None):
    """One slice, one head: the gradients of  sum_t o_t . do_t + <S_final,
    ds_final>  through gated_delta_segment.  q, k [L, d_k], v, do [L, d_v],
    g, beta [L], s0 and ds_final [d_k, d_v] (zero when None).
    Returns (dq, dk [L, d_k], dv [L, d_v], dg, dbeta [L], ds0 [d_k, d_v]).

    Forward step t, as in gated_delta_segment:
        Sd = exp(g_t) S_prev;  pred = Sd^T k_t;  u = beta_t (v_t - pred);
        S_t = Sd + k_t u^T;  o_t = scale S_t^T q_t.
    Backward step t (dS holds the gradient with respect to S_t):
        dS += scale q_t do_t^T;          dq_t = scale S_t do_t
        du = dS^T k_t;                    dk_t = dS u
        dbeta_t = du . (v_t - pred);      dv_t = beta_t du
        dpred = -beta_t du;               dSd = dS + k_t dpred^T;  dk_t += Sd dpred
        dg_t = <dSd, Sd>;                 dS (for S_prev) = exp(g_t) dSd
    and ds0 is the last dS."""
    L, dk_ = k.shape
    dv_ = v.shape[1]
    S = np.zeros((dk_, dv_)) if s0 is None else np.array(s0, dtype=np.float64, copy=True)
    keep = []
    for t in range(L):
        Sd = np.exp(g[t]) * S
        pred = Sd.T @ k[t]
        u = beta[t] * (v[t] - pred)
        S = Sd + np.outer(k[t], u)
        keep.append((Sd, pred, u, S))
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    dg = np.zeros(L)
    dbeta = np.zeros(L)
    dS = np.zeros((dk_, dv_)) if ds_final is None else np.array(ds_final, dtype=np.float64, copy=True)
    for t in range(L - 1, -1, -1):
        Sd, pred, u, St = keep[t]
        dS = dS + scale * np.outer(q[t], do[t])
        dq[t] = scale * (St @ do[t])
        du = dS.T @ k[t]
        dk[t] = dS @ u
        dbeta[t] = du @ (v[t] - pred)
        dv[t] = beta[t] * du
        dpred = -beta[t] * du
        dSd = dS + np.outer(k[t], dpred)
        dk[t] += Sd @ dpred
        dg[t] = np.sum(dSd * Sd)
        dS = np.exp(g[t]) * dSd
    return dq, dk, dv, dg, dbeta, dS


def gated_delta_varlen_backward(q, k, v, g, beta, cu, scale, do, initial_state=None, dht=None):
    """O12 over the packed stream: every slice and head runs
    gated_delta_segment_backward from its own initial state and final-state
    gradient (zero when None).  Returns (dq, dk [T, H_k, d_k], dv [T, H, d_v],
    dg, dbeta [T, H], dh0 [B, H, d_k, d_v]); dq and dk of a query/key head sum
    the value heads that share it."""
    T, Hk, dk_ = q.shape
    H, dv_ = v.shape[1], v.shape[2]
    if k.shape != q.shape or H % Hk != 0:
        raise ValueError("q and k share a shape [T, H_k, d_k], and H is a multiple of H_k")
    G = H // Hk
    cu = _check_cu(cu, T)
    B = len(cu) - 1
    dq = np.zeros((T, Hk, dk_))
    dk = np.zeros((T, Hk, dk_))
    dv = np.zeros((T, H, dv_))
    dg = np.zeros((T, H))
    dbeta = np.zeros((T, H))
    dh0 = np.zeros((B, H, dk_, dv_))
    for b in range(B):
        a, e = cu[b], cu[b + 1]
        for h in range(H):
            s0 = None if initial_state is None else initial_state[b, h]
            dsf = None if dht is None else dht[b, h]
            r = gated_delta_segment_backward(q[a:e, h // G], k[a:e, h // G], v[a:e, h], g[a:e, h], beta[a:e, h],
                                             scale, do[a:e, h], s0, dsf)
            dq[a:e, h // G] += r[0]
            dk[a:e, h // G] += r[1]
            dv[a:e, h] = r[2]
            dg[a:e, h] = r[3]
            dbeta[a:e, h] = r[4]
            dh0[b, h] = r[5]
    return dq, dk, dv, dg, dbeta, dh0
