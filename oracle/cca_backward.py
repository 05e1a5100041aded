"""CPU fp64 oracle for the gradients of CCA attention -- test infrastructure only.

The CCA write-up ("ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展",
Triton section) says the fused operator serves training as well as prefill and
decode, and the models are fine-tuned with it (experiments section).  This
module gives the gradients of the prefill output O with respect to Q, K and V
for an upstream gradient dO, by the chain rule through the three steps of the
forward ([P1] global-aware pooling, locality-preserving module, global-local
fusion):

  pooling    a_j = softmax_i(s_j,i),  s_j,i = scale * q_hat_j . K[jg+i],  q_hat_j = Q[jg+g-1]
             Kc[j] = sum_i a_j,i K[jg+i],   Vc[j] = sum_i a_j,i V[jg+i]
  attention  for query t: keys = [Kc[0:n_c]; K[n_c g .. t]], vals likewise,
             p = softmax(scale * keys @ Q[t]),  O[t] = p @ vals

Backward, per query t (one softmax over the visible set):
  dp_i   = dO[t] . val_i
  ds_i   = p_i * (dp_i - sum_j p_j dp_j)            (softmax Jacobian)
  dQ[t] += scale * sum_i ds_i key_i
  dkey_i += scale * ds_i * Q[t]
  dval_i += p_i * dO[t]
then the core part of dkey/dval (dKc, dVc) flows through the pooling:
  dV[jg+i] += a_j,i dVc[j]
  da_j,i  = dKc[j] . K[jg+i] + dVc[j] . V[jg+i]
  dz_j,i  = a_j,i (da_j,i - sum_l a_j,l da_j,l)     (softmax Jacobian)
  dK[jg+i] += a_j,i dKc[j] + scale * dz_j,i * q_hat_j
  dQ[jg+g-1] += scale * sum_i dz_j,i K[jg+i]
When the core tokens are stored rounded (`core_dtype`), the forward uses the
rounded values and the derivative treats the rounding as the identity.

Everything is float64; loops are per query and per group so each step can be
read against the formulas above.  Pinned by finite differences and, in the
cases where CCA is plain causal attention, by torch's autograd of its
scaled-dot-product attention (tests/backward_pins.py).
"""

from __future__ import annotations

import numpy as np

from . import cca_oracle as _o

__all__ = ["softmax_backward", "pool_backward_group", "cca_backward_slice", "cca_backward",
           "cca_forward_lse_slice"]


def softmax_backward(p, dp):
    """Gradient at the logits of a softmax with output p, given the gradient dp at p."""
    p = np.asarray(p, dtype=np.float64)
    dp = np.asarray(dp, dtype=np.float64)
    return p * (dp - p @ dp)


def pool_backward_group(a, Kg, Vg, q_hat, dKc_j, dVc_j, scale: float):
    """Gradients of one group's rows and of its scoring query from dKc[j], dVc[j].

    Kc[j] = a @ Kg, Vc[j] = a @ Vg with a = softmax(scale * Kg @ q_hat) ([P1]
    core-token and core K/V equations).  Returns (dKg [g,d], dVg [g,d], dq_hat [d]).
    """
    dVg = np.outer(a, dVc_j)
    da = Kg @ dKc_j + Vg @ dVc_j
    dz = softmax_backward(a, da)
    dKg = np.outer(a, dKc_j) + scale * np.outer(dz, q_hat)
    dq_hat = scale * (dz @ Kg)
    return dKg, dVg, dq_hat


def cca_forward_lse_slice(Q, K, V, g: int, k: int, scale: float, core_dtype=None):
    """Forward output [L, d] and per-query log-sum-exp of the scaled scores (natural log)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, d = Q.shape
    Kc, Vc, _ = _o.pool(Q, K, V, g, scale, core_dtype)
    out = np.empty((L, d))
    lse = np.empty(L)
    for t in range(L):
        n_c = _o.visible_core_count(t, g, k)
        lo, hi = _o.raw_window(t, g, k)
        keys = np.concatenate([Kc[:n_c], K[lo:hi + 1]])
        vals = np.concatenate([Vc[:n_c], V[lo:hi + 1]])
        z = scale * (keys @ Q[t])
        mx = z.max()
        e = np.exp(z - mx)
        lse[t] = mx + np.log(e.sum())
        out[t] = (e / e.sum()) @ vals
    return out, lse


def cca_backward_slice(Q, K, V, dO, g: int, k: int, scale: float, core_dtype=None):
    """(dQ, dK, dV) of one slice [L, d] for the upstream gradient dO [L, d]."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    L, d = Q.shape
    m = _o.n_core_groups(L, g)
    Kc, Vc, A = _o.pool(Q, K, V, g, scale, core_dtype)
    dQ = np.zeros((L, d))
    dK = np.zeros((L, d))
    dV = np.zeros((L, d))
    dKc = np.zeros((m, d))
    dVc = np.zeros((m, d))
    # attention over the unified key set, query by query
    for t in range(L):
        n_c = _o.visible_core_count(t, g, k)
        lo, hi = _o.raw_window(t, g, k)
        keys = np.concatenate([Kc[:n_c], K[lo:hi + 1]])
        vals = np.concatenate([Vc[:n_c], V[lo:hi + 1]])
        p = _o.softmax(scale * (keys @ Q[t]))
        dp = vals @ dO[t]
        ds = softmax_backward(p, dp)
        dQ[t] += scale * (ds @ keys)
        dkey = scale * np.outer(ds, Q[t])
        dval = np.outer(p, dO[t])
        dKc[:n_c] += dkey[:n_c]
        dVc[:n_c] += dval[:n_c]
        dK[lo:hi + 1] += dkey[n_c:]
        dV[lo:hi + 1] += dval[n_c:]
    # pooling, group by group
    for j in range(m):
        rows = slice(j * g, (j + 1) * g)
        qh_row = _o.group_query_row(j, g)
        dKg, dVg, dqh = pool_backward_group(A[j], K[rows], V[rows], Q[qh_row], dKc[j], dVc[j], scale)
        dK[rows] += dKg
        dV[rows] += dVg
        dQ[qh_row] += dqh
    return dQ, dK, dV


def cca_backward(Q, K, V, dO, g: int, k: int, scale: float, core_dtype=None):
    """(dQ, dK, dV) for arrays [..., L, d] (any leading batch/head dims)."""
    Q = np.asarray(Q)
    lead = Q.shape[:-2]
    outs = [np.empty(Q.shape, dtype=np.float64) for _ in range(3)]
    for idx in np.ndindex(*lead):
        r = cca_backward_slice(Q[idx], np.asarray(K)[idx], np.asarray(V)[idx], np.asarray(dO)[idx], g, k, scale,
                               core_dtype)
        for o, x in zip(outs, r):
            o[idx] = x
    return tuple(outs)
