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

Grouped-query attention (cca_backward_gqa; the forward of oracle/cca_serving.py,
readings R14/R15: r = H / H_kv query heads share one key/value head, whose core
tokens are pooled once with the mean over the r heads of the group's last-token
query): the attention part runs per query head against its key/value head and
the raw and core gradients of the r heads add up; the pooling backward runs once
per key/value head with q_hat = that mean, and its gradient dq_hat reaches each
of the r heads' last-row queries with weight 1/r.

Everything is float64; loops are per query and per group so each step can be
read against the formulas above.  Pinned by finite differences and, in the
cases where CCA is plain causal attention, by torch's autograd of its
scaled-dot-product attention (tests/backward_pins.py).
"""

from __future__ import annotations

import numpy as np

from . import cca_oracle as _o

__all__ = ["softmax_backward", "pool_backward_group", "cca_backward_slice", "cca_backward",
           "cca_forward_lse_slice", "cca_backward_gqa", "cca_backward_sampled_slice"]


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


def _attention_backward(Qh, K, V, Kc, Vc, dOh, g: int, k: int, scale: float):
    """Attention part of the backward for one query head against given raw and core K/V:
    (dQ [L,d], dK_raw [L,d], dV_raw [L,d], dKc [m,d], dVc [m,d])."""
    L, d = Qh.shape
    m = Kc.shape[0]
    dQ = np.zeros((L, d))
    dK = np.zeros((L, d))
    dV = np.zeros((L, d))
    dKc = np.zeros((m, d))
    dVc = np.zeros((m, d))
    for t in range(L):
        n_c = _o.visible_core_count(t, g, k)
        lo, hi = _o.raw_window(t, g, k)
        keys = np.concatenate([Kc[:n_c], K[lo:hi + 1]])
        vals = np.concatenate([Vc[:n_c], V[lo:hi + 1]])
        p = _o.softmax(scale * (keys @ Qh[t]))
        ds = softmax_backward(p, vals @ dOh[t])
        dQ[t] = scale * (ds @ keys)
        dkey = scale * np.outer(ds, Qh[t])
        dval = np.outer(p, dOh[t])
        dKc[:n_c] += dkey[:n_c]
        dVc[:n_c] += dval[:n_c]
        dK[lo:hi + 1] += dkey[n_c:]
        dV[lo:hi + 1] += dval[n_c:]
    return dQ, dK, dV, dKc, dVc


def cca_backward_gqa(Q, K, V, dO, g: int, k: int, scale: float, core_dtype=None):
    """(dQ [B,H,L,d], dK [B,H_kv,L,d], dV [B,H_kv,L,d]) of the grouped-query CCA prefill.

    Q, dO: [B, H, L, d]; K, V: [B, H_kv, L, d], H a multiple of H_kv.  Query head h
    reads key/value head h // r (R15); each key/value head's core tokens are pooled
    once with the mean last-token query of its r heads (R14).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, H, L, d = Q.shape
    Hkv = K.shape[1]
    if H % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    r = H // Hkv
    m = _o.n_core_groups(L, g)
    dQ = np.zeros(Q.shape)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    for b in range(B):
        for hk in range(Hkv):
            heads = range(hk * r, (hk + 1) * r)
            q_mean = Q[b, hk * r:(hk + 1) * r].sum(axis=0) / r
            Kc, Vc, A = _o.pool(q_mean, K[b, hk], V[b, hk], g, scale, core_dtype)
            dKc = np.zeros((m, d))
            dVc = np.zeros((m, d))
            for h in heads:
                gq, gk, gv, gkc, gvc = _attention_backward(Q[b, h], K[b, hk], V[b, hk], Kc, Vc, dO[b, h], g, k,
                                                           scale)
                dQ[b, h] += gq
                dK[b, hk] += gk
                dV[b, hk] += gv
                dKc += gkc
                dVc += gvc
            for j in range(m):
                rows = slice(j * g, (j + 1) * g)
                row = _o.group_query_row(j, g)
                dKg, dVg, dqh = pool_backward_group(A[j], K[b, hk, rows], V[b, hk, rows], q_mean[row], dKc[j],
                                                    dVc[j], scale)
                dK[b, hk, rows] += dKg
                dV[b, hk, rows] += dVg
                for h in heads:
                    dQ[b, h, row] += dqh / r
    return dQ, dK, dV


def cca_backward_sampled_slice(Q, K, V, dO, g: int, k: int, scale: float, rows, keys, core_dtype=None):
    """(dQ[rows], dK[keys], dV[keys]) of one key/value slice, for sizes where the full backward is too slow.

    Q, dO: [L, d] (one query head) or [r, L, d] (the r query heads that share K, V [L, d],
    readings R14/R15: the core tokens are pooled with their mean last-token query); dQ is
    then [r, len(rows), d].  The same chain rule as cca_backward_slice / cca_backward_gqa,
    organised per requested entry: every query's log-sum-exp and D = dO . O, then
      dKc[j], dVc[j] (core token j) as sums over the queries (of every head) that see it,
      the pooling backward of each group a requested key or row belongs to,
      dK[u], dV[u] of a raw key as sums over the queries whose window holds it, plus the
      pooling part when u lies in a complete group,
      dQ[t] over t's visible keys, plus (1/r) d q_hat when t is the last row of a complete group.
    """
    single = np.asarray(Q).ndim == 2
    Qh = np.asarray(Q, dtype=np.float64).reshape((-1,) + np.asarray(Q).shape[-2:])
    dOh = np.asarray(dO, dtype=np.float64).reshape(Qh.shape)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    r, L, d = Qh.shape
    m = _o.n_core_groups(L, g)
    q_mean = Qh.sum(axis=0) / r
    Kc, Vc, A = _o.pool(q_mean, K, V, g, scale, core_dtype)
    # forward output and log-sum-exp of the queries, one query group at a time (the group's
    # rows share the core tokens and the window start; the causal end hides later raw keys);
    # a group's statistics are computed the first time one of its queries is needed, so that
    # at long L only the queries the requested entries depend on are evaluated
    group_stats = {}

    def stats_of_group(beta):
        if beta not in group_stats:
            t0, t1 = beta * g, min(L, beta * g + g)
            n_c = _o.visible_core_count(t0, g, k)
            lo, _ = _o.raw_window(t0, g, k)
            keys_b = np.concatenate([Kc[:n_c], K[lo:t1]])
            vals_b = np.concatenate([Vc[:n_c], V[lo:t1]])
            lse_b = np.empty((r, t1 - t0))
            d_b = np.empty((r, t1 - t0))
            for h in range(r):
                z = scale * (Qh[h, t0:t1] @ keys_b.T)
                hidden = np.arange(lo, t1)[None, :] > np.arange(t0, t1)[:, None]
                z[:, n_c:][hidden] = -np.inf
                mx = z.max(axis=1, keepdims=True)
                e = np.exp(z - mx)
                lse_b[h] = mx[:, 0] + np.log(e.sum(axis=1))
                out = (e / e.sum(axis=1, keepdims=True)) @ vals_b
                d_b[h] = np.einsum("td,td->t", dOh[h, t0:t1], out)
            group_stats[beta] = (lse_b, d_b)
        return group_stats[beta]

    def stats(ts):
        """(lse [r, len(ts)], D = dO . O [r, len(ts)]) of the queries ts (ascending)."""
        ts = np.asarray(ts)
        lse_t = np.empty((r, len(ts)))
        d_t = np.empty((r, len(ts)))
        for beta in np.unique(ts // g):
            sel = (ts // g) == beta
            lse_b, d_b = stats_of_group(int(beta))
            lse_t[:, sel] = lse_b[:, ts[sel] - beta * g]
            d_t[:, sel] = d_b[:, ts[sel] - beta * g]
        return lse_t, d_t

    t_all = np.arange(L)

    core_cache = {}

    def core_grads(j):
        # queries that see core token j: n_c(t) > j, i.e. t >= (j + k + 1) g
        if j not in core_cache:
            ts = t_all[t_all >= (j + k + 1) * g]
            lse_t, d_t = stats(ts)
            dkc = np.zeros(d)
            dvc = np.zeros(d)
            for h in range(r):
                p = np.exp(scale * (Qh[h, ts] @ Kc[j]) - lse_t[h])
                ds = p * (dOh[h, ts] @ Vc[j] - d_t[h])
                dkc += scale * (ds @ Qh[h, ts])
                dvc += p @ dOh[h, ts]
            core_cache[j] = (dkc, dvc)
        return core_cache[j]

    pool_cache = {}

    def pool_grads(j):
        if j not in pool_cache:
            dkc, dvc = core_grads(j)
            rg = slice(j * g, (j + 1) * g)
            pool_cache[j] = pool_backward_group(A[j], K[rg], V[rg], q_mean[_o.group_query_row(j, g)], dkc, dvc,
                                                scale)
        return pool_cache[j]

    dQ = np.zeros((r, len(rows), d))
    for i, t in enumerate(rows):
        n_c = _o.visible_core_count(t, g, k)
        lo, hi = _o.raw_window(t, g, k)
        keys_t = np.concatenate([Kc[:n_c], K[lo:hi + 1]])
        vals_t = np.concatenate([Vc[:n_c], V[lo:hi + 1]])
        lse_t, d_t = stats([t])
        for h in range(r):
            p = np.exp(scale * (keys_t @ Qh[h, t]) - lse_t[h, 0])
            ds = p * (vals_t @ dOh[h, t] - d_t[h, 0])
            dQ[h, i] = scale * (ds @ keys_t)
            if t % g == g - 1 and t // g < m:
                dQ[h, i] += pool_grads(t // g)[2] / r
    dK = np.zeros((len(keys), d))
    dV = np.zeros((len(keys), d))
    for i, u in enumerate(keys):
        # queries whose raw window holds u: u <= t <= (u // g + k + 1) g - 1
        ts = t_all[(t_all >= u) & (t_all <= min(L - 1, (u // g + k + 1) * g - 1))]
        lse_t, d_t = stats(ts)
        for h in range(r):
            p = np.exp(scale * (Qh[h, ts] @ K[u]) - lse_t[h])
            ds = p * (dOh[h, ts] @ V[u] - d_t[h])
            dK[i] += scale * (ds @ Qh[h, ts])
            dV[i] += p @ dOh[h, ts]
        if u // g < m:
            dKg, dVg, _ = pool_grads(u // g)
            dK[i] += dKg[u % g]
            dV[i] += dVg[u % g]
    return (dQ[0] if single else dQ), dK, dV
