"""Pins for the gradient oracle (oracle/cca_backward.py).

Each pin takes the backward module (so a test can plant a mistake in it) and
returns (ok, detail).  References: central finite differences of the forward
oracle (itself pinned by `oracle_pins`) -- the definition of the derivative --
and, where CCA is plain causal attention (g = 1, or a window covering the whole
sequence), torch's autograd of its scaled-dot-product attention in float64 (a
library routine).  Page: the CCA write-up "ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"
(Triton section: the fused operator also serves training).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.cca_oracle as fwd
from long_context_sparse_cca_amd.synth import np_inputs


def _err(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def _loss(Q, K, V, W, g, k, scale):
    return float(np.sum(fwd.cca_slice(Q, K, V, g, k, scale) * W))


def pin_finite_differences(b):
    """Every gradient entry against a central difference of sum(O * dO) (step 1e-6, fp64)."""
    worst = 0.0
    for (L, g, k, d, seed) in [(12, 3, 1, 3, 1), (13, 2, 0, 2, 2), (10, 4, 1, 3, 3), (9, 3, 5, 2, 4)]:
        Q, K, V = (x[0, 0].astype(np.float64) for x in np_inputs(1, 1, L, d, "f32", seed))
        W = np.random.default_rng(seed + 50).standard_normal((L, d))
        sc = 0.7
        dQ, dK, dV = b.cca_backward_slice(Q, K, V, W, g, k, sc)
        h = 1e-6
        for X, dX in ((Q, dQ), (K, dK), (V, dV)):
            num = np.zeros_like(X)
            for idx in np.ndindex(*X.shape):
                x0 = X[idx]
                X[idx] = x0 + h
                fp = _loss(Q, K, V, W, g, k, sc)
                X[idx] = x0 - h
                fm = _loss(Q, K, V, W, g, k, sc)
                X[idx] = x0
                num[idx] = (fp - fm) / (2 * h)
            worst = max(worst, _err(num, dX))
    return worst < 1e-7, f"max err {worst:.3e}"


def _torch_causal_grads(Q, K, V, W, scale):
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
    (o * torch.tensor(W, dtype=torch.float64)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def pin_causal_special_cases_match_autograd(b):
    """g = 1 (every core token is its own token) and k >= (L-1)/g (no core token visible) are
    causal attention: the gradients equal torch's autograd of causal SDPA."""
    worst = 0.0
    for (L, g, k, d, seed) in [(40, 1, 0, 8, 5), (33, 1, 3, 4, 6), (50, 5, 9, 6, 7), (37, 4, 20, 5, 8)]:
        Q, K, V = (x[0, 0].astype(np.float64) for x in np_inputs(1, 1, L, d, "f32", seed))
        W = np.random.default_rng(seed + 60).standard_normal((L, d))
        sc = 1.0 / math.sqrt(d)
        got = b.cca_backward_slice(Q, K, V, W, g, k, sc)
        want = _torch_causal_grads(Q, K, V, W, sc)
        worst = max(worst, *(_err(x, y) for x, y in zip(got, want)))
    return worst < 1e-12, f"max err {worst:.3e}"


def pin_lse_matches_library_logsumexp(b):
    """With no core token visible the log-sum-exp is torch.logsumexp over the causal scores."""
    L, d, g = 30, 4, 3
    Q, K, V = (x[0, 0].astype(np.float64) for x in np_inputs(1, 1, L, d, "f32", 9))
    sc = 0.5
    out, lse = b.cca_forward_lse_slice(Q, K, V, g, L, sc)
    z = torch.tensor(sc * Q @ K.T)
    z = z.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    want = torch.logsumexp(z, dim=-1).numpy()
    e = max(_err(lse, want), _err(out, fwd.cca_slice(Q, K, V, g, L, sc)))
    return e < 1e-12, f"max err {e:.3e}"


def pin_gqa_finite_differences(b):
    """Grouped-query gradients (r = 2 and r = 3 query heads per key/value head) against central
    differences of the grouped-query forward of oracle/cca_serving.py."""
    import oracle.cca_serving as serving
    worst = 0.0
    for (H, Hkv, L, g, k, d, seed) in [(4, 2, 9, 3, 1, 2, 11), (3, 1, 8, 2, 1, 2, 12)]:
        Q = np_inputs(1, H, L, d, "f32", seed)[0].astype(np.float64)
        K, V = (x[:, :Hkv].astype(np.float64) for x in np_inputs(1, H, L, d, "f32", seed + 1)[1:])
        W = np.random.default_rng(seed + 70).standard_normal((1, H, L, d))
        sc = 0.6
        dQ, dK, dV = b.cca_backward_gqa(Q, K, V, W, g, k, sc)

        def loss():
            return float(np.sum(serving.cca_gqa(Q, K, V, g, k, sc) * W))

        h = 1e-6
        for X, dX in ((Q, dQ), (K, dK), (V, dV)):
            num = np.zeros_like(X)
            for idx in np.ndindex(*X.shape):
                x0 = X[idx]
                X[idx] = x0 + h
                fp = loss()
                X[idx] = x0 - h
                fm = loss()
                X[idx] = x0
                num[idx] = (fp - fm) / (2 * h)
            worst = max(worst, _err(num, dX))
    return worst < 1e-7, f"max err {worst:.3e}"


def pin_sampled_entries_match_full_backward(b):
    """The per-entry form (used at full sizes on sampled rows and keys) gives the entries of the
    full backward, core-token, raw-window and group-last rows included."""
    worst = 0.0
    for (L, g, k, d, seed) in [(50, 4, 2, 5, 13), (37, 3, 0, 4, 14), (64, 8, 1, 6, 15)]:
        Q, K, V = (x[0, 0].astype(np.float64) for x in np_inputs(1, 1, L, d, "f32", seed))
        W = np.random.default_rng(seed + 80).standard_normal((L, d))
        sc = 0.6
        fQ, fK, fV = b.cca_backward_slice(Q, K, V, W, g, k, sc)
        rows = list(range(L))
        sQ, sK, sV = b.cca_backward_sampled_slice(Q, K, V, W, g, k, sc, rows, rows)
        worst = max(worst, _err(sQ, fQ), _err(sK, fK), _err(sV, fV))
    # grouped-query: r = 3 query heads over one key/value head
    L, g, k, d = 40, 4, 1, 4
    Q = np_inputs(1, 3, L, d, "f32", 16)[0].astype(np.float64)
    K, V = (x[:, :1].astype(np.float64) for x in np_inputs(1, 3, L, d, "f32", 17)[1:])
    W = np.random.default_rng(18).standard_normal((1, 3, L, d))
    fQ, fK, fV = b.cca_backward_gqa(Q, K, V, W, g, k, 0.6)
    rows = list(range(L))
    sQ, sK, sV = b.cca_backward_sampled_slice(Q[0], K[0, 0], V[0, 0], W[0], g, k, 0.6, rows, rows)
    worst = max(worst, _err(sQ, fQ[0]), _err(sK, fK[0, 0]), _err(sV, fV[0, 0]))
    return worst < 1e-10, f"max err {worst:.3e}"


ALL_BACKWARD_PINS = [pin_finite_differences, pin_causal_special_cases_match_autograd,
                     pin_lse_matches_library_logsumexp, pin_gqa_finite_differences,
                     pin_sampled_entries_match_full_backward]
