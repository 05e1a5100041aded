"""Pins for the serving part of the oracle (grouped-query attention, per-position rows).

Each pin takes the serving oracle module as its argument (so a test can plant
a mistake in it) and returns (ok, detail).  They use only hand-derived closed
forms, the core oracle (itself pinned by `oracle_pins`), and structural facts:
with one query head per key/value head grouped-query CCA is CCA; with the
query heads of a group identical it is CCA with the key/value heads
repeated; streaming the tokens through a cache reproduces prefill rows.

Pages cited: the CCA write-up "ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"
(global-aware pooling, global-local fusion, Triton section: KV cache in
decode) and "Latent-Condensed Transformer for Efficient Long Context
Modeling" (section 2: mean-query importance; section 3: grouped-query
attention).
"""

from __future__ import annotations

import math

import numpy as np

import oracle.cca_oracle as core_oracle
from long_context_sparse_cca_amd.synth import np_inputs

TOL = 1e-12


def _err(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def _gqa_inputs(B, H, Hkv, L, d, seed, dtype="f32"):
    Q, _, _ = np_inputs(B, H, L, d, dtype, seed)
    _, K, V = np_inputs(B, Hkv, L, d, dtype, seed + 1000)
    return Q, K, V


def pin_gqa_one_query_head_per_kv_head_is_cca(s):
    """H == H_kv: grouped-query CCA is the CCA of the core oracle."""
    worst = 0.0
    for (L, g, k, d, seed) in [(37, 4, 1, 8, 1), (50, 5, 0, 6, 4)]:
        Q, K, V = _gqa_inputs(2, 3, 3, L, d, seed)
        sc = 1.0 / math.sqrt(d)
        worst = max(worst, _err(s.cca_gqa(Q, K, V, g, k, sc), core_oracle.cca(Q, K, V, g, k, sc)))
    return worst < TOL, f"max err {worst:.3e}"


def pin_gqa_identical_heads_is_repeated_cca(s):
    """Query heads equal within each group: output of head h = CCA of key/value head h // r.

    Catches a wrong head grouping (distinct key/value heads make every other
    assignment give different outputs).
    """
    worst = 0.0
    for (H, Hkv, L, g, k, d, seed) in [(6, 2, 29, 4, 1, 5, 2), (8, 4, 40, 5, 2, 4, 3), (4, 1, 24, 3, 1, 6, 4)]:
        r = H // Hkv
        X, K, V = _gqa_inputs(1, Hkv, Hkv, L, d, seed)
        Q = np.repeat(X, r, axis=1)  # heads hk*r .. hk*r + r - 1 all equal X[:, hk]
        sc = 1.0 / math.sqrt(d)
        out = s.cca_gqa(Q, K, V, g, k, sc)
        ref = core_oracle.cca(X, K, V, g, k, sc)
        for h in range(H):
            worst = max(worst, _err(out[:, h], ref[:, h // r]))
    return worst < TOL, f"max err {worst:.3e}"


def pin_gqa_mean_query_closed_form(s):
    """Hand-derived values: d = 1, g = 2, k = 0, L = 4, two query heads, one key/value head, scale 1.

    Queries: head 0 = (0, 1, 0, 0), head 1 = (0, 3, 0, 0); keys (0, x, 0, 0) with
    x = ln(3)/2; values (1, 2, 3, 4).  Group 0 is pooled with the mean of the
    two heads' queries at row 1, (1 + 3)/2 = 2: scores (0, 2x) = (0, ln 3), weights
    (1/4, 3/4), so Kc0 = 3x/4 and Vc0 = 7/4 (the first head alone would give
    weights prop. to (1, sqrt 3); the sum of the heads (1/10, 9/10)).
    Outputs (k = 0):
      t=0: 1 for both heads;
      t=1: raw {0, 1}; head 0 (q=1): weights prop. to (1, 3^(1/2)) -> (1 + 2*3^(1/2)) / (1 + 3^(1/2));
           head 1 (q=3): weights prop. to (1, 3^(3/2)) -> (1 + 2*3^(3/2)) / (1 + 3^(3/2));
      t=2: {Kc0, k2} with q = 0: equal weights -> (7/4 + 3)/2 = 19/8;
      t=3: {Kc0, k2, k3} with q = 0: (7/4 + 3 + 4)/3 = 35/12.
    """
    x = math.log(3.0) / 2.0
    Q = np.zeros((1, 2, 4, 1))
    Q[0, 0, 1, 0], Q[0, 1, 1, 0] = 1.0, 3.0
    K = np.array([0.0, x, 0.0, 0.0]).reshape(1, 1, 4, 1)
    V = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 4, 1)
    Kc, Vc, A = s.pool_gqa(Q[0], K[0, 0], V[0, 0], 2, 1.0)
    out = s.cca_gqa(Q, K, V, 2, 0, 1.0)
    r3 = math.sqrt(3.0)
    want = np.array([[1.0, (1 + 2 * r3) / (1 + r3), 19 / 8, 35 / 12],
                     [1.0, (1 + 2 * r3 ** 3) / (1 + r3 ** 3), 19 / 8, 35 / 12]])
    e = max(_err(A[0], [0.25, 0.75]), _err(Kc[0], [3 * x / 4]), _err(Vc[0], [7 / 4]),
            _err(out[0, :, :, 0], want))
    return e < TOL, f"max err {e:.3e}"


def pin_gqa_stream_matches_prefill(s):
    """Streaming one key/value head and its query heads through the cache gives the prefill rows."""
    worst = 0.0
    for (H, Hkv, L, g, k, d, seed, cd) in [(4, 2, 37, 4, 1, 8, 5, None), (6, 2, 45, 5, 2, 4, 6, "bf16"),
                                           (3, 1, 33, 3, 0, 5, 7, None)]:
        Q, K, V = _gqa_inputs(1, H, Hkv, L, d, seed, "bf16" if cd else "f32")
        sc = 1.0 / math.sqrt(d)
        pre = s.cca_gqa(Q, K, V, g, k, sc, core_dtype=cd)
        r = H // Hkv
        for hk in range(Hkv):
            st = s.decode_stream_gqa(Q[0, hk * r:(hk + 1) * r], K[0, hk], V[0, hk], g, k, sc, t_begin=3,
                                     core_dtype=cd)
            worst = max(worst, _err(st, pre[0, hk * r:(hk + 1) * r, 3:]))
    return worst < TOL, f"max err {worst:.3e}"


def pin_serve_rows_match_prefill(s):
    """Rows at chosen positions (a chunk, single tokens) equal the prefill rows (R16)."""
    worst = 0.0
    for (H, Hkv, L, g, k, d, seed) in [(4, 2, 60, 4, 2, 8, 8), (2, 2, 41, 5, 1, 6, 9)]:
        Q, K, V = _gqa_inputs(1, H, Hkv, L, d, seed)
        sc = 1.0 / math.sqrt(d)
        pre = s.cca_gqa(Q, K, V, g, k, sc)
        pos = [0, 1, g - 1, g, L // 2, L // 2 + 1, L // 2 + 2, L - 1]
        rows = s.serve_rows(Q[0], K[0], V[0], pos, g, k, sc)
        worst = max(worst, _err(rows, pre[0][:, pos]))
    return worst < TOL, f"max err {worst:.3e}"


ALL_SERVING_PINS = [
    pin_gqa_one_query_head_per_kv_head_is_cca,
    pin_gqa_identical_heads_is_repeated_cca,
    pin_gqa_mean_query_closed_form,
    pin_gqa_stream_matches_prefill,
    pin_serve_rows_match_prefill,
]
