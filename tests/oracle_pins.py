"""Pins that tie the CPU oracle to facts fixed outside itself.

Each pin takes the oracle module as an argument (so a test can plant a
mistake in it and check that some pin notices) and returns (ok, detail).
The pins use only: library routines (torch's scaled-dot-product attention in
float64 on the CPU), closed forms derived by hand, structural invariants of
the method as the CCA write-up states it, and that page's printed figures.

Page cited: "ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"
(the CCA write-up), sections on global-aware pooling, the locality-preserving
module, global-local fusion and compute/memory efficiency (Fig. 3).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from long_context_sparse_cca_amd.synth import np_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TOL = 1e-12


def _sdpa_causal(Q, K, V, scale):
    """Textbook causal softmax attention via torch (library routine), float64 CPU."""
    q = torch.from_numpy(np.asarray(Q, np.float64))
    k = torch.from_numpy(np.asarray(K, np.float64))
    v = torch.from_numpy(np.asarray(V, np.float64))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale).numpy()


def _err(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def _cases():
    # (L, g, k, d, seed): ragged tails, k = 0, g = L, windows wider than the sequence
    return [(37, 4, 1, 8, 1), (64, 8, 2, 16, 2), (29, 29, 0, 4, 3), (50, 5, 0, 6, 4), (33, 3, 20, 5, 5)]


def pin_g1_is_causal_attention(o):
    """Group size 1: each core token is its single raw token, so CCA is causal attention."""
    worst = 0.0
    for (L, _, _, d, seed) in _cases():
        Q, K, V = np_inputs(1, 2, L, d, "f32", seed)
        scale = 1.0 / math.sqrt(d)
        for k in (0, 1, 3):
            out = o.cca(Q, K, V, 1, k, scale)
            worst = max(worst, _err(out, _sdpa_causal(Q, K, V, scale)))
    return worst < TOL, f"max err {worst:.3e}"


def pin_full_window_is_causal_attention(o):
    """k >= floor((L-1)/g): no core token is ever visible and the window covers [0, t]."""
    worst = 0.0
    for (L, g, _, d, seed) in _cases():
        Q, K, V = np_inputs(1, 2, L, d, "f32", seed)
        scale = 1.0 / math.sqrt(d)
        k = (L - 1) // g
        out = o.cca(Q, K, V, g, k, scale)
        worst = max(worst, _err(out, _sdpa_causal(Q, K, V, scale)))
    return worst < TOL, f"max err {worst:.3e}"


def pin_pool_weights_sum_to_one(o):
    """The per-group importance weights are a softmax: non-negative, summing to one."""
    Q, K, _ = np_inputs(1, 1, 45, 8, "f32", 7)
    A = o.pool_weights(Q[0, 0], K[0, 0], 5, 0.3)
    ok = A.shape == (9, 5) and np.all(A >= 0) and _err(A.sum(axis=1), np.ones(9)) < TOL
    return ok, f"shape {A.shape}"


def pin_identical_keys_mean_pool(o):
    """Identical keys in a group give equal weights: Kc is that key, Vc the mean of V."""
    L, g, d = 24, 6, 4
    Q, K, V = np_inputs(1, 1, L, d, "f32", 8)
    K = K[0, 0].copy()
    for j in range(L // g):
        K[j * g:(j + 1) * g] = K[j * g]
    Kc, Vc, _ = o.pool(Q[0, 0], K, V[0, 0], g, 0.5)
    want_v = V[0, 0].astype(np.float64).reshape(L // g, g, d).mean(axis=1)
    want_k = K[::g]
    e = max(_err(Kc, want_k), _err(Vc, want_v))
    return e < TOL, f"max err {e:.3e}"


def pin_pool_is_last_query_attention(o):
    """Vc[j] (Kc[j]) equals one-query softmax attention of the group's last query over the group's keys."""
    L, g, d = 40, 8, 16
    Q, K, V = np_inputs(1, 1, L, d, "f32", 9)
    Q, K, V = Q[0, 0], K[0, 0], V[0, 0]
    scale = 1.0 / math.sqrt(d)
    Kc, Vc, _ = o.pool(Q, K, V, g, scale)
    worst = 0.0
    for j in range(L // g):
        qh = torch.from_numpy(Q[j * g + g - 1].astype(np.float64))[None, None, None, :]
        kk = torch.from_numpy(K[j * g:(j + 1) * g].astype(np.float64))[None, None]
        vv = torch.from_numpy(V[j * g:(j + 1) * g].astype(np.float64))[None, None]
        sdpa = torch.nn.functional.scaled_dot_product_attention
        worst = max(worst, _err(Vc[j], sdpa(qh, kk, vv, scale=scale)[0, 0, 0].numpy()))
        worst = max(worst, _err(Kc[j], sdpa(qh, kk, kk, scale=scale)[0, 0, 0].numpy()))
    return worst < TOL, f"max err {worst:.3e}"


def pin_one_hot_limit(o):
    """A key far more aligned with the group's last query than the others takes all the weight."""
    g, d = 4, 3
    rng = np.random.default_rng(10)
    Q = rng.standard_normal((8, d))
    K = rng.standard_normal((8, d)) * 0.01
    V = rng.standard_normal((8, d))
    # group 0 is scored by Q[3], group 1 by Q[7]; make key 1 (group 0) and key 6 (group 1) dominant
    K[1] = 200.0 * Q[3]
    K[6] = 200.0 * Q[7]
    Kc, Vc, A = o.pool(Q, K, V, g, 1.0)
    e = max(_err(Vc[0], V[1]), _err(Vc[1], V[6]), _err(Kc[0], K[1]), _err(Kc[1], K[6]))
    return e < 1e-9, f"max err {e:.3e}"


def pin_closed_form_tiny(o):
    """Hand-derived values for d = 1, g = 2, k = 0, L = 4, scale 1.

    Q = (5, 1, 0, 1), K = (0, ln 3, 0, ln 2), V = (1, 2, 3, 4).
    Group 0 is scored by q1 = 1 against keys (0, ln 3): weights (1/4, 3/4), so
    Kc0 = 3 ln3 / 4 and Vc0 = 1/4 * 1 + 3/4 * 2 = 7/4.  Group 1 is scored by
    q3 = 1 against keys (0, ln 2): weights (1/3, 2/3), so Kc1 = 2 ln2 / 3 and
    Vc1 = 3/3 + 2*4/3 = 11/3.
    Outputs (k = 0: query t sees core tokens of groups before its own group):
      t=0: only itself -> v0 = 1
      t=1: raw {0,1} scored by q1 = 1 -> (1/4, 3/4) -> 7/4
      t=2: {Kc0, k2} scored by q2 = 0 -> equal weights -> (7/4 + 3)/2 = 19/8
      t=3: {Kc0, k2, k3} scored by q3 = 1 -> weights prop. to (3^(3/4), 1, 2)
           -> (3^(3/4) * 7/4 + 3 + 2*4) / (3^(3/4) + 3)
    """
    ln2, ln3 = math.log(2.0), math.log(3.0)
    Q = np.array([[5.0], [1.0], [0.0], [1.0]])
    K = np.array([[0.0], [ln3], [0.0], [ln2]])
    V = np.array([[1.0], [2.0], [3.0], [4.0]])
    Kc, Vc, A = o.pool(Q, K, V, 2, 1.0)
    c = 3.0 ** 0.75
    want_out = np.array([[1.0], [7 / 4], [19 / 8], [(c * 7 / 4 + 3 + 8) / (c + 3)]])
    e = max(
        _err(A, [[0.25, 0.75], [1 / 3, 2 / 3]]),
        _err(Kc, [[3 * ln3 / 4], [2 * ln2 / 3]]),
        _err(Vc, [[7 / 4], [11 / 3]]),
        _err(o.cca_slice(Q, K, V, 2, 0, 1.0), want_out),
    )
    return e < TOL, f"max err {e:.3e}"


def pin_formulations_agree(o):
    """Vectorised, masked-dense and scalar brute-force formulations agree on tiny inputs."""
    worst = 0.0
    for (L, g, k, d, seed) in _cases():
        Q, K, V = np_inputs(1, 1, L, d, "f32", seed)
        q, kk, v = Q[0, 0], K[0, 0], V[0, 0]
        s = 1.0 / math.sqrt(d)
        a = o.cca_slice(q, kk, v, g, k, s)
        b = o.cca_masked_dense(q, kk, v, g, k, s)
        c = np.array(o.cca_bruteforce(q, kk, v, g, k, s))
        worst = max(worst, _err(a, b), _err(a, c))
    return worst < TOL, f"max err {worst:.3e}"


def pin_coverage_partition(o):
    """Reachability: visible core groups plus the raw window cover [0, t] exactly once."""
    for (g, k) in [(1, 0), (1, 3), (4, 0), (4, 1), (16, 1), (16, 64), (5, 7)]:
        for t in range(0, 600, 7):
            n_c = o.visible_core_count(t, g, k)
            lo, hi = o.raw_window(t, g, k)
            covered = []
            for j in range(n_c):
                covered.extend(range(j * g, j * g + g))
            covered.extend(range(lo, hi + 1))
            if sorted(covered) != list(range(t + 1)):
                return False, f"g={g} k={k} t={t}"
            # every visible core token belongs to a complete group
            if n_c > o.n_core_groups(t + 1, g):
                return False, f"incomplete core g={g} k={k} t={t}"
            # the window keeps at least the k*g previous raw tokens
            if hi - lo < min(t, k * g):
                return False, f"window too short g={g} k={k} t={t}"
    return True, ""


def pin_decode_matches_prefill(o):
    """Streaming the tokens through the explicit compressed cache reproduces prefill rows."""
    worst = 0.0
    for (L, g, k, d, seed) in _cases():
        Q, K, V = np_inputs(1, 1, L, d, "f32", seed)
        q, kk, v = Q[0, 0], K[0, 0], V[0, 0]
        s = 1.0 / math.sqrt(d)
        worst = max(worst, _err(o.decode_stream(q, kk, v, g, k, s), o.cca_slice(q, kk, v, g, k, s)))
    return worst < TOL, f"max err {worst:.3e}"


def pin_kv_reduction_matches_page(o):
    """At 128K with g = 16 and a 1024-token window the cache keeps about 7% of the KV (page: 93% less)."""
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        fig = json.load(f)
    red_page = fig["kv_cache_reduction_128k"]["value"]
    res, full = o.kv_cache_bytes(131072, 16, 64, 1, 32, 128, 2)
    red = 1.0 - res / full
    c = o.kv_cache_tokens(131072, 16, 64)
    ok = (round(red, 2) == red_page and c["stored_core"] == 8192 and c["ring_slots"] == 1040
          and c["visible_core"] == 8128 and c["visible_raw"] == 1024)
    return ok, f"reduction {red:.4f} vs page {red_page}; {c}"


def pin_pair_count_closed_form(o):
    """Pair counts against the closed form for L a multiple of g and k*g < L.

    Query group beta (g rows) sees max(0, beta-k) core tokens; raw keys per row
    are (beta - n_c)*g + r + 1 for row r of the group.  Summing by hand:
      core = g * sum_{beta=k}^{m-1} (beta - k) = g * (m-k)(m-k-1)/2
      raw  = sum over groups of g*(min(beta,k)*g) + g(g+1)/2
    """
    for (L, g, k) in [(8192, 16, 64), (4096, 8, 3), (1000, 10, 0)]:
        m = L // g
        core = g * (m - k) * (m - k - 1) // 2
        raw = sum(g * min(b, k) * g for b in range(m)) + m * g * (g + 1) // 2
        if o.attention_pairs(L, g, k) != (core, raw):
            return False, f"L={L} g={g} k={k}: {o.attention_pairs(L, g, k)} vs {(core, raw)}"
    return True, ""


ALL_PINS = [
    pin_g1_is_causal_attention,
    pin_full_window_is_causal_attention,
    pin_pool_weights_sum_to_one,
    pin_identical_keys_mean_pool,
    pin_pool_is_last_query_attention,
    pin_one_hot_limit,
    pin_closed_form_tiny,
    pin_formulations_agree,
    pin_coverage_partition,
    pin_decode_matches_prefill,
    pin_kv_reduction_matches_page,
    pin_pair_count_closed_form,
]


def pin_storage_rounding_is_rne(o):
    """round_storage matches torch's float64 -> bfloat16 / float16 / float32 conversions (library routines)."""
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-3, 4, 20000),
                        # exact bf16 ties: round to the even neighbour
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -8 * 1.5])])
    # torch rounds float64 -> float32 -> bfloat16; on float32 values that is one rounding
    x32 = x.astype(np.float32).astype(np.float64)
    want16 = torch.from_numpy(x32).float().to(torch.bfloat16).to(torch.float64).numpy()
    want32 = torch.from_numpy(x).to(torch.float32).to(torch.float64).numpy()
    ok = np.array_equal(o.round_storage(x32, "bf16"), want16) and np.array_equal(o.round_storage(x, "f32"), want32)
    ok = ok and np.array_equal(o.round_storage(x, None), x)
    # binary16: against torch's float -> float16 conversion on float32 values (one rounding there),
    # in range and at exact ties
    xh = np.concatenate([x32[np.abs(x32) < 6.0e4], np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2.0 ** -24 * 1.5])])
    wanth = torch.from_numpy(xh).float().to(torch.float16).to(torch.float64).numpy()
    ok = ok and np.array_equal(o.round_storage(xh, "f16"), wanth)
    ok = ok and o.round_storage(np.array([1.0 + 2.0 ** -11]), "f16")[0] == 1.0
    # just above a binary16 tie: one rounding goes up (through float32 it would tie to even)
    ok = ok and o.round_storage(np.array([1.0 + 2.0 ** -11 + 2.0 ** -40]), "f16")[0] == 1.0 + 2.0 ** -10
    # a value just above a bf16 tie rounds up when rounded once (through float32 it would tie to even)
    ok = ok and o.round_storage(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]), "bf16")[0] == 1.0 + 2.0 ** -7
    # stored core tokens are the exact ones rounded once
    Q, K, V = np_inputs(1, 1, 40, 8, "bf16", 12)
    Kc, Vc, _ = o.pool(Q[0, 0], K[0, 0], V[0, 0], 4, 0.3)
    Kb, Vb, _ = o.pool(Q[0, 0], K[0, 0], V[0, 0], 4, 0.3, "bf16")
    ok = ok and np.array_equal(Kb, want_b(Kc)) and np.array_equal(Vb, want_b(Vc))
    return bool(ok), ""


def want_b(x):
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def pin_stored_core_decode_matches_prefill(o):
    """With bf16 storage of the core tokens, streaming decode still reproduces prefill rows."""
    worst = 0.0
    for (L, g, k, d, seed) in _cases():
        Q, K, V = np_inputs(1, 1, L, d, "bf16", seed)
        q, kk, v = Q[0, 0], K[0, 0], V[0, 0]
        s = 1.0 / math.sqrt(d)
        worst = max(worst, _err(o.decode_stream(q, kk, v, g, k, s, core_dtype="bf16"),
                                o.cca_slice(q, kk, v, g, k, s, core_dtype="bf16")))
    return worst < TOL, f"max err {worst:.3e}"


ALL_PINS.extend([pin_storage_rounding_is_rne, pin_stored_core_decode_matches_prefill])
