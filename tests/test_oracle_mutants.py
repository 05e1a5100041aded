"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

This is what makes the pins worth trusting: a dropped term, a wrong index or
a transposed operand anywhere in the oracle must turn at least one pin red.
"""
import numpy as np
import pytest

import oracle.cca_oracle as o
from tests import oracle_pins


def _first_query_row(j, g):
    return j * g  # the group's FIRST token instead of its last


def _window_without_self(t, g, k):
    return max(0, t // g - k) * g, t - 1  # query does not see itself


def _window_one_group_early(t, g, k):
    return max(0, t // g - k - 1) * g, t  # window overlaps the last visible core token


def _all_complete_groups_visible(t, g, k):
    return (t + 1) // g  # core tokens of every complete group, overlapping the window


def _pool_weights_unscaled(Q, K, g, scale):
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    m = K.shape[0] // g
    return np.stack([o.softmax(K[j * g:(j + 1) * g] @ Q[j * g + g - 1]) for j in range(m)]).reshape(m, g)


def _pool_keys_from_values(Q, K, V, g, scale):
    A = o.pool_weights(Q, K, g, scale)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    m = A.shape[0]
    Kc = np.stack([A[j] @ V[j * g:(j + 1) * g] for j in range(m)]).reshape(m, -1)
    Vc = np.stack([A[j] @ V[j * g:(j + 1) * g] for j in range(m)]).reshape(m, -1)
    return Kc, Vc, A


def _softmax_unnormalised(x):
    x = np.asarray(x, np.float64)
    return np.exp(x - x.max(axis=-1, keepdims=True))


def _pairs_dropped_self(L, g, k):
    t = np.arange(L, dtype=np.int64)
    n_c = np.maximum(0, t // g - k)
    return int(n_c.sum()), int((t - n_c * g).sum())


def _cache_tokens_small_ring(n, g, k):
    return {"stored_core": n // g, "ring_slots": k * g, "visible_core": max(0, n // g - k),
            "visible_raw": n - max(0, n // g - k) * g, "full": n}


MUTANTS = {
    "pool scored by first query": ("group_query_row", _first_query_row),
    "window excludes the query itself": ("raw_window", _window_without_self),
    "window overlaps a core token": ("raw_window", _window_one_group_early),
    "core of all complete groups visible": ("visible_core_count", _all_complete_groups_visible),
    "pool softmax without temperature": ("pool_weights", _pool_weights_unscaled),
    "core keys pooled from values": ("pool", _pool_keys_from_values),
    "softmax denominator dropped": ("softmax", _softmax_unnormalised),
    "pair count drops the diagonal": ("attention_pairs", _pairs_dropped_self),
    "ring one group short": ("kv_cache_tokens", _cache_tokens_small_ring),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(o, attr, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            ok, _ = pin(o)
        except Exception:  # a crash also counts as the pin noticing
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant '{name}'"


import oracle.cca_serving as serving
from tests import serving_pins


def _kv_head_modulo(h, H, H_kv):
    return h % H_kv  # interleaved grouping instead of consecutive runs


def _mean_is_first_head(Qh):
    return np.asarray(Qh, np.float64)[0]


def _mean_is_sum(Qh):
    return np.asarray(Qh, np.float64).sum(axis=0)


def _pool_gqa_per_head_last(Qh, K, V, g, scale, core_dtype=None):
    return o.pool(np.asarray(Qh, np.float64)[-1], K, V, g, scale, core_dtype)


SERVING_MUTANTS = {
    "kv head of h is h mod H_kv": ("kv_head_of", _kv_head_modulo),
    "pooling query is the first head's": ("mean_query", _mean_is_first_head),
    "pooling query is the sum of the heads": ("mean_query", _mean_is_sum),
    "gqa pooling with the last head only": ("pool_gqa", _pool_gqa_per_head_last),
}


@pytest.mark.parametrize("name", list(SERVING_MUTANTS))
def test_some_serving_pin_catches(name, monkeypatch):
    attr, fn = SERVING_MUTANTS[name]
    monkeypatch.setattr(serving, attr, fn)
    failed = []
    for pin in serving_pins.ALL_SERVING_PINS:
        try:
            ok, _ = pin(serving)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no serving pin caught mutant '{name}'"


import oracle.cca_backward as bwd
from tests import backward_pins


def _softmax_backward_sign(p, dp):
    p = np.asarray(p, np.float64)
    dp = np.asarray(dp, np.float64)
    return p * (p @ dp - dp)


def _pool_backward_no_weight_grad(a, Kg, Vg, q_hat, dKc_j, dVc_j, scale):
    return np.outer(a, dKc_j), np.outer(a, dVc_j), np.zeros_like(q_hat, dtype=np.float64)


_orig_pool_backward = bwd.pool_backward_group


def _pool_backward_no_query_grad(a, Kg, Vg, q_hat, dKc_j, dVc_j, scale):
    dKg, dVg, _ = _orig_pool_backward(a, Kg, Vg, q_hat, dKc_j, dVc_j, scale)
    return dKg, dVg, np.zeros_like(q_hat, dtype=np.float64)


_orig_attention_backward = bwd._attention_backward


def _attention_only_dq(Q, K, V, dO, g, k, scale, core_dtype=None):
    """dQ of the attention part alone (no pooling backward), per query head."""
    import oracle.cca_serving as serving
    Q, K, V, dO = (np.asarray(x, np.float64) for x in (Q, K, V, dO))
    B, H, L, d = Q.shape
    r = H // K.shape[1]
    out = np.zeros_like(Q)
    for b in range(B):
        for h in range(H):
            hk = h // r
            Kc, Vc, _ = serving.pool_gqa(Q[b, hk * r:(hk + 1) * r], K[b, hk], V[b, hk], g, scale, core_dtype)
            out[b, h] = _orig_attention_backward(Q[b, h], K[b, hk], V[b, hk], Kc, Vc, dO[b, h], g, k, scale)[0]
    return out


def _gqa_dq_hat_to_first_head(Q, K, V, dO, g, k, scale, core_dtype=None):
    """Grouped-query backward whose pooling gradient dq_hat reaches only the first query head of a group."""
    dQ, dK, dV = _orig_gqa_backward(Q, K, V, dO, g, k, scale, core_dtype)
    H = dQ.shape[1]
    r = H // np.asarray(K).shape[1]
    dq_pool = dQ - _attention_only_dq(Q, K, V, dO, g, k, scale, core_dtype)
    for h in range(H):
        if h % r:
            dQ[:, h] -= dq_pool[:, h]
            dQ[:, h - h % r] += dq_pool[:, h]
    return dQ, dK, dV


def _core_key_grads_doubled(Qh, K, V, Kc, Vc, dOh, g, k, scale):
    """Attention backward (grouped-query path) with the core-key gradients doubled."""
    dQ, dK, dV, dKc, dVc = _orig_attention_backward(Qh, K, V, Kc, Vc, dOh, g, k, scale)
    return dQ, dK, dV, dKc * 2.0, dVc


_orig_gqa_backward = bwd.cca_backward_gqa

BACKWARD_MUTANTS = {
    "grouped-query dq_hat to the first head only": ("cca_backward_gqa", _gqa_dq_hat_to_first_head),
    "core-key gradients doubled (grouped-query path)": ("_attention_backward", _core_key_grads_doubled),
    "softmax backward with the wrong sign": ("softmax_backward", _softmax_backward_sign),
    "pooling weights treated as constants": ("pool_backward_group", _pool_backward_no_weight_grad),
    "no gradient into the scoring query": ("pool_backward_group", _pool_backward_no_query_grad),
}


@pytest.mark.parametrize("name", list(BACKWARD_MUTANTS))
def test_some_backward_pin_catches(name, monkeypatch):
    attr, fn = BACKWARD_MUTANTS[name]
    monkeypatch.setattr(bwd, attr, fn)
    failed = []
    for pin in backward_pins.ALL_BACKWARD_PINS:
        try:
            ok, _ = pin(bwd)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no backward pin caught mutant '{name}'"


import oracle.cca_lca as lca
from tests import lca_pins


def _last_query_instead_of_mean(Q, j, g):
    return np.asarray(Q, np.float64)[j * g + g - 1]


def _sum_instead_of_mean(Q, j, g):
    return np.asarray(Q, np.float64)[j * g:(j + 1) * g].sum(axis=0)


_orig_lca_pool = lca.lca_pool


def _pooled_positional_dims(Q, K, V, g, scale, d_rope, anchors=None, core_dtype=None):
    return _orig_lca_pool(Q, K, V, g, scale, 0, anchors, core_dtype)


def _anchor_is_argmin(Q, K, V, g, scale, d_rope, anchors=None, core_dtype=None):
    S = lca.lca_scores(Q, K, g, scale)
    return _orig_lca_pool(Q, K, V, g, scale, d_rope, np.argmin(S, axis=1), core_dtype)


_orig_lca_gqa = lca.lca_gqa


def _lca_gqa_first_head_only(Q, K, V, g, k, scale, d_rope, anchors=None, core_dtype=None):
    """Grouped-query condensation scored with the first query head of each group of heads only."""
    Q = np.asarray(Q, np.float64).copy()
    r = Q.shape[1] // np.asarray(K).shape[1]
    Qs = Q.copy()
    for h in range(Q.shape[1]):
        Qs[:, h] = Q[:, h - h % r]
    _, Kc, Vc, anc = _orig_lca_gqa(Qs, K, V, g, k, scale, d_rope, anchors, core_dtype)
    out = _orig_lca_gqa(Q, K, V, g, k, scale, d_rope, anc, core_dtype)[0]
    return out, Kc, Vc, anc


def _lca_gqa_sum_over_heads(Q, K, V, g, k, scale, d_rope, anchors=None, core_dtype=None):
    """Grouped-query condensation scored with the sum (not the mean) over the query heads."""
    Q = np.asarray(Q, np.float64)
    r = Q.shape[1] // np.asarray(K).shape[1]
    Qs = Q.copy()
    for h in range(Q.shape[1]):
        base = h - h % r
        Qs[:, h] = Q[:, base:base + r].sum(axis=1)
    _, Kc, Vc, anc = _orig_lca_gqa(Qs, K, V, g, k, scale, d_rope, anchors, core_dtype)
    return _orig_lca_gqa(Q, K, V, g, k, scale, d_rope, anc, core_dtype)[0], Kc, Vc, anc


LCA_MUTANTS = {
    "grouped-query importance from the first head": ("lca_gqa", _lca_gqa_first_head_only),
    "grouped-query importance from the summed heads": ("lca_gqa", _lca_gqa_sum_over_heads),
    "importance from the last query": ("group_mean_query", _last_query_instead_of_mean),
    "importance from the summed queries": ("group_mean_query", _sum_instead_of_mean),
    "positional dims pooled": ("lca_pool", _pooled_positional_dims),
    "anchor at the lowest score": ("lca_pool", _anchor_is_argmin),
}


@pytest.mark.parametrize("name", list(LCA_MUTANTS))
def test_some_lca_pin_catches(name, monkeypatch):
    attr, fn = LCA_MUTANTS[name]
    monkeypatch.setattr(lca, attr, fn)
    failed = []
    for pin in lca_pins.ALL_LCA_PINS:
        try:
            ok, _ = pin(lca)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no LCA pin caught mutant '{name}'"
