"""CPU fp64 oracle for CCA attention in a serving setting -- test infrastructure only.

Grouped-query attention (several query heads per key/value head), sequences
of different lengths in one batch, and several new tokens appended to a
sequence in one call.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; it shares no code with
the HIP library.

Sources (by page title and section):

  [P1] "ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展",
       global-aware pooling (core-token and core K/V equations), locality-
       preserving module, global-local fusion, Triton acceleration (the fused
       operator serves training, prefill and decode with a KV cache).
  [P3] "Latent-Condensed Transformer for Efficient Long Context Modeling",
       section 2 (importance of a token in a group scored with a MEAN query;
       inference flow: old groups are condensed as tokens arrive) and
       section 3 (the approach carries over to grouped-query attention).

Readings (the pages do not define CCA for grouped-query attention):

  R14  With r = H / H_kv query heads sharing one key/value head, the core
       token of a group of that key/value head is pooled ONCE, with the mean
       over the r heads of the group's last-token query.  One core token per
       key/value head keeps the compressed cache as small as the raw cache
       of a grouped-query model allows; the mean follows [P3]'s mean-query
       importance score.  With r = 1 this is exactly the pooling of [P1].
  R15  Query head h reads key/value head h // r (the grouping used by
       grouped-query attention: consecutive query heads share a head).
  R16  Variable lengths and chunked appends change nothing in the method:
       the output of a token depends only on its position and on the tokens
       before it, so a token appended at position p (alone, or inside a
       chunk of several) has exactly the prefill output of row p.

Everything is float64; inputs are upcast exactly.
"""

from __future__ import annotations

import math

import numpy as np

from . import cca_oracle as _o

__all__ = [
    "kv_head_of",
    "mean_query",
    "pool_gqa",
    "attend_with_core",
    "cca_gqa",
    "serve_rows",
    "decode_stream_gqa",
]


def kv_head_of(h: int, H: int, H_kv: int) -> int:
    """Key/value head read by query head h (R15: runs of r = H / H_kv consecutive heads share one)."""
    return h // (H // H_kv)


def mean_query(Qh) -> np.ndarray:
    """Mean over the query heads sharing one key/value head: [r, L, d] -> [L, d] (R14)."""
    Qh = np.asarray(Qh, dtype=np.float64)
    return Qh.sum(axis=0) / Qh.shape[0]


def pool_gqa(Qh, K, V, g: int, scale: float, core_dtype=None):
    """Core K/V of one key/value head shared by the query heads Qh [r, L, d].

    [P1] global-aware pooling with the group's last-token query replaced by
    the mean of that query over the r heads (R14).
    """
    return _o.pool(mean_query(Qh), K, V, g, scale, core_dtype)


def attend_with_core(Q, K, V, Kc, Vc, g: int, k: int, scale: float) -> np.ndarray:
    """CCA output [L, d] of one query head given its head's raw and core K/V.

    [P1] global-local fusion: for each query group beta, the visible core
    tokens Kc[0:n_c] and the raw keys K[n_c*g .. t] form one key set and the
    output is one softmax over it; inside the current group the causal end
    hides later raw keys.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Kc = np.asarray(Kc, dtype=np.float64)
    Vc = np.asarray(Vc, dtype=np.float64)
    L, d = Q.shape
    out = np.empty((L, d), dtype=np.float64)
    for beta in range((L + g - 1) // g):
        t0, t1 = beta * g, min(L, beta * g + g)
        n_c = _o.visible_core_count(t0, g, k)
        lo, _ = _o.raw_window(t0, g, k)
        keys = np.concatenate([Kc[:n_c], K[lo:t1]], axis=0)
        vals = np.concatenate([Vc[:n_c], V[lo:t1]], axis=0)
        scores = scale * (Q[t0:t1] @ keys.T)
        hidden = np.arange(lo, t1)[None, :] > np.arange(t0, t1)[:, None]
        scores[:, n_c:][hidden] = -np.inf
        out[t0:t1] = _o.softmax(scores) @ vals
    return out


def _heads(Q, K):
    H, Hkv = np.asarray(Q).shape[-3], np.asarray(K).shape[-3]
    if H % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    return H, Hkv, H // Hkv


def cca_gqa(Q, K, V, g: int, k: int, scale: float | None = None, core_dtype=None) -> np.ndarray:
    """CCA prefill with grouped-query attention.

    Q: [B, H, L, d]; K, V: [B, H_kv, L, d] with H a multiple of H_kv.
    Returns [B, H, L, d].  Each key/value head is pooled once (R14) and
    query head h attends to key/value head h // r (R15).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, L, d = Q.shape
    _, Hkv, r = _heads(Q, K)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.empty((B, H, L, d), dtype=np.float64)
    for b in range(B):
        core = {}
        for hk in range(Hkv):
            sharing = [h for h in range(H) if kv_head_of(h, H, Hkv) == hk]
            core[hk] = pool_gqa(Q[b, sharing], K[b, hk], V[b, hk], g, scale, core_dtype)
        for h in range(H):
            hk = kv_head_of(h, H, Hkv)
            Kc, Vc, _ = core[hk]
            out[b, h] = attend_with_core(Q[b, h], K[b, hk], V[b, hk], Kc, Vc, g, k, scale)
    return out


def serve_rows(Q, K, V, positions, g: int, k: int, scale: float, core_dtype=None) -> np.ndarray:
    """Outputs of one sequence at the given positions (appended tokens, R16).

    Q: [H, T, d], K, V: [H_kv, T, d] hold the sequence up to at least the
    largest position.  Returns [H, len(positions), d]: for every position p
    and query head h, one softmax over the core tokens visible to p (pooled
    per key/value head with the mean query, R14) and the raw window of p.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    H, _, d = Q.shape
    Hkv = K.shape[0]
    positions = [int(p) for p in positions]
    out = np.empty((H, len(positions), d), dtype=np.float64)
    core = {}
    for hk in range(Hkv):
        sharing = [h for h in range(H) if kv_head_of(h, H, Hkv) == hk]
        core[hk] = pool_gqa(Q[sharing], K[hk], V[hk], g, scale, core_dtype)
    for h in range(H):
        hk = kv_head_of(h, H, Hkv)
        Kc, Vc, _ = core[hk]
        for i, p in enumerate(positions):
            out[h, i] = _o.cca_row(Q[h, p], p, K[hk], V[hk], Kc, Vc, g, k, scale)
    return out


def decode_stream_gqa(Qh, K, V, g: int, k: int, scale: float, t_begin: int = 0, core_dtype=None) -> np.ndarray:
    """Feed one key/value head and its r query heads token by token through a cache.

    The streaming counterpart of `cca_gqa` ([P1] Triton section: the KV cache
    in decode; [P3] inference flow).  The cache holds core tokens plus a raw
    ring of R = (k+1)*g slots; a group is pooled when its last token arrives,
    with the mean of that token's r queries (R14); every query head of the
    token then attends to the visible core tokens and the raw window.
    Qh: [r, L, d]; K, V: [L, d].  Returns [r, L - t_begin, d].
    """
    Qh = np.asarray(Qh, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    r, L, d = Qh.shape
    R = (k + 1) * g
    ring_k = np.zeros((R, d))
    ring_v = np.zeros((R, d))
    ring_pos = np.full(R, -1, dtype=np.int64)
    core_k: list = []
    core_v: list = []
    outs = [[] for _ in range(r)]
    for t in range(L):
        slot = t % R
        ring_k[slot], ring_v[slot], ring_pos[slot] = K[t], V[t], t
        if (t + 1) % g == 0:
            base = ((t // g) * g) % R
            assert np.array_equal(ring_pos[base:base + g], np.arange(t + 1 - g, t + 1))
            q_bar = mean_query(Qh[:, t:t + 1])[0]
            a = _o.softmax(scale * (ring_k[base:base + g] @ q_bar))
            core_k.append(_o.round_storage(a @ ring_k[base:base + g], core_dtype))
            core_v.append(_o.round_storage(a @ ring_v[base:base + g], core_dtype))
        if t < t_begin:
            continue
        n_c = max(0, t // g - k)
        lo = n_c * g
        slots = np.array([u % R for u in range(lo, t + 1)], dtype=np.int64)
        assert np.array_equal(ring_pos[slots], np.arange(lo, t + 1))
        keys = np.concatenate([np.array(core_k[:n_c]).reshape(n_c, d), ring_k[slots]])
        vals = np.concatenate([np.array(core_v[:n_c]).reshape(n_c, d), ring_v[slots]])
        for h in range(r):
            p = _o.softmax(scale * (keys @ Qh[h, t]))
            outs[h].append(p @ vals)
    return np.array(outs).reshape(r, -1, d)
