"""CPU fp64 oracle for the LCA-style pooling variant -- test infrastructure only.

Source: "Latent-Condensed Transformer for Efficient Long Context Modeling"
(gist.science), section 2 "Methodology": the context is split into groups; the
importance of a token in its group is scored with the dot product of the
group's MEAN query and the token's key; the content part of the representation
is pooled with those weights (semantic condensation, weighted pooling); the
positional part -- the RoPE key, which cannot be mixed -- is not pooled: the
token with the highest importance is the group's anchor and its positional key
is kept as is (positional anchoring, maximum selection); the most recent w
tokens stay uncondensed (local context).  The attention over condensed groups
plus the local window is the one of the CCA write-up ("ICML 2025 | 全局池化+局部保留，
CCA-Attention为LLM长文本建模带来突破性进展", global-local fusion).

Readings (the page describes the method in MLA's latent space; these kernels
take per-head keys and values):
  R18  the last d_rope dimensions of each key are its positional (RoPE) part,
       the first d - d_rope its content part; values have no positional part;
  R19  the mean query of group j is the mean of Q over the group's g positions;
       the scores use the full key (content and positional dimensions), with the
       attention scale;
  R20  the anchor is the first position with the largest score; where several
       scores are equal to within rounding, any of them is a valid anchor (tests
       check the GPU's choice is such a maximum and compare the rest with the
       oracle evaluated at that choice).
  R21  with grouped-query heads (r = H / H_kv query heads sharing a key/value
       head, as in oracle/cca_serving.py's R14/R15), a key/value head is condensed
       once; its group importance query is the mean over the group's g positions
       and over the r query heads (R14's mean over heads with R19's mean over the
       group), and each query head attends to its key/value head's condensed
       tokens and raw window.
Everything is float64.
"""

from __future__ import annotations

import numpy as np

from . import cca_oracle as _o

__all__ = ["group_mean_query", "lca_scores", "lca_pool", "lca_slice", "lca_gqa", "lca_decode_stream"]


def group_mean_query(Q, j: int, g: int) -> np.ndarray:
    """Mean of the group's g queries (R19)."""
    Q = np.asarray(Q, dtype=np.float64)
    return Q[j * g:(j + 1) * g].sum(axis=0) / g


def lca_scores(Q, K, g: int, scale: float) -> np.ndarray:
    """Importance scores [m, g]: scale * mean query . key, per complete group."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    m = _o.n_core_groups(K.shape[0], g)
    S = np.empty((m, g))
    for j in range(m):
        S[j] = scale * (K[j * g:(j + 1) * g] @ group_mean_query(Q, j, g))
    return S


def lca_pool(Q, K, V, g: int, scale: float, d_rope: int, anchors=None, core_dtype=None):
    """(Kc [m,d], Vc [m,d], anchors [m]) of one slice.

    Content dims of Kc and all of Vc: importance-weighted sums (softmax of the
    scores); positional dims of Kc: the anchor token's key (argmax of the
    scores, or the given `anchors`).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, d = K.shape
    dc = d - d_rope
    S = lca_scores(Q, K, g, scale)
    m = S.shape[0]
    if anchors is None:
        anchors = np.array([int(np.argmax(S[j])) for j in range(m)], dtype=np.int64)
    Kc = np.empty((m, d))
    Vc = np.empty((m, d))
    for j in range(m):
        a = _o.softmax(S[j])
        rows = slice(j * g, (j + 1) * g)
        Kc[j, :dc] = a @ K[rows, :dc]
        Kc[j, dc:] = K[j * g + int(anchors[j]), dc:]
        Vc[j] = a @ V[rows]
    return _o.round_storage(Kc, core_dtype), _o.round_storage(Vc, core_dtype), np.asarray(anchors)


def lca_slice(Q, K, V, g: int, k: int, scale: float, d_rope: int, anchors=None, core_dtype=None) -> np.ndarray:
    """Output [L, d] of one slice: LCA core tokens, then CCA's unified attention."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, d = Q.shape
    Kc, Vc, _ = lca_pool(Q, K, V, g, scale, d_rope, anchors, core_dtype)
    out = np.empty((L, d))
    for t in range(L):
        out[t] = _o.cca_row(Q[t], t, K, V, Kc, Vc, g, k, scale)
    return out


def lca_gqa(Q, K, V, g: int, k: int, scale: float, d_rope: int, anchors=None, core_dtype=None):
    """Grouped-query LCA-style prefill (R21): (out [B,H,L,d], Kc, Vc [B,H_kv,m,d], anchors [B,H_kv,m]).

    Q: [B, H, L, d]; K, V: [B, H_kv, L, d].  `anchors`, if given, fixes the anchor of
    every condensed token (the tests pass the GPU's choice, R20).
    """
    from . import cca_serving as _s
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, L, d = Q.shape
    Hkv = K.shape[1]
    if H % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    r = H // Hkv
    m = _o.n_core_groups(L, g)
    out = np.empty((B, H, L, d))
    Kc = np.empty((B, Hkv, m, d))
    Vc = np.empty((B, Hkv, m, d))
    anc = np.empty((B, Hkv, m), dtype=np.int64)
    for b in range(B):
        for hk in range(Hkv):
            q_mean = Q[b, hk * r:(hk + 1) * r].sum(axis=0) / r       # mean over the r heads, per position
            a_in = None if anchors is None else np.asarray(anchors)[b, hk]
            Kc[b, hk], Vc[b, hk], anc[b, hk] = lca_pool(q_mean, K[b, hk], V[b, hk], g, scale, d_rope, a_in,
                                                        core_dtype)
            for h in range(hk * r, (hk + 1) * r):
                out[b, h] = _s.attend_with_core(Q[b, h], K[b, hk], V[b, hk], Kc[b, hk], Vc[b, hk], g, k, scale)
    return out, Kc, Vc, anc


def lca_decode_stream(Q, K, V, L0: int, g: int, k: int, scale: float, d_rope: int, anchors=None, core_dtype=None):
    """Outputs [L - L0, d] of tokens L0 .. L-1 appended one by one after a prefill of L0 tokens.

    The inference flow of the page (section 2): a group is condensed as soon as its last
    token has arrived, from the queries, keys and values of its g tokens (mean query,
    weighted content, anchored positional part); the token then attends to the condensed
    groups before its window and to the raw window, as in the prefill.  `anchors`, if
    given, fixes each group's anchor (the tests pass the GPU's choice).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, d = Q.shape
    dc = d - d_rope
    Kc, Vc = [], []

    def condense(j):
        s = lca_scores(Q[j * g:(j + 1) * g], K[j * g:(j + 1) * g], g, scale)[0]
        a = _o.softmax(s)
        anc = int(np.argmax(s)) if anchors is None else int(np.asarray(anchors)[j])
        kc = np.empty(d)
        kc[:dc] = a @ K[j * g:(j + 1) * g, :dc]
        kc[dc:] = K[j * g + anc, dc:]
        vc = a @ V[j * g:(j + 1) * g]
        Kc.append(_o.round_storage(kc, core_dtype))
        Vc.append(_o.round_storage(vc, core_dtype))

    for j in range(L0 // g):          # the prefill's condensed groups
        condense(j)
    out = np.empty((L - L0, d))
    for t in range(L0, L):
        if (t + 1) % g == 0:          # the token completes its group
            condense(t // g)
        n_c = _o.visible_core_count(t, g, k)
        lo, hi = _o.raw_window(t, g, k)
        keys = np.concatenate([np.array(Kc[:n_c]).reshape(n_c, d), K[lo:hi + 1]])
        vals = np.concatenate([np.array(Vc[:n_c]).reshape(n_c, d), V[lo:hi + 1]])
        out[t - L0] = _o.softmax(scale * (keys @ Q[t])) @ vals
    return out
