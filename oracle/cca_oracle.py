"""Plain CPU fp64 oracle for Core Context Aware (CCA) attention.

TEST INFRASTRUCTURE ONLY.  This module is the checker the HIP path is
compared against.  Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import it; the library itself never does,
and this module imports nothing from the library (the two share no code).

Sources (cited by page title and section; the pages' equations did not
survive extraction, so equations are named by what they define):

  [P1] "ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"
       (xinfinite.net topic 12717), a write-up of the ICML 2025 paper
       "Core Context Aware Transformers for Long Context Language Modeling".
       Sections used: global-aware pooling (全局感知池化) with its core-token
       equation and core K/V equation; locality-preserving module (局部保留模块)
       with its local-window equation; differentiable global-local fusion
       (全局-局部模块可微融合) with its unified-K/V and per-position output
       equations; Triton acceleration (基于 Triton 的底层加速); compute and
       memory efficiency (计算和存储效率对比, Fig. 3).
  [P3] "Latent-Condensed Transformer for Efficient Long Context Modeling"
       (gist.science), section 2 "Methodology", inference flow: used only as
       corroboration of the streaming decode cache.

What is computed, per (batch, head) slice with Q, K, V of shape [L, d]:

  1. Groups: positions [j*g, (j+1)*g) for j < m = floor(L/g).  A trailing
     partial group has no core token.
  2. Core tokens: the query of the group's LAST token scores every key of the
     group; a softmax over those g scores weights the group's keys and values:
        a_j = softmax_i(scale * q_hat_j . K[j*g+i]),  Kc[j] = sum_i a_j,i K[j*g+i],
        Vc[j] = sum_i a_j,i V[j*g+i],   q_hat_j = Q[j*g+g-1].
     Pooling post-projection K and V with the same weights equals projecting
     the pooled hidden states (linearity of W_K, W_V).
  3. Visible set of query t: beta = floor(t/g), n_c = max(0, beta - k);
     core tokens Kc[0:n_c] plus raw keys K[n_c*g .. t] (inclusive).
  4. Output: one softmax over the whole visible set (unified K/V).

Storage precision of the core tokens (a reading of the pages): the
core K/V are the projections of the core tokens ([P1] core K/V equation) and
live in the KV cache ([P1] Triton section).  In a model computing in bf16 those
are bf16 tensors, and the page's 93% KV-cache reduction at 128K (Fig. 3) is
what 2-byte core tokens give.  `pool`, `cca_slice` and `decode_stream` therefore
take `core_dtype`: None keeps the core tokens exact (float64); "bf16" / "f16" / "f32"
round each element once, to nearest even, to that storage type before use.
Everything else stays float64.

Readings taken where the pages are silent:
  * pooling temperature = the attention scale (1/sqrt(d) by default) --
    PARITY UNPINNED against the pages: every invariant below is invariant to
    this temperature, and the paper's equation did not survive extraction;
  * only core tokens of groups before the raw window are visible
    (n_c = beta - k), decided by the g = 1 => causal-attention invariant;
  * the query attends to itself (inclusive causal).

Floating point: everything is float64; inputs are upcast exactly.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "softmax",
    "round_storage",
    "group_query_row",
    "n_core_groups",
    "pool_weights",
    "pool",
    "visible_core_count",
    "raw_window",
    "cca_slice",
    "cca",
    "cca_masked_dense",
    "cca_bruteforce",
    "cca_row",
    "decode_stream",
    "kv_cache_tokens",
    "kv_cache_bytes",
    "attention_pairs",
]


# ---------------------------------------------------------------------------
# small building blocks
# ---------------------------------------------------------------------------

def softmax(x: np.ndarray) -> np.ndarray:
    """Explicit max-subtracted softmax along the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    z = x - x.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def round_storage(x: np.ndarray, core_dtype) -> np.ndarray:
    """Round float64 values once to the storage type of the core tokens.

    None: unchanged.  "f32": IEEE float32 (numpy's cast rounds to nearest
    even).  "f16": IEEE binary16 (numpy's cast from float64 rounds to nearest
    even in one step; overflow gives infinity).  "bf16": the 16 high bits of the
    float32 pattern, ties to even, computed from the float64 value directly
    (round-to-odd to float32 first, so the double rounding cannot create a false tie).
    """
    x = np.asarray(x, dtype=np.float64)
    if core_dtype is None:
        return x
    if core_dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if core_dtype == "f16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).astype(np.float64)
    if core_dtype != "bf16":
        raise ValueError(core_dtype)
    f = x.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    # round-to-odd: if the float32 cast was inexact, force its last bit to 1
    inexact = f.astype(np.float64) != x
    u = np.where(inexact, u | 1, u)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def group_query_row(j: int, g: int) -> int:
    """Row whose query scores group j: the group's last token.

    [P1] global-aware pooling, core-token equation: the importance scores of
    group i use the query vector of that group's last token.
    """
    return j * g + g - 1


def n_core_groups(L: int, g: int) -> int:
    """Number of complete, non-overlapping groups of size g in length L.

    [P1] global-aware pooling: the input is split into non-overlapping groups
    of size g.  A trailing partial group produces no core token (reading).
    """
    return L // g


def visible_core_count(t: int, g: int, k: int) -> int:
    """Core tokens visible to query t: groups strictly before its raw window.

    [P1] locality-preserving module (local-window equation, window aligned to
    the group size) and global-local fusion (unified K/V): query t in group
    beta = t // g keeps the k previous groups and its own group raw; every
    earlier group is seen through its core token.
    """
    return max(0, t // g - k)


def raw_window(t: int, g: int, k: int) -> tuple[int, int]:
    """Inclusive range [lo, hi] of raw positions visible to query t.

    [P1] locality-preserving module: every token sees at least the w = k*g
    previous raw tokens; the window start is aligned to a group boundary so
    that nothing between the last visible core token and the window is lost.
    """
    return visible_core_count(t, g, k) * g, t


# ---------------------------------------------------------------------------
# step 1-2: pooling into core tokens
# ---------------------------------------------------------------------------

def pool_weights(Q: np.ndarray, K: np.ndarray, g: int, scale: float) -> np.ndarray:
    """Per-group softmax importance weights a[j, i], shape [m, g].

    [P1] global-aware pooling, core-token equation: scores of every key of
    group j against the query of the group's last token, then a softmax
    over the group.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    L = K.shape[0]
    m = n_core_groups(L, g)
    A = np.empty((m, g), dtype=np.float64)
    for j in range(m):
        q_hat = Q[group_query_row(j, g)]
        scores = scale * (K[j * g:(j + 1) * g] @ q_hat)
        A[j] = softmax(scores)
    return A


def pool(Q, K, V, g: int, scale: float, core_dtype=None):
    """Core keys and values of one slice: (Kc [m,d], Vc [m,d], weights [m,g]).

    [P1] global-aware pooling: core token = importance-weighted sum of the
    group's tokens (core-token equation); the core K/V are that core token
    projected by W_K and W_V (core K/V equation).  By linearity the same
    weights applied to the projected K and V give the same result.
    `core_dtype` rounds the core K/V to their storage type (see module doc).
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, d = K.shape
    m = n_core_groups(L, g)
    A = pool_weights(Q, K, g, scale)
    Kc = np.empty((m, d), dtype=np.float64)
    Vc = np.empty((m, d), dtype=np.float64)
    for j in range(m):
        Kc[j] = A[j] @ K[j * g:(j + 1) * g]
        Vc[j] = A[j] @ V[j * g:(j + 1) * g]
    return round_storage(Kc, core_dtype), round_storage(Vc, core_dtype), A


# ---------------------------------------------------------------------------
# step 3-4: attention over the unified visible set
# ---------------------------------------------------------------------------

def cca_slice(Q, K, V, g: int, k: int, scale: float, core_dtype=None) -> np.ndarray:
    """CCA output [L, d] of one slice, evaluated one query group at a time.

    [P1] global-local fusion: the core K/V of earlier groups and the raw K/V
    of the aligned local window form one key/value set, and each position's
    output is a single softmax attention over it (per-position output
    equation).  All rows of one query group share the same visible core
    count and window start; they differ only in the causal end.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, d = Q.shape
    Kc, Vc, _ = pool(Q, K, V, g, scale, core_dtype)
    out = np.empty((L, d), dtype=np.float64)
    n_groups_total = (L + g - 1) // g
    for beta in range(n_groups_total):
        t0 = beta * g
        t1 = min(L, t0 + g)
        n_c = visible_core_count(t0, g, k)
        lo, _ = raw_window(t0, g, k)
        keys = np.concatenate([Kc[:n_c], K[lo:t1]], axis=0)
        vals = np.concatenate([Vc[:n_c], V[lo:t1]], axis=0)
        scores = scale * (Q[t0:t1] @ keys.T)
        # causal end inside the current group: raw key u is visible to t iff u <= t
        raw_pos = np.arange(lo, t1)
        rows = np.arange(t0, t1)
        hidden = raw_pos[None, :] > rows[:, None]
        scores[:, n_c:][hidden] = -np.inf
        out[t0:t1] = softmax(scores) @ vals
    return out


def _over_slices(fn, Q, K, V, *args):
    Q = np.asarray(Q)
    lead = Q.shape[:-2]
    out = np.empty(Q.shape, dtype=np.float64)
    for idx in np.ndindex(*lead):
        out[idx] = fn(np.asarray(Q)[idx], np.asarray(K)[idx], np.asarray(V)[idx], *args)
    return out


def cca(Q, K, V, g: int, k: int, scale: float | None = None, core_dtype=None) -> np.ndarray:
    """CCA prefill output for arrays [..., L, d] (any leading batch/head dims)."""
    d = np.asarray(Q).shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return _over_slices(cca_slice, Q, K, V, g, k, scale, core_dtype)


def cca_masked_dense(Q, K, V, g: int, k: int, scale: float) -> np.ndarray:
    """Second formulation of one slice: scores against [Kc; K] with a mask.

    Same definition as `cca_slice` ([P1] global-local fusion), written as a
    dense [L, m+L] score matrix and a boolean visibility mask, so that a
    slicing mistake in one formulation shows up as a disagreement.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, _ = Q.shape
    Kc, Vc, _ = pool(Q, K, V, g, scale)
    m = Kc.shape[0]
    keys = np.concatenate([Kc, K], axis=0)
    vals = np.concatenate([Vc, V], axis=0)
    visible = np.zeros((L, m + L), dtype=bool)
    for t in range(L):
        n_c = visible_core_count(t, g, k)
        lo, hi = raw_window(t, g, k)
        visible[t, :n_c] = True
        visible[t, m + lo:m + hi + 1] = True
    scores = scale * (Q @ keys.T)
    scores[~visible] = -np.inf
    return softmax(scores) @ vals


def cca_bruteforce(Q, K, V, g: int, k: int, scale: float) -> list:
    """Third formulation of one slice: scalar pure-Python loops (tiny inputs).

    Follows the steps of [P1] in order: pool every complete group with its
    last token's query, then for each position build its visible list and
    take one softmax over it.
    """
    Q = [[float(x) for x in row] for row in np.asarray(Q)]
    K = [[float(x) for x in row] for row in np.asarray(K)]
    V = [[float(x) for x in row] for row in np.asarray(V)]
    L = len(Q)
    d = len(Q[0])
    m = L // g
    core_k, core_v = [], []
    for j in range(m):
        qh = Q[j * g + g - 1]
        s = [scale * sum(qh[e] * K[j * g + i][e] for e in range(d)) for i in range(g)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        z = sum(w)
        a = [x / z for x in w]
        core_k.append([sum(a[i] * K[j * g + i][e] for i in range(g)) for e in range(d)])
        core_v.append([sum(a[i] * V[j * g + i][e] for i in range(g)) for e in range(d)])
    out = []
    for t in range(L):
        beta = t // g
        n_c = max(0, beta - k)
        keys = core_k[:n_c] + [K[u] for u in range(n_c * g, t + 1)]
        vals = core_v[:n_c] + [V[u] for u in range(n_c * g, t + 1)]
        s = [scale * sum(Q[t][e] * key[e] for e in range(d)) for key in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        z = sum(w)
        out.append([sum(w[i] * vals[i][e] for i in range(len(vals))) / z for e in range(d)])
    return out


def cca_row(q_t, t: int, K, V, Kc, Vc, g: int, k: int, scale: float) -> np.ndarray:
    """Output of the single query t given the slice's raw K/V and core K/V.

    Used for sampled rows at full sizes: same definition as `cca_slice`
    ([P1] global-local fusion, per-position output equation).
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    n_c = visible_core_count(t, g, k)
    lo, hi = raw_window(t, g, k)
    keys = np.concatenate([np.asarray(Kc[:n_c], np.float64), np.asarray(K[lo:hi + 1], np.float64)])
    vals = np.concatenate([np.asarray(Vc[:n_c], np.float64), np.asarray(V[lo:hi + 1], np.float64)])
    p = softmax(scale * (keys @ q_t))
    return p @ vals


# ---------------------------------------------------------------------------
# step 5: decode through an explicit compressed cache
# ---------------------------------------------------------------------------

def decode_stream(Q, K, V, g: int, k: int, scale: float, t_begin: int = 0, core_dtype=None) -> np.ndarray:
    """Feed one slice token by token through an explicit compressed KV cache.

    [P1] Triton acceleration section (the operator supports the KV cache in
    decode) and compute/memory efficiency (both prefill and decode are sped
    up); [P3] methodology, inference flow (old groups are condensed into the
    cache as tokens arrive, the recent tokens stay raw).  The cache is a list
    of core tokens plus a raw ring of R = (k+1)*g slots.  A group is pooled
    when its last token arrives, with that token's query; the output of token
    t is one softmax over the visible core tokens and the raw ring window.
    Returns outputs for t in [t_begin, L).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, d = Q.shape
    R = (k + 1) * g
    ring_k = np.zeros((R, d))
    ring_v = np.zeros((R, d))
    ring_pos = np.full(R, -1, dtype=np.int64)
    core_k: list = []
    core_v: list = []
    outs = []
    for t in range(L):
        slot = t % R
        ring_k[slot] = K[t]
        ring_v[slot] = V[t]
        ring_pos[slot] = t
        if (t + 1) % g == 0:
            beta = t // g
            base = (beta * g) % R
            assert np.array_equal(ring_pos[base:base + g], np.arange(beta * g, beta * g + g))
            a = softmax(scale * (ring_k[base:base + g] @ Q[t]))
            core_k.append(round_storage(a @ ring_k[base:base + g], core_dtype))
            core_v.append(round_storage(a @ ring_v[base:base + g], core_dtype))
        if t < t_begin:
            continue
        n_c = max(0, t // g - k)
        lo = n_c * g
        slots = np.array([u % R for u in range(lo, t + 1)], dtype=np.int64)
        # the ring must still hold every raw position of the window
        assert np.array_equal(ring_pos[slots], np.arange(lo, t + 1))
        keys = np.concatenate([np.array(core_k[:n_c]).reshape(n_c, d), ring_k[slots]])
        vals = np.concatenate([np.array(core_v[:n_c]).reshape(n_c, d), ring_v[slots]])
        p = softmax(scale * (keys @ Q[t]))
        outs.append(p @ vals)
    return np.array(outs).reshape(-1, d)


# ---------------------------------------------------------------------------
# accounting
# ---------------------------------------------------------------------------

def kv_cache_tokens(n_tokens: int, g: int, k: int) -> dict:
    """Token counts held by the compressed cache after n_tokens tokens.

    [P1] compute and memory efficiency (Fig. 3): the cache keeps core tokens
    plus the local raw tokens instead of every token.  Counted by walking the
    groups: one stored core token per completed group, a raw ring of (k+1)*g
    slots, and for reference the part visible to the next query.
    """
    stored_core = sum(1 for j in range(n_tokens) if (j + 1) % g == 0)
    ring = (k + 1) * g
    nxt = n_tokens
    visible_core = visible_core_count(nxt, g, k)
    lo, hi = raw_window(nxt, g, k)
    return {
        "stored_core": stored_core,
        "ring_slots": ring,
        "visible_core": visible_core,
        "visible_raw": hi - lo,  # raw tokens already cached (excludes the new token)
        "full": n_tokens,
    }


def kv_cache_bytes(n_tokens: int, g: int, k: int, B: int, H: int, d: int, elem_bytes: int):
    """(resident compressed-cache bytes, full KV-cache bytes) for K and V."""
    c = kv_cache_tokens(n_tokens, g, k)
    per_token = B * H * 2 * d * elem_bytes
    return (c["stored_core"] + c["ring_slots"]) * per_token, c["full"] * per_token


def attention_pairs(L: int, g: int, k: int) -> tuple[int, int]:
    """(core pairs, raw pairs) summed over all queries of one slice.

    Counts, for every query t, the visible core tokens and raw keys defined by
    `visible_core_count` and `raw_window`.
    """
    t = np.arange(L, dtype=np.int64)
    n_c = np.maximum(0, t // g - k)
    raw = t - n_c * g + 1
    return int(n_c.sum()), int(raw.sum())
