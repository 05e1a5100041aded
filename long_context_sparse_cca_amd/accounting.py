"""Algorithmic work of the CCA hot path (host integer arithmetic, closed forms).

Used by the benchmark to turn measured times into roofline fractions.
For one (b, h) slice with L queries, group size g and k raw groups:
  query t of group beta sees n_c = max(0, beta - k) core tokens and
  t - n_c*g + 1 raw keys.  Summed over t in closed form below.
"""
from __future__ import annotations


def _tri(n: int) -> int:
    return n * (n + 1) // 2


def attention_pairs(L: int, g: int, k: int) -> tuple[int, int]:
    """(core pairs, raw pairs) over all L queries of one slice."""
    full = L // g          # complete query groups
    rem = L - full * g     # rows of the trailing partial group
    # core: every row of group beta sees max(0, beta - k) core tokens
    core = g * _tri(max(0, full - 1 - k)) + rem * max(0, full - k)
    # raw: row r of group beta sees min(beta, k)*g + r + 1 keys
    raw = g * g * sum_min(full, k) + full * _tri(g)
    raw += rem * min(full, k) * g + _tri(rem)
    return core, raw


def sum_min(n: int, k: int) -> int:
    """sum_{beta=0}^{n-1} min(beta, k)."""
    if n <= 0:
        return 0
    a = min(n, k + 1)
    s = _tri(a - 1)
    if n > a:
        s += (n - a) * k
    return s


def prefill_flops(B: int, H: int, L: int, d: int, g: int, k: int) -> int:
    """QK^T + PV multiply-adds of the fused attention: 4*d per visible (query, key) pair."""
    c, r = attention_pairs(L, g, k)
    return 4 * d * (c + r) * B * H


def pool_bytes(B: int, H: int, L: int, d: int, g: int, elem: int) -> int:
    """HBM bytes of the pooling pass: K and V of complete groups, one query row per group, core K/V out."""
    m = L // g
    return B * H * elem * d * (2 * m * g + m + 2 * m)


def lca_pool_bytes(B: int, H: int, L: int, d: int, g: int, elem: int) -> int:
    """HBM bytes of the LCA-style pooling pass: Q, K and V of complete groups read once
    (the anchor's key row is a re-read of a row already fetched), condensed K/V out."""
    m = L // g
    return B * H * elem * d * (3 * m * g + 2 * m)


def attention_min_bytes(B: int, H: int, L: int, d: int, g: int, elem: int, out_elem: int) -> int:
    """Compulsory HBM bytes of the fused attention: Q, K, V and core K/V read once, O written once."""
    m = L // g
    return B * H * d * (elem * (3 * L + 2 * m) + out_elem * L)


def decode_keys(t: int, g: int, k: int) -> int:
    """Visible keys (core + raw) of the query at position t."""
    n_c = max(0, t // g - k)
    return n_c + (t - n_c * g + 1)


def decode_bytes(B: int, H: int, d: int, t: int, g: int, k: int, elem: int, n_chunks: int) -> int:
    """HBM bytes of one decode step: every visible K and V row once, q, the chunk
    partial states (written then read back by the merge) and the output row."""
    kv = decode_keys(t, g, k) * 2 * d * elem
    partials = 2 * n_chunks * (d + 2) * 4
    return B * H * (kv + d * elem + partials + d * elem)


def serve_bytes(lens, H_q: int, H_kv: int, d: int, g: int, k: int, elem: int, n_chunks: int) -> int:
    """HBM bytes of one serving decode step (sequence b's new token at position lens[b]):
    every visible K and V row once per key/value head (shared by its query heads), q,
    the output, and the chunk partials of every query head (written then read back)."""
    total = 0
    for t in lens:
        total += H_kv * decode_keys(int(t), g, k) * 2 * d * elem
        total += H_q * (2 * d * elem + 2 * n_chunks * (d + 2) * 4)
    return total


def backward_flops(B: int, H: int, L: int, d: int, g: int, k: int) -> int:
    """Algorithmic FLOPs of the attention backward: five products per visible (query, key)
    pair given the forward's log-sum-exp (scores recomputed, dP, dV, dK, dQ), 2*d each."""
    core, raw = attention_pairs(L, g, k)
    return 10 * d * (core + raw) * B * H


def extend_flops(lens, n: int, H_q: int, d: int, g: int, k: int) -> int:
    """Algorithmic FLOPs of one chunked append: 4*d per visible (new token, key) pair and
    query head, for the n tokens at positions lens[b] .. lens[b]+n-1 of every sequence."""
    total = 0
    for t0 in lens:
        for p in range(int(t0), int(t0) + n):
            total += decode_keys(p, g, k)
    return 4 * d * H_q * total


def kv_cache_bytes(n_tokens: int, g: int, k: int, B: int, H: int, d: int, elem: int) -> tuple[int, int]:
    per_token = B * H * 2 * d * elem
    return per_token * (n_tokens // g + (k + 1) * g), per_token * n_tokens
