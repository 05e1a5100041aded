"""Decode through the compressed cache vs the oracle's prefill rows.

A sequence of T tokens is prefilled for its first L0 tokens (pooling on the
GPU, then the cache is seeded), and the remaining tokens are appended one at
a time; every decode output must equal the oracle's prefill row of that
position (steps where a group completes and is pooled in place included).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_cca_amd import binding
from long_context_sparse_cca_amd.synth import np_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 5e-3}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# (B, H, d, g, k, L0, T, dtype, seed)
DECODE_CASES = [
    (2, 3, 128, 16, 2, 100, 260, "bf16", 0),
    (1, 2, 64, 16, 1, 37, 150, "f32", 1),
    (2, 2, 128, 5, 3, 0, 90, "f32", 2),      # empty cache: every token appended
    (1, 2, 128, 16, 64, 1500, 1600, "bf16", 3),  # window of 1024 raw tokens, ring wraps
    (1, 1, 64, 1, 4, 20, 60, "bf16", 4),     # g = 1: pooling every step
    (1, 1, 128, 512, 1, 1000, 1100, "bf16", 5),  # groups of 512 pooled in place from the ring
    (1, 2, 128, 16, 4, 300, 400, "f16", 6),   # binary16 cache
    (2, 1, 64, 7, 2, 30, 120, "f16", 7),
]


def _id(c):
    return f"B{c[0]}H{c[1]}d{c[2]}g{c[3]}k{c[4]}L0{c[5]}T{c[6]}-{c[7]}"


@pytest.mark.parametrize("case", DECODE_CASES, ids=_id)
def test_decode_matches_prefill_rows(gpu, case):
    B, H, d, g, k, L0, T, dt, seed = case
    print(f"decode case {_id(case)}", flush=True)
    sys.stdout.flush()
    Q, K, V = np_inputs(B, H, T, d, dt, seed)
    q, kk, v = (torch.from_numpy(x).to(device=gpu, dtype=TDT[dt]).contiguous() for x in (Q, K, V))
    scale = 1.0 / math.sqrt(d)
    cache = binding.KVCache(B, H, d, g, k, max_tokens=T + g, dtype=TDT[dt], device=gpu)
    if L0 > 0:
        kc, vc = binding.pool_kv(q[:, :, :L0].contiguous(), kk[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(),
                                 g, scale)
        cache.load_prefill(kk[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(), kc, vc)
    assert cache.n_tokens == L0
    outs = torch.empty((T - L0, B, H, d), dtype=torch.float32, device=gpu)
    for t in range(L0, T):
        qt = q[:, :, t].contiguous()
        cache.append(qt, kk[:, :, t].contiguous(), v[:, :, t].contiguous(), scale)
        cache.decode(qt, out_dtype=torch.float32, out=outs[t - L0])
    torch.cuda.synchronize()
    assert cache.n_tokens == T
    got = outs.cpu().numpy()
    for b in range(B):
        for h in range(H):
            want = oracle.cca_slice(Q[b, h], K[b, h], V[b, h], g, k, scale, core_dtype=dt)[L0:]
            err = np.abs(got[:, b, h] - want).max()
            assert err <= TOL[dt], f"slice ({b},{h}) max abs err {err:.3e}"


def test_decode_capacity_error(gpu):
    B, H, d, g, k = 1, 1, 64, 4, 1
    cache = binding.KVCache(B, H, d, g, k, max_tokens=8, dtype=torch.float32, device=gpu)
    x = torch.zeros((B, H, d), device=gpu)
    for _ in range(11):
        cache.append(x, x, x)
    with pytest.raises(binding.CCAError, match="capacity"):
        cache.append(x, x, x)
    assert cache.n_tokens == 11


def test_decode_bf16_output_matches_f32_output(gpu):
    B, H, d, g, k, T = 1, 2, 128, 16, 2, 80
    Q, K, V = np_inputs(B, H, T, d, "bf16", 9)
    q, kk, v = (torch.from_numpy(x).to(device=gpu, dtype=torch.bfloat16).contiguous() for x in (Q, K, V))
    cache = binding.KVCache(B, H, d, g, k, max_tokens=T, dtype=torch.bfloat16, device=gpu)
    for t in range(T):
        cache.append(q[:, :, t].contiguous(), kk[:, :, t].contiguous(), v[:, :, t].contiguous())
    qt = q[:, :, T - 1].contiguous()
    a = cache.decode(qt, out_dtype=torch.float32)
    b = cache.decode(qt)
    torch.cuda.synchronize()
    assert b.dtype == torch.bfloat16
    assert torch.equal(a.to(torch.bfloat16), b)


@pytest.mark.parametrize("case", DECODE_CASES, ids=_id)
def test_fused_append_decode_matches_prefill_rows(gpu, case):
    """cca_cache_append_decode (append + attention in one launch) against the oracle and the two-call path."""
    B, H, d, g, k, L0, T, dt, seed = case
    print(f"fused decode case {_id(case)}", flush=True)
    Q, K, V = np_inputs(B, H, T, d, dt, seed)
    q, kk, v = (torch.from_numpy(x).to(device=gpu, dtype=TDT[dt]).contiguous() for x in (Q, K, V))
    scale = 1.0 / math.sqrt(d)
    caches = [binding.KVCache(B, H, d, g, k, max_tokens=T + g, dtype=TDT[dt], device=gpu) for _ in range(2)]
    if L0 > 0:
        kc, vc = binding.pool_kv(q[:, :, :L0].contiguous(), kk[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(),
                                 g, scale)
        for c in caches:
            c.load_prefill(kk[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(), kc, vc)
    fused = torch.empty((T - L0, B, H, d), dtype=torch.float32, device=gpu)
    split = torch.empty_like(fused)
    for t in range(L0, T):
        qt, kt, vt = q[:, :, t].contiguous(), kk[:, :, t].contiguous(), v[:, :, t].contiguous()
        caches[0].append_decode(qt, kt, vt, out_dtype=torch.float32, out=fused[t - L0], scale=scale)
        caches[1].append(qt, kt, vt, scale)
        caches[1].decode(qt, out_dtype=torch.float32, out=split[t - L0], scale=scale)
    torch.cuda.synchronize()
    assert caches[0].n_tokens == T
    # same cache contents and the same outputs as the two-call sequence
    assert torch.equal(caches[0].ring_k, caches[1].ring_k) and torch.equal(caches[0].core_v, caches[1].core_v)
    assert torch.equal(fused, split)
    got = fused.cpu().numpy()
    for b in range(B):
        for h in range(H):
            want = oracle.cca_slice(Q[b, h], K[b, h], V[b, h], g, k, scale, core_dtype=dt)[L0:]
            err = np.abs(got[:, b, h] - want).max()
            assert err <= TOL[dt], f"slice ({b},{h}) max abs err {err:.3e}"


def test_fused_append_decode_capacity_error(gpu):
    B, H, d, g, k = 1, 1, 64, 4, 1
    cache = binding.KVCache(B, H, d, g, k, max_tokens=8, dtype=torch.float32, device=gpu)
    x = torch.zeros((B, H, d), device=gpu)
    for _ in range(11):
        cache.append_decode(x, x, x)
    with pytest.raises(binding.CCAError, match="capacity"):
        cache.append_decode(x, x, x)
    assert cache.n_tokens == 11
