"""Calls on different streams are independent.

Every entry point reads and writes only the buffers the caller passes (the allocation-free
decode, which shares one scratch array per GPU, is the documented exception and is not used
here), so work enqueued on two streams at once must give the same bits as the same calls run
one after the other on one stream: prefill, the fused decode step and the serving step (CCA
and LCA-style caches), each problem on its own stream, interleaved call by call.
Both streams have the default priority.
"""
import math
import sys

import numpy as np
import pytest
import torch

from long_context_sparse_cca_amd import binding
from long_context_sparse_cca_amd.synth import np_inputs

pytestmark = pytest.mark.gpu

TDT = torch.bfloat16


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x, device):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=TDT).contiguous()


def _problem(seed, B, H, L, d, device):
    return [_dev(x, device) for x in np_inputs(B, H, L, d, "bf16", seed)]


def test_prefill_on_two_streams(gpu):
    _say("prefill on two streams")
    probs = [(_problem(61, 1, 4, 3000, 128, gpu), 16, 4), (_problem(62, 2, 2, 2500, 128, gpu), 7, 9)]
    want = [binding.prefill(*qkv, g, k, out_dtype=torch.float32) for qkv, g, k in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [[], []]
    for _ in range(3):
        for i, (qkv, g, k) in enumerate(probs):
            with torch.cuda.stream(streams[i]):
                got[i].append(binding.prefill(*qkv, g, k, out_dtype=torch.float32))
    torch.cuda.synchronize()
    for i in range(2):
        for o in got[i]:
            assert torch.equal(o, want[i])


def _decode_run(cache_args, prefix, steps, device, stream=None):
    q, k, v = prefix
    L0 = q.shape[2] - steps
    B, H, d, g, kl = cache_args
    cache = binding.KVCache(B, H, d, g, kl, max_tokens=L0 + steps, dtype=TDT, device=device)
    kc, vc = binding.pool_kv(q[:, :, :L0].contiguous(), k[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(), g)
    cache.load_prefill(k[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(), kc, vc)
    xs = [[x[:, :, t].contiguous() for x in (q, k, v)] for t in range(L0, L0 + steps)]
    return cache, xs


def test_decode_on_two_streams(gpu):
    _say("fused decode on two streams")
    specs = [((2, 3, 128, 16, 2), _problem(63, 2, 3, 340, 128, gpu)), ((1, 4, 128, 8, 3), _problem(64, 1, 4, 300, 128, gpu))]
    steps = 40
    want = []
    for args, prob in specs:
        cache, xs = _decode_run(args, prob, steps, gpu)
        want.append([cache.append_decode(*x, out_dtype=torch.float32) for x in xs])
    torch.cuda.synchronize()
    runs = [_decode_run(args, prob, steps, gpu) for args, prob in specs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [[], []]
    for s in range(steps):
        for i, (cache, xs) in enumerate(runs):
            with torch.cuda.stream(streams[i]):
                got[i].append(cache.append_decode(*xs[s], out_dtype=torch.float32))
    torch.cuda.synchronize()
    for i in range(2):
        for a, b in zip(got[i], want[i]):
            assert torch.equal(a, b)


def _serve_cache(lca, lens0, device, seed):
    B, Hq, Hkv, d, g, k = len(lens0), 8, 2, 128, 16, 2
    total = max(lens0) + 64
    Q = np_inputs(B, Hq, total, d, "bf16", seed)[0]
    _, K, V = np_inputs(B, Hkv, total, d, "bf16", seed + 1)
    mk = binding.LCAServeCache if lca else binding.ServeCache
    args = (B, Hq, Hkv, d, g, k, total)
    cache = mk(*args, 64, dtype=TDT, device=device) if lca else mk(*args, dtype=TDT, device=device)
    for b, L in enumerate(lens0):
        if L == 0:
            continue
        qb, kb, vb = (_dev(x[b:b + 1, :, :L], device) for x in (Q, K, V))
        if lca:
            kc, vc, _ = binding.pool_kv_lca(qb, kb, vb, g, 64)
            cache.load_sequence(b, qb, kb, vb, kc, vc)
        else:
            kc, vc = binding.pool_kv(qb, kb, vb, g)
            cache.load_sequence(b, kb, vb, kc, vc)
    steps = [[_dev(np.stack([X[b, :, lens0[b] + s] for b in range(B)]), device) for X in (Q, K, V)]
             for s in range(30)]
    return cache, steps


@pytest.mark.parametrize("lca", [False, True], ids=["cca", "lca"])
def test_serving_on_two_streams(gpu, lca):
    _say(f"serving on two streams ({'lca' if lca else 'cca'})")
    specs = [([150, 37, 0], 71), ([90, 260], 73)]
    want, want_caches = [], []
    for lens0, seed in specs:
        cache, steps = _serve_cache(lca, lens0, gpu, seed)
        want.append([cache.step(*x, out_dtype=torch.float32) for x in steps])
        want_caches.append(cache)
    torch.cuda.synchronize()
    runs = [_serve_cache(lca, lens0, gpu, seed) for lens0, seed in specs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [[], []]
    for s in range(30):
        for i, (cache, steps) in enumerate(runs):
            with torch.cuda.stream(streams[i]):
                got[i].append(cache.step(*steps[s], out_dtype=torch.float32))
    torch.cuda.synchronize()
    for i in range(2):
        for a, b in zip(got[i], want[i]):
            assert torch.equal(a, b)
        names = ["core_k", "core_v", "ring_k", "ring_v", "lens"] + (["qsum"] if lca else [])
        for nm in names:
            assert torch.equal(getattr(runs[i][0], nm), getattr(want_caches[i], nm)), nm
