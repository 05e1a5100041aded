"""Determinism and out-of-bounds guards beyond the prefill (the prefill's own are in
test_gpu_parity.py): decode, serving and backward.

Determinism: every kernel on these paths writes each output element from one place (split
partial states merged in a fixed order, no atomics), so two runs on the same inputs must agree
bit for bit.  Guards: the cache buffers, workspaces and outputs are views into larger buffers
filled with a sentinel; after the calls the sentinel regions must be untouched.
"""
import math

import numpy as np
import pytest
import torch

from long_context_sparse_cca_amd import binding
from long_context_sparse_cca_amd.synth import np_inputs

pytestmark = pytest.mark.gpu

PAD = 4096


def _dev(x, dtype, device):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dtype).contiguous()


def _guarded(shape, dtype, device, fill):
    """A view of `shape` inside a buffer padded with PAD sentinel elements on both sides."""
    n = int(np.prod(shape))
    big = torch.full((n + 2 * PAD,), fill, dtype=dtype, device=device)
    return big, big[PAD:PAD + n].view(shape)


def _intact(big, fill):
    return bool(torch.all(big[:PAD] == fill)) and bool(torch.all(big[-PAD:] == fill))


def _guard_cache(cache, device):
    """Move a cache's buffers and workspace into guarded allocations (descriptor pointers updated)."""
    bigs = []
    for name, fill in (("core_k", -3.0), ("core_v", -5.0), ("ring_k", 7.0), ("ring_v", 9.0)):
        t = getattr(cache, name)
        big, view = _guarded(tuple(t.shape), t.dtype, device, fill)
        view.copy_(t)
        setattr(cache, name, view)
        setattr(cache.desc, name, view.data_ptr())
        bigs.append((big, fill))
    big, view = _guarded(tuple(cache.workspace.shape), torch.float32, device, 1234.5)
    cache.workspace = view
    bigs.append((big, 1234.5))
    return bigs


def _decode_run(device, guard):
    B, H, d, g, k, L0, S = 2, 3, 128, 16, 2, 200, 40
    Q, K, V = np_inputs(B, H, L0 + S, d, "bf16", 81)
    q, kk, v = (_dev(x, torch.bfloat16, device) for x in (Q, K, V))
    scale = 1.0 / math.sqrt(d)
    cache = binding.KVCache(B, H, d, g, k, max_tokens=L0 + S, dtype=torch.bfloat16, device=device)
    kc, vc = binding.pool_kv(q[:, :, :L0].contiguous(), kk[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(), g,
                             scale)
    bigs = _guard_cache(cache, device) if guard else []
    cache.load_prefill(kk[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(), kc, vc)
    obig, outs = _guarded((S, B, H, d), torch.float32, device, 77.0)
    for s in range(S):
        t = L0 + s
        cache.append_decode(*(x[:, :, t].contiguous() for x in (q, kk, v)), out_dtype=torch.float32, out=outs[s],
                            scale=scale)
    torch.cuda.synchronize()
    return outs.clone(), cache, bigs + [(obig, 77.0)]


def test_decode_deterministic_and_in_bounds(gpu):
    a, ca, bigs = _decode_run(gpu, guard=True)
    b, cb, _ = _decode_run(gpu, guard=False)
    assert torch.equal(a, b)
    for name in ("core_k", "core_v", "ring_k", "ring_v"):
        assert torch.equal(getattr(ca, name), getattr(cb, name)), name
    for big, fill in bigs:
        assert _intact(big, fill)


def _serve_run(device):
    B, Hq, Hkv, d, g, k, T = 3, 8, 2, 128, 16, 2, 30
    lens0 = [150, 37, 0]
    Q = np_inputs(B, Hq, max(lens0) + T, d, "bf16", 82)[0]
    _, K, V = np_inputs(B, Hkv, max(lens0) + T, d, "bf16", 83)
    scale = 1.0 / math.sqrt(d)
    cache = binding.ServeCache(B, Hq, Hkv, d, g, k, max(lens0) + T + g, dtype=torch.bfloat16, device=device)
    for b, L in enumerate(lens0):
        if L == 0:
            continue
        qb, kb, vb = (_dev(x[b:b + 1, :, :L], torch.bfloat16, device) for x in (Q, K, V))
        kc, vc = binding.pool_kv(qb, kb, vb, g, scale)
        cache.load_sequence(b, kb, vb, kc, vc)
    wbig, ws = _guarded(tuple(cache.serve_ws.shape), torch.float32, device, 4321.0)
    cache.serve_ws = ws
    obig, outs = _guarded((T, B, Hq, d), torch.float32, device, 55.0)
    for i in range(T):
        pos = [L + i for L in lens0]
        q, kk, v = (_dev(np.stack([X[b, :, pos[b]] for b in range(B)]), torch.bfloat16, device) for X in (Q, K, V))
        cache.step(q, kk, v, out_dtype=torch.float32, out=outs[i], scale=scale)
    torch.cuda.synchronize()
    return outs.clone(), cache, [(wbig, 4321.0), (obig, 55.0)]


def test_serving_deterministic_and_in_bounds(gpu):
    a, ca, bigs = _serve_run(gpu)
    b, cb, _ = _serve_run(gpu)
    assert torch.equal(a, b)
    assert torch.equal(ca.core_k, cb.core_k) and torch.equal(ca.ring_v, cb.ring_v)
    for big, fill in bigs:
        assert _intact(big, fill)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_deterministic(gpu, dt):
    """The matrix-core backward (bf16, d = 128) and the vector one (float32, d = 64)."""
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    d = 128 if dt == "bf16" else 64
    B, H, L, g, k = 1, 2, 700, 16, 3
    Q, K, V = np_inputs(B, H, L, d, dt, 84)
    dO = np_inputs(B, H, L, d, dt, 85)[0]
    q, kk, v, do = (_dev(x, tdt, gpu) for x in (Q, K, V, dO))
    runs = []
    for _ in range(2):
        out, lse, kc, vc = binding.prefill_lse(q, kk, v, g, k)
        runs.append(binding.backward(q, kk, v, kc, vc, out, lse, do, g, k))
    torch.cuda.synchronize()
    for x, y in zip(*runs):
        assert torch.equal(x, y)
