"""The allocation-free fused decode (cca_cache_append_decode_noalloc) against the
workspace form (cca_cache_append_decode), through the C ABI.

The no-alloc call keeps the chunk partial states in the library's per-GPU device
array, so consecutive calls of different shapes reuse memory that still holds the
previous call's states.  Each case drives two caches with the same tokens, one per
entry point, and requires equal outputs and caches bit for bit (the same kernels run
on the same inputs).  The larger shape runs first, then a smaller one.
"""
import math

import numpy as np
import pytest
import torch

from long_context_sparse_cca_amd import binding
from long_context_sparse_cca_amd.synth import np_inputs, torch_inputs

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _dev(x, dt, device):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=TDT[dt]).contiguous()


def _run_pair(device, B, H, d, g, k, L0, S, dt, seed, out_dtype, on_gpu=False):
    """Seed two caches with a prefill of L0 tokens, then S steps through each entry point
    (inputs drawn on the GPU for the long context)."""
    L = L0 + S
    if on_gpu:
        q, kk, v = torch_inputs(B, H, L, d, TDT[dt], device, seed=seed, heavy_frac=0.01)
    else:
        q, kk, v = (_dev(x, dt, device) for x in np_inputs(B, H, L, d, dt, seed))
    scale = 1.0 / math.sqrt(d)
    caches = [binding.KVCache(B, H, d, g, k, max_tokens=L, dtype=TDT[dt], device=device) for _ in range(2)]
    if L0 > 0:
        pre = [x[:, :, :L0].contiguous() for x in (q, kk, v)]
        kc, vc = binding.pool_kv(*pre, g, scale)
        for c in caches:
            c.load_prefill(pre[1], pre[2], kc, vc)
    ref = torch.empty((S, B, H, d), dtype=out_dtype, device=device)
    got = torch.full((S, B, H, d), float("nan"), dtype=out_dtype, device=device)
    for s in range(S):
        t = L0 + s
        x = [y[:, :, t].contiguous() for y in (q, kk, v)]
        caches[0].append_decode(*x, out_dtype=out_dtype, out=ref[s], scale=scale)
        caches[1].append_decode_noalloc(*x, out=got[s], out_dtype=out_dtype, scale=scale)
    torch.cuda.synchronize()
    assert caches[0].n_tokens == caches[1].n_tokens == L
    assert torch.equal(ref, got), f"outputs differ: max {float((ref.float() - got.float()).abs().max()):.3e}"
    for name in ("core_k", "core_v", "ring_k", "ring_v"):
        assert torch.equal(getattr(caches[0], name), getattr(caches[1], name)), f"{name} differs"
    return ref


def test_noalloc_matches_workspace_call_large_then_small(gpu):
    # first: 32 slices at d = 128, bf16, 4 chunks per slice, pooling steps inside
    _run_pair(gpu, B=4, H=8, d=128, g=16, k=2, L0=300, S=40, dt="bf16", seed=90, out_dtype=torch.float32)
    # then a smaller call: 2 slices at d = 64, float32, from an empty cache (fewer chunk records
    # than the first call left behind in the shared array)
    _run_pair(gpu, B=1, H=2, d=64, g=8, k=1, L0=0, S=30, dt="f32", seed=91, out_dtype=torch.float32)


def test_noalloc_16bit_output_and_context_at_scale(gpu):
    """bf16 output, a long context (streaming loads: more than 384 MiB of K/V per step)."""
    _run_pair(gpu, B=3, H=32, d=128, g=16, k=64, L0=131072, S=20, dt="bf16", seed=92, out_dtype=torch.bfloat16,
              on_gpu=True)
    _run_pair(gpu, B=1, H=4, d=128, g=16, k=4, L0=1000, S=20, dt="f16", seed=93, out_dtype=torch.float16)


def test_noalloc_rejects_states_beyond_the_array(gpu):
    """B*H*chunks*(d+2)*4 bytes above 4 MiB is refused before any launch; the cache is untouched."""
    B, H, d, g, k = 128, 64, 128, 16, 1
    cache = binding.KVCache(B, H, d, g, k, max_tokens=g, dtype=torch.bfloat16, device=gpu)
    assert cache.ws_bytes > 4 << 20
    x = torch.zeros((B, H, d), dtype=torch.bfloat16, device=gpu)
    out = torch.empty_like(x)
    with pytest.raises(binding.CCAError, match="workspace"):
        cache.append_decode_noalloc(x, x, x, out=out)
    assert cache.n_tokens == 0
