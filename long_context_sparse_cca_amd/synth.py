"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the attention arithmetic.

Distribution (stands in for LLaMA2-7B long-context attention inputs, whose
weights and datasets are not available): Q, K, V i.i.d. N(0, 1); optionally a
fraction of key positions per (batch, head), chosen uniformly without
replacement, has its K row scaled by 4 ("heavy hitters", mimicking the sparse
attention maps the CCA write-up shows for LLaMA2-7B in its Fig. 1).  Values are
then rounded to the storage dtype with round-to-nearest-even.
"""

from __future__ import annotations

import numpy as np

HEAVY_SCALE = 4.0


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    r = ((u + bias) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def np_inputs(B: int, H: int, L: int, d: int, dtype: str = "f32", seed: int = 0,
              heavy_frac: float = 0.0, tensor_ids=(0, 1, 2)):
    """Q, K, V as float32 numpy arrays [B, H, L, d] whose values are exact in `dtype`.

    Each tensor comes from its own PCG64 stream seeded with (seed, tensor_id).
    """
    out = []
    for tid in tensor_ids:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid])))
        out.append(rng.standard_normal((B, H, L, d)).astype(np.float32))
    Q, K, V = out
    if heavy_frac > 0.0:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
        n = max(1, int(round(heavy_frac * L)))
        for b in range(B):
            for h in range(H):
                idx = rng.choice(L, size=n, replace=False)
                K[b, h, idx] *= np.float32(HEAVY_SCALE)
    if dtype == "bf16":
        Q, K, V = round_to_bf16(Q), round_to_bf16(K), round_to_bf16(V)
    elif dtype == "f16":
        Q, K, V = (x.astype(np.float16).astype(np.float32) for x in (Q, K, V))
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype}")
    return Q, K, V


def torch_inputs(B: int, H: int, L: int, d: int, dtype, device, seed: int = 0,
                 heavy_frac: float = 0.0):
    """Q, K, V as device tensors [B, H, L, d] of `dtype`, drawn on `device`.

    Drawn one batch row at a time in float32 and rounded (RNE) to `dtype`, so
    the peak extra memory is one [H, L, d] float32 slab.
    """
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    tensors = []
    for _ in range(3):
        tensors.append(torch.empty((B, H, L, d), dtype=dtype, device=device))
    Q, K, V = tensors
    n = max(1, int(round(heavy_frac * L))) if heavy_frac > 0.0 else 0
    for b in range(B):
        for t in (Q, K, V):
            x = torch.randn((H, L, d), generator=gen, device=device, dtype=torch.float32)
            if t is K and n > 0:
                order = torch.rand((H, L), generator=gen, device=device).argsort(dim=-1)
                sel = order[:, :n]
                scale = torch.ones((H, L), device=device, dtype=torch.float32)
                scale.scatter_(1, sel, HEAVY_SCALE)
                x.mul_(scale.unsqueeze(-1))
            t[b].copy_(x)
            del x
    return Q, K, V
