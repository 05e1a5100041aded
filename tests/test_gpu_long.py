"""Sequences beyond the pages' 128K: a 1M-token prefill and decode at 1M context, on sampled outputs.

The pages evaluate CCA up to 128K tokens; these cases check that nothing in the
indexing (positions, tile and group counts, cache offsets) depends on staying
there.  Inputs are drawn on the GPU (seeded, 1% heavy-hitter keys x4, bf16); the
sampled heads are copied back so the oracle sees the GPU's exact inputs.  Parity
is against core tokens stored in bf16; the bound is the bf16 tolerance 2e-2.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_cca_amd import binding
from long_context_sparse_cca_amd.synth import torch_inputs

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
D, G, KL = 128, 16, 64
L1M = 1 << 20


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_prefill_1m_tokens_sampled(gpu):
    H = 4
    _say(f"prefill L={L1M} H={H}")
    q, k, v = torch_inputs(1, H, L1M, D, torch.bfloat16, gpu, seed=3, heavy_frac=0.01)
    out = binding.prefill(q, k, v, G, KL, out_dtype=torch.float32)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(D)
    rng = np.random.default_rng(11)
    for h in (0, H - 1):
        Q = q[0, h].float().cpu().numpy().astype(np.float64)
        K = k[0, h].float().cpu().numpy().astype(np.float64)
        V = v[0, h].float().cpu().numpy().astype(np.float64)
        Kc, Vc, _ = oracle.pool(Q, K, V, G, scale, core_dtype="bf16")
        rows = sorted({0, KL * G, L1M // 2, L1M - G, L1M - 1, *rng.integers(0, L1M, size=12).tolist()})
        got = out[0, h, rows].cpu().numpy()
        for i, t in enumerate(rows):
            want = oracle.cca_row(Q[t], t, K, V, Kc, Vc, G, KL, scale)
            err = np.abs(got[i] - want).max()
            assert err <= TOL_BF16, f"head {h} row {t}: max abs err {err:.3e}"


def test_decode_at_1m_context(gpu):
    B, H, S = 1, 2, 20
    L0 = L1M - 7                       # the prefix ends inside a group; a group completes during the steps
    _say(f"decode at context {L0} B={B} H={H}, {S} steps")
    q, k, v = torch_inputs(B, H, L0 + S, D, torch.bfloat16, gpu, seed=4, heavy_frac=0.01)
    pre = [x[:, :, :L0].contiguous() for x in (q, k, v)]
    kc, vc = binding.pool_kv(*pre, G)
    cache = binding.KVCache(B, H, D, G, KL, max_tokens=L0 + S, dtype=torch.bfloat16, device=gpu)
    cache.load_prefill(pre[1], pre[2], kc, vc)
    del pre
    outs = [cache.append_decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                                out_dtype=torch.float32) for t in range(L0, L0 + S)]
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(D)
    for h in range(H):
        Q = q[0, h].float().cpu().numpy().astype(np.float64)
        K = k[0, h].float().cpu().numpy().astype(np.float64)
        V = v[0, h].float().cpu().numpy().astype(np.float64)
        Kc, Vc, _ = oracle.pool(Q, K, V, G, scale, core_dtype="bf16")
        for i, t in enumerate(range(L0, L0 + S)):
            want = oracle.cca_row(Q[t], t, K, V, Kc, Vc, G, KL, scale)
            err = np.abs(outs[i][0, h].cpu().numpy() - want).max()
            assert err <= TOL_BF16, f"head {h} step {t}: max abs err {err:.3e}"
