"""Grouped-query CCA prefill (H query heads over H_kv key/value heads): HIP path vs the oracle.

Small shapes spanning several query tiles and key tiles with ragged tails, r = H/H_kv in
{2, 3, 4, 8}, MQA (H_kv = 1), fp32 and bf16, the bf16 d=128 fast kernels and the generic
ones; then a full-size bf16 layer (L = 32768, H = 32, H_kv = 8) on sampled rows.
Tolerances (max-abs): fp32 1e-4, bf16 2e-2.  The oracle stores core tokens in the input
dtype (one rounding of the exact core token).
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import cca_serving
from long_context_sparse_cca_amd import binding
from long_context_sparse_cca_amd.synth import np_inputs, torch_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 5e-3}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _dev(x, dt, device):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=TDT[dt]).contiguous()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# (B, H, H_kv, L, d, g, k, dtype, seed)
GQA_CASES = [
    (1, 4, 2, 300, 64, 16, 1, "f32", 20),
    (2, 6, 2, 517, 64, 7, 3, "bf16", 21),     # r = 3, ragged group, generic bf16 kernels
    (1, 8, 2, 1000, 128, 16, 4, "bf16", 22),  # r = 4, fast kernels, ragged tiles
    (1, 8, 1, 700, 128, 16, 2, "bf16", 23),   # MQA
    (1, 8, 8, 400, 128, 16, 2, "bf16", 24),   # r = 1 through the grouped-query entry points' path
    (1, 4, 1, 333, 128, 8, 5, "f32", 25),     # fp32, g = 8
    (1, 16, 2, 1300, 128, 16, 64, "bf16", 26),  # r = 8, window wider than most of the sequence
]


def _id(c):
    B, H, Hkv, L, d, g, k, dt, seed = c
    return f"B{B}H{H}kv{Hkv}L{L}d{d}g{g}k{k}-{dt}"


def _gqa_inputs(B, H, Hkv, L, d, dt, seed):
    Q, _, _ = np_inputs(B, H, L, d, dt, seed)
    _, K, V = np_inputs(B, Hkv, L, d, dt, seed + 1000)
    return Q, K, V


@pytest.mark.parametrize("case", GQA_CASES, ids=_id)
def test_gqa_prefill_matches_oracle(gpu, case):
    B, H, Hkv, L, d, g, k, dt, seed = case
    _say(f"gqa prefill case {_id(case)} seed {seed}")
    Q, K, V = _gqa_inputs(B, H, Hkv, L, d, dt, seed)
    q, kk, v = (_dev(x, dt, gpu) for x in (Q, K, V))
    scale = 1.0 / math.sqrt(d)
    out, kc, vc = binding.prefill(q, kk, v, g, k, scale, out_dtype=torch.float32, return_core=True)
    torch.cuda.synchronize()
    want = cca_serving.cca_gqa(Q, K, V, g, k, scale, core_dtype=dt)
    err = np.abs(out.cpu().numpy().astype(np.float64) - want).max()
    assert np.isfinite(err) and err <= TOL[dt], f"max abs err {err:.3e}"
    # core tokens of every key/value head: pooled once with the mean query of its r heads
    r = H // Hkv
    m = L // g
    ulp = 2.0 ** -8 if dt == "bf16" else 2.0 ** -22
    if m:
        for b in range(B):
            for hk in range(Hkv):
                Kc, Vc, _ = cca_serving.pool_gqa(Q[b, hk * r:(hk + 1) * r], K[b, hk], V[b, hk], g, scale)
                for got, ref in ((kc[b, hk], Kc), (vc[b, hk], Vc)):
                    got = got.float().cpu().numpy()
                    assert np.all(np.abs(got - ref) <= TOL[dt] + ulp * np.abs(ref)), \
                        f"core err {np.abs(got - ref).max():.3e}"
    # the attention step alone on the same core tokens gives the same output, bit for bit
    again = binding.attention(q, kk, v, kc, vc, g, k, scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(again, out)


def test_gqa_invalid_head_counts(gpu):
    q = torch.zeros((1, 6, 32, 64), dtype=torch.float32, device=gpu)
    k = torch.zeros((1, 4, 32, 64), dtype=torch.float32, device=gpu)
    with pytest.raises(binding.CCAError):
        binding.prefill(q, k, k.clone(), 16, 1)


def test_gqa_fullsize_sampled(gpu):
    """One bf16 layer at L = 32768, H = 32, H_kv = 8, g = 16, k = 64 on the fast kernels: sampled rows."""
    B, H, Hkv, L, d, g, k = 1, 32, 8, 32768, 128, 16, 64
    _say(f"gqa full size B{B} H{H} H_kv{Hkv} L{L}")
    q, _, _ = torch_inputs(B, H, L, d, torch.bfloat16, gpu, seed=5, heavy_frac=0.01)
    _, kk, v = torch_inputs(B, Hkv, L, d, torch.bfloat16, gpu, seed=6, heavy_frac=0.01)
    scale = 1.0 / math.sqrt(d)
    out, kc, vc = binding.prefill(q, kk, v, g, k, scale, out_dtype=torch.float32, return_core=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    pos = sorted(set([0, 15, 16, 1039, 1040, L - 1] + rng.integers(0, L, 26).tolist()))
    Qn = q[0].float().cpu().numpy()
    Kn = kk[0].float().cpu().numpy()
    Vn = v[0].float().cpu().numpy()
    for hk in (0, 5):
        heads = list(range(hk * 4, hk * 4 + 4))
        sub_q = Qn[heads]
        want = cca_serving.serve_rows(sub_q, Kn[hk:hk + 1], Vn[hk:hk + 1], pos, g, k, scale, core_dtype="bf16")
        got = out[0, heads][:, pos].cpu().numpy()
        err = np.abs(got - want).max()
        _say(f"  kv head {hk}: max err {err:.3e} over {len(pos)} rows x 4 heads")
        assert np.isfinite(err) and err <= TOL["bf16"], f"kv head {hk}: max abs err {err:.3e}"
