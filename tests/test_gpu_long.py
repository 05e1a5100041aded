"""Sequences beyond the pages' 128K: a 1M-token prefill, decode at 1M context and a 1M-token
backward, on sampled outputs.

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


def test_backward_1m_tokens_sampled(gpu):
    """Training at L = 2^20 (H = 2, bf16): the full backward on the GPU, then sampled dQ rows
    (early, middle and last rows, a group's last row) and dK/dV keys in the last 2048
    positions (raw keys, keys of the last complete groups) of head 1 against the per-entry
    gradient oracle, which evaluates only the queries those entries depend on.  Bound: the
    bf16 gradient bound of the 32K backward test, 2e-2 of the sampled gradients' scale."""
    from oracle import cca_backward
    H = 2
    L = L1M
    _say(f"backward L={L} H={H}")
    q, k, v = torch_inputs(1, H, L, D, torch.bfloat16, gpu, seed=5, heavy_frac=0.01)
    gen = torch.Generator(device=gpu)
    gen.manual_seed(6)
    do = torch.randn((1, H, L, D), generator=gen, device=gpu).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(D)
    out, lse, kc, vc = binding.prefill_lse(q, k, v, G, KL, scale)
    dq, dk, dv = binding.backward(q, k, v, kc, vc, out, lse, do, G, KL, scale)
    torch.cuda.synchronize()
    h = 1
    rows = [0, 1, G, KL * G, L // 2 + 3, L - 2 * G - 2, L - G - 1, L - 2, L - 1]
    keys = [L - 2048, L - (KL + 1) * G, L - 2 * G - 1, L - G - 1, L - G, L - 2, L - 1]
    _say("backward L=1M: oracle on sampled entries")
    wq, wk, wv = cca_backward.cca_backward_sampled_slice(
        q[0, h].double().cpu().numpy(), k[0, h].double().cpu().numpy(), v[0, h].double().cpu().numpy(),
        do[0, h].double().cpu().numpy(), G, KL, scale, rows, keys, core_dtype="bf16")
    got = (dq[0, h, rows].cpu().numpy(), dk[0, h, keys].cpu().numpy(), dv[0, h, keys].cpu().numpy())
    for name, g_, ref in zip(("dq", "dk", "dv"), got, (wq, wk, wv)):
        err = np.abs(g_.astype(np.float64) - ref).max()
        bound = 2e-2 * max(1.0, np.abs(ref).max())
        _say(f"  {name}: max abs err {err:.3e} (bound {bound:.3e})")
        assert np.isfinite(err) and err <= bound, f"{name}: max abs err {err:.3e} > {bound:.3e}"


def test_serving_at_1m_context(gpu):
    """The serving cache (per-sequence lengths, grouped-query heads) past the pages' lengths:
    two sequences at 2^20 - 5 and 2^19 + 7 tokens, 8 query heads over 2 key/value heads,
    seeded by grouped-query pooling of each prefix, then 20 single-token steps (each sequence
    completes a group during them) and one chunked append of 256 tokens.  For one key/value
    head per sequence the oracle computes the rows at the appended positions from the whole
    sequence (stored-core reading); bound 2e-2."""
    from oracle import cca_serving
    B, HQ, HKV, S, N_EXT = 2, 8, 2, 20, 256
    R = HQ // HKV
    lens0 = [L1M - 5, L1M // 2 + 7]
    scale = 1.0 / math.sqrt(D)
    _say(f"serving at 1M context: lengths {lens0}, {HQ} query heads over {HKV}")
    cache = binding.ServeCache(B, HQ, HKV, D, G, KL, max(lens0) + S + N_EXT + G, dtype=torch.bfloat16, device=gpu)
    prefix = []
    for b, L in enumerate(lens0):
        q, _, _ = torch_inputs(1, HQ, L, D, torch.bfloat16, gpu, seed=60 + b, heavy_frac=0.01)
        _, k, v = torch_inputs(1, HKV, L, D, torch.bfloat16, gpu, seed=70 + b, heavy_frac=0.01)
        kc, vc = binding.pool_kv(q, k, v, G, scale)
        cache.load_sequence(b, k, v, kc, vc)
        prefix.append((q, k, v))
        del kc, vc
    gen = torch.Generator(device=gpu)
    gen.manual_seed(80)
    qs = torch.randn((S, B, HQ, D), generator=gen, device=gpu).to(torch.bfloat16)
    ks = torch.randn((S, B, HKV, D), generator=gen, device=gpu).to(torch.bfloat16)
    vs = torch.randn((S, B, HKV, D), generator=gen, device=gpu).to(torch.bfloat16)
    outs = torch.empty((S, B, HQ, D), dtype=torch.float32, device=gpu)
    for s in range(S):
        cache.step(qs[s], ks[s], vs[s], out_dtype=torch.float32, out=outs[s], scale=scale)
    qe = torch.randn((B, HQ, N_EXT, D), generator=gen, device=gpu).to(torch.bfloat16)
    ke = torch.randn((B, HKV, N_EXT, D), generator=gen, device=gpu).to(torch.bfloat16)
    ve = torch.randn((B, HKV, N_EXT, D), generator=gen, device=gpu).to(torch.bfloat16)
    ext = cache.extend(qe, ke, ve, out_dtype=torch.float32, scale=scale)
    torch.cuda.synchronize()
    assert cache.lens.cpu().tolist() == [L + S + N_EXT for L in lens0]
    ext_rows = [0, 1, G - 1, N_EXT // 2, N_EXT - 1]
    for (b, hk) in [(0, 1), (1, 0)]:
        heads = slice(hk * R, (hk + 1) * R)
        q, k, v = prefix[b]
        L = lens0[b]
        Q = torch.cat([q[0, heads], qs[:, b, heads].permute(1, 0, 2), qe[b, heads]], dim=1).double().cpu().numpy()
        K = torch.cat([k[0, hk:hk + 1], ks[:, b, hk:hk + 1].permute(1, 0, 2), ke[b, hk:hk + 1]], dim=1)
        V = torch.cat([v[0, hk:hk + 1], vs[:, b, hk:hk + 1].permute(1, 0, 2), ve[b, hk:hk + 1]], dim=1)
        K, V = K.double().cpu().numpy(), V.double().cpu().numpy()
        pos = [L + s for s in range(S)] + [L + S + i for i in ext_rows]
        want = cca_serving.serve_rows(Q, K, V, pos, G, KL, scale, core_dtype="bf16")
        got_steps = outs[:, b, heads].permute(1, 0, 2).cpu().numpy()
        got_ext = ext[b, heads][:, ext_rows].cpu().numpy()
        err_s = np.abs(got_steps - want[:, :S]).max()
        err_e = np.abs(got_ext - want[:, S:]).max()
        _say(f"serving at 1M (b={b}, kv head {hk}): steps err {err_s:.2e}, chunked append err {err_e:.2e}")
        assert np.isfinite(err_s) and err_s <= TOL_BF16, f"steps: max abs err {err_s:.3e}"
        assert np.isfinite(err_e) and err_e <= TOL_BF16, f"chunked append: max abs err {err_e:.3e}"
