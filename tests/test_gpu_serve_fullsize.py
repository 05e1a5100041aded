"""The serving workload the benchmark times, at its full size, on sampled outputs.

B = 8 sequences at 65536 + 9362*b tokens, 32 query heads over 8 key/value heads (r = 4),
d = 128, g = 16, k = 64, bf16: the same cache, launch shapes and kernels as the benchmark's
serving leg (4 query heads per workgroup, 16 chunks per key/value slice, ordinary loads).
Each sequence is seeded from its own grouped-query pooling, then 24 single-token steps
(every sequence completes at least one group, so the fused pooling runs) and one chunked
append of 512 tokens per sequence.  For sampled (sequence, key/value head) pairs the oracle
takes the whole sequence of that key/value head and its 4 query heads (GPU inputs copied
back) and computes the rows at the appended positions (stored-core reading: core tokens
rounded once to bf16).  Bound: 2e-2 max-abs, as for every bf16 output.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import cca_serving
from long_context_sparse_cca_amd import binding
from long_context_sparse_cca_amd.synth import torch_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2
B, HQ, HKV, D, G, KL = 8, 32, 8, 128, 16, 64
R = HQ // HKV
S, N_EXT = 24, 512


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_serving_fullsize_sampled(gpu):
    lens0 = [65536 + 9362 * b for b in range(B)]
    scale = 1.0 / math.sqrt(D)
    _say("serving full size: seeding 8 sequences (64K..128K)")
    cache = binding.ServeCache(B, HQ, HKV, D, G, KL, max(lens0) + S + N_EXT + G, dtype=torch.bfloat16, device=gpu)
    prefix = []
    for b, L in enumerate(lens0):
        q, _, _ = torch_inputs(1, HQ, L, D, torch.bfloat16, gpu, seed=110 + b, heavy_frac=0.01)
        _, k, v = torch_inputs(1, HKV, L, D, torch.bfloat16, gpu, seed=130 + b, heavy_frac=0.01)
        kc, vc = binding.pool_kv(q, k, v, G, scale)
        cache.load_sequence(b, k, v, kc, vc)
        prefix.append((q, k, v))
        del kc, vc
    gen = torch.Generator(device=gpu)
    gen.manual_seed(150)
    qs = torch.randn((S, B, HQ, D), generator=gen, device=gpu).to(torch.bfloat16)
    ks = torch.randn((S, B, HKV, D), generator=gen, device=gpu).to(torch.bfloat16)
    vs = torch.randn((S, B, HKV, D), generator=gen, device=gpu).to(torch.bfloat16)
    _say("serving full size: stepping")
    outs = torch.empty((S, B, HQ, D), dtype=torch.float32, device=gpu)
    for s in range(S):
        cache.step(qs[s], ks[s], vs[s], out_dtype=torch.float32, out=outs[s], scale=scale)
    qe = torch.randn((B, HQ, N_EXT, D), generator=gen, device=gpu).to(torch.bfloat16)
    ke = torch.randn((B, HKV, N_EXT, D), generator=gen, device=gpu).to(torch.bfloat16)
    ve = torch.randn((B, HKV, N_EXT, D), generator=gen, device=gpu).to(torch.bfloat16)
    _say("serving full size: chunked append")
    ext = cache.extend(qe, ke, ve, out_dtype=torch.float32, scale=scale)
    torch.cuda.synchronize()
    assert cache.lens.cpu().tolist() == [L + S + N_EXT for L in lens0]
    rng = np.random.default_rng(9)
    ext_rows = sorted({0, 1, G - 1, N_EXT // 2, N_EXT - 1, *rng.integers(0, N_EXT, 8).tolist()})
    for (b, hk) in [(0, 0), (3, 5), (B - 1, HKV - 1)]:
        heads = slice(hk * R, (hk + 1) * R)
        q, k, v = prefix[b]
        L = lens0[b]
        Q = torch.cat([q[0, heads], qs[:, b, heads].permute(1, 0, 2), qe[b, heads]], dim=1).double().cpu().numpy()
        K = torch.cat([k[0, hk:hk + 1], ks[:, b, hk:hk + 1].permute(1, 0, 2), ke[b, hk:hk + 1]], dim=1)
        V = torch.cat([v[0, hk:hk + 1], vs[:, b, hk:hk + 1].permute(1, 0, 2), ve[b, hk:hk + 1]], dim=1)
        K, V = K.double().cpu().numpy(), V.double().cpu().numpy()
        pos = [L + s for s in range(S)] + [L + S + i for i in ext_rows]
        want = cca_serving.serve_rows(Q, K, V, pos, G, KL, scale, core_dtype="bf16")   # [R, len(pos), D]
        got_steps = outs[:, b, heads].permute(1, 0, 2).cpu().numpy()                   # [R, S, D]
        got_ext = ext[b, heads][:, ext_rows].cpu().numpy()                              # [R, rows, D]
        err_s = np.abs(got_steps - want[:, :S]).max()
        err_e = np.abs(got_ext - want[:, S:]).max()
        _say(f"serving full size (b={b}, kv head {hk}): steps err {err_s:.2e}, chunked append err {err_e:.2e}")
        assert np.isfinite(err_s) and err_s <= TOL, f"steps: max abs err {err_s:.3e}"
        assert np.isfinite(err_e) and err_e <= TOL, f"chunked append: max abs err {err_e:.3e}"


def test_lca_serving_fullsize_sampled(gpu):
    """The LCA-style serving leg at full size (d_rope = 64): same workload, LCA-style cache.
    The oracle checks the GPU's anchors against its fp64 scores, condenses every group itself
    at those anchors (mean over the group's positions and the 4 query heads), and computes the
    rows at the appended positions."""
    from oracle import cca_lca, cca_oracle
    d_rope = 64
    lens0 = [65536 + 9362 * b for b in range(B)]
    scale = 1.0 / math.sqrt(D)
    _say("lca serving full size: seeding 8 sequences (64K..128K)")
    cache = binding.LCAServeCache(B, HQ, HKV, D, G, KL, max(lens0) + S + N_EXT + G, d_rope, dtype=torch.bfloat16,
                                  device=gpu)
    prefix = []
    for b, L in enumerate(lens0):
        q, _, _ = torch_inputs(1, HQ, L, D, torch.bfloat16, gpu, seed=210 + b, heavy_frac=0.01)
        _, k, v = torch_inputs(1, HKV, L, D, torch.bfloat16, gpu, seed=230 + b, heavy_frac=0.01)
        kc, vc, _ = binding.pool_kv_lca(q, k, v, G, d_rope, scale)
        cache.load_sequence(b, q, k, v, kc, vc)
        prefix.append((q, k, v))
        del kc, vc
    gen = torch.Generator(device=gpu)
    gen.manual_seed(250)
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
    rng = np.random.default_rng(11)
    ext_rows = sorted({0, G - 1, N_EXT - 1, *rng.integers(0, N_EXT, 6).tolist()})
    dc = D - d_rope
    for (b, hk) in [(1, 2), (B - 2, HKV - 1)]:
        heads = slice(hk * R, (hk + 1) * R)
        q, k, v = prefix[b]
        L = lens0[b]
        T = L + S + N_EXT
        m = T // G
        Q = torch.cat([q[0, heads], qs[:, b, heads].permute(1, 0, 2), qe[b, heads]], dim=1).double().cpu().numpy()
        K = torch.cat([k[0, hk], ks[:, b, hk], ke[b, hk]], dim=0).double().cpu().numpy()
        V = torch.cat([v[0, hk], vs[:, b, hk], ve[b, hk]], dim=0).double().cpu().numpy()
        q_mean = Q.sum(axis=0) / R
        # the GPU's anchors: the group row whose positional dims each condensed key carries
        gk = cache.core_k[b, hk, :m].double().cpu().numpy()
        Kg = K[:m * G].reshape(m, G, D)[:, :, dc:]
        hits = np.all(Kg == gk[:, None, dc:], axis=2)
        assert hits.any(axis=1).all(), "a condensed key's positional dims match no key of its group"
        anc = hits.argmax(axis=1)
        S_sc = cca_lca.lca_scores(q_mean, K, G, scale)
        best = S_sc.max(axis=1)
        picked = S_sc[np.arange(m), anc]
        assert np.all(picked >= best - 1e-5 * np.maximum(1.0, np.abs(S_sc).max(axis=1))), "anchor not a maximum"
        Kc, Vc, _ = cca_lca.lca_pool(q_mean, K, V, G, scale, d_rope, anchors=anc, core_dtype="bf16")
        pos = [L + s for s in range(S)] + [L + S + i for i in ext_rows]
        want = np.stack([[cca_oracle.cca_row(Q[h, p], p, K, V, Kc, Vc, G, KL, scale) for p in pos] for h in range(R)])
        got_steps = outs[:, b, heads].permute(1, 0, 2).cpu().numpy()
        got_ext = ext[b, heads][:, ext_rows].cpu().numpy()
        err_s = np.abs(got_steps - want[:, :S]).max()
        err_e = np.abs(got_ext - want[:, S:]).max()
        _say(f"lca serving full size (b={b}, kv head {hk}): steps err {err_s:.2e}, chunked append err {err_e:.2e}")
        assert np.isfinite(err_s) and err_s <= TOL, f"steps: max abs err {err_s:.3e}"
        assert np.isfinite(err_e) and err_e <= TOL, f"chunked append: max abs err {err_e:.3e}"
