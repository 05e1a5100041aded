"""Serving decode step (per-sequence lengths, grouped-query attention): HIP path vs the oracle.

Each case seeds every sequence of the batch with its own prefix (a GPU prefill of that
prefix, loaded into a one-sequence view of the cache; length 0 = empty sequence), then
appends tokens one step at a time for all sequences at once; every step's outputs are
compared with the oracle's rows at those positions (a token appended at position p has
the prefill output of row p).  Steps cross group boundaries, so the in-place pooling
with the mean query of the heads sharing a key/value head is exercised too.
Tolerances (max-abs): fp32 1e-4, bf16 2e-2 (core tokens stored in the input dtype).
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import cca_serving
from long_context_sparse_cca_amd import binding
from long_context_sparse_cca_amd.synth import np_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 5e-3}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _dev(x, dt, device):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=TDT[dt]).contiguous()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# (B, H_q, H_kv, d, g, k, dtype, initial lengths, steps, seed)
SERVE_CASES = [
    (3, 4, 2, 128, 16, 2, "bf16", [100, 37, 0], 40, 30),
    (2, 8, 1, 128, 16, 64, "bf16", [1500, 1100], 20, 31),   # MQA, r = 8, windows of 1024
    (2, 6, 2, 64, 5, 3, "f32", [0, 23], 30, 32),             # r = 3: three blocks of one head
    (4, 2, 2, 64, 16, 1, "f32", [37, 0, 16, 15], 24, 33),    # r = 1, sequences at group edges
    (2, 12, 2, 128, 16, 4, "bf16", [260, 300], 20, 34),      # r = 6: blocks of two heads
    (2, 16, 4, 128, 16, 8, "bf16", [700, 64], 18, 35),       # r = 4
    (2, 4, 2, 128, 16, 2, "f16", [150, 9], 24, 39),          # binary16 cache
    (3, 3, 1, 64, 5, 3, "f16", [0, 44, 12], 20, 29),         # binary16, d = 64, MQA
    # several chunks per sequence (each cut from its own length): a 3-token sequence has
    # fewer keys than chunks, so some of its chunks are empty
    (2, 4, 2, 128, 16, 64, "bf16", [3, 6000], 20, 36),
]


def _id(c):
    B, Hq, Hkv, d, g, k, dt, lens, T, seed = c
    return f"B{B}Hq{Hq}kv{Hkv}d{d}g{g}k{k}-{dt}-L{'_'.join(map(str, lens))}-T{T}"


def lib_chunks(cache):
    """Chunks per sequence of the library's serving split, from its workspace size (one
    (d + 2)-float partial state per sequence, query head and chunk)."""
    B, _, d = cache.shape_bhd
    return cache.serve_ws_bytes // (B * cache.H_q * (d + 2) * 4)


def _setup(case, device, capacity=None):
    B, Hq, Hkv, d, g, k, dt, lens0, T, seed = case
    total = max(lens0) + T
    Q, _, _ = np_inputs(B, Hq, total, d, dt, seed)
    _, K, V = np_inputs(B, Hkv, total, d, dt, seed + 1000)
    cache = binding.ServeCache(B, Hq, Hkv, d, g, k, capacity or total + g, dtype=TDT[dt], device=device)
    scale = 1.0 / math.sqrt(d)
    for b, L in enumerate(lens0):
        if L == 0:
            continue
        qb, kb, vb = (_dev(x[b:b + 1, :, :L], dt, device) for x in (Q, K, V))
        _, kc, vc = binding.prefill(qb, kb, vb, g, k, scale, return_core=True)
        cache.load_sequence(b, kb, vb, kc, vc)
    return Q, K, V, cache, scale


# (case, cache capacity in tokens): a large cache splits each sequence into many chunks; with
# sequences a few tokens long most of the chunks hold no key
CAPACITY_CASES = [((2, 4, 2, 128, 16, 4, "bf16", [0, 5], 20, 37), 70000),
                  ((3, 2, 1, 64, 16, 2, "f32", [1, 0, 17], 12, 38), 1 << 17)]


def _serve_steps(gpu, case, capacity=None):
    B, Hq, Hkv, d, g, k, dt, lens0, T, seed = case
    _say(f"serve case {_id(case)} seed {seed} capacity {capacity}")
    Q, K, V, cache, scale = _setup(case, gpu, capacity)
    outs = []
    for i in range(T):
        q = _dev(np.stack([Q[b, :, lens0[b] + i] for b in range(B)]), dt, gpu)
        kk = _dev(np.stack([K[b, :, lens0[b] + i] for b in range(B)]), dt, gpu)
        v = _dev(np.stack([V[b, :, lens0[b] + i] for b in range(B)]), dt, gpu)
        outs.append(cache.step(q, kk, v, out_dtype=torch.float32, scale=scale).cpu().numpy())
    torch.cuda.synchronize()
    assert cache.lens.cpu().tolist() == [L + T for L in lens0]
    got = np.stack(outs, axis=2)  # [B, H_q, T, d]
    for b in range(B):
        pos = [lens0[b] + i for i in range(T)]
        want = cca_serving.serve_rows(Q[b], K[b], V[b], pos, g, k, scale, core_dtype=dt)
        err = np.abs(got[b] - want).max()
        assert np.isfinite(err) and err <= TOL[dt], f"sequence {b}: max abs err {err:.3e}"
    return cache


@pytest.mark.parametrize("case", SERVE_CASES, ids=_id)
def test_serve_steps_match_oracle(gpu, case):
    _serve_steps(gpu, case)


@pytest.mark.parametrize("case,capacity", CAPACITY_CASES, ids=lambda c: _id(c) if isinstance(c, tuple) else f"cap{c}")
def test_serve_short_sequences_in_a_large_cache(gpu, case, capacity):
    cache = _serve_steps(gpu, case, capacity)
    nch = lib_chunks(cache)
    assert nch > max(case[7]) + 1, f"only {nch} chunks: the case does not reach empty chunks"


def test_serve_bf16_output_matches_f32_output(gpu):
    case = (2, 8, 2, 128, 16, 2, "bf16", [90, 33], 1, 36)
    B, Hq, Hkv, d, g, k, dt, lens0, T, seed = case
    Q, K, V, cache, scale = _setup(case, gpu)
    q = _dev(np.stack([Q[b, :, lens0[b]] for b in range(B)]), dt, gpu)
    kk = _dev(np.stack([K[b, :, lens0[b]] for b in range(B)]), dt, gpu)
    v = _dev(np.stack([V[b, :, lens0[b]] for b in range(B)]), dt, gpu)
    # same state twice: a second cache seeded identically
    Q2, K2, V2, cache2, _ = _setup(case, gpu)
    o32 = cache.step(q, kk, v, out_dtype=torch.float32, scale=scale)
    o16 = cache2.step(q, kk, v, out_dtype=torch.bfloat16, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16)


def test_serve_out_of_range_length_gives_nan_and_leaves_cache(gpu):
    """A device length beyond max_len (forced from the host) yields NaN for that sequence only."""
    case = (2, 4, 2, 128, 16, 2, "bf16", [60, 70], 1, 37)
    B, Hq, Hkv, d, g, k, dt, lens0, T, seed = case
    Q, K, V, cache, scale = _setup(case, gpu)
    cache.lens[1] = 10 ** 6          # the host still believes 70 (max_len = 70)
    ring_before = cache.ring_k[1].clone()
    core_before = cache.core_k[1].clone()
    q = _dev(np.stack([Q[b, :, lens0[b]] for b in range(B)]), dt, gpu)
    kk = _dev(np.stack([K[b, :, lens0[b]] for b in range(B)]), dt, gpu)
    v = _dev(np.stack([V[b, :, lens0[b]] for b in range(B)]), dt, gpu)
    out = cache.step(q, kk, v, out_dtype=torch.float32, scale=scale)
    torch.cuda.synchronize()
    assert torch.isnan(out[1]).all()
    assert torch.equal(cache.ring_k[1], ring_before) and torch.equal(cache.core_k[1], core_before)
    assert cache.lens.cpu().tolist() == [lens0[0] + 1, 10 ** 6]   # only the valid sequence advanced
    want = cca_serving.serve_rows(Q[0], K[0], V[0], [lens0[0]], g, k, scale, core_dtype=dt)
    err = np.abs(out[0].cpu().numpy()[:, None, :] - want).max()
    assert err <= TOL[dt]


def test_serve_capacity_error(gpu):
    B, Hq, Hkv, d, g, k = 1, 2, 1, 64, 16, 1
    cache = binding.ServeCache(B, Hq, Hkv, d, g, k, 32, dtype=torch.float32, device=gpu)
    Q, K, V = np_inputs(1, Hq, 31, d, "f32", 38)
    _, Kk, Vv = np_inputs(1, Hkv, 31, d, "f32", 39)
    qb, kb, vb = _dev(Q, "f32", gpu), _dev(Kk, "f32", gpu), _dev(Vv, "f32", gpu)
    _, kc, vc = binding.prefill(qb, kb, vb, g, k, return_core=True)
    cache.load_sequence(0, kb, vb, kc, vc)           # 31 tokens
    step = [torch.zeros((1, h, d), device=gpu) for h in (Hq, Hkv, Hkv)]
    for _ in range(16):                              # positions 31..46 fit (group 1 pooled into slot 1 of 2)
        cache.step(*step)
    with pytest.raises(binding.CCAError):
        cache.step(*step)                            # position 47 completes group 2: a third core slot
    # the failed call changed nothing on the host side
    assert cache.lens_host == [47]


@pytest.mark.parametrize("lca", [False, True], ids=["cca", "lca"])
def test_serve_graph_replay_matches_eager(gpu, lca):
    """A serving step captured in a HIP graph and replayed once per token gives bit-identical
    outputs, caches and lengths to the eager calls with the same length bound.  Eager
    work and synchronisations run between the replays, and every replay is checked."""
    B, Hq, Hkv, d, g, k, dt, lens0, T, seed = (3, 4, 2, 128, 16, 2, "bf16", [100, 37, 0], 40, 38)
    bound = max(lens0) + T
    total = bound + 1
    Q, _, _ = np_inputs(B, Hq, total, d, dt, seed)
    _, K, V = np_inputs(B, Hkv, total, d, dt, seed + 1000)
    scale = 1.0 / math.sqrt(d)

    def make():
        if lca:
            c = binding.LCAServeCache(B, Hq, Hkv, d, g, k, total + g, 64, dtype=TDT[dt], device=gpu)
        else:
            c = binding.ServeCache(B, Hq, Hkv, d, g, k, total + g, dtype=TDT[dt], device=gpu)
        for b, L in enumerate(lens0):
            if L:
                qb, kb, vb = (_dev(x[b:b + 1, :, :L], dt, gpu) for x in (Q, K, V))
                if lca:
                    _, kc, vc, _ = binding.prefill_lca(qb, kb, vb, g, k, 64, scale)
                    c.load_sequence(b, qb, kb, vb, kc, vc)
                else:
                    _, kc, vc = binding.prefill(qb, kb, vb, g, k, scale, return_core=True)
                    c.load_sequence(b, kb, vb, kc, vc)
        return c

    eager, graphed = make(), make()
    torch.cuda.synchronize()
    gr = graphed.graph(bound, out_dtype=torch.float32, scale=scale)
    assert graphed.lens.cpu().tolist() == lens0          # capturing ran nothing
    for i in range(T):
        q = _dev(np.stack([Q[b, :, lens0[b] + i] for b in range(B)]), dt, gpu)
        kk = _dev(np.stack([K[b, :, lens0[b] + i] for b in range(B)]), dt, gpu)
        v = _dev(np.stack([V[b, :, lens0[b] + i] for b in range(B)]), dt, gpu)
        want = eager.step(q, kk, v, out_dtype=torch.float32, scale=scale, max_len=bound)
        got = gr.step(q, kk, v)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {i}: replay differs from the eager call"
    assert graphed.lens.cpu().tolist() == eager.lens.cpu().tolist() == [L + T for L in lens0]
    assert graphed.lens_host == eager.lens_host
    for name in ("core_k", "core_v", "ring_k", "ring_v") + (("qsum",) if lca else ()):
        assert torch.equal(getattr(graphed, name), getattr(eager, name)), name


@pytest.mark.parametrize("kind", ["sharp", "ramp"])
def test_serve_extreme_score_ranges(gpu, kind):
    """Serving steps under score ranges far from N(0,1): 'sharp' scales Q by 8 and K by 4
    (nearly one-hot softmaxes); 'ramp' adds a component shared by every query whose key weight
    grows with the position, so the scores rise by about 150 (log2 units) along a sequence and
    the running reference point of the online softmax moves many times within a chunk."""
    B, Hq, Hkv, d, g, k, dt, lens0, T = 2, 4, 2, 128, 16, 4, "bf16", [700, 1900], 12
    _say(f"serve extreme scores {kind}")
    total = max(lens0) + T
    Q, _, _ = np_inputs(B, Hq, total, d, "f32", 60)
    _, K, V = np_inputs(B, Hkv, total, d, "f32", 61)
    if kind == "sharp":
        Q, K = Q * 8.0, K * 4.0
    else:
        u = np.ones(d, dtype=np.float32) / np.sqrt(d)
        Q = Q + 6.0 * u
        K = K + (np.arange(total, dtype=np.float32)[:, None] * (200.0 / total)) * u
    Q, K, V = (torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).float().numpy() for x in (Q, K, V))
    scale = 1.0 / math.sqrt(d)
    cache = binding.ServeCache(B, Hq, Hkv, d, g, k, total + g, dtype=TDT[dt], device=gpu)
    for b, L in enumerate(lens0):
        qb, kb, vb = (_dev(x[b:b + 1, :, :L], dt, gpu) for x in (Q, K, V))
        _, kc, vc = binding.prefill(qb, kb, vb, g, k, scale, return_core=True)
        cache.load_sequence(b, kb, vb, kc, vc)
    outs = []
    for i in range(T):
        q = _dev(np.stack([Q[b, :, lens0[b] + i] for b in range(B)]), dt, gpu)
        kk = _dev(np.stack([K[b, :, lens0[b] + i] for b in range(B)]), dt, gpu)
        v = _dev(np.stack([V[b, :, lens0[b] + i] for b in range(B)]), dt, gpu)
        outs.append(cache.step(q, kk, v, out_dtype=torch.float32, scale=scale).cpu().numpy())
    torch.cuda.synchronize()
    got = np.stack(outs, axis=2)
    for b in range(B):
        pos = [lens0[b] + i for i in range(T)]
        want = cca_serving.serve_rows(Q[b].astype(np.float64), K[b].astype(np.float64), V[b].astype(np.float64),
                                      pos, g, k, scale, core_dtype=dt)
        # a float32 score of |q|.|k| carries a rounding error of about sqrt(d) 2^-24 sum|q_i k_i| scale,
        # a weight the same relative error: added to the bf16 bound, as for the prefill
        ds = math.sqrt(d) * 2.0 ** -24 * (np.abs(Q[b]).reshape(-1, d) @ np.abs(K[b]).reshape(-1, d).T).max() * scale
        tol = TOL[dt] + 2.0 * ds * np.abs(V).max()
        err = np.abs(got[b] - want).max()
        assert np.isfinite(err) and err <= tol, f"sequence {b}: max abs err {err:.3e} > {tol:.3e}"
