"""Chunked append (n new tokens per sequence per call): HIP path vs the oracle.

Every sequence starts from its own prefix (a GPU prefill loaded into a one-sequence view
of the cache; length 0 = empty), then receives a series of chunks of different sizes --
single tokens, chunks that cross group boundaries, the largest chunk one call takes
(k*g + 1) and longer ones that the binding splits -- and every returned row is compared
with the oracle's row at its position (a token's output is its prefill row).  Chunked
prefill from an empty cache and single-token steps after chunks are covered as well.
Tolerances (max-abs): fp32 1e-4, bf16 2e-2 (core tokens stored in the input dtype).
"""
import ctypes
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


# (B, H_q, H_kv, d, g, k, dtype, initial lengths, chunk sizes, seed)
EXTEND_CASES = [
    (2, 4, 2, 128, 16, 2, "bf16", [100, 37], [1, 5, 17, 33, 40], 40),   # 40 > k*g+1 = 33: split
    (2, 8, 2, 128, 16, 4, "bf16", [0, 300], [65, 64, 3], 41),          # chunked prefill from empty
    (1, 2, 2, 64, 5, 3, "f32", [0], [16, 16, 16, 1, 7], 42),           # k*g+1 = 16, ragged group size
    (2, 6, 3, 64, 16, 1, "f32", [20, 3], [17, 2, 17], 43),             # r = 2, d = 64 fp32
    (1, 16, 2, 128, 16, 64, "bf16", [1500], [1025, 300], 44),          # the largest chunk, r = 8
    (3, 4, 4, 128, 8, 3, "f32", [9, 0, 50], [25, 4], 45),              # fp32 d = 128, r = 1
    (2, 4, 2, 128, 16, 2, "f16", [100, 0], [1, 40, 17], 46),           # binary16 cache
    (1, 2, 1, 64, 7, 2, "f16", [30], [15, 3, 22], 47),                 # binary16, d = 64
]


def _id(c):
    B, Hq, Hkv, d, g, k, dt, lens, chunks, seed = c
    return f"B{B}Hq{Hq}kv{Hkv}d{d}g{g}k{k}-{dt}-L{'_'.join(map(str, lens))}-n{'_'.join(map(str, chunks))}"


def _setup(B, Hq, Hkv, d, g, k, dt, lens0, total, seed, device):
    Q, _, _ = np_inputs(B, Hq, total, d, dt, seed)
    _, K, V = np_inputs(B, Hkv, total, d, dt, seed + 1000)
    cache = binding.ServeCache(B, Hq, Hkv, d, g, k, total + g, dtype=TDT[dt], device=device)
    scale = 1.0 / math.sqrt(d)
    for b, L in enumerate(lens0):
        if L:
            qb, kb, vb = (_dev(x[b:b + 1, :, :L], dt, device) for x in (Q, K, V))
            _, kc, vc = binding.prefill(qb, kb, vb, g, k, scale, return_core=True)
            cache.load_sequence(b, kb, vb, kc, vc)
    return Q, K, V, cache, scale


@pytest.mark.parametrize("case", EXTEND_CASES, ids=_id)
def test_extend_chunks_match_oracle(gpu, case):
    B, Hq, Hkv, d, g, k, dt, lens0, chunks, seed = case
    _say(f"extend case {_id(case)} seed {seed}")
    total = max(lens0) + sum(chunks) + 3
    Q, K, V, cache, scale = _setup(B, Hq, Hkv, d, g, k, dt, lens0, total, seed, gpu)
    pos = list(lens0)
    got = {b: [] for b in range(B)}
    want_pos = {b: [] for b in range(B)}
    for n in chunks:
        q = _dev(np.stack([Q[b, :, pos[b]:pos[b] + n] for b in range(B)]), dt, gpu)
        kk = _dev(np.stack([K[b, :, pos[b]:pos[b] + n] for b in range(B)]), dt, gpu)
        v = _dev(np.stack([V[b, :, pos[b]:pos[b] + n] for b in range(B)]), dt, gpu)
        out = cache.extend(q, kk, v, out_dtype=torch.float32, scale=scale).cpu().numpy()
        for b in range(B):
            got[b].append(out[b])
            want_pos[b].extend(range(pos[b], pos[b] + n))
            pos[b] += n
    # three single-token steps after the chunks
    for _ in range(3):
        q = _dev(np.stack([Q[b, :, pos[b]] for b in range(B)]), dt, gpu)
        kk = _dev(np.stack([K[b, :, pos[b]] for b in range(B)]), dt, gpu)
        v = _dev(np.stack([V[b, :, pos[b]] for b in range(B)]), dt, gpu)
        out = cache.step(q, kk, v, out_dtype=torch.float32, scale=scale).cpu().numpy()
        for b in range(B):
            got[b].append(out[b][:, None, :])
            want_pos[b].append(pos[b])
            pos[b] += 1
    torch.cuda.synchronize()
    assert cache.lens.cpu().tolist() == pos
    for b in range(B):
        g_b = np.concatenate(got[b], axis=1)
        want = cca_serving.serve_rows(Q[b], K[b], V[b], want_pos[b], g, k, scale, core_dtype=dt)
        err = np.abs(g_b - want).max()
        assert np.isfinite(err) and err <= TOL[dt], f"sequence {b}: max abs err {err:.3e}"


def test_extend_rejects_oversized_chunk_and_capacity(gpu):
    B, Hq, Hkv, d, g, k = 1, 2, 1, 64, 4, 2
    cache = binding.ServeCache(B, Hq, Hkv, d, g, k, 20, dtype=torch.float32, device=gpu)
    lib = binding.load_library()
    n = k * g + 2   # one more than a call takes
    q = torch.zeros((B, Hq, n, d), device=gpu)
    kv = torch.zeros((B, Hkv, n, d), device=gpu)
    out = torch.empty_like(q)
    ws = torch.empty((lib.cca_extend_workspace_bytes(ctypes.byref(cache.desc), n) + 3) // 4, device=gpu)
    st = lib.cca_cache_extend(ctypes.byref(cache.desc), ctypes.c_void_p(cache.lens.data_ptr()), 0, Hq, n,
                              ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv.data_ptr()),
                              ctypes.c_void_p(kv.data_ptr()), ctypes.c_void_p(out.data_ptr()), 0,
                              ctypes.c_void_p(ws.data_ptr()), ws.numel() * 4, 0.125, None)
    assert st == -1   # CCA_ERR_INVALID
    # capacity: 20 tokens = 5 core slots; a chunk whose last token would complete group 5 is refused
    cache.extend(torch.zeros((B, Hq, 9, d), device=gpu), torch.zeros((B, Hkv, 9, d), device=gpu),
                 torch.zeros((B, Hkv, 9, d), device=gpu))
    cache.extend(torch.zeros((B, Hq, 9, d), device=gpu), torch.zeros((B, Hkv, 9, d), device=gpu),
                 torch.zeros((B, Hkv, 9, d), device=gpu))   # positions 9..17: groups up to 3 pooled
    with pytest.raises(binding.CCAError):
        cache.extend(torch.zeros((B, Hq, 6, d), device=gpu), torch.zeros((B, Hkv, 6, d), device=gpu),
                     torch.zeros((B, Hkv, 6, d), device=gpu))  # positions 18..23 would need core slot 5
    assert cache.lens.cpu().tolist() == [18]


def test_extend_work_order_ties_and_out_of_range(gpu):
    """The extend attention takes the sequences longest first, ranked on the device from their
    lengths: here the lengths are out of order, two are equal, one sequence is empty and one is
    beyond max_len.  The out-of-range sequence gets NaN rows and keeps its length; every other
    row matches the oracle, and every other length advances by n."""
    B, Hq, Hkv, d, g, k, dt, seed = 6, 4, 2, 128, 16, 2, "bf16", 48
    lens0 = [60, 200, 60, 0, 130, 33]
    max_len, n = 150, 20
    _say(f"extend work order: lengths {lens0}, max_len {max_len}, n {n}")
    total = max(lens0) + n + 3
    Q, K, V, cache, scale = _setup(B, Hq, Hkv, d, g, k, dt, lens0, total, seed, gpu)
    q, kk, v = (_dev(np.stack([X[b, :, lens0[b]:lens0[b] + n] for b in range(B)]), dt, gpu) for X in (Q, K, V))
    out = torch.empty((B, Hq, n, d), dtype=torch.float32, device=gpu)
    lib = binding.load_library()
    ws = torch.empty((lib.cca_extend_workspace_bytes(ctypes.byref(cache.desc), n) + 15) // 16 * 4, device=gpu)
    st = lib.cca_cache_extend(ctypes.byref(cache.desc), ctypes.c_void_p(cache.lens.data_ptr()), max_len, Hq, n,
                              ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kk.data_ptr()),
                              ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()), 0,
                              ctypes.c_void_p(ws.data_ptr()), ws.numel() * 4, scale, None)
    assert st == 0
    torch.cuda.synchronize()
    assert cache.lens.cpu().tolist() == [L + n if L <= max_len else L for L in lens0]
    got = out.cpu().numpy()
    assert np.isnan(got[1]).all()
    for b, L in enumerate(lens0):
        if L > max_len:
            continue
        want = cca_serving.serve_rows(Q[b], K[b], V[b], range(L, L + n), g, k, scale, core_dtype=dt)
        err = np.abs(got[b] - want).max()
        assert np.isfinite(err) and err <= TOL[dt], f"sequence {b}: max abs err {err:.3e}"


def test_extend_window_beyond_one_grid_column(gpu):
    """A raw window of (k+1)*g = 524288 rows (g = 64, k = 8191, float32, d = 128): the staging
    copy of the window needs more than 65535 blocks of the gather's second grid dimension, so
    the gather strides over the rest.  Every appended row matches the oracle."""
    B, Hq, Hkv, d, g, k, dt, seed = 1, 1, 1, 128, 64, 8191, "f32", 49
    L0, n = (k + 1) * g + 100, 50
    _say(f"extend with a {(k + 1) * g}-row window, prefix {L0}")
    total = L0 + n
    Q, K, V, cache, scale = _setup(B, Hq, Hkv, d, g, k, dt, [L0], total, seed, gpu)
    q, kk, v = (_dev(X[:, :, L0:L0 + n], dt, gpu) for X in (Q, K, V))
    out = cache.extend(q, kk, v, out_dtype=torch.float32, scale=scale)
    torch.cuda.synchronize()
    assert cache.lens.cpu().tolist() == [L0 + n]
    want = cca_serving.serve_rows(Q[0], K[0], V[0], range(L0, L0 + n), g, k, scale, core_dtype=dt)
    err = np.abs(out[0].cpu().numpy() - want).max()
    assert np.isfinite(err) and err <= TOL[dt], f"max abs err {err:.3e}"
