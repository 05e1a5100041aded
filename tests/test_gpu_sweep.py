"""Seeded random sweeps of the HIP entry points against the oracle.

The hand-picked cases of the other GPU tests aim at known edges; these draw shapes at
random (fixed seeds, so a failure names a reproducible case): sequence lengths from 1
to ~1300 (ragged against every tile size), group sizes from 1 to 64 including primes,
windows from 0 to 64 groups, head dims 64 and 128, fp32, bf16 and binary16, 1 to 4 query heads
per key/value head, per-sequence lengths in the serving cache (some empty), chunked
appends up to the largest allowed chunk, the LCA-style serving cache (steps and chunks
mixed), and the backward pass (matrix-core and vector paths).  Tolerances as for the
other parity tests: max-abs 1e-4 (fp32), 2e-2 (bf16), 5e-3 (binary16); gradients the same
fractions of their scale.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import cca_backward, cca_lca, cca_serving
from long_context_sparse_cca_amd import binding
from long_context_sparse_cca_amd.synth import np_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 5e-3}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
GROUPS = [1, 2, 3, 5, 8, 13, 16, 17, 32, 64]
WINDOWS = [0, 1, 2, 3, 7, 64]


def _dev(x, dt, device):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=TDT[dt]).contiguous()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(B, H, Hkv, L, d, dt, seed):
    Q = np_inputs(B, H, L, d, dt, seed)[0]
    K, V = np_inputs(B, Hkv, L, d, dt, seed + 1000)[1:]
    return Q, K, V


def _prefill_cases(n=20, seed=2024, dtypes=("f32", "bf16")):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        Hkv = int(rng.integers(1, 3))
        r = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(list(dtypes)))
        g = int(rng.choice(GROUPS))
        k = int(rng.choice(WINDOWS))
        # half the lengths log-uniform (many below one tile), half uniform up to 1300
        L = int(np.exp(rng.uniform(0, np.log(1300)))) if i % 2 else int(rng.integers(1, 1300))
        L = max(1, min(L, 4000 // (B * Hkv * r)))
        cases.append((B, Hkv * r, Hkv, L, d, g, k, dt, 500 + i))
    return cases


def _pid(c):
    B, H, Hkv, L, d, g, k, dt, seed = c
    return f"B{B}H{H}kv{Hkv}L{L}d{d}g{g}k{k}-{dt}-s{seed}"


@pytest.mark.parametrize("case", _prefill_cases() + _prefill_cases(n=6, seed=4242, dtypes=("f16",)), ids=_pid)
def test_prefill_sweep(gpu, case):
    B, H, Hkv, L, d, g, k, dt, seed = case
    _say(f"prefill sweep {_pid(case)}")
    Q, K, V = _inputs(B, H, Hkv, L, d, dt, seed)
    q, kk, v = (_dev(x, dt, gpu) for x in (Q, K, V))
    scale = 1.0 / math.sqrt(d)
    out = binding.prefill(q, kk, v, g, k, scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = cca_serving.cca_gqa(Q, K, V, g, k, scale, core_dtype=dt)
    err = np.abs(out.cpu().numpy().astype(np.float64) - want).max()
    assert np.isfinite(err) and err <= TOL[dt], f"max abs err {err:.3e}"


def _serve_cases(n=6, seed=77, dtypes=("f32", "bf16")):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.integers(1, 3))
        r = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(list(dtypes)))
        g = int(rng.choice([2, 5, 8, 16]))
        k = int(rng.choice([0, 1, 3, 8]))
        lens = [int(x) if rng.uniform() > 0.2 else 0 for x in rng.integers(1, 400, size=B)]
        T = int(rng.integers(5, 26))
        cases.append((B, Hkv * r, Hkv, d, g, k, dt, lens, T, 600 + i))
    return cases


def _sid(c):
    B, Hq, Hkv, d, g, k, dt, lens, T, seed = c
    return f"B{B}Hq{Hq}kv{Hkv}d{d}g{g}k{k}-{dt}-L{'_'.join(map(str, lens))}-T{T}-s{seed}"


def _serve_setup(B, Hq, Hkv, d, g, k, dt, lens0, total, seed, device):
    Q, K, V = _inputs(B, Hq, Hkv, total, d, dt, seed)
    cache = binding.ServeCache(B, Hq, Hkv, d, g, k, total + g, dtype=TDT[dt], device=device)
    scale = 1.0 / math.sqrt(d)
    for b, L in enumerate(lens0):
        if L:
            qb, kb, vb = (_dev(x[b:b + 1, :, :L], dt, device) for x in (Q, K, V))
            _, kc, vc = binding.prefill(qb, kb, vb, g, k, scale, return_core=True)
            cache.load_sequence(b, kb, vb, kc, vc)
    return Q, K, V, cache, scale


@pytest.mark.parametrize("case", _serve_cases() + _serve_cases(n=3, seed=7077, dtypes=("f16",)), ids=_sid)
def test_serve_sweep(gpu, case):
    B, Hq, Hkv, d, g, k, dt, lens0, T, seed = case
    _say(f"serve sweep {_sid(case)}")
    Q, K, V, cache, scale = _serve_setup(B, Hq, Hkv, d, g, k, dt, lens0, max(lens0) + T, seed, gpu)
    outs = []
    for i in range(T):
        q, kk, v = (_dev(np.stack([x[b, :, lens0[b] + i] for b in range(B)]), dt, gpu) for x in (Q, K, V))
        outs.append(cache.step(q, kk, v, out_dtype=torch.float32, scale=scale).cpu().numpy())
    torch.cuda.synchronize()
    assert cache.lens.cpu().tolist() == [L + T for L in lens0]
    got = np.stack(outs, axis=2)
    for b in range(B):
        want = cca_serving.serve_rows(Q[b], K[b], V[b], [lens0[b] + i for i in range(T)], g, k, scale,
                                      core_dtype=dt)
        err = np.abs(got[b] - want).max()
        assert np.isfinite(err) and err <= TOL[dt], f"sequence {b}: max abs err {err:.3e}"


def _extend_cases(n=4, seed=99, dtypes=("f32", "bf16")):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        Hkv = int(rng.integers(1, 3))
        r = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(list(dtypes)))
        g = int(rng.choice([4, 8, 16]))
        k = int(rng.choice([1, 2, 4]))
        lens = [int(x) for x in rng.integers(0, 300, size=B)]
        chunks = [int(x) for x in rng.integers(1, k * g + 2, size=3)]   # up to the largest allowed chunk
        cases.append((B, Hkv * r, Hkv, d, g, k, dt, lens, chunks, 700 + i))
    return cases


def _eid(c):
    B, Hq, Hkv, d, g, k, dt, lens, chunks, seed = c
    return f"B{B}Hq{Hq}kv{Hkv}d{d}g{g}k{k}-{dt}-L{'_'.join(map(str, lens))}-n{'_'.join(map(str, chunks))}-s{seed}"


@pytest.mark.parametrize("case", _extend_cases() + _extend_cases(n=2, seed=9099, dtypes=("f16",)), ids=_eid)
def test_extend_sweep(gpu, case):
    B, Hq, Hkv, d, g, k, dt, lens0, chunks, seed = case
    _say(f"extend sweep {_eid(case)}")
    total = max(lens0) + sum(chunks)
    Q, K, V, cache, scale = _serve_setup(B, Hq, Hkv, d, g, k, dt, lens0, total, seed, gpu)
    pos = list(lens0)
    got = {b: [] for b in range(B)}
    rows = {b: [] for b in range(B)}
    for n in chunks:
        q, kk, v = (_dev(np.stack([x[b, :, pos[b]:pos[b] + n] for b in range(B)]), dt, gpu) for x in (Q, K, V))
        out = cache.extend(q, kk, v, out_dtype=torch.float32, scale=scale).cpu().numpy()
        for b in range(B):
            got[b].append(out[b])
            rows[b].extend(range(pos[b], pos[b] + n))
            pos[b] += n
    torch.cuda.synchronize()
    assert cache.lens.cpu().tolist() == pos
    for b in range(B):
        want = cca_serving.serve_rows(Q[b], K[b], V[b], rows[b], g, k, scale, core_dtype=dt)
        err = np.abs(np.concatenate(got[b], axis=1) - want).max()
        assert np.isfinite(err) and err <= TOL[dt], f"sequence {b}: max abs err {err:.3e}"


def _backward_cases(n=4, seed=123):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Hkv = int(rng.integers(1, 3))
        r = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 3, 8, 16, 17]))
        k = int(rng.choice([0, 1, 2, 5]))
        L = int(rng.integers(40, 700))
        cases.append((1, Hkv * r, Hkv, L, g, k, 800 + i))
    return cases


def _bid(c):
    B, H, Hkv, L, g, k, seed = c
    return f"B{B}H{H}kv{Hkv}L{L}g{g}k{k}-s{seed}"


@pytest.mark.parametrize("case", _backward_cases(), ids=_bid)
def test_backward_sweep(gpu, case):
    B, H, Hkv, L, g, k, seed = case
    d = 128
    _say(f"backward sweep {_bid(case)}")
    Q, K, V = _inputs(B, H, Hkv, L, d, "bf16", seed)
    dO = np_inputs(B, H, L, d, "bf16", seed + 2000)[0]
    q, kk, v, do = (_dev(x, "bf16", gpu) for x in (Q, K, V, dO))
    scale = 1.0 / math.sqrt(d)
    out, lse, kc, vc = binding.prefill_lse(q, kk, v, g, k, scale)
    dq, dk, dv = binding.backward(q, kk, v, kc, vc, out, lse, do, g, k, scale)
    torch.cuda.synchronize()
    want = cca_backward.cca_backward_gqa(Q, K, V, dO, g, k, scale, core_dtype="bf16")
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        err = np.abs(got.cpu().numpy().astype(np.float64) - ref).max()
        bound = 2e-2 * max(1.0, np.abs(ref).max())
        assert np.isfinite(err) and err <= bound, f"{name}: max abs err {err:.3e} > {bound:.3e}"


def _lca_cases(n=4, seed=321, dtypes=("f32", "bf16")):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Hkv = int(rng.integers(1, 3))
        r = int(rng.choice([1, 2]))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(list(dtypes)))
        g = int(rng.choice([2, 5, 16, 33]))
        k = int(rng.choice([0, 1, 3]))
        d_rope = int(rng.choice([0, 8, d // 2, d]))
        L = int(rng.integers(1, 900))
        cases.append((1, Hkv * r, Hkv, L, d, g, k, d_rope, dt, 900 + i))
    return cases


def _lca_d128_cases(n=8, seed=4321):
    """The 16-bit d = 128, g = 16 condensation kernel: head ratios 1..8, ragged lengths (also
    shorter than one group), odd d_rope (a lane's two columns straddle the content/positional
    split)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Hkv = int(rng.integers(1, 3))
        r = int(rng.choice([1, 2, 4, 8]))
        dt = str(rng.choice(["bf16", "f16"]))
        k = int(rng.choice([0, 1, 4]))
        d_rope = int(rng.choice([0, 1, 17, 64, 127, 128]))
        L = int(rng.integers(1, 16)) if rng.random() < 0.15 else int(rng.integers(16, 1500))
        cases.append((1, Hkv * r, Hkv, L, 128, 16, k, d_rope, dt, 1900 + i))
    return cases


def _lid(c):
    B, H, Hkv, L, d, g, k, r, dt, seed = c
    return f"B{B}H{H}kv{Hkv}L{L}d{d}g{g}k{k}rope{r}-{dt}-s{seed}"


@pytest.mark.parametrize("case", _lca_cases() + _lca_cases(n=2, seed=3321, dtypes=("f16",)) + _lca_d128_cases(),
                         ids=_lid)
def test_lca_sweep(gpu, case):
    B, H, Hkv, L, d, g, k, d_rope, dt, seed = case
    _say(f"lca sweep {_lid(case)}")
    Q, K, V = _inputs(B, H, Hkv, L, d, dt, seed)
    q, kk, v = (_dev(x, dt, gpu) for x in (Q, K, V))
    scale = 1.0 / math.sqrt(d)
    out, kc, vc, anchors = binding.prefill_lca(q, kk, v, g, k, d_rope, scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    anc = anchors.cpu().numpy()
    r = H // Hkv
    if L // g and d_rope:
        for hk in range(Hkv):
            q_mean = Q[0, hk * r:(hk + 1) * r].astype(np.float64).mean(axis=0)
            S = cca_lca.lca_scores(q_mean, K[0, hk].astype(np.float64), g, scale)
            picked = S[np.arange(S.shape[0]), anc[0, hk]]
            assert np.all(picked >= S.max(axis=1) - 1e-5 * np.maximum(1.0, np.abs(S).max(axis=1)))
    want = cca_lca.lca_gqa(Q, K, V, g, k, scale, d_rope, anchors=anc if L // g else None, core_dtype=dt)[0]
    err = np.abs(out.cpu().numpy().astype(np.float64) - want).max()
    assert np.isfinite(err) and err <= TOL[dt], f"max abs err {err:.3e}"


def _lca_serve_cases(n=4, seed=55, dtypes=("f32", "bf16")):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.integers(1, 3))
        r = int(rng.choice([1, 2, 3]))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(list(dtypes)))
        g = int(rng.choice([2, 5, 8, 16]))
        k = int(rng.choice([0, 1, 3]))
        d_rope = int(rng.choice([0, 8, d // 2, d]))
        lens = [int(x) if rng.uniform() > 0.25 else 0 for x in rng.integers(1, 300, size=B)]
        # a mix of chunked appends (n <= k*g + 1) and single steps
        ops = [int(rng.integers(1, k * g + 2)) if rng.uniform() < 0.5 else 1 for _ in range(int(rng.integers(3, 8)))]
        cases.append((B, Hkv * r, Hkv, d, g, k, d_rope, dt, lens, ops, 950 + i))
    return cases


def _lsid(c):
    B, Hq, Hkv, d, g, k, r, dt, lens, ops, seed = c
    return (f"B{B}Hq{Hq}kv{Hkv}d{d}g{g}k{k}rope{r}-{dt}-L{'_'.join(map(str, lens))}"
            f"-ops{'_'.join(map(str, ops))}-s{seed}")


def _anchor_rows(gk, K, g, d_rope):
    m, d = gk.shape
    anc = np.zeros(m, dtype=np.int64)
    if d_rope == 0:
        return anc
    for j in range(m):
        hits = [i for i in range(g) if np.array_equal(gk[j, d - d_rope:], K[j * g + i, d - d_rope:])]
        assert hits, f"condensed key {j}: positional dims match no key of its group"
        anc[j] = hits[0]
    return anc


@pytest.mark.parametrize("case", _lca_serve_cases() + _lca_serve_cases(n=2, seed=5055, dtypes=("f16",)), ids=_lsid)
def test_lca_serve_sweep(gpu, case):
    """LCA-style serving cache: chunked appends (op n > 1, or n = 1 through the chunk path when
    drawn as a chunk) and single steps, every row against the LCA-style prefill rows."""
    B, Hq, Hkv, d, g, k, d_rope, dt, lens0, ops, seed = case
    _say(f"lca serve sweep {_lsid(case)}")
    total = max(lens0) + sum(ops)
    Q, K, V = _inputs(B, Hq, Hkv, total, d, dt, seed)
    scale = 1.0 / math.sqrt(d)
    cache = binding.LCAServeCache(B, Hq, Hkv, d, g, k, total + g, d_rope, dtype=TDT[dt], device=gpu)
    for b, L in enumerate(lens0):
        if L:
            qb, kb, vb = (_dev(x[b:b + 1, :, :L], dt, gpu) for x in (Q, K, V))
            _, kc, vc, _ = binding.prefill_lca(qb, kb, vb, g, k, d_rope, scale)
            cache.load_sequence(b, qb, kb, vb, kc, vc)
    pos = list(lens0)
    got = {b: [] for b in range(B)}
    for j, n in enumerate(ops):
        if n == 1 and j % 2:
            q, kk, v = (_dev(np.stack([x[b, :, pos[b]] for b in range(B)]), dt, gpu) for x in (Q, K, V))
            out = cache.step(q, kk, v, out_dtype=torch.float32, scale=scale).cpu().numpy()[:, :, None, :]
        else:
            q, kk, v = (_dev(np.stack([x[b, :, pos[b]:pos[b] + n] for b in range(B)]), dt, gpu) for x in (Q, K, V))
            out = cache.extend(q, kk, v, out_dtype=torch.float32, scale=scale).cpu().numpy()
        for b in range(B):
            got[b].append(out[b])
            pos[b] += n
    torch.cuda.synchronize()
    assert cache.lens.cpu().tolist() == pos
    for b in range(B):
        n_tot = pos[b]
        m = n_tot // g
        Qb, Kb, Vb = (x[b, :, :n_tot].astype(np.float64) for x in (Q, K, V))
        anc = np.stack([_anchor_rows(cache.core_k[b, hk, :m].float().cpu().numpy(), Kb[hk], g, d_rope)
                        for hk in range(Hkv)])
        want = cca_lca.lca_gqa(Qb[None], Kb[None], Vb[None], g, k, scale, d_rope, anchors=anc[None],
                               core_dtype=dt)[0][0][:, lens0[b]:n_tot]
        err = np.abs(np.concatenate(got[b], axis=1) - want).max()
        assert np.isfinite(err) and err <= TOL[dt], f"sequence {b}: max abs err {err:.3e}"


def _generic_backward_cases(n=4, seed=131, kinds=(("f32", 64), ("f32", 128), ("bf16", 64))):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt, d = kinds[int(rng.integers(0, len(kinds)))]
        Hkv = int(rng.integers(1, 3))
        r = int(rng.choice([1, 2, 3]))
        g = int(rng.choice([1, 3, 8, 16, 17]))
        k = int(rng.choice([0, 1, 2, 5]))
        L = int(rng.integers(1, 500))
        cases.append((dt, d, Hkv * r, Hkv, L, g, k, 1300 + i))
    return cases


def _gbid(c):
    dt, d, H, Hkv, L, g, k, seed = c
    return f"{dt}d{d}H{H}kv{Hkv}L{L}g{g}k{k}-s{seed}"


@pytest.mark.parametrize("case", _generic_backward_cases() + _generic_backward_cases(
    n=2, seed=1131, kinds=(("f16", 64), ("f16", 128))), ids=_gbid)
def test_generic_backward_sweep(gpu, case):
    """Backward pass on the vector path (float32, bf16 and binary16 inputs) at random shapes."""
    dt, d, H, Hkv, L, g, k, seed = case
    _say(f"generic backward sweep {_gbid(case)}")
    Q, K, V = _inputs(1, H, Hkv, L, d, dt, seed)
    dO = np_inputs(1, H, L, d, dt, seed + 2000)[0]
    q, kk, v, do = (_dev(x, dt, gpu) for x in (Q, K, V, dO))
    scale = 1.0 / math.sqrt(d)
    out, lse, kc, vc = binding.prefill_lse(q, kk, v, g, k, scale)
    dq, dk, dv = binding.backward(q, kk, v, kc, vc, out, lse, do, g, k, scale)
    torch.cuda.synchronize()
    core = None if dt == "f32" else dt
    tol = {"f32": 1e-4, "bf16": 2e-2, "f16": 5e-3}[dt]
    want = cca_backward.cca_backward_gqa(Q, K, V, dO, g, k, scale, core_dtype=core)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        err = np.abs(got.cpu().numpy().astype(np.float64) - ref).max()
        bound = tol * max(1.0, np.abs(ref).max())
        assert np.isfinite(err) and err <= bound, f"{name}: max abs err {err:.3e} > {bound:.3e}"


def _ring_cases(n=8, seed=4242, serve=False):
    """Small rings (R = (k+1) g from 1 to 15 slots) stepped through several wraps: the ring slot
    of every key is stepped per key in the decode and serving loops, which these cases exercise
    with steps both smaller and larger than R."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        g = int(rng.choice([1, 2, 3, 4, 5]))
        k = int(rng.choice([0, 1, 2]))
        R = (k + 1) * g
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["f32", "bf16"]))
        if serve:
            B = int(rng.integers(1, 4))
            Hkv = int(rng.integers(1, 3))
            r = int(rng.choice([1, 2, 4]))
            lens = [int(x) for x in rng.integers(0, 40, size=B)]
            cases.append((B, Hkv * r, Hkv, d, g, k, dt, lens, 4 * R + 7, 900 + i))
        else:
            B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
            L0 = int(rng.integers(0, 30))
            cases.append((B, H, d, g, k, L0, L0 + 4 * R + 9, dt, 950 + i))
    return cases


def _rid(c):
    B, H, d, g, k, L0, T, dt, seed = c
    return f"B{B}H{H}d{d}g{g}k{k}R{(k + 1) * g}-{dt}-L{L0}-T{T}-s{seed}"


@pytest.mark.parametrize("case", _ring_cases(), ids=_rid)
def test_decode_small_ring_sweep(gpu, case):
    """The fused append+decode over several wraps of a small ring, every step against the
    oracle's rows of the whole sequence."""
    from oracle import cca_oracle
    B, H, d, g, k, L0, T, dt, seed = case
    _say(f"decode ring sweep {_rid(case)}")
    Q, K, V = np_inputs(B, H, T, d, dt, seed)
    q, kk, v = (_dev(x, dt, gpu) for x in (Q, K, V))
    scale = 1.0 / math.sqrt(d)
    cache = binding.KVCache(B, H, d, g, k, max_tokens=T + g, dtype=TDT[dt], device=gpu)
    if L0 > 0:
        kc, vc = binding.pool_kv(q[:, :, :L0].contiguous(), kk[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(),
                                 g, scale)
        cache.load_prefill(kk[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(), kc, vc)
    got = torch.empty((T - L0, B, H, d), dtype=torch.float32, device=gpu)
    for t in range(L0, T):
        cache.append_decode(q[:, :, t].contiguous(), kk[:, :, t].contiguous(), v[:, :, t].contiguous(),
                            out_dtype=torch.float32, out=got[t - L0], scale=scale)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    for b in range(B):
        for h in range(H):
            want = cca_oracle.cca_slice(Q[b, h], K[b, h], V[b, h], g, k, scale, core_dtype=dt)[L0:]
            err = np.abs(got[:, b, h] - want).max()
            assert np.isfinite(err) and err <= TOL[dt], f"slice ({b},{h}): max abs err {err:.3e}"


@pytest.mark.parametrize("case", _ring_cases(serve=True, seed=4343), ids=_sid)
def test_serve_small_ring_sweep(gpu, case):
    """Serving steps over several wraps of a small ring, per-sequence lengths and grouped-query
    heads, every step against the oracle."""
    B, Hq, Hkv, d, g, k, dt, lens0, T, seed = case
    _say(f"serve ring sweep {_sid(case)}")
    Q, K, V, cache, scale = _serve_setup(B, Hq, Hkv, d, g, k, dt, lens0, max(lens0) + T, seed, gpu)
    outs = []
    for i in range(T):
        q, kk, v = (_dev(np.stack([x[b, :, lens0[b] + i] for b in range(B)]), dt, gpu) for x in (Q, K, V))
        outs.append(cache.step(q, kk, v, out_dtype=torch.float32, scale=scale).cpu().numpy())
    torch.cuda.synchronize()
    got = np.stack(outs, axis=2)
    for b in range(B):
        want = cca_serving.serve_rows(Q[b], K[b], V[b], [lens0[b] + i for i in range(T)], g, k, scale,
                                      core_dtype=dt)
        err = np.abs(got[b] - want).max()
        assert np.isfinite(err) and err <= TOL[dt], f"sequence {b}: max abs err {err:.3e}"
