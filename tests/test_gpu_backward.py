"""Backward pass of CCA prefill: HIP path vs the gradient oracle (bf16 d = 128 on the
matrix cores; float32 inputs and d = 64 on the vector path, further down).

Shapes span several 256-query and 128-key tiles with ragged tails, g not a power of
two, g = 1 (causal attention), a window wider than the sequence, and core tiles seen by
many query tiles.  The oracle recomputes the forward with core tokens stored in bf16
(the forward's stored core tokens) and differentiates in fp64.
Tolerance: the bf16 bound 2e-2, taken relative to the gradient's own scale
(max-abs error <= 2e-2 * max(1, max|reference|)): the softmax weights and dS are
rounded to bf16 as matrix-core operands (relative 2^-9 each), and D = dO.O uses the
bf16-rounded forward output.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import cca_backward
from long_context_sparse_cca_amd import binding
from long_context_sparse_cca_amd.synth import np_inputs

pytestmark = pytest.mark.gpu


TDT = {"bf16": torch.bfloat16, "f16": torch.float16}
# gradient bound (fraction of the gradient's scale) and log-sum-exp bound per input type
GRAD_TOL = {"bf16": 2e-2, "f16": 5e-3}
LSE_TOL = {"bf16": 1e-2, "f16": 2e-3}


def _dev(x, device, dt="bf16"):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=TDT[dt]).contiguous()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# matrix-core path (16-bit inputs, d = 128): (B, H, L, g, k, dtype, seed)
BWD_CASES = [
    (1, 2, 300, 16, 2, "bf16", 70),
    (1, 1, 700, 16, 4, "bf16", 71),     # core tiles seen by several query tiles
    (2, 1, 517, 7, 3, "bf16", 72),      # g not a power of two, ragged tiles
    (1, 1, 200, 1, 0, "bf16", 73),      # g = 1: causal attention
    (1, 1, 640, 16, 100, "bf16", 74),   # window wider than the sequence
    (1, 1, 1500, 32, 5, "bf16", 75),    # many core tokens per key tile
    (1, 2, 300, 16, 2, "f16", 76),      # binary16 inputs
    (2, 1, 517, 7, 3, "f16", 77),
    (1, 1, 1500, 32, 5, "f16", 78),
    # shorter than a group or a tile: no core token at all, exactly one group, one visible
    # core token (k = 0), and the first and second 64-query tile
    (1, 2, 1, 16, 2, "bf16", 60),
    (1, 1, 5, 16, 2, "bf16", 61),
    (2, 1, 15, 16, 1, "bf16", 62),
    (1, 2, 16, 16, 0, "bf16", 63),
    (1, 1, 17, 16, 0, "bf16", 64),
    (1, 1, 63, 16, 1, "bf16", 65),
    (1, 2, 65, 16, 1, "f16", 66),
]


def _id(c):
    B, H, L, g, k, dt, seed = c
    return f"B{B}H{H}L{L}g{g}k{k}-{dt}"


@pytest.mark.parametrize("case", BWD_CASES, ids=_id)
def test_backward_matches_oracle(gpu, case):
    """Gradients of the matrix-core path against the fp64 oracle, whose core tokens are
    rounded to the input type as the forward stores them.  P and dS are rounded to that
    type as MFMA operands, so the bound is the type's tolerance times the gradient's scale."""
    B, H, L, g, k, dt, seed = case
    d = 128
    _say(f"backward case {_id(case)} seed {seed}")
    Q, K, V = np_inputs(B, H, L, d, dt, seed)
    dO = np_inputs(B, H, L, d, dt, seed + 500)[0]
    q, kk, v, do = (_dev(x, gpu, dt) for x in (Q, K, V, dO))
    scale = 1.0 / math.sqrt(d)
    out, lse, kc, vc = binding.prefill_lse(q, kk, v, g, k, scale)
    dq, dk, dv = binding.backward(q, kk, v, kc, vc, out, lse, do, g, k, scale)
    torch.cuda.synchronize()
    # the training forward is the plain forward, plus the log-sum-exp
    assert torch.equal(out, binding.prefill(q, kk, v, g, k, scale))
    for b in range(B):
        for h in range(H):
            _, lse_ref = cca_backward.cca_forward_lse_slice(Q[b, h], K[b, h], V[b, h], g, k, scale, core_dtype=dt)
            e = np.abs(lse[b, h].cpu().numpy() - lse_ref).max()
            assert e <= LSE_TOL[dt], f"lse err {e:.3e}"
    # gradients against the oracle, using the GPU's 16-bit forward output for D = dO.O is not
    # needed: the oracle is exact and the tolerance covers the rounding of O
    want = cca_backward.cca_backward(Q, K, V, dO, g, k, scale, core_dtype=dt)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        err = np.abs(got.cpu().numpy().astype(np.float64) - ref).max()
        bound = GRAD_TOL[dt] * max(1.0, np.abs(ref).max())
        _say(f"  {name}: max abs err {err:.3e} (bound {bound:.3e})")
        assert np.isfinite(err) and err <= bound, f"{name}: max abs err {err:.3e} > {bound:.3e}"


def test_autograd_function_matches_backward(gpu):
    B, H, L, d, g, k = 1, 2, 400, 128, 16, 3
    Q, K, V = np_inputs(B, H, L, d, "bf16", 80)
    q, kk, v = (_dev(x, gpu).requires_grad_(True) for x in (Q, K, V))
    out = binding.CCAAttention.apply(q, kk, v, g, k)
    dO = _dev(np_inputs(B, H, L, d, "bf16", 81)[0], gpu)
    out.backward(dO)
    o2, lse, kc, vc = binding.prefill_lse(q.detach(), kk.detach(), v.detach(), g, k)
    dq, dk, dv = binding.backward(q.detach(), kk.detach(), v.detach(), kc, vc, o2, lse, dO, g, k)
    torch.cuda.synchronize()
    assert torch.equal(q.grad, dq.to(torch.bfloat16)) and torch.equal(kk.grad, dk.to(torch.bfloat16))
    assert torch.equal(v.grad, dv.to(torch.bfloat16))


def test_backward_unsupported_shapes(gpu):
    q = torch.zeros((1, 1, 64, 96), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(binding.CCAError):
        binding.prefill_lse(q, q.clone(), q.clone(), 16, 1)


# The vector path: float32 inputs at d = 64 and 128, 16-bit inputs at d = 64 (binary16 at
# d = 128 takes the matrix-core path, the case is kept as one more check of it).
# (dtype, d, B, H, H_kv, L, g, k, seed)
GEN_CASES = [
    ("f32", 64, 1, 2, 2, 256, 16, 1, 110),    # the small float32 layer (B=1, H=2, d=64, L=256, g=16, k=1)
    ("f32", 64, 2, 1, 1, 517, 7, 3, 111),     # g not a power of two, ragged tail
    ("f32", 64, 1, 1, 1, 200, 1, 0, 112),     # g = 1: causal attention
    ("f32", 64, 1, 1, 1, 640, 16, 100, 113),  # window wider than the sequence
    ("f32", 64, 1, 4, 2, 300, 16, 2, 114),    # grouped-query, r = 2
    ("f32", 128, 1, 1, 1, 700, 16, 4, 115),
    ("f32", 128, 2, 8, 2, 260, 7, 1, 116),    # grouped-query, r = 4
    ("bf16", 64, 1, 2, 2, 300, 16, 2, 117),
    ("bf16", 64, 1, 4, 1, 520, 16, 3, 118),   # multi-query
    ("f32", 64, 1, 1, 1, 15, 16, 1, 119),     # shorter than one group: no core tokens
    ("f16", 128, 1, 2, 2, 300, 16, 2, 123),   # binary16 inputs
    ("f16", 64, 1, 4, 2, 517, 7, 3, 124),     # binary16, grouped-query, ragged tail
]


def _gen_id(c):
    dt, d, B, H, Hkv, L, g, k, seed = c
    return f"{dt}d{d}B{B}H{H}Hkv{Hkv}L{L}g{g}k{k}"


@pytest.mark.parametrize("case", GEN_CASES, ids=_gen_id)
def test_generic_backward_matches_oracle(gpu, case):
    """Gradients of the float32 vector path against the fp64 oracle.  Float32 inputs:
    every product and sum in float32 (relative rounding ~1e-7 per step over at most a few
    thousand terms), so the bound is 1e-4 * max(1, max|reference|) and the oracle's core
    tokens are unrounded.  16-bit inputs: the core tokens and the output the gradients read
    are stored in the input type, so that type's bound applies (bf16 2e-2, binary16 5e-3),
    with the oracle's core tokens rounded to it."""
    dt, d, B, H, Hkv, L, g, k, seed = case
    _say(f"generic backward case {_gen_id(case)} seed {seed}")
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dt]
    Q = np_inputs(B, H, L, d, dt, seed)[0]
    K, V = (x[:, :Hkv] for x in np_inputs(B, H, L, d, dt, seed + 1)[1:])
    dO = np_inputs(B, H, L, d, dt, seed + 500)[0]
    q, kk, v, do = (torch.from_numpy(np.ascontiguousarray(x)).to(device=gpu, dtype=tdt) for x in (Q, K, V, dO))
    scale = 1.0 / math.sqrt(d)
    out, lse, kc, vc = binding.prefill_lse(q, kk, v, g, k, scale)
    dq, dk, dv = binding.backward(q, kk, v, kc, vc, out, lse, do, g, k, scale)
    torch.cuda.synchronize()
    assert torch.equal(out, binding.prefill(q, kk, v, g, k, scale))
    core = None if dt == "f32" else dt
    tol = {"f32": 1e-4, "bf16": 2e-2, "f16": 5e-3}[dt]
    lse_tol = {"f32": 1e-4, "bf16": 1e-2, "f16": 2e-3}[dt]
    if Hkv == H:
        for b in range(B):
            for h in range(H):
                _, lse_ref = cca_backward.cca_forward_lse_slice(Q[b, h], K[b, h], V[b, h], g, k, scale,
                                                                core_dtype=core)
                e = np.abs(lse[b, h].cpu().numpy() - lse_ref).max() if L else 0.0
                assert e <= lse_tol, f"lse err {e:.3e}"
        want = cca_backward.cca_backward(Q, K, V, dO, g, k, scale, core_dtype=core)
    else:
        want = cca_backward.cca_backward_gqa(Q, K, V, dO, g, k, scale, core_dtype=core)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        err = np.abs(got.cpu().numpy().astype(np.float64) - ref).max()
        bound = tol * max(1.0, np.abs(ref).max())
        _say(f"  {name}: max abs err {err:.3e} (bound {bound:.3e})")
        assert np.isfinite(err) and err <= bound, f"{name}: max abs err {err:.3e} > {bound:.3e}"


def test_generic_autograd_function(gpu):
    """The autograd function on float32 inputs at d = 64 routes through the vector path."""
    B, H, Hkv, L, d, g, k = 1, 4, 2, 260, 64, 16, 2
    Q = np_inputs(B, H, L, d, "f32", 120)[0]
    K, V = (x[:, :Hkv] for x in np_inputs(B, H, L, d, "f32", 121)[1:])
    q, kk, v = (torch.from_numpy(np.ascontiguousarray(x)).to(gpu).requires_grad_(True) for x in (Q, K, V))
    out = binding.CCAAttention.apply(q, kk, v, g, k)
    dO = torch.from_numpy(np.ascontiguousarray(np_inputs(B, H, L, d, "f32", 122)[0])).to(gpu)
    out.backward(dO)
    torch.cuda.synchronize()
    o2, lse, kc, vc = binding.prefill_lse(q.detach(), kk.detach(), v.detach(), g, k)
    dq, dk, dv = binding.backward(q.detach(), kk.detach(), v.detach(), kc, vc, o2, lse, dO, g, k)
    torch.cuda.synchronize()
    assert torch.equal(q.grad, dq) and torch.equal(kk.grad, dk) and torch.equal(v.grad, dv)


# grouped-query training: (B, H, H_kv, L, g, k, dtype, seed)
GQA_BWD_CASES = [
    (1, 4, 2, 300, 16, 2, "bf16", 90),    # r = 2
    (1, 4, 1, 520, 16, 3, "bf16", 91),    # multi-query (r = 4), ragged tiles
    (2, 8, 2, 260, 7, 1, "bf16", 92),     # r = 4, g not a power of two
    (1, 4, 1, 520, 16, 3, "f16", 93),     # binary16, multi-query
]


def _gid(c):
    B, H, Hkv, L, g, k, dt, seed = c
    return f"B{B}H{H}Hkv{Hkv}L{L}g{g}k{k}-{dt}"


@pytest.mark.parametrize("case", GQA_BWD_CASES, ids=_gid)
def test_gqa_backward_matches_oracle(gpu, case):
    B, H, Hkv, L, g, k, dt, seed = case
    d = 128
    _say(f"gqa backward case {_gid(case)} seed {seed}")
    Q = np_inputs(B, H, L, d, dt, seed)[0]
    K, V = (x[:, :Hkv] for x in np_inputs(B, H, L, d, dt, seed + 1)[1:])
    dO = np_inputs(B, H, L, d, dt, seed + 500)[0]
    q, kk, v, do = (_dev(x, gpu, dt) for x in (Q, K, V, dO))
    scale = 1.0 / math.sqrt(d)
    out, lse, kc, vc = binding.prefill_lse(q, kk, v, g, k, scale)
    dq, dk, dv = binding.backward(q, kk, v, kc, vc, out, lse, do, g, k, scale)
    torch.cuda.synchronize()
    assert tuple(dk.shape) == (B, Hkv, L, d) and tuple(kc.shape) == (B, Hkv, L // g, d)
    assert torch.equal(out, binding.prefill(q, kk, v, g, k, scale))
    want = cca_backward.cca_backward_gqa(Q, K, V, dO, g, k, scale, core_dtype=dt)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        err = np.abs(got.cpu().numpy().astype(np.float64) - ref).max()
        bound = GRAD_TOL[dt] * max(1.0, np.abs(ref).max())
        _say(f"  {name}: max abs err {err:.3e} (bound {bound:.3e})")
        assert np.isfinite(err) and err <= bound, f"{name}: max abs err {err:.3e} > {bound:.3e}"


def test_gqa_autograd_function(gpu):
    B, H, Hkv, L, d, g, k = 1, 4, 2, 300, 128, 16, 2
    Q = np_inputs(B, H, L, d, "bf16", 95)[0]
    K, V = (x[:, :Hkv] for x in np_inputs(B, H, L, d, "bf16", 96)[1:])
    q, kk, v = (_dev(x, gpu).requires_grad_(True) for x in (Q, K, V))
    out = binding.CCAAttention.apply(q, kk, v, g, k)
    dO = _dev(np_inputs(B, H, L, d, "bf16", 97)[0], gpu)
    out.backward(dO)
    torch.cuda.synchronize()
    assert tuple(kk.grad.shape) == (B, Hkv, L, d) and tuple(q.grad.shape) == (B, H, L, d)
    o2, lse, kc, vc = binding.prefill_lse(q.detach(), kk.detach(), v.detach(), g, k)
    dq, dk, dv = binding.backward(q.detach(), kk.detach(), v.detach(), kc, vc, o2, lse, dO, g, k)
    torch.cuda.synchronize()
    assert torch.equal(q.grad, dq.to(torch.bfloat16)) and torch.equal(kk.grad, dk.to(torch.bfloat16))
    assert torch.equal(v.grad, dv.to(torch.bfloat16))


@pytest.mark.parametrize("Hkv,dt", [(32, "bf16"), (8, "bf16"), (32, "f16")], ids=["mha", "gqa8", "mha-f16"])
def test_backward_fullsize_32k_sampled(gpu, Hkv, dt):
    """L = 32768, H = 32, d = 128, g = 16, k = 64 (the 32K prefill layer), full backward on
    the GPU; one query head's sampled dQ rows and its key/value head's sampled dK/dV keys
    (core-token groups, window edges, group-last rows) against the per-entry oracle.
    binary16 too: its softmax weights (about 1/3000 here) and dS are matrix-core operands
    near binary16's subnormal range, so precision loss at long context shows up here."""
    from long_context_sparse_cca_amd.synth import torch_inputs
    H, L, d, g, k = 32, 32768, 128, 16, 64
    _say(f"backward full size L={L} H={H} H_kv={Hkv} {dt}")
    q, kk, v = torch_inputs(1, H, L, d, TDT[dt], gpu, seed=31, heavy_frac=0.01)
    if Hkv != H:
        kk, v = kk[:, :Hkv].contiguous(), v[:, :Hkv].contiguous()
    gen = torch.Generator(device=gpu)
    gen.manual_seed(32)
    do = torch.randn((1, H, L, d), generator=gen, device=gpu).to(TDT[dt])
    scale = 1.0 / math.sqrt(d)
    out, lse, kc, vc = binding.prefill_lse(q, kk, v, g, k, scale)
    dq, dk, dv = binding.backward(q, kk, v, kc, vc, out, lse, do, g, k, scale)
    torch.cuda.synchronize()
    r = H // Hkv
    h = 5                        # query head; its key/value head is h // r
    hk = h // r
    rng = np.random.default_rng(7)
    rows = sorted({0, 1, g - 1, g, k * g - 1, k * g, (k + 1) * g - 1, L // 2 - 1, L - g - 1, L - 1,
                   *rng.integers(0, L, size=16).tolist()})
    keys = sorted({0, g - 1, g, k * g, L // 2, L - g, L - 1, *rng.integers(0, L, size=16).tolist()})
    heads = range(hk * r, (hk + 1) * r)
    Qh = np.stack([q[0, i].double().cpu().numpy() for i in heads])
    dOh = np.stack([do[0, i].double().cpu().numpy() for i in heads])
    Kk = kk[0, hk].double().cpu().numpy()
    Vk = v[0, hk].double().cpu().numpy()
    wq, wk, wv = cca_backward.cca_backward_sampled_slice(Qh, Kk, Vk, dOh, g, k, scale, rows, keys,
                                                         core_dtype=dt)
    got_q = np.stack([dq[0, i, rows].cpu().numpy() for i in heads])
    got_k = dk[0, hk, keys].cpu().numpy()
    got_v = dv[0, hk, keys].cpu().numpy()
    for name, got, ref in (("dq", got_q, wq), ("dk", got_k, wk), ("dv", got_v, wv)):
        err = np.abs(got.astype(np.float64) - ref).max()
        bound = GRAD_TOL[dt] * max(1.0, np.abs(ref).max())
        _say(f"  {name}: max abs err {err:.3e} (bound {bound:.3e})")
        assert np.isfinite(err) and err <= bound, f"{name}: max abs err {err:.3e} > {bound:.3e}"
