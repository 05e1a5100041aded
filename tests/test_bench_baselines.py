"""CPU checks of the benchmark's CPU-oracle legs (no GPU).

The decode baseline replays the decode workload step by step (pool the group a token
completes, then that token's row); fed the oracle's own streaming decode
(oracle.decode_stream, a different formulation: an explicit core list and raw ring) as the
"GPU outputs", its parity error must vanish.  The prefill baseline runs oracle.cca_slice per
head and compares with given outputs the same way.  These pin what the benchmark's CPU
baselines compute, so that their timings are of the stated workloads.
"""
import math

import numpy as np
import torch

import bench
import oracle
from long_context_sparse_cca_amd.synth import np_inputs


def test_decode_sample_slices_cover_every_sequence():
    s = bench.decode_sample_slices(8, 32)
    assert len(s) == len(set(s)) == 16
    assert sorted({b for b, _ in s}) == list(range(8))
    assert all(0 <= h < 32 for _, h in s)


def test_cpu_decode_replays_the_decode_workload():
    B, H, d, g, k, L0, S = 2, 4, 16, 4, 2, 48, 20
    cfg = {"B": B, "H": H, "d": d, "g": g, "k_local": k, "context": L0, "steps": S, "dtype": "f32"}
    Q, K, V = np_inputs(B, H, L0 + S, d, "f32", 5)
    scale = 1.0 / math.sqrt(d)
    want = np.zeros((S, B, H, d))
    for b in range(B):
        for h in range(H):
            want[:, b, h] = oracle.decode_stream(Q[b, h], K[b, h], V[b, h], g, k, scale, t_begin=L0, core_dtype="f32")
    sample = {(b, h): tuple(torch.from_numpy(x[b, h].copy()) for x in (Q, K, V))
              for (b, h) in bench.decode_sample_slices(B, H)}
    res = bench.cpu_decode(sample, want, cfg, S)
    assert res["parity_max_abs_err"] < 1e-9
    assert res["unit"] == "ms/step" and res["value"] > 0
    # S = 20 steps from position 48 with g = 4: the steps at t = 51, 55, ..., 67 complete a group
    assert "5 pooling step(s) per slice" in res["sample"]


def test_cpu_prefill_heads_runs_the_prefill_workload():
    B, H, L, d, g, k = 1, 3, 70, 16, 8, 2
    cfg = {"B": B, "H": H, "L": L, "d": d, "g": g, "k_local": k, "dtype": "f32"}
    Q, K, V = np_inputs(B, H, L, d, "f32", 6)
    out = torch.from_numpy(oracle.cca(Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64), g, k,
                                      1.0 / math.sqrt(d), core_dtype="f32"))
    res = bench.cpu_prefill_heads(*(torch.from_numpy(x) for x in (Q, K, V)), out, cfg, seconds=60.0)
    # the leg reads the given outputs as float32 (the GPU's output type): one float32 rounding
    assert res["parity_max_abs_err"] < 1e-6
    assert res["parity_rows"] == B * H * L and res["value"] > 0
