#!/usr/bin/env python3
"""CCA attention benchmark on one MI355X: prefill tokens/s and decode step latency at 128K.

One step = one pass of the whole hot path on synthetic inputs:
  * prefill of one attention layer, B=1, H=32, d=128, L=131072, g=16, k=64, bf16:
    pooling into core tokens (cca_pool_kv) + fused core/local attention (cca_attention);
  * decode, B=8, H=32, d=128, context 131072 tokens held as core tokens plus a
    1040-slot raw ring: 256 steps, each one launch that appends the token (pooling
    every 16th step) and computes its attention (cca_cache_append_decode).
The decode cache is re-seeded from the prefilled state before each step's
decode phase (outside the per-phase timings).

Prints one JSON line.  `value` is the prefill throughput (tokens/s); decode
latency, KV-cache bytes, the roofline of the dominant kernel (the fused
attention, bf16 MFMA bound) and a CPU-oracle baseline ride along.  The shorter
prefill workloads (256 tokens in float32; 8K and 32K in bf16) are measured
beside the timed steps (`prefill_workloads`), each with its roofline and its own
CPU-oracle baseline; the oracle's decode step is timed too (`cpu_baseline.decode`).

`--config N` times one workload of WORKLOADS alone instead (1: 256-token float32
prefill, 2: 8K, 3: 32K, 4: 128K bf16 prefill, 5: 128K-context bf16 decode).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CCA prefill tokens/s & decode step latency at 128K; % MFMA / HBM roofline"
H, D, G, KL = 32, 128, 16, 64
PREFILL_B, PREFILL_L = 1, 131072
DEC_B, DEC_L0, DEC_STEPS = 8, 131072, 256
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEAVY = 0.01

# The workloads, each one layer of per-head attention inputs (LLaMA2-7B's H=32, d=128 for
# the long ones).  Prefill: one pass of pooling + fused attention over L tokens.  Decode:
# `steps` single-token steps after a `context`-token prefill, one fused launch each.
WORKLOADS = {
    1: {"kind": "prefill", "B": 1, "H": 2, "d": 64, "L": 256, "g": 16, "k_local": 1, "dtype": "f32", "heavy": 0.0},
    2: {"kind": "prefill", "B": 1, "H": 32, "d": 128, "L": 8192, "g": 16, "k_local": 64, "dtype": "bf16",
        "heavy": HEAVY},
    3: {"kind": "prefill", "B": 1, "H": 32, "d": 128, "L": 32768, "g": 16, "k_local": 64, "dtype": "bf16",
        "heavy": HEAVY},
    4: {"kind": "prefill", "B": PREFILL_B, "H": H, "d": D, "L": PREFILL_L, "g": G, "k_local": KL, "dtype": "bf16",
        "heavy": HEAVY},
    5: {"kind": "decode", "B": DEC_B, "H": H, "d": D, "context": DEC_L0, "steps": DEC_STEPS, "g": G, "k_local": KL,
        "dtype": "bf16", "heavy": HEAVY},
}


def workload_name(cfg) -> str:
    if cfg["kind"] == "prefill":
        return (f"CCA prefill of one attention layer B={cfg['B']} H={cfg['H']} d={cfg['d']} L={cfg['L']} "
                f"g={cfg['g']} k={cfg['k_local']} {cfg['dtype']}")
    return (f"CCA decode B={cfg['B']} H={cfg['H']} d={cfg['d']} context {cfg['context']} "
            f"g={cfg['g']} k={cfg['k_local']} {cfg['dtype']}, {cfg['steps']} steps")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--config", type=int, choices=sorted(WORKLOADS), default=None,
                    help="time one workload alone (1: 256-token fp32 prefill, 2: 8K, 3: 32K, 4: 128K bf16 prefill, "
                         "5: 128K-context bf16 decode); default: 4 and 5 in each step, the others beside them")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="time budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the standard-attention comparison")
    ap.add_argument("--no-training", action="store_true", help="skip the forward+backward measurement")
    ap.add_argument("--no-serving", action="store_true",
                    help="skip the serving decode measurement (per-sequence lengths, grouped-query heads)")
    ap.add_argument("--no-lca", action="store_true", help="skip the LCA-style variant measurement")
    ap.add_argument("--no-f16", action="store_true", help="skip the binary16 prefill measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the shorter prefill workloads (256-token fp32, 8K, 32K) beside the timed steps")
    ap.add_argument("--phase", choices=["all", "prefill", "decode", "serving", "training", "lca", "copy"],
                    default="all",
                    help="profiling aid: run only one phase (the JSON line is then not the benchmark result); "
                         "'copy' runs a plain 1 GiB device copy whose counter readings calibrate FETCH_SIZE/WRITE_SIZE")
    return ap.parse_args()


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_sparse_cca_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kind: str, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if the kernel source is unchanged."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            rec = json.load(f).get(kind)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


class CpuEnv:
    """Thread pools of the oracle's BLAS sized to the cores this process may use, and a
    description of the host (core count, CPU model, BLAS build) for the report."""

    def __enter__(self):
        self.n_cpu = len(os.sched_getaffinity(0))
        self.blas = "unknown"
        self.limiter = None
        try:
            import threadpoolctl
            self.limiter = threadpoolctl.threadpool_limits(limits=self.n_cpu)
            info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
            self.threads = sum(i.get("num_threads", 0) for i in info)
            self.blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in info) or "none found"
        except Exception:  # noqa: BLE001
            self.threads = 1
        self.threads = self.threads or 1
        self.cpu_model = platform.processor() or platform.machine()
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        self.cpu_model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        return self

    def __exit__(self, *exc):
        if self.limiter is not None:
            self.limiter.restore_original_limits()
        return False

    def fields(self):
        return {"cores": self.threads, "kind": "oracle", "cpu": self.cpu_model, "cpus_available": self.n_cpu,
                "blas": self.blas}


def _np64(t):
    import numpy as np
    return t.float().cpu().numpy().astype(np.float64)


def cpu_baseline(q, k, v, out, seconds: float):
    """Time the CPU oracle on a bounded sample of the 128K prefill workload (head 0).

    The same sampled rows are compared with `out` (the GPU prefill of the same
    inputs, fp32 output): against the oracle with bf16-stored core tokens (the
    parity bar) and against exact fp64 core tokens (context)."""
    import numpy as np

    import oracle
    with CpuEnv() as env:
        scale = 1.0 / math.sqrt(D)
        Q, K, V = _np64(q[0, 0]), _np64(k[0, 0]), _np64(v[0, 0])
        got = out[0, 0].float().cpu().numpy()
        t0 = time.perf_counter()
        Kc, Vc, _ = oracle.pool(Q, K, V, G, scale, core_dtype="bf16")
        t_pool = time.perf_counter() - t0
        rng = np.random.default_rng(0)
        rows = rng.permutation(PREFILL_L)
        n = 0
        err = 0.0
        t1 = time.perf_counter()
        while n < len(rows) and (time.perf_counter() - t1) < seconds:
            t = int(rows[n])
            ref = oracle.cca_row(Q[t], t, K, V, Kc, Vc, G, KL, scale)
            err = max(err, float(np.abs(got[t] - ref).max()))
            n += 1
        t_rows = time.perf_counter() - t1
        Kx, Vx, _ = oracle.pool(Q, K, V, G, scale)
        err_exact = max(float(np.abs(got[int(t)] - oracle.cca_row(Q[t], int(t), K, V, Kx, Vx, G, KL, scale)).max())
                        for t in rows[:min(n, 2000)])
    per_row = t_rows / n
    layer_s = H * PREFILL_B * (t_pool + PREFILL_L * per_row)
    return {
        "value": PREFILL_B * PREFILL_L / layer_s,
        "unit": "tokens/s",
        **env.fields(),
        "sample": (f"head 0 of the prefill input: full pooling ({t_pool:.2f} s) + {n} uniformly drawn query rows "
                   f"({t_rows:.1f} s); extrapolated to all {H} heads x {PREFILL_L} rows"),
        "parity_max_abs_err": err,
        "parity_rows": n,
        "err_vs_exact_core_tokens": err_exact,
    }


def cpu_prefill_heads(q, k, v, out, cfg, seconds: float):
    """The oracle's whole-slice prefill (oracle.cca_slice: pooling, then every row) on as many
    heads of the workload as fit in `seconds` (at least one), extrapolated to all heads, and
    its rows compared with `out` (the GPU's fp32-output prefill of the same inputs)."""
    import numpy as np

    import oracle
    B, Hh, L, d, g, kl = cfg["B"], cfg["H"], cfg["L"], cfg["d"], cfg["g"], cfg["k_local"]
    scale = 1.0 / math.sqrt(d)
    core = cfg["dtype"]
    with CpuEnv() as env:
        spent, n, err = 0.0, 0, 0.0
        for b in range(B):
            for h in range(Hh):
                Q, K, V = _np64(q[b, h]), _np64(k[b, h]), _np64(v[b, h])
                t0 = time.perf_counter()
                ref = oracle.cca_slice(Q, K, V, g, kl, scale, core_dtype=core)
                spent += time.perf_counter() - t0
                err = max(err, float(np.abs(out[b, h].float().cpu().numpy() - ref).max()))
                n += 1
                if spent >= seconds:
                    break
            if spent >= seconds:
                break
    slices = B * Hh
    layer_s = spent / n * slices
    return {"value": B * L / layer_s, "unit": "tokens/s", **env.fields(),
            "sample": (f"{n} of {slices} (b,h) slices, every row ({spent:.1f} s)"
                       + ("" if n == slices else f"; extrapolated to all {slices}")),
            "parity_max_abs_err": err, "parity_rows": n * L}


def decode_sample_slices(B: int, Hh: int, per_seq: int = 2):
    """(b, h) slices of the decode workload whose steps the oracle replays: `per_seq` heads per
    sequence, spread over the heads and shifted from one sequence to the next."""
    step = Hh // per_seq
    return [(b, (b + j * step) % Hh) for b in range(B) for j in range(per_seq)]


def cpu_decode(sample, gpu_out, cfg, steps: int):
    """The oracle's decode step on a sample of (b, h) slices of the decode workload.

    `sample` maps (b, h) to that slice's host Q, K, V (context + steps tokens);
    `gpu_out` [steps, B, H, d] holds the GPU's fp32 outputs of the same steps.  Each slice
    is seeded untimed (the oracle pools the context); each step then appends the token,
    pooling the group it completes (oracle.pool over that group), and computes the new
    token's output (oracle.cca_row).  The time per step over the sample is scaled to all
    B*H slices: ms per decode step of the whole batch."""
    import numpy as np

    import oracle
    Bb, Hh, d, g, kl, L0 = cfg["B"], cfg["H"], cfg["d"], cfg["g"], cfg["k_local"], cfg["context"]
    scale = 1.0 / math.sqrt(d)
    core = cfg["dtype"]
    with CpuEnv() as env:
        spent, err, pools = 0.0, 0.0, 0
        for (b, h), (q, k, v) in sample.items():
            Q, K, V = _np64(q), _np64(k), _np64(v)
            m_max = (L0 + steps) // g
            Kc = np.zeros((m_max, d))
            Vc = np.zeros((m_max, d))
            Kc[:L0 // g], Vc[:L0 // g], _ = oracle.pool(Q[:L0], K[:L0], V[:L0], g, scale, core_dtype=core)
            t0 = time.perf_counter()
            for s in range(steps):
                t = L0 + s
                if (t + 1) % g == 0:
                    j = t // g
                    rows = slice(j * g, (j + 1) * g)
                    kj, vj, _ = oracle.pool(Q[rows], K[rows], V[rows], g, scale, core_dtype=core)
                    Kc[j], Vc[j] = kj[0], vj[0]
                    pools += 1
                o = oracle.cca_row(Q[t], t, K, V, Kc, Vc, g, kl, scale)
                err = max(err, float(np.abs(gpu_out[s, b, h] - o).max()))
            spent += time.perf_counter() - t0
    per_slice_step = spent / (len(sample) * steps)
    ms_step = per_slice_step * Bb * Hh * 1e3
    return {"value": ms_step, "unit": "ms/step", "higher_is_better": False, **env.fields(),
            "tokens_per_s": Bb / (ms_step * 1e-3),
            "sample": (f"{len(sample)} of {Bb * Hh} (b,h) slices x {steps} steps from position {L0} "
                       f"({pools // len(sample)} pooling step(s) per slice; {spent:.1f} s), seeded untimed; "
                       f"scaled to all {Bb * Hh} slices"),
            "parity_max_abs_err": err, "parity_rows": len(sample) * steps}


def dense_comparison(binding, accounting, dev, seed):
    """Standard causal attention on the same kernels (k >= floor((L-1)/g): no core token is
    visible and the window is [0, t]) against CCA (k = 64) at 64K and 128K, one layer, B=1,
    H=32, d=128, bf16: MI355X context for the write-up's end-to-end speed ratios (Fig. 3).
    Outside the timed steps."""
    import torch

    from long_context_sparse_cca_amd.synth import torch_inputs
    out = {}
    for L in (65536, 131072):
        q, k, v = torch_inputs(1, H, L, D, torch.bfloat16, dev, seed=seed, heavy_frac=HEAVY)
        kc, vc = binding.pool_kv(q, k, v, G)
        o = torch.empty_like(q)
        times = {}
        for name, kl in (("cca", KL), ("dense", L)):
            binding.attention(q, k, v, kc, vc, G, kl, out=o)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(2):
                binding.attention(q, k, v, kc, vc, G, kl, out=o)
            e1.record()
            torch.cuda.synchronize()
            times[name] = e0.elapsed_time(e1) / 2
        fl_dense = accounting.prefill_flops(1, H, L, D, G, L)
        res_b, full_b = accounting.kv_cache_bytes(L, G, KL, 1, H, D, 2)
        out[str(L)] = {"cca_attention_ms": times["cca"], "dense_attention_ms": times["dense"],
                       "speedup": times["dense"] / times["cca"],
                       "dense_tflops": fl_dense / (times["dense"] * 1e-3) / 1e12,
                       "kv_cache_fraction": res_b / full_b}
        del q, k, v, kc, vc, o
        torch.cuda.empty_cache()
    out["page_context"] = {"speedup_64k": 5.7, "speedup_128k": 7.9, "kv_reduction_128k": 0.93,
                           "note": "end-to-end LLaMA2-7B inference on unnamed hardware; ours is one attention layer"}
    return out


def binary16_prefill(binding, accounting, dev, seed, reps: int = 5):
    """The prefill step of the headline workload (B=1, H=32, d=128, L=131072, g=16, k=64) on
    IEEE binary16 inputs: the same attention kernel instantiated for half precision, with
    pooling on the generic kernel.  Outside the timed steps."""
    import torch

    from long_context_sparse_cca_amd.synth import torch_inputs
    L = PREFILL_L
    q, k, v = torch_inputs(1, H, L, D, torch.float16, dev, seed=seed, heavy_frac=HEAVY)
    kc, vc = binding.pool_kv(q, k, v, G)
    o = torch.empty_like(q)
    binding.prefill(q, k, v, G, KL, out=o)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    pool_ms = attn_ms = 0.0
    for _ in range(reps):
        ev[0].record()
        binding.pool_kv(q, k, v, G, kc=kc, vc=vc)
        ev[1].record()
        binding.attention(q, k, v, kc, vc, G, KL, out=o)
        ev[2].record()
        torch.cuda.synchronize()
        pool_ms += ev[0].elapsed_time(ev[1]) / reps
        attn_ms += ev[1].elapsed_time(ev[2]) / reps
    fl = accounting.prefill_flops(1, H, L, D, G, KL)
    tflops = fl / (attn_ms * 1e-3) / 1e12
    del q, k, v, kc, vc, o
    torch.cuda.empty_cache()
    return {"config": {"B": 1, "H": H, "d": D, "L": L, "g": G, "k_local": KL, "dtype": "f16"},
            "ms": pool_ms + attn_ms, "pool_ms": pool_ms, "attention_ms": attn_ms,
            "tokens_per_s": L / ((pool_ms + attn_ms) * 1e-3),
            "roofline": {"kernel": "cca_prefill_d128_kernel<f16>", "bound": "mfma", "achieved": tflops,
                         "peak": 2500.0, "unit": "TFLOP/s", "frac": tflops / 2500.0}}


def serving_decode(binding, accounting, dev, seed, steps: int = 64):
    """Serving with per-sequence lengths and grouped-query attention, outside the timed steps:
    B=8 sequences at lengths 65536 + 9362*b (64K .. 128K), H_q=32 query heads over H_kv=8
    key/value heads (r=4), d=128, g=16, k=64, bf16.  Decode: each step is one
    cca_cache_append_decode_varlen call (append + pooling + attention of one token per
    sequence).  Chunked append: cca_cache_extend calls of 1024 tokens per sequence."""
    import torch

    from long_context_sparse_cca_amd.synth import torch_inputs
    B, Hq, Hkv = 8, 32, 8
    lens0 = [65536 + 9362 * b for b in range(B)]
    n_ext, chunks = 1024, 3
    cache = binding.ServeCache(B, Hq, Hkv, D, G, KL, max(lens0) + steps + 32 + chunks * n_ext + G,
                               dtype=torch.bfloat16, device=dev)
    for b, L in enumerate(lens0):
        q, _, _ = torch_inputs(1, Hq, L, D, torch.bfloat16, dev, seed=seed + 10 + b, heavy_frac=HEAVY)
        _, k, v = torch_inputs(1, Hkv, L, D, torch.bfloat16, dev, seed=seed + 30 + b, heavy_frac=HEAVY)
        kc, vc = binding.pool_kv(q, k, v, G)
        cache.load_sequence(b, k, v, kc, vc)
        del q, k, v, kc, vc
    torch.cuda.empty_cache()
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 50)
    qs = torch.randn((steps, B, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
    ks = torch.randn((steps, B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    vs = torch.randn((steps, B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    lens_at = []
    for s in range(steps):
        lens_at.append(list(cache.lens_host))
        ev[2 * s].record(stream)
        cache.step(qs[s], ks[s], vs[s], out=out)
        ev[2 * s + 1].record(stream)
    torch.cuda.synchronize()
    warm = 8
    us = [ev[2 * s].elapsed_time(ev[2 * s + 1]) * 1e3 for s in range(warm, steps)]
    nchunks = cache.serve_ws_bytes // (B * Hq * (D + 2) * 4)
    byt = [accounting.serve_bytes(lens_at[s], Hq, Hkv, D, G, KL, 2, nchunks) for s in range(warm, steps)]
    us_mean = sum(us) / len(us)
    gbs = sum(byt) / len(byt) / (us_mean * 1e-6) / 1e9
    # the same step captured once in a HIP graph (work split bounded by the length after the replays)
    g_steps = 32
    gr = cache.graph(max(cache.lens_host) + g_steps)
    gev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for s in range(4):
        gr.step(qs[s], ks[s], vs[s])
    torch.cuda.synchronize()
    gev[0].record(stream)
    for s in range(4, g_steps):   # replays alone (the static inputs hold the last token copied in)
        gr.graph.replay()
    gev[1].record(stream)
    torch.cuda.synchronize()
    cache.lens_host = [x + g_steps - 4 for x in cache.lens_host]
    graph_us = gev[0].elapsed_time(gev[1]) / (g_steps - 4) * 1e3
    # chunked append: 1024 new tokens for every sequence per call (four 256-query tiles; one call takes up to k*g+1)
    qe = torch.randn((B, Hq, n_ext, D), generator=gen, device=dev).to(torch.bfloat16)
    ke = torch.randn((B, Hkv, n_ext, D), generator=gen, device=dev).to(torch.bfloat16)
    ve = torch.randn((B, Hkv, n_ext, D), generator=gen, device=dev).to(torch.bfloat16)
    cache.extend(qe, ke, ve)   # first call sizes the staging workspace
    torch.cuda.synchronize()
    ext_ms, ext_fl = [], []
    for _ in range(chunks - 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        lens_now = list(cache.lens_host)
        e0.record(stream)
        cache.extend(qe, ke, ve)
        e1.record(stream)
        torch.cuda.synchronize()
        ext_ms.append(e0.elapsed_time(e1))
        ext_fl.append(accounting.extend_flops(lens_now, n_ext, Hq, D, G, KL))
    ms = sum(ext_ms) / len(ext_ms)
    tf = sum(ext_fl) / len(ext_fl) / (ms * 1e-3) / 1e12
    return {"config": {"B": B, "H_q": Hq, "H_kv": Hkv, "d": D, "g": G, "k_local": KL,
                       "lengths": lens0, "steps_timed": steps - warm},
            "us_per_step": us_mean, "bytes_per_step": sum(byt) / len(byt),
            "roofline": {"kernel": "cca_serve_decode_kernel<bf16,128,4> + cca_decode_merge_kernel", "bound": "hbm",
                         "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS},
            "graph_replay": {"us_per_step": graph_us, "steps_timed": g_steps - 4,
                             "note": "the step captured once in a HIP graph and replayed back to back"},
            "chunked_append": {"tokens_per_sequence": n_ext, "ms_per_call": ms,
                               "tokens_per_s": B * n_ext / (ms * 1e-3), "flops_per_call": sum(ext_fl) / len(ext_fl),
                               "roofline": {"kernel": "cca_prefill_d128_kernel<bf16,extend> (+ gather, append)",
                                            "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                                            "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS}}}


def training_step(binding, accounting, dev, seed, L: int = PREFILL_L, reps: int = 3, H_kv: int = H,
                  dtype: str = "bf16"):
    """Forward with log-sum-exp (cca_prefill_lse) and backward (cca_backward) of one layer,
    B=1, H=32 (H_kv key/value heads), d=128, g=16, k=64, bf16 (or binary16 with
    dtype="f16"), outside the timed steps."""
    import torch

    from long_context_sparse_cca_amd.synth import torch_inputs
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    q, k, v = torch_inputs(1, H, L, D, tdt, dev, seed=seed + 7, heavy_frac=HEAVY)
    if H_kv != H:
        k = k[:, :H_kv].contiguous()
        v = v[:, :H_kv].contiguous()
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 8)
    dout = torch.randn((1, H, L, D), generator=gen, device=dev).to(tdt)
    out, lse, kc, vc = binding.prefill_lse(q, k, v, G, KL)
    binding.backward(q, k, v, kc, vc, out, lse, dout, G, KL)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    fw, bw = [], []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        out, lse, kc, vc = binding.prefill_lse(q, k, v, G, KL)
        e[1].record(stream)
        binding.backward(q, k, v, kc, vc, out, lse, dout, G, KL)
        e[2].record(stream)
        torch.cuda.synchronize()
        fw.append(e[0].elapsed_time(e[1]))
        bw.append(e[1].elapsed_time(e[2]))
    fw_ms, bw_ms = sum(fw) / reps, sum(bw) / reps
    fl = accounting.backward_flops(1, H, L, D, G, KL)
    tf = fl / (bw_ms * 1e-3) / 1e12
    del q, k, v, dout, out, lse, kc, vc
    torch.cuda.empty_cache()
    return {"config": {"B": 1, "H": H, "H_kv": H_kv, "d": D, "L": L, "g": G, "k_local": KL, "dtype": dtype},
            "forward_ms": fw_ms, "backward_ms": bw_ms, "backward_flops": fl,
            "roofline": {"kernel": "cca_bwd_dq_kernel + cca_bwd_dkdv16_kernel (+ prep, pooling backward)",
                         "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / PEAK_BF16_TFLOPS,
                         "per_unit": "10*d FLOPs per visible (query, key) pair"}}


def lca_variant(binding, accounting, dev, seed, L: int = PREFILL_L, d_rope: int = 64, reps: int = 10):
    """LCA-style condensation (cca_pool_kv_lca) and the prefill built on it (cca_prefill_lca),
    B=1, H=32, d=128, g=16, k=64, bf16, last 64 dims of each key positional; outside the timed steps."""
    import torch

    from long_context_sparse_cca_amd.synth import torch_inputs
    q, k, v = torch_inputs(1, H, L, D, torch.bfloat16, dev, seed=seed + 9, heavy_frac=HEAVY)
    binding.prefill_lca(q, k, v, G, KL, d_rope)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    tp, tf = [], []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        binding.pool_kv_lca(q, k, v, G, d_rope)
        e[1].record(stream)
        e[2].record(stream)
        binding.prefill_lca(q, k, v, G, KL, d_rope)
        e[3].record(stream)
        torch.cuda.synchronize()
        tp.append(e[0].elapsed_time(e[1]))
        tf.append(e[2].elapsed_time(e[3]))
    pool_ms, prefill_ms = _median(tp), _median(tf)
    byt = accounting.lca_pool_bytes(1, H, L, D, G, 2)
    gbs = byt / (pool_ms * 1e-3) / 1e9
    del q, k, v
    torch.cuda.empty_cache()

    # decode with the LCA-style cache: B=8 sequences at context 131072, 64 steps (4 condensations)
    steps = 64
    dq, dk, dv = torch_inputs(DEC_B, H, DEC_L0 + steps, D, torch.bfloat16, dev, seed=seed + 10, heavy_frac=HEAVY)
    pre = [x[:, :, :DEC_L0].contiguous() for x in (dq, dk, dv)]
    _, kc, vc, _ = binding.prefill_lca(*pre, G, KL, d_rope)
    cache = binding.LCACache(DEC_B, H, D, G, KL, max_tokens=DEC_L0 + steps, d_rope=d_rope, dtype=torch.bfloat16,
                             device=dev)
    cache.load_prefill(*pre, kc, vc)
    del pre, kc, vc
    xs = [x[:, :, DEC_L0:].permute(2, 0, 1, 3).contiguous() for x in (dq, dk, dv)]
    del dq, dk, dv
    out = torch.empty((DEC_B, H, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for s_ in range(steps):
        cache.append_decode(xs[0][s_], xs[1][s_], xs[2][s_], out=out)
    ev[1].record(stream)
    torch.cuda.synchronize()
    dec_us = ev[0].elapsed_time(ev[1]) / steps * 1e3
    nchunks = cache.ws_bytes // (DEC_B * H * (D + 2) * 4)
    dbytes = sum(accounting.decode_bytes(DEC_B, H, D, DEC_L0 + s_, G, KL, 2, nchunks) for s_ in range(steps)) / steps
    dgbs = dbytes / (dec_us * 1e-6) / 1e9
    del cache, xs
    torch.cuda.empty_cache()
    serving = lca_serving(binding, accounting, dev, seed, d_rope)
    return {"config": {"B": 1, "H": H, "d": D, "L": L, "g": G, "k_local": KL, "d_rope": d_rope},
            "pool_ms": pool_ms, "prefill_ms": prefill_ms, "prefill_tokens_per_s": L / (prefill_ms * 1e-3),
            "pool_bytes": byt,
            "roofline": {"kernel": "cca_pool_lca_d128_g16_kernel", "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                         "per_unit": "(3*g + 2)*d*2 bytes per group"},
            "decode": {"config": {"B": DEC_B, "H": H, "context": DEC_L0, "steps": steps},
                       "us_per_step": dec_us, "bytes_per_step": dbytes,
                       "roofline": {"kernel": "cca_decode_kernel<bf16,128,lca append> + cca_decode_merge_kernel",
                                    "bound": "hbm", "achieved": dgbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": dgbs / PEAK_HBM_GBS}},
            "serving": serving}


def lca_serving(binding, accounting, dev, seed, d_rope: int, steps: int = 64):
    """Serving steps with the LCA-style cache (cca_cache_append_decode_varlen_lca), on the workload of
    serving_decode: B=8 sequences at lengths 65536 + 9362*b, H_q=32 over H_kv=8, d=128, g=16, k=64, bf16."""
    import torch

    from long_context_sparse_cca_amd.synth import torch_inputs
    B, Hq, Hkv = 8, 32, 8
    lens0 = [65536 + 9362 * b for b in range(B)]
    n_ext, chunks = 1024, 3
    cache = binding.LCAServeCache(B, Hq, Hkv, D, G, KL, max(lens0) + steps + chunks * n_ext + G, d_rope,
                                  dtype=torch.bfloat16, device=dev)
    for b, L in enumerate(lens0):
        q, _, _ = torch_inputs(1, Hq, L, D, torch.bfloat16, dev, seed=seed + 60 + b, heavy_frac=HEAVY)
        _, k, v = torch_inputs(1, Hkv, L, D, torch.bfloat16, dev, seed=seed + 80 + b, heavy_frac=HEAVY)
        kc, vc, _ = binding.pool_kv_lca(q, k, v, G, d_rope)
        cache.load_sequence(b, q, k, v, kc, vc)
        del q, k, v, kc, vc
    torch.cuda.empty_cache()
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 90)
    qs = torch.randn((steps, B, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
    ks = torch.randn((steps, B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    vs = torch.randn((steps, B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    lens_at = []
    for s in range(steps):
        lens_at.append(list(cache.lens_host))
        ev[2 * s].record(stream)
        cache.step(qs[s], ks[s], vs[s], out=out)
        ev[2 * s + 1].record(stream)
    torch.cuda.synchronize()
    warm = 8
    us = [ev[2 * s].elapsed_time(ev[2 * s + 1]) * 1e3 for s in range(warm, steps)]
    nchunks = cache.serve_ws_bytes // (B * Hq * (D + 2) * 4)
    byt = [accounting.serve_bytes(lens_at[s], Hq, Hkv, D, G, KL, 2, nchunks) for s in range(warm, steps)]
    us_mean = sum(us) / len(us)
    gbs = sum(byt) / len(byt) / (us_mean * 1e-6) / 1e9
    # chunked append: 1024 new tokens for every sequence per call
    qe = torch.randn((B, Hq, n_ext, D), generator=gen, device=dev).to(torch.bfloat16)
    ke = torch.randn((B, Hkv, n_ext, D), generator=gen, device=dev).to(torch.bfloat16)
    ve = torch.randn((B, Hkv, n_ext, D), generator=gen, device=dev).to(torch.bfloat16)
    cache.extend(qe, ke, ve)   # first call sizes the staging workspace
    torch.cuda.synchronize()
    ext_ms, ext_fl = [], []
    for _ in range(chunks - 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        lens_now = list(cache.lens_host)
        e0.record(stream)
        cache.extend(qe, ke, ve)
        e1.record(stream)
        torch.cuda.synchronize()
        ext_ms.append(e0.elapsed_time(e1))
        ext_fl.append(accounting.extend_flops(lens_now, n_ext, Hq, D, G, KL))
    ms = sum(ext_ms) / len(ext_ms)
    tf = sum(ext_fl) / len(ext_fl) / (ms * 1e-3) / 1e12
    return {"config": {"B": B, "H_q": Hq, "H_kv": Hkv, "d": D, "g": G, "k_local": KL, "d_rope": d_rope,
                       "lengths": lens0, "steps_timed": steps - warm},
            "us_per_step": us_mean, "bytes_per_step": sum(byt) / len(byt),
            "roofline": {"kernel": "cca_serve_decode_kernel<bf16,128,4,lca> + cca_decode_merge_kernel",
                         "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS},
            "chunked_append": {"tokens_per_sequence": n_ext, "ms_per_call": ms,
                               "tokens_per_s": B * n_ext / (ms * 1e-3), "flops_per_call": sum(ext_fl) / len(ext_fl),
                               "roofline": {"kernel": "cca_prefill_d128_kernel<bf16,extend> (+ gather, lca append)",
                                            "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                                            "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS}}}


def prefill_workload(binding, accounting, dev, seed, cfg, reps: int = 10, cpu_seconds: float = 0.0):
    """GPU prefill (pooling + fused attention, one event pair around each launch) of one
    prefill workload, outside the timed steps; medians over `reps` runs.  With cpu_seconds
    > 0 the oracle is timed on the same inputs too (cpu_prefill_heads)."""
    import torch

    from long_context_sparse_cca_amd.synth import torch_inputs
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[cfg["dtype"]]
    B, Hh, L, d, g, kl = cfg["B"], cfg["H"], cfg["L"], cfg["d"], cfg["g"], cfg["k_local"]
    scale = 1.0 / math.sqrt(d)
    q, k, v = torch_inputs(B, Hh, L, d, tdt, dev, seed=seed, heavy_frac=cfg["heavy"])
    kc, vc = binding.pool_kv(q, k, v, g, scale)
    o = torch.empty_like(q)
    binding.attention(q, k, v, kc, vc, g, kl, scale, out=o)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    tp, ta = [], []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        binding.pool_kv(q, k, v, g, scale, kc=kc, vc=vc)
        e[1].record(stream)
        binding.attention(q, k, v, kc, vc, g, kl, scale, out=o)
        e[2].record(stream)
        torch.cuda.synchronize()
        tp.append(e[0].elapsed_time(e[1]))
        ta.append(e[1].elapsed_time(e[2]))
    pool_ms, attn_ms = _median(tp), _median(ta)
    flops = accounting.prefill_flops(B, Hh, L, d, g, kl)
    elem = 4 if cfg["dtype"] == "f32" else 2
    pool_b = accounting.pool_bytes(B, Hh, L, d, g, elem)
    peak = PEAK_F32_TFLOPS if cfg["dtype"] == "f32" else PEAK_BF16_TFLOPS
    tflops = flops / (attn_ms * 1e-3) / 1e12
    kernel = "cca_prefill_d128_kernel<bf16>" if (d == 128 and elem == 2) else f"cca_prefill_kernel<{cfg['dtype']},{d}>"
    res = {"config": {key: cfg[key] for key in ("B", "H", "d", "L", "g", "k_local", "dtype")},
           "ms": pool_ms + attn_ms, "pool_ms": pool_ms, "attention_ms": attn_ms,
           "tokens_per_s": B * L / ((pool_ms + attn_ms) * 1e-3),
           "pool_gbs": pool_b / (pool_ms * 1e-3) / 1e9,
           "roofline": {"kernel": kernel, "bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                        "frac": tflops / peak, "flops_per_launch": flops,
                        "per_unit": "4*d FLOPs per visible (query, key) pair; pairs in closed form"}}
    if cpu_seconds > 0:
        out32 = binding.prefill(q, k, v, g, kl, scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        res["cpu_baseline"] = cpu_prefill_heads(q, k, v, out32, cfg, cpu_seconds)
        del out32
    del q, k, v, kc, vc, o
    torch.cuda.empty_cache()
    return res


def _leg(name: str):
    print(f"leg: {name}", file=sys.stderr, flush=True)


def _median(xs):
    if not xs:
        return float("nan")
    ys = sorted(xs)
    h = len(ys) // 2
    return ys[h] if len(ys) % 2 else 0.5 * (ys[h - 1] + ys[h])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the CCA path here has no "
              "multi-GPU code. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    from long_context_sparse_cca_amd import accounting, binding
    from long_context_sparse_cca_amd.synth import torch_inputs

    binding.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.phase == "copy":
        n = 1 << 29  # bf16 elements: 1 GiB
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"phase": "copy", "bytes_read": 2 * n, "bytes_written": 2 * n, "ms": dt * 1e3,
                          "gbs": 4 * n / dt / 1e9}), flush=True)
        return
    if args.phase == "training":
        print(json.dumps({"phase": "training", "training": training_step(binding, accounting, dev, args.seed),
                          "training_gqa": training_step(binding, accounting, dev, args.seed, H_kv=8)}), flush=True)
        return
    if args.phase == "lca":
        print(json.dumps({"phase": "lca", "lca_variant": lca_variant(binding, accounting, dev, args.seed)}),
              flush=True)
        return
    if args.phase == "serving":
        print(json.dumps({"phase": "serving",
                          "serving_decode": serving_decode(binding, accounting, dev, args.seed)}), flush=True)
        return
    stream = torch.cuda.current_stream()
    if args.config is None:
        pcfg = WORKLOADS[4] if args.phase in ("all", "prefill") else None
        dcfg = WORKLOADS[5] if args.phase in ("all", "decode") else None
    else:
        sel = WORKLOADS[args.config]
        pcfg = sel if sel["kind"] == "prefill" else None
        dcfg = sel if sel["kind"] == "decode" else None
    do_prefill = pcfg is not None
    do_decode = dcfg is not None
    extras = args.config is None and args.phase == "all"
    cpu_dec_steps = 64    # steps of the decode workload the oracle replays (four pooling steps)

    # ---- inputs (resident in HBM before timing)
    if do_prefill:
        ptdt = torch.float32 if pcfg["dtype"] == "f32" else torch.bfloat16
        PB, PH, PL, Pd, Pg, Pk = (pcfg[x] for x in ("B", "H", "L", "d", "g", "k_local"))
        pscale = 1.0 / math.sqrt(Pd)
        q, k, v = torch_inputs(PB, PH, PL, Pd, ptdt, dev, seed=args.seed, heavy_frac=pcfg["heavy"])
        kc = torch.empty((PB, PH, PL // Pg, Pd), dtype=ptdt, device=dev)
        vc = torch.empty_like(kc)
        out = torch.empty_like(q)
    if do_decode:
        DB, DH, Dd, Dg, Dk, DL0, DS = (dcfg[x] for x in ("B", "H", "d", "g", "k_local", "context", "steps"))
        dscale = 1.0 / math.sqrt(Dd)
        dq, dk, dv = torch_inputs(DB, DH, DL0 + DS, Dd, torch.bfloat16, dev, seed=args.seed + 1,
                                  heavy_frac=dcfg["heavy"])
        k0 = dk[:, :, :DL0].contiguous()
        v0 = dv[:, :, :DL0].contiguous()
        kc0, vc0 = binding.pool_kv(dq[:, :, :DL0].contiguous(), k0, v0, Dg, dscale)
        qs = dq[:, :, DL0:].permute(2, 0, 1, 3).contiguous()
        ks = dk[:, :, DL0:].permute(2, 0, 1, 3).contiguous()
        vs = dv[:, :, DL0:].permute(2, 0, 1, 3).contiguous()
        dec_sample = {}
        if not args.no_cpu_baseline:   # host copies of the slices whose steps the oracle replays
            for (b, h) in decode_sample_slices(DB, DH):
                n = DL0 + cpu_dec_steps
                dec_sample[(b, h)] = tuple(x[b, h, :n].cpu() for x in (dq, dk, dv))
        del dq, dk, dv
        cache = binding.KVCache(DB, DH, Dd, Dg, Dk, max_tokens=DL0 + DS, dtype=torch.bfloat16, device=dev)
        dout = torch.empty((DB, DH, Dd), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    pe = [ev() for _ in range(3)]
    de = [ev() for _ in range(2 * DS)] if do_decode else []
    t_pool, t_attn, t_dec, t_decstep, dec_all = [], [], [], [], []

    def one_step(record: bool):
        if do_prefill:
            pe[0].record(stream)
            binding.pool_kv(q, k, v, Pg, pscale, kc=kc, vc=vc)
            pe[1].record(stream)
            binding.attention(q, k, v, kc, vc, Pg, Pk, pscale, out=out)
            pe[2].record(stream)
        if do_decode:
            cache.desc.n_tokens = 0
            cache.desc.n_pooled = 0
            cache.load_prefill(k0, v0, kc0, vc0)
            for s in range(DS):
                de[2 * s].record(stream)
                cache.append_decode(qs[s], ks[s], vs[s], out=dout, scale=dscale)
                de[2 * s + 1].record(stream)
        torch.cuda.synchronize()
        if not record:
            return
        if do_prefill:
            t_pool.append(pe[0].elapsed_time(pe[1]))
            t_attn.append(pe[1].elapsed_time(pe[2]))
        if do_decode:
            per = [de[2 * s].elapsed_time(de[2 * s + 1]) for s in range(DS)]
            dec_all.extend(per)
            d = sum(per)
            w = de[0].elapsed_time(de[2 * DS - 1])
            t_dec.append(d / DS)       # kernel time per step
            t_decstep.append(w / DS)   # step-to-step time, launch gaps included

    for _ in range(args.warmup):
        one_step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    mean = lambda xs: sum(xs) / len(xs) if xs else float("nan")  # noqa: E731
    median = _median
    names = [workload_name(c) for c in (pcfg, dcfg) if c is not None]
    res = {
        "metric": METRIC,
        "value": None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": pcfg["dtype"] if do_prefill else dcfg["dtype"],
        "data": (f"synthetic: Q,K,V ~ N(0,1)"
                 + (", 1% of key rows x4 (heavy hitters)" if (pcfg or dcfg)["heavy"] else "")
                 + f", rounded (RNE) to the input type; seed {args.seed}"),
        "config": {
            "workload": ", then ".join(names),
            "phase": args.phase,
        },
    }
    if do_prefill:
        res["config"]["prefill"] = {x: pcfg[x] for x in ("B", "H", "d", "L", "g", "k_local", "dtype")}
    if do_decode:
        res["config"]["decode"] = {"B": DB, "H": DH, "d": Dd, "context": DL0, "steps": DS, "g": Dg, "k_local": Dk}
    if args.config is not None:
        res["config"]["index"] = args.config
    src_attn = source_hash("prefill.hip", "prefill_d128.hip", "cca_device.h")
    if do_prefill:
        ms_pool, ms_attn = median(t_pool), median(t_attn)   # medians over the timed steps
        ms_prefill = ms_pool + ms_attn
        elem = 4 if pcfg["dtype"] == "f32" else 2
        flops = accounting.prefill_flops(PB, PH, PL, Pd, Pg, Pk)
        pool_b = accounting.pool_bytes(PB, PH, PL, Pd, Pg, elem)
        tflops = flops / (ms_attn * 1e-3) / 1e12
        peak = PEAK_F32_TFLOPS if pcfg["dtype"] == "f32" else PEAK_BF16_TFLOPS
        res["value"] = PB * PL / (ms_prefill * 1e-3)
        res["prefill"] = {
            "ms": ms_prefill, "pool_ms": ms_pool, "attention_ms": ms_attn,
            "attention_ms_mean": mean(t_attn), "attention_ms_min": min(t_attn), "attention_ms_max": max(t_attn),
            "attention_tflops": tflops, "attention_flops": flops,
            "pool_gbs": pool_b / (ms_pool * 1e-3) / 1e9, "pool_bytes": pool_b,
            "pool_hbm_frac": pool_b / (ms_pool * 1e-3) / 1e9 / PEAK_HBM_GBS,
        }
        big = Pd == 128 and elem == 2
        res["roofline"] = {
            "kernel": "cca_prefill_d128_kernel<bf16>" if big else f"cca_prefill_kernel<{pcfg['dtype']},{Pd}>",
            "bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
            "frac": tflops / peak,
            "traffic": load_traffic("prefill_attention", src_attn) if pcfg is WORKLOADS[4] else None,
            "per_unit": "4*d FLOPs per visible (query, key) pair; pairs in closed form",
        }
        res_b, full_b = accounting.kv_cache_bytes(PL, Pg, Pk, PB, PH, Pd, elem)
        lib_res, lib_full = binding.kv_cache_bytes(PL, Pg, Pk, PB, PH, Pd, ptdt)
        assert (lib_res, lib_full) == (res_b, full_b)
        res["kv_cache"] = {"resident_bytes": res_b, "full_kv_bytes": full_b, "fraction": res_b / full_b,
                           "reduction": 1 - res_b / full_b, "page_reduction_128k": 0.93}
    if do_decode:
        nchunks = cache.ws_bytes // (DB * DH * (Dd + 2) * 4)   # chunk count the library chose
        byt = [accounting.decode_bytes(DB, DH, Dd, DL0 + s, Dg, Dk, 2, nchunks) for s in range(DS)]
        mean_bytes = sum(byt) / len(byt)
        us_dec = median(t_dec) * 1e3
        gbs = mean_bytes / (us_dec * 1e-6) / 1e9
        res["decode"] = {
            "us_per_step": median(t_decstep) * 1e3, "us_per_step_mean": mean(t_decstep) * 1e3,
            "kernel_us": us_dec, "kernel_us_mean": mean(t_dec) * 1e3, "kernel_us_p50_over_steps": median(dec_all) * 1e3,
            "chunks": nchunks,
            "bytes_per_step": mean_bytes,
            "tokens_per_s": DB / (median(t_decstep) * 1e-3),
            "roofline": {"kernel": "cca_decode_kernel<bf16,128,append> + cca_decode_merge_kernel",
                         "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS,
                         "traffic": load_traffic("decode", source_hash("decode.hip", "pool_group.h", "cca_device.h"))},
        }
        if not do_prefill:
            res["value"] = DB / (median(t_decstep) * 1e-3)   # tokens generated per second over the batch
            res["roofline"] = res["decode"]["roofline"]
        dec_gpu_out = None
        if not args.no_cpu_baseline:
            # the first steps again with fp32 outputs, for the oracle's parity check of the same steps
            cache.desc.n_tokens = 0
            cache.desc.n_pooled = 0
            cache.load_prefill(k0, v0, kc0, vc0)
            o32 = torch.empty((cpu_dec_steps, DB, DH, Dd), dtype=torch.float32, device=dev)
            for s in range(cpu_dec_steps):
                cache.append_decode(qs[s], ks[s], vs[s], out_dtype=torch.float32, out=o32[s], scale=dscale)
            torch.cuda.synchronize()
            dec_gpu_out = o32.cpu().numpy()
            del o32
    cpu = {}
    if do_decode and not args.no_cpu_baseline:
        _leg("cpu oracle: decode")
        cpu["decode"] = cpu_decode(dec_sample, dec_gpu_out, dcfg, cpu_dec_steps)
        del dec_sample
    if do_decode and not args.no_serving and extras:
        del cache, qs, ks, vs, k0, v0, kc0, vc0
        torch.cuda.empty_cache()
        _leg("serving")
        res["serving_decode"] = serving_decode(binding, accounting, dev, args.seed)
    if do_prefill and extras and not args.no_workloads:
        pw = {}
        for i in (1, 2, 3):
            c = WORKLOADS[i]
            name = f"prefill_{c['L']}_{c['dtype']}"
            _leg(name)
            pw[name] = prefill_workload(binding, accounting, dev, args.seed, c,
                                        cpu_seconds=0.0 if args.no_cpu_baseline else args.cpu_seconds)
            if "cpu_baseline" in pw[name]:
                cpu[name] = pw[name].pop("cpu_baseline")
        res["prefill_workloads"] = pw
    if do_prefill and not args.no_training and extras:
        _leg("training")
        res["training"] = training_step(binding, accounting, dev, args.seed)
        torch.cuda.empty_cache()
        res["training_gqa"] = training_step(binding, accounting, dev, args.seed, H_kv=8)
        torch.cuda.empty_cache()
    if do_prefill and not args.no_lca and extras:
        _leg("lca")
        res["lca_variant"] = lca_variant(binding, accounting, dev, args.seed)
        torch.cuda.empty_cache()
    if do_prefill and not args.no_f16 and extras:
        _leg("binary16")
        res["binary16_prefill"] = binary16_prefill(binding, accounting, dev, args.seed)
        if not args.no_training:
            res["binary16_training"] = training_step(binding, accounting, dev, args.seed, reps=2, dtype="f16")
    if do_prefill and not args.no_dense and extras:
        _leg("dense comparison")
        res["dense_comparison"] = dense_comparison(binding, accounting, dev, args.seed)
    if not args.no_cpu_baseline:
        _leg("cpu oracle: prefill")
        if do_prefill and pcfg is WORKLOADS[4]:
            out32 = binding.prefill(q, k, v, Pg, Pk, pscale, out_dtype=torch.float32)
            torch.cuda.synchronize()
            res["cpu_baseline"] = {**cpu_baseline(q, k, v, out32, args.cpu_seconds), **cpu}
        elif do_prefill:
            out32 = binding.prefill(q, k, v, Pg, Pk, pscale, out_dtype=torch.float32)
            torch.cuda.synchronize()
            res["cpu_baseline"] = cpu_prefill_heads(q, k, v, out32, pcfg, args.cpu_seconds)
        elif "decode" in cpu:
            res["cpu_baseline"] = cpu["decode"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
