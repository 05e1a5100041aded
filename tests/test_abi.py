"""CPU checks of the C ABI: the library loads, exports every declared entry point,
and its host-side validation / accounting behave as include/cca.h states.
None of these calls reaches the GPU (validation fails before any launch)."""
import ctypes
import os
import re

import pytest

import oracle
from long_context_sparse_cca_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from long_context_sparse_cca_amd import build
        build.build()
    return binding.load_library()


def _declared():
    text = open(os.path.join(ROOT, "include", "cca.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cca_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert "cca_prefill" in names and "cca_decode_step" in names and len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert set(names) == set(binding.EXPORTS), "binding and header disagree"


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.cca_status_string(code)
    assert lib.cca_status_string(123) == b"unknown status"


def test_validation_without_gpu(lib):
    NULL = None
    # null pointers
    assert lib.cca_pool_kv(NULL, NULL, NULL, NULL, NULL, 1, 1, 16, 128, 16, 0.1, 1, NULL) == -1
    # unsupported head dim / dtype are reported before pointers are looked at
    assert lib.cca_pool_kv(NULL, NULL, NULL, NULL, NULL, 1, 1, 16, 96, 16, 0.1, 1, NULL) == -2
    assert lib.cca_prefill(NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 16, 128, 16, 1, 0.1, 7, 0, NULL) == -2
    # group size out of range
    assert lib.cca_prefill(NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 16, 128, 0, 1, 0.1, 1, 0, NULL) == -1
    # cache calls with a null / inconsistent descriptor
    assert lib.cca_cache_append(None, NULL, NULL, NULL, 0.1, NULL) == -1
    d = binding.CacheDesc(16, 16, 16, 16, 1, 1, 128, 16, 2, 1, 4, 0, 1)  # n_pooled inconsistent
    assert lib.cca_cache_append(ctypes.byref(d), 16, 16, 16, 0.1, NULL) == -1
    d = binding.CacheDesc(16, 16, 16, 16, 1, 1, 128, 16, 2, 1, 4, 0, 0)
    assert lib.cca_decode_step(ctypes.byref(d), 16, 16, 0, 16, 0, 0.1, NULL) == -1  # no token yet
    d.n_tokens, d.n_pooled = 5, 0
    assert lib.cca_decode_step(ctypes.byref(d), 16, 16, 0, 16, 0, 0.1, NULL) == -3  # workspace too small
    assert lib.cca_cache_ring_slots(ctypes.byref(d)) == 48
    d.n_tokens, d.n_pooled = 79, 4   # next append would complete group 4 with max_groups = 4
    assert lib.cca_cache_append(ctypes.byref(d), 16, 16, 16, 0.1, NULL) == -5
    assert d.n_tokens == 79


def test_noalloc_decode_validation_without_gpu(lib):
    """The allocation-free decode validates the descriptor, then the size of its partial states
    against the library's fixed array, before touching the device."""
    NULL = None
    assert lib.cca_cache_append_decode_noalloc(None, 16, 16, 16, 16, 0, 0.1, NULL) == -1
    d = binding.CacheDesc(16, 16, 16, 16, 1, 1, 128, 16, 2, 1, 4, 0, 1)  # n_pooled inconsistent
    assert lib.cca_cache_append_decode_noalloc(ctypes.byref(d), 16, 16, 16, 16, 0, 0.1, NULL) == -1
    # B*H = 8192 slices at d = 128: one chunk each, 8192*130*4 bytes > 4 MiB
    d = binding.CacheDesc(16, 16, 16, 16, 128, 64, 128, 16, 1, 1, 1, 0, 0)
    assert lib.cca_decode_workspace_bytes(ctypes.byref(d)) > 4 << 20
    assert lib.cca_cache_append_decode_noalloc(ctypes.byref(d), 16, 16, 16, 16, 0, 0.1, NULL) == -3
    assert d.n_tokens == 0


def test_workspace_size(lib):
    d = binding.CacheDesc(16, 16, 16, 16, 8, 32, 128, 16, 64, 1, 8208, 0, 0)
    n = lib.cca_decode_workspace_bytes(ctypes.byref(d))
    assert n > 0 and n % (8 * 32 * 130 * 4) == 0   # whole chunks of (d+2)-float partial states
    d.max_groups = 0
    assert lib.cca_decode_workspace_bytes(ctypes.byref(d)) == 0


@pytest.mark.parametrize("n,g,k,B,H,d,dt", [(131072, 16, 64, 1, 32, 128, 1), (1000, 7, 3, 2, 4, 64, 0),
                                            (5, 16, 0, 1, 1, 128, 1), (0, 4, 2, 1, 1, 64, 0),
                                            (65536, 16, 64, 2, 8, 128, 2)])
def test_kv_cache_bytes_match_oracle(lib, n, g, k, B, H, d, dt):
    r, f = ctypes.c_int64(), ctypes.c_int64()
    assert lib.cca_kv_cache_bytes(n, g, k, B, H, d, dt, ctypes.byref(r), ctypes.byref(f)) == 0
    assert (r.value, f.value) == oracle.kv_cache_bytes(n, g, k, B, H, d, 4 if dt == 0 else 2)


@pytest.mark.parametrize("L,g,k", [(131072, 16, 64), (8192, 16, 64), (256, 16, 1), (1000, 7, 3), (37, 4, 1),
                                   (10, 16, 1), (5, 1, 0), (100, 3, 50), (4097, 64, 2)])
def test_benchmark_pair_count_matches_oracle(L, g, k):
    """The closed form the benchmark uses for FLOPs equals the oracle's per-query enumeration."""
    from long_context_sparse_cca_amd import accounting
    assert accounting.attention_pairs(L, g, k) == oracle.attention_pairs(L, g, k)
    assert accounting.kv_cache_bytes(L, g, k, 2, 3, 64, 2) == oracle.kv_cache_bytes(L, g, k, 2, 3, 64, 2)
    assert sum(accounting.attention_pairs(L, g, k)) == sum(
        accounting.decode_keys(t, g, k) for t in range(L))


def test_validation_of_training_lca_and_serving_calls(lib):
    """Host-side validation of the training, LCA-style and serving entry points (no launch)."""
    P = ctypes.c_void_p(256)          # a 16-byte aligned stand-in that is never dereferenced
    NULL = None
    # training: head counts that do not divide, an unbuilt head dim, a short workspace
    assert lib.cca_prefill_lse_gqa(P, P, P, P, P, P, P, 1, 4, 3, 64, 128, 16, 1, 0.1, 1, 1, NULL) == -1
    assert lib.cca_backward_gqa(P, P, P, P, P, P, P, P, P, P, P, P, 1 << 30, 1, 2, 2, 64, 96, 16, 1, 0.1, 1,
                                NULL) == -2
    need = lib.cca_backward_gqa_workspace_bytes(1, 4, 2, 640, 128, 16)
    assert need == (2 * 4 * 640 + 2 * 2 * (640 // 16) * 128) * 4
    assert lib.cca_backward_gqa(P, P, P, P, P, P, P, P, P, P, P, P, need - 1, 1, 4, 2, 640, 128, 16, 1, 0.1, 1,
                                NULL) == -3
    assert lib.cca_backward_gqa_workspace_bytes(1, 4, 3, 640, 128, 16) == 0
    # LCA-style: positional width outside [0, d]
    assert lib.cca_pool_kv_lca(P, P, P, P, P, NULL, 1, 1, 64, 128, 16, 129, 0.1, 1, NULL) == -1
    assert lib.cca_pool_kv_lca(P, P, P, P, P, NULL, 1, 1, 64, 128, 16, -1, 0.1, 1, NULL) == -1
    # LCA-style serving: running sums missing, positional width, head multiple, chunk size
    d = binding.CacheDesc(256, 256, 256, 256, 2, 2, 128, 16, 2, 1, 64, 0, 0)
    assert lib.cca_cache_append_decode_varlen_lca(ctypes.byref(d), NULL, 64, P, 10, 4, P, P, P, P, 1, P, 1 << 30,
                                                  0.1, NULL) == -1
    assert lib.cca_cache_append_decode_varlen_lca(ctypes.byref(d), P, 129, P, 10, 4, P, P, P, P, 1, P, 1 << 30,
                                                  0.1, NULL) == -1
    assert lib.cca_cache_append_decode_varlen_lca(ctypes.byref(d), P, 64, P, 10, 3, P, P, P, P, 1, P, 1 << 30,
                                                  0.1, NULL) == -1
    assert lib.cca_cache_extend_lca(ctypes.byref(d), P, 64, P, 10, 4, 2 * 16 + 2, P, P, P, P, 1, P, 1 << 30, 0.1,
                                    NULL) == -1
    assert lib.cca_cache_extend_lca(ctypes.byref(d), NULL, 64, P, 10, 4, 4, P, P, P, P, 1, P, 1 << 30, 0.1,
                                    NULL) == -1
    # capacity: 64 core slots hold 1024 tokens; a step at position 1023 completes group 63, 1039 needs slot 64
    assert lib.cca_cache_append_decode_varlen(ctypes.byref(d), P, 1040, 4, P, P, P, P, 1, P, 1 << 30, 0.1,
                                              NULL) == -5
    assert lib.cca_cache_load_prefill_lca_gqa(ctypes.byref(d), P, 3, P, P, P, P, P, 100, NULL) == -1
    # a short serving workspace
    ws = lib.cca_serve_workspace_bytes(ctypes.byref(d), 4)
    assert ws > 0 and lib.cca_serve_workspace_bytes(ctypes.byref(d), 3) == 0
    assert lib.cca_cache_append_decode_varlen(ctypes.byref(d), P, 100, 4, P, P, P, P, 1, P, ws - 1, 0.1,
                                              NULL) == -3


def test_extend_rejects_chunks_completing_too_many_groups(lib):
    """A chunk completes at most n/g + 1 groups, each pooled by one wave of the finish launch;
    beyond 131068 groups the call is refused before any launch (g = 1 and a window of 200000
    groups allow such chunks).  At the limit validation goes on (here: to the workspace check)."""
    P = ctypes.c_void_p(256)
    d = binding.CacheDesc(256, 256, 256, 256, 1, 1, 64, 1, 200000, 0, 1 << 20, 0, 0)
    assert lib.cca_cache_extend(ctypes.byref(d), P, 10, 1, 131068, P, P, P, P, 0, P, 1, 0.1, None) == -2
    assert lib.cca_cache_extend(ctypes.byref(d), P, 10, 1, 131067, P, P, P, P, 0, P, 1, 0.1, None) == -3


def test_extend_chunk_size_bounds(lib):
    """A chunk holds 1 .. k*g + 1 tokens (then no query of the chunk sees a core token pooled
    from the chunk itself); an empty or longer chunk is refused before any launch."""
    P = ctypes.c_void_p(256)
    g, k = 16, 4
    d = binding.CacheDesc(256, 256, 256, 256, 1, 1, 64, g, k, 0, 1 << 20, 0, 0)
    for n in (0, -1, k * g + 2):
        assert lib.cca_cache_extend(ctypes.byref(d), P, 10, 1, n, P, P, P, P, 0, P, 1 << 30, 0.1, None) == -1
    # the largest chunk passes validation up to the workspace check (workspace of 1 byte)
    assert lib.cca_cache_extend(ctypes.byref(d), P, 10, 1, k * g + 1, P, P, P, P, 0, P, 1, 0.1, None) == -3


def test_unknown_dtype_rejected_before_any_launch(lib):
    """A dtype code outside {F32, BF16, F16} is refused by host-side validation (no device
    call is made, so this runs without a GPU)."""
    r, f = ctypes.c_int64(), ctypes.c_int64()
    assert lib.cca_kv_cache_bytes(100, 16, 2, 1, 1, 128, 3, ctypes.byref(r), ctypes.byref(f)) == -2
    null = ctypes.c_void_p(0)
    assert lib.cca_prefill(null, null, null, null, null, null, 1, 1, ctypes.c_int64(64), 128, 16, 1,
                           ctypes.c_float(0.1), 3, 3, null) == -2
    assert lib.cca_pool_kv(null, null, null, null, null, 1, 1, ctypes.c_int64(64), 128, 16,
                           ctypes.c_float(0.1), 7, null) == -2


def test_empty_sequence_is_a_no_op_with_null_pointers(lib):
    """L = 0: sizes, dtypes and scalars are still checked; then the pooling, prefill, attention
    and backward calls return 0 without looking at their (here NULL) data pointers and
    without touching the device."""
    N = None
    nan = float("nan")
    for B, H, Hkv in ((1, 1, 1), (2, 8, 2)):
        assert lib.cca_pool_kv_gqa(N, N, N, N, N, B, H, Hkv, 0, 128, 16, 0.1, 1, N) == 0
        assert lib.cca_prefill_gqa(N, N, N, N, N, N, B, H, Hkv, 0, 128, 16, 4, 0.1, 1, 0, N) == 0
        assert lib.cca_attention_gqa(N, N, N, N, N, N, B, H, Hkv, 0, 64, 16, 4, 0.1, 0, 0, N) == 0
        assert lib.cca_prefill_lse_gqa(N, N, N, N, N, N, N, B, H, Hkv, 0, 128, 16, 4, 0.1, 2, 2, N) == 0
        assert lib.cca_backward_gqa(N, N, N, N, N, N, N, N, N, N, N, N, 0, B, H, Hkv, 0, 128, 16, 4, 0.1, 1, N) == 0
        assert lib.cca_pool_kv_lca_gqa(N, N, N, N, N, N, B, H, Hkv, 0, 128, 16, 32, 0.1, 1, N) == 0
        assert lib.cca_prefill_lca_gqa(N, N, N, N, N, N, N, B, H, Hkv, 0, 128, 16, 4, 32, 0.1, 1, 0, N) == 0
    assert lib.cca_pool_kv(N, N, N, N, N, 1, 1, 0, 64, 7, 0.1, 0, N) == 0
    assert lib.cca_prefill(N, N, N, N, N, N, 1, 1, 0, 64, 7, 0, 0.1, 0, 0, N) == 0
    # the checks before the no-op still apply
    assert lib.cca_prefill(N, N, N, N, N, N, 1, 1, 0, 96, 16, 1, 0.1, 1, 0, N) == -2      # head dim
    assert lib.cca_prefill(N, N, N, N, N, N, 1, 1, 0, 128, 16, 1, 0.1, 1, 2, N) == -2     # out dtype
    assert lib.cca_prefill(N, N, N, N, N, N, 1, 1, 0, 128, 0, 1, 0.1, 1, 0, N) == -1      # g = 0
    assert lib.cca_prefill(N, N, N, N, N, N, 1, 1, 0, 128, 16, -1, 0.1, 1, 0, N) == -1    # k_local < 0
    assert lib.cca_prefill(N, N, N, N, N, N, 1, 1, 0, 128, 16, 1, nan, 1, 0, N) == -1     # scale
    assert lib.cca_prefill(N, N, N, N, N, N, 1, 1, -1, 128, 16, 1, 0.1, 1, 0, N) == -1    # L < 0
    assert lib.cca_prefill_gqa(N, N, N, N, N, N, 1, 6, 4, 0, 128, 16, 1, 0.1, 1, 0, N) == -1  # head multiple
    assert lib.cca_pool_kv(N, N, N, N, N, 1, 1, 0, 128, 16, nan, 1, N) == -1
    assert lib.cca_prefill_lca_gqa(N, N, N, N, N, N, N, 1, 1, 1, 0, 128, 16, 4, 129, 0.1, 1, 0, N) == -1  # d_rope
    assert lib.cca_pool_kv_lca_gqa(N, N, N, N, N, N, 1, 1, 1, 0, 128, 16, -1, 0.1, 1, N) == -1
    # one token: the pointers are looked at again
    assert lib.cca_prefill(N, N, N, N, N, N, 1, 1, 1, 128, 16, 1, 0.1, 1, 0, N) == -1
