// Chunked append: n new tokens per sequence in one call, each sequence at its own
// length, grouped-query heads; returns the attention output of every new token.
//
// Method: the CCA write-up ("ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"):
// a token at position p attends, in one softmax, to the core tokens of the groups
// before its raw window and to the raw keys (p/g - k)*g .. p (locality-preserving
// module, global-local fusion); a group's core token is pooled from its tokens with
// the group's last query (global-aware pooling) as soon as the group is complete,
// and the cache keeps core tokens plus the local raw tokens (Triton section, Fig. 3).
// A token's output depends only on its position and the tokens before it, so a
// chunk of n tokens gives the same rows as n single-token steps.
//
// Three launches:
//   1. gather: the raw keys/values a chunk can see -- positions raw0 .. pos+n-1 with
//      raw0 = max(0, pos/g - k)*g -- into one contiguous scratch slice per key/value
//      head: the cached part from the ring, the rest from the chunk itself;
//   2. attention: the prefill attention kernels in extend mode over that scratch
//      slice and the cached core tokens (MFMA, one softmax per query);
//   3. append: the chunk's keys/values go to their ring slots, every group the chunk
//      completes is pooled into its core slot (mean query over the query heads that
//      share the key/value head), and the sequence length advances by n.
// LCA-style cache: launch 3 condenses a completed group instead (mean of the group's
// queries over its positions and the query heads sharing the key/value head, positional
// dims from the top-scored token; "Latent-Condensed Transformer for Efficient Long Context
// Modeling", sections 2 and 3), taking the queries of the group's tokens before the chunk
// from the running sum qsum; a fourth launch then leaves in qsum the sum of the chunk's
// trailing incomplete group.
// With n <= k*g + 1 no token of the chunk can see a core token pooled from the same
// chunk (the earliest group it completes becomes visible k*g+1 positions after the
// chunk's first token), so pooling can follow the attention.  Launch 3 overwrites
// only ring slots whose positions no later step needs, after launches 1-2 read them.
#include <algorithm>

#include "cca_internal.h"
#include "lca_group.h"
#include "pool_group.h"

namespace cca {
namespace {

// Workspace head: the per-sequence start positions (int32), padded to 256 bytes.
size_t pos_bytes(int B) { return ((size_t)B * sizeof(int32_t) + 255) / 256 * 256; }

template <typename T, int D>
__global__ __launch_bounds__(256) void cca_extend_gather_kernel(const int32_t* __restrict__ lens, int64_t max_len,
                                                                int32_t* __restrict__ pos_ws,
                                                                const T* __restrict__ k_chunk,
                                                                const T* __restrict__ v_chunk,
                                                                const T* __restrict__ ring_k,
                                                                const T* __restrict__ ring_v, T* __restrict__ sk,
                                                                T* __restrict__ sv, int Hkv, int n, int64_t R, int g,
                                                                int k_local, int64_t raw_rows) {
  constexpr int CPR = D * (int)sizeof(T) / 16;
  const int64_t bkv = blockIdx.x;
  const int64_t b = bkv / Hkv;
  const int64_t t = lens[b];
  const bool valid = t >= 0 && t <= max_len;
  if (blockIdx.y == 0 && threadIdx.x == 0 && bkv % Hkv == 0) pos_ws[b] = valid ? (int32_t)t : -1;
  if (!valid) return;
  const int64_t raw0 = std::max<int64_t>(0, t / g - k_local) * g;
  const int64_t rows = t + n - raw0;
  const int64_t idx = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
  const int64_t u = idx / CPR;
  const int c = (int)(idx % CPR);
  if (u >= rows) return;
  const int64_t pos = raw0 + u;
  const T* srck;
  const T* srcv;
  if (pos < t) {
    const int64_t slot = pos % R;
    srck = ring_k + ((size_t)bkv * R + slot) * D;
    srcv = ring_v + ((size_t)bkv * R + slot) * D;
  } else {
    srck = k_chunk + ((size_t)bkv * n + (pos - t)) * D;
    srcv = v_chunk + ((size_t)bkv * n + (pos - t)) * D;
  }
  const size_t dst = ((size_t)bkv * raw_rows + u) * D;
  st16(reinterpret_cast<uint4*>(sk + dst) + c, ld16(reinterpret_cast<const uint4*>(srck) + c));
  st16(reinterpret_cast<uint4*>(sv + dst) + c, ld16(reinterpret_cast<const uint4*>(srcv) + c));
}

// Sum over the nq query heads h*nq .. of chunk row `row` for this lane's D/64 columns,
// added to s (q_chunk [B*Hq][n][D], head slices of sequence b).
template <typename T, int D>
__device__ __forceinline__ void add_query_row(const T* __restrict__ q_chunk, int64_t b, int Hq, int hk, int nq,
                                              int n, int64_t row, int col, float* s) {
  constexpr int CPL = D / kWave;
  float t[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) t[e] = 0.f;
  for (int h = 0; h < nq; ++h) {
    float f[CPL];
    lca_load_cols<T, D>(q_chunk + (((size_t)b * Hq + (size_t)hk * nq + h) * n + row) * D + col, f);
#pragma unroll
    for (int e = 0; e < CPL; ++e) t[e] += f[e];
  }
#pragma unroll
  for (int e = 0; e < CPL; ++e) s[e] += t[e];
}

// One wave per new token: its ring slot, and the pooling (LCA: condensation) of the group
// it completes.
template <typename T, int D, bool LCA>
__global__ __launch_bounds__(256) void cca_extend_append_kernel(
    int32_t* __restrict__ lens, const int32_t* __restrict__ pos_ws, const T* __restrict__ q_chunk,
    const T* __restrict__ k_chunk, const T* __restrict__ v_chunk, const T* __restrict__ sk,
    const T* __restrict__ sv, T* __restrict__ ring_k, T* __restrict__ ring_v, T* __restrict__ core_k,
    T* __restrict__ core_v, int Hkv, int nq, int n, int64_t R, int64_t max_groups, int g, int k_local,
    int64_t raw_rows, float scale, const float* __restrict__ qsum, int d_rope) {
  extern __shared__ float w_lds[];
  const int64_t bkv = blockIdx.x;
  const int64_t b = bkv / Hkv;
  const int hk = (int)(bkv - b * Hkv);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int64_t t = pos_ws[b];
  if (t < 0) return;
  if (blockIdx.y == 0 && threadIdx.x == 0 && hk == 0) lens[b] = (int32_t)(t + n);
  const int i = blockIdx.y * (blockDim.x / kWave) + wave;
  if (i >= n) return;
  const int64_t p = t + i;
  const T* kr = k_chunk + ((size_t)bkv * n + i) * D;
  const T* vr = v_chunk + ((size_t)bkv * n + i) * D;
  constexpr int CPR = D * (int)sizeof(T) / 16;
  const int64_t slot = p % R;
  if (lane < CPR) {
    st16(reinterpret_cast<uint4*>(ring_k + ((size_t)bkv * R + slot) * D) + lane,
         ld16(reinterpret_cast<const uint4*>(kr) + lane));
    st16(reinterpret_cast<uint4*>(ring_v + ((size_t)bkv * R + slot) * D) + lane,
         ld16(reinterpret_cast<const uint4*>(vr) + lane));
  }
  if ((p + 1) % g != 0) return;
  // group beta = p/g: positions p-g+1 .. p, all inside the scratch slice (they start at
  // or after the chunk's own group, which is not before raw0)
  const int64_t beta = p / g;
  const int64_t raw0 = std::max<int64_t>(0, t / g - k_local) * g;
  const size_t first = ((size_t)bkv * raw_rows + (p - g + 1 - raw0)) * D;
  const size_t last = ((size_t)bkv * raw_rows + (p - raw0)) * D;
  const int Hq = Hkv * nq;
  if constexpr (LCA) {
    // the group's queries: chunk rows i-g+1 .. i, or the running sum of its tokens before
    // the chunk followed by rows 0 .. i (token order, heads first, as the decode steps add them)
    constexpr int CPL = D / kWave;
    const int col = lane * CPL;
    float s[CPL];
    int64_t r0 = (int64_t)i - g + 1;
    if (r0 < 0) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) s[e] = qsum[(size_t)bkv * D + col + e];
      r0 = 0;
    } else {
#pragma unroll
      for (int e = 0; e < CPL; ++e) s[e] = 0.f;
    }
    for (int64_t r = r0; r <= i; ++r) add_query_row<T, D>(q_chunk, b, Hq, hk, nq, n, r, col, s);
    float* qbar = w_lds + wave * (D + g);
    const float inv = 1.0f / ((float)g * (float)nq);
#pragma unroll
    for (int e = 0; e < CPL; ++e) qbar[col + e] = s[e] * inv;
    wave_lds_sync();
    lca_condense_wave<T, D>(qbar, sk + first, sv + first, sk + last, sv + last, g, scale, d_rope,
                            core_k + ((size_t)bkv * max_groups + beta) * D,
                            core_v + ((size_t)bkv * max_groups + beta) * D, qbar + D, nullptr);
  } else {
    pool_group_wave<T, D>(q_chunk + (((size_t)b * Hq + (size_t)hk * nq) * n + i) * D, (int64_t)n * D, nq,
                          sk + first, sv + first, sk + last, sv + last, g, scale,
                          core_k + ((size_t)bkv * max_groups + beta) * D,
                          core_v + ((size_t)bkv * max_groups + beta) * D, w_lds + wave * g);
  }
}

// LCA-style cache, after the append launch (which read the sums at the chunk's start): one
// wave per key/value slice leaves in qsum the sum of the queries of the trailing incomplete
// group -- the chunk's rows after its last completed group, plus the previous sum when the
// chunk completes no group.
template <typename T, int D>
__global__ __launch_bounds__(64) void cca_extend_qsum_kernel(const int32_t* __restrict__ pos_ws,
                                                            const T* __restrict__ q_chunk, float* __restrict__ qsum,
                                                            int Hkv, int nq, int n, int g) {
  constexpr int CPL = D / kWave;
  const int64_t bkv = blockIdx.x;
  const int64_t b = bkv / Hkv;
  const int hk = (int)(bkv - b * Hkv);
  const int64_t t = pos_ws[b];
  if (t < 0) return;
  const int col = threadIdx.x * CPL;
  const int64_t end = t + n;
  const bool completes = end / g > t / g;
  float s[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) s[e] = completes ? 0.f : qsum[(size_t)bkv * D + col + e];
  const int64_t r0 = completes ? end / g * g - t : 0;
  for (int64_t r = r0; r < n; ++r) add_query_row<T, D>(q_chunk, b, Hkv * nq, hk, nq, n, r, col, s);
#pragma unroll
  for (int e = 0; e < CPL; ++e) qsum[(size_t)bkv * D + col + e] = s[e];
}

template <typename T, int D>
hipError_t launch_extend_t(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q, int n, const void* q,
                           const void* k, const void* v, void* out, int out_f32, void* workspace, float scale,
                           float* qsum, int d_rope, hipStream_t stream) {
  const int64_t R = (int64_t)(c->k_local + 1) * c->g;
  const int64_t raw_rows = R + n;
  const int64_t BHkv = (int64_t)c->B * c->H;
  const int nq = H_q / c->H;
  int32_t* pos_ws = (int32_t*)workspace;
  T* sk = (T*)((uint8_t*)workspace + pos_bytes(c->B));
  T* sv = sk + (size_t)BHkv * raw_rows * D;
  constexpr int CPR = D * (int)sizeof(T) / 16;
  const int64_t gy = (raw_rows * CPR + 255) / 256;
  hipLaunchKernelGGL((cca_extend_gather_kernel<T, D>), dim3((unsigned)BHkv, (unsigned)gy), dim3(256), 0, stream, lens,
                     max_len, pos_ws, (const T*)k, (const T*)v, (const T*)c->ring_k, (const T*)c->ring_v, sk, sv, c->H,
                     n, R, c->g, c->k_local, raw_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const ExtendArgs ext{pos_ws, H_q, n, raw_rows, c->max_groups};
  e = launch_extend_attention(c->dt, D, q, sk, sv, c->core_k, c->core_v, out, out_f32, c->B * H_q, nq, c->g,
                              c->k_local, scale, ext, stream);
  if (e != hipSuccess) return e;
  const dim3 agrid((unsigned)BHkv, (unsigned)((n + 3) / 4));
  if (qsum == nullptr) {
    hipLaunchKernelGGL((cca_extend_append_kernel<T, D, false>), agrid, dim3(256), (size_t)4 * c->g * sizeof(float),
                       stream, lens, pos_ws, (const T*)q, (const T*)k, (const T*)v, (const T*)sk, (const T*)sv,
                       (T*)c->ring_k, (T*)c->ring_v, (T*)c->core_k, (T*)c->core_v, c->H, nq, n, R, c->max_groups,
                       c->g, c->k_local, raw_rows, scale, (const float*)nullptr, 0);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((cca_extend_append_kernel<T, D, true>), agrid, dim3(256),
                     (size_t)4 * (D + c->g) * sizeof(float), stream, lens, pos_ws, (const T*)q, (const T*)k,
                     (const T*)v, (const T*)sk, (const T*)sv, (T*)c->ring_k, (T*)c->ring_v, (T*)c->core_k,
                     (T*)c->core_v, c->H, nq, n, R, c->max_groups, c->g, c->k_local, raw_rows, scale,
                     (const float*)qsum, d_rope);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((cca_extend_qsum_kernel<T, D>), dim3((unsigned)BHkv), dim3(64), 0, stream,
                     (const int32_t*)pos_ws, (const T*)q, qsum, c->H, nq, n, c->g);
  return hipGetLastError();
}

}  // namespace

size_t extend_workspace_bytes(const cca_cache_t* c, int n) {
  const size_t R = (size_t)(c->k_local + 1) * c->g;
  const size_t esz = (size_t)dtype_bytes(c->dt);
  return pos_bytes(c->B) + 2 * (size_t)c->B * c->H * (R + (size_t)n) * c->d * esz;
}

hipError_t launch_extend(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q, int n, const void* q,
                         const void* k, const void* v, void* out, int out_f32, void* workspace, float scale,
                         hipStream_t stream, float* qsum, int d_rope) {
  return dispatch_td(c->dt, c->d, [&](auto t, auto dd) {
    using T = decltype(t);
    return launch_extend_t<T, decltype(dd)::value>(c, lens, max_len, H_q, n, q, k, v, out,
                                                   sizeof(T) == 4 ? 1 : out_f32, workspace, scale, qsum, d_rope,
                                                   stream);
  });
}

}  // namespace cca
