// LCA-style pooling variant: group importance from the group's mean query, content
// dimensions pooled, positional dimensions taken from the top-scored token.
//
// Method: "Latent-Condensed Transformer for Efficient Long Context Modeling",
// section 2: tokens of a group are scored by the dot product of the group's mean
// query with their keys; the content part is condensed by importance-weighted
// pooling; the positional (RoPE) part is not mixed -- the highest-scoring token is
// the group's anchor and keeps its positional key.  Here the last d_rope dims of
// a key are its positional part; values are pooled entirely.  The condensed
// groups then take the place of CCA's core tokens in the unified attention.
//
// One wave per group, HBM-bound: the group's g query rows (of each of the nq query
// heads that share the key/value head), key rows and value rows are each read once.
// 16-bit inputs at d = 128, g = 16 take a kernel that stages the whole group in LDS up front.
#include <type_traits>

#include "cca_internal.h"
#include "lca_group.h"

namespace cca {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(64) void cca_pool_lca_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                          const T* __restrict__ V, T* __restrict__ Kc,
                                                          T* __restrict__ Vc, int32_t* __restrict__ anchors,
                                                          int64_t L, int g, int64_t m, int nq, int d_rope,
                                                          float scale) {
  extern __shared__ float sm[];   // mean query [D], then scores [g]
  float* qbar = sm;
  constexpr int CPL = D / kWave;
  const int64_t gid = blockIdx.x;
  const int64_t bh = gid / m, j = gid - bh * m;   // key/value slice, group
  const int lane = threadIdx.x;
  const size_t row0 = ((size_t)bh * L + (size_t)j * g) * D;
  const int col = lane * CPL;

  // ---- mean query of the group: each lane sums its columns over the g rows of each of
  // the nq query slices bh*nq .. that read this key/value slice
  {
    float s[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) s[e] = 0.f;
    for (int h = 0; h < nq; ++h) {
      const T* qg = Q + (((size_t)bh * nq + h) * L + (size_t)j * g) * D;
      for (int r = 0; r < g; ++r) {
        float f[CPL];
        lca_load_cols<T, D>(qg + (size_t)r * D + col, f);
#pragma unroll
        for (int e = 0; e < CPL; ++e) s[e] += f[e];
      }
    }
    const float inv_g = 1.0f / ((float)g * (float)nq);
#pragma unroll
    for (int e = 0; e < CPL; ++e) qbar[col + e] = s[e] * inv_g;
  }
  wave_lds_sync();
  const size_t out = ((size_t)bh * m + j) * D;
  lca_condense_wave<T, D>(qbar, K + row0, V + row0, K + row0 + (size_t)(g - 1) * D, V + row0 + (size_t)(g - 1) * D,
                          g, scale, d_rope, Kc + out, Vc + out, sm + D,
                          anchors != nullptr ? anchors + (size_t)bh * m + j : nullptr);
}

// 16-bit inputs, d = 128, g = 16: the same arithmetic as the kernel above (the mean query
// summed head by head and row by row, then lca_condense_math, so every caller of the group
// routine reaches the same condensed tokens), with the group's rows staged in LDS up front
// instead of fetched pass by pass: the key and value rows and the first head's query rows go
// straight from HBM into LDS (global_load_lds, 16 bytes per lane, each row fetched once), and
// every pass then reads LDS.  Four waves per workgroup, one group each, 12 KB of LDS per wave.
// STREAM: query and value rows, read once, carry the nontemporal hint (passes larger than
// the last-level cache).
template <typename T, bool STREAM>
__global__ __launch_bounds__(256) void cca_pool_lca_d128_g16_kernel(const T* __restrict__ Q,
                                                                    const T* __restrict__ K,
                                                                    const T* __restrict__ V, T* __restrict__ Kc,
                                                                    T* __restrict__ Vc,
                                                                    int32_t* __restrict__ anchors, int64_t L,
                                                                    int64_t m, int64_t n_groups, int nq,
                                                                    int d_rope, float scale) {
  constexpr int D = 128, G = 16, CPL = D / kWave, ROW = D * 2, MAT = G * ROW;
  __shared__ __attribute__((aligned(16))) uint8_t rows_lds[4][3 * MAT];   // per wave: Q, K, V rows
  __shared__ float sm[4][D + G];                                          // mean query, scores
  const int wv = threadIdx.x >> 6;
  const int64_t gid = (int64_t)blockIdx.x * 4 + wv;
  if (gid >= n_groups) return;     // whole waves only; the waves never synchronise with each other
  const int lane = threadIdx.x & (kWave - 1);
  const int col = lane * CPL;
  const int rsub = lane >> 2, seg = lane & 3;   // scoring pass: 4 lanes per key row
  const int64_t bh = gid / m, j = gid - bh * m;
  const size_t row0 = ((size_t)bh * L + (size_t)j * G) * D;
  uint8_t* qs = rows_lds[wv];
  uint8_t* ks = qs + MAT;
  uint8_t* vs = ks + MAT;
  // one fill instruction: rows 4i .. 4i+3 of a matrix; lane l brings 16-byte chunk l%16 of row 4i + l/16
  const int fill = (lane >> 4) * D + (lane & 15) * 8;   // element offset of this lane's chunk
  // stream_tag: std::true_type for rows read once (nontemporal cache policy), else false_type
  auto fill_rows = [&](const T* src, uint8_t* dst, auto stream_tag) {
    constexpr int kPolicy = decltype(stream_tag)::value ? 2 : 0;
#pragma unroll
    for (int i = 0; i < G / 4; ++i)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + (size_t)i * 4 * D + fill),
                                       (__attribute__((address_space(3))) void*)(dst + i * 4 * ROW), 16, 0,
                                       kPolicy);
  };
  using once = std::integral_constant<bool, STREAM>;
  fill_rows(K + row0, ks, std::false_type{});
  fill_rows(V + row0, vs, once{});
  const T* q0 = Q + ((size_t)bh * nq * L + (size_t)j * G) * D;
  fill_rows(q0, qs, once{});

  // ---- mean query of the group, summed in the order of the generic kernel
  float* qbar = sm[wv];
  {
    float s[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) s[e] = 0.f;
    for (int h = 0; h < nq; ++h) {
      if (h > 0) {
        // the previous head's rows are consumed (their values sit in s; lgkmcnt(0) makes sure
        // its LDS reads have completed): refill the buffer
        __builtin_amdgcn_s_waitcnt(0xC07F);
        fill_rows(q0 + (size_t)h * L * D, qs, once{});
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this head's rows (and K, V) are in LDS
#pragma unroll
      for (int r = 0; r < G; ++r) {
        float f[CPL];
        Elem<T>::pair_to_f32(*reinterpret_cast<const uint32_t*>(qs + r * ROW + col * 2), f);
#pragma unroll
        for (int e = 0; e < CPL; ++e) s[e] += f[e];
      }
    }
    const float inv_g = 1.0f / ((float)G * (float)nq);
#pragma unroll
    for (int e = 0; e < CPL; ++e) qbar[col + e] = s[e] * inv_g;
  }
  wave_lds_sync();
  const size_t out = ((size_t)bh * m + j) * D;
  lca_condense_math<T, D, G>(
      qbar, G, scale, d_rope, Kc + out, Vc + out, sm[wv] + D,
      anchors != nullptr ? anchors + (size_t)bh * m + j : nullptr,
      [&](int r, int c) { return *reinterpret_cast<const uint4*>(ks + r * ROW + seg * (ROW / 4) + c * 16); },
      [&](int r, float* f) { Elem<T>::pair_to_f32(*reinterpret_cast<const uint32_t*>(ks + r * ROW + col * 2), f); },
      [&](int r, float* f) { Elem<T>::pair_to_f32(*reinterpret_cast<const uint32_t*>(vs + r * ROW + col * 2), f); },
      [&](int r, float* f) { Elem<T>::pair_to_f32(*reinterpret_cast<const uint32_t*>(ks + r * ROW + col * 2), f); });
}

template <typename T, int D>
hipError_t launch_t(const void* q, const void* k, const void* v, void* kc, void* vc, int32_t* anchors, int BHkv,
                    int64_t L, int g, int nq, int d_rope, float scale, hipStream_t stream) {
  const int64_t m = L / g;
  const int64_t n = (int64_t)BHkv * m;
  if (n == 0) return hipSuccess;
  if constexpr (D == 128 && sizeof(T) == 2) {
    if (g == 16) {
      const dim3 grid((unsigned)((n + 3) / 4));
      if (n * 16 * 128 * 2 * (2 + nq) > kStreamBytes)
        hipLaunchKernelGGL((cca_pool_lca_d128_g16_kernel<T, true>), grid, dim3(256), 0, stream, (const T*)q,
                           (const T*)k, (const T*)v, (T*)kc, (T*)vc, anchors, L, m, n, nq, d_rope, scale);
      else
        hipLaunchKernelGGL((cca_pool_lca_d128_g16_kernel<T, false>), grid, dim3(256), 0, stream, (const T*)q,
                           (const T*)k, (const T*)v, (T*)kc, (T*)vc, anchors, L, m, n, nq, d_rope, scale);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((cca_pool_lca_kernel<T, D>), dim3((unsigned)n), dim3(64), (size_t)(D + g) * sizeof(float),
                     stream, (const T*)q, (const T*)k, (const T*)v, (T*)kc, (T*)vc, anchors, L, g, m, nq, d_rope,
                     scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool_lca(int dt, int d, const void* q, const void* k, const void* v, void* kc, void* vc,
                           int32_t* anchors, int BHkv, int64_t L, int g, int nq, int d_rope, float scale,
                           hipStream_t stream) {
  return dispatch_td(dt, d, [&](auto t, auto dd) {
    return launch_t<decltype(t), decltype(dd)::value>(q, k, v, kc, vc, anchors, BHkv, L, g, nq, d_rope, scale,
                                                      stream);
  });
}

}  // namespace cca
