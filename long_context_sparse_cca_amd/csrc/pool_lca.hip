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
// 16-bit inputs at d = 128, g = 16 take a kernel that fetches the whole group up front.
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
// routine reaches the same condensed tokens), with every row of the group fetched up front
// instead of pass by pass: the query rows of the nq heads (this lane's two columns), the key
// segment of the scoring pass, and the key and value columns of the weighted sums (the
// second fetch of a key row hits the cache).  Four waves per workgroup, one group each.
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
  constexpr int D = 128, G = 16, CPL = D / kWave;
  __shared__ float sm[4][D + G];   // per wave: mean query [D], then scores [G]
  const int wv = threadIdx.x >> 6;
  const int64_t gid = (int64_t)blockIdx.x * 4 + wv;
  if (gid >= n_groups) return;     // whole waves only; the waves never synchronise with each other
  const int lane = threadIdx.x & (kWave - 1);
  const int col = lane * CPL;
  const int rsub = lane >> 2, seg = lane & 3;   // scoring pass: 4 lanes per key row
  const int64_t bh = gid / m, j = gid - bh * m;
  const size_t row0 = ((size_t)bh * L + (size_t)j * G) * D;
  const T* kg = K + row0;
  const T* vg = V + row0;

  uint4 kseg[D / 4 / 8];
#pragma unroll
  for (int c = 0; c < D / 4 / 8; ++c) kseg[c] = ld16(kg + (size_t)rsub * D + seg * (D / 4) + c * 8);
  auto ld4 = [](const T* p) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
    if constexpr (STREAM) return __builtin_nontemporal_load(w);
    else return *w;
  };
  uint32_t kcol[G], vcol[G];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    kcol[r] = *reinterpret_cast<const uint32_t*>(kg + (size_t)r * D + col);
    vcol[r] = ld4(vg + (size_t)r * D + col);
  }

  // ---- mean query of the group, summed in the order of the generic kernel
  float* qbar = sm[wv];
  {
    float s[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) s[e] = 0.f;
    for (int h = 0; h < nq; ++h) {
      const T* qg = Q + (((size_t)bh * nq + h) * L + (size_t)j * G) * D + col;
      uint32_t qw[G];
#pragma unroll
      for (int r = 0; r < G; ++r) qw[r] = ld4(qg + (size_t)r * D);
#pragma unroll
      for (int r = 0; r < G; ++r) {
        float f[CPL];
        Elem<T>::pair_to_f32(qw[r], f);
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
      [&](int, int c) { return kseg[c]; },   // this lane's row is rsub, the only one it scores
      [&](int r, float* f) { Elem<T>::pair_to_f32(kcol[r], f); },
      [&](int r, float* f) { Elem<T>::pair_to_f32(vcol[r], f); },
      [&](int r, float* f) {
        uint32_t x = kcol[0];
#pragma unroll
        for (int i = 1; i < G; ++i) x = r == i ? kcol[i] : x;
        Elem<T>::pair_to_f32(x, f);
      });
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
