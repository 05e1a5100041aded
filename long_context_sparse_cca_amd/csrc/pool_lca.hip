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

template <typename T, int D>
hipError_t launch_t(const void* q, const void* k, const void* v, void* kc, void* vc, int32_t* anchors, int BHkv,
                    int64_t L, int g, int nq, int d_rope, float scale, hipStream_t stream) {
  const int64_t m = L / g;
  const int64_t n = (int64_t)BHkv * m;
  if (n == 0) return hipSuccess;
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
