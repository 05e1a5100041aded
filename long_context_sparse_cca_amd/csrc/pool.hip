// Prefill pooling: every complete group of every (b,h) slice becomes one core
// key and one core value (the CCA write-up, global-aware pooling section,
// core-token and core K/V equations).  One wave per group; HBM-bound.
#include "cca_internal.h"
#include "pool_group.h"

namespace cca {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(64) void cca_pool_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                      const T* __restrict__ V, T* __restrict__ Kc,
                                                      T* __restrict__ Vc, int64_t L, int g, int64_t m,
                                                      float scale) {
  extern __shared__ float w_lds[];
  const int64_t gid = blockIdx.x;  // (bh, j) flattened
  const int64_t bh = gid / m;
  const int64_t j = gid - bh * m;
  const size_t base = ((size_t)bh * L + (size_t)j * g) * D;
  const size_t last = base + (size_t)(g - 1) * D;
  const size_t out = ((size_t)bh * m + j) * D;
  pool_group_wave<T, D>(Q + last, K + base, V + base, K + last, V + last, g, scale, Kc + out, Vc + out, w_lds);
}

template <typename T, int D>
hipError_t launch_pool_t(const void* q, const void* k, const void* v, void* kc, void* vc, int BH, int64_t L,
                         int g, float scale, hipStream_t stream) {
  const int64_t m = L / g;
  const int64_t n = (int64_t)BH * m;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((cca_pool_kernel<T, D>), dim3((unsigned)n), dim3(64), (size_t)g * sizeof(float), stream,
                     (const T*)q, (const T*)k, (const T*)v, (T*)kc, (T*)vc, L, g, m, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(int dt, int d, const void* q, const void* k, const void* v, void* kc, void* vc, int BH,
                       int64_t L, int g, float scale, hipStream_t stream) {
  if (dt == CCA_BF16) {
    if (d == 128) return launch_pool_t<bf16_t, 128>(q, k, v, kc, vc, BH, L, g, scale, stream);
    return launch_pool_t<bf16_t, 64>(q, k, v, kc, vc, BH, L, g, scale, stream);
  }
  if (d == 128) return launch_pool_t<float, 128>(q, k, v, kc, vc, BH, L, g, scale, stream);
  return launch_pool_t<float, 64>(q, k, v, kc, vc, BH, L, g, scale, stream);
}

}  // namespace cca
