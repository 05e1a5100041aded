// Prefill pooling: every complete group of every (b,h) slice becomes one core
// key and one core value (the CCA write-up, global-aware pooling section,
// core-token and core K/V equations).  With grouped-query attention a
// key/value head is pooled once, scored by the mean of the last-token queries
// of the query heads that share it.  One wave per group; HBM-bound.  A
// dedicated kernel covers 16-bit inputs (bf16, binary16) at d = 128, g = 16;
// other shapes use the generic group routine shared with the decode cache.
#include "cca_internal.h"
#include "pool_group.h"

namespace cca {
namespace {

// Slices: K, V, Kc, Vc are indexed by the key/value slice bkv = b*H_kv + h_kv; the
// nq = H / H_kv query heads sharing it are the query slices bkv*nq .. bkv*nq + nq-1.
template <typename T, int D>
__global__ __launch_bounds__(64) void cca_pool_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                      const T* __restrict__ V, T* __restrict__ Kc,
                                                      T* __restrict__ Vc, int64_t L, int g, int64_t m, int nq,
                                                      float scale) {
  extern __shared__ float w_lds[];
  const int64_t gid = blockIdx.x;  // (bkv, j) flattened
  const int64_t bkv = gid / m;
  const int64_t j = gid - bkv * m;
  const size_t base = ((size_t)bkv * L + (size_t)j * g) * D;
  const size_t last = base + (size_t)(g - 1) * D;
  const size_t qlast = ((size_t)bkv * nq * L + (size_t)j * g + g - 1) * D;
  const size_t out = ((size_t)bkv * m + j) * D;
  pool_group_wave<T, D>(Q + qlast, (int64_t)L * D, nq, K + base, V + base, K + last, V + last, g, scale, Kc + out,
                        Vc + out, w_lds);
}

// 16-bit inputs, d = 128, g = 16: one wave per group, every load of the group issued
// up front.  Lane (rq = lane/16, c = lane%16) owns the 16-byte column chunk c
// (dims 8c..8c+7) of the rows rq, rq+4, rq+8, rq+12.
template <typename T, bool STREAM>
__global__ __launch_bounds__(256) void cca_pool_d128_g16_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                              const T* __restrict__ V, T* __restrict__ Kc,
                                                              T* __restrict__ Vc, int64_t L, int64_t m,
                                                              int64_t n_groups, int nq, float scale) {
  constexpr int D = 128, G = 16;
  const int64_t gid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gid >= n_groups) return;
  const int lane = threadIdx.x & 63;
  const int rq = lane >> 4, c = lane & 15;
  const int64_t bh = gid / m, j = gid - bh * m;   // bh: key/value slice
  const T* kg = K + ((size_t)bh * L + (size_t)j * G) * D;
  const T* vg = V + ((size_t)bh * L + (size_t)j * G) * D;
  const T* qh = Q + ((size_t)bh * nq * L + (size_t)j * G + G - 1) * D;
  uint4 kr[4], vr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kr[i] = ld16_kv<STREAM>(kg + (size_t)(rq + 4 * i) * D + 8 * c);
    vr[i] = ld16_kv<STREAM>(vg + (size_t)(rq + 4 * i) * D + 8 * c);
  }
  float qf[8];
  Elem<T>::chunk_to_f32(ld16(qh + 8 * c), qf);
  if (nq > 1) {
    // grouped-query attention: the mean of the nq heads' last-token queries
    for (int h = 1; h < nq; ++h) {
      float f[8];
      Elem<T>::chunk_to_f32(ld16(qh + (size_t)h * L * D + 8 * c), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[e] += f[e];
    }
    const float inv = 1.0f / (float)nq;
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] *= inv;
  }
  const float sc = scale * kLog2e;
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float kf[8];
    Elem<T>::chunk_to_f32(kr[i], kf);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) d = fmaf(qf[e], kf[e], d);
    d = wave_sum_xor(d, 1, 16);   // over the 16 column chunks of the row
    s[i] = d * sc;
  }
  float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  mx = wave_max_xor(mx, 16, 64);  // over the 4 row quarters
  float p[4], sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = fast_exp2(s[i] - mx);
    sum += p[i];
  }
  sum = wave_sum_xor(sum, 16, 64);
  const float inv = 1.0f / sum;
  float ak[8], av[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ak[e] = av[e] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float kf[8], vf[8];
    Elem<T>::chunk_to_f32(kr[i], kf);
    Elem<T>::chunk_to_f32(vr[i], vf);
    const float a = p[i] * inv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ak[e] = fmaf(a, kf[e], ak[e]);
      av[e] = fmaf(a, vf[e], av[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ak[e] = wave_sum_xor(ak[e], 16, 64);
    av[e] = wave_sum_xor(av[e], 16, 64);
  }
  if (rq == 0) {
    uint4 ko, vo;
    ko.x = Elem<T>::pack2(ak[0], ak[1]); ko.y = Elem<T>::pack2(ak[2], ak[3]);
    ko.z = Elem<T>::pack2(ak[4], ak[5]); ko.w = Elem<T>::pack2(ak[6], ak[7]);
    vo.x = Elem<T>::pack2(av[0], av[1]); vo.y = Elem<T>::pack2(av[2], av[3]);
    vo.z = Elem<T>::pack2(av[4], av[5]); vo.w = Elem<T>::pack2(av[6], av[7]);
    st16(Kc + ((size_t)bh * m + j) * D + 8 * c, ko);
    st16(Vc + ((size_t)bh * m + j) * D + 8 * c, vo);
  }
}

template <typename T, int D>
hipError_t launch_pool_t(const void* q, const void* k, const void* v, void* kc, void* vc, int BHkv, int64_t L,
                         int g, int nq, float scale, hipStream_t stream) {
  const int64_t m = L / g;
  const int64_t n = (int64_t)BHkv * m;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((cca_pool_kernel<T, D>), dim3((unsigned)n), dim3(64), (size_t)g * sizeof(float), stream,
                     (const T*)q, (const T*)k, (const T*)v, (T*)kc, (T*)vc, L, g, m, nq, scale);
  return hipGetLastError();
}

template <typename T>
void launch_pool_d128_g16(const void* q, const void* k, const void* v, void* kc, void* vc, int64_t L, int64_t m,
                          int64_t n, int nq, float scale, hipStream_t stream) {
  // K and V are read once here; past the last-level cache they are streamed
  if (n * 16 * 128 * 2 * 2 > kStreamBytes)
    hipLaunchKernelGGL((cca_pool_d128_g16_kernel<T, true>), dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream,
                       (const T*)q, (const T*)k, (const T*)v, (T*)kc, (T*)vc, L, m, n, nq, scale);
  else
    hipLaunchKernelGGL((cca_pool_d128_g16_kernel<T, false>), dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream,
                       (const T*)q, (const T*)k, (const T*)v, (T*)kc, (T*)vc, L, m, n, nq, scale);
}

}  // namespace

hipError_t launch_pool(int dt, int d, const void* q, const void* k, const void* v, void* kc, void* vc, int BHkv,
                       int64_t L, int g, int nq, float scale, hipStream_t stream) {
  if (dt != CCA_F32 && d == 128 && g == 16) {
    const int64_t m = L / 16, n = (int64_t)BHkv * m;
    if (n == 0) return hipSuccess;
    if (dt == CCA_F16)
      launch_pool_d128_g16<f16_t>(q, k, v, kc, vc, L, m, n, nq, scale, stream);
    else
      launch_pool_d128_g16<bf16_t>(q, k, v, kc, vc, L, m, n, nq, scale, stream);
    return hipGetLastError();
  }
  return dispatch_td(dt, d, [&](auto t, auto dd) {
    return launch_pool_t<decltype(t), decltype(dd)::value>(q, k, v, kc, vc, BHkv, L, g, nq, scale, stream);
  });
}

}  // namespace cca
