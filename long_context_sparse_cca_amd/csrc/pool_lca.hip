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

namespace cca {
namespace {

template <typename T, int D>
__device__ __forceinline__ void load_cols(const T* p, float* f) {
  constexpr int CPL = D / kWave;   // columns per lane: 1 or 2
  if constexpr (sizeof(T) == 2) {
    if constexpr (CPL == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
      f[0] = __uint_as_float(w << 16);
      f[1] = __uint_as_float(w & 0xffff0000u);
    } else {
      f[0] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[0]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < CPL; ++e) f[e] = p[e];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void cca_pool_lca_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                          const T* __restrict__ V, T* __restrict__ Kc,
                                                          T* __restrict__ Vc, int32_t* __restrict__ anchors,
                                                          int64_t L, int g, int64_t m, int nq, int d_rope,
                                                          float scale) {
  extern __shared__ float sm[];   // mean query [D], then scores [g]
  float* qbar = sm;
  float* w = sm + D;
  constexpr int CPL = D / kWave;
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int LPR = 4;            // lanes per row in the scoring pass
  constexpr int SEG = D / LPR;
  constexpr int SEGC = SEG / EPC;
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
        load_cols<T, D>(qg + (size_t)r * D + col, f);
#pragma unroll
        for (int e = 0; e < CPL; ++e) s[e] += f[e];
      }
    }
    const float inv_g = 1.0f / ((float)g * (float)nq);
#pragma unroll
    for (int e = 0; e < CPL; ++e) qbar[col + e] = s[e] * inv_g;
  }
  wave_lds_sync();

  // ---- scores s_r = scale log2(e) qbar . K_r (4 lanes per row)
  const int rsub = lane / LPR, seg = lane % LPR;
  float qf[SEG];
#pragma unroll
  for (int e = 0; e < SEG; ++e) qf[e] = qbar[seg * SEG + e];
  const float sc = scale * kLog2e;
  for (int r0 = 0; r0 < g; r0 += kWave / LPR) {
    const int r = r0 + rsub;
    float part = 0.f;
    if (r < g) {
#pragma unroll
      for (int c = 0; c < SEGC; ++c) {
        float kf[EPC];
        Elem<T>::chunk_to_f32(ld16(K + row0 + (size_t)r * D + seg * SEG + c * EPC), kf);
#pragma unroll
        for (int e = 0; e < EPC; ++e) part = fmaf(qf[c * EPC + e], kf[e], part);
      }
    }
    part = lane_group_sum<LPR>(part);
    if (seg == 0 && r < g) w[r] = part * sc;
  }
  wave_lds_sync();

  // ---- softmax weights and the anchor (first position with the largest score)
  float mx = -INFINITY;
  for (int r = lane; r < g; r += kWave) mx = fmaxf(mx, w[r]);
  mx = wave_max_xor(mx, 1, kWave);
  int arg = 0x7fffffff;
  float sum = 0.f;
  for (int r = lane; r < g; r += kWave) {
    const float x = w[r];
    if (x == mx && r < arg) arg = r;
    sum += fast_exp2(x - mx);
  }
  for (int b = 1; b < kWave; b <<= 1) arg = min(arg, __shfl_xor(arg, b, kWave));
  if (arg >= g) arg = 0;   // no score compared equal to the max (NaN inputs): stay inside the group
  sum = wave_sum_xor(sum, 1, kWave);
  const float inv = 1.0f / sum;
  wave_lds_sync();
  for (int r = lane; r < g; r += kWave) w[r] = fast_exp2(w[r] - mx) * inv;
  wave_lds_sync();

  // ---- content dims and values: weighted sums; positional dims: the anchor's key
  float ak[CPL], av[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) ak[e] = av[e] = 0.f;
  for (int r = 0; r < g; ++r) {
    const float a = w[r];
    float kf[CPL], vf[CPL];
    load_cols<T, D>(K + row0 + (size_t)r * D + col, kf);
    load_cols<T, D>(V + row0 + (size_t)r * D + col, vf);
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      ak[e] = fmaf(a, kf[e], ak[e]);
      av[e] = fmaf(a, vf[e], av[e]);
    }
  }
  float kanc[CPL];
  load_cols<T, D>(K + row0 + (size_t)arg * D + col, kanc);
  const size_t out = ((size_t)bh * m + j) * D;
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    const bool positional = col + e >= D - d_rope;
    Elem<T>::store1(Kc + out + col + e, positional ? kanc[e] : ak[e]);
    Elem<T>::store1(Vc + out + col + e, av[e]);
  }
  if (anchors != nullptr && lane == 0) anchors[(size_t)bh * m + j] = arg;
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
  if (dt == CCA_BF16) {
    if (d == 128) return launch_t<bf16_t, 128>(q, k, v, kc, vc, anchors, BHkv, L, g, nq, d_rope, scale, stream);
    return launch_t<bf16_t, 64>(q, k, v, kc, vc, anchors, BHkv, L, g, nq, d_rope, scale, stream);
  }
  if (d == 128) return launch_t<float, 128>(q, k, v, kc, vc, anchors, BHkv, L, g, nq, d_rope, scale, stream);
  return launch_t<float, 64>(q, k, v, kc, vc, anchors, BHkv, L, g, nq, d_rope, scale, stream);
}

}  // namespace cca
