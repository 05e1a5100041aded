// Pooling of one group of g tokens into one core token, done by one wave.
//
// Method: the CCA write-up ("ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"),
// global-aware pooling section, core-token and core K/V equations: the query
// of the group's last token scores each key of the group, a softmax over the
// group turns the scores into weights, and the weighted sums of the group's
// keys and values are the core key and core value.
#pragma once

#include "cca_device.h"

namespace cca {

// Load `N` consecutive elements starting at p as floats (N*sizeof(T) is 2..8 bytes).
template <typename T, int N>
__device__ __forceinline__ void load_n(const T* p, float* f) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (N == 2) {
      Elem<T>::pair_to_f32(*reinterpret_cast<const uint32_t*>(p), f);
    } else {
      static_assert(N == 1, "");
      f[0] = Elem<T>::bits_to_f32(reinterpret_cast<const uint16_t*>(p)[0]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = p[i];
  }
}

// One wave pools rows 0..g-1 of a group (the other waves of its workgroup, if
// any, are not involved: only wave-level synchronisation is used).
//   rows r < g-1 are read at k_rows + r*D / v_rows + r*D; row g-1 at k_last / v_last
//   (the decode cache passes the newest token there, the prefill passes row g-1);
//   the scoring query is the mean of the nq query rows q_hat + h*q_stride, h < nq:
//   the queries of the group's last token in the nq heads that share this
//   key/value head (one row, nq = 1, without grouped-query attention);
//   w_lds is LDS scratch of g floats owned by this wave.
// Math in float32; kc/vc receive one rounding to T.
template <typename T, int D>
__device__ __forceinline__ void pool_group_wave(const T* __restrict__ q_hat, int64_t q_stride, int nq,
                                                const T* __restrict__ k_rows,
                                                const T* __restrict__ v_rows, const T* __restrict__ k_last,
                                                const T* __restrict__ v_last, int g, float scale,
                                                T* __restrict__ kc, T* __restrict__ vc,
                                                float* __restrict__ w_lds) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int LPR = 4;            // lanes per row in the scoring pass
  constexpr int SEG = D / LPR;      // elements of a row per lane
  constexpr int SEGC = SEG / EPC;   // 16-byte chunks per lane
  const int rsub = lane / LPR;      // row within a pass of 16 rows
  const int seg = lane % LPR;

  // ---- pass 1: scores s_r = scale * log2(e) * q_hat . K[r] (row-major, 16-byte loads)
  float qf[SEG];
#pragma unroll
  for (int c = 0; c < SEGC; ++c) Elem<T>::chunk_to_f32(ld16(q_hat + seg * SEG + c * EPC), qf + c * EPC);
  if (nq > 1) {
    for (int h = 1; h < nq; ++h) {
#pragma unroll
      for (int c = 0; c < SEGC; ++c) {
        float f[EPC];
        Elem<T>::chunk_to_f32(ld16(q_hat + (size_t)h * q_stride + seg * SEG + c * EPC), f);
#pragma unroll
        for (int e = 0; e < EPC; ++e) qf[c * EPC + e] += f[e];
      }
    }
    const float inv = 1.0f / (float)nq;
#pragma unroll
    for (int e = 0; e < SEG; ++e) qf[e] *= inv;
  }
  const float sc = scale * kLog2e;
  for (int r0 = 0; r0 < g; r0 += kWave / LPR) {
    const int r = r0 + rsub;
    float part = 0.f;
    if (r < g) {
      const T* kr = (r == g - 1) ? k_last : k_rows + (size_t)r * D;
#pragma unroll
      for (int c = 0; c < SEGC; ++c) {
        float kf[EPC];
        Elem<T>::chunk_to_f32(ld16(kr + seg * SEG + c * EPC), kf);
#pragma unroll
        for (int e = 0; e < EPC; ++e) part = fmaf(qf[c * EPC + e], kf[e], part);
      }
    }
    part += __shfl_xor(part, 1, kWave);
    part += __shfl_xor(part, 2, kWave);
    if (seg == 0 && r < g) w_lds[r] = part * sc;
  }
  wave_lds_sync();

  // ---- softmax over the group (base-2 exponent of pre-scaled scores)
  float mx = -INFINITY;
  for (int r = lane; r < g; r += kWave) mx = fmaxf(mx, w_lds[r]);
  mx = wave_max_xor(mx, 1, kWave);
  float sum = 0.f;
  for (int r = lane; r < g; r += kWave) sum += fast_exp2(w_lds[r] - mx);
  sum = wave_sum_xor(sum, 1, kWave);
  const float inv = 1.0f / sum;
  wave_lds_sync();
  for (int r = lane; r < g; r += kWave) w_lds[r] = fast_exp2(w_lds[r] - mx) * inv;
  wave_lds_sync();

  // ---- pass 2: weighted sums, each lane owns D/64 consecutive columns
  constexpr int CPL = D / kWave;
  float ak[CPL], av[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) ak[e] = av[e] = 0.f;
  const int col = lane * CPL;
  int r = 0;
  for (; r + 4 <= g - 1; r += 4) {
    float kf[4][CPL], vf[4][CPL];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      load_n<T, CPL>(k_rows + (size_t)(r + u) * D + col, kf[u]);
      load_n<T, CPL>(v_rows + (size_t)(r + u) * D + col, vf[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float a = w_lds[r + u];
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        ak[e] = fmaf(a, kf[u][e], ak[e]);
        av[e] = fmaf(a, vf[u][e], av[e]);
      }
    }
  }
  for (; r < g; ++r) {
    const T* kr = (r == g - 1) ? k_last : k_rows + (size_t)r * D;
    const T* vr = (r == g - 1) ? v_last : v_rows + (size_t)r * D;
    float kf[CPL], vf[CPL];
    load_n<T, CPL>(kr + col, kf);
    load_n<T, CPL>(vr + col, vf);
    const float a = w_lds[r];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      ak[e] = fmaf(a, kf[e], ak[e]);
      av[e] = fmaf(a, vf[e], av[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    Elem<T>::store1(kc + col + e, ak[e]);
    Elem<T>::store1(vc + col + e, av[e]);
  }
}

}  // namespace cca
