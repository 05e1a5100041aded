// Backward pass of CCA prefill attention for the shapes the matrix-core path does not
// take: float32 inputs, and bf16 or float32 at head dim 64 (float32 gradients).
//
// Method: the CCA write-up ("ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"),
// Triton section (the fused operator serves training), with the chain rule through the
// attention softmax and the pooling softmax as in backward.hip:
//   p = exp(scale k.q - lse), dp = dO.v, ds = p (dp - D), D = dO.O;
//   dQ += scale sum ds k;  dkey += scale ds q;  dval += p dO;
//   then dKc, dVc of the core tokens through the pooling (cca_bwd_pool_kernel, templated).
// All arithmetic in float32 on the vector ALUs: one wave per query (dQ) and one wave per
// key (dK, dV), lanes splitting the other side of the pairs, a reduction over the lanes in
// LDS.  Plain and correct rather than fast: the bf16 d = 128 path is the fast one.
#include "cca_internal.h"

namespace cca {
namespace {

// Lane layout of the dQ and dK/dV kernels: 16 lanes per row (part = lane % 16 owns the
// D/16 dims part*DPL .. +DPL-1), 4 rows per wave step (slot = lane / 16); a row's dot
// products are summed over its 16 lanes with DPP row operations.
template <typename T, int D>
struct GenCfg {
  static constexpr int DPL = D / 16;                       // dims per lane: 4 or 8
  static constexpr int BYTES = DPL * (int)sizeof(T);       // 8, 16 or 32
};

template <typename T, int D>
__device__ __forceinline__ void load_dims(const T* p, float* f) {
  constexpr int DPL = GenCfg<T, D>::DPL;
  if constexpr (sizeof(T) == 2) {
    if constexpr (DPL == 8) {
      Elem<T>::chunk_to_f32(ld16(p), f);
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      Elem<T>::pair_to_f32(w.x, f);
      Elem<T>::pair_to_f32(w.y, f + 2);
    }
  } else {
#pragma unroll
    for (int c = 0; c < DPL; c += 4) Elem<T>::chunk_to_f32(ld16(p + c), f + c);
  }
}

// D[t] = dO[t].O[t] and the log-sum-exp in log2 units, one thread per row
template <typename T, int D>
__global__ __launch_bounds__(256) void cca_bwdg_prep_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                            const float* __restrict__ lse, float* __restrict__ Dv,
                                                            float* __restrict__ lse2, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  constexpr int EPC = Elem<T>::kPerChunk;
  float s = 0.f;
  for (int c = 0; c < D; c += EPC) {
    float o[EPC], g[EPC];
    Elem<T>::chunk_to_f32(ld16(O + (size_t)r * D + c), o);
    Elem<T>::chunk_to_f32(ld16(dO + (size_t)r * D + c), g);
#pragma unroll
    for (int e = 0; e < EPC; ++e) s = fmaf(o[e], g[e], s);
  }
  Dv[r] = s;
  lse2[r] = lse[r] * kLog2e;
}

// dQ (attention part) of one query per wave: 4 keys per step, 16 lanes per key.
template <typename T, int D>
__global__ __launch_bounds__(64) void cca_bwdg_dq_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                         const T* __restrict__ V, const T* __restrict__ Kc,
                                                         const T* __restrict__ Vc, const T* __restrict__ dO,
                                                         const float* __restrict__ lse2,
                                                         const float* __restrict__ Dv, float* __restrict__ dQ,
                                                         int64_t L, int g, int k_local, int nq, float scale) {
  constexpr int DPL = GenCfg<T, D>::DPL;
  const int64_t row = blockIdx.x;                 // bh * L + t
  const int64_t bh = row / L, t = row - bh * L;
  const int64_t bkv = bh / nq;
  const int lane = threadIdx.x, part = lane & 15, slot = lane >> 4;
  const int64_t m = L / g;
  float q[DPL], go[DPL], acc[DPL];
  load_dims<T, D>(Q + (size_t)row * D + part * DPL, q);
  load_dims<T, D>(dO + (size_t)row * D + part * DPL, go);
#pragma unroll
  for (int c = 0; c < DPL; ++c) acc[c] = 0.f;
  const float sc = scale * kLog2e, l2 = lse2[row], dd = Dv[row];
  int64_t n_c = t / g - k_local;
  if (n_c < 0) n_c = 0;
  const int64_t raw_lo = n_c * g;
  const int64_t n_keys = n_c + (t - raw_lo + 1);
  for (int64_t i0 = 0; i0 < n_keys; i0 += 4) {
    const int64_t i = min(i0 + slot, n_keys - 1);
    const T* kr = i < n_c ? Kc + ((size_t)bkv * m + i) * D : K + ((size_t)bkv * L + raw_lo + (i - n_c)) * D;
    const T* vr = i < n_c ? Vc + ((size_t)bkv * m + i) * D : V + ((size_t)bkv * L + raw_lo + (i - n_c)) * D;
    float kf[DPL], vf[DPL];
    load_dims<T, D>(kr + part * DPL, kf);
    load_dims<T, D>(vr + part * DPL, vf);
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int c = 0; c < DPL; ++c) {
      s = fmaf(q[c], kf[c], s);
      dp = fmaf(go[c], vf[c], dp);
    }
    s = lane_group_sum<16>(s);
    dp = lane_group_sum<16>(dp);
    const float p = fast_exp2(s * sc - l2);
    const float ds = i0 + slot < n_keys ? p * (dp - dd) : 0.f;
#pragma unroll
    for (int c = 0; c < DPL; ++c) acc[c] = fmaf(ds, kf[c], acc[c]);
  }
#pragma unroll
  for (int c = 0; c < DPL; ++c) {
    acc[c] += __shfl_xor(acc[c], 16, kWave);
    acc[c] += __shfl_xor(acc[c], 32, kWave);
  }
  if (slot == 0) {
#pragma unroll
    for (int c = 0; c < DPL; ++c) dQ[(size_t)row * D + part * DPL + c] = acc[c] * scale;
  }
}

// dK or dV of one key per wave (MODE 0: dV, MODE 1: dK): key index i < m is core token i,
// else raw position i - m; 4 of the queries that see it per step (over the nq query heads
// that read this key/value slice), 16 lanes per query.
template <typename T, int D, int MODE>
__global__ __launch_bounds__(64) void cca_bwdg_dkdv_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                           const T* __restrict__ V, const T* __restrict__ Kc,
                                                           const T* __restrict__ Vc, const T* __restrict__ dO,
                                                           const float* __restrict__ lse2,
                                                           const float* __restrict__ Dv, float* __restrict__ dKV,
                                                           float* __restrict__ dKVc, int64_t L, int g, int k_local,
                                                           int nq, float scale) {
  constexpr int DPL = GenCfg<T, D>::DPL;
  const int64_t m = L / g;
  const int64_t nk = m + L;
  const int64_t gid = blockIdx.x;
  const int64_t bkv = gid / nk, i = gid - bkv * nk;
  const bool core = i < m;
  const int lane = threadIdx.x, part = lane & 15, slot = lane >> 4;
  const T* kr = core ? Kc + ((size_t)bkv * m + i) * D : K + ((size_t)bkv * L + (i - m)) * D;
  const T* vr = core ? Vc + ((size_t)bkv * m + i) * D : V + ((size_t)bkv * L + (i - m)) * D;
  float kf[DPL], vf[DPL], acc[DPL];
  load_dims<T, D>(kr + part * DPL, kf);
  load_dims<T, D>(vr + part * DPL, vf);
#pragma unroll
  for (int c = 0; c < DPL; ++c) acc[c] = 0.f;
  // queries that see this key: core token j from (j + k + 1) g on; raw u from u to (u/g + k + 1) g - 1
  int64_t t_lo, t_hi;
  if (core) {
    t_lo = (i + k_local + 1) * g;
    t_hi = L - 1;
  } else {
    const int64_t u = i - m;
    t_lo = u;
    t_hi = min(L - 1, (u / g + k_local + 1) * g - 1);
  }
  const float sc = scale * kLog2e;
  const int64_t nt = t_hi >= t_lo ? t_hi - t_lo + 1 : 0;
  const int64_t total = nt * nq;
  for (int64_t e0 = 0; e0 < total; e0 += 4) {
    const int64_t e = min(e0 + slot, total - 1);
    const int64_t h = e / nt, t = t_lo + (e - h * nt);
    const int64_t row = ((size_t)bkv * nq + h) * L + t;
    float qf[DPL], gf[DPL];
    load_dims<T, D>(Q + (size_t)row * D + part * DPL, qf);
    load_dims<T, D>(dO + (size_t)row * D + part * DPL, gf);
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int c = 0; c < DPL; ++c) {
      s = fmaf(qf[c], kf[c], s);
      dp = fmaf(gf[c], vf[c], dp);
    }
    s = lane_group_sum<16>(s);
    dp = lane_group_sum<16>(dp);
    float p = fast_exp2(s * sc - lse2[row]);
    if (e0 + slot >= total) p = 0.f;
    if constexpr (MODE == 0) {
#pragma unroll
      for (int c = 0; c < DPL; ++c) acc[c] = fmaf(p, gf[c], acc[c]);
    } else {
      const float ds = p * (dp - Dv[row]);
#pragma unroll
      for (int c = 0; c < DPL; ++c) acc[c] = fmaf(ds, qf[c], acc[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < DPL; ++c) {
    acc[c] += __shfl_xor(acc[c], 16, kWave);
    acc[c] += __shfl_xor(acc[c], 32, kWave);
  }
  const float f = MODE == 1 ? scale : 1.0f;
  float* o = core ? dKVc + ((size_t)bkv * m + i) * D : dKV + ((size_t)bkv * L + (i - m)) * D;
  if (slot == 0) {
#pragma unroll
    for (int c = 0; c < DPL; ++c) o[part * DPL + c] = acc[c] * f;
  }
}

// Pooling backward, one wave per (key/value slice, group): the group's scores against the
// mean of its nq scoring queries, softmax, da = dKc.K + dVc.V, dz = a (da - a.da); then
// dK += a dKc + scale dz q_hat, dV += a dVc on the group's rows and each scoring query
// gets scale (1/nq) sum dz K.
template <typename T, int D>
__global__ __launch_bounds__(64) void cca_bwdg_pool_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                           const T* __restrict__ V, const float* __restrict__ dKc,
                                                           const float* __restrict__ dVc, float* __restrict__ dQ,
                                                           float* __restrict__ dK, float* __restrict__ dV, int64_t L,
                                                           int g, int64_t m, int nq, float scale) {
  extern __shared__ float sm[];   // a[g], then da / dz[g], then q_hat[D]
  float* a_l = sm;
  float* z_l = sm + g;
  float* qh = sm + 2 * g;
  const int64_t gid = blockIdx.x;
  const int64_t bkv = gid / m, j = gid - bkv * m;
  const int lane = threadIdx.x;
  const size_t row0 = (size_t)bkv * L + (size_t)j * g;
  const size_t qrow0 = ((size_t)bkv * nq * L + (size_t)j * g + g - 1) * D;
  const size_t qstride = (size_t)L * D;
  const float* dkc = dKc + ((size_t)bkv * m + j) * D;
  const float* dvc = dVc + ((size_t)bkv * m + j) * D;
  for (int c = lane; c < D; c += kWave) {
    float s = 0.f;
    for (int h = 0; h < nq; ++h) s += Elem<T>::load1(Q + qrow0 + h * qstride + c);
    qh[c] = s * (1.0f / (float)nq);
  }
  wave_lds_sync();
  // scores and da, one row per lane pass
  const float sc = scale * kLog2e;
  for (int r = lane; r < g; r += kWave) {
    float s = 0.f, da = 0.f;
    const T* kr = K + (row0 + r) * D;
    const T* vr = V + (row0 + r) * D;
    for (int c = 0; c < D; ++c) {
      const float kv = Elem<T>::load1(kr + c);
      s = fmaf(qh[c], kv, s);
      da = fmaf(dkc[c], kv, fmaf(dvc[c], Elem<T>::load1(vr + c), da));
    }
    a_l[r] = s * sc;
    z_l[r] = da;
  }
  wave_lds_sync();
  float mx = -INFINITY;
  for (int r = lane; r < g; r += kWave) mx = fmaxf(mx, a_l[r]);
  mx = wave_max_xor(mx, 1, kWave);
  float sum = 0.f;
  for (int r = lane; r < g; r += kWave) sum += fast_exp2(a_l[r] - mx);
  sum = wave_sum_xor(sum, 1, kWave);
  const float inv = 1.0f / sum;
  float ada = 0.f;
  for (int r = lane; r < g; r += kWave) ada += fast_exp2(a_l[r] - mx) * inv * z_l[r];
  ada = wave_sum_xor(ada, 1, kWave);
  wave_lds_sync();
  for (int r = lane; r < g; r += kWave) {
    const float a = fast_exp2(a_l[r] - mx) * inv;
    z_l[r] = a * (z_l[r] - ada);
    a_l[r] = a;
  }
  wave_lds_sync();
  for (int c = lane; c < D; c += kWave) {
    float dq = 0.f;
    for (int r = 0; r < g; ++r) {
      const float a = a_l[r], dz = z_l[r];
      const size_t o = (row0 + r) * D + c;
      dK[o] += a * dkc[c] + scale * dz * qh[c];
      dV[o] += a * dvc[c];
      dq = fmaf(dz, Elem<T>::load1(K + o), dq);
    }
    for (int h = 0; h < nq; ++h) dQ[qrow0 + h * qstride + c] += scale * (1.0f / (float)nq) * dq;
  }
}

template <typename T, int D>
hipError_t launch_t(const void* q, const void* k, const void* v, const void* kc, const void* vc, const void* out,
                    const float* lse, const void* dout, float* dq, float* dk, float* dv, void* workspace, int BH,
                    int nq, int64_t L, int g, int k_local, float scale, hipStream_t stream) {
  const int64_t m = L / g;
  const int BHkv = BH / nq;
  float* Dv = (float*)workspace;
  float* lse2 = Dv + (size_t)BH * L;
  float* dKc = lse2 + (size_t)BH * L;
  float* dVc = dKc + (size_t)BHkv * m * D;
  const int64_t rows = (int64_t)BH * L;
  hipLaunchKernelGGL((cca_bwdg_prep_kernel<T, D>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream,
                     (const T*)out, (const T*)dout, lse, Dv, lse2, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((cca_bwdg_dq_kernel<T, D>), dim3((unsigned)rows), dim3(kWave), 0, stream, (const T*)q,
                     (const T*)k, (const T*)v, (const T*)kc, (const T*)vc, (const T*)dout, (const float*)lse2,
                     (const float*)Dv, dq, L, g, k_local, nq, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nkeys = (int64_t)BHkv * (m + L);
  hipLaunchKernelGGL((cca_bwdg_dkdv_kernel<T, D, 0>), dim3((unsigned)nkeys), dim3(kWave), 0, stream, (const T*)q,
                     (const T*)k, (const T*)v, (const T*)kc, (const T*)vc, (const T*)dout, (const float*)lse2,
                     (const float*)Dv, dv, dVc, L, g, k_local, nq, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((cca_bwdg_dkdv_kernel<T, D, 1>), dim3((unsigned)nkeys), dim3(kWave), 0, stream, (const T*)q,
                     (const T*)k, (const T*)v, (const T*)kc, (const T*)vc, (const T*)dout, (const float*)lse2,
                     (const float*)Dv, dk, dKc, L, g, k_local, nq, scale);
  e = hipGetLastError();
  if (e != hipSuccess || m == 0) return e;
  hipLaunchKernelGGL((cca_bwdg_pool_kernel<T, D>), dim3((unsigned)((int64_t)BHkv * m)), dim3(kWave),
                     (size_t)(2 * g + D) * sizeof(float), stream, (const T*)q, (const T*)k, (const T*)v,
                     (const float*)dKc, (const float*)dVc, dq, dk, dv, L, g, m, nq, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_generic(int dt, int d, const void* q, const void* k, const void* v, const void* kc,
                                   const void* vc, const void* out, const float* lse, const void* dout, float* dq,
                                   float* dk, float* dv, void* workspace, int BH, int nq, int64_t L, int g,
                                   int k_local, float scale, hipStream_t stream) {
  return dispatch_td(dt, d, [&](auto t, auto dd) {
    return launch_t<decltype(t), decltype(dd)::value>(q, k, v, kc, vc, out, lse, dout, dq, dk, dv, workspace, BH, nq,
                                                      L, g, k_local, scale, stream);
  });
}

}  // namespace cca
