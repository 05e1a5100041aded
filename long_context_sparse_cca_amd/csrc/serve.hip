// Serving decode step over the compressed CCA cache: one new token per sequence,
// each sequence at its own position, grouped-query attention.
//
// Method: the CCA write-up ("ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"):
// the token at position t attends, in one softmax, to the core tokens of the
// groups before its raw window and to the raw keys (t/g - k)*g .. t (global-aware
// pooling, locality-preserving module, global-local fusion sections); the fused
// operator serves decode from a KV cache of core tokens plus local raw tokens
// (Triton section, Fig. 3).  A group is pooled when its last token arrives.
// With grouped-query attention the cache holds one core token per key/value
// head, pooled with the mean of the last-token queries of the query heads that
// share it (the mean-query importance of "Latent-Condensed Transformer for
// Efficient Long Context Modeling", section 2, which its section 3 extends to
// grouped-query attention).
//
// LCA-style cache (LCA): a group is condensed instead, with the mean of all its queries
// (its g tokens times the query heads sharing the key/value head; "Latent-Condensed
// Transformer for Efficient Long Context Modeling", sections 2 and 3) as importance and
// the top-scored token's positional dims (lca_group.h).  The running sum of the current
// group's queries lives in qsum [B*H_kv][D] between calls.
//
// One workgroup = (sequence b, key/value head, block of RH query heads, chunk of
// the key index space); each sequence's keys are cut into the same number of
// equal chunks, sized on the device from its own length, and the chunk index runs
// fastest in the grid, so that the workgroups resident on one compute unit (a
// stride of the unit count apart) belong to different sequences and the units
// read about equal shares.  Every key/value row is loaded once per workgroup and
// scored against all RH query heads, so grouped-query attention reads the cache
// once per key/value head instead of once per query head.  Partial softmax
// states go to the workspace; the decode merge kernel combines the chunks.
#include <algorithm>

#include "cca_internal.h"
#include "lca_group.h"
#include "pool_group.h"

namespace cca {
namespace {

template <typename T, int D, int RH>
struct ServeCfg {
  static constexpr int NWAVE = 4;
  static constexpr int NT = NWAVE * kWave;
  static constexpr int EPC = 16 / (int)sizeof(T);     // elements per lane (one 16-byte chunk)
  static constexpr int LPK = D / EPC;                 // lanes per key row
  static constexpr int KPW = kWave / LPK;             // key rows per wave per load
  // loads of K and V in flight per lane; with 4 query heads, 3 keeps the kernel within 128
  // registers (4 waves per SIMD: a 1024-workgroup grid is resident at once; 4 took 152
  // registers and left a quarter of the grid for a second round, 10% slower)
  static constexpr int U = RH >= 8 ? 2 : (RH >= 4 ? 3 : 4);
  static constexpr int KPI = NWAVE * KPW * U;         // key rows per workgroup iteration
  // minimum waves per SIMD: 4 query heads at d = 128 fit four (the 1024-workgroup grid resident)
  static constexpr int WPE = (RH == 4 && D == 128) ? 4 : 1;
};

template <typename T, int D, int RH, bool STREAM, bool LCA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ServeCfg<T, D, RH>::WPE))) void cca_serve_decode_kernel(
    const int32_t* __restrict__ lens, int64_t max_len, const T* __restrict__ q, const T* __restrict__ k_new,
    const T* __restrict__ v_new, T* __restrict__ core_k, T* __restrict__ core_v, T* __restrict__ ring_k,
    T* __restrict__ ring_v, float* __restrict__ ws_acc, float* __restrict__ ws_ml, int Hkv, int nq, int nhb,
    int64_t max_groups, int64_t R, int g, int k_local, int nchunks, float scale,
    float* __restrict__ qsum, int d_rope) {
  using C = ServeCfg<T, D, RH>;
  __shared__ float red[C::NWAVE][RH][D + 2];
  extern __shared__ float pool_lds[];
  // chunk index fastest: the workgroups that share a compute unit (one grid stride of the
  // compute-unit count apart) then come from different sequences
  const int64_t xb = blockIdx.x / nchunks;
  const int ci = (int)(blockIdx.x - xb * nchunks);
  const int hb = (int)(xb % nhb);
  const int64_t bkv = xb / nhb;             // key/value slice b*Hkv + hk
  const int64_t b = bkv / Hkv;
  const int hk = (int)(bkv - b * Hkv);
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  const int kg = lane / C::LPK;
  const int part = lane % C::LPK;
  const int Hq = Hkv * nq;
  const int h0 = hk * nq + hb * RH;         // first query head of this block
  const int64_t t = lens[b];                // position of the token appended by this call
  const bool valid = t >= 0 && t <= max_len;

  // ---- append: ring slot t mod R; pool the group the token completes (once per key/value slice)
  if (valid && ci == 0 && hb == 0 && wave == 0) {
    const T* kt = k_new + (size_t)bkv * D;
    const T* vt = v_new + (size_t)bkv * D;
    const int64_t slot = t % R;
    constexpr int CPR = D * (int)sizeof(T) / 16;
    if (lane < CPR) {
      st16(reinterpret_cast<uint4*>(ring_k + ((size_t)bkv * R + slot) * D) + lane,
           ld16(reinterpret_cast<const uint4*>(kt) + lane));
      st16(reinterpret_cast<uint4*>(ring_v + ((size_t)bkv * R + slot) * D) + lane,
           ld16(reinterpret_cast<const uint4*>(vt) + lane));
    }
    if constexpr (LCA) {
      // running sum of the group's queries: this token's, over the nq query heads
      constexpr int CPL = D / kWave;
      const int col = lane * CPL;
      float qs[CPL];
      float* qsum_row = qsum + (size_t)bkv * D + col;
#pragma unroll
      for (int e = 0; e < CPL; ++e) qs[e] = 0.f;
      for (int h = 0; h < nq; ++h) {
        float qf[CPL];
        lca_load_cols<T, D>(q + ((size_t)b * Hq + (size_t)hk * nq + h) * D + col, qf);
#pragma unroll
        for (int e = 0; e < CPL; ++e) qs[e] += qf[e];
      }
#pragma unroll
      for (int e = 0; e < CPL; ++e) qs[e] += qsum_row[e];
      if ((t + 1) % g == 0) {
        const float inv = 1.0f / ((float)g * (float)nq);
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          pool_lds[col + e] = qs[e] * inv;
          qsum_row[e] = 0.f;
        }
        wave_lds_sync();
        const int64_t beta = t / g;
        const int64_t first = slot - (g - 1);
        lca_condense_wave<T, D>(pool_lds, ring_k + ((size_t)bkv * R + first) * D,
                                ring_v + ((size_t)bkv * R + first) * D, kt, vt, g, scale, d_rope,
                                core_k + ((size_t)bkv * max_groups + beta) * D,
                                core_v + ((size_t)bkv * max_groups + beta) * D, pool_lds + D, nullptr);
      } else {
#pragma unroll
        for (int e = 0; e < CPL; ++e) qsum_row[e] = qs[e];
      }
    } else if ((t + 1) % g == 0) {
      // the group occupies slots slot-g+1 .. slot (R is a multiple of g); its last row is the new token
      const int64_t beta = t / g;
      const int64_t first = slot - (g - 1);
      pool_group_wave<T, D>(q + ((size_t)b * Hq + (size_t)hk * nq) * D, D, nq,
                            ring_k + ((size_t)bkv * R + first) * D, ring_v + ((size_t)bkv * R + first) * D, kt, vt,
                            g, scale, core_k + ((size_t)bkv * max_groups + beta) * D,
                            core_v + ((size_t)bkv * max_groups + beta) * D, pool_lds);
    }
  }

  // ---- this token's visible keys: core [0, n_c) then raw positions raw_lo .. t
  int64_t n_c = 0, raw_lo = 0, n_keys = 0;
  if (valid) {
    n_c = t / g - k_local;
    n_c = n_c > 0 ? n_c : 0;
    raw_lo = n_c * g;
    n_keys = n_c + (t - raw_lo + 1);
  }
  // this sequence's keys in nchunks equal parts
  const int64_t chunk = (n_keys + nchunks - 1) / nchunks;
  const int64_t start = (int64_t)ci * chunk;
  const int64_t end = min(n_keys, start + chunk);

  const float sc = scale * kLog2e;
  float qf[RH][C::EPC];
#pragma unroll
  for (int j = 0; j < RH; ++j) {
    Elem<T>::chunk_to_f32(ld16(q + ((size_t)b * Hq + h0 + j) * D + part * C::EPC), qf[j]);
#pragma unroll
    for (int e = 0; e < C::EPC; ++e) qf[j][e] *= sc;
  }
  const T* ck = core_k + (size_t)bkv * max_groups * D;
  const T* cv = core_v + (size_t)bkv * max_groups * D;
  const T* rk = ring_k + (size_t)bkv * R * D;
  const T* rv = ring_v + (size_t)bkv * R * D;
  const T* kt_new = k_new + (size_t)bkv * D;
  const T* vt_new = v_new + (size_t)bkv * D;

  float m_run[RH], l_run[RH], acc[RH][C::EPC];
#pragma unroll
  for (int j = 0; j < RH; ++j) {
    m_run[j] = kNegBig;
    l_run[j] = 0.f;
#pragma unroll
    for (int e = 0; e < C::EPC; ++e) acc[j][e] = 0.f;
  }

  // ring slot (raw_lo + n - n_c) mod R of the keys this lane loads, without a division per
  // load: the slot of its u = 0 key is carried from iteration to iteration, key u adds u steps
  // of NWAVE*KPW keys (R < 2^30, so the sums stay in 32 bits)
  const int Ri = (int)R;
  const int r_step = (int)(C::KPI % R), r_u = (int)((C::NWAVE * C::KPW) % R);
  int slot0 = (int)((raw_lo - n_c + start + (int64_t)wave * C::KPW + kg) % R);
  if (slot0 < 0) slot0 += Ri;
  int slot_start = (int)((raw_lo - n_c + start) % R);   // key `start`, read by the lanes past `end`
  if (slot_start < 0) slot_start += Ri;
  for (int64_t base = start; base < end; base += C::KPI) {
    uint4 kr[C::U], vr[C::U];
    bool ok[C::U];
    int sl = slot0;   // slot of key u of this lane
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      const int64_t n = base + (int64_t)(u * C::NWAVE + wave) * C::KPW + kg;
      ok[u] = n < end;
      const int64_t nn = ok[u] ? n : start;
      const T* kp;
      const T* vp;
      if (nn < n_c) {
        kp = ck + (size_t)nn * D;
        vp = cv + (size_t)nn * D;
      } else if (nn == n_keys - 1) {
        kp = kt_new;   // the token appended by this very call
        vp = vt_new;
      } else {
        const int slot = ok[u] ? sl : slot_start;
        kp = rk + (size_t)slot * D;
        vp = rv + (size_t)slot * D;
      }
      kr[u] = ld16_kv<STREAM>(kp + part * C::EPC);
      vr[u] = ld16_kv<STREAM>(vp + part * C::EPC);
      sl += r_u;
      if (sl >= Ri) sl -= Ri;
    }
    slot0 += r_step;
    if (slot0 >= Ri) slot0 -= Ri;
    float s[C::U][RH];
    float vf[C::U][C::EPC];
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      float kf[C::EPC];
      Elem<T>::chunk_to_f32(kr[u], kf);
      Elem<T>::chunk_to_f32(vr[u], vf[u]);
#pragma unroll
      for (int j = 0; j < RH; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < C::EPC; ++e) dot = fmaf(qf[j][e], kf[e], dot);
        if constexpr (C::LPK <= 16) {
          dot = lane_group_sum<C::LPK>(dot);
        } else {
          dot = lane_group_sum<16>(dot);
#pragma unroll
          for (int bb = 16; bb < C::LPK; bb <<= 1) dot += __shfl_xor(dot, bb, kWave);
        }
        s[u][j] = ok[u] ? dot : -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < RH; ++j) {
      float mx = s[0][j];
#pragma unroll
      for (int u = 1; u < C::U; ++u) mx = fmaxf(mx, s[u][j]);
      // the reference point moves only when a score exceeds it by more than 16 (weights
      // stay <= 2^16); the wave skips the rescale when no lane needs it
      const bool move = mx > m_run[j] + 16.f;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float m_new = move ? mx : m_run[j];
        const float alpha = fast_exp2(m_run[j] - m_new);
        m_run[j] = m_new;
        l_run[j] *= alpha;
#pragma unroll
        for (int e = 0; e < C::EPC; ++e) acc[j][e] *= alpha;
      }
      const float m_new = m_run[j];
#pragma unroll
      for (int u = 0; u < C::U; ++u) {
        const float p = fast_exp2(s[u][j] - m_new);
        l_run[j] += p;
#pragma unroll
        for (int e = 0; e < C::EPC; ++e) acc[j][e] = fmaf(p, vf[u][e], acc[j][e]);
      }
    }
  }

  // ---- combine the key slots of the wave (lanes with equal `part`), then the waves
#pragma unroll
  for (int j = 0; j < RH; ++j) {
#pragma unroll
    for (int bb = C::LPK; bb < kWave; bb <<= 1) {
      const float mo = __shfl_xor(m_run[j], bb, kWave);
      const float lo = __shfl_xor(l_run[j], bb, kWave);
      const float M = fmaxf(m_run[j], mo);
      const float a1 = fast_exp2(m_run[j] - M), a2 = fast_exp2(mo - M);
      l_run[j] = l_run[j] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < C::EPC; ++e) {
        const float ao = __shfl_xor(acc[j][e], bb, kWave);
        acc[j][e] = acc[j][e] * a1 + ao * a2;
      }
      m_run[j] = M;
    }
    if (lane < C::LPK) {
#pragma unroll
      for (int e = 0; e < C::EPC; ++e) red[wave][j][part * C::EPC + e] = acc[j][e];
      if (lane == 0) {
        red[wave][j][D] = m_run[j];
        red[wave][j][D + 1] = l_run[j];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < RH * D; idx += C::NT) {
    const int j = idx / D, col = idx - j * D;
    float M = red[0][j][D];
#pragma unroll
    for (int w = 1; w < C::NWAVE; ++w) M = fmaxf(M, red[w][j][D]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < C::NWAVE; ++w) {
      const float f = fast_exp2(red[w][j][D] - M);
      a = fmaf(f, red[w][j][col], a);
      l = fmaf(f, red[w][j][D + 1], l);
    }
    const size_t rec = ((size_t)b * Hq + h0 + j) * nchunks + ci;
    ws_acc[rec * D + col] = a;
    if (col == 0) {
      ws_ml[rec * 2] = M;
      ws_ml[rec * 2 + 1] = l;
    }
  }
}

int heads_per_block(int nq) {
  if (nq % 8 == 0) return 8;
  if (nq % 4 == 0) return 4;
  if (nq % 2 == 0) return 2;
  return 1;
}

template <typename T, int D, int RH, bool STREAM, bool LCA>
void launch_serve_kernel(dim3 grid, size_t lds, hipStream_t stream, const cca_cache_t* c, int32_t* lens,
                         int64_t max_len, const void* q, const void* k, const void* v, float* ws_acc, float* ws_ml,
                         int nq, int nhb, int64_t R, int nchunks, float scale, float* qsum,
                         int d_rope) {
  hipLaunchKernelGGL((cca_serve_decode_kernel<T, D, RH, STREAM, LCA>), grid, dim3(256), lds, stream, lens, max_len,
                     (const T*)q, (const T*)k, (const T*)v, (T*)c->core_k, (T*)c->core_v, (T*)c->ring_k,
                     (T*)c->ring_v, ws_acc, ws_ml, c->H, nq, nhb, c->max_groups, R, c->g, c->k_local, nchunks,
                     scale, qsum, d_rope);
}

template <typename T, int D, int RH>
hipError_t launch_serve_t(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q, const void* q,
                          const void* k, const void* v, void* out, int out_f32, void* workspace, float scale,
                          float* qsum, int d_rope, hipStream_t stream) {
  const int nq = H_q / c->H;
  const int nhb = nq / RH;
  const int64_t R = (int64_t)(c->k_local + 1) * c->g;
  const int nchunks = serve_num_chunks(c, H_q, max_len);
  // Upper bound of a sequence's key count, for the choice of streaming loads: a token at
  // t <= max_len has n_c(t) <= n_c(max_len) core tokens plus at most min(t+1, (k_local+1)*g)
  // raw ones.  (A shorter sequence can have more keys than the longest: the raw part
  // grows with t mod g.)
  const int64_t n_c_max = std::max<int64_t>(0, max_len / c->g - c->k_local);
  const int64_t n_keys_max = n_c_max + std::min<int64_t>(max_len + 1, R);
  float* ws_acc = (float*)workspace;
  float* ws_ml = ws_acc + (size_t)c->B * H_q * nchunks * D;
  const int64_t nblk = (int64_t)c->B * c->H * nhb;
  // K/V bytes of the step if every sequence were max_len long (an upper bound)
  const bool stream_kv = (int64_t)c->B * c->H * n_keys_max * D * (int64_t)sizeof(T) * 2 > kStreamBytes;
  const dim3 grid((unsigned)(nblk * nchunks));
  // pooling scratch: g scores (CCA); the mean query and g scores (LCA-style)
  const bool lca = qsum != nullptr;
  const size_t lds = (size_t)(lca ? D + c->g : c->g) * sizeof(float);
  if (lca) {
    if (stream_kv)
      launch_serve_kernel<T, D, RH, true, true>(grid, lds, stream, c, lens, max_len, q, k, v, ws_acc, ws_ml, nq, nhb,
                                                R, nchunks, scale, qsum, d_rope);
    else
      launch_serve_kernel<T, D, RH, false, true>(grid, lds, stream, c, lens, max_len, q, k, v, ws_acc, ws_ml, nq,
                                                 nhb, R, nchunks, scale, qsum, d_rope);
  } else {
    if (stream_kv)
      launch_serve_kernel<T, D, RH, true, false>(grid, lds, stream, c, lens, max_len, q, k, v, ws_acc, ws_ml, nq,
                                                 nhb, R, nchunks, scale, nullptr, 0);
    else
      launch_serve_kernel<T, D, RH, false, false>(grid, lds, stream, c, lens, max_len, q, k, v, ws_acc, ws_ml, nq,
                                                  nhb, R, nchunks, scale, nullptr, 0);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_merge(D, ws_acc, ws_ml, out, out_mode(out_f32, c->dt), (int64_t)c->B * H_q, nchunks, lens, H_q,
                             max_len,
                             stream);
}

template <typename T, int D>
hipError_t launch_serve_d(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q, const void* q,
                          const void* k, const void* v, void* out, int out_f32, void* ws, float scale, float* qsum,
                          int d_rope, hipStream_t stream) {
  switch (heads_per_block(H_q / c->H)) {
    case 8:
      return launch_serve_t<T, D, 8>(c, lens, max_len, H_q, q, k, v, out, out_f32, ws, scale, qsum, d_rope, stream);
    case 4:
      return launch_serve_t<T, D, 4>(c, lens, max_len, H_q, q, k, v, out, out_f32, ws, scale, qsum, d_rope, stream);
    case 2:
      return launch_serve_t<T, D, 2>(c, lens, max_len, H_q, q, k, v, out, out_f32, ws, scale, qsum, d_rope, stream);
    default:
      return launch_serve_t<T, D, 1>(c, lens, max_len, H_q, q, k, v, out, out_f32, ws, scale, qsum, d_rope, stream);
  }
}

}  // namespace

int serve_num_chunks(const cca_cache_t* c, int H_q, int64_t max_len) {
  // About 1024 workgroups in total, as for the uniform decode; at least 256 keys
  // of the cache's capacity per chunk, at most 64 chunks.  max_len is not used:
  // the workspace size depends on the cache and the head count only.
  (void)max_len;
  const int nq = H_q / c->H;
  const int64_t nblk = (int64_t)c->B * c->H * (nq / heads_per_block(nq));
  const int64_t cap = c->max_groups + (int64_t)(c->k_local + 1) * c->g;
  int64_t n = (1024 + nblk - 1) / nblk;
  n = std::min<int64_t>(n, std::max<int64_t>(1, cap / 256));
  n = std::max<int64_t>(1, std::min<int64_t>(n, 64));
  return (int)n;
}

size_t serve_workspace_bytes(const cca_cache_t* c, int H_q) {
  return (size_t)c->B * H_q * (size_t)serve_num_chunks(c, H_q, 0) * ((size_t)c->d + 2) * sizeof(float);
}

hipError_t launch_serve_append_decode(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q,
                                      const void* q, const void* k, const void* v, void* out, int out_f32,
                                      void* workspace, float scale, hipStream_t stream, float* qsum, int d_rope) {
  return dispatch_td(c->dt, c->d, [&](auto t, auto dd) {
    using T = decltype(t);
    return launch_serve_d<T, decltype(dd)::value>(c, lens, max_len, H_q, q, k, v, out, sizeof(T) == 4 ? 1 : out_f32,
                                                  workspace, scale, qsum, d_rope, stream);
  });
}

}  // namespace cca
