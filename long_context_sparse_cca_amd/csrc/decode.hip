// Decode against the compressed CCA KV cache (core-token array + raw ring).
//
// Method: the CCA write-up ("ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"):
// the Triton section says the fused operator serves decode with a KV cache,
// and the compute/memory-efficiency section (Fig. 3) that the cache holds the
// core tokens plus the local raw tokens.  A group is pooled as soon as its last
// token arrives (its query is the group's last query, global-aware pooling
// section); the core token becomes visible once the group has left the
// window (locality-preserving module, group-aligned window).
//
//   cca_copy_rows_kernel    : seed the cache from a prefill (core tokens + raw tail)
//   cca_append_kernel       : write the newest k,v into its ring slot; pool a completed group
//   cca_decode_kernel       : one chunk of the visible keys per workgroup -> (m, l, acc[d]);
//                             optionally also performs the append of the new token, with
//                             CCA pooling or the LCA-style condensation ("Latent-Condensed
//                             Transformer for Efficient Long Context Modeling", section 2,
//                             inference flow) of a completed group
//   cca_decode_merge_kernel : log-sum-exp combination of the chunk states -> out[d]
//   cca_qsum_seed_kernel    : running query sums of the trailing partial group (LCA-style cache)
#include <algorithm>

#include "cca_internal.h"
#include "lca_group.h"
#include "pool_group.h"

namespace cca {
namespace {

// ---------------------------------------------------------------------------
// row copies (cache seeding)
// ---------------------------------------------------------------------------
// For every slice bh and row r < nrows: dst[bh][(dst_row0 + r) % dst_mod] = src[bh][src_row0 + r],
// for the two (src, dst) pairs (K and V).  Rows are `cpr` 16-byte chunks.
__global__ __launch_bounds__(256) void cca_copy_rows_kernel(const uint4* __restrict__ src0, uint4* __restrict__ dst0,
                                                            const uint4* __restrict__ src1, uint4* __restrict__ dst1,
                                                            int64_t BH, int64_t nrows, int cpr, int64_t src_rows,
                                                            int64_t src_row0, int64_t dst_rows, int64_t dst_row0,
                                                            int64_t dst_mod) {
  const int64_t total = BH * nrows * cpr;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = idx % cpr;
    const int64_t rr = idx / cpr;
    const int64_t r = rr % nrows;
    const int64_t bh = rr / nrows;
    const int64_t s = (bh * src_rows + src_row0 + r) * cpr + c;
    const int64_t d = (bh * dst_rows + (dst_row0 + r) % dst_mod) * cpr + c;
    dst0[d] = src0[s];
    dst1[d] = src1[s];
  }
}

hipError_t copy_rows(const void* s0, void* d0, const void* s1, void* d1, int64_t BH, int64_t nrows, int cpr,
                     int64_t src_rows, int64_t src_row0, int64_t dst_rows, int64_t dst_row0, int64_t dst_mod,
                     hipStream_t stream) {
  const int64_t total = BH * nrows * cpr;
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(cca_copy_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint4*)s0,
                     (uint4*)d0, (const uint4*)s1, (uint4*)d1, BH, nrows, cpr, src_rows, src_row0, dst_rows,
                     dst_row0, dst_mod);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// append one token per sequence (+ in-place pooling of a completed group)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void cca_append_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                        const T* __restrict__ v, T* __restrict__ ring_k,
                                                        T* __restrict__ ring_v, T* __restrict__ core_k,
                                                        T* __restrict__ core_v, int64_t R, int64_t max_groups,
                                                        int64_t t, int g, float scale) {
  extern __shared__ float w_lds[];
  const int64_t bh = blockIdx.x;
  const int lane = threadIdx.x;
  constexpr int CPR = D * (int)sizeof(T) / 16;
  const T* qt = q + (size_t)bh * D;
  const T* kt = k + (size_t)bh * D;
  const T* vt = v + (size_t)bh * D;
  const int64_t slot = t % R;
  T* rk = ring_k + ((size_t)bh * R + slot) * D;
  T* rv = ring_v + ((size_t)bh * R + slot) * D;
  if (lane < CPR) {
    st16(reinterpret_cast<uint4*>(rk) + lane, ld16(reinterpret_cast<const uint4*>(kt) + lane));
    st16(reinterpret_cast<uint4*>(rv) + lane, ld16(reinterpret_cast<const uint4*>(vt) + lane));
  }
  if ((t + 1) % g != 0) return;
  // the group [beta*g, beta*g+g) occupies slots slot-g+1 .. slot (R is a multiple of g)
  const int64_t beta = t / g;
  const int64_t first = slot - (g - 1);
  const T* gk = ring_k + ((size_t)bh * R + first) * D;
  const T* gv = ring_v + ((size_t)bh * R + first) * D;
  T* ck = core_k + ((size_t)bh * max_groups + beta) * D;
  T* cv = core_v + ((size_t)bh * max_groups + beta) * D;
  pool_group_wave<T, D>(qt, 0, 1, gk, gv, kt, vt, g, scale, ck, cv, w_lds);
}

template <typename T, int D>
hipError_t launch_append_t(const cca_cache_t* c, const void* q, const void* k, const void* v, float scale,
                           hipStream_t stream) {
  const int64_t BH = (int64_t)c->B * c->H;
  const int64_t R = (int64_t)(c->k_local + 1) * c->g;
  hipLaunchKernelGGL((cca_append_kernel<T, D>), dim3((unsigned)BH), dim3(64), (size_t)c->g * sizeof(float), stream,
                     (const T*)q, (const T*)k, (const T*)v, (T*)c->ring_k, (T*)c->ring_v, (T*)c->core_k,
                     (T*)c->core_v, R, c->max_groups, c->n_tokens, c->g, scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// split-KV decode with the chunk merge fused in (and, optionally, the append)
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DecodeCfg {
  static constexpr int NWAVE = 4;
  static constexpr int NT = NWAVE * kWave;
  static constexpr int EPC = 16 / (int)sizeof(T);     // elements per lane (one 16-byte chunk)
  static constexpr int LPK = D / EPC;                 // lanes per key
  static constexpr int KPW = kWave / LPK;             // keys per wave per load
  static constexpr int U = 4;                         // loads in flight per lane (per K and V)
  static constexpr int KPI = NWAVE * KPW * U;         // keys per workgroup iteration
};

// Workspace layout (floats): acc [BH][NC][D], then ml [BH][NC][2] (running max in
// log2 units, running sum) of every chunk.
struct DecodeWs {
  float* acc;
  float* ml;
};

// One workgroup = one chunk of the key index space [0, n_keys) of one slice:
// keys [0, n_c) are core tokens, keys [n_c, n_keys) the raw window read from the ring
// (with APPEND, the last key is the new token, read from the inputs).  It writes its
// partial softmax state; cca_decode_merge_kernel combines the chunks of a slice.
// With APPEND, wave 0 of chunk 0 also writes the new token into its ring slot and,
// when the token completes a group, pools that group into the core array (the new
// core token is not visible to this step, so nothing here reads it).  APPEND = 1
// pools as CCA does (the last query scores the group); APPEND = 2 condenses the
// LCA way: qsum [B*H, D] (float32) holds the running sum of the current group's
// queries, the completed group is scored with their mean, and its positional dims
// (the last d_rope) come from the top-scored token.
template <typename T, int D, int APPEND, bool STREAM>
__global__ __launch_bounds__(256) void cca_decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new, T* __restrict__ core_k,
    T* __restrict__ core_v, T* __restrict__ ring_k, T* __restrict__ ring_v, DecodeWs ws, int64_t max_groups,
    int64_t R, int64_t t, int g, int64_t n_c, int64_t raw_lo, int64_t n_keys, int64_t chunk, int nchunks,
    float scale, float* __restrict__ qsum, int d_rope) {
  using C = DecodeCfg<T, D>;
  __shared__ float red[C::NWAVE][D + 2];
  extern __shared__ float pool_lds[];
  const int64_t bh = blockIdx.x;
  const int ci = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  const int kg = lane / C::LPK;      // key slot within the wave
  const int part = lane % C::LPK;    // which 16-byte chunk of the row
  const int64_t start = (int64_t)ci * chunk;
  const int64_t end = min(n_keys, start + chunk);
  const T* qrow = q + (size_t)bh * D;

  if constexpr (APPEND != 0) {
    if (ci == 0 && wave == 0) {
      const T* kt = k_new + (size_t)bh * D;
      const T* vt = v_new + (size_t)bh * D;
      const int64_t slot = t % R;
      constexpr int CPR = D * (int)sizeof(T) / 16;
      if (lane < CPR) {
        st16(reinterpret_cast<uint4*>(ring_k + ((size_t)bh * R + slot) * D) + lane,
             ld16(reinterpret_cast<const uint4*>(kt) + lane));
        st16(reinterpret_cast<uint4*>(ring_v + ((size_t)bh * R + slot) * D) + lane,
             ld16(reinterpret_cast<const uint4*>(vt) + lane));
      }
      if constexpr (APPEND == 1) {
        if ((t + 1) % g == 0) {
          const int64_t beta = t / g;
          const int64_t first = slot - (g - 1);
          pool_group_wave<T, D>(qrow, 0, 1, ring_k + ((size_t)bh * R + first) * D,
                                ring_v + ((size_t)bh * R + first) * D, kt, vt, g, scale,
                                core_k + ((size_t)bh * max_groups + beta) * D,
                                core_v + ((size_t)bh * max_groups + beta) * D, pool_lds);
        }
      } else {
        // running sum of the group's queries (in token order, as the prefill sums them)
        constexpr int CPL = D / kWave;
        const int col = lane * CPL;
        float qf[CPL], qs[CPL];
        lca_load_cols<T, D>(qrow + col, qf);
        float* qsum_row = qsum + (size_t)bh * D + col;
#pragma unroll
        for (int e = 0; e < CPL; ++e) qs[e] = qsum_row[e] + qf[e];
        if ((t + 1) % g == 0) {
          const float inv_g = 1.0f / ((float)g * 1.0f);
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            pool_lds[col + e] = qs[e] * inv_g;
            qsum_row[e] = 0.f;
          }
          wave_lds_sync();
          const int64_t beta = t / g;
          const int64_t first = slot - (g - 1);
          lca_condense_wave<T, D>(pool_lds, ring_k + ((size_t)bh * R + first) * D,
                                  ring_v + ((size_t)bh * R + first) * D, kt, vt, g, scale, d_rope,
                                  core_k + ((size_t)bh * max_groups + beta) * D,
                                  core_v + ((size_t)bh * max_groups + beta) * D, pool_lds + D, nullptr);
        } else {
#pragma unroll
          for (int e = 0; e < CPL; ++e) qsum_row[e] = qs[e];
        }
      }
    }
  }

  float qf[C::EPC];
  Elem<T>::chunk_to_f32(ld16(qrow + part * C::EPC), qf);
  const float sc = scale * kLog2e;
#pragma unroll
  for (int e = 0; e < C::EPC; ++e) qf[e] *= sc;

  const T* ck = core_k + (size_t)bh * max_groups * D;
  const T* cv = core_v + (size_t)bh * max_groups * D;
  const T* rk = ring_k + (size_t)bh * R * D;
  const T* rv = ring_v + (size_t)bh * R * D;

  float m_run = kNegBig, l_run = 0.f;
  float acc[C::EPC];
#pragma unroll
  for (int e = 0; e < C::EPC; ++e) acc[e] = 0.f;

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
      } else if (APPEND != 0 && nn == n_keys - 1) {
        kp = k_new + (size_t)bh * D;   // the token appended by this very launch
        vp = v_new + (size_t)bh * D;
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
    float s[C::U];
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      float kf[C::EPC];
      Elem<T>::chunk_to_f32(kr[u], kf);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < C::EPC; ++e) dot = fmaf(qf[e], kf[e], dot);
#pragma unroll
      for (int b = 1; b < C::LPK; b <<= 1) dot += __shfl_xor(dot, b, kWave);
      s[u] = ok[u] ? dot : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int u = 1; u < C::U; ++u) mx = fmaxf(mx, s[u]);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < C::EPC; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      const float p = fast_exp2(s[u] - m_new);
      l_run += p;
      float vf[C::EPC];
      Elem<T>::chunk_to_f32(vr[u], vf);
#pragma unroll
      for (int e = 0; e < C::EPC; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
    }
  }

  // combine the key slots of the wave (lanes with equal `part`)
#pragma unroll
  for (int b = C::LPK; b < kWave; b <<= 1) {
    const float mo = __shfl_xor(m_run, b, kWave);
    const float lo = __shfl_xor(l_run, b, kWave);
    const float M = fmaxf(m_run, mo);
    const float a1 = fast_exp2(m_run - M), a2 = fast_exp2(mo - M);
    l_run = l_run * a1 + lo * a2;
#pragma unroll
    for (int e = 0; e < C::EPC; ++e) {
      const float ao = __shfl_xor(acc[e], b, kWave);
      acc[e] = acc[e] * a1 + ao * a2;
    }
    m_run = M;
  }
  if (lane < C::LPK) {
#pragma unroll
    for (int e = 0; e < C::EPC; ++e) red[wave][part * C::EPC + e] = acc[e];
    if (lane == 0) {
      red[wave][D] = m_run;
      red[wave][D + 1] = l_run;
    }
  }
  __syncthreads();
  // combine the waves: thread x < D owns column x; publish the chunk's partial state
  const size_t rec = (size_t)bh * nchunks + ci;
  if (tid < D) {
    float M = red[0][D];
#pragma unroll
    for (int w = 1; w < C::NWAVE; ++w) M = fmaxf(M, red[w][D]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < C::NWAVE; ++w) {
      const float f = fast_exp2(red[w][D] - M);
      a = fmaf(f, red[w][tid], a);
      l = fmaf(f, red[w][D + 1], l);
    }
    ws.acc[rec * D + tid] = a;
    if (tid == 0) {
      ws.ml[rec * 2] = M;
      ws.ml[rec * 2 + 1] = l;
    }
  }
}

// One wave per slice.  Lane c reads chunk c's (max, sum) -- all chunks in parallel --
// then every lane accumulates its D/64 columns over the chunks, the chunk weight
// taken from lane c with a scalar read.  With `lens` non-null (serving step), the
// first slice of every sequence then advances that sequence's length by one, after
// the decode kernel of the same call has read it.
template <int D>
__global__ __launch_bounds__(64) void cca_decode_merge_kernel(const float* __restrict__ ws_acc,
                                                              const float* __restrict__ ws_ml, void* __restrict__ out,
                                                              int out_mode, int nchunks, int32_t* __restrict__ lens,
                                                              int slices_per_seq, int64_t max_len) {
  const int64_t bh = blockIdx.x;
  const int lane = threadIdx.x;
  constexpr int CPL = D / kWave;
  const float* ml = ws_ml + (size_t)bh * nchunks * 2;
  float mc = kNegBig, lc = 0.f;
  if (lane < nchunks) {
    mc = ml[2 * lane];
    lc = ml[2 * lane + 1];
  }
  const float M = wave_max_xor(mc, 1, kWave);
  const float f = fast_exp2(mc - M);
  const float l = wave_sum_xor(lane < nchunks ? f * lc : 0.f, 1, kWave);
  float a[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) a[e] = 0.f;
  const float* ac = ws_acc + (size_t)bh * nchunks * D + lane * CPL;
  int c = 0;
  for (; c + 4 <= nchunks; c += 4) {
    float x[4][CPL];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < CPL; ++e) x[u][e] = ac[(size_t)(c + u) * D + e];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float fc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), c + u));
#pragma unroll
      for (int e = 0; e < CPL; ++e) a[e] = fmaf(fc, x[u][e], a[e]);
    }
  }
  for (; c < nchunks; ++c) {
    const float fc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), c));
#pragma unroll
    for (int e = 0; e < CPL; ++e) a[e] = fmaf(fc, ac[(size_t)c * D + e], a[e]);
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    const size_t o = (size_t)bh * D + lane * CPL + e;
    if (out_mode == 1) reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_bits(a[e] * inv);
    else if (out_mode == 2) reinterpret_cast<uint16_t*>(out)[o] = f32_to_f16_bits(a[e] * inv);
    else reinterpret_cast<float*>(out)[o] = a[e] * inv;
  }
  if (lens != nullptr && lane == 0 && bh % slices_per_seq == 0) {
    const int64_t b = bh / slices_per_seq;
    const int32_t t = lens[b];
    if (t >= 0 && t <= max_len) lens[b] = t + 1;
  }
}

template <typename T, int D, int APPEND>
hipError_t launch_decode_t(const cca_cache_t* c, const void* q, const void* k_new, const void* v_new, void* out,
                           int out_f32, void* workspace, float scale, float* qsum, int d_rope, hipStream_t stream) {
  const int64_t BH = (int64_t)c->B * c->H;
  const int64_t R = (int64_t)(c->k_local + 1) * c->g;
  const int64_t t = APPEND ? c->n_tokens : c->n_tokens - 1;   // position of the query
  const int64_t n_c = std::max<int64_t>(0, t / c->g - c->k_local);
  const int64_t raw_lo = n_c * c->g;
  const int64_t n_keys = n_c + (t - raw_lo + 1);
  const int nchunks = decode_num_chunks(c);
  int64_t chunk = (n_keys + nchunks - 1) / nchunks;
  chunk = (chunk + 15) / 16 * 16;
  DecodeWs ws;
  ws.acc = (float*)workspace;
  ws.ml = ws.acc + (size_t)BH * nchunks * D;
  // pooling scratch: g scores (CCA); the mean query and g scores (LCA-style)
  const size_t dyn_lds = APPEND == 1 ? (size_t)c->g * sizeof(float)
                                     : (APPEND == 2 ? (size_t)(D + c->g) * sizeof(float) : 0);
  const bool stream_kv = BH * n_keys * D * (int64_t)sizeof(T) * 2 > kStreamBytes;
  if (stream_kv)
    hipLaunchKernelGGL((cca_decode_kernel<T, D, APPEND, true>), dim3((unsigned)BH, nchunks), dim3(256), dyn_lds,
                       stream, (const T*)q, (const T*)k_new, (const T*)v_new, (T*)c->core_k, (T*)c->core_v,
                       (T*)c->ring_k, (T*)c->ring_v, ws, c->max_groups, R, t, c->g, n_c, raw_lo, n_keys, chunk,
                       nchunks, scale, qsum, d_rope);
  else
    hipLaunchKernelGGL((cca_decode_kernel<T, D, APPEND, false>), dim3((unsigned)BH, nchunks), dim3(256), dyn_lds,
                       stream, (const T*)q, (const T*)k_new, (const T*)v_new, (T*)c->core_k, (T*)c->core_v,
                       (T*)c->ring_k, (T*)c->ring_v, ws, c->max_groups, R, t, c->g, n_c, raw_lo, n_keys, chunk,
                       nchunks, scale, qsum, d_rope);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((cca_decode_merge_kernel<D>), dim3((unsigned)BH), dim3(64), 0, stream, ws.acc, ws.ml, out,
                     out_mode(out_f32, c->dt), nchunks, (int32_t*)nullptr, 1, (int64_t)0);
  return hipGetLastError();
}

template <int APPEND>
hipError_t launch_decode_any(const cca_cache_t* c, const void* q, const void* k, const void* v, void* out,
                             int out_f32, void* workspace, float scale, float* qsum, int d_rope,
                             hipStream_t stream) {
  return dispatch_td(c->dt, c->d, [&](auto t, auto dd) {
    using T = decltype(t);
    return launch_decode_t<T, decltype(dd)::value, APPEND>(c, q, k, v, out, sizeof(T) == 4 ? 1 : out_f32, workspace,
                                                           scale, qsum, d_rope, stream);
  });
}

// Running sums of the queries of each slice's trailing partial group (rows m*g .. L-1)
// of a prefill, over the nq query slices bh*nq .. that share cached slice bh, to seed the
// LCA-style cache: one wave per cached slice, D/64 columns per lane; token by token,
// each token's heads first (the order in which decode steps add them).
template <typename T, int D>
__global__ __launch_bounds__(64) void cca_qsum_seed_kernel(const T* __restrict__ q, float* __restrict__ qsum,
                                                           int64_t L, int64_t row0, int nq) {
  constexpr int CPL = D / kWave;
  const int64_t bh = blockIdx.x;
  const int col = threadIdx.x * CPL;
  float s[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) s[e] = 0.f;
  for (int64_t r = row0; r < L; ++r) {
    float t[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) t[e] = 0.f;
    for (int h = 0; h < nq; ++h) {
      float f[CPL];
      lca_load_cols<T, D>(q + (((size_t)bh * nq + h) * L + r) * D + col, f);
#pragma unroll
      for (int e = 0; e < CPL; ++e) t[e] += f[e];
    }
#pragma unroll
    for (int e = 0; e < CPL; ++e) s[e] += t[e];
  }
#pragma unroll
  for (int e = 0; e < CPL; ++e) qsum[(size_t)bh * D + col + e] = s[e];
}

template <typename T, int D>
hipError_t launch_qsum_seed_t(const cca_cache_t* c, const void* q, float* qsum, int64_t L, int nq,
                              hipStream_t stream) {
  const int64_t BH = (int64_t)c->B * c->H;
  const int64_t row0 = L / c->g * c->g;
  hipLaunchKernelGGL((cca_qsum_seed_kernel<T, D>), dim3((unsigned)BH), dim3(64), 0, stream, (const T*)q, qsum, L,
                     row0, nq);
  return hipGetLastError();
}

}  // namespace

int decode_num_chunks(const cca_cache_t* c) {
  // About 1024 workgroups in total (4 per CU of a 256-CU MI355X; measured best
  // against 2..19 per slice at B=8, H=32): long contiguous chunks, all resident
  // at once.  At least 256 keys of the cache's capacity per chunk, at most 64
  // chunks per slice.
  const int64_t BH = (int64_t)c->B * c->H;
  const int64_t cap = c->max_groups + (int64_t)(c->k_local + 1) * c->g;
  int64_t n = (1024 + BH - 1) / BH;
  n = std::min<int64_t>(n, std::max<int64_t>(1, cap / 256));
  n = std::max<int64_t>(1, std::min<int64_t>(n, 64));
  return (int)n;
}

size_t decode_workspace_bytes(const cca_cache_t* c) {
  const size_t BH = (size_t)c->B * c->H;
  return BH * (size_t)decode_num_chunks(c) * ((size_t)c->d + 2) * sizeof(float);
}

hipError_t launch_cache_load(const cca_cache_t* c, const void* k, const void* v, const void* kc, const void* vc,
                             int64_t L, hipStream_t stream) {
  const int64_t BH = (int64_t)c->B * c->H;
  const int cpr = c->d * dtype_bytes(c->dt) / 16;
  const int64_t m = L / c->g;
  const int64_t R = (int64_t)(c->k_local + 1) * c->g;
  hipError_t e = copy_rows(kc, c->core_k, vc, c->core_v, BH, m, cpr, m, 0, c->max_groups, 0, INT64_MAX, stream);
  if (e != hipSuccess) return e;
  const int64_t lo = std::max<int64_t>(0, m - c->k_local) * c->g;
  return copy_rows(k, c->ring_k, v, c->ring_v, BH, L - lo, cpr, L, lo, R, lo, R, stream);
}

hipError_t launch_cache_append(const cca_cache_t* c, const void* q, const void* k, const void* v, float scale,
                               hipStream_t stream) {
  return dispatch_td(c->dt, c->d, [&](auto t, auto dd) {
    return launch_append_t<decltype(t), decltype(dd)::value>(c, q, k, v, scale, stream);
  });
}

hipError_t launch_decode_merge(int d, const float* ws_acc, const float* ws_ml, void* out, int out_mode,
                               int64_t nslices, int nchunks, int32_t* lens, int slices_per_seq, int64_t max_len,
                               hipStream_t stream) {
  if (nslices == 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL((cca_decode_merge_kernel<128>), dim3((unsigned)nslices), dim3(64), 0, stream, ws_acc, ws_ml,
                       out, out_mode, nchunks, lens, slices_per_seq, max_len);
  else
    hipLaunchKernelGGL((cca_decode_merge_kernel<64>), dim3((unsigned)nslices), dim3(64), 0, stream, ws_acc, ws_ml,
                       out, out_mode, nchunks, lens, slices_per_seq, max_len);
  return hipGetLastError();
}

hipError_t launch_decode(const cca_cache_t* c, const void* q, void* out, int out_f32, void* workspace, float scale,
                         hipStream_t stream) {
  return launch_decode_any<0>(c, q, nullptr, nullptr, out, out_f32, workspace, scale, nullptr, 0, stream);
}

hipError_t launch_append_decode(const cca_cache_t* c, const void* q, const void* k, const void* v, void* out,
                                int out_f32, void* workspace, float scale, hipStream_t stream) {
  return launch_decode_any<1>(c, q, k, v, out, out_f32, workspace, scale, nullptr, 0, stream);
}

hipError_t launch_append_decode_lca(const cca_cache_t* c, float* qsum, int d_rope, const void* q, const void* k,
                                    const void* v, void* out, int out_f32, void* workspace, float scale,
                                    hipStream_t stream) {
  return launch_decode_any<2>(c, q, k, v, out, out_f32, workspace, scale, qsum, d_rope, stream);
}

hipError_t launch_qsum_seed(const cca_cache_t* c, const void* q, float* qsum, int64_t L, int nq,
                            hipStream_t stream) {
  return dispatch_td(c->dt, c->d, [&](auto t, auto dd) {
    return launch_qsum_seed_t<decltype(t), decltype(dd)::value>(c, q, qsum, L, nq, stream);
  });
}

}  // namespace cca
