// Fused CCA prefill attention for gfx950: one online softmax per query over the
// union of the visible core tokens and the group-aligned raw window.
//
// Method: the CCA write-up ("ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"),
// locality-preserving module (local-window equation) and global-local fusion
// (unified K/V and per-position output equations): query t of group
// beta = t/g sees core tokens Kc[0 : beta-k) and raw keys K[(beta-k)*g .. t]
// (lower bound clamped at 0), and one softmax spans both.  The Triton section
// of the same page describes fusing both parts into one flash-style operator;
// this kernel is an MI355X design of that idea, not a translation.
//
// Structure (per workgroup = 4 waves = 128 consecutive queries of one (b,h)):
//   * key tiles of BN keys are staged in LDS: K row-major, V transposed so that
//     the PV product reads 4 or 8 consecutive keys per lane;
//   * the tile loop visits the core tiles [0, n_c_max) then the raw tiles
//     [rl_min, t_max]; each wave classifies every 32-key sub-block as skipped,
//     fully visible or masked for its own 32 queries;
//   * S^T = K Q^T on MFMA (32x32 output: lane = query, 16 keys per lane), so the
//     running max / sum are per-lane scalars and a row max needs one shuffle;
//   * O^T += V^T P^T on MFMA with P rounded to the input type (bf16 or binary16) or
//     kept fp32.
#include "cca_internal.h"

namespace cca {
namespace {

template <typename T, int D>
struct PrefillCfg {
  static constexpr int BM = 128;                        // queries per workgroup
  static constexpr int NWAVE = 4;
  static constexpr int NT = NWAVE * kWave;              // threads
  static constexpr int EB = sizeof(T);
  static constexpr int EPC = 16 / EB;                   // elements per 16-byte chunk
  static constexpr int BN = (EB == 2) ? 64 : 32;        // keys per LDS tile
  static constexpr int NSB = BN / 32;                   // 32-key sub-blocks per tile
  static constexpr int KP = D + 16 / EB;                // K tile pitch (elements), +16 B
  static constexpr int VP = BN + 16 / EB;               // V^T tile pitch (elements), +16 B
  static constexpr int KPT = 8 / EB;                    // keys packed per 8-byte V^T store
  static constexpr int CPR = D / EPC;                   // 16-byte chunks per row
  static constexpr int KCH = BN * CPR / NT;             // K chunks per thread
  static constexpr int KG = BN / KPT;                   // key groups per V tile
  static constexpr int VUNITS = KG * CPR;               // V^T transpose units
  static constexpr int VU = (VUNITS + NT - 1) / NT;     // units per thread
  static constexpr int NDT = D / 32;                    // 32-wide output tiles along d
  static constexpr int LDS_K = BN * KP;                 // elements per buffer
  static constexpr int LDS_V = D * VP;
  static_assert(BN * CPR % NT == 0, "K tile must split evenly");
};

enum : int { kSkip = 0, kFull = 1, kMask = 2 };

// 32x32x16 MFMA on 16-bit operands of type T (bf16_t or f16_t) held as 16-byte chunks.
template <typename T>
__device__ __forceinline__ f32x16_t mfma_32x32x16(const uint4& a, const uint4& b, const f32x16_t& c) {
  if constexpr (std::is_same_v<T, bf16_t>)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

// Running-max threshold (log2 units) below which the accumulators are not
// rescaled: exp2(s - m_run) then stays <= 2^8, far from overflow in fp32 and
// bf16, and the final division by the row sum is exact in real arithmetic for
// any reference point, so skipping the rescale changes nothing but rounding.
constexpr float kRescaleThreshold = 8.0f;

// Column of key j (0..BN-1) in a bf16 V^T row.  Inside each 16-key chunk the
// quads are stored in the order (0-3, 8-11, 4-7, 12-15): lane half hf of the PV
// product then reads its 8 keys {4hf..4hf+3, 8+4hf..8+4hf+3} as one 16-byte load.
__device__ __forceinline__ int vt_col_bf16(int quad) {  // quad = first key / 4
  const int q4 = quad & 3;
  return (quad >> 2) * 16 + (q4 & 1) * 8 + (q4 >> 1) * 4;
}

// EXT: attention of new tokens over a cached prefix (ExtendArgs): positions are absolute,
// query i of the slice is at ext.pos[b] + i, raw key u is row u - raw0 of the raw slice.
// Without EXT the slice is a whole sequence: pos0 = raw0 = 0, L queries, L raw rows.
template <typename T, int D, bool EXT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void cca_prefill_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ Kc, const T* __restrict__ Vc, void* __restrict__ Out, int out_f32,
    int BH, int nq, int64_t L, int g, int k_local, float scale, int ntiles, ExtendArgs ext,
    float* __restrict__ lse) {
  using C = PrefillCfg<T, D>;
  __shared__ __attribute__((aligned(16))) T lds_k[2][C::LDS_K];
  __shared__ __attribute__((aligned(16))) T lds_v[2][C::LDS_V];

  int bh, qtile;
  map_block(BH * ntiles, ntiles, bh, qtile);
  if constexpr (EXT) bh = kv_major_slice(bh, BH, ext.Hq, nq, ext.order);
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // absolute position of query 0, first raw position of the raw slice, queries per slice
  int64_t pos0 = 0, raw0 = 0, nQ = L, raw_rows = L, core_rows = L / g;
  if constexpr (EXT) {
    pos0 = ext.pos[bh / ext.Hq];
    nQ = ext.n;
    raw_rows = ext.raw_rows;
    core_rows = ext.core_rows;
    if (pos0 < 0) {
      // invalid sequence: NaN outputs, nothing read
      const int64_t i = (int64_t)qtile * C::BM + wave * 32 + l32;
      if (i < nQ) {
        const size_t o = ((size_t)bh * nQ + i) * D;
        for (int c = hf; c < D; c += 2) {
          if (out_f32) reinterpret_cast<float*>(Out)[o + c] = __builtin_nanf("");
          else if constexpr (sizeof(T) == 2) reinterpret_cast<uint16_t*>(Out)[o + c] = Elem<T>::kNaNBits;
        }
      }
      return;
    }
    raw0 = max<int64_t>(0, pos0 / g - k_local) * g;
  }
  const int64_t Lend = pos0 + nQ;                       // one past the last query position
  const int64_t m = core_rows;

  const int64_t q0 = pos0 + (int64_t)qtile * C::BM;
  const int64_t q_last = min(q0 + C::BM - 1, Lend - 1);
  const int64_t nc_wg = max<int64_t>(0, q_last / g - k_local);      // core tokens any row sees
  const int64_t rl_wg = max<int64_t>(0, q0 / g - k_local) * g;      // first raw key any row sees
  const int n_core_tiles = (int)((nc_wg + C::BN - 1) / C::BN);
  const int n_raw_tiles = (int)((q_last - rl_wg + C::BN) / C::BN);
  const int n_tiles = n_core_tiles + n_raw_tiles;

  // ---- this wave's queries
  const int64_t qa = q0 + wave * 32;
  const bool wave_live = qa < Lend;
  const int64_t qb = min(qa + 31, Lend - 1);
  const int64_t q_lane = min(qa + l32, Lend - 1);
  const int64_t cl_lane = q_lane / g - k_local;                      // core visible iff j < cl_lane
  const int64_t rl_lane = max<int64_t>(0, cl_lane) * g;              // raw visible iff rl <= u <= q
  const int64_t cl_min = qa / g - k_local, cl_max = qb / g - k_local;
  const int64_t rl_min = max<int64_t>(0, cl_min) * g, rl_max = max<int64_t>(0, cl_max) * g;

  const int bkv = bh / nq;  // key/value slice read by query slice bh (grouped-query attention)
  const T* Qs = Q + (size_t)bh * nQ * D;                // query slice; row = position - pos0
  const T* Ks = K + (size_t)bkv * raw_rows * D;
  const T* Vs = V + (size_t)bkv * raw_rows * D;
  const T* Kcs = Kc + (size_t)bkv * m * D;
  const T* Vcs = Vc + (size_t)bkv * m * D;

  // ---- Q operand in registers (B operand of S^T = K Q^T).
  // bf16: slice s of 16 dims, lane half hf holds dims 16s+8hf .. +8.
  // f32 : lane half hf holds dims hf*D/2 + s for the D/2 single-K MFMAs.
  constexpr int QREG = (C::EB == 2) ? D / 16 : D / 8;
  uint4 qop[QREG];
  {
    const T* qrow = Qs + (size_t)(q_lane - pos0) * D;
#pragma unroll
    for (int s = 0; s < QREG; ++s) {
      if constexpr (C::EB == 2) qop[s] = ld16(qrow + s * 16 + hf * 8);
      else qop[s] = ld16(qrow + hf * (D / 2) + s * 4);
    }
  }

  f32x16_t acc[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = kNegBig, l_run = 0.f;
  const float sc = scale * kLog2e;

  // ---- tile staging: global -> registers (prefetch) -> LDS (double buffered)
  uint4 kreg[C::KCH];
  uint4 vreg[C::VU][C::KPT];

  auto load_tile = [&](int it) {
    const T *ks, *vs;
    int64_t base, lim, off0;   // tile's first key, last valid key, key of row 0 of the slice
    if (it < n_core_tiles) {
      ks = Kcs; vs = Vcs; base = (int64_t)it * C::BN; lim = m - 1; off0 = 0;
    } else {
      ks = Ks; vs = Vs; base = rl_wg + (int64_t)(it - n_core_tiles) * C::BN; lim = Lend - 1; off0 = raw0;
    }
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
      const int id = tid + i * C::NT;
      const int row = id / C::CPR, c = id % C::CPR;
      const int64_t gr = min(base + row, lim) - off0;
      kreg[i] = ld16(ks + (size_t)gr * D + c * C::EPC);
    }
#pragma unroll
    for (int u = 0; u < C::VU; ++u) {
      const int id = tid + u * C::NT;
      if (id < C::VUNITS) {
        const int a = id % C::KG, c = id / C::KG;   // key group fastest: conflict-free V^T stores
#pragma unroll
        for (int e = 0; e < C::KPT; ++e) {
          const int64_t gr = min(base + a * C::KPT + e, lim) - off0;
          vreg[u][e] = ld16(vs + (size_t)gr * D + c * C::EPC);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
      const int id = tid + i * C::NT;
      const int row = id / C::CPR, c = id % C::CPR;
      st16(&lds_k[buf][row * C::KP + c * C::EPC], kreg[i]);
    }
#pragma unroll
    for (int u = 0; u < C::VU; ++u) {
      const int id = tid + u * C::NT;
      if (id < C::VUNITS) {
        const int a = id % C::KG, c = id / C::KG;
        // transpose: KPT keys x EPC dims -> EPC rows of KPT consecutive keys (8 bytes each)
#pragma unroll
        for (int x = 0; x < C::EPC; ++x) {
          uint2 w;
          int col;
          if constexpr (C::EB == 2) {
            const uint32_t* h0 = reinterpret_cast<const uint32_t*>(&vreg[u][0]);
            const uint32_t* h1 = reinterpret_cast<const uint32_t*>(&vreg[u][1]);
            const uint32_t* h2 = reinterpret_cast<const uint32_t*>(&vreg[u][2]);
            const uint32_t* h3 = reinterpret_cast<const uint32_t*>(&vreg[u][3]);
            const int sh = (x & 1) * 16;
            w.x = ((h0[x >> 1] >> sh) & 0xffffu) | (((h1[x >> 1] >> sh) & 0xffffu) << 16);
            w.y = ((h2[x >> 1] >> sh) & 0xffffu) | (((h3[x >> 1] >> sh) & 0xffffu) << 16);
            col = vt_col_bf16(a);
          } else {
            w.x = reinterpret_cast<const uint32_t*>(&vreg[u][0])[x];
            w.y = reinterpret_cast<const uint32_t*>(&vreg[u][1])[x];
            col = a * C::KPT;
          }
          *reinterpret_cast<uint2*>(&lds_v[buf][(c * C::EPC + x) * C::VP + col]) = w;
        }
      }
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_tiles) load_tile(it + 1);   // global loads stay in flight during the compute

    if (wave_live) {
      const bool core = it < n_core_tiles;
      const int64_t tbase = core ? (int64_t)it * C::BN : rl_wg + (int64_t)(it - n_core_tiles) * C::BN;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
        const int64_t kb = tbase + sb * 32;
        int cls;
        if (core) {
          cls = (kb >= cl_max) ? kSkip : ((kb + 32 <= cl_min) ? kFull : kMask);
        } else {
          if (kb + 31 < rl_min || kb > qb) cls = kSkip;
          else if (kb >= rl_max && kb + 31 <= qa) cls = kFull;
          else cls = kMask;
        }
        if (cls == kSkip) continue;

        // ---- S^T = K Q^T for 32 keys x 32 queries
        f32x16_t s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        if constexpr (C::EB == 2) {
          const T* krow = &lds_k[buf][(sb * 32 + l32) * C::KP + hf * 8];
#pragma unroll
          for (int d16 = 0; d16 < D / 16; ++d16)
            s = mfma_32x32x16<T>(*reinterpret_cast<const uint4*>(krow + d16 * 16), qop[d16], s);
        } else {
          const T* krow = &lds_k[buf][(sb * 32 + l32) * C::KP + hf * (D / 2)];
#pragma unroll
          for (int c4 = 0; c4 < D / 8; ++c4) {
            const float4 a = *reinterpret_cast<const float4*>(krow + c4 * 4);
            const float4 b = __builtin_bit_cast(float4, qop[c4]);
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, s, 0, 0, 0);
          }
        }
        if (cls == kMask) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int64_t key = kb + 8 * i + 4 * hf + j;
              const bool vis = core ? (key < cl_lane) : (key >= rl_lane && key <= q_lane);
              if (!vis) s[4 * i + j] = -INFINITY;
            }
        }

        // ---- online softmax with a lazily moved reference point
        float bmax = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) bmax = fmaxf(fmaxf(bmax, s[r]), s[r + 1]);
        bmax = fmaxf(bmax, s[15]);
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, kWave)) * sc;
        if (__any(bmax > m_run + kRescaleThreshold)) {
          const float m_new = fmaxf(m_run, bmax);
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
        }
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(s[r], sc, -m_run));

        if constexpr (C::EB == 2) {
          // P^T as B operand: keys 16u + {4hf..4hf+3, 8+4hf..8+4hf+3} = S registers 8u..8u+7.
          // The row sum takes the weights rounded to T, the values the MFMA multiplies
          // (weights stay <= 2^8 by the rescale threshold, within binary16's range too).
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            uint4 pb;
            uint32_t* pw = reinterpret_cast<uint32_t*>(&pb);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pw[e] = Elem<T>::pack2(p[8 * u + 2 * e], p[8 * u + 2 * e + 1]);
              float f[2];
              Elem<T>::pair_to_f32(pw[e], f);
              l_run += f[0];
              l_run += f[1];
            }
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) {
              const uint4 w = *reinterpret_cast<const uint4*>(
                  &lds_v[buf][(dt * 32 + l32) * C::VP + sb * 32 + 16 * u + 8 * hf]);
              acc[dt] = mfma_32x32x16<T>(w, pb, acc[dt]);
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) l_run += p[r];
          // one single-K MFMA per S register 4i+j (key 8i+4hf+j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) {
              const float4 a = *reinterpret_cast<const float4*>(
                  &lds_v[buf][(dt * 32 + l32) * C::VP + sb * 32 + 8 * i + 4 * hf]);
              acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, p[4 * i + 0], acc[dt], 0, 0, 0);
              acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, p[4 * i + 1], acc[dt], 0, 0, 0);
              acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, p[4 * i + 2], acc[dt], 0, 0, 0);
              acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, p[4 * i + 3], acc[dt], 0, 0, 0);
            }
        }
      }
    }
    if (it + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  // ---- normalise and store: lane (query l32, half hf) holds O[q][dt*32 + 8i + 4hf + j]
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = 1.0f / l_tot;
  const int64_t q_row = qa + l32 - pos0;                 // row within the slice
  if (q_row >= nQ) return;
  if (lse != nullptr && hf == 0) {
    // natural-log log-sum-exp of the scaled scores: (m_run + log2 l) * ln 2
    lse[(size_t)bh * nQ + q_row] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
  if (out_f32) {
    float* o = reinterpret_cast<float*>(Out) + ((size_t)bh * nQ + q_row) * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 v = make_float4(acc[dt][4 * i] * inv, acc[dt][4 * i + 1] * inv, acc[dt][4 * i + 2] * inv,
                               acc[dt][4 * i + 3] * inv);
        *reinterpret_cast<float4*>(o + dt * 32 + 8 * i + 4 * hf) = v;
      }
  } else if constexpr (C::EB == 2) {
    T* o = reinterpret_cast<T*>(Out) + ((size_t)bh * nQ + q_row) * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 w;
        w.x = Elem<T>::pack2(acc[dt][4 * i] * inv, acc[dt][4 * i + 1] * inv);
        w.y = Elem<T>::pack2(acc[dt][4 * i + 2] * inv, acc[dt][4 * i + 3] * inv);
        *reinterpret_cast<uint2*>(o + dt * 32 + 8 * i + 4 * hf) = w;
      }
  }
}

}  // namespace
}  // namespace cca

namespace cca {
namespace {

template <typename T, int D>
hipError_t launch_prefill_t(const void* q, const void* k, const void* v, const void* kc, const void* vc,
                            void* out, int out_f32, int BH, int nq, int64_t L, int g, int k_local, float scale,
                            hipStream_t stream, float* lse = nullptr) {
  using C = PrefillCfg<T, D>;
  const int ntiles = (int)((L + C::BM - 1) / C::BM);
  const int64_t nblocks = (int64_t)BH * ntiles;
  if (nblocks == 0) return hipSuccess;
  const ExtendArgs none{nullptr, 1, 0, 0, 0, nullptr};
  hipLaunchKernelGGL((cca_prefill_kernel<T, D, false>), dim3((unsigned)nblocks), dim3(C::NT), 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)kc, (const T*)vc, out, out_f32, BH, nq, L, g,
                     k_local, scale, ntiles, none, lse);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_extend_t(const void* q, const void* k, const void* v, const void* kc, const void* vc, void* out,
                           int out_f32, int BH, int nq, int g, int k_local, float scale, const ExtendArgs& ext,
                           hipStream_t stream) {
  using C = PrefillCfg<T, D>;
  const int ntiles = (ext.n + C::BM - 1) / C::BM;
  const int64_t nblocks = (int64_t)BH * ntiles;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL((cca_prefill_kernel<T, D, true>), dim3((unsigned)nblocks), dim3(C::NT), 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)kc, (const T*)vc, out, out_f32, BH, nq,
                     (int64_t)0, g, k_local, scale, ntiles, ext, (float*)nullptr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_attention(int dt, int d, const void* q, const void* k, const void* v, const void* kc,
                                    const void* vc, void* out, int out_f32, int BH, int nq, int64_t L, int g,
                                    int k_local, float scale, hipStream_t stream, float* lse) {
  if (dt != CCA_F32 && d == 128)
    return launch_prefill_d128(dt, q, k, v, kc, vc, out, out_f32, BH, nq, L, g, k_local, scale, stream, lse);
  return dispatch_td(dt, d, [&](auto t, auto dd) {
    using T = decltype(t);
    return launch_prefill_t<T, decltype(dd)::value>(q, k, v, kc, vc, out, sizeof(T) == 4 ? 1 : out_f32, BH, nq, L, g,
                                                    k_local, scale, stream, lse);
  });
}

hipError_t launch_extend_attention(int dt, int d, const void* q, const void* k, const void* v, const void* kc,
                                   const void* vc, void* out, int out_f32, int BH, int nq, int g, int k_local,
                                   float scale, const ExtendArgs& ext, hipStream_t stream) {
  if (dt != CCA_F32 && d == 128)
    return launch_extend_attention_d128(dt, q, k, v, kc, vc, out, out_f32, BH, nq, g, k_local, scale, ext, stream);
  return dispatch_td(dt, d, [&](auto t, auto dd) {
    using T = decltype(t);
    return launch_extend_t<T, decltype(dd)::value>(q, k, v, kc, vc, out, sizeof(T) == 4 ? 1 : out_f32, BH, nq, g,
                                                   k_local, scale, ext, stream);
  });
}

}  // namespace cca
