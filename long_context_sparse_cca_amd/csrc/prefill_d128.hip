// Fused CCA prefill attention, 16-bit inputs (bf16 or IEEE binary16), head dim 128: the
// gfx950 fast path.
//
// Same computation as the generic kernel in prefill.hip (the CCA write-up,
// "ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展": query t of
// group beta = t/g attends, in one softmax, to the core tokens Kc[0 : beta-k) and
// the raw keys K[(beta-k)*g .. t]; locality-preserving module and global-local
// fusion sections), restructured around three CDNA4 features:
//   * K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4): no
//     staging registers and no VALU work to fill the tiles;
//   * tiles stay row-major in LDS with a 16-byte XOR swizzle of the chunk index
//     (chunk c of row r sits at c ^ swz(r)), which keeps both operand reads
//     below free of bank conflicts without padding;
//   * the V^T operand of the PV product is read with ds_read_b64_tr_b16, the
//     LDS transpose read: in each 16-lane group, lane j receives element j%4 of
//     the 8-byte pieces read by lanes 4e + j/4 (e = 0..3).  With lane s reading
//     key row kbase + s/4, dims d0 + 4(s%4) .. +3, lane j ends up holding the
//     four keys kbase..kbase+3 at dim d0 + j, i.e. one quarter of an MFMA A operand.
// Softmax bookkeeping uses v_permlane32_swap for the cross-half row max / sum and
// v_dot2_f32_bf16 (v_dot2_f32_f16) against (1, 1) for the row sum of the weights as
// rounded to the input type.
// A workgroup is 8 waves (256 queries, 2 waves per SIMD) sharing each K/V tile;
// each wave raises its priority while it issues its MFMA burst so that the two
// waves of a SIMD tend to alternate between matrix and vector work.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int kBM = 256;                 // queries per workgroup (8 waves x 32)
constexpr int kBN = 64;                  // keys per tile
constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;        // 256
constexpr int kTileBytes = kBN * kRowBytes;  // 16 KB
constexpr int kBufBytes = 2 * kTileBytes;    // K tile + V tile
// Lazy rescaling: the reference point of the exponentials moves only when a row's
// weights in a sub-block sum above kSumLimit (then to the row's running max).  The
// weights thus stay <= 2^16, so the fp32 row sums and accumulators cannot overflow
// unless the sum of |V| over a row exceeds ~2^112; the final division by the row sum
// makes the result independent of the reference point up to rounding.  In binary16 a
// weight above 65519 rounds to infinity; the row sum then exceeds the limit too, so the
// wave rescales and recomputes the weights in that case as well.
constexpr float kSumLimit = 65536.0f;

typedef short v4s_t __attribute__((ext_vector_type(4)));

// 16-byte chunk swizzle of a tile row (16 chunks per 256-byte row).  It is a
// bijection on any 16 consecutive rows (the K operand read: 16 lanes, 16 rows, one
// logical chunk), and the 4 rows of one transpose read (4-aligned, 4 logical chunks
// per row across a 32-lane pass) land in 4 distinct 64-byte bank groups.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// EXT: attention of new tokens over a cached prefix (ExtendArgs): positions are absolute,
// query i of the slice is at ext.pos[b] + i, raw key u is row u - raw0 of the raw slice.
// Without EXT the slice is a whole sequence: pos0 = raw0 = 0, L queries, L raw rows.
template <typename T, bool EXT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void cca_prefill_d128_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ Kc, const T* __restrict__ Vc, void* __restrict__ Out, int out_f32, int BH,
    int nq, int L, int g, int k_local, float scale, int ntiles, ExtendArgs ext, float* __restrict__ lse) {
  // one array per buffer: the LDS-DMA fill of one buffer then provably does not
  // alias the operand reads of the other, so no wait is forced between them
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kBufBytes];

  int bh, qtile;
  map_block(BH * ntiles, ntiles, bh, qtile);
  if constexpr (EXT) bh = kv_major_slice(bh, BH, ext.Hq, nq, ext.order);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // absolute position of query 0, first raw position of the raw slice, queries per slice
  int pos0 = 0, raw0 = 0, nQ = L;
  int64_t raw_rows = L, core_rows = L / g;
  if constexpr (EXT) {
    pos0 = ext.pos[bh / ext.Hq];
    nQ = ext.n;
    raw_rows = ext.raw_rows;
    core_rows = ext.core_rows;
    if (pos0 < 0) {
      // invalid sequence: NaN outputs, nothing read
      const int i = qtile * kBM + wave * 32 + l32;
      if (i < nQ) {
        const size_t o = ((size_t)bh * nQ + i) * kD;
        for (int c = hf; c < kD; c += 2) {
          if (out_f32) reinterpret_cast<float*>(Out)[o + c] = __builtin_nanf("");
          else reinterpret_cast<uint16_t*>(Out)[o + c] = Elem<T>::kNaNBits;
        }
      }
      return;
    }
    raw0 = max(0, pos0 / g - k_local) * g;
  }
  const int Lend = pos0 + nQ;                             // one past the last query position
  const int m = (int)core_rows;

  const int q0 = pos0 + qtile * kBM;
  const int q_last = min(q0 + kBM - 1, Lend - 1);
  const int nc_wg = max(0, q_last / g - k_local);        // core tokens any row sees
  const int rl_wg = max(0, q0 / g - k_local) * g;        // first raw key any row sees
  const int n_core_tiles = (nc_wg + kBN - 1) / kBN;
  const int n_raw_tiles = (q_last - rl_wg + kBN) / kBN;
  const int n_tiles = n_core_tiles + n_raw_tiles;

  // ---- this wave's 32 queries (wave-uniform bounds in scalar registers)
  const int qa = q0 + wave * 32;
  const bool wave_live = qa < Lend;
  const int qb = min(qa + 31, Lend - 1);
  const int cl_min = qa / g - k_local, cl_max = qb / g - k_local;
  const int rl_min = max(0, cl_min) * g, rl_max = max(0, cl_max) * g;
  const int q_lane = min(qa + l32, Lend - 1);
  const int cl_lane = q_lane / g - k_local;              // core j visible iff j < cl_lane
  const int rl_lane = max(0, cl_lane) * g;               // raw u visible iff rl_lane <= u <= q_lane

  const size_t slice = (size_t)bh * nQ * kD;             // query / output slice
  const int bkv = bh / nq;  // key/value slice read by query slice bh (grouped-query attention)
  const T* Ks = K + (size_t)bkv * raw_rows * kD;
  const T* Vs = V + (size_t)bkv * raw_rows * kD;
  const T* Kcs = Kc + (size_t)bkv * core_rows * kD;
  const T* Vcs = Vc + (size_t)bkv * core_rows * kD;

  // ---- Q operand (B of S^T = K Q^T): slice d16 holds dims 16*d16 + 8*hf .. +8
  uint4 qop[kD / 16];
  {
    const T* qrow = Q + slice + (size_t)(q_lane - pos0) * kD;
#pragma unroll
    for (int s = 0; s < kD / 16; ++s) qop[s] = ld16(qrow + s * 16 + hf * 8);
  }

  // ---- tile fill: wave w, instruction i writes rows 8w + 4i .. +3 (1 KB of LDS);
  // lane l lands in physical chunk l%16 of row 8w + 4i + l/16 and so fetches the
  // logical chunk (l%16) ^ swz(row).
  int fill_row[2], fill_off[2], fill_lin[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wave * 8 + i * 4 + (lane >> 4);
    fill_row[i] = r;
    fill_off[i] = ((lane & 15) ^ swz(r)) * 16;
    fill_lin[i] = r * kRowBytes + fill_off[i];
  }
  auto issue_tile = [&](int it, int buf) {
    const T *ks, *vs;
    int base, lim, off0;   // tile's first key, last valid key, key of row 0 of the slice
    if (it < n_core_tiles) {
      ks = Kcs; vs = Vcs; base = it * kBN; lim = m - 1; off0 = 0;
    } else {
      ks = Ks; vs = Vs; base = rl_wg + (it - n_core_tiles) * kBN; lim = Lend - 1; off0 = raw0;
    }
    uint8_t* dst0 = (buf ? lds1 : lds0) + wave * 8 * kRowBytes;
    if (base + kBN - 1 <= lim) {
      // whole tile in range: uniform tile base + per-lane 32-bit offset
      const uint8_t* kt = (const uint8_t*)ks + (size_t)(base - off0) * kRowBytes;
      const uint8_t* vt = (const uint8_t*)vs + (size_t)(base - off0) * kRowBytes;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint8_t* dst = dst0 + i * 4 * kRowBytes;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kt + fill_lin[i]),
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vt + fill_lin[i]),
                                         (__attribute__((address_space(3))) void*)(dst + kTileBytes), 16, 0, 0);
      }
    } else {
      // last tile of a range: rows past the end repeat the last valid row
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const size_t goff = (size_t)(min(base + fill_row[i], lim) - off0) * kRowBytes + fill_off[i];
        uint8_t* dst = dst0 + i * 4 * kRowBytes;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)((const uint8_t*)ks + goff),
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)((const uint8_t*)vs + goff),
                                         (__attribute__((address_space(3))) void*)(dst + kTileBytes), 16, 0, 0);
      }
    }
  };

  // ---- operand read offsets inside a tile (bytes)
  // K (A of QK^T): row l32 of the sub-block, logical chunk 2*d16 + hf.
  int koff[kD / 16];
#pragma unroll
  for (int d16 = 0; d16 < kD / 16; ++d16) koff[d16] = l32 * kRowBytes + (((2 * d16 + hf) ^ swz(l32)) * 16);
  // V (A of V^T P^T via transpose reads): 16-lane group G = lane/16 covers dims
  // dt*32 + 16*(G&1) .. +15 for the four keys 16u + 4*(G>>1) + 8*r .. +3.
  int voff[2][kD / 32];
  {
    const int s = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 4 * (grp >> 1) + 8 * r + (s >> 2);
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) {
        const int chunk = dt * 4 + 2 * (grp & 1) + ((s & 3) >> 1);
        voff[r][dt] = row * kRowBytes + ((chunk ^ swz(row)) * 16) + (s & 1) * 8;
      }
    }
  }

  f32x16_t acc[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = kNegBig, l_run = 0.f;
  const float sc = scale * kLog2e;
  using Ops = Mma16<T>;
  const typename Ops::x2 ones = Ops::round2(1.0f, 1.0f);

  // Visible window [lo, lo + span] of each lane in the key index space of a tile kind:
  // core key j visible iff 0 <= j <= cl_lane - 1 (empty when cl_lane <= 0, encoded
  // with a base below every key index); raw key u iff rl_lane <= u <= q_lane.
  const int core_lo = (cl_lane > 0) ? 0 : -0x40000000;
  const unsigned core_span = (unsigned)max(cl_lane - 1, 0);
  const unsigned raw_span = (unsigned)(q_lane - rl_lane);

  auto compute_tile = [&](const uint8_t* kt, const uint8_t* vt, int it) {
    const bool core = it < n_core_tiles;
    const int tbase = core ? it * kBN : rl_wg + (it - n_core_tiles) * kBN;
    const int lo = core ? core_lo : rl_lane;
    const unsigned span = core ? core_span : raw_span;
#pragma unroll
    for (int sb = 0; sb < kBN / 32; ++sb) {
      const int kb = tbase + sb * 32;
      int cls;
      if (core) {
        cls = (kb >= cl_max) ? 0 : ((kb + 32 <= cl_min) ? 1 : 2);
      } else {
        if (kb + 31 < rl_min || kb > qb) cls = 0;
        else if (kb >= rl_max && kb + 31 <= qa) cls = 1;
        else cls = 2;
      }
      if (cls == 0) continue;

      // all K operand reads in flight at once, then the MFMA chain consumes them in order
      uint4 ka[kD / 16];
#pragma unroll
      for (int d16 = 0; d16 < kD / 16; ++d16)
        ka[d16] = *reinterpret_cast<const uint4*>(kt + sb * 32 * kRowBytes + koff[d16]);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      f32x16_t s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int d16 = 0; d16 < kD / 16; ++d16)
        s = Ops::mfma32(ka[d16], qop[d16], s);
      // V operand transpose reads for this sub-block, issued behind the QK MFMAs so
      // their latency hides under the softmax arithmetic
      v4s_t vop[2][2][kD / 32];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int dt = 0; dt < kD / 32; ++dt)
            vop[u][r][dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(
                vt + (sb * 32 + 16 * u) * kRowBytes + voff[r][dt]));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      if (cls == 2) {
        // key = kb + 8i + 4hf + j; visible iff (unsigned)(key - lo) <= span
        const int k0 = kb + 4 * hf - lo;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool vis = (unsigned)(k0 + 8 * i + j) <= span;
            s[4 * i + j] = vis ? s[4 * i + j] : -INFINITY;
          }
      }

      // Weights P^T (B operand) against the current reference point m_run.  The maximum of
      // the sub-block is not computed up front: a lane whose 16 weights sum above 2^16 (some
      // weight may exceed it, or the reference is still unset) makes the wave move the
      // reference to the running maximum and recompute the weights (rare after the first
      // sub-blocks).  Weights therefore stay <= 2^16, as with an explicit threshold check.
      typename Ops::x2 pp[2][4];
      float bsum;
      auto weights = [&]() {
        // two partial row sums (one per 16-key half) halve the dependent dot2 chain
        float h0 = 0.f, h1 = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(fmaf(s[8 * u + 2 * e], sc, -m_run));
            const float p1 = fast_exp2(fmaf(s[8 * u + 2 * e + 1], sc, -m_run));
            pp[u][e] = Ops::round2(p0, p1);
            if (u == 0) h0 = Ops::dot2(pp[u][e], ones, h0);
            else h1 = Ops::dot2(pp[u][e], ones, h1);
          }
        bsum = h0 + h1;
      };
      weights();
      if (__builtin_amdgcn_ballot_w64(bsum > kSumLimit) != 0) {
        // an empty asm with a memory clobber keeps the compiler from hoisting the maximum's
        // arithmetic above the (rarely taken) branch
        asm volatile("" ::: "memory");
        float bmax = max3f(s[0], s[1], s[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) bmax = max3f(bmax, s[r], s[r + 1]);
        bmax = fmaxf(bmax, s[15]);
        bmax = xhalf_max(bmax) * sc;
        const float m_new = fmaxf(m_run, bmax);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
        weights();
      }
      l_run += bsum;

#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // P^T: keys 16u + {4hf..4hf+3, 8+4hf..8+4hf+3} = S registers 8u .. 8u+7
        const uint4 pb = __builtin_bit_cast(uint4, pp[u]);
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) {
          const v4s_t both[2] = {vop[u][0][dt], vop[u][1][dt]};
          acc[dt] = Ops::mfma32(__builtin_bit_cast(uint4, both), pb, acc[dt]);
        }
      }
    }
  };

  if (n_tiles > 0) issue_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tile has landed in LDS
  __syncthreads();
  // two tiles per trip, buffer 0 then buffer 1, so the accumulators flow straight through
  for (int it = 0; it < n_tiles; it += 2) {
    if (it + 1 < n_tiles) issue_tile(it + 1, 1);  // lands while tile `it` is being used
    if (wave_live) compute_tile(lds0, lds0 + kTileBytes, it);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (it + 1 >= n_tiles) break;
    if (it + 2 < n_tiles) issue_tile(it + 2, 0);
    if (wave_live) compute_tile(lds1, lds1 + kTileBytes, it + 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }

  if (!wave_live) return;
  // ---- normalise and store: lane (query l32, half hf) holds O[q][dt*32 + 8i + 4hf + j]
  const float l_tot = xhalf_sum(l_run);
  const float inv = 1.0f / l_tot;
  const int q_row = qa + l32 - pos0;                     // row within the slice
  if (q_row >= nQ) return;
  if (lse != nullptr && hf == 0) {
    // natural-log log-sum-exp of the scaled scores: (m_run + log2 l) * ln 2
    lse[(size_t)bh * nQ + q_row] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
  if (out_f32) {
    float* o = reinterpret_cast<float*>(Out) + slice + (size_t)q_row * kD;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = make_float4(acc[dt][4 * i] * inv, acc[dt][4 * i + 1] * inv, acc[dt][4 * i + 2] * inv,
                                     acc[dt][4 * i + 3] * inv);
        *reinterpret_cast<float4*>(o + dt * 32 + 8 * i + 4 * hf) = v;
      }
  } else {
    T* o = reinterpret_cast<T*>(Out) + slice + (size_t)q_row * kD;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 w;
        w.x = Elem<T>::pack2(acc[dt][4 * i] * inv, acc[dt][4 * i + 1] * inv);
        w.y = Elem<T>::pack2(acc[dt][4 * i + 2] * inv, acc[dt][4 * i + 3] * inv);
        *reinterpret_cast<uint2*>(o + dt * 32 + 8 * i + 4 * hf) = w;
      }
  }
}

template <typename T>
void launch_prefill_t(const void* q, const void* k, const void* v, const void* kc, const void* vc, void* out,
                      int out_f32, int BH, int nq, int64_t L, int g, int k_local, float scale, int ntiles,
                      const ExtendArgs& ext, bool extend, float* lse, hipStream_t stream) {
  const int64_t nblocks = (int64_t)BH * ntiles;
  if (extend)
    hipLaunchKernelGGL((cca_prefill_d128_kernel<T, true>), dim3((unsigned)nblocks), dim3(512), 0, stream, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)kc, (const T*)vc, out, out_f32, BH, nq, 0, g, k_local,
                       scale, ntiles, ext, (float*)nullptr);
  else
    hipLaunchKernelGGL((cca_prefill_d128_kernel<T, false>), dim3((unsigned)nblocks), dim3(512), 0, stream,
                       (const T*)q, (const T*)k, (const T*)v, (const T*)kc, (const T*)vc, out, out_f32, BH, nq,
                       (int)L, g, k_local, scale, ntiles, ext, lse);
}

}  // namespace

hipError_t launch_prefill_d128(int dt, const void* q, const void* k, const void* v, const void* kc, const void* vc,
                               void* out, int out_f32, int BH, int nq, int64_t L, int g, int k_local, float scale,
                               hipStream_t stream, float* lse) {
  const int ntiles = (int)((L + kBM - 1) / kBM);
  if ((int64_t)BH * ntiles == 0) return hipSuccess;
  const ExtendArgs none{nullptr, 1, 0, 0, 0, nullptr};
  if (dt == CCA_F16)
    launch_prefill_t<f16_t>(q, k, v, kc, vc, out, out_f32, BH, nq, L, g, k_local, scale, ntiles, none, false, lse,
                            stream);
  else
    launch_prefill_t<bf16_t>(q, k, v, kc, vc, out, out_f32, BH, nq, L, g, k_local, scale, ntiles, none, false, lse,
                             stream);
  return hipGetLastError();
}

hipError_t launch_extend_attention_d128(int dt, const void* q, const void* k, const void* v, const void* kc,
                                        const void* vc, void* out, int out_f32, int BH, int nq, int g, int k_local,
                                        float scale, const ExtendArgs& ext, hipStream_t stream) {
  const int ntiles = (ext.n + kBM - 1) / kBM;
  if ((int64_t)BH * ntiles == 0) return hipSuccess;
  if (dt == CCA_F16)
    launch_prefill_t<f16_t>(q, k, v, kc, vc, out, out_f32, BH, nq, 0, g, k_local, scale, ntiles, ext, true, nullptr,
                            stream);
  else
    launch_prefill_t<bf16_t>(q, k, v, kc, vc, out, out_f32, BH, nq, 0, g, k_local, scale, ntiles, ext, true, nullptr,
                             stream);
  return hipGetLastError();
}

}  // namespace cca
