// Backward pass of CCA prefill attention (16-bit inputs: bf16 or IEEE binary16; head dim
// 128; float32 gradients).
//
// Method: the CCA write-up ("ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"):
// the fused operator serves training (Triton section); the forward pools each
// group with its last query (global-aware pooling, core-token and core K/V
// equations) and attends, in one softmax, to the core tokens before the raw
// window and the raw keys of the window (locality-preserving module, global-local
// fusion).  The gradients follow the chain rule through both softmaxes:
//
//   attention  p = softmax(scale k.q) over the visible keys, ds = p (dp - D),
//              dp = dO.v, D = dO.O (= sum_i p_i dp_i);
//              dQ += scale sum ds k;  dkey += scale ds q;  dval += p dO
//   pooling    (core keys/values of group j: Kc = a.K_group, Vc = a.V_group,
//              a = softmax(scale q_hat.K_group))
//              dV_group += a dVc;  da = dKc.K + dVc.V;  dz = a (da - a.da);
//              dK_group += a dKc + scale dz q_hat;  dQ[last row] += scale dz.K_group
//
// Launches:
//   1. cca_bwd_prep_kernel     D[t] = dO[t].O[t]; the log-sum-exp in log2 units
//   2. cca_bwd_dq_kernel       per 256-query tile: recompute scores and p from the
//                              forward's log-sum-exp, dQ = scale (P o (dP - D)) K
//   3. cca_bwd_dkdv16_kernel   per 192-key tile (core tokens or raw keys): loop over
//                              the query tiles that see it; dV and dK of raw keys go
//                              to dv, dk, those of core tokens to dVc, dKc (workspace)
//   4. cca_bwd_pool_kernel     per group: dKc, dVc through the pooling into dk, dv,
//                              and into dq at the group's last row
// The score and gradient products run on MFMA of the input type (32x32x16 for dQ,
// 16x16x32 for dK and dV) with float32 accumulation; P and dS are rounded to that type as
// MFMA operands, as P is in the forward.  Tiles are staged HBM -> LDS with global_load_lds and read with the
// same 16-byte XOR swizzle and transpose reads as the forward kernel.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;
constexpr int kTileRows = 64;                       // rows per staged tile
constexpr int kTileBytes = kTileRows * kRowBytes;   // 16 KB
constexpr float kLn2 = 0.69314718055994531f;

typedef short v4s_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// Swizzle of the dK/dV kernel's query-side tiles (Q, dO).  Measured on this part (per-dispatch
// LDS bank-conflict counts of a one-wave probe): a 16-byte-per-lane LDS read serves each
// 32-lane half in two passes of 16 lanes, split by the parity of lane bits 2-4, over 64
// four-byte banks.  The dK/dV row-operand read (lane l: row l%16, chunk 4kk + l/16) then puts
// rows {0-3, 12-15} of one chunk and rows {4-11} of the next in the same pass, which any
// swizzle of the row alone maps onto repeated banks; this one (r, with bits 2 and 3 flipped
// on odd rows) keeps both passes on 16 distinct chunks, keeps the transpose reads (8 rows x
// 2 chunks per half-wave) on 16 distinct chunks, and is a bijection on 16 rows.
__device__ __forceinline__ int swz_t(int r) { return (r & 15) ^ ((r & 1) * 12); }

// Operand read offsets inside a row-major swizzled tile (bytes, relative to the
// first row of a 32-row sub-block).
//   rows operand (A of X.Y^T with X rows from LDS): row l32, logical chunk 2*d16 + hf;
//   transpose operand (A of X^T.P with X rows from LDS): the four 8-byte pieces
//   that ds_read_b64_tr_b16 turns into rows 16u + 4*(G>>1) + 8r .. +3 at dims
//   dt*32 + 16*(G&1) + lane%16, matching the register order of a 32x32 MFMA
//   output used as the B operand.
struct TileOffsets {
  int rows[kD / 16];
  int tr[2][kD / 32];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int d16 = 0; d16 < kD / 16; ++d16) rows[d16] = l32 * kRowBytes + (((2 * d16 + hf) ^ swz(l32)) * 16);
    const int s = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 4 * (grp >> 1) + 8 * r + (s >> 2);
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) {
        const int chunk = dt * 4 + 2 * (grp & 1) + ((s & 3) >> 1);
        tr[r][dt] = row * kRowBytes + ((chunk ^ swz(row)) * 16) + (s & 1) * 8;
      }
    }
  }
};


// Transpose-operand accumulation acc[dt] += X_subblock^T (d x 32 rows from LDS) . W,
// W [32 rows x 32 cols] the fp32 32x32 MFMA output `w` rounded to T, in two halves:
// the transpose reads of half u (rows 16u .. 16u+15) are issued early (tr_read), the
// MFMAs later (tr_mfma).
struct TrHalf {
  v4s_t r[2][kD / 32];
};
__device__ __forceinline__ void tr_read(const uint8_t* tile_sb, const TileOffsets& o, int u, TrHalf& t) {
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) {
    t.r[0][dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s_t*)(tile_sb + 16 * u * kRowBytes + o.tr[0][dt]));
    t.r[1][dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s_t*)(tile_sb + 16 * u * kRowBytes + o.tr[1][dt]));
  }
}
template <typename T>
__device__ __forceinline__ void tr_mfma(const TrHalf& t, const f32x16_t& w, int u, f32x16_t* acc) {
  typename Mma16<T>::x2 pp[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) pp[e] = Mma16<T>::round2(w[8 * u + 2 * e], w[8 * u + 2 * e + 1]);
  const uint4 pb = __builtin_bit_cast(uint4, pp);
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) {
    const v4s_t both[2] = {t.r[0][dt], t.r[1][dt]};
    acc[dt] = Mma16<T>::mfma32(__builtin_bit_cast(uint4, both), pb, acc[dt]);
  }
}

// Rows-operand chain out = X_subblock (32 rows from LDS) . Y^T, Y's 32 rows in registers
// as B operands yop[d16]: the reads (rows_read) are issued before the MFMAs (rows_mfma).
__device__ __forceinline__ void rows_read(const uint8_t* tile_sb, const TileOffsets& o, uint4* xa) {
#pragma unroll
  for (int d16 = 0; d16 < kD / 16; ++d16) xa[d16] = *reinterpret_cast<const uint4*>(tile_sb + o.rows[d16]);
}
template <typename T>
__device__ __forceinline__ f32x16_t rows_mfma(const uint4* xa, const uint4* yop) {
  f32x16_t s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int d16 = 0; d16 < kD / 16; ++d16) s = Mma16<T>::mfma32(xa[d16], yop[d16], s);
  return s;
}

// Fill a 64-row tile (rows base .. base+63 of a row-major [*, 128] 16-bit array,
// rows past `lim` repeat row `lim`) into LDS with the chunk swizzle (swz, or swz_t with
// TSWZ).  nw waves share the fill: wave w writes rows w*64/nw .. in groups of 4 rows per
// instruction.
template <int NW, bool TSWZ = false>
__device__ __forceinline__ void fill_tile(const void* src, int64_t base, int64_t lim, uint8_t* dst, int wave,
                                          int lane) {
  constexpr int ITERS = kTileRows / (4 * NW);
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int r = wave * (4 * ITERS) + i * 4 + (lane >> 4);
    const int off = ((lane & 15) ^ (TSWZ ? swz_t(r) : swz(r))) * 16;
    const int64_t gr = min(base + r, lim);
    uint8_t* d = dst + (wave * (4 * ITERS) + i * 4) * kRowBytes;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)((const uint8_t*)src +
                                                                                      (size_t)gr * kRowBytes + off),
                                     (__attribute__((address_space(3))) void*)d, 16, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// 1. D[t] = dO[t] . O[t]  (16 lanes per row)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void cca_bwd_prep_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                           const float* __restrict__ lse, float* __restrict__ Dv,
                                                           float* __restrict__ lse2, int64_t rows) {
  const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 16;
  const int c = threadIdx.x & 15;
  float s = 0.f;
  if (row < rows) {
    float a[8], b[8];
    Elem<T>::chunk_to_f32(ld16(O + (size_t)row * kD + 8 * c), a);
    Elem<T>::chunk_to_f32(ld16(dO + (size_t)row * kD + 8 * c), b);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(a[e], b[e], s);
  }
  s = lane_group_sum<16>(s);
  if (row < rows && c == 0) {
    Dv[row] = s;
    lse2[row] = lse[row] * kLog2e;   // log-sum-exp in log2 units, as the kernels use it
  }
}

// ---------------------------------------------------------------------------
// 2. dQ: 256 queries per workgroup (8 waves x 32), loop over the visible key tiles
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void cca_bwd_dq_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ Kc, const T* __restrict__ Vc, const T* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ Dv, float* __restrict__ dQ, int BH, int nq, int L,
    int g, int k_local, float scale, int ntiles) {
  constexpr int kBM = 256, kBN = 64;
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[2 * kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[2 * kTileBytes];
  int bh, qtile;
  map_block(BH * ntiles, ntiles, bh, qtile);
  const int m = L / g;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int l32 = lane & 31, hf = lane >> 5;

  const int q0 = qtile * kBM;
  const int q_last = min(q0 + kBM - 1, L - 1);
  const int nc_wg = max(0, q_last / g - k_local);
  const int rl_wg = max(0, q0 / g - k_local) * g;
  const int n_core_tiles = (nc_wg + kBN - 1) / kBN;
  const int n_tiles = n_core_tiles + (q_last - rl_wg + kBN) / kBN;

  const int qa = q0 + wave * 32;
  const bool wave_live = qa < L;
  const int qb = min(qa + 31, L - 1);
  const int cl_min = qa / g - k_local, cl_max = qb / g - k_local;
  const int rl_min = max(0, cl_min) * g, rl_max = max(0, cl_max) * g;
  const int q_lane = min(qa + l32, L - 1);
  const int cl_lane = q_lane / g - k_local;
  const int rl_lane = max(0, cl_lane) * g;
  const int core_lo = (cl_lane > 0) ? 0 : -0x40000000;
  const unsigned core_span = (unsigned)max(cl_lane - 1, 0);
  const unsigned raw_span = (unsigned)(q_lane - rl_lane);

  const size_t slice = (size_t)bh * L * kD;              // query / dQ slice
  const int bkv = bh / nq;  // key/value slice read by query slice bh (grouped-query attention)
  const T* Ks = K + (size_t)bkv * L * kD;
  const T* Vs = V + (size_t)bkv * L * kD;
  const T* Kcs = Kc + (size_t)bkv * m * kD;
  const T* Vcs = Vc + (size_t)bkv * m * kD;

  // B operands of the score and dP chains: this lane's query / upstream-gradient row
  uint4 qop[kD / 16], dop[kD / 16];
#pragma unroll
  for (int s = 0; s < kD / 16; ++s) {
    qop[s] = ld16(Q + slice + (size_t)q_lane * kD + s * 16 + hf * 8);
    dop[s] = ld16(dO + slice + (size_t)q_lane * kD + s * 16 + hf * 8);
  }
  const float sc = scale * kLog2e;
  const float lse2 = lse[(size_t)bh * L + q_lane];   // log2 units
  const float Dq = Dv[(size_t)bh * L + q_lane];

  TileOffsets off;
  off.init(lane);
  f32x16_t acc[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

  auto issue = [&](int it, uint8_t* buf) {
    const T *ks, *vs;
    int base, lim;
    if (it < n_core_tiles) {
      ks = Kcs; vs = Vcs; base = it * kBN; lim = m - 1;
    } else {
      ks = Ks; vs = Vs; base = rl_wg + (it - n_core_tiles) * kBN; lim = L - 1;
    }
    fill_tile<8>(ks, base, lim, buf, wave, lane);
    fill_tile<8>(vs, base, lim, buf + kTileBytes, wave, lane);
  };

  auto compute = [&](const uint8_t* kt, const uint8_t* vt, int it) {
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
      const uint8_t* ksb = kt + sb * 32 * kRowBytes;
      const uint8_t* vsb = vt + sb * 32 * kRowBytes;
      // operand reads up front; score and dP chains at raised priority, the first half of the
      // K^T transpose reads issued behind them so that their latency hides under dS
      uint4 xa[kD / 16], ya[kD / 16];
      rows_read(ksb, off, xa);
      rows_read(vsb, off, ya);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      f32x16_t s = rows_mfma<T>(xa, qop);           // S^T: keys x queries
      f32x16_t dp = rows_mfma<T>(ya, dop);          // dP^T
      TrHalf th;
      tr_read(ksb, off, 0, th);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      if (cls == 2) {
        const int k0 = kb + 4 * hf - lo;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool vis = (unsigned)(k0 + 8 * i + j) <= span;
            s[4 * i + j] = vis ? s[4 * i + j] : -INFINITY;
          }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[r], sc, -lse2));
        dp[r] = p * (dp[r] - Dq);                 // dS^T
      }
      tr_mfma<T>(th, dp, 0, acc);                   // dQ^T += K^T dS^T
      tr_read(ksb, off, 1, th);
      tr_mfma<T>(th, dp, 1, acc);
    }
  };

  if (n_tiles > 0) issue(0, lds0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int it = 0; it < n_tiles; it += 2) {
    if (it + 1 < n_tiles) issue(it + 1, lds1);
    if (wave_live) compute(lds0, lds0 + kTileBytes, it);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (it + 1 >= n_tiles) break;
    if (it + 2 < n_tiles) issue(it + 2, lds0);
    if (wave_live) compute(lds1, lds1 + kTileBytes, it + 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  if (!wave_live) return;
  const int q_row = qa + l32;
  if (q_row >= L) return;
  float* o = dQ + slice + (size_t)q_row * kD;
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<float4*>(o + dt * 32 + 8 * i + 4 * hf) =
          make_float4(acc[dt][4 * i] * scale, acc[dt][4 * i + 1] * scale, acc[dt][4 * i + 2] * scale,
                      acc[dt][4 * i + 3] * scale);
}

// ---------------------------------------------------------------------------
// 3. dK and dV: 192 keys per workgroup (12 waves x 16 keys, three waves per SIMD) on
//    16x16x32 MFMAs, so that the scores and weights of a (query, key) pair are computed
//    once for both gradients.  A workgroup loops over the 64-query tiles that see its
//    keys (core token j: queries from (j+k+1) g; raw key u: queries u .. (u/g+k+1) g - 1),
//    with Q, dO and the tile's statistics DMA'd into LDS, two tiles in flight.
//    Lane l of a wave holds key l%16; with G = l/16, its score registers are the queries
//    16b + 4G + i (b = 0, 1, i = 0..3) of a 32-query sub-block.  Those 8 values are
//    exactly the B operand of the gradient MFMAs when their reduction index k = 8G + t
//    stands for query 4G + t (t < 4) or 16 + 4G + t - 4 (t >= 4); the A operands (dO^T,
//    Q^T) are read from the tiles in that query order with transpose reads.  At three
//    waves per SIMD (168 registers each) the LDS operand traffic of the 16-key layout
//    (64 bytes per MFMA cycle and wave) has enough waves to hide behind.
// ---------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(768) __attribute__((amdgpu_waves_per_eu(3, 3))) void cca_bwd_dkdv16_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ Kc, const T* __restrict__ Vc, const T* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ Dv, float* __restrict__ dK, float* __restrict__ dV,
    float* __restrict__ dKc, float* __restrict__ dVc, int BHkv, int nq, int L, int g, int k_local, float scale,
    int n_core_wg) {
  constexpr int kBK = 192;  // keys per workgroup
  constexpr int kBufBytes = 2 * kTileBytes + 2 * kTileRows * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[kBufBytes];
  // heaviest work first across all slices (workgroup index wi is the slow index)
  const int wi = blockIdx.x / BHkv;
  const int bkv = blockIdx.x - wi * BHkv;   // key/value slice
  const bool core = wi < n_core_wg;
  const int m = L / g;
  const int key0 = core ? wi * kBK : (wi - n_core_wg) * kBK;
  const int key_end = core ? m : L;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int n16 = lane & 15, G = lane >> 4;
  const int c0 = key0 + wave * 16;         // this wave's first key
  const int c_last = min(key0 + kBK, key_end) - 1;

  // Visibility in query positions, so that the loops need no division by g:
  //   core token j is seen by the queries t >= (j + k + 1) g,
  //   raw key u by the queries u <= t <= (u / g + k + 1) g - 1.
  auto core_first = [&](int j) { return (int)min((int64_t)L, ((int64_t)j + k_local + 1) * g); };
  auto raw_last = [&](int u) { return (int)min((int64_t)L - 1, ((int64_t)(u / g) + k_local + 1) * g - 1); };
  int t_lo, t_hi;
  if (core) {
    t_lo = core_first(key0);
    t_hi = L - 1;
  } else {
    t_lo = key0;
    t_hi = raw_last(c_last);
  }
  const int tq0 = (t_lo / kTileRows) * kTileRows;
  const int n_qt = (t_lo <= t_hi) ? (t_hi - tq0) / kTileRows + 1 : 0;
  // the nq query heads that read this key/value slice each see the same query tiles:
  // iteration it covers tile it % n_qt of head it / n_qt
  const int n_it = n_qt * nq;

  const size_t slice = (size_t)bkv * L * kD;              // key/value (and dK/dV) slice
  const T* Ks = core ? Kc + (size_t)bkv * m * kD : K + slice;
  const T* Vs = core ? Vc + (size_t)bkv * m * kD : V + slice;
  const size_t qslice0 = (size_t)bkv * nq;                // first query slice that reads it
  // B operands of the score and dP products: dims 32kk + 8G .. +7 of this lane's key
  const int key_lane = min(c0 + n16, key_end - 1);
  uint4 kop[kD / 32], vop[kD / 32];
#pragma unroll
  for (int kk = 0; kk < kD / 32; ++kk) {
    kop[kk] = ld16(Ks + (size_t)key_lane * kD + kk * 32 + G * 8);
    vop[kk] = ld16(Vs + (size_t)key_lane * kD + kk * 32 + G * 8);
  }
  const float sc = scale * kLog2e;
  // A-operand read offsets inside a sub-block (bytes): rows operand, row n16 (+16b),
  // logical chunk 4kk + G; transpose operand, rows 4G + n16/4 (+16 for the second
  // half), dims 16 blk + 4 (n16 % 4) .. +3
  int roff[kD / 32];
#pragma unroll
  for (int kk = 0; kk < kD / 32; ++kk) roff[kk] = n16 * kRowBytes + (((4 * kk + G) ^ swz_t(n16)) * 16);
  int toff[2][kD / 16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 16 * h + 4 * G + (n16 >> 2);
#pragma unroll
    for (int blk = 0; blk < kD / 16; ++blk) {
      const int chunk = 2 * blk + ((n16 & 3) >> 1);
      toff[h][blk] = row * kRowBytes + ((chunk ^ swz_t(row)) * 16) + (n16 & 1) * 8;
    }
  }
  f32x4_t acc_v[kD / 16], acc_k[kD / 16];
#pragma unroll
  for (int blk = 0; blk < kD / 16; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_v[blk][i] = acc_k[blk][i] = 0.f;

  const bool wave_live = c0 < key_end;
  const int c_hi = min(c0 + 15, key_end - 1);
  const int w_none_below = core ? core_first(c0) : c0;
  const int w_none_above = core ? L - 1 : raw_last(c_hi);
  const int w_all_from = core ? core_first(c_hi) : c_hi;
  const int w_all_to = core ? L - 1 : raw_last(c0);
  int q_lo;
  unsigned q_span;
  {
    const int key = c0 + n16;
    const int a = core ? core_first(key) : key;
    const int b = core ? L - 1 : raw_last(key);
    const bool ok = key <= c_hi && a <= b;
    q_lo = ok ? a : -0x40000000;
    q_span = ok ? (unsigned)(b - a) : 0u;
  }

  // query tiles from the last one down (the workgroups of a slice that run together
  // then stream the same tiles)
  auto tile_base = [&](int it) { return tq0 + (n_qt - 1 - it % n_qt) * kTileRows; };
  auto issue = [&](int it, uint8_t* buf) {
    const int base = tile_base(it);
    const size_t qs = qslice0 + it / n_qt;                // query slice of this iteration
    if (wave < 8) {
      fill_tile<8, true>(Q + qs * L * kD, base, L - 1, buf, wave, lane);
      fill_tile<8, true>(dO + qs * L * kD, base, L - 1, buf + kTileBytes, wave, lane);
    } else if (wave < 10) {
      const int t = min(base + lane, L - 1);
      const float* src = (wave == 8 ? lse : Dv) + qs * L + t;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(buf + 2 * kTileBytes +
                                                                                  (wave - 8) * kTileRows * 4),
                                       4, 0, 0);
    }
  };

  auto compute = [&](const uint8_t* buf, int qt) {
    const float* lse_t = reinterpret_cast<const float*>(buf + 2 * kTileBytes);
    const float* d_t = lse_t + kTileRows;
#pragma unroll
    for (int sb = 0; sb < kTileRows / 32; ++sb) {
      const int t0 = tile_base(qt) + sb * 32;
      const int t1 = min(t0 + 31, L - 1);
      if (t0 >= L) continue;
      int cls;   // 0: nothing visible, 1: everything visible, 2: mixed
      if (t1 < w_none_below || t0 > w_none_above) cls = 0;
      else if (t0 >= w_all_from && t1 <= w_all_to && t0 + 31 < L) cls = 1;
      else cls = 2;
      if (cls == 0) continue;
      const uint8_t* qsb = buf + sb * 32 * kRowBytes;
      const uint8_t* dsb = buf + kTileBytes + sb * 32 * kRowBytes;
      // scores S and dP for the two 16-query blocks (queries 16b + 4G + i in lane registers)
      f32x4_t s[2], dp[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint4 xa[kD / 32], ya[kD / 32];
#pragma unroll
        for (int kk = 0; kk < kD / 32; ++kk) {
          xa[kk] = *reinterpret_cast<const uint4*>(qsb + 16 * b * kRowBytes + roff[kk]);
          ya[kk] = *reinterpret_cast<const uint4*>(dsb + 16 * b * kRowBytes + roff[kk]);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[b][i] = dp[b][i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < kD / 32; ++kk) s[b] = Mma16<T>::mfma16(xa[kk], kop[kk], s[b]);
#pragma unroll
        for (int kk = 0; kk < kD / 32; ++kk) dp[b] = Mma16<T>::mfma16(ya[kk], vop[kk], dp[b]);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
      }
      // transpose operands (dO^T, Q^T) of gradient block blk: four 8-byte transpose reads
      auto tr4 = [&](int blk, v4s_t* t) {
        t[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(dsb + toff[0][blk]));
        t[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(dsb + toff[1][blk]));
        t[2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(qsb + toff[0][blk]));
        t[3] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(qsb + toff[1][blk]));
      };
      // the first kPre blocks' operands are read before the weights, so that the weight
      // arithmetic covers their latency (the compiler waits for all outstanding transpose
      // reads before their first use, so reads are grouped rather than pipelined one by one)
      constexpr int kPre = 2, kBatch = 3;
      v4s_t ta[kPre][4];
#pragma unroll
      for (int i = 0; i < kPre; ++i) tr4(i, ta[i]);
      __builtin_amdgcn_sched_barrier(0);
      // weights and dS; per-query statistics of the lane's 8 queries
      float pw[8], dsw[8];
      const int tq = t0 + 4 * G - q_lo;   // query t0 + 16b + 4G + i visible iff (tq + 16b + i) <= q_span
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const float4 lv = *reinterpret_cast<const float4*>(lse_t + sb * 32 + 16 * b + 4 * G);
        const float4 dv = *reinterpret_cast<const float4*>(d_t + sb * 32 + 16 * b + 4 * G);
        const float lr[4] = {lv.x, lv.y, lv.z, lv.w};
        const float dr[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = fast_exp2(fmaf(s[b][i], sc, -lr[i]));
          if (cls == 2) p = ((unsigned)(tq + 16 * b + i) <= q_span) ? p : 0.f;
          pw[4 * b + i] = p;
          dsw[4 * b + i] = p * (dp[b][i] - dr[i]);
        }
      }
      typename Mma16<T>::x2 pp[4], qq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pp[e] = Mma16<T>::round2(pw[2 * e], pw[2 * e + 1]);
        qq[e] = Mma16<T>::round2(dsw[2 * e], dsw[2 * e + 1]);
      }
      const uint4 pb = __builtin_bit_cast(uint4, pp);
      const uint4 db = __builtin_bit_cast(uint4, qq);
      // dV^T += dO^T P and dK^T += Q^T dS, 16 dims per MFMA
      auto grad = [&](int blk, const v4s_t* t) {
        const v4s_t ob[2] = {t[0], t[1]};
        const v4s_t qb[2] = {t[2], t[3]};
        acc_v[blk] = Mma16<T>::mfma16(__builtin_bit_cast(uint4, ob), pb, acc_v[blk]);
        acc_k[blk] = Mma16<T>::mfma16(__builtin_bit_cast(uint4, qb), db, acc_k[blk]);
      };
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kPre; ++i) grad(i, ta[i]);
      // the remaining blocks in batches of kBatch: reads of a batch, then its MFMAs
#pragma unroll
      for (int b0 = kPre; b0 < kD / 16; b0 += kBatch) {
        v4s_t tb[kBatch][4];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          if (b0 + i < kD / 16) tr4(b0 + i, tb[i]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          if (b0 + i < kD / 16) grad(b0 + i, tb[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // the tile before the newest one has landed: waves 0-7 issue 4 loads per tile, waves 8-9 one
  auto wait_older = [&]() {
    if (wave < 8) __builtin_amdgcn_s_waitcnt(0x0F74);
    else __builtin_amdgcn_s_waitcnt(0x0F71);
  };
  if (n_it > 0) issue(0, lds0);
  if (n_it > 1) issue(1, lds1);
  if (n_it > 1) wait_older();
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int qt = 0; qt < n_it; qt += 3) {
    if (qt + 2 < n_it) issue(qt + 2, lds2);
    if (wave_live) compute(lds0, qt);
    if (qt + 2 < n_it) wait_older();
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (qt + 1 >= n_it) break;
    if (qt + 3 < n_it) issue(qt + 3, lds0);
    if (wave_live) compute(lds1, qt + 1);
    if (qt + 3 < n_it) wait_older();
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (qt + 2 >= n_it) break;
    if (qt + 4 < n_it) issue(qt + 4, lds1);
    if (wave_live) compute(lds2, qt + 2);
    if (qt + 4 < n_it) wait_older();
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  if (!wave_live) return;
  const int key = c0 + n16;
  if (key >= key_end) return;
  float* ov = core ? dVc + ((size_t)bkv * m + key) * kD : dV + slice + (size_t)key * kD;
  float* ok = core ? dKc + ((size_t)bkv * m + key) * kD : dK + slice + (size_t)key * kD;
  // lane holds dims 16 blk + 4G + i of its key
#pragma unroll
  for (int blk = 0; blk < kD / 16; ++blk) {
    *reinterpret_cast<float4*>(ov + 16 * blk + 4 * G) =
        make_float4(acc_v[blk][0], acc_v[blk][1], acc_v[blk][2], acc_v[blk][3]);
    *reinterpret_cast<float4*>(ok + 16 * blk + 4 * G) =
        make_float4(acc_k[blk][0] * scale, acc_k[blk][1] * scale, acc_k[blk][2] * scale, acc_k[blk][3] * scale);
  }
}

// ---------------------------------------------------------------------------
// 4. pooling backward: one wave per group
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void cca_bwd_pool_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                          const T* __restrict__ V,
                                                          const float* __restrict__ dKc,
                                                          const float* __restrict__ dVc, float* __restrict__ dQ,
                                                          float* __restrict__ dK, float* __restrict__ dV, int64_t L,
                                                          int g, int64_t m, int nq, float scale) {
  extern __shared__ float sm[];   // a[g], then da / dz[g]
  float* a_l = sm;
  float* z_l = sm + g;
  const int64_t gid = blockIdx.x;
  const int64_t bkv = gid / m, j = gid - bkv * m;           // key/value slice, group
  const int lane = threadIdx.x;
  const size_t row0 = (size_t)bkv * L + (size_t)j * g;       // first row of the group
  // its scoring query: row j*g+g-1 of each of the nq query slices bkv*nq .. (their mean)
  const size_t qrow0 = ((size_t)bkv * nq * L + (size_t)j * g + g - 1) * kD;
  const size_t qstride = (size_t)L * kD;
  const float inv_nq = 1.0f / (float)nq;
  const float* dkc = dKc + ((size_t)bkv * m + j) * kD;
  const float* dvc = dVc + ((size_t)bkv * m + j) * kD;
  // scoring pass: 4 lanes per row, 32 dims each (q_hat, dKc, dVc slices in registers)
  const int rsub = lane >> 2, seg = lane & 3;
  float qf[32], kcf[32], vcf[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) Elem<T>::chunk_to_f32(ld16(Q + qrow0 + seg * 32 + c * 8), qf + c * 8);
  if (nq > 1) {
    for (int h = 1; h < nq; ++h) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float f[8];
        Elem<T>::chunk_to_f32(ld16(Q + qrow0 + h * qstride + seg * 32 + c * 8), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[c * 8 + e] += f[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) qf[e] *= inv_nq;
  }
#pragma unroll
  for (int e = 0; e < 32; e += 4) {
    const float4 x = *reinterpret_cast<const float4*>(dkc + seg * 32 + e);
    const float4 y = *reinterpret_cast<const float4*>(dvc + seg * 32 + e);
    kcf[e] = x.x; kcf[e + 1] = x.y; kcf[e + 2] = x.z; kcf[e + 3] = x.w;
    vcf[e] = y.x; vcf[e + 1] = y.y; vcf[e + 2] = y.z; vcf[e + 3] = y.w;
  }
  const float sc = scale * kLog2e;
  for (int r0 = 0; r0 < g; r0 += 16) {
    const int r = r0 + rsub;
    float s = 0.f, da = 0.f;
    if (r < g) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float kf[8], vf[8];
        Elem<T>::chunk_to_f32(ld16(K + (row0 + r) * kD + seg * 32 + c * 8), kf);
        Elem<T>::chunk_to_f32(ld16(V + (row0 + r) * kD + seg * 32 + c * 8), vf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s = fmaf(qf[c * 8 + e], kf[e], s);
          da = fmaf(kcf[c * 8 + e], kf[e], fmaf(vcf[c * 8 + e], vf[e], da));
        }
      }
    }
    s = lane_group_sum<4>(s);
    da = lane_group_sum<4>(da);
    if (seg == 0 && r < g) {
      a_l[r] = s * sc;
      z_l[r] = da;
    }
  }
  wave_lds_sync();
  // softmax of the group scores, then dz = a (da - a.da)
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
  // row updates: each lane owns 2 consecutive dims
  const int col = lane * 2;
  float q2[2] = {0.f, 0.f}, kc2[2], vc2[2], dq2[2] = {0.f, 0.f};
  {
    for (int h = 0; h < nq; ++h) {
      float f[2];
      Elem<T>::pair_to_f32(*reinterpret_cast<const uint32_t*>(Q + qrow0 + h * qstride + col), f);
      q2[0] += f[0];
      q2[1] += f[1];
    }
    if (nq > 1) {
      q2[0] *= inv_nq;
      q2[1] *= inv_nq;
    }
    kc2[0] = dkc[col]; kc2[1] = dkc[col + 1];
    vc2[0] = dvc[col]; vc2[1] = dvc[col + 1];
  }
  for (int r = 0; r < g; ++r) {
    const float a = a_l[r], dz = z_l[r];
    float kf[2];
    Elem<T>::pair_to_f32(*reinterpret_cast<const uint32_t*>(K + (row0 + r) * kD + col), kf);
    const float k0 = kf[0], k1 = kf[1];
    float2* pk = reinterpret_cast<float2*>(dK + (row0 + r) * kD + col);
    float2* pv = reinterpret_cast<float2*>(dV + (row0 + r) * kD + col);
    float2 xk = *pk, xv = *pv;
    xk.x += a * kc2[0] + scale * dz * q2[0];
    xk.y += a * kc2[1] + scale * dz * q2[1];
    xv.x += a * vc2[0];
    xv.y += a * vc2[1];
    *pk = xk;
    *pv = xv;
    dq2[0] = fmaf(dz, k0, dq2[0]);
    dq2[1] = fmaf(dz, k1, dq2[1]);
  }
  // d q_hat reaches each of the nq scoring queries with weight 1/nq
  for (int h = 0; h < nq; ++h) {
    float2* pq = reinterpret_cast<float2*>(dQ + qrow0 + h * qstride + col);
    float2 xq = *pq;
    xq.x += scale * inv_nq * dq2[0];
    xq.y += scale * inv_nq * dq2[1];
    *pq = xq;
  }
}

}  // namespace

size_t backward_workspace_bytes(int B, int H, int H_kv, int64_t L, int d, int g) {
  const size_t BH = (size_t)B * H, BHkv = (size_t)B * H_kv;
  const size_t m = (size_t)(L / g);
  return (2 * BH * (size_t)L + 2 * BHkv * m * (size_t)d) * sizeof(float);
}

template <typename T>
hipError_t launch_backward_t(const void* q, const void* k, const void* v, const void* kc, const void* vc,
                                     const void* out, const float* lse, const void* dout, float* dq, float* dk,
                                     float* dv, void* workspace, int BH, int nq, int64_t L, int g, int k_local,
                                     float scale, hipStream_t stream) {
  const int64_t m = L / g;
  const int BHkv = BH / nq;
  float* Dv = (float*)workspace;
  float* lse2 = Dv + (size_t)BH * L;
  float* dKc = lse2 + (size_t)BH * L;
  float* dVc = dKc + (size_t)BHkv * m * kD;
  const int64_t rows = (int64_t)BH * L;
  hipLaunchKernelGGL(cca_bwd_prep_kernel<T>, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, stream,
                     (const T*)out, (const T*)dout, lse, Dv, lse2, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ntiles = (int)((L + 255) / 256);
  hipLaunchKernelGGL(cca_bwd_dq_kernel<T>, dim3((unsigned)(BH * ntiles)), dim3(512), 0, stream, (const T*)q,
                     (const T*)k, (const T*)v, (const T*)kc, (const T*)vc, (const T*)dout,
                     (const float*)lse2, (const float*)Dv, dq, BH, nq, (int)L, g, k_local, scale, ntiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_core_wg = (int)((m + 191) / 192);
  const int n_wg = n_core_wg + (int)((L + 191) / 192);
  hipLaunchKernelGGL(cca_bwd_dkdv16_kernel<T>, dim3((unsigned)((int64_t)BHkv * n_wg)), dim3(768), 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)kc, (const T*)vc,
                     (const T*)dout, (const float*)lse2, (const float*)Dv, dk, dv, dKc, dVc, BHkv, nq, (int)L,
                     g, k_local, scale, n_core_wg);
  e = hipGetLastError();
  if (e != hipSuccess || m == 0) return e;
  hipLaunchKernelGGL(cca_bwd_pool_kernel<T>, dim3((unsigned)((int64_t)BHkv * m)), dim3(64),
                     (size_t)2 * g * sizeof(float), stream, (const T*)q, (const T*)k, (const T*)v,
                     (const float*)dKc, (const float*)dVc, dq, dk, dv, L, g, m, nq, scale);
  return hipGetLastError();
}

hipError_t launch_backward_d128(int dt, const void* q, const void* k, const void* v, const void* kc, const void* vc,
                                const void* out, const float* lse, const void* dout, float* dq, float* dk, float* dv,
                                void* workspace, int BH, int nq, int64_t L, int g, int k_local, float scale,
                                hipStream_t stream) {
  if (dt == CCA_F16)
    return launch_backward_t<f16_t>(q, k, v, kc, vc, out, lse, dout, dq, dk, dv, workspace, BH, nq, L, g, k_local,
                                    scale, stream);
  return launch_backward_t<bf16_t>(q, k, v, kc, vc, out, lse, dout, dq, dk, dv, workspace, BH, nq, L, g, k_local,
                                   scale, stream);
}

}  // namespace cca
