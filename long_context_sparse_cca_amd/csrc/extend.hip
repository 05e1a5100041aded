// Chunked append: n new tokens per sequence in one call, each sequence at its own
// length, grouped-query heads; returns the attention output of every new token.
//
// Method: the CCA write-up ("ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"):
// a token at position p attends, in one softmax, to the core tokens of the groups
// before its raw window and to the raw keys (p/g - k)*g .. p (locality-preserving
// module, global-local fusion); a group's core token is pooled from its tokens with
// the group's last query (global-aware pooling) as soon as the group is complete,
// and the cache keeps core tokens plus the local raw tokens (Triton section, Fig. 3).
// A token's output depends only on its position and the tokens before it, so a
// chunk of n tokens gives the same rows as n single-token steps.
//
// Three launches:
//   1. gather: the raw keys/values a chunk can see -- positions raw0 .. pos+n-1 with
//      raw0 = max(0, pos/g - k)*g -- into one contiguous scratch slice per key/value
//      head: the cached part from the ring, the rest from the chunk itself;
//   2. attention: the prefill attention kernels in extend mode over that scratch
//      slice and the cached core tokens (MFMA, one softmax per query);
//   3. finish: the chunk's keys/values go to their ring slots, every group the chunk
//      completes is pooled into its core slot (mean query over the query heads that
//      share the key/value head; one wave per group), and the sequence length advances
//      by n.
// LCA-style cache: launch 3 condenses a completed group instead (mean of the group's
// queries over its positions and the query heads sharing the key/value head, positional
// dims from the top-scored token; "Latent-Condensed Transformer for Efficient Long Context
// Modeling", sections 2 and 3), taking the queries of the group's tokens before the chunk
// from the running sum qsum, and then leaves in qsum the sum of the chunk's trailing
// incomplete group.
// With n <= k*g + 1 no token of the chunk can see a core token pooled from the same
// chunk (the earliest group it completes becomes visible k*g+1 positions after the
// chunk's first token), so pooling can follow the attention.  Launch 3 overwrites
// only ring slots whose positions no later step needs, after launches 1-2 read them.
#include <algorithm>

#include "cca_internal.h"
#include "lca_group.h"
#include "pool_group.h"

namespace cca {
namespace {

// Workspace head: the per-sequence start positions (int32), then the sequences ordered by
// length, longest first (int32), each padded to 256 bytes.
size_t pos_bytes(int B) { return ((size_t)B * sizeof(int32_t) + 255) / 256 * 256; }
size_t head_bytes(int B) { return 2 * pos_bytes(B); }

template <typename T, int D>
__global__ __launch_bounds__(256) void cca_extend_gather_kernel(const int32_t* __restrict__ lens, int64_t max_len,
                                                                int32_t* __restrict__ pos_ws,
                                                                int32_t* __restrict__ order_ws,
                                                                const T* __restrict__ k_chunk,
                                                                const T* __restrict__ v_chunk,
                                                                const T* __restrict__ ring_k,
                                                                const T* __restrict__ ring_v, T* __restrict__ sk,
                                                                T* __restrict__ sv, int Hkv, int n, int64_t R, int g,
                                                                int k_local, int64_t raw_rows) {
  constexpr int CPR = D * (int)sizeof(T) / 16;
  const int64_t bkv = blockIdx.x;
  const int64_t b = bkv / Hkv;
  const int64_t t = lens[b];
  const bool valid = t >= 0 && t <= max_len;
  if (blockIdx.y == 0 && bkv % Hkv == 0) {
    // one block per sequence: its start position, and its rank by length (longest first,
    // ties by index, out-of-range sequences last), so order_ws is a permutation of 0..B-1
    __shared__ int rank;
    if (threadIdx.x == 0) rank = 0;
    __syncthreads();
    const int64_t B = gridDim.x / Hkv;
    const int64_t key = valid ? t : -1;
    int before = 0;
    for (int64_t i = threadIdx.x; i < B; i += blockDim.x) {
      const int64_t ti = lens[i];
      const int64_t ki = (ti >= 0 && ti <= max_len) ? ti : -1;
      before += (ki > key || (ki == key && i < b)) ? 1 : 0;
    }
    atomicAdd(&rank, before);
    __syncthreads();
    if (threadIdx.x == 0) {
      pos_ws[b] = valid ? (int32_t)t : -1;
      order_ws[rank] = (int32_t)b;
    }
  }
  if (!valid) return;
  const int64_t raw0 = std::max<int64_t>(0, t / g - k_local) * g;
  const int64_t rows = t + n - raw0;
  // grid-stride over the (row, 16-byte piece) pairs: the y extent is capped at launch
  for (int64_t idx = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; idx < rows * CPR;
       idx += (int64_t)gridDim.y * blockDim.x) {
    const int64_t u = idx / CPR;
    const int c = (int)(idx % CPR);
    const int64_t pos = raw0 + u;
    const T* srck;
    const T* srcv;
    if (pos < t) {
      const int64_t slot = (uint32_t)pos % (uint32_t)R;   // positions and R fit in 32 bits
      srck = ring_k + ((size_t)bkv * R + slot) * D;
      srcv = ring_v + ((size_t)bkv * R + slot) * D;
    } else {
      srck = k_chunk + ((size_t)bkv * n + (pos - t)) * D;
      srcv = v_chunk + ((size_t)bkv * n + (pos - t)) * D;
    }
    const size_t dst = ((size_t)bkv * raw_rows + u) * D;
    st16(reinterpret_cast<uint4*>(sk + dst) + c, ld16(reinterpret_cast<const uint4*>(srck) + c));
    st16(reinterpret_cast<uint4*>(sv + dst) + c, ld16(reinterpret_cast<const uint4*>(srcv) + c));
  }
}

// Add to s, row by row over chunk rows r0 .. r1, the sum of the nq query heads' rows (this
// lane's D/64 columns of q_chunk [B*Hq][n][D], head slices of sequence b): each row's heads
// are summed first, in head order, then the row sum is added -- the order in which the decode
// steps add a token's queries.  The loads of up to 16 rows of one head are issued together.
template <typename T, int D>
__device__ __forceinline__ void add_query_rows(const T* __restrict__ q_chunk, int64_t b, int Hq, int hk, int nq,
                                               int n, int64_t r0, int64_t r1, int col, float* s) {
  constexpr int CPL = D / kWave;
  constexpr int RB = 16;
  for (int64_t rb = r0; rb <= r1; rb += RB) {
    const int cnt = (int)std::min<int64_t>(RB, r1 - rb + 1);
    float t[RB][CPL];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int e = 0; e < CPL; ++e) t[r][e] = 0.f;
    for (int h = 0; h < nq; ++h) {
      const T* qh = q_chunk + (((size_t)b * Hq + (size_t)hk * nq + h) * n + rb) * D + col;
      float f[RB][CPL];
#pragma unroll
      for (int r = 0; r < RB; ++r) lca_load_cols<T, D>(qh + (size_t)std::min(r, cnt - 1) * D, f[r]);
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int e = 0; e < CPL; ++e) t[r][e] += f[r][e];
    }
#pragma unroll
    for (int r = 0; r < RB; ++r)
      if (r < cnt) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) s[e] += t[r][e];
      }
  }
}

// Launch 3.  Blocks y < ring_blocks: the chunk's key/value rows into their ring slots
// (16-byte pieces, grid-stride) and the new length.  The other blocks: one wave per group
// the chunk completes (the w-th such group for wave w; the caller sizes the grid for the
// n/g + 1 groups a chunk can complete), pooled -- LCA: condensed -- from the staged rows; for
// the LCA-style cache, wave 0 then leaves in qsum the query sum of the trailing incomplete
// group (it alone reads the previous sum, for the chunk's first group).
template <typename T, int D, bool LCA>
__global__ __launch_bounds__(256) void cca_extend_finish_kernel(
    int32_t* __restrict__ lens, const int32_t* __restrict__ pos_ws, const T* __restrict__ q_chunk,
    const T* __restrict__ k_chunk, const T* __restrict__ v_chunk, const T* __restrict__ sk,
    const T* __restrict__ sv, T* __restrict__ ring_k, T* __restrict__ ring_v, T* __restrict__ core_k,
    T* __restrict__ core_v, int Hkv, int nq, int n, int64_t R, int64_t max_groups, int g, int k_local,
    int64_t raw_rows, float scale, float* __restrict__ qsum, int d_rope, int ring_blocks) {
  extern __shared__ float w_lds[];
  constexpr int CPR = D * (int)sizeof(T) / 16;
  constexpr int CPL = D / kWave;
  const int64_t bkv = blockIdx.x;
  const int64_t b = bkv / Hkv;
  const int hk = (int)(bkv - b * Hkv);
  const int64_t t = pos_ws[b];
  if (t < 0) return;
  if ((int)blockIdx.y < ring_blocks) {
    if (blockIdx.y == 0 && threadIdx.x == 0 && hk == 0) lens[b] = (int32_t)(t + n);
    for (int64_t idx = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; idx < (int64_t)n * CPR;
         idx += (int64_t)ring_blocks * blockDim.x) {
      const int64_t i = idx / CPR;
      const int c = (int)(idx - i * CPR);
      const int64_t slot = (uint32_t)(t + i) % (uint32_t)R;   // positions and R fit in 32 bits
      st16(reinterpret_cast<uint4*>(ring_k + ((size_t)bkv * R + slot) * D) + c,
           ld16(reinterpret_cast<const uint4*>(k_chunk + ((size_t)bkv * n + i) * D) + c));
      st16(reinterpret_cast<uint4*>(ring_v + ((size_t)bkv * R + slot) * D) + c,
           ld16(reinterpret_cast<const uint4*>(v_chunk + ((size_t)bkv * n + i) * D) + c));
    }
    return;
  }
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int w = ((int)blockIdx.y - ring_blocks) * (int)(blockDim.x / kWave) + wave;
  const int64_t ngroups = (t + n) / g - t / g;   // groups whose last token is in the chunk
  const bool has_group = w < ngroups;
  if (!has_group && !(LCA && w == 0)) return;
  const int Hq = Hkv * nq;
  const int col = lane * CPL;
  if (has_group) {
    // group beta: positions p-g+1 .. p, all inside the staged slice (they start at or after
    // the group of the chunk's first token, which is not before raw0)
    const int64_t beta = t / g + w;
    const int64_t p = beta * g + g - 1;
    const int64_t i = p - t;                     // chunk row of the group's last token
    const int64_t raw0 = std::max<int64_t>(0, t / g - k_local) * g;
    const size_t first = ((size_t)bkv * raw_rows + (p - g + 1 - raw0)) * D;
    const size_t last = first + (size_t)(g - 1) * D;
    T* kc = core_k + ((size_t)bkv * max_groups + beta) * D;
    T* vc = core_v + ((size_t)bkv * max_groups + beta) * D;
    if constexpr (LCA) {
      constexpr bool kFast = D == 128 && sizeof(T) == 2;
      // d = 128, g = 16: the group's staged rows fetched up front (scoring segments, then the
      // columns of the weighted sums), while the query rows are summed
      constexpr int G16 = 16;
      uint4 kseg[kFast ? 4 : 1];
      uint32_t kcol[kFast ? G16 : 1], vcol[kFast ? G16 : 1];
      const bool fast = kFast && g == G16;
      if constexpr (kFast) {
        if (fast) {
          const int rsub = lane >> 2, seg = lane & 3;
#pragma unroll
          for (int c = 0; c < 4; ++c) kseg[c] = ld16(sk + first + (size_t)rsub * D + seg * (D / 4) + c * 8);
#pragma unroll
          for (int r = 0; r < G16; ++r) {
            kcol[r] = *reinterpret_cast<const uint32_t*>(sk + first + (size_t)r * D + col);
            vcol[r] = *reinterpret_cast<const uint32_t*>(sv + first + (size_t)r * D + col);
          }
        }
      }
      // the group's queries: the running sum of its tokens before the chunk, then chunk rows
      float s[CPL];
      int64_t r0 = i - g + 1;
      if (r0 < 0) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) s[e] = qsum[(size_t)bkv * D + col + e];
        r0 = 0;
      } else {
#pragma unroll
        for (int e = 0; e < CPL; ++e) s[e] = 0.f;
      }
      add_query_rows<T, D>(q_chunk, b, Hq, hk, nq, n, r0, i, col, s);
      float* qbar = w_lds + wave * (D + g);
      const float inv = 1.0f / ((float)g * (float)nq);
#pragma unroll
      for (int e = 0; e < CPL; ++e) qbar[col + e] = s[e] * inv;
      wave_lds_sync();
      if constexpr (kFast) {
        if (fast) {
          lca_condense_math<T, D, G16>(
              qbar, G16, scale, d_rope, kc, vc, qbar + D, nullptr, [&](int, int c) { return kseg[c]; },
              [&](int r, float* f) { Elem<T>::pair_to_f32(kcol[r], f); },
              [&](int r, float* f) { Elem<T>::pair_to_f32(vcol[r], f); },
              [&](int r, float* f) { lca_load_cols<T, D>(sk + first + (size_t)r * D + col, f); });
        }
      }
      if (!fast)
        lca_condense_wave<T, D>(qbar, sk + first, sv + first, sk + last, sv + last, g, scale, d_rope, kc, vc,
                                qbar + D, nullptr);
    } else {
      pool_group_wave<T, D>(q_chunk + (((size_t)b * Hq + (size_t)hk * nq) * n + i) * D, (int64_t)n * D, nq,
                            sk + first, sv + first, sk + last, sv + last, g, scale, kc, vc, w_lds + wave * g);
    }
  }
  if constexpr (LCA) {
    if (w == 0) {
      // the query sum of the trailing incomplete group: the chunk's rows after its last
      // completed group, on top of the previous sum when the chunk completes no group
      float s[CPL];
      const int64_t end = t + n;
#pragma unroll
      for (int e = 0; e < CPL; ++e) s[e] = ngroups > 0 ? 0.f : qsum[(size_t)bkv * D + col + e];
      const int64_t r0 = ngroups > 0 ? end / g * g - t : 0;
      if (r0 < n) add_query_rows<T, D>(q_chunk, b, Hq, hk, nq, n, r0, n - 1, col, s);
#pragma unroll
      for (int e = 0; e < CPL; ++e) qsum[(size_t)bkv * D + col + e] = s[e];
    }
  }
}

template <typename T, int D>
hipError_t launch_extend_t(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q, int n, const void* q,
                           const void* k, const void* v, void* out, int out_f32, void* workspace, float scale,
                           float* qsum, int d_rope, hipStream_t stream) {
  const int64_t R = (int64_t)(c->k_local + 1) * c->g;
  const int64_t raw_rows = R + n;
  const int64_t BHkv = (int64_t)c->B * c->H;
  const int nq = H_q / c->H;
  int32_t* pos_ws = (int32_t*)workspace;
  int32_t* order_ws = (int32_t*)((uint8_t*)workspace + pos_bytes(c->B));
  T* sk = (T*)((uint8_t*)workspace + head_bytes(c->B));
  T* sv = sk + (size_t)BHkv * raw_rows * D;
  constexpr int CPR = D * (int)sizeof(T) / 16;
  const int64_t gy = std::min<int64_t>((raw_rows * CPR + 255) / 256, 65535);   // the kernel strides over the rest
  hipLaunchKernelGGL((cca_extend_gather_kernel<T, D>), dim3((unsigned)BHkv, (unsigned)gy), dim3(256), 0, stream, lens,
                     max_len, pos_ws, order_ws, (const T*)k, (const T*)v, (const T*)c->ring_k, (const T*)c->ring_v, sk, sv, c->H,
                     n, R, c->g, c->k_local, raw_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const ExtendArgs ext{pos_ws, H_q, n, raw_rows, c->max_groups, order_ws};
  e = launch_extend_attention(c->dt, D, q, sk, sv, c->core_k, c->core_v, out, out_f32, c->B * H_q, nq, c->g,
                              c->k_local, scale, ext, stream);
  if (e != hipSuccess) return e;
  // launch 3: ring copies, then one wave per completed group (at most n/g + 1 groups)
  const int ring_blocks = (int)std::min<int64_t>(((int64_t)n * CPR + 255) / 256, 32768);
  const int pool_blocks = (int)((n / c->g + 1 + 3) / 4);   // n/g + 1 <= kExtendMaxGroupWaves (checked by the caller)
  const dim3 fgrid((unsigned)BHkv, (unsigned)(ring_blocks + pool_blocks));
  if (qsum == nullptr) {
    hipLaunchKernelGGL((cca_extend_finish_kernel<T, D, false>), fgrid, dim3(256), (size_t)4 * c->g * sizeof(float),
                       stream, lens, pos_ws, (const T*)q, (const T*)k, (const T*)v, (const T*)sk, (const T*)sv,
                       (T*)c->ring_k, (T*)c->ring_v, (T*)c->core_k, (T*)c->core_v, c->H, nq, n, R, c->max_groups,
                       c->g, c->k_local, raw_rows, scale, (float*)nullptr, 0, ring_blocks);
  } else {
    hipLaunchKernelGGL((cca_extend_finish_kernel<T, D, true>), fgrid, dim3(256), (size_t)4 * (D + c->g) * sizeof(float),
                       stream, lens, pos_ws, (const T*)q, (const T*)k, (const T*)v, (const T*)sk, (const T*)sv,
                       (T*)c->ring_k, (T*)c->ring_v, (T*)c->core_k, (T*)c->core_v, c->H, nq, n, R, c->max_groups,
                       c->g, c->k_local, raw_rows, scale, qsum, d_rope, ring_blocks);
  }
  return hipGetLastError();
}

}  // namespace

size_t extend_workspace_bytes(const cca_cache_t* c, int n) {
  const size_t R = (size_t)(c->k_local + 1) * c->g;
  const size_t esz = (size_t)dtype_bytes(c->dt);
  return head_bytes(c->B) + 2 * (size_t)c->B * c->H * (R + (size_t)n) * c->d * esz;
}

hipError_t launch_extend(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q, int n, const void* q,
                         const void* k, const void* v, void* out, int out_f32, void* workspace, float scale,
                         hipStream_t stream, float* qsum, int d_rope) {
  return dispatch_td(c->dt, c->d, [&](auto t, auto dd) {
    using T = decltype(t);
    return launch_extend_t<T, decltype(dd)::value>(c, lens, max_len, H_q, n, q, k, v, out,
                                                   sizeof(T) == 4 ? 1 : out_f32, workspace, scale, qsum, d_rope,
                                                   stream);
  });
}

}  // namespace cca
