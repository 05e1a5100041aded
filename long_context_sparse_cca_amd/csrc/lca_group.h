// LCA-style condensation of one group of g tokens into one core token, done by one wave.
//
// Method: "Latent-Condensed Transformer for Efficient Long Context Modeling",
// section 2: the tokens of a group are scored by the dot product of the group's
// mean query with their keys; the content part of the key and the value are
// condensed by importance-weighted pooling (softmax of the scores); the positional
// (RoPE) part of the key is not mixed: the top-scored token is the group's anchor
// and keeps its positional key.  Here the last d_rope dims of a key are its
// positional part.  Shared by the prefill condensation and the decode cache, so
// that both reach the same core token (and anchor) from the same mean query.
#pragma once

#include "cca_device.h"

namespace cca {

// Load the D/64 consecutive columns of a row that lane `lane` owns, as floats.
template <typename T, int D>
__device__ __forceinline__ void lca_load_cols(const T* p, float* f) {
  constexpr int CPL = D / kWave;   // columns per lane: 1 or 2
  if constexpr (sizeof(T) == 2) {
    if constexpr (CPL == 2) {
      Elem<T>::pair_to_f32(*reinterpret_cast<const uint32_t*>(p), f);
    } else {
      f[0] = Elem<T>::bits_to_f32(reinterpret_cast<const uint16_t*>(p)[0]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < CPL; ++e) f[e] = p[e];
  }
}

// The arithmetic of one group's condensation by one wave, with the group's rows supplied by
// accessors (so that every caller, whichever way it fetches the rows, computes the same
// floats in the same order):
//   kseg(r, c)     16-byte chunk c of the 32-dim segment (lane % 4) of key row r (scores)
//   kcols(r, f)    this lane's D/64 columns of key row r, as floats (weighted sums)
//   vcols(r, f)    the same for value row r
//   kanchor(r, f)  kcols for the anchor row r (a wave-uniform runtime index)
// G > 0 fixes the group size at compile time (g must equal it); G = 0 takes g at run time.
//   qbar  : the group's mean query, D floats in LDS (written before the call and ordered
//           with wave_lds_sync by the caller)
//   w     : LDS scratch of g floats owned by this wave
//   anchor: if non-null, lane 0 stores the anchor (position in the group) there
// The scores use scale * log2(e) (exp2 softmax); the anchor is the first position whose
// score equals the maximum.  Math in float32; kc/vc receive one rounding to T.
template <typename T, int D, int G, class KSeg, class KCols, class VCols, class KAnchor>
__device__ __forceinline__ void lca_condense_math(const float* qbar, int g_rt, float scale, int d_rope,
                                                  T* __restrict__ kc, T* __restrict__ vc, float* w,
                                                  int32_t* anchor, KSeg kseg, KCols kcols, VCols vcols,
                                                  KAnchor kanchor) {
  constexpr int CPL = D / kWave;
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int LPR = 4;            // lanes per row in the scoring pass
  constexpr int SEG = D / LPR;
  constexpr int SEGC = SEG / EPC;
  const int g = G > 0 ? G : g_rt;
  const int lane = threadIdx.x & (kWave - 1);
  const int col = lane * CPL;

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
        Elem<T>::chunk_to_f32(kseg(r, c), kf);
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
  auto accumulate = [&](int r) {
    const float a = w[r];
    float kf[CPL], vf[CPL];
    kcols(r, kf);
    vcols(r, vf);
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      ak[e] = fmaf(a, kf[e], ak[e]);
      av[e] = fmaf(a, vf[e], av[e]);
    }
  };
  if constexpr (G > 0) {
#pragma unroll
    for (int r = 0; r < G; ++r) accumulate(r);
  } else {
    for (int r = 0; r < g; ++r) accumulate(r);
  }
  float kanc[CPL];
  kanchor(arg, kanc);
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    const bool positional = col + e >= D - d_rope;
    Elem<T>::store1(kc + col + e, positional ? kanc[e] : ak[e]);
    Elem<T>::store1(vc + col + e, av[e]);
  }
  if (anchor != nullptr && lane == 0) *anchor = arg;
}

// One wave condenses rows 0..g-1 of a group read from memory: rows r < g-1 at
// k_rows + r*D / v_rows + r*D, row g-1 at k_last / v_last (the decode cache passes the newest
// token there).  Arguments as for lca_condense_math.
template <typename T, int D>
__device__ __forceinline__ void lca_condense_wave(const float* qbar, const T* __restrict__ k_rows,
                                                  const T* __restrict__ v_rows, const T* __restrict__ k_last,
                                                  const T* __restrict__ v_last, int g, float scale, int d_rope,
                                                  T* __restrict__ kc, T* __restrict__ vc, float* w,
                                                  int32_t* anchor) {
  constexpr int CPL = D / kWave;
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int SEG = D / 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int col = lane * CPL;
  const int seg = lane % 4;
  auto krow = [&](int r) { return r == g - 1 ? k_last : k_rows + (size_t)r * D; };
  auto vrow = [&](int r) { return r == g - 1 ? v_last : v_rows + (size_t)r * D; };
  lca_condense_math<T, D, 0>(
      qbar, g, scale, d_rope, kc, vc, w, anchor,
      [&](int r, int c) { return ld16(krow(r) + seg * SEG + c * EPC); },
      [&](int r, float* f) { lca_load_cols<T, D>(krow(r) + col, f); },
      [&](int r, float* f) { lca_load_cols<T, D>(vrow(r) + col, f); },
      [&](int r, float* f) { lca_load_cols<T, D>(krow(r) + col, f); });
}

}  // namespace cca
