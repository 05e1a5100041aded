// Internal launch interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <type_traits>

#include "cca_device.h"
#include "cca.h"

namespace cca {

// Calls fn(T{}, std::integral_constant<int, D>{}) with the element type T of cca_dtype_t
// dt (bf16_t, f16_t or float) and the head dim D (64 or 128; validated by the caller).
template <typename Fn>
hipError_t dispatch_td(int dt, int d, Fn&& fn) {
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (dt == CCA_BF16) return d == 128 ? fn(bf16_t{}, D128{}) : fn(bf16_t{}, D64{});
  if (dt == CCA_F16) return d == 128 ? fn(f16_t{}, D128{}) : fn(f16_t{}, D64{});
  return d == 128 ? fn(float{}, D128{}) : fn(float{}, D64{});
}

// Output encoding of the decode merge: 0 float32, 1 bf16, 2 binary16.
inline int out_mode(int out_f32, int dt) {
  if (out_f32) return 0;
  return dt == CCA_BF16 ? 1 : (dt == CCA_F16 ? 2 : 0);
}

// Bytes per element of a cca_dtype_t.
inline int dtype_bytes(int dt) { return dt == CCA_F32 ? 4 : 2; }

// Each launcher enqueues its kernels on `stream` and returns the launch status.
// Arguments have been validated by the caller (api.hip).
// Attention of new tokens over a cached prefix (chunked append), run by the
// prefill attention kernels with offsets: query i of a slice sits at absolute
// position pos[b] + i; the raw key at absolute position u is row u - raw0 of the
// raw K/V slice, raw0 = max(0, pos[b]/g - k_local)*g (the first raw position any
// query of the slice sees); core token j is row j of the core slice.
// Waves the chunked append's finish launch can give to completed groups (one each): a chunk
// of n tokens completes at most n/g + 1 groups.
constexpr int64_t kExtendMaxGroupWaves = (int64_t)4 * 32767;

struct ExtendArgs {
  const int32_t* pos;  // device [B]: position of the first new token; < 0 marks an invalid sequence
  int Hq;              // query heads: query slice bh belongs to sequence bh / Hq
  int n;               // new tokens (queries) per slice
  int64_t raw_rows;    // rows per raw K/V slice
  int64_t core_rows;   // rows per core K/V slice
  const int32_t* order;  // device [B]: the sequences by length, longest first (work order)
};

// LCA-style pooling (pool_lca.hip): mean-query importance (over the group and the nq query
// heads of a key/value head), the last d_rope dims of a core key taken from the group's
// top-scored token; anchors (optional) receive its index.
hipError_t launch_pool_lca(int dt, int d, const void* q, const void* k, const void* v, void* kc, void* vc,
                           int32_t* anchors, int BHkv, int64_t L, int g, int nq, int d_rope, float scale,
                           hipStream_t stream);

// Grouped-query attention: nq = H / H_kv query heads share each key/value head.
// Query/output slices are (b, h) = b*H + h; key/value and core slices are
// (b, h_kv) = b*H_kv + h_kv, and query slice s reads key/value slice s / nq.
hipError_t launch_pool(int dt, int d, const void* q, const void* k, const void* v, void* kc, void* vc,
                       int BHkv, int64_t L, int g, int nq, float scale, hipStream_t stream);

// lse (optional, float32 [BH][L]): each query's natural-log log-sum-exp of its scaled scores.
hipError_t launch_prefill_attention(int dt, int d, const void* q, const void* k, const void* v,
                                    const void* kc, const void* vc, void* out, int out_f32, int BH, int nq,
                                    int64_t L, int g, int k_local, float scale, hipStream_t stream,
                                    float* lse = nullptr);

// 16-bit (dt = CCA_BF16 or CCA_F16), head dim 128 fast path of the fused attention
// (prefill_d128.hip).  lse (optional, float32 [BH][L]): natural-log log-sum-exp of each
// query's scaled scores.
hipError_t launch_prefill_d128(int dt, const void* q, const void* k, const void* v, const void* kc, const void* vc,
                               void* out, int out_f32, int BH, int nq, int64_t L, int g, int k_local, float scale,
                               hipStream_t stream, float* lse = nullptr);

// Extend-mode attention (16-bit d=128 fast kernel or the generic one): q, out [B*H][n][d];
// k, v [B*H_kv][ext.raw_rows][d]; kc, vc [B*H_kv][ext.core_rows][d].
hipError_t launch_extend_attention(int dt, int d, const void* q, const void* k, const void* v, const void* kc,
                                   const void* vc, void* out, int out_f32, int BH, int nq, int g, int k_local,
                                   float scale, const ExtendArgs& ext, hipStream_t stream);
hipError_t launch_extend_attention_d128(int dt, const void* q, const void* k, const void* v, const void* kc,
                                        const void* vc, void* out, int out_f32, int BH, int nq, int g, int k_local,
                                        float scale, const ExtendArgs& ext, hipStream_t stream);

hipError_t launch_cache_load(const cca_cache_t* c, const void* k, const void* v, const void* kc,
                             const void* vc, int64_t L, hipStream_t stream);

hipError_t launch_cache_append(const cca_cache_t* c, const void* q, const void* k, const void* v,
                               float scale, hipStream_t stream);

int decode_num_chunks(const cca_cache_t* c);
size_t decode_workspace_bytes(const cca_cache_t* c);

hipError_t launch_decode(const cca_cache_t* c, const void* q, void* out, int out_f32, void* workspace,
                         float scale, hipStream_t stream);

// Append (ring write + in-place pooling) and decode of the new token in one launch.
hipError_t launch_append_decode(const cca_cache_t* c, const void* q, const void* k, const void* v, void* out,
                                int out_f32, void* workspace, float scale, hipStream_t stream);
// LCA-style cache (decode.hip): qsum [B*H][d] float32 holds the running sum of the
// current group's queries; a completed group is condensed with their mean.
hipError_t launch_append_decode_lca(const cca_cache_t* c, float* qsum, int d_rope, const void* q, const void* k,
                                    const void* v, void* out, int out_f32, void* workspace, float scale,
                                    hipStream_t stream);
// q [B*c->H*nq][L][d]: nq query heads per cached head; qsum sums over them.
hipError_t launch_qsum_seed(const cca_cache_t* c, const void* q, float* qsum, int64_t L, int nq,
                            hipStream_t stream);

// Log-sum-exp combination of per-chunk decode partials (workspace layout: acc
// [nslices][nchunks][d] floats, then ml [nslices][nchunks][2]) into out [nslices][d].
// With lens non-null, lens[b] (b = slice / slices_per_seq) is then advanced by one
// when it lies in [0, max_len].
hipError_t launch_decode_merge(int d, const float* ws_acc, const float* ws_ml, void* out, int out_mode,
                               int64_t nslices, int nchunks, int32_t* lens, int slices_per_seq, int64_t max_len,
                               hipStream_t stream);

// Serving decode step: one new token per sequence at its own position lens[b]
// (device), H_q = nq * c->H query heads (grouped-query attention), append fused.
int serve_num_chunks(const cca_cache_t* c, int H_q, int64_t max_len);
size_t serve_workspace_bytes(const cca_cache_t* c, int H_q);
// qsum (optional, float32 [B*c->H][d]): the LCA-style cache's running query sums; with it
// a completed group is condensed the LCA way (d_rope positional dims) instead of pooled.
hipError_t launch_serve_append_decode(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q,
                                      const void* q, const void* k, const void* v, void* out, int out_f32,
                                      void* workspace, float scale, hipStream_t stream, float* qsum = nullptr,
                                      int d_rope = 0);

// Backward pass, 16-bit inputs (dt = CCA_BF16 or CCA_F16), head dim 128 (backward.hip);
// BH query slices, nq query heads per
// key/value head.  Workspace: D [BH][L], the log-sum-exp in log2 units [BH][L], then dKc
// and dVc [BH/nq][L/g][d], all float32.
size_t backward_workspace_bytes(int B, int H, int H_kv, int64_t L, int d, int g);
hipError_t launch_backward_d128(int dt, const void* q, const void* k, const void* v, const void* kc, const void* vc,
                                const void* out, const float* lse, const void* dout, float* dq, float* dk, float* dv,
                                void* workspace, int BH, int nq, int64_t L, int g, int k_local, float scale,
                                hipStream_t stream);

// Backward pass for the other shapes (backward_generic.hip): float32 inputs at head dim
// 64 or 128, 16-bit inputs at head dim 64; same arguments, gradients and workspace layout as above,
// out and dout in the input type.
hipError_t launch_backward_generic(int dt, int d, const void* q, const void* k, const void* v, const void* kc,
                                   const void* vc, const void* out, const float* lse, const void* dout, float* dq,
                                   float* dk, float* dv, void* workspace, int BH, int nq, int64_t L, int g,
                                   int k_local, float scale, hipStream_t stream);

// Chunked append of n tokens per sequence (extend.hip); qsum (optional): the LCA-style
// cache's running query sums, as for launch_serve_append_decode.
size_t extend_workspace_bytes(const cca_cache_t* c, int n);
hipError_t launch_extend(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q, int n, const void* q,
                         const void* k, const void* v, void* out, int out_f32, void* workspace, float scale,
                         hipStream_t stream, float* qsum = nullptr,
                         int d_rope = 0);

}  // namespace cca
