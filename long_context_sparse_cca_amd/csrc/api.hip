// C ABI of libcca.so: host-side validation, then stream-ordered kernel launches.
// Every declaration, with its argument contract, is in include/cca.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "cca_internal.h"

namespace {

constexpr int kMaxGroup = 4096;  // pooling keeps one float score per group row in LDS

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

int check_shape(int B, int H, int64_t L, int d, int g, int dt) {
  if (dt != CCA_F32 && dt != CCA_BF16 && dt != CCA_F16) return CCA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return CCA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || L < 0 || g < 1 || g > kMaxGroup) return CCA_ERR_INVALID;
  if ((int64_t)B * H > (int64_t)1 << 24) return CCA_ERR_INVALID;
  return CCA_OK;
}

int check_cache(const cca_cache_t* c) {
  if (c == nullptr) return CCA_ERR_INVALID;
  int s = check_shape(c->B, c->H, 0, c->d, c->g, c->dt);
  if (s != CCA_OK) return s;
  if (!aligned16(c->core_k) || !aligned16(c->core_v) || !aligned16(c->ring_k) || !aligned16(c->ring_v))
    return CCA_ERR_INVALID;
  if (c->k_local < 0 || c->max_groups < 1 || c->n_tokens < 0) return CCA_ERR_INVALID;
  if ((int64_t)(c->k_local + 1) * c->g > ((int64_t)1 << 30)) return CCA_ERR_INVALID;
  if (c->n_pooled != c->n_tokens / c->g) return CCA_ERR_INVALID;
  if (c->n_pooled > c->max_groups) return CCA_ERR_INVALID;
  return CCA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CCA_OK : CCA_ERR_HIP; }

}  // namespace

extern "C" {

const char* cca_status_string(int status) {
  switch (status) {
    case CCA_OK: return "ok";
    case CCA_ERR_INVALID: return "invalid argument";
    case CCA_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
    case CCA_ERR_WORKSPACE: return "workspace too small";
    case CCA_ERR_HIP: return "HIP kernel launch failed";
    case CCA_ERR_CAPACITY: return "cache capacity exceeded";
    default: return "unknown status";
  }
}

int cca_pool_kv_gqa(const void* q, const void* k, const void* v, void* kc, void* vc, int B, int H, int H_kv,
                    int64_t L, int d, int g, float scale, int dt, hipStream_t stream) {
  int s = check_shape(B, H, L, d, g, dt);
  if (s != CCA_OK) return s;
  if (H_kv < 1 || H % H_kv != 0) return CCA_ERR_INVALID;
  if (!isfinite(scale)) return CCA_ERR_INVALID;
  if (L == 0) return CCA_OK;   // nothing is read or written: the data pointers may be NULL
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return CCA_ERR_INVALID;
  if (L / g > 0 && (!aligned16(kc) || !aligned16(vc))) return CCA_ERR_INVALID;
  const int64_t BH = (int64_t)B * H;
  if (BH * (L / g) >= INT32_MAX || BH * L >= ((int64_t)1 << 40)) return CCA_ERR_INVALID;
  return hip_status(cca::launch_pool(dt, d, q, k, v, kc, vc, B * H_kv, L, g, H / H_kv, scale, stream));
}

int cca_pool_kv(const void* q, const void* k, const void* v, void* kc, void* vc, int B, int H, int64_t L, int d,
                int g, float scale, int dt, hipStream_t stream) {
  return cca_pool_kv_gqa(q, k, v, kc, vc, B, H, H, L, d, g, scale, dt, stream);
}

namespace {

int check_prefill(const void* q, const void* k, const void* v, const void* kc, const void* vc, const void* out, int B,
                  int H, int H_kv, int64_t L, int d, int g, int k_local, float scale, int dt, int out_dt) {
  int s = check_shape(B, H, L, d, g, dt);
  if (s != CCA_OK) return s;
  if (H_kv < 1 || H % H_kv != 0) return CCA_ERR_INVALID;
  if (out_dt != CCA_F32 && out_dt != dt) return CCA_ERR_UNSUPPORTED;
  if (k_local < 0 || !isfinite(scale)) return CCA_ERR_INVALID;
  if (L == 0) return CCA_OK;   // nothing is read or written: the data pointers may be NULL
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return CCA_ERR_INVALID;
  if (L / g > 0 && (!aligned16(kc) || !aligned16(vc))) return CCA_ERR_INVALID;
  const int64_t BH = (int64_t)B * H;
  if (L > INT32_MAX || BH * (L / g) >= INT32_MAX || BH * ((L + 127) / 128) >= INT32_MAX) return CCA_ERR_INVALID;
  return CCA_OK;
}

}  // namespace

int cca_prefill_gqa(const void* q, const void* k, const void* v, void* kc, void* vc, void* out, int B, int H,
                    int H_kv, int64_t L, int d, int g, int k_local, float scale, int dt, int out_dt,
                    hipStream_t stream) {
  int s = check_prefill(q, k, v, kc, vc, out, B, H, H_kv, L, d, g, k_local, scale, dt, out_dt);
  if (s != CCA_OK || L == 0) return s;
  const int nq = H / H_kv;
  hipError_t e = cca::launch_pool(dt, d, q, k, v, kc, vc, B * H_kv, L, g, nq, scale, stream);
  if (e != hipSuccess) return CCA_ERR_HIP;
  e = cca::launch_prefill_attention(dt, d, q, k, v, kc, vc, out, out_dt == CCA_F32, B * H, nq, L, g, k_local, scale,
                                    stream);
  return hip_status(e);
}

int cca_prefill(const void* q, const void* k, const void* v, void* kc, void* vc, void* out, int B, int H, int64_t L,
                int d, int g, int k_local, float scale, int dt, int out_dt, hipStream_t stream) {
  return cca_prefill_gqa(q, k, v, kc, vc, out, B, H, H, L, d, g, k_local, scale, dt, out_dt, stream);
}

int cca_attention_gqa(const void* q, const void* k, const void* v, const void* kc, const void* vc, void* out, int B,
                      int H, int H_kv, int64_t L, int d, int g, int k_local, float scale, int dt, int out_dt,
                      hipStream_t stream) {
  int s = check_prefill(q, k, v, kc, vc, out, B, H, H_kv, L, d, g, k_local, scale, dt, out_dt);
  if (s != CCA_OK || L == 0) return s;
  return hip_status(cca::launch_prefill_attention(dt, d, q, k, v, kc, vc, out, out_dt == CCA_F32, B * H, H / H_kv,
                                                  L, g, k_local, scale, stream));
}

int cca_attention(const void* q, const void* k, const void* v, const void* kc, const void* vc, void* out, int B, int H,
                  int64_t L, int d, int g, int k_local, float scale, int dt, int out_dt, hipStream_t stream) {
  return cca_attention_gqa(q, k, v, kc, vc, out, B, H, H, L, d, g, k_local, scale, dt, out_dt, stream);
}

int cca_prefill_lse_gqa(const void* q, const void* k, const void* v, void* kc, void* vc, void* out, float* lse,
                        int B, int H, int H_kv, int64_t L, int d, int g, int k_local, float scale, int dt,
                        int out_dt, hipStream_t stream) {
  int s = check_prefill(q, k, v, kc, vc, out, B, H, H_kv, L, d, g, k_local, scale, dt, out_dt);
  if (s != CCA_OK) return s;
  if (L > 0 && (lse == nullptr || ((uintptr_t)lse & 3u) != 0)) return CCA_ERR_INVALID;
  if (L == 0) return CCA_OK;
  const int nq = H / H_kv;
  hipError_t e = cca::launch_pool(dt, d, q, k, v, kc, vc, B * H_kv, L, g, nq, scale, stream);
  if (e != hipSuccess) return CCA_ERR_HIP;
  return hip_status(cca::launch_prefill_attention(dt, d, q, k, v, kc, vc, out, out_dt == CCA_F32, B * H, nq, L, g,
                                                  k_local, scale, stream, lse));
}

int cca_prefill_lse(const void* q, const void* k, const void* v, void* kc, void* vc, void* out, float* lse, int B,
                    int H, int64_t L, int d, int g, int k_local, float scale, int dt, int out_dt, hipStream_t stream) {
  return cca_prefill_lse_gqa(q, k, v, kc, vc, out, lse, B, H, H, L, d, g, k_local, scale, dt, out_dt, stream);
}

size_t cca_backward_gqa_workspace_bytes(int B, int H, int H_kv, int64_t L, int d, int g) {
  if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0 || L < 0 || g < 1 || (d != 64 && d != 128)) return 0;
  return cca::backward_workspace_bytes(B, H, H_kv, L, d, g);
}

size_t cca_backward_workspace_bytes(int B, int H, int64_t L, int d, int g) {
  return cca_backward_gqa_workspace_bytes(B, H, H, L, d, g);
}

int cca_backward_gqa(const void* q, const void* k, const void* v, const void* kc, const void* vc, const void* out,
                     const float* lse, const void* dout, float* dq, float* dk, float* dv, void* workspace,
                     size_t workspace_bytes, int B, int H, int H_kv, int64_t L, int d, int g, int k_local,
                     float scale, int dt, hipStream_t stream) {
  int s = check_prefill(q, k, v, kc, vc, out, B, H, H_kv, L, d, g, k_local, scale, dt, dt);
  if (s != CCA_OK) return s;
  if (L == 0) return CCA_OK;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
      lse == nullptr || ((uintptr_t)lse & 3u) != 0)
    return CCA_ERR_INVALID;
  const bool fast = dt != CCA_F32 && d == 128;
  if (fast && (int64_t)B * H * ((L + 127) / 128 + L / g / 128 + 1) >= INT32_MAX) return CCA_ERR_INVALID;
  // the other shapes launch one 64-lane wave per query row and per key
  if (!fast && (int64_t)B * H * (L + L / g + 1) * 64 >= (int64_t)UINT32_MAX) return CCA_ERR_INVALID;
  if (workspace_bytes < cca_backward_gqa_workspace_bytes(B, H, H_kv, L, d, g)) return CCA_ERR_WORKSPACE;
  if (fast)
    return hip_status(cca::launch_backward_d128(dt, q, k, v, kc, vc, out, lse, dout, dq, dk, dv, workspace, B * H,
                                                H / H_kv, L, g, k_local, scale, stream));
  return hip_status(cca::launch_backward_generic(dt, d, q, k, v, kc, vc, out, lse, dout, dq, dk, dv, workspace,
                                                 B * H, H / H_kv, L, g, k_local, scale, stream));
}

int cca_backward(const void* q, const void* k, const void* v, const void* kc, const void* vc, const void* out,
                 const float* lse, const void* dout, float* dq, float* dk, float* dv, void* workspace,
                 size_t workspace_bytes, int B, int H, int64_t L, int d, int g, int k_local, float scale, int dt,
                 hipStream_t stream) {
  return cca_backward_gqa(q, k, v, kc, vc, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, H, L, d, g,
                          k_local, scale, dt, stream);
}

int cca_pool_kv_lca_gqa(const void* q, const void* k, const void* v, void* kc, void* vc, int32_t* anchors, int B,
                        int H, int H_kv, int64_t L, int d, int g, int d_rope, float scale, int dt,
                        hipStream_t stream) {
  int s = check_shape(B, H, L, d, g, dt);
  if (s != CCA_OK) return s;
  if (H_kv < 1 || H % H_kv != 0) return CCA_ERR_INVALID;
  if (d_rope < 0 || d_rope > d) return CCA_ERR_INVALID;
  if (!isfinite(scale)) return CCA_ERR_INVALID;
  if (L == 0) return CCA_OK;   // nothing is read or written: the data pointers may be NULL
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return CCA_ERR_INVALID;
  if (L / g > 0 && (!aligned16(kc) || !aligned16(vc))) return CCA_ERR_INVALID;
  if (anchors != nullptr && ((uintptr_t)anchors & 3u) != 0) return CCA_ERR_INVALID;
  const int64_t BHkv = (int64_t)B * H_kv;
  if (BHkv * (L / g) >= INT32_MAX) return CCA_ERR_INVALID;
  return hip_status(cca::launch_pool_lca(dt, d, q, k, v, kc, vc, anchors, (int)BHkv, L, g, H / H_kv, d_rope, scale,
                                         stream));
}

int cca_pool_kv_lca(const void* q, const void* k, const void* v, void* kc, void* vc, int32_t* anchors, int B, int H,
                    int64_t L, int d, int g, int d_rope, float scale, int dt, hipStream_t stream) {
  return cca_pool_kv_lca_gqa(q, k, v, kc, vc, anchors, B, H, H, L, d, g, d_rope, scale, dt, stream);
}

int cca_prefill_lca_gqa(const void* q, const void* k, const void* v, void* kc, void* vc, void* out,
                        int32_t* anchors, int B, int H, int H_kv, int64_t L, int d, int g, int k_local, int d_rope,
                        float scale, int dt, int out_dt, hipStream_t stream) {
  int s = check_prefill(q, k, v, kc, vc, out, B, H, H_kv, L, d, g, k_local, scale, dt, out_dt);
  if (s != CCA_OK) return s;
  if (d_rope < 0 || d_rope > d) return CCA_ERR_INVALID;
  if (L == 0) return CCA_OK;
  s = cca_pool_kv_lca_gqa(q, k, v, kc, vc, anchors, B, H, H_kv, L, d, g, d_rope, scale, dt, stream);
  if (s != CCA_OK) return s;
  return hip_status(cca::launch_prefill_attention(dt, d, q, k, v, kc, vc, out, out_dt == CCA_F32, B * H, H / H_kv, L,
                                                  g, k_local, scale, stream));
}

int cca_prefill_lca(const void* q, const void* k, const void* v, void* kc, void* vc, void* out, int32_t* anchors,
                    int B, int H, int64_t L, int d, int g, int k_local, int d_rope, float scale, int dt, int out_dt,
                    hipStream_t stream) {
  return cca_prefill_lca_gqa(q, k, v, kc, vc, out, anchors, B, H, H, L, d, g, k_local, d_rope, scale, dt, out_dt,
                             stream);
}

int64_t cca_cache_ring_slots(const cca_cache_t* c) {
  if (c == nullptr) return 0;
  return (int64_t)(c->k_local + 1) * c->g;
}

int cca_cache_load_prefill(cca_cache_t* c, const void* k, const void* v, const void* kc, const void* vc, int64_t L,
                           hipStream_t stream) {
  int s = check_cache(c);
  if (s != CCA_OK) return s;
  if (c->n_tokens != 0 || L < 1) return CCA_ERR_INVALID;
  if (!aligned16(k) || !aligned16(v)) return CCA_ERR_INVALID;
  const int64_t m = L / c->g;
  if (m > 0 && (!aligned16(kc) || !aligned16(vc))) return CCA_ERR_INVALID;
  if (m > c->max_groups) return CCA_ERR_CAPACITY;
  hipError_t e = cca::launch_cache_load(c, k, v, kc, vc, L, stream);
  if (e != hipSuccess) return CCA_ERR_HIP;
  c->n_tokens = L;
  c->n_pooled = m;
  return CCA_OK;
}

int cca_cache_append(cca_cache_t* c, const void* q, const void* k, const void* v, float scale, hipStream_t stream) {
  int s = check_cache(c);
  if (s != CCA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !isfinite(scale)) return CCA_ERR_INVALID;
  const int64_t t = c->n_tokens;
  if ((t + 1) / c->g > c->max_groups) return CCA_ERR_CAPACITY;
  hipError_t e = cca::launch_cache_append(c, q, k, v, scale, stream);
  if (e != hipSuccess) return CCA_ERR_HIP;
  c->n_tokens = t + 1;
  c->n_pooled = (t + 1) / c->g;
  return CCA_OK;
}

size_t cca_decode_workspace_bytes(const cca_cache_t* c) {
  if (c == nullptr || c->B < 1 || c->H < 1 || (c->d != 64 && c->d != 128) || c->g < 1 || c->k_local < 0 ||
      c->max_groups < 1)
    return 0;
  return cca::decode_workspace_bytes(c);
}

int cca_decode_step(const cca_cache_t* c, const void* q, void* out, int out_dt, void* workspace,
                    size_t workspace_bytes, float scale, hipStream_t stream) {
  int s = check_cache(c);
  if (s != CCA_OK) return s;
  if (out_dt != CCA_F32 && out_dt != c->dt) return CCA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace) || !isfinite(scale)) return CCA_ERR_INVALID;
  if (c->n_tokens < 1) return CCA_ERR_INVALID;
  if (workspace_bytes < cca_decode_workspace_bytes(c)) return CCA_ERR_WORKSPACE;
  return hip_status(cca::launch_decode(c, q, out, out_dt == CCA_F32, workspace, scale, stream));
}

int cca_cache_append_decode(cca_cache_t* c, const void* q, const void* k, const void* v, void* out, int out_dt,
                            void* workspace, size_t workspace_bytes, float scale, hipStream_t stream) {
  int s = check_cache(c);
  if (s != CCA_OK) return s;
  if (out_dt != CCA_F32 && out_dt != c->dt) return CCA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace) ||
      !isfinite(scale))
    return CCA_ERR_INVALID;
  const int64_t t = c->n_tokens;
  if ((t + 1) / c->g > c->max_groups) return CCA_ERR_CAPACITY;
  if (workspace_bytes < cca_decode_workspace_bytes(c)) return CCA_ERR_WORKSPACE;
  hipError_t e = cca::launch_append_decode(c, q, k, v, out, out_dt == CCA_F32, workspace, scale, stream);
  if (e != hipSuccess) return CCA_ERR_HIP;
  c->n_tokens = t + 1;
  c->n_pooled = (t + 1) / c->g;
  return CCA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// allocation-free fused decode: the chunk partial states live in a library-owned
// device array instead of a caller workspace
// ---------------------------------------------------------------------------
namespace {

constexpr int kMaxDevices = 64;
// One copy per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in: kernels get the device address from hipGetSymbolAddress.
__device__ __align__(256) float scratch[CCA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

std::mutex scratch_mu;
void* scratch_addr[kMaxDevices];

// Device address of `scratch` on the device of `stream` (which must be the current
// device), looked up once per device with that device current.
int scratch_for_stream(hipStream_t stream, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return CCA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return CCA_ERR_UNSUPPORTED;
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return CCA_ERR_HIP;
    if (sdev != dev) return CCA_ERR_INVALID;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CCA_ERR_HIP;
    scratch_addr[dev] = p;
  }
  *ptr = scratch_addr[dev];
  return CCA_OK;
}

}  // namespace

extern "C" {

int cca_cache_append_decode_noalloc(cca_cache_t* c, const void* q, const void* k, const void* v, void* out,
                                    int out_dt, float scale, hipStream_t stream) {
  int s = check_cache(c);
  if (s != CCA_OK) return s;
  const size_t need = cca_decode_workspace_bytes(c);
  if (need > (size_t)CCA_NOALLOC_SCRATCH_BYTES) return CCA_ERR_WORKSPACE;
  void* ws = nullptr;
  s = scratch_for_stream(stream, &ws);
  if (s != CCA_OK) return s;
  // every chunk record is written before the merge reads it: nothing to clear
  return cca_cache_append_decode(c, q, k, v, out, out_dt, ws, need, scale, stream);
}

int cca_cache_load_prefill_lca_gqa(cca_cache_t* c, float* qsum, int H_q, const void* q, const void* k,
                                   const void* v, const void* kc, const void* vc, int64_t L, hipStream_t stream) {
  int s = check_cache(c);
  if (s != CCA_OK) return s;
  if (qsum == nullptr || !aligned16(qsum) || !aligned16(q)) return CCA_ERR_INVALID;
  if (H_q < 1 || H_q % c->H != 0) return CCA_ERR_INVALID;
  // validate as cca_cache_load_prefill does before enqueueing anything, so that the
  // descriptor changes only once all of the seeding is enqueued
  if (c->n_tokens != 0 || L < 1 || !aligned16(k) || !aligned16(v)) return CCA_ERR_INVALID;
  const int64_t m = L / c->g;
  if (m > 0 && (!aligned16(kc) || !aligned16(vc))) return CCA_ERR_INVALID;
  if (m > c->max_groups) return CCA_ERR_CAPACITY;
  if (cca::launch_qsum_seed(c, q, qsum, L, H_q / c->H, stream) != hipSuccess) return CCA_ERR_HIP;
  return cca_cache_load_prefill(c, k, v, kc, vc, L, stream);
}

int cca_cache_load_prefill_lca(cca_cache_t* c, float* qsum, const void* q, const void* k, const void* v,
                               const void* kc, const void* vc, int64_t L, hipStream_t stream) {
  if (c == nullptr) return CCA_ERR_INVALID;
  return cca_cache_load_prefill_lca_gqa(c, qsum, c->H, q, k, v, kc, vc, L, stream);
}

int cca_cache_append_decode_lca(cca_cache_t* c, float* qsum, int d_rope, const void* q, const void* k, const void* v,
                                void* out, int out_dt, void* workspace, size_t workspace_bytes, float scale,
                                hipStream_t stream) {
  int s = check_cache(c);
  if (s != CCA_OK) return s;
  if (out_dt != CCA_F32 && out_dt != c->dt) return CCA_ERR_UNSUPPORTED;
  if (d_rope < 0 || d_rope > c->d) return CCA_ERR_INVALID;
  if (qsum == nullptr || !aligned16(qsum) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(workspace) || !isfinite(scale))
    return CCA_ERR_INVALID;
  const int64_t t = c->n_tokens;
  if ((t + 1) / c->g > c->max_groups) return CCA_ERR_CAPACITY;
  if (workspace_bytes < cca_decode_workspace_bytes(c)) return CCA_ERR_WORKSPACE;
  hipError_t e = cca::launch_append_decode_lca(c, qsum, d_rope, q, k, v, out, out_dt == CCA_F32, workspace, scale,
                                               stream);
  if (e != hipSuccess) return CCA_ERR_HIP;
  c->n_tokens = t + 1;
  c->n_pooled = (t + 1) / c->g;
  return CCA_OK;
}

size_t cca_serve_workspace_bytes(const cca_cache_t* c, int H_q) {
  if (c == nullptr || c->B < 1 || c->H < 1 || (c->d != 64 && c->d != 128) || c->g < 1 || c->k_local < 0 ||
      c->max_groups < 1 || H_q < 1 || H_q % c->H != 0)
    return 0;
  return cca::serve_workspace_bytes(c, H_q);
}

static int append_decode_varlen(const cca_cache_t* c, float* qsum, int d_rope, int32_t* lens, int64_t max_len,
                                int H_q, const void* q, const void* k, const void* v, void* out, int out_dt,
                                void* workspace, size_t workspace_bytes, float scale, hipStream_t stream) {
  int s = check_cache(c);
  if (s != CCA_OK) return s;
  if (out_dt != CCA_F32 && out_dt != c->dt) return CCA_ERR_UNSUPPORTED;
  if (H_q < 1 || H_q % c->H != 0 || (int64_t)c->B * H_q > ((int64_t)1 << 24)) return CCA_ERR_INVALID;
  if (lens == nullptr || ((uintptr_t)lens & 3u) != 0 || max_len < 0 || max_len >= INT32_MAX) return CCA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace) ||
      !isfinite(scale))
    return CCA_ERR_INVALID;
  if ((max_len + 1) / c->g > c->max_groups) return CCA_ERR_CAPACITY;
  if (workspace_bytes < cca_serve_workspace_bytes(c, H_q)) return CCA_ERR_WORKSPACE;
  return hip_status(cca::launch_serve_append_decode(c, lens, max_len, H_q, q, k, v, out, out_dt == CCA_F32,
                                                    workspace, scale, stream, qsum, d_rope));
}

int cca_cache_append_decode_varlen(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q,
                                   const void* q, const void* k, const void* v, void* out, int out_dt,
                                   void* workspace, size_t workspace_bytes, float scale, hipStream_t stream) {
  return append_decode_varlen(c, nullptr, 0, lens, max_len, H_q, q, k, v, out, out_dt, workspace, workspace_bytes,
                              scale, stream);
}

int cca_cache_append_decode_varlen_lca(const cca_cache_t* c, float* qsum, int d_rope, int32_t* lens,
                                       int64_t max_len, int H_q, const void* q, const void* k, const void* v,
                                       void* out, int out_dt, void* workspace, size_t workspace_bytes, float scale,
                                       hipStream_t stream) {
  if (c == nullptr || qsum == nullptr || !aligned16(qsum) || d_rope < 0 || d_rope > c->d) return CCA_ERR_INVALID;
  return append_decode_varlen(c, qsum, d_rope, lens, max_len, H_q, q, k, v, out, out_dt, workspace, workspace_bytes,
                              scale, stream);
}

size_t cca_extend_workspace_bytes(const cca_cache_t* c, int n) {
  if (c == nullptr || c->B < 1 || c->H < 1 || (c->d != 64 && c->d != 128) || c->g < 1 || c->k_local < 0 ||
      c->max_groups < 1 || n < 1)
    return 0;
  return cca::extend_workspace_bytes(c, n);
}

static int cache_extend(const cca_cache_t* c, float* qsum, int d_rope, int32_t* lens, int64_t max_len, int H_q, int n,
                        const void* q, const void* k, const void* v, void* out, int out_dt, void* workspace,
                        size_t workspace_bytes, float scale, hipStream_t stream) {
  int s = check_cache(c);
  if (s != CCA_OK) return s;
  if (out_dt != CCA_F32 && out_dt != c->dt) return CCA_ERR_UNSUPPORTED;
  if (H_q < 1 || H_q % c->H != 0 || (int64_t)c->B * H_q > ((int64_t)1 << 24)) return CCA_ERR_INVALID;
  if (n < 1 || (int64_t)n > (int64_t)c->k_local * c->g + 1) return CCA_ERR_INVALID;
  if ((int64_t)n / c->g + 1 > cca::kExtendMaxGroupWaves) return CCA_ERR_UNSUPPORTED;
  if (lens == nullptr || ((uintptr_t)lens & 3u) != 0 || max_len < 0 || max_len + n >= INT32_MAX)
    return CCA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace) ||
      !isfinite(scale))
    return CCA_ERR_INVALID;
  if ((max_len + n) / c->g > c->max_groups) return CCA_ERR_CAPACITY;
  if ((int64_t)c->B * H_q * ((n + 127) / 128) >= INT32_MAX) return CCA_ERR_INVALID;
  if (workspace_bytes < cca_extend_workspace_bytes(c, n)) return CCA_ERR_WORKSPACE;
  return hip_status(cca::launch_extend(c, lens, max_len, H_q, n, q, k, v, out, out_dt == CCA_F32, workspace, scale,
                                       stream, qsum, d_rope));
}

int cca_cache_extend(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q, int n, const void* q,
                     const void* k, const void* v, void* out, int out_dt, void* workspace, size_t workspace_bytes,
                     float scale, hipStream_t stream) {
  return cache_extend(c, nullptr, 0, lens, max_len, H_q, n, q, k, v, out, out_dt, workspace, workspace_bytes, scale,
                      stream);
}

int cca_cache_extend_lca(const cca_cache_t* c, float* qsum, int d_rope, int32_t* lens, int64_t max_len, int H_q,
                         int n, const void* q, const void* k, const void* v, void* out, int out_dt, void* workspace,
                         size_t workspace_bytes, float scale, hipStream_t stream) {
  if (c == nullptr || qsum == nullptr || !aligned16(qsum) || d_rope < 0 || d_rope > c->d) return CCA_ERR_INVALID;
  return cache_extend(c, qsum, d_rope, lens, max_len, H_q, n, q, k, v, out, out_dt, workspace, workspace_bytes, scale,
                      stream);
}

int cca_kv_cache_bytes(int64_t n_tokens, int g, int k_local, int B, int H, int d, int dt, int64_t* resident_bytes,
                       int64_t* full_bytes) {
  if (n_tokens < 0 || g < 1 || k_local < 0 || B < 1 || H < 1 || d < 1) return CCA_ERR_INVALID;
  if (dt != CCA_F32 && dt != CCA_BF16 && dt != CCA_F16) return CCA_ERR_UNSUPPORTED;
  const int64_t per_token = (int64_t)B * H * 2 * d * cca::dtype_bytes(dt);
  if (resident_bytes) *resident_bytes = per_token * (n_tokens / g + (int64_t)(k_local + 1) * g);
  if (full_bytes) *full_bytes = per_token * n_tokens;
  return CCA_OK;
}

}  // extern "C"
