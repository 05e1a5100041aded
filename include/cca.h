/*
 * cca.h -- C ABI of libcca.so: Core Context Aware (CCA) attention on MI355X (gfx950).
 *
 * Method source: the page "ICML 2025 | 全局池化+局部保留，CCA-Attention为LLM长文本建模带来突破性进展"
 * (a write-up of "Core Context Aware Transformers for Long Context Language
 * Modeling"), referred to below as [CCA].  Its equations did not survive text
 * extraction, so they are named by what they define.
 *
 * Problem statement, per (batch b, head h) slice, following [CCA]:
 *   Q, K, V : [L, d] per-head queries, keys, values (already projected; any
 *             positional encoding has been applied by the caller).
 *   g       : group size; groups are positions [j*g, (j+1)*g), j < m = floor(L/g).
 *   k_local : number of previous groups kept raw (local window w = k_local*g).
 *   scale   : softmax temperature of both the pooling and the attention
 *             (callers normally pass 1/sqrt(d)).
 *   Pooling ([CCA] global-aware pooling, core-token and core K/V equations):
 *     a_j = softmax_i(scale * Q[j*g+g-1] . K[j*g+i]),
 *     Kc[j] = sum_i a_j,i K[j*g+i],  Vc[j] = sum_i a_j,i V[j*g+i].
 *   Attention ([CCA] locality-preserving module and global-local fusion,
 *   local-window, unified K/V and per-position output equations):
 *     query t, beta = floor(t/g), n_c = max(0, beta - k_local);
 *     keys = Kc[0:n_c] followed by K[n_c*g .. t]; one softmax over all of them;
 *     O[t] = sum of softmax weights times the matching Vc / V rows.
 *
 * Conventions shared by every entry point:
 *   - Device pointers are plain HIP device addresses; the library never
 *     allocates, frees, or keeps them.  The caller owns every buffer.
 *   - Tensors are dense row-major in the stated shapes, element type given by
 *     a cca_dtype_t, base addresses aligned to 16 bytes.
 *   - All device work is enqueued on `stream` (0 = legacy default stream);
 *     no entry point synchronises the host with the device.
 *   - Arguments are validated on the host before anything is enqueued.  On any
 *     non-zero return nothing has been enqueued and no output or descriptor
 *     field has been modified, except CCA_ERR_HIP, which reports a failed
 *     kernel launch (see hipGetLastError); then outputs are undefined.
 *   - A call on an empty sequence (L == 0 in the pooling, prefill, attention
 *     and backward calls) checks its sizes, dtypes and scalars as usual and
 *     then returns CCA_OK without reading, writing or enqueuing anything; its
 *     data pointers are not looked at and may be NULL.
 *   - Calls on one stream are ordered; concurrent calls on different streams
 *     that write the same buffers race (the library has no locks).
 */
#ifndef CCA_H
#define CCA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CCA_OK = 0,
  CCA_ERR_INVALID = -1,     /* null pointer, misaligned pointer, bad size or count */
  CCA_ERR_UNSUPPORTED = -2, /* head dim not 64/128, unknown dtype code, dtype combination not built */
  CCA_ERR_WORKSPACE = -3,   /* workspace smaller than the matching *_workspace_bytes() */
  CCA_ERR_HIP = -4,         /* a kernel launch failed */
  CCA_ERR_CAPACITY = -5     /* the cache has no room for another token */
} cca_status_t;

typedef enum {
  CCA_F32 = 0,  /* IEEE float32 */
  CCA_BF16 = 1, /* bfloat16 (upper half of a float32; conversions round to nearest even) */
  CCA_F16 = 2   /* IEEE binary16 (conversions round to nearest even; overflow gives infinity) */
} cca_dtype_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* cca_status_string(int status);

/*
 * Pooling into core tokens ([CCA] global-aware pooling, core-token and core
 * K/V equations).
 *   q, k, v : device, [B, H, L, d] of dtype dt (only rows j*g+g-1 of q are read).
 *   kc, vc  : device, [B, H, floor(L/g), d] of dtype dt, written.  Math is
 *             float32; results are rounded once to dt.  A trailing partial
 *             group (L mod g tokens) produces no core token.  When
 *             floor(L/g) == 0 they are not touched and may be NULL.
 *   d in {64, 128}; 1 <= g <= 4096; L >= 0 (L < g writes nothing).
 */
int cca_pool_kv(const void* q, const void* k, const void* v, void* kc, void* vc,
                int B, int H, int64_t L, int d, int g, float scale,
                int dt, hipStream_t stream);

/*
 * Prefill: pooling followed by the fused core+local causal attention
 * ([CCA] all three modules; one softmax per query over the unified K/V).
 *   q, k, v : device, [B, H, L, d] of dtype dt.
 *   kc, vc  : device, [B, H, floor(L/g), d] of dtype dt: written by the pooling
 *             step and then read by the attention step (the caller may keep
 *             them, e.g. to seed a decode cache with cca_cache_load_prefill).
 *             May be NULL when floor(L/g) == 0.
 *   out     : device, [B, H, L, d] of dtype out_dt, written.  out_dt is CCA_F32
 *             or equal to dt.  Accumulation is float32; for dt = CCA_BF16 or
 *             CCA_F16 the QK^T and PV products run on matrix cores of that type
 *             with the softmax weights rounded to it, for dt = CCA_F32 on
 *             float32 matrix cores.
 *   k_local >= 0 (any value >= floor((L-1)/g) gives plain causal attention);
 *   L <= INT32_MAX; B*H*ceil(L/128) and B*H*floor(L/g) below INT32_MAX.
 */
int cca_prefill(const void* q, const void* k, const void* v, void* kc, void* vc, void* out,
                int B, int H, int64_t L, int d, int g, int k_local, float scale,
                int dt, int out_dt, hipStream_t stream);

/*
 * The attention step of cca_prefill alone, for callers that already hold the
 * pooled core tokens of the same q, k, v (e.g. from cca_pool_kv).  Same
 * arguments and contract as cca_prefill, except that kc and vc are read only.
 */
int cca_attention(const void* q, const void* k, const void* v, const void* kc, const void* vc, void* out,
                  int B, int H, int64_t L, int d, int g, int k_local, float scale,
                  int dt, int out_dt, hipStream_t stream);

/*
 * Grouped-query attention (GQA): H query heads share H_kv key/value heads,
 * H a multiple of H_kv, r = H / H_kv.  The pages define CCA for one query
 * head per key/value head; with r > 1 this library takes the following
 * reading (with r = 1 the calls below are exactly the ones above):
 *   - query head h reads key/value head h / r (runs of r consecutive heads);
 *   - a group of key/value head h_kv is pooled ONCE, scored by the mean over
 *     its r query heads of the group's last-token query (the importance score
 *     with a mean query of "Latent-Condensed Transformer for Efficient Long
 *     Context Modeling", section 2; its section 3 extends that method to GQA),
 *     so the core tokens, like the raw K/V, exist per key/value head.
 *   q, out : device, [B, H, L, d];  k, v : device, [B, H_kv, L, d];
 *   kc, vc : device, [B, H_kv, floor(L/g), d].
 * Everything else (dtypes, NULL core buffers when floor(L/g) == 0, limits,
 * error behaviour) is as for cca_pool_kv / cca_prefill / cca_attention;
 * H_kv < 1 or H not a multiple of H_kv gives CCA_ERR_INVALID.
 */
int cca_pool_kv_gqa(const void* q, const void* k, const void* v, void* kc, void* vc,
                    int B, int H, int H_kv, int64_t L, int d, int g, float scale,
                    int dt, hipStream_t stream);
int cca_prefill_gqa(const void* q, const void* k, const void* v, void* kc, void* vc, void* out,
                    int B, int H, int H_kv, int64_t L, int d, int g, int k_local, float scale,
                    int dt, int out_dt, hipStream_t stream);
int cca_attention_gqa(const void* q, const void* k, const void* v, const void* kc, const void* vc, void* out,
                      int B, int H, int H_kv, int64_t L, int d, int g, int k_local, float scale,
                      int dt, int out_dt, hipStream_t stream);

/*
 * LCA-style pooling variant ("Latent-Condensed Transformer for Efficient Long
 * Context Modeling", section 2: importance from the mean query of the group,
 * weighted pooling of the content part, positional anchoring of the RoPE part).
 * Per group j: q_bar = mean of Q[j*g .. j*g+g-1]; s_i = scale * q_bar . K[j*g+i];
 * a = softmax(s); the first d - d_rope dims of Kc[j] are sum_i a_i K[j*g+i], its
 * last d_rope dims are those of K[j*g + anchor], anchor = the first i with the
 * largest s_i; Vc[j] = sum_i a_i V[j*g+i].  The last d_rope dims of a key are
 * taken to be its positional (RoPE) part; d_rope = 0 pools every dim.
 *   anchors : optional device int32 [B, H, floor(L/g)], receives each anchor
 *             (position within its group); may be NULL.
 * cca_prefill_lca: this pooling followed by the attention of cca_prefill (the
 * condensed groups in the role of the core tokens; raw local window as in CCA).
 * Other arguments, limits and errors as for cca_pool_kv / cca_prefill;
 * 0 <= d_rope <= d else CCA_ERR_INVALID.
 */
int cca_pool_kv_lca(const void* q, const void* k, const void* v, void* kc, void* vc, int32_t* anchors,
                    int B, int H, int64_t L, int d, int g, int d_rope, float scale,
                    int dt, hipStream_t stream);
int cca_prefill_lca(const void* q, const void* k, const void* v, void* kc, void* vc, void* out, int32_t* anchors,
                    int B, int H, int64_t L, int d, int g, int k_local, int d_rope, float scale,
                    int dt, int out_dt, hipStream_t stream);
/*
 * Grouped-query form: k, v, kc, vc, anchors have H_kv heads; the importance query of a
 * group of key/value head h is the mean over the group's g positions and over the r =
 * H/H_kv query heads h*r .. h*r+r-1 that read it (the mean-over-heads reading of
 * cca_pool_kv_gqa with the LCA page's mean over the group).  cca_pool_kv_lca /
 * cca_prefill_lca are these with H_kv = H.  H % H_kv != 0 gives CCA_ERR_INVALID.
 */
int cca_pool_kv_lca_gqa(const void* q, const void* k, const void* v, void* kc, void* vc, int32_t* anchors,
                        int B, int H, int H_kv, int64_t L, int d, int g, int d_rope, float scale,
                        int dt, hipStream_t stream);
int cca_prefill_lca_gqa(const void* q, const void* k, const void* v, void* kc, void* vc, void* out,
                        int32_t* anchors, int B, int H, int H_kv, int64_t L, int d, int g, int k_local,
                        int d_rope, float scale, int dt, int out_dt, hipStream_t stream);

/*
 * Training ([CCA] Triton section: the fused operator serves training as well;
 * the models are fine-tuned with it).  bf16, binary16 or float32 inputs, d = 64 or 128,
 * one query head per key/value head.  bf16 and binary16 at d = 128 run on the matrix cores;
 * the other combinations run a plain float32 vector path, correct but far slower.
 *
 * cca_prefill_lse: cca_prefill that also writes, for every query t, the
 *   natural-log log-sum-exp of its scaled scores over its visible keys,
 *   lse[t] = log sum_i exp(scale * key_i . Q[t])  (device float32 [B, H, L]),
 *   which the backward pass uses to recompute the softmax weights.
 *
 * cca_backward: gradients of sum(out * dout) with respect to q, k, v, by the
 *   chain rule through the attention softmax and through the pooling softmax
 *   (core token j: Kc = a.K_group, Vc = a.V_group, a = softmax(scale q_hat.K_group),
 *   so the gradients of Kc and Vc reach the group's keys and values and its
 *   scoring query Q[j*g+g-1]).  The forward's rounding of the core tokens to
 *   a 16-bit dt is treated as the identity.
 *   q, k, v, kc, vc, out : the forward's inputs and results, all of type dt
 *           (out_dt of the forward must equal dt);
 *   lse   : device float32 [B, H, L] from cca_prefill_lse;
 *   dout  : device [B, H, L, d] of type dt, the gradient of the output;
 *   dq, dk, dv : device float32 [B, H, L, d], written (every element);
 *   workspace : device, >= cca_backward_workspace_bytes(B, H, L, d, g) bytes.
 *   Limits and errors as for cca_prefill; outside 16-bit inputs at d = 128 also
 *   B*H*(L + L/g + 1) < 2^26 (one 64-lane wave per row and per key).
 */
int cca_prefill_lse(const void* q, const void* k, const void* v, void* kc, void* vc, void* out, float* lse,
                    int B, int H, int64_t L, int d, int g, int k_local, float scale,
                    int dt, int out_dt, hipStream_t stream);
size_t cca_backward_workspace_bytes(int B, int H, int64_t L, int d, int g);
int cca_backward(const void* q, const void* k, const void* v, const void* kc, const void* vc, const void* out,
                 const float* lse, const void* dout, float* dq, float* dk, float* dv, void* workspace,
                 size_t workspace_bytes, int B, int H, int64_t L, int d, int g, int k_local, float scale,
                 int dt, hipStream_t stream);

/*
 * Training with grouped-query attention (readings as for cca_prefill_gqa: the r = H/H_kv
 * query heads h*r .. h*r+r-1 read key/value head h, whose core tokens are pooled once with
 * the mean over those heads of the group's last-token query).  The gradient of that mean
 * reaches each of the r queries with weight 1/r; the key/value gradients sum over the r
 * heads.  k, v, kc, vc, dk, dv have H_kv heads ([B, H_kv, ...]); q, out, lse, dout, dq
 * have H.  cca_prefill_lse / cca_backward are these with H_kv = H.  Errors as for
 * cca_prefill_gqa.
 */
int cca_prefill_lse_gqa(const void* q, const void* k, const void* v, void* kc, void* vc, void* out, float* lse,
                        int B, int H, int H_kv, int64_t L, int d, int g, int k_local, float scale,
                        int dt, int out_dt, hipStream_t stream);
size_t cca_backward_gqa_workspace_bytes(int B, int H, int H_kv, int64_t L, int d, int g);
int cca_backward_gqa(const void* q, const void* k, const void* v, const void* kc, const void* vc, const void* out,
                     const float* lse, const void* dout, float* dq, float* dk, float* dv, void* workspace,
                     size_t workspace_bytes, int B, int H, int H_kv, int64_t L, int d, int g, int k_local,
                     float scale, int dt, hipStream_t stream);

/*
 * Compressed KV cache for decode ([CCA] Triton section: the fused operator
 * serves decode with a KV cache holding core tokens plus local raw tokens;
 * compute/memory efficiency section, Fig. 3).  Plain-old-data descriptor;
 * every device buffer is caller-owned.
 *   core_k, core_v : device, [B, H, max_groups, d]: core token j of every
 *                    completed group j (pooled as soon as the group completes).
 *   ring_k, ring_v : device, [B, H, (k_local+1)*g, d]: raw token u lives in
 *                    slot u mod ((k_local+1)*g); the ring always holds the raw
 *                    window of the newest token.
 *   n_tokens       : tokens appended so far (same for every sequence).
 *   n_pooled       : core tokens written = floor(n_tokens/g).
 * The library updates n_tokens/n_pooled on the host only after it has
 * successfully enqueued the matching device work.
 */
typedef struct {
  void* core_k;
  void* core_v;
  void* ring_k;
  void* ring_v;
  int B, H, d, g, k_local;
  int dt;              /* cca_dtype_t of every cache buffer */
  int64_t max_groups;  /* capacity of core_k/core_v in core tokens */
  int64_t n_tokens;
  int64_t n_pooled;
} cca_cache_t;

/* Ring slots of a cache: (k_local+1)*g. */
int64_t cca_cache_ring_slots(const cca_cache_t* c);

/*
 * Seed an empty cache (n_tokens == 0) with the state after a prefill of L tokens.
 *   k, v   : device, [B, H, L, d] of the cache dtype (the prefill's K and V).
 *   kc, vc : device, [B, H, floor(L/g), d] (the prefill's pooled core tokens).
 * Copies every core token into core_k/core_v and the raw window of token L
 * (positions max(0, floor(L/g)-k_local)*g .. L-1) into its ring slots, then
 * sets n_tokens = L, n_pooled = floor(L/g).  Needs floor(L/g) <= max_groups.
 */
int cca_cache_load_prefill(cca_cache_t* c, const void* k, const void* v,
                           const void* kc, const void* vc, int64_t L, hipStream_t stream);

/*
 * Append one token per sequence: q, k, v are device [B, H, d] of the cache dtype.
 * Writes k, v into ring slot t mod R (t = n_tokens).  When the token completes
 * a group (t+1 divisible by g) that group is pooled in place from the ring
 * with this token's query (the group's last query, [CCA] core-token equation)
 * into core_k/core_v[t/g].  Returns CCA_ERR_CAPACITY when the completed group
 * would not fit in max_groups.
 */
int cca_cache_append(cca_cache_t* c, const void* q, const void* k, const void* v,
                     float scale, hipStream_t stream);

/* Bytes of device workspace cca_decode_step / cca_cache_append_decode need for
 * this cache (depends only on B, H, d and the capacity max_groups + ring
 * slots).  0 for an invalid descriptor. */
size_t cca_decode_workspace_bytes(const cca_cache_t* c);

/*
 * Attention of the newest token against the cache (row n_tokens-1 of the
 * prefill output, [CCA] per-position output equation).
 *   q         : device [B, H, d] of the cache dtype: the query of the token
 *               appended last (call cca_cache_append first).
 *   out       : device [B, H, d] of out_dt (CCA_F32 or the cache dtype).
 *   workspace : device, >= cca_decode_workspace_bytes(c) bytes, 16-byte
 *               aligned: per-chunk partial softmax states; no contents needed
 *               on entry, clobbered on return (concurrent calls sharing a
 *               workspace race).
 * The visible keys of each (b,h) are split into chunks handled by separate
 * workgroups; a second, small kernel merges their partial states.
 * Reads the cache only.  Requires n_tokens >= 1.
 */
int cca_decode_step(const cca_cache_t* c, const void* q, void* out, int out_dt,
                    void* workspace, size_t workspace_bytes, float scale,
                    hipStream_t stream);

/*
 * cca_cache_append followed by cca_decode_step, in one launch: appends the
 * token (q, k, v: device [B, H, d]) exactly as cca_cache_append does (ring slot,
 * in-place pooling of a completed group) and writes its attention output to
 * out.  The new token's key/value are read from k, v for its own attention; a
 * group pooled by this call is not yet visible to this token (it is still in
 * the raw window), so the result equals the two-call sequence.  Same
 * workspace contract as cca_decode_step; same CCA_ERR_CAPACITY rule as
 * cca_cache_append.  Updates n_tokens/n_pooled after a successful launch.
 * (Two kernel launches instead of three.)
 */
int cca_cache_append_decode(cca_cache_t* c, const void* q, const void* k, const void* v,
                            void* out, int out_dt, void* workspace, size_t workspace_bytes,
                            float scale, hipStream_t stream);

/*
 * cca_cache_append_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  It allocates nothing (no hipMalloc, no
 * allocating library call).
 *   The chunk partial states go to a library-owned device array of
 *   CCA_NOALLOC_SCRATCH_BYTES (4 MiB), one copy per GPU, held until the process
 *   ends; its address is looked up on the first call on each device.
 *   stream must belong to the current device (CCA_ERR_INVALID otherwise).
 *   CCA_ERR_WORKSPACE when cca_decode_workspace_bytes(c) exceeds the array
 *   (B*H*chunks*(d+2)*4 bytes: 0.5 MiB for B=8, H=32, d=128).
 *   Calls on one GPU share the array: calls that can overlap on that GPU (on
 *   different streams) race; calls ordered on one stream do not.  No contents are
 *   needed on entry.  Otherwise as cca_cache_append_decode (same kernels, same
 *   results bit for bit).
 */
#define CCA_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int cca_cache_append_decode_noalloc(cca_cache_t* c, const void* q, const void* k, const void* v,
                                    void* out, int out_dt, float scale, hipStream_t stream);

/*
 * LCA-style decode cache ("Latent-Condensed Transformer for Efficient Long Context
 * Modeling", section 2, inference flow: a group is condensed as soon as its last token
 * arrives, with the mean-query importance and positional anchoring of cca_pool_kv_lca;
 * the attention is that of cca_cache_append_decode, over the condensed tokens and the
 * raw ring).  The same cca_cache_t holds the condensed tokens in core_k/core_v.
 *   qsum  : device float32 [B, H, d], caller-owned: the running sum of the queries of
 *           each sequence's current (incomplete) group, in token order.  Zero for an
 *           empty cache; cca_cache_load_prefill_lca sets it from the prefill's last
 *           partial group; the append call adds the new query and, when the group
 *           completes, condenses it with the mean (sum / g) and zeroes the sum.
 *   d_rope: 0 <= d_rope <= d, the positional dims (as for cca_pool_kv_lca).
 * cca_cache_load_prefill_lca: cca_cache_load_prefill (kc, vc from cca_prefill_lca of
 *   the same prefix) plus qsum from q [B, H, L, d].
 * cca_cache_append_decode_lca: as cca_cache_append_decode, with the LCA-style
 *   condensation; workspace as cca_decode_workspace_bytes.  Errors as for those calls.
 */
int cca_cache_load_prefill_lca(cca_cache_t* c, float* qsum, const void* q, const void* k, const void* v,
                               const void* kc, const void* vc, int64_t L, hipStream_t stream);
int cca_cache_append_decode_lca(cca_cache_t* c, float* qsum, int d_rope, const void* q, const void* k,
                                const void* v, void* out, int out_dt, void* workspace,
                                size_t workspace_bytes, float scale, hipStream_t stream);

/*
 * Serving decode step: every sequence of the batch at its own length, and
 * grouped-query attention (see the GQA reading above cca_pool_kv_gqa).  The
 * cache descriptor is the same; its H is the number of key/value heads and its
 * n_tokens / n_pooled fields are neither read (beyond the consistency check of
 * every cache call) nor written: per-sequence lengths live on the device.
 *   lens    : device int32 [B]; lens[b] = tokens already in sequence b's cache,
 *             i.e. the position of the token this call appends.  The call
 *             advances it: after the call (in stream order) lens[b] is one larger
 *             for every sequence whose length was in [0, max_len].
 *   max_len : host value >= every lens[b]; validates capacity
 *             ((max_len+1)/g <= max_groups, else CCA_ERR_CAPACITY) and bounds
 *             the step's K/V bytes (which selects streaming loads); the work
 *             split follows the device-side lengths.  A sequence with lens[b] < 0
 *             or > max_len gets NaN outputs, and its cache and length are left
 *             untouched.
 *   H_q     : query heads, a multiple of c->H.
 *   q       : device [B, H_q, d]: the new token's queries.
 *   k, v    : device [B, c->H, d]: its keys and values.
 *   out     : device [B, H_q, d] of out_dt (CCA_F32 or c->dt).
 *   workspace : device, >= cca_serve_workspace_bytes(c, H_q) bytes.
 * Per sequence this is cca_cache_append followed by the attention of the new
 * token ([CCA] Triton section): the token is written to ring slot lens[b] mod
 * ((k_local+1)*g) and, when it completes a group, that group is pooled into
 * core slot lens[b]/g with the mean of the token's queries over the query heads
 * sharing each key/value head; the token then attends to the core tokens
 * before its raw window and to the window itself, itself included.  One kernel
 * reads every cached key/value row once per key/value head for all the query
 * heads that share it.
 */
size_t cca_serve_workspace_bytes(const cca_cache_t* c, int H_q);
int cca_cache_append_decode_varlen(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q,
                                   const void* q, const void* k, const void* v, void* out, int out_dt,
                                   void* workspace, size_t workspace_bytes, float scale, hipStream_t stream);

/*
 * Serving with the LCA-style condensation ("Latent-Condensed Transformer for
 * Efficient Long Context Modeling", sections 2 and 3: mean-query importance,
 * positional dims from the top-scored token, grouped-query heads):
 * cca_cache_append_decode_varlen, except that the group a token completes is
 * condensed as by cca_pool_kv_lca_gqa.  Its importance query is the mean of the
 * group's g queries over the r = H_q / c->H query heads that share each
 * key/value head.
 *   qsum   : device float32 [B, c->H, d], caller-owned.  Per sequence and
 *            key/value head, it is the running sum of the queries of the current
 *            (incomplete) group, over its tokens and the r query heads.  It is
 *            zero for an empty sequence.  cca_cache_load_prefill_lca_gqa, run on a
 *            one-sequence view of the cache, seeds it for that sequence.  Each
 *            call adds the new token's r queries.  When the token completes the
 *            group, the call condenses the group with sum / (g*r) and zeroes the
 *            sum.  A sequence whose length is out of range is left as is.
 *   d_rope : 0 <= d_rope <= d, as for cca_pool_kv_lca.
 * Other arguments, workspace and errors are as for
 * cca_cache_append_decode_varlen.
 *
 * cca_cache_load_prefill_lca_gqa: cca_cache_load_prefill (kc, vc from
 *   cca_prefill_lca_gqa of the same prefix) plus qsum from q [B, H_q, L, d];
 *   H_q is a multiple of c->H.  cca_cache_load_prefill_lca is this call with
 *   H_q = c->H.
 */
int cca_cache_append_decode_varlen_lca(const cca_cache_t* c, float* qsum, int d_rope, int32_t* lens,
                                       int64_t max_len, int H_q, const void* q, const void* k, const void* v,
                                       void* out, int out_dt, void* workspace, size_t workspace_bytes,
                                       float scale, hipStream_t stream);
int cca_cache_load_prefill_lca_gqa(cca_cache_t* c, float* qsum, int H_q, const void* q, const void* k,
                                   const void* v, const void* kc, const void* vc, int64_t L, hipStream_t stream);

/*
 * Chunked append: n new tokens for every sequence in one call (chunked prefill
 * into an existing cache, several draft tokens, ...), with per-sequence lengths
 * and grouped-query heads as in cca_cache_append_decode_varlen.  Returns the
 * attention output of every new token: the token at position p = lens[b] + i
 * attends to the core tokens before its raw window and to the raw keys
 * (p/g - k_local)*g .. p, i.e. exactly the prefill output of row p ([CCA]
 * locality-preserving module and global-local fusion; a token's output depends
 * only on the tokens before it).  Afterwards the chunk is in the cache: its
 * keys/values in their ring slots, every group it completes pooled into its core
 * slot (mean query over the query heads sharing each key/value head), and
 * lens[b] advanced by n.
 *   n       : 1 <= n <= k_local*g + 1 (then no token of the chunk can see a core
 *             token pooled from the same chunk); longer chunks are split by the
 *             caller into consecutive calls.  CCA_ERR_INVALID otherwise.  A chunk
 *             may complete at most 131068 groups (n/g + 1 <= 131068, i.e. k_local
 *             below about 131K); CCA_ERR_UNSUPPORTED above.
 *   lens, max_len, H_q : as for cca_cache_append_decode_varlen; capacity needs
 *             (max_len + n)/g <= max_groups (else CCA_ERR_CAPACITY).  A sequence
 *             with lens[b] outside [0, max_len] gets NaN outputs and is left as is.
 *   q       : device [B, H_q, n, d];  k, v : device [B, c->H, n, d];
 *   out     : device [B, H_q, n, d] of out_dt (CCA_F32 or c->dt).
 *   workspace : device, >= cca_extend_workspace_bytes(c, n) bytes (start
 *             positions and the sequences ordered by length, longest first,
 *             for the work order of the attention, plus a staging copy of the
 *             raw window of every key/value head: about
 *             2*B*H*((k_local+1)*g + n)*d elements).
 * The attention runs on the same MFMA kernels as cca_attention.
 */
size_t cca_extend_workspace_bytes(const cca_cache_t* c, int n);
int cca_cache_extend(const cca_cache_t* c, int32_t* lens, int64_t max_len, int H_q, int n,
                     const void* q, const void* k, const void* v, void* out, int out_dt,
                     void* workspace, size_t workspace_bytes, float scale, hipStream_t stream);

/*
 * Chunked append for the LCA-style serving cache: cca_cache_extend, except that every
 * group the chunk completes is condensed as by cca_cache_append_decode_varlen_lca.  The
 * mean query covers the group's tokens and the r query heads.  Queries of its tokens
 * before the chunk come from qsum; the others come from q.  Afterwards qsum holds,
 * per sequence and key/value head, the sum of the queries of the trailing incomplete
 * group.  qsum and d_rope are as for cca_cache_append_decode_varlen_lca.  Everything
 * else is as for cca_cache_extend.
 */
int cca_cache_extend_lca(const cca_cache_t* c, float* qsum, int d_rope, int32_t* lens, int64_t max_len,
                         int H_q, int n, const void* q, const void* k, const void* v, void* out, int out_dt,
                         void* workspace, size_t workspace_bytes, float scale, hipStream_t stream);

/*
 * KV-cache accounting ([CCA] compute/memory efficiency, Fig. 3: the cache
 * holds core plus local tokens instead of every token).  Host-only integer
 * arithmetic, no device work.  After n_tokens tokens with group size g and
 * k_local raw groups:
 *   *resident_bytes = B*H*2*d*elem * (floor(n_tokens/g) + (k_local+1)*g)
 *   *full_bytes     = B*H*2*d*elem * n_tokens            (standard KV cache)
 * elem = 2 for CCA_BF16 and CCA_F16, 4 for CCA_F32; any other dt gives
 * CCA_ERR_UNSUPPORTED.  Either output pointer may be NULL.
 */
int cca_kv_cache_bytes(int64_t n_tokens, int g, int k_local, int B, int H, int d, int dt,
                       int64_t* resident_bytes, int64_t* full_bytes);

#ifdef __cplusplus
}
#endif

#endif /* CCA_H */
