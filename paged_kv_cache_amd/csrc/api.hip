// api.hip -- the extern "C" entry points declared in include/pagedattn.h.
// Host-side argument checks, then one or two kernel launches on the caller's
// stream.  Nothing here allocates or synchronises.

#include <hip/hip_runtime.h>

#include "kernels.h"
#include "pagedattn.h"

namespace pa {

int device_cu_count() {
  static int count[64];   // per device; written once with the same value by any thread
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (count[dev] <= 0) {
    hipDeviceProp_t prop;
    count[dev] = (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
                     ? prop.multiProcessorCount
                     : 256;
  }
  return count[dev];
}

}  // namespace pa

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_head_dim(int d) { return d == 64 || d == 128; }

// The kernels fold the scale into the exponent (exp2(s*scale*log2e - m)) and
// mask keys with -inf scores, which only works for a finite positive scale.
bool valid_scale(float s) { return s > 0.f && s <= 3.402823466e38f; }

// Common checks of the paged-cache description.
int check_cache(const void *kv_cache, int64_t n_pages, const int32_t *block_table, int n_slots,
                int n_layers, int mbps, int layer, int n_kv_heads, int head_dim) {
  if (!kv_cache || !block_table) return PA_ERR_NULL;
  if (n_pages <= 0 || n_slots <= 0 || n_layers <= 0 || mbps <= 0 || n_kv_heads <= 0 ||
      head_dim <= 0)
    return PA_ERR_SHAPE;
  if (layer < 0 || layer >= n_layers) return PA_ERR_SHAPE;
  if (!aligned16(kv_cache)) return PA_ERR_ALIGN;
  const int64_t page = pa_page_bytes(n_kv_heads, head_dim);
  if (n_pages > INT64_MAX / page) return PA_ERR_RANGE;
  if (n_pages > 0x7fffffffLL) return PA_ERR_RANGE;                      // int32 page ids
  if ((int64_t)n_slots * n_layers * mbps > 0x7fffffffLL) return PA_ERR_RANGE;
  if ((int64_t)mbps * 16 > 0x7fffffffLL) return PA_ERR_RANGE;
  return PA_OK;
}

// Shared checks and launch of attn_prefill / attn_prefill_chunk.
int prefill_common(const void *q, const void *kv_cache, int64_t n_pages, const int32_t *block_table,
                   int n_slots, int n_layers, int max_blocks_per_seq, int layer,
                   const int32_t *slot_ids, const int32_t *seq_lens, const int32_t *q_lens, int B,
                   int T, int Hq, int Hkv, int head_dim, float scale, int causal, void *O,
                   float *LSE, int32_t *err, void *stream) {
  if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return PA_ERR_SHAPE;
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (!valid_scale(scale)) return PA_ERR_VALUE;
  int rc = check_cache(kv_cache, n_pages, block_table, n_slots, n_layers, max_blocks_per_seq, layer,
                       Hkv, head_dim);
  if (rc != PA_OK) return rc;
  if (B == 0 || T == 0) return PA_OK;
  if (!q || !seq_lens || !O || !LSE) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(O)) return PA_ERR_ALIGN;
  if ((int64_t)B * T * Hq > 0x7fffffffLL) return PA_ERR_RANGE;
  return pa::launch_prefill_paged(q, kv_cache, n_pages, block_table, n_slots, n_layers,
                                  max_blocks_per_seq, layer, slot_ids, seq_lens, q_lens, B, T, Hq,
                                  Hkv, head_dim, scale, causal, O, LSE, err,
                                  static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

const char *pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "required pointer is NULL";
    case PA_ERR_SHAPE: return "invalid or inconsistent size";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim or group size";
    case PA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_RANGE: return "index or byte offset overflow";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_VALUE: return "scale must be finite and > 0";
    default: return "unknown status";
  }
}

int64_t pa_page_bytes(int n_kv_heads, int head_dim) {
  if (n_kv_heads <= 0 || head_dim <= 0) return 0;
  return 2LL * 16 * n_kv_heads * head_dim * 2;
}

int pa_clock_probe(float *ghz, int n_waves, int iters, void *stream) {
  if (n_waves < 0 || iters < 0) return PA_ERR_SHAPE;
  if (n_waves == 0) return PA_OK;
  if (!ghz) return PA_ERR_NULL;
  return pa::launch_clock_probe(ghz, n_waves, iters, static_cast<hipStream_t>(stream));
}

int kv_scatter(const void *k, const void *v, int64_t n_tokens, const int32_t *slot_ids,
               const int32_t *positions, void *kv_cache, int64_t n_pages,
               const int32_t *block_table, int n_slots, int n_layers, int max_blocks_per_seq,
               int layer, int n_kv_heads, int head_dim, int32_t *err, void *stream) {
  if (n_tokens < 0) return PA_ERR_SHAPE;
  int rc = check_cache(kv_cache, n_pages, block_table, n_slots, n_layers, max_blocks_per_seq, layer,
                       n_kv_heads, head_dim);
  if (rc != PA_OK) return rc;
  if (((int64_t)n_kv_heads * head_dim) % 8 != 0) return PA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return PA_OK;
  if (!k || !v || !slot_ids || !positions) return PA_ERR_NULL;
  if (!aligned16(k) || !aligned16(v)) return PA_ERR_ALIGN;
  return pa::launch_kv_scatter(k, v, n_tokens, slot_ids, positions, kv_cache, n_pages, block_table,
                               n_slots, n_layers, max_blocks_per_seq, layer, n_kv_heads, head_dim,
                               err, static_cast<hipStream_t>(stream));
}

int attn_prefill(const void *q, const void *kv_cache, int64_t n_pages, const int32_t *block_table,
                 int n_slots, int n_layers, int max_blocks_per_seq, int layer,
                 const int32_t *slot_ids, const int32_t *seq_lens, int B, int T, int Hq, int Hkv,
                 int head_dim, float scale, int causal, void *O, float *LSE, int32_t *err,
                 void *stream) {
  return prefill_common(q, kv_cache, n_pages, block_table, n_slots, n_layers, max_blocks_per_seq,
                        layer, slot_ids, seq_lens, nullptr, B, T, Hq, Hkv, head_dim, scale, causal,
                        O, LSE, err, stream);
}

int attn_prefill_append(const void *q, const void *k, const void *v, void *kv_cache, int64_t n_pages,
                        const int32_t *block_table, int n_slots, int n_layers, int max_blocks_per_seq,
                        int layer, const int32_t *slot_ids, const int32_t *seq_lens, int B, int T,
                        int Hq, int Hkv, int head_dim, float scale, int causal, void *O, float *LSE,
                        int32_t *err, void *stream) {
  if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return PA_ERR_SHAPE;
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (!valid_scale(scale)) return PA_ERR_VALUE;
  int rc = check_cache(kv_cache, n_pages, block_table, n_slots, n_layers, max_blocks_per_seq, layer,
                       Hkv, head_dim);
  if (rc != PA_OK) return rc;
  if (B == 0 || T == 0) return PA_OK;
  if (!q || !k || !v || !seq_lens || !O || !LSE) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(O)) return PA_ERR_ALIGN;
  if ((int64_t)B * T * Hq > 0x7fffffffLL) return PA_ERR_RANGE;
  return pa::launch_prefill_store(q, k, v, kv_cache, n_pages, block_table, n_slots, n_layers,
                                  max_blocks_per_seq, layer, slot_ids, seq_lens, B, T, Hq, Hkv,
                                  head_dim, scale, causal, O, LSE, err,
                                  static_cast<hipStream_t>(stream));
}

int attn_prefill_chunk(const void *q, const void *kv_cache, int64_t n_pages,
                       const int32_t *block_table, int n_slots, int n_layers,
                       int max_blocks_per_seq, int layer, const int32_t *slot_ids,
                       const int32_t *q_lens, const int32_t *kv_lens, int B, int T, int Hq,
                       int Hkv, int head_dim, float scale, int causal, void *O, float *LSE,
                       int32_t *err, void *stream) {
  if (B > 0 && T > 0 && !q_lens) return PA_ERR_NULL;
  return prefill_common(q, kv_cache, n_pages, block_table, n_slots, n_layers, max_blocks_per_seq,
                        layer, slot_ids, kv_lens, q_lens, B, T, Hq, Hkv, head_dim, scale, causal,
                        O, LSE, err, stream);
}

int attn_prefill_packed_plan(const int32_t *q_lens, const int32_t *kv_lens, int B, int Hq, int Hkv,
                             int head_dim, int causal, int32_t *plan, int64_t plan_capacity,
                             int64_t *n_work, int64_t *n_merge, size_t *workspace_bytes) {
  if (!n_work || !n_merge || !workspace_bytes) return PA_ERR_NULL;
  *n_work = 0;
  *n_merge = 0;
  *workspace_bytes = 0;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || plan_capacity < 0) return PA_ERR_SHAPE;
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return PA_ERR_UNSUPPORTED;
  if (B == 0) return PA_OK;
  if (!q_lens || !kv_lens) return PA_ERR_NULL;
  return pa::plan_prefill_packed(q_lens, kv_lens, B, Hq, Hkv, head_dim, causal ? 1 : 0,
                                 pa::device_cu_count(), plan, plan_capacity, n_work, n_merge,
                                 workspace_bytes);
}

int attn_prefill_packed(const void *q, const void *kv_cache, int64_t n_pages,
                        const int32_t *block_table, int n_slots, int n_layers,
                        int max_blocks_per_seq, int layer, const int32_t *slot_ids,
                        const int32_t *kv_lens, const int32_t *q_start, int B, int64_t total_q,
                        int Hq, int Hkv, int head_dim, float scale, int causal,
                        const int32_t *plan, int64_t n_work, int64_t n_merge, void *workspace,
                        size_t workspace_bytes, void *O, float *LSE, int32_t *err, void *stream) {
  if (B < 0 || total_q < 0 || n_work < 0 || n_merge < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return PA_ERR_SHAPE;
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return PA_ERR_UNSUPPORTED;
  if (!valid_scale(scale)) return PA_ERR_VALUE;
  int rc = check_cache(kv_cache, n_pages, block_table, n_slots, n_layers, max_blocks_per_seq, layer,
                       Hkv, head_dim);
  if (rc != PA_OK) return rc;
  if (B == 0 || total_q == 0 || n_work == 0) return PA_OK;
  if (!q || !kv_lens || !q_start || !plan || !O || !LSE) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(O)) return PA_ERR_ALIGN;
  if (n_merge > 0 && !workspace) return PA_ERR_NULL;
  if (workspace && !aligned16(workspace)) return PA_ERR_ALIGN;
  if (total_q > INT64_MAX / ((int64_t)Hq * head_dim * 2)) return PA_ERR_RANGE;
  const int64_t tile_bytes = (int64_t)pa::prefill_rows_per_block(G) * pa::prefill_heads_per_block(G) *
                             (head_dim + 1) * 4;
  const int64_t n_part_slots = workspace ? (int64_t)(workspace_bytes / tile_bytes) : 0;
  return pa::launch_prefill_packed(q, kv_cache, n_pages, block_table, n_slots, n_layers,
                                   max_blocks_per_seq, layer, slot_ids, kv_lens, q_start, B, total_q,
                                   Hq, Hkv, head_dim, scale, causal, plan, n_work, n_merge, workspace,
                                   n_part_slots, O, LSE, err, static_cast<hipStream_t>(stream));
}

int attn_decode_whole_pages(int B, int Hq, int Hkv, int head_dim, int max_ctx) {
  return pa::rows_path(B, Hq, Hkv, head_dim, max_ctx, false) ? 1 : 0;
}

size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int head_dim, int max_ctx) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || head_dim <= 0 || max_ctx < 0) return 0;
  return pa::decode_workspace_bytes(B, Hq, Hkv, head_dim, max_ctx);
}

}  // extern "C"

namespace {

// Host checks shared by attn_decode and attn_decode_noalloc (PA_OK: launch).
int decode_checks(const void *q, const void *kv_cache, int64_t n_pages, const int32_t *block_table,
                  int n_slots, int n_layers, int max_blocks_per_seq, int layer,
                  const int32_t *ctx_lens, int B, int Hq, int Hkv, int head_dim, float scale,
                  int max_ctx, const void *O, const float *LSE) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_ctx < 0) return PA_ERR_SHAPE;
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return PA_ERR_UNSUPPORTED;
  if (!valid_scale(scale)) return PA_ERR_VALUE;
  int rc = check_cache(kv_cache, n_pages, block_table, n_slots, n_layers, max_blocks_per_seq, layer,
                       Hkv, head_dim);
  if (rc != PA_OK) return rc;
  if (B == 0) return PA_OK;
  if (!q || !ctx_lens || !O || !LSE) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(O)) return PA_ERR_ALIGN;
  return PA_OK;
}

}  // namespace

extern "C" {

int attn_decode(const void *q, const void *kv_cache, int64_t n_pages, const int32_t *block_table,
                int n_slots, int n_layers, int max_blocks_per_seq, int layer,
                const int32_t *slot_ids, const int32_t *ctx_lens, int B, int Hq, int Hkv,
                int head_dim, float scale, int max_ctx, void *workspace, size_t workspace_bytes,
                void *O, float *LSE, int32_t *err, void *stream) {
  int rc = decode_checks(q, kv_cache, n_pages, block_table, n_slots, n_layers, max_blocks_per_seq,
                         layer, ctx_lens, B, Hq, Hkv, head_dim, scale, max_ctx, O, LSE);
  if (rc != PA_OK || B == 0) return rc;
  const size_t ws_need = pa::decode_workspace_bytes(B, Hq, Hkv, head_dim, max_ctx);
  if (ws_need > 0 && !workspace) return PA_ERR_NULL;
  if (ws_need > 0 && !aligned16(workspace)) return PA_ERR_ALIGN;
  if (workspace_bytes < ws_need) return PA_ERR_WORKSPACE;
  return pa::launch_decode(q, kv_cache, n_pages, block_table, n_slots, n_layers,
                           max_blocks_per_seq, layer, slot_ids, ctx_lens, B, Hq, Hkv, head_dim,
                           scale, max_ctx, workspace, O, LSE, err,
                           static_cast<hipStream_t>(stream));
}

int attn_decode_append(const void *q, const void *k_new, const void *v_new, void *kv_cache,
                       int64_t n_pages, const int32_t *block_table, int n_slots, int n_layers,
                       int max_blocks_per_seq, int layer, const int32_t *slot_ids,
                       const int32_t *ctx_lens, int B, int Hq, int Hkv, int head_dim, float scale,
                       int max_ctx, void *workspace, size_t workspace_bytes, void *O, float *LSE,
                       int32_t *err, void *stream) {
  int rc = decode_checks(q, kv_cache, n_pages, block_table, n_slots, n_layers, max_blocks_per_seq,
                         layer, ctx_lens, B, Hq, Hkv, head_dim, scale, max_ctx, O, LSE);
  if (rc != PA_OK || B == 0) return rc;
  if (!k_new || !v_new) return PA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return PA_ERR_ALIGN;
  const size_t ws_need = pa::decode_workspace_bytes(B, Hq, Hkv, head_dim, max_ctx);
  if (ws_need > 0 && !workspace) return PA_ERR_NULL;
  if (ws_need > 0 && !aligned16(workspace)) return PA_ERR_ALIGN;
  if (workspace_bytes < ws_need) return PA_ERR_WORKSPACE;
  return pa::launch_decode(q, kv_cache, n_pages, block_table, n_slots, n_layers,
                           max_blocks_per_seq, layer, slot_ids, ctx_lens, B, Hq, Hkv, head_dim,
                           scale, max_ctx, workspace, O, LSE, err, static_cast<hipStream_t>(stream),
                           k_new, v_new);
}

int attn_decode_noalloc(const void *q, const void *kv_cache, int64_t n_pages,
                        const int32_t *block_table, int n_slots, int n_layers,
                        int max_blocks_per_seq, int layer, const int32_t *slot_ids,
                        const int32_t *ctx_lens, int B, int Hq, int Hkv, int head_dim, float scale,
                        int max_ctx, void *O, float *LSE, int32_t *err, void *stream) {
  int rc = decode_checks(q, kv_cache, n_pages, block_table, n_slots, n_layers, max_blocks_per_seq,
                         layer, ctx_lens, B, Hq, Hkv, head_dim, scale, max_ctx, O, LSE);
  if (rc != PA_OK || B == 0) return rc;
  if (pa::decode_workspace_bytes(B, Hq, Hkv, head_dim, max_ctx) > pa::decode_scratch_bytes())
    return PA_ERR_WORKSPACE;
  void *ws = pa::decode_scratch_ptr();
  if (!ws) return PA_ERR_LAUNCH;
  return pa::launch_decode(q, kv_cache, n_pages, block_table, n_slots, n_layers,
                           max_blocks_per_seq, layer, slot_ids, ctx_lens, B, Hq, Hkv, head_dim,
                           scale, max_ctx, ws, O, LSE, err, static_cast<hipStream_t>(stream));
}

int attn_prefill_dense(const void *q, const void *k, const void *v, int B, int T, int Hq, int Hkv,
                       int head_dim, float scale, int causal, void *O, float *LSE, void *stream) {
  if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return PA_ERR_SHAPE;
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return PA_ERR_UNSUPPORTED;
  if (!valid_scale(scale)) return PA_ERR_VALUE;
  if (B == 0 || T == 0) return PA_OK;
  if (!q || !k || !v || !O || !LSE) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(O)) return PA_ERR_ALIGN;
  if ((int64_t)B * T * Hq > 0x7fffffffLL) return PA_ERR_RANGE;
  return pa::launch_prefill_dense(q, k, v, B, T, Hq, Hkv, head_dim, scale, causal, O, LSE,
                                  static_cast<hipStream_t>(stream));
}

int kv_append(const void *k, const void *v, const void *q_in, void *q_out, int Hq, int B,
              const int32_t *slot_ids, const int32_t *positions, const float *cos_t,
              const float *sin_t, int max_pos, void *kv_cache, int64_t n_pages,
              int32_t *block_table, int n_slots, int n_layers, int max_blocks_per_seq, int layer,
              const int32_t *free_pages, int capacity, int32_t *alloc_state, int n_kv_heads,
              int head_dim, int32_t *err, void *stream) {
  if (B < 0 || max_pos <= 0 || capacity < 0) return PA_ERR_SHAPE;
  int rc = check_cache(kv_cache, n_pages, block_table, n_slots, n_layers, max_blocks_per_seq, layer,
                       n_kv_heads, head_dim);
  if (rc != PA_OK) return rc;
  if (head_dim % 16 != 0) return PA_ERR_UNSUPPORTED;
  if ((int64_t)n_kv_heads * head_dim > 8192) return PA_ERR_UNSUPPORTED;  // K+V row staged in LDS
  if ((q_in == nullptr) != (q_out == nullptr)) return PA_ERR_NULL;
  if (q_in && Hq <= 0) return PA_ERR_SHAPE;
  if ((int64_t)max_pos * (head_dim / 2) > 0x7fffffffLL) return PA_ERR_RANGE;
  if (B == 0) return PA_OK;
  if (!k || !v || !positions || !cos_t || !sin_t || !free_pages || !alloc_state) return PA_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(cos_t) || !aligned16(sin_t)) return PA_ERR_ALIGN;
  if (q_in && (!aligned16(q_in) || !aligned16(q_out))) return PA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(alloc_state) & 3u) != 0) return PA_ERR_ALIGN;
  return pa::launch_kv_append(k, v, q_in, q_out, q_in ? Hq : 0, B, slot_ids, positions, cos_t,
                              sin_t, max_pos, kv_cache, n_pages, block_table, n_slots, n_layers,
                              max_blocks_per_seq, layer, free_pages, capacity, alloc_state,
                              n_kv_heads, head_dim, err, static_cast<hipStream_t>(stream));
}

int kv_release(const int32_t *slots, int n, int32_t *block_table, int n_slots, int n_layers,
               int max_blocks_per_seq, int32_t *free_pages, int capacity, int32_t *alloc_state,
               int32_t *err, void *stream) {
  if (n < 0 || n_slots <= 0 || n_layers <= 0 || max_blocks_per_seq <= 0 || capacity < 0)
    return PA_ERR_SHAPE;
  if ((int64_t)n_slots * n_layers * max_blocks_per_seq > 0x7fffffffLL) return PA_ERR_RANGE;
  if (n == 0) return PA_OK;
  if (!slots || !block_table || !free_pages || !alloc_state) return PA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(alloc_state) & 3u) != 0) return PA_ERR_ALIGN;
  return pa::launch_kv_release(slots, n, block_table, n_slots, n_layers, max_blocks_per_seq,
                               free_pages, capacity, alloc_state, err,
                               static_cast<hipStream_t>(stream));
}

size_t attn_backward_workspace_size(int B, int T, int Hq) {
  if (B <= 0 || T <= 0 || Hq <= 0) return 0;
  return pa::backward_workspace_bytes(B, T, Hq);
}

int attn_backward_dense(const void *q, const void *k, const void *v, const void *o,
                        const void *dout, const float *lse, int B, int T, int Hq, int Hkv,
                        int head_dim, float scale, int causal, void *dq, void *dk, void *dv,
                        void *workspace, size_t workspace_bytes, void *stream) {
  if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return PA_ERR_SHAPE;
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return PA_ERR_UNSUPPORTED;
  if (!valid_scale(scale)) return PA_ERR_VALUE;
  if (B == 0 || T == 0) return PA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) || !aligned16(lse))
    return PA_ERR_ALIGN;
  if ((int64_t)B * T * Hq > 0x7fffffffLL / 16) return PA_ERR_RANGE;
  if (workspace_bytes < pa::backward_workspace_bytes(B, T, Hq)) return PA_ERR_WORKSPACE;
  return pa::launch_backward_dense(q, k, v, o, dout, lse, B, T, Hq, Hkv, head_dim, scale, causal,
                                   dq, dk, dv, workspace, static_cast<hipStream_t>(stream));
}

}  // extern "C"
