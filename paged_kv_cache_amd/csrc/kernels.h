// kernels.h -- host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// packed prefill: work list (host), prefill launch and merge of split row blocks
int prefill_rows_per_block(int G);
int prefill_heads_per_block(int G);
int plan_prefill_packed(const int32_t *q_lens, const int32_t *kv_lens, int B, int Hq, int Hkv, int D,
                        int causal, int n_cu, int32_t *plan, int64_t capacity, int64_t *n_work,
                        int64_t *n_merge, size_t *part_bytes);
int launch_prefill_packed(const void *q, const void *kv_cache, int64_t n_pages,
                          const int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                          const int32_t *slot_ids, const int32_t *kv_lens, const int32_t *q_start, int B,
                          int64_t total_q, int Hq, int Hkv, int D, float scale, int causal,
                          const int32_t *plan, int64_t n_work, int64_t n_merge, void *part,
                          int64_t n_part_slots, void *O, float *LSE, int32_t *err, hipStream_t stream);
int launch_packed_merge(const int32_t *merge, int64_t n_merge, const int32_t *q_start, int B,
                        const float *part, int64_t n_part_slots, void *O, float *LSE, int32_t *err,
                        int64_t total_q, int Hq, int Hkv, int D, hipStream_t stream);
int launch_clock_probe(float *ghz, int n_waves, int iters, hipStream_t stream);
int launch_kv_scatter(const void *k, const void *v, int64_t n_tokens, const int32_t *slot_ids,
                      const int32_t *positions, void *kv_cache, int64_t n_pages,
                      const int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                      int n_kv_heads, int head_dim, int32_t *err, hipStream_t stream);

int launch_prefill_paged(const void *q, const void *kv_cache, int64_t n_pages,
                         const int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                         const int32_t *slot_ids, const int32_t *seq_lens, const int32_t *q_lens,
                         int B, int T, int Hq, int Hkv, int D, float scale, int causal, void *O,
                         float *LSE, int32_t *err, hipStream_t stream);

int launch_prefill_dense(const void *q, const void *k, const void *v, int B, int T, int Hq, int Hkv,
                         int D, float scale, int causal, void *O, float *LSE, hipStream_t stream);

// attn_prefill_append: the prefill of whole prompts on the inputs k, v
// [B][T][Hkv][D], which also writes every prompt token's K/V row to its page.
int launch_prefill_store(const void *q, const void *k, const void *v, void *kv_cache, int64_t n_pages,
                         const int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                         const int32_t *slot_ids, const int32_t *seq_lens, int B, int T, int Hq, int Hkv,
                         int D, float scale, int causal, void *O, float *LSE, int32_t *err,
                         hipStream_t stream);

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int D, int max_ctx);
// whether attn_decode streams whole pages for this shape (decode_rows_kernel)
bool rows_path(int B, int Hq, int Hkv, int D, int max_ctx, bool append);

// attn_decode_noalloc's workspace: the capacity of the static device array and
// the current device's address of it (looked up on the first call on each
// device; nullptr if the lookup fails).
size_t decode_scratch_bytes();
void *decode_scratch_ptr();

// k_new, v_new (attn_decode_append): the new token of every sequence, written
// to kv_cache at position ctx_lens[b] - 1 by the same launch; null: none.
int launch_decode(const void *q, const void *kv_cache, int64_t n_pages, const int32_t *block_table,
                  int n_slots, int n_layers, int mbps, int layer, const int32_t *slot_ids,
                  const int32_t *ctx_lens, int B, int Hq, int Hkv, int D, float scale, int max_ctx,
                  void *workspace, void *O, float *LSE, int32_t *err, hipStream_t stream,
                  const void *k_new = nullptr, const void *v_new = nullptr);

int launch_kv_append(const void *k, const void *v, const void *q_in, void *q_out, int Hq, int B,
                     const int32_t *slot_ids, const int32_t *positions, const float *cos_t,
                     const float *sin_t, int max_pos, void *kv_cache, int64_t n_pages,
                     int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                     const int32_t *free_pages, int capacity, int32_t *alloc_state, int n_kv_heads,
                     int head_dim, int32_t *err, hipStream_t stream);

int launch_kv_release(const int32_t *slots, int n, int32_t *block_table, int n_slots, int n_layers,
                      int mbps, int32_t *free_pages, int capacity, int32_t *alloc_state,
                      int32_t *err, hipStream_t stream);

size_t backward_workspace_bytes(int B, int T, int Hq);

// Compute units of the current device (queried once per device; 256 if the
// query fails).  Launchers use it to lay workgroups out in layers of one per CU.
int device_cu_count();

int launch_backward_dense(const void *q, const void *k, const void *v, const void *o,
                          const void *dout, const float *lse, int B, int T, int Hq, int Hkv, int D,
                          float scale, int causal, void *dq, void *dk, void *dv, void *workspace,
                          hipStream_t stream);

}  // namespace pa
