// scatter.hip -- kv_scatter: copy the K and V rows of new tokens into their
// 16-token pages (tiny-vllm part 3, "Distributing K/V into paged blocks";
// tiny-vllm part 6, "Block contents: K in front, V after V_OFFSET").
//
// The reference copies a whole page per host-issued memcpy pair after a host
// lookup.  Here one launch covers any number of tokens: every thread moves one
// 16-byte chunk of one token's K or V row, looks the page up in the block
// table itself and stores with a single 16-byte write, so a token's
// 2 x Hkv x d x 2 bytes are spread over 2 x Hkv x d / 8 lanes and consecutive
// lanes write consecutive bytes of a row.

#include "device.h"
#include "kernels.h"

namespace pa {

__global__ __launch_bounds__(256) void kv_scatter_kernel(
    const uint4 *__restrict__ k, const uint4 *__restrict__ v, int64_t n_tokens,
    const int32_t *__restrict__ slot_ids, const int32_t *__restrict__ positions,
    uint8_t *__restrict__ pool, int64_t n_pages, const int32_t *__restrict__ block_table,
    int n_slots, int n_layers, int mbps, int layer, int chunks_per_row, int64_t page_bytes,
    int64_t v_offset, int32_t *err) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = 2 * (int64_t)chunks_per_row;
  const int64_t tok = gid / per_token;
  if (tok >= n_tokens) return;
  const int r = (int)(gid - tok * per_token);
  const bool is_v = r >= chunks_per_row;
  const int c = is_v ? r - chunks_per_row : r;

  const int slot = slot_ids[tok];
  const int pos = positions[tok];
  if (slot < 0 || slot >= n_slots) {
    if (r == 0) raise_err(err, PA_DEVERR_BAD_SLOT);
    return;
  }
  if (pos < 0 || pos >= mbps * kPageTokens) {
    if (r == 0) raise_err(err, PA_DEVERR_BAD_POS);
    return;
  }
  const int32_t page = block_table[((int64_t)slot * n_layers + layer) * mbps + pos / kPageTokens];
  if (page < 0 || (int64_t)page >= n_pages) {
    if (r == 0) raise_err(err, PA_DEVERR_BAD_PAGE);
    return;
  }
  const int64_t row_bytes = (int64_t)chunks_per_row * 16;
  uint8_t *dst = pool + (int64_t)page * page_bytes + (is_v ? v_offset : 0) +
                 (int64_t)(pos % kPageTokens) * row_bytes + (int64_t)c * 16;
  const uint4 *src = (is_v ? v : k) + tok * chunks_per_row + c;
  *reinterpret_cast<uint4 *>(dst) = *src;
}

int launch_kv_scatter(const void *k, const void *v, int64_t n_tokens, const int32_t *slot_ids,
                      const int32_t *positions, void *kv_cache, int64_t n_pages,
                      const int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                      int n_kv_heads, int head_dim, int32_t *err, hipStream_t stream) {
  const int chunks_per_row = n_kv_heads * head_dim * 2 / 16;
  const int64_t page_bytes = 2LL * kPageTokens * n_kv_heads * head_dim * 2;
  const int64_t v_offset = page_bytes / 2;
  const int64_t threads = n_tokens * 2 * chunks_per_row;
  const int block = 256;
  const int64_t grid = (threads + block - 1) / block;
  if (grid > 0x7fffffff) return PA_ERR_RANGE;
  hipLaunchKernelGGL(kv_scatter_kernel, dim3((unsigned)grid), dim3(block), 0, stream,
                     static_cast<const uint4 *>(k), static_cast<const uint4 *>(v), n_tokens,
                     slot_ids, positions, static_cast<uint8_t *>(kv_cache), n_pages, block_table,
                     n_slots, n_layers, mbps, layer, chunks_per_row, page_bytes, v_offset, err);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
