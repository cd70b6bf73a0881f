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

// WIDE: 64-bit thread index (more than 2^31 - 1 chunks in one call).  The
// source chunk is loaded together with the slot and position: its address
// does not depend on the block table, so the copy waits for one lookup chain
// (slot and position, then the table entry) instead of that chain and then
// the load.
template <bool WIDE>
__global__ __launch_bounds__(256) void kv_scatter_kernel(
    const uint4 *__restrict__ k, const uint4 *__restrict__ v, int64_t n_tokens,
    const int32_t *__restrict__ slot_ids, const int32_t *__restrict__ positions,
    uint8_t *__restrict__ pool, int64_t n_pages, const int32_t *__restrict__ block_table,
    int n_slots, int n_layers, int mbps, int layer, int chunks_per_row, int64_t page_bytes,
    int64_t v_offset, int32_t *err) {
  int64_t tok, src;   // token, and the source chunk's index in k or v
  int r;
  if constexpr (WIDE) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_token = 2 * (int64_t)chunks_per_row;
    tok = gid / per_token;
    r = (int)(gid - tok * per_token);
    src = tok * chunks_per_row + (r >= chunks_per_row ? r - chunks_per_row : r);
  } else {
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t per_token = 2u * (uint32_t)chunks_per_row;
    const uint32_t t = gid / per_token;
    tok = t;
    r = (int)(gid - t * per_token);
    src = (uint32_t)(t * (uint32_t)chunks_per_row + (uint32_t)(r >= chunks_per_row ? r - chunks_per_row : r));
  }
  if (tok >= n_tokens) return;
  const bool is_v = r >= chunks_per_row;
  const int c = is_v ? r - chunks_per_row : r;
  int slot_raw = slot_ids[tok];
  int pos_raw = positions[tok];
  u32x4 data = *reinterpret_cast<const u32x4 *>((is_v ? v : k) + src);
  // the three loads are issued together and have landed here (an empty asm
  // that takes their registers; else the compiler sinks the data load below
  // the table lookup, behind a second memory latency)
  asm volatile("" : "+v"(data), "+v"(slot_raw), "+v"(pos_raw));
  // a bad slot or position looks up entry 0 of slot 0 instead (the host
  // checks n_slots, n_layers and the blocks per sequence are positive) and
  // stores nothing
  const bool slot_ok = slot_raw >= 0 && slot_raw < n_slots;
  const bool pos_ok = pos_raw >= 0 && pos_raw < mbps * kPageTokens;
  const int slot = slot_ok && pos_ok ? slot_raw : 0;
  const int pos = slot_ok && pos_ok ? pos_raw : 0;
  const int32_t page = block_table[((int64_t)slot * n_layers + layer) * mbps + pos / kPageTokens];
  const bool page_ok = page >= 0 && (int64_t)page < n_pages;
  if (!(slot_ok && pos_ok && page_ok)) {
    if (r == 0) raise_err(err, !slot_ok ? PA_DEVERR_BAD_SLOT : !pos_ok ? PA_DEVERR_BAD_POS : PA_DEVERR_BAD_PAGE);
    return;
  }
  const int64_t row_bytes = (int64_t)chunks_per_row * 16;
  uint8_t *dst = pool + (int64_t)page * page_bytes + (is_v ? v_offset : 0) +
                 (int64_t)(pos % kPageTokens) * row_bytes + (int64_t)c * 16;
  // non-temporal: the new rows are not read again by this kernel, and lines
  // that leave L2 as they are written do not wait to be written back when it
  // ends (4096-token prompt 3.8-4.0 -> 3.3 us, the attention after it unchanged)
  __builtin_nontemporal_store(data, reinterpret_cast<u32x4 *>(dst));
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
  auto kern = grid * block <= 0x7fffffffLL ? kv_scatter_kernel<false> : kv_scatter_kernel<true>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(block), 0, stream,
                     static_cast<const uint4 *>(k), static_cast<const uint4 *>(v), n_tokens,
                     slot_ids, positions, static_cast<uint8_t *>(kv_cache), n_pages, block_table,
                     n_slots, n_layers, mbps, layer, chunks_per_row, page_bytes, v_offset, err);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
