// append.hip -- the writes of one decode step, fused in one launch
// (kv_append), and the release of finished slots' pages (kv_release).
//
// kv_append, per new token (tiny-vllm part 3, "RoPE: a rotation that references
// a table" and "Distributing K/V into paged blocks"; tiny-vllm part 6, "The
// lifetime of a physical block: free_blocks"):
//   - a token whose position opens a block (pos % 16 == 0, the decode rule)
//     takes a page from the back of the caller's free stack, in batch order,
//     and records it in the block table;
//   - its K row is rotated by RoPE (pair i = elements i and i + d/2 of a head,
//     angle from row pos of the cos/sin tables) and written with its V row
//     into the page; the query can be rotated in the same launch.
//
// One workgroup per token.  Pop order without any cross-workgroup wait: wave 0
// of every workgroup counts, over the whole batch, the openers before its own
// token (its rank r) and all openers (n); an opener takes free_pages[top-1-r]
// with top read from the allocator state.  The stack top is lowered once, by
// whichever opener arrives last on a counter next to it (each opener has read
// top before it arrives, so nobody reads a lowered top), and that opener
// resets the counter for the next call.  The top and the counter are only
// touched by device-scope atomics, so no memory fence is needed.
//
// Rotation arithmetic is fp64: a bf16 times an fp32 table value is exact in
// fp64, so each output is the exact x1*c - x2*s (or x1*s + x2*c) rounded once,
// then rounded to the nearest bf16 (ties to even).  The result is thus a
// function of the inputs alone, bit for bit.
//
// kv_release is one workgroup: for each released slot in order, its table
// entries (layer-major, logical blocks ascending) are scanned 1024 at a time;
// the entries that hold a page are compacted onto the top of the free stack
// by a workgroup prefix count and reset to -1.

#include "device.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kAppendThreads = 512;
// wave 0 takes the page, waves 1-2 rotate K and stage K/V, waves 3-7 rotate
// the query: the three dependency chains run side by side
constexpr int kKvThreads = 128;
constexpr int kReleaseThreads = 1024;

// Nearest bf16 of a double, ties to even.  The double is first rounded to fp32
// (nearest even); a second rounding to bf16 can only go wrong when that fp32
// value lies exactly halfway between two bf16 values while the double did not,
// and then the side of the double decides.
__device__ __forceinline__ uint32_t f64_to_bf16(double r) {
  const float f = (float)r;
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  if ((u & 0xffffu) == 0x8000u && (double)f != r)
    return (u >> 16) + (fabs(r) > fabs((double)f) ? 1u : 0u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) { return (double)__uint_as_float(w & 0xffff0000u); }

// Rotate 8 pairs: x1 = elements [c0, c0+8) of the first half, x2 = the same
// elements of the second half, angles cs/sn (8 fp32 each).
__device__ __forceinline__ void rotate8(const u32x4 &x1, const u32x4 &x2, const float *cs,
                                        const float *sn, u32x4 &y1, u32x4 &y2) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t o1 = 0, o2 = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const double a = h ? bf16_hi(x1[w]) : bf16_lo(x1[w]);
      const double b = h ? bf16_hi(x2[w]) : bf16_lo(x2[w]);
      const double c = (double)cs[2 * w + h], s = (double)sn[2 * w + h];
      const uint32_t r1 = f64_to_bf16(a * c - b * s);
      const uint32_t r2 = f64_to_bf16(a * s + b * c);
      o1 |= r1 << (16 * h);
      o2 |= r2 << (16 * h);
    }
    y1[w] = o1;
    y2[w] = o2;
  }
}

struct AppendArgs {
  const uint8_t *k, *v;            // [B][Hkv][d] bf16
  const uint8_t *q_in;             // [B][Hq][d] bf16 or null
  uint8_t *q_out;
  const int32_t *slot_ids;         // null: identity
  const int32_t *positions;
  const float *cos_t, *sin_t;      // [max_pos][d/2]
  uint8_t *pool;
  int32_t *block_table;
  const int32_t *free_pages;
  int32_t *alloc;                  // [0] top, [1] arrivals (0 between calls)
  int capacity;                    // entries of free_pages
  int32_t *err;
  int64_t n_pages, page_bytes, v_offset;
  int B, Hq, Hkv, d, max_pos, n_slots, n_layers, mbps, layer;
};

__device__ __forceinline__ bool token_valid(const AppendArgs &a, int slot, int pos) {
  return slot >= 0 && slot < a.n_slots && pos >= 0 && pos < a.max_pos && pos < a.mbps * kPageTokens;
}

// Rotate (and write) every 16-byte chunk pair of n_heads head vectors of one
// token; the chunk pairs are spread over nthreads threads, this one taking
// items tid, tid + nthreads, ...
__device__ __forceinline__ void rope_rows(const uint8_t *src, uint8_t *dst, int n_heads, int d,
                                          const float *cs_row, const float *sn_row, int tid,
                                          int nthreads) {
  const int cpp = d / 16;  // chunk pairs per head: 8 elements of each half
  for (int it = tid; it < n_heads * cpp; it += nthreads) {
    const int h = it / cpp, c = it - h * cpp;
    const uint8_t *x = src + (int64_t)h * d * 2;
    const u32x4 x1 = *reinterpret_cast<const u32x4 *>(x + c * 16);
    const u32x4 x2 = *reinterpret_cast<const u32x4 *>(x + d + c * 16);
    float cs[8], sn[8];
    *reinterpret_cast<f32x4 *>(cs) = *reinterpret_cast<const f32x4 *>(cs_row + c * 8);
    *reinterpret_cast<f32x4 *>(cs + 4) = *reinterpret_cast<const f32x4 *>(cs_row + c * 8 + 4);
    *reinterpret_cast<f32x4 *>(sn) = *reinterpret_cast<const f32x4 *>(sn_row + c * 8);
    *reinterpret_cast<f32x4 *>(sn + 4) = *reinterpret_cast<const f32x4 *>(sn_row + c * 8 + 4);
    u32x4 y1, y2;
    rotate8(x1, x2, cs, sn, y1, y2);
    uint8_t *y = dst + (int64_t)h * d * 2;
    *reinterpret_cast<u32x4 *>(y + c * 16) = y1;
    *reinterpret_cast<u32x4 *>(y + d + c * 16) = y2;
  }
}

}  // namespace

__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendArgs a) {
  // stage: the rotated K row then the V row of this token (2 * Hkv * d * 2 bytes)
  extern __shared__ u32x4 stage[];
  __shared__ int page_s;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int slot = a.slot_ids ? a.slot_ids[b] : b;
  const int pos = a.positions[b];
  const bool pos_ok = pos >= 0 && pos < a.max_pos;
  const bool valid = token_valid(a, slot, pos);
  const bool opens = valid && (pos % kPageTokens) == 0;
  const float *cs_row = a.cos_t + (int64_t)(pos_ok ? pos : 0) * (a.d / 2);
  const float *sn_row = a.sin_t + (int64_t)(pos_ok ? pos : 0) * (a.d / 2);
  const int64_t row_bytes = (int64_t)a.Hkv * a.d * 2;
  int32_t *entry = a.block_table + ((int64_t)(valid ? slot : 0) * a.n_layers + a.layer) * a.mbps +
                   (valid ? pos : 0) / kPageTokens;
  int top = 0, old_entry = -1, rank = 0, total = 0;

  if (tid < 64) {
    // wave 0: the page.  The stack top, the first 64 tokens' slots and
    // positions and this token's entry are all requested at once; then the
    // rank of this token among the openers of the batch, their count, and
    // whether another token names the same slot.
    top = __hip_atomic_load(&a.alloc[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    top = top < 0 ? 0 : (top > a.capacity ? a.capacity : top);
    bool dup = false;
    for (int base = 0; base < a.B; base += 64) {
      const int i = base + lane;
      const int ic = i < a.B ? i : a.B - 1;
      const int si = a.slot_ids ? a.slot_ids[ic] : ic;
      const int pi = a.positions[ic];
      if (base == 0 && valid) old_entry = *entry;
      const bool need = i < a.B && token_valid(a, si, pi) && (pi % kPageTokens) == 0;
      const bool same = i < a.B && i != b && si == slot;
      rank += __popcll(__ballot(need && i < b));
      total += __popcll(__ballot(need));
      dup |= __ballot(same) != 0;
    }
    if (lane == 0) {
      int page = -1;
      if (dup) raise_err(a.err, PA_DEVERR_DUP_SLOT);
      if (!(slot >= 0 && slot < a.n_slots)) {
        raise_err(a.err, PA_DEVERR_BAD_SLOT);
      } else if (!valid) {
        raise_err(a.err, PA_DEVERR_BAD_POS);
      } else if (opens) {
        if (rank >= top) {
          raise_err(a.err, PA_DEVERR_NO_FREE_PAGE);
        } else {
          const int popped = a.free_pages[top - 1 - rank];
          if (popped < 0 || (int64_t)popped >= a.n_pages)
            raise_err(a.err, PA_DEVERR_BAD_PAGE);
          else
            page = popped;
        }
      } else if (old_entry < 0 || (int64_t)old_entry >= a.n_pages) {
        raise_err(a.err, PA_DEVERR_BAD_PAGE);
      } else {
        page = old_entry;
      }
      page_s = page;
    }
  } else if (tid < 64 + kKvThreads) {
    // rotate K and copy V into the stage
    const int t = tid - 64;
    if (valid) {
      const int vchunks = (int)(row_bytes / 16);
      const u32x4 *vsrc = reinterpret_cast<const u32x4 *>(a.v + (int64_t)b * row_bytes);
      for (int c = t; c < vchunks; c += kKvThreads) stage[vchunks + c] = vsrc[c];
      rope_rows(a.k + (int64_t)b * row_bytes, reinterpret_cast<uint8_t *>(stage), a.Hkv, a.d, cs_row,
                sn_row, t, kKvThreads);
    }
  } else if (a.q_in && pos_ok) {
    // rotate the query
    const int t = tid - 64 - kKvThreads;
    rope_rows(a.q_in + (int64_t)b * a.Hq * a.d * 2, a.q_out + (int64_t)b * a.Hq * a.d * 2, a.Hq,
              a.d, cs_row, sn_row, t, kAppendThreads - 64 - kKvThreads);
  }
  __syncthreads();
  const int page = page_s;
  if (tid == 0 && opens) {
    // Every opener has read top before it arrives (its value was used above,
    // before the barrier, so the load has completed), and the last one to
    // arrive lowers it and resets the counter for the next call.  No fence:
    // an agent-scope fence here would write back this XCD's whole L2.
    if (atomicAdd(&a.alloc[1], 1) == total - 1) {
      atomicExch(&a.alloc[0], top > total ? top - total : 0);
      atomicExch(&a.alloc[1], 0);
    }
    if (page >= 0) {
      if (old_entry != -1) raise_err(a.err, PA_DEVERR_REASSIGNED);
      *entry = page;
    }
  }
  if (page < 0) return;
  uint8_t *kdst = a.pool + (int64_t)page * a.page_bytes + (int64_t)(pos % kPageTokens) * row_bytes;
  const int vchunks = (int)(row_bytes / 16);
  for (int c = tid; c < 2 * vchunks; c += kAppendThreads) {
    uint8_t *dst = kdst + (c < vchunks ? (int64_t)c * 16 : a.v_offset + (int64_t)(c - vchunks) * 16);
    *reinterpret_cast<u32x4 *>(dst) = stage[c];
  }
}

__global__ __launch_bounds__(kReleaseThreads) void kv_release_kernel(
    const int32_t *__restrict__ slots, int n, int32_t *__restrict__ block_table, int n_slots,
    int n_layers, int mbps, int32_t *__restrict__ free_pages, int capacity, int32_t *alloc,
    int32_t *err) {
  __shared__ int wave_cnt[kReleaseThreads / 64];
  __shared__ int top_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    const int t = alloc[0];
    top_s = t < 0 ? 0 : (t > capacity ? capacity : t);
  }
  // the released entries in push order (slot of the list, then layer, then
  // logical block) as one flat index; 1024 of them per pass
  const int per_slot = n_layers * mbps;
  const int64_t n_entries = (int64_t)n * per_slot;
  for (int64_t base = 0; base < n_entries; base += kReleaseThreads) {
    const int64_t j = base + tid;
    int e = -1;
    int32_t *ent = nullptr;
    if (j < n_entries) {
      const int i = (int)(j / per_slot);
      const int slot = slots[i];
      const int r = (int)(j - (int64_t)i * per_slot);
      if (slot >= 0 && slot < n_slots) {
        ent = block_table + (int64_t)slot * per_slot + r;
        e = *ent;
      } else if (r == 0) {
        raise_err(err, PA_DEVERR_BAD_SLOT);
      }
    }
    const bool keep = e != -1;
    const uint64_t m = __ballot(keep);
    const int before_in_wave = __popcll(m & ((1ull << lane) - 1));
    if (lane == 0) wave_cnt[wave] = __popcll(m);
    __syncthreads();
    int before = before_in_wave, cnt = 0;
    for (int w = 0; w < kReleaseThreads / 64; ++w) {
      const int c = wave_cnt[w];
      before += w < wave ? c : 0;
      cnt += c;
    }
    const int top = top_s;
    if (keep) {
      const int at = top + before;
      if (at < capacity) {
        free_pages[at] = e;
        *ent = -1;
      } else {
        raise_err(err, PA_DEVERR_STACK_FULL);
      }
    }
    __syncthreads();
    if (tid == 0) top_s = top + cnt < capacity ? top + cnt : capacity;
    __syncthreads();
  }
  if (tid == 0) alloc[0] = top_s;
}

int launch_kv_append(const void *k, const void *v, const void *q_in, void *q_out, int Hq, int B,
                     const int32_t *slot_ids, const int32_t *positions, const float *cos_t,
                     const float *sin_t, int max_pos, void *kv_cache, int64_t n_pages,
                     int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                     const int32_t *free_pages, int capacity, int32_t *alloc_state, int n_kv_heads,
                     int head_dim, int32_t *err, hipStream_t stream) {
  AppendArgs a;
  a.k = static_cast<const uint8_t *>(k);
  a.v = static_cast<const uint8_t *>(v);
  a.q_in = static_cast<const uint8_t *>(q_in);
  a.q_out = static_cast<uint8_t *>(q_out);
  a.slot_ids = slot_ids;
  a.positions = positions;
  a.cos_t = cos_t;
  a.sin_t = sin_t;
  a.pool = static_cast<uint8_t *>(kv_cache);
  a.block_table = block_table;
  a.free_pages = free_pages;
  a.alloc = alloc_state;
  a.capacity = capacity;
  a.err = err;
  a.n_pages = n_pages;
  a.page_bytes = 2LL * kPageTokens * n_kv_heads * head_dim * 2;
  a.v_offset = a.page_bytes / 2;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = n_kv_heads;
  a.d = head_dim;
  a.max_pos = max_pos;
  a.n_slots = n_slots;
  a.n_layers = n_layers;
  a.mbps = mbps;
  a.layer = layer;
  const size_t stage_bytes = 2 * (size_t)n_kv_heads * head_dim * 2;
  hipLaunchKernelGGL(kv_append_kernel, dim3(B), dim3(kAppendThreads), stage_bytes, stream, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int launch_kv_release(const int32_t *slots, int n, int32_t *block_table, int n_slots, int n_layers,
                      int mbps, int32_t *free_pages, int capacity, int32_t *alloc_state,
                      int32_t *err, hipStream_t stream) {
  hipLaunchKernelGGL(kv_release_kernel, dim3(1), dim3(kReleaseThreads), 0, stream, slots, n,
                     block_table, n_slots, n_layers, mbps, free_pages, capacity, alloc_state, err);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
