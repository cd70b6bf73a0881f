// decode.hip -- attn_decode: one query token per sequence against its whole
// paged context (tiny-vllm part 6, "pagedAttentionKernel" and "logical block
// -> physical block -> byte address"), with the context split across
// wavefronts and merged by the log-sum-exp rule (tiny-vllm part 3, "causalMask
// and online softmax": partial results are rescaled to the larger maximum and
// added).
//
// Work split.  One wavefront owns (sequence b, kv head, split of S tokens).
// The reference launches one 64-thread block per (sequence, q head), reads
// each kv head once per q head of its group, and reduces every single
// q.k over shuffles and two barriers.  Here the G = Hq/Hkv query heads of a
// group ride in the columns of one MFMA, so each K/V byte is read from HBM
// exactly once, and the tokens ride in its rows:
//
//   S^T[16 tok][16 col] = K[16 tok][32 d] x Q^T[32 d][16 col]   (v_mfma_f32_16x16x32_bf16)
//   O^T[16 d][16 col]  += V^T[16 d][32 tok] x P^T[32 tok][16 col]
//
// Column c carries q head (c mod G) of the group, so columns repeat when
// G < 16.  K rows are loaded straight from the page into the A operand with
// 16-byte loads: lane l takes token l%16 and 16-byte pieces of its head row,
// so four lanes cover one 128-byte row.  P^T needs no data movement: the
// 8 probabilities a lane holds after the first MFMA are exactly its B operand
// of the second one, once the contraction slots are assigned to the tokens
// that lane already holds.  V^T needs the tokens along the contraction, so the
// V chunk is staged through LDS (written as loaded, read back column-wise).
//
// Each chunk is 32 tokens (two pages).  Loads of chunk c+1 are issued before
// chunk c is computed, so every wave keeps 8 KB (K+V of two pages for one kv
// head) in flight while it works.

#include "device.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kChunk = 32;

template <int D>
struct ChunkRegs {
  // [half][piece]: D/32 16-byte pieces per token row per lane
  uint4 k[2][D / 32];
  uint4 v[2][D / 32];
};

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(64) void decode_partial_kernel(
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ pool, int64_t n_pages,
    const int32_t *__restrict__ block_table, int n_slots, int n_layers, int mbps, int layer,
    const int32_t *__restrict__ slot_ids, const int32_t *__restrict__ ctx_lens, int Hkv,
    float scale_log2, int max_ctx, int split_tokens, int n_splits, float *__restrict__ ws_o,
    float *__restrict__ ws_lse, int32_t *__restrict__ ws_nsplit, uint16_t *__restrict__ out,
    float *__restrict__ lse_out, int32_t *err) {
  static_assert(D % 32 == 0 && 16 % G == 0, "unsupported shape");
  constexpr int P = D / 32;          // 16-byte pieces per lane per token row
  constexpr int ROW = D + 8;         // LDS row (bf16 elements), padded against bank conflicts
  __shared__ __attribute__((aligned(16))) uint16_t vlds[kChunk * ROW];

  const int lane = threadIdx.x;
  const int lrow = lane & 15;        // MFMA row/column lane index
  const int lgrp = lane >> 4;        // MFMA k-group / output row group
  const int split = blockIdx.x % n_splits;
  const int rest = blockIdx.x / n_splits;
  const int kvh = rest % Hkv;
  const int b = rest / Hkv;
  const int Hq = Hkv * G;

  int ctx = ctx_lens[b];
  const int slot = slot_ids ? slot_ids[b] : b;
  if (slot < 0 || slot >= n_slots) {
    if (split == 0 && kvh == 0 && lane == 0) raise_err(err, PA_DEVERR_BAD_SLOT);
    ctx = 0;
  }
  if (ctx < 0 || ctx > max_ctx || ctx > mbps * kPageTokens) {
    if (split == 0 && kvh == 0 && lane == 0) raise_err(err, PA_DEVERR_BAD_POS);
    ctx = ctx < 0 ? 0 : min(min(ctx, max_ctx), mbps * kPageTokens);
  }
  const int my_splits = ctx == 0 ? 1 : (ctx + split_tokens - 1) / split_tokens;
  if (split >= my_splits) return;
  if (split == 0 && kvh == 0 && lane == 0) ws_nsplit[b] = my_splits;

  const int t_begin = split * split_tokens;
  const int t_end = min(ctx, t_begin + split_tokens);

  PageTable pt;
  pt.pool = pool;
  pt.row = block_table + ((int64_t)(slot < 0 || slot >= n_slots ? 0 : slot) * n_layers + layer) * mbps;
  pt.n_pages = n_pages;
  pt.page_bytes = 2LL * kPageTokens * Hkv * D * 2;
  pt.v_offset = pt.page_bytes / 2;
  pt.mbps = mbps;
  const int64_t row_bytes = (int64_t)Hkv * D * 2;
  // byte offset of this lane's pieces inside a page (token lrow, kv head, d-range)
  const int64_t lane_off = (int64_t)lrow * row_bytes + (int64_t)kvh * D * 2 + (int64_t)lgrp * (D / 4) * 2;

  // Q^T as the B operand: column lrow -> q head kvh*G + lrow%G; the lane's
  // contraction slots hold d = lgrp*(D/4) + piece*8 + i.
  bf16x8 qb[P];
  {
    const int hq = kvh * G + (lrow % G);
    const uint4 *qp = reinterpret_cast<const uint4 *>(q + ((int64_t)b * Hq + hq) * D + lgrp * (D / 4));
#pragma unroll
    for (int p = 0; p < P; ++p) qb[p] = __builtin_bit_cast(bf16x8, qp[p]);
  }

  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max (log2 units) of this lane's column
  float l_lane = 0.f;        // this lane's share of the column's exp-sum

  auto load_chunk = [&](int c0, ChunkRegs<D> &r, bool ok[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int first = c0 + 16 * h;
      int64_t page = -1;
      if (first < t_end) {
        page = pt.page(first / kPageTokens);
        if (page < 0 && lane == 0) raise_err(err, PA_DEVERR_BAD_PAGE);
      }
      ok[h] = page >= 0;
      const bool tok_ok = ok[h] && (first + lrow) < t_end;
      const uint8_t *base = pool + (page < 0 ? 0 : page) * pt.page_bytes + lane_off;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (tok_ok) {
          r.k[h][p] = *reinterpret_cast<const uint4 *>(base + p * 16);
          r.v[h][p] = *reinterpret_cast<const uint4 *>(base + pt.v_offset + p * 16);
        } else {
          r.k[h][p] = uint4{0u, 0u, 0u, 0u};
          r.v[h][p] = uint4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  ChunkRegs<D> cur, nxt;
  bool ok_cur[2], ok_nxt[2];
  if (t_begin < t_end) load_chunk(t_begin, cur, ok_cur);

  for (int c0 = t_begin; c0 < t_end; c0 += kChunk) {
    if (c0 + kChunk < t_end) load_chunk(c0 + kChunk, nxt, ok_nxt);

    // stage V rows in LDS: token (16h + lrow), d = lgrp*(D/4) + p*8 .. +8
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int p = 0; p < P; ++p)
        *reinterpret_cast<uint4 *>(&vlds[(16 * h + lrow) * ROW + lgrp * (D / 4) + p * 8]) = cur.v[h][p];

    // S^T = K Q^T for the two 16-token halves
    f32x4 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < P; ++p) s[h] = mfma16(__builtin_bit_cast(bf16x8, cur.k[h][p]), qb[p], s[h]);
    }

    // online softmax over the chunk (log2 domain); the lane holds tokens
    // 16h + 4*lgrp + r of column lrow
    float x[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = c0 + 16 * h + 4 * lgrp + r;
        const bool valid = ok_cur[h] && t < t_end;
        const float v = valid ? s[h][r] * scale_log2 : -INFINITY;
        x[4 * h + r] = v;
        cmax = fmaxf(cmax, v);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const bool live = m_new != -INFINITY;
    const float corr = live ? fast_exp2(m_run - m_new) : 1.f;
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = live ? fast_exp2(x[i] - m_new) : 0.f;
      psum += p;
      pb[i] = (__bf16)p;
    }
    l_lane = l_lane * corr + psum;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mb][r] *= corr;

    __syncthreads();
    // O^T += V^T P^T; contraction slot (lgrp*8 + i) is token 16*(i/4) + 4*lgrp + i%4
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      bf16x8 va;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = 16 * (i / 4) + 4 * lgrp + (i % 4);
        va[i] = __builtin_bit_cast(__bf16, vlds[t * ROW + mb * 16 + lrow]);
      }
      acc[mb] = mfma16(va, pb, acc[mb]);
    }
    __syncthreads();

    if (c0 + kChunk < t_end) {
      cur = nxt;
      ok_cur[0] = ok_nxt[0];
      ok_cur[1] = ok_nxt[1];
    }
  }

  // column totals: the four lane groups hold disjoint tokens of the column
  float l_tot = l_lane + __shfl_xor(l_lane, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const bool empty = !(l_tot > 0.f);
  const float inv_l = empty ? 0.f : 1.f / l_tot;
  const float lse = empty ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;

  if (lrow < G) {
    const int hq = kvh * G + lrow;
    const int64_t bh = (int64_t)b * Hq + hq;
    if (my_splits == 1) {
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb) {
        uint2 w;
        w.x = pack_bf16x2(acc[mb][0] * inv_l, acc[mb][1] * inv_l);
        w.y = pack_bf16x2(acc[mb][2] * inv_l, acc[mb][3] * inv_l);
        *reinterpret_cast<uint2 *>(out + bh * D + mb * 16 + 4 * lgrp) = w;
      }
      if (lgrp == 0) lse_out[bh] = lse;
    } else {
      float *dst = ws_o + (bh * n_splits + split) * D;
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb)
        *reinterpret_cast<float4 *>(dst + mb * 16 + 4 * lgrp) =
            float4{acc[mb][0] * inv_l, acc[mb][1] * inv_l, acc[mb][2] * inv_l, acc[mb][3] * inv_l};
      if (lgrp == 0) ws_lse[bh * n_splits + split] = lse;
    }
  }
}

// Merge the split partials of one (sequence, q head): O = sum_i w_i O_i / sum_i w_i,
// w_i = exp(LSE_i - max LSE), LSE = max + ln(sum_i w_i).
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_lse,
    const int32_t *__restrict__ ws_nsplit, int Hq, int n_splits, uint16_t *__restrict__ out,
    float *__restrict__ lse_out) {
  const int64_t bh = blockIdx.x;
  const int b = (int)(bh / Hq);
  const int n = ws_nsplit[b];
  if (n <= 1) return;
  const int lane = threadIdx.x;
  const float *lp = ws_lse + bh * n_splits;
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, lp[i]);
  constexpr int E = D / 64;
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    for (int i = 0; i < n; ++i) {
      const float w = fast_exp2((lp[i] - M) * kLog2e);
      L += w;
      const float *op = ws_o + (bh * n_splits + i) * D;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] += w * op[lane + 64 * e];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) out[bh * D + lane + 64 * e] = f32_to_bf16(o[e] * inv);
  if (lane == 0) lse_out[bh] = L > 0.f ? M + fast_log2(L) * kLn2 : -INFINITY;
}

int decode_split_tokens(int B, int max_ctx) {
  // Aim for a few thousand wavefronts over the batch; 32-token multiples.
  int64_t s = ((int64_t)B * max_ctx) / 512;
  s = (s + kChunk - 1) / kChunk * kChunk;
  if (s < 64) s = 64;
  if (s > 512) s = 512;
  return (int)s;
}

size_t decode_workspace_bytes(int B, int Hq, int D, int max_ctx) {
  const int split = decode_split_tokens(B, max_ctx);
  const int64_t n_splits = max_ctx <= 0 ? 1 : (max_ctx + split - 1) / split;
  const int64_t o = (int64_t)B * Hq * n_splits * D * 4;
  const int64_t l = (int64_t)B * Hq * n_splits * 4;
  const int64_t n = (int64_t)B * 4;
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  return (size_t)(up(o) + up(l) + up(n));
}

template <int D, int G>
static int launch_decode_t(const void *q, const void *kv_cache, int64_t n_pages,
                           const int32_t *block_table, int n_slots, int n_layers, int mbps,
                           int layer, const int32_t *slot_ids, const int32_t *ctx_lens, int B,
                           int Hkv, float scale, int max_ctx, void *workspace, void *O, float *LSE,
                           int32_t *err, hipStream_t stream) {
  const int Hq = Hkv * G;
  const int split = decode_split_tokens(B, max_ctx);
  const int n_splits = max_ctx <= 0 ? 1 : (max_ctx + split - 1) / split;
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  float *ws_o = reinterpret_cast<float *>(ws);
  float *ws_lse = reinterpret_cast<float *>(ws + up((int64_t)B * Hq * n_splits * D * 4));
  int32_t *ws_n = reinterpret_cast<int32_t *>(ws + up((int64_t)B * Hq * n_splits * D * 4) +
                                              up((int64_t)B * Hq * n_splits * 4));
  const int64_t grid = (int64_t)B * Hkv * n_splits;
  if (grid > 0x7fffffff) return PA_ERR_RANGE;
  hipLaunchKernelGGL((decode_partial_kernel<D, G>), dim3((unsigned)grid), dim3(64), 0, stream,
                     static_cast<const uint16_t *>(q), static_cast<const uint8_t *>(kv_cache),
                     n_pages, block_table, n_slots, n_layers, mbps, layer, slot_ids, ctx_lens, Hkv,
                     scale * kLog2e, max_ctx, split, n_splits, ws_o, ws_lse, ws_n,
                     static_cast<uint16_t *>(O), LSE, err);
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  if (n_splits > 1) {
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(B * Hq)), dim3(64), 0, stream,
                       ws_o, ws_lse, ws_n, Hq, n_splits, static_cast<uint16_t *>(O), LSE);
    if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  }
  return PA_OK;
}

int launch_decode(const void *q, const void *kv_cache, int64_t n_pages, const int32_t *block_table,
                  int n_slots, int n_layers, int mbps, int layer, const int32_t *slot_ids,
                  const int32_t *ctx_lens, int B, int Hq, int Hkv, int D, float scale, int max_ctx,
                  void *workspace, void *O, float *LSE, int32_t *err, hipStream_t stream) {
  const int G = Hq / Hkv;
#define PA_DECODE_CASE(DD, GG)                                                                  \
  if (D == DD && G == GG)                                                                       \
    return launch_decode_t<DD, GG>(q, kv_cache, n_pages, block_table, n_slots, n_layers, mbps,  \
                                   layer, slot_ids, ctx_lens, B, Hkv, scale, max_ctx, workspace, \
                                   O, LSE, err, stream);
  PA_DECODE_CASE(64, 1)
  PA_DECODE_CASE(64, 2)
  PA_DECODE_CASE(64, 4)
  PA_DECODE_CASE(64, 8)
  PA_DECODE_CASE(64, 16)
  PA_DECODE_CASE(128, 1)
  PA_DECODE_CASE(128, 2)
  PA_DECODE_CASE(128, 4)
  PA_DECODE_CASE(128, 8)
  PA_DECODE_CASE(128, 16)
#undef PA_DECODE_CASE
  return PA_ERR_UNSUPPORTED;
}

}  // namespace pa
