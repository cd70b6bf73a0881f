// decode.hip -- attn_decode: one query token per sequence against its whole
// paged context (tiny-vllm part 6, "pagedAttentionKernel" and "logical block
// -> physical block -> byte address"), the context split across wavefronts
// and the splits merged by the log-sum-exp rule (tiny-vllm part 3, "causalMask
// and online softmax": partial results are rescaled to the larger maximum and
// added).
//
// Work split.  A workgroup of kWaves wavefronts owns (sequence b, kv head,
// cross-split of the context); its wavefronts take interleaved chunks (two
// pages at d=64, one page at d=128: 8 KB of K and V either way) and merge
// their partial results through LDS at the end.  Only when the
// batch is too small to fill the GPU (few long sequences) is a context also
// split across workgroups, whose partials a small second kernel merges.
//
// The reference launches one 64-thread block per (sequence, q head), reads
// each kv head once per q head of its group, and reduces every single q.k over
// shuffles and two barriers.  Here the G = Hq/Hkv query heads of a group ride
// in the columns of one MFMA, so each K/V byte is read from HBM exactly once,
// and the tokens ride in its rows (v_mfma_f32_16x16x32_bf16):
//
//   S^T[16 tok][16 col] = K[16 tok][32 d] x Q^T[32 d][16 col]
//   O^T[16 d][16 col]  += V^T[16 d][32 tok] x P^T[32 tok][16 col]
//
// (d=128 takes one-page chunks, and its second product contracts over the 16
// tokens of the page on v_mfma_f32_16x16x16_bf16.)
//
// Column c carries q head (c mod G) of the group (columns repeat when G < 16).
// K rows go straight from the page into the A operand with 16-byte loads:
// lane l takes token l%16 and 16-byte pieces of its head row, four lanes per
// 128-byte row.  P^T needs no data movement: the 8 probabilities a lane holds
// after the first product are its B operand of the second one.  V^T needs the
// tokens along the contraction, so V is staged row-major in LDS (16-byte
// chunks XOR-swizzled per token against bank conflicts) and read back with
// the gfx950 transposing LDS read, 4 tokens of one d column per read.
//
// Pipeline.  Two register steps used in turn: the loads of a wavefront's
// next step are in flight while its current step is computed.  Exactly one
// step is in flight at the top of every iteration on every path (the last
// step is processed in a branch of its own), so the compiler's wait before a
// chunk's first use covers that chunk only, and nothing is loaded past the
// end.  A missing page is never dereferenced: its lanes read a safe page (the
// split's first valid one) instead and its tokens are masked.
//
// Order.  Workgroups are launched in id order into free slots; the r-th row
// of workgroups takes the r-th longest context, so the longest work starts
// first and the CUs finish together (contexts differ by up to 2048x).

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kChunk = 32;             // split granularity in tokens (a whole number of chunks)
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 8
#endif
#ifndef PA_DECODE_MIN_WAVES_PER_SIMD
#define PA_DECODE_MIN_WAVES_PER_SIMD 2
#endif
#ifndef PA_DECODE_SUB
#define PA_DECODE_SUB 1
#endif
constexpr int kWaves = PA_DECODE_WAVES;  // wavefronts per workgroup
constexpr float kRescaleSlack = 8.f;   // see prefill.hip: lazy max, p <= 2^8
constexpr float kMaxFloor = -1e30f;

// Batches up to this are scheduled longest context first.  Each workgroup
// ranks the B lengths itself (O(B) per lane); past 128 sequences the launch
// has enough workgroups that launch order matters less than that cost
// (B = 160 and 192 with the ranking: 93 / 121 us, without: 75 / 98 us).
constexpr int kSortMax = 128;

struct DecodeArgs {
  int B;
  const uint16_t *q;            // [B][Hq][D]
  const uint8_t *pool;
  int64_t n_pages;
  const int32_t *block_table;
  const int32_t *slot_ids;
  const int32_t *ctx_lens;
  int n_slots, n_layers, mbps, layer;
  int Hkv;
  float scale_log2;
  int max_ctx;
  int xsplit_tokens;            // tokens per workgroup split of a context
  int n_xsplits;                // workgroup splits per (sequence, kv head)
  float *ws_o;                  // [B][Hq][n_xsplits][D] normalised partials (n_xsplits > 1)
  float *ws_lse;                // [B][Hq][n_xsplits] partial LSE, natural log
  int32_t *ws_seg;              // whole-page path: [B][2] first partial slot, partial count
  uint16_t *out;                // [B][Hq][D]
  float *lse;                   // [B][Hq]
  int32_t *err;
  // attn_decode_append: the new token of every sequence, [B][Hkv][D] each,
  // written to its page (position ctx_lens[b] - 1) by the same launch
  const uint16_t *k_new, *v_new;
  uint8_t *pool_w;              // the pool, for those writes
};

// max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float rows_max(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <int D, int NH>
struct Chunk {
  u32x4 k[NH][D / 32];   // [16-token half][16-byte piece]
  u32x4 v[NH][D / 32];
  bool ok[NH];           // the half's page exists
};

// Context length actually used for sequence b: bad lengths and slots are
// clamped and their error bits returned through *err_bits.
__device__ __forceinline__ int clamped_ctx(const DecodeArgs &a, int b, int *slot_out, int *err_bits) {
  int ctx = a.ctx_lens[b];
  const int slot = a.slot_ids ? a.slot_ids[b] : b;
  const bool slot_ok = slot >= 0 && slot < a.n_slots;
  if (!slot_ok) {
    *err_bits |= PA_DEVERR_BAD_SLOT;
    ctx = 0;
  }
  if (ctx < 0 || ctx > a.max_ctx || ctx > a.mbps * kPageTokens) {
    *err_bits |= PA_DEVERR_BAD_POS;
    ctx = ctx < 0 ? 0 : min(min(ctx, a.max_ctx), a.mbps * kPageTokens);
  }
  *slot_out = uniform(slot_ok ? slot : 0);
  return uniform(ctx);
}

}  // namespace

template <int D, int G, bool APPEND>
__global__ __launch_bounds__(64 * kWaves, PA_DECODE_MIN_WAVES_PER_SIMD) void decode_kernel(DecodeArgs a) {
  constexpr int kSub = D == 64 ? PA_DECODE_SUB : 1;   // chunks per step (registers: d=128 one)
  static_assert(D % 32 == 0 && 16 % G == 0, "unsupported shape");
  constexpr int P = D / 32;          // 16-byte pieces per lane per token row
  constexpr int CH = D / 8;          // 16-byte chunks per V row
  // tokens per chunk: two pages at d=64, one at d=128 (the same bytes, so the
  // same registers per chunk in flight)
  constexpr int NH = D == 128 ? 1 : 2;
  constexpr int CT = 16 * NH;
  __shared__ __attribute__((aligned(16))) uint16_t vl[kWaves][CT * D];
  __shared__ float red_o[kWaves][G][D];
  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];
  // chunk swizzle: the 8 token rows read together by a half-wave land on
  // 8 distinct 32-byte bank groups
  auto swz = [](int tok) { return 2 * ((tok / (128 / D)) % (CH / 2)); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15;        // MFMA row/column lane index
  const int lgrp = lane >> 4;        // MFMA k-group / output row group
  // ---- workgroup -> (sequence rank, kv head, split).  Sequences are taken
  // longest context first (rank r is the r-th longest sequence, ties by
  // index): workgroups are launched in id order into free slots, so this
  // schedules the longest work first and the CUs finish together.  Batches
  // above kSortMax keep the identity order.
  int xs, kvh, b;
  {
    const int per = a.Hkv * a.n_xsplits;   // workgroups of one sequence
    const int w = blockIdx.x;
    if ((a.B & 7) == 0) {
      // consecutive ids go to the 8 XCDs in turn: keep all the workgroups of
      // a sequence on one XCD (its pages are then read whole, every kv head
      // at about the same time, by that XCD)
      const int j = w >> 3;
      b = (j / per) * 8 + (w & 7);
      const int within = j % per;
      kvh = within / a.n_xsplits;
      xs = within % a.n_xsplits;
    } else {
      xs = w % a.n_xsplits;
      kvh = (w / a.n_xsplits) % a.Hkv;
      b = w / per;
    }
  }
  if (a.B <= kSortMax) {
    __shared__ int lens_s[kSortMax];
    __shared__ int sorted_b;
    auto key = [&](int x) { return x < 0 ? 0 : min(x, a.max_ctx); };
    for (int i = tid; i < a.B; i += 64 * kWaves) lens_s[i] = key(a.ctx_lens[i]);
    __syncthreads();
    // rank of sequence i = number of sequences ahead of it; S adjacent lanes
    // share one i, each counting every S-th j, and add up their counts
    constexpr int kT = 64 * kWaves;
    int S = 64;
    while (S > 1 && S * a.B > kT) S >>= 1;
    const int i = tid / S, s = tid % S;
    const int li = i < a.B ? lens_s[i] : 0;
    int rank = 0;
    if (i < a.B)
      for (int j = s; j < a.B; j += S) {
        const int lj = lens_s[j];
        rank += (lj > li) | ((lj == li) & (j < i));
      }
    for (int o = 1; o < S; o <<= 1) rank += __shfl_xor(rank, o);
    if (i < a.B && s == 0 && rank == b) sorted_b = i;
    __syncthreads();
    b = uniform(sorted_b);
  }
  const int Hq = a.Hkv * G;

  // Errors are collected here and reported once at the end: a global atomic
  // before the chunk loop would make the compiler treat the block table as
  // possibly clobbered and keep its (uniform) reads off the scalar unit.
  int err_bits = 0;
  int slot;
  const int ctx = clamped_ctx(a, b, &slot, &err_bits);
  const bool ctx_ok = err_bits == 0;         // neither the slot nor the length was cut
  if (xs != 0 || kvh != 0) err_bits = 0;     // one workgroup per sequence reports these
  const int t_begin = xs * a.xsplit_tokens;
  const int t_split = min(ctx, t_begin + a.xsplit_tokens);
  // attn_decode_append: the split holding the new token (position ctx-1)
  // streams its other tokens from the pages and takes the new one from
  // k_new / v_new after its chunk loop
  const int new_tok = ctx - 1;
  const bool has_new = APPEND && ctx_ok && new_tok >= t_begin && new_tok < t_split;
  const int t_end = has_new ? new_tok : t_split;   // the chunk loop's end

  const int32_t *trow = a.block_table + ((int64_t)slot * a.n_layers + a.layer) * a.mbps;
  const int64_t row_bytes = (int64_t)a.Hkv * D * 2;
  const int64_t page_bytes = row_bytes * 2 * kPageTokens;
  const int64_t v_offset = page_bytes / 2;
  // this lane's pieces inside a page: token lrow, kv head, 16 bytes at
  // p*64 + lgrp*16 of the head row for piece p, so that each load
  // instruction reads 64 contiguous bytes of every one of its 16 rows
  const int64_t lane_off = (int64_t)lrow * row_bytes + (int64_t)kvh * D * 2 + (int64_t)lgrp * 16;

  // Q^T as the B operand: column lrow -> q head kvh*G + lrow%G; the
  // contraction slots of piece p hold d = p*32 + lgrp*8 + i (as K's)
  bf16x8 qb[P];
  {
    const int hq = kvh * G + (lrow % G);
    const uint16_t *qp = a.q + ((int64_t)b * Hq + hq) * D + lgrp * 8;
#pragma unroll
    for (int p = 0; p < P; ++p) qb[p] = *reinterpret_cast<const bf16x8 *>(qp + p * 32);
  }

  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kMaxFloor;   // reference max (log2 units) of this lane's column
  float l_lane = 0.f;        // this lane's share of the column's exp-sum
  const float c = a.scale_log2;
  uint16_t *vw = vl[w];

  // ---- this wavefront's steps: step i covers the kSub chunks from token
  // t_begin + (w + kWaves*i)*CT*kSub
  const int stride = kWaves * CT * kSub;
  const int first_tok = t_begin + w * CT * kSub;
  const int n_my = first_tok < t_end ? (t_end - first_tok + stride - 1) / stride : 0;
  // block-table row read through the constant address space: a uniform
  // entry is then always a scalar load
  const const_i32_ptr trow_c = as_const(trow);
  // page the loads of a missing page or of a chunk past the end read
  // instead (their tokens never count): the split's first page, else page 0
  int64_t safe_page = 0;
  if (t_end > t_begin) {
    const int32_t e = trow_c[t_begin / kPageTokens];
    if (e >= 0 && (int64_t)e < a.n_pages) safe_page = e;
  }
  // The new token's K and V row of this kv head go to its page (wave 0 of
  // the split holding it, one 16-byte piece per lane); nothing in the launch
  // reads that write back.
  const int64_t new_row = ((int64_t)b * a.Hkv + kvh) * D;   // the new row in k_new / v_new
  if constexpr (APPEND) {
    if (has_new) {
      if (w == 0 && lane < 2 * (D / 8)) {
        const bool isv = lane >= D / 8;
        const int cc = isv ? lane - D / 8 : lane;
        const u32x4 x = *reinterpret_cast<const u32x4 *>((isv ? a.v_new : a.k_new) + new_row + 8 * cc);
        const int32_t e = trow_c[new_tok / kPageTokens];
        if (e >= 0 && (int64_t)e < a.n_pages) {   // a missing page is flagged after the chunk loop
          uint8_t *dst = a.pool_w + (int64_t)e * page_bytes + (isv ? v_offset : 0) +
                         (int64_t)(new_tok % kPageTokens) * row_bytes + (int64_t)kvh * D * 2 + 16 * cc;
          __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(dst));
        }
      }
    }
  }

  // Issue the loads of chunk i.  Every call issues the same loads, also past
  // the end, so that the number of loads in flight is the same on every path
  // and the compiler's wait before a chunk's use covers exactly that chunk.
  auto issue = [&](Chunk<D, NH> &r, int c0) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int first = c0 + 16 * h;
      int64_t page = -1;
      if (first < t_end) {                  // uniform: the same entry for every lane
        const int32_t e = trow_c[first / kPageTokens];
        page = (e < 0 || (int64_t)e >= a.n_pages) ? -1 : (int64_t)e;
        if (page < 0) err_bits |= PA_DEVERR_BAD_PAGE;
      }
      r.ok[h] = page >= 0;
      const uint8_t *base = a.pool + (page < 0 ? safe_page : page) * page_bytes + lane_off;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        r.k[h][p] = *reinterpret_cast<const u32x4 *>(base + p * 64);
        r.v[h][p] = *reinterpret_cast<const u32x4 *>(base + v_offset + p * 64);
      }
    }
  };

  auto process = [&](const Chunk<D, NH> &r, int c0) {
    bool tail = c0 + CT > t_end;
#pragma unroll
    for (int h = 0; h < NH; ++h) tail |= !r.ok[h];
    // stage V (token 16h + lrow, chunk 4p + lgrp), zero rows that must not count
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int tok = 16 * h + lrow;
      const bool keep = !tail || (r.ok[h] && c0 + tok < t_end);
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int ch = 4 * p + lgrp;
        *reinterpret_cast<u32x4 *>(&vw[tok * D + (ch ^ swz(tok)) * 8]) =
            keep ? r.v[h][p] : u32x4{0u, 0u, 0u, 0u};
      }
    }

    // S^T = K Q^T for the 16-token halves
    f32x4 s[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < P; ++p) s[h] = mfma16(__builtin_bit_cast(bf16x8, r.k[h][p]), qb[p], s[h]);
    }
    // the lane holds tokens c0 + 16h + 4*lgrp + i of its column
    if (tail) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool vis = r.ok[h] && (c0 + 16 * h + 4 * lgrp + i) < t_end;
          s[h][i] = vis ? s[h][i] : -INFINITY;
        }
    }
    float cmax = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
#pragma unroll
    for (int h = 1; h < NH; ++h) cmax = fmaxf(cmax, fmaxf(fmaxf(s[h][0], s[h][1]), fmaxf(s[h][2], s[h][3])));
    cmax = rows_max(cmax);
    const float mt = cmax * c;
    if (__any(mt > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mt);
      const float corr = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_lane *= corr;
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mb][i] *= corr;
    }
    __bf16 pv[4 * NH];
    float psum = 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(__builtin_fmaf(s[h][i], c, -m_run));
        psum += p;
        pv[4 * h + i] = (__bf16)p;
      }
    l_lane += psum;
    if constexpr (NH == 1) {
      // one page: O^T += V^T P^T on 16x16x16 products, contraction slot
      // 4*lgrp + k = token 4*lgrp + k (the lane's own probabilities)
      bf16x4 pb4;
#pragma unroll
      for (int i = 0; i < 4; ++i) pb4[i] = pv[i];
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb) {
        const int tok = 4 * lgrp + (lrow >> 2);
        const int d = 16 * mb + 4 * (lrow & 3);
        const uint16_t *src = &vw[tok * D + ((d / 8) ^ swz(tok)) * 8 + (d % 8)];
        const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(src));
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, __builtin_bit_cast(i16x4, pb4), acc[mb], 0, 0, 0);
      }
    } else {
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = pv[i];

    // O^T += V^T P^T.  Contraction slot lgrp*8 + 4*half + k is token
    // 16*half + 4*lgrp + k; one transposing read per half: lane lrow points at
    // V[16*half + 4*lgrp + lrow/4][16*mb + 4*(lrow%4)] and receives
    // V[16*half + 4*lgrp + k][16*mb + lrow], k = 0..3.
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      uint2 part[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int tok = 16 * half + 4 * lgrp + (lrow >> 2);
        const int d = 16 * mb + 4 * (lrow & 3);
        const uint16_t *src = &vw[tok * D + ((d / 8) ^ swz(tok)) * 8 + (d % 8)];
        part[half] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (__attribute__((address_space(3))) i16x4 *)(src)));
      }
      const bf16x8 va = __builtin_bit_cast(bf16x8, uint4{part[0].x, part[0].y, part[1].x, part[1].y});
      acc[mb] = mfma16(va, pb, acc[mb]);
    }
    }
  };

  {
    // ---- ring of register steps: step i is processed while step i+1 is in
    // flight.  A step is kSub chunks (kSub*32 tokens): the more bytes a step
    // moves, the fewer latency-bound steps a workgroup takes.
    struct Step {
      Chunk<D, NH> c[kSub];
    };
    Step r0, r1;
    auto issue_step = [&](Step &st, int i) {
  #pragma unroll
      for (int j = 0; j < kSub; ++j) issue(st.c[j], t_begin + ((w + kWaves * i) * kSub + j) * CT);
    };
    auto process_step = [&](Step &st, int i) {
  #pragma unroll
      for (int j = 0; j < kSub; ++j) {
        const int c0 = t_begin + ((w + kWaves * i) * kSub + j) * CT;
        if (c0 < t_end) process(st.c[j], c0);
      }
    };
    // Exactly one step is in flight at the top of every iteration, on every
    // path; the last step is processed in a branch of its own, with nothing
    // issued after it, so no load is made past the end.
    if (n_my > 0) {
      issue_step(r0, 0);
      for (int i = 0;;) {
        if (i + 1 >= n_my) {
          process_step(r0, i);
          break;
        }
        issue_step(r1, i + 1);
        process_step(r0, i);
        ++i;
        if (i + 1 >= n_my) {
          process_step(r1, i);
          break;
        }
        issue_step(r0, i + 1);
        process_step(r1, i);
        ++i;
      }
    }
  }

  if constexpr (APPEND) {
    if (has_new && w == 0) {
      // the new token: its score for this lane's column (the Q operand's d
      // order: d = p*32 + lgrp*8 + i, the four lanes of a column summed), the
      // exponential against the reference max, p * v_new into the output
      const int32_t e = trow_c[new_tok / kPageTokens];
      if (e < 0 || (int64_t)e >= a.n_pages) {
        err_bits |= PA_DEVERR_BAD_PAGE;   // masked, as a token on a missing page
      } else {
        const uint16_t *kn = a.k_new + new_row;
        const uint16_t *vn = a.v_new + new_row;
        float dot = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const bf16x8 kk = *reinterpret_cast<const bf16x8 *>(kn + p * 32 + lgrp * 8);
#pragma unroll
          for (int i = 0; i < 8; ++i) dot = __builtin_fmaf((float)qb[p][i], (float)kk[i], dot);
        }
        const float mt = rows_sum(dot) * c;
        if (__any(mt > m_run + kRescaleSlack)) {
          const float m_new = fmaxf(m_run, mt);
          const float corr = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_lane *= corr;
#pragma unroll
          for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mb][i] *= corr;
        }
        const float pn = fast_exp2(mt - m_run);
        if (lgrp == 0) l_lane += pn;   // one lane of the column counts it
#pragma unroll
        for (int mb = 0; mb < D / 16; ++mb) {
          const bf16x4 vv = *reinterpret_cast<const bf16x4 *>(vn + 16 * mb + 4 * lgrp);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mb][i] = __builtin_fmaf(pn, (float)vv[i], acc[mb][i]);
        }
      }
    }
  }

  if (err_bits && lane == 0) raise_err(a.err, err_bits);

  // ---- merge the wavefronts: unnormalised outputs, maxima and sums via LDS
  {
    const float l_tot = rows_sum(l_lane);
    if (lrow < G) {
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_o[w][lrow][mb * 16 + 4 * lgrp + i] = acc[mb][i];
      if (lgrp == 0) {
        red_m[w][lrow] = m_run;
        red_l[w][lrow] = l_tot;
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 64 * kWaves) {
    const int j = idx / D;
    const int d = idx % D;
    float M = kMaxFloor;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, red_m[v][j]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float sc = fast_exp2(red_m[v][j] - M);
      o += sc * red_o[v][j][d];
      L += sc * red_l[v][j];
    }
    const bool empty = !(L > 0.f);
    const float val = empty ? 0.f : o / L;
    const float lse_v = empty ? -INFINITY : (M + fast_log2(L)) * kLn2;
    const int64_t bh = (int64_t)b * Hq + kvh * G + j;
    if (a.n_xsplits == 1) {
      a.out[bh * D + d] = f32_to_bf16(val);
      if (d == 0) a.lse[bh] = lse_v;
    } else {
      a.ws_o[(bh * a.n_xsplits + xs) * D + d] = val;
      if (d == 0) a.ws_lse[bh * a.n_xsplits + xs] = lse_v;
    }
  }
}

// Merge the workgroup splits of one (sequence, q head): O = sum_i w_i O_i /
// sum_i w_i with w_i = exp(LSE_i - max LSE), LSE = max + ln(sum_i w_i).
// Splits past the end of a context hold LSE = -inf and weigh nothing.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a, int Hq) {
  const int64_t bh = blockIdx.x;
  const int lane = threadIdx.x;
  const float *lp = a.ws_lse + bh * a.n_xsplits;
  float M = -INFINITY;
  for (int i = 0; i < a.n_xsplits; ++i) M = fmaxf(M, lp[i]);
  constexpr int E = D / 64;
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    for (int i = 0; i < a.n_xsplits; ++i) {
      const float wgt = fast_exp2((lp[i] - M) * kLog2e);
      L += wgt;
      const float *op = a.ws_o + (bh * a.n_xsplits + i) * D;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] += wgt * op[lane + 64 * e];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) a.out[bh * D + lane + 64 * e] = f32_to_bf16(o[e] * inv);
  if (lane == 0) a.lse[bh] = L > 0.f ? M + fast_log2(L) * kLn2 : -INFINITY;
}


// ---- whole-page decode: 8 kv heads, head_dim 64, head groups up to 8 ------
//
// A token row of a page holds every kv head ([token][kv head][d], tiny-vllm
// part 6, "block contents"), 1 KB here.  Reading one head's 128-byte slice
// of each row, as decode_kernel does, HBM delivers far less than for whole
// rows (loads alone, the 64-sequence batch on MI355X: about 4.7 TB/s for the
// slices against 6.6 TB/s for whole rows).  So here a workgroup streams whole
// pages (K and V of every head, 32 KB) into LDS and each of its 8 wavefronts
// computes one kv head from them: S^T = K Q^T and O^T += V^T P^T on 16x16
// MFMAs with the G query heads of the group in the columns, as in
// decode_kernel, and the same online softmax.
//
// Work split: the pages of all sequences, in batch order, form one list;
// workgroup g takes pages [g*total/n_wg, (g+1)*total/n_wg), one workgroup per
// CU, so every CU streams the same bytes (to a page) in one round and no
// ordering by length is needed.  Every (sequence, workgroup) piece leaves
// its partial (normalised O, LSE) in workspace slot b + g, and a second
// kernel merges each sequence's slots by the log-sum-exp rule (tiny-vllm part
// 3, "causalMask and online softmax": partials rescaled to the larger
// maximum and added).
//
// Ring: NS stages of [K rows 16 x 1 KB][V rows 16 x 1 KB][Q, G KB], filled by
// direct global->LDS transfers NS-1 pages ahead; wave w transfers rows
// 4w..4w+3 of the 32 K/V rows on every step (also past the end, from a safe
// page), and Q row w % G of the page's sequence with the first page of each
// sequence piece only (every workgroup of a long context re-reading the same
// 4 KB of Q with each page concentrates its L2 lines).  The wait for a page
// then counts the transfers of the newer page in flight: 4, or 5 when that
// page carries Q.  Chunks of 16 bytes are XOR-swizzled per
// row so that the operand reads are free of bank conflicts: K chunk c of row
// t sits at c ^ (t & 15) (a K read, 16 rows of one chunk, hits the 16 chunks
// of one 256-byte group), V chunk c at c ^ 2(t & 7) (a transposing read, 8
// rows of one chunk pair per half wave, hits 8 distinct pairs).  A wave's
// logical chunks map to physical chunks no other wave reads, so a wave may
// zero its own V rows of tokens that must not count.
constexpr int kRowsMaxB = 512;
constexpr int kRowsList = 1024;   // pages of a workgroup's range resolved up front
#ifndef PA_ROWS_WGPC
#define PA_ROWS_WGPC 1
#endif
// workgroups per CU of the whole-page path (2 needs a 2-stage ring, groups up to 4)
template <int G>
constexpr int rows_wgpc() { return G <= 4 ? PA_ROWS_WGPC : 1; }

template <int G>
__global__ __launch_bounds__(512, rows_wgpc<G>()) void decode_rows_kernel(DecodeArgs a, int n_wg) {
  constexpr int D = 64, HKV = 8, ROW = HKV * D * 2;   // bytes of one token row
  constexpr int QB = G * ROW;                          // Q of one sequence (Hq x D bf16)
  constexpr int STAGE = 32 * ROW + QB;
  constexpr int NS = rows_wgpc<G>() == 2 ? 2 : G <= 4 ? 4 : 3;   // LDS: NS x (32 + G) KB
  constexpr int PAGE = 2 * kPageTokens * ROW;          // 32 KB
  constexpr int VOFF = PAGE / 2;
  static_assert(G >= 1 && G <= 8, "head group");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * STAGE];
  __shared__ int s_ctx[kRowsMaxB], s_start[kRowsMaxB], s_slot[kRowsMaxB];
  __shared__ int s_wsum[8];
  __shared__ int s_first;
  // physical page of each page of the range (-1: missing; the host sends only
  // batches whose ranges fit), resolved in one parallel pass before the ring
  // starts: a block-table read per page on the ring's path would stall the
  // transfers behind it on every scalar-cache miss
  __shared__ int s_page[kRowsList];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);     // wavefront = kv head
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  const int g = blockIdx.x;
  const int B = a.B;
  const int Hq = HKV * G;
  int err_bits = 0;

  // ---- lengths (cut as decode_kernel cuts them), slots, page counts and
  // their prefix sum over the batch
  int np = 0, seq_err = 0;
  if (tid < B) {
    int ctx = a.ctx_lens[tid];
    const int slot = a.slot_ids ? a.slot_ids[tid] : tid;
    const bool slot_ok = slot >= 0 && slot < a.n_slots;
    if (!slot_ok) {
      seq_err |= PA_DEVERR_BAD_SLOT;
      ctx = 0;
    }
    if (ctx < 0 || ctx > a.max_ctx || ctx > a.mbps * kPageTokens) {
      seq_err |= PA_DEVERR_BAD_POS;
      ctx = ctx < 0 ? 0 : min(min(ctx, a.max_ctx), a.mbps * kPageTokens);
    }
    s_ctx[tid] = ctx;
    s_slot[tid] = slot_ok ? slot : 0;
    np = (ctx + kPageTokens - 1) / kPageTokens;
  }
  int incl = np;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int x = s_wsum[v];
    before += v < w ? x : 0;
    total += x;
  }
  total = uniform(total);
  // workgroup g < n_eff = min(n_wg, total) takes pages [g*total/n_eff,
  // (g+1)*total/n_eff): floor or ceil of total/n_eff pages, at least one, so
  // the workgroups holding a sequence's pages are consecutive and each holds
  // some; page j is workgroup owner(j)'s; workgroups past n_eff have none
  const int n_eff = max(1, min(n_wg, total));
  auto first_of = [&](int gg) { return (int)(((int64_t)min(gg, n_eff) * total) / n_eff); };
  auto owner = [&](int j) { return (int)((((int64_t)j + 1) * n_eff - 1) / total); };
  const int lo = uniform(first_of(g));
  const int n_my = uniform(first_of(g + 1) - lo);
  if (tid < B) {
    const int start = before + incl - np;
    s_start[tid] = start;
    // the workgroup holding a sequence's first page reports its length and
    // slot errors and writes where its partials are (the first workgroup
    // does so for sequences without pages)
    const int gf = np > 0 ? owner(start) : 0;
    if (gf == g) {
      const int gl = np > 0 ? owner(start + np - 1) : -1;
      a.ws_seg[2 * tid] = tid + gf;
      a.ws_seg[2 * tid + 1] = gl - gf + 1;
      if (seq_err) raise_err(a.err, seq_err);
    }
    if (np > 0 && start <= lo && lo < start + np) s_first = tid;
  }
  __syncthreads();
  // the range's pages: sequence by binary search over the starts, then the
  // table entry, all threads' loads in flight together
  for (int i = tid; i < min(n_my, kRowsList); i += 512) {
    const int j = lo + i;
    int lo_b = 0, hi_b = B - 1;   // last sequence with start <= j and pages
    while (lo_b < hi_b) {
      const int mid = (lo_b + hi_b + 1) >> 1;
      if (s_start[mid] <= j) lo_b = mid; else hi_b = mid - 1;
    }
    // sequences without pages share the start of the next: step back to the
    // one that holds page j
    while (lo_b > 0 && s_ctx[lo_b] == 0) --lo_b;
    const int k = j - s_start[lo_b];
    const int32_t e = a.block_table[((int64_t)s_slot[lo_b] * a.n_layers + a.layer) * a.mbps + k];
    s_page[i] = (e >= 0 && (int64_t)e < a.n_pages) ? e : -1;
  }
  __syncthreads();

  auto pages_of = [&](int b) { return (uniform(s_ctx[b]) + kPageTokens - 1) / kPageTokens; };
  // next page of the list after (b, k); b == B past the last sequence
  auto advance = [&](int &b, int &k) {
    if (++k < pages_of(b)) return;
    k = 0;
    do {
      ++b;
    } while (b < B && pages_of(b) == 0);
  };

  // physical page u of the range, -1 when missing
  auto page_at = [&](int u) -> int32_t { return uniform(s_page[u]); };

  // ---- transfers of page u of the range (sequence b, block k; and, with_q,
  // the sequence's Q) into a stage
  auto fetch = [&](int u, int b, int k, bool real, bool with_q, int stage) {
    uint8_t *st = ring + stage * STAGE;
    int64_t page = 0;   // a missing page, or a step past the end: pool page 0 (masked)
    int qs = 0;
    if (real) {
      const int32_t e = page_at(u);
      if (e >= 0) page = e;
      qs = b;
    }
    const uint8_t *pbase = a.pool + page * PAGE;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t32 = 4 * w + r;       // K rows 0..15, then V rows 0..15
      const int t = t32 & 15;
      const bool isv = t32 >= 16;      // wave-uniform
      const int chunk = isv ? (lane ^ ((t & 7) << 1)) : (lane ^ (t & 15));
      dma16(pbase, (uint32_t)((isv ? VOFF : 0) + t * ROW + chunk * 16), st + t32 * ROW);
    }
    if (with_q) {
      const uint8_t *qbase = reinterpret_cast<const uint8_t *>(a.q) + (int64_t)qs * QB;
      dma16(qbase, (uint32_t)((w % G) * ROW + lane * 16), st + 32 * ROW + (w % G) * ROW);
    }
  };

  f32x4 acc[D / 16];
  bf16x8 qf[2];
  float m_run = kMaxFloor;
  float l_lane = 0.f;
  const float c = a.scale_log2;
  int cur_b = -1;

  // partial of the current sequence piece into slot cur_b + g
  auto flush = [&]() {
    const float l_tot = rows_sum(l_lane);
    if (lrow < G) {
      const int hq = w * G + lrow;
      const int64_t sidx = (int64_t)(cur_b + g) * Hq + hq;
      const bool empty = !(l_tot > 0.f);
      const float inv = empty ? 0.f : 1.f / l_tot;
      float *op = a.ws_o + sidx * D;
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = acc[mb][i] * inv;
        *reinterpret_cast<f32x4 *>(op + 16 * mb + 4 * lgrp) = v;
      }
      if (lgrp == 0) a.ws_lse[sidx] = empty ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
    }
  };

  auto compute = [&](int u, int b, int k, int stage) {
    const uint8_t *st = ring + stage * STAGE;
    if (b != cur_b) {
      cur_b = b;
      const uint8_t *qp = st + 32 * ROW + (w * G + lrow % G) * (D * 2) + lgrp * 16;
      qf[0] = *reinterpret_cast<const bf16x8 *>(qp);
      qf[1] = *reinterpret_cast<const bf16x8 *>(qp + 64);
      m_run = kMaxFloor;
      l_lane = 0.f;
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int ctx = uniform(s_ctx[b]);
    const bool ok = page_at(u) >= 0;
    if (!ok) err_bits |= PA_DEVERR_BAD_PAGE;
    const int nv = ok ? min(kPageTokens, ctx - kPageTokens * k) : 0;   // tokens that count
    // S^T = K Q^T: lane holds tokens 4*lgrp + i of column lrow
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int chunk = (8 * w + 4 * p + lgrp) ^ lrow;
      s = mfma16(*reinterpret_cast<const bf16x8 *>(st + lrow * ROW + chunk * 16), qf[p], s);
    }
    if (nv < kPageTokens) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = (4 * lgrp + i) < nv ? s[i] : -INFINITY;
      // rows of tokens that must not count (past the context, or a missing
      // page) may hold anything, NaN included: zero this head's V of them
      for (int j = lane; j < (kPageTokens - nv) * 8; j += 64) {
        const int t = nv + j / 8;
        const int chunk = (8 * w + j % 8) ^ ((t & 7) << 1);
        *reinterpret_cast<u32x4 *>(const_cast<uint8_t *>(st) + VOFF + t * ROW + chunk * 16) =
            u32x4{0u, 0u, 0u, 0u};
      }
    }
    float cmax = rows_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
    const float mt = cmax * c;
    if (__any(mt > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mt);
      const float corr = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_lane *= corr;
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mb][i] *= corr;
    }
    bf16x4 pb4;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pr = fast_exp2(__builtin_fmaf(s[i], c, -m_run));
      psum += pr;
      pb4[i] = (__bf16)pr;
    }
    l_lane += psum;
    // O^T += V^T P^T (16x16x16): lane lrow points at V[4*lgrp + lrow/4][16*mb +
    // 4*(lrow%4)] and receives V[4*lgrp + k][16*mb + lrow], k = 0..3
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const int t = 4 * lgrp + (lrow >> 2);
      const int d = 16 * mb + 4 * (lrow & 3);
      const int chunk = (8 * w + d / 8) ^ ((t & 7) << 1);
      const uint8_t *src = st + VOFF + t * ROW + chunk * 16 + (d % 8) * 2;
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(src));
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, __builtin_bit_cast(i16x4, pb4), acc[mb], 0, 0, 0);
    }
  };

  if (n_my > 0) {
    int fb = uniform(s_first), fk = lo - uniform(s_start[fb]);   // fetch cursor
    int cb = fb, ck = fk;                                         // compute cursor
    // Q goes with the first page of each sequence piece: the range's first
    // page and every page that opens a sequence
    int q_stages = 0;   // bit s: the page in stage s carries Q
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) {
      const bool wq = u < n_my && (u == 0 || fk == 0);
      q_stages |= wq ? 1 << u : 0;
      fetch(u, fb, fk, u < n_my, wq, u);
      if (u < n_my) advance(fb, fk);
    }
    for (int u = 0; u < n_my; ++u) {
      // this wave's transfers of page u have landed once only those of the
      // NS-2 newer pages are left (4 each, 5 with Q); after the barrier every
      // wave's have, and every wave is done with page u-1, whose stage the
      // next fetch refills
      int nq = 0;
#pragma unroll
      for (int j = 1; j <= NS - 2; ++j) nq += (q_stages >> ((u + j) % NS)) & 1;
      if constexpr (NS == 2) {
        wait_vm_lgkm0<0>();
      } else if constexpr (NS == 3) {
        if (nq) wait_vm_lgkm0<5>(); else wait_vm_lgkm0<4>();
      } else {
        if (nq == 2) wait_vm_lgkm0<10>(); else if (nq == 1) wait_vm_lgkm0<9>(); else wait_vm_lgkm0<8>();
      }
      __builtin_amdgcn_s_barrier();
      // a piece that ends here is written before the next transfers are
      // issued, so the wait above never has to wait for them
      if (cur_b >= 0 && cb != cur_b) flush();
      const int uf = u + NS - 1;
      const bool wq = uf < n_my && fk == 0;
      q_stages = (q_stages & ~(1 << (uf % NS))) | (wq ? 1 << (uf % NS) : 0);
      fetch(uf, fb, fk, uf < n_my, wq, uf % NS);
      if (uf < n_my) advance(fb, fk);
      compute(u, cb, ck, u % NS);
      advance(cb, ck);
    }
    if (cur_b >= 0) flush();
    // no transfer may still be writing LDS when the workgroup ends
    wait_vm_lgkm0<0>();
  }
  if (err_bits && lane == 0) raise_err(a.err, err_bits);
}

// Merge the partials of a sequence: O = sum_i w_i O_i / sum_i w_i, w_i =
// exp(LSE_i - max LSE), LSE = max + ln(sum_i w_i) per q head; no partial (an
// empty context): O = 0, LSE = -inf.  One workgroup per (sequence, 8 q heads):
// thread t owns 8 dimensions of one head (lanes 8h..8h+7 of each wave) and
// the partials i = t/64 mod 4, eight at a time with all their loads issued
// together, merged online (rescaled to the larger maximum); the four groups
// are merged through LDS.
__global__ __launch_bounds__(256) void decode_rows_combine_kernel(DecodeArgs a, int Hq) {
  constexpr int D = 64, NB = 8;
  __shared__ float s_m[4][64], s_l[4][64];
  __shared__ f32x4 s_o[4][64][2];
  const int hgroups = Hq / 8;
  const int b = blockIdx.x / hgroups;
  const int tid = threadIdx.x, lane = tid & 63, grp = tid >> 6;
  const int hq = (blockIdx.x % hgroups) * 8 + lane / 8;
  const int d0 = (lane % 8) * 8;
  const int s0 = a.ws_seg[2 * b], n = a.ws_seg[2 * b + 1];
  float M = -INFINITY, L = 0.f;
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = grp; i0 < n; i0 += 4 * NB) {
    float x[NB];
    f32x4 y0[NB], y1[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int i = i0 + 4 * k;
      const int64_t sidx = (int64_t)(s0 + min(i, n - 1)) * Hq + hq;
      x[k] = a.ws_lse[sidx];
      const f32x4 *op = reinterpret_cast<const f32x4 *>(a.ws_o + sidx * D + d0);
      y0[k] = op[0];
      y1[k] = op[1];
    }
    float mb = M;
#pragma unroll
    for (int k = 0; k < NB; ++k)
      if (i0 + 4 * k < n) mb = fmaxf(mb, x[k]);
    if (mb != -INFINITY) {
      const float corr = fast_exp2((M - mb) * kLog2e);   // M = -inf: 0
      L *= corr;
      o0 *= corr;
      o1 *= corr;
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const float wgt = i0 + 4 * k < n ? fast_exp2((x[k] - mb) * kLog2e) : 0.f;
        L += wgt;
        o0 += wgt * y0[k];
        o1 += wgt * y1[k];
      }
      M = mb;
    }
  }
  s_m[grp][lane] = M;
  s_l[grp][lane] = L;
  s_o[grp][lane][0] = o0;
  s_o[grp][lane][1] = o1;
  __syncthreads();
  if (grp == 0) {
    const float Mt = fmaxf(fmaxf(s_m[0][lane], s_m[1][lane]), fmaxf(s_m[2][lane], s_m[3][lane]));
    float Lt = 0.f;
    f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
    if (Mt != -INFINITY) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float wgt = fast_exp2((s_m[j][lane] - Mt) * kLog2e);
        Lt += wgt * s_l[j][lane];
        t0 += wgt * s_o[j][lane][0];
        t1 += wgt * s_o[j][lane][1];
      }
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    uint16_t *out = a.out + ((int64_t)b * Hq + hq) * D + d0;
    u32x4 pk;
    pk[0] = pack_bf16x2(t0[0] * inv, t0[1] * inv);
    pk[1] = pack_bf16x2(t0[2] * inv, t0[3] * inv);
    pk[2] = pack_bf16x2(t1[0] * inv, t1[1] * inv);
    pk[3] = pack_bf16x2(t1[2] * inv, t1[3] * inv);
    *reinterpret_cast<u32x4 *>(out) = pk;
    if (d0 == 0) a.lse[(int64_t)b * Hq + hq] = Lt > 0.f ? Mt + fast_log2(Lt) * kLn2 : -INFINITY;
  }
}

namespace {
struct Split {
  int tokens, n;                // tokens per workgroup split, splits per context
  int64_t o_bytes, lse_bytes;   // workspace parts (zero when n == 1)
};
Split split_policy(int B, int Hq, int Hkv, int D, int max_ctx) {
  // Split a context across workgroups only when the B * Hkv workgroups leave
  // CUs without one, and then into as many pieces as give every CU one
  // workgroup (a single round: 16 splits of the 4 x 16384 batch, two rounds,
  // ran 35.8 us against 34.0 us for 8), never below 2 chunks per wavefront.
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  Split s{};
  const int64_t groups = (int64_t)B * Hkv;
  const int64_t n_cu = device_cu_count();
  int64_t n = (n_cu + groups - 1) / groups;
  const int64_t min_tokens = 2LL * kWaves * kChunk;
  const int64_t n_max = max_ctx <= 0 ? 1 : (max_ctx + min_tokens - 1) / min_tokens;
  if (n > n_max) n = n_max;
  if (n < 1) n = 1;
  int64_t t = max_ctx <= 0 ? kChunk : (max_ctx + n - 1) / n;
  t = (t + kChunk - 1) / kChunk * kChunk;
  s.tokens = (int)t;
  s.n = max_ctx <= 0 ? 1 : (int)((max_ctx + t - 1) / t);
  if (s.n > 1) {
    s.o_bytes = up((int64_t)B * Hq * s.n * D * 4);
    s.lse_bytes = up((int64_t)B * Hq * s.n * 4);
  }
  return s;
}
}  // namespace

// The whole-page path: 8 kv heads of head_dim 64, head groups up to 8, up to
// kRowsMaxB sequences (its length scan holds one sequence per thread), not
// the appending variant; except where the batch makes one to two (sequence,
// kv head) units per CU, where decode_kernel's two rounds, longest context
// first, pair the units of a CU well and measured faster on MI355X (64
// sequences, ctx ~ U[1, 2048], 32/8/64: 36.1 against 37.3-37.7 us; at 16,
// 32, 128, 256 sequences and 4 x 16384 the whole-page path is 2-14% faster).
bool rows_path(int B, int Hq, int Hkv, int D, int max_ctx, bool append) {
#ifdef PA_ROWS_DISABLE
  return false;
#endif
  if (append || D != 64 || Hkv != 8 || Hq % Hkv != 0 || Hq / Hkv > 8 || B < 1 || B > kRowsMaxB) return false;
  const int64_t units = (int64_t)B * Hkv, n_cu = device_cu_count();
  // every workgroup's range fits the page list it resolves up front
  const int64_t pages = (int64_t)B * ((std::max(max_ctx, 0) + kPageTokens - 1) / kPageTokens);
  if (pages > (int64_t)kRowsList * n_cu) return false;
  return !(units > n_cu && units <= 2 * n_cu);
}

// Workgroups of the whole-page path: one per CU, fewer when the batch cannot
// have that many pages (so no range exceeds kRowsList pages: rows_path).
int rows_groups(int B, int G, int max_ctx) {
  const int64_t pages = (int64_t)B * ((max_ctx + kPageTokens - 1) / kPageTokens);
  const int wgpc = G <= 4 ? PA_ROWS_WGPC : 1;
  const int64_t n = std::min<int64_t>((int64_t)wgpc * device_cu_count(), pages);
  return (int)std::max<int64_t>(1, n);
}

namespace {
struct RowsWs {
  int64_t o_bytes, lse_bytes, seg_bytes;   // partials [slot][Hq][64], LSE [slot][Hq], [B][2]
};
RowsWs rows_ws(int B, int Hq, int n_wg) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t slots = (int64_t)n_wg + B;   // slot b + g, g < n_wg
  return RowsWs{up(slots * Hq * 64 * 4), up(slots * Hq * 4), up((int64_t)B * 2 * 4)};
}
}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int D, int max_ctx) {
  const Split s = split_policy(B, Hq, Hkv, D, max_ctx);
  int64_t need = s.o_bytes + s.lse_bytes;   // decode_kernel (also attn_decode_append's)
  if (rows_path(B, Hq, Hkv, D, max_ctx, false)) {
    const RowsWs r = rows_ws(B, Hq, rows_groups(B, Hq / Hkv, max_ctx));
    need = std::max<int64_t>(need, r.o_bytes + r.lse_bytes + r.seg_bytes);
  }
  return (size_t)need;
}

// ---- the workspace of attn_decode_noalloc: a static device array, one copy
// per GPU, held until the process ends.  Splits are only made while B * Hkv
// workgroups leave CUs idle, so on a 256-CU part the partials need at most
// G * (256 + B * Hkv) * (D + 1) * 4 bytes, under 4.3 MB; 8 MiB leaves room.
constexpr size_t kScratchBytes = 8u << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

size_t decode_scratch_bytes() { return kScratchBytes; }

void *decode_scratch_ptr() {
  // `scratch` names a host-side stand-in in host code: the device address of
  // the current GPU's copy is looked up once per device and kept.
  static std::mutex mu;
  static void *ptr[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

template <int D, int G>
static int launch_decode_t(DecodeArgs a, int B, hipStream_t stream) {
  const int64_t grid = (int64_t)B * a.Hkv * a.n_xsplits;
  if (grid > 0x7fffffff) return PA_ERR_RANGE;
  if (a.k_new)
    hipLaunchKernelGGL((decode_kernel<D, G, true>), dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, G, false>), dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  if (a.n_xsplits > 1) {
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(B * a.Hkv * G)), dim3(64), 0,
                       stream, a, a.Hkv * G);
    if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  }
  return PA_OK;
}

template <int G>
static int launch_decode_rows(DecodeArgs a, int B, int max_ctx, hipStream_t stream) {
  const int n_wg = rows_groups(B, G, max_ctx);
  hipLaunchKernelGGL((decode_rows_kernel<G>), dim3((unsigned)n_wg), dim3(512), 0, stream, a, n_wg);
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  hipLaunchKernelGGL(decode_rows_combine_kernel, dim3((unsigned)(B * G)), dim3(256), 0, stream, a, 8 * G);
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

int launch_decode(const void *q, const void *kv_cache, int64_t n_pages, const int32_t *block_table,
                  int n_slots, int n_layers, int mbps, int layer, const int32_t *slot_ids,
                  const int32_t *ctx_lens, int B, int Hq, int Hkv, int D, float scale, int max_ctx,
                  void *workspace, void *O, float *LSE, int32_t *err, hipStream_t stream,
                  const void *k_new, const void *v_new) {
  const Split s = split_policy(B, Hq, Hkv, D, max_ctx);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  DecodeArgs a{};
  a.B = B;
  a.q = static_cast<const uint16_t *>(q);
  a.pool = static_cast<const uint8_t *>(kv_cache);
  a.n_pages = n_pages;
  a.block_table = block_table;
  a.slot_ids = slot_ids;
  a.ctx_lens = ctx_lens;
  a.n_slots = n_slots;
  a.n_layers = n_layers;
  a.mbps = mbps;
  a.layer = layer;
  a.Hkv = Hkv;
  a.scale_log2 = scale * kLog2e;
  a.max_ctx = max_ctx;
  a.xsplit_tokens = s.tokens;
  a.n_xsplits = s.n;
  a.ws_o = s.n > 1 ? reinterpret_cast<float *>(ws) : nullptr;
  a.ws_lse = s.n > 1 ? reinterpret_cast<float *>(ws + s.o_bytes) : nullptr;
  a.out = static_cast<uint16_t *>(O);
  a.lse = LSE;
  a.err = err;
  a.k_new = static_cast<const uint16_t *>(k_new);
  a.v_new = static_cast<const uint16_t *>(v_new);
  a.pool_w = k_new ? static_cast<uint8_t *>(const_cast<void *>(kv_cache)) : nullptr;
  const int G = Hq / Hkv;
  if (rows_path(B, Hq, Hkv, D, max_ctx, k_new != nullptr)) {
    const RowsWs r = rows_ws(B, Hq, rows_groups(B, G, max_ctx));
    a.ws_o = reinterpret_cast<float *>(ws);
    a.ws_lse = reinterpret_cast<float *>(ws + r.o_bytes);
    a.ws_seg = reinterpret_cast<int32_t *>(ws + r.o_bytes + r.lse_bytes);
    if (G == 1) return launch_decode_rows<1>(a, B, max_ctx, stream);
    if (G == 2) return launch_decode_rows<2>(a, B, max_ctx, stream);
    if (G == 4) return launch_decode_rows<4>(a, B, max_ctx, stream);
    if (G == 8) return launch_decode_rows<8>(a, B, max_ctx, stream);
  }
#define PA_DECODE_CASE(DD, GG) \
  if (D == DD && G == GG) return launch_decode_t<DD, GG>(a, B, stream);
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
