// prefill.hip -- attn_prefill / attn_prefill_dense: FlashAttention-2-style
// exact attention of whole prompts, K/V read through the block table (paged)
// or from contiguous tensors (dense).
//
// Algorithm (FlashAttention-2 explainer, "Step by step (the two forward
// tweaks)"): walk the key tiles of a query tile, keep a running max m and an
// unnormalised output, rescale both when m grows, divide by l once at the end
// and store LSE = m + ln l.  The exponentials are taken base 2 on scores
// pre-multiplied by scale*log2(e) (same values; v_exp_f32 is a base-2 unit).
// Causal tiles wholly above the diagonal are never visited and the mask is
// evaluated only on tiles that cross the diagonal or the sequence end
// (explainer, "causal mask" paragraph).
//
// Work split (explainer, "Parallelise along the sequence length" and "Work
// partitioning between warps"): one workgroup of four wavefronts owns a query
// tile of one GQA group; the grid is batch x head-group x query tile, all
// independent.  The four wavefronts split the queries (split-Q): with a group
// of four q heads they take the four heads of the same 32 rows, so a K/V tile
// staged once in LDS serves 4 x 32 query rows; with smaller groups they take
// more rows of fewer heads.  No wavefront ever reads another's results.
//
// Tile products on gfx950 bf16 MFMA with fp32 accumulation, 32x32x16 shape:
//   S^T[32 keys][32 rows] = K[32 keys][16 d] x Q^T[16 d][32 rows]
//   O^T[32 d][32 rows]   += V^T[32 d][16 keys] x P^T[16 keys][32 rows]
// Lane l owns query row l%32 throughout, so the row max, the exponentials and
// the row sum of P stay in-lane (one cross-half exchange per tile), and the
// probabilities a lane produces are already its B operand of the PV product.
// K is kept row-major in LDS (a 16-byte read gives an A operand); V is
// transposed when it is written to LDS so that the keys of a PV operand are
// contiguous.
//
// Workgroup order: consecutive workgroup ids go to different XCDs, so the id
// is remapped to keep every tile of one (sequence, head group) on one XCD
// (its K/V then stays in that XCD's L2), and causal query tiles are issued
// longest first.

#include "device.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct PrefillArgs {
  const uint16_t *q;           // [B][T][Hq][D]
  const uint8_t *pool;         // paged source
  int64_t n_pages;
  const int32_t *block_table;
  const int32_t *slot_ids;
  const int32_t *seq_lens;
  int n_slots, n_layers, mbps, layer;
  const uint16_t *k;           // dense source [B][T][Hkv][D]
  const uint16_t *v;
  int B, T, Hkv;
  float scale_log2;
  int causal;
  int n_hgroups;               // head groups per sequence
  int n_rowblocks;             // query tiles per sequence
  uint16_t *O;                 // [B][T][Hq][D]
  float *LSE;                  // [B][Hq][T]
  int32_t *err;
};

}  // namespace

template <int D, int G, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int HW = G < kWaves ? G : kWaves;      // heads per workgroup
  constexpr int RW = kWaves / HW;                  // 32-row blocks per workgroup
  constexpr int BM = 32 * RW;                      // query rows per workgroup
  constexpr int KROW = D + 8;                      // K row in LDS (bf16), padded
  constexpr int VROW = kBN + 2;                    // V^T row in LDS (bf16), padded
  constexpr int CH = D / 8;                        // 16-byte chunks per K/V row
  constexpr int NLD = kBN * CH / kThreads;         // 16-byte loads per thread per tile (K, and V)
  static_assert(NLD >= 1 && kBN * CH % kThreads == 0, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) uint16_t ks[kBN * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;      // query row within the wave's 32 rows
  const int lh = lane >> 5;      // lane half

  // ---- workgroup -> (sequence, head group, query tile)
  const int n_pairs = a.B * a.n_hgroups;
  const int wg = blockIdx.x;
  int pair, rank;
  if ((n_pairs & 7) == 0) {
    const int ppx = n_pairs >> 3;
    const int k8 = wg >> 3;
    rank = k8 / ppx;
    pair = (wg & 7) * ppx + k8 % ppx;
  } else {
    rank = wg / n_pairs;
    pair = wg % n_pairs;
  }
  const int rb = a.causal ? a.n_rowblocks - 1 - rank : rank;
  const int b = pair / a.n_hgroups;
  const int hg = pair % a.n_hgroups;
  const int Hq = a.Hkv * G;
  const int kvh = (hg * HW) / G;
  const int head = hg * HW + (wave % HW);
  const int row0 = rb * BM + 32 * (wave / HW);
  const int T = a.T;

  int len = T;
  PageTable pt{};
  if constexpr (PAGED) {
    len = a.seq_lens[b];
    if (len < 0 || len > T) {
      if (tid == 0 && hg == 0 && rb == 0) raise_err(a.err, PA_DEVERR_BAD_POS);
      len = len < 0 ? 0 : T;
    }
    const int slot = a.slot_ids ? a.slot_ids[b] : b;
    if (slot < 0 || slot >= a.n_slots) {
      if (tid == 0 && hg == 0 && rb == 0) raise_err(a.err, PA_DEVERR_BAD_SLOT);
      len = 0;
    }
    if (len > a.mbps * kPageTokens) {
      if (tid == 0 && hg == 0 && rb == 0) raise_err(a.err, PA_DEVERR_BAD_POS);
      len = a.mbps * kPageTokens;
    }
    pt.pool = a.pool;
    pt.row = a.block_table + ((int64_t)(len > 0 ? slot : 0) * a.n_layers + a.layer) * a.mbps;
    pt.n_pages = a.n_pages;
    pt.page_bytes = 2LL * kPageTokens * a.Hkv * D * 2;
    pt.v_offset = pt.page_bytes / 2;
    pt.mbps = a.mbps;
  }

  const int row = row0 + lr;
  const int wg_row_end = min(rb * BM + BM, len);
  const int kv_end = a.causal ? wg_row_end : len;
  const int n_tiles = (kv_end > 0 && rb * BM < len) ? (kv_end + kBN - 1) / kBN : 0;

  // ---- Q^T as B operands: lane holds row `row`, d = lh*(D/2) + ks*8 + i
  bf16x8 qf[D / 16];
  {
    const bool ok = row < len;
    const uint4 *qp = reinterpret_cast<const uint4 *>(
        a.q + (((int64_t)b * T + (ok ? row : 0)) * Hq + head) * D + lh * (D / 2));
#pragma unroll
    for (int k = 0; k < D / 16; ++k)
      qf[k] = __builtin_bit_cast(bf16x8, ok ? qp[k] : uint4{0u, 0u, 0u, 0u});
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float m_run = -INFINITY;
  float l_lane = 0.f;

  // ---- K/V tile loader: thread covers (key tid/CH + c*(256/CH), chunk tid%CH)
  uint4 kr[NLD], vr[NLD];
  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int c = 0; c < NLD; ++c) {
      const int idx = c * kThreads + tid;
      const int key = idx / CH;
      const int ch = idx % CH;
      const int j = kv0 + key;
      kr[c] = uint4{0u, 0u, 0u, 0u};
      vr[c] = uint4{0u, 0u, 0u, 0u};
      if (j < kv_end) {
        if constexpr (PAGED) {
          const int64_t page = pt.page(j / kPageTokens);
          if (page >= 0) {
            const uint8_t *p = pt.pool + page * pt.page_bytes +
                               (int64_t)(j % kPageTokens) * a.Hkv * D * 2 + (int64_t)kvh * D * 2 + ch * 16;
            kr[c] = *reinterpret_cast<const uint4 *>(p);
            vr[c] = *reinterpret_cast<const uint4 *>(p + pt.v_offset);
          }
        } else {
          const int64_t off = (((int64_t)b * T + j) * a.Hkv + kvh) * D + ch * 8;
          kr[c] = *reinterpret_cast<const uint4 *>(a.k + off);
          vr[c] = *reinterpret_cast<const uint4 *>(a.v + off);
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < NLD; ++c) {
      const int idx = c * kThreads + tid;
      const int key = idx / CH;
      const int ch = idx % CH;
      *reinterpret_cast<uint4 *>(&ks[key * KROW + ch * 8]) = kr[c];
      const uint32_t w[4] = {vr[c].x, vr[c].y, vr[c].z, vr[c].w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        vt[(ch * 8 + i) * VROW + key] = (uint16_t)(w[i / 2] >> (16 * (i % 2)));
    }
  };

  if (n_tiles > 0) load_tile(0);

  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = t * kBN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(kv0 + kBN);

    // pages of this tile that are needed but missing from the table: their
    // keys are left out (the same four table entries in every lane)
    uint32_t bad_pages = 0;
    if constexpr (PAGED) {
#pragma unroll
      for (int p = 0; p < kBN / kPageTokens; ++p) {
        const int blk = kv0 / kPageTokens + p;
        if (blk * kPageTokens < kv_end && pt.page(blk) < 0) bad_pages |= 1u << p;
      }
      if (bad_pages && tid == 0) raise_err(a.err, PA_DEVERR_BAD_PAGE);
    }

    // a wave whose rows all precede this tile sees none of it (causal)
    if (a.causal && kv0 > row0 + 31) continue;
    const bool need_mask = (a.causal && kv0 + kBN - 1 > row0) || (kv0 + kBN > len) || bad_pages;

    // S^T = K Q^T: two 32-key halves
    f32x16 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[h][r] = 0.f;
#pragma unroll
      for (int k = 0; k < D / 16; ++k) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&ks[(h * 32 + lr) * KROW + lh * (D / 2) + k * 8]);
        s[h] = mfma32(kf, qf[k], s[h]);
      }
    }

    // scale, mask, row max (lane holds keys h*32 + 8*(r/4) + 4*lh + r%4)
    float cmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[h][r] * a.scale_log2;
        if (need_mask) {
          const int j = kv0 + h * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
          const bool vis = j < len && (!a.causal || j <= row) &&
                           !((bad_pages >> ((j - kv0) / kPageTokens)) & 1u);
          x = vis ? x : -INFINITY;
        }
        s[h][r] = x;
        cmax = fmaxf(cmax, x);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const bool live = m_new != -INFINITY;
    const float corr = live ? fast_exp2(m_run - m_new) : 1.f;
    m_run = m_new;

    // P (bf16) as B operands of the PV product: 16 keys per operand
    bf16x8 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = live ? fast_exp2(s[h][r] - m_new) : 0.f;
        psum += p;
        pb[h * 2 + r / 8][r % 8] = (__bf16)p;
      }
    l_lane = l_lane * corr + psum;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] *= corr;

    // O^T += V^T P^T; operand kk covers keys 16kk..16kk+15, slot (lh*8 + i)
    // is key 16kk + 8*(i/4) + 4*lh + i%4
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint16_t *vrow = &vt[(mb * 32 + lr) * VROW + 16 * kk + 4 * lh];
        bf16x8 va;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          va[i] = __builtin_bit_cast(__bf16, vrow[i]);
          va[4 + i] = __builtin_bit_cast(__bf16, vrow[8 + i]);
        }
        acc[mb] = mfma32(va, pb[kk], acc[mb]);
      }
    }
  }

  // ---- epilogue: one divide per row, LSE in natural-log units
  float l_row = l_lane + __shfl_xor(l_lane, 32);
  const bool has = row < len && l_row > 0.f;
  const float inv_l = has ? 1.f / l_row : 0.f;
  if (row < T) {
    uint16_t *op = a.O + (((int64_t)b * T + row) * Hq + head) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = has ? pack_bf16x2(acc[mb][4 * g + 0] * inv_l, acc[mb][4 * g + 1] * inv_l) : 0u;
        w.y = has ? pack_bf16x2(acc[mb][4 * g + 2] * inv_l, acc[mb][4 * g + 3] * inv_l) : 0u;
        *reinterpret_cast<uint2 *>(op + mb * 32 + 8 * g + 4 * lh) = w;
      }
    if (lh == 0)
      a.LSE[((int64_t)b * Hq + head) * T + row] = has ? (m_run + fast_log2(l_row)) * kLn2 : -INFINITY;
  }
}

template <int D, int G, bool PAGED>
static int launch_prefill_t(PrefillArgs a, hipStream_t stream) {
  constexpr int HW = G < kWaves ? G : kWaves;
  constexpr int RW = kWaves / HW;
  constexpr int BM = 32 * RW;
  const int Hq = a.Hkv * G;
  a.n_hgroups = Hq / HW;
  a.n_rowblocks = (a.T + BM - 1) / BM;
  const int64_t grid = (int64_t)a.B * a.n_hgroups * a.n_rowblocks;
  if (grid == 0) return PA_OK;
  if (grid > 0x7fffffff) return PA_ERR_RANGE;
  hipLaunchKernelGGL((prefill_kernel<D, G, PAGED>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <bool PAGED>
static int dispatch_prefill(const PrefillArgs &a, int D, int G, hipStream_t stream) {
#define PA_PREFILL_CASE(DD, GG) \
  if (D == DD && G == GG) return launch_prefill_t<DD, GG, PAGED>(a, stream);
  PA_PREFILL_CASE(64, 1)
  PA_PREFILL_CASE(64, 2)
  PA_PREFILL_CASE(64, 4)
  PA_PREFILL_CASE(64, 8)
  PA_PREFILL_CASE(128, 1)
  PA_PREFILL_CASE(128, 2)
  PA_PREFILL_CASE(128, 4)
  PA_PREFILL_CASE(128, 8)
#undef PA_PREFILL_CASE
  return PA_ERR_UNSUPPORTED;
}

int launch_prefill_paged(const void *q, const void *kv_cache, int64_t n_pages,
                         const int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                         const int32_t *slot_ids, const int32_t *seq_lens, int B, int T, int Hq,
                         int Hkv, int D, float scale, int causal, void *O, float *LSE, int32_t *err,
                         hipStream_t stream) {
  PrefillArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.pool = static_cast<const uint8_t *>(kv_cache);
  a.n_pages = n_pages;
  a.block_table = block_table;
  a.slot_ids = slot_ids;
  a.seq_lens = seq_lens;
  a.n_slots = n_slots;
  a.n_layers = n_layers;
  a.mbps = mbps;
  a.layer = layer;
  a.B = B;
  a.T = T;
  a.Hkv = Hkv;
  a.scale_log2 = scale * kLog2e;
  a.causal = causal ? 1 : 0;
  a.O = static_cast<uint16_t *>(O);
  a.LSE = LSE;
  a.err = err;
  return dispatch_prefill<true>(a, D, Hq / Hkv, stream);
}

int launch_prefill_dense(const void *q, const void *k, const void *v, int B, int T, int Hq, int Hkv,
                         int D, float scale, int causal, void *O, float *LSE, hipStream_t stream) {
  PrefillArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.B = B;
  a.T = T;
  a.Hkv = Hkv;
  a.scale_log2 = scale * kLog2e;
  a.causal = causal ? 1 : 0;
  a.O = static_cast<uint16_t *>(O);
  a.LSE = LSE;
  return dispatch_prefill<false>(a, D, Hq / Hkv, stream);
}

}  // namespace pa
