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
  constexpr int CH = D / 8;                        // 16-byte chunks per K/V row
  constexpr int NLD = kBN * CH / kThreads;         // 16-byte loads per thread per tile (K, and V)
  constexpr int KTILE = kBN * KROW;                // bf16 elements of one K tile in LDS
  constexpr int VTILE = kBN * D;                   // bf16 elements of one V tile in LDS
  static_assert(NLD >= 1 && kBN * CH % kThreads == 0, "tile/thread mismatch");
  static_assert(kPageTokens % (64 / CH) == 0, "a wave load step must stay inside one page");
  // A running max is only raised when a row's tile max exceeds it by more
  // than this (log2 units), so most tiles skip the rescale; p stays <= 2^8.
  constexpr float kRescaleSlack = 8.f;
  constexpr float kMaxFloor = -1e30f;              // finite start of the running max

  // Two K and two V tiles: tile t+1 is written while tile t is read.
  // V is row-major [key][d] with its 16-byte chunks XOR-swizzled per key so
  // that the transposing reads of the PV operands hit 64 distinct banks.
  __shared__ __attribute__((aligned(16))) uint16_t ks[2 * KTILE];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2 * VTILE];
  auto vswz = [](int key) { return 4 * ((key / (128 / D)) % (CH / 4)); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;      // query row within the wave's 32 rows
  const int lh = lane >> 5;      // lane half
  const int l16 = lane & 15;     // lane within its 16-lane group
  const int g16 = lane >> 4;     // 16-lane group

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
  // Errors are collected here and reported once at the end: a global atomic
  // before the key loop would make the compiler treat the block table as
  // possibly clobbered and keep its (uniform) reads off the scalar unit.
  int err_bits = 0;
  // paged source of this sequence: table row and page geometry
  const int32_t *trow = nullptr;
  const int64_t page_bytes = 2LL * kPageTokens * a.Hkv * D * 2;
  const int64_t v_offset = page_bytes / 2;
  if constexpr (PAGED) {
    const bool reporter = hg == 0 && rb == 0;   // one workgroup per sequence reports
    len = a.seq_lens[b];
    if (len < 0 || len > T) {
      if (reporter) err_bits |= PA_DEVERR_BAD_POS;
      len = len < 0 ? 0 : T;
    }
    const int slot = a.slot_ids ? a.slot_ids[b] : b;
    if (slot < 0 || slot >= a.n_slots) {
      if (reporter) err_bits |= PA_DEVERR_BAD_SLOT;
      len = 0;
    }
    if (len > a.mbps * kPageTokens) {
      if (reporter) err_bits |= PA_DEVERR_BAD_POS;
      len = a.mbps * kPageTokens;
    }
    len = uniform(len);
    trow = a.block_table + ((int64_t)uniform(len > 0 ? slot : 0) * a.n_layers + a.layer) * a.mbps;
  }

  const int row = row0 + lr;
  const int wg_row_end = min(rb * BM + BM, len);
  const int kv_end = a.causal ? wg_row_end : len;
  const int n_tiles = (kv_end > 0 && rb * BM < len) ? (kv_end + kBN - 1) / kBN : 0;
  // last key this lane's row may see (-1: padding row, sees nothing)
  const int lim = row < len ? (a.causal ? row : len - 1) : -1;

  // ---- Q^T as B operands: lane holds row `row`, d = lh*(D/2) + k*8 + i
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
  float m_run = kMaxFloor;   // reference max of the row (log2 units)
  float l_lane = 0.f;        // this lane's half of the row's exp-sum
  const float c = a.scale_log2;

  // ---- physical page of logical block blk, -1 when missing.  Every lane of
  // a wave asks for the same block, so this is a scalar load.
  auto page_of = [&](int blk) -> int64_t {
    blk = uniform(blk);
    if (blk * kPageTokens >= kv_end || blk >= a.mbps) return -1;
    const int32_t v = trow[blk];
    return (v < 0 || (int64_t)v >= a.n_pages) ? -1 : (int64_t)v;
  };
  // In one load step the 64 lanes of a wave cover 64/CH consecutive keys of a
  // single page, so the page index is uniform per (step, wave).
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // ---- K/V tile loader: thread covers (key idx/CH, chunk idx%CH), idx = c*256 + tid
  uint4 kr[NLD], vr[NLD];
  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int cc = 0; cc < NLD; ++cc) {
      const int idx = cc * kThreads + tid;
      const int key = idx / CH;
      const int ch = idx % CH;
      const int j = kv0 + key;
      kr[cc] = uint4{0u, 0u, 0u, 0u};
      vr[cc] = uint4{0u, 0u, 0u, 0u};
      if constexpr (PAGED) {
        const int64_t page = page_of(kv0 / kPageTokens + ((cc * kThreads + 64 * wv) / CH) / kPageTokens);
        if (j < kv_end && page >= 0) {
          const uint8_t *src = a.pool + page * page_bytes +
                               (int64_t)(j % kPageTokens) * a.Hkv * D * 2 + (int64_t)kvh * D * 2 + ch * 16;
          kr[cc] = *reinterpret_cast<const uint4 *>(src);
          vr[cc] = *reinterpret_cast<const uint4 *>(src + v_offset);
        }
      } else {
        if (j < kv_end) {
          const int64_t off = (((int64_t)b * T + j) * a.Hkv + kvh) * D + ch * 8;
          kr[cc] = *reinterpret_cast<const uint4 *>(a.k + off);
          vr[cc] = *reinterpret_cast<const uint4 *>(a.v + off);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int cc = 0; cc < NLD; ++cc) {
      const int idx = cc * kThreads + tid;
      const int key = idx / CH;
      const int ch = idx % CH;
      *reinterpret_cast<uint4 *>(&ks[buf * KTILE + key * KROW + ch * 8]) = kr[cc];
      *reinterpret_cast<uint4 *>(&vs[buf * VTILE + key * D + ((ch ^ vswz(key)) * 8)]) = vr[cc];
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
    if (n_tiles > 1) load_tile(kBN);
    __syncthreads();
  }

  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = t * kBN;
    const int buf = t & 1;
    uint32_t bad_pages = 0;    // needed pages of this tile missing from the table
    if constexpr (PAGED) {
#pragma unroll
      for (int p = 0; p < kBN / kPageTokens; ++p) {
        const int blk = kv0 / kPageTokens + p;
        if (blk * kPageTokens < kv_end && page_of(blk) < 0) bad_pages |= 1u << p;
      }
      if (bad_pages) err_bits |= PA_DEVERR_BAD_PAGE;
    }

    // a wave whose rows all precede this tile sees none of it (causal)
    if (!(a.causal && kv0 > row0 + 31)) {
      const uint16_t *kt = &ks[buf * KTILE];
      const uint16_t *vtile = &vs[buf * VTILE];
      // S^T = K Q^T: two 32-key halves
      f32x16 s[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[h][r] = 0.f;
#pragma unroll
        for (int k = 0; k < D / 16; ++k) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&kt[(h * 32 + lr) * KROW + lh * (D / 2) + k * 8]);
          s[h] = mfma32(kf, qf[k], s[h]);
        }
      }

      // mask: only tiles that cross the diagonal, the sequence end or a missing
      // page.  The lane holds keys kv0 + h*32 + 8*(r/4) + 4*lh + r%4.
      const bool need_mask = (kv0 + kBN - 1 > row0 && a.causal) | (kv0 + kBN > len) | (bad_pages != 0);
      if (need_mask) {
        const int rel = lim - (kv0 + 4 * lh);      // visible iff key offset <= rel
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = h * 32 + 8 * (r / 4) + (r % 4);
            s[h][r] = off <= rel ? s[h][r] : -INFINITY;
          }
        if (bad_pages) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int pidx = (h * 32 + 8 * (r / 4) + 4 * lh) / kPageTokens;
              s[h][r] = ((bad_pages >> pidx) & 1u) ? -INFINITY : s[h][r];
            }
        }
      }

      // tile row max of the raw scores (scale >= 0 keeps the order)
      float rmax = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) rmax = fmaxf(rmax, s[h][r]);
      rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
      const float mt = rmax * c;
      if (__any(mt > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mt);
        const float corr = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_lane *= corr;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] *= corr;
      }

      // P = 2^(s*c - m) (bf16) as B operands of the PV product: 16 keys each
      bf16x8 pb[4];
      float psum = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[h][r], c, -m_run));
          psum += p;
          pb[h * 2 + r / 8][r % 8] = (__bf16)p;
        }
      l_lane += psum;

      // O^T += V^T P^T.  Operand kk covers keys 16kk..16kk+15; contraction slot
      // (lh*8 + i) is key 16kk + 8*(i/4) + 4*lh + i%4.  Each half of the A
      // operand is one transposing LDS read: in 16-lane group g, lane L points
      // at V[key0 + L/4][d0 + 4*(L%4)] and receives V[key0..key0+3][d0 + L].
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
        const int dcol = mb * 32 + 16 * (g16 & 1) + 4 * (l16 & 3);   // this lane's 4 d values
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          uint2 part[2];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int key = 16 * kk + 8 * half + 4 * (g16 >> 1) + (l16 >> 2);
            const int ch = dcol / 8;
            const uint16_t *src = &vtile[key * D + ((ch ^ vswz(key)) * 8) + (dcol % 8)];
            part[half] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                       (__attribute__((address_space(3))) i16x4 *)(src)));
          }
          const bf16x8 va = __builtin_bit_cast(bf16x8, uint4{part[0].x, part[0].y, part[1].x, part[1].y});
          acc[mb] = mfma32(va, pb[kk], acc[mb]);
        }
      }
    }

    // stage tile t+1 into the other buffer, then prefetch tile t+2
    if (t + 1 < n_tiles) {
      store_tile(buf ^ 1);
      if (t + 2 < n_tiles) load_tile(kv0 + 2 * kBN);
    }
    __syncthreads();
  }

  if (err_bits && tid == 0) raise_err(a.err, err_bits);

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
