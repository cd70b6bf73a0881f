// prefill.hip -- attn_prefill / attn_prefill_dense / attn_prefill_append:
// FlashAttention-2-style exact attention of whole prompts, K/V read through
// the block table (paged) or from contiguous tensors (dense; the storing
// instance behind attn_prefill_append also writes those rows to their pages,
// as the pages' prefill copies the K/V it has computed into the cache while
// attending to them: page "3. The prefill path").
//
// Algorithm (FlashAttention-2 explainer, "Step by step (the two forward
// tweaks)"): walk the key tiles of a query tile, keep a running max m and an
// unnormalised output, rescale both when m grows, divide by l once at the end
// and store LSE = m + ln l.  The exponentials are taken base 2 on scores
// pre-multiplied by scale*log2(e) (same values; v_exp_f32 is a base-2 unit).
// m need not be the exact running max: any reference value works as long as
// the exponentials neither overflow nor lose the row, so m is moved (and O, l
// rescaled) only on a row's first half tile or when some p of a half tile
// would reach 2^64; the others take p = 2^(s*c - m) against the old m, with
// no tile max.
// Causal tiles wholly above the diagonal are never visited and the mask is
// evaluated only on tiles that cross the diagonal or the sequence end
// (explainer, "causal mask" paragraph).
//
// Work split (explainer, "Parallelise along the sequence length" and "Work
// partitioning between warps"): one workgroup owns four 32-column blocks
// (query rows x heads) of one GQA group; the grid is batch x head-group x
// query tile, all independent.  The wavefronts split the queries (split-Q):
// with a group of four q heads the blocks are the four heads of the same 32
// rows, so a K/V tile staged once in LDS serves 4 x 32 query rows; with
// smaller groups they are more rows of fewer heads.  Each wavefront owns one
// block and never reads another's results.  A tile is taken as two 32-key
// halves one after the other, so that few registers are live: at d=64 the
// kernel fits 128 registers and 4 workgroups share a CU.
//
// Tile products on gfx950 bf16 MFMA with fp32 accumulation, 32x32x16 shape:
//   S^T[32 keys][32 rows] = K[32 keys][16 d] x Q^T[16 d][32 rows]
//   O^T[32 d][32 rows]   += V^T[32 d][16 keys] x P^T[16 keys][32 rows]
// Lane l owns query row l%32 throughout, so the row max, the exponentials and
// the row sum of P stay in-lane (one cross-half exchange per tile), and the
// probabilities a lane produces are already its B operand of the PV product.
//
// K/V staging: tiles go from HBM straight into LDS (global_load_lds, 16 bytes
// per lane, no staging registers) into a ring of NS stages, fetched NS-1
// tiles ahead.  Each wave fetches one 16-token page of every tile (one scalar
// block-table read per tile).  Rows are stored [key][16-byte chunk] with XOR
// swizzles chosen so that both the K operand reads and the transposing V
// reads are free of bank conflicts.
//
// Workgroup order: consecutive workgroup ids go to different XCDs, so the id
// is remapped to keep every tile of one (sequence, head group) on one XCD
// (its K/V then stays in that XCD's L2), and causal query tiles are issued
// longest first.

#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kBlocks = 4;     // 32-column (query row x head) blocks per workgroup

struct PrefillArgs {
  const uint16_t *q;           // [B][T][Hq][D]
  const uint8_t *pool;         // paged source
  int64_t n_pages;
  const int32_t *block_table;
  const int32_t *slot_ids;
  const int32_t *seq_lens;     // cached tokens (keys) per sequence
  const int32_t *q_lens;       // query rows per sequence, the last of its tokens (null: all)
  int n_slots, n_layers, mbps, layer;
  const uint16_t *k;           // dense source [B][T][Hkv][D]
  const uint16_t *v;
  int B, T, Hkv;
  float scale_log2;
  int causal;
  int n_hgroups;               // head groups per sequence
  int n_rowblocks;             // query tiles per sequence
  int layer_ranks;             // query-tile ranks per layer of one workgroup per CU
  uint16_t *O;                 // [B][T][Hq][D]  (packed: [total_q][Hq][D])
  float *LSE;                  // [B][Hq][T]     (packed: [total_q][Hq])
  int32_t *err;
  // packed rows (attn_prefill_packed): sequence b's queries are rows
  // q_start[b] .. q_start[b+1]-1 of q, O and LSE; workgroup i runs work item
  // work[6i..6i+5] = (b, row block, head group, first key tile, end key tile,
  // partial slot or -1); a split row block leaves its partial tile (O
  // normalised, then LSE, fp32) in part for the merge kernel.
  const int32_t *q_start;
  const int32_t *work;
  float *part;
  int64_t total_q;
  int64_t n_part_slots;        // partial tiles the workspace holds
  // attn_prefill_append: the same pool, writable; the prompt's K/V rows (k, v)
  // are also written to their pages
  uint8_t *pool_w;
};

}  // namespace

// LDS placement of the 16-byte chunks of a K or V row (XOR swizzles).
template <int D>
struct Swz {
  // K: chunk c of key j sits at c ^ k(j).  The QK operand reads (lanes 0..31
  // = 32 consecutive keys, same chunk) then hit distinct banks in every group
  // of 8 or 16 lanes.
  __device__ static int k(int key) { return D == 64 ? ((key & 7) ^ ((key >> 3) & 1)) : (key & 15); }
  // V: chunk c of key j sits at c ^ v(j); the transposing PV reads (4 keys x
  // 4 columns per 16-lane group) then hit 64 distinct banks.
  __device__ static int v(int key) { return 4 * ((key / (128 / D)) % (D / 32)); }
};

template <int D, int G, bool PAGED, int NS, int OCC, bool PACKED, bool STORE>
__global__ __launch_bounds__(64 * kBlocks, OCC) void prefill_kernel(PrefillArgs a) {
  static_assert(PAGED || !PACKED, "packed rows are read through the block table");
  static_assert(!(PAGED && STORE), "a storing prefill reads its K/V from the inputs");
  constexpr int NW = kBlocks;                      // waves per workgroup, one block each
  constexpr int HW = G < kBlocks ? G : kBlocks;    // heads per workgroup
  constexpr int RW = kBlocks / HW;                 // 32-row blocks per workgroup
  constexpr int BM = 32 * RW;                      // query rows per workgroup
  constexpr int CH = D / 8;                        // 16-byte chunks per K/V row
  constexpr int ROWB = D * 2;                      // bytes of one K/V row (one head)
  constexpr int TILEB = kBN * ROWB;                // bytes of one K (or V) tile
  constexpr int KPI = 64 / CH;                     // keys per 1-KB wave transfer
  constexpr int NDMA = TILEB / (NW * 1024);        // transfers per wave per tile, for K and for V
  constexpr int PPW = NDMA * KPI / kPageTokens;    // pages per wave per tile
  constexpr int TPP = kPageTokens / KPI;           // transfers per page
  static_assert(PPW >= 1 && PPW * kPageTokens == NDMA * KPI, "each wave fetches whole pages of every key tile");
  static_assert(NS >= 2 && NS <= 4, "LDS ring depth");
  // The running max m is only moved when some p = 2^(s*c - m) of a half tile
  // would reach 2^64: fp32 and bf16 hold such p exactly as well as p <= 1,
  // and O, l stay far from overflow, so most tiles skip the tile max and the
  // rescale altogether.  m starts at -1e30, so a row's first half tile with
  // a visible key always moves it.
  constexpr float kSpecLimit = 0x1p64f;
  constexpr float kMaxFloor = -1e30f;              // finite start of the running max
  constexpr int kStoreDevice = 16;                 // buffer-store cache policy: sc1 (device scope)


  // Ring of NS stages, each a K tile and a V tile ([key][chunk], swizzled).
  // Tile u lives in stage u % NS; it is fetched NS-1 tiles ahead of use.
  // Every tile buffer is a variable of its own so that the compiler can tell
  // the stages apart.
  __shared__ __attribute__((aligned(1024))) uint8_t lk0[TILEB], lv0[TILEB], lk1[TILEB], lv1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lk2[NS > 2 ? TILEB : 16], lv2[NS > 2 ? TILEB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lk3[NS > 3 ? TILEB : 16], lv3[NS > 3 ? TILEB : 16];
  auto kbuf = [&](auto S_) -> uint8_t * {
    constexpr int S = decltype(S_)::value;
    if constexpr (S == 0) return lk0;
    else if constexpr (S == 1) return lk1;
    else if constexpr (S == 2) return lk2;
    else return lk3;
  };
  auto vbuf = [&](auto S_) -> uint8_t * {
    constexpr int S = decltype(S_)::value;
    if constexpr (S == 0) return lv0;
    else if constexpr (S == 1) return lv1;
    else if constexpr (S == 2) return lv2;
    else return lv3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar branches)
  const int lr = lane & 31;      // query row within a 32-row block
  const int lh = lane >> 5;      // lane half
  const int l16 = lane & 15;     // lane within its 16-lane group
  const int g16 = lane >> 4;     // 16-lane group

  // ---- workgroup -> (sequence, head group, query tile)
  const int n_pairs = a.B * a.n_hgroups;
  const int wg = blockIdx.x;
  int pair = 0, rank = 0;
  int item_t0 = 0, item_t1 = 0x7fffffff, slot = -1;   // key tiles and partial slot (packed)
  if constexpr (PACKED) {
    const int32_t *it = a.work + 6 * (int64_t)wg;
    pair = it[0] * a.n_hgroups + it[2];
    rank = it[1];
    item_t0 = it[3];
    item_t1 = it[4];
    slot = it[5];
    // a work item naming no row block of this batch, or a slot past the
    // workspace: flagged, nothing read or written
    if (it[0] < 0 || it[0] >= a.B || it[2] < 0 || it[2] >= a.n_hgroups || rank < 0 || item_t0 < 0 ||
        item_t1 < item_t0 || slot < -1 || slot >= a.n_part_slots) {
      if (threadIdx.x == 0) raise_err(a.err, PA_DEVERR_BAD_PLAN);
      return;
    }
  } else if ((n_pairs & 7) == 0) {
    const int ppx = n_pairs >> 3;
    const int k8 = wg >> 3;
    rank = k8 / ppx;
    pair = (wg & 7) * ppx + k8 % ppx;
  } else {
    rank = wg / n_pairs;
    pair = wg % n_pairs;
  }
  if (!PACKED && a.causal && a.layer_ranks > 1) {
    // Workgroups are dispatched in id order, one per CU at a time, so the
    // ids fill the CUs in layers.  Causal tiles are taken longest first,
    // snaking over the layers (odd layers in reverse), so that the tiles
    // sharing a CU add up to about the same number of key tiles.
    const int L = a.layer_ranks;
    const int layer = rank / L, pos = rank % L;
    if (layer & 1) rank = layer * L + (min(L, a.n_rowblocks - layer * L) - 1 - pos);
  }
  const int rb = (a.causal && !PACKED) ? a.n_rowblocks - 1 - rank : rank;
  const int b = pair / a.n_hgroups;
  const int hg = pair % a.n_hgroups;
  const int Hq = a.Hkv * G;
  const int kvh = (hg * HW) / G;
  const int T = a.T;
  // this wave's column block: head hg*HW + wave%HW, rows row0 .. row0+31
  const int head = hg * HW + wave % HW;
  const int row0 = rb * BM + 32 * (wave / HW);
  const int wave_row_end = row0 + 31;

  int len = T;    // keys of this sequence (its cached tokens)
  int qlen = T;   // its query rows: the last qlen of its len tokens
  int64_t qstart = 0;   // packed: row of q / O / LSE holding its query row 0
  // Errors are collected here and reported once at the end.
  int err_bits = 0;
  const int64_t page_bytes = 2LL * kPageTokens * a.Hkv * ROWB;
  const uint32_t v_offset = (uint32_t)(page_bytes / 2);
  const int32_t *trow_v = nullptr;   // block-table row (vector reads)
  const_i32_ptr trow = nullptr;      // the same row (scalar reads)
  if constexpr (PAGED) {
    const bool reporter = hg == 0 && rb == 0;   // one workgroup per sequence reports
    len = a.seq_lens[b];
    if (len < 0 || (!PACKED && !a.q_lens && len > T)) {
      if (reporter) err_bits |= PA_DEVERR_BAD_POS;
      len = len < 0 ? 0 : T;
    }
    if constexpr (PACKED) {
      const int64_t s0 = a.q_start[b], s1 = a.q_start[b + 1];
      qstart = s0;
      qlen = (s0 < 0 || s1 < s0 || s1 > a.total_q) ? -1 : (int)min(s1 - s0, (int64_t)0x7fffffff);
      if (qlen < 0) {
        if (reporter) err_bits |= PA_DEVERR_BAD_POS;
        qlen = 0;
      }
    } else {
      qlen = a.q_lens ? a.q_lens[b] : len;
    }
    if (qlen < 0 || (!PACKED && qlen > T) || qlen > len) {
      if (reporter) err_bits |= PA_DEVERR_BAD_POS;
      qlen = qlen < 0 ? 0 : min(PACKED ? qlen : min(qlen, T), len);
    }
    const int slot = a.slot_ids ? a.slot_ids[b] : b;
    if (slot < 0 || slot >= a.n_slots) {
      if (reporter) err_bits |= PA_DEVERR_BAD_SLOT;
      len = 0;
      qlen = 0;
    }
    if (len > a.mbps * kPageTokens) {
      if (reporter) err_bits |= PA_DEVERR_BAD_POS;
      len = a.mbps * kPageTokens;
      qlen = min(qlen, len);
    }
    len = uniform(len);
    qlen = uniform(qlen);
    trow_v = a.block_table + ((int64_t)uniform(len > 0 ? slot : 0) * a.n_layers + a.layer) * a.mbps;
    trow = as_const(trow_v);
  }
  if constexpr (STORE) {
    // a whole prompt (query row t is token t) attended from the inputs k, v,
    // whose rows also go to the pages: length and slot checked as above
    const bool reporter = hg == 0 && rb == 0;
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
    qlen = len;
    trow_v = a.block_table + ((int64_t)uniform(len > 0 ? slot : 0) * a.n_layers + a.layer) * a.mbps;
    trow = as_const(trow_v);
  }

  // query row t is the token at position off + t (a chunk continuing a cached
  // prefix is aligned to the end of the sequence; off = 0 for a whole prompt)
  const int off = len - qlen;
  const int wg_row_end = min(rb * BM + BM, qlen);
  const int kv_end = a.causal ? off + wg_row_end : len;   // keys past this are never visible here
  const int n_tiles = (kv_end > 0 && rb * BM < qlen) ? (kv_end + kBN - 1) / kBN : 0;
  // key tiles of this workgroup: all of them, or (packed) the work item's share
  const int t_begin = PACKED ? min(item_t0, n_tiles) : 0;
  const int t_end = PACKED ? (slot < 0 ? n_tiles : min(item_t1, n_tiles)) : n_tiles;
  // a partial tile: O (normalised), then LSE, of BM rows x HW heads
  float *const part = PACKED && slot >= 0 ? a.part + (int64_t)slot * (BM * HW * (D + 1)) : nullptr;
  if constexpr (PACKED) {
    if (t_begin >= t_end) {
      // nothing to attend (a row block past the query rows, or a split past
      // the keys): an empty partial if one is expected, else nothing (packed
      // rows past a sequence's length do not exist)
      if (err_bits && tid == 0) raise_err(a.err, err_bits);
      if (part) {
        const int r = 32 * (wave / HW) + lr, h = wave % HW;
        float *op = part + (r * HW + h) * D;
        for (int d = lh; d < D; d += 2) op[d] = 0.f;
        if (lh == 0) part[BM * HW * D + r * HW + h] = -INFINITY;
      }
      return;
    }
  }
  if (n_tiles == 0) {
    // every row of this workgroup is padding (rows past the query length of a
    // short sequence in a padded batch): O = 0, LSE = -inf, nothing else
    if (err_bits && tid == 0) raise_err(a.err, err_bits);
    const int row = row0 + lr;
    if (row < T) {
      uint16_t *op = a.O + (((int64_t)b * T + row) * Hq + head) * D;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2 *>(op + mb * 32 + 8 * g + 4 * lh) = make_uint2(0u, 0u);
      if (lh == 0) a.LSE[((int64_t)b * Hq + head) * T + row] = -INFINITY;
    }
    return;
  }
  const int nblk = (kv_end + kPageTokens - 1) / kPageTokens;   // blocks read (paged)
  // A narrow row block (packed; a decode row, a short chunk tail): its rows
  // fit the 32 columns of one wave as HW heads x NR rows (column lr is head
  // lr / NR, row lr % NR).  Wave 0 then computes every head of the block and
  // the other waves only fetch their share of each tile, so a decode row costs
  // one wave's products per key tile instead of HW waves' with a single row.
  constexpr int NR = 32 / HW;
  const bool narrow = PACKED && HW > 1 && qlen - rb * BM <= NR;
  // this lane's query row and head; the last key its row may see (-1: a
  // padding row, sees nothing)
  const int row = narrow ? rb * BM + lr % NR : row0 + lr;
  const int head_l = narrow ? hg * HW + lr / NR : head;
  const int lim = row < qlen ? (a.causal ? off + row : len - 1) : -1;

  // ---- Q^T as B operands: lane holds row row0 + lr, d = lh*(D/2) + k*8 + e
  // A padding row (row >= qlen) takes the sequence's row 0 instead: its
  // results are never written (O = 0, LSE = -inf), and a real row keeps its
  // scores finite.  (Unconditional loads: no wait between them.)
  bf16x8 qf[D / 16];
  {
    const int64_t qrow = PACKED ? qstart + (row < qlen ? row : 0) : (int64_t)b * T + (row < qlen ? row : 0);
    const bf16x8 *qp = reinterpret_cast<const bf16x8 *>(a.q + (qrow * Hq + head_l) * D + lh * (D / 2));
#pragma unroll
    for (int k = 0; k < D / 16; ++k) qf[k] = qp[k];
  }

  // ---- pages: validated once for the whole workgroup.  A key that must not
  // count (past kv_end, or on a missing page) is fetched from a safe token
  // instead (token 0 of the first valid block the workgroup reads, or of pool
  // page 0 if there is none) so that its V row stays finite; its score is
  // masked.
  bool any_bad = false;
  int64_t safe_page = 0;
  int32_t raw0[PPW];   // first window of this wave's pages, read with the pass below
  if constexpr (PAGED || STORE) {
#pragma unroll
    for (int pp = 0; pp < PPW; ++pp) {
      const int blk = (64 * (t_begin >> 6) + lane) * (kBN / kPageTokens) + wave * PPW + pp;
      raw0[pp] = blk < nblk ? trow_v[blk] : -1;
    }
    // the blocks of this workgroup's key tiles, 64 entries of the table per
    // pass; a packed piece reads only its own range, four rows per pass with
    // their loads in flight together (measured on the whole-prompt grid, the
    // four-row pass is 1% slower there, so that one keeps a row per pass)
    const int blk_lo = PACKED ? t_begin * (kBN / kPageTokens) : 0;
    const int blk_hi = PACKED ? min(nblk, t_end * (kBN / kPageTokens)) : nblk;
    constexpr int NROW = PACKED ? 4 : 1;
    bool found = false;
    for (int b0 = blk_lo; b0 < blk_hi; b0 += 64 * NROW) {
      int p[NROW];
      bool in[NROW];
#pragma unroll
      for (int u = 0; u < NROW; ++u) {
        const int blk = b0 + 64 * u + lane;
        in[u] = blk < blk_hi;
        p[u] = in[u] ? trow_v[blk] : 0;
      }
#pragma unroll
      for (int u = 0; u < NROW; ++u) {
        const bool bad = in[u] && (p[u] < 0 || (int64_t)p[u] >= a.n_pages);
        const uint64_t badm = __ballot(bad);
        const uint64_t goodm = __ballot(in[u] && !bad);
        if (badm) any_bad = true;
        if (!found && goodm) {
          safe_page = __builtin_amdgcn_readlane(p[u], (int)__builtin_ctzll(goodm));
          found = true;
        }
      }
    }
    if (any_bad) err_bits |= PA_DEVERR_BAD_PAGE;
  }
  auto page_ok = [&](int blk) -> bool {   // only for blk < nblk
    const int32_t v = trow[blk];
    return v >= 0 && (int64_t)v < a.n_pages;
  };

  // ---- per-lane transfer offsets, the same for every tile.  Transfer i of
  // this wave carries tile keys kt = (wave*NDMA + i)*KPI + lane/CH, on page
  // wave*PPW + i/TPP of the tile, at key (i%TPP)*KPI + lane/CH of that page.
  // ksafe/vsafe: the same chunks of the safe token.  All of these stay in
  // registers for the whole kernel, so a transfer never waits on a register.
  const int64_t tok_bytes = (int64_t)a.Hkv * ROWB;   // one token, all KV heads
  uint32_t koff[NDMA], voff[NDMA], ksafe[NDMA], vsafe[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int kt = (wave * NDMA + i) * KPI + lane / CH;
    const int pos = lane % CH;
    const uint32_t kc = (uint32_t)(pos ^ Swz<D>::k(kt)) * 16;
    const uint32_t vc = (uint32_t)(pos ^ Swz<D>::v(kt)) * 16;
    if constexpr (PAGED) {
      const uint32_t h = (uint32_t)(kvh * ROWB);
      const uint32_t r = (uint32_t)(((i % TPP) * KPI + lane / CH) * tok_bytes);
      koff[i] = r + h + kc;
      voff[i] = v_offset + r + h + vc;
      ksafe[i] = h + kc;
      vsafe[i] = v_offset + h + vc;
    } else {
      koff[i] = (uint32_t)(kt * tok_bytes) + kc;
      voff[i] = (uint32_t)(kt * tok_bytes) + vc;
      ksafe[i] = kc;
      vsafe[i] = vc;
    }
  }

  // ---- byte offsets of this wave's pages, 64 tiles at a time (paged): lane
  // u holds the offset of its page of tile 64*win + u (the safe page's when
  // the page is missing or past the end); bit u of good_m / clean_m: the page
  // exists / every key on it counts.  One vector read of the block table per
  // 64 tiles; a tile then costs two lane reads.  Tiles are fetched in order,
  // so the window only moves forward.
  uint32_t off_lo[PPW], off_hi[PPW];
  uint64_t good_m[PPW], clean_m[PPW];
  int win = -1;
  // raw table entries of a window (-1 past nblk): read first, used later
  auto window_raw = [&](int w_, int32_t (&raw)[PPW]) {
#pragma unroll
    for (int pp = 0; pp < PPW; ++pp) {
      const int blk = (64 * w_ + lane) * (kBN / kPageTokens) + wave * PPW + pp;
      raw[pp] = blk < nblk ? trow_v[blk] : -1;
    }
  };
  auto window_set = [&](int w_, const int32_t (&raw)[PPW]) {
    win = w_;
#pragma unroll
    for (int pp = 0; pp < PPW; ++pp) {
      const int blk = (64 * w_ + lane) * (kBN / kPageTokens) + wave * PPW + pp;
      const bool good = blk < nblk && raw[pp] >= 0 && (int64_t)raw[pp] < a.n_pages;
      const int64_t page = good ? (int64_t)raw[pp] : safe_page;
      const bool clean = good && (blk + 1) * kPageTokens <= kv_end;
      const uint64_t off = (uint64_t)page * (uint64_t)page_bytes;
      off_lo[pp] = (uint32_t)off;
      off_hi[pp] = (uint32_t)(off >> 32);
      good_m[pp] = __ballot(good);
      clean_m[pp] = __ballot(clean);
    }
  };
  auto load_window = [&](int w_) {
    int32_t raw[PPW];
    window_raw(w_, raw);
    window_set(w_, raw);
  };
  const uint8_t *safe_base = a.pool + safe_page * page_bytes;

  // ---- fetch tile u (K and V) into stage S: 2*NDMA transfers per wave, always
  auto fetch = [&](int u, auto S_) {
    uint8_t *kdst = kbuf(S_) + wave * NDMA * 1024;
    uint8_t *vdst = vbuf(S_) + wave * NDMA * 1024;
    if constexpr (PAGED) {
      if ((u >> 6) != win) load_window(u >> 6);
    }
#pragma unroll
    for (int pp = 0; pp < PPW; ++pp) {
      const int key0 = u * kBN + (wave * PPW + pp) * kPageTokens;   // first key of the page
      const uint8_t *kb, *vb, *sk, *sv;                             // normal and safe bases
      bool page_good = true, clean;
      if constexpr (PAGED) {
        const int idx = u & 63;
        const uint64_t off = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(off_hi[pp], idx) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane(off_lo[pp], idx);
        page_good = (good_m[pp] >> idx) & 1;
        clean = (clean_m[pp] >> idx) & 1;
        kb = a.pool + off;
        vb = kb;
        sk = safe_base;
        sv = sk;
      } else {
        const int64_t base = (((int64_t)b * T + u * kBN) * a.Hkv + kvh) * ROWB;
        const int64_t safe = ((int64_t)b * T * a.Hkv + kvh) * ROWB;
        kb = reinterpret_cast<const uint8_t *>(a.k) + base;
        vb = reinterpret_cast<const uint8_t *>(a.v) + base;
        sk = reinterpret_cast<const uint8_t *>(a.k) + safe;
        sv = reinterpret_cast<const uint8_t *>(a.v) + safe;
        clean = key0 + kPageTokens <= kv_end;
      }
      if (clean) {
#pragma unroll
        for (int e = 0; e < TPP; ++e) {
          const int i = pp * TPP + e;
          dma16(kb, koff[i], kdst + i * 1024);
          dma16(vb, voff[i], vdst + i * 1024);
        }
      } else {
        // some keys of this page must not count: those lanes fetch the safe
        // token instead (two masked transfers; at least one per chunk runs;
        // the safe ones carry the non-temporal hint)
#pragma unroll
        for (int e = 0; e < TPP; ++e) {
          const int i = pp * TPP + e;
          const bool ok = page_good && key0 + e * KPI + lane / CH < kv_end;
          if (ok) {
            dma16(kb, koff[i], kdst + i * 1024);
            dma16(vb, voff[i], vdst + i * 1024);
          } else {
            dma16<1>(sk, ksafe[i], kdst + i * 1024);
            dma16<1>(sv, vsafe[i], vdst + i * 1024);
          }
        }
      }
    }
  };

  // ---- per-lane LDS read offsets (the stage and tile position are immediates)
  // QK: lane reads key h*32 + lr, chunk lh*(CH/2) + k; the swizzle of key
  // h*32 + lr depends on lr only.
  uint32_t kaddr[CH / 2];
#pragma unroll
  for (int k = 0; k < CH / 2; ++k)
    kaddr[k] = lr * ROWB + (uint32_t)(((lh * (CH / 2) + k) ^ Swz<D>::k(lr)) * 16);
  // PV: operand kk covers keys 16kk..16kk+15; contraction slot (lh*8 + e) is
  // key 16kk + 8*(e/4) + 4*lh + e%4.  Each half of the A operand is one
  // transposing LDS read: in 16-lane group g, lane L points at
  // V[key0 + L/4][d0 + 4*(L%4)] and receives V[key0..key0+3][d0 + L].
  uint32_t vaddr[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    const int key = 4 * (g16 >> 1) + (l16 >> 2);   // + 16kk + 8half (swizzle unchanged)
    const int dcol = mb * 32 + 16 * (g16 & 1) + 4 * (l16 & 3);
    vaddr[mb] = key * ROWB + (uint32_t)((((dcol / 8) ^ Swz<D>::v(key)) * 16) + (dcol % 8) * 2);
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  float m_run = kMaxFloor;   // reference max of the row (log2 units)
  float l_lane = 0.f;        // this lane's half of l
  // first tile whose scores need the mask: the first tile holding a key past
  // the position of the block's first row (off + row0), or the tile that
  // crosses kv_end
  const int t_mask = min(a.causal ? (off + row0 + 1) / kBN : 0x7fffffff, kv_end / kBN);
  const float c = a.scale_log2;


  // ---- one key tile: S = K Q^T, online softmax, O^T += V^T P^T, as two
  // 32-key halves one after the other (each an online-softmax step), so that
  // only one half's scores and operands are live at a time.  The lane holds
  // keys kv0 + 32h + 8*(r/4) + 4*lh + r%4 of its row in s[r].
  // the last key any row of this wave may see: a 32-key half past it (the
  // half beyond the diagonal in the last tile of an even causal row block,
  // or past the end of the keys) is skipped, since all its scores are masked
  const int wave_last_key =
      uniform(min(kv_end - 1, a.causal ? off + (narrow ? rb * BM + NR - 1 : wave_row_end) : 0x7fffffff));
  auto compute = [&](int t, auto S_) {
    const uint8_t *kt = kbuf(S_);
    const uint8_t *vt = vbuf(S_);
    // mask: only tiles that cross a diagonal, kv_end or a missing page
    uint32_t bad_pages = 0;
    if constexpr (PAGED || STORE) {
      if (any_bad) {
#pragma unroll
        for (int p = 0; p < kBN / kPageTokens; ++p) {
          const int blk = t * (kBN / kPageTokens) + p;
          if (blk < nblk && !page_ok(blk)) bad_pages |= 1u << p;
        }
      }
    }
    const bool need_mask = (t >= t_mask) | (bad_pages != 0);
    const int rel = lim - (t * kBN + 4 * lh);   // key offset o is visible iff o <= rel
    // S^T = K Q^T of half h (CH/2 MFMAs, K from LDS)
    auto qk = [&](int h) {
      bf16x8 kf[CH / 2];
#pragma unroll
      for (int k = 0; k < CH / 2; ++k) kf[k] = *reinterpret_cast<const bf16x8 *>(kt + kaddr[k] + h * 32 * ROWB);
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
      // the matrix phases of a wave run at raised priority: a wave about to
      // feed the MFMA unit issues ahead of the waves in their vector phase
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int k = 0; k < CH / 2; ++k) s = mfma32(kf[k], qf[k], s);
      __builtin_amdgcn_s_setprio(0);
      return s;
    };
    auto vread = [&](int h, bf16x8 (&vop)[D / 32][2]) {
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          uint2 part[2];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint8_t *src = vt + vaddr[mb] + (32 * h + 16 * q + 8 * half) * ROWB;
            part[half] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                       (__attribute__((address_space(3))) i16x4 *)(src)));
          }
          vop[mb][q] = __builtin_bit_cast(bf16x8, u32x4{part[0].x, part[0].y, part[1].x, part[1].y});
        }
    };
    // mask, exponentials and PV of half h
    auto soft_pv = [&](f32x16 &s, int h) {
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = h * 32 + 8 * (r / 4) + (r % 4);
          s[r] = o <= rel ? s[r] : -INFINITY;
        }
        if (bad_pages) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int pidx = (h * 32 + 8 * (r / 4) + 4 * lh) / kPageTokens;
            s[r] = ((bad_pages >> pidx) & 1u) ? -INFINITY : s[r];
          }
        }
      }
      bf16x8 vop[D / 32][2];
      bf16x8 pb[2];
      auto exps = [&]() -> float {
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[r], c, -m_run));
          sum = r == 0 ? p : sum + p;   // (p >= 0: the same value as 0 + p, one add fewer)
          pb[r / 8][r % 8] = (__bf16)p;
        }
        return sum;
      };
      float ps = exps();
      if (__any(!(ps < kSpecLimit))) {
        float rmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) rmax = fmaxf(rmax, s[r]);
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax), __float_as_uint(rmax), false, false);
        rmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const float m_new = fmaxf(m_run, rmax * c);
        const float corr = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_lane *= corr;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mb][r] *= corr;
        ps = exps();
      }
      l_lane += ps;
      vread(h, vop);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) acc[mb] = mfma32(vop[mb][q], pb[q], acc[mb]);
      __builtin_amdgcn_s_setprio(0);
    };
    // both halves' QK products are issued first, so the second half's run on
    // the matrix unit while the first half's exponentials run; each half's V
    // operands are read after its exponentials (read before them, they would
    // push the wave past the 128 registers of four workgroups per CU)
    const bool half1 = t * kBN + 32 <= wave_last_key;
    f32x16 s0 = qk(0);
    f32x16 s1;
    if (half1) s1 = qk(1);
    soft_pv(s0, 0);
    if (half1) soft_pv(s1, 1);
  };

  // ---- the ring.  Step t: wait for this wave's transfers of tile t, barrier
  // (now every wave's transfers of tile t have landed and every wave is done
  // with tile t-1), fetch tile t+NS-1 into the stage tile t-1 used, compute t.
  // Every step issues its transfers, also for tiles past the end (they carry
  // the safe token), so the number in flight is the same on every path and
  // one constant wait is exact; the compiler's own bookkeeping then agrees
  // and adds no drain of its own.
  // last tile this wave's rows see (causal): later tiles are skipped
  const int t_last = narrow ? (wave != 0 ? -1 : a.causal ? (off + rb * BM + NR - 1) / kBN : 0x7fffffff)
                            : (a.causal ? (off + wave_row_end) / kBN : 0x7fffffff);
  auto skip = [&](int t) { return t > t_last; };
  auto step = [&](int t, auto S_) {
    constexpr int S = decltype(S_)::value;
    wait_vm_lgkm0<(NS - 2) * 2 * NDMA>();
    __builtin_amdgcn_s_barrier();
    fetch(t + NS - 1, std::integral_constant<int, (S + NS - 1) % NS>{});
    if (!skip(t)) compute(t, S_);
  };

  // Let Q land before the first K/V transfer is issued, so that no wait for
  // Q sits inside the loop (it would drain the transfers in flight).  (An
  // empty asm that takes the Q registers forces the wait; the Q loads and the
  // block-table reads above are in flight together until here.)
#pragma unroll
  for (int k = 0; k < D / 16; ++k) asm("" : "+v"(qf[k]));
  // (stages are numbered from the first tile of the range: tile t_begin + j
  // lives in stage j % NS)
  if (t_end > t_begin) {
    if constexpr (PAGED) window_set(t_begin >> 6, raw0);
    fetch(t_begin, std::integral_constant<int, 0>{});
    if constexpr (NS > 2) fetch(t_begin + 1, std::integral_constant<int, 1>{});
    if constexpr (NS > 3) fetch(t_begin + 2, std::integral_constant<int, 2>{});
    for (int t = t_begin;;) {
      step(t, std::integral_constant<int, 0>{});
      if (++t >= t_end) break;
      step(t, std::integral_constant<int, 1 % NS>{});
      if (++t >= t_end) break;
      if constexpr (NS > 2) {
        step(t, std::integral_constant<int, 2 % NS>{});
        if (++t >= t_end) break;
      }
      if constexpr (NS > 3) {
        step(t, std::integral_constant<int, 3 % NS>{});
        if (++t >= t_end) break;
      }
    }
    // no transfer may still be writing LDS when the workgroup ends
    wait_vm_lgkm0<0>();
  }

  // attn_prefill_append: the prompt's K and V rows of this workgroup's tokens
  // go to their pages, 16 bytes per lane, once per kv head (by the kv head's
  // first head group).  They are loaded here and stored after O, so that the
  // loads' latency passes while O is staged.  A missing page is flagged and
  // its rows are not written (its keys were masked above, as attn_prefill
  // masks them).
  constexpr int HPK = G > HW ? G / HW : 1;                   // head groups per kv head
  constexpr int NCP = STORE ? BM * 2 * CH / (64 * NW) : 1;   // 16-byte pieces per lane
  static_assert(!STORE || NCP * 64 * NW == BM * 2 * CH, "whole pieces per lane");
  u32x4 cp[NCP];
  const bool cp_on = STORE && hg % HPK == 0;
  if constexpr (STORE) {
    if (cp_on) {
#pragma unroll
      for (int j = 0; j < NCP; ++j) {
        const int ci = tid + j * 64 * NW;
        const int r = ci / (2 * CH), part = ci % (2 * CH);
        const int t = rb * BM + r;
        const uint16_t *src = (part >= CH ? a.v : a.k) + (((int64_t)b * T + t) * a.Hkv + kvh) * D + (part % CH) * 8;
        cp[j] = t < len ? *reinterpret_cast<const u32x4 *>(src) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  if (err_bits && tid == 0) raise_err(a.err, err_bits);

  // ---- epilogue: one divide per row, LSE in natural-log units.  O leaves
  // through LDS: the workgroup's tile (BM rows x HW heads x D, bf16; the HW
  // heads of a row are adjacent in O) is staged row by row in the ring's
  // first stage and stored with 16-byte writes covering whole rows, at device
  // scope (sc1), so the lines go out while other workgroups still compute
  // instead of staying dirty in L2 until the kernel ends.
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_lane), __float_as_uint(l_lane), false, false);
    const float l_row = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const bool has = row < qlen && l_row > 0.f;
    const float inv_l = has ? 1.f / l_row : 0.f;
    const float lse_row = has ? (m_run + fast_log2(l_row)) * kLn2 : -INFINITY;
    if constexpr (PACKED) {
      if (narrow) {
        // wave 0 holds every row of the block: O (or the partial) straight
        // from its registers, row lr % NR of the block, head lr / NR
        if (wave != 0) return;
        const int r = lr % NR, h = lr / NR;
        if (part) {
          float *op = part + (r * HW + h) * D;
#pragma unroll
          for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              float4 v;
              v.x = acc[mb][4 * g + 0] * inv_l;
              v.y = acc[mb][4 * g + 1] * inv_l;
              v.z = acc[mb][4 * g + 2] * inv_l;
              v.w = acc[mb][4 * g + 3] * inv_l;
              *reinterpret_cast<float4 *>(op + mb * 32 + 8 * g + 4 * lh) = v;
            }
          if (lh == 0) part[BM * HW * D + r * HW + h] = lse_row;
        } else if (row < qlen) {
          uint16_t *op = a.O + ((qstart + row) * Hq + head_l) * D;
#pragma unroll
          for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *reinterpret_cast<uint2 *>(op + mb * 32 + 8 * g + 4 * lh) =
                  make_uint2(pack_bf16x2(acc[mb][4 * g + 0] * inv_l, acc[mb][4 * g + 1] * inv_l),
                             pack_bf16x2(acc[mb][4 * g + 2] * inv_l, acc[mb][4 * g + 3] * inv_l));
          if (lh == 0) a.LSE[(qstart + row) * Hq + head_l] = lse_row;
        }
        return;
      }
      if (part) {
        // a split row block: this wave's 32 rows x 1 head, straight from the
        // registers (row r = 32*(wave/HW) + lr of the tile, head wave % HW)
        const int r = 32 * (wave / HW) + lr, h = wave % HW;
        float *op = part + (r * HW + h) * D;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float4 v;
            v.x = acc[mb][4 * g + 0] * inv_l;
            v.y = acc[mb][4 * g + 1] * inv_l;
            v.z = acc[mb][4 * g + 2] * inv_l;
            v.w = acc[mb][4 * g + 3] * inv_l;
            *reinterpret_cast<float4 *>(op + mb * 32 + 8 * g + 4 * lh) = v;
          }
        if (lh == 0) part[BM * HW * D + r * HW + h] = lse_row;
        return;
      }
      if (row < qlen && lh == 0) a.LSE[(qstart + row) * Hq + head] = lse_row;
    } else {
      if (row < T && lh == 0) a.LSE[((int64_t)b * Hq + head) * T + row] = lse_row;
    }
    constexpr int RB = HW * ROWB;   // bytes of one staged row
    constexpr int RC = RB / 16;     // its 16-byte chunks (chunk c sits at c ^ (row % 8))
    static_assert(RC % 8 == 0 && BM * RB == 2 * TILEB, "O tile = one ring stage");
    auto srow = [&](int r) -> uint8_t * { return r < BM / 2 ? lk0 + r * RB : lv0 + (r - BM / 2) * RB; };
    __syncthreads();   // every wave is done with the ring (its transfers have landed)
    {
      const int r = 32 * (wave / HW) + lr;
      uint8_t *dst = srow(r);
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = ((wave % HW) * D + mb * 32 + 8 * g) / 8;
          uint2 w;
          w.x = has ? pack_bf16x2(acc[mb][4 * g + 0] * inv_l, acc[mb][4 * g + 1] * inv_l) : 0u;
          w.y = has ? pack_bf16x2(acc[mb][4 * g + 2] * inv_l, acc[mb][4 * g + 3] * inv_l) : 0u;
          *reinterpret_cast<uint2 *>(dst + (c ^ (r & 7)) * 16 + 8 * lh) = w;
        }
    }
    __syncthreads();
    const int rows = min(BM, (PACKED ? qlen : T) - rb * BM);   // staged rows inside O
    const int64_t row_stride = (int64_t)Hq * ROWB;
    const int64_t orow0 = PACKED ? qstart + rb * BM : (int64_t)b * T + rb * BM;
    uint8_t *obase = reinterpret_cast<uint8_t *>(a.O) + (orow0 * Hq + hg * HW) * ROWB;
    const int64_t span = (int64_t)(rows - 1) * row_stride + RB;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(obase, (short)0, (int)min(span, (int64_t)0x7fffffff), 0x00020000);
    for (int ci = tid; ci < rows * RC; ci += 64 * NW) {
      const int r = ci / RC, cc = ci % RC;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(srow(r) + (cc ^ (r & 7)) * 16);
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)(r * row_stride) + cc * 16, 0, kStoreDevice);
    }
  }
  if constexpr (STORE) {
    // The rows a wave stores with one instruction (64 lanes / (2 CH) pieces
    // per row: 2 or 4 consecutive rows, starting at a multiple of that) lie on
    // one page, so the page is wave-uniform and the store goes through a
    // buffer resource over that page, at device scope like O's stores.
    constexpr int RPW = 64 / (2 * CH);   // rows per wave and piece
    static_assert(RPW >= 1 && kPageTokens % RPW == 0 && BM % RPW == 0, "a wave's rows on one page");
    if (cp_on) {
      bool bad = false;
#pragma unroll
      for (int j = 0; j < NCP; ++j) {
        const int ci = tid + j * 64 * NW;
        const int r = ci / (2 * CH), part = ci % (2 * CH);
        const int t = rb * BM + r;
        const int tw = rb * BM + uniform((64 * wave + j * 64 * NW) / (2 * CH));   // the wave's first row
        if (tw < len) {
          const int32_t e = trow[tw / kPageTokens];
          if (e >= 0 && (int64_t)e < a.n_pages) {
            const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
                a.pool_w + (int64_t)e * page_bytes, (short)0, (int)page_bytes, 0x00020000);
            const int off = (part >= CH ? (int)v_offset : 0) + (t % kPageTokens) * a.Hkv * ROWB + kvh * ROWB +
                            (part % CH) * 16;
            if (t < len) __builtin_amdgcn_raw_buffer_store_b128(cp[j], prs, off, 0, kStoreDevice);
          } else {
            bad = true;
          }
        }
      }
      if (bad && lane == 0) raise_err(a.err, PA_DEVERR_BAD_PAGE);
    }
  }
}


// Per head size: LDS ring depth and target workgroups per CU.  d=64 takes a
// 2-stage ring (32 KB of LDS) and fits 128 registers, so that 4 workgroups
// share a CU; d=128 keeps a 2-stage ring (64 KB) at 2 workgroups per CU.
template <int D>
struct PrefillCfg {
  static constexpr int NS = 2;
  static constexpr int OCC = D == 64 ? 4 : 2;
};

template <int D, int G, bool PAGED, bool STORE>
static int launch_prefill_t(PrefillArgs a, hipStream_t stream) {
  using C = PrefillCfg<D>;
  constexpr int HW = G < kBlocks ? G : kBlocks;
  constexpr int RW = kBlocks / HW;
  constexpr int BM = 32 * RW;
  const int Hq = a.Hkv * G;
  a.n_hgroups = Hq / HW;
  a.n_rowblocks = (a.T + BM - 1) / BM;
  const int64_t n_pairs = (int64_t)a.B * a.n_hgroups;
  a.layer_ranks = n_pairs > 0 ? (int)(device_cu_count() / n_pairs) : 0;
  const int64_t grid = (int64_t)a.B * a.n_hgroups * a.n_rowblocks;
  if (grid == 0) return PA_OK;
  if (grid > 0x7fffffff) return PA_ERR_RANGE;
  hipLaunchKernelGGL((prefill_kernel<D, G, PAGED, C::NS, C::OCC, false, STORE>), dim3((unsigned)grid),
                     dim3(64 * kBlocks), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <int D, int G>
static int launch_prefill_packed_t(PrefillArgs a, int64_t n_work, hipStream_t stream) {
  using C = PrefillCfg<D>;
  constexpr int HW = G < kBlocks ? G : kBlocks;
  a.n_hgroups = a.Hkv * G / HW;
  if (n_work <= 0) return PA_OK;
  if (n_work > 0x7fffffffLL) return PA_ERR_RANGE;
  hipLaunchKernelGGL((prefill_kernel<D, G, true, C::NS, C::OCC, true, false>), dim3((unsigned)n_work),
                     dim3(64 * kBlocks), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <bool PAGED, bool STORE = false>
static int dispatch_prefill(const PrefillArgs &a, int D, int G, hipStream_t stream) {
#define PA_PREFILL_CASE(DD, GG) \
  if (D == DD && G == GG) return launch_prefill_t<DD, GG, PAGED, STORE>(a, stream);
  PA_PREFILL_CASE(64, 1)
  PA_PREFILL_CASE(64, 2)
  PA_PREFILL_CASE(64, 4)
  PA_PREFILL_CASE(64, 8)
  PA_PREFILL_CASE(64, 16)
  PA_PREFILL_CASE(128, 1)
  PA_PREFILL_CASE(128, 2)
  PA_PREFILL_CASE(128, 4)
  PA_PREFILL_CASE(128, 8)
  PA_PREFILL_CASE(128, 16)
#undef PA_PREFILL_CASE
  return PA_ERR_UNSUPPORTED;
}

int launch_prefill_paged(const void *q, const void *kv_cache, int64_t n_pages,
                         const int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                         const int32_t *slot_ids, const int32_t *seq_lens, const int32_t *q_lens,
                         int B, int T, int Hq, int Hkv, int D, float scale, int causal, void *O,
                         float *LSE, int32_t *err, hipStream_t stream) {
  PrefillArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.pool = static_cast<const uint8_t *>(kv_cache);
  a.n_pages = n_pages;
  a.block_table = block_table;
  a.slot_ids = slot_ids;
  a.seq_lens = seq_lens;
  a.q_lens = q_lens;
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

int launch_prefill_packed(const void *q, const void *kv_cache, int64_t n_pages,
                          const int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                          const int32_t *slot_ids, const int32_t *kv_lens, const int32_t *q_start, int B,
                          int64_t total_q, int Hq, int Hkv, int D, float scale, int causal,
                          const int32_t *plan, int64_t n_work, int64_t n_merge, void *part,
                          int64_t n_part_slots, void *O, float *LSE, int32_t *err, hipStream_t stream) {
  PrefillArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.pool = static_cast<const uint8_t *>(kv_cache);
  a.n_pages = n_pages;
  a.block_table = block_table;
  a.slot_ids = slot_ids;
  a.seq_lens = kv_lens;
  a.n_slots = n_slots;
  a.n_layers = n_layers;
  a.mbps = mbps;
  a.layer = layer;
  a.B = B;
  a.T = 0;
  a.Hkv = Hkv;
  a.scale_log2 = scale * kLog2e;
  a.causal = causal ? 1 : 0;
  a.O = static_cast<uint16_t *>(O);
  a.LSE = LSE;
  a.err = err;
  a.q_start = q_start;
  a.work = plan;
  a.part = static_cast<float *>(part);
  a.total_q = total_q;
  a.n_part_slots = n_part_slots;
  const int G = Hq / Hkv;
  int rc = PA_ERR_UNSUPPORTED;
#define PA_PACKED_CASE(DD, GG) \
  if (D == DD && G == GG) rc = launch_prefill_packed_t<DD, GG>(a, n_work, stream);
  PA_PACKED_CASE(64, 1)
  PA_PACKED_CASE(64, 2)
  PA_PACKED_CASE(64, 4)
  PA_PACKED_CASE(64, 8)
  PA_PACKED_CASE(64, 16)
  PA_PACKED_CASE(128, 1)
  PA_PACKED_CASE(128, 2)
  PA_PACKED_CASE(128, 4)
  PA_PACKED_CASE(128, 8)
  PA_PACKED_CASE(128, 16)
#undef PA_PACKED_CASE
  if (rc != PA_OK) return rc;
  return launch_packed_merge(plan + 6 * n_work, n_merge, q_start, B, static_cast<const float *>(part),
                             n_part_slots, O, LSE, err, total_q, Hq, Hkv, D, stream);
}

int launch_prefill_store(const void *q, const void *k, const void *v, void *kv_cache, int64_t n_pages,
                         const int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                         const int32_t *slot_ids, const int32_t *seq_lens, int B, int T, int Hq, int Hkv,
                         int D, float scale, int causal, void *O, float *LSE, int32_t *err,
                         hipStream_t stream) {
  PrefillArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.pool = static_cast<const uint8_t *>(kv_cache);
  a.pool_w = static_cast<uint8_t *>(kv_cache);
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
  return dispatch_prefill<false, true>(a, D, Hq / Hkv, stream);
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
