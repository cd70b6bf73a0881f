// packed.hip -- the work list of attn_prefill_packed (host) and the merge of
// its split row blocks (device).
//
// A packed batch holds the query rows of every sequence back to back: a
// prompt chunk continuing a cached prefix, a whole prompt, or a single
// decode row, all in one call (tiny-vllm part 6: every step of a sequence is
// attention of its new queries over all of its cached keys; FlashAttention-2
// explainer, "Parallelise along the sequence length").  The unit of work is
// a row block of one sequence (BM query rows x HW heads of one head group, as
// in the padded prefill) against its visible key tiles.  Row blocks of very
// different lengths share the GPU: a decode row sees up to its whole context,
// a chunk row block after a long prefix sees many more key tiles than one
// near the start of a prompt.  The planner cuts every row block into pieces
// of at most the even share of the batch's key tiles per CU (at least
// kMinSplitTiles tiles; a narrow row block, whose HW heads one wave computes,
// counts 1/HW of its tiles), so that no row block outlasts the rest by more than
// a share; each piece is a work item of its own, and the pieces of one row
// block leave partial results (O normalised, LSE) that the merge kernel
// combines by the log-sum-exp rule (tiny-vllm part 3, "causalMask and online
// softmax": rescale to the larger maximum and add).  A piece costs a start
// (Q, page offsets) and a partial tile written and read again.  Where the
// share leaves under two items per CU (a few long row blocks, as a chunk of
// 128 rows after 16384 cached tokens: one item per CU), it is halved until
// there are two (that chunk 37.9 -> 33.7 us); a mixed batch and two prompt
// chunks, with 3-4 items per CU already, are slower with half the share, and
// pieces sized to fill all four workgroup slots of a CU are slower on all
// three (the starts and the partial traffic outweigh the occupancy).
//
// Order.  Workgroup i runs on XCD i % 8, and the row blocks of one (sequence,
// head group) read the same K/V: the planner gives every (sequence, head
// group) to one XCD (groups dealt largest first to the least loaded XCD),
// sorts each XCD's items longest first, reverses every other layer of
// n_cu / 8 items (the items that start together, one per CU of the XCD), and
// interleaves the eight lists, so that each XCD's L2 holds the K/V of its own
// groups, the long items start first, and the items sharing a CU add up to
// about the same number of key tiles (long with short).
//
// The plan depends only on the lengths, so one plan serves every layer of a
// model step.

#include <algorithm>
#include <vector>

#include "device.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kTileKeys = 64;          // keys per tile of the prefill kernel
constexpr int kMinSplitTiles = 8;      // a piece holds at least this many key tiles
constexpr int kXcds = 8;               // workgroup i runs on XCD i % 8

struct Tile {
  int b, rb, hg, n_tiles;
};

}  // namespace

int prefill_rows_per_block(int G) { return 32 * (4 / std::min(G, 4)); }
int prefill_heads_per_block(int G) { return std::min(G, 4); }

int plan_prefill_packed(const int32_t *q_lens, const int32_t *kv_lens, int B, int Hq, int Hkv, int D,
                        int causal, int n_cu, int32_t *plan, int64_t capacity, int64_t *n_work,
                        int64_t *n_merge, size_t *part_bytes) {
  const int G = Hq / Hkv;
  const int HW = prefill_heads_per_block(G), BM = prefill_rows_per_block(G);
  const int n_hgroups = Hq / HW;
  std::vector<Tile> tiles;
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    const int ql = q_lens[b], kv = kv_lens[b];
    if (ql < 0 || kv < ql) return PA_ERR_SHAPE;
    const int off = kv - ql;
    for (int rb = 0; rb * BM < ql; ++rb) {
      const int row_end = std::min((rb + 1) * BM, ql);
      const int kv_end = causal ? off + row_end : kv;
      const int nt = (kv_end + kTileKeys - 1) / kTileKeys;
      if (nt == 0) continue;
      for (int hg = 0; hg < n_hgroups; ++hg) tiles.push_back({b, rb, hg, nt});
      // (a narrow row block -- rows that fit one wave as HW heads x 32/HW
      // rows -- computes with one of its HW waves: it counts 1/HW)
      const bool narrow = HW > 1 && row_end - rb * BM <= 32 / HW;
      total += (int64_t)nt * n_hgroups / (narrow ? HW : 1);
    }
  }
  // pieces per row block: at most the even share of key tiles per CU; while
  // that leaves fewer than two items per CU (a few long row blocks), the share
  // is halved (down to kMinSplitTiles), so that a CU runs two workgroups
  const int64_t cus = std::max(1, n_cu);
  int64_t share = std::max<int64_t>(kMinSplitTiles, (total + cus - 1) / cus);
  std::vector<int> pieces(tiles.size(), 1);
  for (;;) {
    int64_t n_items = 0;
    for (size_t i = 0; i < tiles.size(); ++i) {
      pieces[i] = (int)((tiles[i].n_tiles + share - 1) / share);
      n_items += pieces[i];
    }
    if (n_items >= 2 * cus || share <= kMinSplitTiles) break;
    share = std::max<int64_t>(kMinSplitTiles, (share + 1) / 2);
  }
  struct Item {
    int b, rb, hg, t0, t1, slot;
  };
  std::vector<Item> items;
  std::vector<int32_t> merges;
  int64_t n_slots = 0;
  for (size_t ti = 0; ti < tiles.size(); ++ti) {
    const Tile &t = tiles[ti];
    const int n = pieces[ti];
    if (n <= 1) {
      items.push_back({t.b, t.rb, t.hg, 0, t.n_tiles, -1});
      continue;
    }
    if (n_slots + n > 0x7fffffffLL) return PA_ERR_RANGE;
    for (int s = 0; s < n; ++s)
      items.push_back({t.b, t.rb, t.hg, (int)((int64_t)s * t.n_tiles / n), (int)((int64_t)(s + 1) * t.n_tiles / n),
                       (int)(n_slots + s)});
    merges.insert(merges.end(), {t.b, t.rb, t.hg, (int32_t)n_slots, n, 0});
    n_slots += n;
  }
  // (sequence, head group) -> XCD: groups largest first, each to the XCD
  // with the fewest key tiles so far (ties: the lower XCD)
  std::vector<int64_t> group_tiles((size_t)B * n_hgroups, 0);
  for (const Tile &t : tiles) group_tiles[(size_t)t.b * n_hgroups + t.hg] += t.n_tiles;
  std::vector<int> order;
  for (int g = 0; g < (int)group_tiles.size(); ++g)
    if (group_tiles[g] > 0) order.push_back(g);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return group_tiles[x] > group_tiles[y]; });
  std::vector<int> xcd_of(group_tiles.size(), 0);
  int64_t load[kXcds] = {};
  for (int g : order) {
    const int x = (int)(std::min_element(load, load + kXcds) - load);
    xcd_of[g] = x;
    load[x] += group_tiles[g];
  }
  // each XCD's items longest first (stable: ties keep sequence order), then
  // dealt in turn; a list that runs out leaves its turns to the longest others
  std::vector<Item> per[kXcds];
  for (const Item &it : items) per[xcd_of[(size_t)it.b * n_hgroups + it.hg]].push_back(it);
  const size_t layer = (size_t)std::max(1, n_cu / kXcds);
  for (auto &v : per) {
    std::stable_sort(v.begin(), v.end(), [](const Item &x, const Item &y) { return x.t1 - x.t0 > y.t1 - y.t0; });
    for (size_t l0 = layer; l0 < v.size(); l0 += 2 * layer)
      std::reverse(v.begin() + l0, v.begin() + std::min(v.size(), l0 + layer));
  }
  size_t next[kXcds] = {};
  std::vector<Item> dealt;
  dealt.reserve(items.size());
  for (size_t i = 0; i < items.size(); ++i) {
    int x = (int)(i % kXcds);
    if (next[x] >= per[x].size()) {
      int best = -1;
      for (int y = 0; y < kXcds; ++y)
        if (next[y] < per[y].size() && (best < 0 || per[y].size() - next[y] > per[best].size() - next[best]))
          best = y;
      x = best;
    }
    dealt.push_back(per[x][next[x]++]);
  }
  items.swap(dealt);
  *n_work = (int64_t)items.size();
  *n_merge = (int64_t)merges.size() / 6;
  *part_bytes = (size_t)n_slots * BM * HW * (D + 1) * sizeof(float);
  const int64_t need = 6 * (*n_work + *n_merge);
  if (!plan) return PA_OK;
  if (capacity < need) return PA_ERR_WORKSPACE;
  int32_t *p = plan;
  for (const Item &it : items) {
    p[0] = it.b;
    p[1] = it.rb;
    p[2] = it.hg;
    p[3] = it.t0;
    p[4] = it.t1;
    p[5] = it.slot;
    p += 6;
  }
  std::copy(merges.begin(), merges.end(), p);
  return PA_OK;
}

namespace {

struct MergeArgs {
  const int32_t *merge;     // [n_merge][6]: b, row block, head group, first slot, pieces, 0
  const int32_t *q_start;   // [B + 1]
  const float *part;        // per slot: O [BM * HW][D] (normalised), then LSE [BM * HW]
  uint16_t *O;              // [total_q][Hq][D]
  float *LSE;               // [total_q][Hq]
  int32_t *err;
  int64_t total_q, n_part_slots;
  int B, Hq, HW, BM;
};

// One workgroup per split row block and group of PPP (row, head) pairs of its
// 128 (BM x HW): D/8 lanes per pair, 8 values per lane.  O = sum_s w_s O_s /
// sum_s w_s with w_s = exp(LSE_s - max LSE), LSE = max + ln(sum_s w_s).  The
// lanes of a pair share the max over the pieces (each reads every LP-th
// piece's LSE), and the weighted sum takes four pieces per step with their
// loads in flight together.
template <int D>
__global__ __launch_bounds__(256) void packed_merge_kernel(MergeArgs a) {
  constexpr int LP = D / 8;          // lanes per pair
  constexpr int PPP = 256 / LP;      // pairs per workgroup
  constexpr int NP = 128;            // pairs per tile (BM * HW)
  constexpr int PT = NP * (D + 1);   // floats per partial tile
  static_assert(64 % LP == 0 && NP % PPP == 0, "a pair's lanes sit in one wave");
  const int32_t *it = a.merge + 6 * (int64_t)blockIdx.x;
  const int b = it[0], rb = it[1], hg = it[2], slot0 = it[3], n = it[4];
  if (b < 0 || b >= a.B || rb < 0 || hg < 0 || hg >= a.Hq / a.HW || slot0 < 0 || n < 1 ||
      (int64_t)slot0 + n > a.n_part_slots) {
    if (threadIdx.x == 0 && blockIdx.y == 0) raise_err(a.err, PA_DEVERR_BAD_PLAN);
    return;
  }
  const int64_t s0 = a.q_start[b], s1 = a.q_start[b + 1];
  if (s0 < 0 || s1 < s0 || s1 > a.total_q) return;   // flagged by the prefill kernel
  const int qlen = (int)min(s1 - s0, (int64_t)0x7fffffff);
  const int j = threadIdx.x % LP;
  const int p = blockIdx.y * PPP + threadIdx.x / LP;
  const int r = p / a.HW, h = p % a.HW;
  const int row = rb * a.BM + r;
  if (row >= qlen) return;   // (every lane of the pair)
  const float *base = a.part + (int64_t)slot0 * PT;
  auto lse = [&](int s) { return base[(int64_t)s * PT + NP * D + p]; };
  float M = -INFINITY;
  for (int s = j; s < n; s += LP) M = fmaxf(M, lse(s));
#pragma unroll
  for (int o = 1; o < LP; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  auto add = [&](float l, float4 x0, float4 x1) {
    const float w = fast_exp2((l - M) * kLog2e);   // 0 for an empty piece
    L += w;
    o[0] += w * x0.x;
    o[1] += w * x0.y;
    o[2] += w * x0.z;
    o[3] += w * x0.w;
    o[4] += w * x1.x;
    o[5] += w * x1.y;
    o[6] += w * x1.z;
    o[7] += w * x1.w;
  };
  if (M != -INFINITY) {
    int s = 0;
    for (; s + 4 <= n; s += 4) {
      float l4[4];
      float4 x0[4], x1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float *tp = base + (int64_t)(s + u) * PT;
        l4[u] = tp[NP * D + p];
        x0[u] = *reinterpret_cast<const float4 *>(tp + p * D + 8 * j);
        x1[u] = *reinterpret_cast<const float4 *>(tp + p * D + 8 * j + 4);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) add(l4[u], x0[u], x1[u]);
    }
    for (; s < n; ++s) {
      const float *tp = base + (int64_t)s * PT;
      add(tp[NP * D + p], *reinterpret_cast<const float4 *>(tp + p * D + 8 * j),
          *reinterpret_cast<const float4 *>(tp + p * D + 8 * j + 4));
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int64_t oh = (s0 + row) * a.Hq + hg * a.HW + h;
  uint4 v;
  v.x = pack_bf16x2(o[0] * inv, o[1] * inv);
  v.y = pack_bf16x2(o[2] * inv, o[3] * inv);
  v.z = pack_bf16x2(o[4] * inv, o[5] * inv);
  v.w = pack_bf16x2(o[6] * inv, o[7] * inv);
  *reinterpret_cast<uint4 *>(a.O + oh * D + 8 * j) = v;
  if (j == 0) a.LSE[oh] = L > 0.f ? M + fast_log2(L) * kLn2 : -INFINITY;
}

}  // namespace

int launch_packed_merge(const int32_t *merge, int64_t n_merge, const int32_t *q_start, int B,
                        const float *part, int64_t n_part_slots, void *O, float *LSE, int32_t *err,
                        int64_t total_q, int Hq, int Hkv, int D, hipStream_t stream) {
  if (n_merge <= 0) return PA_OK;
  if (n_merge > 0x7fffffffLL) return PA_ERR_RANGE;
  const int G = Hq / Hkv;
  MergeArgs a{merge, q_start, part, static_cast<uint16_t *>(O), LSE, err, total_q, n_part_slots, B, Hq,
              prefill_heads_per_block(G), prefill_rows_per_block(G)};
  // grid.y: the groups of 256 / (D/8) pairs of a tile's 128
  if (D == 64)
    hipLaunchKernelGGL(packed_merge_kernel<64>, dim3((unsigned)n_merge, 4), dim3(256), 0, stream, a);
  else if (D == 128)
    hipLaunchKernelGGL(packed_merge_kernel<128>, dim3((unsigned)n_merge, 8), dim3(256), 0, stream, a);
  else
    return PA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
