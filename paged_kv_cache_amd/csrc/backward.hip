// backward.hip -- attn_backward_dense: gradients dQ, dK, dV of exact attention
// on contiguous Q, K, V (FlashAttention-2 explainer, "Parallelise along the
// sequence length" and the MQA/GQA paragraph: P is recomputed from the stored
// log-sum-exp, and the key/value gradients of a GQA group are the sums over
// its query heads).
//
// For query row i and visible key j (S = scale * q K^T, P = exp(S - LSE)):
//   dV_j = sum_i P_ij dO_i            dP_ij = dO_i . V_j
//   D_i  = sum_c dO_ic O_ic           dS_ij = P_ij (dP_ij - D_i)
//   dQ_i = scale sum_j dS_ij K_j      dK_j  = scale sum_i dS_ij q_i
//
// The explainer's design runs one pass over key blocks and adds the dQ
// contributions of every key block with atomics.  On this chip each XCD has
// its own L2, and dQ of a long sequence does not fit in it, so those atomics
// would travel to HBM once per key block.  Here two passes avoid them:
//   bwd_dkdv_kernel  one workgroup per (sequence, kv head, 128 keys); each wave
//                    owns 32 keys (K, V in registers, dK, dV accumulated in
//                    registers over every query row and every q head of the
//                    group); Q and dO tiles of 64 rows are staged in LDS.
//   bwd_dq_kernel    one workgroup per (sequence, head group, query tile),
//                    laid out like the forward kernel; K and V tiles of 64
//                    keys are staged in LDS; dQ accumulates in registers.
// Both recompute S and dP (7 matrix products in all instead of 5) and write
// every gradient exactly once, so the result is deterministic.
//
// Tile products on 32x32x16 bf16 MFMA with fp32 accumulation.  P and dS are
// rounded to bf16 only as MFMA operands; in each kernel the lane layout of
// the scores is already the B-operand layout of the next product, and the
// transposed A operands (dO^T, Q^T, K^T) come from transposing LDS reads.
// bwd_dq_kernel runs first and also computes D_i of its rows (it holds their
// dO already) for bwd_dkdv_kernel.

#include "device.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kBT = 64;   // rows (dK/dV kernel) or keys (dQ kernel) per staged tile

struct BwdArgs {
  const uint16_t *q, *k, *v, *o, *dout;   // [B][T][H][D] bf16
  const float *lse;                       // [B][Hq][T] natural log
  float *dvec;                            // workspace [B][Hq][T]: D_i (written by bwd_dq_kernel)
  uint16_t *dq, *dk, *dv;
  int B, T, Hq, Hkv;
  float scale, scale_log2;
  int causal;
};

// LDS placement of 16-byte chunk c of tile row r: c ^ swz(r).  Row operand
// reads (32 consecutive rows, one chunk) hit distinct banks; the swizzle has
// period 16 in r.
template <int D>
__device__ __forceinline__ int bswz(int r) {
  return D == 64 ? ((r & 7) ^ ((r >> 3) & 1)) : (r & 15);
}

template <int D>
__device__ __forceinline__ uint32_t lds_off(int r, int dcol) {
  return (uint32_t)(r * (D * 2) + (((dcol >> 3) ^ bswz<D>(r)) << 4) + (dcol & 7) * 2);
}

// One 32x16 transposed operand for the products whose contraction runs over
// the 32 rows (or keys) of a half tile: slot (lh*8 + e) of operand q is tile
// row 16q + 8*(e/4) + 4*lh + e%4 -- the order in which a lane holds the rows
// of a 32x32 MFMA result -- and the lane's M index is column dcol0 + lane%32.
// Each 4-row half is one transposing read: in 16-lane group g, lane L points
// at row r0 + 4*(g>>1) + L/4, column d0 + 16*(g&1) + 4*(L%4).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint8_t *tile, const uint32_t (&addr)[2]) {
  uint2 part[2];
#pragma unroll
  for (int half = 0; half < 2; ++half)
    part[half] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                               (__attribute__((address_space(3))) i16x4 *)(tile + addr[half])));
  return __builtin_bit_cast(bf16x8, u32x4{part[0].x, part[0].y, part[1].x, part[1].y});
}

}  // namespace

// ---- dK, dV: one workgroup per (sequence, kv head, 128 keys)
template <int D, int G>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int CH = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = kBT * ROWB;
  constexpr int NLD = kBT * CH / 256;        // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint8_t qs[2][TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t os[2][TILEB];
  __shared__ __attribute__((aligned(16))) float ls[2][kBT];
  __shared__ __attribute__((aligned(16))) float dsv[2][kBT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5, l16 = lane & 15, g16 = lane >> 4;
  const int T = a.T, Hq = a.Hq, Hkv = a.Hkv;
  const int n_kb = (T + 127) / 128;
  const int n_pairs = a.B * Hkv;
  // workgroup -> (pair, key block): the key blocks of one (sequence, kv head)
  // stay on one XCD (its Q and dO rows are read by all of them), and key block
  // 0 (the most rows under a causal mask) goes first
  const int wg = blockIdx.x;
  int pair, kb;
  if ((n_pairs & 7) == 0) {
    const int ppx = n_pairs >> 3, k8 = wg >> 3;
    kb = k8 / ppx;
    pair = (wg & 7) * ppx + k8 % ppx;
  } else {
    kb = wg / n_pairs;
    pair = wg % n_pairs;
  }
  const int b = pair / Hkv, kvh = pair % Hkv;
  const int key0 = kb * 128;
  const int keyw = key0 + 32 * wave;           // first key of this wave
  const int key = keyw + lr;                   // this lane's key

  // K and V rows of the lane's key as B operands: slot (lh*8 + e) of operand
  // kk is d = lh*(D/2) + 8kk + e (the row-operand reads below use the same d order)
  bf16x8 kreg[D / 16], vreg[D / 16];
  {
    const int kr = key < T ? key : T - 1;
    const int64_t off = (((int64_t)b * T + kr) * Hkv + kvh) * D + lh * (D / 2);
    const bf16x8 *kp = reinterpret_cast<const bf16x8 *>(a.k + off);
    const bf16x8 *vp = reinterpret_cast<const bf16x8 *>(a.v + off);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kreg[kk] = kp[kk];
      vreg[kk] = vp[kk];
    }
  }
  // row-operand LDS offsets: lane reads row lr (+32 h2), chunk lh*(CH/2) + kk
  uint32_t raddr[CH / 2];
#pragma unroll
  for (int kk = 0; kk < CH / 2; ++kk) raddr[kk] = lds_off<D>(lr, (lh * (CH / 2) + kk) * 8);
  // transposed-operand offsets: [mb][q][half] for rows 16q + 8half + 4(g>>1) + L/4
  uint32_t taddr[D / 32][2][2];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        taddr[mb][q][half] = lds_off<D>(16 * q + 8 * half + 4 * (g16 >> 1) + (l16 >> 2),
                                        mb * 32 + 16 * (g16 & 1) + 4 * (l16 & 3));

  f32x16 dk[D / 32], dvacc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[mb][r] = dvacc[mb][r] = 0.f;

  // iterations: (q head of the group, 64-row tile); under a causal mask rows
  // before key0 see none of these keys
  const int n_rt = (T + kBT - 1) / kBT;
  const int rt0 = a.causal ? key0 / kBT : 0;
  const int per_head = n_rt - rt0;
  const int n_it = G * per_head;

  u32x4 pq[NLD], po[NLD];
  float pl = 0.f, pd = 0.f;
  auto gload = [&](int it) {
    const int h = kvh * G + it / per_head;
    const int rt = rt0 + it % per_head;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int c = tid + 256 * j;
      const int r = c / CH, pos = c % CH;
      int row = rt * kBT + r;
      row = row < T ? row : T - 1;
      const int64_t off = (((int64_t)b * T + row) * Hq + h) * D + pos * 8;
      pq[j] = *reinterpret_cast<const u32x4 *>(a.q + off);
      po[j] = *reinterpret_cast<const u32x4 *>(a.dout + off);
    }
    if (tid < kBT) {
      const int row = rt * kBT + tid;
      const int64_t o = ((int64_t)b * Hq + h) * T + (row < T ? row : 0);
      pl = row < T ? a.lse[o] * kLog2e : INFINITY;   // padding rows: P = 0
      pd = row < T ? a.dvec[o] : 0.f;
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int c = tid + 256 * j;
      const int r = c / CH, pos = c % CH;
      const uint32_t o = lds_off<D>(r, pos * 8);
      *reinterpret_cast<u32x4 *>(&qs[st][o]) = pq[j];
      *reinterpret_cast<u32x4 *>(&os[st][o]) = po[j];
    }
    if (tid < kBT) {
      ls[st][tid] = pl;
      dsv[st][tid] = pd;
    }
  };

  const float c = a.scale_log2;
  auto compute = [&](int it, int st) {
    const int rt = rt0 + it % per_head;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int row0 = rt * kBT + 32 * h2;
      if (a.causal && keyw > row0 + 31) continue;     // every key of the wave after every row
      const uint8_t *qt = qs[st] + h2 * 32 * ROWB;
      const uint8_t *ot = os[st] + h2 * 32 * ROWB;
      // S, dP [32 rows x 32 keys]: lane = key, acc r = row 8(r/4) + 4lh + r%4
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(qt + raddr[kk]);
        const bf16x8 oa = *reinterpret_cast<const bf16x8 *>(ot + raddr[kk]);
        s = mfma32(qa, kreg[kk], s);
        dp = mfma32(oa, vreg[kk], dp);
      }
      // LSE and D of the lane's 16 rows
      f32x4 l4[4], d4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        l4[g] = *reinterpret_cast<const f32x4 *>(&ls[st][32 * h2 + 8 * g + 4 * lh]);
        d4[g] = *reinterpret_cast<const f32x4 *>(&dsv[st][32 * h2 + 8 * g + 4 * lh]);
      }
      const bool diag = a.causal && keyw + 31 > row0;   // some key after some row
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[r], c, -l4[r / 4][r % 4]));
        if (diag) p = key > row0 + 8 * (r / 4) + 4 * lh + (r % 4) ? 0.f : p;
        const float dsr = p * (dp[r] - d4[r / 4][r % 4]);
        pb[r / 8][r % 8] = (__bf16)p;
        sb[r / 8][r % 8] = (__bf16)dsr;
      }
      // dV^T += dO^T P, dK^T += Q^T dS  (M = d, N = keys, contraction over rows)
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const bf16x8 oT = tr_operand<D>(ot, taddr[mb][q]);
          const bf16x8 qT = tr_operand<D>(qt, taddr[mb][q]);
          dvacc[mb] = mfma32(oT, pb[q], dvacc[mb]);
          dk[mb] = mfma32(qT, sb[q], dk[mb]);
        }
    }
  };

  if (n_it > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
    for (int it = 0; it < n_it; ++it) {
      const int st = it & 1;
      const bool more = it + 1 < n_it;
      if (more) gload(it + 1);
      compute(it, st);
      if (more) lstore(st ^ 1);
      __syncthreads();
    }
  }

  // ---- dK = scale * dK^T, dV: lane = key, acc r = d 8(r/4) + 4lh + r%4
  if (key < T) {
    const int64_t off = (((int64_t)b * T + key) * Hkv + kvh) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * lh;
        uint2 wk, wv;
        wk.x = pack_bf16x2(dk[mb][4 * g + 0] * a.scale, dk[mb][4 * g + 1] * a.scale);
        wk.y = pack_bf16x2(dk[mb][4 * g + 2] * a.scale, dk[mb][4 * g + 3] * a.scale);
        wv.x = pack_bf16x2(dvacc[mb][4 * g + 0], dvacc[mb][4 * g + 1]);
        wv.y = pack_bf16x2(dvacc[mb][4 * g + 2], dvacc[mb][4 * g + 3]);
        *reinterpret_cast<uint2 *>(a.dk + off + d0) = wk;
        *reinterpret_cast<uint2 *>(a.dv + off + d0) = wv;
      }
  }
}

// ---- dQ: one workgroup per (sequence, head group, query tile), four 32-row
// column blocks as in the forward kernel
template <int D, int G>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int HW = G < 4 ? G : 4;   // heads per workgroup
  constexpr int RW = 4 / HW;          // 32-row blocks per workgroup
  constexpr int BM = 32 * RW;
  constexpr int CH = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = kBT * ROWB;
  constexpr int NLD = kBT * CH / 256;
  __shared__ __attribute__((aligned(16))) uint8_t ks[2][TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t vs[2][TILEB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5, l16 = lane & 15, g16 = lane >> 4;
  const int T = a.T, Hq = a.Hq, Hkv = a.Hkv;
  const int n_hg = Hq / HW;
  const int n_rb = (T + BM - 1) / BM;
  const int n_pairs = a.B * n_hg;
  const int wg = blockIdx.x;
  int pair, rank;
  if ((n_pairs & 7) == 0) {
    const int ppx = n_pairs >> 3, k8 = wg >> 3;
    rank = k8 / ppx;
    pair = (wg & 7) * ppx + k8 % ppx;
  } else {
    rank = wg / n_pairs;
    pair = wg % n_pairs;
  }
  const int rb = a.causal ? n_rb - 1 - rank : rank;   // causal: longest first
  const int b = pair / n_hg, hg = pair % n_hg;
  const int head = hg * HW + wave % HW;
  const int kvh = head / G;
  const int row0 = rb * BM + 32 * (wave / HW);
  const int row = row0 + lr;                   // this lane's query row
  const int rowc = row < T ? row : T - 1;

  // q and dO of the lane's row as B operands (slot lh*8 + e of operand kk is
  // d = lh*(D/2) + 8kk + e), its LSE (log2 units) and D
  bf16x8 qreg[D / 16], oreg[D / 16];
  {
    const int64_t off = (((int64_t)b * T + rowc) * Hq + head) * D + lh * (D / 2);
    const bf16x8 *qp = reinterpret_cast<const bf16x8 *>(a.q + off);
    const bf16x8 *op = reinterpret_cast<const bf16x8 *>(a.dout + off);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qreg[kk] = qp[kk];
      oreg[kk] = op[kk];
    }
  }
  // D of the lane's row: its dO times the forward's O (each lane half holds
  // half of the row), written for bwd_dkdv_kernel
  const int64_t so = ((int64_t)b * Hq + head) * T + rowc;
  const float l2 = row < T ? a.lse[so] * kLog2e : INFINITY;
  float dr;
  {
    const int64_t off = (((int64_t)b * T + rowc) * Hq + head) * D + lh * (D / 2);
    const u32x4 *op = reinterpret_cast<const u32x4 *>(a.o + off);
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const u32x4 ov = op[kk];
      const u32x4 dv = __builtin_bit_cast(u32x4, oreg[kk]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        part += __uint_as_float(ov[w] << 16) * __uint_as_float(dv[w] << 16);
        part += __uint_as_float(ov[w] & 0xffff0000u) * __uint_as_float(dv[w] & 0xffff0000u);
      }
    }
    dr = part + __shfl_xor(part, 32, 64);
    if (row < T && lh == 0) a.dvec[so] = dr;
    dr = row < T ? dr : 0.f;
  }

  uint32_t raddr[CH / 2];
#pragma unroll
  for (int kk = 0; kk < CH / 2; ++kk) raddr[kk] = lds_off<D>(lr, (lh * (CH / 2) + kk) * 8);
  uint32_t taddr[D / 32][2][2];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        taddr[mb][q][half] = lds_off<D>(16 * q + 8 * half + 4 * (g16 >> 1) + (l16 >> 2),
                                        mb * 32 + 16 * (g16 & 1) + 4 * (l16 & 3));

  f32x16 dq[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[mb][r] = 0.f;

  // key tiles: all of them, or up to the workgroup's last row (causal)
  const int wg_row_end = min(rb * BM + BM, T);   // exclusive
  const int kv_end = a.causal ? wg_row_end : T;
  const int n_it = rb * BM < T ? (kv_end + kBT - 1) / kBT : 0;
  const int wave_last = row0 + 31;

  u32x4 pk[NLD], pv[NLD];
  auto gload = [&](int t) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int c = tid + 256 * j;
      const int r = c / CH, pos = c % CH;
      int kr = t * kBT + r;
      kr = kr < T ? kr : T - 1;
      const int64_t off = (((int64_t)b * T + kr) * Hkv + kvh) * D + pos * 8;
      pk[j] = *reinterpret_cast<const u32x4 *>(a.k + off);
      pv[j] = *reinterpret_cast<const u32x4 *>(a.v + off);
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int c = tid + 256 * j;
      const int r = c / CH, pos = c % CH;
      const uint32_t o = lds_off<D>(r, pos * 8);
      *reinterpret_cast<u32x4 *>(&ks[st][o]) = pk[j];
      *reinterpret_cast<u32x4 *>(&vs[st][o]) = pv[j];
    }
  };
  const float c = a.scale_log2;
  auto compute = [&](int t, int st) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int kv0 = t * kBT + 32 * h2;        // first key of this half
      if (a.causal && kv0 > wave_last) continue;
      const uint8_t *kt = ks[st] + h2 * 32 * ROWB;
      const uint8_t *vt = vs[st] + h2 * 32 * ROWB;
      // S^T, dP^T [32 keys x 32 rows]: lane = row, acc r = key 8(r/4) + 4lh + r%4
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(kt + raddr[kk]);
        const bf16x8 va = *reinterpret_cast<const bf16x8 *>(vt + raddr[kk]);
        s = mfma32(ka, qreg[kk], s);
        dp = mfma32(va, oreg[kk], dp);
      }
      const bool edge = (a.causal && kv0 + 31 > row0) || kv0 + 32 > T;
      bf16x8 sb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[r], c, -l2));
        if (edge) {
          const int kk_ = kv0 + 8 * (r / 4) + 4 * lh + (r % 4);
          p = (kk_ >= T || (a.causal && kk_ > row)) ? 0.f : p;
        }
        sb[r / 8][r % 8] = (__bf16)(p * (dp[r] - dr));
      }
      // dQ^T += K^T dS^T  (M = d, N = rows, contraction over keys)
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int q = 0; q < 2; ++q) dq[mb] = mfma32(tr_operand<D>(kt, taddr[mb][q]), sb[q], dq[mb]);
    }
  };

  if (n_it > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
    for (int t = 0; t < n_it; ++t) {
      const int st = t & 1;
      const bool more = t + 1 < n_it;
      if (more) gload(t + 1);
      compute(t, st);
      if (more) lstore(st ^ 1);
      __syncthreads();
    }
  }

  // ---- dQ = scale * dQ^T: lane = row, acc r = d 8(r/4) + 4lh + r%4
  if (row < T) {
    const int64_t off = (((int64_t)b * T + row) * Hq + head) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack_bf16x2(dq[mb][4 * g + 0] * a.scale, dq[mb][4 * g + 1] * a.scale);
        w.y = pack_bf16x2(dq[mb][4 * g + 2] * a.scale, dq[mb][4 * g + 3] * a.scale);
        *reinterpret_cast<uint2 *>(a.dq + off + mb * 32 + 8 * g + 4 * lh) = w;
      }
  }
}

namespace {

template <int D, int G>
int launch_bwd_t(const BwdArgs &a, hipStream_t stream) {
  constexpr int HW = G < 4 ? G : 4;
  constexpr int BM = 32 * (4 / HW);
  const int64_t kv_grid = (int64_t)a.B * a.Hkv * ((a.T + 127) / 128);
  const int64_t q_grid = (int64_t)a.B * (a.Hq / HW) * ((a.T + BM - 1) / BM);
  if (kv_grid > 0x7fffffff || q_grid > 0x7fffffff) return PA_ERR_RANGE;
  hipLaunchKernelGGL((bwd_dq_kernel<D, G>), dim3((unsigned)q_grid), dim3(256), 0, stream, a);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, G>), dim3((unsigned)kv_grid), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

size_t backward_workspace_bytes(int B, int T, int Hq) { return (size_t)B * Hq * T * sizeof(float); }

int launch_backward_dense(const void *q, const void *k, const void *v, const void *o,
                          const void *dout, const float *lse, int B, int T, int Hq, int Hkv, int D,
                          float scale, int causal, void *dq, void *dk, void *dv, void *workspace,
                          hipStream_t stream) {
  BwdArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.o = static_cast<const uint16_t *>(o);
  a.dout = static_cast<const uint16_t *>(dout);
  a.lse = lse;
  a.dvec = static_cast<float *>(workspace);
  a.dq = static_cast<uint16_t *>(dq);
  a.dk = static_cast<uint16_t *>(dk);
  a.dv = static_cast<uint16_t *>(dv);
  a.B = B;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.causal = causal ? 1 : 0;
  const int G = Hq / Hkv;
#define PA_BWD_CASE(DD, GG) \
  if (D == DD && G == GG) return launch_bwd_t<DD, GG>(a, stream);
  PA_BWD_CASE(64, 1)
  PA_BWD_CASE(64, 2)
  PA_BWD_CASE(64, 4)
  PA_BWD_CASE(64, 8)
  PA_BWD_CASE(64, 16)
  PA_BWD_CASE(128, 1)
  PA_BWD_CASE(128, 2)
  PA_BWD_CASE(128, 4)
  PA_BWD_CASE(128, 8)
  PA_BWD_CASE(128, 16)
#undef PA_BWD_CASE
  return PA_ERR_UNSUPPORTED;
}

}  // namespace pa
