/*
 * oracle.c -- plain, slow, fp64 CPU definition of paged causal GQA attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this file:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load it.  It shares no code, header or constant with the HIP library; the
 * page geometry below is written out again from the pages on purpose.
 *
 * What it computes is the plain definition of exact attention (FlashAttention-2
 * explainer, "FlashAttention-2: better parallelism", opening summary: the result
 * is exact attention with no approximation), so no blocking, online rescaling or
 * reordering appears here: for one query row all scores are formed, the maximum
 * is taken, the exponentials are summed and the weighted sum of V is divided
 * once.
 *
 *   s_j   = scale * sum_c q[c] * K[j][c]            (scaled dot product)
 *   m     = max_j s_j
 *   l     = sum_j exp(s_j - m)
 *   O[c]  = sum_j exp(s_j - m) * V[j][c] / l
 *   LSE   = m + ln(l)                               (natural log of the scaled scores;
 *                                                    FA2 explainer worked example: L = m + log l)
 *
 * Visible keys for one query:
 *   causal prefill    keys 0..t of its own sequence (tiny-vllm part 3, "causalMask and
 *                     online softmax": a score whose column exceeds its row is masked,
 *                     and a masked score has probability exactly 0, so it is skipped)
 *   full prefill      keys 0..seq_len-1
 *   decode            keys 0..ctx_len-1, the newest token included (tiny-vllm part 6,
 *                     "logical block -> physical block -> byte address": the kernel reads
 *                     exactly seq_len tokens, which already count the token just written)
 *
 * GQA head mapping: kv_head = q_head / (Hq / Hkv), consecutive groups (tiny-vllm
 * part 3, "Per-head attention scores and GQA": q heads 0-3 use K head 0).
 *
 * Paged layout (tiny-vllm part 6, "Block contents: K in front, V after V_OFFSET"
 * and "block table" sections):
 *   a page holds 16 tokens; its first half is K as [token][kv_head][dim] bf16,
 *   its second half, V_OFFSET = 16 * Hkv * d * 2 bytes in, is V in the same order;
 *   page bytes = 2 * V_OFFSET.
 *   block_table is int32 [n_slots][n_layers][max_blocks_per_seq]; the entry for
 *   (slot, layer, position p) is at slot*n_layers*mbps + layer*mbps + p/16,
 *   -1 meaning "no page".
 *   byte address of K[p][h][i] = page*page_bytes + (p%16)*Hkv*d*2 + h*d*2 + i*2,
 *   V = the same plus V_OFFSET.
 *
 * Inputs are bf16 bit patterns (uint16); each is widened exactly to double.
 * Where a needed table entry is -1 or outside [0, n_pages) (or the slot or
 * position is out of range) that key is left out of the sum and counted; the
 * functions return the number of such lookups.  A query with no key left gets
 * O = 0 and LSE = -infinity.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_PAGE_TOKENS 16

static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int64_t oracle_page_bytes(int n_kv_heads, int head_dim)
{
    return 2LL * ORACLE_PAGE_TOKENS * n_kv_heads * head_dim * 2;
}

/* Description of one paged pool plus its block table. */
typedef struct {
    const uint8_t *pool;
    int64_t n_pages;
    const int32_t *table;
    int n_slots, n_layers, mbps, layer;
    int n_kv_heads, head_dim;
} paged_src;

/* Physical page holding position p of a slot, or -1 when the lookup is invalid. */
static int64_t page_of(const paged_src *s, int slot, int64_t p)
{
    if (slot < 0 || slot >= s->n_slots || p < 0 || p >= (int64_t)s->mbps * ORACLE_PAGE_TOKENS)
        return -1;
    int64_t e = (int64_t)slot * s->n_layers * s->mbps + (int64_t)s->layer * s->mbps
              + p / ORACLE_PAGE_TOKENS;
    int32_t page = s->table[e];
    if (page < 0 || (int64_t)page >= s->n_pages)
        return -1;
    return page;
}

/* Byte offset of element (p, h, 0) of K inside the pool (V: add V_OFFSET). */
static int64_t k_offset(const paged_src *s, int64_t page, int64_t p, int h)
{
    int64_t row = (int64_t)s->n_kv_heads * s->head_dim * 2;
    return page * oracle_page_bytes(s->n_kv_heads, s->head_dim)
         + (p % ORACLE_PAGE_TOKENS) * row + (int64_t)h * s->head_dim * 2;
}

static int64_t v_offset_bytes(const paged_src *s)
{
    return (int64_t)ORACLE_PAGE_TOKENS * s->n_kv_heads * s->head_dim * 2;
}

/*
 * Attention of one query vector qd[0..d) over keys 0..n_keys-1, whose K and V
 * rows are given as pointers (NULL = key absent).  scores is scratch of n_keys.
 */
static void attend(const double *qd, int d, double scale, int64_t n_keys,
                   const uint16_t *const *krow, const uint16_t *const *vrow,
                   double *scores, double *out, double *lse)
{
    double m = -INFINITY;
    int64_t present = 0;
    for (int64_t j = 0; j < n_keys; ++j) {
        if (!krow[j]) {
            scores[j] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += qd[c] * bf16_to_double(krow[j][c]);
        scores[j] = scale * dot;
        if (scores[j] > m)
            m = scores[j];
        ++present;
    }
    for (int c = 0; c < d; ++c)
        out[c] = 0.0;
    if (present == 0) {
        *lse = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        if (!krow[j])
            continue;
        double w = exp(scores[j] - m);
        l += w;
        for (int c = 0; c < d; ++c)
            out[c] += w * bf16_to_double(vrow[j][c]);
    }
    for (int c = 0; c < d; ++c)
        out[c] /= l;
    *lse = m + log(l);
}

/*
 * Write the K and V rows of n_tokens tokens into their pages.
 * k, v: [n_tokens][n_kv_heads][head_dim] bf16.  Token i belongs to slot
 * slot_ids[i] at sequence position positions[i].  Every byte not named by a
 * token stays as it was.  Returns the number of tokens not written because
 * their lookup was invalid.
 */
int64_t oracle_kv_scatter(uint8_t *pool, int64_t n_pages,
                          const uint16_t *k, const uint16_t *v, int64_t n_tokens,
                          const int32_t *slot_ids, const int32_t *positions,
                          const int32_t *block_table, int n_slots, int n_layers, int mbps,
                          int layer, int n_kv_heads, int head_dim)
{
    paged_src s = {pool, n_pages, block_table, n_slots, n_layers, mbps, layer, n_kv_heads, head_dim};
    int64_t row_elems = (int64_t)n_kv_heads * head_dim;
    int64_t bad = 0;
    for (int64_t i = 0; i < n_tokens; ++i) {
        int64_t page = page_of(&s, slot_ids[i], positions[i]);
        if (page < 0) {
            ++bad;
            continue;
        }
        for (int h = 0; h < n_kv_heads; ++h) {
            int64_t off = k_offset(&s, page, positions[i], h);
            for (int c = 0; c < head_dim; ++c) {
                uint16_t kb = k[i * row_elems + (int64_t)h * head_dim + c];
                uint16_t vb = v[i * row_elems + (int64_t)h * head_dim + c];
                memcpy(pool + off + 2 * c, &kb, 2);
                memcpy(pool + off + v_offset_bytes(&s) + 2 * c, &vb, 2);
            }
        }
    }
    return bad;
}

/*
 * Paged prefill.  q: [B][T][Hq][d]; sequence b lives in block-table slot
 * slot_ids[b] (NULL: slot b) and has seq_lens[b] tokens in the cache.  Its
 * queries are the last q_lens[b] of those tokens (q_lens NULL: all of them,
 * q_len = seq_len <= T): query row t sits at position seq_len - q_len + t, so
 * a chunk continuing a cached prefix is aligned to the end of the sequence
 * (bottom-right), and a single query row (q_len 1) is a decode step.  Rows to
 * evaluate are the (b, t) pairs rows[2i], rows[2i+1] (rows == NULL: all B*T in
 * order).  O: [n_rows][Hq][d], LSE: [n_rows][Hq].  A padding row (t >= q_len)
 * gets O = 0, LSE = -infinity.
 */
int64_t oracle_attn_prefill(const uint16_t *q, const uint8_t *pool, int64_t n_pages,
                            const int32_t *block_table, int n_slots, int n_layers, int mbps,
                            int layer, const int32_t *slot_ids, const int32_t *seq_lens,
                            const int32_t *q_lens, int B, int T, int Hq, int Hkv, int d,
                            double scale, int causal, const int32_t *rows, int64_t n_rows,
                            double *O, double *LSE)
{
    paged_src s = {pool, n_pages, block_table, n_slots, n_layers, mbps, layer, Hkv, d};
    int g = Hq / Hkv;
    if (!rows)
        n_rows = (int64_t)B * T;
    int64_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        int b = rows ? rows[2 * r] : (int)(r / T);
        int t = rows ? rows[2 * r + 1] : (int)(r % T);
        int slot = slot_ids ? slot_ids[b] : b;
        int64_t len = seq_lens[b];
        int64_t qlen = q_lens ? q_lens[b] : len;
        int64_t pos = len - qlen + t; /* position of query row t */
        int64_t n_keys = t < qlen ? (causal ? pos + 1 : len) : 0;
        const uint16_t **krow = malloc(sizeof(*krow) * (size_t)(n_keys + 1));
        const uint16_t **vrow = malloc(sizeof(*vrow) * (size_t)(n_keys + 1));
        double *scores = malloc(sizeof(double) * (size_t)(n_keys + 1));
        double *qd = malloc(sizeof(double) * (size_t)d);
        for (int h = 0; h < Hq; ++h) {
            int kvh = h / g;
            for (int64_t j = 0; j < n_keys; ++j) {
                int64_t page = page_of(&s, slot, j);
                if (page < 0) {
                    krow[j] = vrow[j] = NULL;
                    ++bad;
                    continue;
                }
                int64_t off = k_offset(&s, page, j, kvh);
                krow[j] = (const uint16_t *)(pool + off);
                vrow[j] = (const uint16_t *)(pool + off + v_offset_bytes(&s));
            }
            const uint16_t *qr = q + (((int64_t)b * T + t) * Hq + h) * d;
            for (int c = 0; c < d; ++c)
                qd[c] = bf16_to_double(qr[c]);
            attend(qd, d, scale, n_keys, krow, vrow, scores, O + (r * Hq + h) * d, LSE + r * Hq + h);
        }
        free(krow);
        free(vrow);
        free(scores);
        free(qd);
    }
    return bad;
}

/*
 * Paged decode.  q: [B][Hq][d], the query of the newest token of each
 * sequence; ctx_lens[b] counts the cached tokens including that newest one,
 * all of which are visible (no mask).  O: [B][Hq][d], LSE: [B][Hq].
 */
int64_t oracle_attn_decode(const uint16_t *q, const uint8_t *pool, int64_t n_pages,
                           const int32_t *block_table, int n_slots, int n_layers, int mbps,
                           int layer, const int32_t *slot_ids, const int32_t *ctx_lens,
                           int B, int Hq, int Hkv, int d, double scale, double *O, double *LSE)
{
    paged_src s = {pool, n_pages, block_table, n_slots, n_layers, mbps, layer, Hkv, d};
    int g = Hq / Hkv;
    int64_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t bh = 0; bh < (int64_t)B * Hq; ++bh) {
        int b = (int)(bh / Hq), h = (int)(bh % Hq);
        int slot = slot_ids ? slot_ids[b] : b;
        int64_t n_keys = ctx_lens[b] > 0 ? ctx_lens[b] : 0;
        const uint16_t **krow = malloc(sizeof(*krow) * (size_t)(n_keys + 1));
        const uint16_t **vrow = malloc(sizeof(*vrow) * (size_t)(n_keys + 1));
        double *scores = malloc(sizeof(double) * (size_t)(n_keys + 1));
        double *qd = malloc(sizeof(double) * (size_t)d);
        int kvh = h / g;
        for (int64_t j = 0; j < n_keys; ++j) {
            int64_t page = page_of(&s, slot, j);
            if (page < 0) {
                krow[j] = vrow[j] = NULL;
                ++bad;
                continue;
            }
            int64_t off = k_offset(&s, page, j, kvh);
            krow[j] = (const uint16_t *)(pool + off);
            vrow[j] = (const uint16_t *)(pool + off + v_offset_bytes(&s));
        }
        for (int c = 0; c < d; ++c)
            qd[c] = bf16_to_double(q[bh * d + c]);
        attend(qd, d, scale, n_keys, krow, vrow, scores, O + bh * d, LSE + bh);
        free(krow);
        free(vrow);
        free(scores);
        free(qd);
    }
    return bad;
}

/*
 * Unpaged attention on contiguous q [B][T][Hq][d], k, v [B][T][Hkv][d]
 * (FlashAttention-2 explainer, "Results": the attention-only benchmark shapes).
 * Rows as in oracle_attn_prefill; every sequence has length T.
 */
void oracle_attn_dense(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       int B, int T, int Hq, int Hkv, int d, double scale, int causal,
                       const int32_t *rows, int64_t n_rows, double *O, double *LSE)
{
    int g = Hq / Hkv;
    if (!rows)
        n_rows = (int64_t)B * T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int b = rows ? rows[2 * r] : (int)(r / T);
        int t = rows ? rows[2 * r + 1] : (int)(r % T);
        int64_t n_keys = causal ? (int64_t)t + 1 : T;
        const uint16_t **krow = malloc(sizeof(*krow) * (size_t)n_keys);
        const uint16_t **vrow = malloc(sizeof(*vrow) * (size_t)n_keys);
        double *scores = malloc(sizeof(double) * (size_t)n_keys);
        double *qd = malloc(sizeof(double) * (size_t)d);
        for (int h = 0; h < Hq; ++h) {
            int kvh = h / g;
            for (int64_t j = 0; j < n_keys; ++j) {
                int64_t idx = (((int64_t)b * T + j) * Hkv + kvh) * d;
                krow[j] = k + idx;
                vrow[j] = v + idx;
            }
            const uint16_t *qr = q + (((int64_t)b * T + t) * Hq + h) * d;
            for (int c = 0; c < d; ++c)
                qd[c] = bf16_to_double(qr[c]);
            attend(qd, d, scale, n_keys, krow, vrow, scores, O + (r * Hq + h) * d, LSE + r * Hq + h);
        }
        free(krow);
        free(vrow);
        free(scores);
        free(qd);
    }
}

/* ------------------------------------------------------------------------ */
/* Decode append: RoPE, page allocation from a free stack, page release.    */
/* ------------------------------------------------------------------------ */

/*
 * Device-error bits of the library's ABI, written out again here (the values
 * are an interface both sides must agree on, not shared code).
 */
#define ORACLE_ERR_BAD_PAGE 1
#define ORACLE_ERR_BAD_SLOT 2
#define ORACLE_ERR_BAD_POS 4
#define ORACLE_ERR_NO_FREE_PAGE 8
#define ORACLE_ERR_DUP_SLOT 16
#define ORACLE_ERR_REASSIGNED 32
#define ORACLE_ERR_STACK_FULL 64

/*
 * Round a double to the nearest bfloat16, ties to even, from the definition:
 * a bfloat16 has 8 significant bits and fp32's exponent range, so the spacing
 * of bfloat16 values around |x| in [2^(e-1), 2^e) is 2^(e-8), and 2^-133 in the
 * subnormal range (|x| < 2^-126).  Dividing by that spacing, rounding to the
 * nearest integer (ties to even, the default rounding mode) and multiplying
 * back is exact in double.  Overflow gives infinity.  Returns the bit pattern.
 */
static uint16_t double_to_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    if (x == 0.0 || isinf(x)) {
        float f = (float)x;
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        return (uint16_t)(u >> 16);
    }
    int e;
    frexp(fabs(x), &e);
    int qexp = (e > -125 ? e : -125) - 8;
    double r = ldexp(nearbyint(ldexp(x, -qexp)), qexp);
    float f = (float)r; /* exact: r is a bfloat16 value (or beyond fp32 range: inf) */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void oracle_round_bf16(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = double_to_bf16(x[i]);
}

/*
 * RoPE of one head vector (tiny-vllm part 3, "RoPE: a rotation that references
 * a table"): element i of the first half and element i + d/2 of the second
 * half form pair i, which is turned by the angle whose cosine and sine sit at
 * row `pos`, column i of the tables ([max_pos][d/2] fp32; the page's tables
 * repeat each value twice, one per element of the pair, which carries the
 * same information):
 *     y[i]       = x[i] * cos - x[i + d/2] * sin
 *     y[i + d/2] = x[i] * sin + x[i + d/2] * cos
 * Each product of a bf16 and an fp32 value is exact in double, so each output
 * is the exact result rounded once to double.
 */
static void rope_head(const uint16_t *x, int d, const float *cos_row, const float *sin_row,
                      double *y)
{
    int half = d / 2;
    for (int i = 0; i < half; ++i) {
        double x1 = bf16_to_double(x[i]), x2 = bf16_to_double(x[i + half]);
        double c = (double)cos_row[i], s = (double)sin_row[i];
        y[i] = x1 * c - x2 * s;
        y[i + half] = x1 * s + x2 * c;
    }
}

/*
 * RoPE of n_tok tokens' head vectors x [n_tok][n_heads][d] at positions[t]:
 * out [n_tok][n_heads][d] in double (unrounded).  A token whose position is
 * outside [0, max_pos) gets NaN rows; the count of such tokens is returned.
 */
int64_t oracle_rope(const uint16_t *x, int64_t n_tok, int n_heads, int d, const int32_t *positions,
                    const float *cos_t, const float *sin_t, int max_pos, double *out)
{
    int64_t bad = 0;
    for (int64_t t = 0; t < n_tok; ++t) {
        int pos = positions[t];
        for (int h = 0; h < n_heads; ++h) {
            double *y = out + (t * n_heads + h) * d;
            if (pos < 0 || pos >= max_pos) {
                for (int c = 0; c < d; ++c)
                    y[c] = NAN;
                continue;
            }
            rope_head(x + (t * n_heads + h) * d, d, cos_t + (int64_t)pos * (d / 2),
                      sin_t + (int64_t)pos * (d / 2), y);
        }
        if (pos < 0 || pos >= max_pos)
            ++bad;
    }
    return bad;
}

/*
 * One decode step's writes for B new tokens, in batch order (tiny-vllm part 3,
 * "RoPE: a rotation that references a table" and "Distributing K/V into paged
 * blocks"; part 6, "The lifetime of a physical block: free_blocks"):
 *
 *   for b = 0 .. B-1:
 *     slot = slot_ids[b] (NULL: b), pos = positions[b], block = pos / 16
 *     if pos % 16 == 0 (the token opens a block, the decode allocation rule):
 *         page = free_pages[top - 1]; top -= 1      (pop from the back)
 *         block_table[slot][layer][block] = page
 *     else page = block_table[slot][layer][block]
 *     K row of the token = bf16(RoPE(k[b], pos)), V row = v[b], written into
 *     the page at row pos % 16 (layout as in oracle_kv_scatter);
 *     q_out[b] = bf16(RoPE(q_in[b], pos)) when q_in is given.
 *
 * Checks, each OR-ing an error bit and skipping what it cannot do:
 *   slot outside [0, n_slots)                 BAD_SLOT  (token not written)
 *   pos outside [0, mbps*16) or >= max_pos    BAD_POS   (token not written;
 *                                             q rotated only if pos < max_pos
 *                                             and pos >= 0)
 *   a slot named twice in the call            DUP_SLOT  (both still processed)
 *   opening token, empty stack                NO_FREE_PAGE (not written, entry kept)
 *   opening token, entry was not -1           REASSIGNED (entry overwritten)
 *   popped page or looked-up entry outside [0, n_pages)   BAD_PAGE (not written)
 * A token that cannot be written still takes its place in the pop order:
 * tokens with invalid slot or position do not pop; opening tokens pop (or
 * find the stack empty) in batch order.
 *
 * pool, block_table, *top are updated in place; free_pages is read only
 * (entries at and above the new top are simply no longer free).  Returns the
 * OR of the error bits.
 */
int oracle_kv_append(uint8_t *pool, int64_t n_pages, const uint16_t *k, const uint16_t *v,
                     const uint16_t *q_in, uint16_t *q_out, int Hq, int B,
                     const int32_t *slot_ids, const int32_t *positions,
                     const float *cos_t, const float *sin_t, int max_pos,
                     int32_t *block_table, int n_slots, int n_layers, int mbps, int layer,
                     const int32_t *free_pages, int32_t *top, int n_kv_heads, int head_dim)
{
    int errs = 0;
    int d = head_dim;
    int64_t row_elems = (int64_t)n_kv_heads * d;
    double *y = malloc(sizeof(double) * (size_t)d);
    paged_src s = {pool, n_pages, block_table, n_slots, n_layers, mbps, layer, n_kv_heads, d};
    for (int b = 0; b < B; ++b) {
        int slot = slot_ids ? slot_ids[b] : b;
        int pos = positions[b];
        for (int o = 0; o < B; ++o)
            if (o != b && (slot_ids ? slot_ids[o] : o) == slot)
                errs |= ORACLE_ERR_DUP_SLOT;
        int pos_ok = pos >= 0 && pos < max_pos;
        if (q_in && pos_ok)
            for (int h = 0; h < Hq; ++h) {
                rope_head(q_in + ((int64_t)b * Hq + h) * d, d, cos_t + (int64_t)pos * (d / 2),
                          sin_t + (int64_t)pos * (d / 2), y);
                oracle_round_bf16(y, d, q_out + ((int64_t)b * Hq + h) * d);
            }
        if (slot < 0 || slot >= n_slots) {
            errs |= ORACLE_ERR_BAD_SLOT;
            continue;
        }
        if (!pos_ok || pos >= mbps * ORACLE_PAGE_TOKENS) {
            errs |= ORACLE_ERR_BAD_POS;
            continue;
        }
        int32_t *entry = block_table + (int64_t)slot * n_layers * mbps + (int64_t)layer * mbps
                       + pos / ORACLE_PAGE_TOKENS;
        int64_t page;
        if (pos % ORACLE_PAGE_TOKENS == 0) {
            if (*top <= 0) {
                errs |= ORACLE_ERR_NO_FREE_PAGE;
                continue;
            }
            page = free_pages[*top - 1];
            *top -= 1;
            if (page < 0 || page >= n_pages) {
                errs |= ORACLE_ERR_BAD_PAGE;
                continue;
            }
            if (*entry != -1)
                errs |= ORACLE_ERR_REASSIGNED;
            *entry = (int32_t)page;
        } else {
            page = *entry;
            if (page < 0 || page >= n_pages) {
                errs |= ORACLE_ERR_BAD_PAGE;
                continue;
            }
        }
        for (int h = 0; h < n_kv_heads; ++h) {
            int64_t off = k_offset(&s, page, pos, h);
            rope_head(k + b * row_elems + (int64_t)h * d, d, cos_t + (int64_t)pos * (d / 2),
                      sin_t + (int64_t)pos * (d / 2), y);
            for (int c = 0; c < d; ++c) {
                uint16_t kb = double_to_bf16(y[c]);
                uint16_t vb = v[b * row_elems + (int64_t)h * d + c];
                memcpy(pool + off + 2 * c, &kb, 2);
                memcpy(pool + off + v_offset_bytes(&s) + 2 * c, &vb, 2);
            }
        }
    }
    free(y);
    return errs;
}

/*
 * Release the pages of n finished slots (tiny-vllm part 6, "The lifetime of a
 * physical block: free_blocks"): for each slot in the given order, for every
 * layer, for every logical block in increasing order, a table entry that is
 * not -1 is pushed onto the back of the free stack and reset to -1.
 * free_pages has room for `capacity` entries; a push beyond it sets
 * STACK_FULL and leaves that entry (and the page) as it was.  A slot outside
 * [0, n_slots) sets BAD_SLOT and is skipped.  Returns the OR of the bits.
 */
int oracle_kv_release(const int32_t *slots, int n, int32_t *block_table, int n_slots,
                      int n_layers, int mbps, int32_t *free_pages, int32_t *top, int capacity)
{
    int errs = 0;
    for (int i = 0; i < n; ++i) {
        int slot = slots[i];
        if (slot < 0 || slot >= n_slots) {
            errs |= ORACLE_ERR_BAD_SLOT;
            continue;
        }
        for (int l = 0; l < n_layers; ++l)
            for (int blk = 0; blk < mbps; ++blk) {
                int32_t *entry = block_table + ((int64_t)slot * n_layers + l) * mbps + blk;
                if (*entry == -1)
                    continue;
                if (*top >= capacity) {
                    errs |= ORACLE_ERR_STACK_FULL;
                    continue;
                }
                free_pages[*top] = *entry;
                *top += 1;
                *entry = -1;
            }
    }
    return errs;
}

/* ------------------------------------------------------------------------ */
/* Backward of the dense attention (FlashAttention-2 explainer, "Results"   */
/* and the MQA/GQA paragraph: gradients of the same exact attention; the     */
/* key/value gradients of a GQA group are summed over its query heads).     */
/* ------------------------------------------------------------------------ */

/*
 * Gradients of loss = sum(O * dO) for O = softmax(scale * q K^T) V over the
 * visible keys, written out from the derivative of that definition, row by
 * row (i = query row, j = visible key):
 *   P_ij  = exp(s_ij - LSE_i)                     (the forward's weights)
 *   dV_j += P_ij dO_i
 *   dP_ij = dO_i . V_j
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij K_j
 *   dK_j += scale * dS_ij q_i
 * Inputs as oracle_attn_dense plus dO [B][T][Hq][d] (bf16); outputs dQ
 * [B][T][Hq][d], dK, dV [B][T][Hkv][d] in double.  aQ, aK, aV (nullable)
 * receive the same sums taken over absolute values of every term
 * (|dS_ij| |K_j| ...), the scale of each output's rounding error.
 * pairs (nullable, n_pairs (b, kv head) pairs): evaluate only those.
 * eQ, eK (nullable): how far dQ, dK move when D_i is taken from an output O
 * that was rounded to bf16 after a product with bf16-rounded weights, as an
 * implementation that reads the forward's O does: with
 *   E_i = 2^-8 * sum_c |dO_ic| (|O_ic| + sum_j P_ij |V_jc|)     (bound on |dD_i|)
 * (2^-8: the largest relative error of rounding to bf16, whose significand
 * holds 8 bits, applied to O itself and to every weight P_ij of its sum)
 * eQ_ic = scale E_i sum_j P_ij |K_jc| and eK_jc = scale sum_i P_ij E_i |q_ic|.
 */
void oracle_attn_dense_backward(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const uint16_t *dout, int B, int T, int Hq, int Hkv, int d,
                                double scale, int causal, const int32_t *pairs, int n_pairs,
                                double *dQ, double *dK, double *dV, double *aQ, double *aK,
                                double *aV, double *eQ, double *eK)
{
    int g = Hq / Hkv;
    int64_t nq = (int64_t)B * T * Hq * d;
    memset(dQ, 0, sizeof(double) * (size_t)nq);
    if (aQ)
        memset(aQ, 0, sizeof(double) * (size_t)nq);
    if (eQ)
        memset(eQ, 0, sizeof(double) * (size_t)nq);
    if (eK)
        memset(eK, 0, sizeof(double) * (size_t)((int64_t)B * T * Hkv * d));
    int64_t nkv = (int64_t)B * T * Hkv * d;
    memset(dK, 0, sizeof(double) * (size_t)nkv);
    memset(dV, 0, sizeof(double) * (size_t)nkv);
    if (aK)
        memset(aK, 0, sizeof(double) * (size_t)nkv);
    if (aV)
        memset(aV, 0, sizeof(double) * (size_t)nkv);
    /* one (sequence, kv head) per task: its dK, dV rows belong to it alone;
       pairs (nullable): only the listed (b, kv head) pairs are evaluated, the
       outputs of the others stay 0 */
    int64_t n_tasks = pairs ? n_pairs : (int64_t)B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < n_tasks; ++task) {
        int64_t bk = pairs ? (int64_t)pairs[2 * task] * Hkv + pairs[2 * task + 1] : task;
        int b = (int)(bk / Hkv), kvh = (int)(bk % Hkv);
        double *s = malloc(sizeof(double) * (size_t)T);
        double *dp = malloc(sizeof(double) * (size_t)T);
        double *qd = malloc(sizeof(double) * (size_t)d);
        double *od = malloc(sizeof(double) * (size_t)d);
        double *oex = malloc(sizeof(double) * (size_t)d);
        double *pva = malloc(sizeof(double) * (size_t)d);
        for (int h = kvh * g; h < (kvh + 1) * g; ++h) {
            for (int i = 0; i < T; ++i) {
                int n = causal ? i + 1 : T;
                const uint16_t *qr = q + (((int64_t)b * T + i) * Hq + h) * d;
                const uint16_t *dor = dout + (((int64_t)b * T + i) * Hq + h) * d;
                for (int c = 0; c < d; ++c) {
                    qd[c] = bf16_to_double(qr[c]);
                    od[c] = bf16_to_double(dor[c]);
                }
                double m = -INFINITY;
                for (int j = 0; j < n; ++j) {
                    const uint16_t *kr = k + (((int64_t)b * T + j) * Hkv + kvh) * d;
                    const uint16_t *vr = v + (((int64_t)b * T + j) * Hkv + kvh) * d;
                    double dot = 0.0, dv = 0.0;
                    for (int c = 0; c < d; ++c) {
                        dot += qd[c] * bf16_to_double(kr[c]);
                        dv += od[c] * bf16_to_double(vr[c]);
                    }
                    s[j] = scale * dot;
                    dp[j] = dv;
                    if (s[j] > m)
                        m = s[j];
                }
                double l = 0.0;
                for (int j = 0; j < n; ++j)
                    l += exp(s[j] - m);
                double lse = m + log(l);
                double D = 0.0;
                for (int j = 0; j < n; ++j)
                    D += exp(s[j] - lse) * dp[j];
                double E = 0.0;
                if (eQ || eK) {
                    for (int c = 0; c < d; ++c)
                        oex[c] = pva[c] = 0.0;
                    for (int j = 0; j < n; ++j) {
                        double p = exp(s[j] - lse);
                        const uint16_t *vr = v + (((int64_t)b * T + j) * Hkv + kvh) * d;
                        for (int c = 0; c < d; ++c) {
                            double vc = bf16_to_double(vr[c]);
                            oex[c] += p * vc;
                            pva[c] += p * fabs(vc);
                        }
                    }
                    for (int c = 0; c < d; ++c)
                        E += fabs(od[c]) * (fabs(oex[c]) + pva[c]);
                    E *= ldexp(1.0, -8);
                }
                double *dq = dQ + (((int64_t)b * T + i) * Hq + h) * d;
                double *aq = aQ ? aQ + (((int64_t)b * T + i) * Hq + h) * d : NULL;
                double *eq = eQ ? eQ + (((int64_t)b * T + i) * Hq + h) * d : NULL;
                for (int c = 0; c < d; ++c) {
                    dq[c] = 0.0;
                    if (aq)
                        aq[c] = 0.0;
                }
                for (int j = 0; j < n; ++j) {
                    double p = exp(s[j] - lse);
                    double ds = p * (dp[j] - D);
                    int64_t kvo = (((int64_t)b * T + j) * Hkv + kvh) * d;
                    const uint16_t *kr = k + kvo;
                    for (int c = 0; c < d; ++c) {
                        double kc = bf16_to_double(kr[c]);
                        dq[c] += scale * ds * kc;
                        dK[kvo + c] += scale * ds * qd[c];
                        dV[kvo + c] += p * od[c];
                        if (aq)
                            aq[c] += scale * fabs(ds * kc);
                        if (aK)
                            aK[kvo + c] += scale * fabs(ds * qd[c]);
                        if (aV)
                            aV[kvo + c] += fabs(p * od[c]);
                        if (eq)
                            eq[c] += scale * E * p * fabs(kc);
                        if (eK)
                            eK[kvo + c] += scale * p * E * fabs(qd[c]);
                    }
                }
            }
        }
        free(s);
        free(dp);
        free(qd);
        free(od);
        free(oex);
        free(pva);
    }
}
