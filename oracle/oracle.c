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
 * slot_ids[b] (NULL: slot b) and has seq_lens[b] <= T tokens, query t sitting
 * at position t.  Rows to evaluate are the (b, t) pairs rows[2i], rows[2i+1]
 * (rows == NULL: all B*T in order).  O: [n_rows][Hq][d], LSE: [n_rows][Hq].
 * A padding row (t >= seq_lens[b]) gets O = 0, LSE = -infinity.
 */
int64_t oracle_attn_prefill(const uint16_t *q, const uint8_t *pool, int64_t n_pages,
                            const int32_t *block_table, int n_slots, int n_layers, int mbps,
                            int layer, const int32_t *slot_ids, const int32_t *seq_lens,
                            int B, int T, int Hq, int Hkv, int d, double scale, int causal,
                            const int32_t *rows, int64_t n_rows, double *O, double *LSE)
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
        int64_t n_keys = t < len ? (causal ? (int64_t)t + 1 : len) : 0;
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
