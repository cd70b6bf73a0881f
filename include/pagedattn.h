/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged causal GQA attention library
 * (libpagedattn.so).
 *
 * Three calls make up the path: kv_scatter writes new K/V rows into 16-token
 * pages, attn_prefill runs exact causal attention of a whole prompt over those
 * pages, attn_decode runs exact attention of one new query per sequence over
 * its cached context.  attn_prefill_dense is the same prefill over contiguous
 * (unpaged) K/V.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor pointer is a DEVICE pointer that the caller allocated and
 *   owns.  The library never allocates, frees or keeps a pointer after return.
 *   Tensor pointers must be 16-byte aligned.
 * - bf16 is IEEE bfloat16 stored as 2 bytes; fp32 is IEEE binary32.
 * - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work on
 *   it and return without waiting; outputs are ready when the stream is.
 * - Return value: PA_OK (0) after a successful enqueue, or a negative
 *   pa_status for an argument the host can check (NULL pointer, bad size,
 *   unsupported head_dim/group, misalignment, small workspace, launch failure).
 *   On a negative return nothing was enqueued.
 * - `err` (nullable, device int32): problems only the device can see (a
 *   block-table entry needed for a visible token that is -1 or >= n_pages, a
 *   slot id outside [0, n_slots), a position or length beyond what the table
 *   or the query tensor can hold) are OR-ed into *err as PA_DEVERR_* bits.
 *   The offending token is then left out (never dereferenced), exactly as if it
 *   were masked.  The caller clears *err beforehand.
 *
 * Paged KV layout (page "6. Splitting the KV cache into 16-token blocks",
 * tiny-vllm part 6, sections "Block contents: K in front, V after V_OFFSET"
 * and "block table")
 * ----------------------------------------------------------------------
 * - kv_cache is one buffer of n_pages physical pages.  A page holds 16 tokens:
 *   K as [token 16][kv_head n_kv_heads][dim head_dim] bf16, then V in the same
 *   order starting V_OFFSET = 16*n_kv_heads*head_dim*2 bytes into the page.
 *   Page bytes = 2*V_OFFSET (32768 for 8 KV heads x 64).
 * - block_table is int32 [n_slots][n_layers][max_blocks_per_seq]: the physical
 *   page of logical block p/16 of sequence slot s in layer l sits at index
 *   s*n_layers*max_blocks_per_seq + l*max_blocks_per_seq + p/16; -1 = none.
 * - So K[p][h][i] of (s, l) is at byte
 *   page*page_bytes + (p%16)*n_kv_heads*head_dim*2 + h*head_dim*2 + i*2,
 *   and V at the same byte + V_OFFSET.
 * - GQA: q head h reads kv head h / (Hq / Hkv) (consecutive groups; page
 *   "3. The prefill path", section "Per-head attention scores and GQA").
 *
 * Results (exact attention, FlashAttention-2 explainer "Step by step (the two
 * forward tweaks)"): O = softmax(scale * q K^T) V over the visible keys, and
 * LSE = m + ln(l), the natural-log log-sum-exp of the scaled scores.  A query
 * with no visible key gets O = 0 and LSE = -INFINITY.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL = -1,        /* a required pointer is NULL                          */
    PA_ERR_SHAPE = -2,       /* a size is negative/zero or sizes disagree            */
    PA_ERR_UNSUPPORTED = -3, /* no kernel for this head_dim / group size            */
    PA_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned              */
    PA_ERR_WORKSPACE = -5,   /* decode workspace smaller than the size it needs      */
    PA_ERR_RANGE = -6,       /* an index or byte offset would overflow its type      */
    PA_ERR_LAUNCH = -7,      /* the HIP runtime refused the launch                   */
    PA_ERR_VALUE = -8        /* a scalar argument is outside its domain (scale)      */
} pa_status;

/* Bits OR-ed into the optional device flag `err`. */
#define PA_DEVERR_BAD_PAGE 1 /* needed block-table entry is -1 or >= n_pages         */
#define PA_DEVERR_BAD_SLOT 2 /* slot id outside [0, n_slots)                          */
#define PA_DEVERR_BAD_POS 4  /* position/length outside the table (mbps*16) or T     */
#define PA_DEVERR_NO_FREE_PAGE 8 /* kv_append: the free stack ran out                 */
#define PA_DEVERR_DUP_SLOT 16    /* kv_append: a slot is named by two tokens           */
#define PA_DEVERR_REASSIGNED 32  /* kv_append: an opened block's entry was not -1      */
#define PA_DEVERR_STACK_FULL 64  /* kv_release: the free stack has no room left        */
#define PA_DEVERR_BAD_PLAN 128   /* attn_prefill_packed: a work item names no row block   */
                                 /* of the batch, or a partial slot past the workspace   */

/* Human-readable name of a pa_status value (static string, never NULL). */
const char *pa_status_string(int status);

/* Bytes of one physical page: 2 * 16 * n_kv_heads * head_dim * 2. */
int64_t pa_page_bytes(int n_kv_heads, int head_dim);

/*
 * pa_clock_probe -- a measurement aid, not a step of the attention path: the
 * shader clock the chip sustains while every SIMD issues bf16 matrix products
 * (32x32x16), so that MFMA throughput can be quoted against the peak at the
 * measured clock as well as at the rated one.  Each of n_waves waves (launched
 * as workgroups of four) runs `iters` steps of four independent products and
 * writes cycles / (100 MHz real-time ticks / 1e8) / 1e9 -- its clock in GHz --
 * to ghz[wave] (device memory, n_waves floats, caller-owned).  4096 waves fill
 * a 256-CU part with four waves per SIMD; 20000 steps last about a millisecond.
 * Errors: PA_ERR_NULL (ghz NULL with n_waves > 0), PA_ERR_SHAPE (n_waves or
 * iters < 0), PA_ERR_LAUNCH.  n_waves == 0 is a no-op.
 */
int pa_clock_probe(float *ghz, int n_waves, int iters, void *stream);

/*
 * kv_scatter -- write the K and V rows of n_tokens tokens into their pages
 * (page "3. The prefill path", section "Distributing K/V into paged blocks";
 * the decode append of page 6, section "Block contents").
 *
 *   k, v         [n_tokens][n_kv_heads][head_dim] bf16, read only.
 *   slot_ids     [n_tokens] int32: block-table slot of each token.
 *   positions    [n_tokens] int32: position of each token in its sequence.
 *   kv_cache     pool of n_pages pages (layout above), written in place: only
 *                the 2*n_kv_heads*head_dim*2 bytes of each token's two rows
 *                change; every other byte is left as it was.
 *   block_table  [n_slots][n_layers][max_blocks_per_seq] int32, read only;
 *                `layer` selects the layer.
 *   Pages are never allocated here: the entry for each token must already
 *   hold its page (the caller's free-list does the allocation).
 *   Two tokens naming the same (slot, position) race; the result is one of
 *   the two rows.  n_tokens == 0 is a no-op.  head_dim*n_kv_heads must be a
 *   multiple of 8.
 */
int kv_scatter(const void *k, const void *v, int64_t n_tokens, const int32_t *slot_ids,
               const int32_t *positions, void *kv_cache, int64_t n_pages,
               const int32_t *block_table, int n_slots, int n_layers, int max_blocks_per_seq,
               int layer, int n_kv_heads, int head_dim, int32_t *err, void *stream);

/*
 * attn_prefill -- causal (or full) grouped-query attention of a batch of
 * prompts over the paged cache (page "3. The prefill path", sections
 * "Per-head attention scores and GQA" and "causalMask and online softmax";
 * FlashAttention-2 explainer, sections "Step by step", "Parallelise along the
 * sequence length" and "Work partitioning between warps").
 *
 *   q            [B][T][Hq][head_dim] bf16; row t of sequence b is the query
 *                of the token at position t.
 *   kv_cache, block_table, n_pages, n_slots, n_layers, max_blocks_per_seq,
 *   layer        the paged cache, as for kv_scatter (read only).  The prompt's
 *                K/V must already be in it (kv_scatter first).
 *   slot_ids     [B] int32 block-table slot of each sequence (NULL: slot b).
 *   seq_lens     [B] int32, 0 <= seq_lens[b] <= T: the prompt length.
 *   causal       nonzero: query t sees keys 0..t; zero: keys 0..seq_len-1.
 *   scale        multiplies q.k (pass 1/sqrt(head_dim) for the usual scaling).
 *                It must be finite and > 0 (the pages scale by 1/sqrt(d));
 *                anything else returns PA_ERR_VALUE.  The same holds for the
 *                scale of every attention call below.
 *   O            [B][T][Hq][head_dim] bf16 output.
 *   LSE          [B][Hq][T] fp32 output (natural log, scaled scores).
 *   Rows t >= seq_lens[b] are written as O = 0, LSE = -INFINITY.
 *   Supported: head_dim 64 or 128, Hq/Hkv in {1, 2, 4, 8, 16}.
 */
int attn_prefill(const void *q, const void *kv_cache, int64_t n_pages, const int32_t *block_table,
                 int n_slots, int n_layers, int max_blocks_per_seq, int layer,
                 const int32_t *slot_ids, const int32_t *seq_lens, int B, int T, int Hq, int Hkv,
                 int head_dim, float scale, int causal, void *O, float *LSE, int32_t *err,
                 void *stream);

/*
 * attn_prefill_append -- a prefill step in one launch: the prompts' K/V rows
 * are written to their pages and the prompts attend to them.  The pages'
 * prefill attends to the K/V it has just computed while it copies them into
 * the cache (page "3. The prefill path", sections "Distributing K/V into paged
 * blocks" and "Per-head attention scores and GQA"); this call does both.  The
 * result is that of kv_scatter of every prompt token (slot slot_ids[b],
 * position t for t < seq_lens[b]) followed by attn_prefill: the pool bytes and
 * O, LSE are identical, errors included (a token on a missing page is flagged
 * PA_DEVERR_BAD_PAGE, not written, and left out of the attention).
 *
 *   q            [B][T][Hq][head_dim] bf16, as for attn_prefill.
 *   k, v         [B][T][Hkv][head_dim] bf16 (16-byte aligned): the prompts'
 *                K and V rows; rows t >= seq_lens[b] are not read.
 *   kv_cache     written (the prompt rows' bytes only); other cache arguments,
 *                slot_ids, seq_lens, causal, scale, O, LSE as for attn_prefill.
 *   slot_ids     must name distinct slots, as for attn_decode_append.
 */
int attn_prefill_append(const void *q, const void *k, const void *v, void *kv_cache, int64_t n_pages,
                        const int32_t *block_table, int n_slots, int n_layers, int max_blocks_per_seq,
                        int layer, const int32_t *slot_ids, const int32_t *seq_lens, int B, int T,
                        int Hq, int Hkv, int head_dim, float scale, int causal, void *O, float *LSE,
                        int32_t *err, void *stream);

/*
 * attn_prefill_chunk -- the prefill of a prompt chunk that continues a cached
 * prefix, and of mixed batches: sequence b has kv_lens[b] tokens in the
 * cache (prefix and chunk, the chunk's K/V already scattered) and its queries
 * are the LAST q_lens[b] of them.  Query row t is the token at position
 * kv_lens[b] - q_lens[b] + t (aligned to the end of the sequence); causal: it
 * sees keys 0 .. that position; full: all kv_lens[b] keys.  q_lens[b] == 1 is
 * a decode row (the newest token sees its whole context), q_lens[b] ==
 * kv_lens[b] is attn_prefill.  The pages only prefill fresh prompts
 * (tiny-vllm part 3, "Distributing K/V into paged blocks": the table entries
 * are still unassigned); the end alignment is the reading that keeps every
 * token's view the same as in a whole-prompt prefill.
 *
 *   q            [B][T][Hq][head_dim] bf16, row t < q_lens[b] as above.
 *   q_lens       [B] int32, 0 <= q_lens[b] <= min(T, kv_lens[b]) (required).
 *   kv_lens      [B] int32, cached tokens (no bound by T).
 *   O, LSE, other arguments as for attn_prefill; rows t >= q_lens[b] are
 *   written as O = 0, LSE = -INFINITY.  A q_len outside its range sets
 *   PA_DEVERR_BAD_POS and is clamped into it.
 */
int attn_prefill_chunk(const void *q, const void *kv_cache, int64_t n_pages,
                       const int32_t *block_table, int n_slots, int n_layers,
                       int max_blocks_per_seq, int layer, const int32_t *slot_ids,
                       const int32_t *q_lens, const int32_t *kv_lens, int B, int T, int Hq,
                       int Hkv, int head_dim, float scale, int causal, void *O, float *LSE,
                       int32_t *err, void *stream);

/*
 * attn_prefill_packed_plan / attn_prefill_packed -- attn_prefill_chunk for
 * PACKED query rows: sequence b's q_lens[b] queries are rows q_start[b] ..
 * q_start[b+1]-1 of q, O and LSE, so a batch mixing prompt chunks and decode
 * rows (q_lens[b] == 1) stores and computes no padding.  The same reading of
 * the pages as attn_prefill_chunk (queries aligned to the end of the sequence;
 * tiny-vllm part 6, "pagedAttentionKernel": a step attends its new queries
 * over all of the sequence's cached keys), with the key range of long row
 * blocks split across workgroups (FlashAttention-2 explainer, "Parallelise
 * along the sequence length") and the pieces merged by the log-sum-exp rule
 * (tiny-vllm part 3, "causalMask and online softmax").
 *
 * attn_prefill_packed_plan runs on the host, once per batch (every layer of
 * a step can reuse it): from HOST copies of q_lens[B] and kv_lens[B]
 * (0 <= q_lens[b] <= kv_lens[b], else PA_ERR_SHAPE) it writes the work list
 * to plan (host int32, plan_capacity entries; 6 * (n_work + n_merge) are
 * needed) and returns the counts and the workspace the run needs.  plan ==
 * NULL only computes the counts; a plan_capacity too small returns
 * PA_ERR_WORKSPACE with the counts set.  The split follows the CU count of
 * the current device.
 *
 * attn_prefill_packed runs the plan, copied to device memory by the caller:
 *   q            [total_q][Hq][head_dim] bf16 (16-byte aligned).
 *   kv_lens      [B] int32 (device), the same lengths the plan was made from.
 *   q_start      [B + 1] int32 (device), q_start[b+1] - q_start[b] == q_lens[b]
 *                of the plan, q_start[B] <= total_q.
 *   plan         the plan's 6 * (n_work + n_merge) int32 (device).
 *   workspace    device memory of at least the plan's workspace_bytes (may be
 *                NULL when n_merge == 0); its contents on entry do not matter.
 *   O            [total_q][Hq][head_dim] bf16; LSE [total_q][Hq] fp32: the
 *                rows of every sequence are written; other rows are left as
 *                they were.
 *   other arguments as for attn_prefill_chunk.  Two launches on `stream`
 *   (the prefill workgroups, then a small merge of the split row blocks).  A
 *   plan that does not match the lengths gives wrong rows but no access out
 *   of bounds: device-side, a length outside its range sets PA_DEVERR_BAD_POS
 *   and a work item naming no row block or a slot past the workspace sets
 *   PA_DEVERR_BAD_PLAN (the item is skipped).  Head groups 1, 2, 4, 8, 16.
 */
int attn_prefill_packed_plan(const int32_t *q_lens, const int32_t *kv_lens, int B, int Hq, int Hkv,
                             int head_dim, int causal, int32_t *plan, int64_t plan_capacity,
                             int64_t *n_work, int64_t *n_merge, size_t *workspace_bytes);
int attn_prefill_packed(const void *q, const void *kv_cache, int64_t n_pages,
                        const int32_t *block_table, int n_slots, int n_layers,
                        int max_blocks_per_seq, int layer, const int32_t *slot_ids,
                        const int32_t *kv_lens, const int32_t *q_start, int B, int64_t total_q,
                        int Hq, int Hkv, int head_dim, float scale, int causal,
                        const int32_t *plan, int64_t n_work, int64_t n_merge, void *workspace,
                        size_t workspace_bytes, void *O, float *LSE, int32_t *err, void *stream);

/*
 * attn_decode -- attention of one new query per sequence over its whole cached
 * context, the newest token included (page 6, sections "pagedAttentionKernel"
 * and "logical block -> physical block -> byte address").  Contexts are cut
 * into pieces across workgroups where needed and the pieces merged with the
 * log-sum-exp rule of the online softmax (page 3, "causalMask and online
 * softmax": two partial results are rescaled to the larger maximum and
 * added).  Two kernels serve it: for 8 kv heads of head_dim 64 (groups up to
 * 8, up to 512 sequences; see attn_decode_whole_pages) each workgroup streams
 * whole pages, all kv heads, of an equal share of the batch's pages and a
 * second small kernel merges the pieces; otherwise a workgroup per (sequence,
 * kv head) reads that head's slice of each page.
 *
 *   q            [B][Hq][head_dim] bf16, the query of the token at ctx_len-1.
 *   ctx_lens     [B] int32, tokens cached for each sequence including the
 *                newest; 0 gives O = 0, LSE = -INFINITY.
 *   max_ctx      host upper bound on every ctx_lens[b] (sizes the split grid);
 *                a larger ctx_lens[b] sets PA_DEVERR_BAD_POS and is cut to max_ctx.
 *   workspace    device scratch of attn_decode_workspace_size(B, Hq, Hkv,
 *                head_dim, max_ctx) bytes, 16-byte aligned, for the partial
 *                results of context pieces; the size is 0 (workspace may be
 *                NULL) when no context is cut.  Contents on entry do not
 *                matter; two calls in flight must not share it.
 *   O            [B][Hq][head_dim] bf16 output;  LSE [B][Hq] fp32 output.
 *   Other arguments as for attn_prefill.  Supported: head_dim 64 or 128,
 *   Hq/Hkv in {1, 2, 4, 8, 16}.
 */
int attn_decode(const void *q, const void *kv_cache, int64_t n_pages, const int32_t *block_table,
                int n_slots, int n_layers, int max_blocks_per_seq, int layer,
                const int32_t *slot_ids, const int32_t *ctx_lens, int B, int Hq, int Hkv,
                int head_dim, float scale, int max_ctx, void *workspace, size_t workspace_bytes,
                void *O, float *LSE, int32_t *err, void *stream);

/*
 * attn_decode_append -- one decode step in one launch: the new token of every
 * sequence is written to its page and attended to with the rest of the
 * context (page 6, "pagedAttentionKernel"; page 3, "Distributing K/V into
 * paged blocks" for the write).  The same result as kv_scatter of the new
 * tokens at positions ctx_lens[b] - 1 followed by attn_decode, to the
 * rounding of one token's contribution (the new token is added after the
 * cached ones instead of among them); the pool bytes are identical.
 *
 *   k_new, v_new [B][Hkv][head_dim] bf16 (16-byte aligned): the new token's
 *                K and V rows; written into kv_cache (which must be writable)
 *                at slot slot_ids[b], position ctx_lens[b] - 1.
 *   ctx_lens     [B] tokens of each sequence including the new one; a
 *                sequence with ctx_lens[b] == 0, a bad slot or a length that
 *                sets PA_DEVERR_BAD_POS writes nothing.  A missing page for
 *                the new token sets PA_DEVERR_BAD_PAGE; the token is then
 *                neither written nor attended to.
 *   slot_ids     must name distinct slots (one sequence per slot): two
 *                entries on one slot would write one position while the other
 *                reads it, and the results of both are then undefined.
 *   Other arguments, workspace and results as for attn_decode.
 */
int attn_decode_append(const void *q, const void *k_new, const void *v_new, void *kv_cache,
                       int64_t n_pages, const int32_t *block_table, int n_slots, int n_layers,
                       int max_blocks_per_seq, int layer, const int32_t *slot_ids,
                       const int32_t *ctx_lens, int B, int Hq, int Hkv, int head_dim, float scale,
                       int max_ctx, void *workspace, size_t workspace_bytes, void *O, float *LSE,
                       int32_t *err, void *stream);

/* Workspace bytes attn_decode needs for this batch shape (0 on bad sizes). */
size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int head_dim, int max_ctx);

/*
 * 1 when attn_decode (and attn_decode_noalloc) take the whole-page kernel for
 * this shape on the current device, 0 when they take the per-head kernel
 * (attn_decode_append always does).  Whole pages: head_dim 64, Hkv 8, Hq/Hkv
 * up to 8, 1 <= B <= 512, B * ceil(max_ctx / 16) pages at most 1024 per CU,
 * except B * Hkv between one and two times the CU count (there the per-head
 * kernel's schedule measured faster).  No device work; 0 on bad sizes.
 */
int attn_decode_whole_pages(int B, int Hq, int Hkv, int head_dim, int max_ctx);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and results, bit for bit, but the
 * partial results of split contexts go to a static device array inside the
 * library instead of a caller workspace.  Nothing is allocated or freed by
 * the call.
 *
 *   Arguments as for attn_decode, without workspace / workspace_bytes.
 *   Limit: the array holds 8 MiB on every GPU the library runs on, kept until
 *   the process ends; a batch shape whose attn_decode_workspace_size exceeds
 *   it returns PA_ERR_WORKSPACE (no shape does on a 256-CU MI355X, where the
 *   largest is about 4.3 MB).  The array's device address is looked up on the
 *   first call on each device (PA_ERR_LAUNCH if that lookup fails).
 *   All calls on one GPU share the array: calls that overlap in time on the
 *   same GPU (two streams, or two host threads) race and may return wrong
 *   results; calls in sequence on one stream are safe.  Every byte a call
 *   reads from the array it has written in the same call.
 */
int attn_decode_noalloc(const void *q, const void *kv_cache, int64_t n_pages,
                        const int32_t *block_table, int n_slots, int n_layers,
                        int max_blocks_per_seq, int layer, const int32_t *slot_ids,
                        const int32_t *ctx_lens, int B, int Hq, int Hkv, int head_dim, float scale,
                        int max_ctx, void *O, float *LSE, int32_t *err, void *stream);

/*
 * attn_prefill_dense -- the prefill on contiguous K/V (FlashAttention-2
 * explainer, section "Results": the attention-only benchmark shapes).
 *
 *   q            [B][T][Hq][head_dim] bf16;  k, v [B][T][Hkv][head_dim] bf16.
 *   O            [B][T][Hq][head_dim] bf16;  LSE [B][Hq][T] fp32.
 *   causal, scale as for attn_prefill; every sequence has length T.
 */
int attn_prefill_dense(const void *q, const void *k, const void *v, int B, int T, int Hq, int Hkv,
                       int head_dim, float scale, int causal, void *O, float *LSE, void *stream);

/*
 * attn_backward_dense -- gradients of exact attention on contiguous Q, K, V
 * (FlashAttention-2 explainer, "Parallelise along the sequence length": P is
 * recomputed from the stored log-sum-exp; MQA/GQA paragraph: dK, dV of a kv
 * head are the sums over the q heads that share it).  With S = scale q K^T,
 * P = exp(S - LSE) over the visible keys and D_i = sum_c dO_ic O_ic:
 *   dV_j = sum_i P_ij dO_i,  dS_ij = P_ij (dO_i . V_j - D_i),
 *   dQ_i = scale sum_j dS_ij K_j,  dK_j = scale sum_i dS_ij q_i.
 *
 *   q, o, dout   [B][T][Hq][head_dim] bf16 (o: the forward's output).
 *   k, v         [B][T][Hkv][head_dim] bf16.
 *   lse          [B][Hq][T] fp32, the forward's LSE (natural log).
 *   dq           [B][T][Hq][head_dim] bf16 output; dk, dv [B][T][Hkv][head_dim]
 *                bf16 outputs (every element written once: deterministic).
 *   workspace    attn_backward_workspace_size(B, T, Hq) bytes, 16-byte
 *                aligned (D of every row); contents on entry do not matter.
 *   causal, scale as for attn_prefill_dense.  Supported: head_dim 64 or 128,
 *   Hq/Hkv in {1, 2, 4, 8, 16}.  Two launches on `stream` (dQ and the per-row D
 *   first, then dK and dV).
 */
int attn_backward_dense(const void *q, const void *k, const void *v, const void *o,
                        const void *dout, const float *lse, int B, int T, int Hq, int Hkv,
                        int head_dim, float scale, int causal, void *dq, void *dk, void *dv,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes attn_backward_dense needs (0 on bad sizes). */
size_t attn_backward_workspace_size(int B, int T, int Hq);

/*
 * kv_append -- the cache writes of one decode step in one launch: for each of
 * B new tokens (one per sequence), in batch order,
 *   1. if its position opens a block (position % 16 == 0: tiny-vllm part 6,
 *      "The lifetime of a physical block: free_blocks", the decode rule), a
 *      page is popped from the back of the free stack and recorded in the
 *      block-table entry of that block;
 *   2. its K row is rotated by RoPE (tiny-vllm part 3, "RoPE: a rotation that
 *      references a table": pair i of a head is elements i and i + head_dim/2,
 *      y_i = x_i cos - x_{i+d/2} sin, y_{i+d/2} = x_i sin + x_{i+d/2} cos, with
 *      the angle of row `position`, column i of the tables) and written with
 *      its V row into the page, as kv_scatter would;
 *   3. if q_in is given, the token's query is rotated the same way into q_out.
 * Rotation arithmetic: fp64 (each product of a bf16 and an fp32 table value
 * is exact), one rounding to double, then to the nearest bf16, ties to even.
 *
 *   k, v         [B][n_kv_heads][head_dim] bf16 (k before rotation).
 *   q_in, q_out  [B][Hq][head_dim] bf16, both NULL (no query rotation) or
 *                both given; they may be the same buffer.  Hq is ignored when
 *                q_in is NULL.
 *   slot_ids     [B] int32 (NULL: slot b); positions [B] int32, the position
 *                of the new token (its sequence's length before the append).
 *   cos_t, sin_t [max_pos][head_dim/2] fp32 angle tables (the pages keep
 *                [max_pos][head_dim] with each value twice; one copy is kept
 *                here).
 *   block_table  as for kv_scatter, READ AND WRITTEN: the entry of each
 *                opened block receives its page.
 *   free_pages   int32 [capacity] stack of free page ids, read only here:
 *                entries [0, top) are free, the last one is popped first
 *                (a top outside [0, capacity] is clamped into it).
 *   alloc_state  int32 [2] device: [0] = top, the number of free pages on the
 *                stack (lowered by the number of opening tokens, not below 0);
 *                [1] = an arrival counter used inside the launch, which must
 *                be 0 between calls (initialise the pair as {top, 0}).
 * Device errors (OR-ed into *err): BAD_SLOT, BAD_POS (position outside the
 * table or >= max_pos; the query is still rotated when 0 <= position <
 * max_pos), DUP_SLOT (two tokens of the call name one slot: their writes
 * race), NO_FREE_PAGE (the opening token finds the stack empty: not written,
 * entry left as it was), REASSIGNED (an opened block's entry was not -1: it
 * is overwritten, the old page is no longer referenced), BAD_PAGE (a popped
 * page or a looked-up entry outside [0, n_pages)).  A token with an invalid
 * slot or position pops nothing; every valid opening token takes its place in
 * the pop order even when it cannot be written.  Calls that overlap in time on
 * the same alloc_state race.  head_dim must be a multiple of 16 and
 * n_kv_heads * head_dim at most 8192; tensors and
 * tables 16-byte aligned, alloc_state 4-byte aligned.  B == 0 is a no-op.
 */
int kv_append(const void *k, const void *v, const void *q_in, void *q_out, int Hq, int B,
              const int32_t *slot_ids, const int32_t *positions, const float *cos_t,
              const float *sin_t, int max_pos, void *kv_cache, int64_t n_pages,
              int32_t *block_table, int n_slots, int n_layers, int max_blocks_per_seq, int layer,
              const int32_t *free_pages, int capacity, int32_t *alloc_state, int n_kv_heads,
              int head_dim, int32_t *err, void *stream);

/*
 * kv_release -- return the pages of finished slots to the free stack
 * (tiny-vllm part 6, "The lifetime of a physical block: free_blocks"): for
 * each slot of slots[0..n) in order, for every layer, for every logical block
 * in increasing order, an entry that is not -1 is pushed onto the back of the
 * stack (free_pages[top++] = entry) and reset to -1.
 *
 *   slots        [n] int32 device array of slot ids.
 *   block_table  [n_slots][n_layers][max_blocks_per_seq] int32, written.
 *   free_pages   int32 [capacity] stack, written at [top, top + pushed).
 *   alloc_state  int32 [2] as for kv_append; [0] is raised by the pushes (a
 *                top outside [0, capacity] is clamped into it first).
 * Device errors: BAD_SLOT (slot skipped), STACK_FULL (a push beyond capacity:
 * that entry and its page stay as they were).  One workgroup does the whole
 * release in order, so it suits occasional calls, not per-token ones.
 * n == 0 is a no-op.
 */
int kv_release(const int32_t *slots, int n, int32_t *block_table, int n_slots, int n_layers,
               int max_blocks_per_seq, int32_t *free_pages, int capacity, int32_t *alloc_state,
               int32_t *err, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
