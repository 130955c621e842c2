/*
 * prefill_attn.h -- C ABI of the MI355X (gfx950) long-context prefill attention library.
 *
 * Four operations make up the path:
 *   prefill_attn_dense        chunked prefill attention under an arbitrary additive mask
 *                             (prefill_attn_dense_causal: causal by position, no mask buffer;
 *                              prefill_attn_dense_bits: a keep/drop mask packed one bit per key)
 *   build_pooled_index        mean-pooled key/value blocks
 *   select_blocks             alpha-threshold block selection plus the local diagonal
 *   prefill_attn_blocksparse  exact attention on selected blocks + pooled correction
 * and the last three have *_ld forms for chunked prefill over a growing history
 * (a pooled index with spare capacity, pooled incrementally).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - bf16 and fp16 values travel as raw 16-bit patterns (uint16_t).
 * - Every tensor pointer is a DEVICE pointer owned by the caller. The library
 *   never allocates, frees, or keeps a pointer after the call returns; scratch
 *   memory comes from the caller through `workspace`.
 * - Tensors are dense and row-major in the order written; "token-major" means
 *   [token][head][head_dim]. Pointers must be 16-byte aligned.
 * - Query head h reads KV head h / (n_q / n_kv)  (grouped-query attention with
 *   contiguous groups). n_q must be a multiple of n_kv.
 * - head_dim d must be 64 or 128; `block` must be a power of two in [16, 256].
 * - `stream` is a hipStream_t (NULL = the null stream). A call validates its
 *   arguments on the host first; on any error it returns a negative status and
 *   enqueues nothing. On success it enqueues its kernels on `stream` and returns
 *   0 without synchronising. No call falls back to another implementation.
 * - Batch size is 1; loop over sequences for a batch.
 *
 * Sources (page title, section):
 *   "ANE Prefill Research" -- How the ANE prefill path works (what crosses the
 *     boundary: the chunk's rows, a token-major K/V history and an additive
 *     mask go in; the attention output comes out; the mask is arbitrary, not
 *     causal by contract); What worked, item 2 (a selection folded into the
 *     mask as -30000 contributes exactly nothing).
 *   "Flash attention on ANE: fast long-context prefill" -- Flash attention:
 *     the core insight (tiles and an online softmax instead of the N x N matrix).
 *   "Wiring CoreML to on-device LLMs: KV-cache, ANE, and the token budget for
 *     iPhone 16" -- The KV-cache growth formula (a static, caller-allocated
 *     cache addressed by position).
 *   "Porting FlashPrefill V2 to Apple silicon for faster prefill" -- Part I
 *     (pooled index, threshold selection plus diagonal, exact peaks and a
 *     pooled correction for the rest).
 */
#ifndef PREFILL_ATTN_H
#define PREFILL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  PA_OK = 0,
  PA_EINVAL = -1,        /* a bad argument: null/misaligned pointer, inconsistent sizes, bad scalar */
  PA_EUNSUPPORTED = -2,  /* valid but outside what the kernels implement (d, block, sizes) */
  PA_EHIP = -3,          /* the HIP runtime reported an error while enqueueing */
  PA_EWORKSPACE = -4,    /* workspace missing or smaller than the size helper returned */
  PA_ESCRATCH = -5       /* prefill_attn_dense_noalloc: the sizes need more than its static scratch */
};

/* Human-readable text for a status; for PA_EHIP it includes the runtime's message
 * of the most recent failure on the calling thread. Never NULL. */
const char* pa_status_string(int status);

/*
 * prefill_attn_dense -- one chunk of prefill attention over its K/V history.
 * ("ANE Prefill Research", How the ANE prefill path works; "Flash attention on
 * ANE", Flash attention: the core insight; "The Four Principles for Optimizing
 * Transformers on the ANE", Principle 3, additive pre-softmax masks.)
 *
 *   Q        bf16 [C][n_q][d]      the chunk's query rows
 *   K, V     bf16 [T][n_kv][d]     token-major keys/values: history plus the chunk's own
 *   mask     fp16 [C][mask_ld]     additive mask, columns 0..T-1 used, shared by all heads;
 *                                  an entry <= -30000 (or -inf) omits the key (weight exactly 0)
 *   scale    softmax scale, finite and > 0
 *   O        fp32 [C][n_q][d]      output; a row whose keys are all omitted gets zeros
 *
 *   O[i][h] = sum_t w_t V[t][g(h)],  w = softmax_t(scale * Q[i][h].K[t][g(h)] + mask[i][t])
 *
 * Arithmetic: scores from bf16 Q and K with fp32 accumulation; the softmax
 * weights are rounded to fp16 and multiplied with V staged as fp16 (times a
 * power of two that keeps max |V| below 2^15; exact for bf16 values in fp16's
 * normal range after that factor), accumulated in fp32.
 *
 * Requires C >= 1, 1 <= T <= 2^22 - 4096, mask_ld >= T (K and V may be any size). The mask alone decides visibility; the
 * library assumes nothing about causality. `workspace` must hold at least
 * prefill_attn_dense_workspace(C, T, n_q, n_kv, d) bytes (tile flags, the staged
 * fp16 copy of V[0..T) -- T * n_kv * d * 2 bytes -- and, when the key range is
 * split across workgroups, partial results); it is scratch, needs no
 * initialisation and may be reused after the stream reaches the call's end.
 * Errors: PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP.
 */
int prefill_attn_dense(const uint16_t* Q, int C, int n_q,
                       const uint16_t* K, const uint16_t* V, int T, int n_kv, int d,
                       const uint16_t* mask, int64_t mask_ld,
                       float scale, float* O,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes prefill_attn_dense needs for these sizes (0 for invalid sizes). */
size_t prefill_attn_dense_workspace(int C, int T, int n_q, int n_kv, int d);

/*
 * prefill_attn_dense_noalloc -- prefill_attn_dense for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation and arguments without
 * `workspace`. Its scratch is a static device array inside the library of
 * PA_NOALLOC_SCRATCH_BYTES (80 MiB), one copy per GPU, held until the process
 * ends. The call allocates nothing (no hipMalloc, no events: the kernel timing
 * hooks do not see it) and needs no initialised scratch.
 * Sizes whose prefill_attn_dense_workspace(C, T, n_q, n_kv, d) exceeds the
 * array return PA_ESCRATCH with nothing enqueued; the largest such size is
 * prefill_attn_dense_noalloc_limit(). The staged values take T * n_kv * d * 2
 * bytes of it, so, for example, 32,768 keys of 8 KV heads at d = 128 fit.
 * Every call on one GPU uses that GPU's one array: calls that may overlap on a
 * GPU (other streams, other host threads) race and must be serialised by the
 * caller; calls in order on one stream are safe.
 * Errors: PA_EINVAL, PA_EUNSUPPORTED, PA_ESCRATCH, PA_EHIP.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)
int prefill_attn_dense_noalloc(const uint16_t* Q, int C, int n_q,
                               const uint16_t* K, const uint16_t* V, int T, int n_kv, int d,
                               const uint16_t* mask, int64_t mask_ld,
                               float scale, float* O, void* stream);
size_t prefill_attn_dense_noalloc_limit(void);

/*
 * prefill_attn_dense_bits -- prefill_attn_dense with a keep/drop mask packed one
 * bit per (row, key) instead of fp16 (16x less mask traffic).
 * ("ANE Prefill Research", What worked, item 2: a -30000 entry drops a key, a 0
 * entry keeps it; the compact mask form of a 0 / -30000 mask.)
 *
 *   mask_bits  uint32 [C][bits_ld]   bit (t % 32) of word t / 32 of row i set: key t
 *                                    kept (additive 0); clear: key t dropped (as -30000).
 *                                    Bits of keys >= T are ignored.
 *
 * Equals prefill_attn_dense with mask[i][t] = bit ? 0 : -30000 (bit-for-bit the
 * same arithmetic). Requires bits_ld >= ceil(T / 32) (words); other requirements
 * and the workspace (prefill_attn_dense_workspace) as prefill_attn_dense.
 * Errors: PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP.
 */
int prefill_attn_dense_bits(const uint16_t* Q, int C, int n_q,
                            const uint16_t* K, const uint16_t* V, int T, int n_kv, int d,
                            const uint32_t* mask_bits, int64_t bits_ld,
                            float scale, float* O,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * prefill_attn_dense_causal -- prefill_attn_dense for a causal chunk without a
 * [C][T] mask buffer, optionally with a per-key mask broadcast over the rows.
 * ("The Four Principles for Optimizing Transformers on the ANE", Principle 3:
 * additive pre-softmax masks, a per-(query, key) mask and a per-key padding
 * mask composed by addition.)
 *
 *   rows are at positions q_start .. q_start+C-1; row i sees key t iff t <= q_start + i
 *   kmask    fp16 [T] or NULL    per-key additive mask (e.g. padding), shared by every row;
 *                                an entry <= -30000 (or -inf) omits the key
 *
 * Equals prefill_attn_dense with mask[i][t] = (t > q_start+i or kmask[t] <= -30000)
 * ? -30000 : kmask[t] (0 without kmask). The causal tile structure is computed,
 * not read, so no C x T mask is stored or scanned.
 * Requires q_start >= 0 and q_start + C <= T; other requirements and the
 * workspace (prefill_attn_dense_workspace) as prefill_attn_dense.
 * Errors: PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP.
 */
int prefill_attn_dense_causal(const uint16_t* Q, int C, int q_start, int n_q,
                              const uint16_t* K, const uint16_t* V, int T, int n_kv, int d,
                              const uint16_t* kmask, float scale, float* O,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * build_pooled_index -- mean of each block of `block` consecutive keys (and values).
 * ("Porting FlashPrefill V2 to Apple silicon", Compress keys before the heavy work.)
 *
 *   K, V            bf16 [T][n_kv][d]
 *   K_pool, V_pool  fp32 [n_kv][ceil(T/block)][d]
 *
 * Each mean is summed in fp64 in increasing key order, divided once by the
 * block's key count (the last block may be partial) and rounded once to fp32,
 * so the result is reproducible bit for bit.
 * Errors: PA_EINVAL, PA_EUNSUPPORTED, PA_EHIP.
 */
int build_pooled_index(const uint16_t* K, const uint16_t* V, int T, int n_kv, int d, int block,
                       float* K_pool, float* V_pool, void* stream);

/*
 * select_blocks -- which key blocks each query block attends to exactly.
 * ("Porting FlashPrefill V2 to Apple silicon", A cheap map of where the
 * attention lives; The algorithm starts here; figure "Where the kept blocks are".)
 *
 *   Q        bf16 [C][n_q][d]   chunk rows at absolute positions q_start .. q_start+C-1
 *   K_pool   fp32 [n_kv][ceil(T/block)][d] from build_pooled_index; T == q_start + C
 *   sel_idx  int32 [n_kv][n_qblk][ceil(T/block)]
 *   sel_cnt  int32 [n_kv][n_qblk],  n_qblk = (q_start+C-1)/block - q_start/block + 1
 *
 * For row i at position p, query block j = p / block, and each fully visible
 * block b < j: r_ib = Q[i].K_pool[b] (fp64, summed over d in increasing order),
 * M_i = max_b r_ib. Row i votes for b iff r_ib - M_i > ln(alpha)/scale (strict;
 * alpha = 0 keeps every block). The selection of (KV head g, query block j) is
 * the union of the votes of this call's rows in block j over g's query heads,
 * plus j itself. sel_idx lists it in ascending order (so j comes last) and is
 * zero past sel_cnt. Until the call completes, sel_idx may also hold partial
 * votes, so it must not overlap Q or K_pool.
 * Requires alpha finite and >= 0, scale finite and > 0,
 * ceil(T/block) <= 8192.
 * Errors: PA_EINVAL, PA_EUNSUPPORTED, PA_EHIP.
 */
int select_blocks(const uint16_t* Q, int C, int q_start, int n_q, int n_kv, int d,
                  const float* K_pool, int T, int block, float alpha, float scale,
                  int32_t* sel_idx, int32_t* sel_cnt, void* stream);

/*
 * prefill_attn_blocksparse -- causal block-sparse prefill attention.
 * ("Porting FlashPrefill V2 to Apple silicon", Compute the peaks, summarize the rest.)
 *
 *   Q, K, V, K_pool, V_pool, sel_idx, sel_cnt as above; T == q_start + C.
 *   O   fp32 [C][n_q][d]
 *
 * Row i (position p, block j) of head h (KV head g) takes exact attention over
 * every key of each selected block b < j and over keys j*block..p of its own
 * block, and, for every unselected block b < j, the pooled pair
 * (K_pool[g][b], V_pool[g][b]) with weight block * exp(scale*Q.K_pool - m):
 * a skipped block stands for its `block` keys. All terms share one softmax.
 * The selection arrays come from select_blocks for the same chunk. A list is
 * read as a set: entries outside [0, j) and duplicates are ignored, the
 * diagonal block j is always taken exactly whatever the list holds, and
 * sel_cnt is clamped to [0, ceil(T/block)].
 * Arithmetic as prefill_attn_dense (pooled keys enter as bf16, pooled values as
 * fp16 with the staged values' factor). `workspace` must hold at least
 * prefill_attn_blocksparse_workspace(T, n_kv, d) bytes (the staged fp16 copy of
 * V[0..T), and the pooled keys and values rounded once per call as they enter
 * the matrix cores, with room for the smallest block size); scratch, as for
 * prefill_attn_dense. Every block size select_blocks
 * takes is supported (tuned for 128; smaller blocks give steps of 64 keys that
 * rows of different query blocks take differently, run with a per-key test).
 * Errors: PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP.
 */
int prefill_attn_blocksparse(const uint16_t* Q, int C, int q_start, int n_q,
                             const uint16_t* K, const uint16_t* V, int T, int n_kv, int d,
                             const float* K_pool, const float* V_pool, int block,
                             const int32_t* sel_idx, const int32_t* sel_cnt,
                             float scale, float* O,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes prefill_attn_blocksparse(_ld) needs for these sizes (0 for invalid sizes). */
size_t prefill_attn_blocksparse_workspace(int T, int n_kv, int d);

/*
 * fold_keep_mask -- a sparse indexer's compacted selection folded into the
 * additive mask that prefill_attn_dense consumes. ("ANE Prefill Research",
 * What worked, item 2: the runtime folds keepIndices / keepCounts into the mask
 * as -30000, which contributes exactly nothing.)
 *
 *   keep_idx  int32 [C][keep_ld]  per row, the kept blocks of `width` keys (block c = keys
 *                                 c*width .. c*width+width-1); may be NULL when keep_ld == 0
 *   keep_cnt  int32 [C]           entries used in each row (clamped to 0 .. keep_ld)
 *   mask      fp16 [C][mask_ld]   output; columns 0..T-1 written, the rest untouched
 *
 * Row i sits at position p = q_start + i. mask[i][t] = 0 when t <= p and t lies in
 * a listed block or among the `recent` keys ending at p; otherwise -30000.
 * Listed blocks outside [0, ceil(T/width)) are ignored.
 * Requires C >= 1, q_start >= 0, q_start + C <= T <= mask_ld, width >= 1, recent >= 0.
 * Errors: PA_EINVAL, PA_EHIP.
 */
int fold_keep_mask(const int32_t* keep_idx, int64_t keep_ld, const int32_t* keep_cnt, int C,
                   int q_start, int T, int width, int recent, uint16_t* mask, int64_t mask_ld,
                   void* stream);

/*
 * fold_keep_bits -- the same fold as fold_keep_mask, written as the bit-packed
 * keep mask that prefill_attn_dense_bits consumes (one bit per row and key
 * instead of an fp16 entry). ("ANE Prefill Research", What worked, item 2.)
 *
 *   keep_idx, keep_cnt  as fold_keep_mask
 *   bits      uint32 [C][bits_ld]  output; bit t % 32 of word t / 32 of row i is set
 *                                  exactly where fold_keep_mask writes 0; bits of keys
 *                                  >= T in the last word are clear; words past
 *                                  ceil(T/32) are untouched
 *
 * Requires C >= 1, q_start >= 0, q_start + C <= T, bits_ld >= ceil(T/32),
 * width >= 1, recent >= 0, keep_cnt and bits 16-byte aligned.
 * Errors: PA_EINVAL, PA_EHIP.
 */
int fold_keep_bits(const int32_t* keep_idx, int64_t keep_ld, const int32_t* keep_cnt, int C,
                   int q_start, int T, int width, int recent, uint32_t* bits, int64_t bits_ld,
                   void* stream);

/*
 * prefill_attn_gather -- attention over a sparse indexer's compacted selection
 * without a mask: each row scores only the keys it keeps. ("ANE Prefill Research",
 * What worked, item 2, for the selection lists; "What would re-open it", for
 * gathering the kept keys instead of masking the history.)
 *
 *   Q         bf16 [C][n_q][d]       row i is at position q_start + i
 *   K, V      bf16 [T][n_kv][d]      token-major history and chunk keys
 *   keep_idx  int32 [C][keep_ld]     per row, kept blocks of `width` keys (block c = keys
 *                                    c*width .. c*width+width-1); may be NULL when keep_ld == 0
 *   keep_cnt  int32 [C]              entries used in each row (clamped to 0 .. keep_ld)
 *   O         fp32 [C][n_q][d]       output
 *
 * The result is prefill_attn_dense over the mask fold_keep_mask builds from the
 * same lists: row i (position p) attends to the keys t <= p of its listed blocks
 * and to the `recent` keys ending at p, each once (duplicate and out-of-range
 * entries are ignored); a row that keeps no key outputs zeros. Scores, weights
 * and sums are fp32 (no fp16 rounding of the weights); K and V are read as given
 * (no value staging), so no workspace is needed.
 * Requires C >= 1, q_start >= 0, q_start + C <= T, n_q % n_kv == 0, width >= 1,
 * recent >= 0, keep_ld >= 0, finite scale > 0.
 * Errors: PA_EINVAL; PA_EUNSUPPORTED for d other than 64 and 128, width above 64, or
 * a history whose per-row block bitmap and list (4 * (ceil(T/width/32) +
 * min(keep_ld, ceil(T/width))) bytes) exceed the 160 KB of a CU's LDS; PA_EHIP.
 */
int prefill_attn_gather(const uint16_t* Q, int C, int q_start, int n_q, const uint16_t* K,
                        const uint16_t* V, int T, int n_kv, int d, const int32_t* keep_idx,
                        int64_t keep_ld, const int32_t* keep_cnt, int width, int recent, float scale,
                        float* O, void* stream);

/*
 * Chunked block-sparse prefill over a growing history: the same three steps
 * with a pooled index that is built incrementally and kept between chunks.
 * ("Porting FlashPrefill V2 to Apple silicon", Part I: the pooled index
 * summarises the history by blocks; "ANE Prefill Research", How the ANE prefill
 * path works: a prompt is prefilled chunk by chunk over the accumulated K/V.)
 *
 * Each takes the pooled arrays with a row capacity `pool_ld` per KV head:
 *   K_pool, V_pool  fp32 [n_kv][pool_ld][d], pool_ld >= ceil(T/block)
 * so one allocation sized for the longest history serves every chunk, and a
 * block pooled once stays valid (its keys never change).
 *
 * build_pooled_index_ld -- pools blocks b_first .. ceil(T/block)-1 of K[0..T) and
 *   V[0..T) (same arithmetic as build_pooled_index) and leaves blocks below
 *   b_first untouched. For chunk after chunk, b_first = floor(T_prev/block)
 *   re-pools the previous partial block, if any, with its new keys.
 *   Requires 0 <= b_first <= ceil(T/block); b_first == ceil(T/block) enqueues nothing.
 * select_blocks_ld, prefill_attn_blocksparse_ld -- as select_blocks and
 *   prefill_attn_blocksparse, reading the pooled rows of blocks 0..ceil(T/block)-1
 *   from arrays with row capacity pool_ld. sel_idx keeps its per-call layout
 *   [n_kv][n_qblk][ceil(T/block)].
 * select_blocks_ld also keeps blocks by rule ("Porting FlashPrefill V2 to Apple
 *   silicon", figure "Where the kept blocks are": sinks, a local window and a
 *   dense tail are kept whatever their scores). For query block j:
 *     sink_tokens        every block b < j holding one of the first sink_tokens keys;
 *     window_blocks      blocks j-window_blocks .. j-1;
 *     dense_tail_blocks  every b < j when j is among the last dense_tail_blocks
 *                        query blocks of this call's rows (pass it on the final chunk).
 *   All three zero gives exactly select_blocks' selection.
 * select_blocks(...) is select_blocks_ld(..., pool_ld = ceil(T/block), no rules, ...),
 * and likewise for the other two (b_first = 0).
 * Errors: as the base calls; pool_ld < ceil(T/block), b_first out of range or a
 * negative rule count is PA_EINVAL.
 */
int build_pooled_index_ld(const uint16_t* K, const uint16_t* V, int T, int n_kv, int d, int block,
                          int b_first, float* K_pool, float* V_pool, int pool_ld, void* stream);

int select_blocks_ld(const uint16_t* Q, int C, int q_start, int n_q, int n_kv, int d,
                     const float* K_pool, int pool_ld, int T, int block, float alpha, float scale,
                     int sink_tokens, int window_blocks, int dense_tail_blocks,
                     int32_t* sel_idx, int32_t* sel_cnt, void* stream);

int prefill_attn_blocksparse_ld(const uint16_t* Q, int C, int q_start, int n_q,
                                const uint16_t* K, const uint16_t* V, int T, int n_kv, int d,
                                const float* K_pool, const float* V_pool, int pool_ld, int block,
                                const int32_t* sel_idx, const int32_t* sel_cnt,
                                float scale, float* O,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel timing (instrumentation for benchmarks; off by default).
 * When enabled, each launch of the named kernels is bracketed by HIP events
 * recorded on the launch stream. pa_timing_read synchronises those events and
 * returns the summed milliseconds and launch count for `kernel`, one of
 * "attn_dense", "attn_blocksparse", "mask_classify", "stage_values", "attn_combine", "pool",
 * "select", "fold", "attn_gather". "stage_values" covers the two passes of the fp16 value
 * staging.
 * "select" covers the selection kernel and, when the call splits
 * its voters over several workgroups, the merge kernel after it.
 * pa_timing_reset clears the totals. Returns PA_OK or PA_EINVAL/PA_EHIP.
 */
int pa_timing_enable(int on);
int pa_timing_reset(void);
int pa_timing_read(const char* kernel, double* total_ms, int64_t* launches);

/* Selection path counters (diagnostics; "Porting FlashPrefill V2 to Apple
 * silicon", A cheap map of where the attention lives: the selection must be
 * exact, so which of its exact paths a run took is worth knowing). Every voter
 * tile of a select_blocks / select_blocks_ld call on the current device adds to
 *   counts[0]  voter tiles scored,
 *   counts[1]  tiles whose ambiguous pairs were decided in fp64 (listed once),
 *   counts[2]  tiles whose ambiguous list overflowed and were relisted group by
 *              group (pass 2),
 *   counts[3]  tiles decided in fp64 pair by pair (magnitudes past the
 *              filter's range, |theta| past fp32's, or a near-max / max-job list
 *              that overflowed).
 * pa_select_path_counts waits for the device, copies the four totals since the
 * last reset into counts (host memory, 4 entries) and, if reset != 0, clears
 * them. The totals are shared by every caller on the device (calls running
 * concurrently add into the same counters). Returns PA_OK, PA_EINVAL (counts
 * null) or PA_EHIP. */
int pa_select_path_counts(int64_t* counts, int reset);

#ifdef __cplusplus
}
#endif

#endif /* PREFILL_ATTN_H */
