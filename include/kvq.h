/*
 * kvq.h -- 2-bit mixed-precision paged KV cache with fused
 * dequantize-in-attention decode, for AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI: no HIP or torch types.  Device pointers are passed as void* /
 * float*, a HIP stream as void* (hipStream_t; NULL = the default stream).
 *
 * What the library computes (sources are web pages on KV-cache quantization):
 *  - KIVI explainer (aibr.jp), section 3: Keys quantized per channel, Values
 *    per token, asymmetric (min/max, zero-point) quantization, a residual kept
 *    in full precision, streaming append into the quantized cache.
 *  - Kitty abstract (fugumt, arXiv 2511.18643): per page, a small fraction of
 *    Key channels ranked by sensitivity is kept at 4 bits; a mixed-precision
 *    Key page is stored as two uniform 2-bit tensors; page-centric layout.
 *  - notes.yuuk.io "KV cache quantization", open questions: magnitude-based
 *    channel selection; boost ratios 12.5 % and 25 %; GQA key sharing.
 *  - MiniKV summary (f-binder), problem setting and method: keep the
 *    attention output close to the unquantized one; fuse the 2-bit unpack
 *    into the decode matmul.
 *
 * Numerics (fixed readings of what the pages leave open):
 *  - page = 128 tokens of one (sequence, KV head); Key groups = 32 tokens of
 *    one channel; Value groups = 32 channels of one token; window = 128;
 *  - quantizer: z = min, s = dtype_rne(fp32((max - min) / L)), code =
 *    clamp(rint_even(fp32(fp32(x - z) * fp32(1 / s))), 0, L), all IEEE fp32;
 *    s == 0 gives code 0; a zero minimum is stored as +0;
 *  - the k Key channels with the largest max|K| over the page (ties: lower
 *    channel) use L = 15, stored as lo = code & 3 (all channels) and hi =
 *    code >> 2 (boosted channels, ascending), others L = 3;
 *  - attention: o = softmax(scale q . k) v over every page token
 *    (dequantized) and every window token (exact), no mask; query head hq
 *    reads KV head hq / (Hq / Hkv); output fp32.
 *
 * Page layout (k boosted channels, dtype of 2 bytes; every segment 16-byte
 * aligned, little-endian 2-bit fields):
 *   K_lo    [128 tok][128 ch] 2-bit, element (t, c) at bit 2 (128 t + c)
 *   K_hi    [128 tok][k] 2-bit, (t, j) at bit 2 (k t + j)
 *   K_scale [4][128] dtype, K_zero [4][128] dtype      (group-major)
 *   K_idx   k bytes (ascending), padded to 16
 *   V_codes 4096 B: token t, channel c at bit 8 byte + 16 half + 2 (c / 16),
 *           byte = 1024 (t / 32) + 16 (16 G + c % 16) + 4 w, with
 *           u = t % 32, r = u % 16, G = r / 4, w = 2 (u / 16) + (r % 4) / 2,
 *           half = r % 2
 *   V_scale [4][128] dtype, V_zero [4][128] dtype      (group-major)
 * = 12816 bytes at k = 16, 13344 at k = 32.
 * Cache memory: page (b, h, p) at ((b Hkv + h) max_pages + p) page_bytes,
 * then per (b, h) a window K_res[128][128] followed by V_res[128][128].
 *
 * Ownership: the caller owns every device buffer (cache memory, inputs,
 * outputs, workspace); the library owns only the host handle, never
 * allocates or frees device memory and never synchronizes.  Every launch is
 * asynchronous on the given stream; inputs must stay valid until the stream
 * passes the call.  A handle is not thread-safe.
 *
 * Errors: 0 on success, a negative KVQ_E* code otherwise.  Every argument
 * check happens before any launch, so a failed call changes no state.
 * Preconditions the library does not check: inputs are finite, and a group's
 * range (max - min) is finite in fp32.
 *
 * Debugging switches (environment, read once per process): KVQ_CHECK=1 makes
 * every decode call walk its launch with the extent check of
 * kvq_check_decode_plan first and refuse it with KVQ_EINVAL, before anything
 * is launched, on a violation (the reason on stderr); KVQ_TRACE=1 prints one
 * line per call on stderr (entry point, shape, counters, split plan).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_OK 0
#define KVQ_EINVAL (-1)     /* bad configuration or argument */
#define KVQ_ECAPACITY (-2)  /* more pages than max_pages */
#define KVQ_ESTATE (-3)     /* call not allowed in the current cache state */
#define KVQ_EEMPTY (-4)     /* attention over an empty cache */
#define KVQ_EWORKSPACE (-5) /* workspace too small */
#define KVQ_EALIGN (-6)     /* a device pointer is not 16-byte aligned */
#define KVQ_EHIP (-7)       /* a kernel launch failed */

typedef enum { KVQ_F16 = 0, KVQ_BF16 = 1 } kvq_dtype;

typedef struct {
    int32_t batch;                /* B >= 1 */
    int32_t num_q_heads;          /* Hq, a multiple of Hkv, Hq / Hkv <= 16 */
    int32_t num_kv_heads;         /* Hkv >= 1 */
    int32_t head_dim;             /* must be 128 */
    int32_t page_tokens;          /* must be 128 */
    int32_t key_group_tokens;     /* must be 32 */
    int32_t value_group_channels; /* must be 32 */
    int32_t residual_tokens;      /* must be 128 (= page_tokens) */
    int32_t boost_channels;       /* k: multiple of 16 in [0, 128] (16 = 12.5 %, 32 = 25 %) */
    int32_t max_pages;            /* page capacity per (sequence, KV head), >= 1 */
    int32_t dtype;                /* kvq_dtype of Q, K, V, window and metadata */
    float softmax_scale;          /* <= 0 selects 1 / sqrt(head_dim) */
} kvq_config;

typedef struct kvq_cache kvq_cache; /* opaque host handle */

/* Device bytes the caller must allocate for a cache with this config
   (pages + window).  Errors: KVQ_EINVAL. */
int kvq_cache_bytes(const kvq_config *cfg, size_t *bytes);

/* Bytes of one packed page for this config (12816 at k = 16). */
int kvq_page_bytes(const kvq_config *cfg, size_t *bytes);

/* Wrap caller-owned device memory (>= kvq_cache_bytes, 16-byte aligned) in a
   new handle with n_pages = n_res = 0.  The memory's prior contents are not
   read.  Errors: KVQ_EINVAL, KVQ_EALIGN. */
int kvq_cache_create(const kvq_config *cfg, void *dev_mem, size_t bytes, kvq_cache **out);

/* Free the host handle (not the device memory). */
int kvq_cache_destroy(kvq_cache *cache);

/* Bulk prefill (Kitty abstract: per-page ranking and boost; KIVI section 3:
   per-channel Keys, per-token Values).  k, v: device [B][Hkv][n_pages*128][128]
   in the cache dtype, contiguous, 16-byte aligned.  Quantizes n_pages new
   pages per (sequence, KV head) after the existing ones.  Requires an empty
   window (n_res == 0; else KVQ_ESTATE) and n_pages + new <= max_pages (else
   KVQ_ECAPACITY).  n_pages == 0 is a no-op. */
int kvq_quantize_page(kvq_cache *cache, const void *k, const void *v, int32_t n_pages,
                      void *stream);

/* Streaming append of one token per (sequence, KV head) (KIVI section 3).
   k, v: device [B][Hkv][128] in the cache dtype.  If the window already holds
   128 tokens it is first quantized into page n_pages (flush-before-insert;
   KVQ_ECAPACITY if no page is free); then the token is written to window slot
   n_res.  *flushed (may be NULL) is set to 1 when a flush happened, else 0. */
int kvq_append_token(kvq_cache *cache, const void *k, const void *v, void *stream,
                     int32_t *flushed);

/* Workspace bytes kvq_decode_attention needs for any state of this cache. */
int kvq_decode_workspace_bytes(const kvq_cache *cache, size_t *bytes);

/* Decode attention of one query token per sequence (MiniKV summary: fused
   2-bit unpack + matmul).  q: device [B][Hq][128] in the cache dtype; out:
   device [B][Hq][128] float32; workspace: device, >= the bytes above (else
   KVQ_EWORKSPACE).  Attends to every page token and window token; KVQ_EEMPTY
   when the cache holds no token.  Split-K over pages, then a merge. */
int kvq_decode_attention(kvq_cache *cache, const void *q, float *out, void *workspace,
                         size_t ws_bytes, void *stream);

/* kvq_decode_attention for callers that cannot allocate device memory (code
   under HIP graph capture, tight serving loops, harnesses that forbid
   allocation): the same kernels and the same output, bit for bit, with the
   split partials in a static device buffer of KVQ_NOALLOC_SCRATCH_BYTES that
   the library holds per GPU until the process ends, instead of a caller's
   workspace.  No allocation of any kind happens in the call.  It needs
   B * Hq * (splits of this call) * 520 bytes (splits = page splits + window
   splits, kvq_get_decode_splits + ceil(n_res / 128)); a call that would need
   more returns KVQ_EWORKSPACE before any launch.  Every no-allocation call on
   one GPU shares that buffer: calls that overlap on one GPU (several streams
   or threads) race and must be ordered by the caller.  Errors: KVQ_EINVAL,
   KVQ_EALIGN, KVQ_EEMPTY, KVQ_EWORKSPACE, KVQ_EHIP. */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int kvq_decode_attention_noalloc(kvq_cache *cache, const void *q, float *out, void *stream);

/* One decode step in fewer launches (NEXT-2 of the design: fused append and
   decode): exactly kvq_append_token(k, v, &flushed) followed by
   kvq_decode_attention(q, out, ...), with the same arguments, results (cache
   bytes and output, bit for bit) and error codes, checked before any launch.
   The new token is read from k, v and stored into its window slot by the
   attention kernel itself, so no separate append kernel runs; a full window
   is still flushed into a page first (one extra launch, as in the append). */
int kvq_append_decode(kvq_cache *cache, const void *k, const void *v, const void *q, float *out,
                      void *workspace, size_t ws_bytes, void *stream, int32_t *flushed);

/* Graph-replayable decode step (same launches, same arguments, every step).
   dev_state: device int32[KVQ_DEVICE_STATE_WORDS] = {pages, window tokens,
   unused (0), error flag, and four words the step's own launches use},
   16-byte aligned, owned by the caller.
   kvq_device_state_init writes the handle's host counters into dev_state (a
   kernel launch, so it may itself be captured); when the window is full and
   a page is free it first flushes the window into that page, the flush the
   next step would start with (the host counters follow).
   kvq_append_decode_device is kvq_append_decode with the counters read from
   and advanced in dev_state by the kernels themselves, in two launches: the
   split attention (which stores the new token into its window slot) and the
   split merge, which also flushes a window the step has just filled into the
   next page (the flush that kvq_append_decode makes at the start of the
   following step; the results are the same) and stores the new counters.
   Its page split count is fixed at the call (kvq_set_decode_splits, else one
   round of resident waves for the host counters at that moment), so the
   launches it records into a HIP graph stay valid for any later state.  The
   host counters of the handle are NOT advanced: read dev_state back and call
   kvq_set_state before using the other entry points again.  When the window
   is full and no page is free the kernels leave the cache unchanged, the
   step skips the new token (attending the cache as it is), and dev_state[3]
   becomes 1.  Results equal kvq_append_decode's up to the rounding of a
   different split count.
   Errors: KVQ_EINVAL, KVQ_EALIGN, KVQ_EWORKSPACE (argument checks only);
   KVQ_EHIP from the initial flush. */
#define KVQ_DEVICE_STATE_WORDS 8
int kvq_device_state_init(kvq_cache *cache, int32_t *dev_state, void *stream);
int kvq_append_decode_device(kvq_cache *cache, const void *k, const void *v, const void *q,
                             float *out, void *workspace, size_t ws_bytes, int32_t *dev_state,
                             void *stream);

/* Number of page splits per (sequence, KV head) decode attention uses.  A
   split is one workgroup of four waves; each wave covers a run of
   ceil(4 n_pages / (4 splits)) consecutive 32-token page groups and the
   workgroup merges the four partial results, so the split count in effect is
   ceil(4 n_pages / (4 run)).  splits = 0 restores the automatic choice (one
   round of resident waves); otherwise it is clamped to
   [1, min(ceil(4 n_pages / 4), 256)] at each call.  Results do not depend on
   it beyond rounding. */
int kvq_set_decode_splits(kvq_cache *cache, int32_t splits);

/* Host-side extent check of the decode launches a call would make now; no
   GPU work and nothing is launched.  It walks every workgroup and wave of the
   grid of kvq_decode_attention (mode 0), of kvq_append_decode (mode 1: a
   full window flushed first, then one more window token) or of
   kvq_append_decode_device as captured now and replayed until the cache is
   full (mode 2), with the kernels' own index arithmetic, and checks that
   every page, window token and split partial they address lies inside the
   cache and inside a workspace of ws_bytes, that every 32-token Key group and
   every window token of every (sequence, KV head) is read by exactly one
   wave, and that the split count fits the combine kernel.  (The kernels load
   pages through buffer descriptors, whose out-of-range reads return zeros
   rather than faulting: this is where an offset mistake would show.)
   slots > 0: the resident waves the split plan assumes (0: the device's,
   from the occupancy API).  Returns KVQ_OK, or KVQ_EINVAL with the first
   violation described in msg (msg_len bytes, may be NULL). */
int kvq_check_decode_plan(const kvq_cache *cache, int32_t mode, int32_t slots, size_t ws_bytes,
                          char *msg, size_t msg_len);

/* The page split count the next kvq_decode_attention call will use. */
int kvq_get_decode_splits(const kvq_cache *cache, int32_t *splits);

/* Host-side counters: pages per sequence and window tokens. */
int kvq_get_state(const kvq_cache *cache, int32_t *n_pages, int32_t *n_res);

/* Restore counters after the device bytes were restored (snapshot/restore).
   Errors: KVQ_EINVAL for out-of-range values. */
int kvq_set_state(kvq_cache *cache, int32_t n_pages, int32_t n_res);

/* Byte offset of page (b, h, page) and of the window of (b, h) inside the
   cache memory (for inspection and snapshots). */
int kvq_page_offset(const kvq_cache *cache, int32_t b, int32_t h, int32_t page, size_t *off);
int kvq_residual_offset(const kvq_cache *cache, int32_t b, int32_t h, size_t *k_off,
                        size_t *v_off);

/* Quantize arbitrary groups with the device quantizer (inspection and
   exhaustive checks).  x: device [n_groups][group_len] dtype; s, z: device
   [n_groups] dtype bits (uint16); codes: device [n_groups][group_len] uint8.
   L in {3, 15}; 1 <= group_len <= 256. */
int kvq_quantize_groups(int32_t dtype, int32_t L, const void *x, int32_t n_groups,
                        int32_t group_len, void *s, void *z, void *codes, void *stream);

/* Query-aware Key channel ranking (MixKVQ abstract, fugumt, arXiv
   2512.19206: a Key channel's need for precision follows its quantization
   difficulty and its relevance to the query).  rel: device [batch][Hkv][128]
   float32 (16-byte aligned, finite, >= 0), read by every later page
   quantization of this cache when its kernel runs (bulk pages and window
   flushes; the caller may rewrite it between calls, stream-ordered).  Page
   channel score = |(sum over the page's four Key groups of (max - min) of
   the channel) * rel[c]| in fp32 (group ranges added pairwise: (g0 + g1) +
   (g2 + g3)), the k largest boosted, ties to the lower channel.  rel = NULL
   restores the magnitude ranking.  The page layout and the decode path are
   unchanged.  Errors: KVQ_EINVAL, KVQ_EALIGN. */
int kvq_set_channel_relevance(kvq_cache *cache, const float *rel);

/* Relevance of one query batch: rel[b][h][c] = sum over the g = Hq / Hkv query
   heads h g + j (j ascending) of |q[b][h g + j][c]|, in fp32.  q: device
   [batch][Hq][128] dtype; rel: device [batch][Hkv][128] float32.  Errors:
   KVQ_EINVAL, KVQ_EALIGN. */
int kvq_query_relevance(int32_t dtype, int32_t batch, int32_t num_q_heads,
                        int32_t num_kv_heads, const void *q, float *rel, void *stream);

/* Optional timing hooks: when set (non-NULL hipEvent_t values), decode
   attention records `before` on its stream just before its split kernel and
   `after` just after it.  NULL, NULL clears them. */
int kvq_set_kernel_events(kvq_cache *cache, void *before, void *after);

/* Static description of an error code. */
const char *kvq_strerror(int code);

/* Bandwidth probe, the measured reference for the decode kernels' HBM rates:
   mode 0 reads `bytes` of src once with 16-byte loads (dst: a device word
   that is almost never written), mode 1 copies src to dst (both `bytes`
   long).  bytes must be a positive multiple of 16; 16-byte aligned device
   pointers; asynchronous on the stream.  Errors: KVQ_EINVAL, KVQ_EALIGN,
   KVQ_EHIP. */
int kvq_probe_bandwidth(int32_t mode, const void *src, void *dst, size_t bytes, void *stream);

/* ------------------------------------------------------------------------
 * Block pool: variable-length batches (a page pool with a block table, as
 * in paged attention; Kitty abstract: page-centric layout).
 *
 * cfg->batch is the number of sequence slots (at most 256) and
 * cfg->max_pages the pages one sequence may hold (at most 65535); n_blocks
 * is the pool capacity.  A block holds the Hkv pages of one 128-token span
 * of one sequence, in the page layout above.  Device memory (caller-owned,
 * one region):
 *   blocks   [n_blocks][Hkv][page_bytes]                 at offset 0
 *   windows  [batch][Hkv][K_res | V_res][128][128] dtype at kvq_pool_window_offset
 *   table    [batch][max_pages] int32 block ids           at kvq_pool_table_offset
 * The library keeps per sequence a live flag, its page count, its window
 * count and its block list, and hands out blocks from a free list (host
 * state; the table on the device is written by the library's kernels).
 * Every call checks everything (arguments, capacity, free blocks) before
 * its first launch; on error no state changes.
 * ------------------------------------------------------------------------ */
typedef struct kvq_pool kvq_pool; /* opaque host handle */

/* Device bytes of a pool with n_blocks blocks (n_blocks >= 1). */
int kvq_pool_bytes(const kvq_config *cfg, int32_t n_blocks, size_t *bytes);

/* Create a handle over dev_mem (16-byte aligned, >= kvq_pool_bytes).  Every
   slot starts free (not live) and every block unused.  Errors: KVQ_EINVAL
   (configuration, batch > 256, max_pages > 65535), KVQ_EALIGN. */
int kvq_pool_create(const kvq_config *cfg, int32_t n_blocks, void *dev_mem, size_t bytes,
                    kvq_pool **out);
int kvq_pool_destroy(kvq_pool *pool); /* frees the host handle only */

/* Start sequence `seq` (a free slot) with n_tokens >= 0 prompt tokens.
   k, v: device [Hkv][n_tokens][128] dtype, contiguous.  The first
   128 * floor(n_tokens / 128) tokens become quantized pages in newly taken
   blocks (kernel quantization, Kitty abstract + KIVI section 3), the rest
   (< 128) the window.  The slot becomes live.
   Errors: KVQ_EINVAL (seq out of range, n_tokens < 0, null k/v with
   n_tokens > 0), KVQ_ESTATE (slot live), KVQ_ECAPACITY (more than
   max_pages pages or not enough free blocks), KVQ_EALIGN. */
int kvq_pool_prefill(kvq_pool *pool, int32_t seq, const void *k, const void *v, int32_t n_tokens,
                     void *stream);

/* Append one token to every live sequence.  k, v: device [batch][Hkv][128]
   dtype (rows of slots that are not live are not read).  A sequence whose
   window is full first has it quantized into a new block (flush before
   insert, as for the dense cache); *n_flushed (optional) receives the number
   of such sequences.  Errors: KVQ_EINVAL, KVQ_EALIGN, KVQ_ECAPACITY (a flush
   needs a page beyond max_pages or more blocks than are free). */
int kvq_pool_append(kvq_pool *pool, const void *k, const void *v, void *stream,
                    int32_t *n_flushed);

/* Workspace bytes of kvq_pool_decode_attention (split partials; fixed per
   pool). */
int kvq_pool_decode_workspace_bytes(const kvq_pool *pool, size_t *bytes);

/* Decode attention of every live sequence over its own pages and window.
   q: device [batch][Hq][128] dtype; out: device [batch][Hq][128] float32.
   Rows of slots that are not live, or live without a token, are set to 0.
   Errors: KVQ_EINVAL, KVQ_EALIGN, KVQ_EWORKSPACE. */
int kvq_pool_decode_attention(kvq_pool *pool, const void *q, float *out, void *workspace,
                              size_t ws_bytes, void *stream);

/* kvq_pool_append followed by kvq_pool_decode_attention in fewer launches:
   the new tokens are read from k, v and written to their window slots by the
   attention kernel itself.  Same results and errors as the two calls. */
int kvq_pool_append_decode(kvq_pool *pool, const void *k, const void *v, const void *q,
                           float *out, void *workspace, size_t ws_bytes, void *stream,
                           int32_t *n_flushed);

/* End sequence `seq`: its blocks return to the free list, the slot becomes
   free.  Errors: KVQ_EINVAL (seq out of range), KVQ_ESTATE (slot not live). */
int kvq_pool_release(kvq_pool *pool, int32_t seq);

/* Host state of slot seq: live flag, pages, window tokens. */
int kvq_pool_get_seq(const kvq_pool *pool, int32_t seq, int32_t *live, int32_t *n_pages,
                     int32_t *n_res);
/* Block holding page `page` of live sequence seq (page < n_pages). */
int kvq_pool_block_of(const kvq_pool *pool, int32_t seq, int32_t page, int32_t *block);
/* Blocks not held by any sequence. */
int kvq_pool_free_blocks(const kvq_pool *pool, int32_t *n_free);
/* Byte offsets inside the pool memory: page of KV head h in block `block`;
   window of (seq, h); the block table. */
int kvq_pool_page_offset(const kvq_pool *pool, int32_t block, int32_t h, size_t *off);
int kvq_pool_window_offset(const kvq_pool *pool, int32_t seq, int32_t h, size_t *k_off,
                           size_t *v_off);
int kvq_pool_table_offset(const kvq_pool *pool, size_t *off);

/* Query-aware ranking for the pool's later pages (prefill and flushes), as
   kvq_set_channel_relevance; rel: device [batch][Hkv][128] float32. */
int kvq_pool_set_channel_relevance(kvq_pool *pool, const float *rel);

/* Timing hooks of the pool's split kernel (as kvq_set_kernel_events). */
int kvq_pool_set_kernel_events(kvq_pool *pool, void *before, void *after);

/* The extent check of kvq_check_decode_plan for the pool's decode launch:
   mode 0 = kvq_pool_decode_attention, mode 1 = kvq_pool_append_decode (full
   windows flushed into the next free blocks first, then one more token per
   live sequence); pages are reached through each sequence's block list. */
int kvq_pool_check_decode_plan(const kvq_pool *pool, int32_t mode, int32_t slots,
                               size_t ws_bytes, char *msg, size_t msg_len);

/* ---- Prefill with cumulative attention scores and token selection ----
   MiniKV summary (f-binder), "proposed method": the prefill processes the
   whole input and keeps the heavy hitters by cumulative attention score plus
   a recent window (25 % of the budget each by default); a two-stage selective
   flash-attention gives the attention output and the cumulative scores in
   linear memory.  One sequence per call:
     q: device [Hq][T][128] dtype; k, v: device [Hkv][T][128] dtype (query
     head hq reads KV head hq / (Hq / Hkv)); softmax_scale <= 0 means
     1/sqrt(128).
     out: device [Hq][T][128] float32, causal attention (row i attends to
     positions j <= i).
     score: device [Hkv][T] float32: score[h][j] = sum over the query heads
     of KV head h and the rows i >= j of the softmax probability P[i][j].
     keep: device [Hkv][n_keep] int32: the last min(recent, T) positions plus
     the min(heavy, T - that) positions of largest score among the others
     (ties to the lower position), ascending; n_keep is returned at once.
     k_sel, v_sel: device [Hkv][n_keep][128] dtype, the kept rows of k and v
     (both NULL: no gather), ready for kvq_quantize_page / kvq_append_token.
     workspace: device, kvq_prefill_workspace_bytes; the caller owns every
     buffer, launches are asynchronous on the stream.
   Preconditions: finite inputs.  Errors: KVQ_EINVAL (shape: 1 <= T <= 2^20,
   Hq a multiple of Hkv with at most 16 query heads per KV head), KVQ_EALIGN
   (16-byte alignment), KVQ_EWORKSPACE, KVQ_EHIP. */
int kvq_prefill_workspace_bytes(int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                                size_t *bytes);
int kvq_prefill_select(int32_t dtype, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                       float softmax_scale, const void *q, const void *k, const void *v,
                       int32_t heavy, int32_t recent, float *out, float *score, int32_t *keep,
                       void *k_sel, void *v_sel, void *workspace, size_t ws_bytes, void *stream,
                       int32_t *n_keep);

/* Optional timing hooks of kvq_prefill_select: when set (non-NULL hipEvent_t
   values), every later call records `before` on its stream just before the
   attention kernel and `after` just after it.  NULL, NULL clears them.  The
   setting is process-wide: not for calls made concurrently from several
   threads. */
int kvq_prefill_set_kernel_events(void *before, void *after);

/* Upper bound on the key chunks of kvq_prefill_select (n = 1..4; 0 restores
   the automatic choice, which splits the keys of a short sequence into up to
   four chunks so that the attention kernel fills the chip, and merges them).
   Results agree with the automatic choice up to fp32 summation order; the
   workspace size does not change.  Process-wide, like the timing hooks.
   Errors: KVQ_EINVAL (n outside 0..4). */
int kvq_prefill_set_max_key_splits(int32_t n);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
