/*
 * dattn -- single-token decode attention over a KV cache, for AMD MI355X (gfx950).
 *
 * C ABI.  Every entry point takes plain pointers and sizes; device pointers
 * are HIP device addresses, `stream` is a hipStream_t passed as void*
 * (NULL = the null stream).  The library:
 *   - never allocates or frees device memory and keeps no pointer past return:
 *     the caller owns every buffer, including the workspace;
 *   - validates the host-side arguments before launching anything; a failure
 *     returns a negative dattn_status and dattn_last_error() explains it
 *     (thread-local message); nothing is printed and nothing is launched;
 *   - launches its kernels asynchronously on `stream` and never synchronises;
 *     outputs are valid once the stream reaches that point;
 *   - fully overwrites every output (never accumulates into it);
 *   - moves data in 16-byte vectors: q, caches, outputs and summaries must
 *     be 16-byte aligned (DATTN_EINVAL otherwise; allocator pointers are).
 * Contents of device-resident index arrays (seq_lens, page_table, topk_idx)
 * are a caller contract: they are not read on the host, so calls can be
 * captured into graphs.
 *
 * Layouts (all row-major, no strides):
 *   KV page:     [num_pages, n_kv_heads, page_size, head_dim]  (K and V alike)
 *   page table:  int32 [B, max_pages], logical page j of sequence b at
 *                physical page page_table[b*max_pages + j]; token t lives in
 *                slot t % page_size of logical page t / page_size.
 *   contiguous:  page_table == NULL means one page per sequence:
 *                [B, n_kv_heads, page_size, head_dim] with page_size = S_max.
 *   latent row:  [c_KV (d_latent) | k_pe (d_rope)], 576 values for DeepSeek-V3.
 *
 * Numerics: scores, softmax and accumulation in fp32; bf16 outputs are rounded
 * to nearest even; lse is the natural-log log-sum-exp of the scaled scores.
 * An empty token set yields a zero output row and lse = -inf.
 */
#ifndef DATTN_H
#define DATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define DATTN_EXPORT __attribute__((visibility("default")))
#else
#define DATTN_EXPORT
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  DATTN_FP8_E4M3 is the OCP fp8 "e4m3fn" format (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits, no infinities), one byte per
 * value; the lightning indexer's inputs only. */
typedef enum { DATTN_F32 = 0, DATTN_BF16 = 1, DATTN_FP8_E4M3 = 2 } dattn_dtype;

typedef enum {
  DATTN_OK = 0,
  DATTN_EINVAL = -1,        /* malformed argument (null pointer, bad size, bad ratio) */
  DATTN_EUNSUPPORTED = -2,  /* well-formed but not built: head dim, dtype, group size */
  DATTN_EWORKSPACE = -3,    /* workspace missing or smaller than the *_workspace() size */
  DATTN_EHIP = -4           /* a HIP call or kernel launch failed */
} dattn_status;

/* ------------------------------------------------------------------------ */
/* Grouped-query decode attention, with optional sliding window and sinks.
 *
 * Computes, for every sequence b and query head h, softmax(scale * q K^T) V
 * over the token set T_b of the one new query token, where query head h
 * reads KV head h / (Hq / Hkv) -- the head sharing of GQA ("All the
 * attentions", section 2 GQA; "Overview of Attention Mechanism", GQA, 分组机制:
 * one KV head is MQA, Hkv = Hq is MHA).  L_b = seq_lens[b] counts the cached
 * tokens, the current one included.
 *   window <= 0:  T_b = [0, L_b)  (full attention).
 *   window  > 0:  T_b = [0, min(n_sink, L_b)) u [L_b - window, L_b): the last
 *                 `window` tokens ("All the attentions", section 4, Sliding
 *                 Window) plus the first n_sink attention sinks ("Attention
 *                 Optimizations", "Attention sinks"); a union, never counted
 *                 twice; window >= L_b is full attention.
 * Tokens outside T_b are skipped, not masked: they are never loaded.
 * The cache is paged as described above (PagedAttention block table, "All
 * the attentions", section 8); physical pages may be shared between
 * sequences (read-only aliasing is allowed).
 *
 *   q          [B, Hq, D]                   dtype
 *   k_cache    [num_pages, Hkv, page_size, D] dtype
 *   v_cache    same layout as k_cache
 *   seq_lens   int32 [B], 0 <= L_b <= page_size * max_pages
 *   page_table int32 [B, max_pages] or NULL (contiguous, page_size = S_max)
 *   out        [B, Hq, D] dtype (written)
 *   lse        fp32 [B, Hq] or NULL
 *   dtype      DATTN_F32 or DATTN_BF16; D in {64, 128}; Hq / Hkv in {1,2,4,8}
 *   page_size  paged: a power of two >= 1; contiguous: S_max
 *   scale      softmax scale; <= 0 means 1/sqrt(D)
 *   num_splits token-range splits per (sequence, KV head); 0 = automatic.
 *              Partial results are merged by log-sum-exp in a second kernel.
 *   workspace  device memory of at least decode_attn_gqa_workspace(...) bytes,
 *              256-byte aligned (may be NULL when that size is 0).  It holds
 *              the split partials and needs no initialisation; calls that
 *              share a workspace must be ordered on one stream.
 */
DATTN_EXPORT int decode_attn_gqa(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seq_lens, const int32_t* page_table,
                    int32_t window, int32_t n_sink,
                    void* out, float* lse,
                    int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                    int32_t page_size, int32_t max_pages, int32_t dtype, float scale,
                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                    void* stream);

/* decode_attn_gqa with an explicit sink logit per query head.
 *
 * Some models carry a learned sink logit instead of (or besides) keeping the
 * first tokens ("Attention Optimizations", "Attention sinks": gpt-oss's
 * explicit sink); softmax-off-by-one adds a zero sink, a token whose key and
 * value are zero vectors ("Overview of Attention Mechanism", StreamingLLM /
 * attention sink).  Both are one more term in the softmax denominator with
 * a zero value:
 *   o = sum_t e^{s_t} v_t / (e^{sink[h]} + sum_t e^{s_t})
 * and lse = log(e^{sink[h]} + sum_t e^{s_t}) (so an empty T_b gives o = 0,
 * lse = sink[h]).
 *   sink_logits  device fp32 [Hq], natural-log units, read-only; NULL gives
 *                exactly decode_attn_gqa.  A zero sink is all zeros.
 * Every other argument, the workspace and the error behaviour are those of
 * decode_attn_gqa (same workspace size).
 */
DATTN_EXPORT int decode_attn_gqa_sink(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seq_lens, const int32_t* page_table,
                    int32_t window, int32_t n_sink, const float* sink_logits,
                    void* out, float* lse,
                    int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                    int32_t page_size, int32_t max_pages, int32_t dtype, float scale,
                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Workspace bytes decode_attn_gqa needs for these sizes (0 if none); pass
 * max_pages = 1 for a contiguous cache. */
DATTN_EXPORT size_t decode_attn_gqa_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t page_size, int32_t max_pages, int32_t window,
                                 int32_t n_sink, int32_t num_splits);

/* decode_attn_gqa_sink for callers that cannot allocate device memory: code
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace: the split partials go to a file-scope device array
 * of the library, 16 MiB per GPU (each GPU the library runs on holds its own
 * copy until the process ends; its address is looked up once per device with
 * hipGetSymbolAddress).  The call allocates nothing.  The caller still passes
 * every input and output, with the meanings, layouts and errors of
 * decode_attn_gqa_sink (sink_logits may be NULL).
 *   num_splits  0 = automatic, lowered when needed until the partials,
 *               B * Hq * splits * (D + 1) fp32 values (each of the two parts
 *               rounded up to 256 bytes), fit the 16 MiB; a requested count
 *               whose partials do not fit returns DATTN_EWORKSPACE.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or different threads without ordering) race and
 * give wrong results.  Calls ordered on one stream are safe; the array keeps
 * the last call's partials, and no call needs it cleared.
 */
DATTN_EXPORT int decode_attn_gqa_noalloc(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seq_lens, const int32_t* page_table,
                    int32_t window, int32_t n_sink, const float* sink_logits,
                    void* out, float* lse,
                    int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                    int32_t page_size, int32_t max_pages, int32_t dtype, float scale,
                    int32_t num_splits, void* stream);

/* ------------------------------------------------------------------------ */
/* Cache append: the new token's entries, written before attending.
 *
 * Decoding writes the current token into the cache and then attends over it
 * ("Attention Optimizations", "DSA: DeepSeek Sparse Attention", "Computation
 * Path": update_cache of the latent row and of the indexer key).  Entry
 * position p of sequence b goes to slot p % page_size of physical page
 * page_table[b][p / page_size] (PagedAttention block table, "All the
 * attentions", section 8), or to [b, p] of a contiguous cache.
 *
 * kv_append_gqa: one K row and one V row per KV head.
 *   k_new, v_new  [B, Hkv, D] dtype, read-only
 *   k_cache, v_cache  [num_pages, Hkv, page_size, D] (the decode_attn_gqa layout),
 *                 written at the appended slots only
 *   positions     device int32 [B]: the position written (the current token
 *                 is position L_b - 1 once seq_lens counts it); a negative
 *                 entry skips the sequence, and so does a position past the
 *                 cache (p >= page_size * max_pages, or >= S_max contiguous)
 *   page_table    device int32 [B, max_pages], or NULL (contiguous,
 *                 page_size = S_max).  Pages the append writes must not be
 *                 shared with another sequence (copy them first).
 *   ring_pages, fixed_pages  rolling buffer for a sliding window ("All the
 *                 attentions", section 4: the cache becomes a rolling buffer
 *                 of fixed size, new entries replacing the oldest).  With
 *                 ring_pages > 0 a write into logical page j >= fixed_pages +
 *                 ring_pages first sets page_table[b][j] = page_table[b][j -
 *                 ring_pages] (so the table is written).  Entries below
 *                 fixed_pages + ring_pages are the caller's: fixed_pages for
 *                 the attention-sink tokens, never recycled, then the ring.
 *                 For window W the ring needs ceil((W - 1) / page_size) + 1
 *                 pages so that a recycled page holds no token any later
 *                 query's window reaches.  0 = no rolling buffer.
 *   D * sizeof(dtype) must be a multiple of 16 bytes; every buffer 16-byte
 *   aligned.  Errors: DATTN_EINVAL / DATTN_EUNSUPPORTED before any launch.
 *
 * kv_append_rows: one row per token (the MLA latent cache [c_KV | k_pe],
 *   576 values, or the indexer key cache, 128 values).
 *   rows_new   [B, row_elems] dtype
 *   cache      [num_pages, page_size, row_elems] or contiguous [B, S_max, row_elems]
 *   the rest as for kv_append_gqa (no rolling buffer).
 */
DATTN_EXPORT int kv_append_gqa(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int32_t* positions, int32_t* page_table, int32_t B, int32_t Hkv,
                  int32_t D, int32_t page_size, int32_t max_pages, int32_t ring_pages,
                  int32_t fixed_pages, int32_t dtype, void* stream);

DATTN_EXPORT int kv_append_rows(const void* rows_new, void* cache, const int32_t* positions,
                  const int32_t* page_table, int32_t B, int32_t row_elems, int32_t page_size,
                  int32_t max_pages, int32_t dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Query-aware page selection (Quest) over a GQA cache.
 *
 * Every query picks, per step, which pages of the cache it reads ("Long
 * context, KV eviction and sparse attention", "Sparse attention: choosing
 * dynamically at every step"; "Attention Optimizations", "Query-aware
 * retrieval").  The cache is cut into blocks of 16 tokens (the pages of that
 * passage); block p of (sequence b, KV head g) keeps kmin_p and kmax_p, the
 * per-dimension minimum and maximum of its 16 keys.  Query head h bounds
 * q . k over block p by
 *   upper[h, p] = sum_d max(q_d kmin_p[d], q_d kmax_p[d])
 * and attends to the `budget` full blocks with the largest bounds (ties go to
 * the lower block) plus the last, partial block (L_b % 16 tokens, always
 * kept); a sequence with at most `budget` full blocks attends to all of them.
 * Each query head chooses its own blocks; query head h reads KV head
 * h / (Hq / Hkv).
 *
 * quest_page_minmax: writes the summaries of blocks [first_block, L_b / 16)
 *   of every sequence and KV head; other slots are left as they are.  After
 *   appending token L_b - 1 a caller refreshes only the block it completed
 *   (first_block = that block; summaries are pure functions of the keys, so
 *   recomputing one is harmless).
 *   k_cache    the decode_attn_gqa K layout and page table; paged caches need
 *              a power-of-two page_size >= 16 (a block never straddles pages)
 *   kminmax    [B, Hkv, n_blocks, 2, D] in dtype, n_blocks = page_size *
 *              max_pages / 16 (contiguous: S_max / 16, max_pages = 1):
 *              [.., 0, :] = kmin, [.., 1, :] = kmax (exact; min and max pick
 *              cached values)
 *   first_block >= 0
 *
 * decode_attn_quest: bounds, selection and attention in one call:
 *   q, k_cache, v_cache, seq_lens, page_table, out, lse, dtype, scale,
 *   num_splits   as for decode_attn_gqa (no window, no sinks); Hq / Hkv in
 *                {1,2,4,8}; paged caches need page_size >= 16
 *   kminmax      the summaries quest_page_minmax wrote, read-only
 *   budget       blocks kept per query head, 1 <= budget <= 16384
 *   selected     NULL, or device int32 [B, Hq, budget]: the chosen blocks in
 *                ascending order, -1 padded (written)
 *   B * Hq <= 65535
 *   workspace    at least decode_attn_quest_workspace(...) bytes, 256-byte
 *                aligned; no initialisation needed; calls sharing it must be
 *                ordered on one stream
 * Bounds run in fp32 on MFMAs (products of bf16 values exact, fp32 sums);
 * the choice is the top-k select of dsa_topk over each query head's bounds.
 * For a group of query heads sharing a KV head, each block any of them chose
 * is read once and attended by the heads that chose it (the result is the
 * per-head attention above); tables of more than 8192 blocks per sequence
 * attend per head.
 * Errors: DATTN_EINVAL / DATTN_EUNSUPPORTED / DATTN_EWORKSPACE before any
 * launch, DATTN_EHIP if a launch fails.
 */
DATTN_EXPORT int quest_page_minmax(const void* k_cache, const int32_t* seq_lens,
                  const int32_t* page_table, void* kminmax, int32_t first_block,
                  int32_t B, int32_t Hkv, int32_t D, int32_t page_size, int32_t max_pages,
                  int32_t dtype, void* stream);

DATTN_EXPORT int decode_attn_quest(const void* q, const void* k_cache, const void* v_cache,
                  const void* kminmax, const int32_t* seq_lens, const int32_t* page_table,
                  int32_t budget, void* out, float* lse, int32_t* selected,
                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                  int32_t max_pages, int32_t dtype, float scale, int32_t num_splits,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes decode_attn_quest needs (an upper bound over `selected`
 * given or not); max_pages = 1 for a contiguous cache. */
DATTN_EXPORT size_t decode_attn_quest_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                  int32_t page_size, int32_t max_pages, int32_t budget, int32_t dtype,
                  int32_t num_splits);

/* ------------------------------------------------------------------------ */
/* Absorbed MLA decode attention over a latent cache.
 *
 * For each sequence b and head h: s_t = scale * q_absorbed[b,h] . row_t over
 * all d_latent + d_rope values of the cached row, softmax over t in
 * [0, seq_lens[b]), output = sum_t p_t row_t[0:d_latent].  The query is the
 * absorbed one, [W_UK^T q_nope ; q_pe] ("Overview of Attention Mechanism",
 * MLA, Method: W_UK folds into the query and W_UV into the output
 * projection), and the cached row is cat(c_KV, k_pe) ("Attention
 * Optimizations", "DSA: DeepSeek Sparse Attention", "Computation Path").
 *
 *   q_absorbed   [B, H, d_latent + d_rope] bf16
 *   latent_cache [num_pages, page_size, d_latent + d_rope] bf16, or contiguous
 *                [B, S_max, d_latent + d_rope] when page_table == NULL
 *   seq_lens     int32 [B], 0 <= L_b <= S_max
 *   page_table   int32 [B, max_pages] or NULL
 *   out          [B, H, d_latent] bf16 (written);  lse fp32 [B, H] or NULL
 *   d_latent 512, d_rope 64, H a multiple of 64, dtype DATTN_BF16 only
 *   S_max        contiguous: rows per sequence; paged: page_size * max_pages
 *   page_size    paged: a power of two; ignored when page_table == NULL
 *   scale        <= 0 means 1/sqrt(192) (DeepSeek-V3: 128 + 64 qk dims)
 *   num_splits   0 = automatic; a split holds at most 3840 tokens, so a
 *                smaller count is raised to ceil(S_max / 3840) (at most 256).
 *                Automatic with H a multiple of 128, B <= 512 and a
 *                contiguous cache cuts every sequence into items of about
 *                equal tokens from the actual seq_lens (long sequences take
 *                more, empty ones none), so that ragged batches keep every
 *                CU busy; otherwise (and for paged caches) every sequence
 *                gets the same number of splits.
 *   workspace    decode_attn_mla_workspace bytes (never 0: the splits' partial
 *                results always go through it)
 * The cache must hold fewer than 2^31 rows (B * S_max contiguous, num_pages *
 * page_size paged); page_table entries must name pages of the cache.
 * Errors: DATTN_EINVAL / DATTN_EUNSUPPORTED for arguments outside the above,
 * DATTN_EWORKSPACE for a missing or short workspace, DATTN_EHIP for a launch
 * failure; nothing is written then.
 */
DATTN_EXPORT int decode_attn_mla(const void* q_absorbed, const void* latent_cache,
                    const int32_t* seq_lens, const int32_t* page_table,
                    void* out, float* lse,
                    int32_t B, int32_t H, int32_t d_latent, int32_t d_rope,
                    int32_t S_max, int32_t page_size, int32_t max_pages,
                    int32_t dtype, float scale, int32_t num_splits,
                    void* workspace, size_t workspace_bytes, void* stream);

DATTN_EXPORT size_t decode_attn_mla_workspace(int32_t B, int32_t H, int32_t d_latent, int32_t S_max,
                                 int32_t num_splits);

/* ------------------------------------------------------------------------ */
/* DSA lightning indexer followed by top-k selection.
 *
 * scores[b,t] = sum_h w[b,h] * ReLU(q_i[b,h] . k_i[b,t]) for t < seq_lens[b]
 * ("Attention Optimizations", "DSA: DeepSeek Sparse Attention", "Computation
 * Path": per-head indexer products mixed by a per-head weight; the ReLU and
 * the sum over heads are the reading this library implements), then the k
 * largest scores of each sequence, ties to the lower token index, written in
 * ascending index order; when k > seq_lens[b] the tail is -1.  The caller
 * folds any positive constant (such as n_heads^-0.5) into w.
 *
 *   q_i        [B, Hi, Di] dtype;  w fp32 [B, Hi];  k_i_cache [B, S_max, Di] dtype
 *              (dtype DATTN_BF16, or DATTN_FP8_E4M3: the indexer in FP8 as
 *              the pages give it ("Long context, KV eviction and sparse
 *              attention", "Sparse attention": a lightweight indexer scoring
 *              all past tokens with few heads in FP8), half the key bytes)
 *   seq_lens   int32 [B], 0 <= L_b <= S_max
 *   k          1 <= k <= 16384
 *   topk_idx   int32 [B, k] (written)
 *   scores_out fp32 [B, S_max] or NULL; when given, receives the scores
 *              (entries t >= seq_lens[b] are -inf)
 *   Hi a multiple of 32 (<= 128), Di = 128, dtype DATTN_BF16 or DATTN_FP8_E4M3, B <= 65535,
 *   S_max <= 2^30
 *   workspace  dsa_indexer_topk_workspace(B, S_max, k) bytes, 256-byte
 *              aligned, always required (the selection keeps histograms and
 *              per-chunk counts there; the first B*S_max*4 bytes, rounded up
 *              to 256, hold the scores when scores_out is NULL).  Its contents
 *              need no initialisation and are not meaningful afterwards.
 * Integer-valued inputs with |sum| < 2^24 give exact scores and therefore an
 * exact, reproducible selection.
 */
DATTN_EXPORT int dsa_indexer_topk(const void* q_i, const float* w, const void* k_i_cache,
                     const int32_t* seq_lens, int32_t k, int32_t* topk_idx, float* scores_out,
                     int32_t B, int32_t Hi, int32_t Di, int32_t S_max, int32_t dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

DATTN_EXPORT size_t dsa_indexer_topk_workspace(int32_t B, int32_t S_max, int32_t k);

/* The selection step alone, on caller-provided fp32 scores [B, S_max]:
 * the k largest of scores[b, 0:seq_lens[b]], ties to the lower index,
 * ascending, -1 padded.  -0.0 and +0.0 are equal; NaN scores are not
 * supported (their position in the order is unspecified).  1 <= k <= 16384,
 * B <= 65535, S_max <= 2^30.  The workspace (dsa_topk_workspace bytes,
 * 256-byte aligned, no initialisation needed) holds four 256-bin radix
 * histograms and one count per 2048-token chunk of each row. */
DATTN_EXPORT int dsa_topk(const float* scores, const int32_t* seq_lens, int32_t k, int32_t* topk_idx,
             int32_t B, int32_t S_max, void* workspace, size_t workspace_bytes, void* stream);

DATTN_EXPORT size_t dsa_topk_workspace(int32_t B, int32_t S_max, int32_t k);

/* ------------------------------------------------------------------------ */
/* Sparse MLA: absorbed MLA decode attention over only the selected rows.
 *
 * Same arithmetic as decode_attn_mla, over the token set
 * { topk_idx[b, j] : 0 <= j < k, topk_idx[b, j] >= 0 } (gather of the
 * selected latent rows, "Attention Optimizations", "Computation Path");
 * entries outside [0, S_max) (-1 by convention) are skipped; an index listed
 * twice counts twice.
 *
 *   q            [B, H, d_latent + d_rope] bf16
 *   latent_cache [B, S_max, d_latent + d_rope] bf16, B * S_max < 2^31
 *   topk_idx     int32 [B, k], entries in [0, S_max); any other value
 *                (such as -1) marks an empty slot
 *   out          [B, H, d_latent] bf16;  lse fp32 [B, H] or NULL
 *   num_splits   as for decode_attn_mla, with k in place of S_max
 * A sequence with no selected token gets out = 0 and lse = -inf.
 */
DATTN_EXPORT int sparse_mla_attn(const void* q, const void* latent_cache, const int32_t* topk_idx, int32_t k,
                    void* out, float* lse,
                    int32_t B, int32_t H, int32_t d_latent, int32_t d_rope, int32_t S_max,
                    int32_t dtype, float scale, int32_t num_splits,
                    void* workspace, size_t workspace_bytes, void* stream);

DATTN_EXPORT size_t sparse_mla_attn_workspace(int32_t B, int32_t H, int32_t d_latent, int32_t k,
                                 int32_t num_splits);

/* ------------------------------------------------------------------------ */
/* Diagnostics. */

/* Message describing the last failure on this thread ("" if none). */
DATTN_EXPORT const char* dattn_last_error(void);

/* ABI version of this library. */
DATTN_EXPORT int32_t dattn_version(void);

/* Debug checking of the device-resident tables.
 *
 * The kernel must follow the block table ("All the attentions", section 8,
 * PagedAttention): a page table or a length outside the contract makes it
 * read outside the cache.  The tables stay on the device and are trusted by
 * default.  With DATTN_DEBUG=1 in the environment, or after
 * dattn_debug_enable(1), decode_attn_gqa(_sink), decode_attn_quest,
 * decode_attn_mla and dsa_indexer_topk first copy seq_lens (and page_table)
 * to the host, synchronously on their stream, and check them as
 * dattn_check_tables does (num_pages taken from the size of the cache's
 * device allocation); a violation returns DATTN_EINVAL, names the first bad
 * entry and launches nothing.  The copy synchronises the stream, so this
 * mode does not suit stream capture.
 *
 * dattn_check_tables: the same check on HOST arrays.
 *   seq_lens    host int32 [B]: each 0 <= L_b <= page_size * max_pages
 *               (contiguous: page_table NULL, page_size = S_max)
 *   page_table  host int32 [B, max_pages] or NULL: the entries of the pages
 *               that hold tokens, j < ceil(L_b / page_size), must lie in
 *               [0, num_pages); num_pages < 0 checks only that they are >= 0
 * Returns DATTN_OK or DATTN_EINVAL (message in dattn_last_error). */
DATTN_EXPORT int dattn_debug_enable(int32_t on);
DATTN_EXPORT int dattn_check_tables(const int32_t* seq_lens, const int32_t* page_table, int32_t B,
                                    int32_t page_size, int32_t max_pages, int64_t num_pages);

/* Per-kernel timing.  While enabled, every call's kernels carry HIP events
 * on the launch stream, bound to the dispatches themselves
 * (hipExtLaunchKernel): one record per launch step (a step of several kernels,
 * such as the top-k levels, spans the first kernel's start to the last one's
 * end), so launch overhead between kernels is not counted.  dattn_profile_read
 * waits for the events and reports, for records whose name contains `name`,
 * the summed duration in milliseconds and the record count.
 * dattn_profile_reset drops all records.  Meant for benchmarks, not
 * production. */
DATTN_EXPORT int dattn_profile_enable(int32_t on);
DATTN_EXPORT int dattn_profile_read(const char* name, double* total_ms, int64_t* count);
DATTN_EXPORT int dattn_profile_reset(void);

/* Streaming-read probe: reads `bytes` (a multiple of 16) from the device
 * buffer src (16-byte aligned) with `grid` workgroups of 256 threads, each
 * workgroup one contiguous range, each thread keeping `depth` (4, 8 or 16)
 * 16-byte nontemporal loads in flight; sink (device, `grid` words) is almost
 * never written.  The best rate over launch shapes is the ceiling that the
 * HBM-bound kernels are compared with besides the specification's peak.
 * Diagnostics only. */
DATTN_EXPORT int dattn_stream_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t grid,
                                         int32_t depth, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DATTN_H */
