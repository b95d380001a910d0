/*
 * xq.h — C ABI of the TurboQuant paged KV cache for MI355X (gfx950).
 *
 * What the operations compute comes from the pages on xInfer's TurboQuant KV cache:
 *   - "xInfer: Pure-Rust LLM Inference Without a Python Runtime" (hysenlabs.com),
 *     section "What actually sits between the request and the tokens": each K/V head
 *     vector is rotated by a Walsh-Hadamard transform, then quantized with one absmax
 *     scale per head, so that the rotation spreads outlier channels before the absmax;
 *     the resulting cache is 2 to 4 bits wide (turbo2 is its 2-bit end).
 *   - same page, section "Getting a server up: the commands in the README": the KV cache
 *     type is one of fp8, turbo8, turbo4, turbo3, and BF16 when no type is given.
 *   - same page, section "TurboQuant is a memory trade, and the README does not price it
 *     fully": a low-bit cache is dequantized on every attention step.
 *   - "infero" landing page (jackwangfeng.github.io/infero), section "Beyond plain text
 *     decode", item "Continuous batching": requests share the GPU through a paged KV cache.
 *
 * The pages leave the number format open. This library fixes it as follows:
 *   - rotation: orthonormal fast Walsh-Hadamard transform over head_dim = 128, natural
 *     (Sylvester) order, no random signs; stages h = 1, 2, 4, ..., 64 of (a+b, a-b) in
 *     fp32, then one multiply by C = fp32(1/sqrt(128)) = 0x3DB504F3;
 *   - scale: one fp16 per (token, kv_head), s = fp16_rne(min(absmax / qmax, 65504)),
 *     qmax = 2^(bits-1) - 1 (127, 7, 3, 1), division in fp32;
 *   - codes: c = clamp(rint_half_even(x / s), -qmax, qmax) in fp32; all zero when s == 0;
 *   - packing: code d of a row occupies bits [bits*d, bits*d + bits) of the row's
 *     little-endian bitstream, as a bits-wide two's complement field.
 *   - fp8 (the page's compression table gives it 2x against BF16, so nothing is stored beside
 *     the elements): each bf16 element becomes the nearest finite OCP FP8 E4M3 value (sign,
 *     4 exponent bits with bias 7, 3 mantissa bits), ties to the even code, magnitudes past
 *     448 saturating to 448, the sign kept on zero; no rotation, no scale.
 *
 * Memory layout (both pools, K and V, have the same layout):
 *   pool + page * page_stride + kv_head * block_bytes   is one (page, kv_head) block;
 *   a turbo block is page_size code rows of 16*bits bytes (slot s at s * 16 * bits),
 *   followed by page_size fp16 scales (slot s at page_size * 16 * bits + 2 * s);
 *   a bf16 block is page_size rows of 128 bf16 values (256 bytes per row);
 *   an fp8 block is page_size rows of 128 E4M3 bytes.
 *   block_bytes is a multiple of 16. Physical page ids come from a per-sequence block
 *   table: token position p of sequence b lives in page block_tables[b][p / page_size],
 *   slot p % page_size.
 *
 * Ownership: the caller owns every buffer (device memory unless noted). The library
 * allocates and frees nothing and keeps no state beyond a thread-local error string.
 * Every operation is enqueued on the caller's HIP stream (NULL = the default stream)
 * and the call returns after the launch; the caller orders appends before the decode
 * that reads them and keeps buffers alive until the stream has run them.
 *
 * Errors: functions return an xq_status. Only host-visible arguments are validated
 * (dtype, head_dim, page_size, head counts, null pointers, 16-byte alignment of pools,
 * workspace size); a failed check launches nothing. A failed launch returns XQ_EHIP.
 * The contents of device arrays are the caller's contract: page ids < num_pages,
 * context_lens[b] <= max_pages_per_seq * page_size and <= max_context_len, and no two
 * tokens of one append writing the same slot. With the environment variable XQ_DEBUG set
 * (to anything but "0") both calls also check those contents before launching: they copy
 * the index arrays (context_lens and the block table rows a decode reads; token_seq,
 * token_pos and block-table rows 0 .. max(token_seq) of an append) to host memory on the
 * caller's stream, wait for it, and return XQ_EINVAL with xq_last_error naming the first
 * bad entry. That mode is synchronous and allocates host memory; it is for debugging.
 * Nothing throws across this boundary.
 */
#ifndef XQ_H
#define XQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* KV cache element type. The value is the code width in bits (0 for bf16). */
typedef enum {
  XQ_KV_BF16 = 0,   /* unquantized: the cache type used when none is given */
  XQ_KV_TURBO8 = 8, /* 8-bit codes, 130 bytes per row (128 codes + fp16 scale) */
  XQ_KV_TURBO4 = 4, /* 4-bit codes, 66 bytes per row */
  XQ_KV_TURBO3 = 3, /* 3-bit codes in a dense bitstream, 50 bytes per row */
  XQ_KV_TURBO2 = 2, /* 2-bit codes (-1, 0, 1), 34 bytes per row */
  XQ_KV_FP8 = 16    /* OCP FP8 E4M3 elements, 128 bytes per row, no rotation and no scale
                       (the value is not a code width) */
} xq_kv_dtype;

typedef enum {
  XQ_OK = 0,
  XQ_EINVAL = 1,        /* an argument is out of range or a pointer is null/misaligned */
  XQ_EUNSUPPORTED = 2,  /* a valid combination this build does not implement */
  XQ_EWORKSPACE = 3,    /* workspace too small or null */
  XQ_EHIP = 4           /* the HIP runtime reported an error */
} xq_status;

/* Geometry of one KV pool (K and V pools share it). */
typedef struct {
  int32_t kv_dtype;     /* an xq_kv_dtype */
  int32_t head_dim;     /* must be 128 */
  int32_t num_kv_heads; /* >= 1 */
  int32_t page_size;    /* tokens per page: a power of two in [16, 256] */
  int64_t num_pages;    /* physical pages in the pool, >= 1 */
} xq_cache_layout;

/* Bytes of one (page, kv_head) block; -1 if the layout is invalid. */
int64_t xq_block_bytes(const xq_cache_layout* layout);
/* Bytes between consecutive pages: num_kv_heads * xq_block_bytes; -1 if invalid. */
int64_t xq_page_stride_bytes(const xq_cache_layout* layout);
/* Bytes of one pool (K or V): num_pages * xq_page_stride_bytes; -1 if invalid. */
int64_t xq_pool_bytes(const xq_cache_layout* layout);

/*
 * Number of sequence partitions ("splits") the decode uses for a sequence of up to
 * max_context_len tokens. num_splits_hint = 0 lets the library choose from the batch
 * shape; a positive hint asks for that many partitions. Partitions are whole pages and
 * whole 32-token tiles, and span at most 128 pages, so the count returned can be smaller
 * (short contexts) or larger (long contexts) than the hint. A negative hint fixes every
 * partition at -num_splits_hint tokens, which must be a multiple of 32 and of page_size and
 * at most 128 pages: the batch-invariant mode, in which a sequence's decode output is
 * bitwise the same whatever else is in the batch and whatever max_context_len is (the
 * xInfer page's decode step is replayed as a captured graph, section "What actually sits
 * between the request and the tokens", which wants shapes that do not change the results).
 * Returns -1 on invalid arguments.
 */
int32_t xq_decode_num_splits(const xq_cache_layout* layout, int32_t batch,
                             int32_t num_q_heads, int32_t max_context_len,
                             int32_t num_splits_hint);

/*
 * Workspace bytes xq_paged_decode_attention needs for these arguments: the partition
 * partials, 0 when every sequence fits one partition. Returns -1 on invalid arguments.
 */
int64_t xq_decode_workspace_bytes(const xq_cache_layout* layout, int32_t batch,
                                  int32_t num_q_heads, int32_t max_context_len,
                                  int32_t num_splits_hint);

/* Static description of a status code. */
const char* xq_status_string(int32_t status);
/* Message of the last failed call on this host thread ("" if none). */
const char* xq_last_error(void);

/*
 * Rotate, quantize and pack new K and V rows, and store them in their pages.
 * Defined by the xInfer page, section "What actually sits between the request and the
 * tokens" (rotation, then per-head absmax quantization), with the number format fixed above.
 *
 *   k_new, v_new       bf16 [n_tokens][num_kv_heads][128], row-major, 16-byte aligned
 *   n_tokens           rows per head to append (0 is a no-op)
 *   token_seq          int32 [n_tokens]: sequence index of each token
 *   token_pos          int32 [n_tokens]: position of the token in its sequence
 *   block_tables       int32 [num_seqs][max_pages_per_seq]: physical page per logical page
 *   k_pool, v_pool     pools of xq_pool_bytes(layout) bytes, 16-byte aligned
 *   stream             hipStream_t (NULL = default stream)
 * Each (token, kv_head) row of K and of V becomes one code row and one fp16 scale at
 * page block_tables[token_seq[i]][token_pos[i] / page_size], slot token_pos[i] % page_size.
 * In bf16 mode the row is copied unchanged; in fp8 mode it becomes 128 E4M3 bytes (no scale).
 * Bytes of other slots are not touched.
 */
xq_status xq_quantize_append(const xq_cache_layout* layout,
                             const void* k_new, const void* v_new, int32_t n_tokens,
                             const int32_t* token_seq, const int32_t* token_pos,
                             const int32_t* block_tables, int32_t max_pages_per_seq,
                             void* k_pool, void* v_pool, void* stream);

/*
 * Single-token decode attention over the paged (and, for turbo types, quantized) cache.
 * Defined by the xInfer page, section "TurboQuant is a memory trade, and the README does
 * not price it fully" (every attention step reads and dequantizes the cache), and the
 * infero page, section "Beyond plain text decode", item "Continuous batching" (paged KV).
 *
 * For sequence b and query head j (kv head j / (num_q_heads / num_kv_heads)):
 *   turbo types:  q' = H q;  k'_t = s_k[t] c_k[t];  v'_t = s_v[t] c_v[t]   (rotated space)
 *                 z_t = softmax_scale * (q' . k'_t);  o = sum_t softmax(z)_t v'_t;  out = H o
 *   bf16, fp8:    the same without H, over the stored bf16 or E4M3 values.
 * H is the orthonormal Walsh-Hadamard matrix (symmetric, its own inverse), t runs over
 * positions 0 .. context_lens[b]-1 with no mask, and context_lens[b] = 0 gives zeros.
 *
 *   q                  bf16 [batch][num_q_heads][128], 16-byte aligned
 *   k_pool, v_pool     pools written by xq_quantize_append
 *   block_tables       int32 [batch][max_pages_per_seq]
 *   context_lens       int32 [batch] (device)
 *   max_context_len    host upper bound of context_lens (sizes the launch)
 *   softmax_scale      multiplies q . k (e.g. 1/sqrt(128))
 *   num_splits_hint    0 = library policy, > 0 a split count, < 0 fixed partitions of
 *                      -num_splits_hint tokens (batch invariant); as for xq_decode_num_splits
 *   workspace          device scratch of >= xq_decode_workspace_bytes(...) bytes, 16-byte
 *                      aligned; may be NULL when that size is 0. Its contents on entry do
 *                      not matter; calls that share a workspace must not overlap.
 *   out                fp32 [batch][num_q_heads][128], 16-byte aligned
 * num_q_heads must be a multiple of num_kv_heads (XQ_EINVAL otherwise); a group size above 16,
 * a batch above 65535, more than 65535 splits or 2^26 or more (split, kv head, sequence) units
 * give XQ_EUNSUPPORTED. Block-table entries read for positions below context_lens[b] must be
 * pages of the pool (not checked on the device).
 */
xq_status xq_paged_decode_attention(const xq_cache_layout* layout,
                                    const void* q, int32_t batch, int32_t num_q_heads,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, int32_t max_pages_per_seq,
                                    const int32_t* context_lens, int32_t max_context_len,
                                    float softmax_scale, int32_t num_splits_hint,
                                    void* workspace, int64_t workspace_bytes,
                                    float* out, void* stream);

/*
 * xq_paged_decode_attention for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same decode, with the
 * split partials in a scratch array built into the library instead of a caller workspace.
 * Arguments, results and errors are those of xq_paged_decode_attention without the workspace;
 * the output is bitwise that of xq_paged_decode_attention with the same arguments.
 *
 * The scratch holds 16 MiB (XQ_NOALLOC_SCRATCH_BYTES) on each GPU the library runs on, until the
 * process ends: a call whose xq_decode_workspace_bytes(...) exceeds it returns XQ_EWORKSPACE and
 * launches nothing. The call allocates and frees nothing (its first call on a device only looks
 * up the array's address there) and ignores XQ_DEBUG (the checked mode copies to host memory).
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.
 */
#define XQ_NOALLOC_SCRATCH_BYTES (16ll << 20)
xq_status xq_paged_decode_attention_noalloc(const xq_cache_layout* layout,
                                            const void* q, int32_t batch, int32_t num_q_heads,
                                            const void* k_pool, const void* v_pool,
                                            const int32_t* block_tables, int32_t max_pages_per_seq,
                                            const int32_t* context_lens, int32_t max_context_len,
                                            float softmax_scale, int32_t num_splits_hint,
                                            float* out, void* stream);

/*
 * Optional host-side plan for a decode (the split into a host "plan" and a device "run" of
 * batched-attention libraries): from the host's copy of the context lengths, where each piece of
 * work runs, so that the SIMDs finish together. With every work unit resident, the GPU fills its
 * SIMDs round-robin by workgroup id (workgroup i runs on SIMD i mod S, S SIMDs). The order changes
 * where work runs, never what it computes: outputs are bitwise those of xq_paged_decode_attention.
 *   - One partition per sequence: a permutation of the batch that puts long and short sequences
 *     on the same SIMDs (the decode's unit order puts sequence slots b, b + S / num_kv_heads, ...
 *     on the same SIMDs; sequences sorted by length are dealt to those slot groups in snake
 *     order); the identity where that cannot help (a batch that is not a multiple of 8).
 *   - Several partitions: a unit plan with one entry per work slot (workgroup id) of the launch:
 *     the work unit (b * nsplits + split) * num_kv_heads + kv_head it runs, or -1. The (sequence,
 *     partition) groups are placed longest first on the least loaded SIMDs, the kv heads of a
 *     group on one XCD.
 *
 *   host_context_lens  int32 [batch], host memory: the lengths the decode will see
 *   host_seq_order     int32 [xq_decode_plan_entries(...)], host memory, written
 * Other arguments as for xq_decode_num_splits. The device is queried for its SIMD count (1024,
 * MI355X's, if that fails). Nothing is launched; XQ_EINVAL on invalid arguments.
 */
xq_status xq_decode_plan(const xq_cache_layout* layout, int32_t batch, int32_t num_q_heads,
                         int32_t max_context_len, int32_t num_splits_hint,
                         const int32_t* host_context_lens, int32_t* host_seq_order);

/* Entries of the plan xq_decode_plan writes for these arguments: batch with one partition per
 * sequence, else the launch's work slots (splits x kv heads x batch). -1 on invalid arguments. */
int32_t xq_decode_plan_entries(const xq_cache_layout* layout, int32_t batch, int32_t num_q_heads,
                               int32_t max_context_len, int32_t num_splits_hint);

/*
 * xq_paged_decode_attention with a plan: seq_order is device int32 [plan_entries], the plan's
 * host_seq_order for the same arguments and host lengths, copied to the device by the caller;
 * plan_entries must equal xq_decode_plan_entries for these arguments (XQ_EINVAL otherwise, nothing
 * launched). The result is bitwise that of xq_paged_decode_attention with the same arguments. A
 * seq_order that is not such a plan (not a permutation; a unit plan that repeats a unit, or misses
 * one with tokens or partition 0 of a sequence, which writes an empty sequence's zeros) is outside
 * the contract: rejected under XQ_DEBUG, otherwise some work is done twice and other work not at
 * all (unit entries outside the units are skipped).
 */
xq_status xq_paged_decode_attention_planned(const xq_cache_layout* layout,
                                            const void* q, int32_t batch, int32_t num_q_heads,
                                            const void* k_pool, const void* v_pool,
                                            const int32_t* block_tables, int32_t max_pages_per_seq,
                                            const int32_t* context_lens, int32_t max_context_len,
                                            float softmax_scale, int32_t num_splits_hint,
                                            void* workspace, int64_t workspace_bytes,
                                            float* out, const int32_t* seq_order, int32_t plan_entries,
                                            void* stream);

/*
 * One decode step in one launch: append each sequence's new K/V row, then decode. Equivalent to
 * xq_quantize_append of row b of k_new/v_new at position context_lens[b] - 1 of sequence b (for
 * every b with context_lens[b] >= 1), followed by xq_paged_decode_attention (or, with a non-NULL
 * seq_order, xq_paged_decode_attention_planned) with the same arguments: the stored bytes and
 * the outputs are bitwise those of the two separate calls. The wave that decodes the last
 * partition of a sequence encodes that sequence's new rows of its kv head first and waits for
 * the stores before it loads the cache, so no separate launch is needed (the xInfer page's
 * decode step, section "What actually sits between the request and the tokens": rotate and
 * quantize the new rows, then attend).
 *
 *   k_new, v_new       bf16 [batch][num_kv_heads][128], 16-byte aligned: the step's new rows
 *   k_pool, v_pool     written (the new rows) and read
 *   seq_order          NULL, or a device plan as for xq_paged_decode_attention_planned
 *   plan_entries       its entries (ignored when seq_order is NULL)
 * Other arguments, errors and the workspace as for xq_paged_decode_attention. context_lens are
 * the lengths after the append; the new row's slot must lie in a page of the block table.
 */
xq_status xq_append_decode_attention(const xq_cache_layout* layout,
                                     const void* k_new, const void* v_new,
                                     const void* q, int32_t batch, int32_t num_q_heads,
                                     void* k_pool, void* v_pool,
                                     const int32_t* block_tables, int32_t max_pages_per_seq,
                                     const int32_t* context_lens, int32_t max_context_len,
                                     float softmax_scale, int32_t num_splits_hint,
                                     void* workspace, int64_t workspace_bytes,
                                     float* out, const int32_t* seq_order, int32_t plan_entries,
                                     void* stream);

/*
 * Length-aware partitions for a decode over sequences of mixed lengths (the infero page, section
 * "Beyond plain text decode", item "Continuous batching": decodes of long and short sequences
 * share one step). Host only; nothing is launched. From the host's copy of the context lengths,
 * every sequence gets its own partition size so that all work units (partition x kv head) hold
 * about the same number of tokens and all fit the waves the GPU keeps resident at once: no
 * unit is left to run alone at the end. Units are ordered longest first and dealt over the
 * compute units, the kv heads of a partition on one XCD.
 *   host_context_lens  int32 [batch], host memory: the lengths the decode will see
 *   host_seq_tps       int32 [batch], host memory, written: tokens per partition of sequence b, a
 *                      multiple of 32 and of page_size, at most 128 pages
 *   host_units         NULL, or int32 pairs [batch * nsplits * num_kv_heads][2], host memory,
 *                      written: pair i = {unit, host_seq_tps[b]} for work slot i, unit =
 *                      (b * nsplits + partition) * num_kv_heads + kv_head, or {-1, 0}
 * Returns nsplits, the partitions' stride (the largest partition count of a sequence, >= 1), or
 * -1 on invalid arguments (xq_last_error says why). Call once with host_units = NULL to size it.
 */
int32_t xq_decode_plan_balanced(const xq_cache_layout* layout, int32_t batch, int32_t num_q_heads,
                                int32_t max_context_len, const int32_t* host_context_lens,
                                int32_t* host_seq_tps, int32_t* host_units);

/* Workspace bytes of xq_decode_attention_balanced for a plan of stride nsplits; -1 on invalid
 * arguments. */
int64_t xq_decode_workspace_bytes_balanced(const xq_cache_layout* layout, int32_t batch,
                                           int32_t num_q_heads, int32_t nsplits);

/*
 * The decode (optionally with the step's append, as xq_append_decode_attention) over a
 * length-aware plan: units and seq_tps are device copies of the plan's host_units (pairs) and
 * host_seq_tps for the same lengths, nsplits its return value. Each unit covers its partition
 * of seq_tps[b] tokens; sequences with several partitions are merged by log-sum-exp as for the
 * other decodes. Results equal xq_paged_decode_attention's up to the rounding of a different
 * partitioning (within the split-agreement bound).
 *   k_new, v_new  NULL (no append), or both bf16 [batch][num_kv_heads][128], 16-byte aligned
 * The same launch can also append rows of sequences it does not decode, as xq_quantize_append
 * does (the step's prefill chunk, continuous batching as the infero page describes it in
 * section "Beyond plain text decode"): the appenders run after the decode's units, in the
 * idle end of the launch, and their codes and scales equal xq_quantize_append's bit for bit.
 *   chunk_tokens  rows to append (0: none; then the chunk pointers may be NULL)
 *   chunk_k, chunk_v, chunk_seq, chunk_pos  as xq_quantize_append's k_new, v_new, token_seq,
 *                 token_pos, with chunk_seq indexing rows of the same block_tables (any row,
 *                 not only the first batch) and at most 2^28 - 1 (token, kv head) rows
 * No chunk row may land in a page that the decode reads (a page holding rows 0 .. L_b - 1 of
 * a decoded sequence b): the decode's units and the appenders run in no fixed order, so such
 * a row would race the decode (rejected under XQ_DEBUG, with xq_quantize_append's checks).
 * Other arguments and errors as for xq_paged_decode_attention; the workspace is
 * xq_decode_workspace_bytes_balanced(layout, batch, num_q_heads, nsplits) bytes. A plan that
 * does not match the lengths (a unit twice or missing, a pair whose size is not its sequence's)
 * is outside the contract: rejected under XQ_DEBUG.
 */
xq_status xq_decode_attention_balanced(const xq_cache_layout* layout, const void* q, int32_t batch,
                                       int32_t num_q_heads, void* k_pool, void* v_pool,
                                       const int32_t* block_tables, int32_t max_pages_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len,
                                       float softmax_scale, int32_t nsplits, const int32_t* units,
                                       const int32_t* seq_tps, const void* k_new, const void* v_new,
                                       const void* chunk_k, const void* chunk_v, int32_t chunk_tokens,
                                       const int32_t* chunk_seq, const int32_t* chunk_pos,
                                       void* workspace, int64_t workspace_bytes, float* out,
                                       void* stream);

/*
 * Workspace bytes xq_paged_prefill_attention needs for these arguments (the partition partials;
 * 0 when the chunk runs in one partition). Returns -1 on invalid arguments.
 */
int64_t xq_prefill_workspace_bytes(const xq_cache_layout* layout, int32_t n_query,
                                   int32_t num_q_heads, int32_t start_pos,
                                   int32_t num_splits_hint);

/*
 * Chunked prefill attention over the paged (and, for turbo types, quantized) cache: the queries
 * of one chunk of one sequence, each attending causally to the sequence's cached rows. Defined
 * by the infero page, section "Beyond plain text decode", item "Continuous batching" (decodes
 * go first, prefill fills the rest of a step and may be split across steps, so a chunk attends
 * to the cached rows of earlier chunks and to its own), with each row read as the decode reads
 * it (the xInfer page's TurboQuant rows, rotated and quantized).
 *
 * Query i sits at position start_pos + i and attends to positions 0 .. start_pos + i (no row
 * after its own); the chunk's own K/V rows must have been appended (xq_quantize_append) before.
 * Per query head j (kv head j / (num_q_heads / num_kv_heads)) the result is the decode's formula
 * with context length start_pos + i + 1.
 *
 *   q                  bf16 [n_query][num_q_heads][128], 16-byte aligned
 *   k_pool, v_pool     pools written by xq_quantize_append
 *   block_table        int32 [max_pages]: the sequence's physical page per logical page
 *   start_pos          position of query 0 (the number of rows cached before the chunk), >= 0
 *   softmax_scale      multiplies q . k
 *   num_splits_hint    as for xq_paged_decode_attention
 *   workspace          device scratch of >= xq_prefill_workspace_bytes(layout, n_query,
 *                      num_q_heads, start_pos, num_splits_hint) bytes (may be NULL when that is
 *                      0); calls that share a workspace must not overlap
 *   out                fp32 [n_query][num_q_heads][128], 16-byte aligned
 * n_query = 0 is a no-op. start_pos + n_query must not exceed max_pages * page_size (XQ_EINVAL);
 * more than 65535 queries, a group size above 16 or 2^26 or more (split, kv head, query) units
 * give XQ_EUNSUPPORTED. The block-table entries of positions below start_pos + n_query must be
 * pages of the pool (checked only under XQ_DEBUG).
 * Kernels: with fixed partitions (num_splits_hint < 0) the queries run on the decode's kernel,
 * and each query's output is bitwise the decode's with the same partition when the group size
 * is 16; otherwise a tile kernel runs the chunk (a workgroup converts each 64-token tile once
 * for 8 * (16 / group) queries), with its own rounding order, within the same tolerance.
 */
xq_status xq_paged_prefill_attention(const xq_cache_layout* layout,
                                     const void* q, int32_t n_query, int32_t num_q_heads,
                                     const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, int32_t max_pages,
                                     int32_t start_pos, float softmax_scale, int32_t num_splits_hint,
                                     void* workspace, int64_t workspace_bytes,
                                     float* out, void* stream);

/*
 * Streaming-read reference for the decode's roofline: a measurement aid, not part of the attention
 * method. The decode reads each cache byte once per step, so its ceiling is the rate at which this
 * GPU's HBM delivers bytes to a kernel that only reads; this call launches such a kernel.
 *
 *   buf            device memory of buf_bytes bytes, 16-byte aligned; only read
 *   n_blocks       blocks to read (0 is a no-op; n_blocks * block_bytes below 2 TiB)
 *   block_bytes    bytes of a block: a power of two from 1024 to 2^20 (a wave reads 1 KiB at a
 *                  time)
 *   block_stride   bytes between block starts (a multiple of 16, >= block_bytes)
 *   block_order    NULL: block i starts at i * block_stride, all within buf_bytes (checked);
 *                  else device int32 [n_blocks]: block i starts at block_order[i] * block_stride,
 *                  which must lie, with its block_bytes, inside buf (the caller's contract,
 *                  not checked on the device)
 *   sink           device uint32 [1]: written only if the XOR of everything read equals a fixed
 *                  value (so the reads cannot be optimised away); its contents do not matter
 * Time it with events on `stream`: bytes read = n_blocks * block_bytes. XQ_EINVAL on invalid
 * arguments, XQ_EHIP if the launch fails.
 */
xq_status xq_hbm_read_probe(const void* buf, int64_t buf_bytes, int64_t n_blocks, int32_t block_bytes,
                            int64_t block_stride, const int32_t* block_order, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* XQ_H */
