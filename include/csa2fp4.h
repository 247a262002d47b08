/*
 * csa2fp4.h -- C ABI of libcsa2fp4.so: the decode / prefill-chunk step of CSA2
 * sparse attention over a sequence-compressed global KV cache stored in FP4,
 * for AMD MI355X (gfx950).
 *
 * What the step computes comes from the pages describing DeepSeek-V4.1-Flash:
 *   - "DeepSeek-V4.1-Flash, expliqué pas à pas", CSA2 section: a shared global cache
 *     of compressed entries (m tokens each, disjoint groups), a light indexer that
 *     scores every entry from an indexer query and one indexer key per entry and
 *     keeps the best k, and a main attention that reads the selected entries plus
 *     the layer's own sliding-window KV; the Full / Reindex / Reuse layer modes.
 *   - same page, FP4 KV cache section: main entries are E2M1 values with one E4M3
 *     scale per 16 channels (288 B per 512-channel entry), quantised after RoPE and
 *     dequantised before attention; indexer keys and queries are OCP MXFP4 (E2M1
 *     values with one E8M0 scale per 32 channels, 68 B per 128-channel key).
 *   - same page, attention forms: the window covers the last 128 tokens.
 *   - "Résumé exécutif", CSA2 mode table: Full computes cache, indexer keys and
 *     indices; Reindex reuses cache and keys and recomputes indices; Reuse reuses all.
 *
 * Conventions for every entry point:
 *   - Array arguments and every pointer inside csa2_fp4_cache are DEVICE pointers,
 *     allocated and owned by the caller.  The cache descriptor struct itself is a
 *     host struct.  The library allocates no memory and never synchronises; work
 *     is enqueued on `stream` in order.  Its only global state is one diagnostic
 *     counter per device (csa2_exact_path_count below) and the static workspace of
 *     index_topk_noalloc.
 *   - Arguments are validated on the host before anything is enqueued, so a bad
 *     argument returns a negative csa2_status and enqueues nothing.  A failed
 *     launch returns CSA2_ERR_LAUNCH (work enqueued before it may have run).
 *   - Device-side preconditions (not checked): slots unique and in range; every
 *     block-table entry read is a valid page; n_visible <= ld and covered by the
 *     block table; indices are < n_visible or -1; inputs are finite.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 */
#ifndef CSA2FP4_H
#define CSA2FP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_NULL = -1,        /* a required pointer is NULL                         */
  CSA2_ERR_SHAPE = -2,       /* a size or count is out of range                    */
  CSA2_ERR_UNSUPPORTED = -3, /* a supported-but-not-built configuration            */
  CSA2_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than the *_workspace_size */
  CSA2_ERR_LAUNCH = -5       /* a kernel launch failed                              */
} csa2_status;

#define CSA2_LATENT_DIM 512 /* channels of a main-cache entry and of a window row */
#define CSA2_INDEX_DIM 128  /* channels of an indexer key / query head             */
#define CSA2_PAGE_SIZE 64   /* cache slots per page                                */
#define CSA2_MAX_K 4096     /* largest top-k                                       */
#define CSA2_MAX_WINDOW 128 /* largest sliding window                              */

/* One global FP4 cache (the cache of one Full layer).  Per slot s:
 *   main_codes [s*256 .. s*256+255]: 512 E2M1 codes, byte i holds channel 2i in
 *                                    bits 0-3 and channel 2i+1 in bits 4-7;
 *                                    code = 8*sign + index into {0,.5,1,1.5,2,3,4,6}
 *   main_scales[s*32 .. s*32+31]   : OCP E4M3FN scale of channels 16g .. 16g+15
 *   idx_codes  [s*64 .. s*64+63]   : 128 E2M1 codes of the indexer key, same order
 *   idx_scales [s*4 .. s*4+3]      : OCP E8M0 scale of channels 32b .. 32b+31
 * That is 288 + 68 = 356 bytes per slot.  num_slots is a multiple of page_size,
 * and a sequence's logical entry j lives in slot
 *   block_table[row][j / page_size] * page_size + j % page_size.            */
typedef struct {
  uint8_t* main_codes;
  uint8_t* main_scales;
  uint8_t* idx_codes;
  uint8_t* idx_scales;
  int64_t num_slots;
  int32_t page_size; /* must be CSA2_PAGE_SIZE */
} csa2_fp4_cache;

/* Human-readable name of a status code (static string). */
const char* csa2_status_string(int status);

/* fp4_cache_write -- quantise n compressed entries into the cache.
 * Source: "DeepSeek-V4.1-Flash, expliqué pas à pas", FP4 KV cache section (E2M1 with
 * one E4M3 scale per 16 channels for the main entry; OCP MXFP4 for the indexer key;
 * quantisation after RoPE, one format for all channels).
 *   latent  bf16 [n][512] : post-RoPE compressed main entries
 *   idx_key bf16 [n][128] : indexer keys of the same entries
 *   slot    int64 [n]     : destination slot of each row, unique, < num_slots
 * Rounding: per 16-channel block the scale is the E4M3FN value nearest to amax/6
 * (ties to even, saturating at 448); per 32-channel indexer block the scale is
 * 2^(floor(log2 amax) - 2) (2^-127 for an all-zero block); each channel takes the
 * nearest of the 8 E2M1 magnitudes times the scale (ties to the even code), keeps
 * its sign bit, and a zero E4M3 scale gives signed zeros.  Bit-exact and
 * deterministic.  n == 0 is a no-op. */
int fp4_cache_write(const csa2_fp4_cache* cache, const uint16_t* latent, const uint16_t* idx_key,
                    const int64_t* slot, int64_t n, hipStream_t stream);

/* index_score -- lightning-indexer scores of visible entries.
 * Source: "DeepSeek-V4.1-Flash, expliqué pas à pas", CSA2 section (the indexer scores
 * each entry from the query's indexer query and the entry's indexer key) and FP4 KV
 * cache section (indexer queries and keys are MXFP4).
 *   q_idx bf16 [nq][Hi][128]  : indexer queries, quantised to MXFP4 inside the call
 *   w     f32  [nq][Hi]       : per-head weights
 *   Hi                        : indexer heads, a multiple of 16, 16 <= Hi <= 128
 *   seq_of_query int32 [nq]   : block-table row of each query (NULL: row q)
 *   n_visible    int32 [nq]   : entries 0 .. n_visible[q]-1 are scored, <= ld
 *   block_table  int32 [rows][max_pages]
 *   scores f32 [nq][ld]       : only positions < n_visible[q] are written
 * score[q][j] = sum over h of w[q][h] * max(d_h, 0), where d_h is the exact dot
 * product of the MXFP4-quantised query head and key rounded once to fp32, and the
 * sum is an fp32 fused-multiply-add chain over h = 0 .. Hi-1 starting from +0.
 * Bit-exact and deterministic. */
int index_score(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* block_table, int32_t max_pages,
                int32_t nq, float* scores, int64_t ld, hipStream_t stream);

/* topk_select -- the k best entries per query.
 * Source: "DeepSeek-V4.1-Flash, expliqué pas à pas", attention forms and CSA2 section
 * (the indexer keeps only the best-scoring entries).
 *   scores f32 [nq][ld]  : positions < n_visible[q] are read
 *   k                    : 1 <= k <= 4096
 *   topk_idx int32 [nq][k]: the min(k, n_visible[q]) entries with the largest score
 *                          (numeric compare; ties go to the lower index), in
 *                          ascending index order, then -1 padding.
 *   ws, ws_bytes          : device workspace of at least
 *                          topk_select_workspace_size(nq, ld, k) bytes.  It must be
 *                          zero-filled before its first use; every call returns its
 *                          counters and histograms to zero (in stream order), so the
 *                          next call needs no clearing.  The rest of it is scratch
 *                          that each call overwrites before reading.  Calls sharing
 *                          one workspace must be stream-ordered.
 * Bit-exact and deterministic. */
size_t topk_select_workspace_size(int32_t nq, int64_t ld, int32_t k);
int topk_select(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k,
                int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t stream);

/* index_topk -- index_score followed by topk_select on the same scores, as one call:
 * the indexer stage of a Full or Reindex layer.
 * Source: as for index_score and topk_select ("DeepSeek-V4.1-Flash, expliqué pas à
 * pas", CSA2 section: the indexer scores every entry, then keeps the best ones).
 * Arguments as for the two calls; ws / ws_bytes as for topk_select (same size, same
 * zero-fill contract).  scores and topk_idx are bit-identical to calling index_score
 * and then topk_select.  When every query reads its own sequence (seq_of_query NULL,
 * or fewer than 64 queries) the selection's first counting pass is folded into the
 * scoring pass, which saves one launch. */
int index_topk(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
               const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* block_table, int32_t max_pages,
               int32_t nq, float* scores, int64_t ld, int32_t k, int32_t* topk_idx, void* ws, size_t ws_bytes,
               hipStream_t stream);

/* index_score_counted, topk_select_counted -- index_topk as two calls, for callers
 * that want the scores before the selection runs (or time the two apart).
 * Source: as for index_topk.
 * index_score_counted: index_score (same arguments and scores) that also leaves the
 *   selection's first-digit histogram of each row with n_visible > k in ws (the
 *   topk_select workspace for (nq, ld, k), same zero-fill contract).  With one query
 *   per workgroup it counts as it scores, the kernel index_topk runs; otherwise a
 *   counting pass follows the scan.
 * topk_select_counted: topk_select (same arguments and indices) that takes those
 *   counts from ws instead of counting; call it next on the same scores, k and ws,
 *   with no other use of ws in between.  It returns ws to its zero state.
 * Together they give scores and indices bit-identical to index_topk.  Errors as for
 * index_score and topk_select. */
int index_score_counted(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                        const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* block_table,
                        int32_t max_pages, int32_t nq, float* scores, int64_t ld, int32_t k, void* ws,
                        size_t ws_bytes, hipStream_t stream);
int topk_select_counted(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k,
                        int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t stream);

/* index_topk_noalloc -- index_topk for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid it.  The
 * same arguments without ws / ws_bytes and the same results (bit for bit): the
 * selection's workspace is a static array of CSA2_NOALLOC_SCRATCH_BYTES in device
 * memory, one per device, held until the process ends.  Calls that need more
 * (topk_select_workspace_size(nq, ld, k) > CSA2_NOALLOC_SCRATCH_BYTES; 1M-entry rows
 * take about 0.37 MB per query) return CSA2_ERR_WORKSPACE and enqueue nothing.  The
 * call allocates nothing (no hipMalloc, no library allocation); it clears the array's
 * counters with a kernel (no memset node, so it may be captured into a graph).  All
 * calls on one device share the array: calls that overlap on one device (different
 * streams, not ordered) race and give undefined results; calls on one stream are
 * safe.  The array's device address is looked up on the first call on each device.
 * A HIP failure in that lookup returns CSA2_ERR_LAUNCH. */
#define CSA2_NOALLOC_SCRATCH_BYTES (32u << 20)
int index_topk_noalloc(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                       const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* block_table,
                       int32_t max_pages, int32_t nq, float* scores, int64_t ld, int32_t k, int32_t* topk_idx,
                       hipStream_t stream);

/* Hierarchical candidate pool.
 * Source: "DeepSeek V4.1 Flash et le cerveau divisé", memory section (the first
 * decoder layer scans the whole global cache and assembles a pool of about 16,000
 * positions organised as 2048 blocks of 8; the layers after it may not search
 * outside the pool); "DeepSeek-V4.1-Flash, expliqué pas à pas", CSA2 section (for a
 * fixed pool the deeper indexers' cost no longer grows with the context).  The rule
 * that picks the blocks is not on the pages; the one here: blocks of CSA2_POOL_BLOCK
 * consecutive entries are ranked by the largest score among their visible members,
 * ties to the lower block.
 *
 * index_pool_build -- the pool of each query from a gatekeeper layer's scores.
 *   scores f32 [nq][ld]  : positions < n_visible[q] are read (e.g. index_topk's scores)
 *   npool                : blocks kept, 1 <= npool <= 4096 (2048 in the pages)
 *   pool int32 [nq][npool]: the min(npool, ceil(n_visible/8)) best blocks, ascending,
 *                          then -1 padding
 *   ws, ws_bytes          : at least index_pool_build_workspace_size(nq, ld, npool)
 *                          bytes, with the zero-fill contract of topk_select.
 * Bit-exact and deterministic. */
#define CSA2_POOL_BLOCK 8
size_t index_pool_build_workspace_size(int32_t nq, int64_t ld, int32_t npool);
int index_pool_build(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t npool,
                     int32_t* pool, void* ws, size_t ws_bytes, hipStream_t stream);

/* index_topk_pool_build -- the gatekeeper layer's indexer stage in one call: index_topk
 * and then index_pool_build on the same scores (the arguments of both; npool and pool
 * as for index_pool_build).  scores, topk_idx and pool are bit-identical to the two
 * calls.  With one query per workgroup (as for index_topk's folded counting) the scan
 * also writes each 8-entry block's largest visible score and counts its first digit,
 * so the pool's selection needs neither the block-maximum launch nor a counting
 * launch.  ws, ws_bytes: at least index_topk_pool_build_workspace_size(nq, ld, k,
 * npool) bytes, zero-filled before the first use (every call leaves its counters
 * zero, as for topk_select). */
size_t index_topk_pool_build_workspace_size(int32_t nq, int64_t ld, int32_t k, int32_t npool);
int index_topk_pool_build(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                          const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* block_table,
                          int32_t max_pages, int32_t nq, float* scores, int64_t ld, int32_t k, int32_t* topk_idx,
                          int32_t npool, int32_t* pool, void* ws, size_t ws_bytes, hipStream_t stream);

/* index_topk_pool -- index_topk restricted to each query's candidate pool: the
 * indexer stage of a Reindex layer behind a gatekeeper layer.
 *   pool int32 [nq][npool] : as written by index_pool_build (blocks ascending, -1 last)
 *   scores_pool f32 [nq][8*npool] out: position 8r + i holds the score (as index_score)
 *                           of member i of block pool[q][r]; only the positions that
 *                           hold a visible entry are written (a prefix of the row)
 *   topk_idx int32 [nq][k] out: the min(k, visible members) members with the largest
 *                           score, ties to the lower entry, as ENTRY indices in
 *                           ascending order, then -1 padding
 *   ws, ws_bytes           : at least index_topk_pool_workspace_size(nq, npool, k)
 *                           bytes, with the zero-fill contract of topk_select.
 * Other arguments as for index_topk (block_table rows cover n_visible).  Bit-exact
 * and deterministic; with a pool that covers every block the result equals
 * index_topk's. */
size_t index_topk_pool_workspace_size(int32_t nq, int32_t npool, int32_t k);
int index_topk_pool(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                    const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* pool, int32_t npool,
                    const int32_t* block_table, int32_t max_pages, int32_t nq, float* scores_pool, int32_t k,
                    int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t stream);

/* sparse_attn_decode -- one softmax over the selected cache entries and the window.
 * Source: "DeepSeek-V4.1-Flash, expliqué pas à pas", CSA2 section (the main query
 * reads the selected entries and the layer's own sliding-window KV; FP4 is only a
 * storage format, dequantised before attention) and intro (softmax-weighted mean);
 * "La lignée DeepSeek" (one latent vector shared by all heads).
 *   q bf16 [B][H][512]        : main queries, H a multiple of 16, 16 <= H <= 128
 *   topk_idx int32 [B][k]     : selected entries of sequence b (-1 = none)
 *   block_table int32 [B][max_pages] : row b belongs to sequence b
 *   swa bf16 [B][window][512] : window rows; rows 0 .. swa_len[b]-1 are valid
 *   softmax_scale             : logit multiplier (1/sqrt(512) in the workloads)
 *   out f32 [B][H][512], lse f32 [B][H]
 * Each dequantised entry and each window row is both key and value for every head:
 * z = softmax_scale * q_h . x, out_h = sum softmax(z)_x x, lse_h = log sum exp z.
 * With no rows at all: out = 0, lse = -inf.  Within 2e-3 absolute of an fp64
 * evaluation on the workloads' data.
 *   ws, ws_bytes: at least sparse_attn_decode_workspace_size(B, H, k, window). */
size_t sparse_attn_decode_workspace_size(int32_t B, int32_t H, int32_t k, int32_t window);
int sparse_attn_decode(const csa2_fp4_cache* cache, const uint16_t* q, int32_t H, const int32_t* topk_idx, int32_t k,
                       const int32_t* block_table, int32_t max_pages, const uint16_t* swa, const int32_t* swa_len,
                       int32_t window, float softmax_scale, int32_t B, float* out, float* lse, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* sparse_attn_prefill_chunk -- decode attention for T consecutive query tokens.
 * Source: as sparse_attn_decode; each query token has its own top-k selection and
 * its own causal window of the last `window` tokens.
 *   q bf16 [T][H][512], topk_idx int32 [T][k]  (row i: query token chunk_start + i)
 *   block_table int32 [max_pages]               : the one sequence's page table
 *   swa bf16 [window-1+T][512]                  : row r holds token
 *                                                 chunk_start - window + 1 + r
 *   swa_first_valid                             : rows below it do not exist
 * Query i attends its selected entries plus window rows max(i, swa_first_valid) ..
 * i + window - 1 under one softmax.  out f32 [T][H][512], lse f32 [T][H].
 * A bounded replay that restarts the window at the chunk's first token s ("DeepSeek-
 * V4.1-Flash, expliqué pas à pas", bounded SWA replay: keys of the window truncated
 * to the replayed segment) passes swa_first_valid = window - 1, so query token t
 * sees window tokens max(s, t - window + 1) .. t. 
 *   ws, ws_bytes: at least sparse_attn_prefill_chunk_workspace_size(T, H, k, window). */
size_t sparse_attn_prefill_chunk_workspace_size(int32_t T, int32_t H, int32_t k, int32_t window);
int sparse_attn_prefill_chunk(const csa2_fp4_cache* cache, const uint16_t* q, int32_t H, const int32_t* topk_idx,
                              int32_t k, const int32_t* block_table, int32_t max_pages, int64_t chunk_start, int32_t T,
                              const uint16_t* swa, int32_t swa_first_valid, int32_t window, float softmax_scale,
                              float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* FP8 window.  "DeepSeek-V4.1-Flash, expliqué pas à pas", FP4 KV cache section: the
 * sliding-window KV stays in FP8 because it is more sensitive to quantisation.  The
 * pages give no format; the one used here: E4M3FN codes and one E8M0 scale per
 * 512-channel row, X = the smallest power of two with amax <= 448 X (no code
 * saturates), code = the E4M3FN value nearest to x / X (ties to even, sign copied);
 * an all-zero row gets X = 2^-127.  Every dequantised value is exact in bf16, so the
 * attention over an FP8 window equals the attention over the bf16 rows holding those
 * values.
 *
 * swa_fp8_write -- quantise n window rows.
 *   rows bf16 [n][512]; codes u8 [n][512] out; scales u8 [n] out (E8M0 byte e + 127).
 *   Rows are independent (any n >= 0).  NULL pointers with n > 0: CSA2_ERR_NULL. */
int swa_fp8_write(const uint16_t* rows, int64_t n, uint8_t* codes, uint8_t* scales, hipStream_t stream);

/* sparse_attn_decode_fp8win / sparse_attn_prefill_chunk_fp8win -- the attention calls
 * above with the window as FP8 rows: swa_codes u8 and swa_scales u8 in place of swa,
 * laid out as swa's rows ([B][window] rows for decode, [window-1+T] rows for the
 * prefill chunk).  Everything else, the workspaces included
 * (sparse_attn_decode_workspace_size, sparse_attn_prefill_chunk_workspace_size), is as
 * for the bf16 calls.  window > 0 with a NULL codes or scales pointer: CSA2_ERR_NULL. */
int sparse_attn_decode_fp8win(const csa2_fp4_cache* cache, const uint16_t* q, int32_t H, const int32_t* topk_idx,
                              int32_t k, const int32_t* block_table, int32_t max_pages, const uint8_t* swa_codes,
                              const uint8_t* swa_scales, const int32_t* swa_len, int32_t window, float softmax_scale,
                              int32_t B, float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);
int sparse_attn_prefill_chunk_fp8win(const csa2_fp4_cache* cache, const uint16_t* q, int32_t H,
                                     const int32_t* topk_idx, int32_t k, const int32_t* block_table,
                                     int32_t max_pages, int64_t chunk_start, int32_t T, const uint8_t* swa_codes,
                                     const uint8_t* swa_scales, int32_t swa_first_valid, int32_t window,
                                     float softmax_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* Diagnostic: the number of (query, entry) index scores that were recomputed on the
 * exact integer path since the last csa2_exact_path_reset(), on the current device.
 * index_score, index_topk and index_topk_pool take an entry's score from the FP4
 * matrix unit only when every partial sum of each head's dot is exactly
 * representable in fp32 (the per-block exponent sums span at most 10 and stay in
 * fp32's normal range, so the result is the exact dot); other entries are
 * recomputed from the definition, with identical results either way.  Both calls
 * are synchronous with respect to the device; the count covers work enqueued and
 * finished before the call.  count NULL: CSA2_ERR_NULL; a HIP failure:
 * CSA2_ERR_LAUNCH. */
int csa2_exact_path_count(unsigned long long* count);
int csa2_exact_path_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2FP4_H */
