/*
 * indexer_fp4.h -- C ABI of the MI355X (gfx950) FP4 sparse-indexer library.
 *
 * What the library computes (sources are web pages, cited by title and section):
 *   [P2] "Score a DSA sparse indexer in FP4" (ROCm/ATOM pull request #2216)
 *   [P1] ROCm/ATOM pull request #2125, Technical Details section 3
 *        "FP4 indexer padding rows"
 *
 * A DSA sparse indexer keeps one 128-dim index key per token. Here the keys are
 * stored in FP4: packed E2M1 codes (64 bytes per key) plus one e8m0 scale byte per
 * 32 elements, in 64-token pages ([P2] commit message and PR description intro).
 * For every query row the scorer computes, per index head, the dot product of the
 * row's query with every key the row may see, applies ReLU, and sums the heads with
 * per-head weights into one fp32 logit per key; a top-k then keeps the index_topk
 * best keys per row.
 *
 * Memory layout (one index region, two planes; [P2] PR description intro):
 *   kv_packed  uint8 [n_pages][64 pos][64 B]  key (page,pos), element d in byte d/2,
 *                                             even d in the low nibble
 *   kv_scale   uint8 [n_pages][4 group][64 slot]  scale of elements 32g..32g+31 of
 *                                             key (page,pos) at slot (pos%16)*4 + pos/16,
 *                                             the 16x4 transpose of the row axis ([P2]
 *                                             second review finding; commit "Use the
 *                                             index scale plane's own row order ...")
 *   q_packed   uint8 [rows][n_heads][64 B]    same packing as keys
 *   q_scale    uint8 [rows][n_heads][4]       scale of elements 32g..32g+31 at [g]
 *   weights    fp32  [rows][n_heads]          per-head weights
 *   block_table int32 [seqs][bt_ld]           page of key j of sequence s at
 *                                             block_table[s][j/64], position j%64
 *   logits     fp32  [rows][logits_ld]        column j = key position j of the row's
 *                                             sequence; only j < row_len[r] is written
 *
 * Encoding (the pages name the format but print no rule; OCP Microscaling v1.0):
 *   scale exponent e = floor(log2(amax of the 32 elements)) - 2, clamped to
 *   [-127, 127], byte e + 127 (0 for an all-zero block); each element is rounded to
 *   the nearest of +-{0, 0.5, 1, 1.5, 2, 3, 4, 6} * 2^e, ties to the even code,
 *   larger magnitudes saturate to 6 * 2^e; the sign bit is the input's sign bit.
 *
 * Conventions shared by every call:
 *   - Pointers are DEVICE pointers unless marked [host]. The caller owns every buffer;
 *     the library keeps no pointer past the call and allocates no device memory.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls are asynchronous on
 *     it, never synchronize, and never read device memory on the host, so a sequence
 *     of calls can be captured into a HIP graph and replayed.
 *   - Return value: INDEXER_FP4_OK (0) or a negative code; nothing is launched when a
 *     call returns an error. indexer_fp4_last_error() then holds a message (per host
 *     thread) that names the offending quantities.
 *   - Problems only visible on the device (a block-table entry outside [0, n_pages),
 *     a context longer than the block table covers) never fault: the kernel skips the
 *     page and ORs a flag into the error word of the schedule buffer it was given
 *     (int32 at byte offset 4 of the buffer; see INDEXER_FP4_DEV_*).
 *   - The library refuses what it cannot do (wrong geometry, wrong GPU); it has no
 *     fallback path ([P2] Scope: the structural gate, with falling back to FP8 left
 *     to the caller).
 */
#ifndef INDEXER_FP4_H
#define INDEXER_FP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  INDEXER_FP4_OK = 0,
  INDEXER_FP4_EINVAL = -1, /* an argument is out of range or inconsistent */
  INDEXER_FP4_ENOSPC = -2, /* a buffer (schedule, workspace, logits, table) is too small */
  INDEXER_FP4_EARCH = -3,  /* the current device is not gfx950 */
  INDEXER_FP4_EHIP = -4    /* the HIP runtime reported an error */
};

/* Flags the kernels OR into the schedule buffer's error word (device-side problems),
 * and (the last two) the fused writer into its caller's error word. */
enum {
  INDEXER_FP4_DEV_BAD_PAGE = 1,      /* block-table entry outside [0, n_pages): page skipped */
  INDEXER_FP4_DEV_TABLE_SHORT = 2,   /* a row needs more pages than bt_ld: rest skipped */
  INDEXER_FP4_DEV_BAD_SCHEDULE = 4,  /* schedule built for other sizes than the call's */
  INDEXER_FP4_DEV_BAD_LENGTH = 8,    /* negative length or cu_rows not ascending */
  INDEXER_FP4_DEV_BAD_POSITION = 16, /* a rotary position outside the cos/sin table: row skipped */
  INDEXER_FP4_DEV_SLOT_OUT_OF_POOL = 32 /* a slot at or past n_pages*64: key skipped */
};

#define INDEXER_FP4_PAGE 64       /* tokens per page ([P2] review fixes: block size 64) */
#define INDEXER_FP4_HEAD_DIM 128  /* index head dimension ([P2] Scope) */
#define INDEXER_FP4_HEAD_MULT 16  /* n_heads must be a multiple of this ([P2] Scope: MFMA_M) */
#define INDEXER_FP4_MAX_HEADS 128
#define INDEXER_FP4_ROW_MULTIPLE 8 /* a prefill step's n_rows_padded is a multiple of this */
#define INDEXER_FP4_TILE_ROWS 16   /* prefill rows per tile (a row group is cut into tiles) */

/* Message of the last failed call on this host thread ("" if none). [host]
 * indexer_last_error is the same function under a shorter name. */
const char *indexer_fp4_last_error(void);
const char *indexer_last_error(void);

/* ---------------------------------------------------------------------------------
 * Cache write and query quantization ([P2] commit message: the fused writer's FP4
 * output mode stores keys as packed E2M1 plus e8m0 scales and emits the quantized
 * query with its scales; review fixes: rows whose slot is negative are skipped).
 *
 *   k_bf16        bf16 [n_tok][k_ld]; elements 0..127 of each row are the key
 *   slot_mapping  int64 [n_tok]; key t goes to page slot/64, position slot%64;
 *                 slot < 0 is skipped, and so (device-side) is slot >= n_pages*64
 *   kv_packed, kv_scale  the two planes (layout above), n_pages pages each; only the
 *                 bytes of the written keys change
 *   q_bf16        bf16 [n_q_rows][n_heads][128], or NULL (no query arm)
 *   q_packed, q_scale  outputs [n_q_rows][n_heads][64] / [n_q_rows][n_heads][4]
 * n_tok may be 0 (query arm only); n_q_rows may be 0 (key arm only).
 * Errors: EINVAL (negative sizes, k_ld < 128, n_heads <= 0 with a query arm, NULL
 * plane or output pointers that a non-empty arm needs), EARCH, EHIP.
 * --------------------------------------------------------------------------------- */
int indexer_fp4_quant_and_cache(const void *k_bf16, int64_t n_tok, int64_t k_ld,
                                const int64_t *slot_mapping, uint8_t *kv_packed,
                                uint8_t *kv_scale, int64_t n_pages, const void *q_bf16,
                                int64_t n_q_rows, int32_t n_heads, uint8_t *q_packed,
                                uint8_t *q_scale, void *stream);

/* ---------------------------------------------------------------------------------
 * Per-step schedules. The scorers run a persistent grid of n_units workgroups that
 * splits the step's work evenly: unit u takes items [floor(u*W/n), floor((u+1)*W/n))
 * of the W work items. The schedule is built once per step into a caller-owned
 * buffer that stays at a fixed address, so a captured graph that reads it can be
 * replayed for a new step after the schedule call is re-run ([P2] Decode grid floor:
 * the CTA schedule is published once a step at a graph-stable address; the pages'
 * floors are 512 units for decode and 4096 for prefill).
 *
 * Decode: rows are next_n query tokens per sequence ([P2] review fixes). A work item
 * is (sequence b, page p < ceil(context_lens[b]/64)), b-major. row_len[b*next_n + t]
 * = context_lens[b] - next_n + 1 + t (the context counts the token just written).
 *   context_lens  int32 [batch]
 *   sched         buffer of indexer_fp4_decode_sched_bytes(batch, next_n, n_units) bytes
 *   row_len       int32 [batch*next_n] output (keys each row sees)
 * Errors: EINVAL (batch < 0, next_n outside 1..4, n_units <= 0), ENOSPC (sched_bytes too
 * small: a schedule is never silently truncated, [P2] review fixes), EARCH, EHIP.
 * --------------------------------------------------------------------------------- */
int64_t indexer_fp4_decode_sched_bytes(int32_t batch, int32_t next_n, int32_t n_units);
int indexer_fp4_decode_schedule(const int32_t *context_lens, int32_t batch, int32_t next_n,
                                int32_t n_units, void *sched, int64_t sched_bytes,
                                int32_t *row_len, void *stream);

/* Prefill: the step's query rows are grouped by request: rows [cu_rows[i],
 * cu_rows[i+1]) belong to request i, and row r sits at position start_pos[i] + r -
 * cu_rows[i] and sees keys [0, position] (causal, inclusive). Rows [cu_rows[n_req],
 * n_rows_padded) are padding: they join the last request's group and see no key
 * ([P1] section 3: padding rows fold into the last request's group, sit at position 0
 * and read no key). Each group is cut into tiles of up to INDEXER_FP4_TILE_ROWS rows
 * starting at the group's first row; a work item is (tile, page), tile-major, for the
 * pages the tile's longest row reaches. The schedule also looks every item's page up in
 * the block table (request i reads its keys through block_table[i]; [P1] section 3: group
 * b -> block_tables[b]), once a step for every layer that shares the table, so the scorer
 * does not read the table; a page the table cannot give (an entry outside [0, n_pages), or
 * past bt_ld) is recorded as unreadable and flagged in the schedule's error word
 * (INDEXER_FP4_DEV_BAD_PAGE, INDEXER_FP4_DEV_TABLE_SHORT); its logits are not written.
 *   cu_rows     int32 [n_req+1], cu_rows[0] = 0, ascending, cu_rows[n_req] <= n_rows_padded
 *   start_pos   int32 [n_req]
 *   n_rows_padded [host] a multiple of INDEXER_FP4_ROW_MULTIPLE
 *   block_table int32 [n_req][bt_ld]: row i = request i of the step
 *   n_pages     pages in the cache planes the scorer will read
 *   sched       indexer_fp4_prefill_sched_bytes(n_req, n_rows_padded, n_units, bt_ld) bytes
 *   row_len     int32 [n_rows_padded] output (0 for padding rows)
 * Errors: EINVAL (n_req <= 0, n_rows_padded not a positive multiple of 8, n_units <= 0,
 * bt_ld outside 1..2^31-1, n_pages < 0), ENOSPC, EARCH, EHIP. Device-side: a descending
 * cu_rows or negative start_pos sets INDEXER_FP4_DEV_BAD_LENGTH and empties the schedule.
 * --------------------------------------------------------------------------------- */
int64_t indexer_fp4_prefill_sched_bytes(int32_t n_req, int32_t n_rows_padded, int32_t n_units, int64_t bt_ld);
int indexer_fp4_prefill_schedule(const int32_t *cu_rows, const int32_t *start_pos, int32_t n_req,
                                 int32_t n_rows_padded, int32_t n_units, const int32_t *block_table,
                                 int64_t bt_ld, int64_t n_pages, void *sched, int64_t sched_bytes,
                                 int32_t *row_len, void *stream);

/* ---------------------------------------------------------------------------------
 * Fused writer: key LayerNorm and RoPE, then the cache write and query quantization
 * above, and the scorer's weights ([P2] commit message: the widened writer emits the
 * quantized query and weights_mqa, k_norm runs before the quantizer; review fixes:
 * slot < 0 rows are skipped and their weights_mqa must be zero). The pages give no
 * formulas; these are the readings:
 *   key   LayerNorm over its 128 elements (biased variance): (x - mean) /
 *         sqrt(var + eps) * k_norm_weight + k_norm_bias (skipped if k_norm_weight is
 *         NULL; a NULL bias is zero), then RoPE;
 *   query RoPE only, per head;
 *   RoPE  rotates pairs of the first rope_dim elements: pair i is (i, i + rope_dim/2),
 *         or (2i, 2i+1) when rope_interleaved, and (a, b) becomes (a cos - b sin,
 *         b cos + a sin) with cos = cos_sin[pos][i], sin = cos_sin[pos][rope_dim/2 + i];
 *   the fp32 result is rounded once to bf16 (nearest, ties to even) and quantized as
 *   indexer_fp4_quant_and_cache quantizes bf16 input;
 *   weights_mqa[t][h] = weight_scale * weights[t][h].
 *
 *   k_bf16        bf16 [n_tok][k_ld] (first 128 used); token t's key
 *   k_norm_weight, k_norm_bias  fp32 [128] or NULL; eps >= 0
 *   positions     int64 [n_tok] (needed when rope_dim > 0)
 *   cos_sin       fp32 [max_pos][rope_dim]; rope_dim a multiple of 16 in 0..128
 *   slot_mapping, kv_packed, kv_scale, n_pages  as for indexer_fp4_quant_and_cache
 *   q_bf16        bf16 [n_tok][n_heads][128] or NULL (no query arm); token t's heads
 *   q_packed, q_scale  outputs [n_tok][n_heads][64] / [n_tok][n_heads][4]
 *   weights       fp32 [n_tok][n_heads]; weights_mqa output of the same shape
 *   all_q         0: a token with slot < 0 gets the zero query (codes 0, scale byte 0)
 *                 and weights_mqa 0; nonzero: its query and weights are computed
 *   err           int32 word or NULL: INDEXER_FP4_DEV_BAD_POSITION (position outside
 *                 [0, max_pos) with rope_dim > 0: key skipped, zero query and weights),
 *                 INDEXER_FP4_DEV_SLOT_OUT_OF_POOL (key skipped, query written)
 * Errors: EINVAL (negative sizes, rope_dim not a multiple of 16 or above 128, a bias
 * without a weight, eps < 0, k_ld < 128 or not a multiple of 8, missing or misaligned
 * pointers an arm needs), EARCH, EHIP.
 * --------------------------------------------------------------------------------- */
int indexer_fp4_norm_rope_quant_and_cache(const void *k_bf16, int64_t n_tok, int64_t k_ld,
                                          const float *k_norm_weight, const float *k_norm_bias, float eps,
                                          const int64_t *positions, const float *cos_sin, int64_t max_pos,
                                          int32_t rope_dim, int32_t rope_interleaved,
                                          const int64_t *slot_mapping, uint8_t *kv_packed, uint8_t *kv_scale,
                                          int64_t n_pages, const void *q_bf16, int32_t n_heads,
                                          uint8_t *q_packed, uint8_t *q_scale, const float *weights,
                                          float weight_scale, float *weights_mqa, int32_t all_q, int32_t *err,
                                          void *stream);

/* ---------------------------------------------------------------------------------
 * Decode scorer ([P2] commit message and PR description: the FP4 mqa-logits kernel
 * scores straight out of the paged FP4 cache on a persistent grid driven by the
 * published CTA schedule).
 *   logits[r][j] = sum_h weights[r][h] * max(0, sum_d q(r,h,d) * k(j,d)),  j < row_len[r]
 * with q and k the dequantized FP4 values; row r = b*next_n + t reads its sequence's
 * pages through block_table[b]. Columns >= row_len[r] are not written.
 *   sched, row_len  as written by indexer_fp4_decode_schedule for the same batch,
 *                   next_n and n_units (sched's error word may be updated); sched_bytes is
 *                   the buffer's size, at least indexer_fp4_decode_sched_bytes(batch,
 *                   next_n, n_units). A buffer whose header names other sizes (stale,
 *                   zeroed) is not read past its header: the call scores nothing and sets
 *                   INDEXER_FP4_DEV_BAD_SCHEDULE.
 *   row_hist        optional (NULL: none), uint32 [batch*next_n][4096], 16-byte aligned,
 *                   zero-filled before its first use: the scorer adds the histogram of
 *                   every written logit's top 12 order-key bits (layout private to the
 *                   library), which indexer_topk takes instead of building its own and
 *                   leaves zero-filled again.
 * Errors: EINVAL (n_heads not a multiple of 16 or above 128, negative sizes, misaligned
 * row_hist), ENOSPC (logits_ld < 64*bt_ld, bt_ld <= 0, sched_bytes too small), EARCH, EHIP.
 * --------------------------------------------------------------------------------- */
int indexer_fp4_score_decode(const uint8_t *q_packed, const uint8_t *q_scale,
                             const float *weights, int32_t n_heads, const uint8_t *kv_packed,
                             const uint8_t *kv_scale, int64_t n_pages,
                             const int32_t *block_table, int64_t bt_ld, int32_t batch,
                             int32_t next_n, void *sched, int64_t sched_bytes, int32_t n_units,
                             const int32_t *row_len, float *logits, int64_t logits_ld,
                             uint32_t *row_hist, void *stream);

/* ---------------------------------------------------------------------------------
 * FP8 comparator ([P2] PR description, Performance: the FP4 scorer is measured against
 * the FP8 indexer's scorer, +2.3 us, and the scan's FP4/FP8 time ratio against the byte
 * ratio). The pages give no FP8 format; these calls use OCP MXFP8: E4M3 elements (bias 7,
 * largest 448, nearest with ties to even, saturating) with one e8m0 scale per 32 elements,
 * scale exponent floor(log2 amax) - 8 clamped to [-127, 127].
 *
 * indexer_fp8_quant_and_cache: as indexer_fp4_quant_and_cache, but kv_packed is
 *   [n_pages][64][128] (element d of a key at byte d) and q_packed [n_q_rows][n_heads][128];
 *   the scale planes are laid out exactly as the FP4 ones.
 * indexer_fp8_score_decode: as indexer_fp4_score_decode over those planes (same schedule,
 *   lengths, logits, optional row histogram, errors).
 * --------------------------------------------------------------------------------- */
int indexer_fp8_quant_and_cache(const void *k_bf16, int64_t n_tok, int64_t k_ld,
                                const int64_t *slot_mapping, uint8_t *kv_packed, uint8_t *kv_scale,
                                int64_t n_pages, const void *q_bf16, int64_t n_q_rows, int32_t n_heads,
                                uint8_t *q_packed, uint8_t *q_scale, void *stream);
int indexer_fp8_score_decode(const uint8_t *q_packed, const uint8_t *q_scale, const float *weights,
                             int32_t n_heads, const uint8_t *kv_packed, const uint8_t *kv_scale,
                             int64_t n_pages, const int32_t *block_table, int64_t bt_ld,
                             int32_t batch, int32_t next_n, void *sched, int64_t sched_bytes, int32_t n_units,
                             const int32_t *row_len, float *logits, int64_t logits_ld,
                             uint32_t *row_hist, void *stream);

/* ---------------------------------------------------------------------------------
 * Write and score in one launch ([P2] PR description, Performance: the FP4 path runs
 * exactly one kernel more than the FP8 one, the fused writer; here that writer's work is
 * done by the decode scorer itself). For next_n = 1 only: the result equals
 * indexer_fp4_norm_rope_quant_and_cache on (k_bf16, q_bf16, weights) with n_tok = batch
 * followed by indexer_fp4_score_decode on its outputs: the cache planes receive the same
 * bytes at slot_mapping, and logits and row_hist the same values. The quantized query rows
 * stay inside the launch (no q_packed, q_scale or weights_mqa output).
 *   k_bf16 ... all_q   as for indexer_fp4_norm_rope_quant_and_cache, with n_tok = batch
 *                      (row b is sequence b); n_heads a multiple of 16, at most 128
 *   kv_packed ... row_hist  as for indexer_fp4_score_decode with next_n = 1; the
 *                      schedule must be built with next_n = 1
 * Each sequence's new key is written by the wave that scores the sequence's last page,
 * before it loads that page: slot_mapping[b] must be the slot of position row_len[b] - 1
 * of sequence b (its block-table page, as the decode step writes it); a key written to
 * another slot is still written but not necessarily seen by this call's scores.
 * Device flags as both: INDEXER_FP4_DEV_BAD_POSITION and _SLOT_OUT_OF_POOL (key skipped)
 * go to the schedule's error word.
 * Errors: EINVAL (n_heads, rope_dim, eps, k_ld, bias without weight, NULL or misaligned
 * pointers), ENOSPC (bt_ld, logits_ld, sched_bytes), EARCH, EHIP.
 * --------------------------------------------------------------------------------- */
int indexer_fp4_write_and_score_decode(
    const void *k_bf16, int64_t k_ld, const float *k_norm_weight, const float *k_norm_bias, float eps,
    const int64_t *positions, const float *cos_sin, int64_t max_pos, int32_t rope_dim, int32_t rope_interleaved,
    const int64_t *slot_mapping, const void *q_bf16, const float *weights, float weight_scale, int32_t all_q,
    int32_t n_heads, uint8_t *kv_packed, uint8_t *kv_scale, int64_t n_pages, const int32_t *block_table, int64_t bt_ld,
    int32_t batch, void *sched, int64_t sched_bytes, int32_t n_units, const int32_t *row_len, float *logits,
    int64_t logits_ld, uint32_t *row_hist, void *stream);

/* ---------------------------------------------------------------------------------
 * Prefill scorer ([P2] commit message: the FP4 prefill variant; [P1] section 3: the
 * row-group kernel finds a group's page table as group b -> block_tables[b], which the
 * schedule has already resolved). Same logit as decode for every valid row of the step;
 * padding rows read nothing and write nothing; items whose page the schedule marked
 * unreadable are skipped.
 *   q_packed/q_scale/weights  [n_rows_padded][n_heads]...
 *   n_pages, bt_ld, n_req, n_units, n_rows_padded  as given to the schedule call
 *   sched                     from indexer_fp4_prefill_schedule; sched_bytes its size
 *   logits                    fp32 [n_rows_padded][logits_ld], logits_ld >= 64*bt_ld
 * More than 64 heads are scored in passes of 64 heads over the same items (two launches
 * at 128 heads); the passes after the first add into the logits.
 * Errors: as decode (a header of other sizes sets INDEXER_FP4_DEV_BAD_SCHEDULE and
 * nothing is scored).
 * --------------------------------------------------------------------------------- */
int indexer_fp4_score_prefill(const uint8_t *q_packed, const uint8_t *q_scale,
                              const float *weights, int32_t n_heads, const uint8_t *kv_packed,
                              const uint8_t *kv_scale, int64_t n_pages, int64_t bt_ld, int32_t n_req,
                              void *sched, int64_t sched_bytes, int32_t n_units, int32_t n_rows_padded,
                              float *logits, int64_t logits_ld, void *stream);

/* ---------------------------------------------------------------------------------
 * Per-row top-k ([P2] review fixes: top_k_per_row bounds its scan by the row's
 * context, so the logits tail past it is never read; PR description Accuracy: a row
 * with at most index_topk keys keeps them all).
 * For row r, topk_idx[r][0 .. min(k, row_len[r])) receives the columns of the
 * min(k, row_len[r]) largest logits[r][0 .. row_len[r]), in ascending column order;
 * among equal logits the lower column is kept (-0.0 counts as equal to +0.0). The
 * rest of the row, up to k, is -1. Logits must be finite.
 *   row_len    int32 [n_rows] (e.g. a schedule's row_len output)
 *   workspace  indexer_topk_workspace_bytes(n_rows, max_len, k) bytes (0 when every
 *              row fits one workgroup: max_len <= 16384 or k >= max_len). Its contents
 *              when a call starts do not matter (a call writes every word it reads
 *              first), so one buffer serves any number of calls, of any shapes, on one
 *              stream. Calls that share it must not overlap.
 *   row_hist   optional (NULL: none): the histogram indexer_fp4_score_decode filled for
 *              exactly these logits and rows; it replaces one pass of this call and is
 *              left zero-filled. A histogram of other logits gives a meaningless (though
 *              in-bounds, -1 padded) selection.
 * Errors: EINVAL (k <= 0, n_rows < 0, max_len < 0, max_len > 2^20 with k < max_len,
 * misaligned row_hist), ENOSPC (topk_ld < k, workspace too small), EARCH, EHIP. Rows
 * longer than max_len are clamped to max_len (device-side; max_len must not exceed
 * logits_ld).
 * --------------------------------------------------------------------------------- */
int64_t indexer_topk_workspace_bytes(int32_t n_rows, int64_t max_len, int32_t k);
int indexer_topk(const float *logits, int64_t logits_ld, int32_t n_rows, const int32_t *row_len,
                 int64_t max_len, int32_t k, int32_t *topk_idx, int64_t topk_ld,
                 void *workspace, int64_t ws_bytes, uint32_t *row_hist, void *stream);

/* ---------------------------------------------------------------------------------
 * indexer_topk without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, selection and errors as indexer_topk, except that the
 * long-row workspace is a fixed array of INDEXER_TOPK_NOALLOC_SCRATCH_BYTES bytes of device
 * memory owned by the library (one copy per GPU, held until the process ends); a call
 * whose indexer_topk_workspace_bytes(n_rows, max_len, k) exceeds it returns ENOSPC
 * (e.g. 16 rows x 131072 keys need 8.7 MB and fit; 64 rows, 34.6 MB, do not). The call
 * allocates nothing. Every call on one GPU shares that GPU's array: calls that overlap on
 * one GPU (different streams, or host threads) race and give undefined selections.
 * --------------------------------------------------------------------------------- */
#define INDEXER_TOPK_NOALLOC_SCRATCH_BYTES (32ll << 20)
int indexer_topk_noalloc(const float *logits, int64_t logits_ld, int32_t n_rows, const int32_t *row_len,
                         int64_t max_len, int32_t k, int32_t *topk_idx, int64_t topk_ld, uint32_t *row_hist,
                         void *stream);

/* ---------------------------------------------------------------------------------
 * Candidate merge for context-parallel decode ([P2] DCP commit: each rank takes a local
 * top-k over its share of a sequence's pages, the ranks exchange candidates, and a merge
 * top-k reads the exchanged fp32 scores).
 * For row r, among the candidates (cand_score[r][c], cand_index[r][c]), c < n_cand, whose
 * index is >= 0 (an index < 0 is an empty slot), topk_idx[r][0 .. m) receives the indices
 * of the m = min(k, #valid) candidates with the largest score, ties to the smaller index
 * (as indexer_topk), in ascending index order; topk_idx[r][m .. k) is -1. Valid indices of
 * a row must be distinct.
 *   cand_score float [n_rows][cand_ld], cand_index int32 [n_rows][cand_ld]
 * Errors: EINVAL (k outside 1..4096, n_cand outside 0..16384, cand_ld < n_cand,
 * n_rows < 0, NULL pointers), ENOSPC (topk_ld < k), EARCH, EHIP.
 * --------------------------------------------------------------------------------- */
int indexer_topk_merge(const float *cand_score, const int32_t *cand_index, int64_t cand_ld,
                       int32_t n_rows, int32_t n_cand, int32_t k, int32_t *topk_idx,
                       int64_t topk_ld, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* INDEXER_FP4_H */
