/*
 * oracle.h -- plain fp64 CPU oracle for the FP4 sparse-indexer scorer.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library. The product
 * (the HIP library and its Python binding) never does, and this oracle shares
 * no code, header, table or constant with it.
 *
 * Sources (web pages, cited by title and section):
 *   [P2] "Score a DSA sparse indexer in FP4" (ROCm/ATOM pull request #2216):
 *        its commit messages, its second review finding, and the PR
 *        description sections Scope, Decode grid floor, Performance,
 *        Accuracy, Decode context parallelism and Notes.
 *   [P1] ROCm/ATOM pull request #2125 (three PCP correctness fixes),
 *        Technical Details section 3 "FP4 indexer padding rows".
 *   [OCP] OCP Microscaling Formats (MX) v1.0: the E2M1 element and E8M0
 *        scale encodings the pages name but do not spell out.
 *
 * All buffers are host memory owned by the caller. Functions return 0 on
 * success and a negative value when an argument is out of range; they never
 * read or write outside the sizes they are given.
 */
#ifndef INDEXER_ORACLE_H
#define INDEXER_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Value of a 4-bit E2M1 code (bit 3 = sign) and of an e8m0 scale byte. */
double oracle_e2m1_value(int code);
double oracle_e8m0_value(int byte);

/* Scale-plane slot of in-page key position pos (0..63). */
int oracle_scale_slot(int pos);

/* Encode n_blocks blocks of 32 bf16 values (bit patterns) each:
 * scale[b] = e8m0 byte, codes[b*32+i] = E2M1 code of element i (one per byte). */
int oracle_mx_encode_blocks(const uint16_t *vals, int64_t n_blocks, uint8_t *scale, uint8_t *codes);

/* Cache write. k is [n_tok][k_ld] bf16 (first 128 used). Token t goes to
 * page slot[t]/64, position slot[t]%64; slot[t] < 0 is skipped.
 * kv_packed is [n_pages][64][64] bytes, kv_scale is [n_pages][4][64] bytes. */
int oracle_quant_and_cache(const uint16_t *k, int64_t n_tok, int64_t k_ld, const int64_t *slot,
                           uint8_t *kv_packed, uint8_t *kv_scale, int64_t n_pages);

/* Query quantization: q [n_rows][n_heads][128] bf16 ->
 * q_packed [n_rows][n_heads][64], q_scale [n_rows][n_heads][4]. */
int oracle_quant_q(const uint16_t *q, int64_t n_rows, int32_t n_heads, uint8_t *q_packed, uint8_t *q_scale);

/* Dequantize one cached key (page, pos) or one query head into out[128]. */
int oracle_dequant_key(const uint8_t *kv_packed, const uint8_t *kv_scale, int64_t n_pages,
                       int64_t page, int pos, double *out);
int oracle_dequant_q(const uint8_t *q_packed, const uint8_t *q_scale, int64_t row, int32_t n_heads,
                     int32_t h, double *out);

/* Row geometry. Decode: row r = b*next_n + t of sequence b, sees
 * ctx[b] - next_n + 1 + t keys. Prefill: row r of request i sits at position
 * start_pos[i] + r - cu_rows[i] and sees keys [0, position]; padding rows
 * [cu_rows[n_req], n_rows_padded) belong to request n_req-1 and see none. */
int oracle_decode_geometry(const int32_t *ctx, int32_t batch, int32_t next_n, int32_t *row_seq,
                           int32_t *row_len);
int oracle_prefill_geometry(const int32_t *cu_rows, const int32_t *start_pos, int32_t n_req,
                            int32_t n_rows_padded, int32_t *row_seq, int32_t *row_len);

/* Index scores, fp64: logits[r*ld + j] for j < row_len[r] (other entries are
 * not touched). Key j of row r is read from page block_table[row_seq[r]*bt_ld
 * + j/64] at position j%64. reads (optional, [n_rows]) counts keys read. */
int oracle_score(const uint8_t *q_packed, const uint8_t *q_scale, const float *w, int32_t n_heads,
                 int64_t n_rows, const int32_t *row_seq, const int32_t *row_len,
                 const uint8_t *kv_packed, const uint8_t *kv_scale, int64_t n_pages,
                 const int32_t *block_table, int64_t bt_ld, double *logits, int64_t ld,
                 int64_t *reads);

/* Top-k by full sort: idx[r*idx_ld + i], i < k, holds the column of the i-th
 * largest s[r][j] over j < row_len[r], ties broken by lower column; entries past
 * min(k, row_len[r]) are -1. */
int oracle_topk(const double *s, int64_t ld, int64_t n_rows, const int32_t *row_len, int32_t k,
                int32_t *idx, int64_t idx_ld);

/* Candidate merge: among the candidates (score[r*ld + c], index[r*ld + c]), c < n_cand, whose
 * index is >= 0, idx[r*idx_ld + i], i < k, holds the index of the i-th largest score, ties to
 * the smaller index; entries past the valid candidates are -1. */
int oracle_topk_merge(const double *score, const int32_t *index, int64_t ld, int64_t n_rows, int32_t n_cand,
                      int32_t k, int32_t *idx, int64_t idx_ld);

/* Decode work split: items are (sequence b, page p < ceil(ctx[b]/64)) in
 * b-major order, cum_pages[b] = first item of b (B+1 entries). Unit u covers
 * items [unit_begin[u], unit_begin[u+1]) with unit_begin[u] = floor(u*W/U);
 * unit_seq[u] = sequence that holds item unit_begin[u] (batch if none). */
int oracle_decode_schedule(const int32_t *ctx, int32_t batch, int32_t n_units, int32_t *cum_pages,
                           int32_t *unit_begin, int32_t *unit_seq);

/* Prefill work split: tiles of at most tile_rows rows that stay inside one
 * request's group and start at the group's first row (the last group runs to
 * n_rows_padded). tiles[4*t..] = {first row, rows, request, pages}; items are
 * (tile, page) in tile-major order, cum_items[t] = first item of tile t
 * (n_tiles+1 entries); units split items as in decode; unit_tile[u] = tile
 * holding item unit_begin[u] (n_tiles if none). max_tiles bounds the output. */
int oracle_prefill_schedule(const int32_t *cu_rows, const int32_t *start_pos, int32_t n_req,
                            int32_t n_rows_padded, int32_t tile_rows, int32_t n_units,
                            int32_t max_tiles, int32_t *n_tiles, int32_t *tiles, int32_t *cum_items,
                            int32_t *unit_begin, int32_t *unit_tile);

/* MXFP8 comparator (reading R16 in oracle.c): E4M3 value of a code; blocks of 32
 * bf16 values -> e8m0 byte + 32 codes; cache write (kv_packed [n_pages][64][128]) and
 * query quantization (q_packed [n_rows][n_heads][128]) with the FP4 scale layout;
 * one dequantized key; the paged score as oracle_score. */
double oracle_e4m3_value(int code);
int oracle_mx8_encode_blocks(const uint16_t *vals, int64_t n_blocks, uint8_t *scale, uint8_t *codes);
int oracle_quant8_and_cache(const uint16_t *k, int64_t n_tok, int64_t k_ld, const int64_t *slot,
                            uint8_t *kv_packed, uint8_t *kv_scale, int64_t n_pages);
int oracle_quant8_q(const uint16_t *q, int64_t n_rows, int32_t n_heads, uint8_t *q_packed, uint8_t *q_scale);
int oracle_dequant8_key(const uint8_t *kv_packed, const uint8_t *kv_scale, int64_t n_pages, int64_t page, int pos,
                        double *out);
int oracle_score8(const uint8_t *q_packed, const uint8_t *q_scale, const float *w, int32_t n_heads,
                  int64_t n_rows, const int32_t *row_seq, const int32_t *row_len, const uint8_t *kv_packed,
                  const uint8_t *kv_scale, int64_t n_pages, const int32_t *block_table, int64_t bt_ld,
                  double *logits, int64_t ld, int64_t *reads);

/* Fused writer pieces and composition (readings R12-R15 in oracle.c). */
uint16_t oracle_bf16_round(double x);
int oracle_layer_norm(const double *x, int32_t n, const float *gamma, const float *beta, float eps, double *y);
int oracle_rope(double *x, int32_t rope_dim, int32_t interleaved, const float *cs);
int oracle_norm_rope_quant_and_cache(const uint16_t *k, int64_t n_tok, int64_t k_ld, const float *gamma,
                                     const float *beta, float eps, const int64_t *pos, const float *cos_sin,
                                     int64_t max_pos, int32_t rope_dim, int32_t interleaved, const int64_t *slot,
                                     uint8_t *kv_packed, uint8_t *kv_scale, int64_t n_pages, const uint16_t *q,
                                     int32_t n_heads, uint8_t *q_packed, uint8_t *q_scale, const float *weights,
                                     float weight_scale, float *weights_mqa, int32_t all_q, double *k_pre,
                                     double *q_pre, int32_t *err);

#ifdef __cplusplus
}
#endif
#endif
