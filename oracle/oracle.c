/*
 * oracle.c -- plain fp64 CPU oracle for the FP4 sparse-indexer scorer.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h). Deliberately slow and literal:
 * every step is written the way its definition reads, in double precision,
 * with no blocking, fusion or reordering. OpenMP only spreads independent
 * rows / keys over threads; it does not change any arithmetic.
 *
 * Readings of the pages that this file commits to (the pages leave them open):
 *   R1 scale rule: e = floor(log2(amax)) - 2 (E2M1's largest exponent is 2),
 *      clamped to [-127, 127], stored as e + 127; amax == 0 gives byte 0.
 *   R2 element rounding: nearest point of the E2M1 grid, ties to the even
 *      code, magnitudes past 6 saturate to 6; the sign bit is the input's.
 *   R3 nibble order: element 2i in the low nibble of byte i.
 *   R4 query format: q is quantized by the same MXFP4 rule per (row, head).
 *   R5 padding rows see an empty key range (they "read no key").
 *   R6 score: sum over heads of w * max(0, q.k); no other factor.
 *   R7 top-k ties: the lower column wins.
 * and, for the fused writer (the pages name k_norm, RoPE on q and k and the
 * weights_mqa output of the widened writer, but print none of their formulas):
 *   R12  k_norm is a LayerNorm over the key's 128 elements with the biased
 *       variance, (x - mean) / sqrt(var + eps) * gamma + beta; keys only, before RoPE.
 *   R13  RoPE rotates pairs of the first rope_dim elements of each key and query
 *       head; the angle table row of the token's position holds cos[0, half) then
 *       sin[0, half); pair i is (i, i + half) (half-split) or (2i, 2i + 1)
 *       (interleaved) and turns (a, b) into (a cos - b sin, b cos + a sin).
 *   R14 the normalized, rotated vectors are rounded to bf16 (nearest, ties to
 *       even) and then quantized exactly like plain bf16 writer input.
 *   R15 weights_mqa = weight_scale * weights; a row the writer skips (slot < 0
 *       unless all_q, or a position outside the table) gets zero weights and
 *       the quantization of a zero query.
 * and, for the FP8 comparator (the pages compare against an FP8 indexer but do not
 * give its format):
 *   R16 FP8 is MXFP8 [OCP MX v1.0]: E4M3 elements (bias 7, largest 448, no
 *       infinities) with one e8m0 scale per 32; scale exponent floor(log2 amax) - 8
 *       clamped to [-127, 127]; elements nearest on the E4M3 grid, ties to the even
 *       code, saturating at 448. The key cache is 128 code bytes per key in a plane
 *       like the FP4 one, and the scale plane is the FP4 scale plane.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define KEY_DIM 128     /* index head dimension (Scope: index_head_dim == 128) */
#define BLOCK_ELEMS 32  /* one e8m0 scale per 32 elements */
#define PAGE_KEYS 64    /* block size 64 */

/* E2M1 magnitudes by 3-bit code [OCP, E2M1]: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_value(int code) {
  double mag = kE2M1[code & 7];
  return (code & 8) ? -mag : mag;
}

/* e8m0: byte b stands for 2^(b - 127) [OCP, E8M0]. */
double oracle_e8m0_value(int byte) { return ldexp(1.0, (byte & 0xFF) - 127); }

/* Scale-plane slot of key position pos inside its 64-key page: the scale
 * plane stores the row axis as a 16x4 transpose, slot = (pos % 16) * 4 + pos / 16
 * ([P2] second review finding; commit "Use the index scale plane's own row
 * order when staging FP4 prefill under DCP"). */
int oracle_scale_slot(int pos) { return (pos % 16) * 4 + pos / 16; }

/* bf16 bit pattern -> double (exact: bf16 is the top half of an fp32). */
static double bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Nearest E2M1 magnitude code for a non-negative x, ties to the even code (R2).
 * Past 6 the nearest grid point is 6 itself, which is the saturation. */
static int e2m1_nearest_code(double x) {
  int best = 0;
  double best_d = fabs(x - kE2M1[0]);
  for (int c = 1; c < 8; c++) {
    double d = fabs(x - kE2M1[c]);
    if (d < best_d || (d == best_d && (c % 2) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return best;
}

/* One MX block: 32 values -> e8m0 byte + 32 E2M1 codes (R1, R2). */
static void encode_block(const double *v, uint8_t *scale, uint8_t *codes) {
  double amax = 0.0;
  for (int i = 0; i < BLOCK_ELEMS; i++)
    if (fabs(v[i]) > amax) amax = fabs(v[i]);
  int e;
  if (amax == 0.0) {
    e = -127;
  } else {
    int ex;
    frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
    e = (ex - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
  }
  *scale = (uint8_t)(e + 127);
  for (int i = 0; i < BLOCK_ELEMS; i++) {
    double x = ldexp(fabs(v[i]), -e); /* exact power-of-two rescale */
    int code = e2m1_nearest_code(x);
    if (signbit(v[i])) code |= 8;
    codes[i] = (uint8_t)code;
  }
}

int oracle_mx_encode_blocks(const uint16_t *vals, int64_t n_blocks, uint8_t *scale, uint8_t *codes) {
  if (n_blocks < 0) return -1;
  for (int64_t b = 0; b < n_blocks; b++) {
    double v[BLOCK_ELEMS];
    for (int i = 0; i < BLOCK_ELEMS; i++) v[i] = bf16_to_double(vals[b * BLOCK_ELEMS + i]);
    encode_block(v, &scale[b], &codes[b * BLOCK_ELEMS]);
  }
  return 0;
}

/* One 128-dim vector -> 64 packed bytes (R3) + 4 scale bytes (one per 32). */
static void encode_vector(const uint16_t *src, uint8_t *packed, uint8_t *scales) {
  for (int g = 0; g < KEY_DIM / BLOCK_ELEMS; g++) {
    double v[BLOCK_ELEMS];
    uint8_t codes[BLOCK_ELEMS];
    for (int i = 0; i < BLOCK_ELEMS; i++) v[i] = bf16_to_double(src[g * BLOCK_ELEMS + i]);
    encode_block(v, &scales[g], codes);
    for (int i = 0; i < BLOCK_ELEMS / 2; i++)
      packed[g * (BLOCK_ELEMS / 2) + i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
  }
}

/* Cache write ([P2] commit "Score a DSA sparse indexer in FP4": keys kept as
 * packed E2M1 plus e8m0 scales in one index region declared as two planes;
 * review fixes: the writer skips rows whose slot is negative). */
int oracle_quant_and_cache(const uint16_t *k, int64_t n_tok, int64_t k_ld, const int64_t *slot,
                           uint8_t *kv_packed, uint8_t *kv_scale, int64_t n_pages) {
  if (n_tok < 0 || k_ld < KEY_DIM || n_pages < 0) return -1;
  for (int64_t t = 0; t < n_tok; t++) {
    if (slot[t] < 0) continue;
    int64_t page = slot[t] / PAGE_KEYS;
    int pos = (int)(slot[t] % PAGE_KEYS);
    if (page >= n_pages) return -2;
    uint8_t packed[64], scales[4];
    encode_vector(&k[t * k_ld], packed, scales);
    memcpy(&kv_packed[(page * PAGE_KEYS + pos) * 64], packed, 64);
    for (int g = 0; g < 4; g++) kv_scale[(page * 4 + g) * PAGE_KEYS + oracle_scale_slot(pos)] = scales[g];
  }
  return 0;
}

/* Query quantization (R4; the FP4 writer emits q_out with q_scale). */
int oracle_quant_q(const uint16_t *q, int64_t n_rows, int32_t n_heads, uint8_t *q_packed, uint8_t *q_scale) {
  if (n_rows < 0 || n_heads <= 0) return -1;
  for (int64_t r = 0; r < n_rows; r++)
    for (int32_t h = 0; h < n_heads; h++) {
      int64_t v = r * n_heads + h;
      encode_vector(&q[v * KEY_DIM], &q_packed[v * 64], &q_scale[v * 4]);
    }
  return 0;
}

/* ---- MXFP8 (R16) ---------------------------------------------------------------- */

/* E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
 * subnormal (m/8 * 2^-6); 0x7F / 0xFF are NaN [OCP 8-bit floating point]. */
double oracle_e4m3_value(int code) {
  int e = (code >> 3) & 15, m = code & 7;
  double mag = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
  if ((code & 0x7F) == 0x7F) mag = NAN;
  return (code & 0x80) ? -mag : mag;
}

/* Nearest finite E4M3 magnitude code (0..0x7E) for x >= 0, ties to the even code;
 * past 448 the nearest point is 448, the saturation. */
static int e4m3_nearest_code(double x) {
  int best = 0;
  double best_d = fabs(x);
  for (int c = 1; c <= 0x7E; c++) {
    double d = fabs(x - oracle_e4m3_value(c));
    if (d < best_d || (d == best_d && (c % 2) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return best;
}

static void encode_block8(const double *v, uint8_t *scale, uint8_t *codes) {
  double amax = 0.0;
  for (int i = 0; i < BLOCK_ELEMS; i++)
    if (fabs(v[i]) > amax) amax = fabs(v[i]);
  int e = -127;
  if (amax > 0.0) {
    int ex;
    frexp(amax, &ex);
    e = (ex - 1) - 8; /* E4M3's largest exponent is 8 */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
  }
  *scale = (uint8_t)(e + 127);
  for (int i = 0; i < BLOCK_ELEMS; i++) {
    int code = e4m3_nearest_code(ldexp(fabs(v[i]), -e));
    if (signbit(v[i])) code |= 0x80;
    codes[i] = (uint8_t)code;
  }
}

/* One 128-dim vector -> 128 code bytes (element d at byte d) + 4 scale bytes. */
static void encode_vector8(const uint16_t *src, uint8_t *packed, uint8_t *scales) {
  for (int g = 0; g < KEY_DIM / BLOCK_ELEMS; g++) {
    double v[BLOCK_ELEMS];
    for (int i = 0; i < BLOCK_ELEMS; i++) v[i] = bf16_to_double(src[g * BLOCK_ELEMS + i]);
    encode_block8(v, &scales[g], &packed[g * BLOCK_ELEMS]);
  }
}

int oracle_mx8_encode_blocks(const uint16_t *vals, int64_t n_blocks, uint8_t *scale, uint8_t *codes) {
  if (n_blocks < 0) return -1;
  for (int64_t b = 0; b < n_blocks; b++) {
    double v[BLOCK_ELEMS];
    for (int i = 0; i < BLOCK_ELEMS; i++) v[i] = bf16_to_double(vals[b * BLOCK_ELEMS + i]);
    encode_block8(v, &scale[b], &codes[b * BLOCK_ELEMS]);
  }
  return 0;
}

int oracle_quant8_and_cache(const uint16_t *k, int64_t n_tok, int64_t k_ld, const int64_t *slot,
                            uint8_t *kv_packed, uint8_t *kv_scale, int64_t n_pages) {
  if (n_tok < 0 || k_ld < KEY_DIM || n_pages < 0) return -1;
  for (int64_t t = 0; t < n_tok; t++) {
    if (slot[t] < 0) continue;
    int64_t page = slot[t] / PAGE_KEYS;
    int pos = (int)(slot[t] % PAGE_KEYS);
    if (page >= n_pages) return -2;
    uint8_t scales[4];
    encode_vector8(&k[t * k_ld], &kv_packed[(page * PAGE_KEYS + pos) * KEY_DIM], scales);
    for (int g = 0; g < 4; g++) kv_scale[(page * 4 + g) * PAGE_KEYS + oracle_scale_slot(pos)] = scales[g];
  }
  return 0;
}

int oracle_quant8_q(const uint16_t *q, int64_t n_rows, int32_t n_heads, uint8_t *q_packed, uint8_t *q_scale) {
  if (n_rows < 0 || n_heads <= 0) return -1;
  for (int64_t v = 0; v < n_rows * n_heads; v++)
    encode_vector8(&q[v * KEY_DIM], &q_packed[v * KEY_DIM], &q_scale[v * 4]);
  return 0;
}

/* Element formats of the packed planes: 4 = MXFP4 (64 bytes a vector), 8 = MXFP8 (128). */
static int vec_bytes(int fmt) { return fmt == 8 ? KEY_DIM : KEY_DIM / 2; }

/* value of element d of a packed 128-dim vector with its 4 scale bytes */
static double element_fmt(int fmt, const uint8_t *packed, const uint8_t scales[4], int d) {
  double v;
  if (fmt == 8) {
    v = oracle_e4m3_value(packed[d]);
  } else {
    uint8_t byte = packed[d / 2];
    v = oracle_e2m1_value((d % 2 == 0) ? (byte & 0xF) : (byte >> 4));
  }
  return v * oracle_e8m0_value(scales[d / BLOCK_ELEMS]);
}

static int dequant_key_fmt(int fmt, const uint8_t *kv_packed, const uint8_t *kv_scale, int64_t n_pages,
                           int64_t page, int pos, double *out) {
  if (page < 0 || page >= n_pages || pos < 0 || pos >= PAGE_KEYS) return -1;
  uint8_t scales[4];
  for (int g = 0; g < 4; g++) scales[g] = kv_scale[(page * 4 + g) * PAGE_KEYS + oracle_scale_slot(pos)];
  const uint8_t *packed = &kv_packed[(page * PAGE_KEYS + pos) * vec_bytes(fmt)];
  for (int d = 0; d < KEY_DIM; d++) out[d] = element_fmt(fmt, packed, scales, d);
  return 0;
}

static int dequant_q_fmt(int fmt, const uint8_t *q_packed, const uint8_t *q_scale, int64_t row, int32_t n_heads,
                         int32_t h, double *out) {
  if (row < 0 || h < 0 || h >= n_heads) return -1;
  int64_t v = row * n_heads + h;
  for (int d = 0; d < KEY_DIM; d++) out[d] = element_fmt(fmt, &q_packed[v * vec_bytes(fmt)], &q_scale[v * 4], d);
  return 0;
}

int oracle_dequant8_key(const uint8_t *kv_packed, const uint8_t *kv_scale, int64_t n_pages, int64_t page, int pos,
                        double *out) {
  return dequant_key_fmt(8, kv_packed, kv_scale, n_pages, page, pos, out);
}

static double element(const uint8_t *packed, const uint8_t scales[4], int d) {
  return element_fmt(4, packed, scales, d);
}

int oracle_dequant_key(const uint8_t *kv_packed, const uint8_t *kv_scale, int64_t n_pages,
                       int64_t page, int pos, double *out) {
  if (page < 0 || page >= n_pages || pos < 0 || pos >= PAGE_KEYS) return -1;
  uint8_t scales[4];
  for (int g = 0; g < 4; g++) scales[g] = kv_scale[(page * 4 + g) * PAGE_KEYS + oracle_scale_slot(pos)];
  const uint8_t *packed = &kv_packed[(page * PAGE_KEYS + pos) * 64];
  for (int d = 0; d < KEY_DIM; d++) out[d] = element(packed, scales, d);
  return 0;
}

int oracle_dequant_q(const uint8_t *q_packed, const uint8_t *q_scale, int64_t row, int32_t n_heads,
                     int32_t h, double *out) {
  if (row < 0 || h < 0 || h >= n_heads) return -1;
  int64_t v = row * n_heads + h;
  for (int d = 0; d < KEY_DIM; d++) out[d] = element(&q_packed[v * 64], &q_scale[v * 4], d);
  return 0;
}

/* Decode rows: a sequence contributes next_n query rows; row t of them sits
 * next_n - 1 - t tokens before the end of the context ([P2] review fixes
 * name next_n rows per sequence; the staggering is the usual layout of
 * speculative rows). */
int oracle_decode_geometry(const int32_t *ctx, int32_t batch, int32_t next_n, int32_t *row_seq,
                           int32_t *row_len) {
  if (batch < 0 || next_n <= 0) return -1;
  for (int32_t b = 0; b < batch; b++)
    for (int32_t t = 0; t < next_n; t++) {
      int32_t len = ctx[b] - next_n + 1 + t;
      if (len < 0) len = 0;
      row_seq[b * next_n + t] = b;
      row_len[b * next_n + t] = len;
    }
  return 0;
}

/* Prefill rows: causal, inclusive of the row's own position. Padding rows join
 * the last request's group at position 0 and read no key ([P1] section 3). */
int oracle_prefill_geometry(const int32_t *cu_rows, const int32_t *start_pos, int32_t n_req,
                            int32_t n_rows_padded, int32_t *row_seq, int32_t *row_len) {
  if (n_req <= 0 || cu_rows[0] != 0 || n_rows_padded < cu_rows[n_req]) return -1;
  for (int32_t i = 0; i < n_req; i++) {
    if (cu_rows[i + 1] < cu_rows[i]) return -1;
    for (int32_t r = cu_rows[i]; r < cu_rows[i + 1]; r++) {
      row_seq[r] = i;
      row_len[r] = start_pos[i] + (r - cu_rows[i]) + 1;
    }
  }
  for (int32_t r = cu_rows[n_req]; r < n_rows_padded; r++) {
    row_seq[r] = n_req - 1;
    row_len[r] = 0;
  }
  return 0;
}

/* s = sum_h w[h] * max(0, sum_d q[h][d] * k[d])  (R6). */
static double score_one(const double *qd, const float *w, int32_t n_heads, const double *kd) {
  double s = 0.0;
  for (int32_t h = 0; h < n_heads; h++) {
    double dot = 0.0;
    for (int d = 0; d < KEY_DIM; d++) dot += qd[h * KEY_DIM + d] * kd[d];
    s += (double)w[h] * (dot > 0.0 ? dot : 0.0);
  }
  return s;
}

static int dequant_row_q(int fmt, const uint8_t *q_packed, const uint8_t *q_scale, int64_t r, int32_t n_heads,
                         double *qd) {
  for (int32_t h = 0; h < n_heads; h++)
    if (dequant_q_fmt(fmt, q_packed, q_scale, r, n_heads, h, &qd[h * KEY_DIM])) return -1;
  return 0;
}

static int score_fmt(int fmt, const uint8_t *q_packed, const uint8_t *q_scale, const float *w, int32_t n_heads,
                     int64_t n_rows, const int32_t *row_seq, const int32_t *row_len, const uint8_t *kv_packed,
                     const uint8_t *kv_scale, int64_t n_pages, const int32_t *block_table, int64_t bt_ld,
                     double *logits, int64_t ld, int64_t *reads);

/* Paged DSA index score ([P2] PR description: logits straight from the
 * paged FP4 cache; the page table maps a row's keys to pages). */
int oracle_score(const uint8_t *q_packed, const uint8_t *q_scale, const float *w, int32_t n_heads,
                 int64_t n_rows, const int32_t *row_seq, const int32_t *row_len,
                 const uint8_t *kv_packed, const uint8_t *kv_scale, int64_t n_pages,
                 const int32_t *block_table, int64_t bt_ld, double *logits, int64_t ld,
                 int64_t *reads) {
  return score_fmt(4, q_packed, q_scale, w, n_heads, n_rows, row_seq, row_len, kv_packed, kv_scale, n_pages,
                   block_table, bt_ld, logits, ld, reads);
}

/* The same score over MXFP8 queries and keys (R16). */
int oracle_score8(const uint8_t *q_packed, const uint8_t *q_scale, const float *w, int32_t n_heads,
                  int64_t n_rows, const int32_t *row_seq, const int32_t *row_len, const uint8_t *kv_packed,
                  const uint8_t *kv_scale, int64_t n_pages, const int32_t *block_table, int64_t bt_ld,
                  double *logits, int64_t ld, int64_t *reads) {
  return score_fmt(8, q_packed, q_scale, w, n_heads, n_rows, row_seq, row_len, kv_packed, kv_scale, n_pages,
                   block_table, bt_ld, logits, ld, reads);
}

static int score_fmt(int fmt, const uint8_t *q_packed, const uint8_t *q_scale, const float *w, int32_t n_heads,
                     int64_t n_rows, const int32_t *row_seq, const int32_t *row_len, const uint8_t *kv_packed,
                     const uint8_t *kv_scale, int64_t n_pages, const int32_t *block_table, int64_t bt_ld,
                     double *logits, int64_t ld, int64_t *reads) {
  if (n_heads <= 0 || n_rows < 0) return -1;
  double *qd = (double *)malloc(sizeof(double) * n_heads * KEY_DIM);
  if (!qd) return -3;
  int err = 0;
  for (int64_t r = 0; r < n_rows && !err; r++) {
    int64_t len = row_len[r];
    if (len > ld || (len + PAGE_KEYS - 1) / PAGE_KEYS > bt_ld) { err = -1; break; }
    if (dequant_row_q(fmt, q_packed, q_scale, r, n_heads, qd)) { err = -1; break; }
    const int32_t *bt = &block_table[(int64_t)row_seq[r] * bt_ld];
    int64_t nread = 0;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : nread) reduction(| : bad)
    for (int64_t j = 0; j < len; j++) {
      double kd[KEY_DIM];
      if (dequant_key_fmt(fmt, kv_packed, kv_scale, n_pages, bt[j / PAGE_KEYS], (int)(j % PAGE_KEYS), kd)) {
        bad = 1;
        continue;
      }
      nread += 1;
      logits[r * ld + j] = score_one(qd, &w[r * n_heads], n_heads, kd);
    }
    if (bad) err = -2;
    if (reads) reads[r] = nread;
  }
  free(qd);
  return err;
}

/* Top-k by a full sort of (score desc, column asc) (R7). The per-row scan is
 * bounded by the row's own length ([P2] review fixes: the top-k bounds its
 * scan by the context, so the logits tail is never read). */
typedef struct {
  double v;
  int32_t j;
} Cand;

static int cand_cmp(const void *a, const void *b) {
  const Cand *x = (const Cand *)a, *y = (const Cand *)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

int oracle_topk(const double *s, int64_t ld, int64_t n_rows, const int32_t *row_len, int32_t k,
                int32_t *idx, int64_t idx_ld) {
  if (k <= 0 || idx_ld < k || n_rows < 0) return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t r = 0; r < n_rows; r++) {
    int64_t len = row_len[r];
    if (len < 0 || len > ld) { bad = 1; continue; }
    Cand *c = (Cand *)malloc(sizeof(Cand) * (len > 0 ? len : 1));
    if (!c) { bad = 1; continue; }
    for (int64_t j = 0; j < len; j++) {
      c[j].v = s[r * ld + j];
      c[j].j = (int32_t)j;
    }
    qsort(c, (size_t)len, sizeof(Cand), cand_cmp);
    for (int32_t i = 0; i < k; i++) idx[r * idx_ld + i] = (i < len) ? c[i].j : -1;
    free(c);
  }
  return bad ? -1 : 0;
}

/* Candidate merge for context-parallel decode ([P2] DCP commit: each rank takes a local
 * top-k over its share of a sequence's pages, the ranks exchange candidates, and a merge
 * top-k reads the exchanged fp32 scores). For row r the candidates are
 * (score[r*ld + c], index[r*ld + c]) for c < n_cand; an index < 0 is an empty slot. The
 * result lists the indices of the min(k, #valid) candidates with the largest score, ties to
 * the smaller index (R7), in that order; entries past them are -1. */
int oracle_topk_merge(const double *score, const int32_t *index, int64_t ld, int64_t n_rows, int32_t n_cand,
                      int32_t k, int32_t *idx, int64_t idx_ld) {
  if (k <= 0 || idx_ld < k || n_rows < 0 || n_cand < 0 || ld < n_cand) return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t r = 0; r < n_rows; r++) {
    Cand *c = (Cand *)malloc(sizeof(Cand) * (n_cand > 0 ? (size_t)n_cand : 1));
    if (!c) { bad = 1; continue; }
    int32_t n = 0;
    for (int32_t j = 0; j < n_cand; j++) {
      if (index[r * ld + j] < 0) continue;
      c[n].v = score[r * ld + j];
      c[n].j = index[r * ld + j];
      n++;
    }
    qsort(c, (size_t)n, sizeof(Cand), cand_cmp);
    for (int32_t i = 0; i < k; i++) idx[r * idx_ld + i] = (i < n) ? c[i].j : -1;
    free(c);
  }
  return bad ? -1 : 0;
}

/* Even split of n_items over n_units contiguous ranges: unit u starts at
 * floor(u * n_items / n_units). (The pages publish a per-step CTA schedule
 * with a persistent grid of max(floor, rows) units -- [P2] Decode grid floor
 * -- but do not print how it divides the work; this even contiguous split is
 * the plainest reading.) */
static void even_split(int64_t n_items, int32_t n_units, int32_t *unit_begin) {
  for (int32_t u = 0; u <= n_units; u++) unit_begin[u] = (int32_t)(((int64_t)u * n_items) / n_units);
}

int oracle_decode_schedule(const int32_t *ctx, int32_t batch, int32_t n_units, int32_t *cum_pages,
                           int32_t *unit_begin, int32_t *unit_seq) {
  if (batch < 0 || n_units <= 0) return -1;
  cum_pages[0] = 0;
  for (int32_t b = 0; b < batch; b++) {
    if (ctx[b] < 0) return -1;
    cum_pages[b + 1] = cum_pages[b] + (ctx[b] + PAGE_KEYS - 1) / PAGE_KEYS;
  }
  even_split(cum_pages[batch], n_units, unit_begin);
  for (int32_t u = 0; u < n_units; u++) {
    int32_t b = 0;
    while (b < batch && cum_pages[b + 1] <= unit_begin[u]) b++;
    unit_seq[u] = b;
  }
  return 0;
}

int oracle_prefill_schedule(const int32_t *cu_rows, const int32_t *start_pos, int32_t n_req,
                            int32_t n_rows_padded, int32_t tile_rows, int32_t n_units,
                            int32_t max_tiles, int32_t *n_tiles, int32_t *tiles, int32_t *cum_items,
                            int32_t *unit_begin, int32_t *unit_tile) {
  if (n_req <= 0 || tile_rows <= 0 || n_units <= 0 || cu_rows[0] != 0 || n_rows_padded < cu_rows[n_req])
    return -1;
  int32_t nt = 0;
  cum_items[0] = 0;
  for (int32_t i = 0; i < n_req; i++) {
    int32_t first = cu_rows[i];
    int32_t valid_end = cu_rows[i + 1];
    /* the last request's group also holds the padding rows ([P1] section 3) */
    int32_t group_end = (i == n_req - 1) ? n_rows_padded : cu_rows[i + 1];
    if (valid_end < first) return -1;
    for (int32_t r0 = first; r0 < group_end; r0 += tile_rows) {
      int32_t rows = group_end - r0 < tile_rows ? group_end - r0 : tile_rows;
      int32_t pages = 0;
      for (int32_t r = r0; r < r0 + rows; r++) {
        if (r >= valid_end) continue; /* padding row: no key */
        int32_t len = start_pos[i] + (r - first) + 1;
        int32_t p = (len + PAGE_KEYS - 1) / PAGE_KEYS;
        if (p > pages) pages = p;
      }
      if (nt >= max_tiles) return -2; /* never truncate silently ([P2] review fixes) */
      tiles[4 * nt + 0] = r0;
      tiles[4 * nt + 1] = rows;
      tiles[4 * nt + 2] = i;
      tiles[4 * nt + 3] = pages;
      cum_items[nt + 1] = cum_items[nt] + pages;
      nt++;
    }
  }
  *n_tiles = nt;
  even_split(cum_items[nt], n_units, unit_begin);
  for (int32_t u = 0; u < n_units; u++) {
    int32_t t = 0;
    while (t < nt && cum_items[t + 1] <= unit_begin[u]) t++;
    unit_tile[u] = t;
  }
  return 0;
}

/* ---- fused writer ([P2] commit message and review fixes: the widened writer
 * normalizes keys with k_norm before the quantizer, applies RoPE to q and k,
 * skips slot < 0 rows and must zero weights_mqa for the rows it skips) ------- */

/* Nearest bf16 to x, ties to even (R14): bf16 keeps fp32's exponent range and 8
 * significant bits; below 2^-126 its step is 2^-133. Returns the bit pattern. */
uint16_t oracle_bf16_round(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex); /* a in [2^(ex-1), 2^ex) */
  int q = (ex - 1 >= -126) ? (ex - 1) - 7 : -133;
  double v = ldexp(rint(ldexp(a, -q)), q); /* rint: nearest, ties to even */
  if (v >= ldexp(1.0, 128)) return sign | 0x7F80;
  float f = (float)v; /* exact */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return sign | (uint16_t)(u >> 16);
}

/* R12 */
int oracle_layer_norm(const double *x, int32_t n, const float *gamma, const float *beta, float eps, double *y) {
  if (n <= 0) return -1;
  double mean = 0.0, var = 0.0;
  for (int i = 0; i < n; i++) mean += x[i];
  mean /= n;
  for (int i = 0; i < n; i++) var += (x[i] - mean) * (x[i] - mean);
  var /= n;
  double inv = 1.0 / sqrt(var + (double)eps);
  for (int i = 0; i < n; i++) y[i] = (x[i] - mean) * inv * (double)gamma[i] + (beta ? (double)beta[i] : 0.0);
  return 0;
}

/* R13, in place on x[0, rope_dim); cs is the table row {cos[half], sin[half]}. */
int oracle_rope(double *x, int32_t rope_dim, int32_t interleaved, const float *cs) {
  if (rope_dim < 0 || rope_dim % 2) return -1;
  int half = rope_dim / 2;
  for (int i = 0; i < half; i++) {
    int ia = interleaved ? 2 * i : i, ib = interleaved ? 2 * i + 1 : i + half;
    double c = cs[i], s = cs[half + i], a = x[ia], b = x[ib];
    x[ia] = a * c - b * s;
    x[ib] = b * c + a * s;
  }
  return 0;
}

static void zero_vector(uint8_t *packed, uint8_t *scales) {
  uint16_t z[KEY_DIM] = {0};
  encode_vector(z, packed, scales);
}

/* The fused writer, token by token (R12-R15). k_pre / q_pre (optional) receive
 * the fp64 vectors just before bf16 rounding (NaN for rows not computed). err
 * gets 16 for a position outside [0, max_pos) with rope_dim > 0 and 32 for a
 * slot past the pool (key skipped). */
int oracle_norm_rope_quant_and_cache(const uint16_t *k, int64_t n_tok, int64_t k_ld, const float *gamma,
                                     const float *beta, float eps, const int64_t *pos, const float *cos_sin,
                                     int64_t max_pos, int32_t rope_dim, int32_t interleaved, const int64_t *slot,
                                     uint8_t *kv_packed, uint8_t *kv_scale, int64_t n_pages, const uint16_t *q,
                                     int32_t n_heads, uint8_t *q_packed, uint8_t *q_scale, const float *weights,
                                     float weight_scale, float *weights_mqa, int32_t all_q, double *k_pre,
                                     double *q_pre, int32_t *err) {
  if (n_tok < 0 || k_ld < KEY_DIM || n_pages < 0 || rope_dim < 0 || rope_dim > KEY_DIM || rope_dim % 2) return -1;
  *err = 0;
  for (int64_t t = 0; t < n_tok; t++) {
    int bad_pos = rope_dim > 0 && (pos[t] < 0 || pos[t] >= max_pos);
    if (bad_pos) *err |= 16;
    const float *cs = bad_pos || rope_dim == 0 ? NULL : &cos_sin[pos[t] * rope_dim];
    double v[KEY_DIM];
    uint16_t bits[KEY_DIM];
    /* key */
    if (k_pre)
      for (int i = 0; i < KEY_DIM; i++) k_pre[t * KEY_DIM + i] = NAN;
    int in_pool = slot[t] >= 0 && slot[t] / PAGE_KEYS < n_pages;
    if (slot[t] >= 0 && !in_pool) *err |= 32;
    if (!bad_pos && in_pool) {
      for (int i = 0; i < KEY_DIM; i++) v[i] = bf16_to_double(k[t * k_ld + i]);
      if (gamma) oracle_layer_norm(v, KEY_DIM, gamma, beta, eps, v);
      if (cs) oracle_rope(v, rope_dim, interleaved, cs);
      for (int i = 0; i < KEY_DIM; i++) {
        if (k_pre) k_pre[t * KEY_DIM + i] = v[i];
        bits[i] = oracle_bf16_round(v[i]);
      }
      int64_t page = slot[t] / PAGE_KEYS;
      int p = (int)(slot[t] % PAGE_KEYS);
      uint8_t packed[64], scales[4];
      encode_vector(bits, packed, scales);
      memcpy(&kv_packed[(page * PAGE_KEYS + p) * 64], packed, 64);
      for (int g = 0; g < 4; g++) kv_scale[(page * 4 + g) * PAGE_KEYS + oracle_scale_slot(p)] = scales[g];
    }
    /* query heads and weights */
    if (!q) continue;
    int live = !bad_pos && (slot[t] >= 0 || all_q);
    for (int32_t h = 0; h < n_heads; h++) {
      int64_t vh = t * n_heads + h;
      if (q_pre)
        for (int i = 0; i < KEY_DIM; i++) q_pre[vh * KEY_DIM + i] = NAN;
      if (!live) {
        zero_vector(&q_packed[vh * 64], &q_scale[vh * 4]);
        weights_mqa[vh] = 0.0f;
        continue;
      }
      for (int i = 0; i < KEY_DIM; i++) v[i] = bf16_to_double(q[vh * KEY_DIM + i]);
      if (cs) oracle_rope(v, rope_dim, interleaved, cs);
      for (int i = 0; i < KEY_DIM; i++) {
        if (q_pre) q_pre[vh * KEY_DIM + i] = v[i];
        bits[i] = oracle_bf16_round(v[i]);
      }
      encode_vector(bits, &q_packed[vh * 64], &q_scale[vh * 4]);
      weights_mqa[vh] = (float)((double)weight_scale * (double)weights[vh]);
    }
  }
  return 0;
}
