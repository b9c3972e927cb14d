/*
 * kvq_oracle.c -- plain, slow CPU oracle for the INT8 paged decode-attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py may load this library.  It shares no code, header, table or constant
 * with the HIP library under decode_attention_quantized_amd/csrc; neither includes or
 * links the other.
 *
 * What it computes, and the passages it follows:
 *   - quantize-on-write (oracle_quantize_group, oracle_kv_write_int8):
 *       "Making a ternary reasoning model fast in vLLM" (half-the-memory page), section
 *       "Is 8 bits enough?": llama.cpp's Q8_0 cache format keeps one scale per 32 values;
 *       gllm page, section "Quantization Design": symmetric, scale = amax/127, round to
 *       nearest, clamp to [-127, 127], dynamic per token, no calibration;
 *       NVFP4 page, section "Writing and reading the packed cache": the writer takes BF16
 *       values plus a token->slot map, computes group maxima, then scales, then codes;
 *       invalid slots do not write.
 *     Arithmetic is IEEE fp32 (no contraction, no flush to zero), the scale is rounded
 *     to fp16 (ties to even) after saturating at 65504, and codes are computed against
 *     the stored fp16 scale with ties to even.
 *   - attention (oracle_decode): the plain definition softmax(q.K^T / sqrt(D)) V over the
 *     dequantized cache, in fp64, per sequence and query head, with GQA head mapping
 *     kv_head = q_head / (Hq / Hkv).  Half-the-memory page, section "Read the compressed
 *     cache without copying it first" (attend straight from the quantized values, V
 *     dequantized); NVFP4 page, section "Testing the cache without loading the model"
 *     (compare with an independent CPU calculation over decoded cache values).
 *   - split/merge (oracle_decode_split): the flash-decoding algorithm of the
 *     long-context page, section "Give more GPU workers a piece of the attention
 *     calculation": cut the context into segments, keep for each a weighted value sum and
 *     its normalisation terms, and combine with those terms (never by averaging).
 *
 *   - the per-head format (oracle_quantize_row_f32, oracle_kv_write_int8_head): the
 *     half-the-memory page, sections on vLLM's int8_per_token_head format and "Is 8 bits
 *     enough?": every value of a (token, head) row as an 8-bit integer with one shared 32-bit
 *     scale, 520 bytes per token per head at D = 256 (one scale per 256 values); the same
 *     symmetric amax/127 rule, with the scale kept in fp32.
 *
 * Cache images here use the LOGICAL layout (the GPU library stores the same bytes in a
 * permuted in-page order):
 *     codes  int8  [num_blocks][Hkv][16][D]
 *     scales fp16  [num_blocks][Hkv][16][D/32]   (raw IEEE binary16 bits)
 *     per-head scales fp32 [num_blocks][Hkv][16]
 *     bf16 cache   [num_blocks][Hkv][16][D]      (raw bfloat16 bits)
 * Token t of sequence s lives in slot block_tables[s][t/16]*16 + t%16.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PAGE 16
#define GROUP 32
#define ORACLE_MAX_D 256      /* head_dim limit of the stack buffers below */
#define ORACLE_MAX_SPLITS 4096

/* ---------------------------------------------------------------- number formats */

/* bfloat16 -> fp32: the 16 stored bits are the top half of an IEEE single. */
float oracle_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* IEEE binary16 bits -> fp32 (exact). */
float oracle_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t exp = (h >> 10) & 0x1Fu;
  uint32_t man = h & 0x3FFu;
  float mag;
  if (exp == 0) {
    mag = ldexpf((float)man, -24); /* zero or subnormal: man * 2^-24 */
  } else if (exp == 31) {
    mag = man ? NAN : INFINITY;
  } else {
    mag = ldexpf((float)(man | 0x400u), (int)exp - 25); /* (1024+man) * 2^(e-15-10) */
  }
  uint32_t u;
  memcpy(&u, &mag, 4);
  u |= sign;
  memcpy(&mag, &u, 4);
  return mag;
}

/* fp32 -> IEEE binary16 bits, round to nearest, ties to even; overflow gives infinity,
 * results below the normal range become subnormals (no flush to zero). */
uint16_t oracle_f32_to_f16(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) { /* inf or nan */
    if (ax == 0x7F800000u) return sign | 0x7C00u;
    return sign | 0x7E00u;
  }
  uint32_t efield = ax >> 23;
  if (efield == 0) return sign; /* fp32 subnormal: far below half the smallest fp16 subnormal */
  int e = (int)efield - 127;    /* unbiased exponent */
  uint32_t man = ax & 0x7FFFFFu;
  if (e > 15) return sign | 0x7C00u;
  if (e >= -14) { /* normal binary16 exponent range; rounding may carry into the exponent */
    uint32_t h = ((uint32_t)(e + 15) << 10) | (man >> 13);
    uint32_t rem = man & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;
    return sign | (uint16_t)h;
  }
  /* below 2^-14: result = round(|f| / 2^-24); |f| = m24 * 2^(e-23), so shift by -(e+1) */
  uint32_t m24 = man | 0x800000u;
  int sh = -(e + 1); /* >= 14 */
  if (sh > 31) return sign;
  uint32_t q = m24 >> sh;
  uint32_t rem = m24 & ((1u << sh) - 1u);
  uint32_t half = 1u << (sh - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1u;
  return sign | (uint16_t)q;
}

/* ---------------------------------------------------------------- quantizer */

/*
 * Quantize one group of n (= 32) bf16 values: amax, fp16 scale, int8 codes.
 * Steps, all fp32: x = float(bf16) (exact); amax = max |x|; d = amax / 127 (correctly
 * rounded division); s = fp16(min(d, 65504)) with ties to even -- the stored scale;
 * if s == 0 every code is 0, else q = clamp(rint(x / s), -127, 127) with the division
 * against the stored scale and rint rounding ties to even.
 */
void oracle_quantize_group(const uint16_t *xb, int n, int8_t *codes, uint16_t *scale_out) {
  float x[GROUP];
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    x[i] = oracle_bf16_to_f32(xb[i]);
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float d = amax / 127.0f;
  if (d > 65504.0f) d = 65504.0f;
  uint16_t s16 = oracle_f32_to_f16(d);
  float s = oracle_f16_to_f32(s16);
  *scale_out = s16;
  for (int i = 0; i < n; ++i) {
    if (s == 0.0f) {
      codes[i] = 0;
      continue;
    }
    float r = rintf(x[i] / s);
    if (r != r) r = 0.0f; /* non-finite input: caller error, keep it defined */
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    codes[i] = (int8_t)r;
  }
}

/*
 * Quantize-on-write.  k, v: bf16 [T][Hkv][D].  slot_mapping[t] < 0: token t is not written.
 * Every (slot, head) that is written gets all D codes and D/32 scales of K and of V; no
 * other byte of the cache is touched.  Valid slots are unique within one call.
 */
void oracle_kv_write_int8(int T, int Hkv, int D, int num_blocks, const uint16_t *k, const uint16_t *v,
                          const int32_t *slot_mapping, int8_t *k_codes, int8_t *v_codes, uint16_t *k_scales,
                          uint16_t *v_scales) {
  int ng = D / GROUP;
  for (int t = 0; t < T; ++t) {
    int32_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_blocks * PAGE) continue;
    int64_t blk = slot / PAGE, off = slot % PAGE;
    for (int h = 0; h < Hkv; ++h) {
      int64_t row = (blk * Hkv + h) * PAGE + off; /* (block, head, offset) */
      const uint16_t *kt = k + ((int64_t)t * Hkv + h) * D;
      const uint16_t *vt = v + ((int64_t)t * Hkv + h) * D;
      for (int g = 0; g < ng; ++g) {
        oracle_quantize_group(kt + g * GROUP, GROUP, k_codes + row * D + g * GROUP, k_scales + row * ng + g);
        oracle_quantize_group(vt + g * GROUP, GROUP, v_codes + row * D + g * GROUP, v_scales + row * ng + g);
      }
    }
  }
}

/*
 * Per-head format: quantize one (token, head) row of n (= D) bf16 values with one fp32 scale.
 * x = float(bf16) (exact); amax = max |x|; s = amax / 127 (correctly rounded fp32 division),
 * stored as is; if s == 0 every code is 0, else q = clamp(rint(x / s), -127, 127), ties to
 * even.
 */
void oracle_quantize_row_f32(const uint16_t *xb, int n, int8_t *codes, float *scale_out) {
  float x[ORACLE_MAX_D];
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    x[i] = oracle_bf16_to_f32(xb[i]);
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float s = amax / 127.0f;
  *scale_out = s;
  for (int i = 0; i < n; ++i) {
    if (s == 0.0f) {
      codes[i] = 0;
      continue;
    }
    float r = rintf(x[i] / s);
    if (r != r) r = 0.0f;
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    codes[i] = (int8_t)r;
  }
}

/* Quantize-on-write into the per-head format: scales fp32 [num_blocks][Hkv][16]. */
void oracle_kv_write_int8_head(int T, int Hkv, int D, int num_blocks, const uint16_t *k, const uint16_t *v,
                               const int32_t *slot_mapping, int8_t *k_codes, int8_t *v_codes, float *k_scales,
                               float *v_scales) {
  for (int t = 0; t < T; ++t) {
    int32_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_blocks * PAGE) continue;
    int64_t blk = slot / PAGE, off = slot % PAGE;
    for (int h = 0; h < Hkv; ++h) {
      int64_t row = (blk * Hkv + h) * PAGE + off;
      oracle_quantize_row_f32(k + ((int64_t)t * Hkv + h) * D, D, k_codes + row * D, k_scales + row);
      oracle_quantize_row_f32(v + ((int64_t)t * Hkv + h) * D, D, v_codes + row * D, v_scales + row);
    }
  }
}

/* BF16 cache variant: the write is a scatter copy of the bf16 bits. */
void oracle_kv_write_bf16(int T, int Hkv, int D, int num_blocks, const uint16_t *k, const uint16_t *v,
                          const int32_t *slot_mapping, uint16_t *k_cache, uint16_t *v_cache) {
  for (int t = 0; t < T; ++t) {
    int32_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_blocks * PAGE) continue;
    int64_t blk = slot / PAGE, off = slot % PAGE;
    for (int h = 0; h < Hkv; ++h) {
      int64_t row = (blk * Hkv + h) * PAGE + off;
      memcpy(k_cache + row * D, k + ((int64_t)t * Hkv + h) * D, (size_t)D * 2);
      memcpy(v_cache + row * D, v + ((int64_t)t * Hkv + h) * D, (size_t)D * 2);
    }
  }
}

/* ---------------------------------------------------------------- cache reads */

typedef struct {
  int dtype; /* 0: int8 codes + fp16 scales, 1: bf16, 2: int8 codes + one fp32 scale per row */
  int Hkv, D, num_blocks;
  const int8_t *k_codes, *v_codes;
  const uint16_t *k_scales, *v_scales;
  const uint16_t *k_bf16, *v_bf16;
  const float *k_row_scales, *v_row_scales;
} cache_view;

/* Decoded K (which = 0) or V (which = 1) row of token t of sequence s, head h, in fp64.
 * INT8: value = code * scale (exact in fp64).  BF16: the stored value. */
static void read_row(const cache_view *c, const int32_t *bt_row, int t, int h, int which, double *dst) {
  int64_t blk = bt_row[t / PAGE];
  int64_t row = (blk * c->Hkv + h) * PAGE + t % PAGE;
  int D = c->D;
  if (c->dtype == 0) {
    const int8_t *codes = (which ? c->v_codes : c->k_codes) + row * D;
    const uint16_t *sc = (which ? c->v_scales : c->k_scales) + row * (D / GROUP);
    for (int i = 0; i < D; ++i) dst[i] = (double)codes[i] * (double)oracle_f16_to_f32(sc[i / GROUP]);
  } else if (c->dtype == 2) {
    const int8_t *codes = (which ? c->v_codes : c->k_codes) + row * D;
    double sc = (double)(which ? c->v_row_scales : c->k_row_scales)[row];
    for (int i = 0; i < D; ++i) dst[i] = (double)codes[i] * sc; /* exact: 8 + 24 significant bits */
  } else {
    const uint16_t *vals = (which ? c->v_bf16 : c->k_bf16) + row * D;
    for (int i = 0; i < D; ++i) dst[i] = (double)oracle_bf16_to_f32(vals[i]);
  }
}

/* Score of token t for query row qd: z = (q . k) / sqrt(D). */
static double score(const cache_view *c, const int32_t *bt_row, int t, int h, const double *qd, double *tmp) {
  read_row(c, bt_row, t, h, 0, tmp);
  double acc = 0.0;
  for (int i = 0; i < c->D; ++i) acc += qd[i] * tmp[i];
  return acc / sqrt((double)c->D);
}

/* The plain definition for one (sequence, query head): out = sum_t e^(z_t-M) V_t / sum_t e^(z_t-M),
 * lse = M + ln sum_t e^(z_t-M).  An empty context gives out = 0 and lse = -inf. */
static void attend_row(const cache_view *c, const int32_t *bt_row, int L, int h, const uint16_t *q_row,
                       double *out, double *lse) {
  int D = c->D;
  double qd[ORACLE_MAX_D], tmp[ORACLE_MAX_D];
  for (int i = 0; i < D; ++i) qd[i] = (double)oracle_bf16_to_f32(q_row[i]);
  for (int i = 0; i < D; ++i) out[i] = 0.0;
  if (L <= 0) {
    *lse = -INFINITY;
    return;
  }
  double M = -INFINITY;
  for (int t = 0; t < L; ++t) {
    double z = score(c, bt_row, t, h, qd, tmp);
    if (z > M) M = z;
  }
  double den = 0.0;
  for (int t = 0; t < L; ++t) {
    double w = exp(score(c, bt_row, t, h, qd, tmp) - M);
    den += w;
    read_row(c, bt_row, t, h, 1, tmp);
    for (int i = 0; i < D; ++i) out[i] += w * tmp[i];
  }
  for (int i = 0; i < D; ++i) out[i] /= den;
  *lse = M + log(den);
}

/*
 * The flash-decoding algorithm for one (sequence, query head).  Pages are cut into
 * contiguous chunks of cpp = ceil(max_pages / num_splits) pages, max_pages =
 * ceil(max_context_len / 16).  Split j keeps m_j = max z, l_j = sum e^(z-m_j) and
 * o_j = sum e^(z-m_j) V over its tokens; an empty split has m_j = -inf, l_j = 0 and is
 * left out of the merge.  Merge: M = max_j m_j, w_j = e^(m_j - M),
 * out = sum_j w_j o_j / sum_j w_j l_j, lse = M + ln sum_j w_j l_j.
 */
static void attend_row_split(const cache_view *c, const int32_t *bt_row, int L, int h, const uint16_t *q_row,
                             int num_splits, int max_context_len, double *out, double *lse) {
  int D = c->D;
  double qd[ORACLE_MAX_D], tmp[ORACLE_MAX_D], o_j[ORACLE_MAX_D];
  for (int i = 0; i < D; ++i) qd[i] = (double)oracle_bf16_to_f32(q_row[i]);
  for (int i = 0; i < D; ++i) out[i] = 0.0;
  if (L <= 0) {
    *lse = -INFINITY;
    return;
  }
  int max_pages = (max_context_len + PAGE - 1) / PAGE;
  int cpp = (max_pages + num_splits - 1) / num_splits;
  /* pass 1: the merge maximum over non-empty splits */
  double M = -INFINITY;
  double m_j_store[ORACLE_MAX_SPLITS];
  for (int j = 0; j < num_splits; ++j) {
    int t0 = j * cpp * PAGE, t1 = (j + 1) * cpp * PAGE;
    if (t1 > L) t1 = L;
    m_j_store[j] = -INFINITY;
    if (t0 >= t1) continue;
    double m = -INFINITY;
    for (int t = t0; t < t1; ++t) {
      double z = score(c, bt_row, t, h, qd, tmp);
      if (z > m) m = z;
    }
    m_j_store[j] = m;
    if (m > M) M = m;
  }
  /* pass 2: each split's partial, weighted into the merge */
  double den = 0.0;
  for (int j = 0; j < num_splits; ++j) {
    int t0 = j * cpp * PAGE, t1 = (j + 1) * cpp * PAGE;
    if (t1 > L) t1 = L;
    if (t0 >= t1) continue;
    double m = m_j_store[j], l = 0.0;
    for (int i = 0; i < D; ++i) o_j[i] = 0.0;
    for (int t = t0; t < t1; ++t) {
      double p = exp(score(c, bt_row, t, h, qd, tmp) - m);
      l += p;
      read_row(c, bt_row, t, h, 1, tmp);
      for (int i = 0; i < D; ++i) o_j[i] += p * tmp[i];
    }
    double w = exp(m - M);
    den += w * l;
    for (int i = 0; i < D; ++i) out[i] += w * o_j[i];
  }
  for (int i = 0; i < D; ++i) out[i] /= den;
  *lse = M + log(den);
}

/*
 * Decode attention for a list of (sequence, query head) rows.
 *   q            bf16 [S][Hq][D]
 *   block_tables int32 [S][max_blocks]
 *   context_lens int32 [S]
 *   rows         flat indices s*Hq + hq to compute (NULL: all S*Hq in order), n_rows of them
 *   out          fp64 [n_rows][D], lse fp64 [n_rows]
 *   num_splits   0: the plain definition; > 0: the split/merge algorithm with that many splits
 * Parallel over rows with OpenMP; each row is computed independently in a fixed order, so
 * the result does not depend on the thread count.
 */
static void decode_rows(const cache_view *c, int S, int Hq, int max_blocks, const uint16_t *q,
                        const int32_t *block_tables, const int32_t *context_lens, const int64_t *rows, int64_t n_rows,
                        int num_splits, int max_context_len, double *out, double *lse) {
  int G = Hq / c->Hkv;
  int64_t n = rows ? n_rows : (int64_t)S * Hq;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n; ++r) {
    int64_t flat = rows ? rows[r] : r;
    int s = (int)(flat / Hq), hq = (int)(flat % Hq);
    const int32_t *bt_row = block_tables + (int64_t)s * max_blocks;
    const uint16_t *q_row = q + flat * c->D;
    if (num_splits > 0)
      attend_row_split(c, bt_row, context_lens[s], hq / G, q_row, num_splits, max_context_len, out + r * c->D,
                       lse + r);
    else
      attend_row(c, bt_row, context_lens[s], hq / G, q_row, out + r * c->D, lse + r);
  }
}

void oracle_decode_int8(int S, int Hq, int Hkv, int D, int num_blocks, int max_blocks, const uint16_t *q,
                        const int32_t *block_tables, const int32_t *context_lens, const int8_t *k_codes,
                        const int8_t *v_codes, const uint16_t *k_scales, const uint16_t *v_scales, const int64_t *rows,
                        int64_t n_rows, int num_splits, int max_context_len, double *out, double *lse) {
  cache_view c = {0, Hkv, D, num_blocks, k_codes, v_codes, k_scales, v_scales, 0, 0, 0, 0};
  decode_rows(&c, S, Hq, max_blocks, q, block_tables, context_lens, rows, n_rows, num_splits, max_context_len, out,
              lse);
}

void oracle_decode_bf16(int S, int Hq, int Hkv, int D, int num_blocks, int max_blocks, const uint16_t *q,
                        const int32_t *block_tables, const int32_t *context_lens, const uint16_t *k_cache,
                        const uint16_t *v_cache, const int64_t *rows, int64_t n_rows, int num_splits,
                        int max_context_len, double *out, double *lse) {
  cache_view c = {1, Hkv, D, num_blocks, 0, 0, 0, 0, k_cache, v_cache, 0, 0};
  decode_rows(&c, S, Hq, max_blocks, q, block_tables, context_lens, rows, n_rows, num_splits, max_context_len, out,
              lse);
}

void oracle_decode_int8_head(int S, int Hq, int Hkv, int D, int num_blocks, int max_blocks, const uint16_t *q,
                             const int32_t *block_tables, const int32_t *context_lens, const int8_t *k_codes,
                             const int8_t *v_codes, const float *k_scales, const float *v_scales, const int64_t *rows,
                             int64_t n_rows, int num_splits, int max_context_len, double *out, double *lse) {
  cache_view c = {2, Hkv, D, num_blocks, k_codes, v_codes, 0, 0, 0, 0, k_scales, v_scales};
  decode_rows(&c, S, Hq, max_blocks, q, block_tables, context_lens, rows, n_rows, num_splits, max_context_len, out,
              lse);
}

/* Array forms of the scalar routines above, for tests. */
void oracle_f32_to_f16_array(const float *x, uint16_t *h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = oracle_f32_to_f16(x[i]);
}

void oracle_f16_to_f32_array(const uint16_t *h, float *x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = oracle_f16_to_f32(h[i]);
}

/* ngroups consecutive groups of 32 bf16 values -> 32 codes and one scale each. */
void oracle_quantize_groups(const uint16_t *x, int64_t ngroups, int8_t *codes, uint16_t *scales) {
  for (int64_t g = 0; g < ngroups; ++g) oracle_quantize_group(x + g * GROUP, GROUP, codes + g * GROUP, scales + g);
}

/* nrows consecutive rows of n bf16 values -> n codes and one fp32 scale each (per-head format). */
void oracle_quantize_rows_f32(const uint16_t *x, int64_t nrows, int n, int8_t *codes, float *scales) {
  for (int64_t r = 0; r < nrows; ++r) oracle_quantize_row_f32(x + r * n, n, codes + r * n, scales + r);
}

/* Thread count OpenMP will use (for reporting), and a way to change it (timing at one thread). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_num_threads(int n) { (void)n; }
#endif
