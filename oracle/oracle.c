/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for paged-KV GQA
 * attention (incremental prefill, initial prefill, decode) and for the
 * kv_append scatter.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The product path
 * (libpagedattn.so and its Python binding) never calls it, links it or shares
 * a line of code with it.
 *
 * Everything is computed in IEEE double precision, one output at a time, in
 * the order the definition states: gather the cached keys through the block
 * table, full logit row, max, exp, sum, weighted sum of values.  No tiling,
 * no online softmax, no blocking, no fused steps.  OpenMP only distributes
 * independent (row, head) outputs over threads; it does not change the order
 * of any sum.
 *
 * Pages cited (title, then section):
 *   [Agentic] "vLLM Agentic 推理｜面向 Agent 负载的推理优化"
 *   [AMPD]    "ICML'26 | AMPD：PD 分离遇上多轮推理，incremental prefill 到底该在哪跑"
 *   [V1Sched] "vLLM/V1 推理调度器"
 *   [V41]     "vLLM 优化 DeepSeek-V4.1-Flash：智能体吞吐提升 5 倍"
 *
 * Readings where the pages are silent (they never write the attention
 * formula, the cache layout or the fp8 format):
 *   - attention is scaled dot-product softmax attention with a causal mask
 *     whose boundary is inclusive: the query at absolute position p sees keys
 *     0..p (its own key was appended before attention, [Agentic] §5.2: the
 *     first kernel writes KV, the second attends);
 *   - query head h reads KV head h / (Hq / Hkv) (contiguous GQA groups;
 *     [Agentic] §4.3.1 says only that GQA has few KV heads);
 *   - cache layout [num_blocks][Hkv][block_size][head_dim];
 *   - fp8 is OCP E4M3 ("e4m3fn": bias 7, no infinities, 0x7F/0xFF NaN,
 *     largest finite 448) with one fp32 scale per (physical block, KV head),
 *     separate for K and V, value = decode(code) * scale.  Encoding rounds
 *     x / scale (fp32 division, correctly rounded) to nearest-even and
 *     saturates to +-448.
 *   - 4-bit KV ([V41] kernels section: an FP4 KV cache, about half the bytes
 *     of FP8) is OCP MXFP4: E2M1 elements (1 sign, 2 exponent bits with bias
 *     1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) sharing one
 *     E8M0 scale (2^(byte - 127), byte 255 = NaN) per 32 consecutive head_dim
 *     elements of one token and KV head.  Encoding a group: its shared
 *     exponent is floor(log2(amax)) - 2 (2 = the largest E2M1 exponent),
 *     clamped to [-127, 127] (amax = 0 gives -127); each element x / 2^that
 *     rounds to the nearest E2M1 value, ties to the even mantissa, and
 *     saturates to +-6; the sign bit is x's.  A group holding a NaN or an
 *     infinity gets the NaN scale and zero codes.
 *
 * Parity pins for every function here live in tests/test_oracle_*.py.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Block count.  [V1Sched] 源码片段 "KVCacheManager.allocate_slots — 块容量":
 * the number of blocks a request needs is the token count divided by the
 * block size, rounded up. */
int64_t orc_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t orc_num_blocks(int64_t ctx, int32_t block_size) {
  if (ctx <= 0) return 0;
  return orc_cdiv(ctx, (int64_t)block_size);
}

/* ------------------------------------------------------------------ */
/* Element decoding. */

/* bfloat16 is the upper half of an IEEE binary32; widening is exact. */
double orc_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP 8-bit floating point, E4M3 variant: 1 sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9;
 * S.1111.111 is NaN; there are no infinities. */
double orc_e4m3_to_double(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* Round a binary32 value to E4M3 with round-half-to-even, saturating every
 * finite or infinite magnitude above 448 to 448.  NaN maps to 0x7F with the
 * input's sign.  The rounding itself is done by nearbyint() in the default
 * round-to-nearest-even mode on a value scaled exactly by a power of two. */
uint8_t orc_e4m3_from_float(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  /* Below the smallest normal 2^-6 the grid is m * 2^-9, m = 0..8 (m = 8 is
   * the smallest normal, whose code is also 8). */
  if (a < ldexp(1.0, -6)) {
    double q = nearbyint(ldexp(a, 9));
    return (uint8_t)(sign | (uint8_t)q);
  }
  int k;
  (void)frexp(a, &k);         /* a = f * 2^k, f in [0.5, 1) */
  int E = k - 1;              /* a in [2^E, 2^(E+1)) */
  double q = nearbyint(ldexp(a, 3 - E)); /* grid step 2^(E-3): q in [8, 16] */
  if (q >= 16.0) {            /* rounded up into the next binade */
    q = 8.0;
    E += 1;
  }
  int field = E + 7;
  int code = (field << 3) | ((int)q - 8);
  if (code > 0x7E) code = 0x7E; /* 480 is not finite in E4M3: saturate */
  return (uint8_t)(sign | code);
}

/* OCP MX E2M1 (the low 4 bits of `code`): exponent field 0 holds the
 * subnormal m * 0.5; otherwise (1 + m / 2) * 2^(e - 1). */
double orc_e2m1_to_double(uint8_t code) {
  int sign = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -v : v;
}

/* OCP MX E8M0 scale: 2^(byte - 127); 0xFF is NaN. */
double orc_e8m0_to_double(uint8_t byte) {
  if (byte == 0xFF) return NAN;
  return ldexp(1.0, (int)byte - 127);
}

/* E2M1 code of a value already divided by its group's scale: the nearest of
 * the eight magnitudes, ties to the even mantissa, magnitudes >= 6 saturate
 * to 6.  The rounding is nearbyint() (round-to-nearest-even) on the value
 * expressed in units of its binade's step: 0.5 below 2, 1 in [2, 4), 2 from
 * 4 on -- an even multiple of the step is a zero mantissa bit. */
uint8_t orc_e2m1_from_double(double v) {
  uint8_t sign = signbit(v) ? 0x8 : 0x0;
  double a = fabs(v);
  double r;
  if (a >= 6.0)
    r = 6.0;
  else if (a < 2.0)
    r = 0.5 * nearbyint(a * 2.0);
  else if (a < 4.0)
    r = nearbyint(a);
  else
    r = 2.0 * nearbyint(a * 0.5);
  for (uint8_t c = 0; c < 8; c++)
    if (orc_e2m1_to_double(c) == r) return (uint8_t)(sign | c);
  return sign; /* not reached: r is one of the magnitudes */
}

/* Shared-exponent byte of a group with largest magnitude amax (finite):
 * floor(log2(amax)) - 2 + 127, clamped to [0, 254]; amax = 0 gives 0. */
uint8_t orc_mxfp4_scale_byte(double amax) {
  if (amax == 0.0) return 0;
  int k;
  (void)frexp(amax, &k); /* amax = f * 2^k, f in [0.5, 1): floor(log2 amax) = k - 1 */
  int e = (k - 1) - 2 + 127;
  if (e < 0) e = 0;
  if (e > 254) e = 254;
  return (uint8_t)e;
}

/* Encode one group of n bf16 values (n = 32) into n E2M1 codes (one per
 * byte, low 4 bits) and its scale byte, by the rule in the header above. */
void orc_mxfp4_encode_group(const uint16_t *x, int32_t n, uint8_t *codes, uint8_t *scale) {
  double amax = 0.0;
  int finite = 1;
  for (int32_t i = 0; i < n; i++) {
    double v = orc_bf16_to_double(x[i]);
    if (!isfinite(v)) finite = 0;
    else if (fabs(v) > amax) amax = fabs(v);
  }
  if (!finite) {
    *scale = 0xFF;
    for (int32_t i = 0; i < n; i++) codes[i] = 0;
    return;
  }
  uint8_t sb = orc_mxfp4_scale_byte(amax);
  double X = orc_e8m0_to_double(sb);
  *scale = sb;
  for (int32_t i = 0; i < n; i++) codes[i] = orc_e2m1_from_double(orc_bf16_to_double(x[i]) / X);
}

/* Correctly rounded binary32 quotient: the binary64 quotient of two binary32
 * values rounded once more to binary32 equals the correctly rounded binary32
 * quotient, because 53 >= 2*24 + 2. */
float orc_div_f32(float x, float s) { return (float)((double)x / (double)s); }

/* ------------------------------------------------------------------ */
/* Cache element access through the block table. */

typedef struct {
  const void *k, *v;
  const void *ks, *vs;
  int32_t num_blocks, hkv, bs, d, dtype;
} cache_view;

/* Value of every E4M3 code, filled once from orc_e4m3_to_double (a memo of
 * the definition above, so the per-element work is a lookup). */
static double e4m3_value[256];
static int e4m3_value_ready = 0;
/* Likewise the 16 E2M1 values and the 256 E8M0 scales (memos of
 * orc_e2m1_to_double and orc_e8m0_to_double). */
static double e2m1_value[16], e8m0_value[256];
static void e4m3_table_init(void) {
  if (e4m3_value_ready) return;
  for (int i = 0; i < 256; i++) e4m3_value[i] = orc_e4m3_to_double((uint8_t)i);
  for (int i = 0; i < 16; i++) e2m1_value[i] = orc_e2m1_to_double((uint8_t)i);
  for (int i = 0; i < 256; i++) e8m0_value[i] = orc_e8m0_to_double((uint8_t)i);
  e4m3_value_ready = 1;
}

/* Element dd of token slot (phys, off), KV head kvh.  MXFP4: codes
 * [nb][hkv][bs][d/2] with element 2i in the low and 2i+1 in the high 4 bits
 * of byte i; scale bytes [nb][hkv][d/32][bs]. */
static double cache_elem(const cache_view *c, const void *base, const void *scale,
                         int64_t phys, int32_t kvh, int32_t off, int32_t dd) {
  int64_t row = (phys * c->hkv + kvh) * (int64_t)c->bs + off;
  if (c->dtype == ORC_KV_BF16) return orc_bf16_to_double(((const uint16_t *)base)[row * c->d + dd]);
  if (c->dtype == ORC_KV_E4M3)
    return e4m3_value[((const uint8_t *)base)[row * c->d + dd]] * (double)((const float *)scale)[phys * c->hkv + kvh];
  uint8_t byte = ((const uint8_t *)base)[row * (c->d / 2) + dd / 2];
  uint8_t code = (dd & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
  uint8_t sb = ((const uint8_t *)scale)[((phys * c->hkv + kvh) * (c->d / 32) + dd / 32) * (int64_t)c->bs + off];
  return e2m1_value[code] * e8m0_value[sb];
}

/* Encode one token's head vector x[d] into MXFP4 codes and scales at slot
 * (blk, off), head h, of a cache with the layout above. */
static void mxfp4_store(uint8_t *codes, uint8_t *scales, int64_t blk, int32_t h, int64_t off, int32_t hkv,
                        int32_t bs, int32_t d, const uint16_t *x) {
  uint8_t c[32], sb;
  uint8_t *row = codes + ((blk * hkv + h) * (int64_t)bs + off) * (d / 2);
  for (int32_t grp = 0; grp < d / 32; grp++) {
    orc_mxfp4_encode_group(x + 32 * grp, 32, c, &sb);
    for (int32_t i = 0; i < 16; i++) row[16 * grp + i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
    scales[((blk * hkv + h) * (d / 32) + grp) * (int64_t)bs + off] = sb;
  }
}

/* ------------------------------------------------------------------ */
/* kv_append.  New tokens' K and V are written into the cache slots the
 * scheduler assigned ([AMPD] §7: the increment's KV is concatenated onto the
 * locally held history; [Agentic] §5.2: the KV write precedes attention).
 * slot = physical_block * block_size + offset; slot < 0 means "skip". */
int orc_kv_append(void *k_cache, void *v_cache, void *k_scale, void *v_scale,
                  int32_t num_blocks, int32_t hkv, int32_t bs, int32_t d, int32_t dtype,
                  const uint16_t *k_new, const uint16_t *v_new, const int64_t *slot_mapping,
                  int64_t num_tokens) {
  for (int64_t t = 0; t < num_tokens; t++) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    int64_t blk = slot / bs, off = slot % bs;
    if (blk >= num_blocks) return ORC_ERR_RANGE;
    for (int32_t h = 0; h < hkv; h++) {
      if (dtype == ORC_KV_MXFP4) {
        mxfp4_store((uint8_t *)k_cache, (uint8_t *)k_scale, blk, h, off, hkv, bs, d, k_new + (t * hkv + h) * (int64_t)d);
        mxfp4_store((uint8_t *)v_cache, (uint8_t *)v_scale, blk, h, off, hkv, bs, d, v_new + (t * hkv + h) * (int64_t)d);
        continue;
      }
      for (int32_t e = 0; e < d; e++) {
        int64_t src = (t * hkv + h) * (int64_t)d + e;
        int64_t dst = ((blk * hkv + h) * (int64_t)bs + off) * (int64_t)d + e;
        if (dtype == ORC_KV_BF16) {
          ((uint16_t *)k_cache)[dst] = k_new[src];
          ((uint16_t *)v_cache)[dst] = v_new[src];
        } else {
          float kx = (float)orc_bf16_to_double(k_new[src]);
          float vx = (float)orc_bf16_to_double(v_new[src]);
          ((uint8_t *)k_cache)[dst] = orc_e4m3_from_float(orc_div_f32(kx, ((const float *)k_scale)[blk * hkv + h]));
          ((uint8_t *)v_cache)[dst] = orc_e4m3_from_float(orc_div_f32(vx, ((const float *)v_scale)[blk * hkv + h]));
        }
      }
    }
  }
  return ORC_OK;
}

/* Encode a whole pool of bf16 values ([nb][hkv][bs][d]) with per-(block,
 * head) scales: the same per-element rule as orc_kv_append. */
void orc_e4m3_quantize_pool(const uint16_t *src, const float *scale, uint8_t *dst,
                            int64_t nb, int32_t hkv, int32_t bs, int32_t d) {
  int64_t per = (int64_t)bs * d;
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < nb * hkv; bh++) {
    float s = scale[bh];
    for (int64_t e = 0; e < per; e++) {
      float x = (float)orc_bf16_to_double(src[bh * per + e]);
      dst[bh * per + e] = orc_e4m3_from_float(orc_div_f32(x, s));
    }
  }
}

/* MXFP4-encode a whole pool of bf16 values ([nb][hkv][bs][d]): the same
 * per-token rule as orc_kv_append, into codes [nb][hkv][bs][d/2] and scales
 * [nb][hkv][d/32][bs]. */
void orc_mxfp4_quantize_pool(const uint16_t *src, uint8_t *codes, uint8_t *scales, int64_t nb, int32_t hkv,
                             int32_t bs, int32_t d) {
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < nb * hkv; bh++)
    for (int32_t off = 0; off < bs; off++)
      mxfp4_store(codes, scales, bh / hkv, (int32_t)(bh % hkv), off, hkv, bs, d, src + (bh * bs + off) * (int64_t)d);
}

/* Values of one sequence's cache through its block-table row, in fp64:
 * out[p][kvh][e] = element e of K (or V) at position p (the same element
 * rule attention uses). */
int orc_gather_values(const void *cache, const void *scale, int32_t dtype, int32_t num_blocks, int32_t hkv,
                      int32_t bs, int32_t d, const int32_t *bt_row, int64_t ctx, double *out) {
  e4m3_table_init();
  cache_view c = {cache, cache, scale, scale, num_blocks, hkv, bs, d, dtype};
  for (int64_t p = 0; p < ctx; p++) {
    int32_t phys = bt_row[p / bs];
    if (phys < 0 || phys >= num_blocks) return ORC_ERR_RANGE;
    for (int32_t h = 0; h < hkv; h++)
      for (int32_t e = 0; e < d; e++) out[(p * hkv + h) * (int64_t)d + e] = cache_elem(&c, cache, scale, phys, h, (int32_t)(p % bs), e);
  }
  return ORC_OK;
}

/* Raw gather of one sequence's cache through its block-table row:
 * out[p][kvh][e] = cache[bt[p / bs]][kvh][p % bs][e] for p < ctx, in the
 * cache's own element type (elem_bytes 2 for bf16, 1 for fp8). */
int orc_gather(const void *cache, int32_t num_blocks, int32_t hkv, int32_t bs, int32_t d,
               int32_t elem_bytes, const int32_t *bt_row, int64_t ctx, void *out) {
  for (int64_t p = 0; p < ctx; p++) {
    int32_t phys = bt_row[p / bs];
    if (phys < 0 || phys >= num_blocks) return ORC_ERR_RANGE;
    for (int32_t h = 0; h < hkv; h++) {
      const char *src = (const char *)cache +
                        (((int64_t)phys * hkv + h) * bs + p % bs) * (int64_t)d * elem_bytes;
      char *dst = (char *)out + ((p * hkv + h) * (int64_t)d) * elem_bytes;
      memcpy(dst, src, (size_t)d * elem_bytes);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Attention for one (row, head) over the key range [k_lo, k_hi) of the
 * sequence, restricted to keys <= pos (causal, inclusive).  Writes the
 * normalised output o[d] and lse = m + ln(sum exp(l - m)) with the logits in
 * natural units (scale * q.k).  An empty range gives lse = -inf, o = 0.
 * If probs != NULL, the probabilities w_j / Z for keys k_lo..min(k_hi,pos+1)-1
 * are stored there. */
static void attend_one(const cache_view *c, const int32_t *bt_row, const uint16_t *qrow,
                       int32_t kvh, int64_t pos, int64_t k_lo, int64_t k_hi, double scale,
                       double *logits, double *o, double *lse, double *probs) {
  int64_t hi = k_hi < pos + 1 ? k_hi : pos + 1;
  int64_t n = hi - k_lo;
  for (int32_t e = 0; e < c->d; e++) o[e] = 0.0;
  if (n <= 0) {
    *lse = -INFINITY;
    return;
  }
  /* logits l_j = scale * sum_e q[e] * K[j][e] */
  for (int64_t j = k_lo; j < hi; j++) {
    int64_t phys = bt_row[j / c->bs];
    int32_t off = (int32_t)(j % c->bs);
    double dot = 0.0;
    for (int32_t e = 0; e < c->d; e++)
      dot += orc_bf16_to_double(qrow[e]) * cache_elem(c, c->k, c->ks, phys, kvh, off, e);
    logits[j - k_lo] = scale * dot;
  }
  double m = -INFINITY;
  for (int64_t j = 0; j < n; j++)
    if (logits[j] > m) m = logits[j];
  double z = 0.0;
  for (int64_t j = 0; j < n; j++) {
    logits[j] = exp(logits[j] - m); /* now w_j */
    z += logits[j];
  }
  for (int64_t j = k_lo; j < hi; j++) {
    int64_t phys = bt_row[j / c->bs];
    int32_t off = (int32_t)(j % c->bs);
    double w = logits[j - k_lo];
    for (int32_t e = 0; e < c->d; e++) o[e] += w * cache_elem(c, c->v, c->vs, phys, kvh, off, e);
  }
  for (int32_t e = 0; e < c->d; e++) o[e] /= z;
  *lse = m + log(z);
  if (probs)
    for (int64_t j = 0; j < n; j++) probs[j] = logits[j] / z;
}

/* Validate lengths and the block-table entries a sequence will read. */
static int check_seq(const cache_view *c, const int32_t *bt_row, int32_t max_blocks,
                     int64_t hist, int64_t incr) {
  if (hist < 0 || incr < 0) return ORC_ERR_RANGE;
  int64_t nblk = orc_num_blocks(hist + incr, c->bs);
  if (nblk > max_blocks) return ORC_ERR_RANGE;
  for (int64_t j = 0; j < nblk; j++)
    if (bt_row[j] < 0 || bt_row[j] >= c->num_blocks) return ORC_ERR_RANGE;
  return ORC_OK;
}

/*
 * Paged attention over [history | increment] for a batch of sequences.
 * [AMPD] §1 and §3: incremental prefill reads the cached history of length
 * l_hist plus l_incr new tokens; initial prefill is l_hist = 0; decode emits
 * one token against the whole cache (l_incr = 1).  Query row i of sequence s
 * (rows packed in sequence order, rowstart[s] = sum of earlier incr) sits at
 * absolute position hist[s] + i.
 *
 * rows: the global query rows to compute (NULL = all total_q rows in order).
 * out:  double [nrows][hq][d];  lse: double [nrows][hq] (may be NULL).
 */
int orc_attention(const uint16_t *q, const void *k_cache, const void *v_cache,
                  const void *k_scale, const void *v_scale, int32_t dtype,
                  int32_t num_blocks, int32_t hkv, int32_t bs, int32_t d,
                  const int32_t *block_tables, int32_t max_blocks,
                  const int32_t *hist, const int32_t *incr, int32_t num_seqs, int32_t hq,
                  float scale, const int64_t *rows, int64_t nrows, double *out, double *lse) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return ORC_ERR_RANGE;
  e4m3_table_init();
  cache_view c = {k_cache, v_cache, k_scale, v_scale, num_blocks, hkv, bs, d, dtype};
  int64_t *rowstart = (int64_t *)malloc(sizeof(int64_t) * (num_seqs + 1));
  rowstart[0] = 0;
  for (int32_t s = 0; s < num_seqs; s++) {
    int rc = check_seq(&c, block_tables + (int64_t)s * max_blocks, max_blocks, hist[s], incr[s]);
    if (rc) {
      free(rowstart);
      return rc;
    }
    rowstart[s + 1] = rowstart[s] + incr[s];
  }
  int64_t total_q = rowstart[num_seqs];
  if (rows == NULL) nrows = total_q;
  for (int64_t i = 0; i < nrows; i++) {
    int64_t r = rows ? rows[i] : i;
    if (r < 0 || r >= total_q) {
      free(rowstart);
      return ORC_ERR_RANGE;
    }
  }
  int32_t group = hq / hkv;
  int rc_all = ORC_OK;
#pragma omp parallel
  {
    double *logits = NULL;
    int64_t cap = 0;
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < nrows * hq; t++) {
      int64_t i = t / hq;
      int32_t h = (int32_t)(t % hq);
      int64_t r = rows ? rows[i] : i;
      int32_t s = 0; /* sequence owning row r */
      while (rowstart[s + 1] <= r) s++;
      int64_t pos = (int64_t)hist[s] + (r - rowstart[s]);
      if (pos + 1 > cap) {
        free(logits);
        cap = pos + 1;
        logits = (double *)malloc(sizeof(double) * cap);
      }
      double l;
      attend_one(&c, block_tables + (int64_t)s * max_blocks, q + (r * hq + h) * (int64_t)d,
                 h / group, pos, 0, pos + 1, (double)scale, logits,
                 out + (i * hq + h) * (int64_t)d, &l, NULL);
      if (lse) lse[i * hq + h] = l;
    }
    free(logits);
  }
  free(rowstart);
  return rc_all;
}

/* Partial attention of one (row, head) over keys [k_lo, k_hi): the pieces a
 * split computation produces.  [Agentic] §4.3.3 merges such partial outputs
 * O_i with their LSE "the online-softmax way". */
int orc_attention_partial(const uint16_t *qrow, const void *k_cache, const void *v_cache,
                          const void *k_scale, const void *v_scale, int32_t dtype,
                          int32_t num_blocks, int32_t hkv, int32_t bs, int32_t d,
                          const int32_t *bt_row, int32_t kvh, int64_t pos, int64_t k_lo,
                          int64_t k_hi, float scale, double *o, double *lse, double *probs) {
  e4m3_table_init();
  cache_view c = {k_cache, v_cache, k_scale, v_scale, num_blocks, hkv, bs, d, dtype};
  int64_t n = (k_hi < pos + 1 ? k_hi : pos + 1) - k_lo;
  double *logits = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
  attend_one(&c, bt_row, qrow, kvh, pos, k_lo, k_hi, (double)scale, logits, o, lse, probs);
  free(logits);
  return ORC_OK;
}

/* Merge n partial results (o_i normalised by their own sums, lse_i) into the
 * whole: L = max lse_i, w_i = exp(lse_i - L), o = sum w_i o_i / sum w_i,
 * lse = L + ln(sum w_i).  Parts with lse = -inf carry no keys and are
 * skipped.  [Agentic] §4.3.3. */
void orc_merge(const double *o_parts, const double *lse_parts, int32_t n, int32_t d,
               double *o, double *lse) {
  double L = -INFINITY;
  for (int32_t i = 0; i < n; i++)
    if (lse_parts[i] > L) L = lse_parts[i];
  for (int32_t e = 0; e < d; e++) o[e] = 0.0;
  if (L == -INFINITY) {
    *lse = -INFINITY;
    return;
  }
  double wsum = 0.0;
  for (int32_t i = 0; i < n; i++) {
    if (lse_parts[i] == -INFINITY) continue;
    double w = exp(lse_parts[i] - L);
    wsum += w;
    for (int32_t e = 0; e < d; e++) o[e] += w * o_parts[(int64_t)i * d + e];
  }
  for (int32_t e = 0; e < d; e++) o[e] /= wsum;
  *lse = L + log(wsum);
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the following calls (n >= 1); returns the previous setting.
 * Only the distribution of independent outputs changes, not the arithmetic. */
int orc_set_num_threads(int n) {
  const int prev = orc_num_threads();
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#endif
  return prev;
}
