/*
 * oracle.h -- fp64 CPU reference for paged-KV GQA attention and kv_append.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product library.  It shares no
 * code, header, table or constant with the GPU path.
 *
 * Layouts (row-major):
 *   q            uint16 (bf16 bits) [total_q][hq][d], sequences packed in order
 *   k/v cache    [num_blocks][hkv][bs][d], uint16 bf16 bits or uint8 E4M3 codes;
 *                MXFP4: uint8 [num_blocks][hkv][bs][d/2], element 2i in the low
 *                and 2i+1 in the high 4 bits of byte i
 *   k/v scale    E4M3: float [num_blocks][hkv] (value = code * scale);
 *                MXFP4: uint8 E8M0 [num_blocks][hkv][d/32][bs]
 *   block_tables int32 [num_seqs][max_blocks]
 *   k/v new      uint16 bf16 bits [num_tokens][hkv][d]
 *   slot_mapping int64 [num_tokens], slot = block * bs + offset, < 0 = skip
 */
#ifndef PAGED_ATTN_ORACLE_H
#define PAGED_ATTN_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_OK = 0, ORC_ERR_RANGE = 1 };
enum { ORC_KV_BF16 = 0, ORC_KV_E4M3 = 1, ORC_KV_MXFP4 = 2 };

int64_t orc_cdiv(int64_t a, int64_t b);
int64_t orc_num_blocks(int64_t ctx, int32_t block_size);
double orc_bf16_to_double(uint16_t bits);
double orc_e4m3_to_double(uint8_t code);
uint8_t orc_e4m3_from_float(float x);
float orc_div_f32(float x, float s);
double orc_e2m1_to_double(uint8_t code);
double orc_e8m0_to_double(uint8_t byte);
uint8_t orc_e2m1_from_double(double v);
uint8_t orc_mxfp4_scale_byte(double amax);
void orc_mxfp4_encode_group(const uint16_t *x, int32_t n, uint8_t *codes, uint8_t *scale);
void orc_mxfp4_quantize_pool(const uint16_t *src, uint8_t *codes, uint8_t *scales, int64_t nb, int32_t hkv,
                             int32_t bs, int32_t d);
int orc_gather_values(const void *cache, const void *scale, int32_t dtype, int32_t num_blocks, int32_t hkv,
                      int32_t bs, int32_t d, const int32_t *bt_row, int64_t ctx, double *out);

int orc_kv_append(void *k_cache, void *v_cache, void *k_scale, void *v_scale,
                  int32_t num_blocks, int32_t hkv, int32_t bs, int32_t d, int32_t dtype,
                  const uint16_t *k_new, const uint16_t *v_new, const int64_t *slot_mapping,
                  int64_t num_tokens);
void orc_e4m3_quantize_pool(const uint16_t *src, const float *scale, uint8_t *dst, int64_t nb,
                            int32_t hkv, int32_t bs, int32_t d);
int orc_gather(const void *cache, int32_t num_blocks, int32_t hkv, int32_t bs, int32_t d,
               int32_t elem_bytes, const int32_t *bt_row, int64_t ctx, void *out);

int orc_attention(const uint16_t *q, const void *k_cache, const void *v_cache,
                  const void *k_scale, const void *v_scale, int32_t dtype,
                  int32_t num_blocks, int32_t hkv, int32_t bs, int32_t d,
                  const int32_t *block_tables, int32_t max_blocks, const int32_t *hist,
                  const int32_t *incr, int32_t num_seqs, int32_t hq, float scale,
                  const int64_t *rows, int64_t nrows, double *out, double *lse);
int orc_attention_partial(const uint16_t *qrow, const void *k_cache, const void *v_cache,
                          const void *k_scale, const void *v_scale, int32_t dtype,
                          int32_t num_blocks, int32_t hkv, int32_t bs, int32_t d,
                          const int32_t *bt_row, int32_t kvh, int64_t pos, int64_t k_lo,
                          int64_t k_hi, float scale, double *o, double *lse, double *probs);
void orc_merge(const double *o_parts, const double *lse_parts, int32_t n, int32_t d, double *o,
               double *lse);
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
