/*
 * nvfp4_oracle.h -- declarations of the CPU oracle (test infrastructure).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg use
 * this library; the GPU library neither includes nor links it.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H

#include <stdint.h>

#define ORC_LAYOUT_1D 0
#define ORC_LAYOUT_2D 1
#define ORC_SEARCH_6 0
#define ORC_SEARCH_4O6 1

float orc_e2m1_value(uint8_t nib);
uint8_t orc_e2m1_encode(float y);
float orc_e4m3_value(uint8_t code);
uint8_t orc_e4m3_encode(float t);
uint16_t orc_bf16_rne(float f);
float orc_amax(const float *x, int64_t n);
void orc_tensor_scales(float amax, float *s_enc, float *s_dec);
int orc_quantize(const float *x, int64_t R, int64_t C, int layout, int search,
                 const float *amax_in, uint8_t *codes, uint8_t *scales, float *s_dec_out,
                 float *err6, float *err4);
float orc_dequant_value(uint8_t nib, uint8_t scale, float s_dec);
void orc_dequantize(const uint8_t *codes, const uint8_t *scales, float s_dec, int64_t R,
                    int64_t C, int layout, float *out);
void orc_to_bf16(const float *x, int64_t n, uint16_t *out);
void orc_kv_mean(const float *K, int64_t T, int64_t HD, float *mu);
int orc_kv_encode_chunk(const float *K, const float *V, int64_t T, int64_t HD, int search,
                        uint8_t *kc, uint8_t *ks, float *sdk, uint8_t *vc, uint8_t *vs,
                        float *sdv, float *mu);
void orc_kv_dequant_tokens(const uint8_t *codes, const uint8_t *scales, float s_dec,
                           const float *mu, int64_t tok0, int64_t ntok, int64_t HD,
                           uint16_t *out);
int64_t orc_effective_tokens(int64_t t, int64_t Tc, int64_t W, int64_t g_tokens,
                             int64_t s_start, int64_t s_tokens, int64_t *out);
int orc_gemm_ref(const uint8_t *a_codes, const uint8_t *a_scales, float a_sdec, int64_t M,
                 int64_t K, const uint8_t *w_codes, const uint8_t *w_scales, float w_sdec,
                 int64_t N, int w_layout, const int64_t *rows, int64_t nrows, double *y,
                 double *abs_sum);
void orc_e2m1_encode_array(const float *y, int64_t n, uint8_t *out);
void orc_rht16(const float *x, int64_t R, int64_t C, uint32_t signs, float *out);
int orc_lora_ref(const float *x, const float *a, const float *b, int64_t M, int64_t K,
                 int64_t N, int64_t r, float scale, const int64_t *rows, int64_t nrows,
                 double *y, double *abs_sum, float *xa);
void orc_e4m3_encode_array(const float *t, int64_t n, uint8_t *out);
int orc_attention_ref(const float *q, const float *k, const float *v, int64_t nq, int64_t nk,
                      int64_t H, int64_t d, double scale, const int64_t *rows, int64_t nrows,
                      double *o, double *abs_o, double *lse);

#endif
