/* Runs every function of the CPU oracle on small, edge-heavy inputs, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer (any finding
 * aborts).  Test infrastructure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/nvfp4_oracle.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static double urand(void)
{
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(st >> 11) * (1.0 / 9007199254740992.0);
}
static float nrand(void)
{
    double u1 = 1.0 - urand(), u2 = urand();
    return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

int main(void)
{
    /* formats over a sweep, specials included */
    const float specials[] = {0.0f, -0.0f, 0.25f, 0.75f, 5.0f, 6.0f, 448.0f, 1e-40f, 3e38f, -7.0f};
    for (size_t i = 0; i < sizeof specials / sizeof *specials; ++i) {
        (void)orc_e2m1_encode(specials[i]);
        (void)orc_e4m3_encode(fabsf(specials[i]));
        (void)orc_bf16_rne(specials[i]);
    }
    for (int c = 0; c < 256; ++c) {
        (void)orc_e4m3_value((uint8_t)c);
        (void)orc_e2m1_value((uint8_t)(c & 15));
    }
    /* quantize / dequantize, 1-D and 2-D, both searches, with and without amax */
    enum { R = 48, C = 64 };
    float *x = malloc(sizeof(float) * R * C), *y = malloc(sizeof(float) * R * C);
    uint8_t *codes = malloc(R * C / 2), *scales = malloc(R * C / 16);
    float e6[R * C / 16], e4[R * C / 16], sd;
    for (int i = 0; i < R * C; ++i)
        x[i] = nrand() * (urand() < 0.02 ? 20.0f : 1.0f);
    x[5] = 0.0f;
    x[7] = 1e-39f;
    for (int layout = 0; layout < 2; ++layout)
        for (int search = 0; search < 2; ++search) {
            if (orc_quantize(x, R, C, layout, search, NULL, codes, scales, &sd, e6, e4))
                return 1;
            orc_dequantize(codes, scales, sd, R, C, layout, y);
            float amax = 2688.0f;
            if (orc_quantize(x, R, C, layout, search, &amax, codes, scales, &sd, NULL, NULL))
                return 1;
        }
    memset(y, 0, sizeof(float) * R * C);
    if (orc_quantize(y, R, C, 0, 1, NULL, codes, scales, &sd, NULL, NULL)) /* all zero */
        return 1;
    if (orc_quantize(x, R, 24, 0, 1, NULL, codes, scales, &sd, NULL, NULL) == 0) /* cols % 16 */
        return 1;
    uint16_t *b16 = malloc(sizeof(uint16_t) * R * C);
    orc_to_bf16(x, R * C, b16);
    (void)orc_amax(x, R * C);
    /* K mean: wide binades, subnormals, one token, cancellation */
    float mu[C];
    orc_kv_mean(x, R, C, mu);
    orc_kv_mean(x, 1, C, mu);
    for (int i = 0; i < R * C; ++i)
        y[i] = ldexpf(nrand(), (int)(urand() * 250) - 140);
    orc_kv_mean(y, R, C, mu);
    /* chunk encode and token dequantize */
    uint8_t *kc = malloc(R * C / 2), *ks = malloc(R * C / 16), *vc = malloc(R * C / 2),
            *vs = malloc(R * C / 16);
    float sdk, sdv;
    if (orc_kv_encode_chunk(x, y, R, C, 1, kc, ks, &sdk, vc, vs, &sdv, mu))
        return 1;
    orc_kv_dequant_tokens(kc, ks, sdk, mu, 3, R - 3, C, b16);
    orc_kv_dequant_tokens(vc, vs, sdv, NULL, 0, R, C, b16);
    /* effective sets against their size */
    int64_t toks[4096];
    for (int64_t t = 0; t < 12; ++t) {
        int64_t n = orc_effective_tokens(t, 48, 3, 16, 4 * 48, 12, NULL);
        if (n > 4096 || orc_effective_tokens(t, 48, 3, 16, 4 * 48, 12, toks) != n)
            return 1;
    }
    /* GEMM reference, all rows and a subset */
    enum { M = 16, N = 32, K = 64 };
    uint8_t ac[M * K / 2], as[M * K / 16], wc[N * K / 2], wsc[N * K / 16];
    float sa, sw;
    if (orc_quantize(x, M, K, 0, 1, NULL, ac, as, &sa, NULL, NULL) ||
        orc_quantize(x + M * K, N, K, 1, 1, NULL, wc, wsc, &sw, NULL, NULL))
        return 1;
    double yr[M * N], ab[M * N];
    if (orc_gemm_ref(ac, as, sa, M, K, wc, wsc, sw, N, 1, NULL, 0, yr, ab))
        return 1;
    const int64_t rows[3] = {0, 7, 15};
    if (orc_gemm_ref(ac, as, sa, M, K, wc, wsc, sw, N, 1, rows, 3, yr, NULL))
        return 1;
    /* RHT, LoRA, attention */
    orc_rht16(x, R, C, 0xB7E1u, y);
    double ly[M * N], lab[M * N];
    float xa[M * 16];
    if (orc_lora_ref(x, x + M * K, x + 2 * M * K, M, K, N, 16, 2.0f, NULL, 0, ly, lab, xa))
        return 1;
    enum { NQ = 5, NK = 9, H = 2, D = 16 };
    double o[NQ * H * D], ao[NQ * H * D], lse[NQ * H];
    if (orc_attention_ref(x, x + 512, x + 1024, NQ, NK, H, D, 0.25, NULL, 0, o, ao, lse) ||
        orc_attention_ref(x, x + 512, x + 1024, NQ, 0, H, D, 0.25, NULL, 0, o, ao, lse))
        return 1;
    free(x); free(y); free(codes); free(scales); free(b16); free(kc); free(ks); free(vc); free(vs);
    puts("oracle ok");
    return 0;
}
