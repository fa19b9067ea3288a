/*
 * nvfp4_oracle.c -- plain, slow CPU reference of the NVFP4 data path.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the GPU library, and it is never
 * on the product path.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (see oracle/build.py).
 * Every float operation below is one IEEE-754 binary32 operation rounded to
 * nearest-even (x86-64 SSE, FLT_EVAL_METHOD == 0, no contraction); fmaf() is
 * the correctly rounded fused multiply-add of C99; double is used only where
 * stated.
 *
 * Sources (the LongLive-2.0 pages):
 *   [DR]  "MCISLAB DeepRead: LongLive2" summary, Method: NVFP4 training
 *         (E2M1 elements, block FP8 E4M3 scale, tensor FP32 scale; 2-D
 *         scaling for weights, 1-D for activations; scale search over the
 *         target magnitudes 6 and 4, keeping the lower-error encoding),
 *         inference infrastructure (chunk-level KV quantization with
 *         F_c = 8 frames, K-smoothing, storage 4*T_c*H*d -> (9/8)*T_c*H*d
 *         bytes) and algorithm design (multi-shot attention sink,
 *         K_eff(t) = A_g u A_s u KV[t-W, t), overlapping tokens removed).
 *   [AU]  ngjoo.com audit of arXiv 2605.18739, claim list: adaptive block
 *         scaling evaluates 6 and 4 per block and selects the lower-error
 *         encoding; the KV storage formula; FP4 GEMM in place of BF16 GEMM.
 *   [IT]  "LongLive-2.0: Infrastruttura Parallela NVFP4 per Video Lunghi",
 *         sections "Addestramento NVFP4" (a random Hadamard transform is
 *         applied before quantization on the gradient-sensitive paths),
 *         "Inferenza W4A4 NVFP4" (micro-block KV scaling with Four Over
 *         Six) and "Multi-Shot Attention Sink".
 * Where the pages leave a step open the reading taken is marked READING.
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Element and scale formats                                          */
/* ------------------------------------------------------------------ */

/* E2M1 magnitudes: 1 sign, 2 exponent (bias 1), 1 mantissa bit; the largest
 * magnitude is 6 ([DR] NVFP4 training: E2M1; [AU]: standard target 6). */
static const float kE2M1Mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float orc_e2m1_value(uint8_t nib)
{
    float v = kE2M1Mag[nib & 7u];
    return (nib & 8u) ? -v : v;
}

/* Nearest E2M1 magnitude to |y|, ties to the even index (= even mantissa
 * bit), saturating at 6; the sign bit copies signbit(y), so a negative value
 * that rounds to zero keeps its sign (READING: -0 is encoded as 0x8).
 * Distances are taken in double; wherever two candidates are close to a tie
 * both differences are exact (Sterbenz), so ties are detected exactly. */
uint8_t orc_e2m1_encode(float y)
{
    uint8_t sign = signbit(y) ? 8u : 0u;
    double a = fabs((double)y);
    uint8_t k = 7;
    if (a < 6.0) {
        double best = a; /* distance to magnitude 0 */
        k = 0;
        for (uint8_t j = 1; j < 8; ++j) {
            double dist = fabs(a - (double)kE2M1Mag[j]);
            if (dist < best || (dist == best && (j & 1u) == 0)) {
                best = dist;
                k = j;
            }
        }
    }
    return (uint8_t)(sign | k);
}

/* OCP FP8 E4M3FN (READING: the pages say "FP8 E4M3"): bias 7, codes
 * 0x00..0x7E finite, 0x7F NaN, largest 448, e = 0 subnormal m * 2^-9. */
float orc_e4m3_value(uint8_t code)
{
    int e = (code >> 3) & 0xF;
    int m = code & 7;
    float v = (e == 0) ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return (code & 0x80u) ? -v : v;
}

/* Nearest of the 127 non-negative finite E4M3 values to t >= 0, ties to the
 * even code; t >= 448 (and +inf) saturates to 448 = 0x7E.  The scale sign
 * bit is always 0. */
uint8_t orc_e4m3_encode(float t)
{
    if (!(t < 448.0f))
        return 0x7E;
    double td = fabs((double)t);
    uint8_t best_code = 0;
    double best = td;
    for (int c = 1; c <= 0x7E; ++c) {
        double dist = fabs(td - (double)orc_e4m3_value((uint8_t)c));
        if (dist < best || (dist == best && (c & 1) == 0)) {
            best = dist;
            best_code = (uint8_t)c;
        }
    }
    return best_code;
}

/* bfloat16 of a float, nearest with ties to even (the usual
 * float -> bf16 conversion); NaN stays a quiet NaN. */
uint16_t orc_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* ------------------------------------------------------------------ */
/* Tensor scale                                                       */
/* ------------------------------------------------------------------ */

float orc_amax(const float *x, int64_t n)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = fabsf(x[i]);
        if (v > a)
            a = v;
    }
    return a;
}

/* FP32 tensor scale ([DR] hierarchical scaling): the tensor amax is mapped to
 * 6 * 448 = 2688, the product of the largest E2M1 and E4M3 magnitudes, so that
 * the block holding the tensor amax gets the largest block scale under the
 * standard target 6.  Both are correctly rounded divisions.  An all-zero
 * tensor gets s_enc = s_dec = 1 (READING).  0 < amax < 2^-100 and non-finite
 * inputs are outside the domain. */
void orc_tensor_scales(float amax, float *s_enc, float *s_dec)
{
    if (amax == 0.0f) {
        *s_enc = 1.0f;
        *s_dec = 1.0f;
        return;
    }
    *s_enc = 2688.0f / amax;
    *s_dec = amax / 2688.0f;
}

/* ------------------------------------------------------------------ */
/* One scaling block, both candidates of the scale search             */
/* ------------------------------------------------------------------ */

/* Encode one scaling block: `nr` rows of 16 consecutive values, row stride
 * `ld` (nr = 1 for a 1x16 activation block, 16 for a 16x16 weight tile).
 *
 * For each candidate target magnitude c (6, then 4 when search == 4/6):
 *   ideal_c = RN(RN(amax_b / c) * s_enc)           block scale before rounding
 *   sc_c    = E4M3(ideal_c),  sigma_c = value(sc_c)  (saturating: READING)
 *   S_c     = RN(sigma_c * s_dec)                  decode scale of the block
 *   r_c     = RN(1 / S_c), or 0 when S_c == 0      encode multiplier
 *   q_i     = E2M1(RN(x_i * r_c))
 *   d_i     = RN(x_i - V(q_i) * S_c)               one fma: exact product
 *   row error  E = RN(E_lo + E_hi), E_lo the fma chain d_i*d_i + acc over
 *                  i = 0..7 from +0, E_hi over i = 8..15      (READING)
 *   err_c   = the row errors summed pairwise, level by level, adjacent
 *             pairs in row order (a single row: its own error)  (READING)
 * The encoding with the lower error is kept; a tie keeps target 6
 * ([DR], [AU]: evaluate 6 and 4, select the lower-error encoding; the
 * squared-error criterion and strict comparison are READINGS).  With
 * sigma_c == 0 every code is a signed zero and d_i = x_i. */
static void encode_block(const float *x, int64_t ld, int nr, float s_enc, float s_dec,
                         int search, uint8_t *nib_out /* nr*16 */, uint8_t *scale_out,
                         float *err6_out, float *err4_out)
{
    float amax = 0.0f;
    for (int r = 0; r < nr; ++r)
        for (int i = 0; i < 16; ++i) {
            float v = fabsf(x[r * ld + i]);
            if (v > amax)
                amax = v;
        }

    const int ncand = (search == ORC_SEARCH_4O6) ? 2 : 1;
    uint8_t nib[2][256];
    uint8_t sc[2];
    float err[2] = {0.0f, 0.0f};

    for (int c = 0; c < ncand; ++c) {
        float ideal = (c == 0) ? (amax / 6.0f) * s_enc : (amax * 0.25f) * s_enc;
        sc[c] = orc_e4m3_encode(ideal);
        float sigma = orc_e4m3_value(sc[c]);
        float S = sigma * s_dec;
        float rcp = (S == 0.0f) ? 0.0f : 1.0f / S;
        float row_err[16];
        for (int r = 0; r < nr; ++r) {
            float half[2];
            for (int h = 0; h < 2; ++h) {
                float acc = 0.0f;
                for (int i = 8 * h; i < 8 * h + 8; ++i) {
                    float xv = x[r * ld + i];
                    float y = xv * rcp;
                    uint8_t q = orc_e2m1_encode(y);
                    nib[c][r * 16 + i] = q;
                    float d = fmaf(-orc_e2m1_value(q), S, xv);
                    acc = fmaf(d, d, acc);
                }
                half[h] = acc;
            }
            row_err[r] = half[0] + half[1];
        }
        /* pairwise tree over rows */
        int n = nr;
        while (n > 1) {
            for (int i = 0; i < n / 2; ++i)
                row_err[i] = row_err[2 * i] + row_err[2 * i + 1];
            n /= 2;
        }
        err[c] = row_err[0];
    }

    int pick = (ncand == 2 && err[1] < err[0]) ? 1 : 0;
    memcpy(nib_out, nib[pick], (size_t)nr * 16);
    *scale_out = sc[pick];
    if (err6_out)
        *err6_out = err[0];
    if (err4_out)
        *err4_out = (ncand == 2) ? err[1] : NAN;
}

/* ------------------------------------------------------------------ */
/* Quantize / dequantize a tensor                                      */
/* ------------------------------------------------------------------ */

/* x: float32 [R, C] row-major.  1-D layout: blocks are 1x16 along a row
 * (the reduction dimension), scales [R, C/16].  2-D layout: blocks are
 * 16x16 tiles, scales [R/16, C/16] ([DR]: weights 2-D, activations and
 * gradients 1-D; the 16x16 tile size is a READING).  Codes [R, C/2]: column
 * 2j in bits 0..3 of byte j, column 2j+1 in bits 4..7 (READING). */
int orc_quantize(const float *x, int64_t R, int64_t C, int layout, int search,
                 const float *amax_in, uint8_t *codes, uint8_t *scales, float *s_dec_out,
                 float *err6, float *err4)
{
    if (C % 16 != 0 || R < 0 || C < 0)
        return -1;
    if (layout == ORC_LAYOUT_2D && R % 16 != 0)
        return -1;
    float amax = amax_in ? *amax_in : orc_amax(x, R * C);
    float s_enc, s_dec;
    orc_tensor_scales(amax, &s_enc, &s_dec);
    *s_dec_out = s_dec;

    const int64_t nbc = C / 16;
    const int nr = (layout == ORC_LAYOUT_2D) ? 16 : 1;
    uint8_t nib[256];
    for (int64_t br = 0; br < R / nr; ++br) {
        for (int64_t bc = 0; bc < nbc; ++bc) {
            const float *xb = x + br * nr * C + bc * 16;
            int64_t bidx = br * nbc + bc;
            encode_block(xb, C, nr, s_enc, s_dec, search, nib, &scales[bidx],
                         err6 ? &err6[bidx] : NULL, err4 ? &err4[bidx] : NULL);
            for (int r = 0; r < nr; ++r) {
                uint8_t *crow = codes + (br * nr + r) * (C / 2) + bc * 8;
                for (int j = 0; j < 8; ++j)
                    crow[j] = (uint8_t)(nib[r * 16 + 2 * j] | (nib[r * 16 + 2 * j + 1] << 4));
            }
        }
    }
    return 0;
}

static uint8_t code_at(const uint8_t *codes, int64_t C, int64_t r, int64_t c)
{
    uint8_t b = codes[r * (C / 2) + c / 2];
    return (c & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0xF);
}

static uint8_t scale_at(const uint8_t *scales, int64_t C, int layout, int64_t r, int64_t c)
{
    if (layout == ORC_LAYOUT_2D)
        return scales[(r / 16) * (C / 16) + c / 16];
    return scales[r * (C / 16) + c / 16];
}

/* x_hat = RN(V(q) * S), S = RN(sigma * s_dec): the block's decode scale is
 * formed first and multiplies the E2M1 value (READING). */
float orc_dequant_value(uint8_t nib, uint8_t scale, float s_dec)
{
    float S = orc_e4m3_value(scale) * s_dec;
    return orc_e2m1_value(nib) * S;
}

void orc_dequantize(const uint8_t *codes, const uint8_t *scales, float s_dec, int64_t R,
                    int64_t C, int layout, float *out)
{
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c)
            out[r * C + c] = orc_dequant_value(code_at(codes, C, r, c),
                                               scale_at(scales, C, layout, r, c), s_dec);
}

void orc_to_bf16(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_rne(x[i]);
}

/* ------------------------------------------------------------------ */
/* KV cache: K-smoothing and chunk encoding                            */
/* ------------------------------------------------------------------ */

/* Exact sum of float values.  Every finite float is M * 2^(P - 149) with
 * an integer 0 <= M < 2^24 and 0 <= P <= 253, so a sum of floats is an
 * integer multiple of 2^-149.  The accumulator holds that integer as
 * KM_DIGITS signed base-2^32 digits, d[0] the least significant, with the
 * carries left unpropagated until the end (each digit stays below 2^63 for
 * fewer than 2^31 terms); the most significant bit a float can set is bit
 * 253 + 24, so 12 digits (384 bits) leave room for the carries of 2^31
 * terms.  No step rounds. */
#define KM_DIGITS 12

static void exact_add(int64_t *d, float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    uint32_t be = (u >> 23) & 0xFFu, frac = u & 0x7FFFFFu;
    uint64_t M = be ? (uint64_t)(frac | 0x800000u) : (uint64_t)frac;
    int P = be ? (int)be - 1 : 0; /* normal: 1.f * 2^(be-127) = M * 2^(be-150) */
    if (M == 0)
        return;
    uint64_t w = M << (P % 32); /* < 2^56 */
    int64_t lo = (int64_t)(w & 0xFFFFFFFFu), hi = (int64_t)(w >> 32);
    if (u >> 31) {
        lo = -lo;
        hi = -hi;
    }
    d[P / 32] += lo;
    d[P / 32 + 1] += hi;
}

/* Sign (+1, -1 or 0) and magnitude (base-2^32 digits) of the accumulated
 * integer: carries propagated in two's complement, a negative result
 * negated. */
static int exact_magnitude(const int64_t *d, uint32_t *mag)
{
    int64_t carry = 0;
    for (int i = 0; i < KM_DIGITS; ++i) {
        int64_t x = d[i] + carry;
        int64_t low = x & 0xFFFFFFFF;
        mag[i] = (uint32_t)low;
        carry = (x - low) / 4294967296LL;
    }
    int sign = carry < 0 ? -1 : 1;
    if (sign < 0) { /* two's complement negation of the digit string */
        uint64_t c = 1;
        for (int i = 0; i < KM_DIGITS; ++i) {
            uint64_t x = (uint64_t)(uint32_t)~mag[i] + c;
            mag[i] = (uint32_t)x;
            c = x >> 32;
        }
    }
    int nz = 0;
    for (int i = 0; i < KM_DIGITS; ++i)
        nz |= mag[i] != 0;
    return nz ? sign : 0;
}

/* RN64(N * 2^-149 / T) for the integer N given by sign and magnitude, T >= 1:
 * the long division of N * 2^96 by T (base 2^32, exact quotient Q and
 * remainder), then Q rounded to 53 significant bits, ties to even, with the
 * bits below the guard bit and the remainder as the sticky bit.  N >= 1 and
 * T < 2^31 make Q >= 2^65, so 53 bits, the guard bit and the sticky bit are
 * all there; the result is a normal double (>= 2^-180). */
static double exact_quotient(int sign, const uint32_t *mag, uint32_t T)
{
    enum { ND = KM_DIGITS + 3 };
    uint32_t num[ND], quo[ND];
    if (sign == 0)
        return 0.0;
    for (int i = 0; i < 3; ++i)
        num[i] = 0;
    for (int i = 0; i < KM_DIGITS; ++i)
        num[i + 3] = mag[i];
    uint64_t rem = 0;
    for (int i = ND - 1; i >= 0; --i) {
        uint64_t cur = (rem << 32) | num[i];
        quo[i] = (uint32_t)(cur / T);
        rem = cur % T;
    }
#define QBIT(b) ((quo[(b) / 32] >> ((b) % 32)) & 1u)
    int p = ND * 32 - 1;
    while (!QBIT(p))
        --p;
    uint64_t mant = 0;
    for (int b = p; b > p - 53; --b)
        mant = 2 * mant + QBIT(b);
    int guard = (int)QBIT(p - 53);
    int sticky = rem != 0;
    for (int b = p - 54; b >= 0; --b)
        sticky |= (int)QBIT(b);
#undef QBIT
    if (guard && (sticky || (mant & 1u)))
        ++mant;
    /* mant = 2^53 after a carry out is still exact in double */
    double q = ldexp((double)mant, p - 52 - 149 - 96);
    return sign < 0 ? -q : q;
}

/* Per-channel mean of the chunk's keys ([DR] inference: keys are
 * K-smoothed before NVFP4 quantization; the pages give no formula, READING:
 * subtract the per-channel mean over the chunk's tokens).  K is [T, HD]
 * (HD = heads * head_dim, token-major).  mu = (float)RN64(S / T), where S is
 * the exact sum of the channel's T values (no rounding, so no summation
 * order enters), S / T is rounded once to double and that double once to
 * float (READING: the mean is formed in double, as a double sum would give
 * it whenever that sum is exact).  T < 2^31. */
void orc_kv_mean(const float *K, int64_t T, int64_t HD, float *mu)
{
    int64_t *acc = (int64_t *)calloc((size_t)(HD > 0 ? HD : 1) * KM_DIGITS, sizeof(int64_t));
    if (!acc)
        abort();
    for (int64_t t = 0; t < T; ++t)
        for (int64_t ch = 0; ch < HD; ++ch)
            exact_add(acc + ch * KM_DIGITS, K[t * HD + ch]);
    for (int64_t ch = 0; ch < HD; ++ch) {
        uint32_t mag[KM_DIGITS];
        int sign = exact_magnitude(acc + ch * KM_DIGITS, mag);
        mu[ch] = (T > 0) ? (float)exact_quotient(sign, mag, (uint32_t)T) : 0.0f;
    }
    free(acc);
}

/* Quantize one KV chunk independently ([DR]: chunk-level, F_c = 8 frames;
 * [IT]: micro-block scaling with the 4/6 scale search).  K_s = RN(K - mu) and
 * V are each quantized 1-D along the flattened (head, dim) axis with one FP32
 * tensor scale per chunk (READING); V is not smoothed (the pages smooth keys
 * only). */
int orc_kv_encode_chunk(const float *K, const float *V, int64_t T, int64_t HD, int search,
                        uint8_t *kc, uint8_t *ks, float *sdk, uint8_t *vc, uint8_t *vs,
                        float *sdv, float *mu)
{
    float *Ks = (float *)malloc((size_t)(T * HD) * sizeof(float) + 1);
    if (!Ks)
        return -2;
    orc_kv_mean(K, T, HD, mu);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t ch = 0; ch < HD; ++ch)
            Ks[t * HD + ch] = K[t * HD + ch] - mu[ch];
    int rc = orc_quantize(Ks, T, HD, ORC_LAYOUT_1D, search, NULL, kc, ks, sdk, NULL, NULL);
    free(Ks);
    if (rc)
        return rc;
    return orc_quantize(V, T, HD, ORC_LAYOUT_1D, search, NULL, vc, vs, sdv, NULL, NULL);
}

/* Dequantize tokens [tok0, tok0 + ntok) of one encoded chunk to bf16 bits.
 * With mu (keys): K_hat = bf16(RN(x_hat + mu)), the stored mean added back
 * (READING: per-chunk means differ inside one attention window, so dropping
 * them would change q.k across chunks); without: bf16(x_hat). */
void orc_kv_dequant_tokens(const uint8_t *codes, const uint8_t *scales, float s_dec,
                           const float *mu, int64_t tok0, int64_t ntok, int64_t HD,
                           uint16_t *out)
{
    for (int64_t t = 0; t < ntok; ++t)
        for (int64_t ch = 0; ch < HD; ++ch) {
            int64_t r = tok0 + t;
            float xh = orc_dequant_value(code_at(codes, HD, r, ch),
                                         scale_at(scales, HD, ORC_LAYOUT_1D, r, ch), s_dec);
            if (mu)
                xh = xh + mu[ch];
            out[t * HD + ch] = orc_bf16_rne(xh);
        }
}

/* Effective key/value set of the multi-shot attention sink at step t, i.e.
 * while chunk t is generated ([DR] algorithm design; [IT] Multi-Shot
 * Attention Sink): token j (global index) belongs to E(t) iff it is already
 * stored (j < t*Tc) and lies in the global sink A_g = [0, g_tokens), in the
 * current shot's sink A_s = [s_start, s_start + s_tokens), or in the window
 * of the last W chunks [max(0, t-W)*Tc, t*Tc).  Each token appears once and
 * in ascending order.  Writes the tokens when `out` is non-NULL; returns
 * |E(t)|.  Brute force over every stored token. */
int64_t orc_effective_tokens(int64_t t, int64_t Tc, int64_t W, int64_t g_tokens,
                             int64_t s_start, int64_t s_tokens, int64_t *out)
{
    int64_t n = 0;
    int64_t win_lo = (t - W > 0 ? t - W : 0) * Tc;
    for (int64_t j = 0; j < t * Tc; ++j) {
        int in = (j < g_tokens) || (j >= s_start && j < s_start + s_tokens) || (j >= win_lo);
        if (in) {
            if (out)
                out[n] = j;
            ++n;
        }
    }
    return n;
}

/* ------------------------------------------------------------------ */
/* W4A4 GEMM reference                                                 */
/* ------------------------------------------------------------------ */

/* y[m, n] = s_A * s_W * sum_k A_hat[m, k] * W_hat[n, k] in double, with
 * A_hat = V(q) * sigma (1-D scales), W_hat likewise (2-D scales); both are
 * exact in double.  abs_sum gets s_A * s_W * sum_k |A_hat * W_hat| (for the
 * error bound).  Only the rows listed in `rows` (nrows of them) are computed
 * when rows != NULL; output row i corresponds to rows[i].  ([DR] inference:
 * the FP4 GEMM replaces the BF16 GEMM; tensor-wise FP32 scales.) */
int orc_gemm_ref(const uint8_t *a_codes, const uint8_t *a_scales, float a_sdec, int64_t M,
                 int64_t K, const uint8_t *w_codes, const uint8_t *w_scales, float w_sdec,
                 int64_t N, int w_layout, const int64_t *rows, int64_t nrows, double *y,
                 double *abs_sum)
{
    int64_t nr = rows ? nrows : M;
    double *Wd = (double *)malloc((size_t)(N * K) * sizeof(double) + 1);
    double *Ad = (double *)malloc((size_t)K * sizeof(double) + 1);
    if (!Wd || !Ad) {
        free(Wd);
        free(Ad);
        return -2;
    }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            Wd[n * K + k] = (double)orc_e2m1_value(code_at(w_codes, K, n, k)) *
                            (double)orc_e4m3_value(scale_at(w_scales, K, w_layout, n, k));
    double s = (double)a_sdec * (double)w_sdec;
    for (int64_t i = 0; i < nr; ++i) {
        int64_t m = rows ? rows[i] : i;
        if (m < 0 || m >= M) {
            free(Wd);
            free(Ad);
            return -1;
        }
        for (int64_t k = 0; k < K; ++k)
            Ad[k] = (double)orc_e2m1_value(code_at(a_codes, K, m, k)) *
                    (double)orc_e4m3_value(scale_at(a_scales, K, ORC_LAYOUT_1D, m, k));
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            const double *wr = Wd + n * K;
            for (int64_t k = 0; k < K; ++k) {
                double p = Ad[k] * wr[k];
                acc += p;
                aacc += fabs(p);
            }
            y[i * N + n] = s * acc;
            if (abs_sum)
                abs_sum[i * N + n] = s * aacc;
        }
    }
    free(Wd);
    free(Ad);
    return 0;
}

/* Vectorised conveniences for the tests. */
void orc_e2m1_encode_array(const float *y, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e2m1_encode(y[i]);
}

void orc_e4m3_encode_array(const float *t, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode(t[i]);
}

/* ------------------------------------------------------------------ */
/* Random Hadamard transform before quantization                      */
/* ------------------------------------------------------------------ */

/* [DR] NVFP4 training (RHT stabilises the weight-gradient GEMM), [IT]
 * Addestramento NVFP4 (an RHT is applied before quantization on the
 * gradient-sensitive paths).  READING: per 1x16 block along a row,
 * y = (1/4) * H16 * diag(s) * x with H16 the Sylvester Hadamard matrix,
 * H16[i][j] = (-1)^popcount(i & j), and s_j = -1 where bit j of `signs` is
 * set; computed as: sign flips (exact), then the fast Walsh-Hadamard
 * butterflies with strides 1, 2, 4, 8 -- (a, b) -> (RN(a + b), RN(a - b)) --
 * then RN(v * 0.25).  The same transform on both GEMM operands along K
 * leaves the product unchanged ((H S / 4)^T (H S / 4) = I). */
void orc_rht16(const float *x, int64_t R, int64_t C, uint32_t signs, float *out) {
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t b = 0; b < C / 16; ++b) {
            float v[16];
            for (int j = 0; j < 16; ++j) {
                float e = x[r * C + b * 16 + j];
                v[j] = ((signs >> j) & 1u) ? -e : e;
            }
            for (int h = 1; h < 16; h *= 2) {
                for (int j = 0; j < 16; ++j) {
                    if (j & h) continue;
                    float a = v[j], c = v[j + h];
                    v[j] = a + c;
                    v[j + h] = a - c;
                }
            }
            for (int j = 0; j < 16; ++j) out[r * C + b * 16 + j] = v[j] * 0.25f;
        }
    }
}

/* ------------------------------------------------------------------ */
/* LoRA adapter on the frozen NVFP4 backbone                          */
/* ------------------------------------------------------------------ */

/* [DR] Few-step distillation: the trainable model is the frozen quantized
 * backbone plus LoRA adapters, W ~ Dequant(Q_search(W_0)) + dW with
 * dW = (alpha / r) B A; [IT] the distillation trains only the LoRA adapters
 * on the frozen quantized backbone.  Forward through dW for activations x:
 * x dW^T = (alpha / r) (x A^T) B^T.  READING: the adapter branch runs in
 * bf16 like the activations: the down projection x A^T is an fp32 result
 * stored as bf16, XA = bf16(fp32(x A^T)) (each nearest-even; fp32 of the
 * exact dot product here), then (alpha / r) * XA B^T, added to the W4A4
 * product.
 * x [M, K], A [r, K], B [N, r] row-major float32 (bf16 values); `scale` is
 * alpha / r as one float.  y[i, n] and abs_sum[i, n] (optional) for the rows
 * `rows` (or all M); xa [M, r] (optional) receives XA as float. */
int orc_lora_ref(const float *x, const float *a, const float *b, int64_t M, int64_t K,
                 int64_t N, int64_t r, float scale, const int64_t *rows, int64_t nrows,
                 double *y, double *abs_sum, float *xa)
{
    int64_t nr = rows ? nrows : M;
    double *xr = (double *)malloc((size_t)(r > 0 ? r : 1) * sizeof(double));
    if (!xr)
        return -2;
    for (int64_t i = 0; i < nr; ++i) {
        int64_t m = rows ? rows[i] : i;
        if (m < 0 || m >= M) {
            free(xr);
            return -1;
        }
        for (int64_t j = 0; j < r; ++j) {
            double d = 0.0;
            for (int64_t k = 0; k < K; ++k)
                d += (double)x[m * K + k] * (double)a[j * K + k];
            /* the double sum of products of bf16 values is exact unless the
             * exponents differ widely; round it to fp32, then to bf16 */
            float f = (float)d;
            uint16_t hb = orc_bf16_rne(f);
            union {
                uint32_t u;
                float f;
            } cv;
            cv.u = (uint32_t)hb << 16;
            xr[j] = (double)cv.f;
            if (xa)
                xa[m * r + j] = cv.f;
        }
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t j = 0; j < r; ++j) {
                double p = xr[j] * (double)b[n * r + j];
                acc += p;
                aacc += fabs(p);
            }
            y[i * N + n] = (double)scale * acc;
            if (abs_sum)
                abs_sum[i * N + n] = fabs((double)scale) * aacc;
        }
    }
    free(xr);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Attention over the effective key/value set                         */
/* ------------------------------------------------------------------ */

/* [DR] Multi-Shot Attention Sink: each step's sliding-window
 * self-attention runs over the effective set K_eff(t) = A_g u A_s u
 * KV[t-W, t) of dequantized keys and values.  READING: scaled dot-product
 * softmax attention per head,
 *   o[i] = sum_j w_j v[j] / sum_j w_j,  w_j = exp(scale q[i].k[j] - m),
 * m = max_j scale q[i].k[j] (a common factor exp(-m) that cancels), and the
 * log-sum-exp lse[i] = m + log(sum_j w_j); all in double.  q [nq, H, d],
 * k and v [nk, H, d] row-major float32 (bf16 values); o [nq, H, d]; abs_o
 * (optional) receives sum_j w_j |v[j]| / sum_j w_j (the error scale of the
 * weighted sum); lse [nq, H] (optional).  nk == 0 gives o = 0, lse = -inf.
 * `rows` (optional) picks the queries computed: output row i is query
 * rows[i]. */
int orc_attention_ref(const float *q, const float *k, const float *v, int64_t nq, int64_t nk,
                      int64_t H, int64_t d, double scale, const int64_t *rows, int64_t nrows,
                      double *o, double *abs_o, double *lse)
{
    int64_t nr = rows ? nrows : nq;
    double *s = (double *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(double));
    double *acc = (double *)malloc((size_t)(2 * d > 0 ? 2 * d : 1) * sizeof(double));
    if (!s || !acc) {
        free(s);
        free(acc);
        return -2;
    }
    double *aacc = acc + d;
    for (int64_t i = 0; i < nr; ++i) {
        int64_t qi = rows ? rows[i] : i;
        if (qi < 0 || qi >= nq) {
            free(s);
            free(acc);
            return -1;
        }
        for (int64_t h = 0; h < H; ++h) {
            const float *qv = q + (qi * H + h) * d;
            double m = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) {
                const float *kv = k + (j * H + h) * d;
                double dot = 0.0;
                for (int64_t e = 0; e < d; ++e)
                    dot += (double)qv[e] * (double)kv[e];
                s[j] = scale * dot;
                if (s[j] > m)
                    m = s[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            double *out = o + (i * H + h) * d;
            double *aout = abs_o ? abs_o + (i * H + h) * d : NULL;
            /* each element's sum runs over j in order; j is the outer loop
             * only so that the rows of v are read contiguously */
            for (int64_t e = 0; e < d; ++e) {
                acc[e] = 0.0;
                aacc[e] = 0.0;
            }
            for (int64_t j = 0; j < nk; ++j) {
                const float *vr = v + (j * H + h) * d;
                for (int64_t e = 0; e < d; ++e) {
                    double x = (double)vr[e];
                    acc[e] += s[j] * x;
                    aacc[e] += s[j] * fabs(x);
                }
            }
            for (int64_t e = 0; e < d; ++e) {
                out[e] = nk > 0 ? acc[e] / l : 0.0;
                if (aout)
                    aout[e] = nk > 0 ? aacc[e] / l : 0.0;
            }
            if (lse)
                lse[i * H + h] = nk > 0 ? m + log(l) : -INFINITY;
        }
    }
    free(s);
    free(acc);
    return 0;
}
