// device.hpp -- gfx950 device helpers shared by the libnvfp4 kernels.
//
// Formats (LongLive-2.0 pages: "MCISLAB DeepRead: LongLive2" summary, Method /
// NVFP4 training -- E2M1 elements, FP8 E4M3 block scales, FP32 tensor scale):
//   E2M1 nibble  s e1 e0 m, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
//   E4M3FN byte  bias 7, max 448 (0x7E), subnormals m * 2^-9
//
// The conversions use gfx950's hardware converters.  Their behaviour was
// checked exhaustively on an MI355X against bit-exact software definitions:
// v_cvt_scalef32_pk_fp4_f32 (scale 1.0) is E2M1 round-to-nearest-even with
// saturation at 6 and a signed zero, over every non-NaN float;
// v_cvt_pk_fp8_f32 is E4M3FN round-to-nearest-even for 0 <= t < 448; the
// float -> bf16 conversion (v_cvt_pk_bf16_f32) is round-to-nearest-even.
// The fp4 -> f32/f16 converters take only the exponent of their scale
// operand (a power of two).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw (untyped) buffer descriptor on CDNA: 32-bit data format,
// no swizzle, no index stride.
constexpr int kBufferWord3 = 0x00020000;

// Largest E2M1 magnitude times largest E4M3 magnitude: the tensor amax maps to it.
constexpr float kTensorTarget = 2688.0f;  // 6 * 448

// ---------------------------------------------------------------------------
// scalar formats
// ---------------------------------------------------------------------------

// Value of a non-negative E4M3FN scale byte.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// E4M3FN byte of t >= 0: nearest-even, saturating to 448 (0x7E) for t >= 448.
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
    uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, t, 0, false) & 0xFFu;
    return (t < 448.0f) ? c : 0x7Eu;
}

// Tensor scales from the tensor amax: s_enc = RN(2688 / amax), s_dec = RN(amax / 2688);
// an all-zero tensor gets 1 and 1.  Correctly rounded divisions.
__device__ __forceinline__ void tensor_scales(float amax, float &s_enc, float &s_dec) {
    if (amax == 0.0f) {
        s_enc = 1.0f;
        s_dec = 1.0f;
    } else {
        s_enc = __fdiv_rn(kTensorTarget, amax);
        s_dec = __fdiv_rn(amax, kTensorTarget);
    }
}

// ---------------------------------------------------------------------------
// E2M1 pack / unpack (8 values <-> one dword, element 2j in bits 8j..8j+3)
// ---------------------------------------------------------------------------

// Codes of y_i = RN(x_i * r), i = 0..7.
__device__ __forceinline__ uint32_t e2m1_pack8(const float (&x)[8], float r) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0] * r, x[1] * r, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2] * r, x[3] * r, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4] * r, x[5] * r, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6] * r, x[7] * r, 1.0f, 3);
    return w;
}

// Signed E2M1 values of byte `sel` of w (low nibble first).
template <int SEL>
__device__ __forceinline__ f32x2 e2m1_unpack2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Sum over i = 0..7 of RN(x_i - V(q_i) * S)^2 as the fma chain acc <- d*d + acc from +0.
__device__ __forceinline__ float half_block_error(const float (&x)[8], uint32_t q, float S) {
    float acc = 0.0f;
    f32x2 v;
#define NVFP4_ERR_PAIR(SEL)                          \
    v = e2m1_unpack2<SEL>(q);                        \
    {                                                \
        float d0 = __builtin_fmaf(-v.x, S, x[2 * SEL]);     \
        acc = __builtin_fmaf(d0, d0, acc);                  \
        float d1 = __builtin_fmaf(-v.y, S, x[2 * SEL + 1]); \
        acc = __builtin_fmaf(d1, d1, acc);                  \
    }
    NVFP4_ERR_PAIR(0)
    NVFP4_ERR_PAIR(1)
    NVFP4_ERR_PAIR(2)
    NVFP4_ERR_PAIR(3)
#undef NVFP4_ERR_PAIR
    return acc;
}

// RN(a / 6) for a >= 0.  For a >= 2^-125, q = RN(a * RN(1/6)) corrected once
// by the exact residual fma(-q, 6, a) is the correctly rounded quotient
// (checked exhaustively over every float in [2^-125, FLT_MAX]); smaller a
// (quotient near or below the subnormal range) takes the IEEE division.
__device__ __forceinline__ float div6_rn(float a) {
    const float c = 0.16666667f;  // RN(1/6)
    const float q0 = a * c;
    const float r = __builtin_fmaf(-q0, 6.0f, a);
    float q = __builtin_fmaf(r, c, q0);
    // the division is skipped by the whole wave unless one of its lanes needs it
    if (__builtin_amdgcn_ballot_w64(a < 0x1p-125f)) q = (a < 0x1p-125f) ? a / 6.0f : q;
    return q;
}

// ---------------------------------------------------------------------------
// random Hadamard transform of one 1x16 block held by one lane
// ---------------------------------------------------------------------------

// (1/4) H16 diag(s) v: bit j of `signs` flips element j (exact), then the
// fast Walsh-Hadamard butterflies with strides 1, 2, 4, 8 -- (a, b) ->
// (RN(a + b), RN(a - b)) -- then RN(v * 0.25).  H16 is the Sylvester
// Hadamard matrix (entry (i, j) = (-1)^popcount(i & j)).
__device__ __forceinline__ void rht16(float (&v)[16], uint32_t signs) {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = ((signs >> j) & 1u) ? -v[j] : v[j];
#pragma unroll
    for (int h = 1; h < 16; h *= 2)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j & h) continue;
            const float a = v[j], c = v[j + h];
            v[j] = a + c;
            v[j + h] = a - c;
        }
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = v[j] * 0.25f;
}

// ---------------------------------------------------------------------------
// one 1x16 block held by one lane: the Four-Over-Six encoder
// ---------------------------------------------------------------------------

// Per-scale-code table entry: (S, r) with S = RN(sigma * s_dec) and
// r = RN(1 / S) (0 when S == 0), sigma the E4M3 value of the code.
__device__ __forceinline__ f32x2 scale_entry(uint32_t code, float s_dec) {
    const float S = e4m3_value(code) * s_dec;
    return f32x2{S, (S == 0.0f) ? 0.0f : 1.0f / S};
}

// Encode x_0..x_15 for the tensor encode scale s_enc.  For each target c in
// {6, 4}: scale code E4M3(RN(RN(amax / c) * s_enc)), codes E2M1(RN(x * r)),
// error RN(E_lo + E_hi) with E_lo / E_hi the fma chains of RN(x - V*S)^2
// over elements 0..7 / 8..15; target 4 is kept only if its error is lower.
// Codes of elements 0..7 go to q_lo, 8..15 to q_hi (element 2j in the low
// nibble of byte j).
template <bool FOUR_OVER_SIX>
__device__ __forceinline__ void encode_block16(const float (&x)[16], float s_enc,
                                               const f32x2 *lut, uint32_t &q_lo, uint32_t &q_hi,
                                               uint32_t &scale) {
    const float(&xl)[8] = *reinterpret_cast<const float(*)[8]>(&x[0]);
    const float(&xh)[8] = *reinterpret_cast<const float(*)[8]>(&x[8]);
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(x[i]));
    const uint32_t sc6 = e4m3_encode(div6_rn(am) * s_enc);
    const f32x2 sr6 = lut[sc6];
    const uint32_t a6 = e2m1_pack8(xl, sr6.y), b6 = e2m1_pack8(xh, sr6.y);
    if (!FOUR_OVER_SIX) {
        q_lo = a6;
        q_hi = b6;
        scale = sc6;
        return;
    }
    const float e6 = half_block_error(xl, a6, sr6.x) + half_block_error(xh, b6, sr6.x);
    const uint32_t sc4 = e4m3_encode((am * 0.25f) * s_enc);
    const f32x2 sr4 = lut[sc4];
    const uint32_t a4 = e2m1_pack8(xl, sr4.y), b4 = e2m1_pack8(xh, sr4.y);
    const float e4 = half_block_error(xl, a4, sr4.x) + half_block_error(xh, b4, sr4.x);
    const bool pick4 = e4 < e6;
    q_lo = pick4 ? a4 : a6;
    q_hi = pick4 ? b4 : b6;
    scale = pick4 ? sc4 : sc6;
}

// ---------------------------------------------------------------------------
// lane exchange
// ---------------------------------------------------------------------------

// Value of the neighbouring lane (lane ^ 1), via DPP quad_perm [1,0,3,2].
__device__ __forceinline__ float swap_pair(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// ---------------------------------------------------------------------------
// bf16 / f32 helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats to packed bf16 (nearest-even), a in the low half: one
// v_cvt_pk_bf16_f32 with both sources.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
    uint32_t u;
    __builtin_memcpy(&u, &v, 4);
    return u;
}

// Raw 16-element block loads (16 bf16 = 2 x 16 B, 16 float = 4 x 16 B).
struct Raw16Bf16 {
    u32x4 a, b;
};
struct Raw16F32 {
    f32x4 a, b, c, d;
};
__device__ __forceinline__ void load_raw16(const uint16_t *p, Raw16Bf16 &r) {
    r.a = *(const u32x4 *)p;
    r.b = *(const u32x4 *)(p + 8);
}
__device__ __forceinline__ void load_raw16(const float *p, Raw16F32 &r) {
    r.a = *(const f32x4 *)p;
    r.b = *(const f32x4 *)(p + 4);
    r.c = *(const f32x4 *)(p + 8);
    r.d = *(const f32x4 *)(p + 12);
}
__device__ __forceinline__ void unpack16(const Raw16Bf16 &r, float (&x)[16]) {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[2 * i] = bf16lo(w[i]);
        x[2 * i + 1] = bf16hi(w[i]);
    }
}
__device__ __forceinline__ void unpack16(const Raw16F32 &r, float (&x)[16]) {
    const f32x4 v[4] = {r.a, r.b, r.c, r.d};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[4 * i] = v[i].x;
        x[4 * i + 1] = v[i].y;
        x[4 * i + 2] = v[i].z;
        x[4 * i + 3] = v[i].w;
    }
}
// The same blocks by raw buffer loads at byte offset `off` (a block past the
// descriptor's end reads as zero).
__device__ __forceinline__ void buffer_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off,
                                              Raw16Bf16 &r) {
    r.a = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    r.b = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0);
}
__device__ __forceinline__ void buffer_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off,
                                              Raw16F32 &r) {
    r.a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    r.b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0));
    r.c = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32, 0, 0));
    r.d = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 48, 0, 0));
}

template <typename T> struct Raw16Of;
template <> struct Raw16Of<uint16_t> { typedef Raw16Bf16 type; };
template <> struct Raw16Of<float> { typedef Raw16F32 type; };

// Load 8 consecutive elements as float.
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    f32x4 a = *(const f32x4 *)p;
    f32x4 b = *(const f32x4 *)(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void load8(const uint16_t *p, float (&x)[8]) {
    u32x4 w = *(const u32x4 *)p;
    x[0] = bf16lo(w.x); x[1] = bf16hi(w.x);
    x[2] = bf16lo(w.y); x[3] = bf16hi(w.y);
    x[4] = bf16lo(w.z); x[5] = bf16hi(w.z);
    x[6] = bf16lo(w.w); x[7] = bf16hi(w.w);
}

__device__ __forceinline__ void store8(float *p, const float (&y)[8]) {
    *(f32x4 *)p = f32x4{y[0], y[1], y[2], y[3]};
    *(f32x4 *)(p + 4) = f32x4{y[4], y[5], y[6], y[7]};
}

__device__ __forceinline__ void store8(uint16_t *p, const float (&y)[8]) {
    *(u32x4 *)p = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                        pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
}

// The same as a non-temporal (streaming) store: the line is not kept dirty
// in the caches for a later write-back.
__device__ __forceinline__ void store8_stream(uint16_t *p, const float (&y)[8]) {
    const u32x4 v = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                          pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
    __builtin_nontemporal_store(v, (u32x4 *)p);
}

// x_hat_i = RN(V(q_i) * S) for the 8 codes of dword q.
__device__ __forceinline__ void dequant8(uint32_t q, float S, float (&y)[8]) {
    f32x2 v;
    v = e2m1_unpack2<0>(q); y[0] = v.x * S; y[1] = v.y * S;
    v = e2m1_unpack2<1>(q); y[2] = v.x * S; y[3] = v.y * S;
    v = e2m1_unpack2<2>(q); y[4] = v.x * S; y[5] = v.y * S;
    v = e2m1_unpack2<3>(q); y[6] = v.x * S; y[7] = v.y * S;
}

}  // namespace nvfp4
