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
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Two floats to packed bf16 (nearest-even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    __bf16 ha = (__bf16)a, hb = (__bf16)b;
    unsigned short ua, ub;
    __builtin_memcpy(&ua, &ha, 2);
    __builtin_memcpy(&ub, &hb, 2);
    return (uint32_t)ua | ((uint32_t)ub << 16);
}

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

// x_hat_i = RN(V(q_i) * S) for the 8 codes of dword q.
__device__ __forceinline__ void dequant8(uint32_t q, float S, float (&y)[8]) {
    f32x2 v;
    v = e2m1_unpack2<0>(q); y[0] = v.x * S; y[1] = v.y * S;
    v = e2m1_unpack2<1>(q); y[2] = v.x * S; y[3] = v.y * S;
    v = e2m1_unpack2<2>(q); y[4] = v.x * S; y[5] = v.y * S;
    v = e2m1_unpack2<3>(q); y[6] = v.x * S; y[7] = v.y * S;
}

}  // namespace nvfp4
