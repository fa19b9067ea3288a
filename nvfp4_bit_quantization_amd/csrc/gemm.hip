// gemm.hip -- W4A4 GEMM on NVFP4 operands for gfx950 (MFMA).
//
// Method (LongLive-2.0 pages): "MCISLAB DeepRead: LongLive2" summary, Method /
// inference infrastructure: the generator runs W4A4, FP4 GEMMs replacing the
// BF16 GEMMs; weights use 2-D block scaling, activations 1-D, with a
// tensor-wise FP32 scale on each ("NVFP4 training").
//
// gfx950 has no MFMA that takes an E4M3 scale per 16 elements (its scaled
// FP4 MFMA takes power-of-two E8M0 scales per 32), so each NVFP4 tile is
// expanded exactly in registers and fed to the fp16 MFMA:
//   A_hat = V(code) * sigma,  sigma = 2^E * F  (E4M3: F = 1 + m/8, or m for a
//   subnormal with E = -9).  v_cvt_scalef32_pk_f16_fp4 gives V * 2^E exactly,
//   one packed fp16 multiply by F gives V * sigma exactly (at most 6
//   significant bits, magnitude in [2^-10, 2688]: exact in fp16, as in bf16).
// The FP32 tensor scales are applied once in the epilogue:
//   Y = RN(RN(s_A * s_W) * acc), acc the fp32 MFMA accumulation.
//
// Tiling: workgroup 256 threads = 4 waves, output tile 128 x 128, K step 64;
// each wave owns a 64 x 64 sub-tile = 2 x 2 MFMA 32x32x16 blocks.  The packed
// tiles are expanded to fp16 in LDS (row stride 72 halfs to spread banks).
#include "device.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // halfs

// sigma = pow2 * F for a non-negative E4M3 byte; F as a packed fp16 pair.
__device__ __forceinline__ void e4m3_split(uint32_t c, float &pow2, f16x2 &F) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    if (e) {
        pow2 = __uint_as_float((e + 120u) << 23);
        const uint16_t fb = (uint16_t)(0x3C00u | (m << 7));
        _Float16 f;
        __builtin_memcpy(&f, &fb, 2);
        F = f16x2{f, f};
    } else {
        pow2 = __uint_as_float(118u << 23);  // 2^-9
        const _Float16 f = (_Float16)(float)m;
        F = f16x2{f, f};
    }
}

// Expand one 16-element block (two code dwords) to 16 fp16 values in `dst`.
__device__ __forceinline__ void expand_block(uint32_t w0, uint32_t w1, uint32_t sc,
                                             _Float16 *dst) {
    float p2;
    f16x2 F;
    e4m3_split(sc, p2, F);
    f16x8 lo, hi;
    f16x2 t;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, p2, 0) * F; lo[0] = t.x; lo[1] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, p2, 1) * F; lo[2] = t.x; lo[3] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, p2, 2) * F; lo[4] = t.x; lo[5] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, p2, 3) * F; lo[6] = t.x; lo[7] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, p2, 0) * F; hi[0] = t.x; hi[1] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, p2, 1) * F; hi[2] = t.x; hi[3] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, p2, 2) * F; hi[4] = t.x; hi[5] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, p2, 3) * F; hi[6] = t.x; hi[7] = t.y;
    *(f16x8 *)dst = lo;
    *(f16x8 *)(dst + 8) = hi;
}

__device__ __forceinline__ void zero_block(_Float16 *dst) {
    *(f16x8 *)dst = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    *(f16x8 *)(dst + 8) = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_w4a4_kernel(
    const uint8_t *__restrict__ a_codes, const uint8_t *__restrict__ a_scales,
    const float *__restrict__ a_sdec, const uint8_t *__restrict__ w_codes,
    const uint8_t *__restrict__ w_scales, const float *__restrict__ w_sdec, int64_t M,
    int64_t N, int64_t K, void *__restrict__ yv) {
    __shared__ __attribute__((aligned(16))) _Float16 As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) _Float16 Ws[BN * LDS_STRIDE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int64_t KB = K >> 4;       // 16-element blocks along K
    const int64_t kbytes = K >> 1;   // code bytes per row

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // loader: thread -> tile row (tid / 2), 32-element half of the K step
    const int lrow = tid >> 1, lseg = (tid & 1) * 32;
    const int64_t arow = m0 + lrow, wrow = n0 + lrow;
    const bool a_ok = arow < M, w_ok = wrow < N;

    for (int64_t k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int64_t kb = (k0 + lseg) / 16 + b;  // block index along K
            _Float16 *ad = &As[lrow * LDS_STRIDE + lseg + b * 16];
            _Float16 *wd = &Ws[lrow * LDS_STRIDE + lseg + b * 16];
            if (a_ok && kb < KB) {
                const uint32_t *src = (const uint32_t *)(a_codes + arow * kbytes + kb * 8);
                expand_block(src[0], src[1], a_scales[arow * KB + kb], ad);
            } else {
                zero_block(ad);
            }
            if (w_ok && kb < KB) {
                const uint32_t *src = (const uint32_t *)(w_codes + wrow * kbytes + kb * 8);
                expand_block(src[0], src[1], w_scales[(wrow >> 4) * KB + kb], wd);
            } else {
                zero_block(wd);
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            f16x8 af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *(const f16x8 *)&As[(wm * 64 + i * 32 + (lane & 31)) * LDS_STRIDE + kk +
                                            (lane >> 5) * 8];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[j] = *(const f16x8 *)&Ws[(wn * 64 + j * 32 + (lane & 31)) * LDS_STRIDE + kk +
                                            (lane >> 5) * 8];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0,
                                                                       0, 0);
        }
        __syncthreads();
    }

    const float scale = (*a_sdec) * (*w_sdec);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (row < M && col < N) {
                    const float v = scale * acc[i][j][r];
                    if (OUT_BF16) {
                        __bf16 h = (__bf16)v;
                        ((__bf16 *)yv)[row * N + col] = h;
                    } else {
                        ((float *)yv)[row * N + col] = v;
                    }
                }
            }
        }
}

hipError_t launch_gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_sdec,
                            const uint8_t *w_codes, const uint8_t *w_scales,
                            const float *w_sdec, int64_t M, int64_t N, int64_t K, void *y,
                            int ydtype, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    if (ydtype == kBF16)
        NVFP4_LAUNCH("gemm_w4a4", gemm_w4a4_kernel<true>, grid, dim3(256), 0, s, a_codes, a_scales,
                           a_sdec, w_codes, w_scales, w_sdec, M, N, K, y);
    else
        NVFP4_LAUNCH("gemm_w4a4", gemm_w4a4_kernel<false>, grid, dim3(256), 0, s, a_codes, a_scales,
                           a_sdec, w_codes, w_scales, w_sdec, M, N, K, y);
    return hipGetLastError();
}

}  // namespace nvfp4
