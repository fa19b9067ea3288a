// gemm.hip -- W4A4 GEMM on NVFP4 operands for gfx950 (MFMA).
//
// Method (LongLive-2.0 pages): "MCISLAB DeepRead: LongLive2" summary, Method /
// inference infrastructure: the generator runs W4A4, FP4 GEMMs replacing the
// BF16 GEMMs; weights use 2-D block scaling, activations 1-D, with a
// tensor-wise FP32 scale on each ("NVFP4 training").
//
// gfx950 has no MFMA that takes an E4M3 scale per 16 elements (its scaled
// FP4 MFMA takes power-of-two E8M0 scales per 32), so each NVFP4 tile is
// expanded exactly and fed to the fp16 MFMA (same dense rate as bf16):
//   A_hat = V(code) * sigma,  sigma = 2^E * F  (E4M3: F = 1 + m/8, or m for a
//   subnormal with E = -9).  v_cvt_scalef32_pk_f16_fp4 gives V * 2^E exactly,
//   one packed fp16 multiply by F gives V * sigma exactly (at most 6
//   significant bits, magnitude in [2^-10, 2688]: exact in fp16, as in bf16).
// The FP32 tensor scales are applied once in the epilogue:
//   Y = RN(RN(s_A * s_W) * acc), acc the fp32 MFMA accumulation.
//
// Tiling: workgroup 256 threads = 4 waves (2 x 2), output tile BM x BN =
// 256 x 256, K step 64.  Each wave owns a 128 x 128 sub-tile = 4 x 4 blocks
// of v_mfma_f32_32x32x16_f16 (256 fp32 accumulators per lane).  Every packed
// tile is expanded once per workgroup into LDS as fp16 (row stride 72 halfs:
// the 16-byte fragment reads of 16 consecutive rows hit disjoint banks), two
// LDS stages: while the MFMAs consume stage k, the packed tile k+1 (already in
// registers) is expanded into the other stage and tile k+2 is fetched.
#include "device.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // halfs per row
constexpr int WM = BM / 2, WN = BN / 2;
constexpr int FM = WM / 32, FN = WN / 32;  // MFMA blocks per wave

// Expand 8 codes (one dword) to 8 fp16 values V * sigma: the hardware
// converter gives V exactly in fp16 (scale 1), one packed multiply by the
// block scale sigma (exact in fp16: E4M3 values lie in [2^-9, 448]) gives
// V * sigma exactly.
__device__ __forceinline__ f16x8 expand8(uint32_t w, f16x2 sig) {
    f16x8 o;
    f16x2 t;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sig; o[0] = t.x; o[1] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sig; o[2] = t.x; o[3] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sig; o[4] = t.x; o[5] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sig; o[6] = t.x; o[7] = t.y;
    return o;
}

// One thread's share of staging one K step: for each of 4 "parts" (A rows
// lrow and lrow + 128, W rows lrow and lrow + 128), 32 consecutive K elements
// = 2 blocks = 16 code bytes + 2 scale bytes.
struct Part {
    u32x4 q;
    uint32_t sc;  // two E4M3 scale bytes in the low 16 bits
};

struct GemmArgs {
    const uint8_t *a_codes, *a_scales, *w_codes, *w_scales;
    int64_t M, N, K;
};

// Per-thread source pointers of the 4 parts at K step 0 (rows clamped into
// range; edge tiles mask them later).
struct PartPtrs {
    const uint8_t *c[4];
    const uint8_t *s[4];
    uint32_t rowmask[4];  // ~0 if the part's row exists, else 0
};

__device__ __forceinline__ void part_ptrs(PartPtrs &pp, const GemmArgs &g, int64_t m0, int64_t n0,
                                          int tid) {
    const int64_t KB = g.K >> 4, kbytes = g.K >> 1;
    const int lrow = tid >> 1, kseg = (tid & 1) * 32;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const bool isA = p < 2;
        const int64_t rows = isA ? g.M : g.N;
        const int64_t r = (isA ? m0 : n0) + lrow + (p & 1) * 128;
        const int64_t rc = r < rows ? r : rows - 1;
        const int64_t srow = isA ? rc : (rc >> 4);
        pp.c[p] = (isA ? g.a_codes : g.w_codes) + rc * kbytes + kseg / 2;
        pp.s[p] = (isA ? g.a_scales : g.w_scales) + srow * KB + kseg / 16;
        pp.rowmask[p] = r < rows ? ~0u : 0u;
    }
}

// Fetch part P of K step kt.  Fast path (EDGE = false): the whole tile lies
// inside the matrices and K % 64 == 0.  Edge path: clamped, in-bounds loads,
// codes of missing rows or blocks zeroed (code 0 is +0 whatever the scale).
template <int P, bool EDGE>
__device__ __forceinline__ void fetch_part(Part &pt, const PartPtrs &pp, const GemmArgs &g,
                                           int64_t kt, int tid) {
    if (!EDGE) {
        pt.q = *(const u32x4 *)(pp.c[P] + kt * (BK / 2));
        pt.sc = *(const uint16_t *)(pp.s[P] + kt * (BK / 16));
        return;
    }
    const int64_t KB = g.K >> 4;
    const int64_t kb0 = kt * (BK / 16) + (tid & 1) * 2;  // first of the two blocks
    const bool b0 = kb0 < KB, b1 = kb0 + 1 < KB;
    // base pointers address block (tid & 1) * 2 of K step 0
    const int64_t kbc = b1 ? kb0 : (KB >= 2 ? KB - 2 : 0);
    const int64_t dblk = kbc - (tid & 1) * 2;  // blocks from the base pointer
    u32x4 q;
    uint32_t sc;
    if (KB >= 2) {
        q = *(const u32x4 *)(pp.c[P] + dblk * 8);
        sc = (uint32_t)pp.s[P][dblk] | ((uint32_t)pp.s[P][dblk + 1] << 8);
    } else {
        const uint2 q2 = *(const uint2 *)(pp.c[P] + dblk * 8);
        q = u32x4{q2.x, q2.y, 0u, 0u};
        sc = pp.s[P][dblk];
    }
    const bool up = KB >= 2 && !b1;  // only the last block is valid: it is in the upper half
    const uint32_t m0k = b0 ? pp.rowmask[P] : 0u, m1k = b1 ? pp.rowmask[P] : 0u;
    pt.q = u32x4{(up ? q.z : q.x) & m0k, (up ? q.w : q.y) & m0k, q.z & m1k, q.w & m1k};
    pt.sc = up ? (sc >> 8) : sc;
}

template <int P>
__device__ __forceinline__ void expand_part(const Part &pt, _Float16 *stage, int tid) {
    const int lrow = tid >> 1, kseg = (tid & 1) * 32;
    _Float16 *d = stage + ((P >= 2 ? BM : 0) + lrow + (P & 1) * 128) * LDS_STRIDE + kseg;
    const f16x2 sg = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pt.sc, 1.0f, false);
    const f16x2 s0 = f16x2{sg.x, sg.x}, s1 = f16x2{sg.y, sg.y};
    *(f16x8 *)(d) = expand8(pt.q.x, s0);
    *(f16x8 *)(d + 8) = expand8(pt.q.y, s0);
    *(f16x8 *)(d + 16) = expand8(pt.q.z, s1);
    *(f16x8 *)(d + 24) = expand8(pt.q.w, s1);
}

template <bool OUT_BF16, bool EDGE>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, const float *__restrict__ a_sdec,
                                          const float *__restrict__ w_sdec, void *__restrict__ yv,
                                          _Float16 *lds, int64_t m0, int64_t n0) {
    auto stage = [&](int s) { return lds + s * (BM + BN) * LDS_STRIDE; };
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = g.M, N = g.N, K = g.K;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nk = (K + BK - 1) / BK;
    PartPtrs pp;
    part_ptrs(pp, g, m0, n0, tid);
    Part p0, p1, p2, p3;
    fetch_part<0, EDGE>(p0, pp, g, 0, tid);
    fetch_part<1, EDGE>(p1, pp, g, 0, tid);
    fetch_part<2, EDGE>(p2, pp, g, 0, tid);
    fetch_part<3, EDGE>(p3, pp, g, 0, tid);
    expand_part<0>(p0, stage(0), tid);
    expand_part<1>(p1, stage(0), tid);
    expand_part<2>(p2, stage(0), tid);
    expand_part<3>(p3, stage(0), tid);
    // the fast path never reads past the last K step
    const int64_t last = EDGE ? (int64_t)1 << 40 : nk - 1;
    fetch_part<0, EDGE>(p0, pp, g, 1 < last ? 1 : last, tid);
    fetch_part<1, EDGE>(p1, pp, g, 1 < last ? 1 : last, tid);
    fetch_part<2, EDGE>(p2, pp, g, 1 < last ? 1 : last, tid);
    fetch_part<3, EDGE>(p3, pp, g, 1 < last ? 1 : last, tid);
    __syncthreads();

    const int frow = lane & 31, fk = (lane >> 5) * 8;
    const int aoff = (wm * WM + frow) * LDS_STRIDE + fk;
    const int woff = (BM + wn * WN + frow) * LDS_STRIDE + fk;
    f16x8 fa[2][FM], fb[2][FN];
    {
        const _Float16 *S = stage(0);
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[0][i] = *(const f16x8 *)(S + aoff + i * 32 * LDS_STRIDE);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[0][j] = *(const f16x8 *)(S + woff + j * 32 * LDS_STRIDE);
    }
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const _Float16 *S = stage(cur);
        _Float16 *Nx = stage(cur ^ 1);
        // K step fetched this iteration (past the end: clamped on the fast
        // path, zeroed on the edge path; either way never used)
        const int64_t kf = (kt + 2 < last) ? kt + 2 : last;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int c = kk & 1;
            if (kk < 3) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    fa[c ^ 1][i] = *(const f16x8 *)(S + aoff + i * 32 * LDS_STRIDE + (kk + 1) * 16);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    fb[c ^ 1][j] = *(const f16x8 *)(S + woff + j * 32 * LDS_STRIDE + (kk + 1) * 16);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[c][i], fb[c][j],
                                                                       acc[i][j], 0, 0, 0);
            // stage the next K step (harmless past the end of K)
            if (kk == 0) { expand_part<0>(p0, Nx, tid); fetch_part<0, EDGE>(p0, pp, g, kf, tid); }
            if (kk == 1) { expand_part<1>(p1, Nx, tid); fetch_part<1, EDGE>(p1, pp, g, kf, tid); }
            if (kk == 2) { expand_part<2>(p2, Nx, tid); fetch_part<2, EDGE>(p2, pp, g, kf, tid); }
            if (kk == 3) { expand_part<3>(p3, Nx, tid); fetch_part<3, EDGE>(p3, pp, g, kf, tid); }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[0][i] = *(const f16x8 *)(Nx + aoff + i * 32 * LDS_STRIDE);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[0][j] = *(const f16x8 *)(Nx + woff + j * 32 * LDS_STRIDE);
    }

    const float scale = (*a_sdec) * (*w_sdec);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t col = n0 + wn * WN + j * 32 + (lane & 31);
            const int64_t rbase = m0 + wm * WM + i * 32 + (lane >> 5) * 4;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = rbase + (r >> 2) * 8 + (r & 3);
                const float v = scale * acc[i][j][r];
                if (!EDGE || (row < M && col < N)) {
                    if (OUT_BF16)
                        ((__bf16 *)yv)[row * N + col] = (__bf16)v;
                    else
                        ((float *)yv)[row * N + col] = v;
                }
            }
        }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_w4a4_kernel(GemmArgs g, const float *__restrict__ a_sdec,
                                                        const float *__restrict__ w_sdec,
                                                        void *__restrict__ yv) {
    extern __shared__ __attribute__((aligned(16))) _Float16 lds[];
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const bool interior = (m0 + BM <= g.M) && (n0 + BN <= g.N) && (g.K % BK == 0);
    if (interior)
        gemm_tile<OUT_BF16, false>(g, a_sdec, w_sdec, yv, lds, m0, n0);
    else
        gemm_tile<OUT_BF16, true>(g, a_sdec, w_sdec, yv, lds, m0, n0);
}

constexpr size_t kLdsBytes = (size_t)2 * (BM + BN) * LDS_STRIDE * sizeof(_Float16);

hipError_t launch_gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_sdec,
                            const uint8_t *w_codes, const uint8_t *w_scales,
                            const float *w_sdec, int64_t M, int64_t N, int64_t K, void *y,
                            int ydtype, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    static bool attr_set = false;
    if (!attr_set) {
        const void *fns[2] = {(const void *)gemm_w4a4_kernel<true>,
                              (const void *)gemm_w4a4_kernel<false>};
        for (const void *f : fns) {
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)kLdsBytes);
            if (e != hipSuccess) return e;
        }
        attr_set = true;
    }
    dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    GemmArgs g{a_codes, a_scales, w_codes, w_scales, M, N, K};
    if (ydtype == kBF16)
        NVFP4_LAUNCH("gemm_w4a4", gemm_w4a4_kernel<true>, grid, dim3(256), kLdsBytes, s, g,
                     a_sdec, w_sdec, y);
    else
        NVFP4_LAUNCH("gemm_w4a4", gemm_w4a4_kernel<false>, grid, dim3(256), kLdsBytes, s, g,
                     a_sdec, w_sdec, y);
    return hipGetLastError();
}

}  // namespace nvfp4
