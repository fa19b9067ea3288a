// quantize.hip -- NVFP4 quantize / dequantize kernels for gfx950.
//
// Method (LongLive-2.0 pages): "MCISLAB DeepRead: LongLive2" summary, Method /
// NVFP4 training: E2M1 elements with block FP8 E4M3 and tensor FP32 scaling,
// 2-D block scaling for weights and 1-D for activations; few-step
// distillation: the adaptive block scaling evaluates target magnitudes 6 and
// 4 per block and keeps the lower-error encoding (also the ngjoo.com audit's
// claim list, and "Inferenza W4A4 NVFP4" on the Italian page: Four Over Six).
//
// Work split (HBM-bound streaming; one pass for the tensor amax, one for the
// encode):
//   amax_kernel      16-byte loads, grid-stride, one partial max per workgroup
//   encode1d_kernel  one lane per 1x16 block (encode_block16: both
//                    candidates in registers), two blocks in flight, raw
//                    buffer loads and stores
//   encode2d_kernel  32 lanes own a 16x16 tile (lane pair = tile row)
//   dequant_kernel   16 output bytes per lane (one 16-byte store)
#include "device.hpp"
#include "launch.hpp"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// Tensor amax partials
// ---------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(256) void amax_kernel(const T *__restrict__ x, int64_t n8,
                                                   float *__restrict__ partials) {
    float m = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n8; u += 4 * stride) {
        float v[4][8];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (u + k * stride < n8) load8(x + (u + k * stride) * 8, v[k]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (u + k * stride < n8)
#pragma unroll
                for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[k][i]));
    }
    m = wave_max(m);
    __shared__ float red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        partials[blockIdx.x] = r;
    }
}

// Amax partials of the random-Hadamard-transformed tensor: one lane per 1x16
// block, two blocks in flight.
template <typename T>
__global__ __launch_bounds__(256) void amax_rht_kernel(const T *__restrict__ x, int64_t nblk,
                                                       uint32_t signs,
                                                       float *__restrict__ partials) {
    typedef typename Raw16Of<T>::type Raw;
    float m = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += 2 * stride) {
        const int64_t b2 = b + stride;
        Raw r0, r1;
        load_raw16(x + b * 16, r0);
        if (b2 < nblk) load_raw16(x + b2 * 16, r1);
        float v[16];
        unpack16(r0, v);
        rht16(v, signs);
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
        if (b2 < nblk) {
            unpack16(r1, v);
            rht16(v, signs);
#pragma unroll
            for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
        }
    }
    m = wave_max(m);
    __shared__ float red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) partials[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// This thread's first four amax partials (i, i + blockDim, ...; zero past
// `np`), loaded together; nothing is loaded when the amax is given.  Issued
// before a kernel's first data loads: the loads return in order, so partials
// requested after the data would wait for the data too.
struct Partials4 {
    float a, b, c, d;
};
__device__ __forceinline__ Partials4 partials_issue(const float *__restrict__ partials, int np,
                                                    const float *__restrict__ amax_in) {
    Partials4 p{0.0f, 0.0f, 0.0f, 0.0f};
    if (amax_in) return p;
    const int st = (int)blockDim.x, i = (int)threadIdx.x;
    if (i < np) p.a = partials[i];
    if (i + st < np) p.b = partials[i + st];
    if (i + 2 * st < np) p.c = partials[i + 2 * st];
    if (i + 3 * st < np) p.d = partials[i + 3 * st];
    return p;
}

// Reduce `np` partial maxima (the first four per thread already loaded in
// `p`; or take *amax_in), derive the tensor scales and build the
// per-scale-code table (S, r): S = RN(sigma * s_dec), r = RN(1 / S) (0 when
// S == 0).  Called by every workgroup of the encode kernels.
__device__ __forceinline__ void encode_prologue(const Partials4 &p,
                                                const float *__restrict__ partials, int np,
                                                const float *__restrict__ amax_in,
                                                float *__restrict__ s_dec_out, f32x2 *lut,
                                                float &s_enc_out) {
    __shared__ float red[4];
    __shared__ float sh_enc;
    __shared__ float sh_dec;
    float m = 0.0f;
    if (amax_in) {
        m = *amax_in;
    } else {
        m = fmaxf(fmaxf(p.a, p.b), fmaxf(p.c, p.d));
        const int st = (int)blockDim.x;
        for (int i = threadIdx.x + 4 * st; i < np; i += st) m = fmaxf(m, partials[i]);
        m = wave_max(m);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = red[0];
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) a = fmaxf(a, red[w]);
        float se, sd;
        tensor_scales(a, se, sd);
        sh_enc = se;
        sh_dec = sd;
        if (blockIdx.x == 0 && blockIdx.y == 0 && s_dec_out) *s_dec_out = sd;
    }
    __syncthreads();
    const float sd = sh_dec;
    for (int c = threadIdx.x; c < 128; c += blockDim.x) {
        float S = e4m3_value((uint32_t)c) * sd;
        float r = (S == 0.0f) ? 0.0f : 1.0f / S;
        lut[c] = f32x2{S, r};
    }
    s_enc_out = sh_enc;
    __syncthreads();
}

// One candidate target for a half block: block scale code, codes and the
// half-block error.  `am` is the block amax (both halves).
template <int TARGET>
__device__ __forceinline__ void candidate(const float (&x)[8], float am, float s_enc,
                                          const f32x2 *lut, uint32_t &sc, uint32_t &q,
                                          float &err_half) {
    float ideal = (TARGET == 6) ? div6_rn(am) * s_enc : (am * 0.25f) * s_enc;
    sc = e4m3_encode(ideal);
    f32x2 sr = lut[sc];
    q = e2m1_pack8(x, sr.y);
    err_half = half_block_error(x, q, sr.x);
}

// ---------------------------------------------------------------------------
// 1-D encode: one lane per 1x16 block, two blocks in flight per lane
// ---------------------------------------------------------------------------

// With RHT every block is first transformed by rht16 (signs).  BUF (arrays
// below 2^31 bytes): raw buffer loads and stores with 32-bit offsets, the
// amax partials and then the first two blocks of each lane requested before
// the prologue and two blocks kept in flight, the loop unrolled three times
// so the block registers rotate without copies; a block past the end loads as
// zero and is not encoded (the last iteration's empty slots would otherwise
// cost a sixth of the encode work at 7040 x 3072 on 512 workgroups).
// Otherwise: two blocks per iteration by pointer.
template <typename T, bool FOUR_OVER_SIX, bool RHT, bool BUF>
__global__ __launch_bounds__(256) void encode1d_kernel(
    const T *__restrict__ x, int64_t nblk, const float *__restrict__ partials, int np,
    const float *__restrict__ amax_in, uint2 *__restrict__ codes, uint8_t *__restrict__ scales,
    float *__restrict__ s_dec_out, uint32_t signs) {
    __shared__ f32x2 lut[128];
    typedef typename Raw16Of<T>::type Raw;
    if (BUF) {
        constexpr uint32_t BB = 16 * sizeof(T);  // bytes per block
        const uint32_t nb = (uint32_t)nblk, stride = gridDim.x * blockDim.x;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)x, (short)0, (int)(nb * BB), kBufferWord3);
        auto off = [nb](uint32_t blk) { return (blk < nb ? blk : nb) * BB; };
        uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
        const Partials4 pp = partials_issue(partials, np, amax_in);
        Raw ra, rb, rc;
        buffer_load16(xr, off(b), ra);
        buffer_load16(xr, off(b + stride), rb);
        float s_enc;
        encode_prologue(pp, partials, np, amax_in, s_dec_out, lut, s_enc);
        const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)codes, (short)0, (int)(nb * 8u), kBufferWord3);
        const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)scales, (short)0, (int)nb, kBufferWord3);
        auto encode = [&](const Raw &r, uint32_t blk) {
            float v[16];
            uint32_t lo, hi, sc;
            unpack16(r, v);
            if (RHT) rht16(v, signs);
            encode_block16<FOUR_OVER_SIX>(v, s_enc, lut, lo, hi, sc);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, cr, blk * 8, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, sr, blk, 0, 0);
        };
        for (; b < nb; b += 3 * stride) {
            buffer_load16(xr, off(b + 2 * stride), rc);
            encode(ra, b);
            buffer_load16(xr, off(b + 3 * stride), ra);
            if (b + stride < nb) encode(rb, b + stride);
            buffer_load16(xr, off(b + 4 * stride), rb);
            if (b + 2 * stride < nb) encode(rc, b + 2 * stride);
        }
        return;
    }
    float s_enc;
    encode_prologue(partials_issue(partials, np, amax_in), partials, np, amax_in, s_dec_out,
                    lut, s_enc);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += 2 * stride) {
        const int64_t b2 = b + stride;
        Raw r0, r1;
        load_raw16(x + b * 16, r0);
        if (b2 < nblk) load_raw16(x + b2 * 16, r1);
        float v[16];
        uint32_t lo, hi, sc;
        unpack16(r0, v);
        if (RHT) rht16(v, signs);
        encode_block16<FOUR_OVER_SIX>(v, s_enc, lut, lo, hi, sc);
        codes[b] = make_uint2(lo, hi);
        scales[b] = (uint8_t)sc;
        if (b2 < nblk) {
            unpack16(r1, v);
            if (RHT) rht16(v, signs);
            encode_block16<FOUR_OVER_SIX>(v, s_enc, lut, lo, hi, sc);
            codes[b2] = make_uint2(lo, hi);
            scales[b2] = (uint8_t)sc;
        }
    }
}

// ---------------------------------------------------------------------------
// 2-D encode: 16x16 tiles, 32 lanes per tile
// ---------------------------------------------------------------------------

__device__ __forceinline__ float xor_sum(float v, int o) { return v + __shfl_xor(v, o); }

template <typename T, bool FOUR_OVER_SIX>
__global__ __launch_bounds__(256) void encode2d_kernel(
    const T *__restrict__ x, int64_t rows, int64_t cols, const float *__restrict__ partials,
    int np, const float *__restrict__ amax_in, uint32_t *__restrict__ codes,
    uint8_t *__restrict__ scales, float *__restrict__ s_dec_out) {
    __shared__ f32x2 lut[128];
    float s_enc;
    encode_prologue(partials_issue(partials, np, amax_in), partials, np, amax_in, s_dec_out,
                    lut, s_enc);
    const int64_t tcols = cols >> 4, trows = rows >> 4;
    const int64_t ntiles = trows * tcols;
    const int lane32 = threadIdx.x & 31;
    const int r = lane32 >> 1, half = lane32 & 1;
    const int64_t groups = (int64_t)gridDim.x * (blockDim.x >> 5);
    for (int64_t tile = (int64_t)blockIdx.x * (blockDim.x >> 5) + (threadIdx.x >> 5);
         tile < ntiles; tile += groups) {
        const int64_t I = tile / tcols, J = tile % tcols;
        const int64_t row = I * 16 + r;
        const int64_t col = J * 16 + half * 8;
        float v[8];
        load8(x + row * cols + col, v);
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
        uint32_t sc6, q6;
        float e6;
        candidate<6>(v, am, s_enc, lut, sc6, q6, e6);
        uint32_t qsel = q6, scsel = sc6;
        if (FOUR_OVER_SIX) {
            uint32_t sc4, q4;
            float e4;
            candidate<4>(v, am, s_enc, lut, sc4, q4, e4);
            // row error, then the pairwise tree over rows (xor 2, 4, 8, 16)
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) {
                e6 = xor_sum(e6, o);
                e4 = xor_sum(e4, o);
            }
            const bool pick4 = e4 < e6;
            qsel = pick4 ? q4 : q6;
            scsel = pick4 ? sc4 : sc6;
        }
        codes[(row * cols + col) >> 3] = qsel;
        if (lane32 == 0) scales[I * tcols + J] = (uint8_t)scsel;
    }
}

// ---------------------------------------------------------------------------
// Dequantize
// ---------------------------------------------------------------------------

// One lane per 16 output bytes (8 bf16 or 4 fp32 elements, inside one
// block): its codes (a dword or a half word), the block's scale byte, one
// 16-byte store, so each store instruction of a wave writes 1 KB
// contiguous.
template <typename TOUT, bool TWO_D>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales,
                                                      const float *__restrict__ s_dec_p,
                                                      int64_t nvec, int64_t cols,
                                                      TOUT *__restrict__ y) {
    constexpr int E = 16 / (int)sizeof(TOUT);  // elements per lane
    const float s_dec = *s_dec_p;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t tcols = cols >> 4;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        const int64_t e0 = v * E, b = e0 >> 4;
        int64_t si = b;
        if (TWO_D) {
            const int64_t row = b / tcols, cb = b - row * tcols;
            si = (row >> 4) * tcols + cb;
        }
        const float S = e4m3_value(scales[si]) * s_dec;
        float out[8];
        if (E == 8) {
            dequant8(((const uint32_t *)codes)[v], S, out);
            store8((uint16_t *)y + e0, out);
        } else {
            const uint32_t q = ((const uint16_t *)codes)[v];
            f32x2 w0 = e2m1_unpack2<0>(q), w1 = e2m1_unpack2<1>(q);
            *(f32x4 *)((float *)y + e0) = f32x4{w0.x * S, w0.y * S, w1.x * S, w1.y * S};
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static int grid_for(int64_t units, int per_block, int cap) {
    int64_t g = (units + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

hipError_t launch_amax(const void *x, int dtype, int64_t n, float *partials, int np,
                       hipStream_t s) {
    const int64_t n8 = n / 8;
    if (dtype == kF32)
        NVFP4_LAUNCH("amax", amax_kernel<float>, dim3(np), dim3(256), 0, s, (const float *)x,
                     n8, partials);
    else
        NVFP4_LAUNCH("amax", amax_kernel<uint16_t>, dim3(np), dim3(256), 0, s,
                     (const uint16_t *)x, n8, partials);
    return hipGetLastError();
}

int amax_partials_for(int64_t n) { return grid_for(n / 8, 256 * 4, kMaxPartials); }

// Workgroups of the streaming kernels: enough to fill every CU several
// times, few enough that the per-workgroup prologue stays small.  The plain
// 1-D encode runs best with two a CU (7040 x 3072 bf16: 14.3-14.5 us at 512
// workgroups, 14.9-15.2 at 1024, 15.4-16.1 at 768, 15.7-16.3 at 2048).
constexpr int kStreamGrid = 1024;
constexpr int kEncode1dGrid = 512;

hipError_t launch_encode(const void *x, int dtype, int64_t rows, int64_t cols, int layout,
                         int search, const float *partials, int np, const float *amax_in,
                         uint8_t *codes, uint8_t *scales, float *s_dec, hipStream_t s) {
    const int64_t n = rows * cols;
    const bool f46 = (search == 1);
    uint32_t *c32 = (uint32_t *)codes;
    if (layout == 0) {
        const int64_t nblk = n / 16;
        const int g = grid_for(nblk, 256, kEncode1dGrid);
        uint2 *c64 = (uint2 *)codes;
        const bool buf = n * (dtype == kF32 ? 4 : 2) < ((int64_t)1 << 31);
#define L1(T, F)                                                                            \
    if (buf)                                                                                \
        NVFP4_LAUNCH("encode1d", (encode1d_kernel<T, F, false, true>), dim3(g), dim3(256), 0, \
                     s, (const T *)x, nblk, partials, np, amax_in, c64, scales, s_dec, 0u);   \
    else                                                                                    \
        NVFP4_LAUNCH("encode1d", (encode1d_kernel<T, F, false, false>), dim3(g), dim3(256), 0,\
                     s, (const T *)x, nblk, partials, np, amax_in, c64, scales, s_dec, 0u);
        if (dtype == kF32) {
            if (f46) { L1(float, true) } else { L1(float, false) }
        } else {
            if (f46) { L1(uint16_t, true) } else { L1(uint16_t, false) }
        }
#undef L1
    } else {
        const int64_t ntiles = (rows / 16) * (cols / 16);
        const int g = grid_for(ntiles, 8, 8192);
#define L2(T, F)                                                                          \
    NVFP4_LAUNCH("encode2d", (encode2d_kernel<T, F>), dim3(g), dim3(256), 0, s, (const T *)x, \
                 rows, cols, partials, np, amax_in, c32, scales, s_dec)
        if (dtype == kF32) {
            if (f46) L2(float, true); else L2(float, false);
        } else {
            if (f46) L2(uint16_t, true); else L2(uint16_t, false);
        }
#undef L2
    }
    return hipGetLastError();
}

int amax_rht_partials_for(int64_t n) { return grid_for(n / 16, 256 * 2, kMaxPartials); }

hipError_t launch_quantize_rht(const void *x, int dtype, int64_t rows, int64_t cols, int search,
                               uint32_t signs, float *partials, const float *amax_in,
                               uint8_t *codes, uint8_t *scales, float *s_dec, hipStream_t s) {
    const int64_t nblk = rows * cols / 16;
    int np = 0;
    if (!amax_in) {
        np = amax_rht_partials_for(rows * cols);
        if (dtype == kF32)
            NVFP4_LAUNCH("amax_rht", amax_rht_kernel<float>, dim3(np), dim3(256), 0, s,
                         (const float *)x, nblk, signs, partials);
        else
            NVFP4_LAUNCH("amax_rht", amax_rht_kernel<uint16_t>, dim3(np), dim3(256), 0, s,
                         (const uint16_t *)x, nblk, signs, partials);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int g = grid_for(nblk, 256, kStreamGrid);
    uint2 *c64 = (uint2 *)codes;
    const bool buf = rows * cols * (dtype == kF32 ? 4 : 2) < ((int64_t)1 << 31);
#define LR(T, F)                                                                               \
    if (buf)                                                                                   \
        NVFP4_LAUNCH("encode1d_rht", (encode1d_kernel<T, F, true, true>), dim3(g), dim3(256), 0, \
                     s, (const T *)x, nblk, partials, np, amax_in, c64, scales, s_dec, signs);   \
    else                                                                                       \
        NVFP4_LAUNCH("encode1d_rht", (encode1d_kernel<T, F, true, false>), dim3(g), dim3(256),   \
                     0, s, (const T *)x, nblk, partials, np, amax_in, c64, scales, s_dec, signs);
    if (dtype == kF32) {
        if (search == 1) { LR(float, true) } else { LR(float, false) }
    } else {
        if (search == 1) { LR(uint16_t, true) } else { LR(uint16_t, false) }
    }
#undef LR
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, const float *s_dec,
                          int64_t rows, int64_t cols, int layout, void *y, int ydtype,
                          hipStream_t s) {
    const int64_t nvec = rows * cols * (ydtype == kF32 ? 4 : 2) / 16;
    const int g = grid_for(nvec, 256 * 4, 8192);
#define LD(T, TWO)                                                                      \
    NVFP4_LAUNCH("dequant", (dequant_kernel<T, TWO>), dim3(g), dim3(256), 0, s, codes, scales, \
                 s_dec, nvec, cols, (T *)y)
    if (ydtype == kF32) {
        if (layout) LD(float, true); else LD(float, false);
    } else {
        if (layout) LD(uint16_t, true); else LD(uint16_t, false);
    }
#undef LD
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MXFP4 quantize (OCP Microscaling v1.0; reference format for the MX GEMM)
// ---------------------------------------------------------------------------

// One lane per 32-element block along a row: shared exponent
// e = floor(log2(amax)) - 2 (2 = the E2M1 maximum exponent), clamped to
// [-127, 127] (0 for an all-zero block's scale byte), E8M0 byte e + 127;
// elements E2M1(RN(x * 2^-e)) with saturation at 6.  A subnormal amax takes
// e = -127.
template <typename T>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const T *__restrict__ x, int64_t nblk,
                                                          uint32_t *__restrict__ codes,
                                                          uint8_t *__restrict__ scales) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
        typename Raw16Of<T>::type r0, r1;
        load_raw16(x + b * 32, r0);
        load_raw16(x + b * 32 + 16, r1);
        float v[32];
        float(&v0)[16] = *reinterpret_cast<float(*)[16]>(&v[0]);
        float(&v1)[16] = *reinterpret_cast<float(*)[16]>(&v[16]);
        unpack16(r0, v0);
        unpack16(r1, v1);
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
        const int be = (int)((__float_as_uint(am) >> 23) & 0xFFu);
        int e = be == 0 ? -127 : be - 127 - 2;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        const float inv = __builtin_ldexpf(1.0f, -e);  // exact power of two
        uint32_t q[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t w = 0;
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * d] * inv, v[8 * d + 1] * inv, 1.0f, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * d + 2] * inv, v[8 * d + 3] * inv, 1.0f, 1);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * d + 4] * inv, v[8 * d + 5] * inv, 1.0f, 2);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * d + 6] * inv, v[8 * d + 7] * inv, 1.0f, 3);
            q[d] = w;
        }
        *(u32x4 *)(codes + b * 4) = u32x4{q[0], q[1], q[2], q[3]};
        scales[b] = (uint8_t)(am == 0.0f ? 0 : e + 127);
    }
}

hipError_t launch_mx_quantize(const void *x, int xdtype, int64_t rows, int64_t cols,
                              uint8_t *codes, uint8_t *scales, hipStream_t s) {
    const int64_t nblk = rows * cols / 32;
    if (nblk == 0) return hipSuccess;
    const int g = grid_for(nblk, 256, 4096);
    if (xdtype == kF32)
        NVFP4_LAUNCH("mx_quantize", mx_quantize_kernel<float>, dim3(g), dim3(256), 0, s,
                     (const float *)x, nblk, (uint32_t *)codes, scales);
    else
        NVFP4_LAUNCH("mx_quantize", mx_quantize_kernel<uint16_t>, dim3(g), dim3(256), 0, s,
                     (const uint16_t *)x, nblk, (uint32_t *)codes, scales);
    return hipGetLastError();
}

}  // namespace nvfp4
