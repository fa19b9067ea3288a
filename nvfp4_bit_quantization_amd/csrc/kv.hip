// kv.hip -- chunk-level NVFP4 KV cache: K-smoothing statistics, chunk encode
// into the ring (with sink capture) and the parallel gather-dequantizer of
// the attention window.
//
// Method (LongLive-2.0 pages): "MCISLAB DeepRead: LongLive2" summary, Method /
// inference infrastructure: the KV cache is quantized per frame chunk
// (F_c = 8), keys are K-smoothed before NVFP4 micro-block quantization, the
// storage falls from 4*T_c*H*d to (9/8)*T_c*H*d bytes, and a parallel
// dequantization kernel feeds attention; algorithm design / Multi-Shot
// Attention Sink: K_eff(t) = A_g u A_s u KV[t-W, t) with overlapping tokens
// removed.  The Italian page ("Inferenza W4A4 NVFP4") adds that the KV cache
// uses micro-block scaling with the Four Over Six selection.
//
// Store = three launches:
//   kv_stats     two waves per (64-token node, 512 channels): per-channel fp64
//                tile sums (token order) combined up to the 64-token node,
//                key max/min, value |max|
//   kv_finalize  one wave per 16 channels: mu = (float)(sum of tile sums / T)
//                by the pairwise tree, and the key amax
//                max_c max(RN(max K - mu), RN(mu - min K)) (equal to the
//                elementwise amax of RN(K - mu) because RN is monotone)
//   kv_encode    reduces the amax partials to the FP32 tensor scales of K_s
//                and V, then the 1-D 4/6 encoder over K_s = RN(K - mu) and V,
//                writing the ring slot and, for sink chunks, the sink copy in
//                the same pass
// Gather = one launch: one workgroup-iteration per kGatherTok output tokens,
// one lane per 16-element block; each token's segment (ring slot or sink
// copy) is found from scalars (sink lengths, window start, W).
#include "device.hpp"
#include "launch.hpp"

namespace nvfp4 {

// Key-mean summation order (fixed, so the result is reproducible): tokens in
// tiles of kSeq = 16, each tile summed in token order in double; the tile
// sums, padded with zeros to a power-of-two count, added pairwise level by
// level.  kv_stats computes the tile sums and the first two tree levels (one
// workgroup = 2 waves = 4 consecutive tiles); kv_finalize finishes the tree.
constexpr int kSeq = 16;            // tokens summed sequentially by one lane
constexpr int kStatsTokens = 64;    // tokens per stats unit (4 tiles of 16)
constexpr int kGroupCh = 512;       // channels per stats unit (64 lanes x 8)
constexpr int kFinCh = 16;          // channels per finalize wave
constexpr int64_t kEncodeGrid = 4096; // encode workgroups per tensor (upper bound)
constexpr int64_t kEncodeBlocks = 6;  // target blocks per encode lane (measured: 6 over ~10)

struct KvWs {
    double *P;      // [nt64, HD]  level-2 tree nodes (64-token sums)
    float *kmax;    // [nt64, HD]
    float *kmin;    // [nt64, HD]
    float *vpart;   // [nt64 * gy] value |max| per stats unit
    float *kpart;   // [nfin]      key amax per finalize wave
};

struct KvDims {
    int64_t nt64;   // stats units along tokens (64-token nodes)
    int64_t gy;     // stats units along channels
    int64_t n2;     // level-2 nodes in the padded tree (power of two)
    int64_t nfin;   // finalize waves (one workgroup each)
};

static inline int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

static KvDims kv_dims(int64_t T, int64_t HD) {
    KvDims d;
    d.nt64 = (T + kStatsTokens - 1) / kStatsTokens;
    d.gy = (HD + kGroupCh - 1) / kGroupCh;
    const int64_t nt16 = (T + kSeq - 1) / kSeq;
    int64_t npad = 1;
    while (npad < nt16) npad *= 2;
    d.n2 = npad >= 4 ? npad / 4 : 1;
    d.nfin = (HD + kFinCh - 1) / kFinCh;
    return d;
}

static KvWs carve_ws(void *ws, int64_t T, int64_t HD) {
    const KvDims d = kv_dims(T, HD);
    uint8_t *p = (uint8_t *)ws;
    KvWs w;
    w.P = (double *)p;
    p += align256(d.nt64 * HD * 8);
    w.kmax = (float *)p;
    p += align256(d.nt64 * HD * 4);
    w.kmin = (float *)p;
    p += align256(d.nt64 * HD * 4);
    w.vpart = (float *)p;
    p += align256(d.nt64 * d.gy * 4);
    w.kpart = (float *)p;
    return w;
}

size_t kv_store_ws_bytes(int64_t T, int64_t HD) {
    const KvDims d = kv_dims(T, HD);
    return (size_t)(align256(d.nt64 * HD * 8) + 2 * align256(d.nt64 * HD * 4) +
                    align256(d.nt64 * d.gy * 4) + align256(d.nfin * 4));
}

constexpr int kHalf = kStatsTokens / 2;  // tokens per stats wave (two tiles)

// The 32 loads of a wave's two tiles (a full node: no token past T) as raw
// buffer loads: the node's wave-uniform base is in the buffer descriptor,
// the token's byte offset in a scalar register and the lane's byte offset in
// one vector register shared by all loads.
__device__ __forceinline__ void stats_load(u32x4 (&r)[kHalf], __amdgpu_buffer_rsrc_t rs,
                                           uint32_t voff, uint32_t tok0, uint32_t row_bytes) {
#pragma unroll
    for (int j = 0; j < kHalf; ++j)
        r[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (tok0 + j) * row_bytes, 0);
}

__device__ __forceinline__ void bf16x8(const u32x4 &r, float (&v)[8]) {
    v[0] = bf16lo(r.x);
    v[1] = bf16hi(r.x);
    v[2] = bf16lo(r.y);
    v[3] = bf16hi(r.y);
    v[4] = bf16lo(r.z);
    v[5] = bf16hi(r.z);
    v[6] = bf16lo(r.w);
    v[7] = bf16hi(r.w);
}

// Key token: add to the running per-channel sums (double), max / min.
__device__ __forceinline__ void stats_key_token(const u32x4 &r, double (&s)[8], float (&mx)[8],
                                                float (&mn)[8]) {
    float v[8];
    bf16x8(r, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        s[i] += (double)v[i];
        mx[i] = fmaxf(mx[i], v[i]);
        mn[i] = fminf(mn[i], v[i]);
        // the extrema are materialised token by token: otherwise the max / min
        // chains get regrouped across tokens and keep every value alive
        asm volatile("" : "+v"(mx[i]), "+v"(mn[i]));
    }
}

__device__ __forceinline__ float stats_value_token(const u32x4 &r, float m) {
    float v[8];
    bf16x8(r, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    return m;
}

// Workgroup = 2 waves = one unit (64-token node p, 512-channel group y);
// blockIdx.y selects keys (0) or values (1).  Wave h takes tokens
// 64 p + 32 h .. +31; lane l owns channels 512 y + 8 l .. +7 (one 16-byte
// load per token), and all 32 loads of a wave are issued before any is
// used.  Keys: each 16-token tile is summed in token order in double; the
// wave adds its two tile sums (tree level 1), wave 1 hands its node to wave
// 0 through LDS, which adds them (level 2) and stores the level-2 node with
// the per-channel max / min.  Values: the |max| of the unit.  The last,
// partial node reads token by token up to T; its absent tiles are +0, the
// value the padded tree gives them.
__global__ __launch_bounds__(128) void kv_stats_kernel(const uint16_t *__restrict__ K,
                                                       const uint16_t *__restrict__ V, int64_t T,
                                                       int64_t HD, int64_t gy, KvWs w) {
    __shared__ double sp[8][64];
    __shared__ float sx[8][64];
    __shared__ float sn[8][64];
    __shared__ float sv;
    const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t unit = blockIdx.x;
    const int64_t p = unit / gy, y = unit - p * gy;
    const int64_t chq = y * kGroupCh + lane * 8;
    const bool ch_ok = chq < HD;  // HD is a multiple of 16: all 8 channels or none
    const uint32_t off = ch_ok ? (uint32_t)lane * 8 : 0u;
    const int64_t t0 = p * kStatsTokens + h * kHalf;
    const uint16_t *row = (blockIdx.y ? V : K) + y * kGroupCh + t0 * HD;  // wave-uniform
    const bool full = t0 + kHalf <= T;
    // descriptor over the wave's rows (32 * HD * 2 bytes < 2^32: HD < 2^26)
    const uint32_t rb = (uint32_t)HD * 2, voff = off * 2;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)row, (short)0, (int)(kHalf * rb), kBufferWord3);
    if (blockIdx.y) {
        float m = 0.0f;
        if (full) {
            u32x4 r[kHalf];
            stats_load(r, rs, voff, 0, rb);
#pragma unroll
            for (int j = 0; j < kHalf; ++j) m = stats_value_token(r[j], m);
        } else {
#pragma unroll 1
            for (int64_t j = 0; t0 + j < T; ++j)
                m = stats_value_token(*(const u32x4 *)(row + j * HD + off), m);
        }
        m = ch_ok ? m : 0.0f;
        m = wave_max(m);
        if (h == 1 && lane == 0) sv = m;
        __syncthreads();
        if (h == 0 && lane == 0) w.vpart[unit] = fmaxf(m, sv);
        return;
    }
    double node[8];
    float mx[8], mn[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        mx[i] = -__builtin_huge_valf();
        mn[i] = __builtin_huge_valf();
    }
    if (full) {
        u32x4 r[kHalf];
        stats_load(r, rs, voff, 0, rb);
        double a[8], b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = b[i] = 0.0;
#pragma unroll
        for (int j = 0; j < kSeq; ++j) stats_key_token(r[j], a, mx, mn);
#pragma unroll
        for (int j = kSeq; j < kHalf; ++j) stats_key_token(r[j], b, mx, mn);
#pragma unroll
        for (int i = 0; i < 8; ++i) node[i] = a[i] + b[i];
    } else {
        double a[8], b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = b[i] = 0.0;
#pragma unroll 1
        for (int64_t j = 0; j < kSeq && t0 + j < T; ++j)
            stats_key_token(*(const u32x4 *)(row + j * HD + off), a, mx, mn);
#pragma unroll 1
        for (int64_t j = kSeq; j < kHalf && t0 + j < T; ++j)
            stats_key_token(*(const u32x4 *)(row + j * HD + off), b, mx, mn);
#pragma unroll
        for (int i = 0; i < 8; ++i) node[i] = a[i] + b[i];
    }
    if (h == 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sp[i][lane] = node[i];
            sx[i][lane] = mx[i];
            sn[i][lane] = mn[i];
        }
    }
    __syncthreads();
    if (h == 1 || !ch_ok) return;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        node[i] = node[i] + sp[i][lane];
        mx[i] = fmaxf(mx[i], sx[i][lane]);
        mn[i] = fminf(mn[i], sn[i][lane]);
    }
    double *P = w.P + p * HD + chq;
    float *X = w.kmax + p * HD + chq;
    float *N = w.kmin + p * HD + chq;
#pragma unroll
    for (int i = 0; i < 8; i += 2) *(f64x2 *)(P + i) = f64x2{node[i], node[i + 1]};
    *(f32x4 *)X = f32x4{mx[0], mx[1], mx[2], mx[3]};
    *(f32x4 *)(X + 4) = f32x4{mx[4], mx[5], mx[6], mx[7]};
    *(f32x4 *)N = f32x4{mn[0], mn[1], mn[2], mn[3]};
    *(f32x4 *)(N + 4) = f32x4{mn[4], mn[5], mn[6], mn[7]};
}

// Tree sum of 32 doubles, adjacent pairs level by level.
__device__ __forceinline__ double tree32(double (&v)[32]) {
#pragma unroll
    for (int w = 16; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) v[i] = v[2 * i] + v[2 * i + 1];
    return v[0];
}

// One wave per 16 channels: lane = (channel c = lane & 15, quarter
// q = lane >> 4).  The level-2 nodes of a channel form blocks of 32 (nodes
// past the last 64-token node are zero); quarter q sums blocks q, q + 4, ...
// with a fixed 32-leaf tree into LDS, then the q = 0 lanes sum the block
// sums with the same tree (zero padded; adding an exact zero changes
// nothing, and no partial sum is -0).  This is the level-by-level pairwise
// tree over the 16-token tile sums.  mu = (float)(S / T); the wave's key
// amax max_c max(RN(max K - mu), RN(mu - min K)) goes to kpart.
__global__ __launch_bounds__(64) void kv_finalize_kernel(KvWs w, int64_t nt64, int64_t n2,
                                                         int64_t T, int64_t HD, float *mu_slot,
                                                         float *mu_g, float *mu_s) {
    __shared__ double bs[32][kFinCh];
    __shared__ float rx[4][kFinCh];
    __shared__ float rn[4][kFinCh];
    const int lane = threadIdx.x, c = lane & (kFinCh - 1), q = lane >> 4;
    const int64_t ch = (int64_t)blockIdx.x * kFinCh + c;
    const int nb = n2 >= 32 ? (int)(n2 / 32) : 1;  // blocks of 32 nodes (<= 32)
    float kx = -__builtin_huge_valf(), kn = __builtin_huge_valf();
    const int64_t chc = ch < HD ? ch : HD - 1;
    for (int b = q; b < nb; b += 4) {
        double v[32];
        float xv[32], nv[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int64_t node = (int64_t)b * 32 + i;
            const int64_t nc = node < nt64 ? node : nt64 - 1;
            v[i] = w.P[nc * HD + chc];
            xv[i] = w.kmax[nc * HD + chc];
            nv[i] = w.kmin[nc * HD + chc];
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const bool ok = (int64_t)b * 32 + i < nt64;
            v[i] = ok ? v[i] : 0.0;
            kx = ok ? fmaxf(kx, xv[i]) : kx;
            kn = ok ? fminf(kn, nv[i]) : kn;
        }
        bs[b][c] = tree32(v);
    }
    rx[q][c] = kx;
    rn[q][c] = kn;
    __syncthreads();
    float amax = 0.0f;
    if (q == 0 && ch < HD) {
        double v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = (i < nb) ? bs[i][c] : 0.0;
        const double S = tree32(v);
        const float mu = (float)(S / (double)T);
        mu_slot[ch] = mu;
        if (mu_g) mu_g[ch] = mu;
        if (mu_s) mu_s[ch] = mu;
        const float x = fmaxf(fmaxf(rx[0][c], rx[1][c]), fmaxf(rx[2][c], rx[3][c]));
        const float n = fminf(fminf(rn[0][c], rn[1][c]), fminf(rn[2][c], rn[3][c]));
        amax = fmaxf(x - mu, mu - n);
    }
    amax = wave_max(amax);
    if (lane == 0) w.kpart[blockIdx.x] = amax;
}

// Raw 16-element bf16 block at byte offset `off` of a buffer (zero past its end).
__device__ __forceinline__ Raw16Bf16 block_load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    Raw16Bf16 r;
    buffer_load16(rs, off, r);
    return r;
}

// Destination of one tensor's blocks: codes (8 bytes per block) and scales
// (1 byte per block) of the slot and of the two sink copies, as buffer
// descriptors whose sizes are the blocks each holds, so a store past them is
// dropped by the hardware range check.
struct EncDst {
    __amdgpu_buffer_rsrc_t c, s, gc, gs, sc, ss;
};

__device__ __forceinline__ void block_store(const EncDst &d, bool sinks, uint32_t b, uint32_t lo,
                                            uint32_t hi, uint32_t sc) {
    const u32x2 q = u32x2{lo, hi};
    __builtin_amdgcn_raw_buffer_store_b64(q, d.c, b * 8, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, d.s, b, 0, 0);
    if (sinks) {  // uniform: the chunk writes a sink copy
        __builtin_amdgcn_raw_buffer_store_b64(q, d.gc, b * 8, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, d.gs, b, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(q, d.sc, b * 8, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, d.ss, b, 0, 0);
    }
}

// One lane per 1x16 block along the (head, dim) axis; blockIdx.y = 0: keys
// (K_s = RN(K - mu)), 1: values.  The first two blocks of each lane are
// loaded before the prologue, which reduces the key / value amax partials,
// derives both tensor scales (workgroup (0,0) stores the decode scales into
// the slot and the sink copies) and builds the (S, r) table of the
// workgroup's tensor; afterwards each lane keeps two blocks in flight, with
// the loop unrolled three times so the three block registers rotate without
// copies.  Loads and stores are raw buffer accesses with 32-bit offsets:
// a block past the end loads as zero and its stores are dropped by the
// range check (also how only the blocks below the sink length reach the
// sink copies).  When the grid stride is a multiple of the blocks per token
// (MU_FIXED) every block of a lane starts at the same channel, and the lane
// holds its 16 key means in registers; otherwise they are re-read per block.
template <bool FOUR_OVER_SIX, bool MU_FIXED>
__global__ __launch_bounds__(256) void kv_encode_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, int64_t nblk, int64_t HD,
    const float *__restrict__ kpart, int nk, const float *__restrict__ vpart, int nv,
    KvRegion slot, KvRegion gsink, KvRegion ssink, int64_t g_blk, int64_t s_blk) {
    __shared__ f32x2 lut[128];
    __shared__ float red[2][4];
    __shared__ float sh[4];
    const int which = blockIdx.y;  // 0: keys, 1: values
    // nblk * 32 = T * HD * 2 < 2^32 bytes; block offsets are clamped to the
    // end so that they never wrap
    const uint32_t nb = (uint32_t)nblk;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(which ? V : K), (short)0, (int)(nb * 32u), kBufferWord3);
    const uint32_t stride = gridDim.x * blockDim.x;
    uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
    auto off = [nb](uint32_t blk) { return (blk < nb ? blk : nb) * 32u; };
    Raw16Bf16 ra = block_load(xr, off(b)), rb = block_load(xr, off(b + stride)), rc;
    // channel of the block's first element, advanced without division: (16 b) mod HD
    int64_t ch0 = ((int64_t)b * 16) % HD;
    const int64_t step = ((int64_t)stride * 16) % HD;
    float mu[16];
    if (MU_FIXED && which == 0 && b < nb) {
        Raw16F32 m;
        load_raw16(slot.mu + ch0, m);
        unpack16(m, mu);
    }
    float ak = 0.0f, av = 0.0f;
    for (int i = threadIdx.x; i < nk; i += blockDim.x) ak = fmaxf(ak, kpart[i]);
    for (int i = threadIdx.x; i < nv; i += blockDim.x) av = fmaxf(av, vpart[i]);
    ak = wave_max(ak);
    av = wave_max(av);
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = ak;
        red[1][threadIdx.x >> 6] = av;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const float a0 = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
        const float a1 = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
        float e0, d0, e1, d1;
        tensor_scales(a0, e0, d0);
        tensor_scales(a1, e1, d1);
        sh[0] = e0;
        sh[1] = d0;
        sh[2] = e1;
        sh[3] = d1;
        if (blockIdx.x == 0 && blockIdx.y == 0) {
            slot.sd[0] = d0;
            slot.sd[1] = d1;
            if (g_blk > 0) {
                gsink.sd[0] = d0;
                gsink.sd[1] = d1;
            }
            if (s_blk > 0) {
                ssink.sd[0] = d0;
                ssink.sd[1] = d1;
            }
        }
    }
    __syncthreads();
    const float s_enc = sh[2 * which];
    const float s_dec = sh[2 * which + 1];
    for (int c = threadIdx.x; c < 128; c += blockDim.x) lut[c] = scale_entry((uint32_t)c, s_dec);
    __syncthreads();
    EncDst d;
    const uint32_t gb = (uint32_t)g_blk, sb = (uint32_t)s_blk;
    d.c = __builtin_amdgcn_make_buffer_rsrc((void *)(which ? slot.vc : slot.kc), (short)0,
                                            (int)(nb * 8u), kBufferWord3);
    d.s = __builtin_amdgcn_make_buffer_rsrc((void *)(which ? slot.vs : slot.ks), (short)0, (int)nb,
                                            kBufferWord3);
    d.gc = __builtin_amdgcn_make_buffer_rsrc((void *)(which ? gsink.vc : gsink.kc), (short)0,
                                             (int)(gb * 8u), kBufferWord3);
    d.gs = __builtin_amdgcn_make_buffer_rsrc((void *)(which ? gsink.vs : gsink.ks), (short)0,
                                             (int)gb, kBufferWord3);
    d.sc = __builtin_amdgcn_make_buffer_rsrc((void *)(which ? ssink.vc : ssink.kc), (short)0,
                                             (int)(sb * 8u), kBufferWord3);
    d.ss = __builtin_amdgcn_make_buffer_rsrc((void *)(which ? ssink.vs : ssink.ks), (short)0,
                                             (int)sb, kBufferWord3);
    const bool sinks = gb > 0 || sb > 0;
    auto encode = [&](const Raw16Bf16 &r, uint32_t blk) {
        float v[16];
        unpack16(r, v);
        if (which == 0) {
            if (!MU_FIXED) {
                Raw16F32 m;
                load_raw16(slot.mu + ch0, m);
                unpack16(m, mu);
                ch0 += step;
                if (ch0 >= HD) ch0 -= HD;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = v[i] - mu[i];
        }
        uint32_t lo, hi, sc;
        encode_block16<FOUR_OVER_SIX>(v, s_enc, lut, lo, hi, sc);
        block_store(d, sinks, blk, lo, hi, sc);
    };
    // blocks b, b + stride, b + 2 stride per iteration (past nblk: zero
    // loads, dropped stores)
    for (; b < nb; b += 3 * stride) {
        rc = block_load(xr, off(b + 2 * stride));
        encode(ra, b);
        ra = block_load(xr, off(b + 3 * stride));
        encode(rb, b + stride);
        rb = block_load(xr, off(b + 4 * stride));
        encode(rc, b + 2 * stride);
    }
}

hipError_t launch_kv_store(const KvStoreArgs &a, hipStream_t s) {
    const KvDims d = kv_dims(a.T, a.HD);
    KvWs w = carve_ws(a.ws, a.T, a.HD);
    NVFP4_LAUNCH("kv_stats", kv_stats_kernel, dim3((unsigned)(d.nt64 * d.gy), 2), dim3(128), 0,
                 s, a.K, a.V, a.T, a.HD, d.gy, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    NVFP4_LAUNCH("kv_finalize", kv_finalize_kernel, dim3((unsigned)d.nfin), dim3(64), 0, s, w,
                 d.nt64, d.n2, a.T, a.HD, a.slot.mu,
                 a.g_tokens > 0 ? a.gsink.mu : (float *)nullptr,
                 a.s_tokens > 0 ? a.ssink.mu : (float *)nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nblk = a.T * a.HD / 16;
    // Grid: about kEncodeBlocks blocks per lane (whole iterations of the
    // three-block loop), at most kEncodeGrid workgroups per tensor.  If a
    // multiple of m = NB / gcd(NB, 256) fits (NB = blocks per token), the grid
    // is the next such multiple, so the stride in blocks is a multiple of NB.
    int64_t g = (nblk + 256 * kEncodeBlocks - 1) / (256 * kEncodeBlocks);
    if (g > kEncodeGrid) g = kEncodeGrid;
    if (g < 1) g = 1;
    const int64_t NB = a.HD / 16;
    int64_t gc = NB, tw = 256;
    while (tw > 1 && gc % 2 == 0) {
        gc /= 2;
        tw /= 2;
    }
    bool fixed = false;
    if (gc <= g) {
        g = ((g + gc - 1) / gc) * gc;
        fixed = true;
    } else if (gc <= 2 * kEncodeGrid) {
        g = gc;
        fixed = true;
    }
    const int64_t g_blk = a.g_tokens * a.HD / 16, s_blk = a.s_tokens * a.HD / 16;
    const int nk = (int)d.nfin, nv = (int)(d.nt64 * d.gy);
#define NVFP4_ENC(F46, FIX)                                                                   \
    NVFP4_LAUNCH("kv_encode", (kv_encode_kernel<F46, FIX>), dim3((unsigned)g, 2), dim3(256), 0, \
                 s, a.K, a.V, nblk, a.HD, (const float *)w.kpart, nk, (const float *)w.vpart, nv, \
                 a.slot, a.gsink, a.ssink, g_blk, s_blk)
    if (a.search == 1) {
        if (fixed)
            NVFP4_ENC(true, true);
        else
            NVFP4_ENC(true, false);
    } else {
        if (fixed)
            NVFP4_ENC(false, true);
        else
            NVFP4_ENC(false, false);
    }
#undef NVFP4_ENC
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gather-dequantize of K_eff(t)
// ---------------------------------------------------------------------------

// Output order: [global-sink tokens outside the window][shot-sink tokens
// outside the window][window chunks c_lo .. c_lo + nwin - 1]; sinks lie below
// the window in token order, so this is ascending token order.
__device__ __forceinline__ void gather_region(const GatherArgs &a, int64_t tok, KvRegion &r,
                                              int64_t &st) {
    if (tok < a.n_g) {
        r = a.gsink;
        st = tok;
    } else if (tok < a.n_g + a.n_s) {
        r = a.ssink;
        st = tok - a.n_g;
    } else {
        const int64_t w = tok - a.n_g - a.n_s;
        const int64_t q = w / a.Tc;
        const int64_t off = ((a.c_lo + q) % a.W) * a.slot_bytes;
        r.kc = a.slot0.kc + off;
        r.ks = a.slot0.ks + off;
        r.vc = a.slot0.vc + off;
        r.vs = a.slot0.vs + off;
        r.mu = (float *)((uint8_t *)a.slot0.mu + off);
        r.sd = (float *)((uint8_t *)a.slot0.sd + off);
        st = w - q * a.Tc;
    }
}

// Each workgroup-iteration covers kGatherTok consecutive output tokens; lane
// j expands block j (16 elements) of K and V of each of them, with the loads
// of all the tokens issued before any of them is expanded.
constexpr int kGatherTok = 4;

__global__ __launch_bounds__(256) void kv_gather_kernel(GatherArgs a) {
    const int64_t NB = a.HD >> 4;  // blocks per token
    for (int64_t tok0 = (int64_t)blockIdx.x * kGatherTok; tok0 < a.n_tokens;
         tok0 += (int64_t)gridDim.x * kGatherTok) {
        for (int64_t j = threadIdx.x; j < NB; j += blockDim.x) {
            uint2 qk[kGatherTok], qv[kGatherTok];
            uint32_t sk[kGatherTok], sv[kGatherTok];
            const float *mup[kGatherTok];
            float sdk[kGatherTok], sdv[kGatherTok];
#pragma unroll
            for (int k = 0; k < kGatherTok; ++k) {
                const int64_t tok = tok0 + k < a.n_tokens ? tok0 + k : a.n_tokens - 1;
                KvRegion r;
                int64_t st;
                gather_region(a, tok, r, st);
                qk[k] = ((const uint2 *)r.kc)[st * NB + j];
                qv[k] = ((const uint2 *)r.vc)[st * NB + j];
                sk[k] = r.ks[st * NB + j];
                sv[k] = r.vs[st * NB + j];
                sdk[k] = r.sd[0];
                sdv[k] = r.sd[1];
                mup[k] = r.mu + j * 16;
            }
#pragma unroll
            for (int k = 0; k < kGatherTok; ++k) {
                const int64_t tok = tok0 + k;
                if (tok >= a.n_tokens) break;
                Raw16F32 m;
                load_raw16(mup[k], m);
                float mu[16];
                unpack16(m, mu);
                const float Sk = e4m3_value(sk[k]) * sdk[k];
                const float Sv = e4m3_value(sv[k]) * sdv[k];
                uint16_t *ko = a.Kout + tok * a.HD + j * 16;
                uint16_t *vo = a.Vout + tok * a.HD + j * 16;
                float y[8];
                dequant8(qk[k].x, Sk, y);
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = y[i] + mu[i];
                store8(ko, y);
                dequant8(qk[k].y, Sk, y);
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = y[i] + mu[8 + i];
                store8(ko + 8, y);
                dequant8(qv[k].x, Sv, y);
                store8(vo, y);
                dequant8(qv[k].y, Sv, y);
                store8(vo + 8, y);
            }
        }
    }
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s) {
    if (a.n_tokens == 0) return hipSuccess;
    const int64_t NB = a.HD >> 4;
    int64_t bs = ((NB + 63) / 64) * 64;
    if (bs > 256) bs = 256;
    int64_t g = (a.n_tokens + kGatherTok - 1) / kGatherTok;
    if (g > 2048) g = 2048;
    NVFP4_LAUNCH("kv_gather", kv_gather_kernel, dim3((unsigned)g), dim3((unsigned)bs), 0, s, a);
    return hipGetLastError();
}

}  // namespace nvfp4
