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
// Store = two launches:
//   kv_stats     four waves per (256-token node, 512 channels): per-channel key
//                sums in double, key max / min and the value |max| over the
//                node, added into the workspace with device-scope atomics
//                (the sums are exact on the key-mean domain, so their order
//                does not matter); the last workgroup of each 512-channel
//                group to finish then finalizes the group: mu = (float)(S /
//                T), the group's key amax max_c max(RN(max K - mu), RN(mu -
//                min K)) (equal to the elementwise amax of RN(K - mu) because
//                RN is monotone) and value amax, and the accumulators cleared
//                for the next call
//   kv_encode    the FP32 tensor scales of K_s and V from the groups'
//                amaxes, then the 1-D 4/6 encoder over K_s = RN(K - mu) and
//                V, writing the ring slot and, for sink chunks, the sink copy
//                in the same pass
// Gather = one launch: workgroups take runs of tokens of one segment (ring
// slot or sink copy) of the effective set, a lane per half block, the bf16
// output written with non-temporal stores.
#include <mutex>

#include "device.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kHalf = 32;             // tokens per stats batch (all its loads in flight at once)
constexpr int kStatsWaves = 4;        // waves per stats workgroup
constexpr int kStatsBatches = 2;      // batches per stats wave
constexpr int kStatsTokens = kHalf * kStatsBatches * kStatsWaves;  // tokens per stats unit
constexpr int kGroupCh = 512;         // channels per stats unit (64 lanes x 8)
constexpr int64_t kEncodeGrid = 4096; // encode workgroups per tensor (upper bound)
constexpr int64_t kEncodeBlocks = 6;  // target blocks per encode lane (measured: 6 over ~10)

// Store workspace.  The accumulators and ticket counters are zero between
// calls: every store leaves them so (the finalizing workgroups clear them),
// and a store of chunk 0 clears them first.
struct KvWs {
    double *sum;     // [HD] per-channel key sums
    uint32_t *kmax;  // [HD] order-preserving bits of the channel's key max
    uint32_t *kneg;  // [HD] order-preserving bits of minus the channel's key min
    uint32_t *vmax;  // [gy] value |max| of each channel group (float bits)
    uint32_t *tick;  // [gy] statistics workgroups of each group done
    float *gamax;    // [gy] this call's key amax of each channel group (read by kv_encode)
    float *gvmax;    // [gy] this call's value amax of each channel group
};

static inline int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

static KvWs carve_ws(void *ws, int64_t HD) {
    const int64_t gy = (HD + kGroupCh - 1) / kGroupCh;
    uint8_t *p = (uint8_t *)ws;
    KvWs w;
    w.sum = (double *)p;
    p += align256(HD * 8);
    w.kmax = (uint32_t *)p;
    p += align256(HD * 4);
    w.kneg = (uint32_t *)p;
    p += align256(HD * 4);
    w.vmax = (uint32_t *)p;
    p += align256(gy * 4);
    w.tick = (uint32_t *)p;
    p += align256(gy * 4);
    w.gamax = (float *)p;
    p += align256(gy * 4);
    w.gvmax = (float *)p;
    return w;
}

// The part that must be zero between calls, and the whole.
static int64_t kv_ws_zero_bytes(int64_t HD) {
    const int64_t gy = (HD + kGroupCh - 1) / kGroupCh;
    return align256(HD * 8) + 2 * align256(HD * 4) + 2 * align256(gy * 4);
}
size_t kv_store_ws_bytes(int64_t T, int64_t HD) {
    (void)T;
    const int64_t gy = (HD + kGroupCh - 1) / kGroupCh;
    return (size_t)(kv_ws_zero_bytes(HD) + 2 * align256(gy * 4));
}

// Bits of a float whose unsigned order is the float order (-0 just below +0).
__device__ __forceinline__ uint32_t ord_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_value(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

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

// Workgroup = 4 waves = one unit (256-token node p, 512-channel group y);
// blockIdx.y selects keys (0) or values (1; absent when the caller supplies
// the value amax).  Wave h takes tokens 256 p + 64 h .. +63 in two batches
// of 32; lane l owns channels 512 y + 8 l .. +7 (one 16-byte load per
// token), and all 32 loads of a batch are issued before any is used; a
// partial batch (past T) reads token by token.  Keys: per-channel double
// sums, max and min over the wave's tokens; the waves put theirs in LDS and
// the workgroup adds the unit's 512 channels to the workspace with atomics,
// thread t taking channels t and t + 256 so that one atomic instruction
// covers consecutive addresses (atomic add of the sums, atomic max of the
// order-preserving bits of max and of -min).  Values: the unit's |max|, one
// atomic max into its channel group's word.  The device-scope atomics bound
// this kernel (774K of them take about 10 us on their own, measured), so a
// unit spans 256 tokens: 3 atomics per channel per 256 tokens.  Each double
// sum and every partial sum the atomics form is exact on the key-mean
// domain (every partial sum of a channel's keys is a multiple of the
// channel's smallest key unit below 2^53 of them), so mu does not depend on
// the order in which units arrive.
//
// Finalize: each wave waits until its atomics are performed (s_waitcnt
// vmcnt(0)), the workgroup meets at a barrier, and thread 0 takes a ticket
// of its channel group (a relaxed device-scope atomic add); the workgroup
// that takes the group's last ticket (per_group: the group's key and value
// units) finalizes the group.  Every other unit's atomics were performed
// before its ticket was taken, and the finalizing workgroup reads the
// accumulators with device-scope atomic loads, so it sees them all.  With
// one round of workgroups (every unit resident at once) the wait before the
// ticket delays nothing else: the store is ~2 us faster than with a
// separate finalize launch (7040 x 24 x 128, 66.7 -> 64.6 us a KV step);
// with 64-token units (1320 workgroups queued behind waiting ones) the same
// scheme was 9-10 us slower.  (Finalizing in every kv_encode workgroup's
// prologue instead: ~5 us slower, since each key workgroup reads all the
// channels' statistics and divides for every channel.)
__device__ __forceinline__ void finalize_group(const KvWs &w, int64_t y, int64_t T, int64_t HD,
                                               float *mu_slot, float *mu_g, float *mu_s,
                                               float *red);

__global__ __launch_bounds__(64 * kStatsWaves) void kv_stats_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, int64_t T, int64_t HD,
    int64_t gy, KvWs w, float *mu_slot, float *mu_g, float *mu_s, uint32_t per_group) {
    __shared__ double sp[kStatsWaves][64][8];
    __shared__ int last;  // [wave][lane][channel of the lane]
    __shared__ float sx[kStatsWaves][64][8];
    __shared__ float sn[kStatsWaves][64][8];
    __shared__ float red[kStatsWaves];
    const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t unit = blockIdx.x;
    const int64_t p = unit / gy, y = unit - p * gy;
    const int64_t chq = y * kGroupCh + lane * 8;
    const bool ch_ok = chq < HD;  // HD is a multiple of 16: all 8 channels or none
    const uint32_t off = ch_ok ? (uint32_t)lane * 8 : 0u;
    const uint32_t rb = (uint32_t)HD * 2, voff = off * 2;
    const uint16_t *X = blockIdx.y ? V : K;
    // batch q of this wave: tokens t0 .. t0 + 31 from `row` (wave-uniform),
    // through a descriptor over its rows (32 * HD * 2 bytes < 2^32: HD < 2^26)
    auto batch = [&](int q, int64_t &t0, const uint16_t *&row, __amdgpu_buffer_rsrc_t &rs) {
        t0 = p * kStatsTokens + (h * kStatsBatches + q) * kHalf;
        row = X + y * kGroupCh + t0 * HD;
        rs = __builtin_amdgcn_make_buffer_rsrc((void *)row, (short)0, (int)(kHalf * rb),
                                               kBufferWord3);
    };
    if (blockIdx.y) {
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < kStatsBatches; ++q) {
            int64_t t0;
            const uint16_t *row;
            __amdgpu_buffer_rsrc_t rs;
            batch(q, t0, row, rs);
            if (t0 + kHalf <= T) {
                u32x4 r[kHalf];
                stats_load(r, rs, voff, 0, rb);
#pragma unroll
                for (int j = 0; j < kHalf; ++j) m = stats_value_token(r[j], m);
            } else {
#pragma unroll 1
                for (int64_t j = 0; t0 + j < T; ++j)
                    m = stats_value_token(*(const u32x4 *)(row + j * HD + off), m);
            }
        }
        m = ch_ok ? m : 0.0f;
        m = wave_max(m);
        if (lane == 0) red[h] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
            float a = red[0];
#pragma unroll
            for (int v = 1; v < kStatsWaves; ++v) a = fmaxf(a, red[v]);
            atomicMax(&w.vmax[y], __float_as_uint(a));
        }
    } else {
        float mx[8], mn[8];
        double a[8], b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mx[i] = -__builtin_huge_valf();
            mn[i] = __builtin_huge_valf();
            a[i] = b[i] = 0.0;
        }
#pragma unroll
        for (int q = 0; q < kStatsBatches; ++q) {
            int64_t t0;
            const uint16_t *row;
            __amdgpu_buffer_rsrc_t rs;
            batch(q, t0, row, rs);
            if (t0 + kHalf <= T) {
                u32x4 r[kHalf];
                stats_load(r, rs, voff, 0, rb);
#pragma unroll
                for (int j = 0; j < kHalf / 2; ++j) stats_key_token(r[j], a, mx, mn);
#pragma unroll
                for (int j = kHalf / 2; j < kHalf; ++j) stats_key_token(r[j], b, mx, mn);
            } else {
#pragma unroll 1
                for (int64_t j = 0; t0 + j < T; ++j)
                    stats_key_token(*(const u32x4 *)(row + j * HD + off), a, mx, mn);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sp[h][lane][i] = a[i] + b[i];
            sx[h][lane][i] = mx[i];
            sn[h][lane][i] = mn[i];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kGroupCh / (64 * kStatsWaves); ++j) {
            const int c = (int)threadIdx.x + 64 * kStatsWaves * j, i = c & 7, l = c >> 3;
            const int64_t ch = y * kGroupCh + c;
            if (ch < HD) {
                double s = sp[0][l][i];
                float x = sx[0][l][i], n = sn[0][l][i];
#pragma unroll
                for (int v = 1; v < kStatsWaves; ++v) {
                    s += sp[v][l][i];
                    x = fmaxf(x, sx[v][l][i]);
                    n = fminf(n, sn[v][l][i]);
                }
                unsafeAtomicAdd(&w.sum[ch], s);
                atomicMax(&w.kmax[ch], ord_bits(x));
                atomicMax(&w.kneg[ch], ord_bits(-n));
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's atomics performed
    __syncthreads();
    if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(&w.tick[y], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               per_group - 1;
    __syncthreads();
    if (last) finalize_group(w, y, T, HD, mu_slot, mu_g, mu_s, red);
}

// Finalize channel group y (one workgroup of 256 threads, two channels a
// thread, loads issued first): mu = (float)(S / T) into the slot (and the
// sink copies), the group's key amax max_c max(RN(max K - mu), RN(mu - min
// K)) and value amax for kv_encode; the group's sums, extrema, value maximum
// and ticket counter go back to zero for the next call.  The accumulators
// are read and cleared with device-scope atomic loads and stores (coherent
// across the chip's L2 caches, like the atomics that filled them).  `red`:
// 4 floats of LDS.
__device__ __forceinline__ void finalize_group(const KvWs &w, int64_t y, int64_t T, int64_t HD,
                                               float *mu_slot, float *mu_g, float *mu_s,
                                               float *red) {
    constexpr int kPer = kGroupCh / 256;
    double S[kPer];
    uint32_t xo[kPer], no[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        int64_t c = y * kGroupCh + (int)threadIdx.x + 256 * j;
        c = c < HD ? c : HD - 1;
        S[j] = __hip_atomic_load(&w.sum[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        xo[j] = __hip_atomic_load(&w.kmax[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        no[j] = __hip_atomic_load(&w.kneg[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int64_t c = y * kGroupCh + (int)threadIdx.x + 256 * j;
        if (c < HD) {
            const float mu = (float)(S[j] / (double)T);
            mu_slot[c] = mu;
            if (mu_g) mu_g[c] = mu;
            if (mu_s) mu_s[c] = mu;
            // RN(max K - mu) and RN(mu - min K) = RN(mu + (-min K))
            am = fmaxf(am, fmaxf(ord_value(xo[j]) - mu, mu + ord_value(no[j])));
            __hip_atomic_store(&w.sum[c], 0.0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&w.kmax[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&w.kneg[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    am = wave_max(am);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t vb = __hip_atomic_load(&w.vmax[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        w.gamax[y] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        w.gvmax[y] = __uint_as_float(vb);
        __hip_atomic_store(&w.vmax[y], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&w.tick[y], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}


// Zero the store workspace (the first store of a ring).
__global__ __launch_bounds__(256) void kv_ws_clear_kernel(uint32_t *__restrict__ p, int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
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
// loaded before the prologue, which takes the key (or value) amax as the
// maximum of the channel groups' (or *v_amax_in), derives the tensor scale
// (workgroup 0 stores the decode scale into the slot and the sink copies)
// and builds the (S, r) table of the workgroup's tensor; afterwards each
// lane keeps two blocks in flight, with the loop unrolled three times so
// the three block registers rotate without copies.  Loads and stores are
// raw buffer accesses with 32-bit offsets: a block past the end loads as
// zero and its stores are dropped by the range check (also how only the
// blocks below the sink length reach the sink copies).  When the grid
// stride is a multiple of the blocks per token (MU_FIXED) every block of a
// lane starts at the same channel, and the lane holds its 16 key means in
// registers; otherwise they are re-read per block.
template <bool FOUR_OVER_SIX, bool MU_FIXED>
__global__ __launch_bounds__(256) void kv_encode_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, int64_t nblk, int64_t HD,
    const float *__restrict__ gamax, const float *__restrict__ gvmax, int gy,
    const float *__restrict__ v_amax_in, KvRegion slot, KvRegion gsink, KvRegion ssink,
    int64_t g_blk, int64_t s_blk) {
    __shared__ f32x2 lut[128];
    __shared__ float sh[2];
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
    if (threadIdx.x == 0) {
        const float *g = which ? gvmax : gamax;
        float a = 0.0f;
        for (int i = 0; i < gy; ++i) a = fmaxf(a, g[i]);
        if (which == 1 && v_amax_in) a = *v_amax_in;
        float e, d;
        tensor_scales(a, e, d);
        sh[0] = e;
        sh[1] = d;
        if (blockIdx.x == 0) {
            slot.sd[which] = d;
            if (g_blk > 0) gsink.sd[which] = d;
            if (s_blk > 0) ssink.sd[which] = d;
        }
    }
    __syncthreads();
    const float s_enc = sh[0];
    const float s_dec = sh[1];
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

// ---------------------------------------------------------------------------
// Store scratch without allocation: the store's workspace as a file-scope
// device array (each device the library runs on holds one until the process
// ends).  Its host-side name is only a stand-in: the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
// ---------------------------------------------------------------------------

constexpr int64_t kNoallocMaxHD = 16384;
constexpr size_t kNoallocScratchBytes =
    (size_t)(((kNoallocMaxHD * 8 + 255) & ~255) + 2 * ((kNoallocMaxHD * 4 + 255) & ~255) +
             4 * 256);
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

int64_t kv_noalloc_max_hd() { return kNoallocMaxHD; }
static_assert(kNoallocMaxHD == 16384, "allocation-free store limit (nvfp4.h)");

hipError_t kv_noalloc_scratch(void **ptr, size_t *bytes, hipStream_t s) {
    static std::mutex mu;
    static void *dev_ptr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!dev_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        // zero the accumulators once, ahead of the first store on the
        // caller's stream (a fill kernel, not a memset node; the array also
        // starts zero-initialised)
        const int64_t n4 = (int64_t)kNoallocScratchBytes / 4;
        hipLaunchKernelGGL(kv_ws_clear_kernel, dim3((unsigned)((n4 + 1023) / 1024)), dim3(256), 0,
                           s, (uint32_t *)p, n4);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        dev_ptr[dev] = p;
    }
    *ptr = dev_ptr[dev];
    *bytes = kNoallocScratchBytes;
    return hipSuccess;
}

hipError_t launch_kv_store(const KvStoreArgs &a, hipStream_t s) {
    const int64_t nodes = (a.T + kStatsTokens - 1) / kStatsTokens;
    const int64_t gy = (a.HD + kGroupCh - 1) / kGroupCh;
    KvWs w = carve_ws(a.ws, a.HD);
    if (a.clear_ws) {
        const int64_t n4 = kv_ws_zero_bytes(a.HD) / 4;
        NVFP4_LAUNCH("kv_ws_clear", kv_ws_clear_kernel, dim3((unsigned)((n4 + 1023) / 1024)),
                     dim3(256), 0, s, (uint32_t *)a.ws, n4);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const unsigned ny = a.v_amax_in ? 1u : 2u;
    NVFP4_LAUNCH("kv_stats", kv_stats_kernel, dim3((unsigned)(nodes * gy), ny),
                 dim3(64 * kStatsWaves), 0, s,
                 a.K, a.V, a.T, a.HD, gy, w, a.slot.mu,
                 a.g_tokens > 0 ? a.gsink.mu : (float *)nullptr,
                 a.s_tokens > 0 ? a.ssink.mu : (float *)nullptr, (uint32_t)(nodes * ny));
    hipError_t e = hipGetLastError();
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
#define NVFP4_ENC(F46, FIX)                                                                   \
    NVFP4_LAUNCH("kv_encode", (kv_encode_kernel<F46, FIX>), dim3((unsigned)g, 2), dim3(256), 0, \
                 s, a.K, a.V, nblk, a.HD, (const float *)w.gamax, (const float *)w.gvmax,       \
                 (int)gy, a.v_amax_in, a.slot, a.gsink, a.ssink, g_blk, s_blk)
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

// Each workgroup takes tpw consecutive tokens of one segment (found once,
// from the plan's first-workgroup table), so every token's region, key mean
// and decode scales are the workgroup's.  Lane i expands half-block i of K
// and V of each token (elements 8 i .. 8 i + 7: block i >> 1's scale and
// one dword of its codes), its 8 key means held in registers, with the
// loads of four tokens issued before any of them is expanded; each store
// instruction of a wave then writes 1 KB contiguous (a lane per whole block
// wrote 32 bytes at a 32-byte stride in two instructions: 141 against
// 113 us for the 33,440-token set of the 64 s ring).  The stores are
// non-temporal: the output is not left dirty in the caches, where its
// write-back slowed the next kernel (the next chunk's statistics pass: 24.3
// against 19.1 us a 7040-token step; the 33,440-token gather itself 108.9
// against 105.4 us).  Output rows follow the segments: ascending token
// order.
constexpr int kGatherTok = 4;

__global__ __launch_bounds__(512) void kv_gather_kernel(GatherArgs a) {
    int s = 0;
    while (s + 1 < a.nseg && (int)blockIdx.x >= a.wg0[s + 1]) ++s;
    const KvSeg &g = a.seg[s];
    const int64_t t_begin = (int64_t)((int)blockIdx.x - a.wg0[s]) * a.tpw;
    const int64_t t_end = t_begin + a.tpw < g.n ? t_begin + a.tpw : g.n;
    const int64_t NB = a.HD >> 4;  // blocks per token
    const float sdk = g.sd[0], sdv = g.sd[1];
    const uint32_t *kc = (const uint32_t *)g.kc, *vc = (const uint32_t *)g.vc;
    uint16_t *Ko = a.Kout + a.out0[s] * a.HD, *Vo = a.Vout + a.out0[s] * a.HD;
    for (int64_t i = threadIdx.x; i < 2 * NB; i += blockDim.x) {
        const int64_t j = i >> 1;
        float mu[8];
        load8(g.mu + i * 8, mu);
        for (int64_t t0 = t_begin; t0 < t_end; t0 += kGatherTok) {
            uint32_t qk[kGatherTok], qv[kGatherTok], sk[kGatherTok], sv[kGatherTok];
#pragma unroll
            for (int k = 0; k < kGatherTok; ++k) {
                const int64_t t = t0 + k < t_end ? t0 + k : t_end - 1;
                qk[k] = kc[t * 2 * NB + i];
                qv[k] = vc[t * 2 * NB + i];
                sk[k] = g.ks[t * NB + j];
                sv[k] = g.vs[t * NB + j];
            }
#pragma unroll
            for (int k = 0; k < kGatherTok; ++k) {
                const int64_t t = t0 + k;
                if (t >= t_end) break;
                const float Sk = e4m3_value(sk[k]) * sdk;
                const float Sv = e4m3_value(sv[k]) * sdv;
                float y[8];
                dequant8(qk[k], Sk, y);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = y[e] + mu[e];
                store8_stream(Ko + t * a.HD + i * 8, y);
                dequant8(qv[k], Sv, y);
                store8_stream(Vo + t * a.HD + i * 8, y);
            }
        }
    }
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s) {
    const int g = a.wg0[a.nseg];
    if (g == 0) return hipSuccess;
    const int64_t NB = a.HD >> 4;
    int64_t bs = ((2 * NB + 63) / 64) * 64;
    if (bs > 512) bs = 512;
    NVFP4_LAUNCH("kv_gather", kv_gather_kernel, dim3((unsigned)g), dim3((unsigned)bs), 0, s, a);
    return hipGetLastError();
}

}  // namespace nvfp4
