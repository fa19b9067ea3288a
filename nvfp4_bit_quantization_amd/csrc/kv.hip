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
//   kv_stats     one wave per (64-token tile, 512 channels): per-channel fp64
//                tile sums (token order), key max/min, value |max|
//   kv_finalize  one workgroup: mu = (float)(sum of tile sums / T), the key
//                amax max_c max(RN(max K - mu), RN(mu - min K)) (equal to the
//                elementwise amax of RN(K - mu) because RN is monotone), the
//                value amax, and the FP32 tensor scales of K_s and V
//   kv_encode    the 1-D 4/6 encoder over K_s = RN(K - mu) and V, writing the
//                ring slot and, for sink chunks, the sink copy in the same pass
// Gather = one launch: one workgroup-iteration per output token, one lane per
// 8 elements; each token's segment (ring slot or sink copy) is found by a
// scalar scan of <= W + 2 segments.
#include "device.hpp"
#include "launch.hpp"

namespace nvfp4 {

// Key-mean summation order (fixed, so the result is reproducible): tokens in
// tiles of kSeq = 16, each tile summed in token order in double; the tile
// sums, padded with zeros to a power-of-two count, added pairwise level by
// level.  kv_stats computes the tile sums and the first two tree levels (one
// workgroup = 4 waves = 4 consecutive tiles); kv_finalize finishes the tree.
constexpr int kSeq = 16;            // tokens summed sequentially by one lane
constexpr int kStatsTokens = 64;    // tokens per stats workgroup (4 waves x 16)
constexpr int kGroupCh = 256;       // channels per stats workgroup (64 lanes x 4)
constexpr int kFinCh = 64;          // channels per finalize workgroup

struct KvWs {
    double *P;      // [nt64, HD]  level-2 tree nodes (64-token sums)
    float *kmax;    // [nt64, HD]
    float *kmin;    // [nt64, HD]
    float *vpart;   // [nt64 * gy] value |max| per stats workgroup
    float *kpart;   // [nfin]      key amax per finalize workgroup
};

struct KvDims {
    int64_t nt64;   // stats workgroups along tokens
    int64_t gy;     // stats workgroups along channels
    int64_t n2;     // level-2 nodes in the padded tree (power of two)
    int64_t nfin;   // finalize workgroups
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

// Workgroup (tile p of 64 tokens, channel group g of 256, blockIdx.z = 0):
// wave w sums tokens 64p + 16w .. +15 of its lane's 4 channels sequentially;
// the four wave sums are combined as ((s0 + s1) + (s2 + s3)); key max/min
// per channel.  blockIdx.z = 1 workgroups take the value |max| of the same
// tile.  Loads are unconditional (token index clamped) so that all 16 of a
// lane's loads are in flight together; out-of-range tokens contribute +0 to
// the sums (no partial sum is -0, so adding +0 changes nothing) and nothing
// to the extrema.
__global__ __launch_bounds__(256) void kv_stats_kernel(const uint16_t *__restrict__ K,
                                                       const uint16_t *__restrict__ V, int64_t T,
                                                       int64_t HD, KvWs w) {
    __shared__ double sp[4][kGroupCh];
    __shared__ float smx[4][kGroupCh];
    __shared__ float smn[4][kGroupCh];
    __shared__ float svm[4];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t p = blockIdx.x;
    const int chl = lane * 4;
    const int64_t chq = (int64_t)blockIdx.y * kGroupCh + chl;
    const bool ch_ok = chq < HD;
    const int64_t ch0 = ch_ok ? chq : 0;
    const int64_t t0 = p * kStatsTokens + wave * kSeq;
    uint2 r[kSeq];
    const uint16_t *src = blockIdx.z ? V : K;
#pragma unroll
    for (int j = 0; j < kSeq; ++j) {
        const int64_t t = (t0 + j < T) ? t0 + j : T - 1;
        r[j] = *(const uint2 *)(src + t * HD + ch0);
    }
    if (blockIdx.z) {
        float vmx = 0.0f;
#pragma unroll
        for (int j = 0; j < kSeq; ++j) {
            const bool ok = ch_ok && (t0 + j < T);
            const float m = fmaxf(fmaxf(fabsf(bf16lo(r[j].x)), fabsf(bf16hi(r[j].x))),
                                  fmaxf(fabsf(bf16lo(r[j].y)), fabsf(bf16hi(r[j].y))));
            vmx = ok ? fmaxf(vmx, m) : vmx;
        }
        vmx = wave_max(vmx);
        if (lane == 0) svm[wave] = vmx;
        __syncthreads();
        if (threadIdx.x == 0)
            w.vpart[p * gridDim.y + blockIdx.y] =
                fmaxf(fmaxf(svm[0], svm[1]), fmaxf(svm[2], svm[3]));
        return;
    }
    double s[4];
    float mx[4], mn[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s[i] = 0.0;
        mx[i] = -__builtin_huge_valf();
        mn[i] = __builtin_huge_valf();
    }
#pragma unroll
    for (int j = 0; j < kSeq; ++j) {
        const bool ok = t0 + j < T;
        const float v[4] = {bf16lo(r[j].x), bf16hi(r[j].x), bf16lo(r[j].y), bf16hi(r[j].y)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] += ok ? (double)v[i] : 0.0;
            mx[i] = ok ? fmaxf(mx[i], v[i]) : mx[i];
            mn[i] = ok ? fminf(mn[i], v[i]) : mn[i];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sp[wave][chl + i] = s[i];
        smx[wave][chl + i] = mx[i];
        smn[wave][chl + i] = mn[i];
    }
    __syncthreads();
    {
        const int c = threadIdx.x;  // 256 threads, 256 channels
        const int64_t ch = (int64_t)blockIdx.y * kGroupCh + c;
        if (ch < HD) {
            const double P = (sp[0][c] + sp[1][c]) + (sp[2][c] + sp[3][c]);
            w.P[p * HD + ch] = P;
            w.kmax[p * HD + ch] = fmaxf(fmaxf(smx[0][c], smx[1][c]), fmaxf(smx[2][c], smx[3][c]));
            w.kmin[p * HD + ch] = fminf(fminf(smn[0][c], smn[1][c]), fminf(smn[2][c], smn[3][c]));
        }
    }
}

// Tree sum of 32 doubles, adjacent pairs level by level.
__device__ __forceinline__ double tree32(double (&v)[32]) {
#pragma unroll
    for (int w = 16; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) v[i] = v[2 * i] + v[2 * i + 1];
    return v[0];
}

// Workgroup of 256 threads = 4 waves over 64 channels (lane = channel).  The
// level-2 nodes of a channel form blocks of 32 (nodes past the last 64-token
// tile are zero); wave q sums blocks q, q+4, ... with a fixed 32-leaf tree
// into LDS, then wave 0 sums the block sums with the same tree (zero padded;
// adding an exact zero changes nothing, and no partial sum is -0).  This is
// the level-by-level pairwise tree over the 16-token tile sums.
// mu = (float)(S / T); the workgroup's key amax
// max_c max(RN(max K - mu), RN(mu - min K)) goes to kpart.
__global__ __launch_bounds__(256) void kv_finalize_kernel(KvWs w, int64_t nt64, int64_t n2,
                                                          int64_t T, int64_t HD, float *mu_slot,
                                                          float *mu_g, float *mu_s) {
    __shared__ double bs[32][kFinCh];
    __shared__ float rx[4][kFinCh];
    __shared__ float rn[4][kFinCh];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t ch = (int64_t)blockIdx.x * kFinCh + lane;
    const int nb = n2 >= 32 ? (int)(n2 / 32) : 1;  // blocks of 32 nodes (<= 32)
    float kx = -__builtin_huge_valf(), kn = __builtin_huge_valf();
    const int64_t chc = ch < HD ? ch : HD - 1;
    for (int b = wave; b < nb; b += 4) {
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
        bs[b][lane] = tree32(v);
    }
    rx[wave][lane] = kx;
    rn[wave][lane] = kn;
    __syncthreads();
    if (wave != 0) return;
    float amax = 0.0f;
    if (ch < HD) {
        double v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = (i < nb) ? bs[i][lane] : 0.0;
        const double S = tree32(v);
        const float mu = (float)(S / (double)T);
        mu_slot[ch] = mu;
        if (mu_g) mu_g[ch] = mu;
        if (mu_s) mu_s[ch] = mu;
        const float x = fmaxf(fmaxf(rx[0][lane], rx[1][lane]), fmaxf(rx[2][lane], rx[3][lane]));
        const float n = fminf(fminf(rn[0][lane], rn[1][lane]), fminf(rn[2][lane], rn[3][lane]));
        amax = fmaxf(x - mu, mu - n);
    }
    amax = wave_max(amax);
    if (lane == 0) w.kpart[blockIdx.x] = amax;
}

// One lane per 1x16 block along the (head, dim) axis; blockIdx.y = 0: keys
// (K_s = RN(K - mu)), 1: values.  The prologue reduces the key / value amax
// partials, derives both tensor scales (workgroup (0,0) stores the decode
// scales into the slot and the sink copies) and builds the (S, r) table of
// the workgroup's tensor.  Blocks below the sink length are also written to
// the sink copies.
template <bool FOUR_OVER_SIX>
__global__ __launch_bounds__(256) void kv_encode_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, int64_t nblk, int64_t HD,
    const float *__restrict__ kpart, int nk, const float *__restrict__ vpart, int nv,
    KvRegion slot, KvRegion gsink, KvRegion ssink, int64_t g_blk, int64_t s_blk) {
    __shared__ f32x2 lut[128];
    __shared__ float red[2][4];
    __shared__ float sh[4];
    const int which = blockIdx.y;  // 0: keys, 1: values
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
    const uint16_t *x = which ? V : K;
    uint2 *codes = (uint2 *)(which ? slot.vc : slot.kc);
    uint8_t *scales = which ? slot.vs : slot.ks;
    uint2 *gcodes = (uint2 *)(which ? gsink.vc : gsink.kc);
    uint8_t *gscales = which ? gsink.vs : gsink.ks;
    uint2 *scodes = (uint2 *)(which ? ssink.vc : ssink.kc);
    uint8_t *sscales = which ? ssink.vs : ssink.ks;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // channel of the block's first element, advanced without division: (16 b) mod HD
    int64_t ch0 = (b * 16) % HD;
    const int64_t step = (stride * 16) % HD;
    Raw16Bf16 rn;
    if (b < nblk) load_raw16(x + b * 16, rn);
    for (; b < nblk; b += stride) {
        // the next block's load is issued before this block is encoded
        const Raw16Bf16 r = rn;
        if (b + stride < nblk) load_raw16(x + (b + stride) * 16, rn);
        float v[16];
        unpack16(r, v);
        if (which == 0) {
            Raw16F32 m;
            load_raw16(slot.mu + ch0, m);
            float mu[16];
            unpack16(m, mu);
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = v[i] - mu[i];
        }
        uint32_t lo, hi, sc;
        encode_block16<FOUR_OVER_SIX>(v, s_enc, lut, lo, hi, sc);
        codes[b] = make_uint2(lo, hi);
        scales[b] = (uint8_t)sc;
        if (b < g_blk) {
            gcodes[b] = make_uint2(lo, hi);
            gscales[b] = (uint8_t)sc;
        }
        if (b < s_blk) {
            scodes[b] = make_uint2(lo, hi);
            sscales[b] = (uint8_t)sc;
        }
        ch0 += step;
        if (ch0 >= HD) ch0 -= HD;
    }
}

hipError_t launch_kv_store(const KvStoreArgs &a, hipStream_t s) {
    const KvDims d = kv_dims(a.T, a.HD);
    KvWs w = carve_ws(a.ws, a.T, a.HD);
    NVFP4_LAUNCH("kv_stats", kv_stats_kernel, dim3((unsigned)d.nt64, (unsigned)d.gy, 2),
                 dim3(256), 0, s, a.K, a.V, a.T, a.HD, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    NVFP4_LAUNCH("kv_finalize", kv_finalize_kernel, dim3((unsigned)d.nfin), dim3(256), 0, s, w,
                 d.nt64, d.n2, a.T, a.HD, a.slot.mu,
                 a.g_tokens > 0 ? a.gsink.mu : (float *)nullptr,
                 a.s_tokens > 0 ? a.ssink.mu : (float *)nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nblk = a.T * a.HD / 16;
    int64_t g = (nblk + 255) / 256;
    if (g > 512) g = 512;
    if (g < 1) g = 1;
    const int64_t g_blk = a.g_tokens * a.HD / 16, s_blk = a.s_tokens * a.HD / 16;
    const int nk = (int)d.nfin, nv = (int)(d.nt64 * d.gy);
    if (a.search == 1)
        NVFP4_LAUNCH("kv_encode", kv_encode_kernel<true>, dim3((unsigned)g, 2), dim3(256), 0, s,
                     a.K, a.V, nblk, a.HD, (const float *)w.kpart, nk, (const float *)w.vpart, nv,
                     a.slot, a.gsink, a.ssink, g_blk, s_blk);
    else
        NVFP4_LAUNCH("kv_encode", kv_encode_kernel<false>, dim3((unsigned)g, 2), dim3(256), 0, s,
                     a.K, a.V, nblk, a.HD, (const float *)w.kpart, nk, (const float *)w.vpart, nv,
                     a.slot, a.gsink, a.ssink, g_blk, s_blk);
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
