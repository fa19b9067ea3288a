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

constexpr int kTile = 64;          // tokens per statistics tile
constexpr int kStatsLanes = 64;    // lanes per stats workgroup (8 channels each)

struct KvWs {
    double *P;       // [ntiles, HD]
    float *kmax;     // [ntiles, HD]
    float *kmin;     // [ntiles, HD]
    float *vpart;    // [ntiles * gy]
    float *senc;     // [2]
};

static inline int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

static KvWs carve_ws(void *ws, int64_t T, int64_t HD) {
    const int64_t ntiles = (T + kTile - 1) / kTile;
    const int64_t gy = (HD / 8 + kStatsLanes - 1) / kStatsLanes;
    uint8_t *p = (uint8_t *)ws;
    KvWs w;
    w.P = (double *)p;
    p += align256(ntiles * HD * 8);
    w.kmax = (float *)p;
    p += align256(ntiles * HD * 4);
    w.kmin = (float *)p;
    p += align256(ntiles * HD * 4);
    w.vpart = (float *)p;
    p += align256(ntiles * gy * 4);
    w.senc = (float *)p;
    return w;
}

size_t kv_store_ws_bytes(int64_t T, int64_t HD) {
    const int64_t ntiles = (T + kTile - 1) / kTile;
    const int64_t gy = (HD / 8 + kStatsLanes - 1) / kStatsLanes;
    return (size_t)(align256(ntiles * HD * 8) + 2 * align256(ntiles * HD * 4) +
                    align256(ntiles * gy * 4) + 256);
}

__global__ __launch_bounds__(64) void kv_stats_kernel(const uint16_t *__restrict__ K,
                                                      const uint16_t *__restrict__ V, int64_t T,
                                                      int64_t HD, KvWs w) {
    const int64_t p = blockIdx.x;
    const int64_t ch0 = ((int64_t)blockIdx.y * kStatsLanes + threadIdx.x) * 8;
    const int64_t t0 = p * kTile;
    const int64_t t1 = (t0 + kTile < T) ? t0 + kTile : T;
    float vmx = 0.0f;
    if (ch0 < HD) {
        double s[8];
        float mx[8], mn[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[i] = 0.0;
            mx[i] = -__builtin_huge_valf();
            mn[i] = __builtin_huge_valf();
        }
        for (int64_t t = t0; t < t1; ++t) {
            float k[8], v[8];
            load8(K + t * HD + ch0, k);
            load8(V + t * HD + ch0, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                s[i] += (double)k[i];
                mx[i] = fmaxf(mx[i], k[i]);
                mn[i] = fminf(mn[i], k[i]);
                vmx = fmaxf(vmx, fabsf(v[i]));
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w.P[p * HD + ch0 + i] = s[i];
            w.kmax[p * HD + ch0 + i] = mx[i];
            w.kmin[p * HD + ch0 + i] = mn[i];
        }
    }
    vmx = wave_max(vmx);
    if (threadIdx.x == 0) w.vpart[p * gridDim.y + blockIdx.y] = vmx;
}

__global__ __launch_bounds__(1024) void kv_finalize_kernel(KvWs w, int64_t ntiles, int64_t nvpart,
                                                           int64_t T, int64_t HD, float *mu_slot,
                                                           float *mu_g, float *mu_s,
                                                           float *sd_slot, float *sd_g,
                                                           float *sd_s) {
    __shared__ float red[2][16];
    float ak = 0.0f, av = 0.0f;
    for (int64_t ch = threadIdx.x; ch < HD; ch += blockDim.x) {
        double S = 0.0;
        float kx = -__builtin_huge_valf(), kn = __builtin_huge_valf();
        for (int64_t p = 0; p < ntiles; ++p) {
            S += w.P[p * HD + ch];
            kx = fmaxf(kx, w.kmax[p * HD + ch]);
            kn = fminf(kn, w.kmin[p * HD + ch]);
        }
        const float mu = (float)(S / (double)T);
        mu_slot[ch] = mu;
        if (mu_g) mu_g[ch] = mu;
        if (mu_s) mu_s[ch] = mu;
        ak = fmaxf(ak, fmaxf(kx - mu, mu - kn));
    }
    for (int64_t i = threadIdx.x; i < nvpart; i += blockDim.x) av = fmaxf(av, w.vpart[i]);
    ak = wave_max(ak);
    av = wave_max(av);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red[0][wave] = ak;
        red[1][wave] = av;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float a0 = 0.0f, a1 = 0.0f;
        for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
            a0 = fmaxf(a0, red[0][i]);
            a1 = fmaxf(a1, red[1][i]);
        }
        float e0, d0, e1, d1;
        tensor_scales(a0, e0, d0);
        tensor_scales(a1, e1, d1);
        w.senc[0] = e0;
        w.senc[1] = e1;
        sd_slot[0] = d0;
        sd_slot[1] = d1;
        if (sd_g) {
            sd_g[0] = d0;
            sd_g[1] = d1;
        }
        if (sd_s) {
            sd_s[0] = d0;
            sd_s[1] = d1;
        }
    }
}

// Encoder core shared in spirit with quantize.hip's 1-D encoder: lane = 8
// elements, lane pair = one 1x16 block along the (head, dim) axis.
template <bool FOUR_OVER_SIX>
__device__ __forceinline__ void kv_encode_half(const float (&x)[8], float s_enc, const f32x2 *lut,
                                               uint32_t &codes, uint32_t &scale) {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(x[i]));
    am = fmaxf(am, swap_pair(am));
    float id6 = (am / 6.0f) * s_enc;
    uint32_t sc6 = e4m3_encode(id6);
    f32x2 sr6 = lut[sc6];
    uint32_t q6 = e2m1_pack8(x, sr6.y);
    if (!FOUR_OVER_SIX) {
        codes = q6;
        scale = sc6;
        return;
    }
    float e6 = half_block_error(x, q6, sr6.x);
    float id4 = (am * 0.25f) * s_enc;
    uint32_t sc4 = e4m3_encode(id4);
    f32x2 sr4 = lut[sc4];
    uint32_t q4 = e2m1_pack8(x, sr4.y);
    float e4 = half_block_error(x, q4, sr4.x);
    e6 = e6 + swap_pair(e6);
    e4 = e4 + swap_pair(e4);
    const bool pick4 = e4 < e6;
    codes = pick4 ? q4 : q6;
    scale = pick4 ? sc4 : sc6;
}

template <bool FOUR_OVER_SIX>
__global__ __launch_bounds__(256) void kv_encode_kernel(const uint16_t *__restrict__ K,
                                                        const uint16_t *__restrict__ V,
                                                        int64_t n8, int64_t HD,
                                                        const float *__restrict__ senc,
                                                        KvRegion slot, KvRegion gsink,
                                                        KvRegion ssink, int64_t g_n8,
                                                        int64_t s_n8) {
    __shared__ f32x2 lut[128];
    const int which = blockIdx.y;  // 0: keys, 1: values
    const float s_dec = slot.sd[which];
    const float s_enc = senc[which];
    for (int c = threadIdx.x; c < 128; c += blockDim.x) {
        float S = e4m3_value((uint32_t)c) * s_dec;
        lut[c] = f32x2{S, (S == 0.0f) ? 0.0f : 1.0f / S};
    }
    __syncthreads();
    const uint16_t *x = which ? V : K;
    uint32_t *codes = (uint32_t *)(which ? slot.vc : slot.kc);
    uint8_t *scales = which ? slot.vs : slot.ks;
    uint32_t *gcodes = (uint32_t *)(which ? gsink.vc : gsink.kc);
    uint8_t *gscales = which ? gsink.vs : gsink.ks;
    uint32_t *scodes = (uint32_t *)(which ? ssink.vc : ssink.kc);
    uint8_t *sscales = which ? ssink.vs : ssink.ks;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // channel of the unit's first element, advanced incrementally (no division
    // in the loop): ch0 = (8u) mod HD
    int64_t ch0 = (u * 8) % HD;
    const int64_t step = (stride * 8) % HD;
    for (; u < n8; u += stride) {
        float v[8];
        load8(x + u * 8, v);
        if (which == 0) {
            float m[8];
            load8(slot.mu + ch0, m);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = v[i] - m[i];
        }
        uint32_t q, sc;
        kv_encode_half<FOUR_OVER_SIX>(v, s_enc, lut, q, sc);
        codes[u] = q;
        const bool lead = (u & 1) == 0;
        if (lead) scales[u >> 1] = (uint8_t)sc;
        if (u < g_n8) {
            gcodes[u] = q;
            if (lead) gscales[u >> 1] = (uint8_t)sc;
        }
        if (u < s_n8) {
            scodes[u] = q;
            if (lead) sscales[u >> 1] = (uint8_t)sc;
        }
        ch0 += step;
        if (ch0 >= HD) ch0 -= HD;
    }
}

hipError_t launch_kv_store(const KvStoreArgs &a, hipStream_t s) {
    const int64_t ntiles = (a.T + kTile - 1) / kTile;
    const int64_t gy = (a.HD / 8 + kStatsLanes - 1) / kStatsLanes;
    KvWs w = carve_ws(a.ws, a.T, a.HD);
    NVFP4_LAUNCH("kv_stats", kv_stats_kernel, dim3((unsigned)ntiles, (unsigned)gy),
                 dim3(kStatsLanes), 0, s, a.K, a.V, a.T, a.HD, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    NVFP4_LAUNCH("kv_finalize", kv_finalize_kernel, dim3(1), dim3(1024), 0, s, w, ntiles, ntiles * gy,
                       a.T, a.HD, a.slot.mu, a.g_tokens > 0 ? a.gsink.mu : (float *)nullptr,
                       a.s_tokens > 0 ? a.ssink.mu : (float *)nullptr, a.slot.sd,
                       a.g_tokens > 0 ? a.gsink.sd : (float *)nullptr,
                       a.s_tokens > 0 ? a.ssink.sd : (float *)nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n8 = a.T * a.HD / 8;
    int64_t g = (n8 + 1023) / 1024;
    if (g > 4096) g = 4096;
    if (g < 1) g = 1;
    const int64_t g_n8 = a.g_tokens * a.HD / 8, s_n8 = a.s_tokens * a.HD / 8;
    if (a.search == 1)
        NVFP4_LAUNCH("kv_encode", kv_encode_kernel<true>, dim3((unsigned)g, 2), dim3(256), 0, s, a.K,
                           a.V, n8, a.HD, (const float *)w.senc, a.slot, a.gsink, a.ssink, g_n8,
                           s_n8);
    else
        NVFP4_LAUNCH("kv_encode", kv_encode_kernel<false>, dim3((unsigned)g, 2), dim3(256), 0, s, a.K,
                           a.V, n8, a.HD, (const float *)w.senc, a.slot, a.gsink, a.ssink, g_n8,
                           s_n8);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gather-dequantize of K_eff(t)
// ---------------------------------------------------------------------------

// Output order: [global-sink tokens outside the window][shot-sink tokens
// outside the window][window chunks c_lo .. c_lo + nwin - 1]; sinks lie below
// the window in token order, so this is ascending token order.
__global__ __launch_bounds__(1024) void kv_gather_kernel(GatherArgs a) {
    const int64_t U = a.HD >> 3;   // 8-element units per token
    const int64_t SB = a.HD >> 4;  // scale bytes per token
    for (int64_t tok = blockIdx.x; tok < a.n_tokens; tok += gridDim.x) {
        KvRegion r;
        int64_t st;
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
        const float sdk = r.sd[0], sdv = r.sd[1];
        const uint32_t *kc = (const uint32_t *)r.kc + st * U;
        const uint32_t *vc = (const uint32_t *)r.vc + st * U;
        const uint8_t *ks = r.ks + st * SB;
        const uint8_t *vs = r.vs + st * SB;
        uint16_t *ko = a.Kout + tok * a.HD;
        uint16_t *vo = a.Vout + tok * a.HD;
        for (int64_t j = threadIdx.x; j < U; j += blockDim.x) {
            const uint32_t qk = kc[j], qv = vc[j];
            const float Sk = e4m3_value(ks[j >> 1]) * sdk;
            const float Sv = e4m3_value(vs[j >> 1]) * sdv;
            float yk[8], yv[8], m[8];
            dequant8(qk, Sk, yk);
            dequant8(qv, Sv, yv);
            load8(r.mu + j * 8, m);
#pragma unroll
            for (int i = 0; i < 8; ++i) yk[i] = yk[i] + m[i];
            store8(ko + j * 8, yk);
            store8(vo + j * 8, yv);
        }
    }
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s) {
    if (a.n_tokens == 0) return hipSuccess;
    const int64_t U = a.HD >> 3;
    int64_t bs = ((U + 63) / 64) * 64;
    if (bs > 1024) bs = 1024;
    int64_t g = a.n_tokens < 4096 ? a.n_tokens : 4096;
    NVFP4_LAUNCH("kv_gather", kv_gather_kernel, dim3((unsigned)g), dim3((unsigned)bs), 0, s, a);
    return hipGetLastError();
}

}  // namespace nvfp4
