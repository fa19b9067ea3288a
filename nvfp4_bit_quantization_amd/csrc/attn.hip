// attn.hip -- attention of a chunk's queries over the NVFP4 KV ring's
// effective set, the dequantization fused into the key/value staging
// (gfx950, bf16 MFMA).
//
// Method (LongLive-2.0 pages): "MCISLAB DeepRead: LongLive2" summary,
// Multi-Shot Attention Sink -- sliding-window self-attention over the
// effective set K_eff(t) = A_g u A_s u KV[t-W, t) -- and parallel KV
// quantization (packed NVFP4 KV cache, a custom dequantization kernel); TX
// page, NVFP4 section: the FP4 KV cache comes with a fused dequantization
// extension.
//
// Per head: O[q] = sum_j softmax_j(scale * Q[q] . K_hat[j]) V_hat[j], with
// K_hat = bf16(RN(RN(V * S) + mu)) and V_hat = bf16(RN(V * S)) exactly as the
// gather-dequantizer writes them (S = RN(sigma * s_dec) per 1x16 block, mu
// the key mean of the token's region).  lse[q] = ln sum_j exp(scale Q.K_j).
//
// Workgroup: 256 queries of one head, 8 waves of 32 queries (two waves a
// SIMD, so one wave's softmax and dequantization run under the other's
// MFMAs).  The effective set is walked segment by segment (each segment one
// region: one key mean, one pair of decode scales), 64 keys a tile, through
// two LDS stages.  Every tile is dequantized once per workgroup straight
// from the packed ring (waves 0-3 the V blocks, 2 keys x 16 d a lane; waves
// 4-7 the K blocks, 2 keys x 16 d a lane) into
//   K tile   [64 keys][128 d] bf16: 16-byte column c of key k in slot c ^ (k & 15)
//   V^T tile [128 d][64 keys] bf16: keys permuted (below); 16-byte slot s of
//            row d in s ^ ((d >> 1) & 7) ^ ((d >> 4) & 7)
// so each fragment read (16 lanes x 16 bytes) meets 16 different groups of
// the 64 banks.  Per tile and wave: S^T = K_hat Q^T on
// v_mfma_f32_32x32x16_bf16 (a lane holds one query and 32 of the tile's
// scores), the online softmax in registers (exp2 of the scores times
// scale * log2 e), P^T rounded to bf16, O^T += V_hat^T P^T.  A lane of the
// 32x32 accumulator holds, for key block kb and element e, key
// kb * 32 + h * 4 + (e >> 2) * 8 + (e & 3) (h = lane >> 5); V^T keeps key k of
// each 16-key group at column ((k >> 2) & 1) * 8 + ((k >> 3) & 1) * 4 + (k & 3),
// so the 8 keys of a lane's P^T operand slots are 16 contiguous bytes of V^T.
// Each wave's queries sit in LDS too (same swizzle as the K tile), read one
// 16-deep fragment at a time.  The global loads of tile j + 1 are issued
// before tile j's MFMAs and dequantized into the other stage after them; one
// barrier per tile.
#include <atomic>

#include "device.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kAD = 128;                   // head dim
constexpr int kAQ = 256;                   // queries per workgroup (8 waves)
constexpr int kAK = 64;                    // keys per tile
constexpr int kATile = kAK * kAD * 2;      // bytes of the K tile (and of V^T)
constexpr int kAStage = 2 * kATile;        // K tile, then V^T tile
constexpr int kAQOff = 2 * kAStage;        // then each wave's 32 queries x 128 d
constexpr int kALds = kAQOff + kAQ * kAD * 2;  // 128 KB

// Column of V^T that holds key k of a tile.
__device__ __forceinline__ int vt_col(int k) {
    return (k & ~15) | (((k >> 2) & 1) << 3) | (((k >> 3) & 1) << 2) | (k & 3);
}

// Segment of tile j (uniform scan over the cumulative tile counts).
__device__ __forceinline__ int seg_of(const AttnArgs &a, int j) {
    int s = 0;
    while (s + 1 < a.nseg && a.tile0[s + 1] <= j) ++s;
    return s;
}

// One lane's packed blocks of a tile: 2 keys x one 16-element block along d.
// A key past the segment's end reads the segment's last token instead: its
// score is masked to -inf, so its weight is exactly 0 and its (finite)
// values never count.
struct TileBlocks {
    u32x2 c[2];
    uint32_t sc[2];
};

// V lanes (waves 0-3, t = threadIdx.x): keys 2 (t >> 3) + i, d block t & 7.
// K lanes (waves 4-7, t = threadIdx.x - 256): keys (t >> 3) + 32 i, d block t & 7.
__device__ __forceinline__ int tile_key(bool vrole, int t, int i) {
    return vrole ? 2 * (t >> 3) + i : (t >> 3) + 32 * i;
}

__device__ __forceinline__ void load_blocks(const AttnArgs &a, const AttnSeg &sg, int64_t tok0,
                                            bool vrole, int t, int head, TileBlocks &tb) {
    const int b = t & 7;
    const uint8_t *codes = vrole ? sg.vc : sg.kc;
    const uint8_t *scales = vrole ? sg.vs : sg.ks;
    const int64_t cstride = a.HD >> 1, sstride = a.HD >> 4;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int64_t tok = tok0 + tile_key(vrole, t, i);
        tok = tok < sg.n ? tok : sg.n - 1;
        tb.c[i] = *(const u32x2 *)(codes + tok * cstride + head * 64 + b * 8);
        tb.sc[i] = scales[tok * sstride + head * 8 + b];
    }
}

// Dequantize a lane's blocks into `stage` (K rows or V^T columns).
__device__ __forceinline__ void store_blocks(uint8_t *stage, const AttnSeg &sg, bool vrole, int t,
                                             int head, const TileBlocks &tb) {
    const int b = t & 7;
    if (vrole) {
        const float sdv = sg.sd[1];
        float S[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) S[i] = e4m3_value(tb.sc[i]) * sdv;
        const int col = vt_col(2 * (t >> 3));  // 2 consecutive columns
        const int slot = col >> 3, off = (col & 7) * 2;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float y[2][8];
#pragma unroll
            for (int i = 0; i < 2; ++i) dequant8(half ? tb.c[i].y : tb.c[i].x, S[i], y[i]);
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                const int d = b * 16 + half * 8 + dd;
                const int phys = slot ^ ((d >> 1) & 7) ^ ((d >> 4) & 7);
                *(uint32_t *)(stage + kATile + d * 128 + phys * 16 + off) =
                    pack_bf16x2(y[0][dd], y[1][dd]);
            }
        }
    } else {
        const float sdk = sg.sd[0];
        Raw16F32 m;
        load_raw16(sg.mu + head * kAD + b * 16, m);
        float mu[16];
        unpack16(m, mu);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int k = tile_key(false, t, i);
            const float S = e4m3_value(tb.sc[i]) * sdk;
            float y0[8], y1[8];
            dequant8(tb.c[i].x, S, y0);
            dequant8(tb.c[i].y, S, y1);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                y0[e] = y0[e] + mu[e];
                y1[e] = y1[e] + mu[8 + e];
            }
            const u32x4 lo{pack_bf16x2(y0[0], y0[1]), pack_bf16x2(y0[2], y0[3]),
                           pack_bf16x2(y0[4], y0[5]), pack_bf16x2(y0[6], y0[7])};
            const u32x4 hi{pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3]),
                           pack_bf16x2(y1[4], y1[5]), pack_bf16x2(y1[6], y1[7])};
            *(u32x4 *)(stage + k * 256 + (((2 * b) ^ (k & 15)) * 16)) = lo;
            *(u32x4 *)(stage + k * 256 + (((2 * b + 1) ^ (k & 15)) * 16)) = hi;
        }
    }
}

__global__ __launch_bounds__(512) void attn_window_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // workgroups of one head run on one XCD (b % 8), sharing its L2
    const int64_t nqt = (a.nq + kAQ - 1) / kAQ;
    const int64_t total = nqt * a.heads;
    const int64_t bid = blockIdx.x;
    const int64_t per = total / 8;
    const int64_t tix = bid < per * 8 ? (bid % 8) * per + bid / 8 : bid;
    const int head = (int)(tix / nqt);
    const int64_t q0 = (tix % nqt) * kAQ;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 31, h = lane >> 5;
    const bool vrole = wave < 4;
    const int t = vrole ? threadIdx.x : threadIdx.x - 256;

    // the wave's queries (Q^T operand rows) into its LDS region: query
    // qw + c in row c, 16-byte column x in slot x ^ (c & 15); lane (c, h)
    // copies columns 2 ks + h
    const int64_t qw = q0 + wave * 32;
    const int64_t qi = qw + c;
    uint8_t *const qs = lds + kAQOff + wave * (32 * kAD * 2);
    {
        const uint16_t *qp = a.q + (qi < a.nq ? qi : a.nq - 1) * a.HD + head * kAD + h * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            *(u32x4 *)(qs + c * 256 + (((2 * ks + h) ^ (c & 15)) * 16)) =
                *(const u32x4 *)(qp + ks * 16);
    }

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = 0.0f;
    float m_run = -__builtin_inff(), l_run = 0.0f;

    const int ntile = a.tile0[a.nseg];
    TileBlocks tb;
    if (ntile > 0) {
        const int s = seg_of(a, 0);
        load_blocks(a, a.seg[s], 0, vrole, t, head, tb);
        store_blocks(lds, a.seg[s], vrole, t, head, tb);
    }
    __syncthreads();

    for (int j = 0; j < ntile; ++j) {
        const bool more = j + 1 < ntile;
        const int sj = seg_of(a, j);
        const int sn = more ? seg_of(a, j + 1) : sj;
        if (more) load_blocks(a, a.seg[sn], (int64_t)(j + 1 - a.tile0[sn]) * kAK, vrole, t, head, tb);

        const uint8_t *st = lds + (j & 1) * kAStage;
        // S^T = K_hat Q^T: two 32-key blocks, alternating so that no MFMA
        // waits for the one before it (keys kb * 32 + c share the swizzle
        // of query row c)
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int col = ((2 * ks + h) ^ (c & 15)) * 16;
            const bf16x8 qv = *(const bf16x8 *)(qs + c * 256 + col);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 kf = *(const bf16x8 *)(st + (kb * 32 + c) * 256 + col);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qv, sacc[kb], 0, 0, 0);
            }
        }
        // keys past the segment's end
        const int64_t nvalid = a.seg[sj].n - (int64_t)(j - a.tile0[sj]) * kAK;
        if (nvalid < kAK) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (kb * 32 + h * 4 + (e >> 2) * 8 + (e & 3) >= nvalid)
                        sacc[kb][e] = -__builtin_inff();
        }
        // online softmax
        float mx = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * a.scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float ps = 0.0f;
        u32x4 pw[4];  // P^T operands: bf16 pairs
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e], a.scale_log2, -m_new));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e + 1], a.scale_log2, -m_new));
                ps += p0;
                ps += p1;
                pw[kb * 2 + (e >> 3)][(e & 7) >> 1] = pack_bf16x2(p0, p1);
            }
        l_run = __builtin_fmaf(l_run, alpha, ps);
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
        }
        m_run = m_new;
        // O^T += V_hat^T P^T
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int d = db * 32 + c;
            const int sw = ((d >> 1) & 7) ^ ((d >> 4) & 7);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 vf =
                    *(const bf16x8 *)(st + kATile + d * 128 + (((2 * kk + h) ^ sw) * 16));
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, pw[kk]),
                                                                o[db], 0, 0, 0);
            }
        }
        if (more) store_blocks(lds + ((j + 1) & 1) * kAStage, a.seg[sn], vrole, t, head, tb);
        __syncthreads();
    }

    // both lane halves saw every score maximum, so m_run agrees; the sums add
    const float lt = l_run + __shfl_xor(l_run, 32);
    if (qi < a.nq) {
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        uint16_t *op = a.o + qi * a.HD + head * kAD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + h * 4 + g * 8;
                *(u32x2 *)(op + d) =
                    u32x2{pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                          pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
            }
        if (a.lse && h == 0)
            a.lse[qi * a.heads + head] =
                lt > 0.0f ? (m_run + log2f(lt)) * 0.69314718055994531f : -__builtin_inff();
    }
}

hipError_t launch_attn_window(const AttnArgs &a, hipStream_t s) {
    if (a.nq == 0) return hipSuccess;
    static std::atomic<uint32_t> lds_set{0};
    const void *fn = (const void *)attn_window_kernel;
    hipError_t e = lds_limit_once(&fn, 1, kALds, lds_set);
    if (e != hipSuccess) return e;
    const int64_t grid = ((a.nq + kAQ - 1) / kAQ) * a.heads;
    NVFP4_LAUNCH("attn_window", attn_window_kernel, dim3((unsigned)grid), dim3(512), kALds, s, a);
    return hipGetLastError();
}

}  // namespace nvfp4
