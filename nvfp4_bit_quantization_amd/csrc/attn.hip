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
// three LDS stages.  Every tile is dequantized once per workgroup straight
// from the packed ring (every lane one K block and half a V block for a
// pair of keys) into
//   K tile   [64 keys][128 d] bf16: 16-byte column c of key k in slot c ^ (k & 15)
//   V^T tile [128 d][64 keys] bf16: keys permuted (below); 16-byte slot s of
//            row d in s ^ ((d >> 1) & 7) ^ ((d >> 4) & 7)
// so each fragment read (16 lanes x 16 bytes) meets 16 different groups of
// the 64 banks.  Per tile and wave: S^T = K_hat Q^T on
// v_mfma_f32_32x32x16_bf16 (a lane holds one query and 32 of the tile's
// scores), the online softmax in registers (exp2 of the scores times
// scale * log2 e, against a reference maximum that moves only when a score
// passes it by more than 2^8), P^T rounded to bf16, O^T += V_hat^T P^T; the
// normaliser sums the same bf16 weights (v_dot2_f32_bf16 against ones, two
// a step).  A lane of the
// 32x32 accumulator holds, for key block kb and element e, key
// kb * 32 + h * 4 + (e >> 2) * 8 + (e & 3) (h = lane >> 5); V^T keeps key k of
// each 16-key group at column ((k >> 2) & 1) * 8 + ((k >> 3) & 1) * 4 + (k & 3),
// so the 8 keys of a lane's P^T operand slots are 16 contiguous bytes of V^T.
// Each wave keeps its 32 queries in registers.  Software pipeline, one
// barrier per tile: during tile j the packed blocks of tile j + 3 are
// loaded, tile j + 1's score MFMAs run among tile j's exponentials, and tile
// j + 2 is dequantized into the third stage among tile j's value MFMAs.
// With key splits, workgroup (split, query block, head) walks its split's
// run of tiles and a merge kernel combines the runs.
#include "device.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kAD = 128;                   // head dim
constexpr int kAQ = 256;                   // queries per workgroup (8 waves)
constexpr int kAK = 64;                    // keys per tile
constexpr int kATile = kAK * kAD * 2;      // bytes of the K tile (and of V^T)
constexpr int kAStage = 2 * kATile;        // K tile, then V^T tile
constexpr int kAVt = 3 * kATile;           // V^T tiles after the three K tiles
constexpr int kALds = 3 * kAStage;         // 96 KB: three stages

// 16-byte slot permutation of V^T row d.  A fragment read (16 lanes: rows
// d0 + c, c = 0..15, one slot each) meets 16 different bank groups, and the
// dequant's 4-byte writes (16 rows 8 apart per 16 lanes) two lanes a bank.
// For row d = 32 db + c it is vt_swz_lo(c) ^ 2 db, so slot 2 kk + h of
// block db is slot 2 (kk ^ db) + h of block 0 moved by db rows of 32: the
// reads of all four blocks share four lane offsets.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) & 7) ^ ((d >> 4) & 7); }
__device__ __forceinline__ int vt_swz_lo(int c) { return ((c >> 1) & 7) ^ (c >> 4); }

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

// One lane's packed blocks of a tile: one K block (16 d of one key) and, of
// V, the 8 d of one half block for a pair of keys.  A key past the
// segment's end reads the segment's last token instead: its score is masked
// to -inf, so its weight is exactly 0 and its (finite) values never count.
struct TileBlocks {
    u32x2 kc;
    uint32_t ks;
    uint32_t vc[2];
    uint32_t vs[2];
};

// Lane t (0..511) of the workgroup: K block of key t >> 3, d block t & 7;
// V keys 2 (t >> 4) and 2 (t >> 4) + 1, d = 8 (t & 15) .. + 8.  Raw buffer
// loads over the segment's arrays: the head's offset is the scalar part,
// token * row bytes (below 2^31, tokens below 2^24) the 24-bit vector part.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seg_rsrc(const void *p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             kBufferWord3);
}

__device__ __forceinline__ void load_blocks(const AttnArgs &a, const AttnSeg &sg, int tok0, int t,
                                            int head, TileBlocks &tb) {
    const uint32_t cs = (uint32_t)(a.HD >> 1), ss = (uint32_t)(a.HD >> 4);
    const int last = (int)sg.n - 1;
    const __amdgpu_buffer_rsrc_t kc = seg_rsrc(sg.kc, sg.n * cs), ks = seg_rsrc(sg.ks, sg.n * ss);
    const __amdgpu_buffer_rsrc_t vc = seg_rsrc(sg.vc, sg.n * cs), vs = seg_rsrc(sg.vs, sg.n * ss);
    {
        const int tk = tok0 + (t >> 3) < last ? tok0 + (t >> 3) : last;
        const int b = t & 7;
        tb.kc = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                              kc, __umul24(tk, cs) + b * 8, head * 64, 0));
        tb.ks = __builtin_amdgcn_raw_buffer_load_b8(ks, __umul24(tk, ss) + b, head * 8, 0);
    }
    const int hb = t & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tv = tok0 + 2 * (t >> 4) + i < last ? tok0 + 2 * (t >> 4) + i : last;
        tb.vc[i] = __builtin_amdgcn_raw_buffer_load_b32(vc, __umul24(tv, cs) + hb * 4, head * 64, 0);
        tb.vs[i] = __builtin_amdgcn_raw_buffer_load_b8(vs, __umul24(tv, ss) + (hb >> 1), head * 8, 0);
    }
}

// Dequantize a lane's blocks into a stage: a K row segment into the K tile
// `kst`, V^T columns into the V^T tile `vst`.
__device__ __forceinline__ void store_blocks(uint8_t *kst, uint8_t *vst, const AttnSeg &sg, int t,
                                             int head, const TileBlocks &tb) {
    {
        const int k = t >> 3, b = t & 7;
        Raw16F32 m;
        buffer_load16(seg_rsrc(sg.mu, (int64_t)head * kAD * 4 + kAD * 4), (uint32_t)(head * kAD + b * 16) * 4, m);
        float mu[16];
        unpack16(m, mu);
        const float S = e4m3_value(tb.ks) * sg.sd[0];
        float y0[8], y1[8];
        dequant8(tb.kc.x, S, y0);
        dequant8(tb.kc.y, S, y1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            y0[e] = y0[e] + mu[e];
            y1[e] = y1[e] + mu[8 + e];
        }
        const u32x4 lo{pack_bf16x2(y0[0], y0[1]), pack_bf16x2(y0[2], y0[3]),
                       pack_bf16x2(y0[4], y0[5]), pack_bf16x2(y0[6], y0[7])};
        const u32x4 hi{pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3]),
                       pack_bf16x2(y1[4], y1[5]), pack_bf16x2(y1[6], y1[7])};
        *(u32x4 *)(kst + k * 256 + (((2 * b) ^ (k & 15)) * 16)) = lo;
        *(u32x4 *)(kst + k * 256 + (((2 * b + 1) ^ (k & 15)) * 16)) = hi;
    }
    {
        const float sdv = sg.sd[1];
        float y[2][8];
#pragma unroll
        for (int i = 0; i < 2; ++i) dequant8(tb.vc[i], e4m3_value(tb.vs[i]) * sdv, y[i]);
        const int col = vt_col(2 * (t >> 4));  // two consecutive columns
        const int slot = col >> 3, off = (col & 7) * 2;
        const int hb = t & 15;
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            const int d = hb * 8 + dd;
            const int phys = slot ^ vt_swz(d);
            *(uint32_t *)(vst + d * 128 + phys * 16 + off) = pack_bf16x2(y[0][dd], y[1][dd]);
        }
    }
}

// max / sum of v over lanes l and l ^ 32 (v_permlane32_swap: the upper half
// of the first operand trades places with the lower half of the second)
__device__ __forceinline__ float half_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// S^T = K_hat Q^T for the K tile of stage `st`: two 32-key blocks,
// alternating so that no MFMA waits for the one before it; fragment reads
// four MFMAs ahead of their use.
__device__ __forceinline__ void scores(const uint8_t *st, const bf16x8 (&qf)[8], int c, int h,
                                       f32x16 (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.0f;
    constexpr int PF = 4;
    bf16x8 kf[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int ks = i >> 1, kb = i & 1;
        kf[i] = *(const bf16x8 *)(st + (kb * 32 + c) * 256 + (((2 * ks + h) ^ (c & 15)) * 16));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int ks = i >> 1, kb = i & 1;
        const bf16x8 cur = kf[i % PF];
        if (i + PF < 16) {
            const int ks2 = (i + PF) >> 1, kb2 = (i + PF) & 1;
            kf[i % PF] = *(const bf16x8 *)(st + (kb2 * 32 + c) * 256 + (((2 * ks2 + h) ^ (c & 15)) * 16));
        }
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[ks], sacc[kb], 0, 0, 0);
    }
}

// One tile of the loop, the stages fixed at compile time (so every LDS
// address is a loop-invariant lane offset plus an immediate): tile j's K
// and V^T tiles in stage CUR, tile j + 1's in NXT, tile j + 2 is written to
// FUT.  sacc holds tile j's scores on entry and tile j + 1's on return.
template <int CUR>
__device__ __forceinline__ void attn_tile(const AttnArgs &a, uint8_t *lds, int j, int je, int t,
                                          int head, int c, int h, bool zero_scale, float scale_log2,
                                          const bf16x8 (&qf)[8], f32x16 (&o)[4], float &m_run,
                                          float &l_run, f32x16 (&sacc)[2], TileBlocks &tb,
                                          int &s_tb, int &sj, int &sj_end, int &s3, int &s3_end) {
    constexpr int NXT = (CUR + 1) % 3, FUT = (CUR + 2) % 3;
    // segment cursors of tile j and of tile j + 3 (both move by at most one
    // tile per tile, and every segment has a tile, so one step suffices)
    if (j >= sj_end) {
        ++sj;
        sj_end = a.tile0[sj + 1];
    }
    const int j3 = j + 3 < je ? j + 3 : je - 1;
    if (j3 >= s3_end) {
        ++s3;
        s3_end = a.tile0[s3 + 1];
    }
    TileBlocks tn;
    load_blocks(a, a.seg[s3], (j3 - a.tile0[s3]) * kAK, t, head, tn);

    if (zero_scale) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.0f;
    }
    // keys past the segment's end
    const int64_t nvalid = a.seg[sj].n - (int64_t)(j - a.tile0[sj]) * kAK;
    if (nvalid < kAK) {
        // key kb*32 + h*4 + (e>>2)*8 + (e&3) against nvalid, the lane's
        // part moved to the right so each compare takes a constant
        const int lim = (int)nvalid - h * 4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (kb * 32 + (e >> 2) * 8 + (e & 3) >= lim) sacc[kb][e] = -__builtin_inff();
    }
    // online softmax against a reference maximum m_run (scale_log2 > 0,
    // so a masked key's -inf stays -inf and its weight is exactly 0).
    // The output and the normaliser are rescaled only when a tile's
    // maximum exceeds the reference by more than 8 (log2 units) in some
    // lane; in between the weights 2^(x - m_run) stay below 2^8, where
    // bf16 and the fp32 sums keep the same relative rounding.
    float mx = sacc[0][0];
#pragma unroll
    for (int e = 1; e < 32; ++e) mx = fmaxf(mx, sacc[e >> 4][e & 15]);
    mx = half_max(mx) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
        l_run *= alpha;
        m_run = m_new;
    }
    // From here to the barrier one basic block: tile j + 1's score MFMAs
    // among the exponentials, the value MFMAs among tile j + 2's
    // dequantization.
    f32x16 snx[2];
    scores(lds + NXT * kATile, qf, c, h, snx);
    float ps = 0.0f;
    const bf16x2 ones2 = __builtin_bit_cast(bf16x2, 0x3F803F80u);
    u32x4 pw[4];  // P^T operands: bf16 pairs
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e], scale_log2, -m_run));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e + 1], scale_log2, -m_run));
            const uint32_t w = pack_bf16x2(p0, p1);
            pw[kb * 2 + (e >> 3)][(e & 7) >> 1] = w;
            ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones2, ps, false);
        }
    l_run += ps;
    // O^T += V_hat^T P^T, the four d blocks in turn (independent MFMAs)
    {
        // fragment reads four MFMAs ahead of their use
        constexpr int PF = 4;
        auto vaddr = [&](int i) {
            const int kk = i >> 2, db = i & 3;
            const int kx = kk ^ db;  // compile-time: the block-0 slot pair
            return (const bf16x8 *)(lds + kAVt + CUR * kATile + db * 4096 + c * 128 +
                                    (((2 * kx + h) ^ vt_swz_lo(c)) * 16));
        };
        bf16x8 vf[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) vf[i] = *vaddr(i);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kk = i >> 2, db = i & 3;
            const bf16x8 cur = vf[i % PF];
            if (i + PF < 16) vf[i % PF] = *vaddr(i + PF);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, __builtin_bit_cast(bf16x8, pw[kk]),
                                                            o[db], 0, 0, 0);
        }
    }
    store_blocks(lds + FUT * kATile, lds + kAVt + FUT * kATile, a.seg[s_tb], t, head, tb);
    tb = tn;
    s_tb = s3;
    sacc[0] = snx[0];
    sacc[1] = snx[1];
    __syncthreads();
}

__global__ __launch_bounds__(512) void attn_window_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // workgroups of one (split, head) run on one XCD (b % 8), sharing its L2
    const int64_t nqt = (a.nq + kAQ - 1) / kAQ;
    const int64_t units = nqt * a.heads;
    const int64_t total = units * a.nsplit;
    const int64_t bid = blockIdx.x;
    const int64_t per = total / 8;
    const int64_t tix = bid < per * 8 ? (bid % 8) * per + bid / 8 : bid;
    const int split = (int)(tix / units);
    const int head = (int)(tix % units / nqt);
    const int64_t q0 = (tix % nqt) * kAQ;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 31, h = lane >> 5;
    const int t = threadIdx.x;

    // Q^T operand in registers: lane (c, h) holds query qw + c (clamped),
    // d = 16 ks + 8 h .. + 8
    const int64_t qw = q0 + wave * 32;
    const int64_t qi = qw + c;
    bf16x8 qf[8];
    {
        const uint16_t *qp = a.q + (qi < a.nq ? qi : a.nq - 1) * a.HD + head * kAD + h * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8 *)(qp + ks * 16);
    }

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = 0.0f;
    float m_run = -__builtin_inff(), l_run = 0.0f;

    // The split's tiles [jb, je), three LDS stages: during iteration j the
    // value MFMAs read tile j's stage, the score MFMAs of tile j + 1 (issued
    // among tile j's exponentials) read the next, and tile j + 2's blocks,
    // loaded one iteration earlier, are dequantized into the third among
    // the value MFMAs; tile j + 3's are requested at the top.  Past the last
    // tile the loads repeat it and the extra stage writes and scores are
    // never used, so a tile has no branch around them.  The loop is unrolled
    // by the three stages (attn_tile<0..2>), tile jb in stage 0.
    const int ntile = a.tile0[a.nseg];
    const int jb = (int)((int64_t)split * ntile / a.nsplit);
    const int je = (int)((int64_t)(split + 1) * ntile / a.nsplit);
    TileBlocks tb;
    int s_tb = 0;
    int sj = seg_of(a, jb);
    int sj_end = a.tile0[sj + 1];
    if (je > jb) {
        int s0 = seg_of(a, jb);
        load_blocks(a, a.seg[s0], (jb - a.tile0[s0]) * kAK, t, head, tb);
        store_blocks(lds, lds + kAVt, a.seg[s0], t, head, tb);
        const int j1 = jb + 1 < je ? jb + 1 : jb;
        s0 = seg_of(a, j1);
        load_blocks(a, a.seg[s0], (j1 - a.tile0[s0]) * kAK, t, head, tb);
        store_blocks(lds + kATile, lds + kAVt + kATile, a.seg[s0], t, head, tb);
        const int j2 = jb + 2 < je ? jb + 2 : je - 1;
        s_tb = seg_of(a, j2);
        load_blocks(a, a.seg[s_tb], (j2 - a.tile0[s_tb]) * kAK, t, head, tb);
    }
    __syncthreads();
    f32x16 sacc[2];
    scores(lds, qf, c, h, sacc);
    // A zero scale (every weight 1: the mean of the values) runs as scores
    // of 0 at scale 1, so that a masked key's -inf is never multiplied by 0.
    const bool zero_scale = a.scale_log2 == 0.0f;
    const float scale_log2 = zero_scale ? 1.0f : a.scale_log2;
    int s3 = s_tb;  // segment of tile min(jb + 2, je - 1)
    int s3_end = a.tile0[s3 + 1];

    for (int j = jb; j < je; j += 3) {
        attn_tile<0>(a, lds, j, je, t, head, c, h, zero_scale, scale_log2, qf, o, m_run, l_run, sacc, tb, s_tb, sj, sj_end, s3, s3_end);
        if (j + 1 >= je) break;
        attn_tile<1>(a, lds, j + 1, je, t, head, c, h, zero_scale, scale_log2, qf, o, m_run, l_run, sacc, tb, s_tb, sj, sj_end, s3, s3_end);
        if (j + 2 >= je) break;
        attn_tile<2>(a, lds, j + 2, je, t, head, c, h, zero_scale, scale_log2, qf, o, m_run, l_run, sacc, tb, s_tb, sj, sj_end, s3, s3_end);
    }

    // both lane halves saw every score maximum, so m_run agrees; the sums add
    const float lt = half_sum(l_run);
    if (a.nsplit > 1) {
        // the split's share: output and sum of weights, both relative to the
        // reference maximum m_run, and m_run itself
        if (qi < a.nq) {
            const int64_t r = ((int64_t)split * a.nq + qi) * a.heads + head;
            float *po = a.part_o + r * kAD;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *(f32x4 *)(po + db * 32 + h * 4 + g * 8) =
                        f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
            if (h == 0) *(f32x2 *)(a.part_ml + 2 * r) = f32x2{m_run, lt};
        }
        return;
    }
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

// Merge of the key splits: thread (query, head, 8 d).  With M the largest
// of the splits' reference maxima and w_s = 2^(m_s - M), o = sum_s w_s o_s / sum_s w_s l_s and
// lse = (M + log2 sum_s w_s l_s) ln 2, splits in index order; a split
// without keys has m = -inf and l = 0, and no keys at all give o = 0 and
// lse = -inf as in the single-split kernel.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
    const int64_t nqh = a.nq * a.heads;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nqh * 16) return;
    const int64_t r = i >> 4;
    const int g = (int)(i & 15);
    float M = -__builtin_inff();
    for (int sp = 0; sp < a.nsplit; ++sp) M = fmaxf(M, a.part_ml[2 * (sp * nqh + r)]);
    float L = 0.0f;
    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
    if (M != -__builtin_inff()) {
        for (int sp = 0; sp < a.nsplit; ++sp) {
            const f32x2 ml = *(const f32x2 *)(a.part_ml + 2 * (sp * nqh + r));
            const float w = __builtin_amdgcn_exp2f(ml.x - M);
            const float *po = a.part_o + (sp * nqh + r) * kAD + g * 8;
            L = __builtin_fmaf(w, ml.y, L);
            acc0 = w * *(const f32x4 *)po + acc0;
            acc1 = w * *(const f32x4 *)(po + 4) + acc1;
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    *(u32x4 *)(a.o + r * kAD + g * 8) =
        u32x4{pack_bf16x2(acc0.x * inv, acc0.y * inv), pack_bf16x2(acc0.z * inv, acc0.w * inv),
              pack_bf16x2(acc1.x * inv, acc1.y * inv), pack_bf16x2(acc1.z * inv, acc1.w * inv)};
    if (a.lse && g == 0)
        a.lse[r] = L > 0.0f ? (M + log2f(L)) * 0.69314718055994531f : -__builtin_inff();
}

size_t attn_workspace_bytes(int64_t nq, int heads, int nsplit) {
    if (nsplit <= 1) return 0;
    const size_t rows = (size_t)nsplit * (size_t)nq * (size_t)heads;
    return (rows * 8 + 255) / 256 * 256 + rows * kAD * 4;
}

// Compute units of each device, read once.
static int device_cus(int dev, hipError_t &e) {
    static std::atomic<int> cache[64];
    e = hipSuccess;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0) return 0;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// One 8-wave workgroup fills a compute unit (two waves a SIMD at the
// kernel's register count), so a launch runs in rounds of `cus` workgroups.
// A split count s costs ceil(units * s / cus) rounds of 1/s of a unit's
// time, times 1 + 0.015 s for what each split adds (its pipeline fill and
// partial output, the merge; measured ~1.5% a split on 7040 queries x 24
// heads over 33,440 keys).  The cheapest s is taken if it saves 3% over one
// split, each split keeping at least 8 tiles.
hipError_t attn_choose_splits(int64_t nq, int heads, int ntile, int requested, int *nsplit) {
    if (requested > 0) {
        *nsplit = requested;
        return hipSuccess;
    }
    *nsplit = 1;
    const int64_t units = (nq + kAQ - 1) / kAQ * heads;
    if (units == 0 || ntile < 16) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int cus = device_cus(dev, e);
    if (e != hipSuccess) return e;
    if (cus <= 0) return hipSuccess;
    auto cost = [&](int sp) {
        return (double)((units * sp + cus - 1) / cus) / sp * (1.0 + 0.015 * sp);
    };
    int best = 1;
    for (int sp = 2; sp <= kAttnMaxSplit && ntile >= 8 * sp; ++sp)
        if (cost(sp) < cost(best)) best = sp;
    if (cost(best) <= 0.97 * cost(1)) *nsplit = best;
    return hipSuccess;
}

hipError_t launch_attn_window(const AttnArgs &a, hipStream_t s) {
    if (a.nq == 0) return hipSuccess;
    static std::atomic<uint32_t> lds_set{0};
    const void *fn = (const void *)attn_window_kernel;
    hipError_t e = lds_limit_once(&fn, 1, kALds, lds_set);
    if (e != hipSuccess) return e;
    const int64_t grid = ((a.nq + kAQ - 1) / kAQ) * a.heads * a.nsplit;
    NVFP4_LAUNCH("attn_window", attn_window_kernel, dim3((unsigned)grid), dim3(512), kALds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.nsplit <= 1) return e;
    const int64_t mgrid = (a.nq * a.heads * 16 + 255) / 256;
    NVFP4_LAUNCH("attn_merge", attn_merge_kernel, dim3((unsigned)mgrid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace nvfp4
