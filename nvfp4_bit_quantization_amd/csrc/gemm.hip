// gemm.hip -- W4A4 GEMM on NVFP4 operands for gfx950 (MFMA).
//
// Method (LongLive-2.0 pages): "MCISLAB DeepRead: LongLive2" summary, Method /
// inference infrastructure: the generator runs W4A4, FP4 GEMMs replacing the
// BF16 GEMMs; weights use 2-D block scaling, activations 1-D, with a
// tensor-wise FP32 scale on each ("NVFP4 training").
//
// gfx950 has no MFMA that takes an E4M3 scale per 16 elements (its scaled
// FP4 MFMA takes power-of-two E8M0 scales per 32), so each NVFP4 operand is
// expanded exactly and fed to the fp16 MFMA (same dense rate as bf16):
//   A_hat = V(code) * sigma,  sigma the E4M3 block scale.
//   v_cvt_scalef32_pk_f16_fp4 gives V exactly, one packed fp16 multiply by
//   sigma gives V * sigma exactly (at most 6 significant bits, magnitude in
//   [2^-10, 2688]: exact in fp16).
// The FP32 tensor scales are applied once in the epilogue:
//   Y = RN(RN(s_A * s_W) * acc), acc the fp32 MFMA accumulation.
// With QUANT the epilogue encodes bf16(Y) straight to NVFP4 (1-D blocks
// along N, the Four-Over-Six encoder of the quantizer) for a tensor amax the
// caller gives, so the next W4A4 GEMM reads it without a bf16 round trip
// through memory.
//
// Operand layout in the MFMA: the 32x32x16 MFMA pairs lane l's 8 K values
// of row (l & 31) with the same 8 K positions of the other operand, and the
// contraction does not care which K positions those are, so lane half
// h = l >> 5 takes the contiguous K range [128 h, 128 h + 128) of each
// 256-deep K step (16 consecutive code dwords = 64 bytes, and the 8 scale
// bytes of those blocks); MFMA substep s uses dword s of both halves.  The
// same assignment on both operands keeps the product exact.
//
// Tiling: workgroup 4 waves (2 x 2), tile BM x BN = 256 x 192; each wave owns
// 128 x 96 = 4 x 3 blocks of v_mfma_f32_32x32x16_f16 (192 fp32 accumulators
// per lane).  Where it shortens the last round, the last rows go in 192 x 192
// tiles (96 x 96 = 3 x 3 blocks a wave) in the same launch (TileSplit).
// Workgroups are mapped to tiles XCD by XCD: XCD x takes the x-th contiguous
// (row-major) range of tiles, so tiles that share operand rows share an L2.
//
// Data flow (K % 256 == 0): the packed tiles of a K step (codes 128 bytes
// per row, scales 16 bytes per row or 16-row group) go from memory straight
// to LDS (global_load_lds, 16 bytes per lane, 8 lanes per 128-byte row, so
// every load instruction covers 8 whole cache lines), two LDS stages.  The
// 16-byte columns of each row are XOR-swizzled by the row (column c of tile
// row r sits in slot c ^ ((r >> 1) & 7)): a fragment read takes one column
// of 16 consecutive rows per 16 lanes, and those 16 slots -- two rows of
// 128 bytes per 256 bytes of LDS -- land in 16 different groups of the 64
// banks, so the reads run without bank conflicts.  Per K step: barrier; each wave
// reads its whole step of fragments from LDS into registers; the loads of
// the next step are issued into the other stage; the 16 MFMA substeps run
// from registers, expanding each fragment dword just before its MFMAs.
// Other K: the same MFMA schedule from per-lane loads straight from memory,
// with blocks past K read as zero.
#include <atomic>
#include <utility>

#include "device.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int FM = 4, FN = 3;               // MFMA blocks per wave
constexpr int WM = 32 * FM, WN = 32 * FN;   // 128 x 96 per wave
constexpr int BM = 2 * WM, BN = 2 * WN;     // 256 x 192 per workgroup
constexpr int BK = 256;                     // K per step
constexpr int NSUB = BK / 16;               // MFMA substeps per step
constexpr int kXcds = 8;

// LDS stage layout (bytes): A codes (BM / 8 blocks of 8 rows x 128 bytes),
// W codes, A scales (16 bytes per row), W scales (16 bytes per row for 1-D
// W, per 16-row group for 2-D W).
constexpr int kAOff = 0;
constexpr int kBOff = kAOff + BM * 128;
constexpr int kASOff = kBOff + BN * 128;
constexpr int kBSOff = kASOff + BM * 16;
constexpr int kStage = kBSOff + BN * 16;  // 64512 bytes
constexpr int kLdsBytes = 2 * kStage;
static_assert(kStage % 256 == 0, "stage alignment");


typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void *lvoid;  // LDS

struct GemmArgs {
    const uint8_t *a_codes, *a_scales, *w_codes, *w_scales;
    int64_t M, N, K;
};

// One lane's share of one operand fragment (32 rows x 256 K) for one K
// step: 16 code dwords (4 chunks of 16 bytes) and 8 scale bytes.
struct Frag {
    u32x4 q[4];
    u32x2 sc;
};

// Eight fp16 values V * sigma from one code dword (8 codes, element 2j in
// the low nibble of byte j).
__device__ __forceinline__ f16x8 expand8(uint32_t w, f16x2 sig) {
    f16x8 o;
    f16x2 t;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sig; o[0] = t.x; o[1] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sig; o[2] = t.x; o[3] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sig; o[4] = t.x; o[5] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sig; o[6] = t.x; o[7] = t.y;
    return o;
}

// Block scales (E4M3) of blocks 2p and 2p + 1 of a fragment's step, as fp16
// (exact: every E4M3 value is an fp16 value).
template <int P>
__device__ __forceinline__ f16x2 sigma_pair(const u32x2 &sc) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(P < 2 ? sc.x : sc.y, 1.0f, (P & 1) != 0);
}

__device__ __forceinline__ uint32_t dword_of(const u32x4 &q, int i) {
    return i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
}

// Row pointers of one lane's fragment (row clamped into range: rows past
// the end compute values that are never stored).
struct FragPtr {
    const uint8_t *c;  // codes of the row, + 64 h bytes
    const uint8_t *s;  // scales of the row (2-D: of its 16-row group), + 8 h
};

__device__ __forceinline__ FragPtr frag_ptr(const uint8_t *codes, const uint8_t *scales,
                                            int64_t row, int64_t rows, int64_t K, bool two_d,
                                            int h) {
    const int64_t r = row < rows ? row : rows - 1;
    const int64_t KB = K >> 4;
    FragPtr p;
    p.c = codes + r * (K >> 1) + h * 64;
    p.s = scales + (two_d ? (r >> 4) : r) * KB + h * 8;
    return p;
}

// General path (any K % 16 == 0): blocks at or past K / 16 read as code 0
// and scale 0 (+0 whatever the other operand); loads are 8-byte (codes) and
// 1-byte (scales) and stay inside the row.
__device__ __forceinline__ void load_frag_general(Frag &f, const FragPtr &p, int64_t kt,
                                                  int64_t K, int h) {
    const int64_t KB = K >> 4;
    const int64_t kb0 = kt * (BK / 16) + h * 8;  // first block of this lane's half
    const uint8_t *crow = p.c - h * 64, *srow = p.s - h * 8;
    uint32_t d[16], sb[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const bool ok = kb0 + b < KB;
        const int64_t kb = ok ? kb0 + b : 0;
        const uint2 v = *(const uint2 *)(crow + kb * 8);
        d[2 * b] = ok ? v.x : 0u;
        d[2 * b + 1] = ok ? v.y : 0u;
        sb[b] = ok ? (uint32_t)srow[kb] : 0u;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) f.q[c] = u32x4{d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]};
    f.sc = u32x2{sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24),
                 sb[4] | (sb[5] << 8) | (sb[6] << 16) | (sb[7] << 24)};
}

// MFMA substep s (K positions 8 s .. 8 s + 7 of each lane half) over the
// wave's 4 x 3 blocks: block s / 2 of the half, scale byte s / 2.
template <int S, int FMT>
__device__ __forceinline__ void substep(f32x16 (&acc)[FMT][FN], const Frag (&A)[FMT],
                                        const Frag (&B)[FN]) {
    constexpr int c = S >> 2, i4 = S & 3, hi = (S >> 1) & 1;
    f16x8 a[FMT], b[FN];
#pragma unroll
    for (int i = 0; i < FMT; ++i) {
        const f16x2 sg = sigma_pair<c>(A[i].sc);
        const _Float16 g = hi ? sg.y : sg.x;
        a[i] = expand8(dword_of(A[i].q[c], i4), f16x2{g, g});
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const f16x2 sg = sigma_pair<c>(B[j].sc);
        const _Float16 g = hi ? sg.y : sg.x;
        b[j] = expand8(dword_of(B[j].q[c], i4), f16x2{g, g});
    }
#pragma unroll
    for (int i = 0; i < FMT; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// Buffer descriptors over the four packed arrays and this lane's byte
// offsets into them for its share of every step's direct-to-LDS loads:
// A code blocks 8w .. 8w + 7 and W code blocks 6w .. 6w + 5 of the tile
// (8 rows each; lane j loads 16-byte column (j & 7) ^ ((R >> 1) & 7) of
// tile row R = 8 * block + (j >> 3) into slot j), the A scales of tile rows 64w + j, and (wave 0, lanes
// below 12) the W scales of the tile's 16-row groups.  Rows past the matrix
// edge are clamped to the last row.  The step's offset is a scalar added at
// each load.  (The host sends matrices of 2^31 bytes or more to the general
// path, so every offset fits.)
struct StageSrc {
    __amdgpu_buffer_rsrc_t ac, wc, as, ws;
    uint32_t a[BM / 32], w[BN / 32], asr, wsr;
};

template <bool SCALES, bool W2D, int FMT = FM>
__device__ __forceinline__ void stage_src(StageSrc &q, const GemmArgs &g, int64_t m0, int64_t n0,
                                          int wave, int lane) {
    constexpr int BMT = 64 * FMT;  // tile rows
    const int64_t kbytes = g.K >> 1, KB = g.K >> 4;
    q.ac = __builtin_amdgcn_make_buffer_rsrc((void *)g.a_codes, (short)0, (int)(g.M * kbytes),
                                             kBufferWord3);
    q.wc = __builtin_amdgcn_make_buffer_rsrc((void *)g.w_codes, (short)0, (int)(g.N * kbytes),
                                             kBufferWord3);
    if (SCALES) {
        q.as = __builtin_amdgcn_make_buffer_rsrc((void *)g.a_scales, (short)0, (int)(g.M * KB),
                                                 kBufferWord3);
        q.ws = __builtin_amdgcn_make_buffer_rsrc((void *)g.w_scales, (short)0,
                                                 (int)((W2D ? g.N >> 4 : g.N) * KB),
                                                 kBufferWord3);
    }
    // block parity gives bit 2 of the swizzle key (8 rows per block; both
    // per-wave block counts are even)
    static_assert((BMT / 32) % 2 == 0 && (BN / 32) % 2 == 0, "block parity");
    const int rib = lane >> 3;
#pragma unroll
    for (int bb = 0; bb < BMT / 32; ++bb) {
        const int64_t row0 = m0 + (wave * (BMT / 32) + bb) * 8 + rib;
        const int64_t row = row0 < g.M ? row0 : g.M - 1;
        const int gcol = (lane & 7) ^ ((bb & 1) << 2 | rib >> 1);
        q.a[bb] = (uint32_t)(row * kbytes) + gcol * 16;
    }
#pragma unroll
    for (int bb = 0; bb < BN / 32; ++bb) {
        const int64_t row0 = n0 + (wave * (BN / 32) + bb) * 8 + rib;
        const int64_t row = row0 < g.N ? row0 : g.N - 1;
        const int gcol = (lane & 7) ^ ((bb & 1) << 2 | rib >> 1);
        q.w[bb] = (uint32_t)(row * kbytes) + gcol * 16;
    }
    const int64_t ar0 = m0 + wave * 64 + lane;
    q.asr = (uint32_t)((ar0 < g.M ? ar0 : g.M - 1) * KB);
    if (W2D) {
        const int64_t gr0 = (n0 >> 4) + lane, glast = (g.N >> 4) - 1;
        q.wsr = (uint32_t)((gr0 < glast ? gr0 : glast) * KB);
    } else {
        const int64_t wr0 = n0 + (wave < BN / 64 ? wave : 0) * 64 + lane;
        q.wsr = (uint32_t)((wr0 < g.N ? wr0 : g.N - 1) * KB);
    }
}

// Issue this wave's direct-to-LDS loads of K step kt into `stage` (codes,
// and with SCALES the NVFP4 block scales).
template <bool SCALES, bool W2D, int FMT = FM>
__device__ __forceinline__ void stage_load(const StageSrc &q, uint8_t *stage, int64_t kt, int wave,
                                           int lane) {
    constexpr int BMT = 64 * FMT;
    const uint32_t kc = (uint32_t)kt * 128, ks = (uint32_t)kt * 16;
#pragma unroll
    for (int bb = 0; bb < BMT / 32; ++bb)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            q.ac, (lvoid)(stage + kAOff + (wave * (BMT / 32) + bb) * 1024), 16, q.a[bb], kc, 0, 0);
#pragma unroll
    for (int bb = 0; bb < BN / 32; ++bb)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            q.wc, (lvoid)(stage + kBOff + (wave * (BN / 32) + bb) * 1024), 16, q.w[bb], kc, 0, 0);
    if (!SCALES) return;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(q.as, (lvoid)(stage + kASOff + wave * 1024), 16,
                                             q.asr, ks, 0, 0);
    if (W2D) {
        if (wave == 0 && lane < BN / 16)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(q.ws, (lvoid)(stage + kBSOff), 16, q.wsr, ks,
                                                     0, 0);
    } else if (wave < BN / 64) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(q.ws, (lvoid)(stage + kBSOff + wave * 1024), 16,
                                                 q.wsr, ks, 0, 0);
    }
}

// The wave's fragments of one K step from LDS: lane (r, h) reads, for each
// fragment row R, the 16-byte columns 4h .. 4h + 3 (un-swizzled) and the 8
// scale bytes of its half.  Fragments start on multiples of 32 tile rows, so
// the swizzle key of row R is (r >> 1) & 7.
template <bool SCALES, bool W2D, int FMT = FM>
__device__ __forceinline__ void stage_read(Frag (&A)[FMT], Frag (&B)[FN], const uint8_t *stage,
                                           int wm, int wn, int r, int h) {
    constexpr int WMT = 32 * FMT;
    const int rib = r & 7, key = (r >> 1) & 7;
    if (SCALES) {
#pragma unroll
        for (int i = 0; i < FMT; ++i)
            A[i].sc = *(const u32x2 *)(stage + kASOff + (wm * WMT + i * 32 + r) * 16 + h * 8);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int R = wn * WN + j * 32 + r;
            B[j].sc = *(const u32x2 *)(stage + kBSOff + (W2D ? R >> 4 : R) * 16 + h * 8);
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int slot = ((h * 4 + c) ^ key) * 16 + rib * 128;
#pragma unroll
        for (int i = 0; i < FMT; ++i)
            A[i].q[c] = *(const u32x4 *)(stage + kAOff + ((wm * WMT + i * 32 + r) >> 3) * 1024 + slot);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            B[j].q[c] = *(const u32x4 *)(stage + kBOff + ((wn * WN + j * 32 + r) >> 3) * 1024 + slot);
    }
}

template <int FMT, int... S>
__device__ __forceinline__ void step_all(f32x16 (&acc)[FMT][FN], const Frag (&A)[FMT],
                                         const Frag (&B)[FN], std::integer_sequence<int, S...>) {
    (substep<S, FMT>(acc, A, B), ...);
}

// LoRA epilogue operands (LORA = true): XA [M, r] and B [N, r] bf16, the
// branch (lora_scale) * XA B^T added to every output.
struct LoraArgs {
    const uint16_t *xa;
    const uint16_t *b;
    int64_t r;
    float scale;
};

// Per-wave LDS of the bf16 and fused-encode epilogues: the wave's 128 x 96
// tile of bf16(Y) (row-major, 192 bytes a row), then (fused encode) the
// (S, 1/S) table of the 128 non-negative scale codes for the tensor's s_dec.
constexpr int kQRowBytes = WN * 2;
constexpr int kQTileBytes = WM * kQRowBytes;           // 24576
constexpr int kQLutOff = kQTileBytes;
constexpr int kQWaveBytes = kQTileBytes + 128 * 8;     // 25600
static_assert(4 * kQWaveBytes <= kLdsBytes, "fused-encode LDS");

// Rows [0, m1) are covered by 256-row tiles (the first t1 workgroups), rows
// [m1, M) by 192-row tiles (the rest of the grid): when the 256-row tiles
// would leave the chip's last round part-empty (7040 x 3072: 448 tiles, 1.72
// rounds on 256 CUs), a first round of 256-row tiles and a second of 256
// 192-row tiles take 1.75 tile times instead of 2.  The host chooses m1.
struct TileSplit {
    int64_t t1;  // workgroups of 256-row tiles
    int64_t m1;  // rows they cover: a multiple of 256, or M
};

// XCD-aware tile order: workgroup b runs on XCD b % 8; XCD x takes the x-th
// contiguous range of the `count` tiles (tiles past 8 * floor(count / 8) map
// to themselves).
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t count) {
    const int64_t per = count / kXcds;
    return b < per * kXcds ? (b % kXcds) * per + b / kXcds : b;
}

// One tile at (m0, n0) of FMT * 64 rows x 192 columns: 4 waves (2 x 2) of
// FMT x 3 MFMA blocks each.
template <bool OUT_BF16, bool KFAST, bool W2D, bool LORA, bool QUANT, int FMT>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, int64_t m0, int64_t n0,
                                          const float *__restrict__ a_sdec,
                                          const float *__restrict__ w_sdec, void *__restrict__ yv,
                                          float *__restrict__ amax_out, const LoraArgs &la,
                                          const QuantOut &qo, uint8_t *lds) {
    constexpr int WMT = 32 * FMT;
    const int64_t M = g.M, N = g.N, K = g.K;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, r = lane & 31, wm = wave >> 1, wn = wave & 1;
    const int64_t mw = m0 + wm * WMT, nw = n0 + wn * WN;
    // a wave whose sub-tile lies wholly past the matrix edge computes nothing
    // (it still takes its share of the loads and every barrier)
    const bool active = mw < M && nw < N;

    f32x16 acc[FMT][FN];
#pragma unroll
    for (int i = 0; i < FMT; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int64_t nk = (K + BK - 1) / BK;
    Frag A[FMT], B[FN];
    if (KFAST) {
        StageSrc src;
        stage_src<true, W2D, FMT>(src, g, m0, n0, wave, lane);
        stage_load<true, W2D, FMT>(src, lds, 0, wave, lane);
        // Each iteration: this wave's loads of step kt have landed; after the
        // barrier so have everyone's, and nobody still reads the stage that
        // the loads of step kt + 1 overwrite.  The last iteration reloads its
        // own step into the idle stage (never read), keeping the loop free of
        // branches.  Both loops take the same barriers.
        if (active) {
            for (int64_t kt = 0; kt < nk; ++kt) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                const int64_t kn = kt + 1 < nk ? kt + 1 : kt;
                stage_read<true, W2D, FMT>(A, B, lds + (kt & 1) * kStage, wm, wn, r, h);
                stage_load<true, W2D, FMT>(src, lds + ((kt + 1) & 1) * kStage, kn, wave, lane);
                step_all(acc, A, B, std::make_integer_sequence<int, NSUB>{});
            }
        } else {
            for (int64_t kt = 0; kt < nk; ++kt) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                const int64_t kn = kt + 1 < nk ? kt + 1 : kt;
                stage_load<true, W2D, FMT>(src, lds + ((kt + 1) & 1) * kStage, kn, wave, lane);
            }
        }
        // no load into LDS is still in flight when the wave leaves
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // the fused encode and the bf16 epilogue reuse the stages: every wave
        // is past its last read
        if (QUANT || OUT_BF16) __syncthreads();
    } else if (active) {
        FragPtr pa[FMT], pb[FN];
#pragma unroll
        for (int i = 0; i < FMT; ++i)
            pa[i] = frag_ptr(g.a_codes, g.a_scales, mw + i * 32 + r, M, K, false, h);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            pb[j] = frag_ptr(g.w_codes, g.w_scales, nw + j * 32 + r, N, K, W2D, h);
        for (int64_t kt = 0; kt < nk; ++kt) {
#pragma unroll
            for (int i = 0; i < FMT; ++i) load_frag_general(A[i], pa[i], kt, K, h);
#pragma unroll
            for (int j = 0; j < FN; ++j) load_frag_general(B[j], pb[j], kt, K, h);
            step_all(acc, A, B, std::make_integer_sequence<int, NSUB>{});
        }
    }
    if (!active) return;

    const float scale = (*a_sdec) * (*w_sdec);
    float amax = 0.0f;  // max |stored y| of this lane
    uint8_t *const qw = lds + wave * kQWaveBytes;  // QUANT: this wave's tile and table
    // LoRA: (XA rows of block i) x (B rows of block j)^T on the bf16 MFMA, 16
    // of r per step, for two row blocks x three column blocks at a time; each
    // step loads those 2 + 3 fragments at once (rows past the edge are
    // clamped, never stored)
    constexpr int FH = FMT % 2 == 0 ? FMT / 2 : 1;  // row blocks per LoRA pass
#pragma unroll
    for (int ih = 0; ih < FMT / FH; ++ih) {
        f32x16 lo[FH][FN];
        if (LORA) {
            const uint16_t *xp[FH], *bp[FN];
#pragma unroll
            for (int i = 0; i < FH; ++i) {
                const int64_t row = mw + (ih * FH + i) * 32 + r;
                xp[i] = la.xa + (row < M ? row : M - 1) * la.r + h * 8;
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) lo[i][j][e] = 0.0f;
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t col = nw + j * 32 + r;
                bp[j] = la.b + (col < N ? col : N - 1) * la.r + h * 8;
            }
            for (int64_t q = 0; q < la.r; q += 16) {
                bf16x8 xf[FH], bfr[FN];
#pragma unroll
                for (int i = 0; i < FH; ++i) xf[i] = *(const bf16x8 *)(xp[i] + q);
#pragma unroll
                for (int j = 0; j < FN; ++j) bfr[j] = *(const bf16x8 *)(bp[j] + q);
#pragma unroll
                for (int i = 0; i < FH; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        lo[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[i], bfr[j],
                                                                           lo[i][j], 0, 0, 0);
            }
        }
#pragma unroll
        for (int ii = 0; ii < FH; ++ii)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int i = ih * FH + ii;
                const int64_t col = nw + j * 32 + r;
                const int64_t rbase = mw + i * 32 + h * 4;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = rbase + (e >> 2) * 8 + (e & 3);
                    float v = scale * acc[i][j][e];
                    if (LORA) v = __builtin_fmaf(la.scale, lo[ii][j][e], v);
                    if (QUANT || (OUT_BF16 && KFAST)) {
                        const __bf16 b = (__bf16)v;
                        if (row < M && col < N) amax = fmaxf(amax, fabsf((float)b));
                        const int rl = i * 32 + h * 4 + (e >> 2) * 8 + (e & 3);
                        *(__bf16 *)(qw + rl * kQRowBytes + (j * 32 + r) * 2) = b;
                    } else if (row < M && col < N) {
                        if (OUT_BF16) {
                            const __bf16 b = (__bf16)v;
                            ((__bf16 *)yv)[row * N + col] = b;
                            amax = fmaxf(amax, fabsf((float)b));
                        } else {
                            ((float *)yv)[row * N + col] = v;
                            amax = fmaxf(amax, fabsf(v));
                        }
                    }
                }
            }
    }
    if (!QUANT && OUT_BF16 && KFAST) {
        // bf16 Y: the wave's tile went to its LDS region (row-major, 192 bytes
        // a row, so 16-byte piece c of the tile sits at byte 16 c); back in
        // 16-byte row pieces, one 16-byte store each (lane-strided 2-byte
        // stores straight from the accumulators took 141 against 131 us on
        // 7040 x 3072 x 3072).  Only this wave touches its region.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        constexpr int kPieces = WN / 8;  // 12 a row
#pragma unroll 4
        for (int k = 0; k < WMT * kPieces / 64; ++k) {
            const int c = lane + 64 * k, rl = c / kPieces, cc = c - rl * kPieces;
            const int64_t row = mw + rl, col = nw + cc * 8;
            const u32x4 v = *(const u32x4 *)(qw + c * 16);
            if (row < M && col < N) *(u32x4 *)((__bf16 *)yv + row * N + col) = v;
        }
    }
    if (QUANT) {
        // 1x16 blocks of the wave's tile, 12 per lane: bf16 values back from
        // LDS, the quantizer's Four-Over-Six encode (same table, same
        // operation order), codes and scale byte to Y.  Only this wave
        // touches its region; the wait (also a compiler barrier) puts every
        // table and tile write before the reads of other lanes' values.
        float s_enc, s_dec;
        tensor_scales(*qo.amax_in, s_enc, s_dec);
        f32x2 *const lut = (f32x2 *)(qw + kQLutOff);
        lut[lane] = scale_entry(lane, s_dec);
        lut[lane + 64] = scale_entry(lane + 64, s_dec);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        constexpr int kBlkRow = WN / 16;  // 6 blocks a row
#pragma unroll 2
        for (int k = 0; k < WMT * kBlkRow / 64; ++k) {
            const int blk = lane + 64 * k;
            const int rl = blk / kBlkRow, cb = blk - rl * kBlkRow;
            const int64_t row = mw + rl, col = nw + cb * 16;
            Raw16Bf16 raw;
            raw.a = *(const u32x4 *)(qw + rl * kQRowBytes + cb * 32);
            raw.b = *(const u32x4 *)(qw + rl * kQRowBytes + cb * 32 + 16);
            float x[16];
            unpack16(raw, x);
            uint32_t q_lo, q_hi, sc;
            if (qo.four_over_six)
                encode_block16<true>(x, s_enc, lut, q_lo, q_hi, sc);
            else
                encode_block16<false>(x, s_enc, lut, q_lo, q_hi, sc);
            if (row < M && col < N) {
                *(u32x2 *)(qo.codes + row * (N >> 1) + (col >> 1)) = u32x2{q_lo, q_hi};
                qo.scales[row * (N >> 4) + (col >> 4)] = (uint8_t)sc;
            }
        }
    }
    if (amax_out) {
        amax = wave_max(amax);
        if (lane == 0) atomicMax((unsigned int *)amax_out, __float_as_uint(amax));
    }
}


template <bool OUT_BF16, bool KFAST, bool W2D, bool LORA, bool QUANT>
__global__ __launch_bounds__(256) void gemm_w4a4_kernel(GemmArgs g, TileSplit ts,
                                                        const float *__restrict__ a_sdec,
                                                        const float *__restrict__ w_sdec,
                                                        void *__restrict__ yv,
                                                        float *__restrict__ amax_out, LoraArgs la,
                                                        QuantOut qo) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    if (QUANT && blockIdx.x == 0 && threadIdx.x == 0) {
        float s_enc, s_dec;
        tensor_scales(*qo.amax_in, s_enc, s_dec);
        *qo.s_dec = s_dec;
    }
    const int64_t tn = (g.N + BN - 1) / BN;
    const int64_t b = blockIdx.x;
    if (b < ts.t1) {
        const int64_t t = xcd_tile(b, ts.t1);
        gemm_tile<OUT_BF16, KFAST, W2D, LORA, QUANT, FM>(g, (t / tn) * BM, (t % tn) * BN, a_sdec,
                                                         w_sdec, yv, amax_out, la, qo, lds);
    } else {
        const int64_t t = xcd_tile(b - ts.t1, (int64_t)gridDim.x - ts.t1);
        gemm_tile<OUT_BF16, KFAST, W2D, LORA, QUANT, 3>(g, ts.m1 + (t / tn) * (64 * 3),
                                                        (t % tn) * BN, a_sdec, w_sdec, yv,
                                                        amax_out, la, qo, lds);
    }
}

// Raise the dynamic-LDS limit of `fns` to `bytes` once per device: `done`
// holds one bit per device id (0..31) already set up.  Threads that race
// both set the attribute, which is harmless.
hipError_t lds_limit_once(const void *const *fns, int n, int bytes,
                                 std::atomic<uint32_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint32_t bit = (dev >= 0 && dev < 32) ? (1u << dev) : 0u;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    for (int i = 0; i < n; ++i) {
        e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess) return e;
    }
    done.fetch_or(bit, std::memory_order_release);
    return hipSuccess;
}

// Compute units of the current device (0 if unknown), cached per device.
static int device_cus() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            c = -1;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c > 0 ? c : 0;
}

// Finish time, in quarters of a 256-row tile, of n1 256-row tiles then n2
// 192-row tiles (3 quarters each) handed to `cus` CUs in workgroup order,
// each to the CU that frees first.  After the first kind every CU is busy
// until a = 4 floor(n1 / cus), or a + 4 for the n1 mod cus that took one
// more; a tile of the second kind then starts at the n-th smallest of the
// times {a + 3 k} and {a + 4 + 3 k} (one sequence per CU), so the last one
// starts at the smallest T by which n2 starts are available.
static int64_t split_makespan(int64_t n1, int64_t n2, int cus) {
    const int64_t q = n1 / cus, r = n1 % cus, a = 4 * q, b = a + 4;
    const int64_t first = r > 0 ? b : a;
    if (n2 == 0) return n1 > 0 ? first : 0;
    auto starts = [&](int64_t t) {  // tile starts of the second kind at or before t
        int64_t n = 0;
        if (t >= a) n += (cus - r) * ((t - a) / 3 + 1);
        if (r > 0 && t >= b) n += r * ((t - b) / 3 + 1);
        return n;
    };
    int64_t lo = a, hi = a + 3 * n2;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (starts(mid) >= n2)
            hi = mid;
        else
            lo = mid + 1;
    }
    return first > lo + 3 ? first : lo + 3;
}

// The row split of an M x N output on `cus` compute units: rows [0, *m1) in
// 256-row tiles, the rest in 192-row tiles, *grid workgroups.  All 256-row
// tiles unless moving the last rows to 192-row tiles finishes more than 3%
// sooner (the earliest finish wins; among equals, the most 256-row tiles).
void gemm_plan(int64_t M, int64_t N, int cus, int64_t *m1, int64_t *grid) {
    const int64_t tn = (N + BN - 1) / BN, kfull = (M + BM - 1) / BM;
    *m1 = M;
    *grid = kfull * tn;
    if (cus <= 0 || M <= 0 || N <= 0) return;
    const int64_t base = split_makespan(kfull * tn, 0, cus);
    int64_t best = base;
    for (int64_t k1 = kfull - 1; k1 >= 0; --k1) {
        const int64_t k2 = (M - k1 * BM + 191) / 192;
        const int64_t t = split_makespan(k1 * tn, k2 * tn, cus);
        if (t < best && t * 100 < base * 97) {
            best = t;
            *m1 = k1 * BM;
            *grid = (k1 + k2) * tn;
        }
    }
}

// The TileSplit of an M x N output on the current device.
static TileSplit choose_split(int64_t M, int64_t N, int64_t &grid) {
    int64_t m1 = M;
    gemm_plan(M, N, device_cus(), &m1, &grid);
    const int64_t tn = (N + BN - 1) / BN;
    return TileSplit{((m1 + BM - 1) / BM) * tn, m1};
}

// s_dec of an empty fused-encode output.
__global__ void quant_sdec_kernel(const float *__restrict__ amax_in, float *__restrict__ s_dec) {
    if (threadIdx.x == 0) {
        float s_enc, sd;
        tensor_scales(*amax_in, s_enc, sd);
        *s_dec = sd;
    }
}

hipError_t launch_gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_sdec,
                            const uint8_t *w_codes, const uint8_t *w_scales,
                            const float *w_sdec, int64_t M, int64_t N, int64_t K, int w_layout,
                            void *y, int ydtype, float *amax_out, const uint16_t *lora_xa,
                            const uint16_t *lora_b, int64_t lora_r, float lora_scale,
                            const QuantOut *quant, hipStream_t s) {
    if (M == 0 || N == 0) {
        if (!quant) return hipSuccess;
        NVFP4_LAUNCH("gemm_w4a4_quant", quant_sdec_kernel, dim3(1), dim3(64), 0, s,
                     quant->amax_in, quant->s_dec);
        return hipGetLastError();
    }
    int64_t ntiles = 0;
    const TileSplit ts = choose_split(M, N, ntiles);
    const dim3 grid((unsigned)ntiles);
    const GemmArgs g{a_codes, a_scales, w_codes, w_scales, M, N, K};
    const LoraArgs la{lora_xa, lora_b, lora_r, lora_scale};
    const QuantOut qo = quant ? *quant : QuantOut{};
    const bool lora = lora_xa != nullptr;
    // LDS path: K a multiple of the step, and buffer offsets that fit 31 bits
    const bool fast = K % BK == 0 && M * (K / 2) < ((int64_t)1 << 31) &&
                      N * (K / 2) < ((int64_t)1 << 31);
    static std::atomic<uint32_t> lds_set{0};
    const void *fns[12] = {(const void *)gemm_w4a4_kernel<true, true, true, false, false>,
                           (const void *)gemm_w4a4_kernel<false, true, true, false, false>,
                           (const void *)gemm_w4a4_kernel<true, true, false, false, false>,
                           (const void *)gemm_w4a4_kernel<false, true, false, false, false>,
                           (const void *)gemm_w4a4_kernel<true, true, true, true, false>,
                           (const void *)gemm_w4a4_kernel<false, true, true, true, false>,
                           (const void *)gemm_w4a4_kernel<true, true, false, true, false>,
                           (const void *)gemm_w4a4_kernel<false, true, false, true, false>,
                           (const void *)gemm_w4a4_kernel<true, true, true, false, true>,
                           (const void *)gemm_w4a4_kernel<true, true, false, false, true>,
                           (const void *)gemm_w4a4_kernel<true, false, true, false, true>,
                           (const void *)gemm_w4a4_kernel<true, false, false, false, true>};
    hipError_t e = lds_limit_once(fns, 12, kLdsBytes, lds_set);
    if (e != hipSuccess) return e;
#define NVFP4_GEMM(BF, KF, W2, LO, Q)                                                       \
    NVFP4_LAUNCH(Q ? "gemm_w4a4_quant" : LO ? "gemm_w4a4_lora" : "gemm_w4a4",                \
                 (gemm_w4a4_kernel<BF, KF, W2, LO, Q>), grid, dim3(256),                      \
                 KF ? kLdsBytes : Q ? 4 * kQWaveBytes : 0, s, g, ts, a_sdec, w_sdec, y,        \
                 amax_out, la, qo)
#define NVFP4_GEMM_K(BF, W2, LO, Q)      \
    if (fast)                            \
        NVFP4_GEMM(BF, true, W2, LO, Q); \
    else                                 \
        NVFP4_GEMM(BF, false, W2, LO, Q);
#define NVFP4_GEMM_W(BF, LO, Q)          \
    if (w_layout) {                      \
        NVFP4_GEMM_K(BF, true, LO, Q)    \
    } else {                             \
        NVFP4_GEMM_K(BF, false, LO, Q)   \
    }
    if (quant) {
        NVFP4_GEMM_W(true, false, true)
    } else if (ydtype == kBF16) {
        if (lora) {
            NVFP4_GEMM_W(true, true, false)
        } else {
            NVFP4_GEMM_W(true, false, false)
        }
    } else {
        if (lora) {
            NVFP4_GEMM_W(false, true, false)
        } else {
            NVFP4_GEMM_W(false, false, false)
        }
    }
#undef NVFP4_GEMM_W
#undef NVFP4_GEMM_K
#undef NVFP4_GEMM
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LoRA down projection XA = bf16(X A^T)
// ---------------------------------------------------------------------------

// Workgroup = 16 ROWT rows of X; its 4 waves split K into quarters
// (32-deep steps) and each accumulates (16 ROWT) x r on the 16x16x32 bf16
// MFMA, so every A fragment a wave loads serves ROWT row tiles; the
// quarters are added in LDS in wave order and stored as bf16
// (nearest-even).  Lane (c = l & 15, g = l >> 4) holds row c of each X
// fragment and of each A fragment, K values 8g .. 8g + 7 of the step; the
// output lane holds column c, rows 4g .. 4g + 3 of a tile.  Rows past M are
// clamped, never stored.
template <int NB, int ROWT>  // r = 16 * NB
__global__ __launch_bounds__(256) void lora_down_kernel(const uint16_t *__restrict__ X,
                                                        const uint16_t *__restrict__ A, int64_t M,
                                                        int64_t K, uint16_t *__restrict__ XA) {
    constexpr int r = 16 * NB;
    constexpr int U = NB * ROWT <= 8 ? 4 : 2;  // steps of loads in flight
    __shared__ f32x4 part[4][ROWT][NB][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * 16 * ROWT;
    const int64_t steps = K / 32;
    const int64_t s0 = steps * wave / 4, s1 = steps * (wave + 1) / 4;
    f32x4 acc[ROWT][NB];
#pragma unroll
    for (int t = 0; t < ROWT; ++t)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[t][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t *xp[ROWT];
#pragma unroll
    for (int t = 0; t < ROWT; ++t) {
        const int64_t xr = m0 + t * 16 + c < M ? m0 + t * 16 + c : M - 1;
        xp[t] = X + xr * K + g * 8;
    }
    const uint16_t *ap = A + (int64_t)c * K + g * 8;
    // U steps of loads in flight before their MFMAs.  A step past s1 reloads
    // step s1 - 1 with its X fragment zeroed, so it adds exact zeros: the
    // loop has no branch for the compiler to sink the loads into.
    const bf16x8 zero = {};
    for (int64_t st = s0; st < s1; st += U) {
        bf16x8 xf[U][ROWT], af[U][NB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = st + u < s1;  // wave-uniform
            const int64_t su = ok ? st + u : s1 - 1;
#pragma unroll
            for (int t = 0; t < ROWT; ++t) {
                const bf16x8 v = *(const bf16x8 *)(xp[t] + su * 32);
                xf[u][t] = ok ? v : zero;
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) af[u][j] = *(const bf16x8 *)(ap + (int64_t)j * 16 * K + su * 32);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < ROWT; ++t)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[u][t], af[u][j],
                                                                        acc[t][j], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < ROWT; ++t)
#pragma unroll
        for (int j = 0; j < NB; ++j) part[wave][t][j][lane] = acc[t][j];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < ROWT; ++t)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const f32x4 v = ((part[0][t][j][lane] + part[1][t][j][lane]) + part[2][t][j][lane]) +
                            part[3][t][j][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + t * 16 + g * 4 + e;
                if (row < M) ((__bf16 *)XA)[row * r + j * 16 + c] = (__bf16)v[e];
            }
        }
}

hipError_t launch_lora_down(const uint16_t *x, const uint16_t *a, int64_t M, int64_t K, int64_t r,
                            uint16_t *xa, hipStream_t s) {
    if (M == 0) return hipSuccess;
    // two 16-row tiles per workgroup (measured against one and four); ROWT x NB
    // <= 16 bounds the LDS hand-off at 64 KB
    constexpr int kRowTiles = 2;
#define NVFP4_LD(NB)                                                                        \
    {                                                                                       \
        constexpr int RT = kRowTiles * (NB) <= 16 ? kRowTiles : 16 / (NB);                   \
        const dim3 grid((unsigned)((M + 16 * RT - 1) / (16 * RT)));                          \
        NVFP4_LAUNCH("lora_down", (lora_down_kernel<NB, RT>), grid, dim3(256), 0, s, x, a, M, \
                     K, xa);                                                                \
    }
    switch (r) {
    case 16: NVFP4_LD(1); break;
    case 32: NVFP4_LD(2); break;
    case 64: NVFP4_LD(4); break;
    case 128: NVFP4_LD(8); break;
    default: return hipErrorInvalidValue;
    }
#undef NVFP4_LD
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MXFP4 reference GEMM (speed reference, not part of the method)
// ---------------------------------------------------------------------------
//
// OCP Microscaling (MX) v1.0 MXFP4: E2M1 elements with one power-of-two E8M0
// scale per 32 consecutive elements (1-D along K for both operands).  gfx950
// multiplies such operands natively: v_mfma_scale_f32_32x32x64_f8f6f4 with
// fp4 A and B takes the packed codes as they are and one E8M0 byte per lane
// per 32 K values.  Lane half h holds K [128 h, 128 h + 128) of a 256-deep
// step as in the NVFP4 kernel, so MFMA substep s (64 K) pairs dwords
// 4s .. 4s + 3 of both halves, each half with its own block scale (byte s of
// the half's scale dword).  Codes are staged through LDS exactly as for
// NVFP4; the scale dword of each fragment is loaded from memory per step.
// Y = sum_k A_mx[m, k] * W_mx[n, k], fp32 accumulation, no tensor scale.
//
// The NVFP4 operands cannot run on this instruction: an E4M3 block scale
// has 3 mantissa bits (E8M0 is a pure power of two), covers 16 elements
// (two per MX block), and E2M1 x E4M3 needs up to 6 significant bits, which
// no FP4/FP6/FP8 element times a power of two holds.

template <int S>
__device__ __forceinline__ void mx_substep(f32x16 (&acc)[FM][FN], const Frag (&A)[FM],
                                           const Frag (&B)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const u32x4 qa = A[i].q[S], qb = B[j].q[S];
            const i32x8 a = {(int)qa.x, (int)qa.y, (int)qa.z, (int)qa.w, 0, 0, 0, 0};
            const i32x8 b = {(int)qb.x, (int)qb.y, (int)qb.z, (int)qb.w, 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                a, b, acc[i][j], 4, 4, S, (int)A[i].sc.x, S, (int)B[j].sc.x);
        }
}

template <int... S>
__device__ __forceinline__ void mx_step(f32x16 (&acc)[FM][FN], const Frag (&A)[FM],
                                        const Frag (&B)[FN], std::integer_sequence<int, S...>) {
    (mx_substep<S>(acc, A, B), ...);
}

// g.a_scales / g.w_scales hold the E8M0 bytes, [rows, K / 32].  K % 256 == 0.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_mx_kernel(GemmArgs g, void *__restrict__ yv) {
    const int64_t M = g.M, N = g.N, K = g.K;
    const int64_t tn_count = (N + BN - 1) / BN;
    const int64_t ntiles = ((M + BM - 1) / BM) * tn_count;
    const int64_t b = blockIdx.x;
    const int64_t per = ntiles / kXcds;
    const int64_t t = b < per * kXcds ? (b % kXcds) * per + b / kXcds : b;
    const int64_t m0 = (t / tn_count) * BM, n0 = (t % tn_count) * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, r = lane & 31, wm = wave >> 1, wn = wave & 1;
    const int64_t mw = m0 + wm * WM, nw = n0 + wn * WN;
    const bool active = mw < M && nw < N;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // scale dword of each fragment row: bytes 8 kt + 4 h .. +3 of the row
    const int64_t SB = K >> 5;
    const uint8_t *sa[FM], *sb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t row = mw + i * 32 + r < M ? mw + i * 32 + r : M - 1;
        sa[i] = g.a_scales + row * SB + h * 4;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t row = nw + j * 32 + r < N ? nw + j * 32 + r : N - 1;
        sb[j] = g.w_scales + row * SB + h * 4;
    }

    const int64_t nk = K / BK;
    Frag A[FM], B[FN];
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    StageSrc src;
    stage_src<false, true>(src, g, m0, n0, wave, lane);
    stage_load<false, true>(src, lds, 0, wave, lane);
    if (active) {
        for (int64_t kt = 0; kt < nk; ++kt) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            const int64_t kn = kt + 1 < nk ? kt + 1 : kt;
#pragma unroll
            for (int i = 0; i < FM; ++i) A[i].sc.x = *(const uint32_t *)(sa[i] + kt * 8);
#pragma unroll
            for (int j = 0; j < FN; ++j) B[j].sc.x = *(const uint32_t *)(sb[j] + kt * 8);
            stage_read<false, true>(A, B, lds + (kt & 1) * kStage, wm, wn, r, h);
            stage_load<false, true>(src, lds + ((kt + 1) & 1) * kStage, kn, wave, lane);
            mx_step(acc, A, B, std::make_integer_sequence<int, 4>{});
        }
    } else {
        for (int64_t kt = 0; kt < nk; ++kt) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            const int64_t kn = kt + 1 < nk ? kt + 1 : kt;
            stage_load<false, true>(src, lds + ((kt + 1) & 1) * kStage, kn, wave, lane);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!active) return;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t col = nw + j * 32 + r;
            const int64_t rbase = mw + i * 32 + h * 4;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = rbase + (e >> 2) * 8 + (e & 3);
                if (row < M && col < N) {
                    if (OUT_BF16)
                        ((__bf16 *)yv)[row * N + col] = (__bf16)acc[i][j][e];
                    else
                        ((float *)yv)[row * N + col] = acc[i][j][e];
                }
            }
        }
}

hipError_t launch_gemm_mx(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_codes,
                          const uint8_t *w_scales, int64_t M, int64_t N, int64_t K, void *y,
                          int ydtype, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    static std::atomic<uint32_t> lds_set{0};
    const void *fns[2] = {(const void *)gemm_mx_kernel<true>, (const void *)gemm_mx_kernel<false>};
    hipError_t e = lds_limit_once(fns, 2, kLdsBytes, lds_set);
    if (e != hipSuccess) return e;
    const int64_t ntiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const GemmArgs g{a_codes, a_scales, w_codes, w_scales, M, N, K};
    if (ydtype == kBF16)
        NVFP4_LAUNCH("gemm_mx", gemm_mx_kernel<true>, dim3((unsigned)ntiles), dim3(256), kLdsBytes,
                     s, g, y);
    else
        NVFP4_LAUNCH("gemm_mx", gemm_mx_kernel<false>, dim3((unsigned)ntiles), dim3(256), kLdsBytes,
                     s, g, y);
    return hipGetLastError();
}

}  // namespace nvfp4
