/*
 * nvfp4.h -- C ABI of libnvfp4, the NVFP4 data path of LongLive-2.0 on
 * AMD Instinct MI355X (gfx950).
 *
 * The library implements four things the LongLive-2.0 pages describe:
 *   1. NVFP4 quantize / dequantize: E2M1 4-bit elements, one FP8 E4M3 scale
 *      per 16-element block, one FP32 scale per tensor; 1-D (1x16) blocks for
 *      activations, 2-D (16x16) blocks for weights; the adaptive "Four Over
 *      Six" search that tries the block targets 6 and 4 and keeps the
 *      encoding with the lower squared error.
 *      ("MCISLAB DeepRead: LongLive2" summary, Method / NVFP4 training;
 *      ngjoo.com audit of arXiv 2605.18739, claim on adaptive block scaling;
 *      "LongLive-2.0: Infrastruttura Parallela NVFP4 per Video Lunghi",
 *      section Addestramento NVFP4.)
 *   2. The chunk-level KV-cache quantizer: keys K-smoothed, each chunk of
 *      F_c frames quantized independently into a ring; storage falls from
 *      4*T_c*H*d to (9/8)*T_c*H*d bytes.  (DeepRead summary, Method /
 *      inference infrastructure, parallel KV quantization.)
 *   3. The parallel gather-dequantizer of the attention window
 *      K_eff(t) = A_g u A_s u KV[t-W, t), overlapping tokens removed, the
 *      shot sink tracked by two scalar pointers and rebound on a prompt
 *      switch.  (DeepRead summary, algorithm design / Multi-Shot Attention
 *      Sink; Italian page, section Multi-Shot Attention Sink.)
 *   4. The W4A4 GEMM on NVFP4 operands.  (DeepRead summary, inference
 *      infrastructure / NVFP4 inference; Italian page, Inferenza W4A4 NVFP4.)
 * Built on these: the GEMM with its epilogue quantizing the output, the LoRA
 * branch on the frozen NVFP4 backbone, the RHT quantizer, and attention over
 * K_eff(t) read packed from the ring (each declared below with its source).
 *
 * Conventions (all entry points):
 *   - Device pointers are HIP device memory owned by the caller; the library
 *     never allocates or frees device memory.  Host structs are caller-owned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls enqueue work on it and return without synchronising the host.
 *   - Every argument is validated on the host before anything is enqueued;
 *     on failure the call returns a negative nvfp4_status, enqueues nothing
 *     and sets a thread-local message readable with nvfp4_last_error().
 *     Numeric problems on the device are not reported (that would need a
 *     synchronisation).
 *   - Device pointers must be 16-byte aligned (NVFP4_EALIGN otherwise).
 *   - Numerics: every result is bit-identical to the CPU oracle's definition
 *     (codes, scales, dequantized values, gathered KV); GEMM outputs differ
 *     from the exact fp64 product only by fp32 accumulation rounding.
 *   - Domain: finite inputs whose tensor amax is 0 or >= 2^-100.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 2

typedef enum nvfp4_status {
    NVFP4_OK = 0,
    NVFP4_EINVAL = -1, /* bad argument value or NULL pointer            */
    NVFP4_EALIGN = -2, /* device pointer not 16-byte aligned            */
    NVFP4_ESHAPE = -3, /* shapes inconsistent or not multiples of 16    */
    NVFP4_ENOSPC = -4, /* workspace / ring / output capacity too small  */
    NVFP4_ESTATE = -5, /* KV ring used out of order                     */
    NVFP4_EHIP = -6    /* the HIP runtime reported an error at launch   */
} nvfp4_status;

enum { NVFP4_DTYPE_F32 = 0, NVFP4_DTYPE_BF16 = 1 };
enum { NVFP4_LAYOUT_1D = 0, NVFP4_LAYOUT_2D = 1 };
enum { NVFP4_SEARCH_6 = 0, NVFP4_SEARCH_4O6 = 1 };

/* Library ABI version (NVFP4_ABI_VERSION of the built library). */
int nvfp4_abi_version(void);
/* Identity of the build: a digest of the sources the library was compiled
 * from (static text).  The Python binding refuses a library whose digest
 * differs from that of the sources next to it. */
const char *nvfp4_build_hash(void);
/* Static text for a status code. */
const char *nvfp4_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char *nvfp4_last_error(void);

/*
 * A packed NVFP4 tensor of logical shape [rows, cols] (row-major).
 *   codes : device, rows * cols / 2 bytes.  Byte j of row r holds column 2j
 *           in bits 0..3 and column 2j+1 in bits 4..7.  A nibble is
 *           s e1 e0 m (bit 3 = sign): E2M1 magnitudes {0,.5,1,1.5,2,3,4,6}.
 *   scales: device, OCP E4M3FN bytes (bias 7, max 448, sign bit 0).
 *           1-D: [rows, cols/16], block (r, j) = row r, columns 16j..16j+15.
 *           2-D: [rows/16, cols/16], block (I, J) = the 16x16 tile.
 *   s_dec : device, one float: the FP32 tensor decode scale.
 *   cols % 16 == 0; for 2-D also rows % 16 == 0.
 * Value of element (r, c): V(code) * RN(E4M3(scale) * s_dec).
 */
typedef struct nvfp4_tensor {
    uint8_t *codes;
    uint8_t *scales;
    float *s_dec;
    int64_t rows;
    int64_t cols;
    int32_t layout; /* NVFP4_LAYOUT_1D or NVFP4_LAYOUT_2D */
    int32_t reserved;
} nvfp4_tensor;

/* Bytes of `codes` and `scales` for a tensor of that shape and layout. */
size_t nvfp4_codes_bytes(int64_t rows, int64_t cols);
size_t nvfp4_scales_bytes(int64_t rows, int64_t cols, int32_t layout);

/*
 * Workspace (device bytes) nvfp4_quantize needs for a tensor of that shape:
 * per-workgroup amax partials.  Pure host function.
 */
size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols, int32_t layout);

/*
 * Quantize x (device, contiguous [out->rows, out->cols], dtype F32 or BF16)
 * into `out` (DeepRead summary, Method / NVFP4 training: hierarchical
 * scaling; 2-D for weights, 1-D for activations; scale search over 6 and 4).
 *   Tensor scale: amax = max|x| (or *amax_in when amax_in != NULL, the value
 *   a fused producer already computed; device pointer), s_enc =
 *   RN(2688/amax), s_dec = RN(amax/2688); amax == 0 gives s_enc = s_dec = 1.
 *   Per block, for each target c in {6, 4} (only 6 with NVFP4_SEARCH_6):
 *   scale = E4M3(RN(RN(amax_b / c) * s_enc)) (saturating at 448), decode
 *   scale S = RN(scale * s_dec), codes = E2M1(RN(x * RN(1/S))) (0 if S == 0),
 *   error = sum of RN(x - V*S)^2 in a fixed order; target 4 is kept only if
 *   its error is strictly lower.
 * Workspace: device, >= nvfp4_quantize_workspace_bytes(); contents on entry
 * are ignored.  Writes out->codes, out->scales and *out->s_dec.
 */
int nvfp4_quantize(const void *x, int32_t x_dtype, const nvfp4_tensor *out, int32_t search,
                   const float *amax_in, void *workspace, size_t workspace_bytes, void *stream);

/*
 * nvfp4_quantize with a random Hadamard transform first (DR NVFP4 training:
 * RHT stabilises the weight-gradient GEMM; IT Addestramento NVFP4: an RHT is
 * applied before quantization on the gradient-sensitive paths).  Every 1x16
 * block along a row is replaced by (1/4) H16 diag(s) x -- H16 the Sylvester
 * Hadamard matrix, s_j = -1 where bit j of `signs` (a 16-bit mask) is set --
 * computed by the fast Walsh-Hadamard butterflies (strides 1, 2, 4, 8, each
 * (a, b) -> (RN(a+b), RN(a-b))) and RN(* 0.25); then the tensor amax (of the
 * transformed values; or *amax_in), scales and 4/6 encode exactly as
 * nvfp4_quantize.  1-D layout only.  Transforming both operands of a GEMM
 * along K with the same signs leaves the product unchanged.
 */
int nvfp4_quantize_rht(const void *x, int32_t x_dtype, const nvfp4_tensor *out, int32_t search,
                       uint32_t signs, const float *amax_in, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * Dequantize `in` into y (device, contiguous [rows, cols], F32 or BF16):
 * y = V(code) * RN(E4M3(scale) * s_dec), rounded to nearest-even for BF16.
 */
int nvfp4_dequantize(const nvfp4_tensor *in, void *y, int32_t y_dtype, void *stream);

/*
 * W4A4 GEMM (DeepRead summary, inference infrastructure: BF16 GEMMs replaced
 * by FP4 GEMMs on NVFP4 weights and activations):
 *   Y[m, n] = RN(RN(s_A * s_W) * sum_k A_hat[m, k] * W_hat[n, k])
 * with A_hat = V * E4M3 scale (exact), likewise W_hat; fp32 accumulation.
 *   a: 1-D layout, [M, K].   w: [N, K] (rows = output features), 2-D layout
 *   for weights, or 1-D for a gradient operand (e.g. the weight-gradient
 *   GEMM of training, both operands 1-D along the reduction dimension).
 *   y: device, contiguous [M, N] in F32 or BF16 (nearest-even).
 *   amax_out: NULL, or a device fp32 that the call raises to
 *     max(*amax_out, max |y| over the stored y values) -- the tensor amax the
 *     next quantize of y needs (pass it as that call's amax_in to skip its
 *     amax pass; same result bit for bit).  The caller sets *amax_out before
 *     the call (0 for a fresh maximum).  Updated with an atomic max on the
 *     fp32 bit pattern, which orders non-negative values correctly.
 * K % 16 == 0, N % 16 == 0, any M >= 0.
 */
int nvfp4_gemm_w4a4(const nvfp4_tensor *a, const nvfp4_tensor *w, void *y, int32_t y_dtype,
                    float *amax_out, void *stream);

/*
 * W4A4 GEMM whose epilogue writes NVFP4 directly (producer-fused
 * requantization; TX page, NVFP4 section: the NVFP4 inference path gained
 * fused kernels and in-place quantization updates; DR summary, inference
 * infrastructure: the activations feeding the next FP4 GEMM are 1-D NVFP4).
 * y (1-D layout, [M, N], caller-owned codes / scales / s_dec) receives
 *   nvfp4_quantize(bf16(Y), search, amax_in)
 * bit for bit, Y the nvfp4_gemm_w4a4 product (bf16 nearest-even), so the
 * next GEMM reads 0.5625 bytes an element instead of a bf16 Y written and
 * read back.  amax_in (device fp32, required) is the tensor amax the encode
 * uses: max|bf16(Y)| gives exactly the unfused result; any other value (an
 * amax from an earlier call, a calibrated one) is used as given, values
 * beyond it saturating as in nvfp4_quantize (block scale 448, codes 6).
 * amax_out: NULL, or raised to max|bf16(Y)| as in nvfp4_gemm_w4a4 (the
 * amax the next call may use).  Shapes and layouts of a and w as
 * nvfp4_gemm_w4a4; y->rows == M, y->cols == N.  M == 0 or N == 0 writes
 * s_dec only.
 */
int nvfp4_gemm_w4a4_quant(const nvfp4_tensor *a, const nvfp4_tensor *w, const nvfp4_tensor *y,
                          int32_t search, const float *amax_in, float *amax_out, void *stream);

/*
 * LoRA on the frozen NVFP4 backbone (DR few-step distillation: the model is
 * the frozen quantized backbone plus LoRA adapters, W ~ Dequant(Q_search(W_0))
 * + (alpha/r) B A; IT: only the LoRA adapters are trained on the frozen
 * quantized backbone).  The layer's output is the W4A4 product plus the
 * adapter branch (alpha/r) (x A^T) B^T, the branch in bf16:
 *
 * nvfp4_lora_down: xa[M, r] = bf16(x A^T), fp32 accumulation, nearest-even;
 *   x [M, K] and a [r, K] bf16, row-major device memory; r in {16, 32, 64,
 *   128}; K % 32 == 0.
 * nvfp4_gemm_w4a4_lora: as nvfp4_gemm_w4a4, with
 *   y = fma(lora_scale, sum_j xa[m, j] b[n, j], RN(RN(s_A s_W) acc))
 *   (the branch on the bf16 MFMA, fp32 accumulation); xa [M, r] and
 *   b [N, r] bf16, r as above; lora_scale = alpha / r.
 */
int nvfp4_lora_down(const void *x_bf16, const void *a_bf16, int64_t M, int64_t K, int64_t r,
                    void *xa_bf16, void *stream);
int nvfp4_gemm_w4a4_lora(const nvfp4_tensor *a, const nvfp4_tensor *w, const void *xa_bf16,
                         const void *b_bf16, int64_t r, float lora_scale, void *y,
                         int32_t y_dtype, float *amax_out, void *stream);

/* ------------------------------------------------------------------------ */
/* MXFP4 speed reference (not part of the method)                            */
/* ------------------------------------------------------------------------ */

/*
 * The W4A4 GEMM is measured beside the gfx950 MFMA that takes FP4 operands
 * with power-of-two block scales: MXFP4 of the OCP Microscaling Formats
 * (MX) v1.0 specification -- E2M1 elements, one E8M0 scale (2^(byte - 127))
 * per 32 consecutive elements along a row.  NVFP4 operands cannot use that
 * instruction (E4M3 scale with mantissa bits, 16-element blocks, products
 * of up to 6 significant bits), so the MX result is a different
 * quantization of the same data, compared for speed and error only.
 *
 * nvfp4_mx_quantize: x (device, F32 or BF16, contiguous [rows, cols],
 *   cols % 32 == 0) -> codes [rows, cols/2] (element 2j in the low nibble of
 *   byte j) and scales [rows, cols/32] E8M0 bytes, all caller-owned device
 *   memory.  Per block: e = floor(log2(amax)) - 2 clamped to [-127, 127]
 *   (a subnormal amax gives -127), scale byte e + 127 (0 for an all-zero
 *   block), elements E2M1(RN(x * 2^-e)) saturating at 6.
 */
int nvfp4_mx_quantize(const void *x, int32_t x_dtype, int64_t rows, int64_t cols,
                      uint8_t *codes, uint8_t *scales, void *stream);

/*
 * nvfp4_gemm_mx: Y[m, n] = sum_k A_mx[m, k] * W_mx[n, k] with fp32
 * accumulation (v_mfma_scale_f32_32x32x64_f8f6f4); A [M, K] and W [N, K] as
 * written by nvfp4_mx_quantize; y device [M, N] F32 or BF16 (nearest-even).
 * K % 256 == 0, M, N >= 0; each code array below 2^31 bytes.
 */
int nvfp4_gemm_mx(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_codes,
                  const uint8_t *w_scales, int64_t M, int64_t N, int64_t K, void *y,
                  int32_t y_dtype, void *stream);

/* ------------------------------------------------------------------------ */
/* KV-cache ring                                                              */
/* ------------------------------------------------------------------------ */

/*
 * Shape of the streaming KV cache (DeepRead summary: chunk of F_c = 8 latent
 * frames; 5B model: 880 tokens per frame, 24 heads of width 128; global sink
 * A_g = first S_g frames, shot sink A_s = first S_s frames of the current
 * shot, window of W chunks).  K and V of a chunk are bf16 [T_c, heads,
 * head_dim], token-major, T_c = tokens_per_frame * frames_per_chunk.
 */
typedef struct nvfp4_kv_config {
    int32_t tokens_per_frame;   /* L_f  (880); T_c <= 65536, T_c*H*d < 2^31 */
    int32_t frames_per_chunk;   /* F_c  (8)   */
    int32_t heads;              /* H    (24)  */
    int32_t head_dim;           /* d    (128), multiple of 16 */
    int32_t sink_frames_global; /* S_g  (3),  0 <= S_g <= F_c */
    int32_t sink_frames_shot;   /* S_s  (3),  0 <= S_s <= F_c */
    int32_t window_chunks;      /* W    (4),  1 <= W <= NVFP4_KV_MAX_WINDOW */
    int32_t search;             /* NVFP4_SEARCH_6 or NVFP4_SEARCH_4O6 */
} nvfp4_kv_config;

#define NVFP4_KV_MAX_WINDOW 16

/*
 * Host-side ring state.  Allocate it yourself (it is plain data), set it up
 * with nvfp4_kv_ring_init and treat every field as read-only.  The device
 * memory it points at is caller-owned.  Layout of that memory: W chunk slots
 * (chunk c lives in slot c mod W), then a global-sink region and a shot-sink
 * region; each region holds packed K codes, K scales, V codes, V scales
 * ((9/8) bytes per K+V element), the chunk's key mean mu[H*d] (fp32) and its
 * two FP32 decode scales.  A ring must not be used from two host threads at
 * once.
 */
typedef struct nvfp4_kv_ring {
    nvfp4_kv_config cfg;
    uint8_t *base;          /* device memory given to nvfp4_kv_ring_init */
    uint64_t bytes;         /* its size */
    int64_t chunk_tokens;   /* T_c */
    int64_t hd;             /* heads * head_dim */
    int64_t slot_bytes;     /* bytes of one chunk slot */
    int64_t gsink_offset;   /* byte offset of the global-sink region */
    int64_t ssink_offset;   /* byte offset of the shot-sink region */
    int64_t next_chunk;     /* number of chunks stored so far */
    int64_t g_end;          /* sink pointer 1: end of A_g (token index) */
    int64_t s_start;        /* sink pointer 2: first token of the current shot */
} nvfp4_kv_ring;

/* Device bytes a ring of this configuration needs (pure host). */
size_t nvfp4_kv_ring_bytes(const nvfp4_kv_config *cfg);
/* Device workspace nvfp4_kv_store_chunk needs (pure host). */
size_t nvfp4_kv_store_workspace_bytes(const nvfp4_kv_config *cfg);

/*
 * Set up `ring` over caller-owned device memory `dev_mem` of `bytes` bytes
 * (>= nvfp4_kv_ring_bytes(cfg)).  No device work is enqueued.  The ring
 * starts empty with chunk 0 as the first shot (s_start = 0).
 */
int nvfp4_kv_ring_init(nvfp4_kv_ring *ring, const nvfp4_kv_config *cfg, void *dev_mem,
                       size_t bytes);

/*
 * Prompt switch: rebind the shot sink A_s to the chunk about to be generated
 * (chunk_idx must equal ring->next_chunk).  Sets s_start = chunk_idx * T_c;
 * the global sink and the history are untouched (DeepRead summary: a prompt
 * switch rebinds A_s and keeps the global sink and history).  Host-only.
 */
int nvfp4_kv_begin_shot(nvfp4_kv_ring *ring, int64_t chunk_idx);

/*
 * Quantize chunk `chunk_idx` (must equal ring->next_chunk) into its ring
 * slot (DeepRead summary: chunk-level KV quantization, keys K-smoothed).
 *   K, V: device bf16 [T_c, H, d].
 *   mu[h, c] = (float)RN64(S / T_c), S the exact sum of the chunk's T_c keys
 *   of channel (h, c) (the exact quotient rounded to double, then to float);
 *   K_s = RN(K - mu).  The kernels sum in double, which is exact, so mu is
 *   exactly that, whenever sum_t |K[t, h, c]| < 2^53 * 2^k with 2^k the
 *   largest power of two dividing every nonzero key of the channel (for
 *   bf16 keys it suffices that their exponents span at most 45 - log2(T_c)
 *   binades: 32 at T_c = 7040); outside that domain mu may differ from it
 *   in the last bit.  K_s and V are each quantized 1-D along (h, c) with one
 *   FP32 tensor scale per chunk.  Chunk 0 also fills the global-sink region
 *   and the first chunk of a shot fills the shot-sink region (byte copies of
 *   the leading sink tokens, written by the same kernel).  Advances
 *   next_chunk.
 *   v_amax_in: NULL, or a device fp32 holding max |V| over the chunk, as a
 *   fused producer has it (e.g. the amax_out of the GEMM that wrote V; the
 *   same applies as for nvfp4_quantize's amax_in): the value tensor scale
 *   then comes from it and the statistics pass reads the keys only.  Another
 *   value is used as given (values beyond it saturate as in nvfp4_quantize).
 * Workspace: device, >= nvfp4_kv_store_workspace_bytes(), 16-byte aligned,
 *   owned by the caller.  It holds accumulators that must be zero when the
 *   store of a chunk > 0 starts: every store leaves them zero, and the store
 *   of chunk 0 clears them first (one small extra launch).  So one workspace
 *   serves one ring's stores, or several rings' stores one after another;
 *   two stores sharing a workspace must not overlap.
 * Two launches (three for chunk 0): statistics (whose last workgroup of
 *   each channel group finalizes the group's mean and amax), encode.
 */
int nvfp4_kv_store_chunk(nvfp4_kv_ring *ring, int64_t chunk_idx, const void *K_bf16,
                         const void *V_bf16, const float *v_amax_in, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * nvfp4_kv_store_chunk without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation).  Same arguments, checks and results as
 * nvfp4_kv_store_chunk, bit for bit; the store's accumulators live in a
 * fixed device array of the library instead (about 257 KB on every device
 * the call runs on, kept until the process ends; located, and cleared by a
 * fill kernel on `stream`, on the first call on each device).  Rejects
 * heads * head_dim above NVFP4_KV_NOALLOC_MAX_CHANNELS with NVFP4_ENOSPC.
 * Calls the library makes no allocation for.  Every call on one GPU shares
 * that array: calls that overlap on one GPU (different streams, or host
 * threads) race, whichever ring they store into; calls that follow one
 * another in stream order do not.
 */
#define NVFP4_KV_NOALLOC_MAX_CHANNELS 16384
int nvfp4_kv_store_chunk_noalloc(nvfp4_kv_ring *ring, int64_t chunk_idx, const void *K_bf16,
                                 const void *V_bf16, const float *v_amax_in, void *stream);

/*
 * Number of tokens in K_eff(step) (step must equal ring->next_chunk: the
 * step that generates chunk `step`).  K_eff(step) = (A_g u A_s u
 * [max(0, step-W)*T_c, step*T_c)) n [0, step*T_c).  Pure host.
 */
int nvfp4_kv_effective_tokens(const nvfp4_kv_ring *ring, int64_t step, int64_t *n_tokens);

/*
 * Dequantize K_eff(step) into K_out / V_out (device bf16 [n, H, d],
 * ascending token order, each token once): K_hat = bf16(RN(x_hat + mu)),
 * V_hat = bf16(x_hat), x_hat = V(code) * RN(scale * s_dec) of the token's
 * own chunk.  capacity_tokens below n gives NVFP4_ENOSPC.  *n_tokens (host)
 * receives n.  One kernel launch.
 */
int nvfp4_gather_window(const nvfp4_kv_ring *ring, int64_t step, void *K_out, void *V_out,
                        int64_t capacity_tokens, int64_t *n_tokens, void *stream);

/*
 * Launch shape nvfp4_gemm_w4a4 (and its variants) takes for an M x N output
 * on a device with `compute_units` CUs (pure host; the launch asks the
 * device for its count).  The output's first *rows_256 rows go in 256 x 192
 * tiles and the rest in 192 x 192 tiles, *workgroups in all: 192-row tiles
 * for the last rows only where greedy in-order dispatch of the two kinds of
 * tile onto the CUs finishes more than 3% sooner than all 256-row tiles (a
 * 192-row tile taken as 3/4 of a 256-row one).  Results do not depend on the
 * split.  M, N >= 0, compute_units >= 1, non-NULL outputs, else
 * NVFP4_EINVAL.
 */
int nvfp4_gemm_plan(int64_t M, int64_t N, int32_t compute_units, int64_t *rows_256,
                    int64_t *workgroups);

/*
 * Attention of step `step`'s queries over K_eff(step), read packed from the
 * ring with the dequantization fused in (DeepRead summary, Multi-Shot
 * Attention Sink: sliding-window self-attention over K_eff(t) = A_g u A_s u
 * KV[t-W, t); TX page, NVFP4 section: the FP4 KV cache with a fused
 * dequantization extension).  Per head hh and query i:
 *   o[i, hh] = sum_j softmax_j(softmax_scale * q[i, hh] . K_hat[j, hh]) V_hat[j, hh]
 *   lse[i, hh] = ln sum_j exp(softmax_scale * q[i, hh] . K_hat[j, hh])
 * over the tokens j of K_eff(step), with K_hat and V_hat the bf16 values
 * nvfp4_gather_window would write (so the result equals attention over the
 * gathered K/V).  Scores and sums in fp32 (the products on the bf16 MFMA),
 * the softmax weights rounded to bf16 for the value product and its
 * normaliser alike (so exp(lse) carries their 2^-9 relative rounding), o
 * rounded to bf16 (nearest-even).
 *   softmax_scale: finite and >= 0 (0 gives the mean of the values).
 *   step: must equal ring->next_chunk, as for the gather.
 *   q, o: device bf16 [n_q, H, 128], row-major, 16-byte aligned; head_dim
 *     must be 128 (else NVFP4_ESHAPE).
 *   lse: NULL, or device fp32 [n_q, H] (for merging with attention over
 *     other keys, e.g. the chunk's own).
 *   key_splits: 0 lets the library choose (see nvfp4_attention_plan), 1 to
 *     NVFP4_ATTN_MAX_SPLITS fixes the count (else NVFP4_EINVAL).  With s > 1
 *     splits the key set's 64-key tiles are cut into s consecutive runs of
 *     near-equal length, each run's partial softmax (fp32 unnormalised output,
 *     reference maximum and sum of weights) goes to the workspace, and a second
 *     kernel combines the runs in index order, rescaling each by 2^(m_s - M)
 *     (the blockwise softmax merge).  Results depend on s only through fp32
 *     rounding and are identical from call to call for the same s.
 *   ws, ws_bytes: device workspace of at least the bytes nvfp4_attention_plan
 *     reports for the same arguments, 256-byte aligned (else NVFP4_ENOSPC /
 *     NVFP4_EALIGN); unused (may be NULL) when the plan has one split.  Owned
 *     by the caller; the call must not overlap another use of it.
 *   An empty K_eff (step 0) gives o = 0 and lse = -inf.  One kernel launch,
 *   two with splits.
 */
int nvfp4_attention_window(const nvfp4_kv_ring *ring, int64_t step, const void *q_bf16,
                           int64_t n_q, float softmax_scale, void *o_bf16, float *lse,
                           int32_t key_splits, void *ws, size_t ws_bytes, void *stream);

#define NVFP4_ATTN_MAX_SPLITS 8

/*
 * Key splits and workspace bytes nvfp4_attention_window takes for the same
 * ring, step, n_q and key_splits (same checks, same errors; host only, but
 * key_splits = 0 reads the current device's compute-unit count).  The
 * automatic choice: a workgroup of 256 queries of one head fills a compute
 * unit, so n = ceil(n_q / 256) * H workgroups run in rounds of one per
 * unit, and s splits take ceil(n s / CUs) rounds of 1/s the time, each split
 * adding about 1.5% (its pipeline fill, its partial output, the merge).  The
 * cheapest s in 1..8 under that model is taken if it saves 3% over one
 * split, each split keeping at least 8 of the 64-key tiles (e.g. 7040 queries
 * x 24 heads on 256 units: 672 workgroups, 3 splits, 8 rounds of a third
 * instead of 3 whole ones; 256 queries x 24 heads: 8 splits).
 * Workspace: the (max, sum) fp32 pairs, 8 s n_q H bytes rounded up to a
 * multiple of 256, then the fp32 outputs, 512 s n_q H bytes; 0 for one split.
 */
int nvfp4_attention_plan(const nvfp4_kv_ring *ring, int64_t step, int64_t n_q, int32_t key_splits,
                         int32_t *splits, size_t *ws_bytes);

/* ------------------------------------------------------------------------ */
/* Kernel timing                                                              */
/* ------------------------------------------------------------------------ */

/*
 * Turn kernel timing on (on != 0) or off.  While on, every kernel launch of
 * the library is bracketed by two HIP events recorded on the launch's
 * stream (HIP events are created on first use and reused; no device memory
 * is allocated).  Process-wide; off by default.
 */
int nvfp4_profile_enable(int on);

/*
 * Wait for every recorded launch, then report per kernel name (sorted):
 * names (cap entries of name_len bytes, NUL-terminated), launch counts and
 * summed event-to-event milliseconds.  Clears the record.  Returns the number
 * of distinct kernels (which may exceed cap), or NVFP4_EHIP.
 */
int nvfp4_profile_collect(char *names, int name_len, int64_t *launches, double *total_ms,
                          int cap);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
