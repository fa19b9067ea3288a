// launch.hpp -- host-side launchers of the libnvfp4 kernels (internal).
// Arguments are validated by the C ABI layer (capi.cpp) before these run.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace nvfp4 {

// ---- profile.cpp: optional HIP-event timing of every launch
bool prof_on();
// Reserves a (start, stop) event pair under NAME; false if none is available.
bool prof_take(const char *name, hipEvent_t *start, hipEvent_t *stop);

// Launch KERNEL (parenthesise template kernels).  When timing is enabled the
// launch goes through hipExtLaunchKernelGGL with an event pair that the
// dispatch itself time-stamps at kernel start and end, on STREAM.
#define NVFP4_LAUNCH(NAME, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                       \
    do {                                                                                 \
        hipEvent_t _e0 = nullptr, _e1 = nullptr;                                         \
        if (::nvfp4::prof_on() && ::nvfp4::prof_take(NAME, &_e0, &_e1))                  \
            hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, _e0, _e1, 0,       \
                                  __VA_ARGS__);                                          \
        else                                                                             \
            hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);         \
    } while (0)

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kMaxPartials = 1024;  // amax partials per quantize call

// ---- quantize.hip
int amax_partials_for(int64_t n);
hipError_t launch_amax(const void *x, int dtype, int64_t n, float *partials, int np,
                       hipStream_t s);
hipError_t launch_encode(const void *x, int dtype, int64_t rows, int64_t cols, int layout,
                         int search, const float *partials, int np, const float *amax_in,
                         uint8_t *codes, uint8_t *scales, float *s_dec, hipStream_t s);
hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, const float *s_dec,
                          int64_t rows, int64_t cols, int layout, void *y, int ydtype,
                          hipStream_t s);

// ---- kv.hip
// Addresses of one ring region (a chunk slot or a sink copy).
struct KvRegion {
    uint8_t *kc;  // K codes   [tokens, HD/2]
    uint8_t *ks;  // K scales  [tokens, HD/16]
    uint8_t *vc;  // V codes
    uint8_t *vs;  // V scales
    float *mu;    // [HD]
    float *sd;    // [2]: s_dec of K_s, s_dec of V
};

struct KvStoreArgs {
    const uint16_t *K;
    const uint16_t *V;
    int64_t T;   // tokens in the chunk
    int64_t HD;  // heads * head_dim
    int search;
    KvRegion slot;
    KvRegion gsink;  // written when g_tokens > 0
    KvRegion ssink;  // written when s_tokens > 0
    int64_t g_tokens;
    int64_t s_tokens;
    const float *v_amax_in;  // nullptr: the stats pass takes the value amax itself
    void *ws;                // accumulators zero unless clear_ws (see kv.hip)
    bool clear_ws;           // zero them first (the first store of a ring)
};
size_t kv_store_ws_bytes(int64_t T, int64_t HD);
hipError_t launch_kv_store(const KvStoreArgs &a, hipStream_t s);
constexpr int kMaxDevices = 64;
// Largest heads * head_dim the allocation-free store takes.
int64_t kv_noalloc_max_hd();
// Device address and size of the allocation-free store's scratch on the
// current device (looked up, and zeroed on stream s, on the first call per
// device).
hipError_t kv_noalloc_scratch(void **ptr, size_t *bytes, hipStream_t s);

// A run of consecutive stored tokens of one ring region (a chunk slot or a
// sink copy): one key mean, one pair of decode scales.  K_eff(t) is up to
// 2 + W such segments in ascending token order (global sink part, shot sink
// part, window chunks).
constexpr int kMaxSeg = 2 + 16;
struct KvSeg {
    const uint8_t *kc, *ks, *vc, *vs;  // codes / scales of the segment's first token
    const float *mu;                   // [HD] key mean of the region
    const float *sd;                   // [2] decode scales (K_s, V)
    int64_t n;                         // tokens
};

// Gather plan: workgroups [wg0[s], wg0[s + 1]) take segment s, tpw tokens
// each (the last one fewer); segment s's tokens go to output rows
// out0[s] .. out0[s] + n - 1.
struct GatherArgs {
    KvSeg seg[kMaxSeg];
    int32_t wg0[kMaxSeg + 1];
    int64_t out0[kMaxSeg];
    int32_t nseg;
    int32_t tpw;
    int64_t HD;
    uint16_t *Kout;
    uint16_t *Vout;
};
hipError_t launch_gather(const GatherArgs &a, hipStream_t s);

// ---- attn.hip
// Attention over K_eff(t) read packed from the ring: the effective set as
// up to 2 + W segments, each a run of consecutive tokens of one region (one
// key mean, one pair of decode scales), in ascending token order.
constexpr int kAttnMaxSeg = kMaxSeg;
typedef KvSeg AttnSeg;
struct AttnArgs {
    AttnSeg seg[kAttnMaxSeg];
    int32_t tile0[kAttnMaxSeg + 1];  // first 64-key tile of each segment, tile0[nseg] = total
    int32_t nseg;
    int32_t heads;
    int64_t HD;                      // heads * 128
    int64_t nq;
    const uint16_t *q;               // [nq, heads, 128] bf16
    uint16_t *o;                     // [nq, heads, 128] bf16
    float *lse;                      // [nq, heads] or nullptr
    float scale_log2;                // softmax scale * log2(e)
    // Key splits: workgroup (split, query block, head) takes the split's
    // share of the tiles; with nsplit > 1 it writes its unnormalised output
    // and (reference max in log2 units, sum of weights) to the workspace and a
    // second kernel merges the splits into o and lse.
    int32_t nsplit;
    float *part_ml;                  // [nsplit][nq][heads] (m, l)
    float *part_o;                   // [nsplit][nq][heads][128]
};
constexpr int kAttnMaxSplit = 8;      // most key splits a call takes
// Workspace bytes of `nsplit` key splits (0 for one split).
size_t attn_workspace_bytes(int64_t nq, int heads, int nsplit);
// Key splits for nq queries over ntile 64-key tiles: `requested` if > 0,
// else the count that best fills the device's compute units.
hipError_t attn_choose_splits(int64_t nq, int heads, int ntile, int requested, int *nsplit);
hipError_t launch_attn_window(const AttnArgs &a, hipStream_t s);

// ---- gemm.hip
// Raise the dynamic-LDS limit of the kernels `fns` to `bytes`, once per
// device (`done`: one bit per device id).
hipError_t lds_limit_once(const void *const *fns, int n, int bytes, std::atomic<uint32_t> &done);

// NVFP4 output of the GEMM's fused encode: Y [M, N] with 1-D blocks.
struct QuantOut {
    uint8_t *codes;         // [M, N / 2]
    uint8_t *scales;        // [M, N / 16]
    float *s_dec;           // one float
    const float *amax_in;   // tensor amax the encode uses (device)
    int four_over_six;
};
// quant == nullptr: Y in ydtype at y.  Otherwise Y goes to *quant (y and
// ydtype unused, no LoRA).
hipError_t launch_gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_sdec,
                            const uint8_t *w_codes, const uint8_t *w_scales,
                            const float *w_sdec, int64_t M, int64_t N, int64_t K, int w_layout,
                            void *y, int ydtype, float *amax_out, const uint16_t *lora_xa,
                            const uint16_t *lora_b, int64_t lora_r, float lora_scale,
                            const QuantOut *quant, hipStream_t s);
// Row split of the W4A4 grid for `cus` compute units (rows [0, *m1) in
// 256-row tiles, the rest in 192-row tiles) and its workgroup count.
void gemm_plan(int64_t M, int64_t N, int cus, int64_t *m1, int64_t *grid);
hipError_t launch_lora_down(const uint16_t *x, const uint16_t *a, int64_t M, int64_t K, int64_t r,
                            uint16_t *xa, hipStream_t s);
hipError_t launch_gemm_mx(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_codes,
                          const uint8_t *w_scales, int64_t M, int64_t N, int64_t K, void *y,
                          int ydtype, hipStream_t s);
hipError_t launch_quantize_rht(const void *x, int dtype, int64_t rows, int64_t cols, int search,
                               uint32_t signs, float *partials, const float *amax_in,
                               uint8_t *codes, uint8_t *scales, float *s_dec, hipStream_t s);
hipError_t launch_mx_quantize(const void *x, int xdtype, int64_t rows, int64_t cols,
                              uint8_t *codes, uint8_t *scales, hipStream_t s);

}  // namespace nvfp4
