// Drives the C ABI's host side -- argument validation, ring bookkeeping, the
// effective-set plan and the launchers' grid arithmetic -- in a build of the
// whole library for the host only, with AddressSanitizer and
// UndefinedBehaviorSanitizer (any finding aborts).  There is no GPU here:
// calls that pass validation reach a launch, which the HIP runtime refuses
// (NVFP4_EHIP).  Device pointers are host-side stand-ins that nothing
// dereferences.  Test infrastructure.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <set>

#include "nvfp4.h"

static int failures = 0;
#define EXPECT(cond)                                                    \
    do {                                                                \
        if (!(cond)) {                                                  \
            std::printf("FAILED line %d: %s (%s)\n", __LINE__, #cond,   \
                        nvfp4_last_error());                            \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static void *const F = (void *)(uintptr_t)0x7F0000000000ull;  // aligned stand-in
static uint8_t *const FB = (uint8_t *)F;

static nvfp4_tensor tensor(int64_t rows, int64_t cols, int32_t layout) {
    nvfp4_tensor t{};
    t.codes = FB;
    t.scales = FB + (1 << 20);
    t.s_dec = (float *)(FB + (2 << 20));
    t.rows = rows;
    t.cols = cols;
    t.layout = layout;
    return t;
}

static bool launched_or_ok(int st) { return st == NVFP4_OK || st == NVFP4_EHIP; }

int main() {
    EXPECT(nvfp4_abi_version() == NVFP4_ABI_VERSION);
    for (int s = 1; s >= -8; --s) EXPECT(nvfp4_status_string(s) != nullptr);
    EXPECT(nvfp4_build_hash() != nullptr);
    EXPECT(nvfp4_codes_bytes(-1, 16) == 0 && nvfp4_scales_bytes(16, -1, 0) == 0);

    // quantize / dequantize
    nvfp4_tensor t = tensor(64, 128, NVFP4_LAYOUT_1D);
    const size_t ws = nvfp4_quantize_workspace_bytes(64, 128, 0);
    EXPECT(nvfp4_quantize(F, NVFP4_DTYPE_BF16, nullptr, 1, nullptr, F, ws, nullptr) == NVFP4_EINVAL);
    EXPECT(nvfp4_quantize(F, 7, &t, 1, nullptr, F, ws, nullptr) == NVFP4_EINVAL);
    EXPECT(nvfp4_quantize(F, 1, &t, 5, nullptr, F, ws, nullptr) == NVFP4_EINVAL);
    EXPECT(nvfp4_quantize(FB + 2, 1, &t, 1, nullptr, F, ws, nullptr) == NVFP4_EALIGN);
    EXPECT(nvfp4_quantize(F, 1, &t, 1, nullptr, F, ws - 1, nullptr) == NVFP4_ENOSPC);
    nvfp4_tensor bad = tensor(64, 24, 0);
    EXPECT(nvfp4_quantize(F, 1, &bad, 1, nullptr, F, ws, nullptr) == NVFP4_ESHAPE);
    bad = tensor(24, 64, 1);
    EXPECT(nvfp4_quantize(F, 1, &bad, 1, nullptr, F, ws, nullptr) == NVFP4_ESHAPE);
    bad = tensor(-1, 64, 0);
    EXPECT(nvfp4_quantize(F, 1, &bad, 1, nullptr, F, ws, nullptr) == NVFP4_ESHAPE);
    EXPECT(launched_or_ok(nvfp4_quantize(F, 1, &t, 1, nullptr, F, ws, nullptr)));
    EXPECT(launched_or_ok(nvfp4_quantize(F, 0, &t, 0, (const float *)F, nullptr, 0, nullptr)));
    EXPECT(launched_or_ok(nvfp4_quantize_rht(F, 1, &t, 1, 0xFFFFu, nullptr, F, ws, nullptr)));
    EXPECT(nvfp4_quantize_rht(F, 1, &t, 1, 0x10000u, nullptr, F, ws, nullptr) == NVFP4_EINVAL);
    EXPECT(launched_or_ok(nvfp4_dequantize(&t, F, NVFP4_DTYPE_F32, nullptr)));
    EXPECT(nvfp4_dequantize(&t, FB + 8, NVFP4_DTYPE_F32, nullptr) == NVFP4_EALIGN);
    nvfp4_tensor empty = tensor(0, 0, 0);
    EXPECT(nvfp4_dequantize(&empty, F, 1, nullptr) == NVFP4_OK);

    // GEMMs
    nvfp4_tensor a = tensor(100, 256, 0), w = tensor(48, 256, 1), w1 = tensor(48, 256, 0);
    EXPECT(launched_or_ok(nvfp4_gemm_w4a4(&a, &w, F, 1, nullptr, nullptr)));
    EXPECT(launched_or_ok(nvfp4_gemm_w4a4(&a, &w1, F, 0, (float *)F, nullptr)));
    EXPECT(nvfp4_gemm_w4a4(&w, &w, F, 1, nullptr, nullptr) == NVFP4_EINVAL);  // A 2-D
    nvfp4_tensor ak = tensor(100, 128, 0);
    EXPECT(nvfp4_gemm_w4a4(&ak, &w, F, 1, nullptr, nullptr) == NVFP4_ESHAPE);
    EXPECT(nvfp4_gemm_w4a4(&a, &w, FB + 4, 1, nullptr, nullptr) == NVFP4_EALIGN);
    nvfp4_tensor y = tensor(100, 48, 0);
    EXPECT(launched_or_ok(nvfp4_gemm_w4a4_quant(&a, &w, &y, 1, (const float *)F, nullptr, nullptr)));
    EXPECT(nvfp4_gemm_w4a4_quant(&a, &w, &y, 1, nullptr, nullptr, nullptr) == NVFP4_EINVAL);
    nvfp4_tensor yb = tensor(100, 32, 0);
    EXPECT(nvfp4_gemm_w4a4_quant(&a, &w, &yb, 1, (const float *)F, nullptr, nullptr) == NVFP4_ESHAPE);
    EXPECT(launched_or_ok(nvfp4_gemm_w4a4_lora(&a, &w, F, F, 32, 1.0f, F, 1, nullptr, nullptr)));
    EXPECT(nvfp4_gemm_w4a4_lora(&a, &w, F, F, 24, 1.0f, F, 1, nullptr, nullptr) == NVFP4_EINVAL);
    EXPECT(launched_or_ok(nvfp4_lora_down(F, F, 100, 256, 64, F, nullptr)));
    EXPECT(nvfp4_lora_down(F, F, 100, 48, 64, F, nullptr) == NVFP4_ESHAPE);
    EXPECT(launched_or_ok(nvfp4_mx_quantize(F, 1, 64, 256, FB, FB, nullptr)));
    EXPECT(nvfp4_mx_quantize(F, 1, 64, 48, FB, FB, nullptr) == NVFP4_ESHAPE);
    EXPECT(launched_or_ok(nvfp4_gemm_mx(FB, FB, FB, FB, 64, 32, 512, F, 1, nullptr)));
    for (int64_t m = 0; m < 9000; m += 137)
        for (int32_t cus : {1, 7, 256}) {
            int64_t r = -1, wg = -1;
            EXPECT(nvfp4_gemm_plan(m, 3072, cus, &r, &wg) == NVFP4_OK);
            EXPECT((r == m || r % 256 == 0) && r <= m && wg >= 0);
            EXPECT(wg == ((r + 255) / 256 + (m - r + 191) / 192) * 16);
        }
    {
        int64_t r, wg;
        EXPECT(nvfp4_gemm_plan(-1, 1, 1, &r, &wg) == NVFP4_EINVAL);
        EXPECT(nvfp4_gemm_plan(1, 1, 0, &r, &wg) == NVFP4_EINVAL);
    }
    EXPECT(nvfp4_gemm_mx(FB, FB, FB, FB, 64, 32, 500, F, 1, nullptr) == NVFP4_ESHAPE);

    // KV ring: many small configurations, the plan checked against brute force
    uint64_t rng = 12345;
    auto next = [&](int n) {
        rng = rng * 6364136223846793005ull + 1442695040888963407ull;
        return (int)((rng >> 33) % (uint64_t)n);
    };
    for (int trial = 0; trial < 300; ++trial) {
        nvfp4_kv_config c{};
        c.tokens_per_frame = 1 + next(20);
        c.frames_per_chunk = 1 + next(6);
        c.heads = 1 + next(3);
        c.head_dim = 16 * (1 + next(8));
        c.sink_frames_global = next(c.frames_per_chunk + 1);
        c.sink_frames_shot = next(c.frames_per_chunk + 1);
        c.window_chunks = 1 + next(NVFP4_KV_MAX_WINDOW);
        c.search = next(2);
        const size_t bytes = nvfp4_kv_ring_bytes(&c);
        EXPECT(bytes > 0);
        nvfp4_kv_ring r{};
        EXPECT(nvfp4_kv_ring_init(&r, &c, F, bytes) == NVFP4_OK);
        const int64_t Tc = (int64_t)c.tokens_per_frame * c.frames_per_chunk;
        int64_t shot = 0;
        for (int64_t t = 0; t < 3 * c.window_chunks + 4; ++t) {
            if (next(4) == 0 && t > 0) {
                EXPECT(nvfp4_kv_begin_shot(&r, t) == NVFP4_OK);
                shot = t;
            }
            int64_t n = -1;
            EXPECT(nvfp4_kv_effective_tokens(&r, t, &n) == NVFP4_OK);
            std::set<int64_t> e;
            const int64_t g = (int64_t)c.sink_frames_global * c.tokens_per_frame;
            const int64_t s = (int64_t)c.sink_frames_shot * c.tokens_per_frame;
            const int64_t lo = (t > c.window_chunks ? t - c.window_chunks : 0) * Tc;
            for (int64_t j = 0; j < t * Tc; ++j)
                if (j < g || (j >= shot * Tc && j < shot * Tc + s) || j >= lo) e.insert(j);
            EXPECT(n == (int64_t)e.size());
            int64_t got = -1;
            if (n > 0) EXPECT(nvfp4_gather_window(&r, t, F, F, n - 1, &got, nullptr) == NVFP4_ENOSPC);
            EXPECT(launched_or_ok(nvfp4_gather_window(&r, t, F, F, n, &got, nullptr)) && got == n);
            if (c.head_dim == 128) {
                int32_t sp = 0;
                size_t wsb = 0;
                EXPECT(nvfp4_attention_plan(&r, t, 300, 3, &sp, &wsb) == NVFP4_OK && sp == 3);
                EXPECT(launched_or_ok(nvfp4_attention_window(&r, t, F, 300, 0.1f, F, nullptr, 3,
                                                             F, wsb, nullptr)));
            }
            const size_t kws = nvfp4_kv_store_workspace_bytes(&c);
            EXPECT(nvfp4_kv_store_chunk(&r, t + 1, F, F, nullptr, F, kws, nullptr) == NVFP4_ESTATE);
            EXPECT(nvfp4_kv_store_chunk(&r, t, F, F, nullptr, F, kws - 1, nullptr) == NVFP4_ENOSPC);
            const int st = nvfp4_kv_store_chunk(&r, t, F, F, nullptr, F, kws, nullptr);
            EXPECT(launched_or_ok(st));
            r.next_chunk = t + 1;  // the launch failed without a GPU: advance by hand
        }
    }
    nvfp4_kv_config big{1, 1, 129, 128, 0, 0, 1, 1};
    nvfp4_kv_ring rb{};
    EXPECT(nvfp4_kv_ring_init(&rb, &big, F, 1ull << 40) == NVFP4_OK);
    EXPECT(nvfp4_kv_store_chunk_noalloc(&rb, 0, F, F, nullptr, nullptr) == NVFP4_ENOSPC);
    nvfp4_kv_config badc{880, 8, 24, 40, 3, 3, 4, 1};
    EXPECT(nvfp4_kv_ring_bytes(&badc) == 0);
    EXPECT(nvfp4_kv_ring_init(&rb, &badc, F, 1ull << 40) == NVFP4_ESHAPE);
    EXPECT(nvfp4_profile_enable(1) == NVFP4_OK && nvfp4_profile_enable(0) == NVFP4_OK);
    if (failures) return 1;
    std::puts("abi ok");
    return 0;
}
