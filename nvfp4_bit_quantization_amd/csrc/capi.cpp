// capi.cpp -- the C ABI of libnvfp4 (declared in include/nvfp4.h).
//
// Host side only: argument validation (before anything is enqueued), ring
// bookkeeping of the multi-shot sink's two scalar pointers, planning of the
// effective set, and kernel launches on the caller's stream.  No call
// allocates device memory or synchronises the host.
#include "../../include/nvfp4.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return NVFP4_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

int check_tensor(const nvfp4_tensor *t, const char *name) {
    if (!t) return fail(NVFP4_EINVAL, "%s: NULL tensor", name);
    if (t->layout != NVFP4_LAYOUT_1D && t->layout != NVFP4_LAYOUT_2D)
        return fail(NVFP4_EINVAL, "%s: layout %d is neither 1-D nor 2-D", name, t->layout);
    if (t->rows < 0 || t->cols < 0)
        return fail(NVFP4_ESHAPE, "%s: negative shape [%lld, %lld]", name, (long long)t->rows,
                    (long long)t->cols);
    if (t->cols % 16)
        return fail(NVFP4_ESHAPE, "%s: cols %lld not a multiple of 16", name, (long long)t->cols);
    if (t->layout == NVFP4_LAYOUT_2D && t->rows % 16)
        return fail(NVFP4_ESHAPE, "%s: 2-D layout needs rows %% 16 == 0, got %lld", name,
                    (long long)t->rows);
    if (!t->s_dec) return fail(NVFP4_EINVAL, "%s: NULL s_dec", name);
    if (t->rows * t->cols > 0 && (!t->codes || !t->scales))
        return fail(NVFP4_EINVAL, "%s: NULL codes or scales", name);
    if (!aligned16(t->codes) || !aligned16(t->scales) || ((uintptr_t)t->s_dec & 3u))
        return fail(NVFP4_EALIGN, "%s: codes/scales must be 16-byte aligned", name);
    return NVFP4_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(NVFP4_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// ---- KV ring layout ---------------------------------------------------------

struct RegionLayout {
    int64_t kc, ks, vc, vs, mu, sd, bytes;
};

RegionLayout region_layout(int64_t tokens, int64_t hd) {
    RegionLayout r;
    int64_t o = 0;
    r.kc = o;
    o += align256(tokens * hd / 2);
    r.ks = o;
    o += align256(tokens * hd / 16);
    r.vc = o;
    o += align256(tokens * hd / 2);
    r.vs = o;
    o += align256(tokens * hd / 16);
    r.mu = o;
    o += align256(hd * 4);
    r.sd = o;
    o += 256;
    r.bytes = o;
    return r;
}

int check_kv_config(const nvfp4_kv_config *c) {
    if (!c) return fail(NVFP4_EINVAL, "NULL kv config");
    if (c->tokens_per_frame < 1 || c->frames_per_chunk < 1 || c->heads < 1 || c->head_dim < 16)
        return fail(NVFP4_EINVAL, "kv config: sizes must be positive (head_dim >= 16)");
    if (c->head_dim % 16) return fail(NVFP4_ESHAPE, "kv config: head_dim %% 16 != 0");
    if (c->sink_frames_global < 0 || c->sink_frames_global > c->frames_per_chunk ||
        c->sink_frames_shot < 0 || c->sink_frames_shot > c->frames_per_chunk)
        return fail(NVFP4_EINVAL, "kv config: sink frames must lie in [0, frames_per_chunk]");
    if (c->window_chunks < 1 || c->window_chunks > NVFP4_KV_MAX_WINDOW)
        return fail(NVFP4_EINVAL, "kv config: window_chunks must lie in [1, %d]",
                    NVFP4_KV_MAX_WINDOW);
    if (c->search != NVFP4_SEARCH_6 && c->search != NVFP4_SEARCH_4O6)
        return fail(NVFP4_EINVAL, "kv config: bad search %d", c->search);
    const int64_t T = (int64_t)c->tokens_per_frame * c->frames_per_chunk;
    const int64_t hd = (int64_t)c->heads * c->head_dim;
    if (T * hd >= ((int64_t)1 << 31) || T > 65536)
        return fail(NVFP4_ESHAPE, "kv config: a chunk of %lld tokens x %lld channels is too large",
                    (long long)T, (long long)hd);
    return NVFP4_OK;
}

nvfp4::KvRegion region_at(uint8_t *base, const RegionLayout &L) {
    nvfp4::KvRegion r;
    r.kc = base + L.kc;
    r.ks = base + L.ks;
    r.vc = base + L.vc;
    r.vs = base + L.vs;
    r.mu = (float *)(base + L.mu);
    r.sd = (float *)(base + L.sd);
    return r;
}

struct Plan {
    int64_t n_g, n_s, c_lo, nwin, total;
};

// K_eff(t) = (A_g u A_s u [max(0, t-W)*Tc, t*Tc)) n [0, t*Tc): the sinks lie
// at the start of their chunks, so a sink either sits inside the window
// (served from the ring slot) or entirely below it (served from its copy).
Plan plan_effective(const nvfp4_kv_ring *r, int64_t t) {
    const int64_t Tc = r->chunk_tokens, W = r->cfg.window_chunks;
    Plan p;
    p.c_lo = t - W > 0 ? t - W : 0;
    p.nwin = t - p.c_lo;
    const int64_t win_lo = p.c_lo * Tc, hi = t * Tc;
    const int64_t g_end = r->g_end < hi ? r->g_end : hi;
    // global sink part below the window
    p.n_g = 0;
    if (g_end > 0 && win_lo > 0) p.n_g = g_end < win_lo ? g_end : win_lo;
    // shot sink part below the window, minus overlap with the global sink
    p.n_s = 0;
    const int64_t s_lo = r->s_start;
    int64_t s_hi = r->s_start + (int64_t)r->cfg.sink_frames_shot * r->cfg.tokens_per_frame;
    if (s_hi > hi) s_hi = hi;
    if (s_hi > win_lo) s_hi = win_lo;
    int64_t lo = s_lo > p.n_g ? s_lo : p.n_g;
    if (s_hi > lo) p.n_s = s_hi - lo;
    p.total = p.n_g + p.n_s + p.nwin * Tc;
    return p;
}

// K_eff(t) as segments (ascending token order): the global sink's part
// below the window, the shot sink's part below the window and above the
// global sink (its copy starts at the shot's first token, so that many
// leading tokens are skipped), then the window chunks, oldest first.
int effective_segments(const nvfp4_kv_ring *r, const Plan &p, nvfp4::KvSeg *seg) {
    const nvfp4_kv_config &c = r->cfg;
    const int64_t T = r->chunk_tokens, hd = r->hd;
    int ns = 0;
    auto add = [&](const nvfp4::KvRegion &g, int64_t skip, int64_t n) {
        nvfp4::KvSeg &s = seg[ns++];
        s.kc = g.kc + skip * hd / 2;
        s.ks = g.ks + skip * hd / 16;
        s.vc = g.vc + skip * hd / 2;
        s.vs = g.vs + skip * hd / 16;
        s.mu = g.mu;
        s.sd = g.sd;
        s.n = n;
    };
    if (p.n_g > 0)
        add(region_at(r->base + r->gsink_offset,
                      region_layout((int64_t)c.sink_frames_global * c.tokens_per_frame, hd)),
            0, p.n_g);
    if (p.n_s > 0) {
        const int64_t skip = (r->s_start > p.n_g ? r->s_start : p.n_g) - r->s_start;
        add(region_at(r->base + r->ssink_offset,
                      region_layout((int64_t)c.sink_frames_shot * c.tokens_per_frame, hd)),
            skip, p.n_s);
    }
    for (int64_t w = 0; w < p.nwin; ++w)
        add(region_at(r->base + ((p.c_lo + w) % c.window_chunks) * r->slot_bytes,
                      region_layout(T, hd)),
            0, T);
    return ns;
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

#ifndef NVFP4_BUILD_HASH
#define NVFP4_BUILD_HASH "unknown"
#endif
const char *nvfp4_build_hash(void) { return NVFP4_BUILD_HASH; }

const char *nvfp4_status_string(int status) {
    switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_EINVAL: return "invalid argument";
    case NVFP4_EALIGN: return "misaligned device pointer";
    case NVFP4_ESHAPE: return "bad shape";
    case NVFP4_ENOSPC: return "buffer too small";
    case NVFP4_ESTATE: return "KV ring used out of order";
    case NVFP4_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *nvfp4_last_error(void) { return g_err; }

size_t nvfp4_codes_bytes(int64_t rows, int64_t cols) {
    return (rows < 0 || cols < 0) ? 0 : (size_t)(rows * cols / 2);
}

size_t nvfp4_scales_bytes(int64_t rows, int64_t cols, int32_t layout) {
    if (rows < 0 || cols < 0) return 0;
    return layout == NVFP4_LAYOUT_2D ? (size_t)((rows / 16) * (cols / 16))
                                     : (size_t)(rows * (cols / 16));
}

size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols, int32_t layout) {
    (void)layout;
    if (rows < 0 || cols < 0) return 0;
    return (size_t)nvfp4::kMaxPartials * sizeof(float);
}

int nvfp4_quantize(const void *x, int32_t x_dtype, const nvfp4_tensor *out, int32_t search,
                   const float *amax_in, void *workspace, size_t workspace_bytes,
                   void *stream) {
    int st = check_tensor(out, "quantize out");
    if (st) return st;
    if (x_dtype != NVFP4_DTYPE_F32 && x_dtype != NVFP4_DTYPE_BF16)
        return fail(NVFP4_EINVAL, "quantize: bad x dtype %d", x_dtype);
    if (search != NVFP4_SEARCH_6 && search != NVFP4_SEARCH_4O6)
        return fail(NVFP4_EINVAL, "quantize: bad search %d", search);
    const int64_t n = out->rows * out->cols;
    if (n > 0 && !x) return fail(NVFP4_EINVAL, "quantize: NULL x");
    if (!aligned16(x)) return fail(NVFP4_EALIGN, "quantize: x not 16-byte aligned");
    if (((uintptr_t)amax_in & 3u)) return fail(NVFP4_EALIGN, "quantize: amax_in misaligned");
    const size_t need = nvfp4_quantize_workspace_bytes(out->rows, out->cols, out->layout);
    if (!amax_in && (!workspace || workspace_bytes < need))
        return fail(NVFP4_ENOSPC, "quantize: workspace %zu < %zu bytes", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(NVFP4_EALIGN, "quantize: workspace misaligned");
    hipStream_t s = (hipStream_t)stream;
    float *partials = (float *)workspace;
    int np = 0;
    if (!amax_in) {
        np = nvfp4::amax_partials_for(n);
        hipError_t e = nvfp4::launch_amax(x, x_dtype, n, partials, np, s);
        if (e != hipSuccess) return hip_status(e, "quantize amax launch");
    }
    hipError_t e = nvfp4::launch_encode(x, x_dtype, out->rows, out->cols, out->layout, search,
                                        partials, np, amax_in, out->codes, out->scales,
                                        out->s_dec, s);
    return hip_status(e, "quantize encode launch");
}

int nvfp4_quantize_rht(const void *x, int32_t x_dtype, const nvfp4_tensor *out, int32_t search,
                       uint32_t signs, const float *amax_in, void *workspace,
                       size_t workspace_bytes, void *stream) {
    int st = check_tensor(out, "quantize_rht out");
    if (st) return st;
    if (out->layout != NVFP4_LAYOUT_1D)
        return fail(NVFP4_EINVAL, "quantize_rht: the transform is along rows: 1-D layout only");
    if (x_dtype != NVFP4_DTYPE_F32 && x_dtype != NVFP4_DTYPE_BF16)
        return fail(NVFP4_EINVAL, "quantize_rht: bad x dtype %d", x_dtype);
    if (search != NVFP4_SEARCH_6 && search != NVFP4_SEARCH_4O6)
        return fail(NVFP4_EINVAL, "quantize_rht: bad search %d", search);
    if (signs > 0xFFFFu) return fail(NVFP4_EINVAL, "quantize_rht: signs is a 16-bit mask");
    const int64_t n = out->rows * out->cols;
    if (n > 0 && !x) return fail(NVFP4_EINVAL, "quantize_rht: NULL x");
    if (!aligned16(x)) return fail(NVFP4_EALIGN, "quantize_rht: x not 16-byte aligned");
    if (((uintptr_t)amax_in & 3u)) return fail(NVFP4_EALIGN, "quantize_rht: amax_in misaligned");
    const size_t need = nvfp4_quantize_workspace_bytes(out->rows, out->cols, out->layout);
    if (!amax_in && (!workspace || workspace_bytes < need))
        return fail(NVFP4_ENOSPC, "quantize_rht: workspace %zu < %zu bytes", workspace_bytes,
                    need);
    if (!aligned16(workspace)) return fail(NVFP4_EALIGN, "quantize_rht: workspace misaligned");
    hipError_t e = nvfp4::launch_quantize_rht(x, x_dtype, out->rows, out->cols, search, signs,
                                              (float *)workspace, amax_in, out->codes,
                                              out->scales, out->s_dec, (hipStream_t)stream);
    return hip_status(e, "quantize_rht launch");
}

int nvfp4_dequantize(const nvfp4_tensor *in, void *y, int32_t y_dtype, void *stream) {
    int st = check_tensor(in, "dequantize in");
    if (st) return st;
    if (y_dtype != NVFP4_DTYPE_F32 && y_dtype != NVFP4_DTYPE_BF16)
        return fail(NVFP4_EINVAL, "dequantize: bad y dtype %d", y_dtype);
    const int64_t n = in->rows * in->cols;
    if (n > 0 && !y) return fail(NVFP4_EINVAL, "dequantize: NULL y");
    if (!aligned16(y)) return fail(NVFP4_EALIGN, "dequantize: y not 16-byte aligned");
    if (n == 0) return ok();
    hipError_t e = nvfp4::launch_dequant(in->codes, in->scales, in->s_dec, in->rows, in->cols,
                                         in->layout, y, y_dtype, (hipStream_t)stream);
    return hip_status(e, "dequantize launch");
}

static int check_gemm(const nvfp4_tensor *a, const nvfp4_tensor *w, const void *y,
                      int32_t y_dtype, const float *amax_out) {
    int st = check_tensor(a, "gemm A");
    if (st) return st;
    st = check_tensor(w, "gemm W");
    if (st) return st;
    if (a->layout != NVFP4_LAYOUT_1D)
        return fail(NVFP4_EINVAL, "gemm: A must use 1-D (1x16) block scaling");
    if (w->layout != NVFP4_LAYOUT_2D && w->layout != NVFP4_LAYOUT_1D)
        return fail(NVFP4_EINVAL, "gemm: bad W layout %d", w->layout);
    if (a->cols != w->cols)
        return fail(NVFP4_ESHAPE, "gemm: K mismatch (A has %lld, W has %lld)",
                    (long long)a->cols, (long long)w->cols);
    if (y_dtype != NVFP4_DTYPE_F32 && y_dtype != NVFP4_DTYPE_BF16)
        return fail(NVFP4_EINVAL, "gemm: bad y dtype %d", y_dtype);
    if (a->rows * w->rows > 0 && !y) return fail(NVFP4_EINVAL, "gemm: NULL y");
    if (!aligned16(y)) return fail(NVFP4_EALIGN, "gemm: y not 16-byte aligned");
    if (((uintptr_t)amax_out & 3u)) return fail(NVFP4_EALIGN, "gemm: amax_out misaligned");
    return NVFP4_OK;
}

static bool lora_rank_ok(int64_t r) { return r == 16 || r == 32 || r == 64 || r == 128; }

int nvfp4_gemm_w4a4(const nvfp4_tensor *a, const nvfp4_tensor *w, void *y, int32_t y_dtype,
                    float *amax_out, void *stream) {
    int st = check_gemm(a, w, y, y_dtype, amax_out);
    if (st) return st;
    hipError_t e = nvfp4::launch_gemm_w4a4(a->codes, a->scales, a->s_dec, w->codes, w->scales,
                                           w->s_dec, a->rows, w->rows, a->cols, w->layout, y,
                                           y_dtype, amax_out, nullptr, nullptr, 0, 0.0f,
                                           nullptr, (hipStream_t)stream);
    return hip_status(e, "gemm launch");
}

int nvfp4_gemm_w4a4_quant(const nvfp4_tensor *a, const nvfp4_tensor *w, const nvfp4_tensor *y,
                          int32_t search, const float *amax_in, float *amax_out, void *stream) {
    int st = check_tensor(y, "gemm_quant Y");
    if (st) return st;
    if (y->layout != NVFP4_LAYOUT_1D)
        return fail(NVFP4_EINVAL, "gemm_quant: Y must use 1-D (1x16) block scaling");
    st = check_gemm(a, w, y->codes, NVFP4_DTYPE_BF16, amax_out);
    if (st) return st;
    if (y->rows != a->rows || y->cols != w->rows)
        return fail(NVFP4_ESHAPE, "gemm_quant: Y is [%lld, %lld], the product [%lld, %lld]",
                    (long long)y->rows, (long long)y->cols, (long long)a->rows,
                    (long long)w->rows);
    if (search != NVFP4_SEARCH_6 && search != NVFP4_SEARCH_4O6)
        return fail(NVFP4_EINVAL, "gemm_quant: bad search %d", search);
    if (!amax_in) return fail(NVFP4_EINVAL, "gemm_quant: NULL amax_in");
    if (((uintptr_t)amax_in & 3u)) return fail(NVFP4_EALIGN, "gemm_quant: amax_in misaligned");
    const nvfp4::QuantOut q{y->codes, y->scales, y->s_dec, amax_in, search == NVFP4_SEARCH_4O6};
    hipError_t e = nvfp4::launch_gemm_w4a4(a->codes, a->scales, a->s_dec, w->codes, w->scales,
                                           w->s_dec, a->rows, w->rows, a->cols, w->layout,
                                           nullptr, NVFP4_DTYPE_BF16, amax_out, nullptr, nullptr,
                                           0, 0.0f, &q, (hipStream_t)stream);
    return hip_status(e, "gemm_quant launch");
}

int nvfp4_gemm_w4a4_lora(const nvfp4_tensor *a, const nvfp4_tensor *w, const void *xa_bf16,
                         const void *b_bf16, int64_t r, float lora_scale, void *y,
                         int32_t y_dtype, float *amax_out, void *stream) {
    int st = check_gemm(a, w, y, y_dtype, amax_out);
    if (st) return st;
    if (!lora_rank_ok(r)) return fail(NVFP4_EINVAL, "gemm_lora: r must be 16, 32, 64 or 128");
    if (a->rows * w->rows > 0 && (!xa_bf16 || !b_bf16))
        return fail(NVFP4_EINVAL, "gemm_lora: NULL xa or b");
    if (!aligned16(xa_bf16) || !aligned16(b_bf16))
        return fail(NVFP4_EALIGN, "gemm_lora: xa and b must be 16-byte aligned");
    hipError_t e = nvfp4::launch_gemm_w4a4(
        a->codes, a->scales, a->s_dec, w->codes, w->scales, w->s_dec, a->rows, w->rows, a->cols,
        w->layout, y, y_dtype, amax_out, (const uint16_t *)xa_bf16, (const uint16_t *)b_bf16, r,
        lora_scale, nullptr, (hipStream_t)stream);
    return hip_status(e, "gemm_lora launch");
}

int nvfp4_lora_down(const void *x_bf16, const void *a_bf16, int64_t M, int64_t K, int64_t r,
                    void *xa_bf16, void *stream) {
    if (M < 0 || K <= 0) return fail(NVFP4_ESHAPE, "lora_down: bad shape");
    if (K % 32) return fail(NVFP4_ESHAPE, "lora_down: K %% 32 != 0 (got %lld)", (long long)K);
    if (!lora_rank_ok(r)) return fail(NVFP4_EINVAL, "lora_down: r must be 16, 32, 64 or 128");
    if (M == 0) return ok();
    if (!x_bf16 || !a_bf16 || !xa_bf16) return fail(NVFP4_EINVAL, "lora_down: NULL pointer");
    if (!aligned16(x_bf16) || !aligned16(a_bf16) || !aligned16(xa_bf16))
        return fail(NVFP4_EALIGN, "lora_down: pointers must be 16-byte aligned");
    hipError_t e = nvfp4::launch_lora_down((const uint16_t *)x_bf16, (const uint16_t *)a_bf16, M,
                                           K, r, (uint16_t *)xa_bf16, (hipStream_t)stream);
    return hip_status(e, "lora_down launch");
}

// ---- MXFP4 speed reference ------------------------------------------------------

int nvfp4_mx_quantize(const void *x, int32_t x_dtype, int64_t rows, int64_t cols,
                      uint8_t *codes, uint8_t *scales, void *stream) {
    if (rows < 0 || cols < 0) return fail(NVFP4_ESHAPE, "mx_quantize: negative shape");
    if (cols % 32) return fail(NVFP4_ESHAPE, "mx_quantize: cols %% 32 != 0 (got %lld)",
                               (long long)cols);
    if (x_dtype != NVFP4_DTYPE_F32 && x_dtype != NVFP4_DTYPE_BF16)
        return fail(NVFP4_EINVAL, "mx_quantize: bad x dtype %d", x_dtype);
    if (rows * cols == 0) return ok();
    if (!x || !codes || !scales) return fail(NVFP4_EINVAL, "mx_quantize: NULL pointer");
    if (!aligned16(x) || !aligned16(codes))
        return fail(NVFP4_EALIGN, "mx_quantize: x and codes must be 16-byte aligned");
    hipError_t e = nvfp4::launch_mx_quantize(x, x_dtype, rows, cols, codes, scales,
                                             (hipStream_t)stream);
    return hip_status(e, "mx_quantize launch");
}

int nvfp4_gemm_mx(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_codes,
                  const uint8_t *w_scales, int64_t M, int64_t N, int64_t K, void *y,
                  int32_t y_dtype, void *stream) {
    if (M < 0 || N < 0 || K <= 0) return fail(NVFP4_ESHAPE, "gemm_mx: bad shape");
    if (K % 256) return fail(NVFP4_ESHAPE, "gemm_mx: K %% 256 != 0 (got %lld)", (long long)K);
    if (M * (K / 2) >= ((int64_t)1 << 31) || N * (K / 2) >= ((int64_t)1 << 31))
        return fail(NVFP4_ESHAPE, "gemm_mx: code arrays must stay below 2^31 bytes");
    if (y_dtype != NVFP4_DTYPE_F32 && y_dtype != NVFP4_DTYPE_BF16)
        return fail(NVFP4_EINVAL, "gemm_mx: bad y dtype %d", y_dtype);
    if (M * N == 0) return ok();
    if (!a_codes || !a_scales || !w_codes || !w_scales || !y)
        return fail(NVFP4_EINVAL, "gemm_mx: NULL pointer");
    if (!aligned16(a_codes) || !aligned16(w_codes) || !aligned16(y) || !aligned16(a_scales) ||
        !aligned16(w_scales))
        return fail(NVFP4_EALIGN, "gemm_mx: device pointers must be 16-byte aligned");
    hipError_t e = nvfp4::launch_gemm_mx(a_codes, a_scales, w_codes, w_scales, M, N, K, y,
                                         y_dtype, (hipStream_t)stream);
    return hip_status(e, "gemm_mx launch");
}

// ---- KV ring ------------------------------------------------------------------

size_t nvfp4_kv_ring_bytes(const nvfp4_kv_config *cfg) {
    if (check_kv_config(cfg)) return 0;
    const int64_t T = (int64_t)cfg->tokens_per_frame * cfg->frames_per_chunk;
    const int64_t hd = (int64_t)cfg->heads * cfg->head_dim;
    const int64_t g = (int64_t)cfg->sink_frames_global * cfg->tokens_per_frame;
    const int64_t sh = (int64_t)cfg->sink_frames_shot * cfg->tokens_per_frame;
    return (size_t)(cfg->window_chunks * region_layout(T, hd).bytes +
                    region_layout(g, hd).bytes + region_layout(sh, hd).bytes);
}

size_t nvfp4_kv_store_workspace_bytes(const nvfp4_kv_config *cfg) {
    if (check_kv_config(cfg)) return 0;
    const int64_t T = (int64_t)cfg->tokens_per_frame * cfg->frames_per_chunk;
    const int64_t hd = (int64_t)cfg->heads * cfg->head_dim;
    return nvfp4::kv_store_ws_bytes(T, hd);
}

int nvfp4_kv_ring_init(nvfp4_kv_ring *ring, const nvfp4_kv_config *cfg, void *dev_mem,
                       size_t bytes) {
    if (!ring) return fail(NVFP4_EINVAL, "kv_ring_init: NULL ring");
    int st = check_kv_config(cfg);
    if (st) return st;
    if (!dev_mem) return fail(NVFP4_EINVAL, "kv_ring_init: NULL device memory");
    if (((uintptr_t)dev_mem & 255u))
        return fail(NVFP4_EALIGN, "kv_ring_init: device memory must be 256-byte aligned");
    const size_t need = nvfp4_kv_ring_bytes(cfg);
    if (bytes < need) return fail(NVFP4_ENOSPC, "kv_ring_init: %zu < %zu bytes", bytes, need);
    memset(ring, 0, sizeof(*ring));
    ring->cfg = *cfg;
    ring->base = (uint8_t *)dev_mem;
    ring->bytes = bytes;
    ring->chunk_tokens = (int64_t)cfg->tokens_per_frame * cfg->frames_per_chunk;
    ring->hd = (int64_t)cfg->heads * cfg->head_dim;
    ring->slot_bytes = region_layout(ring->chunk_tokens, ring->hd).bytes;
    ring->gsink_offset = cfg->window_chunks * ring->slot_bytes;
    ring->ssink_offset =
        ring->gsink_offset +
        region_layout((int64_t)cfg->sink_frames_global * cfg->tokens_per_frame, ring->hd).bytes;
    ring->next_chunk = 0;
    ring->g_end = (int64_t)cfg->sink_frames_global * cfg->tokens_per_frame;
    ring->s_start = 0;
    return ok();
}

static int check_ring(const nvfp4_kv_ring *r) {
    if (!r || !r->base) return fail(NVFP4_EINVAL, "NULL or uninitialised ring");
    return check_kv_config(&r->cfg);
}

int nvfp4_kv_begin_shot(nvfp4_kv_ring *ring, int64_t chunk_idx) {
    int st = check_ring(ring);
    if (st) return st;
    if (chunk_idx != ring->next_chunk)
        return fail(NVFP4_ESTATE, "kv_begin_shot: chunk %lld is not the next chunk (%lld)",
                    (long long)chunk_idx, (long long)ring->next_chunk);
    ring->s_start = chunk_idx * ring->chunk_tokens;
    return ok();
}

static_assert(NVFP4_KV_NOALLOC_MAX_CHANNELS == 16384, "allocation-free store limit");

static int kv_store(nvfp4_kv_ring *ring, int64_t chunk_idx, const void *K_bf16,
                    const void *V_bf16, const float *v_amax_in, void *workspace,
                    size_t workspace_bytes, void *stream, bool noalloc) {
    const char *who = noalloc ? "kv_store_chunk_noalloc" : "kv_store_chunk";
    int st = check_ring(ring);
    if (st) return st;
    if (chunk_idx != ring->next_chunk)
        return fail(NVFP4_ESTATE, "%s: chunk %lld stored out of order (next %lld)", who,
                    (long long)chunk_idx, (long long)ring->next_chunk);
    if (!K_bf16 || !V_bf16) return fail(NVFP4_EINVAL, "%s: NULL K or V", who);
    if (!aligned16(K_bf16) || !aligned16(V_bf16))
        return fail(NVFP4_EALIGN, "%s: K and V must be 16-byte aligned", who);
    if ((uintptr_t)v_amax_in & 3u) return fail(NVFP4_EALIGN, "%s: v_amax_in misaligned", who);
    const size_t need = nvfp4_kv_store_workspace_bytes(&ring->cfg);
    if (noalloc) {
        if (ring->hd > nvfp4::kv_noalloc_max_hd())
            return fail(NVFP4_ENOSPC,
                        "%s: heads * head_dim = %lld exceeds the %lld channels its fixed scratch "
                        "holds (use nvfp4_kv_store_chunk with a workspace)",
                        who, (long long)ring->hd, (long long)nvfp4::kv_noalloc_max_hd());
        hipError_t e = nvfp4::kv_noalloc_scratch(&workspace, &workspace_bytes, (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e, "kv_store_chunk_noalloc scratch");
        if (workspace_bytes < need)
            return fail(NVFP4_ENOSPC, "%s: scratch %zu < %zu bytes", who, workspace_bytes, need);
    } else {
        if (!aligned16(workspace))
            return fail(NVFP4_EALIGN, "%s: workspace must be 16-byte aligned", who);
        if (!workspace || workspace_bytes < need)
            return fail(NVFP4_ENOSPC, "%s: workspace %zu < %zu bytes", who, workspace_bytes,
                        need);
    }
    const nvfp4_kv_config &c = ring->cfg;
    const int64_t T = ring->chunk_tokens, hd = ring->hd;
    const int64_t gtok = (int64_t)c.sink_frames_global * c.tokens_per_frame;
    const int64_t stok = (int64_t)c.sink_frames_shot * c.tokens_per_frame;
    nvfp4::KvStoreArgs a;
    a.K = (const uint16_t *)K_bf16;
    a.V = (const uint16_t *)V_bf16;
    a.T = T;
    a.HD = hd;
    a.search = c.search;
    a.slot = region_at(ring->base + (chunk_idx % c.window_chunks) * ring->slot_bytes,
                       region_layout(T, hd));
    a.gsink = region_at(ring->base + ring->gsink_offset, region_layout(gtok, hd));
    a.ssink = region_at(ring->base + ring->ssink_offset, region_layout(stok, hd));
    a.g_tokens = (chunk_idx == 0) ? gtok : 0;
    a.s_tokens = (chunk_idx * T == ring->s_start) ? stok : 0;
    a.v_amax_in = v_amax_in;
    a.ws = workspace;
    a.clear_ws = (chunk_idx == 0);
    hipError_t e = nvfp4::launch_kv_store(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, noalloc ? "kv_store_chunk_noalloc launch"
                                                      : "kv_store_chunk launch");
    ring->next_chunk = chunk_idx + 1;
    return ok();
}

int nvfp4_kv_store_chunk(nvfp4_kv_ring *ring, int64_t chunk_idx, const void *K_bf16,
                         const void *V_bf16, const float *v_amax_in, void *workspace,
                         size_t workspace_bytes, void *stream) {
    return kv_store(ring, chunk_idx, K_bf16, V_bf16, v_amax_in, workspace, workspace_bytes,
                    stream, false);
}

int nvfp4_kv_store_chunk_noalloc(nvfp4_kv_ring *ring, int64_t chunk_idx, const void *K_bf16,
                                 const void *V_bf16, const float *v_amax_in, void *stream) {
    return kv_store(ring, chunk_idx, K_bf16, V_bf16, v_amax_in, nullptr, 0, stream, true);
}

int nvfp4_kv_effective_tokens(const nvfp4_kv_ring *ring, int64_t step, int64_t *n_tokens) {
    int st = check_ring(ring);
    if (st) return st;
    if (!n_tokens) return fail(NVFP4_EINVAL, "kv_effective_tokens: NULL n_tokens");
    if (step != ring->next_chunk)
        return fail(NVFP4_ESTATE, "kv_effective_tokens: step %lld != next chunk %lld",
                    (long long)step, (long long)ring->next_chunk);
    *n_tokens = plan_effective(ring, step).total;
    return ok();
}

int nvfp4_gather_window(const nvfp4_kv_ring *ring, int64_t step, void *K_out, void *V_out,
                        int64_t capacity_tokens, int64_t *n_tokens, void *stream) {
    int st = check_ring(ring);
    if (st) return st;
    if (step != ring->next_chunk)
        return fail(NVFP4_ESTATE, "gather_window: step %lld != next chunk %lld",
                    (long long)step, (long long)ring->next_chunk);
    const Plan p = plan_effective(ring, step);
    if (n_tokens) *n_tokens = p.total;
    if (p.total > capacity_tokens)
        return fail(NVFP4_ENOSPC, "gather_window: %lld tokens exceed capacity %lld",
                    (long long)p.total, (long long)capacity_tokens);
    if (p.total > 0 && (!K_out || !V_out)) return fail(NVFP4_EINVAL, "gather_window: NULL output");
    if (!aligned16(K_out) || !aligned16(V_out))
        return fail(NVFP4_EALIGN, "gather_window: outputs must be 16-byte aligned");
    nvfp4::GatherArgs a;
    a.nseg = effective_segments(ring, p, a.seg);
    // tokens per workgroup: enough workgroups to fill the chip many times
    // (about 4096), each at least one four-token iteration (measured at
    // 33,440 tokens: 8 a workgroup 141.5 us, 16 143.7, 32 151)
    int64_t tpw = (p.total + 4095) / 4096;
    tpw = tpw < 4 ? 4 : (tpw > 32 ? 32 : (tpw + 3) / 4 * 4);
    a.tpw = (int32_t)tpw;
    a.wg0[0] = 0;
    int64_t out = 0;
    for (int i = 0; i < a.nseg; ++i) {
        a.out0[i] = out;
        out += a.seg[i].n;
        a.wg0[i + 1] = a.wg0[i] + (int32_t)((a.seg[i].n + tpw - 1) / tpw);
    }
    a.HD = ring->hd;
    a.Kout = (uint16_t *)K_out;
    a.Vout = (uint16_t *)V_out;
    hipError_t e = nvfp4::launch_gather(a, (hipStream_t)stream);
    return hip_status(e, "gather_window launch");
}

static_assert(nvfp4::kAttnMaxSplit == NVFP4_ATTN_MAX_SPLITS, "attention key splits");
static_assert(nvfp4::kAttnMaxSeg >= 2 + NVFP4_KV_MAX_WINDOW,
              "attention segments: two sinks and every window chunk");

// Host checks shared by the plan and the call, and the effective set as
// segments (ascending token order, the gather's segments).
static int attn_setup(const nvfp4_kv_ring *ring, int64_t step, int64_t n_q, int32_t key_splits,
                      const char *who, nvfp4::AttnArgs &a) {
    int st = check_ring(ring);
    if (st) return st;
    if (step != ring->next_chunk)
        return fail(NVFP4_ESTATE, "%s: step %lld != next chunk %lld", who, (long long)step,
                    (long long)ring->next_chunk);
    if (ring->cfg.head_dim != 128)
        return fail(NVFP4_ESHAPE, "%s: head_dim must be 128 (got %d)", who, ring->cfg.head_dim);
    if (n_q < 0) return fail(NVFP4_ESHAPE, "%s: negative query count", who);
    if (key_splits < 0 || key_splits > nvfp4::kAttnMaxSplit)
        return fail(NVFP4_EINVAL, "%s: key_splits must be 0 (automatic) or 1..%d (got %d)", who,
                    nvfp4::kAttnMaxSplit, key_splits);
    if ((n_q + 255) / 256 * (int64_t)ring->cfg.heads * nvfp4::kAttnMaxSplit >= ((int64_t)1 << 31))
        return fail(NVFP4_ESHAPE, "%s: too many queries", who);
    const Plan p = plan_effective(ring, step);
    const nvfp4_kv_config &c = ring->cfg;
    const int64_t hd = ring->hd;
    a = nvfp4::AttnArgs{};
    const int ns = effective_segments(ring, p, a.seg);
    a.nseg = ns;
    a.tile0[0] = 0;
    for (int i = 0; i < ns; ++i) a.tile0[i + 1] = a.tile0[i] + (int32_t)((a.seg[i].n + 63) / 64);
    a.heads = c.heads;
    a.HD = hd;
    a.nq = n_q;
    hipError_t e =
        nvfp4::attn_choose_splits(n_q, c.heads, a.tile0[ns], key_splits, &a.nsplit);
    return hip_status(e, "attention: device query");
}

int nvfp4_gemm_plan(int64_t M, int64_t N, int32_t compute_units, int64_t *rows_256,
                    int64_t *workgroups) {
    if (!rows_256 || !workgroups) return fail(NVFP4_EINVAL, "gemm_plan: NULL output");
    if (M < 0 || N < 0 || compute_units < 1)
        return fail(NVFP4_EINVAL, "gemm_plan: M, N must be >= 0 and compute_units >= 1");
    nvfp4::gemm_plan(M, N, compute_units, rows_256, workgroups);
    return ok();
}

int nvfp4_attention_plan(const nvfp4_kv_ring *ring, int64_t step, int64_t n_q, int32_t key_splits,
                         int32_t *splits, size_t *ws_bytes) {
    if (!splits || !ws_bytes) return fail(NVFP4_EINVAL, "attention_plan: NULL output");
    nvfp4::AttnArgs a;
    const int st = attn_setup(ring, step, n_q, key_splits, "attention_plan", a);
    if (st) return st;
    *splits = a.nsplit;
    *ws_bytes = nvfp4::attn_workspace_bytes(n_q, a.heads, a.nsplit);
    return NVFP4_OK;
}

int nvfp4_attention_window(const nvfp4_kv_ring *ring, int64_t step, const void *q_bf16,
                           int64_t n_q, float softmax_scale, void *o_bf16, float *lse,
                           int32_t key_splits, void *ws, size_t ws_bytes, void *stream) {
    if (!(softmax_scale >= 0.0f && softmax_scale <= 3.4e38f))
        return fail(NVFP4_EINVAL, "attention_window: softmax_scale must be finite and >= 0");
    if (n_q > 0 && (!q_bf16 || !o_bf16))
        return fail(NVFP4_EINVAL, "attention_window: NULL q or o");
    if (!aligned16(q_bf16) || !aligned16(o_bf16) || ((uintptr_t)lse & 3u))
        return fail(NVFP4_EALIGN, "attention_window: q and o must be 16-byte aligned, lse 4");
    nvfp4::AttnArgs a;
    const int st = attn_setup(ring, step, n_q, key_splits, "attention_window", a);
    if (st) return st;
    const size_t need = nvfp4::attn_workspace_bytes(n_q, a.heads, a.nsplit);
    if (need > 0) {
        if (!ws || ws_bytes < need)
            return fail(NVFP4_ENOSPC, "attention_window: %d key splits need %zu workspace bytes (got %zu)",
                        a.nsplit, need, ws ? ws_bytes : (size_t)0);
        if ((uintptr_t)ws & 255u)
            return fail(NVFP4_EALIGN, "attention_window: workspace must be 256-byte aligned");
        const size_t rows = (size_t)a.nsplit * (size_t)n_q * (size_t)a.heads;
        a.part_ml = (float *)ws;
        a.part_o = (float *)((uint8_t *)ws + (rows * 8 + 255) / 256 * 256);
    }
    a.q = (const uint16_t *)q_bf16;
    a.o = (uint16_t *)o_bf16;
    a.lse = lse;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    hipError_t e = nvfp4::launch_attn_window(a, (hipStream_t)stream);
    return hip_status(e, "attention_window launch");
}

}  // extern "C"
