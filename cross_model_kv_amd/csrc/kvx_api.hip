// C ABI of libkvx: argument validation (host only, before any GPU work is enqueued), workspace
// sizing and the launch sequence of every entry point declared in include/kvx.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "kvx_internal.h"

using namespace kvx;

namespace {

thread_local std::string g_err;

kvx_status fail(kvx_status code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

kvx_status ok() {
    g_err.clear();
    return KVX_OK;
}

kvx_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(KVX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define KVX_TRY_HIP(expr, what)                              \
    do {                                                     \
        hipError_t e_ = (expr);                              \
        if (e_ != hipSuccess) return hip_status(e_, what);   \
    } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the gathered QKV projection: the K-slice partials of its split tail (bf16 only).
size_t qkv_split_bytes(int32_t dtype, int64_t n_sel, int32_t D, int n_qkv) {
    if (dtype != KVX_BF16 || n_sel == 0 || n_sel > INT32_MAX) return 0;
    return round256(gemm_bf16_split_bytes((int)n_sel, n_qkv, D, 1, EPI_STORE));
}


// KVX_DEBUG set to anything but "" or "0": every call first copies the device-side index data
// it is about to trust (batch prefix arrays, position lists, page tables) to the host and checks
// it.  Read on every call, so a process can switch it on and off.
bool debug_checks() {
    const char* v = getenv("KVX_DEBUG");
    return v && v[0] && v[0] != '0';
}

#define KVX_REQUIRE(cond, ...)                                         \
    do {                                                               \
        if (!(cond)) return fail(KVX_ERR_INVALID, __VA_ARGS__);        \
    } while (0)

#define KVX_REQUIRE_PTR(p, name)                                                        \
    do {                                                                                \
        if (!(p)) return fail(KVX_ERR_INVALID, "%s must not be null", name);            \
        if (!aligned16(p)) return fail(KVX_ERR_INVALID, "%s must be 16-byte aligned", name); \
    } while (0)

kvx_status check_dtype(int32_t dtype) {
    if (dtype != KVX_F32 && dtype != KVX_BF16)
        return fail(KVX_ERR_UNSUPPORTED, "dtype %d is not KVX_F32 (0) or KVX_BF16 (1)", dtype);
    return KVX_OK;
}

size_t elem_size(int32_t dtype) { return dtype == KVX_BF16 ? 2 : 4; }

struct BatchInfo {
    int n_req;
    int64_t n_tokens, n_sel, n_rest;
    int max_T;
};

kvx_status check_batch(const kvx_batch* bt, BatchInfo* out) {
    KVX_REQUIRE(bt, "batch must not be null");
    KVX_REQUIRE(bt->n_req >= 1, "batch.n_req must be >= 1 (got %d)", bt->n_req);
    KVX_REQUIRE(bt->cu_tokens_h && bt->cu_sel_h, "batch host prefix arrays must not be null");
    KVX_REQUIRE(bt->cu_tokens_d && bt->cu_sel_d, "batch device prefix arrays must not be null");
    KVX_REQUIRE(bt->cu_tokens_h[0] == 0 && bt->cu_sel_h[0] == 0, "batch prefix arrays must start at 0");
    int max_T = 0;
    for (int b = 0; b < bt->n_req; ++b) {
        const int T = bt->cu_tokens_h[b + 1] - bt->cu_tokens_h[b];
        const int k = bt->cu_sel_h[b + 1] - bt->cu_sel_h[b];
        KVX_REQUIRE(T >= 0, "batch.cu_tokens must be non-decreasing (request %d)", b);
        KVX_REQUIRE(k >= 0 && k <= T, "request %d selects %d of %d positions", b, k, T);
        if (T > max_T) max_T = T;
    }
    if (debug_checks()) {
        KVX_TRY_HIP(hipDeviceSynchronize(), "debug synchronisation");
        std::vector<int32_t> t(bt->n_req + 1), s(bt->n_req + 1);
        KVX_TRY_HIP(hipMemcpy(t.data(), bt->cu_tokens_d, t.size() * 4, hipMemcpyDeviceToHost), "debug copy");
        KVX_TRY_HIP(hipMemcpy(s.data(), bt->cu_sel_d, s.size() * 4, hipMemcpyDeviceToHost), "debug copy");
        for (int b = 0; b <= bt->n_req; ++b)
            KVX_REQUIRE(t[b] == bt->cu_tokens_h[b] && s[b] == bt->cu_sel_h[b],
                        "batch device prefix arrays differ from the host copies at %d", b);
    }
    out->n_req = bt->n_req;
    out->n_tokens = bt->cu_tokens_h[bt->n_req];
    out->n_sel = bt->cu_sel_h[bt->n_req];
    out->n_rest = out->n_tokens - out->n_sel;
    out->max_T = max_T;
    return KVX_OK;
}

kvx_status check_cache(const kvx_cache* c, const BatchInfo& bi, int32_t dtype, int32_t H_kv,
                       int32_t d_h, int min_layers) {
    KVX_REQUIRE(c, "cache must not be null");
    KVX_REQUIRE(c->layout == KVX_CONTIGUOUS || c->layout == KVX_PAGED, "cache.layout %d is unknown", c->layout);
    KVX_REQUIRE_PTR(c->k, "cache.k");
    KVX_REQUIRE_PTR(c->v, "cache.v");
    KVX_REQUIRE(c->n_layers >= min_layers, "cache.n_layers (%d) must be >= %d", c->n_layers, min_layers);
    if (c->layout == KVX_CONTIGUOUS) {
        KVX_REQUIRE(c->n_slots >= bi.n_tokens, "contiguous cache.n_slots (%lld) < tokens (%lld)",
                    (long long)c->n_slots, (long long)bi.n_tokens);
        return KVX_OK;
    }
    KVX_REQUIRE(c->page_size > 0, "paged cache.page_size must be > 0");
    KVX_REQUIRE(c->page_table, "paged cache.page_table must not be null");
    KVX_REQUIRE(c->n_slots % c->page_size == 0, "paged cache.n_slots must be a multiple of page_size");
    const int need = (bi.max_T + c->page_size - 1) / c->page_size;
    KVX_REQUIRE(c->max_pages >= need, "paged cache.max_pages (%d) < %d pages of the longest request",
                c->max_pages, need);
    (void)dtype; (void)H_kv; (void)d_h;
    return KVX_OK;
}

kvx_status check_page_table_debug(const kvx_cache* c, const kvx_batch* bt) {
    if (!debug_checks() || c->layout != KVX_PAGED) return KVX_OK;
    KVX_TRY_HIP(hipDeviceSynchronize(), "debug synchronisation");
    std::vector<int32_t> pt((size_t)bt->n_req * c->max_pages);
    KVX_TRY_HIP(hipMemcpy(pt.data(), c->page_table, pt.size() * 4, hipMemcpyDeviceToHost), "debug copy");
    const int64_t n_pages = c->n_slots / c->page_size;
    std::vector<char> used((size_t)n_pages, 0);
    for (int b = 0; b < bt->n_req; ++b) {
        const int T = bt->cu_tokens_h[b + 1] - bt->cu_tokens_h[b];
        const int np = (T + c->page_size - 1) / c->page_size;
        for (int i = 0; i < np; ++i) {
            const int32_t p = pt[(size_t)b * c->max_pages + i];
            KVX_REQUIRE(p >= 0 && p < n_pages, "page_table[%d][%d] = %d is outside [0, %lld)", b, i, p,
                        (long long)n_pages);
            KVX_REQUIRE(!used[p], "page %d is mapped twice", p);
            used[p] = 1;
        }
    }
    return KVX_OK;
}

// KVX_DEBUG: a per-request position list (selected positions, or with `rest` the complement
// lists, which start at cu_tokens[b] - cu_sel[b]) must be strictly ascending within each request
// and inside [0, T_b): the kernels index the rotary table, the cache slots and the query blocks'
// key ranges with these values without checking them.
kvx_status check_positions_debug(const int32_t* list, const kvx_batch* bt, bool rest, const char* name) {
    if (!debug_checks() || !list) return KVX_OK;
    const int n_req = bt->n_req;
    const int64_t count = rest ? (int64_t)bt->cu_tokens_h[n_req] - bt->cu_sel_h[n_req] : bt->cu_sel_h[n_req];
    if (count <= 0) return KVX_OK;
    KVX_TRY_HIP(hipDeviceSynchronize(), "debug synchronisation");
    std::vector<int32_t> h((size_t)count);
    KVX_TRY_HIP(hipMemcpy(h.data(), list, h.size() * 4, hipMemcpyDeviceToHost), "debug copy");
    for (int b = 0; b < n_req; ++b) {
        const int T = bt->cu_tokens_h[b + 1] - bt->cu_tokens_h[b];
        const int k = bt->cu_sel_h[b + 1] - bt->cu_sel_h[b];
        const int64_t start = rest ? (int64_t)bt->cu_tokens_h[b] - bt->cu_sel_h[b] : bt->cu_sel_h[b];
        const int n = rest ? T - k : k;
        for (int i = 0; i < n; ++i) {
            const int32_t v = h[(size_t)(start + i)];
            KVX_REQUIRE(v >= 0 && v < T, "%s[%lld] = %d (request %d) is outside [0, %d)", name,
                        (long long)(start + i), v, b, T);
            KVX_REQUIRE(i == 0 || v > h[(size_t)(start + i - 1)],
                        "%s of request %d is not strictly ascending at entry %lld (%d after %d)", name, b,
                        (long long)(start + i), v, h[(size_t)(start + i - 1)]);
        }
    }
    return KVX_OK;
}

SlotMap slot_map(const kvx_cache* c, const kvx_batch* bt) {
    SlotMap s;
    s.cu_tok = bt->cu_tokens_d;
    s.paged = c->layout == KVX_PAGED ? 1 : 0;
    s.page_table = s.paged ? c->page_table : nullptr;
    s.max_pages = s.paged ? c->max_pages : 0;
    s.page_size = s.paged ? c->page_size : 1;
    s.page_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((1 << sh) == s.page_size) s.page_shift = sh;
    return s;
}

int32_t budget_of(int32_t T, int32_t pct) { return (int32_t)(((int64_t)pct * T + 99) / 100); }

// Workspace of the attention's key-range split (bf16; 0 when the batch fills the GPU without it).
size_t attn_split_bytes(int32_t dtype, const kvx_batch* batch, const BatchInfo& bi, int H_q, int H_kv, int d_h) {
    if (dtype != KVX_BF16 || H_kv <= 0 || H_q % H_kv != 0 || bi.n_sel == 0) return 0;
    const int bq = attn_bf16_block_queries(H_q / H_kv);
    if (bq == 0) return 0;
    int64_t n_blocks = 0;
    for (int b = 0; b < bi.n_req; ++b) n_blocks += (batch->cu_sel_h[b + 1] - batch->cu_sel_h[b] + bq - 1) / bq;
    if (n_blocks > INT32_MAX) return 0;
    return attn_bf16_split_bytes(bi.n_sel, H_q, d_h, attn_bf16_split((int)n_blocks, H_kv, bi.max_T));
}

}  // namespace

extern "C" {

const char* kvx_last_error(void) { return g_err.c_str(); }

const char* kvx_version(void) { return "kvx 0.1 (gfx950)"; }

int32_t kvx_budget(int32_t T, int32_t pct) {
    if (T < 0 || pct < 0 || pct > 100) {
        fail(KVX_ERR_INVALID, "kvx_budget: need T >= 0 and 0 <= pct <= 100");
        return -1;
    }
    return budget_of(T, pct);
}

kvx_status kvx_map_latent_workspace(int32_t dtype, int64_t n, int32_t d_src, int32_t r, size_t* bytes) {
    if (kvx_status st = check_dtype(dtype)) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(n >= 0 && n <= INT32_MAX, "n (%lld) must be in [0, 2^31)", (long long)n);
    KVX_REQUIRE(d_src > 0 && r > 0, "d_src (%d) and r (%d) must be positive", d_src, r);
    *bytes = (dtype == KVX_BF16 && n > 0) ? round256(gemm_bf16_split_bytes((int)n, r, d_src, 1, EPI_STORE)) : 0;
    return ok();
}

kvx_status kvx_map_latent(void* stream, int32_t dtype, const void* x_src, const void* w_s, void* z,
                          int64_t n, int32_t d_src, int32_t r, void* ws, size_t ws_bytes) {
    if (kvx_status st = check_dtype(dtype)) return st;
    KVX_REQUIRE_PTR(x_src, "x_src");
    KVX_REQUIRE_PTR(w_s, "w_s");
    KVX_REQUIRE_PTR(z, "z");
    KVX_REQUIRE(n >= 0 && n <= INT32_MAX, "n (%lld) must be in [0, 2^31)", (long long)n);
    KVX_REQUIRE(d_src > 0 && r > 0, "d_src (%d) and r (%d) must be positive", d_src, r);
    if (dtype == KVX_BF16) {
        KVX_REQUIRE(d_src % 64 == 0, "bf16 needs d_src %% 64 == 0 (got %d)", d_src);
        KVX_REQUIRE(r % 8 == 0, "bf16 needs r %% 8 == 0 (got %d)", r);
    }
    if (n == 0) return ok();
    size_t need = 0;
    kvx_map_latent_workspace(dtype, n, d_src, r, &need);
    if (need && (!ws || ws_bytes < need))
        return fail(KVX_ERR_WORKSPACE, "map_latent needs %zu workspace bytes (got %zu)", need, ws_bytes);
    if (need) KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    if (dtype == KVX_BF16) {
        GemmArgs a{};
        a.A = (const bf16*)x_src; a.lda = d_src; a.K_a = d_src;
        a.B = (const bf16*)w_s; a.ldb = d_src; a.b_group_stride = 0;
        a.M = (int)n; a.N = r; a.K = d_src; a.groups = 1;
        a.rows.mode = 0;
        a.epi = EPI_STORE; a.C = (bf16*)z; a.ldc = r;
        a.split_ws = need ? (float*)ws : nullptr;
        return hip_status(launch_gemm_bf16(a, s), "map_latent");
    }
    GemmF32Args a{};
    a.A = (const float*)x_src; a.lda = d_src; a.K_a = d_src;
    a.B = (const float*)w_s; a.ldb = d_src;
    a.M = (int)n; a.N = r; a.K = d_src; a.groups = 1;
    a.rows.mode = 0;
    a.epi = EPI_STORE; a.C = (float*)z; a.ldc = r;
    return hip_status(launch_gemm_f32(a, s), "map_latent");
}

kvx_status kvx_score_prepare_workspace(int32_t r, int32_t d_t, int32_t c, size_t* bytes) {
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(r > 0 && d_t > 0 && c >= 0 && c <= d_t, "need r > 0, d_t > 0, 0 <= c <= d_t");
    *bytes = round256((size_t)c * r * 8) + round256((size_t)d_t * r * 8) + round256((size_t)r * r * 8);
    return ok();
}

kvx_status kvx_score_prepare(void* stream, int32_t dtype, const void* w_l, const float* u, int32_t L_t,
                             int32_t r, int32_t d_t, int32_t c, void* op, void* ws, size_t ws_bytes) {
    if (kvx_status st = check_dtype(dtype)) return st;
    KVX_REQUIRE_PTR(w_l, "w_l");
    KVX_REQUIRE_PTR(op, "op");
    KVX_REQUIRE(L_t > 0 && r > 0 && d_t > 0, "L_t, r and d_t must be positive");
    KVX_REQUIRE(c >= 0 && c <= d_t, "calibration rank c (%d) must be in [0, d_t]", c);
    if (c > 0) KVX_REQUIRE_PTR(u, "u");
    size_t need = 0;
    kvx_score_prepare_workspace(r, d_t, c, &need);
    if (!ws || ws_bytes < need)
        return fail(KVX_ERR_WORKSPACE, "score_prepare needs %zu workspace bytes (got %zu)", need, ws_bytes);
    KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    char* p = (char*)ws;
    double* G = (double*)p; p += round256((size_t)c * r * 8);
    double* R = (double*)p; p += round256((size_t)d_t * r * 8);
    double* A = (double*)p;
    const int tw = dtype == KVX_BF16 ? ET_BF16 : ET_F32;
    const size_t es = elem_size(dtype);
    KVX_TRY_HIP(launch_zero_f64(A, (int64_t)r * r, s), "score_prepare");
    for (int l = 0; l < L_t; ++l) {
        const void* W = (const char*)w_l + (size_t)l * d_t * r * es;     // [d_t][r]
        const float* U = u ? u + (size_t)l * d_t * c : nullptr;          // [d_t][c]
        KVX_TRY_HIP(launch_to_f64(W, tw, R, (int64_t)d_t * r, s), "score_prepare");
        if (c > 0) {
            // G = U^T W  [c][r]
            KVX_TRY_HIP(launch_gemm_f64(c, r, d_t, 1.0, U, ET_F32, 1, c, W, tw, r, 1, G, r, false, s),
                        "score_prepare");
            // R = W - U G  [d_t][r]: the part of every column of W outside span(U)
            KVX_TRY_HIP(launch_gemm_f64(d_t, r, c, -1.0, U, ET_F32, c, 1, G, ET_F64, r, 1, R, r, true, s),
                        "score_prepare");
        }
        // A += R^T R  [r][r]
        KVX_TRY_HIP(launch_gemm_f64(r, r, d_t, 1.0, R, ET_F64, 1, r, R, ET_F64, r, 1, A, r, true, s),
                    "score_prepare");
    }
    return hip_status(launch_pack_operator(A, r, dtype, op, s), "score_prepare");
}

}  // extern "C"

namespace {

kvx_status check_fit_mapper(int32_t dtype, int32_t n, int32_t d_src, int32_t L_t, int32_t d_t, int32_t r) {
    if (kvx_status st = check_dtype(dtype)) return st;
    KVX_REQUIRE(n > 0 && d_src > 0 && L_t > 0 && d_t > 0 && r > 0, "n, d_src, L_t, d_t and r must be positive");
    KVX_REQUIRE((int64_t)L_t * d_t <= INT32_MAX, "L_t * d_t too large");
    const int m = L_t * d_t;
    KVX_REQUIRE(r <= n && r <= d_src && r <= m, "r (%d) must not exceed n (%d), d_src (%d) or L_t * d_t (%d): the "
                "fitted values have at most that rank", r, n, d_src, m);
    if (dtype == KVX_BF16) {
        KVX_REQUIRE(d_src % 64 == 0 && m % 64 == 0, "bf16 needs d_src %% 64 == 0 and L_t * d_t %% 64 == 0");
        KVX_REQUIRE(n % 8 == 0, "bf16 needs n %% 8 == 0 (got %d)", n);
    }
    return KVX_OK;
}

kvx_status check_fit_calibration(int32_t n, int32_t L_t, int32_t d_t, int32_t r, int32_t c) {
    KVX_REQUIRE(n > 0 && L_t > 0 && d_t > 0 && r > 0 && c > 0, "n, L_t, d_t, r and c must be positive");
    KVX_REQUIRE(c <= d_t && c <= r && c <= n, "c (%d) must not exceed d_t (%d), r (%d) or n (%d): the mapped "
                "calibration KV has at most that rank", c, d_t, r, n);
    return KVX_OK;
}

}  // namespace

extern "C" {

kvx_status kvx_fit_mapper_workspace(int32_t dtype, int32_t n, int32_t d_src, int32_t L_t, int32_t d_t, int32_t r,
                                    size_t* bytes) {
    if (kvx_status st = check_fit_mapper(dtype, n, d_src, L_t, d_t, r)) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    *bytes = fit_mapper_bytes(n, d_src, L_t * d_t, r);
    return ok();
}

kvx_status kvx_fit_mapper(void* stream, int32_t dtype, const void* x, const void* y, int32_t n, int32_t d_src,
                          int32_t L_t, int32_t d_t, int32_t r, double lambda, int32_t iters, void* w_s, void* w_l,
                          void* ws, size_t ws_bytes) {
    if (kvx_status st = check_fit_mapper(dtype, n, d_src, L_t, d_t, r)) return st;
    KVX_REQUIRE_PTR(x, "x");
    KVX_REQUIRE_PTR(y, "y");
    KVX_REQUIRE_PTR(w_s, "w_s");
    KVX_REQUIRE_PTR(w_l, "w_l");
    KVX_REQUIRE(lambda > 0.0 && lambda < INFINITY, "lambda must be positive and finite");
    KVX_REQUIRE(iters >= 1 && iters <= 10000, "iters must be in [1, 10000] (got %d)", iters);
    const size_t need = fit_mapper_bytes(n, d_src, L_t * d_t, r);
    if (!ws || ws_bytes < need)
        return fail(KVX_ERR_WORKSPACE, "fit_mapper needs %zu workspace bytes (got %zu)", need, ws_bytes);
    KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    return hip_status(launch_fit_mapper((hipStream_t)stream, dtype, x, y, n, d_src, L_t * d_t, r, lambda, iters, w_s,
                                        w_l, ws),
                      "fit_mapper");
}

kvx_status kvx_fit_calibration_workspace(int32_t n, int32_t L_t, int32_t d_t, int32_t r, int32_t c, size_t* bytes) {
    if (kvx_status st = check_fit_calibration(n, L_t, d_t, r, c)) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    *bytes = fit_calibration_bytes(n, d_t, r, c);
    return ok();
}

kvx_status kvx_fit_calibration(void* stream, int32_t dtype, const void* z, const void* w_l, int32_t n, int32_t L_t,
                               int32_t d_t, int32_t r, int32_t c, int32_t iters, float* u, void* ws, size_t ws_bytes) {
    if (kvx_status st = check_dtype(dtype)) return st;
    if (kvx_status st = check_fit_calibration(n, L_t, d_t, r, c)) return st;
    KVX_REQUIRE_PTR(z, "z");
    KVX_REQUIRE_PTR(w_l, "w_l");
    KVX_REQUIRE_PTR(u, "u");
    KVX_REQUIRE(iters >= 1 && iters <= 10000, "iters must be in [1, 10000] (got %d)", iters);
    const size_t need = fit_calibration_bytes(n, d_t, r, c);
    if (!ws || ws_bytes < need)
        return fail(KVX_ERR_WORKSPACE, "fit_calibration needs %zu workspace bytes (got %zu)", need, ws_bytes);
    KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    return hip_status(launch_fit_calibration((hipStream_t)stream, dtype, z, w_l, n, L_t, d_t, r, c, iters, u, ws),
                      "fit_calibration");
}

kvx_status kvx_select_topk(void* stream, const float* scores, const kvx_batch* batch, int32_t* sel,
                           int32_t* rest) {
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE_PTR(scores, "scores");
    if (bi.n_sel > 0) KVX_REQUIRE_PTR(sel, "sel");
    if (bi.n_rest > 0) KVX_REQUIRE_PTR(rest, "rest");
    return hip_status(launch_select(nullptr, 0, bi.n_tokens, (float*)scores, batch->cu_tokens_d,
                                    batch->cu_sel_d, bi.n_req, sel, rest, (hipStream_t)stream),
                      "select_topk");
}

kvx_status kvx_score_select_workspace(int32_t dtype, int32_t r, int64_t n, size_t* bytes) {
    if (kvx_status st = check_dtype(dtype)) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(r > 0 && n >= 0, "need r > 0 and n >= 0");
    if (dtype == KVX_BF16) {
        const int nt = cdiv(r, gemm_bf16_block_n());
        *bytes = round256((size_t)nt * n * 4);
    } else {
        *bytes = round256((size_t)n * r * 4) + round256((size_t)n * 4);
    }
    return ok();
}

}  // extern "C"

namespace {

// Every request's selected count is the budget of its percentage.
kvx_status check_budgets(const kvx_batch* batch, const BatchInfo& bi, const int32_t* budget_pct) {
    for (int b = 0; b < bi.n_req; ++b) {
        const int T = batch->cu_tokens_h[b + 1] - batch->cu_tokens_h[b];
        const int k = batch->cu_sel_h[b + 1] - batch->cu_sel_h[b];
        KVX_REQUIRE(budget_pct[b] >= 0 && budget_pct[b] <= 100, "budget_pct[%d] = %d outside [0, 100]", b,
                    budget_pct[b]);
        KVX_REQUIRE(k == budget_of(T, budget_pct[b]), "request %d: cu_sel gives %d positions but the "
                    "budget of %d%% of %d is %d", b, k, budget_pct[b], T, budget_of(T, budget_pct[b]));
    }
    return KVX_OK;
}

// Arguments of kvx_score_select other than its workspace.
kvx_status check_score_select(int32_t dtype, const void* z, const void* op, int32_t r, const kvx_batch* batch,
                              const int32_t* budget_pct, const float* scores, const int32_t* sel,
                              const int32_t* rest, BatchInfo* bi_out) {
    if (kvx_status st = check_dtype(dtype)) return st;
    BatchInfo& bi = *bi_out;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE_PTR(z, "z");
    KVX_REQUIRE_PTR(op, "op");
    KVX_REQUIRE_PTR(scores, "scores");
    KVX_REQUIRE(budget_pct, "budget_pct must not be null");
    KVX_REQUIRE(r > 0, "r must be positive");
    if (dtype == KVX_BF16) KVX_REQUIRE(r % 64 == 0, "bf16 needs r %% 64 == 0 (got %d)", r);
    if (bi.n_sel > 0) KVX_REQUIRE_PTR(sel, "sel");
    if (bi.n_rest > 0) KVX_REQUIRE_PTR(rest, "rest");
    if (kvx_status st = check_budgets(batch, bi, budget_pct)) return st;
    KVX_REQUIRE(bi.n_tokens <= INT32_MAX, "too many rows");
    return KVX_OK;
}

// Partial sums of z^T A z per row into ws (bf16: one per 256-column block of the operator, from the
// score GEMM's epilogue; fp32: P = z A, then one row dot per row).  Returns the number of partials
// per row and where they start.
hipError_t score_partials(hipStream_t s, int32_t dtype, const void* z, const void* op, int32_t r,
                          const BatchInfo& bi, void* ws, const float** partial, int* n_part) {
    if (dtype == KVX_BF16) {
        GemmArgs a{};
        a.A = (const bf16*)z; a.lda = r; a.K_a = r;
        a.B = (const bf16*)op; a.ldb = 2 * r; a.b_group_stride = 0;
        a.M = (int)bi.n_tokens; a.N = r; a.K = 2 * r; a.groups = 1;
        a.rows.mode = 0;
        a.epi = EPI_SCORE; a.partial = (float*)ws; a.Z = (const bf16*)z; a.ldz = r;
        *partial = (const float*)ws;
        *n_part = cdiv(r, gemm_bf16_block_n());
        return launch_gemm_bf16(a, s);
    }
    float* P = (float*)ws;
    float* rows = (float*)((char*)ws + round256((size_t)bi.n_tokens * r * 4));
    GemmF32Args a{};
    a.A = (const float*)z; a.lda = r; a.K_a = r;
    a.B = (const float*)op; a.ldb = r;
    a.M = (int)bi.n_tokens; a.N = r; a.K = r; a.groups = 1;
    a.rows.mode = 0;
    a.epi = EPI_STORE; a.C = P; a.ldc = r;
    if (hipError_t e = launch_gemm_f32(a, s)) return e;
    *partial = rows;
    *n_part = 1;
    return launch_rowdot_f32(P, (const float*)z, bi.n_tokens, r, rows, s);
}

size_t score_ws_bytes(int32_t dtype, int32_t r, int64_t n) {
    size_t b = 0;
    kvx_score_select_workspace(dtype, r, n, &b);
    return b;
}

// Score GEMM and the top-k.  Every byte of ws that is read was written by this call.  With op2
// (the total-energy operator) the score is the ratio of the two quadratic forms; its partials go
// to the second half of ws.
kvx_status run_score_select(hipStream_t s, int32_t dtype, const void* z, const void* op, int32_t r,
                            const kvx_batch* batch, const BatchInfo& bi, float* scores, int32_t* sel, int32_t* rest,
                            void* ws, const void* op2 = nullptr) {
    if (bi.n_tokens == 0) return ok();
    const float* part = nullptr;
    const float* part2 = nullptr;
    int np = 0, np2 = 0;
    KVX_TRY_HIP(score_partials(s, dtype, z, op, r, bi, ws, &part, &np), "score");
    if (op2)
        KVX_TRY_HIP(score_partials(s, dtype, z, op2, r, bi, (char*)ws + score_ws_bytes(dtype, r, bi.n_tokens), &part2,
                                   &np2), "score (total energy)");
    return hip_status(launch_select(part, np, bi.n_tokens, scores, batch->cu_tokens_d, batch->cu_sel_d, bi.n_req,
                                    sel, rest, s, part2, np2),
                      "select");
}

// Scratch of kvx_score_select_noalloc: one array per device, in the code object (so it exists
// from the library's load on that device until the process ends).  Host code never uses the
// array's name as an address: its device address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)KVX_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES];

kvx_status scratch_of_current_device(void** out) {
    int dev = -1;
    KVX_TRY_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
        return fail(KVX_ERR_UNSUPPORTED, "device %d: the no-allocation scratch covers devices 0..%d", dev,
                    NOALLOC_MAX_DEVICES - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        KVX_TRY_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (!p) return fail(KVX_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KVX_OK;
}

}  // namespace

extern "C" {

kvx_status kvx_score_select(void* stream, int32_t dtype, const void* z, const void* op, int32_t r,
                            const kvx_batch* batch, const int32_t* budget_pct, float* scores,
                            int32_t* sel, int32_t* rest, void* ws, size_t ws_bytes) {
    BatchInfo bi;
    if (kvx_status st = check_score_select(dtype, z, op, r, batch, budget_pct, scores, sel, rest, &bi)) return st;
    size_t need = 0;
    kvx_score_select_workspace(dtype, r, bi.n_tokens, &need);
    if (!ws || ws_bytes < need)
        return fail(KVX_ERR_WORKSPACE, "score_select needs %zu workspace bytes (got %zu)", need, ws_bytes);
    KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    return run_score_select((hipStream_t)stream, dtype, z, op, r, batch, bi, scores, sel, rest, ws);
}

kvx_status kvx_score_select_noalloc(void* stream, int32_t dtype, const void* z, const void* op, int32_t r,
                                    const kvx_batch* batch, const int32_t* budget_pct, float* scores,
                                    int32_t* sel, int32_t* rest) {
    BatchInfo bi;
    if (kvx_status st = check_score_select(dtype, z, op, r, batch, budget_pct, scores, sel, rest, &bi)) return st;
    size_t need = 0;
    kvx_score_select_workspace(dtype, r, bi.n_tokens, &need);
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(KVX_ERR_WORKSPACE, "score_select_noalloc: this batch needs %zu scratch bytes, more than the "
                    "%zu the library holds (use kvx_score_select with a workspace)", need, NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (kvx_status st = scratch_of_current_device(&ws)) return st;
    return run_score_select((hipStream_t)stream, dtype, z, op, r, batch, bi, scores, sel, rest, ws);
}

kvx_status kvx_score_select_normalized_workspace(int32_t dtype, int32_t r, int64_t n, size_t* bytes) {
    if (kvx_status st = kvx_score_select_workspace(dtype, r, n, bytes)) return st;
    *bytes *= 2;
    return ok();
}

kvx_status kvx_score_select_normalized(void* stream, int32_t dtype, const void* z, const void* op,
                                       const void* op_total, int32_t r, const kvx_batch* batch,
                                       const int32_t* budget_pct, float* scores, int32_t* sel, int32_t* rest,
                                       void* ws, size_t ws_bytes) {
    BatchInfo bi;
    if (kvx_status st = check_score_select(dtype, z, op, r, batch, budget_pct, scores, sel, rest, &bi)) return st;
    KVX_REQUIRE_PTR(op_total, "op_total");
    size_t need = 0;
    kvx_score_select_normalized_workspace(dtype, r, bi.n_tokens, &need);
    if (!ws || ws_bytes < need)
        return fail(KVX_ERR_WORKSPACE, "score_select_normalized needs %zu workspace bytes (got %zu)", need, ws_bytes);
    KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    return run_score_select((hipStream_t)stream, dtype, z, op, r, batch, bi, scores, sel, rest, ws, op_total);
}

}  // extern "C"

namespace {

// Reconstruction of the listed rows (all rows when rows is null) into every layer's cache; with
// rope set (bf16 only) the key columns are rotated at their rows' positions on the way.
kvx_status run_reconstruct(void* stream, int32_t dtype, const void* z, const void* w_l, int32_t L_t, int32_t r,
                           int32_t H_kv, int32_t d_h, const float* rope, const kvx_batch* batch,
                           const int32_t* rows, const kvx_cache* cache) {
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE_PTR(z, "z");
    KVX_REQUIRE_PTR(w_l, "w_l");
    KVX_REQUIRE(L_t > 0 && r > 0 && H_kv > 0 && d_h > 0, "L_t, r, H_kv and d_h must be positive");
    KVX_REQUIRE(d_h % 8 == 0, "d_h must be a multiple of 8 (got %d)", d_h);
    if (dtype == KVX_BF16) KVX_REQUIRE(r % 64 == 0, "bf16 needs r %% 64 == 0 (got %d)", r);
    if (kvx_status st = check_cache(cache, bi, dtype, H_kv, d_h, L_t)) return st;
    if (kvx_status st = check_page_table_debug(cache, batch)) return st;
    if (rows) KVX_REQUIRE(aligned16(rows), "rows must be 16-byte aligned");
    if (kvx_status st = check_positions_debug(rows, batch, true, "rows")) return st;
    const int64_t M = rows ? bi.n_rest : bi.n_tokens;
    if (M == 0) return ok();
    hipStream_t s = (hipStream_t)stream;
    const int hd = H_kv * d_h, d_t = 2 * hd;
    RowMap rm{};
    rm.mode = rows ? 2 : 1;
    rm.list = rows;
    rm.list_is_rest = 1;
    rm.cu_tok = batch->cu_tokens_d;
    rm.cu_sel = batch->cu_sel_d;
    rm.n_req = bi.n_req;
    if (dtype == KVX_BF16) {
        GemmArgs a{};
        a.A = (const bf16*)z; a.lda = r; a.K_a = r;
        a.B = (const bf16*)w_l; a.ldb = r; a.b_group_stride = (int64_t)d_t * r;
        a.M = (int)M; a.N = d_t; a.K = r; a.groups = L_t;
        a.rows = rm;
        a.epi = EPI_CACHE;
        a.kc = (bf16*)cache->k; a.vc = (bf16*)cache->v;
        a.layer_elems = cache->n_slots * hd; a.hd = hd; a.slots = slot_map(cache, batch);
        a.rope = rope; a.d_h = d_h;
        return hip_status(launch_gemm_bf16(a, s), "reconstruct");
    }
    GemmF32Args a{};
    a.A = (const float*)z; a.lda = r; a.K_a = r;
    a.B = (const float*)w_l; a.ldb = r; a.b_group_stride = (int64_t)d_t * r;
    a.M = (int)M; a.N = d_t; a.K = r; a.groups = L_t;
    a.rows = rm;
    a.epi = EPI_CACHE;
    a.kc = (float*)cache->k; a.vc = (float*)cache->v;
    a.layer_elems = cache->n_slots * hd; a.hd = hd; a.slots = slot_map(cache, batch);
    if (!rope) return hip_status(launch_gemm_f32(a, s), "reconstruct");
    KVX_TRY_HIP(launch_gemm_f32(a, s), "reconstruct");
    return hip_status(launch_rope_cache_rows_f32((float*)cache->k, a.layer_elems, L_t, hd, d_h, rope, rm, a.slots, M, s),
                      "reconstruct (key rotation)");
}

}  // namespace

extern "C" {

kvx_status kvx_reconstruct(void* stream, int32_t dtype, const void* z, const void* w_l, int32_t L_t,
                           int32_t r, int32_t H_kv, int32_t d_h, const kvx_batch* batch,
                           const int32_t* rows, const kvx_cache* cache) {
    if (kvx_status st = check_dtype(dtype)) return st;
    return run_reconstruct(stream, dtype, z, w_l, L_t, r, H_kv, d_h, nullptr, batch, rows, cache);
}

kvx_status kvx_reconstruct_rope(void* stream, int32_t dtype, const void* z, const void* w_l, int32_t L_t,
                                int32_t r, int32_t H_kv, int32_t d_h, const float* rope, int32_t max_pos,
                                const kvx_batch* batch, const int32_t* rows, const kvx_cache* cache) {
    if (kvx_status st = check_dtype(dtype)) return st;
    if (dtype == KVX_BF16 && d_h != 64 && d_h != 128)
        return fail(KVX_ERR_UNSUPPORTED, "bf16 needs d_h 64 or 128 (got %d)", d_h);
    KVX_REQUIRE_PTR(rope, "rope");
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE(max_pos >= bi.max_T, "rope table has %d positions, the longest request %d", max_pos, bi.max_T);
    return run_reconstruct(stream, dtype, z, w_l, L_t, r, H_kv, d_h, rope, batch, rows, cache);
}

kvx_status kvx_rope_table(void* stream, double base, int32_t d_h, int32_t max_pos, float* table) {
    KVX_REQUIRE_PTR(table, "table");
    KVX_REQUIRE(d_h >= 2 && d_h % 2 == 0, "d_h must be even and >= 2 (got %d)", d_h);
    KVX_REQUIRE(max_pos >= 1, "max_pos must be >= 1");
    KVX_REQUIRE(base > 0.0, "base must be positive");
    return hip_status(launch_rope_table(base, d_h, max_pos, table, (hipStream_t)stream), "rope_table");
}

kvx_status kvx_recompute_attn_workspace(int32_t dtype, const kvx_batch* batch, int32_t D, int32_t H_q,
                                        int32_t H_kv, int32_t d_h, size_t* bytes) {
    if (kvx_status st = check_dtype(dtype)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(H_q > 0 && H_kv > 0 && d_h > 0, "H_q, H_kv and d_h must be positive");
    KVX_REQUIRE(D > 0, "D must be positive");
    const int n_qkv = (H_q + 2 * H_kv) * d_h;
    *bytes = round256((size_t)bi.n_sel * n_qkv * elem_size(dtype)) +
             std::max(qkv_split_bytes(dtype, bi.n_sel, D, n_qkv), attn_split_bytes(dtype, batch, bi, H_q, H_kv, d_h));
    return ok();
}

kvx_status kvx_sparse_attention_workspace(int32_t dtype, const kvx_batch* batch, int32_t H_q, int32_t H_kv,
                                          int32_t d_h, size_t* bytes) {
    if (kvx_status st = check_dtype(dtype)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(H_q > 0 && H_kv > 0 && d_h > 0, "H_q, H_kv and d_h must be positive");
    *bytes = attn_split_bytes(dtype, batch, bi, H_q, H_kv, d_h);
    return ok();
}

kvx_status kvx_qkv_project_workspace(int32_t dtype, const kvx_batch* batch, int32_t D, int32_t H_q, int32_t H_kv,
                                     int32_t d_h, size_t* bytes) {
    if (kvx_status st = check_dtype(dtype)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(H_q > 0 && H_kv > 0 && d_h > 0, "H_q, H_kv and d_h must be positive");
    KVX_REQUIRE(D > 0, "D must be positive");
    *bytes = qkv_split_bytes(dtype, bi.n_sel, D, (H_q + 2 * H_kv) * d_h);
    return ok();
}

}  // extern "C"

namespace {

// Head shape and batch checks shared by the recompute steps.
kvx_status check_heads(int32_t dtype, int32_t H_q, int32_t H_kv, int32_t d_h) {
    if (kvx_status st = check_dtype(dtype)) return st;
    KVX_REQUIRE(H_q > 0 && H_kv > 0, "H_q and H_kv must be positive");
    if (d_h != 64 && d_h != 128) return fail(KVX_ERR_UNSUPPORTED, "d_h must be 64 or 128 (got %d)", d_h);
    KVX_REQUIRE(H_q % H_kv == 0, "H_q (%d) must be a multiple of H_kv (%d)", H_q, H_kv);
    const int g = H_q / H_kv;
    if (g > 16) return fail(KVX_ERR_UNSUPPORTED, "H_q / H_kv = %d > 16", g);
    if (dtype == KVX_BF16 && attn_bf16_block_queries(g) == 0)
        return fail(KVX_ERR_UNSUPPORTED, "bf16 attention supports H_q / H_kv <= 16 (got %d)", g);
    return KVX_OK;
}

kvx_status check_layer_cache(const kvx_cache* cache, const kvx_batch* batch, const BatchInfo& bi, int32_t dtype,
                             int32_t H_kv, int32_t d_h, int32_t layer, const float* rope, int32_t max_pos) {
    KVX_REQUIRE_PTR(rope, "rope");
    KVX_REQUIRE(max_pos >= bi.max_T, "rope table has %d positions, the longest request %d", max_pos, bi.max_T);
    if (kvx_status st = check_cache(cache, bi, dtype, H_kv, d_h, 1)) return st;
    KVX_REQUIRE(layer >= 0 && layer < cache->n_layers, "layer %d outside [0, %d)", layer, cache->n_layers);
    return check_page_table_debug(cache, batch);
}

RowMap sel_rows(const kvx_batch* batch, const int32_t* sel, int n_req) {
    RowMap rm{};
    rm.mode = 2;
    rm.list = sel;
    rm.list_is_rest = 0;
    rm.cu_tok = batch->cu_tokens_d;
    rm.cu_sel = batch->cu_sel_d;
    rm.n_req = n_req;
    return rm;
}

hipError_t run_qkv(hipStream_t s, int32_t dtype, const void* x_l, const void* w_qkv, int32_t D, int n_qkv,
                   const kvx_batch* batch, const BatchInfo& bi, const int32_t* sel, void* qkv, void* split_ws) {
    const RowMap rm = sel_rows(batch, sel, bi.n_req);
    if (dtype == KVX_BF16) {
        GemmArgs a{};
        a.A = (const bf16*)x_l; a.lda = D; a.K_a = D;
        a.B = (const bf16*)w_qkv; a.ldb = D;
        a.M = (int)bi.n_sel; a.N = n_qkv; a.K = D; a.groups = 1;
        a.rows = rm;
        a.epi = EPI_STORE; a.C = (bf16*)qkv; a.ldc = n_qkv;
        a.split_ws = (float*)split_ws;
        return launch_gemm_bf16(a, s);
    }
    GemmF32Args a{};
    a.A = (const float*)x_l; a.lda = D; a.K_a = D;
    a.B = (const float*)w_qkv; a.ldb = D;
    a.M = (int)bi.n_sel; a.N = n_qkv; a.K = D; a.groups = 1;
    a.rows = rm;
    a.epi = EPI_STORE; a.C = (float*)qkv; a.ldc = n_qkv;
    return launch_gemm_f32(a, s);
}

void* layer_base(void* base, const kvx_cache* cache, int layer, int hd, int32_t dtype) {
    return (char*)base + (int64_t)layer * cache->n_slots * hd * (int64_t)elem_size(dtype);
}

hipError_t run_scatter(hipStream_t s, int32_t dtype, int32_t layer, const void* qkv, int32_t H_q, int32_t H_kv,
                       int32_t d_h, const float* rope, const kvx_batch* batch, const BatchInfo& bi,
                       const int32_t* sel, const kvx_cache* cache) {
    const int hd = H_kv * d_h;
    ScatterArgs sc{};
    sc.qkv = qkv; sc.ld = (H_q + 2 * H_kv) * d_h;
    sc.H_q = H_q; sc.H_kv = H_kv; sc.d_h = d_h;
    sc.rope = rope;
    sc.sel = sel; sc.cu_sel = batch->cu_sel_d; sc.n_req = bi.n_req; sc.n_sel = bi.n_sel;
    sc.slots = slot_map(cache, batch);
    sc.kc = layer_base(cache->k, cache, layer, hd, dtype);
    sc.vc = layer_base(cache->v, cache, layer, hd, dtype);
    return launch_rope_scatter(sc, dtype, s);
}

// Steps 1-3 of one layer.  bf16: one GEMM whose epilogue rounds every output to bf16, keeps
// the q columns in qkv and writes rotated k and v to the cache slots, with the arithmetic of
// the separate steps (bit-identical to run_qkv + run_scatter).  fp32: the two separate kernels.
// compact_rows: row i of x_l is the i-th selected row itself (the chained layer's rows), not
// row cu_tokens[b] + sel[i] of the batch.
hipError_t run_qkv_rope_scatter(hipStream_t s, int32_t dtype, int32_t layer, const void* x_l, const void* w_qkv,
                                int32_t D, int32_t H_q, int32_t H_kv, int32_t d_h, const float* rope,
                                const kvx_batch* batch, const BatchInfo& bi, const int32_t* sel,
                                const kvx_cache* cache, void* qkv, void* split_ws, bool compact_rows = false,
                                const float* q_gain = nullptr, const float* k_gain = nullptr, float eps = 0.f) {
    const int n_qkv = (H_q + 2 * H_kv) * d_h;
    if (dtype != KVX_BF16) {
        if (hipError_t e = run_qkv(s, dtype, x_l, w_qkv, D, n_qkv, batch, bi, sel, qkv, split_ws)) return e;
        if (q_gain)                      // QK-norm: q and k heads normalised in place before the rotation
            if (hipError_t e = launch_qknorm_rows_f32((float*)qkv, bi.n_sel, n_qkv, H_q, H_kv, d_h, q_gain, k_gain,
                                                      eps, s))
                return e;
        return run_scatter(s, dtype, layer, qkv, H_q, H_kv, d_h, rope, batch, bi, sel, cache);
    }
    const int hd = H_kv * d_h;
    GemmArgs a{};
    a.A = (const bf16*)x_l; a.lda = D; a.K_a = D;
    a.B = (const bf16*)w_qkv; a.ldb = D;
    a.M = (int)bi.n_sel; a.N = n_qkv; a.K = D; a.groups = 1;
    a.rows = sel_rows(batch, sel, bi.n_req);
    if (compact_rows) a.rows.mode = 3;
    a.epi = EPI_QKV; a.C = (bf16*)qkv; a.ldc = n_qkv;
    a.kc = (bf16*)layer_base(cache->k, cache, layer, hd, dtype);
    a.vc = (bf16*)layer_base(cache->v, cache, layer, hd, dtype);
    a.hd = hd; a.slots = slot_map(cache, batch);
    a.rope = rope; a.q_cols = H_q * d_h; a.d_h = d_h;
    a.split_ws = (float*)split_ws;
    if (q_gain) {                    // QK-norm: whole tiles only (the split reduce has no normalisation)
        a.qk_gain_q = q_gain; a.qk_gain_k = k_gain; a.qk_eps = eps;
        a.split_ws = nullptr;
    }
    return launch_gemm_bf16(a, s);
}

// Layers [layer, layer + n) of one launch (bf16 only when n > 1): q columns, outputs and
// log-sum-exps of layer layer + j at qkv, out, lse + j * the strides (elements).
struct LayerSpan {
    int n;
    int64_t q_stride, out_stride, lse_stride;
};

// Steps 1-3 of layers [l0, l0 + n) in one grouped GEMM (bf16): group j reads x + j * N * D and
// w_qkv + j * n_qkv * D, keeps its q columns in qkv + j * q_stride and writes its rotated k
// and v into cache layer l0 + j.  The same epilogue arithmetic as run_qkv_rope_scatter, without a
// K split: a whole tile of a group accumulates in the order a single-layer call without a
// workspace uses, so the two agree bit for bit.
hipError_t run_qkv_rope_scatter_layers(hipStream_t s, int32_t l0, int32_t n, const void* x, const void* w_qkv,
                                       int32_t D, int32_t H_q, int32_t H_kv, int32_t d_h, const float* rope,
                                       const kvx_batch* batch, const BatchInfo& bi, const int32_t* sel,
                                       const kvx_cache* cache, void* qkv, int64_t q_stride) {
    const int n_qkv = (H_q + 2 * H_kv) * d_h;
    const int hd = H_kv * d_h;
    GemmArgs a{};
    a.A = (const bf16*)x; a.lda = D; a.K_a = D; a.a_group_stride = bi.n_tokens * D;
    a.B = (const bf16*)w_qkv; a.ldb = D; a.b_group_stride = (int64_t)n_qkv * D;
    a.M = (int)bi.n_sel; a.N = n_qkv; a.K = D; a.groups = n;
    a.rows = sel_rows(batch, sel, bi.n_req);
    a.epi = EPI_QKV; a.C = (bf16*)qkv; a.ldc = n_qkv; a.c_group_stride = q_stride;
    a.kc = (bf16*)layer_base(cache->k, cache, l0, hd, KVX_BF16);
    a.vc = (bf16*)layer_base(cache->v, cache, l0, hd, KVX_BF16);
    a.layer_elems = cache->n_slots * hd; a.hd = hd; a.slots = slot_map(cache, batch);
    a.rope = rope; a.q_cols = H_q * d_h; a.d_h = d_h;
    return launch_gemm_bf16(a, s);
}

hipError_t run_attention(hipStream_t s, int32_t dtype, int32_t layer, const void* qkv, int32_t H_q,
                         int32_t H_kv, int32_t d_h, const float* rope, const kvx_batch* batch,
                         const BatchInfo& bi, const int32_t* sel, const kvx_cache* cache, void* out,
                         float* lse, void* split_ws, const LayerSpan& span = LayerSpan{1, 0, 0, 0}) {
    const int hd = H_kv * d_h;
    AttnArgs at{};
    at.n_split = 1;
    at.n_layers = span.n;
    at.q_layer_stride = span.q_stride;
    at.kv_layer_elems = cache->n_slots * hd;
    at.out_layer_stride = span.out_stride;
    at.lse_layer_stride = span.lse_stride;
    if (span.n > 1 && dtype != KVX_BF16) return hipErrorInvalidValue;
    at.qkv = qkv; at.ld = (H_q + 2 * H_kv) * d_h;
    at.H_q = H_q; at.H_kv = H_kv; at.d_h = d_h;
    at.rope = rope;
    at.sel = sel; at.cu_sel = batch->cu_sel_d; at.n_req = bi.n_req;
    at.slots = slot_map(cache, batch);
    at.kc = layer_base(cache->k, cache, layer, hd, dtype);
    at.vc = layer_base(cache->v, cache, layer, hd, dtype);
    at.out = out; at.lse = lse;
    if (dtype == KVX_BF16) {
        at.bq = attn_bf16_block_queries(H_q / H_kv);
        at.blk_cu[0] = 0;
        for (int b = 0; b < bi.n_req; ++b) {
            const int k = batch->cu_sel_h[b + 1] - batch->cu_sel_h[b];
            at.blk_cu[b + 1] = at.blk_cu[b] + (k + at.bq - 1) / at.bq;
        }
        at.n_blocks = at.blk_cu[bi.n_req];
        if (split_ws && span.n == 1) {
            at.n_split = attn_bf16_split(at.n_blocks, H_kv, bi.max_T);
            if (at.n_split > 1) {
                const int max_tiles = (bi.max_T + ATTN_KEY_TILE - 1) / ATTN_KEY_TILE;
                at.split_len = (max_tiles + at.n_split - 1) / at.n_split;
                at.part = (float*)split_ws;
                at.part_ml = at.part + round256((size_t)bi.n_sel * H_q * at.n_split * d_h * 4) / 4;
                at.n_rows_total = bi.n_sel;
            }
        }
        return launch_attn_bf16(at, s);
    }
    at.bq = 1;
    at.n_blocks = (int)bi.n_sel;     // one wave per (selected row, head)
    return launch_attn_f32(at, s);
}

// ---- chained target layer (bf16)

size_t gemm_split_ws(int64_t M, int N, int K, int epi) {
    if (M <= 0 || M > INT32_MAX || N <= 0 || K <= 0) return 0;
    return round256(gemm_bf16_split_bytes((int)M, N, K, 1, epi));
}

// out = resid + a w^T (compact rows)
hipError_t run_linear_residual(hipStream_t s, const void* a, const void* w, const void* resid, void* out, int64_t M,
                               int N, int K, void* split_ws) {
    GemmArgs g{};
    g.A = (const bf16*)a; g.lda = K; g.K_a = K;
    g.B = (const bf16*)w; g.ldb = K;
    g.M = (int)M; g.N = N; g.K = K; g.groups = 1;
    g.epi = EPI_RESID; g.C = (bf16*)out; g.ldc = N; g.R = (const bf16*)resid; g.ldr = N;
    g.split_ws = (float*)split_ws;
    return launch_gemm_bf16(g, s);
}

// out = a w^T (compact rows)
hipError_t run_linear(hipStream_t s, const void* a, const void* w, void* out, int64_t M, int N, int K, void* split_ws) {
    GemmArgs g{};
    g.A = (const bf16*)a; g.lda = K; g.K_a = K;
    g.B = (const bf16*)w; g.ldb = K;
    g.M = (int)M; g.N = N; g.K = K; g.groups = 1;
    g.epi = EPI_STORE; g.C = (bf16*)out; g.ldc = N;
    g.split_ws = (float*)split_ws;
    return launch_gemm_bf16(g, s);
}

// h = silu(x w_gate^T) * (x w_up^T)
hipError_t run_swiglu(hipStream_t s, const void* x, const void* w_gate, const void* w_up, void* h, int64_t M, int D,
                      int F, void* split_ws) {
    GemmArgs g{};
    g.A = (const bf16*)x; g.lda = D; g.K_a = D;
    g.B = (const bf16*)w_gate; g.B2 = (const bf16*)w_up; g.ldb = D;
    g.M = (int)M; g.N = 2 * F; g.K = D; g.groups = 1;
    g.epi = EPI_SWIGLU; g.C = (bf16*)h; g.ldc = F;
    g.split_ws = (float*)split_ws;
    return launch_gemm_bf16(g, s);
}

struct LayerWs {
    size_t xn, qkv, attn, mlp, split, total;
};

LayerWs layer_ws(int64_t k, int D, int F, int H_q, int H_kv, int d_h, size_t attn_split) {
    const int n_qkv = (H_q + 2 * H_kv) * d_h;
    LayerWs w{};
    w.xn = round256((size_t)k * D * 2);
    w.qkv = round256((size_t)k * n_qkv * 2);
    w.attn = round256((size_t)k * H_q * d_h * 2);
    w.mlp = round256((size_t)k * F * 2);
    w.split = std::max(std::max(gemm_split_ws(k, n_qkv, D, EPI_QKV), gemm_split_ws(k, D, H_q * d_h, EPI_RESID)),
                       std::max(gemm_split_ws(k, 2 * F, D, EPI_SWIGLU), gemm_split_ws(k, D, F, EPI_RESID)));
    w.split = std::max(w.split, attn_split);
    w.total = w.xn + w.qkv + w.attn + w.mlp + w.split;
    return w;
}

kvx_status check_bf16_only(int32_t dtype, const char* what) {
    if (kvx_status st = check_dtype(dtype)) return st;
    if (dtype != KVX_BF16) return fail(KVX_ERR_UNSUPPORTED, "%s supports KVX_BF16 only", what);
    return KVX_OK;
}

kvx_status check_ws(size_t need, const void* ws, size_t ws_bytes, const char* what) {
    if (need && (!ws || ws_bytes < need))
        return fail(KVX_ERR_WORKSPACE, "%s needs %zu workspace bytes (got %zu)", what, need, ws_bytes);
    if (need && !aligned16(ws)) return fail(KVX_ERR_INVALID, "ws must be 16-byte aligned");
    return KVX_OK;
}

}  // namespace

extern "C" {

kvx_status kvx_qkv_project(void* stream, int32_t dtype, const void* x_l, const void* w_qkv, int32_t D,
                           int32_t H_q, int32_t H_kv, int32_t d_h, const kvx_batch* batch, const int32_t* sel,
                           void* qkv, void* ws, size_t ws_bytes) {
    if (kvx_status st = check_heads(dtype, H_q, H_kv, d_h)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE_PTR(x_l, "x_l");
    KVX_REQUIRE_PTR(w_qkv, "w_qkv");
    KVX_REQUIRE(D > 0, "D must be positive");
    if (dtype == KVX_BF16) KVX_REQUIRE(D % 64 == 0, "bf16 needs D %% 64 == 0 (got %d)", D);
    if (bi.n_sel == 0) return ok();
    KVX_REQUIRE(bi.n_sel <= INT32_MAX, "too many selected rows");
    KVX_REQUIRE_PTR(sel, "sel");
    if (kvx_status st = check_positions_debug(sel, batch, false, "sel")) return st;
    KVX_REQUIRE_PTR(qkv, "qkv");
    const int n_qkv = (H_q + 2 * H_kv) * d_h;
    const size_t need = qkv_split_bytes(dtype, bi.n_sel, D, n_qkv);
    if (need && (!ws || ws_bytes < need))
        return fail(KVX_ERR_WORKSPACE, "qkv_project needs %zu workspace bytes (got %zu)", need, ws_bytes);
    if (need) KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    return hip_status(run_qkv((hipStream_t)stream, dtype, x_l, w_qkv, D, n_qkv, batch, bi, sel, qkv, need ? ws : nullptr),
                      "qkv_project");
}

kvx_status kvx_rope_scatter(void* stream, int32_t dtype, int32_t layer, const void* qkv, int32_t H_q,
                            int32_t H_kv, int32_t d_h, const float* rope, int32_t max_pos, const kvx_batch* batch,
                            const int32_t* sel, const kvx_cache* cache) {
    if (kvx_status st = check_heads(dtype, H_q, H_kv, d_h)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    if (kvx_status st = check_layer_cache(cache, batch, bi, dtype, H_kv, d_h, layer, rope, max_pos)) return st;
    if (bi.n_sel == 0) return ok();
    KVX_REQUIRE_PTR(sel, "sel");
    if (kvx_status st = check_positions_debug(sel, batch, false, "sel")) return st;
    KVX_REQUIRE_PTR(qkv, "qkv");
    return hip_status(run_scatter((hipStream_t)stream, dtype, layer, qkv, H_q, H_kv, d_h, rope, batch, bi, sel,
                                  cache), "rope_scatter");
}

kvx_status kvx_qkv_rope_scatter(void* stream, int32_t dtype, int32_t layer, const void* x_l, const void* w_qkv,
                                int32_t D, int32_t H_q, int32_t H_kv, int32_t d_h, const float* rope,
                                int32_t max_pos, const kvx_batch* batch, const int32_t* sel,
                                const kvx_cache* cache, void* qkv, void* ws, size_t ws_bytes) {
    if (kvx_status st = check_heads(dtype, H_q, H_kv, d_h)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE_PTR(x_l, "x_l");
    KVX_REQUIRE_PTR(w_qkv, "w_qkv");
    KVX_REQUIRE(D > 0, "D must be positive");
    if (dtype == KVX_BF16) KVX_REQUIRE(D % 64 == 0, "bf16 needs D %% 64 == 0 (got %d)", D);
    if (kvx_status st = check_layer_cache(cache, batch, bi, dtype, H_kv, d_h, layer, rope, max_pos)) return st;
    if (bi.n_sel == 0) return ok();
    KVX_REQUIRE(bi.n_sel <= INT32_MAX, "too many selected rows");
    KVX_REQUIRE_PTR(sel, "sel");
    if (kvx_status st = check_positions_debug(sel, batch, false, "sel")) return st;
    KVX_REQUIRE_PTR(qkv, "qkv");
    const int n_qkv = (H_q + 2 * H_kv) * d_h;
    const size_t need = qkv_split_bytes(dtype, bi.n_sel, D, n_qkv);
    if (need && (!ws || ws_bytes < need))
        return fail(KVX_ERR_WORKSPACE, "qkv_rope_scatter needs %zu workspace bytes (got %zu)", need, ws_bytes);
    if (need) KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    return hip_status(run_qkv_rope_scatter((hipStream_t)stream, dtype, layer, x_l, w_qkv, D, H_q, H_kv, d_h, rope,
                                           batch, bi, sel, cache, qkv, need ? ws : nullptr),
                      "qkv_rope_scatter");
}

kvx_status kvx_qkv_rope_scatter_qknorm(void* stream, int32_t dtype, int32_t layer, const void* x_l,
                                       const void* w_qkv, int32_t D, int32_t H_q, int32_t H_kv, int32_t d_h,
                                       const float* q_gain, const float* k_gain, float eps, const float* rope,
                                       int32_t max_pos, const kvx_batch* batch, const int32_t* sel,
                                       const kvx_cache* cache, void* qkv) {
    if (kvx_status st = check_heads(dtype, H_q, H_kv, d_h)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE_PTR(x_l, "x_l");
    KVX_REQUIRE_PTR(w_qkv, "w_qkv");
    KVX_REQUIRE(q_gain && k_gain, "q_gain and k_gain must not be null");
    KVX_REQUIRE(eps >= 0.f && eps < INFINITY, "eps must be finite and >= 0");
    if (dtype == KVX_BF16) KVX_REQUIRE(D > 0 && D % 64 == 0, "bf16 needs D %% 64 == 0 (got %d)", D);
    else KVX_REQUIRE(D > 0, "D must be positive (got %d)", D);
    if (kvx_status st = check_layer_cache(cache, batch, bi, dtype, H_kv, d_h, layer, rope, max_pos)) return st;
    if (bi.n_sel == 0) return ok();
    KVX_REQUIRE(bi.n_sel <= INT32_MAX, "too many selected rows");
    KVX_REQUIRE_PTR(sel, "sel");
    if (kvx_status st = check_positions_debug(sel, batch, false, "sel")) return st;
    KVX_REQUIRE_PTR(qkv, "qkv");
    return hip_status(run_qkv_rope_scatter((hipStream_t)stream, dtype, layer, x_l, w_qkv, D, H_q, H_kv, d_h, rope,
                                           batch, bi, sel, cache, qkv, nullptr, false, q_gain, k_gain, eps),
                      "qkv_rope_scatter_qknorm");
}

kvx_status kvx_sparse_attention(void* stream, int32_t dtype, int32_t layer, const void* qkv, int32_t H_q,
                                int32_t H_kv, int32_t d_h, const float* rope, int32_t max_pos,
                                const kvx_batch* batch, const int32_t* sel, const kvx_cache* cache, void* out,
                                float* lse, void* ws, size_t ws_bytes) {
    if (kvx_status st = check_heads(dtype, H_q, H_kv, d_h)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    if (bi.n_req > MAX_ATTN_REQ)
        return fail(KVX_ERR_UNSUPPORTED, "at most %d requests per call (got %d)", MAX_ATTN_REQ, bi.n_req);
    if (kvx_status st = check_layer_cache(cache, batch, bi, dtype, H_kv, d_h, layer, rope, max_pos)) return st;
    if (bi.n_sel == 0) return ok();
    KVX_REQUIRE_PTR(sel, "sel");
    if (kvx_status st = check_positions_debug(sel, batch, false, "sel")) return st;
    KVX_REQUIRE_PTR(qkv, "qkv");
    KVX_REQUIRE_PTR(out, "out");
    if (lse) KVX_REQUIRE(aligned16(lse), "lse must be 16-byte aligned");
    // no workspace: no key-range split; otherwise the full size is required
    const size_t need = attn_split_bytes(dtype, batch, bi, H_q, H_kv, d_h);
    const bool split = need && (ws || ws_bytes);
    if (split) {
        if (!ws || ws_bytes < need)
            return fail(KVX_ERR_WORKSPACE, "sparse_attention needs %zu workspace bytes (got %zu)", need, ws_bytes);
        KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    }
    return hip_status(run_attention((hipStream_t)stream, dtype, layer, qkv, H_q, H_kv, d_h, rope, batch, bi, sel,
                                    cache, out, lse, split ? ws : nullptr), "sparse_attention");
}

kvx_status kvx_recompute_attn(void* stream, int32_t dtype, int32_t layer, const void* x_l, const void* w_qkv,
                              int32_t D, int32_t H_q, int32_t H_kv, int32_t d_h, const float* rope,
                              int32_t max_pos, const kvx_batch* batch, const int32_t* sel,
                              const kvx_cache* cache, void* out, float* lse, void* ws, size_t ws_bytes) {
    if (kvx_status st = check_heads(dtype, H_q, H_kv, d_h)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE_PTR(x_l, "x_l");
    KVX_REQUIRE_PTR(w_qkv, "w_qkv");
    KVX_REQUIRE(D > 0, "D must be positive");
    if (dtype == KVX_BF16) KVX_REQUIRE(D % 64 == 0, "bf16 needs D %% 64 == 0 (got %d)", D);
    if (bi.n_req > MAX_ATTN_REQ)
        return fail(KVX_ERR_UNSUPPORTED, "at most %d requests per call (got %d)", MAX_ATTN_REQ, bi.n_req);
    if (kvx_status st = check_layer_cache(cache, batch, bi, dtype, H_kv, d_h, layer, rope, max_pos)) return st;
    size_t need = 0;
    kvx_recompute_attn_workspace(dtype, batch, D, H_q, H_kv, d_h, &need);
    if (bi.n_sel == 0) return ok();
    KVX_REQUIRE(bi.n_sel <= INT32_MAX, "too many selected rows");
    KVX_REQUIRE_PTR(sel, "sel");
    if (kvx_status st = check_positions_debug(sel, batch, false, "sel")) return st;
    KVX_REQUIRE_PTR(out, "out");
    if (lse) KVX_REQUIRE(aligned16(lse), "lse must be 16-byte aligned");
    if (!ws || ws_bytes < need)
        return fail(KVX_ERR_WORKSPACE, "recompute_attn needs %zu workspace bytes (got %zu)", need, ws_bytes);
    KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const int n_qkv = (H_q + 2 * H_kv) * d_h;
    const size_t qkv_bytes = round256((size_t)bi.n_sel * n_qkv * elem_size(dtype));
    void* split_ws = qkv_split_bytes(dtype, bi.n_sel, D, n_qkv) ? (char*)ws + qkv_bytes : nullptr;
    void* attn_ws = attn_split_bytes(dtype, batch, bi, H_q, H_kv, d_h) ? (char*)ws + qkv_bytes : nullptr;
    KVX_TRY_HIP(run_qkv_rope_scatter(s, dtype, layer, x_l, w_qkv, D, H_q, H_kv, d_h, rope, batch, bi, sel, cache,
                                     ws, split_ws), "recompute qkv/rope/scatter");
    return hip_status(run_attention(s, dtype, layer, ws, H_q, H_kv, d_h, rope, batch, bi, sel, cache, out, lse,
                                    attn_ws), "attention");
}

}  // extern "C"

namespace {

// Shared checks of the several-layer entry points.
kvx_status check_layers(const kvx_cache* cache, const kvx_batch* batch, const BatchInfo& bi, int32_t dtype,
                        int32_t H_kv, int32_t d_h, int32_t l0, int32_t n_layers, const float* rope,
                        int32_t max_pos) {
    KVX_REQUIRE(n_layers >= 1, "n_layers must be >= 1 (got %d)", n_layers);
    if (kvx_status st = check_layer_cache(cache, batch, bi, dtype, H_kv, d_h, l0, rope, max_pos)) return st;
    KVX_REQUIRE((int64_t)l0 + n_layers <= cache->n_layers, "layers [%d, %d) outside the cache's %d layers", l0,
                l0 + n_layers, cache->n_layers);
    return KVX_OK;
}

size_t layers_qkv_bytes(int32_t dtype, int64_t n_sel, int n_qkv) {
    return round256((size_t)n_sel * n_qkv * elem_size(dtype));
}

}  // namespace

extern "C" {

kvx_status kvx_qkv_rope_scatter_layers(void* stream, int32_t dtype, int32_t l0, int32_t n_layers, const void* x,
                                       const void* w_qkv, int32_t D, int32_t H_q, int32_t H_kv, int32_t d_h,
                                       const float* rope, int32_t max_pos, const kvx_batch* batch,
                                       const int32_t* sel, const kvx_cache* cache, void* qkv) {
    if (kvx_status st = check_heads(dtype, H_q, H_kv, d_h)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE_PTR(x, "x");
    KVX_REQUIRE_PTR(w_qkv, "w_qkv");
    KVX_REQUIRE(D > 0, "D must be positive");
    if (dtype == KVX_BF16) KVX_REQUIRE(D % 64 == 0, "bf16 needs D %% 64 == 0 (got %d)", D);
    if (kvx_status st = check_layers(cache, batch, bi, dtype, H_kv, d_h, l0, n_layers, rope, max_pos)) return st;
    if (bi.n_sel == 0) return ok();
    KVX_REQUIRE(bi.n_sel <= INT32_MAX, "too many selected rows");
    KVX_REQUIRE_PTR(sel, "sel");
    if (kvx_status st = check_positions_debug(sel, batch, false, "sel")) return st;
    KVX_REQUIRE_PTR(qkv, "qkv");
    hipStream_t s = (hipStream_t)stream;
    const int n_qkv = (H_q + 2 * H_kv) * d_h;
    if (dtype == KVX_BF16)
        return hip_status(run_qkv_rope_scatter_layers(s, l0, n_layers, x, w_qkv, D, H_q, H_kv, d_h, rope, batch, bi,
                                                      sel, cache, qkv, bi.n_sel * n_qkv), "qkv_rope_scatter_layers");
    for (int j = 0; j < n_layers; ++j)       // fp32: the single-layer kernels, layer by layer
        KVX_TRY_HIP(run_qkv_rope_scatter(s, dtype, l0 + j, (const float*)x + (int64_t)j * bi.n_tokens * D,
                                         (const float*)w_qkv + (int64_t)j * n_qkv * D, D, H_q, H_kv, d_h, rope,
                                         batch, bi, sel, cache, (float*)qkv + (int64_t)j * bi.n_sel * n_qkv,
                                         nullptr), "qkv_rope_scatter_layers");
    return ok();
}

kvx_status kvx_sparse_attention_layers(void* stream, int32_t dtype, int32_t l0, int32_t n_layers, const void* qkv,
                                       int32_t H_q, int32_t H_kv, int32_t d_h, const float* rope, int32_t max_pos,
                                       const kvx_batch* batch, const int32_t* sel, const kvx_cache* cache,
                                       void* out, float* lse) {
    if (kvx_status st = check_heads(dtype, H_q, H_kv, d_h)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    if (bi.n_req > MAX_ATTN_REQ)
        return fail(KVX_ERR_UNSUPPORTED, "at most %d requests per call (got %d)", MAX_ATTN_REQ, bi.n_req);
    if (kvx_status st = check_layers(cache, batch, bi, dtype, H_kv, d_h, l0, n_layers, rope, max_pos)) return st;
    if (bi.n_sel == 0) return ok();
    KVX_REQUIRE_PTR(sel, "sel");
    if (kvx_status st = check_positions_debug(sel, batch, false, "sel")) return st;
    KVX_REQUIRE_PTR(qkv, "qkv");
    KVX_REQUIRE_PTR(out, "out");
    if (lse) KVX_REQUIRE(aligned16(lse), "lse must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const int n_qkv = (H_q + 2 * H_kv) * d_h;
    const int64_t q_stride = bi.n_sel * n_qkv, o_stride = bi.n_sel * H_q * d_h, l_stride = bi.n_sel * H_q;
    if (dtype == KVX_BF16)
        return hip_status(run_attention(s, dtype, l0, qkv, H_q, H_kv, d_h, rope, batch, bi, sel, cache, out, lse,
                                        nullptr, LayerSpan{n_layers, q_stride, o_stride, l_stride}),
                          "sparse_attention_layers");
    for (int j = 0; j < n_layers; ++j)
        KVX_TRY_HIP(run_attention(s, dtype, l0 + j, (const float*)qkv + j * q_stride, H_q, H_kv, d_h, rope, batch,
                                  bi, sel, cache, (float*)out + j * o_stride, lse ? lse + j * l_stride : nullptr,
                                  nullptr), "sparse_attention_layers");
    return ok();
}

kvx_status kvx_recompute_attn_layers_workspace(int32_t dtype, const kvx_batch* batch, int32_t D, int32_t H_q,
                                               int32_t H_kv, int32_t d_h, int32_t n_layers, size_t* bytes) {
    if (kvx_status st = check_dtype(dtype)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(H_q > 0 && H_kv > 0 && d_h > 0 && D > 0, "D, H_q, H_kv and d_h must be positive");
    KVX_REQUIRE(n_layers >= 1, "n_layers must be >= 1 (got %d)", n_layers);
    *bytes = (size_t)n_layers * layers_qkv_bytes(dtype, bi.n_sel, (H_q + 2 * H_kv) * d_h);
    return ok();
}

kvx_status kvx_recompute_attn_layers(void* stream, int32_t dtype, int32_t l0, int32_t n_layers, const void* x,
                                     const void* w_qkv, int32_t D, int32_t H_q, int32_t H_kv, int32_t d_h,
                                     const float* rope, int32_t max_pos, const kvx_batch* batch,
                                     const int32_t* sel, const kvx_cache* cache, void* out, float* lse, void* ws,
                                     size_t ws_bytes) {
    if (kvx_status st = check_heads(dtype, H_q, H_kv, d_h)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE_PTR(x, "x");
    KVX_REQUIRE_PTR(w_qkv, "w_qkv");
    KVX_REQUIRE(D > 0, "D must be positive");
    if (dtype == KVX_BF16) KVX_REQUIRE(D % 64 == 0, "bf16 needs D %% 64 == 0 (got %d)", D);
    if (bi.n_req > MAX_ATTN_REQ)
        return fail(KVX_ERR_UNSUPPORTED, "at most %d requests per call (got %d)", MAX_ATTN_REQ, bi.n_req);
    if (kvx_status st = check_layers(cache, batch, bi, dtype, H_kv, d_h, l0, n_layers, rope, max_pos)) return st;
    if (bi.n_sel == 0) return ok();
    KVX_REQUIRE(bi.n_sel <= INT32_MAX, "too many selected rows");
    KVX_REQUIRE_PTR(sel, "sel");
    if (kvx_status st = check_positions_debug(sel, batch, false, "sel")) return st;
    KVX_REQUIRE_PTR(out, "out");
    if (lse) KVX_REQUIRE(aligned16(lse), "lse must be 16-byte aligned");
    const size_t per = layers_qkv_bytes(dtype, bi.n_sel, (H_q + 2 * H_kv) * d_h);
    const size_t need = (size_t)n_layers * per;
    if (!ws || ws_bytes < need)
        return fail(KVX_ERR_WORKSPACE, "recompute_attn_layers needs %zu workspace bytes (got %zu)", need, ws_bytes);
    KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const int n_qkv = (H_q + 2 * H_kv) * d_h;
    const int64_t q_stride = (int64_t)(per / elem_size(dtype)), o_stride = bi.n_sel * H_q * d_h,
                  l_stride = bi.n_sel * H_q;
    if (dtype == KVX_BF16) {
        // the q rows of layer j sit at ws + j * per; the grouped GEMM writes them there
        KVX_TRY_HIP(run_qkv_rope_scatter_layers(s, l0, n_layers, x, w_qkv, D, H_q, H_kv, d_h, rope, batch, bi, sel,
                                                cache, ws, q_stride), "recompute_attn_layers qkv/rope/scatter");
        return hip_status(run_attention(s, dtype, l0, ws, H_q, H_kv, d_h, rope, batch, bi, sel, cache, out, lse,
                                        nullptr, LayerSpan{n_layers, q_stride, o_stride, l_stride}),
                          "recompute_attn_layers attention");
    }
    for (int j = 0; j < n_layers; ++j) {
        void* q = (char*)ws + j * per;
        KVX_TRY_HIP(run_qkv_rope_scatter(s, dtype, l0 + j, (const float*)x + (int64_t)j * bi.n_tokens * D,
                                         (const float*)w_qkv + (int64_t)j * n_qkv * D, D, H_q, H_kv, d_h, rope,
                                         batch, bi, sel, cache, q, nullptr), "recompute_attn_layers qkv");
        KVX_TRY_HIP(run_attention(s, dtype, l0 + j, q, H_q, H_kv, d_h, rope, batch, bi, sel, cache,
                                  (float*)out + j * o_stride, lse ? lse + j * l_stride : nullptr, nullptr),
                    "recompute_attn_layers attention");
    }
    return ok();
}

kvx_status kvx_gather_rows(void* stream, int32_t dtype, const void* src, int32_t D, const kvx_batch* batch,
                           const int32_t* sel, void* dst) {
    if (kvx_status st = check_bf16_only(dtype, "gather_rows")) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE(D > 0 && D % 8 == 0, "D must be a positive multiple of 8 (got %d)", D);
    if (bi.n_sel == 0) return ok();
    KVX_REQUIRE(bi.n_sel <= INT32_MAX, "too many selected rows");
    KVX_REQUIRE_PTR(src, "src");
    KVX_REQUIRE_PTR(sel, "sel");
    if (kvx_status st = check_positions_debug(sel, batch, false, "sel")) return st;
    KVX_REQUIRE_PTR(dst, "dst");
    return hip_status(launch_gather_rows_bf16((const bf16*)src, D, sel, batch->cu_tokens_d, batch->cu_sel_d, bi.n_req,
                                              bi.n_sel, (bf16*)dst, (hipStream_t)stream),
                      "gather_rows");
}

kvx_status kvx_rmsnorm(void* stream, int32_t dtype, const void* x, const void* gamma, float eps, int64_t n,
                       int32_t D, void* y) {
    if (kvx_status st = check_bf16_only(dtype, "rmsnorm")) return st;
    KVX_REQUIRE(n >= 0 && n <= INT32_MAX, "n must be in [0, 2^31) (got %lld)", (long long)n);
    KVX_REQUIRE(D > 0 && D % 8 == 0 && D <= rmsnorm_max_dim(), "D must be a multiple of 8 in [8, %d] (got %d)",
                rmsnorm_max_dim(), D);
    KVX_REQUIRE(eps >= 0.f && eps < INFINITY, "eps must be finite and >= 0");
    if (n == 0) return ok();
    KVX_REQUIRE_PTR(x, "x");
    KVX_REQUIRE_PTR(gamma, "gamma");
    KVX_REQUIRE_PTR(y, "y");
    return hip_status(launch_rmsnorm_bf16((const bf16*)x, (const bf16*)gamma, eps, n, D, (bf16*)y, (hipStream_t)stream),
                      "rmsnorm");
}

kvx_status kvx_linear_residual_workspace(int32_t dtype, int64_t M, int32_t N, int32_t K, size_t* bytes) {
    if (kvx_status st = check_bf16_only(dtype, "linear_residual")) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(M >= 0 && M <= INT32_MAX && N > 0 && K > 0, "M must be in [0, 2^31), N and K positive");
    *bytes = gemm_split_ws(M, N, K, EPI_RESID);
    return ok();
}

kvx_status kvx_linear_residual(void* stream, int32_t dtype, const void* a, const void* w, const void* resid, void* out,
                               int64_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes) {
    if (kvx_status st = check_bf16_only(dtype, "linear_residual")) return st;
    KVX_REQUIRE(M >= 0 && M <= INT32_MAX, "M must be in [0, 2^31)");
    KVX_REQUIRE(N > 0 && N % 8 == 0, "N must be a positive multiple of 8 (got %d)", N);
    KVX_REQUIRE(K > 0 && K % 64 == 0, "K must be a positive multiple of 64 (got %d)", K);
    if (M == 0) return ok();
    KVX_REQUIRE_PTR(a, "a");
    KVX_REQUIRE_PTR(w, "w");
    KVX_REQUIRE_PTR(resid, "resid");
    KVX_REQUIRE_PTR(out, "out");
    const size_t need = gemm_split_ws(M, N, K, EPI_RESID);
    if (kvx_status st = check_ws(need, ws, ws_bytes, "linear_residual")) return st;
    return hip_status(run_linear_residual((hipStream_t)stream, a, w, resid, out, M, N, K, need ? ws : nullptr),
                      "linear_residual");
}

kvx_status kvx_swiglu_workspace(int32_t dtype, int64_t M, int32_t D, int32_t F, size_t* bytes) {
    if (kvx_status st = check_bf16_only(dtype, "swiglu")) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(M >= 0 && M <= INT32_MAX && D > 0 && F > 0 && F <= INT32_MAX / 2,
                "M must be in [0, 2^31), D and F positive");
    *bytes = gemm_split_ws(M, 2 * F, D, EPI_SWIGLU);
    return ok();
}

kvx_status kvx_swiglu(void* stream, int32_t dtype, const void* x, const void* w_gate, const void* w_up, void* h,
                      int64_t M, int32_t D, int32_t F, void* ws, size_t ws_bytes) {
    if (kvx_status st = check_bf16_only(dtype, "swiglu")) return st;
    KVX_REQUIRE(M >= 0 && M <= INT32_MAX, "M must be in [0, 2^31)");
    KVX_REQUIRE(D > 0 && D % 64 == 0, "D must be a positive multiple of 64 (got %d)", D);
    KVX_REQUIRE(F > 0 && F % 8 == 0 && F <= INT32_MAX / 2, "F must be a positive multiple of 8 (got %d)", F);
    if (M == 0) return ok();
    KVX_REQUIRE_PTR(x, "x");
    KVX_REQUIRE_PTR(w_gate, "w_gate");
    KVX_REQUIRE_PTR(w_up, "w_up");
    KVX_REQUIRE_PTR(h, "h");
    const size_t need = gemm_split_ws(M, 2 * F, D, EPI_SWIGLU);
    if (kvx_status st = check_ws(need, ws, ws_bytes, "swiglu")) return st;
    return hip_status(run_swiglu((hipStream_t)stream, x, w_gate, w_up, h, M, D, F, need ? ws : nullptr), "swiglu");
}

kvx_status kvx_target_layer_workspace(int32_t dtype, const kvx_batch* batch, int32_t D, int32_t F, int32_t H_q,
                                      int32_t H_kv, int32_t d_h, size_t* bytes) {
    if (kvx_status st = check_bf16_only(dtype, "target_layer")) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(D > 0 && F > 0 && H_q > 0 && H_kv > 0 && d_h > 0 && F <= INT32_MAX / 2,
                "D, F, H_q, H_kv and d_h must be positive");
    *bytes = layer_ws(bi.n_sel, D, F, H_q, H_kv, d_h, attn_split_bytes(dtype, batch, bi, H_q, H_kv, d_h)).total;
    return ok();
}

kvx_status kvx_target_layer(void* stream, int32_t dtype, int32_t layer, void* x, const kvx_layer_weights* w,
                            int32_t D, int32_t F, int32_t H_q, int32_t H_kv, int32_t d_h, float eps,
                            const float* rope, int32_t max_pos, const kvx_batch* batch, const int32_t* sel,
                            const kvx_cache* cache, void* attn_out, float* lse, void* ws, size_t ws_bytes) {
    if (kvx_status st = check_bf16_only(dtype, "target_layer")) return st;
    if (kvx_status st = check_heads(dtype, H_q, H_kv, d_h)) return st;
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    if (bi.n_req > MAX_ATTN_REQ)
        return fail(KVX_ERR_UNSUPPORTED, "at most %d requests per call (got %d)", MAX_ATTN_REQ, bi.n_req);
    KVX_REQUIRE(D > 0 && D % 64 == 0 && D <= rmsnorm_max_dim(), "D must be a multiple of 64 in [64, %d] (got %d)",
                rmsnorm_max_dim(), D);
    KVX_REQUIRE(F > 0 && F % 64 == 0 && F <= INT32_MAX / 2, "F must be a positive multiple of 64 (got %d)", F);
    KVX_REQUIRE(eps >= 0.f && eps < INFINITY, "eps must be finite and >= 0");
    KVX_REQUIRE(w, "w must not be null");
    KVX_REQUIRE_PTR(w->gamma_in, "w.gamma_in");
    KVX_REQUIRE_PTR(w->w_qkv, "w.w_qkv");
    KVX_REQUIRE_PTR(w->w_o, "w.w_o");
    KVX_REQUIRE_PTR(w->gamma_post, "w.gamma_post");
    KVX_REQUIRE_PTR(w->w_gate, "w.w_gate");
    KVX_REQUIRE_PTR(w->w_up, "w.w_up");
    KVX_REQUIRE_PTR(w->w_down, "w.w_down");
    if (kvx_status st = check_layer_cache(cache, batch, bi, dtype, H_kv, d_h, layer, rope, max_pos)) return st;
    if (bi.n_sel == 0) return ok();
    KVX_REQUIRE(bi.n_sel <= INT32_MAX, "too many selected rows");
    KVX_REQUIRE_PTR(x, "x");
    KVX_REQUIRE_PTR(sel, "sel");
    if (kvx_status st = check_positions_debug(sel, batch, false, "sel")) return st;
    if (attn_out) KVX_REQUIRE(aligned16(attn_out), "attn_out must be 16-byte aligned");
    if (lse) KVX_REQUIRE(aligned16(lse), "lse must be 16-byte aligned");
    const int64_t k = bi.n_sel;
    const size_t attn_split = attn_split_bytes(dtype, batch, bi, H_q, H_kv, d_h);
    const LayerWs L = layer_ws(k, D, F, H_q, H_kv, d_h, attn_split);
    if (!ws || ws_bytes < L.total)
        return fail(KVX_ERR_WORKSPACE, "target_layer needs %zu workspace bytes (got %zu)", L.total, ws_bytes);
    KVX_REQUIRE(aligned16(ws), "ws must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    char* base = (char*)ws;
    bf16* xn = (bf16*)base;
    void* qkv = base + L.xn;
    void* attn = attn_out ? attn_out : (void*)(base + L.xn + L.qkv);
    bf16* mlp = (bf16*)(base + L.xn + L.qkv + L.attn);
    void* split = L.split ? (void*)(base + L.xn + L.qkv + L.attn + L.mlp) : nullptr;
    bf16* xr = (bf16*)x;
    KVX_TRY_HIP(launch_rmsnorm_bf16(xr, (const bf16*)w->gamma_in, eps, k, D, xn, s), "input norm");
    KVX_TRY_HIP(run_qkv_rope_scatter(s, dtype, layer, xn, w->w_qkv, D, H_q, H_kv, d_h, rope, batch, bi, sel, cache,
                                     qkv, split, true), "qkv/rope/scatter");
    KVX_TRY_HIP(run_attention(s, dtype, layer, qkv, H_q, H_kv, d_h, rope, batch, bi, sel, cache, attn, lse,
                              attn_split ? split : nullptr), "attention");
    KVX_TRY_HIP(run_linear_residual(s, attn, w->w_o, xr, xr, k, D, H_q * d_h, split), "output projection");
    KVX_TRY_HIP(launch_rmsnorm_bf16(xr, (const bf16*)w->gamma_post, eps, k, D, xn, s), "post-attention norm");
    KVX_TRY_HIP(run_swiglu(s, xn, w->w_gate, w->w_up, mlp, k, D, F, split), "gate/up");
    return hip_status(run_linear_residual(s, mlp, w->w_down, xr, xr, k, D, F, split), "down projection");
}

kvx_status kvx_linear_workspace(int32_t dtype, int64_t M, int32_t N, int32_t K, size_t* bytes) {
    if (kvx_status st = check_bf16_only(dtype, "linear")) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(M >= 0 && M <= INT32_MAX && N > 0 && K > 0, "M must be in [0, 2^31), N and K positive");
    *bytes = gemm_split_ws(M, N, K, EPI_STORE);
    return ok();
}

kvx_status kvx_linear(void* stream, int32_t dtype, const void* a, const void* w, void* out, int64_t M, int32_t N,
                      int32_t K, void* ws, size_t ws_bytes) {
    if (kvx_status st = check_bf16_only(dtype, "linear")) return st;
    KVX_REQUIRE(M >= 0 && M <= INT32_MAX, "M must be in [0, 2^31)");
    KVX_REQUIRE(N > 0 && N % 8 == 0, "N must be a positive multiple of 8 (got %d)", N);
    KVX_REQUIRE(K > 0 && K % 64 == 0, "K must be a positive multiple of 64 (got %d)", K);
    if (M == 0) return ok();
    KVX_REQUIRE_PTR(a, "a");
    KVX_REQUIRE_PTR(w, "w");
    KVX_REQUIRE_PTR(out, "out");
    const size_t need = gemm_split_ws(M, N, K, EPI_STORE);
    if (kvx_status st = check_ws(need, ws, ws_bytes, "linear")) return st;
    return hip_status(run_linear((hipStream_t)stream, a, w, out, M, N, K, need ? ws : nullptr), "linear");
}

kvx_status kvx_argmax(void* stream, int32_t dtype, const void* logits, int64_t n, int32_t V, int32_t* out) {
    if (kvx_status st = check_bf16_only(dtype, "argmax")) return st;
    KVX_REQUIRE(n >= 0 && n <= INT32_MAX, "n must be in [0, 2^31)");
    KVX_REQUIRE(V > 0, "V must be positive (got %d)", V);
    if (n == 0) return ok();
    KVX_REQUIRE_PTR(logits, "logits");
    KVX_REQUIRE(out && aligned16(out), "out must be a 16-byte aligned pointer");
    return hip_status(launch_argmax_bf16((const bf16*)logits, n, V, out, (hipStream_t)stream), "argmax");
}

}  // extern "C"

namespace {

// Arguments of the direct scoring calls other than the outputs and the workspace.
kvx_status check_score_cache(int32_t dtype, const kvx_cache* cache, int32_t layer0, int32_t n_layers, int32_t H_kv,
                             int32_t d_h, const void* op, int32_t c, const kvx_batch* batch, BatchInfo* bi) {
    if (kvx_status st = check_dtype(dtype)) return st;
    if (kvx_status st = check_batch(batch, bi)) return st;
    KVX_REQUIRE(layer0 >= 0 && n_layers >= 1 && n_layers <= 65535, "need layer0 >= 0 and n_layers in [1, 65535] "
                "(got %d, %d)", layer0, n_layers);
    KVX_REQUIRE(H_kv > 0 && d_h > 0 && d_h % 8 == 0, "H_kv must be positive and d_h a positive multiple of 8");
    KVX_REQUIRE((int64_t)H_kv * d_h <= (1 << 20), "H_kv * d_h too large");
    const int d_t = 2 * H_kv * d_h;
    KVX_REQUIRE(c >= 1 && c <= d_t, "c must be in [1, d_t = %d] (got %d)", d_t, c);
    if (dtype == KVX_BF16) {
        KVX_REQUIRE((H_kv * d_h) % 64 == 0, "bf16 needs H_kv * d_h %% 64 == 0 (got %d)", H_kv * d_h);
        KVX_REQUIRE(c % 8 == 0, "bf16 needs c %% 8 == 0 (got %d)", c);
    } else {
        KVX_REQUIRE(d_t <= 8192, "fp32 needs d_t <= 8192 (got %d)", d_t);
    }
    KVX_REQUIRE_PTR(op, "op");
    if (kvx_status st = check_cache(cache, *bi, dtype, H_kv, d_h, 1)) return st;
    KVX_REQUIRE((int64_t)layer0 + n_layers <= cache->n_layers, "layers [%d, %d) outside the cache's %d layers",
                layer0, layer0 + n_layers, cache->n_layers);
    KVX_REQUIRE(bi->n_tokens <= INT32_MAX, "too many rows");
    KVX_REQUIRE((uintptr_t)cache->k % 16 == 0 && (uintptr_t)cache->v % 16 == 0, "cache.k and cache.v must be "
                "16-byte aligned");
    return check_page_table_debug(cache, batch);
}

size_t score_cache_ws_bytes(int32_t dtype, int32_t n_layers, int32_t c, int64_t n) {
    const int64_t inner = dtype == KVX_BF16 ? cdiv(c, gemm_bf16_block_n()) : 1;
    return round256((size_t)n_layers * inner * n * 4);
}

// Per-layer energies of the scored layers as partials in ws: [n_layers][*n_inner][N].
hipError_t score_cache_parts(hipStream_t s, int32_t dtype, const kvx_cache* cache, int32_t layer0, int32_t n_layers,
                             int32_t H_kv, int32_t d_h, const void* op, int32_t c, const kvx_batch* batch,
                             const BatchInfo& bi, float* parts, int* n_inner) {
    const int hd = H_kv * d_h, d_t = 2 * hd;
    const int64_t layer_elems = cache->n_slots * hd;
    const SlotMap slots = slot_map(cache, batch);
    if (dtype == KVX_F32) {
        *n_inner = 1;
        return launch_score_cache_f32((const float*)cache->k + layer0 * layer_elems,
                                      (const float*)cache->v + layer0 * layer_elems, layer_elems, hd, slots, bi.n_req,
                                      bi.n_tokens, n_layers, (const float*)op, c, parts, s);
    }
    GemmArgs a{};
    a.A = (const bf16*)cache->k + layer0 * layer_elems; a.lda = hd; a.K_a = d_t;
    a.kv_delta = ((int64_t)(uintptr_t)cache->v - (int64_t)(uintptr_t)cache->k) / (int64_t)sizeof(bf16);
    a.kv_split = hd;
    a.a_group_stride = layer_elems;
    a.B = (const bf16*)op; a.ldb = 2 * d_t; a.b_group_stride = (int64_t)c * 2 * d_t;
    a.M = (int)bi.n_tokens; a.N = c; a.K = 2 * d_t; a.groups = n_layers;
    a.rows.mode = 1; a.rows.cu_tok = batch->cu_tokens_d; a.rows.cu_sel = batch->cu_sel_d; a.rows.n_req = bi.n_req;
    a.slots = slots;
    a.epi = EPI_SQNORM; a.partial = parts;
    *n_inner = cdiv(c, gemm_bf16_block_n());
    return launch_gemm_bf16(a, s);
}

}  // namespace

extern "C" {

kvx_status kvx_score_cache_prepare(void* stream, int32_t dtype, const float* u, int32_t n_layers, int32_t d_t,
                                   int32_t c, void* op) {
    if (kvx_status st = check_dtype(dtype)) return st;
    KVX_REQUIRE(n_layers >= 1 && d_t >= 1 && c >= 1 && c <= d_t, "need n_layers >= 1 and 1 <= c <= d_t "
                "(got %d, %d, %d)", n_layers, c, d_t);
    KVX_REQUIRE((int64_t)n_layers * d_t * c <= ((int64_t)1 << 40), "basis too large");
    if (dtype == KVX_BF16) {
        KVX_REQUIRE(d_t % 128 == 0, "bf16 needs d_t %% 128 == 0 (got %d)", d_t);
        KVX_REQUIRE(c % 8 == 0, "bf16 needs c %% 8 == 0 (got %d)", c);
    }
    KVX_REQUIRE_PTR(u, "u");
    KVX_REQUIRE_PTR(op, "op");
    return hip_status(launch_pack_cache_basis(u, n_layers, d_t, c, dtype, op, (hipStream_t)stream),
                      "score_cache_prepare");
}

kvx_status kvx_score_cache_workspace(int32_t dtype, int32_t n_layers, int32_t c, int64_t n, size_t* bytes) {
    if (kvx_status st = check_dtype(dtype)) return st;
    KVX_REQUIRE(bytes, "bytes must not be null");
    KVX_REQUIRE(n_layers >= 1 && c >= 1 && n >= 0 && n <= INT32_MAX, "need n_layers >= 1, c >= 1 and n in [0, 2^31)");
    *bytes = score_cache_ws_bytes(dtype, n_layers, c, n);
    return ok();
}

kvx_status kvx_score_cache(void* stream, int32_t dtype, const kvx_cache* cache, int32_t layer0, int32_t n_layers,
                           int32_t H_kv, int32_t d_h, const void* op, int32_t c, const kvx_batch* batch,
                           float* energy, void* ws, size_t ws_bytes) {
    BatchInfo bi;
    if (kvx_status st = check_score_cache(dtype, cache, layer0, n_layers, H_kv, d_h, op, c, batch, &bi)) return st;
    if (bi.n_tokens == 0) return ok();
    KVX_REQUIRE_PTR(energy, "energy");
    const size_t need = score_cache_ws_bytes(dtype, n_layers, c, bi.n_tokens);
    if (kvx_status st = check_ws(need, ws, ws_bytes, "score_cache")) return st;
    hipStream_t s = (hipStream_t)stream;
    int inner = 0;
    if (dtype == KVX_F32)       // one partial per layer: the energies are written in place
        return hip_status(score_cache_parts(s, dtype, cache, layer0, n_layers, H_kv, d_h, op, c, batch, bi, energy,
                                            &inner),
                          "score_cache");
    KVX_TRY_HIP(score_cache_parts(s, dtype, cache, layer0, n_layers, H_kv, d_h, op, c, batch, bi, (float*)ws, &inner),
                "score_cache");
    return hip_status(launch_sum_parts((const float*)ws, n_layers, inner, bi.n_tokens, true, energy, s),
                      "score_cache (layer sums)");
}

kvx_status kvx_score_cache_select(void* stream, int32_t dtype, const kvx_cache* cache, int32_t layer0,
                                  int32_t n_layers, int32_t H_kv, int32_t d_h, const void* op, int32_t c,
                                  const kvx_batch* batch, const int32_t* budget_pct, float* scores, int32_t* sel,
                                  int32_t* rest, void* ws, size_t ws_bytes) {
    BatchInfo bi;
    if (kvx_status st = check_score_cache(dtype, cache, layer0, n_layers, H_kv, d_h, op, c, batch, &bi)) return st;
    KVX_REQUIRE(budget_pct, "budget_pct must not be null");
    if (kvx_status st = check_budgets(batch, bi, budget_pct)) return st;
    if (bi.n_tokens == 0) return ok();
    KVX_REQUIRE_PTR(scores, "scores");
    if (bi.n_sel > 0) KVX_REQUIRE_PTR(sel, "sel");
    if (bi.n_rest > 0) KVX_REQUIRE_PTR(rest, "rest");
    const size_t need = score_cache_ws_bytes(dtype, n_layers, c, bi.n_tokens);
    if (kvx_status st = check_ws(need, ws, ws_bytes, "score_cache_select")) return st;
    hipStream_t s = (hipStream_t)stream;
    int inner = 0;
    KVX_TRY_HIP(score_cache_parts(s, dtype, cache, layer0, n_layers, H_kv, d_h, op, c, batch, bi, (float*)ws, &inner),
                "score_cache");
    KVX_TRY_HIP(launch_sum_parts((const float*)ws, n_layers, inner, bi.n_tokens, false, scores, s),
                "score_cache (sums)");
    return hip_status(launch_select(nullptr, 0, bi.n_tokens, scores, batch->cu_tokens_d, batch->cu_sel_d, bi.n_req,
                                    sel, rest, s),
                      "select");
}

kvx_status kvx_select_topk_layers(void* stream, const float* scores, int32_t n_layers, const kvx_batch* batch,
                                  int32_t* sel, int32_t* rest) {
    BatchInfo bi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    KVX_REQUIRE(n_layers >= 1 && n_layers <= 65535, "n_layers must be in [1, 65535] (got %d)", n_layers);
    if (bi.n_tokens == 0) return ok();
    KVX_REQUIRE_PTR(scores, "scores");
    if (bi.n_sel > 0) KVX_REQUIRE_PTR(sel, "sel");
    if (bi.n_rest > 0) KVX_REQUIRE_PTR(rest, "rest");
    return hip_status(launch_select(nullptr, 0, bi.n_tokens, (float*)scores, batch->cu_tokens_d, batch->cu_sel_d,
                                    bi.n_req, sel, rest, (hipStream_t)stream, nullptr, 0, n_layers, bi.n_sel),
                      "select_topk_layers");
}

kvx_status kvx_select_pages(void* stream, const float* scores, const kvx_batch* batch, int32_t page_size,
                            const kvx_batch* pages, float* page_scores, int32_t* sel_pages, int32_t* rest_pages,
                            int32_t* cu_sel, int32_t* sel, int32_t* rest) {
    BatchInfo bi, pi;
    if (kvx_status st = check_batch(batch, &bi)) return st;
    if (kvx_status st = check_batch(pages, &pi)) return st;
    KVX_REQUIRE(page_size >= 1, "page_size must be >= 1 (got %d)", page_size);
    KVX_REQUIRE(pages->n_req == batch->n_req, "pages has %d requests, batch %d", pages->n_req, batch->n_req);
    for (int b = 0; b < bi.n_req; ++b) {
        const int64_t T = batch->cu_tokens_h[b + 1] - batch->cu_tokens_h[b];
        const int64_t np = pages->cu_tokens_h[b + 1] - pages->cu_tokens_h[b];
        KVX_REQUIRE(np == (T + page_size - 1) / page_size, "request %d: %lld positions make %lld pages of %d, "
                    "pages gives %lld", b, (long long)T, (long long)((T + page_size - 1) / page_size), page_size,
                    (long long)np);
    }
    KVX_REQUIRE(pi.n_sel * (int64_t)page_size <= INT32_MAX, "too many selected positions");
    KVX_REQUIRE_PTR(cu_sel, "cu_sel");
    if (bi.n_tokens > 0) KVX_REQUIRE_PTR(scores, "scores");
    if (pi.n_tokens > 0) KVX_REQUIRE_PTR(page_scores, "page_scores");
    if (pi.n_sel > 0) {
        KVX_REQUIRE_PTR(sel_pages, "sel_pages");
        KVX_REQUIRE_PTR(sel, "sel");
    }
    if (pi.n_rest > 0) {
        KVX_REQUIRE_PTR(rest_pages, "rest_pages");
        KVX_REQUIRE_PTR(rest, "rest");
    }
    return hip_status(launch_select_pages(scores, batch->cu_tokens_d, bi.n_req, page_size, pages->cu_tokens_d,
                                          pages->cu_sel_d, pi.n_tokens, page_scores, sel_pages, rest_pages, cu_sel, sel,
                                          rest, (hipStream_t)stream),
                      "select_pages");
}

}  // extern "C"
