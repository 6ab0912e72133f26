// Non-matrix-core kernels of the handoff: the fp64 score-operator preparation, the radix
// top-k selection, the rotary table, rotate-and-scatter of recomputed K/V, and the fp32
// storage path (GEMM, row dot, attention).
#include <climits>
#include <math.h>

#include "kvx_internal.h"

namespace kvx {
namespace {

template <typename T> __device__ __forceinline__ double to_d(T x) { return (double)x; }
template <> __device__ __forceinline__ double to_d<bf16>(bf16 x) { return (double)(float)x; }
template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

// =========================================================================== fp64 GEMM
// 64x64 output tile, 16-deep K slices, 256 threads with 4x4 outputs each.  Used once per
// (mapper, calibration) pair, so it favours generality (arbitrary strides and input types).
template <typename TA, typename TB>
__global__ __launch_bounds__(256) void gemm_f64_kernel(int M, int N, int K, double alpha,
                                                       const TA* A, int64_t sam, int64_t sak,
                                                       const TB* B, int64_t sbk, int64_t sbn,
                                                       double* C, int64_t ldc, int accumulate) {
    __shared__ double As[16][65];
    __shared__ double Bs[16][65];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    double acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += 16) {
        for (int e = tid; e < 1024; e += 256) {
            const int mm = e & 63, kk = e >> 6;        // consecutive threads walk m (A) / n (B)
            const int m = m0 + mm, n = n0 + mm, k = k0 + kk;
            As[kk][mm] = (m < M && k < K) ? to_d(A[m * sam + k * sak]) : 0.0;
            Bs[kk][mm] = (n < N && k < K) ? to_d(B[k * sbk + n * sbn]) : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= N) continue;
            double v = alpha * acc[i][j];
            if (accumulate) v += C[m * ldc + n];
            C[m * ldc + n] = v;
        }
    }
}

template <typename T>
__global__ void to_f64_kernel(const T* src, double* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = to_d(src[i]);
}

__global__ void zero_f64_kernel(double* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = 0.0;
}

__global__ void pack_operator_kernel(const double* A, int r, int dtype, void* op) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)r * r) return;
    const double a = A[i];
    if (dtype == KVX_F32) {
        ((float*)op)[i] = (float)a;
        return;
    }
    const int row = (int)(i / r), col = (int)(i % r);
    const bf16 hi = (bf16)(float)a;
    const bf16 lo = (bf16)(float)(a - (double)(float)hi);
    bf16* o = (bf16*)op + (int64_t)row * 2 * r;
    o[col] = hi;
    o[r + col] = lo;
}

// =========================================================================== direct scoring of a stored cache
// Calibration basis for the direct scoring: u [L][d_t][c] fp32 (columns orthonormal).  bf16: the
// score GEMM's B operand [L][c][2 d_t], row j = direction j, its columns in 128-wide pairs of
// chunks: [128 q, 128 q + 64) the bf16-rounded u[64 q + e][j] and [128 q + 64, 128 q + 128) the
// bf16 rounding of what is left (so hi + lo carries u to about 2^-17); fp32: u copied as is.
__global__ void pack_cache_basis_kernel(const float* u, int d_t, int c, int64_t n, int dtype, void* op) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float x = u[i];
    if (dtype == KVX_F32) {
        ((float*)op)[i] = x;
        return;
    }
    const int64_t l = i / ((int64_t)d_t * c);
    const int rem = (int)(i - l * d_t * c);
    const int ch = rem / c, j = rem % c;
    const bf16 hi = (bf16)x;
    const bf16 lo = (bf16)(x - (float)hi);
    bf16* o = (bf16*)op + (l * c + j) * 2 * d_t + (ch >> 6) * 128 + (ch & 63);
    o[0] = hi;
    o[64] = lo;
}

// fp32 cache: one 256-thread block per (position, layer).  The stored vector y = [K heads | V
// heads] of the position's slot goes to LDS; the block sums y_i^2 and, one direction per thread
// in turn, p_j = sum_i y_i u[i][j] (reads of u coalesced over j), then p_j^2; both block sums in
// a fixed order.  energy[l][m] = |y|^2 - |p|^2.
constexpr int DSC_THREADS = 256;
__global__ __launch_bounds__(DSC_THREADS) void score_cache_f32_kernel(const float* kc, const float* vc,
                                                                      int64_t layer_elems, int hd, SlotMap slots,
                                                                      int n_req, const float* u, int c, float* energy,
                                                                      int64_t M) {
    extern __shared__ float s_y[];
    __shared__ float red[2][DSC_THREADS / 64];
    const int m = blockIdx.x, l = blockIdx.y;
    const int b = find_request(slots.cu_tok, n_req, m);
    const int64_t slot = slots.slot(b, m - slots.cu_tok[b]);
    const int d_t = 2 * hd;
    const float* kr = kc + l * layer_elems + slot * hd;
    const float* vr = vc + l * layer_elems + slot * hd;
    float yy = 0.f;
    for (int i = threadIdx.x; i < hd; i += DSC_THREADS) {
        const float a = kr[i], v = vr[i];
        s_y[i] = a;
        s_y[hd + i] = v;
        yy = fmaf(a, a, yy);
        yy = fmaf(v, v, yy);
    }
    __syncthreads();
    const float* ul = u + (int64_t)l * d_t * c;
    float pp = 0.f;
    for (int j = threadIdx.x; j < c; j += DSC_THREADS) {
        float p = 0.f;
        for (int i = 0; i < d_t; ++i) p = fmaf(s_y[i], ul[(int64_t)i * c + j], p);
        pp = fmaf(p, p, pp);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        yy += __shfl_xor(yy, o);
        pp += __shfl_xor(pp, o);
    }
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = yy;
        red[1][threadIdx.x >> 6] = pp;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float ty = 0.f, tp = 0.f;
#pragma unroll
        for (int w = 0; w < DSC_THREADS / 64; ++w) {
            ty += red[0][w];
            tp += red[1][w];
        }
        energy[(int64_t)l * M + m] = ty - tp;
    }
}

// out[o][m] = sum_{i < n_inner} parts[(o * n_inner + i) * M + m] for o < n_outer (per_outer), or
// out[m] = the sum over every o and i (both in ascending order, so the result is deterministic)
__global__ void sum_parts_kernel(const float* parts, int n_outer, int n_inner, int64_t M, int per_outer,
                                 float* out) {
    const int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= M) return;
    if (per_outer) {
        const int o = blockIdx.y;
        float s = 0.f;
        for (int i = 0; i < n_inner; ++i) s += parts[((int64_t)o * n_inner + i) * M + m];
        out[(int64_t)o * M + m] = s;
        return;
    }
    float s = 0.f;
    for (int j = 0; j < n_outer * n_inner; ++j) s += parts[(int64_t)j * M + m];
    out[m] = s;
}

// =========================================================================== fp32 variants
// QK-norm on fp32 projection rows: one wave per (row, q or k head); the head's sum of squares over
// its d_h channels (lanes stride the channels, then a wave tree), x = x * inv * gain with
// inv = 1 / sqrt(mean square + eps), in place; v is left as it is.
__global__ __launch_bounds__(256) void qknorm_rows_f32_kernel(float* qkv, int64_t n_rows, int n_qkv, int H_q,
                                                              int H_kv, int d_h, const float* gq, const float* gk,
                                                              float eps) {
    const int heads = H_q + H_kv;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (item >= n_rows * heads) return;
    const int64_t row = item / heads;
    const int hs = (int)(item - row * heads);
    float* x = qkv + row * n_qkv + (int64_t)hs * d_h;
    const float* g = hs < H_q ? gq : gk;
    float ss = 0.f;
    for (int j = lane; j < d_h; j += 64) ss = fmaf(x[j], x[j], ss);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float inv = 1.f / sqrtf(ss / (float)d_h + eps);
    for (int j = lane; j < d_h; j += 64) x[j] = x[j] * inv * g[j];
}

// Keys of the listed rows rotated in place in every layer of an fp32 cache (the rotary phase of
// a mapper whose keys carry none): thread per (row, layer, rotation pair of one head), rope_lo /
// rope_hi with the table's (cos, sin) at the row's position.
__global__ void rope_cache_rows_f32_kernel(float* kc, int64_t layer_elems, int L, int hd, int d_h, const float* rope,
                                           RowMap rm, SlotMap sl, int64_t M) {
    const int half = d_h / 2, pairs = hd / 2;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= M * L * pairs) return;
    const int p = (int)(i % pairs);
    const int64_t ml = i / pairs;
    const int l = (int)(ml % L);
    const int m = (int)(ml / L);
    const RowInfo ri = row_info(rm, m);
    const int64_t slot = sl.slot(ri.b, ri.pos);
    const int h = p / half, j = p % half;
    float* base = kc + l * layer_elems + slot * hd + (int64_t)h * d_h;
    const float* cs = rope + ((int64_t)ri.pos * half + j) * 2;
    const float x1 = base[j], x2 = base[j + half];
    base[j] = rope_lo(x1, x2, cs[0], cs[1]);
    base[j + half] = rope_hi(x1, x2, cs[0], cs[1]);
}

// =========================================================================== page-granular selection
// Page j of request b holds positions [j ps, min((j + 1) ps, T_b)); one thread per page sums its
// positions' scores in position order.
__global__ void page_scores_kernel(const float* scores, const int32_t* cu_tok, const int32_t* cu_pages, int n_req,
                                   int ps, int64_t total_pages, float* out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= total_pages) return;
    const int b = find_request(cu_pages, n_req, (int)g);
    const int j = (int)g - cu_pages[b];
    const int T = cu_tok[b + 1] - cu_tok[b];
    const int p0 = j * ps, p1 = min(p0 + ps, T);
    const float* sb = scores + cu_tok[b];
    float sum = 0.f;
    for (int p = p0; p < p1; ++p) sum += sb[p];
    out[g] = sum;
}

// cu_sel[b + 1] = cu_sel[b] + positions of request b's selected pages (the last page of a request
// may be short; it is the last of the ascending selected pages when it is selected).  One thread.
__global__ void page_counts_kernel(const int32_t* cu_tok, const int32_t* cu_pages, const int32_t* cu_kpages,
                                   const int32_t* sel_pages, int n_req, int ps, int32_t* cu_sel) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int acc = 0;
    cu_sel[0] = 0;
    for (int b = 0; b < n_req; ++b) {
        const int kp = cu_kpages[b + 1] - cu_kpages[b];
        const int np = cu_pages[b + 1] - cu_pages[b];
        const int T = cu_tok[b + 1] - cu_tok[b];
        int cnt = kp * ps;
        if (kp > 0 && sel_pages[cu_kpages[b] + kp - 1] == np - 1) cnt -= np * ps - T;
        acc += cnt;
        cu_sel[b + 1] = acc;
    }
}

// Positions of request b's selected pages (ascending) at sel + cu_sel[b] and of its other pages at
// rest + cu_tok[b] - cu_sel[b]; entry i * ps + e is position e of the i-th page (only a request's
// last page can be short, and it comes last in either list).  One block per request.
__global__ void expand_pages_kernel(const int32_t* cu_tok, const int32_t* cu_pages, const int32_t* cu_kpages,
                                    const int32_t* sel_pages, const int32_t* rest_pages, const int32_t* cu_sel, int ps,
                                    int32_t* sel, int32_t* rest) {
    const int b = blockIdx.x;
    const int T = cu_tok[b + 1] - cu_tok[b];
    const int kp = cu_kpages[b + 1] - cu_kpages[b];
    const int nr = cu_pages[b + 1] - cu_pages[b] - kp;
    const int32_t* sp = sel_pages + cu_kpages[b];
    const int32_t* rp = rest_pages + (cu_pages[b] - cu_kpages[b]);
    int32_t* so = sel + cu_sel[b];
    int32_t* ro = rest + (cu_tok[b] - cu_sel[b]);
    for (int64_t i = threadIdx.x; i < (int64_t)kp * ps; i += blockDim.x) {
        const int pos = sp[i / ps] * ps + (int)(i % ps);
        if (pos < T) so[i] = pos;
    }
    for (int64_t i = threadIdx.x; i < (int64_t)nr * ps; i += blockDim.x) {
        const int pos = rp[i / ps] * ps + (int)(i % ps);
        if (pos < T) ro[i] = pos;
    }
}

// =========================================================================== select
// One workgroup of 1024 threads per request.  Keys are the fp32 score bits made
// order-preserving as unsigned integers (-0.0 folded onto +0.0).  The k-th largest key is
// found by radix passes of 8 bits over the bits below the common prefix of the request's
// min and max keys; the histogram's top-down cumulative count picks each digit.  Keys equal
// to the k-th are taken lowest position first, then positions are written in ascending
// order with two block-wide prefix sums.  Integer-only after the scores: deterministic.
// The keys are formed once (summing the score GEMM's per-column-block partials) and kept in
// LDS for every later pass when the request has at most SEL_CAP positions (else re-read from
// the scores written by the first pass).
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_CAP = 32768;

__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ int block_excl_scan(int v, int* s_wave, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_wave[w] = x;
    __syncthreads();
    if (w == 0) {
        int t = lane < SEL_WAVES ? s_wave[lane] : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(t, o);
            if (lane >= o) t += y;
        }
        if (lane < SEL_WAVES) s_wave[lane] = t;
    }
    __syncthreads();
    const int base = w > 0 ? s_wave[w - 1] : 0;
    if (total) *total = s_wave[SEL_WAVES - 1];
    __syncthreads();
    return base + x - v;
}

__global__ __launch_bounds__(SEL_THREADS) void select_kernel(const float* partial, int n_part,
                                                            const float* partial2, int n_part2,
                                                            int64_t n_rows, float* scores,
                                                            const int32_t* cu_tok,
                                                            const int32_t* cu_sel, int32_t* sel,
                                                            int32_t* rest, int64_t n_sel_all) {
    __shared__ int hist[SEL_WAVES][256];
    __shared__ uint32_t s_key[SEL_CAP];
    __shared__ int s_wave[SEL_WAVES];
    __shared__ uint32_t s_mm[2][SEL_WAVES];
    __shared__ int s_bc[2];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int b = blockIdx.x;
    // blockIdx.y: the layer of per-layer scores (no partials then), each with its own outputs
    scores += (int64_t)blockIdx.y * n_rows;
    sel += (int64_t)blockIdx.y * n_sel_all;
    rest += (int64_t)blockIdx.y * (n_rows - n_sel_all);
    const int base = cu_tok[b], T = cu_tok[b + 1] - base;
    const int k = cu_sel[b + 1] - cu_sel[b];
    int32_t* so = sel + cu_sel[b];
    int32_t* ro = rest + (base - cu_sel[b]);

    // the score: the sum of the partials, or (n_part2 > 0) that sum over the sum of partial2's
    // partials (0 where the denominator is 0), each sum in partial order
    auto score_at = [&](int t) -> float {
        if (n_part == 0) return scores[base + t];
        float s = 0.f;
        for (int p = 0; p < n_part; ++p) s += partial[(int64_t)p * n_rows + base + t];
        if (n_part2 > 0) {
            float d = 0.f;
            for (int p = 0; p < n_part2; ++p) d += partial2[(int64_t)p * n_rows + base + t];
            s = d > 0.f ? s / d : 0.f;
        }
        return s;
    };
    const bool in_lds = T <= SEL_CAP;
    for (int t = tid; t < T; t += SEL_THREADS) {
        const float sc = score_at(t);
        if (n_part > 0) scores[base + t] = sc;
        if (in_lds) s_key[t] = order_key(sc);
    }
    __syncthreads();
    auto key_at = [&](int t) -> uint32_t { return in_lds ? s_key[t] : order_key(scores[base + t]); };
    if (k == 0) {
        for (int t = tid; t < T; t += SEL_THREADS) ro[t] = t;
        return;
    }
    if (k == T) {
        for (int t = tid; t < T; t += SEL_THREADS) so[t] = t;
        return;
    }

    // common prefix of all keys of this request
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int t = tid; t < T; t += SEL_THREADS) {
        const uint32_t key = key_at(t);
        kmin = min(kmin, key);
        kmax = max(kmax, key);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    }
    if (lane == 0) { s_mm[0][w] = kmin; s_mm[1][w] = kmax; }
    __syncthreads();
    kmin = s_mm[0][0];
    kmax = s_mm[1][0];
    for (int i = 1; i < SEL_WAVES; ++i) { kmin = min(kmin, s_mm[0][i]); kmax = max(kmax, s_mm[1][i]); }
    const uint32_t diff = kmin ^ kmax;
    int nb = diff ? 32 - __clz(diff) : 0;              // bits below the common prefix
    uint32_t prefix = nb == 32 ? 0u : (kmax >> nb) << nb;
    uint32_t mask = nb == 32 ? 0u : ~((1u << nb) - 1u);
    int want = k;                                       // rank from the top among matches

    while (nb > 0) {
        const int d = nb < 8 ? nb : 8;
        const int shift = nb - d;
        const int nbins = 1 << d;
        for (int i = tid; i < SEL_WAVES * 256; i += SEL_THREADS) (&hist[0][0])[i] = 0;
        __syncthreads();
        for (int t = tid; t < T; t += SEL_THREADS) {
            const uint32_t key = key_at(t);
            if ((key & mask) == prefix) atomicAdd(&hist[w][(key >> shift) & (nbins - 1)], 1);
        }
        __syncthreads();
        if (tid < 256) {
            int s = 0;
            for (int i = 0; i < SEL_WAVES; ++i) s += hist[i][tid];
            hist[0][tid] = s;
        }
        __syncthreads();
        if (w == 0) {
            // lane l owns bins top-4l .. top-4l-3 (top = nbins-1), cumulative from the top
            int cnt[4], c = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int bin = nbins - 1 - 4 * lane - q;
                cnt[q] = bin >= 0 ? hist[0][bin] : 0;
                c += cnt[q];
            }
            int cum = c;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(cum, o);
                if (lane >= o) cum += y;
            }
            const unsigned long long hit = __ballot(cum >= want);
            const int L = __ffsll((long long)hit) - 1;
            if (lane == L) {
                int before = cum - c, bin = nbins - 1 - 4 * lane;
                for (int q = 0; q < 4; ++q, --bin) {
                    if (before + cnt[q] >= want) break;
                    before += cnt[q];
                }
                s_bc[0] = bin;
                s_bc[1] = want - before;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)s_bc[0] << shift;
        mask |= (uint32_t)(nbins - 1) << shift;
        want = s_bc[1];
        nb = shift;
        __syncthreads();
    }
    const uint32_t tau = prefix;      // the k-th largest key
    const int take_eq = want;         // how many keys equal to tau are selected

    const int chunk = (T + SEL_THREADS - 1) / SEL_THREADS;
    const int t0 = min(T, tid * chunk), t1 = min(T, t0 + chunk);
    int n_eq = 0;
    for (int t = t0; t < t1; ++t) n_eq += key_at(t) == tau;
    const int eq_before = block_excl_scan(n_eq, s_wave, nullptr);
    int n_take = 0;
    {
        int e = eq_before;
        for (int t = t0; t < t1; ++t) {
            const uint32_t key = key_at(t);
            n_take += key > tau || (key == tau && e++ < take_eq);
        }
    }
    int j = block_excl_scan(n_take, s_wave, nullptr);
    int e = eq_before;
    for (int t = t0; t < t1; ++t) {
        const uint32_t key = key_at(t);
        const bool take = key > tau || (key == tau && e++ < take_eq);
        if (take) so[j++] = t;
        else ro[t - j] = t;
    }
}

// =========================================================================== rope
__global__ void rope_table_kernel(double base, int d_h, int max_pos, float* table) {
    const int half = d_h / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)max_pos * half) return;
    const int p = (int)(idx / half), j = (int)(idx % half);
    const double theta = pow(base, -2.0 * (double)j / (double)d_h);
    const double ang = (double)p * theta;
    table[2 * idx] = (float)cos(ang);
    table[2 * idx + 1] = (float)sin(ang);
}

// fp32: one thread per (selected row, KV head, rotation pair j): rotates k's pair and copies v's
// two elements at j and j + d_h/2
__global__ void rope_scatter_kernel(ScatterArgs a) {
    typedef float TE;
    const int half = a.d_h / 2;
    const int64_t per_row = (int64_t)a.H_kv * half;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= a.n_sel * per_row) return;
    const int i = (int)(idx / per_row);
    const int rem = (int)(idx % per_row);
    const int h = rem / half, j = rem % half;
    const int b = find_request(a.cu_sel, a.n_req, i);
    const int p = a.sel[i];
    const int64_t slot = a.slots.slot(b, p);
    const TE* row = (const TE*)a.qkv + (int64_t)i * a.ld;
    const TE* kr = row + (int64_t)(a.H_q + h) * a.d_h;
    const TE* vr = row + (int64_t)(a.H_q + a.H_kv + h) * a.d_h;
    const float c = a.rope[((int64_t)p * half + j) * 2], s = a.rope[((int64_t)p * half + j) * 2 + 1];
    const float x1 = to_f(kr[j]), x2 = to_f(kr[j + half]);
    TE* kd = (TE*)a.kc + (slot * a.H_kv + h) * a.d_h;
    TE* vd = (TE*)a.vc + (slot * a.H_kv + h) * a.d_h;
    kd[j] = (TE)rope_lo(x1, x2, c, s);
    kd[j + half] = (TE)rope_hi(x1, x2, c, s);
    vd[j] = vr[j];
    vd[j + half] = vr[j + half];
}

// bf16 with 16-byte rows: one thread per (selected row, KV head, run of 8 rotation pairs).  It
// reads 16 bytes of k at j0 and at j0 + d_h/2, the same of v, and the 8 (cos, sin) pairs, and
// writes four 16-byte chunks; the rotation is the same rope_lo / rope_hi as the scalar kernel.
__global__ __launch_bounds__(256) void rope_scatter_vec_kernel(ScatterArgs a) {
    const int half = a.d_h / 2, runs = half / 8;
    const int64_t per_row = (int64_t)a.H_kv * runs;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= a.n_sel * per_row) return;
    const int i = (int)(idx / per_row);
    const int rem = (int)(idx % per_row);
    const int h = rem / runs, j0 = (rem % runs) * 8;
    const int b = find_request(a.cu_sel, a.n_req, i);
    const int p = a.sel[i];
    const int64_t slot = a.slots.slot(b, p);
    const bf16* row = (const bf16*)a.qkv + (int64_t)i * a.ld;
    const bf16* kr = row + (int64_t)(a.H_q + h) * a.d_h + j0;
    const bf16* vr = row + (int64_t)(a.H_q + a.H_kv + h) * a.d_h + j0;
    const bf16x8 k1 = *(const bf16x8*)kr, k2 = *(const bf16x8*)(kr + half);
    const bf16x8 v1 = *(const bf16x8*)vr, v2 = *(const bf16x8*)(vr + half);
    const float4* cs = (const float4*)(a.rope + ((int64_t)p * half + j0) * 2);
    bf16x8 o1, o2;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
        const float4 t = cs[e2];       // (cos, sin) of pairs j0 + 2 e2 and j0 + 2 e2 + 1
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = 2 * e2 + u;
            const float c = u ? t.z : t.x, sn = u ? t.w : t.y;
            const float x1 = (float)k1[e], x2 = (float)k2[e];
            o1[e] = (bf16)rope_lo(x1, x2, c, sn);
            o2[e] = (bf16)rope_hi(x1, x2, c, sn);
        }
    }
    bf16* kd = (bf16*)a.kc + (slot * a.H_kv + h) * a.d_h + j0;
    bf16* vd = (bf16*)a.vc + (slot * a.H_kv + h) * a.d_h + j0;
    *(bf16x8*)kd = o1;
    *(bf16x8*)(kd + half) = o2;
    *(bf16x8*)vd = v1;
    *(bf16x8*)(vd + half) = v2;
}

// =========================================================================== fp32 path
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Args a) {
    __shared__ float As[16][65];
    __shared__ float Bs[16][65];
    __shared__ int s_src[64];
    __shared__ int64_t s_slot[64];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int g = blockIdx.z, m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    if (tid < 64) {
        const int m = m0 + tid;
        int src = -1;
        int64_t slot = 0;
        if (m < a.M) {
            const RowInfo ri = row_info(a.rows, m);
            src = ri.src;
            if (a.epi == EPI_CACHE) slot = a.slots.slot(ri.b, ri.pos);
        }
        s_src[tid] = src;
        s_slot[tid] = slot;
    }
    __syncthreads();
    const float* Bg = a.B + (int64_t)g * a.b_group_stride;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < a.K; k0 += 16) {
        for (int e = tid; e < 1024; e += 256) {
            const int kk = e & 15, mm = e >> 4;         // consecutive threads walk k
            const int k = k0 + kk;
            const int src = s_src[mm];
            As[kk][mm] = (src >= 0 && k < a.K) ? a.A[(int64_t)src * a.lda + k % a.K_a] : 0.f;
            const int n = n0 + mm;
            Bs[kk][mm] = (n < a.N && k < a.K) ? Bg[(int64_t)n * a.ldb + k] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float x[4], y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(x[i], y[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ml = ty * 4 + i;
        if (s_src[ml] < 0) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= a.N) continue;
            if (a.epi == EPI_STORE) {
                a.C[(int64_t)(m0 + ml) * a.ldc + n] = acc[i][j];
            } else {
                const bool is_k = n < a.hd;
                float* dst = (is_k ? a.kc : a.vc) + (int64_t)g * a.layer_elems + s_slot[ml] * a.hd +
                             (is_k ? n : n - a.hd);
                *dst = acc[i][j];
            }
        }
    }
}

// one wave per row: out[t] = sum_n P[t][n] * Z[t][n] in a fixed order
__global__ void rowdot_f32_kernel(const float* P, const float* Z, int64_t n, int r, float* out) {
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= n) return;
    float s = 0.f;
    for (int c = lane; c < r; c += 64) s = fmaf(P[row * r + c], Z[row * r + c], s);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) out[row] = s;
}

// fp32 attention: one wave per (selected query, head).  Keys are spread over the lanes
// (one dot product per lane), the softmax is online over chunks of 64 keys in the log2
// domain, and every lane accumulates the output dims lane and lane + 64.
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
    __shared__ float s_q[4][128];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t item = (int64_t)blockIdx.x * 4 + wv;            // one (row, head) per wave
    if (item >= (int64_t)a.n_blocks * a.H_q) return;               // whole wave leaves
    const int i = (int)(item / a.H_q), h = (int)(item % a.H_q);
    const int g = a.H_q / a.H_kv, hk = h / g;
    const int d_h = a.d_h, half = d_h / 2;
    const int b = find_request(a.cu_sel, a.n_req, i);
    const int p = a.sel[i];
    const float* q = (const float*)a.qkv + (int64_t)i * a.ld + (int64_t)h * d_h;
    if (lane < half) {
        const float c = a.rope[((int64_t)p * half + lane) * 2], s = a.rope[((int64_t)p * half + lane) * 2 + 1];
        const float x1 = q[lane], x2 = q[lane + half];
        s_q[wv][lane] = x1 * c - x2 * s;
        s_q[wv][lane + half] = x2 * c + x1 * s;
    }
    // s_q[wv] is private to this wave: a wave-level barrier orders its LDS writes and reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const float* K = (const float*)a.kc;
    const float* V = (const float*)a.vc;
    const float scale = 1.4426950408889634f / sqrtf((float)d_h);
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int j0 = 0; j0 <= p; j0 += 64) {
        const int j = j0 + lane;
        float x = -INFINITY;
        int64_t slot_j = 0;
        if (j <= p) {
            slot_j = a.slots.slot(b, j);
            const float* kr = K + (slot_j * a.H_kv + hk) * d_h;
            float dot = 0.f;
            for (int d = 0; d < d_h; ++d) dot = fmaf(s_q[wv][d], kr[d], dot);
            x = dot * scale;
        }
        float cm = x;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) cm = fmaxf(cm, __shfl_xor(cm, o));
        const float mn = fmaxf(m, cm);
        const float corr = exp2f(m - mn);
        const float pj = j <= p ? exp2f(x - mn) : 0.f;
        float ps = pj;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ps += __shfl_xor(ps, o);
        l = l * corr + ps;
        o0 *= corr;
        o1 *= corr;
        const int nj = min(64, p + 1 - j0);
        for (int jj = 0; jj < nj; ++jj) {
            const float w = __shfl(pj, jj);
            const int64_t sj = __shfl((long long)slot_j, jj);
            const float* vr = V + (sj * a.H_kv + hk) * d_h;
            o0 = fmaf(w, vr[lane], o0);
            if (lane + 64 < d_h) o1 = fmaf(w, vr[lane + 64], o1);
        }
        m = mn;
    }
    float* out = (float*)a.out + ((int64_t)i * a.H_q + h) * d_h;
    if (lane < d_h) out[lane] = o0 / l;
    if (lane + 64 < d_h) out[lane + 64] = o1 / l;
    if (a.lse && lane == 0) a.lse[(int64_t)i * a.H_q + h] = (m + log2f(l)) * 0.6931471805599453f;
}

}  // namespace

// =========================================================================== target layer rows
namespace {
constexpr int NORM_THREADS = 256;
constexpr int NORM_MAXC = 8;   // 16-byte chunks per thread: D <= 256 * 8 * 8

// y[i] = x[i] / sqrt(mean_j(x[i][j]^2) + eps) * gamma: one row per block, fp32 arithmetic, the
// sum of squares in a fixed order (per-thread chunks, then the wave and block trees)
__global__ __launch_bounds__(NORM_THREADS) void rmsnorm_bf16_kernel(const bf16* x, const bf16* gamma, float eps,
                                                                     int D, bf16* y) {
    __shared__ float red[NORM_THREADS / 64];
    const int64_t row = blockIdx.x;
    const int nch = D / 8;
    const bf16x8* xr = (const bf16x8*)(x + row * D);
    bf16x8 v[NORM_MAXC];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NORM_MAXC; ++c) {
        const int idx = threadIdx.x + c * NORM_THREADS;
        if (idx < nch) {
            v[c] = xr[idx];
#pragma unroll
            for (int j = 0; j < 8; ++j) ss = __builtin_fmaf((float)v[c][j], (float)v[c][j], ss);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NORM_THREADS / 64; ++w) tot += red[w];
    const float inv = 1.f / sqrtf(tot / (float)D + eps);
    const bf16x8* gr = (const bf16x8*)gamma;
    bf16x8* yr = (bf16x8*)(y + row * D);
#pragma unroll
    for (int c = 0; c < NORM_MAXC; ++c) {
        const int idx = threadIdx.x + c * NORM_THREADS;
        if (idx < nch) {
            const bf16x8 g = gr[idx];
            bf16x8 o;
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = (bf16)((float)v[c][j] * inv * (float)g[j]);
            yr[idx] = o;
        }
    }
}

// out[i] = the index of the largest logits[i][j]; ties go to the lowest index (one 1024-thread
// block per row: per-thread scan of 8-element chunks in ascending order, then a wave and a
// block reduction on (value, index))
constexpr int ARGMAX_THREADS = 1024;
__global__ __launch_bounds__(ARGMAX_THREADS) void argmax_bf16_kernel(const bf16* logits, int V, int32_t* out) {
    __shared__ float sv[ARGMAX_THREADS / 64];
    __shared__ int si[ARGMAX_THREADS / 64];
    const bf16* row = logits + (int64_t)blockIdx.x * V;
    float best = -INFINITY;
    int bi = INT_MAX;
    const bool vec = (V % 8) == 0;
    if (vec) {
        for (int c = threadIdx.x; c < V / 8; c += ARGMAX_THREADS) {
            const bf16x8 x = *(const bf16x8*)(row + (int64_t)c * 8);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if ((float)x[j] > best) { best = (float)x[j]; bi = c * 8 + j; }   // first maximum stays
        }
    } else {
        for (int j = threadIdx.x; j < V; j += ARGMAX_THREADS) {
            const float x = (float)row[j];
            if (x > best) { best = x; bi = j; }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
    }
    if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = best; si[threadIdx.x >> 6] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < ARGMAX_THREADS / 64; ++w)
            if (sv[w] > best || (sv[w] == best && si[w] < bi)) { best = sv[w]; bi = si[w]; }
        out[blockIdx.x] = bi == INT_MAX ? 0 : bi;
    }
}

// dst[i] = src[cu_tok[b] + sel[i]] (the selected rows of a batch, compact)
__global__ __launch_bounds__(256) void gather_rows_bf16_kernel(const bf16* src, int D, const int32_t* sel,
                                                                const int32_t* cu_tok, const int32_t* cu_sel,
                                                                int n_req, bf16* dst) {
    const int i = blockIdx.x;
    const int b = find_request(cu_sel, n_req, i);
    const bf16x8* sr = (const bf16x8*)(src + (int64_t)(cu_tok[b] + sel[i]) * D);
    bf16x8* dr = (bf16x8*)(dst + (int64_t)i * D);
    for (int c = threadIdx.x; c < D / 8; c += 256) dr[c] = sr[c];
}

}  // namespace

// =========================================================================== launchers
int rmsnorm_max_dim() { return NORM_THREADS * NORM_MAXC * 8; }

hipError_t launch_rmsnorm_bf16(const bf16* x, const bf16* gamma, float eps, int64_t n, int D, bf16* y,
                               hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (D % 8 || D > rmsnorm_max_dim() || n > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rmsnorm_bf16_kernel, dim3((unsigned)n), dim3(NORM_THREADS), 0, s, x, gamma, eps, D, y);
    return hipGetLastError();
}

hipError_t launch_argmax_bf16(const bf16* logits, int64_t n, int V, int32_t* out, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (n > INT32_MAX || V <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(argmax_bf16_kernel, dim3((unsigned)n), dim3(ARGMAX_THREADS), 0, s, logits, V, out);
    return hipGetLastError();
}

hipError_t launch_gather_rows_bf16(const bf16* src, int D, const int32_t* sel, const int32_t* cu_tok,
                                   const int32_t* cu_sel, int n_req, int64_t n_sel, bf16* dst, hipStream_t s) {
    if (n_sel == 0) return hipSuccess;
    if (D % 8 || n_sel > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gather_rows_bf16_kernel, dim3((unsigned)n_sel), dim3(256), 0, s, src, D, sel, cu_tok, cu_sel,
                       n_req, dst);
    return hipGetLastError();
}

hipError_t launch_gemm_f64(int M, int N, int K, double alpha, const void* A, int ta, int64_t sam,
                           int64_t sak, const void* B, int tb, int64_t sbk, int64_t sbn, double* C,
                           int64_t ldc, bool accumulate, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    dim3 grid(cdiv(N, 64), cdiv(M, 64));
    const int acc = accumulate ? 1 : 0;
#define KVX_F64_CASE(TA_, TB_)                                                                    \
    hipLaunchKernelGGL((gemm_f64_kernel<TA_, TB_>), grid, dim3(256), 0, s, M, N, K, alpha,         \
                       (const TA_*)A, sam, sak, (const TB_*)B, sbk, sbn, C, ldc, acc)
    if (ta == ET_F32 && tb == ET_BF16) KVX_F64_CASE(float, bf16);
    else if (ta == ET_F32 && tb == ET_F32) KVX_F64_CASE(float, float);
    else if (ta == ET_F32 && tb == ET_F64) KVX_F64_CASE(float, double);
    else if (ta == ET_F64 && tb == ET_F64) KVX_F64_CASE(double, double);
    else if (ta == ET_BF16 && tb == ET_F64) KVX_F64_CASE(bf16, double);
    else if (ta == ET_F64 && tb == ET_BF16) KVX_F64_CASE(double, bf16);
    else if (ta == ET_F64 && tb == ET_F32) KVX_F64_CASE(double, float);
    else return hipErrorInvalidValue;
#undef KVX_F64_CASE
    return hipGetLastError();
}

hipError_t launch_to_f64(const void* src, int t, double* dst, int64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (t == ET_BF16) hipLaunchKernelGGL(to_f64_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (const bf16*)src, dst, n);
    else hipLaunchKernelGGL(to_f64_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)src, dst, n);
    return hipGetLastError();
}

hipError_t launch_zero_f64(double* dst, int64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_f64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, n);
    return hipGetLastError();
}

hipError_t launch_pack_operator(const double* A, int r, int dtype, void* op, hipStream_t s) {
    const int64_t n = (int64_t)r * r;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_operator_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, A, r, dtype, op);
    return hipGetLastError();
}

hipError_t launch_select(const float* partial, int n_part, int64_t n_rows, float* scores,
                         const int32_t* cu_tok, const int32_t* cu_sel, int n_req, int32_t* sel,
                         int32_t* rest, hipStream_t s, const float* partial2, int n_part2, int n_layers,
                         int64_t n_sel_all) {
    if (n_req == 0 || n_layers == 0) return hipSuccess;
    if (n_layers > 1 && (n_part > 0 || n_part2 > 0)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(select_kernel, dim3(n_req, n_layers), dim3(SEL_THREADS), 0, s, partial, n_part, partial2,
                       n_part2, n_rows, scores, cu_tok, cu_sel, sel, rest, n_sel_all);
    return hipGetLastError();
}

hipError_t launch_rope_table(double base, int d_h, int max_pos, float* table, hipStream_t s) {
    const int64_t n = (int64_t)max_pos * (d_h / 2);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, base, d_h, max_pos, table);
    return hipGetLastError();
}

hipError_t launch_rope_scatter(const ScatterArgs& a, int dtype, hipStream_t s) {
    const int64_t n = a.n_sel * a.H_kv * (a.d_h / 2);
    if (n == 0) return hipSuccess;
    if (dtype == KVX_BF16) {
        // 16-byte rows: d_h / 2 a multiple of 8 (d_h is 64 or 128) and 16-byte aligned rows and table
        // (the C ABI checks the alignment of every pointer)
        if (a.d_h % 16 != 0 || a.ld % 8 != 0 ||
            ((uintptr_t)a.qkv | (uintptr_t)a.kc | (uintptr_t)a.vc | (uintptr_t)a.rope) % 16 != 0)
            return hipErrorInvalidValue;
        const int64_t nv = n / 8;
        hipLaunchKernelGGL(rope_scatter_vec_kernel, dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL(rope_scatter_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmF32Args& a, hipStream_t s) {
    if (a.M == 0 || a.N == 0 || a.groups == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(cdiv(a.N, 64), cdiv(a.M, 64), a.groups), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_rowdot_f32(const float* P, const float* Z, int64_t n, int r, float* out, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(rowdot_f32_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, P, Z, n, r, out);
    return hipGetLastError();
}

hipError_t launch_pack_cache_basis(const float* u, int L, int d_t, int c, int dtype, void* op, hipStream_t s) {
    const int64_t n = (int64_t)L * d_t * c;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_cache_basis_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, u, d_t, c, n, dtype,
                       op);
    return hipGetLastError();
}

hipError_t launch_score_cache_f32(const float* kc, const float* vc, int64_t layer_elems, int hd, const SlotMap& slots,
                                  int n_req, int64_t M, int L, const float* u, int c, float* energy, hipStream_t s) {
    if (M == 0 || L == 0) return hipSuccess;
    hipLaunchKernelGGL(score_cache_f32_kernel, dim3((unsigned)M, (unsigned)L), dim3(DSC_THREADS),
                       (size_t)2 * hd * sizeof(float), s, kc, vc, layer_elems, hd, slots, n_req, u, c, energy, M);
    return hipGetLastError();
}

hipError_t launch_sum_parts(const float* parts, int n_outer, int n_inner, int64_t M, bool per_outer, float* out,
                            hipStream_t s) {
    if (M == 0 || n_outer == 0) return hipSuccess;
    hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)((M + 255) / 256), per_outer ? n_outer : 1), dim3(256), 0, s,
                       parts, n_outer, n_inner, M, per_outer ? 1 : 0, out);
    return hipGetLastError();
}

hipError_t launch_select_pages(const float* scores, const int32_t* cu_tok, int n_req, int ps, const int32_t* cu_pages,
                               const int32_t* cu_kpages, int64_t total_pages, float* page_scores, int32_t* sel_pages,
                               int32_t* rest_pages, int32_t* cu_sel, int32_t* sel, int32_t* rest, hipStream_t s) {
    if (n_req == 0) return hipSuccess;
    if (total_pages > 0) {
        hipLaunchKernelGGL(page_scores_kernel, dim3((unsigned)((total_pages + 255) / 256)), dim3(256), 0, s, scores,
                           cu_tok, cu_pages, n_req, ps, total_pages, page_scores);
        if (hipError_t e = hipGetLastError()) return e;
        if (hipError_t e = launch_select(nullptr, 0, total_pages, page_scores, cu_pages, cu_kpages, n_req, sel_pages,
                                         rest_pages, s))
            return e;
    }
    hipLaunchKernelGGL(page_counts_kernel, dim3(1), dim3(64), 0, s, cu_tok, cu_pages, cu_kpages, sel_pages, n_req, ps,
                       cu_sel);
    if (hipError_t e = hipGetLastError()) return e;
    hipLaunchKernelGGL(expand_pages_kernel, dim3(n_req), dim3(256), 0, s, cu_tok, cu_pages, cu_kpages, sel_pages,
                       rest_pages, cu_sel, ps, sel, rest);
    return hipGetLastError();
}

hipError_t launch_qknorm_rows_f32(float* qkv, int64_t n_rows, int n_qkv, int H_q, int H_kv, int d_h, const float* gq,
                                  const float* gk, float eps, hipStream_t s) {
    const int64_t items = n_rows * (H_q + H_kv);
    if (items == 0) return hipSuccess;
    hipLaunchKernelGGL(qknorm_rows_f32_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, qkv, n_rows, n_qkv,
                       H_q, H_kv, d_h, gq, gk, eps);
    return hipGetLastError();
}

hipError_t launch_rope_cache_rows_f32(float* kc, int64_t layer_elems, int L, int hd, int d_h, const float* rope,
                                      const RowMap& rm, const SlotMap& sl, int64_t M, hipStream_t s) {
    const int64_t n = M * L * (hd / 2);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_cache_rows_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, kc, layer_elems,
                       L, hd, d_h, rope, rm, sl, M);
    return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
    const int64_t items = (int64_t)a.n_blocks * a.H_q;   // n_blocks = selected rows here
    if (items == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvx
