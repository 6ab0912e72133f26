// Closed-form fit of the factorized mapper and of the calibration subspaces: a one-time
// preparation per model pair, before any handoff.
//
//  * PANORAMA abstract: the mapper is factorized into one shared source projection and a
//    layer-specific reconstruction, and is first fitted for translation alone.  RaReCache
//    abstract: closed-form linear maps translate KV between models of one family.  The fit is
//    reduced-rank ridge regression: the ridge least-squares map B from the source KV x [n, d_src]
//    of n calibration positions to the target KV y [n, m] of all layers (m = L_t d_t, layer-major),
//    truncated to the top-r right singular directions V of its fitted values y^ = x B, and
//    factored as w_s = (B V)^T, w_l = the rows of V that belong to layer l.
//  * RaReCache abstract: the calibration data supports some output directions weakly.  Each
//    layer's calibration subspace is the span of the top-c left singular vectors of the mapped
//    calibration KV (columns w_l z_t), i.e. the top-c eigenspace of w_l (z^T z) w_l^T.
//
// Everything large is a product of n x n matrices (n calibration positions <= d_src), so the fit
// never forms a d_src x d_src or m x m matrix:
//    G = x x^T, K = y y^T                     bf16 matrix-core GEMM with fp32 output (or the fp32
//                                             GEMM), then fp64
//    C = G + lambda I = L L^T                 blocked fp64 Cholesky
//    C^-1 = L^-T L^-1,  H = G C^-1 = I - lambda C^-1   (y^ = H y)
//    M = H K H = y^ y^T                       its top-r eigenspace (subspace iteration with
//                                             Cholesky-QR) is the left singular space Q of y^
//    T = Q^T M Q = L_T L_T^T                  V = y^T H Q L_T^-T has orthonormal columns
//    w_l rows = (y^T R) for R = H Q L_T^-T,   w_s = L_T^-1 (H Q)^T K C^-1 x
// The latent is only defined up to a rotation (every quantity the handoff uses - the mapped KV,
// the composite map, the score - is invariant), so no eigen-decomposition of T is needed: its
// Cholesky factor gives an orthonormal V directly.
#include <math.h>

#include <algorithm>

#include "kvx_internal.h"

namespace kvx {
namespace {

constexpr int NB = 64;        // block size of the fp64 factorizations
constexpr int EW = 256;       // threads of the element-wise kernels

// ---------------------------------------------------------------------------- element-wise
__global__ __launch_bounds__(EW) void gram_to_f64_kernel(const float* g, double* c, int n, double diag) {
    const int64_t i = (int64_t)blockIdx.x * EW + threadIdx.x;
    if (i >= (int64_t)n * n) return;
    c[i] = (double)g[i] + ((i / n == i % n) ? diag : 0.0);
}

// h = delta_ij + alpha * a_ij
__global__ __launch_bounds__(EW) void identity_plus_kernel(const double* a, double alpha, double* h, int n) {
    const int64_t i = (int64_t)blockIdx.x * EW + threadIdx.x;
    if (i >= (int64_t)n * n) return;
    h[i] = alpha * a[i] + ((i / n == i % n) ? 1.0 : 0.0);
}

// dst[r][c] = src[r][c] for a rows x cols block (leading dimensions lds, ldd)
__global__ __launch_bounds__(EW) void copy2d_kernel(const double* src, int lds, double* dst, int ldd, int rows, int cols) {
    const int64_t i = (int64_t)blockIdx.x * EW + threadIdx.x;
    if (i >= (int64_t)rows * cols) return;
    const int r = (int)(i / cols), c = (int)(i % cols);
    dst[(int64_t)r * ldd + c] = src[(int64_t)r * lds + c];
}

__global__ __launch_bounds__(EW) void fill_kernel(double* dst, int64_t n, double v) {
    const int64_t i = (int64_t)blockIdx.x * EW + threadIdx.x;
    if (i < n) dst[i] = v;
}

// strict upper triangle of an n x n matrix (leading dimension ld) set to zero
__global__ __launch_bounds__(EW) void zero_upper_kernel(double* a, int n, int ld) {
    const int64_t i = (int64_t)blockIdx.x * EW + threadIdx.x;
    if (i >= (int64_t)n * n) return;
    const int r = (int)(i / n), c = (int)(i % n);
    if (c > r) a[(int64_t)r * ld + c] = 0.0;
}

// the fixed starting block of the subspace iterations: q[i][j] uniform in [-1, 1) from an
// integer hash of (i, j, salt) (the iterations only need it not to be orthogonal to the wanted
// subspace, which a fixed pseudo-random block is not, except on a set of measure zero)
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
    return x;
}
__global__ __launch_bounds__(EW) void start_block_kernel(double* q, int n, int k, uint32_t salt) {
    const int64_t i = (int64_t)blockIdx.x * EW + threadIdx.x;
    if (i >= (int64_t)n * k) return;
    const uint32_t h = mix32(mix32((uint32_t)(i / k) * 0x9e3779b9u + salt) ^ (uint32_t)(i % k));
    q[i] = (double)h * (2.0 / 4294967296.0) - 1.0;
}

template <typename T>
__global__ __launch_bounds__(EW) void from_f64_kernel(const double* src, T* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * EW + threadIdx.x;
    if (i < n) dst[i] = (T)src[i];
}
template <>
__global__ __launch_bounds__(EW) void from_f64_kernel<bf16>(const double* src, bf16* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * EW + threadIdx.x;
    if (i < n) dst[i] = (bf16)(float)src[i];
}

unsigned blocks_of(int64_t n) { return (unsigned)((n + EW - 1) / EW); }

// ---------------------------------------------------------------------------- Cholesky
// Diagonal block [j0, j0 + jb) of a (jb <= NB): factor it in place (lower) and write the inverse
// of the factor to dinv [jb][NB].  One workgroup; the block lives in LDS.  A pivot that is not
// positive (a matrix that is not positive definite to working precision) is replaced by the
// smallest positive normal number, so that the factor stays finite.
__global__ __launch_bounds__(256) void chol_diag_kernel(double* a, int lda, int j0, int jb, double* dinv) {
    __shared__ double t[NB][NB + 1];
    __shared__ double x[NB][NB + 1];
    const int tid = threadIdx.x;
    for (int e = tid; e < jb * jb; e += 256) {
        const int r = e / jb, c = e % jb;
        t[r][c] = c <= r ? a[(int64_t)(j0 + r) * lda + j0 + c] : 0.0;
    }
    __syncthreads();
    for (int k = 0; k < jb; ++k) {
        if (tid == 0) {
            const double d = t[k][k];
            t[k][k] = d > 0.0 ? sqrt(d) : 2.2250738585072014e-308;
        }
        __syncthreads();
        const double dk = t[k][k];
        for (int r = k + 1 + tid; r < jb; r += 256) t[r][k] /= dk;
        __syncthreads();
        const int rem = jb - k - 1;
        for (int e = tid; e < rem * rem; e += 256) {
            const int r = k + 1 + e / rem, c = k + 1 + e % rem;
            if (c <= r) t[r][c] -= t[r][k] * t[c][k];
        }
        __syncthreads();
    }
    // inverse of the lower-triangular factor, one column per thread (forward substitution)
    if (tid < jb) {
        const int c = tid;
        for (int r = 0; r < jb; ++r) {
            if (r < c) { x[r][c] = 0.0; continue; }
            double v = r == c ? 1.0 : 0.0;
            for (int k = c; k < r; ++k) v -= t[r][k] * x[k][c];
            x[r][c] = v / t[r][r];
        }
    }
    __syncthreads();
    for (int e = tid; e < jb * jb; e += 256) {
        const int r = e / jb, c = e % jb;
        a[(int64_t)(j0 + r) * lda + j0 + c] = c <= r ? t[r][c] : 0.0;
        dinv[(int64_t)r * NB + c] = x[r][c];
    }
}

// C = alpha * op(A) op(B) (+ C), row-major fp64 (op = transpose when the flag is set)
hipError_t mm(hipStream_t s, int M, int N, int K, double alpha, const double* A, bool ta, int64_t lda,
              const double* B, bool tb, int64_t ldb, double* C, int64_t ldc, bool acc) {
    return launch_gemm_f64(M, N, K, alpha, A, ET_F64, ta ? 1 : lda, ta ? lda : 1, B, ET_F64, tb ? 1 : ldb,
                           tb ? ldb : 1, C, ldc, acc, s);
}

#define KVX_HIP(expr)                                   \
    do {                                                \
        hipError_t e_ = (expr);                         \
        if (e_ != hipSuccess) return e_;                \
    } while (0)

// In-place lower Cholesky factor of the SPD matrix a (n x n, leading dimension lda), strict upper
// triangle zeroed.  dinv [n][NB]: inverses of the diagonal blocks; panel: n * NB scratch.
hipError_t chol(hipStream_t s, double* a, int n, int lda, double* dinv, double* panel) {
    for (int j0 = 0; j0 < n; j0 += NB) {
        const int jb = std::min(NB, n - j0);
        hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, s, a, lda, j0, jb, dinv + (int64_t)j0 * NB);
        KVX_HIP(hipGetLastError());
        const int rem = n - j0 - jb;
        if (rem == 0) break;
        double* a21 = a + (int64_t)(j0 + jb) * lda + j0;
        // panel = a21 L_jj^-T, then a21 = panel and a22 -= panel panel^T
        KVX_HIP(mm(s, rem, jb, jb, 1.0, a21, false, lda, dinv + (int64_t)j0 * NB, true, NB, panel, jb, false));
        hipLaunchKernelGGL(copy2d_kernel, dim3(blocks_of((int64_t)rem * jb)), dim3(EW), 0, s, panel, jb, a21, lda,
                           rem, jb);
        KVX_HIP(hipGetLastError());
        KVX_HIP(mm(s, rem, rem, jb, -1.0, panel, false, jb, panel, true, jb, a21 + jb, lda, true));
    }
    hipLaunchKernelGGL(zero_upper_kernel, dim3(blocks_of((int64_t)n * n)), dim3(EW), 0, s, a, n, lda);
    return hipGetLastError();
}

// x = l^-1 for the lower-triangular l (n x n) whose diagonal-block inverses chol left in dinv;
// block forward substitution: x_ii = l_ii^-1, x_ij = -l_ii^-1 sum_{k<i} l_ik x_kj.  tmp: NB * n.
hipError_t trinv(hipStream_t s, const double* l, int n, int ldl, const double* dinv, double* x, int ldx, double* tmp) {
    hipLaunchKernelGGL(fill_kernel, dim3(blocks_of((int64_t)n * ldx)), dim3(EW), 0, s, x, (int64_t)n * ldx, 0.0);
    KVX_HIP(hipGetLastError());
    for (int i0 = 0; i0 < n; i0 += NB) {
        const int ib = std::min(NB, n - i0);
        hipLaunchKernelGGL(copy2d_kernel, dim3(blocks_of((int64_t)ib * ib)), dim3(EW), 0, s,
                           dinv + (int64_t)i0 * NB, NB, x + (int64_t)i0 * ldx + i0, ldx, ib, ib);
        KVX_HIP(hipGetLastError());
        if (i0 == 0) continue;
        KVX_HIP(mm(s, ib, i0, i0, 1.0, l + (int64_t)i0 * ldl, false, ldl, x, false, ldx, tmp, i0, false));
        KVX_HIP(mm(s, ib, i0, ib, -1.0, dinv + (int64_t)i0 * NB, false, NB, tmp, false, i0, x + (int64_t)i0 * ldx, ldx,
                   false));
    }
    return hipSuccess;
}

// Scratch of the small dense steps on k x k matrices and n x k blocks.
struct Small {
    double* a;       // k x k
    double* ainv;    // k x k
    double* dinv;    // max(n, k) x NB
    double* panel;   // max(n, k) x NB
    double* tmp;     // NB x max(n, k)
};

// q (n x k) <- an orthonormal basis of its column span: Cholesky-QR, twice (the second pass
// restores the orthogonality the first loses on ill-conditioned blocks).  w: n x k scratch.
hipError_t orthonormalize(hipStream_t s, double* q, int n, int k, double* w, const Small& sm) {
    for (int pass = 0; pass < 2; ++pass) {
        KVX_HIP(mm(s, k, k, n, 1.0, q, true, k, q, false, k, sm.a, k, false));
        KVX_HIP(chol(s, sm.a, k, k, sm.dinv, sm.panel));
        KVX_HIP(trinv(s, sm.a, k, k, sm.dinv, sm.ainv, k, sm.tmp));
        KVX_HIP(mm(s, n, k, k, 1.0, q, false, k, sm.ainv, true, k, w, k, false));
        hipLaunchKernelGGL(copy2d_kernel, dim3(blocks_of((int64_t)n * k)), dim3(EW), 0, s, w, k, q, k, n, k);
        KVX_HIP(hipGetLastError());
    }
    return hipSuccess;
}

// q (n x k): orthonormal basis of the top-k eigenspace of the symmetric positive semidefinite
// m (n x n), after `iters` block power steps q <- orth(m q) from the fixed start block.
hipError_t top_eigenspace(hipStream_t s, const double* m, int n, int k, int iters, uint32_t salt, double* q, double* w,
                          const Small& sm) {
    hipLaunchKernelGGL(start_block_kernel, dim3(blocks_of((int64_t)n * k)), dim3(EW), 0, s, q, n, k, salt);
    KVX_HIP(hipGetLastError());
    KVX_HIP(orthonormalize(s, q, n, k, w, sm));
    for (int it = 0; it < iters; ++it) {
        KVX_HIP(mm(s, n, k, n, 1.0, m, false, n, q, false, k, w, k, false));
        hipLaunchKernelGGL(copy2d_kernel, dim3(blocks_of((int64_t)n * k)), dim3(EW), 0, s, w, k, q, k, n, k);
        KVX_HIP(hipGetLastError());
        KVX_HIP(orthonormalize(s, q, n, k, w, sm));
    }
    return hipSuccess;
}

// Gram matrix out = a a^T (rows x rows, fp32) of a [rows][cols] in the storage dtype
hipError_t gram(hipStream_t s, int dtype, const void* a, int rows, int cols, float* out) {
    if (dtype == KVX_BF16) {
        GemmArgs g{};
        g.A = (const bf16*)a; g.lda = cols; g.K_a = cols;
        g.B = (const bf16*)a; g.ldb = cols;
        g.M = rows; g.N = rows; g.K = cols; g.groups = 1;
        g.rows.mode = 0;
        g.epi = EPI_F32; g.C32 = out; g.ldc = rows;
        return launch_gemm_bf16(g, s);
    }
    GemmF32Args g{};
    g.A = (const float*)a; g.lda = cols; g.K_a = cols;
    g.B = (const float*)a; g.ldb = cols;
    g.M = rows; g.N = rows; g.K = cols; g.groups = 1;
    g.rows.mode = 0;
    g.epi = EPI_STORE; g.C = out; g.ldc = rows;
    return launch_gemm_f32(g, s);
}

hipError_t store(hipStream_t s, int dtype, const double* src, void* dst, int64_t n) {
    if (dtype == KVX_BF16)
        hipLaunchKernelGGL(from_f64_kernel<bf16>, dim3(blocks_of(n)), dim3(EW), 0, s, src, (bf16*)dst, n);
    else
        hipLaunchKernelGGL(from_f64_kernel<float>, dim3(blocks_of(n)), dim3(EW), 0, s, src, (float*)dst, n);
    return hipGetLastError();
}

size_t al(size_t bytes) { return (bytes + 255) & ~(size_t)255; }

struct MapperWs {
    double *c, *x, *cinv, *h, *k, *m, *dinv, *panel, *tmp, *q, *w, *hq, *rr, *t, *tinv, *sa, *sainv, *sdinv, *spanel,
        *stmp, *s1, *s2, *sf, *ws64, *wl64;
    float* g32;
    size_t bytes;
};

MapperWs carve_mapper(void* base, int n, int d_src, int m, int r) {
    MapperWs w{};
    char* p = (char*)base;
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* q = p ? p + off : nullptr;
        off += al(bytes);
        return q;
    };
    const size_t nn = (size_t)n * n * 8, nr = (size_t)n * r * 8, rr = (size_t)r * r * 8;
    const int big = std::max(n, r);
    w.c = (double*)take(nn); w.x = (double*)take(nn); w.cinv = (double*)take(nn); w.h = (double*)take(nn);
    w.k = (double*)take(nn); w.m = (double*)take(nn);
    w.g32 = (float*)take((size_t)n * n * 4);
    w.dinv = (double*)take((size_t)big * NB * 8); w.panel = (double*)take((size_t)big * NB * 8);
    w.tmp = (double*)take((size_t)NB * big * 8);
    w.q = (double*)take(nr); w.w = (double*)take(nr); w.hq = (double*)take(nr); w.rr = (double*)take(nr);
    w.t = (double*)take(rr); w.tinv = (double*)take(rr); w.sa = (double*)take(rr); w.sainv = (double*)take(rr);
    w.sdinv = (double*)take((size_t)r * NB * 8); w.spanel = (double*)take((size_t)r * NB * 8);
    w.stmp = (double*)take((size_t)NB * r * 8);
    w.s1 = (double*)take(nr); w.s2 = (double*)take(nr); w.sf = (double*)take(nr);
    w.ws64 = (double*)take((size_t)r * d_src * 8);
    w.wl64 = (double*)take((size_t)m * r * 8);
    w.bytes = off;
    return w;
}

struct CalibWs {
    double *z, *gz, *wl, *a1, *sl, *q, *w, *sa, *sainv, *sdinv, *spanel, *stmp;
    size_t bytes;
};

CalibWs carve_calib(void* base, int n, int d_t, int r, int c) {
    CalibWs w{};
    char* p = (char*)base;
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* q = p ? p + off : nullptr;
        off += al(bytes);
        return q;
    };
    const int big = std::max(d_t, c);
    w.z = (double*)take((size_t)n * r * 8);
    w.gz = (double*)take((size_t)r * r * 8);
    w.wl = (double*)take((size_t)d_t * r * 8);
    w.a1 = (double*)take((size_t)d_t * r * 8);
    w.sl = (double*)take((size_t)d_t * d_t * 8);
    w.q = (double*)take((size_t)d_t * c * 8);
    w.w = (double*)take((size_t)d_t * c * 8);
    w.sa = (double*)take((size_t)c * c * 8);
    w.sainv = (double*)take((size_t)c * c * 8);
    w.sdinv = (double*)take((size_t)big * NB * 8);
    w.spanel = (double*)take((size_t)big * NB * 8);
    w.stmp = (double*)take((size_t)NB * big * 8);
    w.bytes = off;
    return w;
}

}  // namespace

size_t fit_mapper_bytes(int n, int d_src, int m, int r) { return carve_mapper(nullptr, n, d_src, m, r).bytes; }

size_t fit_calibration_bytes(int n, int d_t, int r, int c) { return carve_calib(nullptr, n, d_t, r, c).bytes; }

hipError_t launch_fit_mapper(hipStream_t s, int dtype, const void* x, const void* y, int n, int d_src, int m, int r,
                             double lambda, int iters, void* w_s, void* w_l, void* ws) {
    const MapperWs w = carve_mapper(ws, n, d_src, m, r);
    const int et = dtype == KVX_BF16 ? ET_BF16 : ET_F32;
    // C = x x^T + lambda I and K = y y^T
    KVX_HIP(gram(s, dtype, x, n, d_src, w.g32));
    hipLaunchKernelGGL(gram_to_f64_kernel, dim3(blocks_of((int64_t)n * n)), dim3(EW), 0, s, w.g32, w.c, n, lambda);
    KVX_HIP(hipGetLastError());
    KVX_HIP(gram(s, dtype, y, n, m, w.g32));
    hipLaunchKernelGGL(gram_to_f64_kernel, dim3(blocks_of((int64_t)n * n)), dim3(EW), 0, s, w.g32, w.k, n, 0.0);
    KVX_HIP(hipGetLastError());
    // C = L L^T; C^-1 = L^-T L^-1; H = I - lambda C^-1
    const Small big{nullptr, nullptr, w.dinv, w.panel, w.tmp};
    KVX_HIP(chol(s, w.c, n, n, big.dinv, big.panel));
    KVX_HIP(trinv(s, w.c, n, n, big.dinv, w.x, n, big.tmp));
    KVX_HIP(mm(s, n, n, n, 1.0, w.x, true, n, w.x, false, n, w.cinv, n, false));
    hipLaunchKernelGGL(identity_plus_kernel, dim3(blocks_of((int64_t)n * n)), dim3(EW), 0, s, w.cinv, -lambda, w.h, n);
    KVX_HIP(hipGetLastError());
    // M = H K H (the Gram matrix of the fitted values; H K is kept for w_s)
    KVX_HIP(mm(s, n, n, n, 1.0, w.h, false, n, w.k, false, n, w.x, n, false));
    KVX_HIP(mm(s, n, n, n, 1.0, w.x, false, n, w.h, false, n, w.m, n, false));
    // Q: top-r eigenspace of M; T = Q^T M Q = L_T L_T^T
    const Small small{w.sa, w.sainv, w.sdinv, w.spanel, w.stmp};
    KVX_HIP(top_eigenspace(s, w.m, n, r, iters, 0x5eedu, w.q, w.w, small));
    KVX_HIP(mm(s, n, r, n, 1.0, w.m, false, n, w.q, false, r, w.w, r, false));
    KVX_HIP(mm(s, r, r, n, 1.0, w.q, true, r, w.w, false, r, w.t, r, false));
    KVX_HIP(chol(s, w.t, r, r, w.sdinv, w.spanel));
    KVX_HIP(trinv(s, w.t, r, r, w.sdinv, w.tinv, r, w.stmp));
    // R = H Q L_T^-T; w_l rows: y^T R (the reconstruction V = y^ ^T Q L_T^-T, orthonormal columns)
    KVX_HIP(mm(s, n, r, n, 1.0, w.h, false, n, w.q, false, r, w.hq, r, false));
    KVX_HIP(mm(s, n, r, r, 1.0, w.hq, false, r, w.tinv, true, r, w.rr, r, false));
    KVX_HIP(launch_gemm_f64(m, r, n, 1.0, y, et, 1, m, w.rr, ET_F64, r, 1, w.wl64, r, false, s));
    KVX_HIP(store(s, dtype, w.wl64, w_l, (int64_t)m * r));
    // w_s = L_T^-1 (H Q)^T (H K)... with H K C^-1 = (H Q)^T K C^-1 = V^T y^T C^-1 rows: S x
    KVX_HIP(mm(s, r, n, n, 1.0, w.hq, true, r, w.k, false, n, w.s1, n, false));
    KVX_HIP(mm(s, r, n, n, 1.0, w.s1, false, n, w.cinv, false, n, w.s2, n, false));
    KVX_HIP(mm(s, r, n, r, 1.0, w.tinv, false, r, w.s2, false, n, w.sf, n, false));
    KVX_HIP(launch_gemm_f64(r, d_src, n, 1.0, w.sf, ET_F64, n, 1, x, et, d_src, 1, w.ws64, d_src, false, s));
    return store(s, dtype, w.ws64, w_s, (int64_t)r * d_src);
}

hipError_t launch_fit_calibration(hipStream_t s, int dtype, const void* z, const void* w_l, int n, int L, int d_t,
                                  int r, int c, int iters, float* u, void* ws) {
    const CalibWs w = carve_calib(ws, n, d_t, r, c);
    const int et = dtype == KVX_BF16 ? ET_BF16 : ET_F32;
    KVX_HIP(launch_to_f64(z, et, w.z, (int64_t)n * r, s));
    KVX_HIP(mm(s, r, r, n, 1.0, w.z, true, r, w.z, false, r, w.gz, r, false));    // z^T z
    const Small small{w.sa, w.sainv, w.sdinv, w.spanel, w.stmp};
    const size_t es = dtype == KVX_BF16 ? 2 : 4;
    for (int l = 0; l < L; ++l) {
        // S_l = w_l (z^T z) w_l^T: the Gram matrix of the layer's mapped calibration KV
        KVX_HIP(launch_to_f64((const char*)w_l + (size_t)l * d_t * r * es, et, w.wl, (int64_t)d_t * r, s));
        KVX_HIP(mm(s, d_t, r, r, 1.0, w.wl, false, r, w.gz, false, r, w.a1, r, false));
        KVX_HIP(mm(s, d_t, d_t, r, 1.0, w.a1, false, r, w.wl, true, r, w.sl, d_t, false));
        KVX_HIP(top_eigenspace(s, w.sl, d_t, c, iters, 0xca1bu + (uint32_t)l, w.q, w.w, small));
        hipLaunchKernelGGL(from_f64_kernel<float>, dim3(blocks_of((int64_t)d_t * c)), dim3(EW), 0, s, w.q,
                           u + (size_t)l * d_t * c, (int64_t)d_t * c);
        KVX_HIP(hipGetLastError());
    }
    return hipSuccess;
}

}  // namespace kvx
