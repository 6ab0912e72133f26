// Internal definitions shared by the kvx HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvx.h"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

namespace kvx {

// ----------------------------------------------------------------------------- rows
// A row of a flattened [N, ...] activation belongs to request b with cu[b] <= m < cu[b+1].
__device__ __forceinline__ int find_request(const int32_t* cu, int n_req, int m) {
    int lo = 0, hi = n_req - 1;            // largest b in [0, n_req) with cu[b] <= m
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= m) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Complement lists start at cu_tokens[b] - cu_sel[b].
__device__ __forceinline__ int find_request_rest(const int32_t* cu_tok, const int32_t* cu_sel,
                                                 int n_req, int m) {
    int lo = 0, hi = n_req - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu_tok[mid] - cu_sel[mid] <= m) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Cache slot of position p of request b.
struct SlotMap {
    const int32_t* cu_tok;      // device [n_req+1]
    const int32_t* page_table;  // device [n_req][max_pages] (paged) or null
    int32_t max_pages;
    int32_t page_size;
    int32_t page_shift;         // log2(page_size) when it is a power of two, else -1
    int32_t paged;
    __device__ __forceinline__ int64_t slot(int b, int p) const {
        if (paged) {
            const int pi = page_shift >= 0 ? p >> page_shift : p / page_size;
            const int po = page_shift >= 0 ? p & (page_size - 1) : p % page_size;
            const int pg = page_table[(int64_t)b * max_pages + pi];
            return (int64_t)pg * page_size + po;
        }
        return (int64_t)cu_tok[b] + p;
    }
};

// ----------------------------------------------------------------------------- misc
__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }

template <typename T>
__device__ __forceinline__ T ldg(const T* p) { return *p; }

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Chunk swizzle for [rows][8 chunks of 16 B] LDS tiles read 16 consecutive rows at a time
// (one chunk column): chunk c of row r lives at c ^ swz(r).  Chosen by measuring
// ds_read_b128 throughput on gfx950 for this access pattern (Gray code of the row).
__device__ __forceinline__ int swz(int key) { return (key ^ (key >> 1)) & 7; }

// 16-byte direct global -> LDS load of one wave: lane i fills bytes 16i..16i+15 of the 1 KB
// block at dst (M0 holds the block's LDS address).  Written as asm so that the compiler does
// not count it among the LDS events: with such a load in flight it would take the LDS counter
// as out of order and drain every fragment read with lgkmcnt(0).  Callers wait for these loads
// themselves (s_waitcnt) before the barrier that publishes the block.  No register outputs, so
// nothing the compiler allocates can be overwritten while a load is in flight.
__device__ __forceinline__ void lds_dma16(const bf16* src, bf16* dst) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)dst;
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(m0) : "memory");
}

}  // namespace kvx

// ----------------------------------------------------------------------------- launchers
// Host-side launch helpers implemented in the .hip files; the C ABI in kvx_api.hip validates
// arguments before calling them.  Each returns hipSuccess or the launch error.
namespace kvx {

struct RowMap {
    int32_t mode;           // 0: row m is source row m; 1: all rows of a batch; 2: listed rows;
                            // 3: row m is source row m, at the position list[m] (selected rows
                            //    already gathered into a compact matrix)
    const int32_t* list;    // mode 2: request-local positions
    int32_t list_is_rest;   // mode 2: list is a complement list (else a selected list)
    const int32_t* cu_tok;  // device [n_req+1]
    const int32_t* cu_sel;  // device [n_req+1]
    int32_t n_req;
};

// Source row, request and request-local position of GEMM row m.
struct RowInfo { int src, b, pos; };
__device__ __forceinline__ RowInfo row_info(const RowMap& rm, int m) {
    RowInfo r{m, 0, m};
    if (rm.mode == 1) {
        r.b = find_request(rm.cu_tok, rm.n_req, m);
        r.pos = m - rm.cu_tok[r.b];
    } else if (rm.mode == 2) {
        r.b = rm.list_is_rest ? find_request_rest(rm.cu_tok, rm.cu_sel, rm.n_req, m)
                              : find_request(rm.cu_sel, rm.n_req, m);
        r.pos = rm.list[m];
        r.src = rm.cu_tok[r.b] + r.pos;
    } else if (rm.mode == 3) {
        r.b = find_request(rm.cu_sel, rm.n_req, m);
        r.pos = rm.list[m];
    }
    return r;
}

enum EpiKind { EPI_STORE = 0, EPI_CACHE = 1, EPI_SCORE = 2, EPI_QKV = 3, EPI_RESID = 4, EPI_SWIGLU = 5, EPI_F32 = 6,
               EPI_SQNORM = 7 };

struct GemmArgs {
    // C[m][n] = sum_k A[src(m)][k mod K_a] * B[n][k]
    const bf16* A; int64_t lda; int32_t K_a;
    const bf16* B; int64_t ldb; int64_t b_group_stride;
    int32_t M, N, K, groups;
    // independent groups (a_group_stride != 0, EPI_QKV): group g reads its own A rows at
    // A + g * a_group_stride and writes its q columns at C + g * c_group_stride and its K/V into
    // cache layer g (kc, vc + g * layer_elems); the tiles run group by group
    int64_t a_group_stride; int64_t c_group_stride;
    RowMap rows;
    int32_t epi;
    // EPI_STORE (and EPI_F32: C32[m][n] = acc in fp32, leading dimension ldc)
    bf16* C; int64_t ldc; float* C32;
    // EPI_CACHE (group = layer)
    bf16* kc; bf16* vc; int64_t layer_elems; int32_t hd; SlotMap slots;
    // EPI_SCORE: partial[n_block][m] = sum_{n in block} C[m][n] * Z[m][n]
    float* partial; const bf16* Z; int64_t ldz;
    // EPI_STORE / EPI_QKV with a split tail (see gemm_bf16_split_bytes): fp32 K-slice partials
    float* split_ws;
    // EPI_QKV (the gathered QKV projection of one layer): columns [0, q_cols) go to C like a
    // store; the K columns are rounded to bf16, rotated (rotate-half, table rope at the row's
    // position) and written with the V columns to the layer's cache slots (kc, vc, hd, slots).
    // EPI_CACHE with rope set: the K columns [0, hd) rotated the same way before they are stored
    const float* rope; int32_t q_cols; int32_t d_h;
    // EPI_QKV with qk_gain_q set (QK-norm): every q and k head RMS-normalised over its d_h
    // channels (mean square + qk_eps) with the per-channel gains qk_gain_q / qk_gain_k [d_h]
    // before the rotation (the value rounded to bf16 first, as without the normalisation)
    const float* qk_gain_q; const float* qk_gain_k; float qk_eps;
    // EPI_RESID: C[m][n] = R[m][n] + acc (C may be R: every element is read, then written, by
    // one thread)
    const bf16* R; int64_t ldr;
    // EPI_SWIGLU: B row n is row (n/16)*8 + n%8 of the gate weight B (n/8 even) or of the up
    // weight B2 (n/8 odd); C[m][f] = silu(gate_f) * up_f for f = (n/16)*8 + n%8, N = 2F
    const bf16* B2;
    // EPI_SQNORM (direct scoring of a stored cache, independent groups = layers): A row m is the
    // stored vector of row m's cache slot, its columns [0, kv_split) in the K array at A and
    // [kv_split, K_a) in the V array at A + kv_delta (elements); K = 2 K_a, and K step kt reads A
    // columns [(kt/2) BK, (kt/2 + 1) BK) against B columns [kt BK, (kt + 1) BK) (each A chunk
    // twice, once against the high and once against the low bf16 half of the basis).
    // partial[(g * nt + tn) * M + m] = (tn == 0 ? sum_k A[m][k]^2 : 0) - sum_{n in tile} C[m][n]^2
    int64_t kv_delta; int32_t kv_split;
};

// Rotate-half of one pair, in the order every kernel uses (results are bit-identical):
//   first half:  x1 * c - x2 * s        second half:  x2 * c + x1 * s
__device__ __forceinline__ float rope_lo(float x1, float x2, float c, float s) { return __builtin_fmaf(x1, c, -(x2 * s)); }
__device__ __forceinline__ float rope_hi(float x1, float x2, float c, float s) { return __builtin_fmaf(x2, c, x1 * s); }

// Compute units and XCDs of the current device (host side; planners size their work to them)
struct DeviceShape { int cus, xcds; };
DeviceShape device_shape();

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s);
int gemm_bf16_block_n();
// Workspace bytes the bf16 GEMM needs to split its last, partly filled round of tiles along K
// (EPI_STORE, one group); 0 when it runs without a split.
size_t gemm_bf16_split_bytes(int M, int N, int K, int groups, int epi);

}  // namespace kvx
