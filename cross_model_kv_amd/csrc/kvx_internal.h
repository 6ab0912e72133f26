// Launchers of the kvx kernels (internal; the C ABI validates arguments before calling).
#pragma once

#include "kvx_common.h"

namespace kvx {

// ---- fp64 strided GEMM used once per model pair by the score-operator preparation:
//      C[m][n] = (accumulate ? C[m][n] : 0) + alpha * sum_k A(m,k) B(k,n)
//      A(m,k) = A[m*sam + k*sak], B(k,n) = B[k*sbk + n*sbn], C row-major with ldc.
enum ElemType { ET_F32 = 0, ET_BF16 = 1, ET_F64 = 2 };
hipError_t launch_gemm_f64(int M, int N, int K, double alpha, const void* A, int ta, int64_t sam,
                           int64_t sak, const void* B, int tb, int64_t sbk, int64_t sbn, double* C,
                           int64_t ldc, bool accumulate, hipStream_t s);
hipError_t launch_to_f64(const void* src, int t, double* dst, int64_t n, hipStream_t s);
hipError_t launch_zero_f64(double* dst, int64_t n, hipStream_t s);
// op = hi/lo bf16 [r][2r] or fp32 [r][r] from the fp64 operator
hipError_t launch_pack_operator(const double* A, int r, int dtype, void* op, hipStream_t s);

// ---- closed-form fit of the mapper (reduced-rank ridge regression in the n x n Gram space of
//      the calibration positions) and of the calibration subspaces; workspace sizes in bytes
size_t fit_mapper_bytes(int n, int d_src, int m, int r);
size_t fit_calibration_bytes(int n, int d_t, int r, int c);
hipError_t launch_fit_mapper(hipStream_t s, int dtype, const void* x, const void* y, int n, int d_src, int m, int r,
                             double lambda, int iters, void* w_s, void* w_l, void* ws);
hipError_t launch_fit_calibration(hipStream_t s, int dtype, const void* z, const void* w_l, int n, int L, int d_t,
                                  int r, int c, int iters, float* u, void* ws);

// ---- selection: scores[t] = sum_p partial[p][t] (when n_part > 0; divided by
//      sum_p partial2[p][t] when n_part2 > 0, 0 where that is 0), then the k_b largest per
//      request (ties to the lower position) written ascending to sel, the rest to rest.
//      n_layers > 1 (scores only, no partials): scores [n_layers][n_rows], every layer selected
//      on its own into sel [n_layers][n_sel_all] and rest [n_layers][n_rows - n_sel_all].
hipError_t launch_select(const float* partial, int n_part, int64_t n_rows, float* scores,
                         const int32_t* cu_tok, const int32_t* cu_sel, int n_req, int32_t* sel,
                         int32_t* rest, hipStream_t s, const float* partial2 = nullptr, int n_part2 = 0,
                         int n_layers = 1, int64_t n_sel_all = 0);

// ---- direct scoring of a stored cache: the calibration bases packed for the score GEMM (bf16:
//      hi/lo pairs of 64-column chunks, [L][c][2 d_t]; fp32: a copy of u [L][d_t][c]), the fp32
//      path's per-layer energies, and fixed-order sums of per-tile partials
hipError_t launch_pack_cache_basis(const float* u, int L, int d_t, int c, int dtype, void* op, hipStream_t s);
hipError_t launch_score_cache_f32(const float* kc, const float* vc, int64_t layer_elems, int hd, const SlotMap& slots,
                                  int n_req, int64_t M, int L, const float* u, int c, float* energy, hipStream_t s);
hipError_t launch_sum_parts(const float* parts, int n_outer, int n_inner, int64_t M, bool per_outer, float* out,
                            hipStream_t s);

// ---- fp32 variants: QK-norm of the projection rows in place; keys of the listed rows of every
//      layer rotated in place at their positions
hipError_t launch_qknorm_rows_f32(float* qkv, int64_t n_rows, int n_qkv, int H_q, int H_kv, int d_h, const float* gq,
                                  const float* gk, float eps, hipStream_t s);
hipError_t launch_rope_cache_rows_f32(float* kc, int64_t layer_elems, int L, int hd, int d_h, const float* rope,
                                      const RowMap& rm, const SlotMap& sl, int64_t M, hipStream_t s);

// ---- page-granular selection: page scores (sums over aligned pages of ps positions), the top
//      pages per request (select over pages), the selected position counts and the positions
hipError_t launch_select_pages(const float* scores, const int32_t* cu_tok, int n_req, int ps, const int32_t* cu_pages,
                               const int32_t* cu_kpages, int64_t total_pages, float* page_scores, int32_t* sel_pages,
                               int32_t* rest_pages, int32_t* cu_sel, int32_t* sel, int32_t* rest, hipStream_t s);

// ---- rotary table [max_pos][d_h/2][2] (cos, sin), angles in fp64
hipError_t launch_rope_table(double base, int d_h, int max_pos, float* table, hipStream_t s);

// ---- rotate recomputed k and write k, v of every selected row into the layer's cache
struct ScatterArgs {
    const void* qkv; int64_t ld;      // [k][n_qkv]
    int H_q, H_kv, d_h;
    const float* rope;
    const int32_t* sel; const int32_t* cu_sel; int n_req; int64_t n_sel;
    SlotMap slots;
    void* kc; void* vc;               // layer base pointers
};
hipError_t launch_rope_scatter(const ScatterArgs& a, int dtype, hipStream_t s);

// Requests per recompute_attn call: the query-block plan travels in the kernel arguments.
constexpr int MAX_ATTN_REQ = 256;
constexpr int ATTN_KEY_TILE = 64;     // keys per tile of the bf16 attention

struct AttnArgs {
    const void* qkv; int64_t ld;      // Q heads are the first H_q*d_h columns
    int H_q, H_kv, d_h;
    const float* rope;
    const int32_t* sel; const int32_t* cu_sel; int n_req;
    int n_blocks;                     // total query blocks over all requests
    int bq;                           // selected queries per block
    SlotMap slots;
    const void* kc; const void* vc;   // layer base pointers
    void* out; float* lse;
    // key-range split (bf16 path): chunk c of a query block is the c-th run of split_len key
    // tiles counted back from the block's last tile (n_split chunks, one workgroup each,
    // chunk-major: every block's chunk 0 first).  A block of at most split_len tiles is whole in
    // its chunk 0, which writes the final rows; its other chunks are empty and write nothing.
    // Each chunk of a longer block leaves its unnormalised output rows (fp32) in
    // part[(row * n_split + c) * d_h] and (m, l) in part_ml[(row * n_split + c) * 2], row =
    // i * H_q + h, l = 0 for rows without keys in it; a combine kernel merges the chunks of those
    // rows only.  n_split = 1: no split, no partials.
    int n_split; int split_len; float* part; float* part_ml; int64_t n_rows_total;
    // several layers in one launch (bf16, n_split = 1): workgroups run layer by layer; layer j
    // reads its q columns at qkv + j * q_layer_stride and the cache at kc, vc + j * kv_layer_elems,
    // and writes out + j * out_layer_stride, lse + j * lse_layer_stride (elements)
    int n_layers; int64_t q_layer_stride, kv_layer_elems, out_layer_stride, lse_layer_stride;
    int32_t blk_cu[MAX_ATTN_REQ + 1];  // blk_cu[b] = sum_{b' < b} ceil(k_b' / bq)
};
// chunks per query block for the key-range split: round(1.25 * 256 / workgroups) (none when the
// blocks alone fill the CUs), chunks of at least 4 key tiles
int attn_bf16_split(int n_blocks, int H_kv, int max_T);
// fp32 partial workspace of a split attention over n_sel selected rows
size_t attn_bf16_split_bytes(int64_t n_sel, int H_q, int d_h, int n_split);
// bf16 matrix-core path (d_h 64 or 128); returns the number of queries per block it uses
int attn_bf16_block_queries(int g);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
// fp32 path: one wave per (query, head)
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

// ---- fp32 GEMM with the same row maps and epilogues as the bf16 matrix-core GEMM
struct GemmF32Args {
    const float* A; int64_t lda; int32_t K_a;
    const float* B; int64_t ldb; int64_t b_group_stride;
    int32_t M, N, K, groups;
    RowMap rows;
    int32_t epi;                      // EPI_STORE or EPI_CACHE
    float* C; int64_t ldc;
    float* kc; float* vc; int64_t layer_elems; int32_t hd; SlotMap slots;
};
hipError_t launch_gemm_f32(const GemmF32Args& a, hipStream_t s);
// partial[t] = sum_n P[t][n] * Z[t][n]
hipError_t launch_rowdot_f32(const float* P, const float* Z, int64_t n, int r, float* out, hipStream_t s);

// ---- rows of the chained target layer (bf16): RMS normalisation and the gather of the
//      selected rows of a batch into a compact matrix
int rmsnorm_max_dim();
hipError_t launch_rmsnorm_bf16(const bf16* x, const bf16* gamma, float eps, int64_t n, int D, bf16* y,
                               hipStream_t s);
// index of each row's largest logit, ties to the lowest index
hipError_t launch_argmax_bf16(const bf16* logits, int64_t n, int V, int32_t* out, hipStream_t s);
hipError_t launch_gather_rows_bf16(const bf16* src, int D, const int32_t* sel, const int32_t* cu_tok,
                                   const int32_t* cu_sel, int n_req, int64_t n_sel, bf16* dst, hipStream_t s);

}  // namespace kvx
