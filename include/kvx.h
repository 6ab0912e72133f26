/*
 * kvx.h - C ABI of the MI355X (gfx950) cross-model KV handoff library, libkvx.so.
 *
 * The handoff (PANORAMA: Cross-Model KV Sharing via Contextual Recomputation, abstract;
 * RaReCache abstract on the CacheReforge card) runs in four calls:
 *
 *   kvx_map_latent      shared source projection: source KV -> compact latent per position
 *   kvx_score_select    rank-disagreement score of every position, then the top-budget set
 *   kvx_reconstruct     layer-specific reconstruction of the target K/V from the latent
 *   kvx_recompute_attn  per layer: recompute Q/K/V of the selected positions, rotate,
 *                       write K/V into the mixed cache, attend causally over that cache
 *
 * plus two one-time preparations per model pair (kvx_score_prepare, kvx_rope_table)
 * and a standalone top-k (kvx_select_topk).
 *
 * Conventions
 *  - Every call returns a kvx_status (0 = KVX_OK).  On failure nothing is enqueued and
 *    kvx_last_error() returns a message (thread-local; valid until the next call on the
 *    same thread).  No C++ exception crosses this ABI.
 *  - All arguments are validated on the host before any GPU work is enqueued.
 *  - Work is asynchronous on `stream` (a hipStream_t; NULL = the null stream).  Faults
 *    inside kernels surface at the caller's next synchronisation.
 *  - The caller allocates and owns every buffer.  Pointers marked (device) are device
 *    memory, (host) are host memory.  The library never allocates device memory and
 *    keeps no state between calls; calls on distinct streams with distinct buffers may
 *    run concurrently.  Scratch memory is passed explicitly as a workspace whose size
 *    the matching *_workspace() call returns.
 *  - Storage dtype KVX_BF16 or KVX_F32 applies to activations, weights, the latent,
 *    the cache, Q and the attention output; accumulation, softmax and scores are fp32.
 *    Device pointers must be 16-byte aligned; all arrays are dense row-major, the last
 *    index fastest.
 *  - Weights are stored output-major: row j holds the weights that produce output j
 *    (y = W x is computed as y_j = sum_c W[j][c] x[c]).
 *  - Device index data is trusted by the kernels, not checked: a position list (`sel`, or
 *    the complement list `rows`) must be strictly ascending within each request with every
 *    entry in [0, T_b); a paged cache's table must map the pages a request uses to distinct
 *    pages inside the pool; the device prefix arrays must equal the host ones.  Violations
 *    give wrong results or out-of-bounds accesses.  With the environment variable KVX_DEBUG
 *    set (to anything but "" or "0"; read on every call), each call first synchronises the
 *    device, copies these arrays to the host and checks them; a violation returns
 *    KVX_ERR_INVALID with nothing enqueued.
 *
 * Shapes (one request of T positions, or a ragged batch of n_req requests flattened
 * into N = sum T_b rows; positions restart at 0 in every request)
 *   d_src = 2 * L_s * H_s * d_hs     source K and V of all source layers per position,
 *                                    channel order (layer, K/V, head, dim)
 *   r                                latent rank
 *   d_t   = 2 * H_kv * d_h           one target layer's [K heads | V heads], head-major
 *   n_qkv = (H_q + 2 H_kv) * d_h     rows [Q heads | K heads | V heads] of W_qkv
 */
#ifndef KVX_H
#define KVX_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define KVX_API __attribute__((visibility("default")))
#else
#define KVX_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvx_status;
#define KVX_OK 0
#define KVX_ERR_INVALID (-1)     /* bad argument: null pointer, size, alignment, shape */
#define KVX_ERR_UNSUPPORTED (-2) /* valid request this library does not implement */
#define KVX_ERR_HIP (-3)         /* a HIP runtime call or kernel launch failed */
#define KVX_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required */

#define KVX_F32 0
#define KVX_BF16 1

#define KVX_CONTIGUOUS 0
#define KVX_PAGED 1

/* Ragged batch.  Request b owns rows [cu_tokens[b], cu_tokens[b+1]) of every [N, ...]
 * activation and selects k_b = cu_sel[b+1] - cu_sel[b] positions.  The host and device
 * copies must hold the same values; cu_*[0] = 0 and both are non-decreasing.  The
 * complement list of request b starts at cu_tokens[b] - cu_sel[b]. */
typedef struct kvx_batch {
    int32_t n_req;
    const int32_t* cu_tokens_h; /* (host)   [n_req + 1] */
    const int32_t* cu_sel_h;    /* (host)   [n_req + 1] */
    const int32_t* cu_tokens_d; /* (device) [n_req + 1] */
    const int32_t* cu_sel_d;    /* (device) [n_req + 1] */
} kvx_batch;

/* Target KV cache of all layers, K and V in separate arrays of the storage dtype.
 *  KVX_CONTIGUOUS: k, v are [n_layers][n_slots][H_kv][d_h]; position p of request b is
 *                  slot cu_tokens[b] + p (n_slots >= N).
 *  KVX_PAGED:      k, v are [n_layers][n_pages][page_size][H_kv][d_h] (n_slots =
 *                  n_pages * page_size); position p of request b is slot
 *                  page_table[b][p / page_size] * page_size + p % page_size.
 * Distinct (request, position) pairs must map to distinct slots. */
typedef struct kvx_cache {
    int32_t layout;
    void* k;                      /* (device) */
    void* v;                      /* (device) */
    int32_t n_layers;
    int64_t n_slots;
    int32_t page_size;            /* KVX_PAGED only, > 0 */
    int32_t max_pages;            /* KVX_PAGED only: row length of page_table */
    const int32_t* page_table;    /* (device) [n_req][max_pages] int32, KVX_PAGED only */
} kvx_cache;

/* Message of the last failed call on this thread ("" if none). */
KVX_API const char* kvx_last_error(void);

/* Library version string. */
KVX_API const char* kvx_version(void);

/* Recompute budget: k = ceil(pct * T / 100) in integer arithmetic (RaReCache abstract:
 * 30% and 40% of positions are recomputed; rounded up so the budget is never
 * under-spent).  Returns -1 if T < 0 or pct is outside [0, 100]. */
KVX_API int32_t kvx_budget(int32_t T, int32_t pct);

/* Source side of the factorized mapper (PANORAMA abstract: one projection shared by all
 * target layers turns each position's source KV into a short latent vector):
 *   z[t][i] = sum_c w_s[i][c] * x_src[t][c].
 *   x_src (device) [n][d_src], w_s (device) [r][d_src], z (device, out) [n][r].
 *   bf16 needs d_src % 64 == 0 and r % 8 == 0.
 *   ws (device): kvx_map_latent_workspace() bytes.  When the product has too few output
 *   tiles to fill the GPU, tiles are split along d_src into fp32 partial sums that a second
 *   kernel adds in a fixed order (results do not depend on timing).  A size of 0 allows
 *   ws = NULL; a smaller non-zero ws_bytes is KVX_ERR_WORKSPACE. */
KVX_API kvx_status kvx_map_latent_workspace(int32_t dtype, int64_t n, int32_t d_src, int32_t r,
                                            size_t* bytes);
KVX_API kvx_status kvx_map_latent(void* stream, int32_t dtype, const void* x_src, const void* w_s,
                          void* z, int64_t n, int32_t d_src, int32_t r, void* ws, size_t ws_bytes);

/* Score operator of the rank-disagreement metric (RaReCache abstract: energy of the
 * mapped KV in output directions weakly supported by the calibration data).  With
 * R_l = (I - U_l U_l^T) W_l the score of a latent z is
 *   s(z) = sum_l |(I - U_l U_l^T) W_l z|^2 = z^T A z,   A = sum_l R_l^T R_l  (r x r),
 * exact for the linear bias-free mapper.  Computed in fp64 on the device, once per
 * (mapper, calibration) pair.
 *   w_l (device) [L_t][d_t][r] storage dtype; u (device) [L_t][d_t][c] fp32 with
 *   orthonormal columns (c may be 0); op (device, out):
 *     bf16: [r][2r] bf16, row i = [hi(A[i][:]) | lo(A[i][:])] with hi = bf16(A),
 *           lo = bf16(A - hi);
 *     f32:  [r][r] fp32.
 *   ws (device) of kvx_score_prepare_workspace() bytes. */
KVX_API kvx_status kvx_score_prepare_workspace(int32_t r, int32_t d_t, int32_t c, size_t* bytes);
KVX_API kvx_status kvx_score_prepare(void* stream, int32_t dtype, const void* w_l, const float* u,
                             int32_t L_t, int32_t r, int32_t d_t, int32_t c, void* op,
                             void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------------
 * Fitting the mapper and the calibration subspaces (one-time, per model pair, before any
 * handoff).
 *
 * kvx_fit_mapper: closed-form fit of the factorized mapper to paired calibration KV of the two
 * models (PANORAMA abstract: the mapper, a shared source projection and layer-specific
 * reconstructions, is fitted for translation; RaReCache abstract: closed-form linear maps
 * translate KV between models).  Reduced-rank ridge regression: with B the ridge least-squares
 * map from x to y (argmin |x B - y|^2 + lambda |B|^2) and V [L_t d_t][r] an orthonormal basis
 * of the top-r right singular space of the fitted values x B, the fitted mapper is the rank-r
 * map B V V^T, factored as w_s = (B V)^T and w_l = the rows of V of layer l.  The latent is
 * defined up to a rotation: every quantity the handoff uses (mapped KV, composite map, scores)
 * does not depend on it.
 *   x (device) [n][d_src] source KV of n calibration positions (channel order as x_src);
 *   y (device) [n][L_t * d_t] the target's K|V of the same positions, layer-major (layer l is
 *   columns l*d_t .. (l+1)*d_t, [K heads | V heads] as a reconstructed layer);
 *   w_s (device, out) [r][d_src], w_l (device, out) [L_t][d_t][r], storage dtype.
 *   lambda > 0; iters in [1, 10000] block power steps for the singular space (the subspace
 *   error shrinks by the ratio of the (r+1)-th to the r-th squared singular value of x B per
 *   step, so a gap there is needed).  r <= min(n, d_src, L_t d_t).  bf16 needs d_src and
 *   L_t d_t multiples of 64 and n a multiple of 8.  Work and memory are those of n x n
 *   matrices (fp64): ws (device) of kvx_fit_mapper_workspace() bytes. */
KVX_API kvx_status kvx_fit_mapper_workspace(int32_t dtype, int32_t n, int32_t d_src, int32_t L_t, int32_t d_t,
                                            int32_t r, size_t* bytes);
KVX_API kvx_status kvx_fit_mapper(void* stream, int32_t dtype, const void* x, const void* y, int32_t n,
                                  int32_t d_src, int32_t L_t, int32_t d_t, int32_t r, double lambda, int32_t iters,
                                  void* w_s, void* w_l, void* ws, size_t ws_bytes);

/* kvx_fit_calibration: the calibration subspace of every target layer (RaReCache abstract:
 * output directions the calibration data supports): u[l] = an orthonormal basis of the top-c
 * left singular space of the layer's mapped calibration KV (the d_t x n matrix whose column t is
 * w_l z_t), found by iters block power steps on w_l (z^T z) w_l^T in fp64.
 *   z (device) [n][r] latents of the calibration positions (kvx_map_latent of their source KV);
 *   w_l (device) [L_t][d_t][r]; u (device, out) [L_t][d_t][c] fp32, ready for kvx_score_prepare.
 *   c <= min(d_t, r, n); iters in [1, 10000].  ws (device) of kvx_fit_calibration_workspace(). */
KVX_API kvx_status kvx_fit_calibration_workspace(int32_t n, int32_t L_t, int32_t d_t, int32_t r, int32_t c,
                                                 size_t* bytes);
KVX_API kvx_status kvx_fit_calibration(void* stream, int32_t dtype, const void* z, const void* w_l, int32_t n,
                                       int32_t L_t, int32_t d_t, int32_t r, int32_t c, int32_t iters, float* u,
                                       void* ws, size_t ws_bytes);

/* The score as a share (an unranked variant of the RaReCache abstract's score; the pages do not
 * say which): s_t = z_t^T A z_t / z_t^T A_tot z_t, the energy of the token's mapped KV outside the
 * calibration subspaces over the energy of all of it (0 where that is 0), then the selection of
 * kvx_score_select.  op: kvx_score_prepare(w_l, u); op_total: kvx_score_prepare(w_l, none), c = 0
 * (A_tot = sum_l W_l^T W_l), same storage.  Both quadratic forms run on the score GEMM; the ratio
 * and the selection in one pass.  ws (device) of kvx_score_select_normalized_workspace() bytes
 * (twice kvx_score_select's); other arguments as in kvx_score_select. */
KVX_API kvx_status kvx_score_select_normalized_workspace(int32_t dtype, int32_t r, int64_t n, size_t* bytes);
KVX_API kvx_status kvx_score_select_normalized(void* stream, int32_t dtype, const void* z, const void* op,
                                               const void* op_total, int32_t r, const kvx_batch* batch,
                                               const int32_t* budget_pct, float* scores, int32_t* sel,
                                               int32_t* rest, void* ws, size_t ws_bytes);

/* Direct scoring of a stored cache (an unranked variant of the RaReCache abstract's score, for a
 * mapper that is not linear, whose cache has no latent form).  For every scored layer l and every
 * position t of the batch, with y = [K heads | V heads] of t's slot in cache layer layer0 + l (the
 * order kvx_reconstruct splits), the energy outside the calibration subspace:
 *   E[l][t] = |y|^2 - |U_l^T y|^2   (= |(I - U_l U_l^T) y|^2 for orthonormal U_l).
 * kvx_score_cache_prepare packs the bases once:
 *   u (device) [n_layers][d_t][c] fp32, orthonormal columns (the bases of the scored layers, in
 *   order); op (device, out) of 4 * n_layers * d_t * c bytes:
 *     bf16: [n_layers][c][2 d_t] bf16, row j: for every 64-channel chunk q the 64 values bf16(u)
 *           then the 64 values bf16(u - bf16(u)) (the two halves of the score GEMM's operand);
 *     f32:  a copy of u.
 *   bf16 needs d_t % 128 == 0 and c % 8 == 0; c in [1, d_t].
 * kvx_score_cache: energy (device, out) [n_layers][N] fp32.  bf16: one matrix-core GEMM over all
 *   scored layers (the stored rows gathered by slot straight from the cache, each 64-channel chunk
 *   against both halves of the basis; |y|^2 from the same fragments), then a fixed-order sum of its
 *   per-256-direction partials; fp32: one block per (position, layer).  Deterministic.
 *   cache as in kvx_reconstruct (contiguous or paged), layers [layer0, layer0 + n_layers) inside
 *   it; H_kv * d_h = d_t / 2 (bf16: a multiple of 64; fp32: d_t <= 8192); op from
 *   kvx_score_cache_prepare with the same dtype, n_layers, d_t and c; ws (device) of
 *   kvx_score_cache_workspace() bytes (bf16: 4 * n_layers * ceil(c / 256) * N rounded up to 256;
 *   fp32: 4 * n_layers * N rounded up).
 * kvx_score_cache_select: scores (device, out) [N] = sum over the scored layers of E (in layer
 *   order), then the selection of kvx_score_select (budget_pct, sel, rest as there). */
KVX_API kvx_status kvx_score_cache_prepare(void* stream, int32_t dtype, const float* u, int32_t n_layers,
                                           int32_t d_t, int32_t c, void* op);
KVX_API kvx_status kvx_score_cache_workspace(int32_t dtype, int32_t n_layers, int32_t c, int64_t n, size_t* bytes);
KVX_API kvx_status kvx_score_cache(void* stream, int32_t dtype, const kvx_cache* cache, int32_t layer0,
                                   int32_t n_layers, int32_t H_kv, int32_t d_h, const void* op, int32_t c,
                                   const kvx_batch* batch, float* energy, void* ws, size_t ws_bytes);
KVX_API kvx_status kvx_score_cache_select(void* stream, int32_t dtype, const kvx_cache* cache, int32_t layer0,
                                          int32_t n_layers, int32_t H_kv, int32_t d_h, const void* op, int32_t c,
                                          const kvx_batch* batch, const int32_t* budget_pct, float* scores,
                                          int32_t* sel, int32_t* rest, void* ws, size_t ws_bytes);

/* Per-layer selection sets (an unranked variant: every layer recomputes its own positions): the
 * selection of kvx_select_topk applied to each layer's scores on its own.  scores (device)
 * [n_layers][N] fp32, finite (e.g. kvx_score_cache's energies); sel (device, out)
 * [n_layers][cu_sel[n_req]] and rest (device, out) [n_layers][N - cu_sel[n_req]], row l laid out
 * as kvx_select_topk lays out its single set.  Every layer takes cu_sel[b+1] - cu_sel[b] positions
 * of request b.  Row l of sel then serves as the `sel` of layer l's kvx_recompute_attn. */
KVX_API kvx_status kvx_select_topk_layers(void* stream, const float* scores, int32_t n_layers,
                                          const kvx_batch* batch, int32_t* sel, int32_t* rest);

/* Page-granular selection (an unranked variant, after the block-rounded repair sets of the
 * PatchKV abstract on the CacheReforge card): request b's positions fall into pages of page_size
 * consecutive positions (page j = [j * page_size, min((j + 1) * page_size, T_b)), the last one
 * possibly short); a page's score is the sum of its positions' scores (fp32, in position order);
 * the request's k_b pages of largest score (ties to the lower page) are recomputed whole.
 *   scores (device) [N] fp32 position scores, finite; batch: the positions (its cu_sel is not read);
 *   page_size >= 1; pages: a batch over pages with the same n_req, request b holding
 *     ceil(T_b / page_size) pages of which cu_sel gives the k_b selected ones;
 *   page_scores (device, out) [pages.cu_tokens[n_req]] fp32;
 *   sel_pages (device, out) [pages.cu_sel[n_req]], rest_pages (device, out) [the other pages], laid
 *     out as kvx_select_topk lays out positions;
 *   cu_sel (device, out) [n_req + 1]: cu_sel[0] = 0, cu_sel[b + 1] - cu_sel[b] = the positions of
 *     request b's selected pages (k_b * page_size less the shortfall of its last page when that page
 *     is selected), so the selected count is known on the device only;
 *   sel (device, out), room for sum_b k_b * page_size entries: request b's selected positions,
 *     ascending, at cu_sel[b]; rest (device, out), room for N entries: its other positions, ascending,
 *     at cu_tokens[b] - cu_sel[b].
 * A caller copies cu_sel to the host to build the kvx_batch of the following steps. */
KVX_API kvx_status kvx_select_pages(void* stream, const float* scores, const kvx_batch* batch, int32_t page_size,
                                    const kvx_batch* pages, float* page_scores, int32_t* sel_pages,
                                    int32_t* rest_pages, int32_t* cu_sel, int32_t* sel, int32_t* rest);

/* Top-k of given scores per request: the k_b largest scores of request b, ties to the
 * lower position, -0.0 equal to +0.0.  scores (device) [N] fp32, finite.
 * sel (device, out) [cu_sel[n_req]] request-local positions, ascending per request;
 * rest (device, out) [N - cu_sel[n_req]] the complement, ascending per request. */
KVX_API kvx_status kvx_select_topk(void* stream, const float* scores, const kvx_batch* batch,
                           int32_t* sel, int32_t* rest);

/* Rank-disagreement score of every position and the top-budget selection.
 *   z (device) [N][r] latent; op (device) from kvx_score_prepare for the same dtype;
 *   budget_pct (host) [n_req]: must satisfy cu_sel[b+1]-cu_sel[b] = kvx_budget(T_b, pct_b);
 *   scores (device, out) [N] fp32 = z^T A z per position;
 *   sel, rest as in kvx_select_topk; ws (device) of kvx_score_select_workspace() bytes. */
KVX_API kvx_status kvx_score_select_workspace(int32_t dtype, int32_t r, int64_t n, size_t* bytes);
KVX_API kvx_status kvx_score_select(void* stream, int32_t dtype, const void* z, const void* op,
                            int32_t r, const kvx_batch* batch, const int32_t* budget_pct,
                            float* scores, int32_t* sel, int32_t* rest, void* ws,
                            size_t ws_bytes);

/* kvx_score_select without a workspace argument, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and errors as kvx_score_select; its scratch (what
 * kvx_score_select_workspace would return for this call) comes from a fixed array of
 * KVX_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on until the
 * process ends.  A call needing more returns KVX_ERR_WORKSPACE with nothing enqueued (bf16:
 * 4 * N * ceil(r / 256) bytes, e.g. N up to 1M positions at r = 1024; fp32: about 4 * N * (r + 1)).
 * The first call on a device looks up that device's array (with the device current), and it
 * allocates nothing.  All calls on one device share its array, and the scratch of a call is
 * fully written before it is read, so nothing carries over between calls, but calls that
 * overlap in time on one device (concurrent streams, or threads) race on it: serialise them. */
#define KVX_NOALLOC_SCRATCH_BYTES (16u << 20)
KVX_API kvx_status kvx_score_select_noalloc(void* stream, int32_t dtype, const void* z, const void* op,
                                            int32_t r, const kvx_batch* batch, const int32_t* budget_pct,
                                            float* scores, int32_t* sel, int32_t* rest);

/* Layer-specific target reconstruction (PANORAMA abstract) into the translated cache:
 * for every layer l and listed position p of request b,
 *   y = W_l z[cu_tokens[b] + p];  K_l[slot(b,p)] = y[0 : H_kv d_h],
 *                                 V_l[slot(b,p)] = y[H_kv d_h : 2 H_kv d_h].
 *   rows (device) NULL = every position; else the complement list from
 *   kvx_score_select (positions about to be recomputed are skipped: kvx_recompute_attn
 *   overwrites them): [N - cu_sel[n_req]], request b's T_b - k_b entries starting at
 *   cu_tokens[b] - cu_sel[b], strictly ascending, each in [0, T_b).
 *   w_l (device) [L_t][d_t][r].  bf16 needs r % 64 == 0.
 *   cache->n_layers must be >= L_t.  No workspace. */
KVX_API kvx_status kvx_reconstruct(void* stream, int32_t dtype, const void* z, const void* w_l,
                           int32_t L_t, int32_t r, int32_t H_kv, int32_t d_h,
                           const kvx_batch* batch, const int32_t* rows,
                           const kvx_cache* cache);

/* kvx_reconstruct for a mapper whose keys carry no rotary phase (the pages do not say whether
 * translated keys are cache-ready; kvx_reconstruct takes them as they are): every key head of
 * every layer is rotated at its row's position as recomputed keys are (rotate-half, pair
 * (j, j + d_h/2) by angle p * base^(-2j/d_h), the table of kvx_rope_table), V unchanged:
 *   K_l[slot(b,p)] = rope(y[0 : H_kv d_h], p) head by head,  V_l[slot(b,p)] = y[H_kv d_h : ].
 * bf16: each key value is rounded to bf16, rotated in fp32 with its partner and rounded again
 * (the order of the fused QKV projection), in the reconstruction's epilogue; d_h 64 or 128.
 * fp32: the reconstruction, then the listed rows' keys rotated in place in fp32.  rope (device)
 * with max_pos >= every T_b; other arguments as in kvx_reconstruct. */
KVX_API kvx_status kvx_reconstruct_rope(void* stream, int32_t dtype, const void* z, const void* w_l,
                                        int32_t L_t, int32_t r, int32_t H_kv, int32_t d_h,
                                        const float* rope, int32_t max_pos, const kvx_batch* batch,
                                        const int32_t* rows, const kvx_cache* cache);

/* Rotary table for positions [0, max_pos): table[p][j] = (cos, sin)(p * base^(-2j/d_h)),
 * j < d_h/2, angles formed in fp64, stored fp32.  table (device, out) [max_pos][d_h/2][2]. */
KVX_API kvx_status kvx_rope_table(void* stream, double base, int32_t d_h, int32_t max_pos,
                          float* table);

/* Contextual recomputation of one target layer (PANORAMA abstract: the selected positions
 * are recomputed over the full KV cache the mapper produced):
 *   1. [q | k | v]_i = W_qkv x_l[cu_tokens[b] + p_i] for every selected position p_i;
 *   2. q and k rotated (rotate-half: pair (j, j + d_h/2) by angle p_i * base^(-2j/d_h));
 *   3. K[layer][slot(b,p_i)] = k_i, V[layer][slot(b,p_i)] = v_i for all i;
 *   4. after all of step 3, for every i and query head h:
 *      out[i][h] = sum_{j <= p_i} softmax_j(q_ih . K_j / sqrt(d_h)) V_j over KV head
 *      h / (H_q / H_kv) of request b's cache;  lse[i][h] = natural log-sum-exp of the
 *      scaled logits.
 *   x_l (device) [N][D]; w_qkv (device) [n_qkv][D]; rope (device) from kvx_rope_table
 *   with max_pos >= every T_b; sel (device) [cu_sel[n_req]]: request b's k_b positions
 *   start at cu_sel[b], strictly ascending, each in [0, T_b) (the attention takes a query
 *   block's key range from its last entry); out (device, out)
 *   [cu_sel[n_req]][H_q][d_h]; lse (device, out, nullable) [cu_sel[n_req]][H_q] fp32.
 *   d_h must be 64 or 128, H_q % H_kv == 0, H_q / H_kv <= 16; bf16 needs D % 64 == 0.
 *   ws (device) of kvx_recompute_attn_workspace() bytes (the qkv rows, then one region
 *   that serves the projection's split tail and then the attention's key-range split). */
KVX_API kvx_status kvx_recompute_attn_workspace(int32_t dtype, const kvx_batch* batch, int32_t D,
                                        int32_t H_q, int32_t H_kv, int32_t d_h, size_t* bytes);
KVX_API kvx_status kvx_recompute_attn(void* stream, int32_t dtype, int32_t layer, const void* x_l,
                              const void* w_qkv, int32_t D, int32_t H_q, int32_t H_kv,
                              int32_t d_h, const float* rope, int32_t max_pos,
                              const kvx_batch* batch, const int32_t* sel,
                              const kvx_cache* cache, void* out, float* lse, void* ws,
                              size_t ws_bytes);

/* The steps of kvx_recompute_attn as separate calls, for callers that schedule or time them
 * individually.  kvx_recompute_attn is kvx_qkv_rope_scatter followed by kvx_sparse_attention;
 * kvx_qkv_project followed by kvx_rope_scatter gives the same cache and q rows (and also the
 * unrotated k and v columns of qkv).
 *
 * Every step takes `sel` as kvx_recompute_attn does (strictly ascending per request, entries
 * in [0, T_b)).
 *
 * kvx_qkv_project: step 1, qkv (device, out) [cu_sel[n_req]][n_qkv] in the storage dtype,
 *   row i = W_qkv x_l[cu_tokens[b] + sel[i]] (not rotated).  bf16 needs D % 64 == 0.
 *   ws (device): kvx_qkv_project_workspace() bytes, fp32 partial sums of output tiles split
 *   along D (the last, partly filled round of tiles, or every tile when there are too few
 *   to fill the GPU); a second kernel adds the slices in a fixed order, so results do not
 *   depend on timing.  When the size is 0, ws may be NULL; a smaller non-zero ws_bytes is
 *   KVX_ERR_WORKSPACE. */
KVX_API kvx_status kvx_qkv_project_workspace(int32_t dtype, const kvx_batch* batch, int32_t D,
                                             int32_t H_q, int32_t H_kv, int32_t d_h, size_t* bytes);
KVX_API kvx_status kvx_qkv_project(void* stream, int32_t dtype, const void* x_l, const void* w_qkv,
                                   int32_t D, int32_t H_q, int32_t H_kv, int32_t d_h,
                                   const kvx_batch* batch, const int32_t* sel, void* qkv,
                                   void* ws, size_t ws_bytes);

/* kvx_rope_scatter: steps 2-3, rotate the k part of every qkv row at its true position and
 * write k and v into layer `layer` of the cache (slots of the selected positions). */
KVX_API kvx_status kvx_rope_scatter(void* stream, int32_t dtype, int32_t layer, const void* qkv,
                                    int32_t H_q, int32_t H_kv, int32_t d_h, const float* rope,
                                    int32_t max_pos, const kvx_batch* batch, const int32_t* sel,
                                    const kvx_cache* cache);

/* kvx_qkv_rope_scatter: steps 1-3 in one call.  Writes the q part of every qkv row (the k and
 * v columns of qkv are left unwritten) and the rotated k and the v rows into layer `layer` of
 * the cache, with results identical to kvx_qkv_project followed by kvx_rope_scatter (bf16:
 * one kernel, whose epilogue rounds to bf16 and rotates as the separate kernel does; fp32:
 * the two kernels).  Arguments as in kvx_qkv_project and kvx_rope_scatter; ws and its size
 * as in kvx_qkv_project (kvx_qkv_project_workspace). */
KVX_API kvx_status kvx_qkv_rope_scatter(void* stream, int32_t dtype, int32_t layer, const void* x_l,
                                        const void* w_qkv, int32_t D, int32_t H_q, int32_t H_kv,
                                        int32_t d_h, const float* rope, int32_t max_pos,
                                        const kvx_batch* batch, const int32_t* sel,
                                        const kvx_cache* cache, void* qkv, void* ws,
                                        size_t ws_bytes);

/* kvx_qkv_rope_scatter_qknorm: steps 1-3 for a target whose layers normalise q and k per head
 * before the rotation (QK-norm; one of the target families the pages name does, the pages do not
 * describe the block): every q and every k head is divided by the root of its mean square over its
 * d_h channels plus eps and multiplied by the layer's per-channel gain (q_gain, k_gain (device)
 * [d_h] fp32, shared by the layer's heads), k is then rotated and written to the cache with v, and
 * the normalised q is left in qkv for kvx_sparse_attention (which rotates it).  bf16: in the
 * projection's epilogue, each value rounded to bf16 before the normalisation as the plain projection
 * stores it, whole output tiles (no workspace); fp32: the projection, then the q and k heads of the
 * rows normalised in place, then the rotation and scatter.  Other arguments as in
 * kvx_qkv_rope_scatter. */
KVX_API kvx_status kvx_qkv_rope_scatter_qknorm(void* stream, int32_t dtype, int32_t layer, const void* x_l,
                                               const void* w_qkv, int32_t D, int32_t H_q, int32_t H_kv,
                                               int32_t d_h, const float* q_gain, const float* k_gain,
                                               float eps, const float* rope, int32_t max_pos,
                                               const kvx_batch* batch, const int32_t* sel,
                                               const kvx_cache* cache, void* qkv);

/* kvx_sparse_attention: step 4, causal attention of the selected queries (the q part of
 * the qkv rows, rotated at their true positions inside the kernel) over layer `layer` of
 * the cache; out and lse as in kvx_recompute_attn.  d_h must be 64 or 128.
 * ws (device): kvx_sparse_attention_workspace() bytes.  When the query blocks are too few
 * to fill the GPU (bf16), each block's keys are cut into equal chunks that run as separate
 * workgroups; every chunk leaves fp32 partial rows (unnormalised output, maximum and sum) in
 * ws, and a second kernel merges them in chunk order (results do not depend on timing).
 * ws = NULL with ws_bytes = 0 runs without the split (slower on small batches; the result
 * differs from the split one only by rounding); a non-NULL ws must hold the full size. */
KVX_API kvx_status kvx_sparse_attention_workspace(int32_t dtype, const kvx_batch* batch,
                                                  int32_t H_q, int32_t H_kv, int32_t d_h,
                                                  size_t* bytes);
KVX_API kvx_status kvx_sparse_attention(void* stream, int32_t dtype, int32_t layer, const void* qkv,
                                        int32_t H_q, int32_t H_kv, int32_t d_h, const float* rope,
                                        int32_t max_pos, const kvx_batch* batch,
                                        const int32_t* sel, const kvx_cache* cache, void* out,
                                        float* lse, void* ws, size_t ws_bytes);

/* Several target layers in one call: kvx_recompute_attn of layers l0 .. l0 + n_layers - 1
 * (PANORAMA abstract, as above), for the path where every layer recomputes from its own given
 * input rows (x of each layer known up front).  Each layer's attention still reads its cache
 * layer only after all of that layer's k and v are written; layers are independent, so the
 * projections of all n_layers run as one grouped launch and the attentions as another, which
 * fills the GPU when one layer's work would not (few selected positions).
 *   x (device) [n_layers][N][D] (layer j's input at x + j N D); w_qkv (device)
 *   [n_layers][n_qkv][D]; out (device, out) [n_layers][cu_sel[n_req]][H_q][d_h]; lse (device,
 *   out, nullable) [n_layers][cu_sel[n_req]][H_q]; l0 + n_layers <= cache->n_layers; the
 *   other arguments as in kvx_recompute_attn.
 *   No K split in the projections and no key-range split in the attention (bf16): each layer's
 *   results equal, bit for bit, kvx_qkv_rope_scatter and kvx_sparse_attention of that layer
 *   called without workspaces.  fp32: the single-layer kernels, layer by layer.
 *   ws (device) of kvx_recompute_attn_layers_workspace() bytes: the qkv rows of every layer.
 * kvx_qkv_rope_scatter_layers / kvx_sparse_attention_layers: the two launches apart (no
 *   workspace); qkv (device) [n_layers][cu_sel[n_req]][n_qkv], only the q columns written. */
KVX_API kvx_status kvx_recompute_attn_layers_workspace(int32_t dtype, const kvx_batch* batch, int32_t D,
                                                       int32_t H_q, int32_t H_kv, int32_t d_h,
                                                       int32_t n_layers, size_t* bytes);
KVX_API kvx_status kvx_recompute_attn_layers(void* stream, int32_t dtype, int32_t l0, int32_t n_layers,
                                             const void* x, const void* w_qkv, int32_t D, int32_t H_q,
                                             int32_t H_kv, int32_t d_h, const float* rope,
                                             int32_t max_pos, const kvx_batch* batch,
                                             const int32_t* sel, const kvx_cache* cache, void* out,
                                             float* lse, void* ws, size_t ws_bytes);
KVX_API kvx_status kvx_qkv_rope_scatter_layers(void* stream, int32_t dtype, int32_t l0, int32_t n_layers,
                                               const void* x, const void* w_qkv, int32_t D, int32_t H_q,
                                               int32_t H_kv, int32_t d_h, const float* rope,
                                               int32_t max_pos, const kvx_batch* batch,
                                               const int32_t* sel, const kvx_cache* cache, void* qkv);
KVX_API kvx_status kvx_sparse_attention_layers(void* stream, int32_t dtype, int32_t l0, int32_t n_layers,
                                               const void* qkv, int32_t H_q, int32_t H_kv, int32_t d_h,
                                               const float* rope, int32_t max_pos,
                                               const kvx_batch* batch, const int32_t* sel,
                                               const kvx_cache* cache, void* out, float* lse);

/* ---------------------------------------------------------------------------------------
 * Target layer chaining (bf16 only; KVX_ERR_UNSUPPORTED for KVX_F32).  PANORAMA abstract:
 * the recomputed positions let the target model's own computation use the translated
 * context.  The selected rows continue through the rest of each target layer, so layer l+1
 * recomputes its Q/K/V from layer l's output rows instead of from a given input.  The block
 * is the plain pre-norm decoder layer of the pages' target families (the pages name the
 * model pairs, not their blocks):
 *   h  = rmsnorm(x, gamma_in);  q, k, v = W_qkv h (k rotated, k and v written into the
 *   cache, q rotated inside the attention);  o = attention over the mixed cache;
 *   x1 = x + W_o o;  x2 = x1 + W_down (silu(W_gate h2) * (W_up h2)), h2 = rmsnorm(x1, gamma_post)
 * with rmsnorm(x, g)_j = x_j / sqrt(mean(x^2) + eps) * g_j and silu(a) = a / (1 + e^-a).
 * Rows are the compact selected rows of the batch (row i = the i-th entry of sel). */

/* Per-layer weights of the chained block, all (device) bf16, output-major.
 *   gamma_in, gamma_post [D];  w_qkv [n_qkv][D];  w_o [D][H_q * d_h];
 *   w_gate, w_up [F][D];  w_down [D][F]. */
typedef struct kvx_layer_weights {
    const void* gamma_in;
    const void* w_qkv;
    const void* w_o;
    const void* gamma_post;
    const void* w_gate;
    const void* w_up;
    const void* w_down;
} kvx_layer_weights;

/* dst[i] = src[cu_tokens[b] + sel[i]] for every selected row i (request b owning row i):
 * the compact input rows of the chain.  src (device) [N][D], dst (device, out)
 * [cu_sel[n_req]][D]; D % 8 == 0; sel as in kvx_recompute_attn. */
KVX_API kvx_status kvx_gather_rows(void* stream, int32_t dtype, const void* src, int32_t D,
                                   const kvx_batch* batch, const int32_t* sel, void* dst);

/* y[i] = rmsnorm(x[i], gamma) for n rows of width D (fp32 arithmetic, eps under the root).
 * x, y (device) [n][D] (y may be x), gamma (device) [D]; D % 8 == 0, D <= 16384, eps >= 0. */
KVX_API kvx_status kvx_rmsnorm(void* stream, int32_t dtype, const void* x, const void* gamma,
                               float eps, int64_t n, int32_t D, void* y);

/* out = resid + a W^T: a (device) [M][K], w (device) [N][K], resid and out (device) [M][N]
 * (out may be resid: every element is read before it is written, by the same thread).
 * One bf16 rounding of the fp32 sum.  K % 64 == 0, N % 8 == 0.  ws as in kvx_qkv_project
 * (fp32 K-slice partials of a split last round, added in a fixed order). */
KVX_API kvx_status kvx_linear_residual_workspace(int32_t dtype, int64_t M, int32_t N, int32_t K,
                                                 size_t* bytes);
KVX_API kvx_status kvx_linear_residual(void* stream, int32_t dtype, const void* a, const void* w,
                                       const void* resid, void* out, int64_t M, int32_t N,
                                       int32_t K, void* ws, size_t ws_bytes);

/* h = silu(x W_gate^T) * (x W_up^T): x (device) [M][D], w_gate, w_up (device) [F][D],
 * h (device, out) [M][F]; gate and up accumulate in fp32, one bf16 rounding of the product.
 * D % 64 == 0, F % 8 == 0.  ws as in kvx_linear_residual. */
KVX_API kvx_status kvx_swiglu_workspace(int32_t dtype, int64_t M, int32_t D, int32_t F, size_t* bytes);
KVX_API kvx_status kvx_swiglu(void* stream, int32_t dtype, const void* x, const void* w_gate,
                              const void* w_up, void* h, int64_t M, int32_t D, int32_t F,
                              void* ws, size_t ws_bytes);

/* One chained target layer on the selected rows.  x (device, in/out) [cu_sel[n_req]][D]:
 * layer l's input rows on entry, its output rows on return.  Cache, rope, batch and sel as
 * in kvx_recompute_attn (layer `layer` of the cache gets the recomputed k and v).
 * attn_out (device, out, nullable) [cu_sel[n_req]][H_q][d_h] and lse (nullable) as in
 * kvx_recompute_attn.  F % 64 == 0, D % 64 == 0, D <= 16384, eps >= 0.  ws (device) of
 * kvx_target_layer_workspace() bytes: normalised rows, qkv rows, attention rows (when
 * attn_out is NULL), MLP rows, then the largest split workspace of the four projections. */
KVX_API kvx_status kvx_target_layer_workspace(int32_t dtype, const kvx_batch* batch, int32_t D,
                                              int32_t F, int32_t H_q, int32_t H_kv, int32_t d_h,
                                              size_t* bytes);
KVX_API kvx_status kvx_target_layer(void* stream, int32_t dtype, int32_t layer, void* x,
                                    const kvx_layer_weights* w, int32_t D, int32_t F,
                                    int32_t H_q, int32_t H_kv, int32_t d_h, float eps,
                                    const float* rope, int32_t max_pos, const kvx_batch* batch,
                                    const int32_t* sel, const kvx_cache* cache, void* attn_out,
                                    float* lse, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------------
 * First token after the handoff (bf16 only).  The time to first token is the handoff plus
 * one step for the last prompt position: that row runs through every target layer as a
 * one-row kvx_target_layer call (its k and v recomputed over the mixed cache), then the
 * final RMS norm (kvx_rmsnorm), the vocabulary projection (kvx_linear) and kvx_argmax.
 * (RaReCache abstract: time to first token at the target's saturation load; PANORAMA
 * abstract: handoff latency against a full re-prefill.) */

/* out = a W^T: a (device) [M][K], w (device) [N][K], out (device, out) [M][N]; fp32
 * accumulation, one bf16 rounding.  K % 64 == 0, N % 8 == 0.  ws as in kvx_qkv_project
 * (split K-slice partials; for a few rows every output tile is split so that all CUs stream
 * the weight, and only the valid rows of a partial are written). */
KVX_API kvx_status kvx_linear_workspace(int32_t dtype, int64_t M, int32_t N, int32_t K, size_t* bytes);
KVX_API kvx_status kvx_linear(void* stream, int32_t dtype, const void* a, const void* w, void* out,
                              int64_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes);

/* out[i] = index of the largest of logits[i][0..V), ties to the lowest index.
 * logits (device) [n][V]; out (device, out) [n] int32. */
KVX_API kvx_status kvx_argmax(void* stream, int32_t dtype, const void* logits, int64_t n, int32_t V,
                              int32_t* out);

#ifdef __cplusplus
}
#endif

#endif /* KVX_H */
