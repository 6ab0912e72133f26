// Sparse-query causal GQA flash attention for gfx950 (bf16 storage, fp32 softmax/accumulate).
//
// A workgroup serves one KV head of one block of consecutive selected queries of a request (a
// request's first block holds the remainder of its queries over the block size, so the partly
// filled block is the one with the fewest key tiles):
// rows = (query, head) pairs for the g = H_q / H_kv query heads that share the KV head, 32
// rows per wave.  The block walks the request's mixed cache in 64-key tiles up to the
// position of its last query; each row masks keys beyond its own position (inclusive).
//
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K is the A operand (16-byte LDS reads), the
//    rotated Q rows are the B operand held in registers for the whole sweep.  In the result
//    every lane holds 16 keys of one row, so the online softmax needs only lane-local work
//    and one exchange with lane ^ 32.
//  * O^T = V^T P^T: P comes straight from the S^T registers (bf16), V^T fragments are read
//    from the row-major V tile with ds_read_b64_tr_b16, and the output rows stay lane-local,
//    so the rescale by exp2(m_old - m_new) needs no cross-lane traffic.
//  * K and V tiles are double-buffered in LDS with per-row XOR-swizzled 16-byte chunks and
//    arrive by direct global -> LDS loads (global_load_lds_dwordx4): each wave fills whole
//    1 KB blocks, every lane fetching the chunk that belongs at its slot; the next tile's
//    loads are in flight while the current tile is consumed.  Keys past the request's end
//    load key 0 instead (finite data; such keys are always masked).  The direct loads are
//    issued from asm and waited for before each barrier, so the fragment reads stay alone on
//    the LDS counter and the look-ahead reads are waited for one at a time.
//  * q is rotated (rotate-half, table angles at the query's true position) and scaled by
//    log2(e)/sqrt(d_h) while it is loaded; k was rotated when it was scattered into the cache.
//    The q rows arrive whole (16 bytes per lane, several rows per load) through LDS rather than
//    as fragments, which would read 32 bytes of each of 32 rows per load.
//  * VALU work per tile is kept small, because on gfx950 a wave's VALU instructions do not
//    overlap its own MFMAs: the causal mask runs only on tiles that reach past the smallest
//    query position of the wave; the scores leave the MFMAs already shifted by a reference
//    maximum (the accumulators start at -m_ref); the row sum is a packed bf16 dot product of
//    the rounded P that the MFMA consumes (so O and l use the same weights; four independent
//    partial sums, since one serial chain of 16 dependent dot products measured 2.5% slower),
//    kept per lane until the end.  The common tile is exp2, bf16 packing and 16 dot products; only when a
//    lane sum exceeds 2^16 (a score far above m_ref) does a slow path take the true maximum
//    and rescale O and l (the ratio O / l does not depend on the reference used); a wave's
//    first tile, with no reference yet, goes to that path directly.
//  * Paged caches run their own instance (PG): the request's page-table entries are staged in
//    LDS once and each tile's block pages are read from there by the instance whose loads know
//    it is LDS (a pointer that could be either LDS or global memory is read with flat loads,
//    which wait on both memory counters); contiguous caches keep their instance unchanged.
//  * The normalised output rows leave through LDS: each wave writes its 32 rows into its own
//    slice of the idle K/V stages and stores whole rows, 16 bytes per lane (the accumulator
//    layout would store 8 bytes to each of 32 rows per instruction, which measured slower for
//    the short workgroups of 4K requests).
//  * Query blocks are issued longest-first, and the KV head is the fastest-varying workgroup
//    index so that, with 8 KV heads, every XCD streams one head's K/V through its own L2.
//  * With fewer blocks than CUs the keys of the long blocks are cut into runs counted back
//    from the block's last tile: a block short enough for one run is done by its chunk 0,
//    which writes the final rows; each run of a longer block writes fp32 partial rows that
//    attn_combine_kernel merges.  Workgroups go chunk-major (every block's chunk 0 first).
#include <algorithm>
#include <climits>

#include "kvx_internal.h"

namespace kvx {
namespace {

constexpr int KT = ATTN_KEY_TILE;

// LDS fragment reads kept in flight ahead of the MFMAs that consume them (measured best)
constexpr int PF_K = 4;   // K fragments (one per MFMA)
constexpr int PF_V = 8;   // transposed V reads (two per MFMA)
constexpr int PT_MAX = 2048;   // page-table entries staged in LDS (longer requests read it from HBM)

// Chunk swizzle of the K/V tiles, chosen by measuring gfx950 LDS throughput for both reads
// of a tile: ds_read_b128 of 32 consecutive keys (K) and ds_read_b64_tr_b16 of 8 keys x 64 B
// (V).  For 8-chunk rows (d_h = 64) the 16-row pattern swizzle is used.
template <int D_H>
__device__ __forceinline__ int kv_swz(int key) {
    if constexpr (D_H == 128) return (key & 15) ^ ((key & 3) << 2);
    else return swz(key);
}

template <int D_H, int W, bool PG>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(AttnArgs a) {
    constexpr int NT = W * 64;
    constexpr int NCH = D_H / 8;               // 16-byte chunks per K/V row
    constexpr int QC = D_H / 16;               // 16-deep k-steps of S^T = K Q^T
    constexpr int DB = D_H / 32;               // 32-wide output blocks
    constexpr int TILE = KT * D_H;             // elements of one K (or V) tile
    constexpr int KPB = 1024 / (2 * D_H);      // keys per 1 KB block
    constexpr int NBLK = 2 * TILE * 2 / 1024;  // 1 KB blocks of a K+V tile
    __shared__ __attribute__((aligned(1024))) bf16 lds0[2 * TILE];
    __shared__ __attribute__((aligned(1024))) bf16 lds1[2 * TILE];
    __shared__ int32_t s_pt[PT_MAX];           // the request's page table (paged caches)
    __shared__ __attribute__((aligned(16))) bf16 s_q[W * 32 * D_H];   // q rows on their way to the fragments

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const int hf = lane >> 5, lr = lane & 31;
    const int H_kv = a.H_kv, g = a.H_q / H_kv;
    // layer of this workgroup (the slowest index), then the KV head, then the block item
    const int per_layer = a.n_blocks * a.n_split * H_kv;
    const int layer = (int)(blockIdx.x / per_layer);
    const int wg = (int)(blockIdx.x - layer * per_layer);
    const int hk = wg % H_kv;
    const int item = wg / H_kv;
    // chunk-major order: every block's chunk 0 (longest blocks first), then the chunk 1s, ...
    const int qb = a.n_blocks - 1 - item % a.n_blocks;
    const int chunk = item / a.n_blocks;

    // request of this query block
    int b = 0;
    {
        int lo = 0, hi = a.n_req - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.blk_cu[mid] <= qb) lo = mid; else hi = mid - 1;
        }
        b = lo;
    }
    const int ks0 = a.cu_sel[b], k_b = a.cu_sel[b + 1] - ks0;
    // request b's first block takes the remainder k_b - (blocks - 1) * bq, the others bq each: the
    // partly filled block is the one with the fewest key tiles
    const int jb = qb - a.blk_cu[b];
    const int first = k_b - (a.blk_cu[b + 1] - a.blk_cu[b] - 1) * a.bq;
    const int qi0 = jb == 0 ? 0 : first + (jb - 1) * a.bq;
    const int nq = jb == 0 ? first : a.bq;
    const int i0 = ks0 + qi0;
    const int T_b = a.slots.cu_tok[b + 1] - a.slots.cu_tok[b];
    const int p_max = a.sel[i0 + nq - 1];

    // this lane's row
    const int row = w * 32 + lr;
    const int qi = row / g, hh = row - qi * g;
    const bool valid = qi < nq;
    const int h = hk * g + hh;
    const int p_row = valid ? a.sel[i0 + qi] : p_max;
    // key tiles of this workgroup: all of the block's tiles, or one chunk of them
    const int n_tiles_all = p_max / KT + 1;
    int t_lo = 0, t_hi = n_tiles_all;
    if (a.n_split > 1) {           // chunk c: the c-th run of split_len tiles from the block's end
        t_hi = max(n_tiles_all - chunk * a.split_len, 0);
        t_lo = max(t_hi - a.split_len, 0);
        if (t_lo >= t_hi) return;  // the block is shorter: nothing to do, nothing written
    }
    // a block of at most split_len tiles is whole in its chunk 0, which writes the final rows
    const bool whole = a.n_split == 1 || n_tiles_all <= a.split_len;
    // a row whose position lies before the chunk has no key in it: its work is discarded
    const bool active = p_row >= t_lo * KT;

    // ---- rotated, scaled Q fragments (B operand: row lr, dims 16c + 8hf + e)
    const float sl2 = 1.4426950408889634f / sqrtf((float)D_H);
    bf16x8 qf[QC];
    {
        // whole q rows, 16 bytes per lane, through this wave's slice of s_q (16-byte chunks
        // XOR-swizzled by row), then read back in the fragment layout
        bf16* sq = s_q + w * 32 * D_H;
        constexpr int RPS = 64 / NCH;
        bf16x8 tmp[32 / RPS];
#pragma unroll
        for (int it = 0; it < 32 / RPS; ++it) {
            const int r = it * RPS + lane / NCH, ch = lane % NCH;
            const int row2 = w * 32 + r, qi2 = row2 / g;
            if (qi2 < nq) {
                const int h2 = hk * g + (row2 - qi2 * g);
                tmp[it] = *(const bf16x8*)((const bf16*)a.qkv + layer * a.q_layer_stride + (int64_t)(i0 + qi2) * a.ld +
                                           (int64_t)h2 * D_H + ch * 8);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) tmp[it][e] = (bf16)0.f;
            }
        }
#pragma unroll
        for (int it = 0; it < 32 / RPS; ++it) {
            const int r = it * RPS + lane / NCH, ch = lane % NCH;
            *(bf16x8*)(sq + r * D_H + ((ch ^ (r & (NCH - 1))) << 3)) = tmp[it];
        }
#pragma unroll
        for (int c = 0; c < QC; ++c)
            qf[c] = *(const bf16x8*)(sq + lr * D_H + (((2 * c + hf) ^ (lr & (NCH - 1))) << 3));
    }
    constexpr int HC = QC / 2;     // chunks of the first half of the dims
    float4 rt[HC][4];
    {
        const float* rp = a.rope + (int64_t)p_row * D_H;   // [d_h/2][2] per position
#pragma unroll
        for (int c = 0; c < HC; ++c)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) rt[c][e2] = ((const float4*)(rp + 2 * (16 * c + 8 * hf)))[e2];
    }
    // the rotation runs after the first tile's loads are issued (its table reads are in flight
    // with them)
    auto rotate_q = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < HC; ++c) {
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float4 t = rt[c][e2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int e = 2 * e2 + u;
                    const float co = u ? t.z : t.x, si = u ? t.w : t.y;
                    const float x1 = (float)qf[c][e], x2 = (float)qf[c + HC][e];
                    qf[c][e] = (bf16)((x1 * co - x2 * si) * sl2);
                    qf[c + HC][e] = (bf16)((x2 * co + x1 * si) * sl2);
                }
            }
        }
    };

    // ---- K/V tile staging: block q of a tile holds KPB consecutive keys of K (q < NBLK/2) or V
    const bf16* kbase = (const bf16*)a.kc + layer * a.kv_layer_elems;
    const int64_t vdelta = (const bf16*)a.vc - (const bf16*)a.kc;   // V addressed relative to K
    // slots of the keys first (page-table loads complete before any of the tile's direct
    // loads is issued), then the direct loads themselves
    constexpr int NBW = (NBLK + W - 1) / W;   // blocks per wave
    const int tok0 = a.slots.cu_tok[b];
    const int32_t* ptab = a.slots.page_table + (int64_t)b * a.slots.max_pages;
    const int psz = a.slots.page_size, psh = a.slots.page_shift;
    const bool paged = PG || a.slots.paged != 0;   // PG: the paged instance (known at compile time)
    // the pages this block's tiles touch, staged in LDS once (made visible by the first barrier)
    const int n_tiles_pt = p_max / KT + 1;
    const int n_pages = !paged ? 0 : psh >= 0 ? ((min(n_tiles_pt * KT, T_b) - 1) >> psh) + 1
                                               : (min(n_tiles_pt * KT, T_b) - 1) / psz + 1;
    const bool pt_lds = n_pages <= PT_MAX;
    if (paged && pt_lds)
        for (int i = tid; i < n_pages; i += NT) s_pt[i] = ptab[i];
    // when W divides 16 every block of the wave sits a lane-independent distance from the
    // wave's first block (same swizzle, keys a multiple of 16 apart): one lane address serves all
    constexpr bool UNIFORM = 16 % W == 0;
    // lane part of every load address: the lane's key within its block, its head and its
    // (swizzled) chunk; blocks add a wave-uniform key offset
    const int key0 = (w % (NBLK / 2)) * KPB + lane / NCH;
    const bf16* lane0 = kbase + ((int64_t)(lane / NCH) * H_kv + hk) * D_H + (((lane % NCH) ^ kv_swz<D_H>(key0)) << 3);
    const int64_t tile_stride = (int64_t)KT * H_kv * D_H;
    // the paged and general paths read page-table entries through page_of: the staged copy in LDS
    // or the table in global memory, each in its own instance (a pointer that could point to either
    // is read with flat loads, which wait on both memory counters)
    auto issue_with = [&](bf16* st, int kt, auto page_of) __attribute__((always_inline)) {
        if (UNIFORM && paged && psh >= 0 && psz >= KPB && (kt + 1) * KT <= T_b) {
            // each 1 KB block holds KPB consecutive keys of one page: one wave-uniform
            // page-table read per block, the lane's key and chunk added on top
            // (all page-table reads before the first load: the loads' asm orders memory accesses)
            int64_t o[NBW];
#pragma unroll
            for (int c = 0; c < NBW; ++c) {
                const int q = w + c * W;
                const int kv = q / (NBLK / 2), ql = q % (NBLK / 2);
                const int j0 = kt * KT + ql * KPB;
                const int page = page_of(__builtin_amdgcn_readfirstlane(j0 >> psh));
                const int64_t slot0 = (int64_t)page * psz + (j0 & (psz - 1));
                // same swizzle as the wave's first block: the blocks' keys differ by multiples of 16
                o[c] = slot0 * H_kv * D_H + (kv ? vdelta : 0);
            }
#pragma unroll
            for (int c = 0; c < NBW; ++c) {
                const int q = w + c * W;
                const int kv = q / (NBLK / 2), ql = q % (NBLK / 2);
                lds_dma16(lane0 + o[c], st + kv * TILE + ql * 512);
            }
            return;
        }
        int64_t off[NBW];
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
            const int q = w + c * W;
            const int kv = q / (NBLK / 2), ql = q % (NBLK / 2);
            const int key = ql * KPB + lane / NCH;
            const int ch = (lane % NCH) ^ kv_swz<D_H>(key);
            int j = kt * KT + key;
            if (j >= T_b) j = 0;
            int64_t slot;
            if (paged) {
                const int pi = psh >= 0 ? j >> psh : j / psz;
                const int po = psh >= 0 ? j & (psz - 1) : j % psz;
                slot = (int64_t)page_of(pi) * psz + po;
            } else {
                slot = tok0 + j;
            }
            off[c] = (slot * H_kv + hk) * D_H + ch * 8 + (kv ? vdelta : 0);
        }
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
            const int q = w + c * W;
            if (NBLK % W == 0 || q < NBLK) {
                const int kv = q / (NBLK / 2), ql = q % (NBLK / 2);
                lds_dma16(kbase + off[c], st + kv * TILE + ql * 512);
            }
        }
    };
    auto issue = [&](bf16* st, int kt) {
        if constexpr (PG) {            // paged caches: the page table read from LDS when staged there
            if (pt_lds) issue_with(st, kt, [&](int i) { return s_pt[i]; });
            else issue_with(st, kt, [&](int i) { return ptab[i]; });
        } else {
            if (UNIFORM && !paged && (kt + 1) * KT <= T_b) {
                const bf16* base = lane0 + (int64_t)(tok0 + (w % (NBLK / 2)) * KPB) * H_kv * D_H + kt * tile_stride;
    #pragma unroll
                for (int c = 0; c < NBW; ++c) {
                    const int q = w + c * W;
                    const int kv = q / (NBLK / 2), ql = q % (NBLK / 2);
                    const int64_t d = (int64_t)(ql - w % (NBLK / 2)) * KPB * H_kv * D_H + (kv ? vdelta : 0);
                    lds_dma16(base + d, st + kv * TILE + ql * 512);
                }
                return;
            }
            if (UNIFORM && paged && psh >= 0 && psz >= KPB && (kt + 1) * KT <= T_b) {
                // each 1 KB block holds KPB consecutive keys of one page: one wave-uniform
                // page-table read per block (a scalar load), the lane's key and chunk added on top
                // (all page-table reads before the first load: the loads' asm orders memory accesses)
                int64_t o[NBW];
    #pragma unroll
                for (int c = 0; c < NBW; ++c) {
                    const int q = w + c * W;
                    const int kv = q / (NBLK / 2), ql = q % (NBLK / 2);
                    const int j0 = kt * KT + ql * KPB;
                    const int page = ptab[__builtin_amdgcn_readfirstlane(j0 >> psh)];
                    const int64_t slot0 = (int64_t)page * psz + (j0 & (psz - 1));
                    // same swizzle as the wave's first block: the blocks' keys differ by multiples of 16
                    o[c] = slot0 * H_kv * D_H + (kv ? vdelta : 0);
                }
    #pragma unroll
                for (int c = 0; c < NBW; ++c) {
                    const int q = w + c * W;
                    const int kv = q / (NBLK / 2), ql = q % (NBLK / 2);
                    lds_dma16(lane0 + o[c], st + kv * TILE + ql * 512);
                }
                return;
            }
            int64_t off[NBW];
    #pragma unroll
            for (int c = 0; c < NBW; ++c) {
                const int q = w + c * W;
                const int kv = q / (NBLK / 2), ql = q % (NBLK / 2);
                const int key = ql * KPB + lane / NCH;
                const int ch = (lane % NCH) ^ kv_swz<D_H>(key);
                int j = kt * KT + key;
                if (j >= T_b) j = 0;
                int64_t slot;
                if (paged) {
                    const int pi = psh >= 0 ? j >> psh : j / psz;
                    const int po = psh >= 0 ? j & (psz - 1) : j % psz;
                    slot = (int64_t)(pt_lds ? s_pt[pi] : ptab[pi]) * psz + po;
                } else {
                    slot = tok0 + j;
                }
                off[c] = (slot * H_kv + hk) * D_H + ch * 8 + (kv ? vdelta : 0);
            }
    #pragma unroll
            for (int c = 0; c < NBW; ++c) {
                const int q = w + c * W;
                if (NBLK % W == 0 || q < NBLK) {
                    const int kv = q / (NBLK / 2), ql = q % (NBLK / 2);
                    lds_dma16(kbase + off[c], st + kv * TILE + ql * 512);
                }
            }
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
    // Online softmax with a reference maximum m_ref (log2 domain; q carries the scale).  The
    // scores come out of the MFMAs already shifted by -m_ref (the accumulators start at
    // -m_ref), so the common tile costs only exp2, the bf16 packing and a packed-dot row sum.
    // m_ref is always a maximum some earlier tile reached, and a tile is accepted only if its
    // lane sums stay <= 2^16 (so every p <= 2^16 and the row's mass stays >= 1); otherwise the
    // rare slow path takes the tile's true maximum and rescales O and l.
    float m_ref = 0.f, l_lane = 0.f;           // l_lane: this lane's half of the row sum
    bool have_ref = false;
    f32x16 negm;
#pragma unroll
    for (int i = 0; i < 16; ++i) negm[i] = 0.f;
    // smallest query position of this wave: tiles ending at or below it need no mask
    int p_min = active ? p_row : INT_MAX;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) p_min = min(p_min, __shfl_xor(p_min, o));

    // value held by lane ^ 32 (the other 16 keys of each row's 32-key half tile)
    auto other_half = [&](float x) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return hf ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
    };
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
    auto compute = [&](const bf16* lk, int kt) {
        const bf16* lv = lk + TILE;
        // S^T - m_ref for the two 32-key halves of the tile
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = kb * 32 + lr;
            sacc[kb] = negm;
#pragma unroll
            for (int c = 0; c < QC; ++c) {
                const bf16x8 kf = *(const bf16x8*)(lk + key * D_H + (((2 * c + hf) ^ kv_swz<D_H>(key)) << 3));
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], sacc[kb], 0, 0, 0);
            }
        }
        // K fragment reads PF_K ahead of the MFMAs that use them
        __builtin_amdgcn_sched_group_barrier(0x100, PF_K, 0);
#pragma unroll
        for (int i = 0; i < 2 * QC - PF_K; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PF_K, 0);
        if (kt * KT + KT - 1 > p_min) {          // tile crosses a row's position (rare)
            asm volatile("");                     // keep this a branch, not per-element selects
            const int jbase = kt * KT + 4 * hf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = jbase + kb * 32 + 8 * (i >> 2) + (i & 3);
                    if (j > p_row) sacc[kb][i] = -INFINITY;
                }
        }
        bf16x8 pf[2][2];
        // P = bf16(exp2(sacc + shift)) (no shift on the common path); returns the lane sum, kept
        // in four partial sums so that the packed dot products do not form one serial chain
        auto exp_pack = [&](bool shifted, float shift) -> float {
            float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    bf16x2 pp;
                    pp[0] = (bf16)__builtin_amdgcn_exp2f(shifted ? sacc[kb][i] + shift : sacc[kb][i]);
                    pp[1] = (bf16)__builtin_amdgcn_exp2f(shifted ? sacc[kb][i + 1] + shift : sacc[kb][i + 1]);
                    pf[kb][i >> 3][i & 7] = pp[0];
                    pf[kb][i >> 3][(i & 7) + 1] = pp[1];
                    rs[2 * kb + ((i >> 1) & 1)] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, rs[2 * kb + ((i >> 1) & 1)], false);
                }
            return (rs[0] + rs[1]) + (rs[2] + rs[3]);
        };
        // a wave with a row that has no reference yet (its first tile) goes straight to the slow
        // path; otherwise the common path, and the slow one only if a score is far above m_ref
        float rs = 0.f;
        const bool no_ref = __any(!have_ref);
        bool slow = no_ref;
        if (!no_ref) {
            rs = exp_pack(false, 0.f);
            slow = __any(!(rs <= 65536.f));
        }
        if (slow) {
            asm volatile("");
            float mx = sacc[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
            mx = fmaxf(mx, other_half(mx)) + m_ref;   // the row's true tile maximum
            // a row with every key of the tile masked (possible only in a chunk that starts
            // past the row's position) keeps its reference: its P is 0
            const bool none = !(mx > -INFINITY);
            const float m_new = none ? m_ref : have_ref ? fmaxf(m_ref, mx) : mx;
            // rows without a reference hold O = 0 and l = 0: a wave without any reference skips the rescale
            if (__any(have_ref)) {
                const float corr = have_ref ? __builtin_amdgcn_exp2f(m_ref - m_new) : 0.f;
                l_lane *= corr;
#pragma unroll
                for (int d = 0; d < DB; ++d)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[d][i] *= corr;
            }
            rs = exp_pack(true, m_ref - m_new);
            m_ref = m_new;
            have_ref = have_ref || !none;
#pragma unroll
            for (int i = 0; i < 16; ++i) negm[i] = -m_new;
        }
        l_lane += rs;

        // O^T += V^T P^T
        const int G = lane >> 4, gi = lane & 15;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int d = 0; d < DB; ++d) {
                    bf16x8 vf;
#pragma unroll
                    for (int E = 0; E < 2; ++E) {
                        const int key = kb * 32 + s * 16 + 8 * E + 4 * (G >> 1) + (gi >> 2);
                        const int d0 = d * 32 + 16 * (G & 1) + 4 * (gi & 3);
                        const bf16* addr = lv + key * D_H + (((d0 >> 3) ^ kv_swz<D_H>(key)) << 3) + (d0 & 7);
                        const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(addr));
                        const bf16x4 tb = __builtin_bit_cast(bf16x4, t);
#pragma unroll
                        for (int v = 0; v < 4; ++v) vf[4 * E + v] = tb[v];
                    }
                    oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][s], oacc[d], 0, 0, 0);
                }
            }
        }
        // V^T fragment reads (two per MFMA: 8 * DB reads, 4 * DB MFMAs) PF_V ahead
        __builtin_amdgcn_sched_group_barrier(0x100, PF_V, 0);
#pragma unroll
        for (int i = 0; i < 4 * DB - PF_V / 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PF_V / 2, 0);
    };

    if (paged && pt_lds) __syncthreads();      // the staged page table, before the first loads
    if (t_lo < t_hi) issue(lds0, t_lo);
    rotate_q();
    if (t_lo < t_hi) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    for (int kt = t_lo; kt < t_hi; kt += 2) {
        if (kt + 1 < t_hi) issue(lds1, kt + 1);
        compute(lds0, kt);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 < t_hi) {
            if (kt + 2 < t_hi) issue(lds0, kt + 2);
            compute(lds1, kt + 1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    const float l_run = l_lane + other_half(l_lane);
    // this lane's output row, formed again from the lane id (behind an opaque copy, so that
    // none of the prologue's row values has to stay live across the key loop)
    int lane_e = __lane_id();
    asm volatile("" : "+v"(lane_e));
    const int row_e = w * 32 + (lane_e & 31);
    const int qi_e = row_e / g;
    if (whole) {
        // final rows: staged in this wave's own 32-row slice of the (now idle) K/V stages
        // (16-byte chunks XOR-swizzled by row), then written 16 bytes per lane, whole rows per
        // store (4 at d_h = 128): a store of the accumulator layout touches 32 rows, 8 bytes each
        const float inv = 1.f / l_run;
        bf16* so = (w < 4 ? lds0 : lds1) + (w & 3) * 32 * D_H;
        const int rr = lane_e & 31, hh2 = lane_e >> 5;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                bf16x4 o;
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = (bf16)(oacc[d][4 * q4 + v] * inv);
                const int c16 = (d * 4 + q4) ^ (rr & (NCH - 1));
                *(bf16x4*)(so + rr * D_H + c16 * 8 + 4 * hh2) = o;
            }
        constexpr int RPS = 64 / NCH;               // rows per store
#pragma unroll
        for (int it = 0; it < 32 / RPS; ++it) {
            const int r = it * RPS + lane_e / NCH, ch = lane_e % NCH;
            const bf16x8 v = *(const bf16x8*)(so + r * D_H + ((ch ^ (r & (NCH - 1))) << 3));
            const int row2 = w * 32 + r, qi2 = row2 / g;
            if (qi2 < nq) {
                const int64_t orow2 = (int64_t)(i0 + qi2) * a.H_q + hk * g + (row2 - qi2 * g);
                *(bf16x8*)((bf16*)a.out + layer * a.out_layer_stride + orow2 * D_H + ch * 8) = v;
            }
        }
        if (qi_e >= nq) return;
        const int64_t out_row = (int64_t)(i0 + qi_e) * a.H_q + hk * g + (row_e - qi_e * g);
        if (a.lse && hf == 0)
            a.lse[layer * a.lse_layer_stride + out_row] = (m_ref + __log2f(l_run)) * 0.6931471805599453f;
        return;
    }
    // partial rows of this chunk: unnormalised O, m (log2), l
    if (qi_e >= nq) return;
    const int64_t out_row = (int64_t)(i0 + qi_e) * a.H_q + hk * g + (row_e - qi_e * g);
    // rows without keys in the chunk leave only l = 0 (the merge skips their output)
    const bool has = active;
    const int64_t prow = out_row * a.n_split + chunk;
    float* po = a.part + prow * D_H;
    if (has)
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 o;
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = oacc[d][4 * q4 + v];
                *(f32x4*)(po + d * 32 + 8 * q4 + 4 * hf) = o;
            }
    if (hf == 0) {
        a.part_ml[prow * 2] = m_ref;
        a.part_ml[prow * 2 + 1] = has ? l_run : 0.f;
    }
}

// Merge of a split attention: out = sum_c 2^(m_c - m) O_c / sum_c 2^(m_c - m) l_c over the
// chunks with l_c > 0 (m their largest m_c), in chunk order.  One wave per (row, head): lane
// c < n_split holds chunk c's weight, every lane then sums D_H / 64 output columns over the
// chunks (the weights broadcast from their lanes).
template <int D_H>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* part, const float* ml, int n_split,
                                                            int split_len, int64_t rows, int H_q,
                                                            const int32_t* sel, const int32_t* cu_sel, int n_req,
                                                            int bq, bf16* out, float* lse) {
    constexpr int CPL = D_H / 64;                 // output columns per lane
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    // the row's query block: its last query's position gives the block's key tiles, and so the
    // chunks that hold partials (none when the block was whole in its chunk 0)
    const int i = (int)(row / H_q);
    int b = 0;
    {
        int lo = 0, hi = n_req - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cu_sel[mid] <= i) lo = mid; else hi = mid - 1;
        }
        b = lo;
    }
    const int qi = i - cu_sel[b];
    // the row's block (the request's first block holds the remainder of k_b over bq): its last query
    const int k_b = cu_sel[b + 1] - cu_sel[b];
    const int first = k_b - ((k_b + bq - 1) / bq - 1) * bq;
    const int last = cu_sel[b] + (qi < first ? first : first + ((qi - first) / bq + 1) * bq) - 1;
    const int n_tiles = sel[last] / KT + 1;
    if (n_tiles <= split_len) return;
    const int nch = min((n_tiles + split_len - 1) / split_len, n_split);
    const float* mlr = ml + row * n_split * 2;
    const float mc = lane < nch ? mlr[2 * lane] : 0.f;
    const float lc = lane < nch ? mlr[2 * lane + 1] : 0.f;
    float m = lc > 0.f ? mc : -INFINITY;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float wgt = lc > 0.f ? __builtin_amdgcn_exp2f(mc - m) : 0.f;
    // chunk-ordered sum of the weighted row sums (lane 0 adds them one by one)
    float L = 0.f;
    for (int c = 0; c < nch; ++c) L += __shfl(wgt, c) * __shfl(lc, c);
    float acc[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) acc[j] = 0.f;
    // eight chunks per pass: their loads are issued together, the sums stay in chunk order
    for (int c0 = 0; c0 < nch; c0 += 8) {
        float v[8][CPL];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = c0 + u;
            const bool use = c < nch && __shfl(wgt, c < nch ? c : 0) != 0.f;
            const float* pc = part + (row * n_split + (use ? c : 0)) * D_H + lane * CPL;
#pragma unroll
            for (int j = 0; j < CPL; ++j) v[u][j] = use ? pc[j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = c0 + u;
            const float wc = c < nch ? __shfl(wgt, c) : 0.f;
            if (wc == 0.f) continue;              // uniform over the wave
#pragma unroll
            for (int j = 0; j < CPL; ++j) acc[j] += wc * v[u][j];
        }
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int j = 0; j < CPL; ++j) out[row * D_H + lane * CPL + j] = (bf16)(acc[j] * inv);
    if (lse && lane == 0) lse[row] = (m + __log2f(L)) * 0.6931471805599453f;
}

template <int D_H>
hipError_t launch_dh(const AttnArgs& a, int W, hipStream_t s) {
    if (W != 8) return hipErrorInvalidValue;
    if (a.n_split < 1 || (a.n_split > 1 && (!a.part || !a.part_ml))) return hipErrorInvalidValue;
    if (a.n_layers < 1 || (a.n_layers > 1 && a.n_split != 1)) return hipErrorInvalidValue;
    const int64_t wgs = (int64_t)a.n_blocks * a.n_split * a.H_kv * a.n_layers;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    if (a.slots.paged)
        hipLaunchKernelGGL((attn_bf16_kernel<D_H, 8, true>), grid, dim3(8 * 64), 0, s, a);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<D_H, 8, false>), grid, dim3(8 * 64), 0, s, a);
    if (a.n_split == 1) return hipGetLastError();
    if (hipError_t e = hipGetLastError()) return e;
    const int64_t rows = a.n_rows_total * a.H_q;   // (selected row, query head) rows
    if (a.n_split > 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_combine_kernel<D_H>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                       (const float*)a.part, (const float*)a.part_ml, a.n_split, a.split_len, rows, a.H_q, a.sel,
                       a.cu_sel, a.n_req, a.bq, (bf16*)a.out, a.lse);
    return hipGetLastError();
}

}  // namespace

// Blocks of 8 waves (256 rows): floor(256 / g) queries, so a g that does not divide 256 leaves
// fewer than g rows of the last wave idle (measured faster than g-wave blocks of 32 queries).
int attn_bf16_split(int n_blocks, int H_kv, int max_T) {
    const int64_t CUS = device_shape().cus;
    const int64_t items = (int64_t)n_blocks * H_kv;
    if (items <= 0 || items >= CUS) return 1;
    const int max_tiles = (max_T + KT - 1) / KT;
    // c = round(1.25 * CUS / items), fitted by measurement (200 workgroups: 2 chunks, 104: 3, 50: 6)
    int c = (int)((5 * CUS + 2 * items) / (4 * items));
    c = std::min(c, std::min(max_tiles / 4, 64));
    return std::max(c, 1);
}

size_t attn_bf16_split_bytes(int64_t n_sel, int H_q, int d_h, int n_split) {
    if (n_split <= 1) return 0;
    const size_t rows = (size_t)n_sel * H_q * n_split;
    return ((rows * d_h * 4 + 255) & ~(size_t)255) + ((rows * 2 * 4 + 255) & ~(size_t)255);
}

int attn_bf16_block_queries(int g) {
    if (g <= 0 || g > 16) return 0;
    return 256 / g;            // 8 waves of 32 rows; g that do not divide 256 leave < g rows idle
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
    if (a.n_blocks == 0) return hipSuccess;
    const int g = a.H_q / a.H_kv;
    const int W = (a.bq * g + 31) / 32;
    if (a.d_h == 128) return launch_dh<128>(a, W, s);
    if (a.d_h == 64) return launch_dh<64>(a, W, s);
    return hipErrorInvalidValue;
}

}  // namespace kvx
