// bf16 GEMM on gfx950 matrix cores:  C[m][n] = sum_k A[src(m)][k] * B[n][k], fp32 accumulate.
//
// Both operands are K-contiguous (weights are stored output-major), so every 16-byte global
// load feeds one LDS chunk and every MFMA operand is one 16-byte LDS read.
//
//  * Block tiles of 256 x 256 x 64 with 8 waves (two per SIMD, so one wave's LDS waits hide
//    behind the other's MFMAs), each wave a 64 x 128 grid of v_mfma_f32_16x16x32_bf16 blocks.
//  * Tiles travel global -> LDS with direct loads (global_load_lds_dwordx4): the first four
//    waves (one per SIMD) fill whole 1 KB blocks of the stage, each lane fetching the chunk
//    that belongs at its slot of the XOR-swizzled layout, while the other wave of each SIMD
//    keeps its matrix core busy (measured 3% faster than every wave loading its share).  No VGPRs hold the next tile; the two LDS stages are
//    separate objects so the next tile's loads stay in flight while the current one is read.
//    The direct loads are issued from asm and waited for explicitly before each barrier, so
//    the compiler sees only fragment reads on the LDS counter and waits for them one group at
//    a time; every fragment is read one group of MFMAs ahead of its use.
//  * Row pointers of the gathered A rows and of the B rows are computed once per block;
//    rows past M or N are clamped to row 0 (their outputs are never stored), so the K loop
//    has no branches.
//  * B fragment j of lane l is tile row (l%16)*FN + j, so after the K loop each lane holds
//    FN consecutive output columns of every row it owns: the epilogue writes 8- or 16-byte
//    chunks with no LDS staging.  In LDS that row is stored at row j*16 + l%16 of the wave's
//    slab, so a fragment read touches 16 consecutive LDS rows (the conflict-free pattern).
//  * Rows of A can be gathered (selected or complement positions of a ragged batch), and
//    the epilogue can write a plain matrix, the K/V cache of a layer (contiguous or paged
//    slots), or per-row partial sums of C[m][n] * Z[m][n] (the score quadratic form).
//  * Tiles are numbered so that every XCD owns one contiguous range of tiles, walked in
//    groups of row panels sized so the tiles in flight on an XCD share operand panels in L2.
#include <algorithm>
#include <atomic>
#include <climits>

#include "kvx_common.h"

namespace kvx {
namespace {

constexpr int BK = 64;

struct Tile { int group, tm, tn; };

// Tile order.  Every XCD (workgroup i runs on XCD i % 8) owns one contiguous range of the linear
// tile index, and its 32 CUs run consecutive indices together.  The linear index walks groups
// of gm row panels: inside a group the row panel varies fastest, then the column panel (the
// columns of all groups side by side), so the 32 tiles in flight on an XCD share gm row panels
// and 32/gm column panels of their operands in that XCD's L2.
__device__ __forceinline__ Tile tile_at(int lin, int mt, int nt, int groups, int gm) {
    const int cols = nt * groups;
    const int band = lin / (gm * cols);
    const int m0 = band * gm;
    const int g = min(mt - m0, gm);
    const int r = lin - band * gm * cols;
    const int cp = r / g;
    Tile t;
    t.tm = m0 + (r - cp * g);
    t.group = cp / nt;
    t.tn = cp - t.group * nt;
    return t;
}

// linear tile index of workgroup bid among `total` tiles: XCD x owns one contiguous range
__device__ __forceinline__ int xcd_linear(int bid, int total, int nx) {
    const int xcd = bid % nx, j = bid / nx;
    const int per = total / nx, rem = total % nx;
    return xcd * per + min(xcd, rem) + j;
}

// Split tail.  When the last round of tiles would leave most CUs idle, the workgroups past
// the whole rounds each take one K slice of a tail tile and write its fp32 partial tile; a
// second kernel adds the slices in order and stores the result (deterministic).
struct SplitPlan { int full, rem, split; };

typedef __attribute__((address_space(3))) void* lds_ptr_t;


// Issue order of one stage of the GEMM's K loop (see compute): before group g its look-ahead
// reads (the next A fragment; during the first substep also FN / FM second-substep B
// fragments), then its FN MFMAs.
template <int G, int FM, int FN>
__device__ __forceinline__ void group_order() {
    if constexpr (G < 2 * FM) {
        constexpr int nr = (G + 1 < 2 * FM ? 1 : 0) + (G < FM ? FN / FM : 0);
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);
        group_order<G + 1, FM, FN>();
    }
}

template <int BM, int BN, int WM, int WN, bool SQ>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4)))
void gemm_bf16_kernel(GemmArgs a, int mt, int nt, int gm, SplitPlan sp, int n_xcd) {
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    static_assert(FN == 4 || FN == 8, "lanes own 4 or 8 consecutive output columns");
    constexpr int STAGE = (BM + BN) * BK;
    __shared__ __attribute__((aligned(1024))) bf16 lds0[STAGE];
    __shared__ __attribute__((aligned(1024))) bf16 lds1[STAGE];
    __shared__ int s_src[BM];
    __shared__ int64_t s_slot[BM];
    __shared__ int s_pos[BM];
    __shared__ float s_red[WN][BM];
    __shared__ float s_yy[SQ ? BM : 1];             // EPI_SQNORM: squared norm of every A row

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int nk_all = a.K / BK;
    const int bid = blockIdx.x;
    const bool tail = bid >= sp.full;                 // a K slice of a tail tile
    const int unit = bid - sp.full;
    Tile t;
    if (a.a_group_stride != 0) {
        // independent groups, one after another in dispatch order, each spread over every XCD
        // like a single-group launch: the CUs work on one group's operands at a time, which
        // keep fitting in the last-level cache
        const int per = mt * nt;
        const int grp = bid / per;
        t = tile_at(xcd_linear(bid - grp * per, per, n_xcd), mt, nt, 1, gm);
        t.group = grp;
    } else {
        t = tail ? tile_at(sp.full + unit / sp.split, mt, nt, a.groups, gm)
                 : tile_at(xcd_linear(bid, sp.full, n_xcd), mt, nt, a.groups, gm);
    }
    const int k_first = tail ? (unit % sp.split) * (nk_all / sp.split) : 0;
    const int nk = tail ? nk_all / sp.split : nk_all;
    const int m0 = t.tm * BM, n0 = t.tn * BN;

    // ---- row map: source row of every tile row, and its cache slot
    for (int r = tid; r < BM; r += NW * 64) {
        const int m = m0 + r;
        int src = -1, pos = 0;
        int64_t slot = 0;
        if (m < a.M) {
            const RowInfo ri = row_info(a.rows, m);
            src = ri.src;
            if (a.epi == EPI_CACHE || a.epi == EPI_QKV || SQ) slot = a.slots.slot(ri.b, ri.pos);
            pos = ri.pos;
        }
        s_src[r] = src;
        s_slot[r] = slot;
        s_pos[r] = pos;
    }
    __syncthreads();

    // ---- per-lane sources of the direct loads: lane owns LDS chunk P = (c*NL + wave)*64 + lane
    const bf16* Bg = a.B + (int64_t)t.group * a.b_group_stride;
    // loader waves: only the first NL waves (one per SIMD) issue the direct loads
    constexpr int NL = NW / 2;
    constexpr int A_L = BM / 8 / NL, B_L = BN / 8 / NL;   // 1 KB direct loads per loader wave
    static_assert(A_L * NL * 8 == BM && B_L * NL * 8 == BN, "tiles split into whole 1 KB blocks per loader wave");
    const int lw = wave % NL;
    const bf16* asrc[A_L];
    const bf16* bsrc[B_L];
#pragma unroll
    for (int c = 0; c < A_L; ++c) {
        const int P = (c * NL + lw) * 64 + lane;
        const int row = P >> 3, ch = (P & 7) ^ swz(row);
        if constexpr (SQ) {              // the row's cache slot (rows past M read slot 0)
            asrc[c] = a.A + (int64_t)t.group * a.a_group_stride + s_slot[row] * a.lda + ch * 8;
        } else {
            const int src = max(s_src[row], 0);
            asrc[c] = a.A + (int64_t)t.group * a.a_group_stride + (int64_t)src * a.lda + ch * 8;
        }
    }
#pragma unroll
    for (int c = 0; c < B_L; ++c) {
        const int P = (c * NL + lw) * 64 + lane;
        const int R = P >> 3, ch = (P & 7) ^ swz(R);          // LDS row R of the B stage
        const int slab = R / WTN, rl = R % WTN;               // rl = j*16 + s  <->  tile row s*FN + j
        const int row = slab * WTN + (rl % 16) * FN + rl / 16;
        const int n = n0 + row < a.N ? n0 + row : 0;
        const bf16* brow = a.epi == EPI_SWIGLU
                               ? ((n >> 3) & 1 ? a.B2 : a.B) + (int64_t)((n >> 4) * 8 + (n & 7)) * a.ldb
                               : Bg + (int64_t)n * a.ldb;
        bsrc[c] = brow + ch * 8;
    }
    auto issue = [&](bf16* st, int kt) {
        if (wave >= NL) return;
        if constexpr (SQ) {
            int64_t ka = (kt >> 1) * BK;
            if (ka >= a.kv_split) ka += a.kv_delta - a.kv_split;
#pragma unroll
            for (int c = 0; c < A_L; ++c)
                lds_dma16(asrc[c] + ka, st + (c * NL + lw) * 512);
        } else {
            const int ka = (kt * BK) % a.K_a;
#pragma unroll
            for (int c = 0; c < A_L; ++c)
                lds_dma16(asrc[c] + ka, st + (c * NL + lw) * 512);
        }
#pragma unroll
        for (int c = 0; c < B_L; ++c)
            lds_dma16(bsrc[c] + kt * BK, st + BM * BK + (c * NL + lw) * 512);
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int lr = lane & 15, lq = lane >> 4;
    // EPI_SQNORM: the first column tile's wn == 0 waves square the A fragments they read on the even
    // K steps (each A chunk once); lane holds row wm*WTM + i*16 + lr, k chunk ks*4 + lq
    float sq[SQ ? FM : 1];
#pragma unroll
    for (int i = 0; i < (SQ ? FM : 1); ++i) sq[i] = 0.f;
    bool sq_on = false;
    // One stage = two 32-deep substeps = 2*FM groups of FN MFMAs (group g: A fragment g % FM of
    // substep g / FM against the substep's FN B fragments).  Reads run one group ahead: before
    // group g the A fragment of group g+1 is read, and during the first substep's groups the
    // second substep's B fragments (FN / FM per group), so only the stage's first reads wait.
    static_assert(BK == 64 && FN % FM == 0, "two substeps per stage, B reads spread over FM groups");
    auto compute = [&](const bf16* st) {
        const bf16* la = st;
        const bf16* lb = st + BM * BK;
        auto rd_b = [&](int ks, int j) {
            const int R = wn * WTN + j * 16 + lr;
            return *(const bf16x8*)(lb + R * BK + (((ks * 4 + lq) ^ swz(R)) << 3));
        };
        auto rd_a = [&](int ks, int i) {
            const int ml = wm * WTM + i * 16 + lr;
            return *(const bf16x8*)(la + ml * BK + (((ks * 4 + lq) ^ swz(ml)) << 3));
        };
        bf16x8 b0[FN], b1[FN], af[2];
#pragma unroll
        for (int j = 0; j < FN; ++j) b0[j] = rd_b(0, j);
        af[0] = rd_a(0, 0);
        constexpr int BPG = FN / FM;        // second-substep B reads per first-substep group
#pragma unroll
        for (int g = 0; g < 2 * FM; ++g) {
            const int ks = g / FM, i = g % FM;
            if (g + 1 < 2 * FM) af[(g + 1) & 1] = rd_a((g + 1) / FM, (g + 1) % FM);
            if (g < FM) {
#pragma unroll
                for (int u = 0; u < BPG; ++u) b1[g * BPG + u] = rd_b(1, g * BPG + u);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[g & 1], ks ? b1[j] : b0[j], acc[i][j], 0, 0, 0);
            if constexpr (SQ) {
                if (sq_on) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float f = (float)af[g & 1][e];
                        sq[i] = __builtin_fmaf(f, f, sq[i]);
                    }
                }
            }
        }
        // issue order: the first reads, then per group its look-ahead reads and its MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, FN + 1, 0);
        group_order<0, FM, FN>();
    };

    // SQ: K steps alternate high and low halves of the basis on the same A chunk, so stage lds0
    // (even steps) carries each chunk once
    if constexpr (SQ) sq_on = t.tn == 0 && wn == 0;
    issue(lds0, k_first);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        if (kt + 1 < nk) issue(lds1, k_first + kt + 1);
        compute(lds0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 < nk) {
            if (kt + 2 < nk) issue(lds0, k_first + kt + 2);
            if constexpr (SQ) { const bool on = sq_on; sq_on = false; compute(lds1); sq_on = on; }
            else compute(lds1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    // ---- epilogue: lane owns rows wm*WTM + i*16 + 4*lq + v and columns nl0 .. nl0+FN-1
    const int nl0 = wn * WTN + lr * FN;
    const int ng = n0 + nl0;
    if (tail) {                               // fp32 partial tile [BM][BN] of this K slice (valid rows)
        float* pt = a.split_ws + (int64_t)unit * BM * BN;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ml = wm * WTM + i * 16 + 4 * lq + v;
                if (s_src[ml] < 0) continue;
#pragma unroll
                for (int j = 0; j < FN; j += 4)
                    *(f32x4*)(pt + ml * BN + nl0 + j) =
                        f32x4{acc[i][j][v], acc[i][j + 1][v], acc[i][j + 2][v], acc[i][j + 3][v]};
            }
        return;
    }
    if constexpr (SQ) {
        if (t.tn == 0 && wn == 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                float v = sq[i];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                if (lq == 0) s_yy[wm * WTM + i * 16 + lr] = v;
            }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ml = wm * WTM + i * 16 + 4 * lq + v;
                float p = 0.f;
                if (s_src[ml] >= 0 && ng < a.N) {
#pragma unroll
                    for (int j = 0; j < FN; ++j) p = __builtin_fmaf(acc[i][j][v], acc[i][j][v], p);
                }
                p += __shfl_xor(p, 1);
                p += __shfl_xor(p, 2);
                p += __shfl_xor(p, 4);
                p += __shfl_xor(p, 8);
                if (lr == 0) s_red[wn][ml] = p;
            }
        }
        __syncthreads();
        float* out = a.partial + ((int64_t)t.group * nt + t.tn) * a.M + m0;
        for (int r = tid; r < BM; r += NW * 64) {
            if (m0 + r >= a.M) continue;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < WN; ++w) s += s_red[w][r];
            out[r] = (t.tn == 0 ? s_yy[r] : 0.f) - s;
        }
        return;
    }
    if (a.epi == EPI_SCORE) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ml = wm * WTM + i * 16 + 4 * lq + v;
                const int src = s_src[ml];
                float p = 0.f;
                if (src >= 0 && ng < a.N) {
                    const bf16* zr = a.Z + (int64_t)src * a.ldz + ng;
#pragma unroll
                    for (int j = 0; j < FN; ++j) p += acc[i][j][v] * (float)zr[j];
                }
                p += __shfl_xor(p, 1);
                p += __shfl_xor(p, 2);
                p += __shfl_xor(p, 4);
                p += __shfl_xor(p, 8);
                if (lr == 0) s_red[wn][ml] = p;
            }
        }
        __syncthreads();
        for (int r = tid; r < BM; r += NW * 64) {
            if (m0 + r >= a.M) continue;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < WN; ++w) s += s_red[w][r];
            a.partial[(int64_t)t.tn * a.M + m0 + r] = s;
        }
        return;
    }
    if (a.epi == EPI_QKV) {
        // columns nl0 .. nl0+7 of one head (heads are 64 or 128 columns, aligned to 8)
        static_assert(FN == 8, "the fused QKV epilogue expects 8 columns per lane");
        const int half = a.d_h / 2;
        // a wave whose 128-column slab touches the K columns exchanges rotation partners:
        // column j of a head pairs with j +- d_h/2, held by lane ^ (d_h/16)
        const int slab0 = n0 + wn * WTN;
        const bool k_slab = slab0 < a.q_cols + a.hd && slab0 + WTN > a.q_cols;
        const int cc = ng - a.q_cols;                 // column in [K | V]
        const bool is_k = ng >= a.q_cols && cc < a.hd;
        const int j0 = (cc % a.d_h) % half;           // rotation index of the first column
        const bool lo = (cc % a.d_h) < half;
        // QK-norm: q and k heads normalised over their d_h columns (16 lanes at d_h = 128, 8 at 64)
        const bool is_q = ng < a.q_cols;
        const bool norm = a.qk_gain_q && (is_q || is_k);
        float gn[8];
        if (a.qk_gain_q) {
            const float* gsrc = (is_q ? a.qk_gain_q : a.qk_gain_k) + (ng % a.d_h);
#pragma unroll
            for (int j = 0; j < 8; ++j) gn[j] = is_q || is_k ? gsrc[j] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ml = wm * WTM + i * 16 + 4 * lq + v;
                float x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = (float)(bf16)acc[i][j][v];
                if (a.qk_gain_q) {
                    float ss = 0.f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) ss = __builtin_fmaf(x[j], x[j], ss);
                    ss += __shfl_xor(ss, 1);
                    ss += __shfl_xor(ss, 2);
                    ss += __shfl_xor(ss, 4);
                    if (a.d_h == 128) ss += __shfl_xor(ss, 8);
                    const float inv = 1.f / sqrtf(ss / (float)a.d_h + a.qk_eps);
                    if (norm)
#pragma unroll
                        for (int j = 0; j < 8; ++j) x[j] = x[j] * inv * gn[j];
                }
                float y[8];
                if (k_slab) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int xi = __float_as_int(x[j]);
                        const int pi = a.d_h == 128 ? __builtin_amdgcn_update_dpp(0, xi, 0x128, 0xF, 0xF, false)
                                                    : __shfl_xor(xi, 4);
                        y[j] = __int_as_float(pi);           // the partner column's value
                    }
                }
                if (ng >= a.N || s_src[ml] < 0) continue;
                bf16x8 o;
                if (is_k) {
                    const float4* cs = (const float4*)(a.rope + ((int64_t)s_pos[ml] * half + j0) * 2);
#pragma unroll
                    for (int j2 = 0; j2 < 4; ++j2) {
                        const float4 t2 = cs[j2];
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int j = 2 * j2 + u;
                            const float c = u ? t2.z : t2.x, sn = u ? t2.w : t2.y;
                            o[j] = (bf16)(lo ? rope_lo(x[j], y[j], c, sn) : rope_hi(y[j], x[j], c, sn));
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) o[j] = (bf16)x[j];
                }
                bf16* dst = ng < a.q_cols ? a.C + (int64_t)t.group * a.c_group_stride + (int64_t)(m0 + ml) * a.ldc + ng
                                          : (is_k ? a.kc : a.vc) + (int64_t)t.group * a.layer_elems +
                                                s_slot[ml] * a.hd + (is_k ? cc : cc - a.hd);
                *(bf16x8*)dst = o;
            }
        }
        return;
    }
    if (a.epi == EPI_SWIGLU) {
        // lane pairs (lr even, lr odd) hold the gate and the up columns of the same 8 features
        const bool gate_lane = (lr & 1) == 0;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ml = wm * WTM + i * 16 + 4 * lq + v;
                float up[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    up[j] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[i][j][v]), 0xB1, 0xF, 0xF,
                                                                       false));
                if (!gate_lane || ng >= a.N || s_src[ml] < 0) continue;
                bf16x8 o;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float g = acc[i][j][v];
                    o[j] = (bf16)(g / (1.f + __expf(-g)) * up[j]);
                }
                *(bf16x8*)(a.C + (int64_t)(m0 + ml) * a.ldc + (ng >> 4) * 8) = o;
            }
        }
        return;
    }
    if (ng >= a.N) return;
    if (a.epi == EPI_F32) {                  // fp32 store (Gram matrices of the mapper fit)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ml = wm * WTM + i * 16 + 4 * lq + v;
                if (s_src[ml] < 0) continue;
                float* dst = a.C32 + (int64_t)(m0 + ml) * a.ldc + ng;
#pragma unroll
                for (int j = 0; j < FN; j += 4)
                    *(f32x4*)(dst + j) = f32x4{acc[i][j][v], acc[i][j + 1][v], acc[i][j + 2][v], acc[i][j + 3][v]};
            }
        return;
    }
    if (a.epi == EPI_RESID) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ml = wm * WTM + i * 16 + 4 * lq + v;
                if (s_src[ml] < 0) continue;
                const bf16x8 r = *(const bf16x8*)(a.R + (int64_t)(m0 + ml) * a.ldr + ng);
                bf16x8 o;
#pragma unroll
                for (int j = 0; j < 8; ++j) o[j] = (bf16)((float)r[j] + acc[i][j][v]);
                *(bf16x8*)(a.C + (int64_t)(m0 + ml) * a.ldc + ng) = o;
            }
        }
        return;
    }
    if (a.epi == EPI_CACHE && a.rope) {
        // translated keys rotated at their rows' positions (the key columns [0, hd) of each
        // layer), with the rounding and rotation order of the fused QKV epilogue: the value is
        // rounded to bf16, rotated in fp32 with its partner column j +- d_h/2 (held by
        // lane ^ (d_h/16)), and rounded again; V columns are stored as they are
        static_assert(FN == 8, "the rotating cache epilogue expects 8 columns per lane");
        const int half = a.d_h / 2;
        const int slab0 = n0 + wn * WTN;
        const bool k_slab = slab0 < a.hd;
        const bool is_k = ng < a.hd;
        const int j0 = (ng % a.d_h) % half;
        const bool lo = (ng % a.d_h) < half;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ml = wm * WTM + i * 16 + 4 * lq + v;
                float x[8], y[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = (float)(bf16)acc[i][j][v];
                if (k_slab) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int xi = __float_as_int(x[j]);
                        const int pi = a.d_h == 128 ? __builtin_amdgcn_update_dpp(0, xi, 0x128, 0xF, 0xF, false)
                                                    : __shfl_xor(xi, 4);
                        y[j] = __int_as_float(pi);
                    }
                }
                if (s_src[ml] < 0) continue;
                bf16x8 o;
                if (is_k) {
                    const float4* cs = (const float4*)(a.rope + ((int64_t)s_pos[ml] * half + j0) * 2);
#pragma unroll
                    for (int j2 = 0; j2 < 4; ++j2) {
                        const float4 t2 = cs[j2];
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int j = 2 * j2 + u;
                            const float c = u ? t2.z : t2.x, sn = u ? t2.w : t2.y;
                            o[j] = (bf16)(lo ? rope_lo(x[j], y[j], c, sn) : rope_hi(y[j], x[j], c, sn));
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) o[j] = (bf16)x[j];
                }
                bf16* dst = (is_k ? a.kc : a.vc) + (int64_t)t.group * a.layer_elems + s_slot[ml] * a.hd +
                            (is_k ? ng : ng - a.hd);
                *(bf16x8*)dst = o;
            }
        }
        return;
    }
    typedef __bf16 vecN __attribute__((ext_vector_type(FN)));
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int ml = wm * WTM + i * 16 + 4 * lq + v;
            if (s_src[ml] < 0) continue;
            vecN o;
#pragma unroll
            for (int j = 0; j < FN; ++j) o[j] = (bf16)acc[i][j][v];
            bf16* dst;
            if (a.epi == EPI_STORE) {
                dst = a.C + (int64_t)(m0 + ml) * a.ldc + ng;
            } else {
                const bool is_k = ng < a.hd;
                dst = (is_k ? a.kc : a.vc) + (int64_t)t.group * a.layer_elems +
                      s_slot[ml] * a.hd + (is_k ? ng : ng - a.hd);
            }
            *(vecN*)dst = o;
        }
    }
}

// Few rows (M <= GEMV_MAX_M): the product is bound by streaming the weight, and 256-row
// matrix-core tiles would spend almost all their work on padding.  Every output tile becomes a
// split unit (full = 0, rem = tiles): workgroup (unit, 32-column group, K slice) computes the
// fp32 dot products of its 32 columns with the M rows over its K slice and writes them to the
// unit's partial tile (only the M valid rows), so gemm_split_reduce_kernel applies the usual
// epilogue.  A wave takes 8 columns at a time: lane l reads 16 bytes of column l/8 at k offset
// 8*(l%8) of each 64-wide k step (each column's 128-byte k chunk in one request), and the
// eight k lanes of a column are summed in a fixed order at the end.
constexpr int GEMV_MAX_M = 16;

template <int MR>   // rows handled (M <= MR; rows past M read row 0 and are not written)
__global__ __launch_bounds__(256) void gemv_bf16_kernel(GemmArgs a, int mt, int nt, int gm, SplitPlan sp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int item = blockIdx.x;
    const int sl = item % sp.split;                        // K slice
    const int cg = (item / sp.split) % 8;                  // 32-column group of the tile
    const int unit = item / (sp.split * 8);
    const Tile t = tile_at(unit, mt, nt, a.groups, gm);
    const int M = a.M;
    const int ks = a.K / sp.split, k_begin = sl * ks;
    const int c_in = lane >> 3, kl = lane & 7;
    const int nl = cg * 32 + wave * 8 + c_in;              // column within the tile
    const int n = t.tn * 256 + nl;
    const bool col_ok = n < a.N;
    const bf16* brow;
    if (a.epi == EPI_SWIGLU)
        brow = ((n >> 3) & 1 ? a.B2 : a.B) + (int64_t)((n >> 4) * 8 + (n & 7)) * a.ldb;
    else
        brow = a.B + (int64_t)n * a.ldb;
    if (!col_ok) brow = a.B;                               // in bounds; the result is not written
    brow += k_begin + kl * 8;
    const bf16* arow[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m)
        arow[m] = a.A + (int64_t)(m < M ? row_info(a.rows, m).src : 0) * a.lda + k_begin + kl * 8;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.f;
    auto dot8 = [&](const bf16x8& w, const bf16x8& x, float c) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x2 wv = {w[2 * j], w[2 * j + 1]}, xv = {x[2 * j], x[2 * j + 1]};
            c = __builtin_amdgcn_fdot2_f32_bf16(wv, xv, c, false);
        }
        return c;
    };
    const int steps = ks / 64;
    int st = 0;
    for (; st + 4 <= steps; st += 4) {                     // four 64-wide k steps per pass
        bf16x8 w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = *(const bf16x8*)(brow + (st + u) * 64);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            bf16x8 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = *(const bf16x8*)(arow[m] + (st + u) * 64);
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[m] = dot8(w[u], x[u], acc[m]);
        }
    }
    for (; st < steps; ++st) {
        const bf16x8 w = *(const bf16x8*)(brow + st * 64);
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[m] = dot8(w, *(const bf16x8*)(arow[m] + st * 64), acc[m]);
    }
    float* pt = a.split_ws + ((int64_t)unit * sp.split + sl) * 65536;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        float v = acc[m];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        if (kl == 0 && col_ok && m < M) pt[m * 256 + nl] = v;
    }
}

// GEMV plan: all tiles are split units; K slices so that about four workgroups per CU stream
// the weight (each slice a whole number of 64-wide k steps, at least 4 of them)
static SplitPlan plan_gemv(int N, int K) {
    const int tiles = cdiv(N, 256);
    const int nk = K / BK;
    const int64_t target = 4 * (int64_t)device_shape().cus;
    int split = 1;
    while (split < 16 && (int64_t)tiles * 8 * split < target && nk % (split * 2) == 0 && nk / (split * 2) >= 4) split *= 2;
    return SplitPlan{0, tiles, split};
}

static bool gemv_eligible(const GemmArgs& a) {
    return a.M >= 1 && a.M <= GEMV_MAX_M && a.groups == 1 && a.K_a == a.K &&
           (a.epi == EPI_STORE || a.epi == EPI_QKV || a.epi == EPI_RESID || a.epi == EPI_SWIGLU);
}

// C rows of the tail tiles: out = sum over the K slices, in slice order.  One thread per 8
// consecutive columns of one tile row.
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(GemmArgs a, int mt, int nt, int gm, SplitPlan sp) {
    const int tile = blockIdx.y;
    const int e = (blockIdx.x * 256 + threadIdx.x) * 8;      // element of the 256 x 256 tile
    const int ml = e >> 8, nl = e & 255;
    const Tile t = tile_at(sp.full + tile, mt, nt, a.groups, gm);
    const int m = t.tm * 256 + ml, n = t.tn * 256 + nl;
    if (m >= a.M || n >= a.N) return;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* p = a.split_ws + (int64_t)tile * sp.split * 65536 + e;
    for (int k = 0; k < sp.split; ++k) {
        const f32x4 x0 = *(const f32x4*)(p + (int64_t)k * 65536);
        const f32x4 x1 = *(const f32x4*)(p + (int64_t)k * 65536 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { s[i] += x0[i]; s[4 + i] += x1[i]; }
    }
    if (a.epi == EPI_SWIGLU) {            // the gate thread of each 16-column group
        if ((n >> 3) & 1) return;
        float u[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < sp.split; ++k) {
            const f32x4 x0 = *(const f32x4*)(p + 8 + (int64_t)k * 65536);
            const f32x4 x1 = *(const f32x4*)(p + 12 + (int64_t)k * 65536);
#pragma unroll
            for (int i = 0; i < 4; ++i) { u[i] += x0[i]; u[4 + i] += x1[i]; }
        }
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (bf16)(s[i] / (1.f + __expf(-s[i])) * u[i]);
        *(bf16x8*)(a.C + (int64_t)m * a.ldc + (n >> 4) * 8) = o;
        return;
    }
    if (a.epi == EPI_RESID) {
        const bf16x8 r = *(const bf16x8*)(a.R + (int64_t)m * a.ldr + n);
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (bf16)((float)r[i] + s[i]);
        *(bf16x8*)(a.C + (int64_t)m * a.ldc + n) = o;
        return;
    }
    if (a.epi == EPI_QKV) {               // same column handling as the tile epilogue
        const RowInfo ri = row_info(a.rows, m);
        const int64_t slot = a.slots.slot(ri.b, ri.pos);
        const int half = a.d_h / 2;
        const int cc = n - a.q_cols;
        const bool is_k = n >= a.q_cols && cc < a.hd;
        bf16x8 o;
        if (is_k) {
            const bool lo = (cc % a.d_h) < half;
            const int j0 = (cc % a.d_h) % half;
            float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            const float* pp = p + (lo ? half : -half);
            for (int k = 0; k < sp.split; ++k) {
                const f32x4 x0 = *(const f32x4*)(pp + (int64_t)k * 65536);
                const f32x4 x1 = *(const f32x4*)(pp + (int64_t)k * 65536 + 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) { y[i] += x0[i]; y[4 + i] += x1[i]; }
            }
            const float4* cs = (const float4*)(a.rope + ((int64_t)ri.pos * half + j0) * 2);
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2) {
                const float4 t2 = cs[j2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int j = 2 * j2 + u;
                    const float c = u ? t2.z : t2.x, sn = u ? t2.w : t2.y;
                    const float xm = (float)(bf16)s[j], xp = (float)(bf16)y[j];
                    o[j] = (bf16)(lo ? rope_lo(xm, xp, c, sn) : rope_hi(xp, xm, c, sn));
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (bf16)s[i];
        }
        bf16* dst = n < a.q_cols ? a.C + (int64_t)m * a.ldc + n
                                 : (is_k ? a.kc : a.vc) + slot * a.hd + (is_k ? cc : cc - a.hd);
        *(bf16x8*)dst = o;
        return;
    }
    bf16* dst = a.C + (int64_t)m * a.ldc + n;
    if (n + 8 <= a.N) {
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (bf16)s[i];
        *(bf16x8*)dst = o;
    } else {
        for (int i = 0; i < a.N - n; ++i) dst[i] = (bf16)s[i];
    }
}

// K splits of a plain store (one group).  Time is counted in tile-times on the device's CUs:
//   whole tiles:            ceil(tiles / CUs)
//   split tail (split s):   floor(tiles / CUs) + ceil(rem * s / CUs) / s, rem = tiles % CUs
//   every tile split (s):   ceil(tiles * s / CUs) / s
// plus, for split plans, the HBM time of writing and re-reading the fp32 partial tiles
// (only the valid rows are written: min(M, 256) * 256 * 4 bytes each way per partial, at
// ~5 TB/s) in units of one tile's compute (2*256*256*K flops at
// ~4.7 TFLOP/s per CU, the rate these tiles reach).  The cheapest wins (ties keep fewer
// partials); every K slice spans at least 4 k-tiles.
SplitPlan plan_split(int M, int N, int K, int groups, int epi) {
    const int64_t tiles = (int64_t)cdiv(M, 256) * cdiv(N, 256) * groups;
    SplitPlan best{(int)tiles, 0, 1};
    if ((epi != EPI_STORE && epi != EPI_QKV && epi != EPI_RESID && epi != EPI_SWIGLU) || groups != 1 || tiles == 0 ||
        tiles > INT32_MAX / 8)
        return best;
    const int nk = K / BK;
    const int64_t cu = device_shape().cus;
    double best_t = (double)((tiles + cu - 1) / cu);
    int64_t best_parts = 0;
    auto consider = [&](int full, int rem, int split) {
        const int64_t parts = (int64_t)rem * split;
        const double partial_s = parts * (std::min(M, 256) * 256.0 * 4.0 * 2.0) / 5e12;
        const double tile_s = 2.0 * 65536.0 * K / 4.7e12;
        const double t = (double)(full / cu) + (double)((rem * (int64_t)split + cu - 1) / cu) / split +
                         partial_s / tile_s;
        if (t < best_t - 1e-9 || (t < best_t + 1e-9 && best_parts && parts < best_parts)) {
            best_t = t; best_parts = parts; best = SplitPlan{full, rem, split};
        }
    };
    for (int split = 2; split <= 8; split *= 2) {
        if (nk % split != 0 || nk / split < 4) continue;
        const int rem = (int)(tiles % cu);
        if (rem) consider((int)(tiles - rem), rem, split);      // split the last round only
        consider(0, (int)tiles, split);                         // split every tile
    }
    return best;
}

}  // namespace

// Compute units and XCDs of the current device, queried once per device.  Without a usable
// device (workspace sizing on a host that has none) the planners assume a whole MI355X: 256
// CUs in 8 XCDs.  A failed query's error is cleared so that it does not surface at the next
// launch check.
DeviceShape device_shape() {
    constexpr int MAX_DEV = 64;
    static std::atomic<int> cache[MAX_DEV];     // (cus << 8) | xcds, 0 = not queried yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) {
        (void)hipGetLastError();
        return DeviceShape{256, 8};
    }
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, xcds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
            (void)hipGetLastError();
            cus = 256;
        }
        if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds <= 0) {
            (void)hipGetLastError();
            xcds = 1;
        }
        v = (cus << 8) | std::min(xcds, 255);
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return DeviceShape{v >> 8, v & 255};
}

// Score partial sums are written per 256-column block of the output.
int gemm_bf16_block_n() { return 256; }

size_t gemm_bf16_split_bytes(int M, int N, int K, int groups, int epi) {
    GemmArgs probe{};
    probe.M = M; probe.N = N; probe.K = K; probe.K_a = K; probe.groups = groups; probe.epi = epi;
    const SplitPlan sp = gemv_eligible(probe) ? plan_gemv(N, K) : plan_split(M, N, K, groups, epi);
    return sp.rem ? (size_t)sp.rem * sp.split * 65536 * sizeof(float) : 0;
}

// Row-panel group size of the tile order: the one that fetches the fewest operand panel bytes
// per window of w concurrent tiles (an XCD's share of one round: its CUs).
static int pick_group_rows(int mt, int cols, double a_panel, double b_panel, int w) {
    int best = 1;
    double best_bytes = 0.0;
    for (int gm = 1; gm <= w; gm *= 2) {
        const int rows_w = std::min(gm, mt);
        const int cols_w = std::min(cols, std::max(1, w / rows_w));
        const int rows_eff = std::min(mt, std::max(rows_w, w / cols_w));
        const double bytes = rows_eff * a_panel + cols_w * b_panel;
        if (gm == 1 || bytes < best_bytes) { best = gm; best_bytes = bytes; }
    }
    return best;
}

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s) {
    const int mt = cdiv(a.M, 256);
    if ((int64_t)mt * a.groups == 0 || a.N == 0) return hipSuccess;
    const int nt = cdiv(a.N, 256);
    // A row operand shared by several groups (the per-layer reconstruction) is small next to the
    // groups' weights: walking all row panels first streams each weight panel through an XCD
    // once while the row operand stays resident in the last-level cache (measured fastest).
    const DeviceShape dv = device_shape();
    const bool indep = a.a_group_stride != 0;
    if (indep && ((a.epi != EPI_QKV && a.epi != EPI_SQNORM) || a.split_ws)) return hipErrorInvalidValue;
    if ((a.epi == EPI_SQNORM) != (indep && a.K == 2 * a.K_a && a.kv_split > 0 && a.kv_split % BK == 0 &&
                                  a.K_a % BK == 0))
        return hipErrorInvalidValue;
    const int gm = a.groups > 1 && !indep ? mt
                                          : pick_group_rows(mt, nt * (indep ? 1 : a.groups), 256.0 * a.K_a,
                                                            256.0 * a.K, std::max(1, dv.cus / dv.xcds));
    if (a.split_ws && gemv_eligible(a)) {           // few rows: stream the weight, reduce with the epilogue
        const SplitPlan sp = plan_gemv(a.N, a.K);
        const dim3 grid((unsigned)(sp.rem * 8 * sp.split));
        if (a.M <= 1) hipLaunchKernelGGL(gemv_bf16_kernel<1>, grid, dim3(256), 0, s, a, mt, nt, gm, sp);
        else if (a.M <= 2) hipLaunchKernelGGL(gemv_bf16_kernel<2>, grid, dim3(256), 0, s, a, mt, nt, gm, sp);
        else if (a.M <= 4) hipLaunchKernelGGL(gemv_bf16_kernel<4>, grid, dim3(256), 0, s, a, mt, nt, gm, sp);
        else if (a.M <= 8) hipLaunchKernelGGL(gemv_bf16_kernel<8>, grid, dim3(256), 0, s, a, mt, nt, gm, sp);
        else hipLaunchKernelGGL(gemv_bf16_kernel<16>, grid, dim3(256), 0, s, a, mt, nt, gm, sp);
        if (hipError_t e = hipGetLastError()) return e;
        hipLaunchKernelGGL(gemm_split_reduce_kernel, dim3(65536 / (256 * 8), sp.rem), dim3(256), 0, s, a, mt, nt, gm, sp);
        return hipGetLastError();
    }
    SplitPlan sp = plan_split(a.M, a.N, a.K, a.groups, a.epi);
    if (sp.rem && !a.split_ws) sp = SplitPlan{sp.full + sp.rem, 0, 1};   // no workspace: whole tiles
    const int64_t grid = (int64_t)sp.full + (int64_t)sp.rem * sp.split;
    if (a.epi == EPI_SQNORM)
        hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 4, 2, true>), dim3((unsigned)grid), dim3(512), 0, s, a, mt, nt,
                           gm, sp, dv.xcds);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 4, 2, false>), dim3((unsigned)grid), dim3(512), 0, s, a, mt, nt,
                           gm, sp, dv.xcds);
    if (sp.rem) {
        if (hipError_t e = hipGetLastError()) return e;
        hipLaunchKernelGGL(gemm_split_reduce_kernel, dim3(65536 / (256 * 8), sp.rem), dim3(256), 0, s, a, mt, nt, gm, sp);
    }
    return hipGetLastError();
}

}  // namespace kvx
