// bf16 GEMM on gfx950 matrix cores:  C[m][n] = sum_k A[src(m)][k] * B[n][k], fp32 accumulate.
//
// Both operands are K-contiguous (weights are stored output-major), so every 16-byte global
// load feeds one LDS chunk and every MFMA operand is one 16-byte LDS read.
//
//  * 256x256x64 block tile, 4 waves in 2x2, each wave a 128x128 tile of 8x8
//    v_mfma_f32_16x16x32_bf16 blocks (256 fp32 accumulators per lane).
//  * LDS holds two stages of A and B ([256 rows][8 chunks of 16 B] each, 128 KB in total);
//    chunks are XOR-swizzled per row so the 16-lane fragment reads hit distinct banks.
//    The next K tile is loaded into registers while the current one feeds the MFMAs.
//  * B fragment j of lane l reads tile row (l%16)*8 + j, so after the K loop each lane
//    holds 8 consecutive output columns of every row it owns: the epilogue writes 16-byte
//    chunks with no LDS staging.
//  * Rows of A can be gathered (selected or complement positions of a ragged batch), and
//    the epilogue can write a plain matrix, the K/V cache of a layer (contiguous or paged
//    slots), or per-row partial sums of C[m][n] * Z[m][n] (the score quadratic form).
//  * Tiles are numbered so that every XCD (workgroup i runs on XCD i % 8) owns one
//    contiguous range of tiles; tiles that share the larger operand's panel share an L2.
#include "kvx_common.h"

namespace kvx {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WM = 2, WN = 2;
constexpr int NTH = WM * WN * 64;
constexpr int WTM = BM / WM, WTN = BN / WN;
constexpr int FM = WTM / 16, FN = WTN / 16;
constexpr int A_CH = BM * 8 / NTH;   // 16-byte chunks per thread per A tile
constexpr int B_CH = BN * 8 / NTH;
constexpr int TILE_ELEMS = (BM + BN) * BK;

static_assert(FN == 8, "the epilogue writes 8 consecutive bf16 columns per lane");

struct Tile { int group, tm, tn; };

__device__ __forceinline__ Tile tile_of(int bid, int mt, int nt, int groups, bool n_major) {
    const int per_group = mt * nt;
    const int total = per_group * groups;
    const int xcd = bid & 7, j = bid >> 3;
    const int per = total >> 3, rem = total & 7;
    const int lin = xcd * per + min(xcd, rem) + j;
    Tile t;
    t.group = lin / per_group;
    const int r = lin - t.group * per_group;
    if (n_major) { t.tn = r / mt; t.tm = r - t.tn * mt; }
    else         { t.tm = r / nt; t.tn = r - t.tm * nt; }
    return t;
}

__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(GemmArgs a, int mt, int nt, int n_major) {
    __shared__ __attribute__((aligned(16))) bf16 lds[2 * TILE_ELEMS];
    __shared__ int s_src[BM];
    __shared__ int64_t s_slot[BM];
    __shared__ float s_red[WN][BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const Tile t = tile_of(blockIdx.x, mt, nt, a.groups, n_major != 0);
    const int m0 = t.tm * BM, n0 = t.tn * BN;

    // ---- row map: source row of every tile row, and its cache slot
    if (tid < BM) {
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

    const bf16* Bg = a.B + (int64_t)t.group * a.b_group_stride;
    const int nk = a.K / BK;

    uint4 ra[A_CH], rb[B_CH];
    auto gload = [&](int kt) {
        const int ka = (kt * BK) % a.K_a;
#pragma unroll
        for (int c = 0; c < A_CH; ++c) {
            const int idx = tid + c * NTH, row = idx >> 3, ch = idx & 7;
            const int src = s_src[row];
            ra[c] = src >= 0 ? *(const uint4*)(a.A + (int64_t)src * a.lda + ka + ch * 8)
                             : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < B_CH; ++c) {
            const int idx = tid + c * NTH, row = idx >> 3, ch = idx & 7;
            const int n = n0 + row;
            rb[c] = n < a.N ? *(const uint4*)(Bg + (int64_t)n * a.ldb + kt * BK + ch * 8)
                            : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int stage) {
        bf16* la = lds + stage * TILE_ELEMS;
        bf16* lb = la + BM * BK;
#pragma unroll
        for (int c = 0; c < A_CH; ++c) {
            const int idx = tid + c * NTH, row = idx >> 3, ch = idx & 7;
            *(uint4*)(la + row * BK + ((ch ^ swz(row)) << 3)) = ra[c];
        }
#pragma unroll
        for (int c = 0; c < B_CH; ++c) {
            const int idx = tid + c * NTH, row = idx >> 3, ch = idx & 7;
            *(uint4*)(lb + row * BK + ((ch ^ swz(row / FN)) << 3)) = rb[c];
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    gload(0);
    lstore(0);
    __syncthreads();

    const int lr = lane & 15, lq = lane >> 4;
    for (int kt = 0; kt < nk; ++kt) {
        const int stage = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const bf16* la = lds + stage * TILE_ELEMS;
        const bf16* lb = la + BM * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int ch = ks * 4 + lq;
            bf16x8 bfr[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int nl = wn * WTN + lr * FN + j;
                bfr[j] = *(const bf16x8*)(lb + nl * BK + ((ch ^ swz(nl / FN)) << 3));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int ml = wm * WTM + i * 16 + lr;
                const bf16x8 afr = *(const bf16x8*)(la + ml * BK + ((ch ^ swz(ml)) << 3));
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) lstore(stage ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane owns rows wm*WTM + i*16 + 4*lq + v and columns nl0 .. nl0+7
    const int nl0 = wn * WTN + lr * FN;
    const int ng = n0 + nl0;
    if (a.epi == EPI_SCORE) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ml = wm * WTM + i * 16 + 4 * lq + v;
                const int src = s_src[ml];
                float p = 0.f;
                if (src >= 0 && ng < a.N) {
                    const bf16x8 z = *(const bf16x8*)(a.Z + (int64_t)src * a.ldz + ng);
#pragma unroll
                    for (int j = 0; j < FN; ++j) p += acc[i][j][v] * (float)z[j];
                }
                p += __shfl_xor(p, 1);
                p += __shfl_xor(p, 2);
                p += __shfl_xor(p, 4);
                p += __shfl_xor(p, 8);
                if (lr == 0) s_red[wn][ml] = p;
            }
        }
        __syncthreads();
        if (tid < BM && m0 + tid < a.M) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < WN; ++w) s += s_red[w][tid];
            a.partial[(int64_t)t.tn * a.M + m0 + tid] = s;
        }
        return;
    }
    if (ng >= a.N) return;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int ml = wm * WTM + i * 16 + 4 * lq + v;
            if (s_src[ml] < 0) continue;
            bf16x8 o;
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
            *(bf16x8*)dst = o;
        }
    }
}

}  // namespace

int gemm_bf16_block_n() { return BN; }

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s) {
    const int mt = cdiv(a.M, BM), nt = cdiv(a.N, BN);
    const int64_t total = (int64_t)mt * nt * a.groups;
    if (total == 0) return hipSuccess;
    // read the larger operand once: keep tiles that share its panel on one XCD
    const double a_bytes = (double)a.M * a.K_a, b_bytes = (double)a.N * a.K * a.groups;
    const int n_major = b_bytes > a_bytes ? 1 : 0;
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)total), dim3(NTH), 0, s, a, mt, nt, n_major);
    return hipGetLastError();
}

}  // namespace kvx
