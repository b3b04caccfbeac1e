// la_lowrank.hip -- low-rank projection y = (x V^T) U^T + bias and its
// gradients on the gfx950 matrix cores (SVD_linear_Attention, "Module
// neuralops.core.triton_kernels.low_rank": fwd, and bwd as the gradient of fwd).
//
// Every product is one bf16 GEMM  C[M x N] = A[M x K] B[K x N]  with fp32
// accumulation.  A is stored K-contiguous ([m][k]) or M-contiguous ([k][m]),
// B K-contiguous ([n][k]) or N-contiguous ([k][n]); with t = x V^T, g = grad_out:
//   fwd:  t = x V^T          A = x [m][k]        B = V [n][k]
//         y = t U^T + bias   A = t [m][k]        B = U [n][k]   (bias added per column)
//   bwd:  grad_t = g U       A = g [m][k]        B = U [k][n]
//         grad_x = grad_t V  A = grad_t [m][k]   B = V [k][n]
//         grad_U = g^T t     A = g [k][m]        B = t [k][n]   (K = tokens: split)
//         grad_V = grad_t^T x  A = grad_t [k][m] B = x [k][n]   (K = tokens: split)
//         grad_bias = column sums of g
// t and grad_t are rounded to bf16 between products, as a bf16 evaluation of
// the page's expression rounds them.  Split products write fp32 partials per
// K range, summed in split order; the bias sum is a fixed-order two-pass sum:
// results are bitwise reproducible.
//
// GEMM tiling: a 512-thread workgroup (two waves per SIMD) computes a
// 256 x 256 tile of C; wave (wm, wn) owns 128 x 64 of it as 4 x 2
// accumulators of the 32x32x16 bf16 MFMA (128 fp32 per lane), each computed
// transposed (B operand first) so a lane holds runs of 4 columns of one row
// for the epilogue.  Per 64-wide K step each wave reads 4 A and 2 B operand
// fragments per 16-wide substep (ld8 for K-contiguous tiles, the transposed
// LDS read for the others) and issues 32 MFMAs.  The next K step's
// tiles are loaded into registers while the current one computes and stored
// to the other half of a double-buffered LDS tile, one barrier per K step;
// the stores go out during the last two sub-steps, one between each pair of
// MFMAs, so the LDS writes overlap the products instead of preceding the
// barrier on their own.
// Loads past M, N or the K range stage zeros.  K-contiguous operands need
// K % 8 == 0, the others M (or N) % 8 == 0, all bases 16-byte aligned.
#include <type_traits>

#include "la_common.h"
#include "la_kernels.h"
#include "la_mfma.h"
#include "la_timing.h"

namespace la {
namespace {

using namespace mf;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WAVES_M = 2, WAVES_N = 4, GT = 64 * WAVES_M * WAVES_N;   // 8 waves, 2 per SIMD
constexpr int FM = BM / WAVES_M / 32, FN = BN / WAVES_N / 32;          // 32x32 blocks per wave: 4 x 2
constexpr int STA = BK / 16 - 2, STB = BK / 16 - 1;   // sub-steps that store the next A and B tiles

// LDS tile of one operand for one K step: K-contiguous operands as
// [256 rows (m or n)][64], the others as [64 rows (k)][256].
template <bool KC>
struct OpTile {
    using L = std::conditional_t<KC, Pad<BK>, PadI<BM>>;
    static constexpr int rows = KC ? BM : BK;
    static constexpr int V8 = (KC ? BK : BM) / 8;   // 16-byte vectors per row
    static constexpr int NV = rows * V8 / GT;        // vectors per thread
    static constexpr int elems = rows * L::ld;
    static_assert(NV * GT == rows * V8, "tile splits evenly over the threads");
};

// Tile (mn0, k0) of an operand [MN x K] stored with leading dimension ld:
// every vector is loaded from a clamped, in-range address.
template <bool KC>
__device__ __forceinline__ void load_tile(uint4 (&r)[OpTile<KC>::NV], const u16 *base, long long ld,
                                          int mn0, int k0, int MN, int K) {
    using T = OpTile<KC>;
#pragma unroll
    for (int j = 0; j < T::NV; ++j) {
        const int v = threadIdx.x + j * GT, row = v / T::V8, c8 = (v % T::V8) * 8;
        const int mn = KC ? mn0 + row : mn0 + c8;
        const int k = KC ? k0 + c8 : k0 + row;
        const u16 *p = KC ? base + (long long)min(mn, MN - 1) * ld + min(k, K - 8)
                          : base + (long long)min(k, K - 1) * ld + min(mn, MN - 8);
        r[j] = *reinterpret_cast<const uint4 *>(p);
    }
}

// Replaces the loaded vectors that lie past MN or kend by zeros; a tile that
// reaches past neither (uniform test) is left as loaded.  Masking after the
// load rather than at it keeps the loads in flight through the K step.
template <bool KC>
__device__ __forceinline__ void mask_tile(uint4 (&r)[OpTile<KC>::NV], int mn0, int k0, int MN, int kend) {
    using T = OpTile<KC>;
    if (mn0 + BM > MN || k0 + BK > kend) {
#pragma unroll
        for (int j = 0; j < T::NV; ++j) {
            const int v = threadIdx.x + j * GT, row = v / T::V8, c8 = (v % T::V8) * 8;
            const int mn = KC ? mn0 + row : mn0 + c8;
            const int k = KC ? k0 + c8 : k0 + row;
            if (!(mn < MN && k < kend)) r[j] = make_uint4(0, 0, 0, 0);
        }
    }
}

// Stores the (masked) tile to LDS.
template <bool KC>
__device__ __forceinline__ void put_tile(u16 *s, uint4 (&r)[OpTile<KC>::NV]) {
    using T = OpTile<KC>;
#pragma unroll
    for (int j = 0; j < T::NV; ++j) {
        const int v = threadIdx.x + j * GT, row = v / T::V8, c8 = (v % T::V8) * 8;
        *reinterpret_cast<uint4 *>(s + T::L::at(row, c8)) = r[j];
    }
}

// Operand fragment: rows mn_off + lane % 32 (mn_off a multiple of 32) and
// k = 16 sub + 8 (lane / 32) + 0..7 of the staged K step.
template <bool KC>
__device__ __forceinline__ bf16x8 frag(const u16 *s, int mn_off, int sub) {
    using L = typename OpTile<KC>::L;
    const int l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
    if constexpr (KC) {
        return ld8<L>(s, mn_off + l32, 16 * sub + 8 * h);
    } else {
        const int k0 = 16 * sub + 8 * h;
        return tr8(tr_addr<L>(s, k0, mn_off), tr_addr<L>(s, k0 + 4, mn_off));
    }
}

struct GemmArgs {
    const u16 *A, *B;
    long long lda, ldb;
    int M, N, K;
    int ksplit;             // K elements per split (a multiple of BK); grid.z splits
    u16 *C;                 // bf16 output [M][ldc] (when C32 is null)
    long long ldc;
    const u16 *bias;        // optional bf16 [N], added before rounding
    float *C32;             // fp32 partials [split][M][N] instead of C
    int tiles_n, tiles;     // tiles per row of C, tiles per split
};

template <bool AKC, bool BKC>
struct GemmSmem {
    static constexpr int a = OpTile<AKC>::elems, b = OpTile<BKC>::elems;
    using LC = Pad<BN>;                                       // the bf16 C tile, [BM][BN]
    static constexpr int c = BM * LC::ld;
    static constexpr int elems = 2 * (a + b) > c ? 2 * (a + b) : c;
};

template <bool AKC, bool BKC>
__global__ __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_lowrank_gemm(GemmArgs g) {
    using SM = GemmSmem<AKC, BKC>;
    using LC = typename SM::LC;
    __shared__ __attribute__((aligned(16))) u16 smem[SM::elems];
    auto sA = [&](int c) { return smem + c * SM::a; };                // double-buffered operand tiles
    auto sB = [&](int c) { return smem + 2 * SM::a + c * SM::b; };
    // tiles of one split go to the 8 XCDs in contiguous ranges (blocks are
    // dealt to the XCDs round-robin), so neighbouring tiles share an L2
    int tile = blockIdx.x;
    if (g.tiles % 8 == 0) tile = (blockIdx.x % 8) * (g.tiles / 8) + blockIdx.x / 8;
    const int bm = tile / g.tiles_n, bn = tile % g.tiles_n;
    const int m0 = bm * BM, n0 = bn * BN;
    const int kbeg = blockIdx.z * g.ksplit, kend = min(kbeg + g.ksplit, g.K);
    const int nkt = (kend - kbeg + BK - 1) / BK;
    const int w = threadIdx.x >> 6, wm = w / WAVES_N, wn = w % WAVES_N;
    constexpr int WTM = 32 * FM, WTN = 32 * FN;   // this wave's 128 x 64 part of the tile
    const int l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;

    // acc[j][i] is the transposed 32x32 block: register r of lane (m, h) holds
    // C[32i + m][32j + acc_row(r, h)], so a lane owns runs of 4 columns of a row
    f32x16 acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = zero16();

    uint4 rA[OpTile<AKC>::NV], rB[OpTile<BKC>::NV];
    load_tile<AKC>(rA, g.A, g.lda, m0, kbeg, g.M, g.K);
    load_tile<BKC>(rB, g.B, g.ldb, n0, kbeg, g.N, g.K);
    mask_tile<AKC>(rA, m0, kbeg, g.M, kend);
    mask_tile<BKC>(rB, n0, kbeg, g.N, kend);
    put_tile<AKC>(sA(0), rA);
    put_tile<BKC>(sB(0), rB);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int cur = kt & 1;
        // the next K step (past the range: zeros staged, never read); the
        // scheduling fence keeps these loads ahead of the products
        const int kn = kbeg + (kt + 1) * BK;
        load_tile<AKC>(rA, g.A, g.lda, m0, kn, g.M, g.K);
        load_tile<BKC>(rB, g.B, g.ldb, n0, kn, g.N, g.K);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sub = 0; sub < BK / 16; ++sub) {
            bf16x8 a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) a[i] = frag<AKC>(sA(cur), wm * WTM + 32 * i, sub);
#pragma unroll
            for (int j = 0; j < FN; ++j) b[j] = frag<BKC>(sB(cur), wn * WTN + 32 * j, sub);
            // the next K step goes to the other buffer (free since the last
            // barrier): A's vectors during sub-step STA, B's during STB, each
            // store issued between two products so the writes overlap them
            if (sub == STA) {
                mask_tile<AKC>(rA, m0, kn, g.M, kend);
                put_tile<AKC>(sA(cur ^ 1), rA);
            }
            if (sub == STB) {
                mask_tile<BKC>(rB, n0, kn, g.N, kend);
                put_tile<BKC>(sB(cur ^ 1), rB);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i) acc[j][i] = mfma(b[j], a[i], acc[j][i]);
            if (sub == STA || sub == STB) {
                const int nst = sub == STA ? OpTile<AKC>::NV : OpTile<BKC>::NV;
#pragma unroll
                for (int q = 0; q < FM * FN; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // one MFMA
                    if (q < nst) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // one LDS write
                }
            }
        }
        __syncthreads();
    }

    if (g.C32) {
        // split partials: 16-byte stores of 4 columns per lane and register group
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = m0 + wm * WTM + 32 * i + l32;
                if (m >= g.M) continue;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int n = n0 + wn * WTN + 32 * j + 8 * q4 + 4 * h;
                    if (n >= g.N) continue;
                    *reinterpret_cast<float4 *>(g.C32 + ((long long)blockIdx.z * g.M + m) * g.N + n) =
                        make_float4(acc[j][i][4 * q4], acc[j][i][4 * q4 + 1], acc[j][i][4 * q4 + 2],
                                    acc[j][i][4 * q4 + 3]);
                }
            }
        return;
    }
    // bf16 output: bias added, rounded, staged as the [BM][BN] tile in LDS (the
    // operand tiles are dead after the last barrier), then whole rows stored
    // with 16-byte vectors
    u16 *sC = smem;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int nl = wn * WTN + 32 * j + 8 * q4 + 4 * h;   // tile column of this run of 4
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if (g.bias && n0 + nl < g.N) {
                const uint2 u = *reinterpret_cast<const uint2 *>(g.bias + n0 + nl);
                bv[0] = __uint_as_float(u.x << 16);
                bv[1] = __uint_as_float(u.x & 0xffff0000u);
                bv[2] = __uint_as_float(u.y << 16);
                bv[3] = __uint_as_float(u.y & 0xffff0000u);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int ml = wm * WTM + 32 * i + l32;
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = acc[j][i][4 * q4 + e] + bv[e];
                st4bf(sC + LC::at(ml, nl), x);
            }
        }
    __syncthreads();
    constexpr int V8 = BN / 8;
#pragma unroll 4
    for (int v = threadIdx.x; v < BM * V8; v += GT) {
        const int row = v / V8, c8 = (v % V8) * 8;
        const int m = m0 + row, n = n0 + c8;
        if (m < g.M && n < g.N)
            *reinterpret_cast<uint4 *>(g.C + (long long)m * g.ldc + n) =
                *reinterpret_cast<const uint4 *>(sC + LC::at(row, c8));
    }
}

// C[M][N] (bf16) = sum over splits of P[split][M][N], in split order.
__global__ __launch_bounds__(256) void k_lowrank_splitsum(const float *P, u16 *C, long long MN, int splits) {
    const long long v = (long long)blockIdx.x * blockDim.x + threadIdx.x;   // 8 elements each
    if (v * 8 >= MN) return;
    float s[8];
    const float4 *p = reinterpret_cast<const float4 *>(P + v * 8);
    float4 a = p[0], b = p[1];
    s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w; s[4] = b.x; s[5] = b.y; s[6] = b.z; s[7] = b.w;
    for (int z = 1; z < splits; ++z) {
        const float4 *q = reinterpret_cast<const float4 *>(P + (long long)z * MN + v * 8);
        a = q[0];
        b = q[1];
        s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w; s[4] += b.x; s[5] += b.y; s[6] += b.z; s[7] += b.w;
    }
    *reinterpret_cast<uint4 *>(C + v * 8) =
        make_uint4(pk2(s[0], s[1]), pk2(s[2], s[3]), pk2(s[4], s[5]), pk2(s[6], s[7]));
}

// Bias gradient, pass 1: partial column sums over row block blockIdx.x
// (rows_per rows, in order) of a slice of nc <= 8 * 256 * kColGroups columns
// of g (row stride ld).  The block reads whole row slices, so its loads sweep
// contiguous memory; thread t sums column groups t, t + 256, ... (8 columns each).
constexpr int kColGroups = 4;
__global__ __launch_bounds__(256) void k_lowrank_colsum_slice(const u16 *G, float *P, int M, int nc, int ld,
                                                              int rows_per) {
    const int r0 = blockIdx.x * rows_per, r1 = min(r0 + rows_per, M);
    const int ng = nc / 8;
    float s[kColGroups][8] = {};
    for (int m = r0; m < r1; m += 4) {
        uint4 u[4][kColGroups];   // 4 rows x the thread's column groups in flight
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < kColGroups; ++q) {
                const int cg = threadIdx.x + 256 * q;
                u[j][q] = (m + j < r1 && cg < ng)
                              ? *reinterpret_cast<const uint4 *>(G + (long long)(m + j) * ld + 8 * cg)
                              : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < kColGroups; ++q) {
                const uint32_t wd[4] = {u[j][q].x, u[j][q].y, u[j][q].z, u[j][q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s[q][2 * e] += __uint_as_float(wd[e] << 16);
                    s[q][2 * e + 1] += __uint_as_float(wd[e] & 0xffff0000u);
                }
            }
    }
#pragma unroll
    for (int q = 0; q < kColGroups; ++q) {
        const int cg = threadIdx.x + 256 * q;
        if (cg < ng)
#pragma unroll
            for (int e = 0; e < 8; ++e) P[(long long)blockIdx.x * ld + 8 * cg + e] = s[q][e];
    }
}

// pass 2: the row blocks' partials summed in order, rounded to bf16.  A
// block takes 64 columns; its 4 thread groups each sum a quarter of the
// partials (16 loads in flight per thread), and the quarters are added in
// order through LDS.
__global__ __launch_bounds__(256) void k_lowrank_colsum2(const float *P, u16 *out, int N, int blocks) {
    __shared__ float part[4][64];
    const int c = blockIdx.x * 64 + (threadIdx.x & 63), grp = threadIdx.x >> 6;
    const int per = (blocks + 3) / 4, b0 = grp * per, b1 = min(b0 + per, blocks);
    float s = 0.f;
    if (c < N) {
        for (int b = b0; b < b1; b += 16) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = b + j < b1 ? P[(long long)(b + j) * N + c] : 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) s += v[j];
        }
    }
    part[grp][threadIdx.x & 63] = s;
    __syncthreads();
    if (grp == 0 && c < N) {
        const int t = threadIdx.x;
        out[c] = __builtin_bit_cast(u16, (__bf16)(((part[0][t] + part[1][t]) + part[2][t]) + part[3][t]));
    }
}

template <bool AKC, bool BKC>
hipError_t gemm(const char *name, const u16 *A, long long lda, const u16 *B, long long ldb, int M, int N, int K,
                u16 *C, long long ldc, const u16 *bias, float *C32, int splits, hipStream_t s) {
    GemmArgs g{};
    g.A = A; g.B = B; g.lda = lda; g.ldb = ldb; g.M = M; g.N = N; g.K = K;
    g.ksplit = (int)(((long long)K + splits - 1) / splits);
    g.ksplit = (g.ksplit + BK - 1) / BK * BK;
    g.C = C; g.ldc = ldc; g.bias = bias; g.C32 = C32;
    g.tiles_n = (N + BN - 1) / BN;
    g.tiles = ((M + BM - 1) / BM) * g.tiles_n;
    TimedLaunch tl(name, s);
    hipLaunchKernelGGL((k_lowrank_gemm<AKC, BKC>), dim3(g.tiles, 1, splits), dim3(GT), 0, s, g);
    return hipGetLastError();
}

}  // namespace

int lowrank_splits(int M, int rows, int cols) {
    // enough tiles x splits to fill the chip once (one workgroup per CU), with at
    // least 1024 tokens per split; twice that many took longer, in the products
    // and in summing twice the partials
    const long long tiles = (long long)((rows + BM - 1) / BM) * ((cols + BN - 1) / BN);
    int s = 1;
    while (tiles * s < 256 && (long long)M / (2 * s) >= 1024) s *= 2;
    return s;
}

// row blocks of 64 rows (at most 512): enough workgroups to stream g at HBM speed
int lowrank_bias_blocks(int M) { return M >= 64 * 512 ? 512 : (M + 63) / 64; }

hipError_t lowrank_fwd_run(const LowRankArgs &a, hipStream_t s) {
    hipError_t e = gemm<true, true>("k_lowrank_gemm_xVt", a.x, a.n_in, a.V, a.n_in, a.M, a.rank, a.n_in,
                                    a.t, a.rank, nullptr, nullptr, 1, s);
    if (e != hipSuccess) return e;
    return gemm<true, true>("k_lowrank_gemm_tUt", a.t, a.rank, a.U, a.rank, a.M, a.n_out, a.rank, a.y,
                            a.n_out, a.bias, nullptr, 1, s);
}

hipError_t lowrank_bwd_run(const LowRankArgs &a, hipStream_t s) {
    hipError_t e;
    if ((e = gemm<true, true>("k_lowrank_gemm_xVt", a.x, a.n_in, a.V, a.n_in, a.M, a.rank, a.n_in, a.t,
                              a.rank, nullptr, nullptr, 1, s)) != hipSuccess) return e;
    if ((e = gemm<true, false>("k_lowrank_gemm_gU", a.g, a.n_out, a.U, a.rank, a.M, a.rank, a.n_out,
                               a.gt, a.rank, nullptr, nullptr, 1, s)) != hipSuccess) return e;
    if ((e = gemm<true, false>("k_lowrank_gemm_gtV", a.gt, a.rank, a.V, a.n_in, a.M, a.n_in, a.rank,
                               a.gx, a.n_in, nullptr, nullptr, 1, s)) != hipSuccess) return e;
    const int sU = lowrank_splits(a.M, a.n_out, a.rank);
    if ((e = gemm<false, false>("k_lowrank_gemm_gTt", a.g, a.n_out, a.t, a.rank, a.n_out, a.rank, a.M,
                                nullptr, 0, nullptr, a.part, sU, s)) != hipSuccess) return e;
    {
        TimedLaunch tl("k_lowrank_splitsum", s);
        const long long mn = (long long)a.n_out * a.rank;
        hipLaunchKernelGGL(k_lowrank_splitsum, dim3((unsigned)((mn / 8 + 255) / 256)), dim3(256), 0, s,
                           a.part, a.gU, mn, sU);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int sV = lowrank_splits(a.M, a.rank, a.n_in);
    if ((e = gemm<false, false>("k_lowrank_gemm_gtTx", a.gt, a.rank, a.x, a.n_in, a.rank, a.n_in, a.M,
                                nullptr, 0, nullptr, a.part, sV, s)) != hipSuccess) return e;
    {
        TimedLaunch tl("k_lowrank_splitsum", s);
        const long long mn = (long long)a.rank * a.n_in;
        hipLaunchKernelGGL(k_lowrank_splitsum, dim3((unsigned)((mn / 8 + 255) / 256)), dim3(256), 0, s,
                           a.part, a.gV, mn, sV);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.gbias) {
        const int blocks = lowrank_bias_blocks(a.M);
        const int rows_per = (a.M + blocks - 1) / blocks;
        {
            TimedLaunch tl("k_lowrank_colsum", s);
            for (int c0 = 0; c0 < a.n_out; c0 += 8 * 256 * kColGroups) {   // column slices of the kernel's width
                const int nc = min(a.n_out - c0, 8 * 256 * kColGroups);
                hipLaunchKernelGGL(k_lowrank_colsum_slice, dim3((unsigned)blocks), dim3(256), 0, s, a.g + c0,
                                   a.bpart + c0, a.M, nc, a.n_out, rows_per);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
        }
        TimedLaunch tl2("k_lowrank_colsum2", s);
        hipLaunchKernelGGL(k_lowrank_colsum2, dim3((unsigned)((a.n_out + 63) / 64)), dim3(256), 0, s,
                           a.bpart, a.gbias, a.n_out, blocks);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace la
