// la_mfma_fwd.hip -- bf16 causal forward on the gfx950 matrix cores.
//
// Method (SVD_linear_Attention, "Module neuralops.core.triton_kernels.
// linear_attn", module docstring: chunked causal streaming, O(N) memory,
// tiled in on-chip memory; cos/sin modulation; fwd arguments): rows are cut
// into chunks of C = 32 (the state pass sums 64- or 128-row chunks); for
// chunk c with exclusive carried state (S, z)
//   A = (Phi(Q_c) Phi(K_c)^T) masked to j <= i,
//   num = A V_c + Phi(Q_c) S,   den = A 1 + Phi(Q_c) z + eps,   out = num / den,
//   S += Phi(K_c)^T V_c,   z += Phi(K_c)^T 1.
// The sequence of each (batch, KV head) is split into segments that run in
// parallel: k_state_mfma sums each segment's (S, z), a scan forms the
// exclusive prefixes, and k_fwd_mfma runs the chunk loop of one segment from
// its prefix.  One workgroup serves all n_rep query heads of its KV head
// (gqa page, bwd: query head h reads KV head h / n_rep), so K, V and the
// state update are shared by the group.
//
// Matrix products use v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32
// accumulate).  Wave w of the D/32 waves owns value columns 32w..32w+31:
// its slice of S (F/32 accumulator tiles, fp32, in registers) and of the
// output.  Per chunk and head each wave computes the three non-zero 32x32
// tiles of A^T (keys x queries) itself, so no C x C data crosses waves.
// Operands come from LDS tiles stored row-major; contractions over the row
// (token) index read them with ds_read_b64_tr_b16.
#include <type_traits>

#include "la_common.h"
#include "la_kernels.h"
#include "la_mfma.h"
#include "la_timing.h"

namespace la {
namespace {

using namespace mf;

// LDS layout of the forward's tiles: the row-permuted padded layout, under
// which every transposed read and every 16-row read is conflict-free.
template <int D, int F>
struct FwdTiles {
    using TF = PadI<F>;
    using TD = PadI<D>;
};

// S += Phi(K)^T V over the CS rows of the staged chunk for one wave's tiles:
// value block vb and feature blocks FBW*fh + i, i < FBW (natural k order:
// lane half h holds rows 16s + 8h .. +7), and z += Phi(K)^T 1 for the blocks
// i = vb + (D/32) c < FBW of that set into Z[c].  The z products read their K
// operands at the wave's own feature columns (a uniform address), so no
// branch depends on the wave index.
template <int D, int F, int FBW, int CS>
__device__ __forceinline__ void state_update(f32x16 *S, f32x16 *Z, const u16 *sK, const u16 *sV,
                                             int vb, int fh) {
    constexpr int NW = D / 32, ZB = (FBW + NW - 1) / NW;
    using TF = typename FwdTiles<D, F>::TF;
    using TD = typename FwdTiles<D, F>::TD;
    const int h = (threadIdx.x & 63) >> 5;
    const bf16x8 one = ones8();
#pragma unroll
    for (int s = 0; s < CS / 16; ++s) {
        const int k0 = 16 * s + 8 * h;
        const bf16x8 vo = tr8(tr_addr<TD>(sV, k0, 32 * vb), tr_addr<TD>(sV, k0 + 4, 32 * vb));
#pragma unroll
        for (int i = 0; i < FBW; ++i) {
            const int fb = FBW * fh + i;
            const bf16x8 ka = tr8(tr_addr<TF>(sK, k0, 32 * fb), tr_addr<TF>(sK, k0 + 4, 32 * fb));
            S[i] = mfma(ka, vo, S[i]);
        }
#pragma unroll
        for (int c = 0; c < ZB; ++c) {
            if (ZB * NW > FBW && vb + NW * c >= FBW) continue;   // uniform: no such block
            const int zc = 32 * (FBW * fh + vb + NW * c);
            Z[c] = mfma(tr8(tr_addr<TF>(sK, k0, zc), tr_addr<TF>(sK, k0 + 4, zc)), one, Z[c]);
        }
    }
}

// ---------------------------------------------------------------------------
// k_state_mfma: per (batch, KV head, segment) the segment sums
// dS = sum_j Phi(k_j) v_j^T (F x D) and dz = sum_j Phi(k_j), written as fp32
// to the workspace record of the segment.  The next chunk's loads are issued
// before the current chunk's products.  NH wave sets of D/32 waves split the
// feature blocks: wave w owns value block w % (D/32) and the feature blocks
// of set w / (D/32) (the tiles are disjoint, so nothing crosses waves).  At
// F = 256 two sets keep 64 accumulator registers per lane instead of 128, and
// two waves share a SIMD instead of one.
// ---------------------------------------------------------------------------
// Occupancy the state pass is built for: it streams K and V, so more waves
// per SIMD hide more load latency (each shape's registers allow this).
template <int D, int F>
constexpr int state_sets() { return D == 128 ? 2 : 1; }
template <int D, int F>
constexpr int state_waves() { return F == 64 ? 4 : F == 128 && D == 128 ? 4 : 2; }
// Rows per chunk: at D = F = 128 the two wave sets have the registers for
// 128-row chunks, which doubles the bytes each workgroup keeps in flight
// (the pass streams K and V, and in-flight bytes set its rate).
template <int D, int F>
constexpr int state_chunk() { return D == 128 && F == 128 ? 128 : kC; }

template <int D, int F, int PHI, bool COS>
__global__ __launch_bounds__((D * 2 * state_sets<D, F>())) __attribute__((amdgpu_waves_per_eu(state_waves<D, F>()))) void k_state_mfma(Args a, int nseg_run) {
    using TF = typename FwdTiles<D, F>::TF;
    using TD = typename FwdTiles<D, F>::TD;
    constexpr int NH = state_sets<D, F>(), NW = D / 32, NT = D * 2 * NH;
    constexpr int FBW = F / 32 / NH, ZB = (FBW + NW - 1) / NW;   // z tiles per wave (at most)
    constexpr int CS = state_chunk<D, F>();
    static_assert(FBW * NH * 32 == F, "feature blocks split evenly");
    __shared__ __attribute__((aligned(16))) u16 sK[CS * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sV[CS * TD::ld];
    const int seg = blockIdx.x % nseg_run, bg = blockIdx.x / nseg_run;   // segments 0 .. nseg_run-1
    const int t = threadIdx.x, l = t & 63, h = l >> 5, l32 = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index, uniform
    const int vb = w % NW, fh = w / NW;                       // value block, feature set
    const u16 *kh = static_cast<const u16 *>(a.k) + (size_t)bg * a.N * D;
    const u16 *vh = static_cast<const u16 *>(a.v) + (size_t)bg * a.N * D;
    f32x16 S[FBW], Z[ZB];
#pragma unroll
    for (int i = 0; i < FBW; ++i) S[i] = zero16();
#pragma unroll
    for (int c = 0; c < ZB; ++c) Z[c] = zero16();
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    // The next chunk's loads are in flight while the current one is summed.
    // Tiles end at the segment end row1 (segments are multiples of 64 rows,
    // chunks may be 128): rows at or past it load as zeros, like rows past N,
    // so they add nothing; a load wholly past it (the prefetch after the
    // last chunk) is unused.
    // Chunks are summed last to first: the rows this pass reads last are
    // the first ones the forward reads back, so they are the most likely to
    // still sit in the device's last-level cache when it does.
    RawTile<D, NT, CS, D == 128> rK, rV;
    const int clast = row0 + (row1 - row0 - 1) / CS * CS;
    rK.template load<COS>(kh, clast, row1, a.cw, a.sw);
    rV.load(vh, clast, row1);
    for (int c0 = clast; c0 >= row0; c0 -= CS) {
        __syncthreads();
        rK.template store_feat<PHI, COS, TF, false>(sK, c0, row1, nullptr, nullptr);
        rV.template store<TD>(sV);
        __syncthreads();
        const int cn = c0 - CS >= row0 ? c0 - CS : row0;   // the next chunk (after the first: unused)
        rK.template load<COS>(kh, cn, row1, a.cw, a.sw);
        rV.load(vh, cn, row1);
        state_update<D, F, FBW, CS>(S, Z, sK, sV, vb, fh);
    }
    float *out = a.ws_S + ((size_t)bg * (a.nseg + 1) + seg) * ((size_t)F * D + F);
#pragma unroll
    for (int i = 0; i < FBW; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int f = 32 * (FBW * fh + i) + acc_row(r, h);
            out[(size_t)f * D + 32 * vb + l32] = S[i][r];
        }
    // every column of a z tile holds z: lane 0 of each half writes its rows
    // (z tile c is block i = vb + (D/32) c of this wave's set, if it exists)
    if (l32 == 0) {
#pragma unroll
        for (int c = 0; c < ZB; ++c)
            if (vb + NW * c < FBW) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    out[(size_t)F * D + 32 * (FBW * fh + vb + NW * c) + acc_row(r, h)] = Z[c][r];
            }
    }
}

constexpr int kCf = 32;   // forward chunk length: one 32x32 tile of A per head

// Waves per SIMD the causal forward is built for: D = F = 64 (two-wave
// workgroups, six per compute unit) three; F = 256 one.
template <int D, int F>
constexpr int fwd_waves() { return D == 64 && F == 64 ? 3 : F <= 128 ? 2 : 1; }

// ---------------------------------------------------------------------------
// k_fwd_mfma: per (batch, KV head, segment): the chunk loop for all n_rep
// query heads of the KV head, from the segment's exclusive prefix state.
// Chunks of 32 rows keep the working set small enough for two workgroups per
// compute unit; the global loads of the next head / chunk are issued as soon
// as the current tiles are in LDS.  z is carried on the matrix cores too
// (z += Phi(K)^T 1, in fp32 accumulators; wave w owns feature blocks
// w, w + D/32, ...) and mirrored to LDS for the Phi(q).z dot of the staging.
// ---------------------------------------------------------------------------
template <int D, int F, int PHI, bool COS>
__global__ __launch_bounds__(D * 2) __attribute__((amdgpu_waves_per_eu(fwd_waves<D, F>()))) void k_fwd_mfma(Args a) {
    using TF = typename FwdTiles<D, F>::TF;
    using TD = typename FwdTiles<D, F>::TD;
    constexpr int NT = D * 2, NW = D / 32, FB = F / 32, ZB = FB / NW;
    __shared__ __attribute__((aligned(16))) u16 sK[kCf * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sQ[kCf * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sV[kCf * TD::ld];
    __shared__ __attribute__((aligned(16))) u16 sO[kCf * TD::ld];   // output rows of one head
    __shared__ __attribute__((aligned(16))) float sz[F];
    __shared__ float sQZ[kCf];
    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int t = threadIdx.x, l = t & 63, h = l >> 5, l32 = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index, uniform
    const size_t SD = (size_t)F * D + F;
    const u16 *kh = static_cast<const u16 *>(a.k) + (size_t)bg * a.N * D;
    const u16 *vh = static_cast<const u16 *>(a.v) + (size_t)bg * a.N * D;
    const size_t bh0 = (size_t)b * a.H + (size_t)g * a.nrep;
    const u16 *qbase = static_cast<const u16 *>(a.q);
    u16 *obase = static_cast<u16 *>(a.out);

    // exclusive prefix state of this segment: S (F/32 tiles of this wave's
    // value block) and this wave's blocks of z (every column of a z tile holds z)
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + seg) * SD;
    f32x16 S[FB], Z[ZB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int f = 32 * fb + 8 * (r >> 2) + 4 * h + (r & 3);
            S[fb][r] = Sp[(size_t)f * D + 32 * w + l32];
        }
#pragma unroll
    for (int c = 0; c < ZB; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            Z[c][r] = Sp[(size_t)F * D + 32 * (w + NW * c) + 8 * (r >> 2) + 4 * h + (r & 3)];
    for (int e = t; e < F; e += NT) sz[e] = Sp[(size_t)F * D + e];
    const bf16x8 one = ones8();
    // the D = F = 128 instance has registers to spare at two waves per SIMD:
    // it keeps the mask words and reads the Phi(Q) operands ahead
    constexpr bool kRich = D == 128 && F == 128;
    const CausalMaskT cmask(kRich ? l32 : 0, h);

    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    // q is read and out written once: streamed past the caches, which keep
    // the K, V rows the state pass has just read
    RawTile<D, NT, kCf, kRich> rK, rV;
    RawTile<D, NT, kCf, kRich, kRich> rQ;
    rK.template load<COS>(kh, row0, a.N, a.cw, a.sw);
    rV.load(vh, row0, a.N);
    rQ.template load<COS>(qbase + bh0 * a.N * D, row0, a.N, a.cw, a.sw);
    // rows staged in sO wait for the next barrier to be stored (pend_* = where)
    u16 *pend_oh = nullptr;
    int pend_c0 = 0;
    for (int c0 = row0; c0 < row1; c0 += kCf) {
        __syncthreads();   // previous chunk: every LDS read done, sz updated, sO complete
        if (pend_oh) store_rows<D, NT, TD, kRich, kRich>(pend_oh, sO, pend_c0, a.N);
        rK.template store_feat<PHI, COS, TF, false>(sK, c0, a.N, nullptr, nullptr);
        rV.template store<TD>(sV);
        // the next chunk's K, V (unconditional: rows past the segment are
        // loaded clamped and never used, and no register copies are needed)
        rK.template load<COS>(kh, c0 + kCf, a.N, a.cw, a.sw);
        rV.load(vh, c0 + kCf, a.N);
        // the first head's rows are staged here, in straight-line code: staged
        // at the top of the head loop, they would share its header with the
        // later heads, whose wait for their own rows would also wait for the
        // K, V loads just issued
        rQ.template store_feat<PHI, COS, TF, true>(sQ, c0, a.N, sz, sQZ);
        for (int rep = 0; rep < a.nrep; ++rep) {
            u16 *oh = obase + (bh0 + rep) * a.N * D;
            if (rep > 0) {
                __syncthreads();   // every wave is done with the previous head's sQ; sO complete
                rQ.template store_feat<PHI, COS, TF, true>(sQ, c0, a.N, sz, sQZ);
                store_rows<D, NT, TD, kRich, kRich>(pend_oh, sO, pend_c0, a.N);   // after the staging's wait
            }
            __syncthreads();
            {   // Q rows of the next head, or of the first head at the next chunk
                const bool last = rep + 1 == a.nrep;
                rQ.load(qbase + (bh0 + (last ? 0 : rep + 1)) * a.N * D, last ? c0 + kCf : c0, a.N);
                if (COS && last) rQ.load_w(a.cw, a.sw, c0 + kCf, a.N);   // new positions
            }

            // A^T (keys x queries) of the chunk, causal mask, bf16 rounding (the
            // values the A V product consumes) and the in-chunk denominators
            // from the same rounded values
            // (fully unrolled: the first product starts from a zero accumulator
            // operand, with no register clearing)
            f32x16 T = zero16();
#pragma unroll
            for (int s = 0; s < F / 16; ++s)
                T = mfma(ld8<TF>(sK, l32, 16 * s + 8 * h), ld8<TF>(sQ, l32, 16 * s + 8 * h), T);
            if constexpr (!kRich) {
#pragma unroll
                for (int r = 0; r < 16; ++r) T[r] = acc_row(r, h) <= l32 ? T[r] : 0.f;
            }
            const bf16x8 B0 = kRich ? cmask.op(T, 0) : acc_pk(T, 0);
            const bf16x8 B1 = kRich ? cmask.op(T, 1) : acc_pk(T, 1);
            // sum_j A_ij on the matrix cores: 1^T A^T, every row holds it
            const float dsum = mfma(one, B1, mfma(one, B0, zero16()))[0];

            // num^T for this wave's value columns: V^T A^T + S^T Phi(Q)^T.  With
            // registers to spare the Phi(Q) operands are all read before the
            // products, so the chain of products waits for the LDS once.
            bf16x8 qop[FB][2];
            if constexpr (kRich) {
#pragma unroll
                for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                    for (int s = 0; s < 2; ++s) qop[fb][s] = ld4x2<TF>(sQ, l32, 32 * fb + 16 * s + 4 * h);
            }
            f32x16 Nt = zero16();
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int k0 = 16 * s + 4 * h;
                const bf16x8 va = tr8(tr_addr<TD>(sV, k0, 32 * w), tr_addr<TD>(sV, k0 + 8, 32 * w));
                Nt = mfma(va, s ? B1 : B0, Nt);
            }
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    Nt = mfma(acc_pk(S[fb], s),
                              kRich ? qop[fb][s] : ld4x2<TF>(sQ, l32, 32 * fb + 16 * s + 4 * h), Nt);
            const float den = dsum + sQZ[l32] + a.eps;
            stage_out<TD>(sO, Nt, rcp(den), 32 * w);
            pend_oh = oh;
            pend_c0 = c0;
        }
        // carry (S, z) past this chunk: S += Phi(K)^T V, z += Phi(K)^T 1 for
        // the z blocks of this wave (feature blocks w, w + D/32, ...).  With
        // registers to spare those read their K operands again at the wave's
        // own columns (no branch on the block index); otherwise they reuse the
        // S operand of the block behind a uniform branch.
#pragma unroll
        for (int s = 0; s < kCf / 16; ++s) {
            const int k0 = 16 * s + 8 * h;
            const bf16x8 vb = tr8(tr_addr<TD>(sV, k0, 32 * w), tr_addr<TD>(sV, k0 + 4, 32 * w));
#pragma unroll
            for (int fb = 0; fb < FB; ++fb) {
                const bf16x8 ka = tr8(tr_addr<TF>(sK, k0, 32 * fb), tr_addr<TF>(sK, k0 + 4, 32 * fb));
                S[fb] = mfma(ka, vb, S[fb]);
                if (!kRich && fb % NW == w) Z[fb / NW] = mfma(ka, one, Z[fb / NW]);
            }
            if constexpr (kRich) {
#pragma unroll
                for (int c = 0; c < ZB; ++c) {
                    const int zc = 32 * (w + NW * c);
                    Z[c] = mfma(tr8(tr_addr<TF>(sK, k0, zc), tr_addr<TF>(sK, k0 + 4, zc)), one, Z[c]);
                }
            }
        }
        // every head's staging has read sz (they all passed the barrier before
        // their products), so it can take the new z now
        if (l32 == 0) {
#pragma unroll
            for (int c = 0; c < ZB; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sz[32 * (w + NW * c) + 8 * (r >> 2) + 4 * h + (r & 3)] = Z[c][r];
        }
    }
    __syncthreads();
    if (pend_oh) store_rows<D, NT, TD, kRich, kRich>(pend_oh, sO, pend_c0, a.N);
}

// ---------------------------------------------------------------------------
// k_fwd_split_mfma: the causal chunk loop of k_fwd_mfma for the wide cos/sin
// features (F = 2D = 256), with the state's feature blocks split over two
// sets of D/32 waves.  A 32-column slice of S over all F features takes 128
// accumulator registers per lane, which leaves one wave per SIMD; split, each
// wave holds F/64 tiles and two waves share a SIMD.  Wave w owns value block
// w % (D/32) and the feature blocks of half w / (D/32) (its z block is
// feature block w).  The first half forms the chunk's masked A tile over all
// F features; the second half's partial numerators reach the first half
// through LDS, which then normalises and stages the output rows.  Phi(Q) and
// Phi(q).z are double-buffered by head: a chunk's later heads are staged
// during the previous head's products, two barriers per head instead of three.
// ---------------------------------------------------------------------------
template <int D, int F, int PHI, bool COS>
__global__ __launch_bounds__(D * 4) __attribute__((amdgpu_waves_per_eu(2))) void k_fwd_split_mfma(Args a) {
    using TF = typename FwdTiles<D, F>::TF;
    using TD = typename FwdTiles<D, F>::TD;
    constexpr int NT = D * 4, NW = D / 32, FH = F / 64;   // FH feature blocks per half
    static_assert(F == 2 * D, "two feature halves of D/32 blocks each");
    __shared__ __attribute__((aligned(16))) u16 sK[kCf * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sQ2[2][kCf * TF::ld];   // Phi(Q) of a head, by head parity
    __shared__ __attribute__((aligned(16))) u16 sV[kCf * TD::ld];
    __shared__ __attribute__((aligned(16))) u16 sO[kCf * TD::ld];   // output rows of one head
    __shared__ __attribute__((aligned(16))) float sNp[NW][64 * 16];   // second half's numerators
    __shared__ __attribute__((aligned(16))) float sz[F];
    __shared__ float sQZ2[2][kCf];
    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int t = threadIdx.x, l = t & 63, h = l >> 5, l32 = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index, uniform
    const int vb = w % NW, fh = w / NW;                       // value block, feature half
    const size_t SD = (size_t)F * D + F;
    const u16 *kh = static_cast<const u16 *>(a.k) + (size_t)bg * a.N * D;
    const u16 *vh = static_cast<const u16 *>(a.v) + (size_t)bg * a.N * D;
    const size_t bh0 = (size_t)b * a.H + (size_t)g * a.nrep;
    const u16 *qbase = static_cast<const u16 *>(a.q);
    u16 *obase = static_cast<u16 *>(a.out);

    // exclusive prefix state of this segment: this wave's FH tiles of S
    // (feature blocks FH*fh .. FH*fh + FH-1, value block vb) and z block w
    // (every column of the z tile holds z)
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + seg) * SD;
    f32x16 S[FH], Z;
#pragma unroll
    for (int i = 0; i < FH; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            S[i][r] = Sp[(size_t)(32 * (FH * fh + i) + acc_row(r, h)) * D + 32 * vb + l32];
#pragma unroll
    for (int r = 0; r < 16; ++r) Z[r] = Sp[(size_t)F * D + 32 * w + acc_row(r, h)];
    for (int e = t; e < F; e += NT) sz[e] = Sp[(size_t)F * D + e];
    const bf16x8 one = ones8();

    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    RawTile<D, NT, kCf> rK, rV, rQ;
    rK.template load<COS>(kh, row0, a.N, a.cw, a.sw);
    rV.load(vh, row0, a.N);
    rQ.template load<COS>(qbase + bh0 * a.N * D, row0, a.N, a.cw, a.sw);
    // rows staged in sO wait for the next barrier to be stored (pend_* = where)
    u16 *pend_oh = nullptr;
    int pend_c0 = 0;
    for (int c0 = row0; c0 < row1; c0 += kCf) {
        __syncthreads();   // previous chunk: every LDS read done, sz updated, sO complete
        if (pend_oh) store_rows<D, NT, TD>(pend_oh, sO, pend_c0, a.N);
        pend_oh = nullptr;
        rK.template store_feat<PHI, COS, TF, false>(sK, c0, a.N, nullptr, nullptr);
        rV.template store<TD>(sV);
        rK.template load<COS>(kh, c0 + kCf, a.N, a.cw, a.sw);   // next chunk (past the segment: clamped, unused)
        rV.load(vh, c0 + kCf, a.N);
        rQ.template store_feat<PHI, COS, TF, true>(sQ2[0], c0, a.N, sz, sQZ2[0]);
        {   // Q rows of the second head, or of the first head at the next chunk
            const bool last = a.nrep == 1;
            rQ.load(qbase + (bh0 + (last ? 0 : 1)) * a.N * D, last ? c0 + kCf : c0, a.N);
            if (COS && last) rQ.load_w(a.cw, a.sw, c0 + kCf, a.N);   // new positions
        }
        for (int rep = 0; rep < a.nrep; ++rep) {
            u16 *oh = obase + (bh0 + rep) * a.N * D;
            const int cur = rep & 1;
            const u16 *const sQ = sQ2[cur];
            __syncthreads();   // this head's Phi(Q) (and the chunk's K, V) staged; sO complete
            if (pend_oh) store_rows<D, NT, TD>(pend_oh, sO, pend_c0, a.N);   // the previous head's rows
            // num^T of value block vb: the first half adds V^T A^T, each half
            // its feature blocks' S^T Phi(Q)^T.  The first half forms A^T
            // (keys x queries) over all F features, causal mask, bf16 rounding
            // (and the in-chunk denominators), as in k_fwd_mfma
            f32x16 Nt = zero16();
            bf16x8 B0, B1;
            if (fh == 0) {
                f32x16 T = mfma_chain<F / 16, 4>([&](int s) { return ld8<TF>(sK, l32, 16 * s + 8 * h); },
                                                 [&](int s) { return ld8<TF>(sQ, l32, 16 * s + 8 * h); }, zero16());
#pragma unroll
                for (int r = 0; r < 16; ++r) T[r] = acc_row(r, h) <= l32 ? T[r] : 0.f;
                B0 = acc_pk(T, 0);
                B1 = acc_pk(T, 1);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int k0 = 16 * s + 4 * h;
                    const bf16x8 va = tr8(tr_addr<TD>(sV, k0, 32 * vb), tr_addr<TD>(sV, k0 + 8, 32 * vb));
                    Nt = mfma(va, s ? B1 : B0, Nt);
                }
            }
            // (the Phi(Q) operands all read before the products: the chain
            // then waits for the LDS once)
            bf16x8 qop[FH][2];
#pragma unroll
            for (int i = 0; i < FH; ++i)
#pragma unroll
                for (int s = 0; s < 2; ++s) qop[i][s] = ld4x2<TF>(sQ, l32, 32 * (FH * fh + i) + 16 * s + 4 * h);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FH; ++i)
#pragma unroll
                for (int s = 0; s < 2; ++s) Nt = mfma(acc_pk(S[i], s), qop[i][s], Nt);
            if (fh == 1) put_acc(sNp[vb], Nt);
            // the next head's Phi(Q) into the other buffer (last read by the
            // previous head, before the barrier above), then the rows after it
            if (rep + 1 < a.nrep) {
                rQ.template store_feat<PHI, COS, TF, true>(sQ2[cur ^ 1], c0, a.N, sz, sQZ2[cur ^ 1]);
                const bool last = rep + 2 >= a.nrep;
                rQ.load(qbase + (bh0 + (last ? 0 : rep + 2)) * a.N * D, last ? c0 + kCf : c0, a.N);
                if (COS && last) rQ.load_w(a.cw, a.sw, c0 + kCf, a.N);   // new positions
            }
            __syncthreads();
            if (fh == 0) {
                const f32x16 P = get_acc(sNp[vb]);
#pragma unroll
                for (int r = 0; r < 16; ++r) Nt[r] += P[r];
                // sum_j A_ij on the matrix cores: 1^T A^T, every row holds it
                const float dsum = mfma(one, B1, mfma(one, B0, zero16()))[0];
                const float den = dsum + sQZ2[cur][l32] + a.eps;
                stage_out<TD>(sO, Nt, rcp(den), 32 * vb);
            }
            pend_oh = oh;
            pend_c0 = c0;
        }
        // carry this wave's part of (S, z) past the chunk
#pragma unroll
        for (int s = 0; s < kCf / 16; ++s) {
            const int k0 = 16 * s + 8 * h;
            const bf16x8 vo = tr8(tr_addr<TD>(sV, k0, 32 * vb), tr_addr<TD>(sV, k0 + 4, 32 * vb));
#pragma unroll
            for (int i = 0; i < FH; ++i) {
                const int fb = FH * fh + i;
                const bf16x8 ka = tr8(tr_addr<TF>(sK, k0, 32 * fb), tr_addr<TF>(sK, k0 + 4, 32 * fb));
                S[i] = mfma(ka, vo, S[i]);
                if (i == vb) Z = mfma(ka, one, Z);   // feature block w = FH * fh + vb
            }
        }
        // every head's staging has read sz (each before a barrier this wave has
        // passed since), so it can take the new z now
        if (l32 == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sz[32 * w + acc_row(r, h)] = Z[r];
        }
    }
    __syncthreads();
    if (pend_oh) store_rows<D, NT, TD>(pend_oh, sO, pend_c0, a.N);
}

// ---------------------------------------------------------------------------
// k_fwd_bidir_mfma: bidirectional row pass (linear_attn page, module
// docstring: the bidirectional parallel reduction), per (batch, KV head,
// segment of query rows), for all n_rep query heads:
//   out_i = Phi(q_i) S / (Phi(q_i) . z + eps)
// against the totals (S, z) over the whole sequence (the scan's last slot).
// The total S is constant, so each wave keeps its slice as bf16 operands.
// ---------------------------------------------------------------------------
template <int D, int F, int PHI, bool COS>
__global__ __launch_bounds__(D * 2) __attribute__((amdgpu_waves_per_eu(2))) void k_fwd_bidir_mfma(Args a) {
    using TF = typename FwdTiles<D, F>::TF;
    using TD = typename FwdTiles<D, F>::TD;
    constexpr int NT = D * 2, FB = F / 32;
    __shared__ __attribute__((aligned(16))) u16 sQ[kCf * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sO[kCf * TD::ld];   // output rows of one head
    __shared__ __attribute__((aligned(16))) float sz[F];
    __shared__ float sQZ[kCf];
    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int t = threadIdx.x, l = t & 63, h = l >> 5, l32 = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index, uniform
    const size_t SD = (size_t)F * D + F;
    const size_t bh0 = (size_t)b * a.H + (size_t)g * a.nrep;
    const u16 *qbase = static_cast<const u16 *>(a.q);
    u16 *obase = static_cast<u16 *>(a.out);

    // total state: this wave's value block as the A operands of S^T Phi(Q)^T
    // (feature k order of an accumulator: 32 fb + 16 s + 8 (e / 4) + 4 h + e % 4)
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + a.nseg) * SD;
    bf16x8 Sop[FB][2];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int f = 32 * fb + 16 * s + 8 * (e >> 2) + 4 * h + (e & 3);
                Sop[fb][s][e] = (__bf16)Sp[(size_t)f * D + 32 * w + l32];
            }
    for (int e = t; e < F; e += NT) sz[e] = Sp[(size_t)F * D + e];

    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    RawTile<D, NT, kCf> rQ;
    rQ.template load<COS>(qbase + bh0 * a.N * D, row0, a.N, a.cw, a.sw);
    u16 *pend_oh = nullptr;   // rows staged in sO, stored after the next barrier
    int pend_c0 = 0;
    for (int c0 = row0; c0 < row1; c0 += kCf) {
        for (int rep = 0; rep < a.nrep; ++rep) {
            __syncthreads();   // previous head: sQ reads done, sO complete (and sz written)
            // staging first: its wait for the Q rows would otherwise also wait
            // for the output stores issued just before
            rQ.template store_feat<PHI, COS, TF, true>(sQ, c0, a.N, sz, sQZ);
            if (pend_oh) store_rows<D, NT, TD>(pend_oh, sO, pend_c0, a.N);
            __syncthreads();
            {   // Q rows of the next head, or of the first head at the next chunk
                const bool last = rep + 1 == a.nrep;
                rQ.load(qbase + (bh0 + (last ? 0 : rep + 1)) * a.N * D, last ? c0 + kCf : c0, a.N);
                if (COS && last) rQ.load_w(a.cw, a.sw, c0 + kCf, a.N);   // new positions
            }
            f32x16 Nt = zero16();
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    Nt = mfma(Sop[fb][s], ld4x2<TF>(sQ, l32, 32 * fb + 16 * s + 4 * h), Nt);
            stage_out<TD>(sO, Nt, rcp(sQZ[l32] + a.eps), 32 * w);
            pend_oh = obase + (bh0 + rep) * a.N * D;
            pend_c0 = c0;
        }
    }
    __syncthreads();
    if (pend_oh) store_rows<D, NT, TD>(pend_oh, sO, pend_c0, a.N);
}

// Per-segment state sums and their exclusive prefix.  Causal passes read only
// exclusive prefixes, which never include the last segment: its sum is not
// computed (and the scan writes no total).
template <int D, int F, int PHI, bool COS>
hipError_t run_state(const Args &a, bool causal, hipStream_t s) {
    constexpr int NT = D * 2;
    const unsigned n_units = (unsigned)(a.B * a.Hkv);
    const int nseg_run = causal ? a.nseg - 1 : a.nseg;
    if (nseg_run > 0) {
        TimedLaunch tl("k_state_mfma", s);
        hipLaunchKernelGGL((k_state_mfma<D, F, PHI, COS>), dim3(n_units * nseg_run),
                           dim3(NT * state_sets<D, F>()), 0, s, a,
                           nseg_run);
    }
    TimedLaunch tl("k_scan_S", s);
    return scan_state(a.ws_S, a.nseg, (size_t)F * D + F, n_units, causal, s);
}

template <int D, int F, int PHI, bool COS>
hipError_t run(const Args &a, bool causal, hipStream_t s) {
    constexpr int NT = D * 2;
    hipError_t e = run_state<D, F, PHI, COS>(a, causal, s);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(a.B * a.Hkv * a.nseg));
    if constexpr (F == 256) {
        if (causal) {   // F = 2D = 256: the feature blocks split over two wave sets
            TimedLaunch tl("k_fwd_split_mfma", s);
            hipLaunchKernelGGL((k_fwd_split_mfma<D, F, PHI, COS>), grid, dim3(2 * NT), 0, s, a);
            return hipGetLastError();
        }
    }
    if (causal) {
        TimedLaunch tl("k_fwd_mfma", s);
        hipLaunchKernelGGL((k_fwd_mfma<D, F, PHI, COS>), grid, dim3(NT), 0, s, a);
    } else {
        TimedLaunch tl("k_fwd_bidir_mfma", s);
        hipLaunchKernelGGL((k_fwd_bidir_mfma<D, F, PHI, COS>), grid, dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

template <int D, bool COS>
hipError_t by_phi(const Args &a, int phi, bool state_only, bool causal, hipStream_t s) {
    constexpr int F = COS ? 2 * D : D;
    switch (phi) {
        case kElu1:
            return state_only ? run_state<D, F, kElu1, COS>(a, causal, s) : run<D, F, kElu1, COS>(a, causal, s);
        case kRelu:
            return state_only ? run_state<D, F, kRelu, COS>(a, causal, s) : run<D, F, kRelu, COS>(a, causal, s);
        default:
            return state_only ? run_state<D, F, kIdentity, COS>(a, causal, s)
                              : run<D, F, kIdentity, COS>(a, causal, s);
    }
}

hipError_t dispatch(const Args &a, int phi, bool state_only, bool causal, hipStream_t s) {
    const bool cos = a.F == 2 * a.D;
    if (a.D == 64)
        return cos ? by_phi<64, true>(a, phi, state_only, causal, s)
                   : by_phi<64, false>(a, phi, state_only, causal, s);
    return cos ? by_phi<128, true>(a, phi, state_only, causal, s)
               : by_phi<128, false>(a, phi, state_only, causal, s);
}

}  // namespace

bool mfma_fwd_serves(int bf16, int D) { return bf16 && (D == 64 || D == 128); }

hipError_t mfma_fwd_run(const Args &a, int phi, int causal, hipStream_t s) {
    return dispatch(a, phi, false, causal != 0, s);
}

hipError_t mfma_state_run(const Args &a, int phi, int causal, hipStream_t s) {
    return dispatch(a, phi, true, causal != 0, s);
}

}  // namespace la
