// la_mfma_bwd.hip -- bf16 causal backward on the gfx950 matrix cores
// (feature width F = D: no cos/sin weights).
//
// The gradient is the exact derivative of the forward (SVD_linear_Attention,
// "Module neuralops.core.triton_kernels.linear_attn", function bwd: autograd
// of fwd with respect to q, k, v).  With g_i = dL/dout_i, gn_i = g_i / den_i,
// c_i = (g_i . out_i) / den_i, and per chunk (C = 64 rows, j <= i masked):
//   A_ij = Phi(q_i).Phi(k_j),  T_ij = g_i.v_j,  U_i = S g_i  (S exclusive),
//   den_i = sum_j A_ij + Phi(q_i).z + eps,
//   c_i   = (sum_j A_ij T_ij + Phi(q_i).U_i) / den_i^2,
//   P_ij  = T_ij / den_i - c_i,
//   dPhi(q_i) = sum_j P_ij Phi(k_j) + U_i / den_i - c_i z
// (k_bwd_q_mfma, forward over chunks), and with (R, r) the exclusive suffix
// sum over later rows of Phi(q_i) gn_i^T and c_i Phi(q_i), summed over the
// n_rep query heads of the KV head (gqa page, bwd: KV gradients are summed
// over the n_rep axis):
//   dPhi(k_j) = sum_i P_ij Phi(q_i) + R v_j - r,
//   dv_j      = sum_i A_ij gn_i + R^T Phi(k_j)
// (k_bwd_kv_mfma, backward over chunks).  k_bwd_q_mfma also writes den_i,
// c_i and each segment's sum of (R, r); a scan forms the suffixes.
//
// Layout of the work: one workgroup per (batch, KV head, segment) serving the
// n_rep query heads; wave w of the D/32 waves owns feature columns
// 32w..32w+31 of the states (S^T in the q-kernel, R^T in the kv-kernel) and of
// dPhi(q), dPhi(k), and value columns 32w..32w+31 of dv.  The three non-zero
// 32x32 tiles of the chunk's C x C matrices are computed by different waves
// and exchanged through LDS (bf16), with the column sums the denominators
// need reduced through LDS in a fixed order.
#include "la_common.h"
#include "la_kernels.h"
#include "la_mfma.h"
#include "la_timing.h"

namespace la {
namespace {

using namespace mf;

constexpr int kLDP = kC + 8;   // row stride of the C x C tiles in LDS

// Tile t of the lower block triangle: (key block, query block).
__device__ __forceinline__ int tile_jb(int t) { return t == 2 ? 1 : 0; }
__device__ __forceinline__ int tile_ib(int t) { return t == 0 ? 0 : 1; }

// A^T and T^T (keys x queries) of tile t, causal mask applied, A rounded to
// bf16.  Ks/Vs: key-side tiles, Qs/Gs: query-side tiles.
template <int F, int D>
__device__ __forceinline__ void tile_AT(int t, const u16 *sK, const u16 *sQ, const u16 *sV,
                                        const u16 *sG, f32x16 &At, f32x16 &Tt) {
    constexpr int LDF = F + 8, LDV = D + 8;
    const int l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
    const int jb = tile_jb(t), ib = tile_ib(t);
    At = zero16();
    Tt = zero16();
#pragma unroll 4
    for (int s = 0; s < F / 16; ++s)
        At = mfma(ld8(sK + (32 * jb + l32) * LDF + 16 * s + 8 * h),
                  ld8(sQ + (32 * ib + l32) * LDF + 16 * s + 8 * h), At);
#pragma unroll 4
    for (int s = 0; s < D / 16; ++s)
        Tt = mfma(ld8(sV + (32 * jb + l32) * LDV + 16 * s + 8 * h),
                  ld8(sG + (32 * ib + l32) * LDV + 16 * s + 8 * h), Tt);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int j = 8 * (r >> 2) + 4 * h + (r & 3);
        const bool keep = jb != ib || j <= l32;
        At[r] = keep ? (float)(__bf16)At[r] : 0.f;
        Tt[r] = keep ? Tt[r] : 0.f;
    }
}

// Store the 32x32 tile (keys x queries accumulator) transposed into a
// row-major [query][key] LDS matrix, bf16.
__device__ __forceinline__ void store_tile_qk(u16 *M, int t, const f32x16 &X) {
    const int l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
    const int jb = tile_jb(t), ib = tile_ib(t);
    u16 *row = M + (32 * ib + l32) * kLDP + 32 * jb + 4 * h;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t lo = (uint32_t)f2bf(X[4 * q4]) | ((uint32_t)f2bf(X[4 * q4 + 1]) << 16);
        const uint32_t hi = (uint32_t)f2bf(X[4 * q4 + 2]) | ((uint32_t)f2bf(X[4 * q4 + 3]) << 16);
        *reinterpret_cast<uint2 *>(row + 8 * q4) = make_uint2(lo, hi);
    }
}

// 4 consecutive bf16 of an LDS row as floats.
__device__ __forceinline__ void ld4f(const u16 *p, float *o) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    o[0] = __uint_as_float(u.x << 16);
    o[1] = __uint_as_float(u.x & 0xffff0000u);
    o[2] = __uint_as_float(u.y << 16);
    o[3] = __uint_as_float(u.y & 0xffff0000u);
}

__device__ __forceinline__ void st4bf(u16 *p, const float *x) {
    const uint32_t lo = (uint32_t)f2bf(x[0]) | ((uint32_t)f2bf(x[1]) << 16);
    const uint32_t hi = (uint32_t)f2bf(x[2]) | ((uint32_t)f2bf(x[3]) << 16);
    *reinterpret_cast<uint2 *>(p) = make_uint2(lo, hi);
}

// ---------------------------------------------------------------------------
// k_bwd_q_mfma: forward over the chunks of one (batch, KV head, segment).
// ---------------------------------------------------------------------------
template <int D, int PHI>
__global__ __launch_bounds__(D * 2) void k_bwd_q_mfma(Args a) {
    constexpr int F = D, NW = D / 32, NT = 2 * D, LDF = F + 8, LDV = D + 8;
    __shared__ __attribute__((aligned(16))) u16 sK[kC * LDF];
    __shared__ __attribute__((aligned(16))) u16 sV[kC * LDV];
    __shared__ __attribute__((aligned(16))) u16 sQ[kC * LDF];
    __shared__ __attribute__((aligned(16))) u16 sG[kC * LDV];
    __shared__ __attribute__((aligned(16))) u16 sQr[kC * LDV];
    __shared__ __attribute__((aligned(16))) u16 sP[kC * kLDP];
    __shared__ float sz[F];
    __shared__ float sDenP[3][32], sAtP[3][32];
    __shared__ float sQU[NW][kC];
    __shared__ float sQZ[kC], sDen[kC], sCc[kC];

    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int t = threadIdx.x, l = t & 63, w = t >> 6, h = l >> 5, l32 = l & 31;
    const size_t SD = (size_t)F * D + F;
    const u16 *kh = static_cast<const u16 *>(a.k) + (size_t)bg * a.N * D;
    const u16 *vh = static_cast<const u16 *>(a.v) + (size_t)bg * a.N * D;

    // S^T tiles (value block db x this wave's feature block), fp32
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + seg) * SD;
    f32x16 St[NW], dR[NW];
#pragma unroll
    for (int db = 0; db < NW; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            St[db][r] = Sp[(size_t)(32 * w + l32) * D + 32 * db + 8 * (r >> 2) + 4 * h + (r & 3)];
        dR[db] = zero16();
    }
    for (int e = t; e < F; e += NT) sz[e] = Sp[(size_t)F * D + e];
    float rr = 0.f;

    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    for (int c0 = row0; c0 < row1; c0 += kC) {
        __syncthreads();
        stage<D, LDF, NT, true, PHI, false>(sK, kh, c0, a.N, a.cw, a.sw);
        stage<D, LDV, NT, false, PHI, false>(sV, vh, c0, a.N, a.cw, a.sw);
        for (int rep = 0; rep < a.nrep; ++rep) {
            const size_t bh = (size_t)b * a.H + (size_t)g * a.nrep + rep;
            const u16 *qh = static_cast<const u16 *>(a.q) + bh * a.N * D;
            const u16 *gh = static_cast<const u16 *>(a.g) + bh * a.N * D;
            u16 *dqh = static_cast<u16 *>(a.dq) + bh * a.N * D;
            if (rep > 0) __syncthreads();
            stage<D, LDF, NT, true, PHI, false>(sQ, qh, c0, a.N, a.cw, a.sw);
            stage<D, LDV, NT, false, PHI, false>(sQr, qh, c0, a.N, a.cw, a.sw);
            stage<D, LDV, NT, false, PHI, false>(sG, gh, c0, a.N, a.cw, a.sw);
            __syncthreads();

            // tiles of A^T, T^T: tile t on wave t % NW
            f32x16 At[2], Tt[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int tt = w + k * NW;
                if (tt < 3) {
                    tile_AT<F, D>(tt, sK, sQ, sV, sG, At[k], Tt[k]);
                    float dA = 0.f, aT = 0.f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        dA += At[k][r];
                        aT += At[k][r] * Tt[k][r];
                    }
                    dA += __shfl_xor(dA, 32);
                    aT += __shfl_xor(aT, 32);
                    if (h == 0) {
                        sDenP[tt][l32] = dA;
                        sAtP[tt][l32] = aT;
                    }
                }
            }
            // U^T = S g for this wave's feature block, both query blocks
            f32x16 U0 = zero16(), U1 = zero16();
#pragma unroll
            for (int db = 0; db < NW; ++db)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const bf16x8 sa = acc_op(St[db], s);
                    const int d0 = 32 * db + 16 * s + 4 * h;
                    U0 = mfma(sa, ld4x2(sG + l32 * LDV + d0), U0);
                    U1 = mfma(sa, ld4x2(sG + (32 + l32) * LDV + d0), U1);
                }
            {   // partial Phi(q_i) . U_i over this wave's features
                float qu0 = 0.f, qu1 = 0.f, x[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int f0 = 32 * w + 8 * q4 + 4 * h;
                    ld4f(sQ + l32 * LDF + f0, x);
#pragma unroll
                    for (int e = 0; e < 4; ++e) qu0 += x[e] * U0[4 * q4 + e];
                    ld4f(sQ + (32 + l32) * LDF + f0, x);
#pragma unroll
                    for (int e = 0; e < 4; ++e) qu1 += x[e] * U1[4 * q4 + e];
                }
                qu0 += __shfl_xor(qu0, 32);
                qu1 += __shfl_xor(qu1, 32);
                if (h == 0) {
                    sQU[w][l32] = qu0;
                    sQU[w][32 + l32] = qu1;
                }
            }
            if (w == NW - 1) {   // Phi(q_i) . z for every row of the chunk
                float acc = 0.f;
                for (int f = 0; f < F; f += 8) {
                    const bf16x8 xq = ld8(sQ + l * LDF + f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc += (float)xq[e] * sz[f + e];
                }
                sQZ[l] = acc;
            }
            __syncthreads();

            // den and c of rows l32 and 32 + l32 (rows past N: neutral)
            float den[2], cc[2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int i = 32 * ib + l32;
                float dsum = ib ? sDenP[1][l32] + sDenP[2][l32] : sDenP[0][l32];
                float gsum = ib ? sAtP[1][l32] + sAtP[2][l32] : sAtP[0][l32];
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) gsum += sQU[ww][i];
                const bool ok = c0 + i < a.N;
                den[ib] = ok ? dsum + sQZ[i] + a.eps : 1.f;
                cc[ib] = ok ? gsum / (den[ib] * den[ib]) : 0.f;
                if (w == 0 && h == 0) {
                    sDen[i] = den[ib];
                    sCc[i] = cc[ib];
                    if (ok) {
                        a.ws_den[bh * a.N + c0 + i] = den[ib];
                        a.ws_c[bh * a.N + c0 + i] = cc[ib];
                    }
                }
            }
            // P tiles into sP as [query][key]
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int tt = w + k * NW;
                if (tt < 3) {
                    const int ib = tile_ib(tt), jb = tile_jb(tt);
                    const float inv = 1.f / den[ib], c = cc[ib];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = 8 * (r >> 2) + 4 * h + (r & 3);
                        const bool keep = jb != ib || j <= l32;
                        Tt[k][r] = keep ? Tt[k][r] * inv - c : 0.f;
                    }
                    store_tile_qk(sP, tt, Tt[k]);
                }
            }
            __syncthreads();
            // G -> gn = G / den, in place (bf16)
            for (int v = t; v < kC * D / 8; v += NT) {
                const int i = v / (D / 8), c8 = (v % (D / 8)) * 8;
                const float inv = 1.f / sDen[i];
                uint4 *p = reinterpret_cast<uint4 *>(sG + i * LDV + c8);
                uint4 u = *p;
                uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = __uint_as_float(wds[e] << 16) * inv;
                    const float hi = __uint_as_float(wds[e] & 0xffff0000u) * inv;
                    wds[e] = (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
                }
                *p = make_uint4(wds[0], wds[1], wds[2], wds[3]);
            }
            if (t < F) {   // r partial: sum_i c_i Phi(q_i)
                float acc = 0.f;
                for (int i = 0; i < kC; ++i) acc += sCc[i] * bf2f(sQ[i * LDF + t]);
                rr += acc;
            }
            __syncthreads();

            // dPhi(q)^T for this wave's feature block
            f32x16 Q0 = zero16(), Q1 = zero16();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k0 = 16 * s + 8 * h;
                const bf16x8 ka = tr8(tr_addr(sK, LDF, k0, 32 * w), tr_addr(sK, LDF, k0 + 4, 32 * w));
                if (s < 2) Q0 = mfma(ka, ld8(sP + l32 * kLDP + 16 * s + 8 * h), Q0);
                Q1 = mfma(ka, ld8(sP + (32 + l32) * kLDP + 16 * s + 8 * h), Q1);
            }
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                f32x16 &Qt = ib ? Q1 : Q0;
                const f32x16 &Ut = ib ? U1 : U0;
                const float inv = 1.f / den[ib], c = cc[ib];
                const int row = c0 + 32 * ib + l32;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int f0 = 32 * w + 8 * q4 + 4 * h;
                    float qr[4], o[4];
                    ld4f(sQr + (32 * ib + l32) * LDV + f0, qr);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float dphi = Qt[4 * q4 + e] + Ut[4 * q4 + e] * inv - sz[f0 + e] * c;
                        o[e] = phi_d<PHI>(qr[e]) * dphi;
                    }
                    if (row < a.N) st4bf(dqh + (size_t)row * D + f0, o);
                }
            }
            // segment partial R += Phi(Q)^T gn (this wave's feature block x all value blocks)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k0 = 16 * s + 8 * h;
                const bf16x8 qa = tr8(tr_addr(sQ, LDF, k0, 32 * w), tr_addr(sQ, LDF, k0 + 4, 32 * w));
#pragma unroll
                for (int db = 0; db < NW; ++db) {
                    const bf16x8 gb = tr8(tr_addr(sG, LDV, k0, 32 * db), tr_addr(sG, LDV, k0 + 4, 32 * db));
                    dR[db] = mfma(qa, gb, dR[db]);
                }
            }
        }
        // carry S^T past this chunk: S^T += V^T Phi(K)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int k0 = 16 * s + 8 * h;
            const bf16x8 kb = tr8(tr_addr(sK, LDF, k0, 32 * w), tr_addr(sK, LDF, k0 + 4, 32 * w));
#pragma unroll
            for (int db = 0; db < NW; ++db) {
                const bf16x8 va = tr8(tr_addr(sV, LDV, k0, 32 * db), tr_addr(sV, LDV, k0 + 4, 32 * db));
                St[db] = mfma(va, kb, St[db]);
            }
        }
        __syncthreads();
        if (t < F) {
            float acc = 0.f;
            for (int j = 0; j < kC; ++j) acc += bf2f(sK[j * LDF + t]);
            sz[t] += acc;
        }
    }
    // this segment's (R, r), summed over the group's query heads
    float *Ro = a.ws_Rp + ((size_t)bg * a.nseg + seg) * SD;
#pragma unroll
    for (int db = 0; db < NW; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            Ro[(size_t)(32 * w + 8 * (r >> 2) + 4 * h + (r & 3)) * D + 32 * db + l32] = dR[db][r];
    if (t < F) Ro[(size_t)F * D + t] = rr;
}

// ---------------------------------------------------------------------------
// k_bwd_kv_mfma: backward over the chunks of one (batch, KV head, segment),
// from the exclusive suffix (R, r) of the segment.
// ---------------------------------------------------------------------------
template <int D, int PHI>
__global__ __launch_bounds__(D * 2) void k_bwd_kv_mfma(Args a) {
    constexpr int F = D, NW = D / 32, NT = 2 * D, LDF = F + 8, LDV = D + 8;
    __shared__ __attribute__((aligned(16))) u16 sK[kC * LDF];
    __shared__ __attribute__((aligned(16))) u16 sV[kC * LDV];
    __shared__ __attribute__((aligned(16))) u16 sKr[kC * LDV];
    __shared__ __attribute__((aligned(16))) u16 sQ[kC * LDF];
    __shared__ __attribute__((aligned(16))) u16 sG[kC * LDV];
    __shared__ __attribute__((aligned(16))) u16 sA[kC * kLDP];
    __shared__ __attribute__((aligned(16))) u16 sP[kC * kLDP];
    __shared__ __attribute__((aligned(16))) u16 sR[F * LDV];
    __shared__ float sr[F], sCc[kC];

    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int t = threadIdx.x, l = t & 63, w = t >> 6, h = l >> 5, l32 = l & 31;
    const size_t SD = (size_t)F * D + F;
    const u16 *kh = static_cast<const u16 *>(a.k) + (size_t)bg * a.N * D;
    const u16 *vh = static_cast<const u16 *>(a.v) + (size_t)bg * a.N * D;
    u16 *dkh = static_cast<u16 *>(a.dk) + (size_t)bg * a.N * D;
    u16 *dvh = static_cast<u16 *>(a.dv) + (size_t)bg * a.N * D;

    // R^T tiles (value block db x this wave's feature block), fp32
    const float *Rp = a.ws_Rs + ((size_t)bg * (a.nseg + 1) + seg) * SD;
    f32x16 Rt[NW];
#pragma unroll
    for (int db = 0; db < NW; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            Rt[db][r] = Rp[(size_t)(32 * w + l32) * D + 32 * db + 8 * (r >> 2) + 4 * h + (r & 3)];
    for (int e = t; e < F; e += NT) sr[e] = Rp[(size_t)F * D + e];

    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    const int nch = (row1 - row0 + kC - 1) / kC;
    for (int ci = nch - 1; ci >= 0; --ci) {
        const int c0 = row0 + ci * kC;
        __syncthreads();
        stage<D, LDF, NT, true, PHI, false>(sK, kh, c0, a.N, a.cw, a.sw);
        stage<D, LDV, NT, false, PHI, false>(sV, vh, c0, a.N, a.cw, a.sw);
        stage<D, LDV, NT, false, PHI, false>(sKr, kh, c0, a.N, a.cw, a.sw);
        // R (bf16, [feature][value]) for the value-gradient's state term
#pragma unroll
        for (int db = 0; db < NW; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = Rt[db][4 * q4 + e];
                st4bf(sR + (32 * w + l32) * LDV + 32 * db + 8 * q4 + 4 * h, x);
            }
        __syncthreads();

        // state terms: dPhi(k)^T = R V^T - r, dv^T = R^T Phi(K)^T
        f32x16 dK[2] = {zero16(), zero16()}, dV[2] = {zero16(), zero16()};
#pragma unroll
        for (int db = 0; db < NW; ++db)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8 ra = acc_op(Rt[db], s);
                const int d0 = 32 * db + 16 * s + 4 * h;
                dK[0] = mfma(ra, ld4x2(sV + l32 * LDV + d0), dK[0]);
                dK[1] = mfma(ra, ld4x2(sV + (32 + l32) * LDV + d0), dK[1]);
            }
#pragma unroll 4
        for (int s = 0; s < F / 16; ++s) {
            const int k0 = 16 * s + 8 * h;
            const bf16x8 ra = tr8(tr_addr(sR, LDV, k0, 32 * w), tr_addr(sR, LDV, k0 + 4, 32 * w));
            dV[0] = mfma(ra, ld8(sK + l32 * LDF + 16 * s + 8 * h), dV[0]);
            dV[1] = mfma(ra, ld8(sK + (32 + l32) * LDF + 16 * s + 8 * h), dV[1]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float rf = sr[32 * w + 8 * (r >> 2) + 4 * h + (r & 3)];
            dK[0][r] -= rf;
            dK[1][r] -= rf;
        }

        for (int rep = 0; rep < a.nrep; ++rep) {
            const size_t bh = (size_t)b * a.H + (size_t)g * a.nrep + rep;
            const u16 *qh = static_cast<const u16 *>(a.q) + bh * a.N * D;
            const u16 *gh = static_cast<const u16 *>(a.g) + bh * a.N * D;
            __syncthreads();   // previous head's tiles and the state-term reads of r are done
            stage<D, LDF, NT, true, PHI, false>(sQ, qh, c0, a.N, a.cw, a.sw);
            // gn = g / den (rows past N: zeros)
            for (int v = t; v < kC * D / 8; v += NT) {
                const int i = v / (D / 8), c8 = (v % (D / 8)) * 8, row = c0 + i;
                uint4 u = make_uint4(0, 0, 0, 0);
                if (row < a.N) {
                    const float inv = 1.f / a.ws_den[bh * a.N + row];
                    u = *reinterpret_cast<const uint4 *>(gh + (size_t)row * D + c8);
                    uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = __uint_as_float(wds[e] << 16) * inv;
                        const float hi = __uint_as_float(wds[e] & 0xffff0000u) * inv;
                        wds[e] = (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
                    }
                    u = make_uint4(wds[0], wds[1], wds[2], wds[3]);
                }
                *reinterpret_cast<uint4 *>(sG + i * LDV + c8) = u;
            }
            for (int i = t; i < kC; i += NT) sCc[i] = c0 + i < a.N ? a.ws_c[bh * a.N + c0 + i] : 0.f;
            __syncthreads();

            // tiles: A (bf16) and P = gn.v - c, stored [query][key]
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int tt = w + k * NW;
                if (tt < 3) {
                    f32x16 At, Tt;
                    tile_AT<F, D>(tt, sK, sQ, sV, sG, At, Tt);
                    const int ib = tile_ib(tt), jb = tile_jb(tt);
                    const float c = sCc[32 * ib + l32];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = 8 * (r >> 2) + 4 * h + (r & 3);
                        const bool keep = jb != ib || j <= l32;
                        Tt[r] = keep ? Tt[r] - c : 0.f;
                    }
                    store_tile_qk(sA, tt, At);
                    store_tile_qk(sP, tt, Tt);
                }
            }
            if (t < F) {
                float acc = 0.f;
                for (int i = 0; i < kC; ++i) acc += sCc[i] * bf2f(sQ[i * LDF + t]);
                sr[t] += acc;
            }
            __syncthreads();

            // in-chunk terms
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k0 = 16 * s + 8 * h;
                const bf16x8 qa = tr8(tr_addr(sQ, LDF, k0, 32 * w), tr_addr(sQ, LDF, k0 + 4, 32 * w));
                const bf16x8 ga = tr8(tr_addr(sG, LDV, k0, 32 * w), tr_addr(sG, LDV, k0 + 4, 32 * w));
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    if (jb == 1 && s < 2) continue;   // queries before key block 1 see none of it
                    const bf16x8 pb = tr8(tr_addr(sP, kLDP, k0, 32 * jb), tr_addr(sP, kLDP, k0 + 4, 32 * jb));
                    const bf16x8 ab = tr8(tr_addr(sA, kLDP, k0, 32 * jb), tr_addr(sA, kLDP, k0 + 4, 32 * jb));
                    dK[jb] = mfma(qa, pb, dK[jb]);
                    dV[jb] = mfma(ga, ab, dV[jb]);
                }
            }
            // R^T += gn^T Phi(Q) for the rows of this chunk
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k0 = 16 * s + 8 * h;
                const bf16x8 qb = tr8(tr_addr(sQ, LDF, k0, 32 * w), tr_addr(sQ, LDF, k0 + 4, 32 * w));
#pragma unroll
                for (int db = 0; db < NW; ++db) {
                    const bf16x8 ga = tr8(tr_addr(sG, LDV, k0, 32 * db), tr_addr(sG, LDV, k0 + 4, 32 * db));
                    Rt[db] = mfma(ga, qb, Rt[db]);
                }
            }
        }
        // dk = phi'(k) dPhi(k), dv; lane holds key j and columns 32w + 8q + 4h + 0..3
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int row = c0 + 32 * jb + l32;
            if (row >= a.N) continue;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int f0 = 32 * w + 8 * q4 + 4 * h;
                float kr[4], ok[4], ov[4];
                ld4f(sKr + (32 * jb + l32) * LDV + f0, kr);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ok[e] = phi_d<PHI>(kr[e]) * dK[jb][4 * q4 + e];
                    ov[e] = dV[jb][4 * q4 + e];
                }
                st4bf(dkh + (size_t)row * D + f0, ok);
                st4bf(dvh + (size_t)row * D + f0, ov);
            }
        }
    }
}

template <int D, int PHI>
hipError_t run(const Args &a, hipStream_t s) {
    constexpr int NT = D * 2, F = D;
    const unsigned n_units = (unsigned)(a.B * a.Hkv);
    const size_t SD = (size_t)F * D + F;
    hipError_t e = mfma_state_run(a, PHI, s);
    if (e != hipSuccess) return e;
    {
        TimedLaunch tl("k_bwd_q_mfma", s);
        hipLaunchKernelGGL((k_bwd_q_mfma<D, PHI>), dim3(n_units * a.nseg), dim3(NT), 0, s, a);
    }
    {
        TimedLaunch tl("k_scan_R", s);
        // per-segment records are already summed over the group's heads
        e = scan_suffix(a.ws_Rp, a.ws_Rs, a.nseg, SD, a.Hkv, a.Hkv, 1, n_units, s);
        if (e != hipSuccess) return e;
    }
    {
        TimedLaunch tl("k_bwd_kv_mfma", s);
        hipLaunchKernelGGL((k_bwd_kv_mfma<D, PHI>), dim3(n_units * a.nseg), dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

bool mfma_bwd_serves(int bf16, int causal, int D, int has_cos) {
    return bf16 && causal && !has_cos && (D == 64 || D == 128);
}

hipError_t mfma_bwd_run(const Args &a, int phi, hipStream_t s) {
    if (a.D == 64) {
        switch (phi) {
            case kElu1: return run<64, kElu1>(a, s);
            case kRelu: return run<64, kRelu>(a, s);
            default: return run<64, kIdentity>(a, s);
        }
    }
    switch (phi) {
        case kElu1: return run<128, kElu1>(a, s);
        case kRelu: return run<128, kRelu>(a, s);
        default: return run<128, kIdentity>(a, s);
    }
}

}  // namespace la
