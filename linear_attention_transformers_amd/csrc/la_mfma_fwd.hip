// la_mfma_fwd.hip -- bf16 causal forward on the gfx950 matrix cores.
//
// Method (SVD_linear_Attention, "Module neuralops.core.triton_kernels.
// linear_attn", module docstring: chunked causal streaming, O(N) memory,
// tiled in on-chip memory; cos/sin modulation; fwd arguments): rows are cut
// into chunks of C = 64; for chunk c with exclusive carried state (S, z)
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
#include "la_common.h"
#include "la_kernels.h"
#include "la_mfma.h"
#include "la_timing.h"

namespace la {
namespace {

using namespace mf;

// S[fb] += Phi(K)^T V over the 64 rows of the staged chunk, for this wave's
// value columns (natural k order: lane half h holds rows 16s + 8h .. +7).
template <int F, int LDF, int LDV>
__device__ __forceinline__ void state_update(f32x16 *S, const u16 *sK, const u16 *sV, int w) {
    const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int s = 0; s < kC / 16; ++s) {
        const int k0 = 16 * s + 8 * h;
        const bf16x8 vb = tr8(tr_addr(sV, LDV, k0, 32 * w), tr_addr(sV, LDV, k0 + 4, 32 * w));
#pragma unroll
        for (int fb = 0; fb < F / 32; ++fb) {
            const bf16x8 ka = tr8(tr_addr(sK, LDF, k0, 32 * fb), tr_addr(sK, LDF, k0 + 4, 32 * fb));
            S[fb] = mfma(ka, vb, S[fb]);
        }
    }
}

// ---------------------------------------------------------------------------
// k_state_mfma: per (batch, KV head, segment) the segment sums
// dS = sum_j Phi(k_j) v_j^T (F x D) and dz = sum_j Phi(k_j), written as fp32
// to the workspace record of the segment.
// ---------------------------------------------------------------------------
template <int D, int F, int PHI, bool COS>
__global__ __launch_bounds__(D * 2) void k_state_mfma(Args a) {
    constexpr int NT = D * 2, LDF = F + 8, LDV = D + 8, FB = F / 32;
    __shared__ __attribute__((aligned(16))) u16 sK[kC * LDF];
    __shared__ __attribute__((aligned(16))) u16 sV[kC * LDV];
    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int t = threadIdx.x, l = t & 63, w = t >> 6, h = l >> 5, l32 = l & 31;
    const u16 *kh = static_cast<const u16 *>(a.k) + (size_t)bg * a.N * D;
    const u16 *vh = static_cast<const u16 *>(a.v) + (size_t)bg * a.N * D;
    f32x16 S[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) S[fb] = zero16();
    float z = 0.f;
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    for (int c0 = row0; c0 < row1; c0 += kC) {
        __syncthreads();
        stage<D, LDF, NT, true, PHI, COS>(sK, kh, c0, a.N, a.cw, a.sw);
        stage<D, LDV, NT, false, PHI, COS>(sV, vh, c0, a.N, a.cw, a.sw);
        __syncthreads();
        state_update<F, LDF, LDV>(S, sK, sV, w);
        if (t < F)
            for (int j = 0; j < kC; ++j) z += bf2f(sK[j * LDF + t]);
    }
    float *out = a.ws_S + ((size_t)bg * (a.nseg + 1) + seg) * ((size_t)F * D + F);
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int f = 32 * fb + 8 * (r >> 2) + 4 * h + (r & 3);
            out[(size_t)f * D + 32 * w + l32] = S[fb][r];
        }
    if (t < F) out[(size_t)F * D + t] = z;
}

// ---------------------------------------------------------------------------
// k_fwd_mfma: per (batch, KV head, segment): the chunk loop for all n_rep
// query heads of the KV head, from the segment's exclusive prefix state.
// ---------------------------------------------------------------------------
template <int D, int F, int PHI, bool COS>
__global__ __launch_bounds__(D * 2) void k_fwd_mfma(Args a) {
    constexpr int NT = D * 2, LDF = F + 8, LDV = D + 8, FB = F / 32;
    __shared__ __attribute__((aligned(16))) u16 sK[kC * LDF];
    __shared__ __attribute__((aligned(16))) u16 sQ[kC * LDF];
    __shared__ __attribute__((aligned(16))) u16 sV[kC * LDV];
    __shared__ float sz[F];
    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int t = threadIdx.x, l = t & 63, w = t >> 6, h = l >> 5, l32 = l & 31;
    const size_t SD = (size_t)F * D + F;
    const u16 *kh = static_cast<const u16 *>(a.k) + (size_t)bg * a.N * D;
    const u16 *vh = static_cast<const u16 *>(a.v) + (size_t)bg * a.N * D;

    // exclusive prefix state of this segment
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + seg) * SD;
    f32x16 S[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int f = 32 * fb + 8 * (r >> 2) + 4 * h + (r & 3);
            S[fb][r] = Sp[(size_t)f * D + 32 * w + l32];
        }
    for (int e = t; e < F; e += NT) sz[e] = Sp[(size_t)F * D + e];

    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    for (int c0 = row0; c0 < row1; c0 += kC) {
        __syncthreads();   // previous chunk: sK, sV, sQ reads and the z update done
        stage<D, LDF, NT, true, PHI, COS>(sK, kh, c0, a.N, a.cw, a.sw);
        stage<D, LDV, NT, false, PHI, COS>(sV, vh, c0, a.N, a.cw, a.sw);
        for (int rep = 0; rep < a.nrep; ++rep) {
            const size_t bh = (size_t)b * a.H + (size_t)g * a.nrep + rep;
            const u16 *qh = static_cast<const u16 *>(a.q) + bh * a.N * D;
            u16 *oh = static_cast<u16 *>(a.out) + bh * a.N * D;
            if (rep > 0) __syncthreads();   // every wave is done with the previous head's sQ
            stage<D, LDF, NT, true, PHI, COS>(sQ, qh, c0, a.N, a.cw, a.sw);
            __syncthreads();

            // A^T tiles (keys x queries): T00 = (j 0-31, i 0-31), T01 = (j 0-31,
            // i 32-63), T11 = (j 32-63, i 32-63); (j 32-63, i 0-31) is masked out.
            f32x16 T00 = zero16(), T01 = zero16(), T11 = zero16();
#pragma unroll 4
            for (int s = 0; s < F / 16; ++s) {
                const int k = 16 * s + 8 * h;
                const bf16x8 k0 = ld8(sK + l32 * LDF + k);
                const bf16x8 k1 = ld8(sK + (32 + l32) * LDF + k);
                const bf16x8 q0 = ld8(sQ + l32 * LDF + k);
                const bf16x8 q1 = ld8(sQ + (32 + l32) * LDF + k);
                T00 = mfma(k0, q0, T00);
                T01 = mfma(k0, q1, T01);
                T11 = mfma(k1, q1, T11);
            }
            // causal mask on the diagonal tiles, bf16 rounding (the values the
            // A V product consumes) and the intra-chunk denominators
            float d0 = 0.f, d1 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = 8 * (r >> 2) + 4 * h + (r & 3);
                const float x00 = (__bf16)(j <= l32 ? T00[r] : 0.f);
                const float x11 = (__bf16)(j <= l32 ? T11[r] : 0.f);
                const float x01 = (__bf16)T01[r];
                T00[r] = x00;
                T11[r] = x11;
                T01[r] = x01;
                d0 += x00;
                d1 += x01 + x11;
            }
            d0 += __shfl_xor(d0, 32);
            d1 += __shfl_xor(d1, 32);
            // Phi(q_i) . z for i = l32 and 32 + l32, the two lane halves splitting F
            float qz0 = 0.f, qz1 = 0.f;
#pragma unroll 2
            for (int f = h * (F / 2); f < (h + 1) * (F / 2); f += 8) {
                const bf16x8 x0 = ld8(sQ + l32 * LDF + f);
                const bf16x8 x1 = ld8(sQ + (32 + l32) * LDF + f);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float zf = sz[f + e];
                    qz0 += (float)x0[e] * zf;
                    qz1 += (float)x1[e] * zf;
                }
            }
            qz0 += __shfl_xor(qz0, 32);
            qz1 += __shfl_xor(qz1, 32);
            const float den0 = d0 + qz0 + a.eps, den1 = d1 + qz1 + a.eps;

            // num^T for this wave's value columns: N0 (queries 0-31), N1 (32-63)
            f32x16 N0 = zero16(), N1 = zero16();
#pragma unroll
            for (int s = 0; s < 2; ++s) {   // keys 0-31
                const int k0 = 16 * s + 4 * h;
                const bf16x8 va = tr8(tr_addr(sV, LDV, k0, 32 * w), tr_addr(sV, LDV, k0 + 8, 32 * w));
                N0 = mfma(va, acc_op(T00, s), N0);
                N1 = mfma(va, acc_op(T01, s), N1);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {   // keys 32-63
                const int k0 = 32 + 16 * s + 4 * h;
                const bf16x8 va = tr8(tr_addr(sV, LDV, k0, 32 * w), tr_addr(sV, LDV, k0 + 8, 32 * w));
                N1 = mfma(va, acc_op(T11, s), N1);
            }
            // inter-chunk term: num^T += S^T Phi(Q)^T (S rounded to bf16)
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const bf16x8 sa = acc_op(S[fb], s);
                    const int f0 = 32 * fb + 16 * s + 4 * h;
                    N0 = mfma(sa, ld4x2(sQ + l32 * LDF + f0), N0);
                    N1 = mfma(sa, ld4x2(sQ + (32 + l32) * LDF + f0), N1);
                }
            // out[i][d] = num / den; lane holds query i (= l32 or 32 + l32) and
            // value columns 32w + 8q + 4h + 0..3, q = 0..3
            const float inv0 = 1.f / den0, inv1 = 1.f / den1;
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int row = c0 + 32 * ib + l32;
                if (row < a.N) {
                    const f32x16 &Nt = ib ? N1 : N0;
                    const float inv = ib ? inv1 : inv0;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const uint32_t lo = (uint32_t)f2bf(Nt[4 * q4] * inv) |
                                            ((uint32_t)f2bf(Nt[4 * q4 + 1] * inv) << 16);
                        const uint32_t hi = (uint32_t)f2bf(Nt[4 * q4 + 2] * inv) |
                                            ((uint32_t)f2bf(Nt[4 * q4 + 3] * inv) << 16);
                        *reinterpret_cast<uint2 *>(oh + (size_t)row * D + 32 * w + 8 * q4 + 4 * h) =
                            make_uint2(lo, hi);
                    }
                }
            }
        }
        // carry the state past this chunk
        state_update<F, LDF, LDV>(S, sK, sV, w);
        __syncthreads();   // all heads have read z
        if (t < F) {
            float acc = 0.f;
            for (int j = 0; j < kC; ++j) acc += bf2f(sK[j * LDF + t]);
            sz[t] += acc;
        }
    }
}

template <int D, int F, int PHI, bool COS>
hipError_t run_state(const Args &a, hipStream_t s) {
    constexpr int NT = D * 2;
    const unsigned n_units = (unsigned)(a.B * a.Hkv);
    {
        TimedLaunch tl("k_state_mfma", s);
        hipLaunchKernelGGL((k_state_mfma<D, F, PHI, COS>), dim3(n_units * a.nseg), dim3(NT), 0, s, a);
    }
    TimedLaunch tl("k_scan_S", s);
    return scan_state(a.ws_S, a.nseg, (size_t)F * D + F, n_units, s);
}

template <int D, int F, int PHI, bool COS>
hipError_t run(const Args &a, hipStream_t s) {
    constexpr int NT = D * 2;
    hipError_t e = run_state<D, F, PHI, COS>(a, s);
    if (e != hipSuccess) return e;
    {
        TimedLaunch tl("k_fwd_mfma", s);
        hipLaunchKernelGGL((k_fwd_mfma<D, F, PHI, COS>), dim3((unsigned)(a.B * a.Hkv * a.nseg)),
                           dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

template <int D, bool COS>
hipError_t by_phi(const Args &a, int phi, bool state_only, hipStream_t s) {
    constexpr int F = COS ? 2 * D : D;
    switch (phi) {
        case kElu1: return state_only ? run_state<D, F, kElu1, COS>(a, s) : run<D, F, kElu1, COS>(a, s);
        case kRelu: return state_only ? run_state<D, F, kRelu, COS>(a, s) : run<D, F, kRelu, COS>(a, s);
        default:
            return state_only ? run_state<D, F, kIdentity, COS>(a, s) : run<D, F, kIdentity, COS>(a, s);
    }
}

hipError_t dispatch(const Args &a, int phi, bool state_only, hipStream_t s) {
    const bool cos = a.F == 2 * a.D;
    if (a.D == 64)
        return cos ? by_phi<64, true>(a, phi, state_only, s) : by_phi<64, false>(a, phi, state_only, s);
    return cos ? by_phi<128, true>(a, phi, state_only, s) : by_phi<128, false>(a, phi, state_only, s);
}

}  // namespace

bool mfma_fwd_serves(int bf16, int causal, int D) {
    return bf16 && causal && (D == 64 || D == 128);
}

hipError_t mfma_fwd_run(const Args &a, int phi, hipStream_t s) { return dispatch(a, phi, false, s); }

hipError_t mfma_state_run(const Args &a, int phi, hipStream_t s) { return dispatch(a, phi, true, s); }

}  // namespace la
