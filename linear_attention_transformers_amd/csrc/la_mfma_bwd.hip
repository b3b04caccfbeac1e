// la_mfma_bwd.hip -- bf16 causal backward on the gfx950 matrix cores
// (feature width F = D: no cos/sin weights).
//
// The gradient is the exact derivative of the forward (SVD_linear_Attention,
// "Module neuralops.core.triton_kernels.linear_attn", function bwd: autograd
// of fwd with respect to q, k, v).  With g_i = dL/dout_i, gn_i = g_i / den_i,
// c_i = (g_i . out_i) / den_i, and per chunk (C = 32 rows, j <= i masked):
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
// c_i and each segment's sum of (R, r); a scan forms the suffixes.  The
// chain rule through phi takes phi' from the staged bf16 features
// (phi_d_feat), so the raw q and k rows are not kept.
//
// LDS tiles use the permuted padded layout (PadI): transposed 4-row reads
// are conflict-free in it.
//
// Layout of the work: one workgroup per (batch, KV head) and run of
// consecutive segments (one, or several where fewer, longer workgroups pay)
// serving the n_rep query heads.  Per chunk and head one wave forms each
// 32x32 C x C tile (A, T in the q-kernel; A, P in the kv-kernel) for the
// workgroup, and each wave owns a 32-wide block of the feature columns of
// the state (S^T in the q-kernel, R^T in the kv-kernel), of dPhi(q) /
// dPhi(k), and of the value columns of dv.  The only cross-wave reduction, Phi(q_i).U_i over the
// feature blocks, goes through LDS in a fixed order.  In the q-kernel a
// second set of waves accumulates the segment's (R, r) so the two
// register-heavy states live in different waves.
#include <atomic>

#include "la_common.h"
#include "la_kernels.h"
#include "la_mfma.h"
#include "la_timing.h"

namespace la {
namespace {

using namespace mf;

constexpr int kCb = 32;   // backward chunk length: one 32x32 tile per head

// ---------------------------------------------------------------------------
// k_bwd_q_mfma: forward over the 32-row chunks of one (batch, KV head,
// segment).  Waves 0 .. D/32-1 ("state waves") hold S^T (z lives in LDS,
// each state wave adding its block's chunk sums) and produce dq; waves
// D/32 .. 2D/32-1 ("R waves") accumulate the segment's
// R = sum_i Phi(q_i) gn_i^T (feature block w - D/32 x all value blocks) and
// r = sum_i c_i Phi(q_i), summed over the group's query heads.  Per chunk and
// head the first two R waves also compute the 32x32 tiles A^T (with the
// denominators) and T^T and pass them to the state waves through LDS, which
// meanwhile form U = S g (the A wave's chain is the longer of the two).
// After that exchange (one barrier) the two wave kinds run independently: the
// R update needs only 1/den, and the R waves recompute c for r.
// ---------------------------------------------------------------------------
template <int D, int PHI, bool CAUSAL, bool MULTI>
__global__ __launch_bounds__(D * 4) __attribute__((amdgpu_waves_per_eu(2)))
void k_bwd_q_mfma(Args a, int qm_arg) {
    constexpr int F = D, NW = D / 32, NT = 4 * D;
    using TF = PadI<F>;
    using TD = PadI<D>;
    __shared__ __attribute__((aligned(16))) u16 sK[kCb * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sV[kCb * TD::ld];
    __shared__ __attribute__((aligned(16))) u16 sQ[kCb * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sG[kCb * TD::ld];
    __shared__ __attribute__((aligned(16))) float sz[F];
    __shared__ __attribute__((aligned(16))) float sInv[kCb];
    __shared__ __attribute__((aligned(16))) float sAt[64 * 16], sTt[64 * 16];   // accumulator tiles
    __shared__ float sQZ[kCb], sDen[kCb], sQU[NW][kCb];
    __shared__ __attribute__((aligned(16))) float sCw[NW][kCb];   // each R wave's c, for its operands

    // this workgroup walks the qm consecutive segments seg0 .. seg0 + qm - 1
    // (its state carry runs through their boundaries) and writes each one's
    // (R, r) record; without MULTI, qm = 1 at compile time and the segment
    // loop below is a single pass
    const int qm = MULTI ? qm_arg : 1;
    const int nq = (a.nseg + qm - 1) / qm;
    const int seg0 = (blockIdx.x % nq) * qm, bg = blockIdx.x / nq;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    // w is left per-lane: declared uniform, the wave-role branches keep both
    // roles' registers live and the kernel spills
    const int t = threadIdx.x, l = t & 63, w = t >> 6, h = l >> 5, l32 = l & 31;
    const bool state_wave = w < NW;
    const int wr = w - NW;   // feature block of an R wave
    const size_t SD = (size_t)F * D + F;
    const u16 *kh = static_cast<const u16 *>(a.k) + (size_t)bg * a.N * D;
    const u16 *vh = static_cast<const u16 *>(a.v) + (size_t)bg * a.N * D;
    const size_t bh0 = (size_t)b * a.H + (size_t)g * a.nrep;
    const u16 *qbase = static_cast<const u16 *>(a.q);
    const u16 *gbase = static_cast<const u16 *>(a.g);
    u16 *dqbase = static_cast<u16 *>(a.dq);

    // state waves: S^T tiles (value block db x feature block w), the
    // segment's exclusive prefix (causal) or the sequence total
    // R waves: R tiles (feature block wr x value block db)
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + (CAUSAL ? seg0 : a.nseg)) * SD;
    f32x16 X[NW];
    if (state_wave) {
#pragma unroll
        for (int db = 0; db < NW; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                X[db][r] = Sp[(size_t)(32 * w + l32) * D + 32 * db + acc_row(r, h)];
    } else {
#pragma unroll
        for (int db = 0; db < NW; ++db) X[db] = zero16();
    }
    for (int e = t; e < F; e += NT) sz[e] = Sp[(size_t)F * D + e];
    // R waves: this lane's part of r for feature 32 wr + l32 (rows of its half)
    float racc = 0.f;
    const bf16x8 one = ones8();

    const int row0 = seg0 * a.L, row1 = min(row0 + qm * a.L, a.N);
    RawTile<D, NT, kCb, true> rK, rV, rQ, rG;
    if constexpr (CAUSAL) {
        rK.load(kh, row0, a.N);
        rV.load(vh, row0, a.N);
    }
    rQ.load(qbase + bh0 * a.N * D, row0, a.N);
    rG.load(gbase + bh0 * a.N * D, row0, a.N);
    for (int seg = seg0; seg < seg0 + qm && seg * a.L < row1; ++seg) {
        const int s1 = min(seg * a.L + a.L, row1);
        for (int c0 = seg * a.L; c0 < s1; c0 += kCb) {
            __syncthreads();
            if constexpr (CAUSAL) {
                rK.template store_feat<PHI, false, TF, false>(sK, c0, a.N, nullptr, nullptr);
                rV.template store<TD>(sV);
                // the next chunk's K, V (unconditional: rows past the workgroup's
                // segments are loaded clamped and never used, and no register
                // copies are needed)
                rK.load(kh, c0 + kCb, a.N);
                rV.load(vh, c0 + kCb, a.N);
            }
            // the first head's rows are staged here, in straight-line code (in the
            // head loop, the wait for them would also wait for the K, V loads
            // just issued: the loop header merges the later heads' path)
            rQ.template store_feat<PHI, false, TF, true>(sQ, c0, a.N, sz, sQZ);
            rG.template store<TD>(sG);
            for (int rep = 0; rep < a.nrep; ++rep) {
                const size_t bh = bh0 + rep;
                if (rep > 0) {
                    __syncthreads();
                    rQ.template store_feat<PHI, false, TF, true>(sQ, c0, a.N, sz, sQZ);
                    rG.template store<TD>(sG);
                }
                __syncthreads();
                {   // Q, G rows of the next head, or of the first head at the next chunk
                    const bool last = rep + 1 == a.nrep;
                    const size_t hn = bh0 + (last ? 0 : rep + 1);
                    const int cn = last ? c0 + kCb : c0;
                    rQ.load(qbase + hn * a.N * D, cn, a.N);
                    rG.load(gbase + hn * a.N * D, cn, a.N);
                }
                const bool ok = c0 + l32 < a.N;   // this lane's query row exists
                f32x16 U;
                if (state_wave) {
                    // U^T = S g (this feature block x the chunk's queries); the g
                    // operands all read before the products
                    U = zero16();
                    bf16x8 gq[NW][2];
#pragma unroll
                    for (int db = 0; db < NW; ++db)
#pragma unroll
                        for (int s = 0; s < 2; ++s) gq[db][s] = ld4x2<TD>(sG, l32, 32 * db + 16 * s + 4 * h);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int db = 0; db < NW; ++db)
#pragma unroll
                        for (int s = 0; s < 2; ++s) {
                            U = mfma(acc_op(X[db], s), gq[db][s], U);
                            // bidirectional: every term goes through the state, and with
                            // few keys dq is a small difference: S in two bf16 parts
                            if constexpr (!CAUSAL) U = mfma(acc_lo(X[db], s), gq[db][s], U);
                        }
                    float qu = 0.f, x4[4];
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        ld4f(sQ + TF::at(l32, 32 * w + 8 * q4 + 4 * h), x4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) qu += x4[e] * U[4 * q4 + e];
                    }
                    qu = sum_halves(qu);
                    if (h == 0) sQU[w][l32] = qu;
                } else if (w == NW) {
                    // causal: A^T (keys x queries), causal mask, rounded to bf16
                    // (the forward's A), the tile for the state waves; the denominators
                    float dA = 0.f;
                    if constexpr (CAUSAL) {
                        f32x16 At = mfma_chain<F / 16, 4>([&](int s) { return ld8<TF>(sK, l32, 16 * s + 8 * h); },
                                                          [&](int s) { return ld8<TF>(sQ, l32, 16 * s + 8 * h); },
                                                          zero16());
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            At[r] = acc_row(r, h) <= l32 ? (float)(__bf16)At[r] : 0.f;
                            dA += At[r];
                        }
                        dA = sum_halves(dA);
                        put_acc(sAt, At);
                    }
                    if (h == 0) {
                        const float den = ok ? dA + sQZ[l32] + a.eps : 1.f;
                        sDen[l32] = den;
                        sInv[l32] = rcp(den);
                    }
                } else if (CAUSAL && w == NW + 1) {
                    // T^T = V G^T (keys x queries), unmasked: the state waves mask
                    const f32x16 Tt = mfma_chain<D / 16, 4>([&](int s) { return ld8<TD>(sV, l32, 16 * s + 8 * h); },
                                                            [&](int s) { return ld8<TD>(sG, l32, 16 * s + 8 * h); },
                                                            zero16());
                    put_acc(sTt, Tt);
                }
                __syncthreads();
                if (state_wave) {
                    // c = (sum_j A_ij T_ij + Phi(q_i).U_i) / den_i^2 (no A term: bidirectional)
                    f32x16 Tt;
                    float aT = 0.f;
                    if constexpr (CAUSAL) {
                        Tt = get_acc(sTt);
                        const f32x16 At = get_acc(sAt);
#pragma unroll
                        for (int r = 0; r < 16; ++r) aT += At[r] * Tt[r];
                        aT = sum_halves(aT);
                    }
                    float gsum = aT;
#pragma unroll
                    for (int ww = 0; ww < NW; ++ww) gsum += sQU[ww][l32];
                    const float inv = sInv[l32];
                    const float c = ok ? gsum * inv * inv : 0.f;
                    f32x16 Qd = zero16();
                    if constexpr (CAUSAL) {
                        if (w == 0 && h == 0 && ok) {   // for the dk/dv pass
                            a.ws_den[bh * a.N + c0 + l32] = sDen[l32];
                            a.ws_c[bh * a.N + c0 + l32] = c;
                        }
                        // P^T = T^T / den - c (masked), then dPhi(q)^T = Phi(K)^T P^T + U^T / den - z c
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            Tt[r] = acc_row(r, h) <= l32 ? Tt[r] * inv - c : 0.f;
#pragma unroll
                        for (int s = 0; s < 2; ++s) {
                            const int k0 = 16 * s + 4 * h;
                            const bf16x8 ka = tr8(tr_addr<TF>(sK, k0, 32 * w), tr_addr<TF>(sK, k0 + 8, 32 * w));
                            Qd = mfma(ka, acc_op(Tt, s), Qd);
                        }
                    }
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int f0 = 32 * w + 8 * q4 + 4 * h;
                        float qf[4];
                        ld4f(sQ + TF::at(l32, f0), qf);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            Qd[4 * q4 + e] = phi_d_feat<PHI>(qf[e]) *
                                             (Qd[4 * q4 + e] + U[4 * q4 + e] * inv - sz[f0 + e] * c);
                    }
                    const int row = c0 + l32;
                    if (row < a.N) {
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const float o[4] = {Qd[4 * q4], Qd[4 * q4 + 1], Qd[4 * q4 + 2], Qd[4 * q4 + 3]};
                            st4bf(dqbase + bh * a.N * D + (size_t)row * D + 32 * w + 8 * q4 + 4 * h, o);
                        }
                    }
                }
                if (!state_wave) {
                    // c_i for this lane's query, as the state waves form it (same
                    // bits), then through this wave's LDS row into operand order:
                    // lane (n, h) needs c of rows 16s + 8h + 0..7
                    float aT = 0.f;
                    if constexpr (CAUSAL) {
                        const f32x16 At = get_acc(sAt), Tt = get_acc(sTt);
#pragma unroll
                        for (int r = 0; r < 16; ++r) aT += At[r] * Tt[r];
                        aT = sum_halves(aT);
                    }
                    float gsum = aT;
#pragma unroll
                    for (int ww = 0; ww < NW; ++ww) gsum += sQU[ww][l32];
                    const float iq = sInv[l32];
                    if (h == 0) sCw[wr][l32] = ok ? gsum * iq * iq : 0.f;
                    // R (feature block wr x every value block) += (Phi(Q) / den)^T G,
                    // r (feature block wr) += Phi(Q)^T c in fp32 from the same Phi(Q)
                    // operand: lane (n, h) holds feature 32 wr + n of rows
                    // 16s + 8h .. +7, so the two halves together cover the chunk
#pragma unroll
                    for (int s = 0; s < kCb / 16; ++s) {
                        const int k0 = 16 * s + 8 * h;
                        bf16x8 qa = tr8(tr_addr<TF>(sQ, k0, 32 * wr), tr_addr<TF>(sQ, k0 + 4, 32 * wr));
                        {
                            const float4 c0v = *reinterpret_cast<const float4 *>(&sCw[wr][k0]);
                            const float4 c1v = *reinterpret_cast<const float4 *>(&sCw[wr][k0 + 4]);
                            const float cv[8] = {c0v.x, c0v.y, c0v.z, c0v.w, c1v.x, c1v.y, c1v.z, c1v.w};
#pragma unroll
                            for (int e = 0; e < 8; ++e) racc += cv[e] * (float)qa[e];
                        }
                        const float4 i0 = *reinterpret_cast<const float4 *>(sInv + k0);
                        const float4 i1 = *reinterpret_cast<const float4 *>(sInv + k0 + 4);
                        const float sc[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
                        bf16x8 qlo;   // bidirectional: Phi(q) / den in two bf16 parts (R v - r is
                                      // a small difference when few queries see a key)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float x = (float)qa[e] * sc[e];
                            qa[e] = (__bf16)x;
                            qlo[e] = (__bf16)(x - (float)qa[e]);
                        }
#pragma unroll
                        for (int db = 0; db < NW; ++db) {
                            const bf16x8 gb = tr8(tr_addr<TD>(sG, k0, 32 * db), tr_addr<TD>(sG, k0 + 4, 32 * db));
                            X[db] = mfma(qa, gb, X[db]);
                            if constexpr (!CAUSAL) X[db] = mfma(qlo, gb, X[db]);
                        }
                    }
                }
            }
            if (CAUSAL && state_wave) {
                // carry (S^T, z) past this chunk: z gets the chunk's sum of its
                // block (every column of Zc holds it)
                f32x16 Zc = zero16();
#pragma unroll
                for (int s = 0; s < kCb / 16; ++s) {
                    const int k0 = 16 * s + 8 * h;
                    const bf16x8 kb = tr8(tr_addr<TF>(sK, k0, 32 * w), tr_addr<TF>(sK, k0 + 4, 32 * w));
                    Zc = mfma(kb, one, Zc);
#pragma unroll
                    for (int db = 0; db < NW; ++db) {
                        const bf16x8 va = tr8(tr_addr<TD>(sV, k0, 32 * db), tr_addr<TD>(sV, k0 + 4, 32 * db));
                        X[db] = mfma(va, kb, X[db]);
                    }
                }
                // every staging of this chunk has read sz (each preceded a barrier
                // this wave has passed), and only this wave reads block w in its
                // dq epilogue, so it can take the new z now
                if (l32 == 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) sz[32 * w + acc_row(r, h)] += Zc[r];
                }
            }
        }
        if (!state_wave) {
            // this segment's (R, r), summed over the group's query heads, and a
            // fresh sum for the next one
            float *Ro = a.ws_Rp + ((size_t)bg * a.nseg + seg) * SD;
#pragma unroll
            for (int db = 0; db < NW; ++db) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    Ro[(size_t)(32 * wr + acc_row(r, h)) * D + 32 * db + l32] = X[db][r];
                X[db] = zero16();
            }
            const float rt = sum_halves(racc);
            if (h == 0) Ro[(size_t)F * D + 32 * wr + l32] = rt;
            racc = 0.f;
        }
    }
}

// Segments per dq workgroup (segments_by_rounds), each build (one segment,
// several) at its own occupancy.
template <int D, int PHI, bool CAUSAL>
int q_segments_per_wg(const Args &a, unsigned n_units) {
    // workgroups per round of the two builds (0: not yet asked).  Calls from
    // several host threads may each ask; they store the same values.
    static std::atomic<int> cached1{0}, cachedm{0};
    int slots1 = cached1.load(std::memory_order_relaxed), slotsm = cachedm.load(std::memory_order_relaxed);
    if (slots1 == 0 || slotsm == 0) {
        slots1 = device_slots(k_bwd_q_mfma<D, PHI, CAUSAL, false>, 4 * D);
        slotsm = device_slots(k_bwd_q_mfma<D, PHI, CAUSAL, true>, 4 * D);
        if (slots1 <= 0 || slotsm <= 0) return 1;
        cached1.store(slots1, std::memory_order_relaxed);
        cachedm.store(slotsm, std::memory_order_relaxed);
    }
    return segments_by_rounds(a.nseg, n_units, slots1, slotsm);
}

// ---------------------------------------------------------------------------
// k_bwd_kv_mfma: backward over the 32-row chunks of one (batch, KV head) and
// qm consecutive segments, from the exclusive suffix (R, r) of the last one.
// Wave w holds R^T (every value block x feature block w) and produces dk for
// feature block w and dv for value block w.  Per head, wave 0 forms the
// masked A tile and wave 1 the P tile as bf16 operands for every wave
// (through LDS), while the waves form the chunk's state terms.
// ---------------------------------------------------------------------------
template <int D, int PHI, bool CAUSAL>
__global__ __launch_bounds__(D * 2) __attribute__((amdgpu_waves_per_eu(2)))
void k_bwd_kv_mfma(Args a, int qm) {
    constexpr int F = D, NW = D / 32, NT = 2 * D;
    using TF = PadI<F>;
    using TD = PadI<D>;
    __shared__ __attribute__((aligned(16))) u16 sK[kCb * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sV[kCb * TD::ld];
    __shared__ __attribute__((aligned(16))) u16 sQ[kCb * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sG[kCb * TD::ld];
    __shared__ __attribute__((aligned(16))) u16 sR[F * TD::ld];
    __shared__ __attribute__((aligned(16))) u16 sGr[kCb * TD::ld];   // raw g rows (for P)
    __shared__ __attribute__((aligned(16))) float sCc[kCb], sIq[kCb];   // c_i, 1 / den_i
    __shared__ __attribute__((aligned(16))) float sr[F];
    __shared__ bf16x8 sAop[2][64];   // A operands of one head, per lane
    // P operands of one head, per lane: in the raw g rows, which only wave 1
    // reads (for P, before it writes them) until the next head is staged
    bf16x8 (*sPop)[64] = reinterpret_cast<bf16x8 (*)[64]>(sGr);
    static_assert(sizeof(bf16x8) * 2 * 64 <= sizeof(u16) * kCb * TD::ld, "P operands fit the g rows");

    // this workgroup walks the qm consecutive segments seg0 .. seg1 (last to
    // first; the R carry runs through their boundaries) from the suffix of
    // the last one
    const int nq = (a.nseg + qm - 1) / qm;
    const int seg0 = (blockIdx.x % nq) * qm, bg = blockIdx.x / nq;
    const int seg1 = min(seg0 + qm, a.nseg) - 1;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int t = threadIdx.x, l = t & 63, h = l >> 5, l32 = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index, uniform
    const size_t SD = (size_t)F * D + F;
    const u16 *kh = static_cast<const u16 *>(a.k) + (size_t)bg * a.N * D;
    const u16 *vh = static_cast<const u16 *>(a.v) + (size_t)bg * a.N * D;
    u16 *dkh = static_cast<u16 *>(a.dk) + (size_t)bg * a.N * D;
    u16 *dvh = static_cast<u16 *>(a.dv) + (size_t)bg * a.N * D;
    const size_t bh0 = (size_t)b * a.H + (size_t)g * a.nrep;
    const u16 *qbase = static_cast<const u16 *>(a.q);
    const u16 *gbase = static_cast<const u16 *>(a.g);

    // the exclusive suffix of (R, r) of segment seg1 (causal) or the sequence total
    const float *Rp = a.ws_Rs + ((size_t)bg * (a.nseg + 1) + (CAUSAL ? seg1 : a.nseg)) * SD;
    f32x16 Rt[NW];
#pragma unroll
    for (int db = 0; db < NW; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) Rt[db][r] = Rp[(size_t)(32 * w + l32) * D + 32 * db + acc_row(r, h)];
    // r (the running suffix): both lanes (n, h) of wave w hold r[32w + n];
    // each chunk publishes the wave's block to sr for the state term
    float racc = Rp[(size_t)F * D + 32 * w + l32];

    const int row0 = seg0 * a.L, row1 = min((seg1 + 1) * a.L, a.N);
    const int nch = (row1 - row0 + kCb - 1) / kCb;
    RawTile<D, NT, kCb> rK, rV, rQ, rG;
    constexpr int NV = RawTile<D, NT, kCb>::NV, V8 = D / 8;
    // prefetched: den of this thread's G rows, c and den of query t % 32
    float pden[NV], pc, pdq;
    auto load_dc = [&](size_t hh, int cc) {
#pragma unroll
        for (int k = 0; k < NV; ++k)
            pden[k] = a.ws_den[hh * a.N + min(cc + (t + k * NT) / V8, a.N - 1)];
        pc = a.ws_c[hh * a.N + min(cc + (t & (kCb - 1)), a.N - 1)];
        pdq = a.ws_den[hh * a.N + min(cc + (t & (kCb - 1)), a.N - 1)];
    };
    {
        const int c0 = row0 + (nch - 1) * kCb;
        rK.load(kh, c0, a.N);
        rV.load(vh, c0, a.N);
        if constexpr (CAUSAL) {   // the in-chunk terms need the queries' rows
            rQ.load(qbase + bh0 * a.N * D, c0, a.N);
            rG.load(gbase + bh0 * a.N * D, c0, a.N);
            load_dc(bh0, c0);
        }
    }
    // this head's query rows into LDS: Phi(Q), gn = g / den, raw g, c, 1 / den
    // (rows past N: zeros), then the next head's (or the next chunk's first
    // head's) loads
    auto stage_head = [&](int c0, int rep, int cn) {
        rQ.template store_feat<PHI, false, TF, false>(sQ, c0, a.N, nullptr, nullptr);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = t + k * NT, i = idx / V8, c8 = (idx % V8) * 8, row = c0 + i;
            const float inv = row < a.N ? rcp(pden[k]) : 0.f;
            const uint4 u = rG.v[k];
            uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                wds[e] = pk2(__uint_as_float(wds[e] << 16) * inv, __uint_as_float(wds[e] & 0xffff0000u) * inv);
            *reinterpret_cast<uint4 *>(sG + TD::at(i, c8)) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
        }
        rG.template store<TD>(sGr);
        if (t < kCb) {
            sCc[t] = c0 + t < a.N ? pc : 0.f;
            sIq[t] = c0 + t < a.N ? rcp(pdq) : 0.f;
        }
        const bool last = rep + 1 == a.nrep;
        const size_t hn = bh0 + (last ? 0 : rep + 1);
        const int cq = last ? cn : c0;
        rQ.load(qbase + hn * a.N * D, cq, a.N);
        rG.load(gbase + hn * a.N * D, cq, a.N);
        load_dc(hn, cq);
    };
    // A = Phi(Q) Phi(K)^T (wave 0) and P = (G V^T) / den - c (wave 1)
    // (queries x keys), i >= j, masked and turned into bf16 operands, for
    // every wave through LDS (each lane's operands in its own slot: every
    // wave's operands of a product sit at the same lanes).  P comes from the
    // raw g rows (exact operands) scaled in fp32: it can be a small
    // difference (one key: P_00 = eps / den_0 * g.v / den_0), which products
    // with bf16-rounded gn would not resolve.
    auto form_ap = [&]() {
        if (w == 0) {
            f32x16 A = mfma_chain<F / 16, 2>([&](int s) { return ld8<TF>(sQ, l32, 16 * s + 8 * h); },
                                             [&](int s) { return ld8<TF>(sK, l32, 16 * s + 8 * h); }, zero16());
#pragma unroll
            for (int r = 0; r < 16; ++r) A[r] = acc_row(r, h) >= l32 ? A[r] : 0.f;
            sAop[0][l] = acc_op(A, 0);
            sAop[1][l] = acc_op(A, 1);
        } else if (w == 1) {
            f32x16 P = mfma_chain<D / 16, 2>([&](int s) { return ld8<TD>(sGr, l32, 16 * s + 8 * h); },
                                             [&](int s) { return ld8<TD>(sV, l32, 16 * s + 8 * h); }, zero16());
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 cv = *reinterpret_cast<const float4 *>(sCc + 8 * q4 + 4 * h);
                const float4 iv = *reinterpret_cast<const float4 *>(sIq + 8 * q4 + 4 * h);
                const float cr[4] = {cv.x, cv.y, cv.z, cv.w}, ir[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * q4 + e;
                    P[r] = acc_row(r, h) >= l32 ? P[r] * ir[e] - cr[e] : 0.f;
                }
            }
            sPop[0][l] = acc_op(P, 0);
            sPop[1][l] = acc_op(P, 1);
        }
    };
    // The dk, dv rows of a chunk are staged in the query tiles sQ, sG and
    // stored as whole rows after the next barrier: by each thread, ahead of
    // its own staging of the next head's rows, which writes exactly the pieces
    // it reads (the same thread-to-piece map), so no barrier separates them.
    // (From the registers, 8-byte pieces scattered over 32 rows per
    // instruction, the stores cost far more.)
    int pend_c0 = -1;
    for (int ci = nch - 1; ci >= 0; --ci) {
        const int c0 = row0 + ci * kCb;
        const int cn = ci > 0 ? c0 - kCb : c0;   // next chunk (none: reload this one)
        __syncthreads();   // every read of the previous chunk's tiles is done
        rK.template store_feat<PHI, false, TF, false>(sK, c0, a.N, nullptr, nullptr);
        rV.template store<TD>(sV);
        rK.load(kh, cn, a.N);
        rV.load(vh, cn, a.N);
        // R (bf16, [feature][value]) for the state terms (bidirectional: the
        // total, staged once), r for the state term
        if (CAUSAL || ci == nch - 1) {
#pragma unroll
            for (int db = 0; db < NW; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    float x[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = Rt[db][4 * q4 + e];
                    st4bf(sR + TD::at(32 * w + l32, 32 * db + 8 * q4 + 4 * h), x);
                }
            if (h == 0) sr[32 * w + l32] = racc;
        }
        if (pend_c0 >= 0) {   // the previous chunk's rows (fences: one tile's registers at a time)
            __builtin_amdgcn_sched_barrier(0);
            store_rows<D, NT, TF, true>(dkh, sQ, pend_c0, a.N);
            __builtin_amdgcn_sched_barrier(0);
            store_rows<D, NT, TD, true>(dvh, sG, pend_c0, a.N);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (CAUSAL) stage_head(c0, 0, cn);
        __syncthreads();
        // causal: the first head's A and P tiles (waves 0 and 1), ahead of the
        // state terms that every wave computes meanwhile
        if constexpr (CAUSAL) form_ap();
        // state terms: dPhi(k)^T = R V^T - r, dv^T = R^T Phi(K)^T
        f32x16 dK = zero16(), dV = zero16();
#pragma unroll
        for (int db = 0; db < NW; ++db)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8 vq = ld4x2<TD>(sV, l32, 32 * db + 16 * s + 4 * h);
                if constexpr (CAUSAL) {
                    dK = mfma(ld4x2<TD>(sR, 32 * w + l32, 32 * db + 16 * s + 4 * h), vq, dK);   // R, as staged
                } else {
                    // R (total) in two bf16 parts: R v - r is a small difference
                    // when few queries see a key
                    dK = mfma(acc_op(Rt[db], s), vq, dK);
                    dK = mfma(acc_lo(Rt[db], s), vq, dK);
                }
            }
#pragma unroll 4
        for (int s = 0; s < F / 16; ++s) {
            const int k0 = 16 * s + 8 * h;
            dV = mfma(tr8(tr_addr<TD>(sR, k0, 32 * w), tr_addr<TD>(sR, k0 + 4, 32 * w)),
                      ld8<TF>(sK, l32, 16 * s + 8 * h), dV);
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {   // rows 8 q4 + 4h + 0..3 are consecutive
            const float4 r4 = *reinterpret_cast<const float4 *>(sr + 32 * w + 8 * q4 + 4 * h);
            dK[4 * q4] -= r4.x;
            dK[4 * q4 + 1] -= r4.y;
            dK[4 * q4 + 2] -= r4.z;
            dK[4 * q4 + 3] -= r4.w;
        }

        // causal: the chunk's own queries (in-chunk terms) and the R update;
        // the first head's rows were staged with the chunk
        for (int rep = 0; rep < (CAUSAL ? a.nrep : 0); ++rep) {
            if (rep > 0) {
                __syncthreads();   // the previous head's LDS reads are done
                stage_head(c0, rep, cn);
                __syncthreads();
                form_ap();
            }
            __syncthreads();   // this head's A, P operands are in LDS
            const bf16x8 Aop[2] = {sAop[0][l], sAop[1][l]}, Pop[2] = {sPop[0][l], sPop[1][l]};
            // in-chunk terms: dPhi(k)^T += Phi(Q)^T P, dv^T += gn^T A
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int k0 = 16 * s + 4 * h;
                dK = mfma(tr8(tr_addr<TF>(sQ, k0, 32 * w), tr_addr<TF>(sQ, k0 + 8, 32 * w)), Pop[s], dK);
                dV = mfma(tr8(tr_addr<TD>(sG, k0, 32 * w), tr_addr<TD>(sG, k0 + 8, 32 * w)), Aop[s], dV);
            }
            // R^T += gn^T Phi(Q) for the rows of this chunk; r += Phi(Q)^T c
            // from the same Phi(Q) operand: lane (n, h) holds feature 32w + n of
            // rows 16s + 8h .. +7, so the two halves together cover the chunk
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < kCb / 16; ++s) {
                const int k0 = 16 * s + 8 * h;
                const bf16x8 qb = tr8(tr_addr<TF>(sQ, k0, 32 * w), tr_addr<TF>(sQ, k0 + 4, 32 * w));
#pragma unroll
                for (int db = 0; db < NW; ++db) {
                    const bf16x8 ga = tr8(tr_addr<TD>(sG, k0, 32 * db), tr_addr<TD>(sG, k0 + 4, 32 * db));
                    Rt[db] = mfma(ga, qb, Rt[db]);
                }
                const float4 c0v = *reinterpret_cast<const float4 *>(sCc + k0);
                const float4 c1v = *reinterpret_cast<const float4 *>(sCc + k0 + 4);
                const float cv[8] = {c0v.x, c0v.y, c0v.z, c0v.w, c1v.x, c1v.y, c1v.z, c1v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) acc += cv[e] * (float)qb[e];
            }
            racc += sum_halves(acc);
        }
        // dk = phi'(k) dPhi(k), dv; lane holds key l32 and columns 32w + 8q + 4h + 0..3,
        // stored straight from the registers (the next chunk's tiles take the LDS)
        if constexpr (CAUSAL) __syncthreads();   // every read of the last head's sQ, sG is done
        {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int f0 = 32 * w + 8 * q4 + 4 * h;
                float kf[4], ok4[4], ov4[4];
                ld4f(sK + TF::at(l32, f0), kf);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ok4[e] = dK[4 * q4 + e] * phi_d_feat<PHI>(kf[e]);
                    ov4[e] = dV[4 * q4 + e];
                }
                st4bf(sQ + TF::at(l32, f0), ok4);
                st4bf(sG + TD::at(l32, f0), ov4);
            }
        }
        pend_c0 = c0;
    }
    if (pend_c0 >= 0) {
        __syncthreads();
        store_rows<D, NT, TF>(dkh, sQ, pend_c0, a.N);
        store_rows<D, NT, TD>(dvh, sG, pend_c0, a.N);
    }
}

template <int D, int PHI, bool CAUSAL>
hipError_t run(const Args &a, hipStream_t s) {
    constexpr int F = D;
    const unsigned n_units = (unsigned)(a.B * a.Hkv);
    const size_t SD = (size_t)F * D + F;
    hipError_t e = a.state_ready ? hipSuccess : mfma_state_run(a, PHI, CAUSAL, s);
    if (e != hipSuccess) return e;
    {
        bool launched = false;
        // segments per workgroup: the one-segment kernel is a separate build
        const int qm = q_segments_per_wg<D, PHI, CAUSAL>(a, n_units);
        const unsigned nq = (unsigned)((a.nseg + qm - 1) / qm);
        TimedLaunch tl(CAUSAL ? "k_bwd_q_mfma" : "k_bwd_q_bidir_mfma", s);
        if (qm > 1) {
            hipLaunchKernelGGL((k_bwd_q_mfma<D, PHI, CAUSAL, true>), dim3(n_units * nq), dim3(4 * D), 0, s, a, qm);
            launched = true;
        }
        if (!launched)
            hipLaunchKernelGGL((k_bwd_q_mfma<D, PHI, CAUSAL, false>), dim3(n_units * nq), dim3(4 * D), 0, s, a, 1);
    }
    {
        TimedLaunch tl("k_scan_R", s);
        // per-segment records are already summed over the group's heads
        e = scan_suffix(a.ws_Rp, a.ws_Rs, a.nseg, SD, a.Hkv, a.Hkv, 1, n_units, CAUSAL, s);
        if (e != hipSuccess) return e;
    }
    {
        TimedLaunch tl(CAUSAL ? "k_bwd_kv_mfma" : "k_bwd_kv_bidir_mfma", s);
        // causal: one segment per workgroup (two workgroups per compute unit;
        // fewer, longer ones leave compute units idle)
        const int kqm = CAUSAL ? 1 : bidir_segments_per_wg(a.nseg, n_units);
        const unsigned nk = (unsigned)((a.nseg + kqm - 1) / kqm);
        hipLaunchKernelGGL((k_bwd_kv_mfma<D, PHI, CAUSAL>), dim3(n_units * nk), dim3(2 * D), 0, s, a, kqm);
    }
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t by_phi(const Args &a, int phi, hipStream_t s) {
    switch (phi) {
        case kElu1: return run<D, kElu1, CAUSAL>(a, s);
        case kRelu: return run<D, kRelu, CAUSAL>(a, s);
        default: return run<D, kIdentity, CAUSAL>(a, s);
    }
}

}  // namespace

int bidir_segments_per_wg(int nseg, unsigned n_units) {
    static std::atomic<int> cached{0};   // compute units (0: not yet asked)
    int cus = cached.load(std::memory_order_relaxed);
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return 1;
        cached.store(cus, std::memory_order_relaxed);
    }
    // the fewest workgroups per unit that still give every compute unit one,
    // then segments spread evenly over them
    const long long groups = std::min<long long>(nseg, ((long long)cus + n_units - 1) / n_units);
    return (int)((nseg + groups - 1) / groups);
}

bool mfma_bwd_serves(int bf16, int causal, int D, int has_cos) {
    (void)causal;
    (void)has_cos;
    return bf16 && (D == 64 || D == 128);
}

hipError_t mfma_bwd_run(const Args &a, int phi, int causal, hipStream_t s) {
    if (a.F == 2 * a.D) return mfma_bwd_cos_run(a, phi, causal, s);
    if (a.D == 64) return causal ? by_phi<64, true>(a, phi, s) : by_phi<64, false>(a, phi, s);
    return causal ? by_phi<128, true>(a, phi, s) : by_phi<128, false>(a, phi, s);
}

}  // namespace la
