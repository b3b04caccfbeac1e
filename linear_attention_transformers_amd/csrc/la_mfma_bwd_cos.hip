// la_mfma_bwd_cos.hip -- bf16 backward with the cos/sin features (F = 2D)
// on the gfx950 matrix cores, causal and bidirectional.
//
// The derivative is the one of la_mfma_bwd.hip (SVD_linear_Attention,
// "Module neuralops.core.triton_kernels.linear_attn", function bwd; module
// docstring: cos/sin modulation) with Phi(x_t) = [cos_t phi(x_t),
// sin_t phi(x_t)] of width F = 2D.  The chain rule through the modulation
// gives, for d < D,
//   dq_d = phi'(q_d) (cos_i dPhi(q_i)_d + sin_i dPhi(q_i)_{D+d}),   likewise dk.
// There are twice as many feature blocks (F/32) as value blocks, so one wave
// per feature block holds its slice of the state (S^T in the dq kernel, R^T
// in the dk/dv kernel): a workgroup is F/32 waves, and the two halves of
// dPhi meet through LDS.  With every wave busy with its own state, the
// per-segment (R, r) sums get a pass of their own (k_bwd_r_cos_mfma) between
// the dq and the dk/dv kernels; it reads the den_i and c_i the dq kernel
// writes.  Causal: per chunk and head wave 0 forms the A tile (over the F
// features) and wave 1 the T (or P) tile for the workgroup.  Bidirectional
// (CAUSAL = false): every term goes through the total state; there are no
// in-chunk tiles or carries, and the products whose results can be small
// differences take two bf16 parts (S for U, gn and c in the R pass, R for
// R v in dk).
#include "la_common.h"
#include "la_kernels.h"
#include "la_mfma.h"
#include "la_timing.h"

namespace la {
namespace {

using namespace mf;

constexpr int kCc = 32;   // chunk length: one 32x32 tile of A per head

// ---------------------------------------------------------------------------
// k_bwd_q_cos_mfma: forward over the 32-row chunks of one (batch, KV head,
// segment) for the n_rep query heads.  Wave w (of F/32) holds S^T for
// feature block w (all value blocks) and z of that block; it forms U = S g
// for its block and dPhi(q) for its block, weighted by cos or sin and by
// phi'; the waves of the sin half pass their terms to those of the cos half,
// which add them and store dq after the next head's exchange barrier.  Wave 0 forms A^T (over all F features) and wave 1 T^T for the
// whole workgroup; they reach every wave through LDS with the Phi(q).U
// partials.  Writes den_i and c_i.
// ---------------------------------------------------------------------------
template <int D, int PHI, bool CAUSAL>
__global__ __launch_bounds__(D * 4) __attribute__((amdgpu_waves_per_eu(2)))
void k_bwd_q_cos_mfma(Args a) {
    constexpr int F = 2 * D, NW = D / 32, FW = F / 32, NT = 64 * FW;
    using TF = PadI<F>;
    using TD = PadI<D>;
    __shared__ __attribute__((aligned(16))) u16 sK[kCc * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sV[kCc * TD::ld];
    __shared__ __attribute__((aligned(16))) u16 sQ[kCc * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sQr[kCc * TD::ld];   // phi(q) rows (unweighted), for phi'
    __shared__ __attribute__((aligned(16))) u16 sG[kCc * TD::ld];
    __shared__ __attribute__((aligned(16))) float sz[F];
    __shared__ __attribute__((aligned(16))) float sX[2][NW][64 * 16];   // sin halves' dq terms, by head parity
    __shared__ __attribute__((aligned(16))) float sAt[64 * 16], sTt[64 * 16];   // A^T, T^T tiles
    __shared__ float sQZ[kCc], sQU[FW][kCc];

    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int t = threadIdx.x, l = t & 63, w = t >> 6, h = l >> 5, l32 = l & 31;
    const size_t SD = (size_t)F * D + F;
    const u16 *kh = static_cast<const u16 *>(a.k) + (size_t)bg * a.N * D;
    const u16 *vh = static_cast<const u16 *>(a.v) + (size_t)bg * a.N * D;
    const size_t bh0 = (size_t)b * a.H + (size_t)g * a.nrep;
    const u16 *qbase = static_cast<const u16 *>(a.q);
    const u16 *gbase = static_cast<const u16 *>(a.g);
    u16 *dqbase = static_cast<u16 *>(a.dq);

    // exclusive prefix state of the segment (causal) or the sequence total:
    // S^T tiles (value block db x feature block w) and the z tile of block w
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + (CAUSAL ? seg : a.nseg)) * SD;
    f32x16 X[NW], Z;
#pragma unroll
    for (int db = 0; db < NW; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) X[db][r] = Sp[(size_t)(32 * w + l32) * D + 32 * db + acc_row(r, h)];
#pragma unroll
    for (int r = 0; r < 16; ++r) Z[r] = Sp[(size_t)F * D + 32 * w + acc_row(r, h)];
    for (int e = t; e < F; e += NT) sz[e] = Sp[(size_t)F * D + e];
    const bf16x8 one = ones8();

    // The cos-half wave of dims 32w .. 32w+31 stores dq from its own term and
    // the sin-half wave's (through sX) after the next head's exchange barrier,
    // so no barrier of its own is needed: its pending term, rows and buffer
    f32x16 Qp;
    bool pend = false;
    int pbuf = 0, prow = 0;
    size_t pbh = 0;
    auto store_pending = [&]() {
        if (w < NW) {
            const f32x16 Qs = get_acc(sX[pbuf][w]);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d0 = 32 * w + 8 * q4 + 4 * h;
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = Qp[4 * q4 + e] + Qs[4 * q4 + e];
                if (prow < a.N) st4bf(dqbase + pbh * a.N * D + (size_t)prow * D + d0, o);
            }
        }
    };
    int step = 0;   // (chunk, head) steps so far: sX buffer parity

    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    RawTile<D, NT, kCc, true> rK, rV, rQ, rG;
    if constexpr (CAUSAL) {   // the in-chunk terms and the carry need the keys
        rK.load(kh, row0, a.N);
        rV.load(vh, row0, a.N);
    }
    rQ.load(qbase + bh0 * a.N * D, row0, a.N);
    rG.load(gbase + bh0 * a.N * D, row0, a.N);
    for (int c0 = row0; c0 < row1; c0 += kCc) {
        __syncthreads();
        if constexpr (CAUSAL) {
            rK.load_w(a.cw, a.sw, c0, a.N);   // read here: read with the rows, a chunk ahead, this kernel ran 2% slower
            rK.template store_feat<PHI, true, TF, false>(sK, c0, a.N, nullptr, nullptr);
            rV.template store<TD>(sV);
            rK.load(kh, c0 + kCc, a.N);   // next chunk (past the segment: unused)
            rV.load(vh, c0 + kCc, a.N);
        }
        const int ti = min(c0 + l32, a.N - 1);
        const float mq = w < NW ? a.cw[ti] : a.sw[ti];   // this lane's query weight for block w
        // the first head's rows are staged here, in straight-line code (in the
        // head loop, the wait for them would also wait for the K, V loads
        // just issued: the loop header merges the later heads' path)
        rQ.load_w(a.cw, a.sw, c0, a.N);   // the chunk's positions, for every head
        rQ.template store_feat<PHI, true, TF, true, TD>(sQ, c0, a.N, sz, sQZ, sQr);
        rG.template store<TD>(sG);
        for (int rep = 0; rep < a.nrep; ++rep) {
            const size_t bh = bh0 + rep;
            if (rep > 0) {
                __syncthreads();
                rQ.template store_feat<PHI, true, TF, true, TD>(sQ, c0, a.N, sz, sQZ, sQr);
                rG.template store<TD>(sG);
            }
            __syncthreads();
            {   // Q, G rows of the next head, or of the first head at the next chunk
                const bool last = rep + 1 == a.nrep;
                const size_t hn = bh0 + (last ? 0 : rep + 1);
                const int cn = last ? c0 + kCc : c0;
                rQ.load(qbase + hn * a.N * D, cn, a.N);
                rG.load(gbase + hn * a.N * D, cn, a.N);
            }
            const bool ok = c0 + l32 < a.N;   // this lane's query row exists

            // causal: A^T over the F features (the cos/sin weighting included)
            // on wave 0, T^T on wave 1, for every wave after the barrier below
            if (CAUSAL && w == 0) {
                const f32x16 At = mfma_chain<F / 16, 2>([&](int s) { return ld8<TF>(sK, l32, 16 * s + 8 * h); },
                                                        [&](int s) { return ld8<TF>(sQ, l32, 16 * s + 8 * h); },
                                                        zero16());
                put_acc(sAt, At);
            } else if (CAUSAL && w == 1) {
                const f32x16 Tt = mfma_chain<D / 16, 2>([&](int s) { return ld8<TD>(sV, l32, 16 * s + 8 * h); },
                                                        [&](int s) { return ld8<TD>(sG, l32, 16 * s + 8 * h); },
                                                        zero16());
                put_acc(sTt, Tt);
            }
            // U^T = S g (feature block w x the chunk's queries), Phi(q).U over the
            // block; bidirectional: every term goes through the state, and dq can
            // be a small difference, so S goes in as two bf16 parts
            f32x16 U = zero16();
#pragma unroll
            for (int db = 0; db < NW; ++db)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const bf16x8 gq = ld4x2<TD>(sG, l32, 32 * db + 16 * s + 4 * h);
                    U = mfma(acc_op(X[db], s), gq, U);
                    if constexpr (!CAUSAL) U = mfma(acc_lo(X[db], s), gq, U);
                }
            float qu = 0.f;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float x4[4];
                ld4f(sQ + TF::at(l32, 32 * w + 8 * q4 + 4 * h), x4);
#pragma unroll
                for (int e = 0; e < 4; ++e) qu += x4[e] * U[4 * q4 + e];
            }
            qu = sum_halves(qu);
            if (h == 0) sQU[w][l32] = qu;
            __syncthreads();
            if (pend) store_pending();   // the previous head's dq rows

            f32x16 Tt;
            float dA = 0.f, aT = 0.f;
            if constexpr (CAUSAL) {
                Tt = get_acc(sTt);
                const f32x16 At = get_acc(sAt);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = acc_row(r, h) <= l32 ? (float)(__bf16)At[r] : 0.f;   // the forward's A
                    dA += x;
                    aT += x * Tt[r];
                }
                dA = sum_halves(dA);
                aT = sum_halves(aT);
            }
            const float den = ok ? dA + sQZ[l32] + a.eps : 1.f;
            float gsum = aT;
#pragma unroll
            for (int ww = 0; ww < FW; ++ww) gsum += sQU[ww][l32];
            const float inv = rcp(den);
            const float c = ok ? gsum * inv * inv : 0.f;
            if (w == 0 && h == 0 && ok) {   // for the R pass and the dk/dv kernel
                a.ws_den[bh * a.N + c0 + l32] = den;
                a.ws_c[bh * a.N + c0 + l32] = c;
            }
            // P^T = T^T / den - c (masked); dPhi(q)^T = Phi(K)^T P^T + U^T / den - z c
            // (no in-chunk term: bidirectional)
            f32x16 Qd = zero16();
            if constexpr (CAUSAL) {
#pragma unroll
                for (int r = 0; r < 16; ++r) Tt[r] = acc_row(r, h) <= l32 ? Tt[r] * inv - c : 0.f;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int k0 = 16 * s + 4 * h;
                    const bf16x8 ka = tr8(tr_addr<TF>(sK, k0, 32 * w), tr_addr<TF>(sK, k0 + 8, 32 * w));
                    Qd = mfma(ka, acc_op(Tt, s), Qd);
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                Qd[r] = mq * (Qd[r] + U[r] * inv - sz[32 * w + acc_row(r, h)] * c);
            // each half's term of dq = phi'(q) (cos dPhi(q)_cos + sin dPhi(q)_sin)
            // for dims 32 (w mod D/32) ..: the sin half's goes through sX
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float qr[4];
                ld4f(sQr + TD::at(l32, 32 * (w % NW) + 8 * q4 + 4 * h), qr);
#pragma unroll
                for (int e = 0; e < 4; ++e) Qd[4 * q4 + e] *= phi_d_feat<PHI>(qr[e]);
            }
            const int buf = step & 1;
            if (w >= NW) put_acc(sX[buf][w - NW], Qd);
            Qp = Qd;
            pend = true;
            pbuf = buf;
            prow = c0 + l32;
            pbh = bh;
            ++step;
        }
        if constexpr (CAUSAL) {
            // carry (S^T, z) past this chunk
#pragma unroll
            for (int s = 0; s < kCc / 16; ++s) {
                const int k0 = 16 * s + 8 * h;
                const bf16x8 kb = tr8(tr_addr<TF>(sK, k0, 32 * w), tr_addr<TF>(sK, k0 + 4, 32 * w));
                Z = mfma(kb, one, Z);
#pragma unroll
                for (int db = 0; db < NW; ++db) {
                    const bf16x8 va = tr8(tr_addr<TD>(sV, k0, 32 * db), tr_addr<TD>(sV, k0 + 4, 32 * db));
                    X[db] = mfma(va, kb, X[db]);
                }
            }
            // every staging of this chunk has read sz; only this wave reads block w
            if (l32 == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sz[32 * w + acc_row(r, h)] = Z[r];
            }
        }
    }
    __syncthreads();   // the last head's sin terms are in sX
    if (pend) store_pending();
}

// ---------------------------------------------------------------------------
// k_bwd_r_cos_mfma: per (batch, KV head, segment) the segment's sums over
// the n_rep query heads of R = sum_i Phi(q_i) gn_i^T (F x D) and
// r = sum_i c_i Phi(q_i), gn_i = g_i / den_i, written as fp32 to the
// workspace record of the segment.  Two sets of D/32 waves split the
// feature blocks: wave w owns value block w % (D/32) and the F/64 R tiles of
// feature half w / (D/32) in that block, and the r tile of feature block w
// (r = Phi(Q)^T c on the matrix cores with c rounded to bf16, every column
// of an r tile holding r).  The tiles are disjoint, so nothing crosses
// waves; split, a wave holds 64 accumulator registers per lane instead of
// 128 and two waves share a SIMD.  Bidirectional: dk = R v - r can be a
// small difference (every term goes through R), so gn and c go in as two
// bf16 parts each (hi, then the rounding remainder).
// ---------------------------------------------------------------------------
template <int D, int PHI, bool CAUSAL>
__global__ __launch_bounds__(D * 4) __attribute__((amdgpu_waves_per_eu(2))) void k_bwd_r_cos_mfma(Args a) {
    constexpr int F = 2 * D, NW = D / 32, FBW = F / 64, NT = 4 * D;
    using TF = PadI<F>;
    using TD = PadI<D>;
    __shared__ __attribute__((aligned(16))) u16 sQ[kCc * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sG[kCc * TD::ld];
    __shared__ __attribute__((aligned(16))) u16 sGl[CAUSAL ? 8 : kCc * TD::ld];   // gn remainders
    __shared__ __attribute__((aligned(16))) float sC[kCc];
    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int t = threadIdx.x, l = t & 63, h = l >> 5, l32 = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index, uniform
    const int vb = w % NW, fh = w / NW;                       // value block, feature half
    const size_t bh0 = (size_t)b * a.H + (size_t)g * a.nrep;
    const u16 *qbase = static_cast<const u16 *>(a.q);
    const u16 *gbase = static_cast<const u16 *>(a.g);
    f32x16 R[FBW], Zr = zero16();
#pragma unroll
    for (int i = 0; i < FBW; ++i) R[i] = zero16();

    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    constexpr int NV = RawTile<D, NT, kCc>::NV, V8 = D / 8;
    RawTile<D, NT, kCc> rQ, rG;
    float pden[NV], pc;   // den of this thread's G rows and c of row t % 32, prefetched
    auto load_dc = [&](size_t hh, int cc) {
#pragma unroll
        for (int k = 0; k < NV; ++k) pden[k] = a.ws_den[hh * a.N + min(cc + (t + k * NT) / V8, a.N - 1)];
        pc = a.ws_c[hh * a.N + min(cc + (t & (kCc - 1)), a.N - 1)];
    };
    rQ.load(qbase + bh0 * a.N * D, row0, a.N);
    rG.load(gbase + bh0 * a.N * D, row0, a.N);
    load_dc(bh0, row0);
    for (int c0 = row0; c0 < row1; c0 += kCc) {
        for (int rep = 0; rep < a.nrep; ++rep) {
            __syncthreads();   // the previous head's LDS reads are done
            rQ.load_w(a.cw, a.sw, c0, a.N);   // read here: read with the rows, a chunk ahead, this kernel ran 2% slower
            rQ.template store_feat<PHI, true, TF, false>(sQ, c0, a.N, nullptr, nullptr);
#pragma unroll
            for (int k = 0; k < NV; ++k) {   // gn = g / den (rows past N: zeros)
                const int idx = t + k * NT, i = idx / V8, c8 = (idx % V8) * 8;
                const float inv = c0 + i < a.N ? rcp(pden[k]) : 0.f;
                const uint4 u = rG.v[k];
                uint32_t wds[4] = {u.x, u.y, u.z, u.w};
                uint32_t lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = __uint_as_float(wds[e] << 16) * inv, x1 = __uint_as_float(wds[e] & 0xffff0000u) * inv;
                    wds[e] = pk2(x0, x1);
                    if constexpr (!CAUSAL)
                        lo[e] = pk2(x0 - __uint_as_float(wds[e] << 16), x1 - __uint_as_float(wds[e] & 0xffff0000u));
                }
                *reinterpret_cast<uint4 *>(sG + TD::at(i, c8)) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
                if constexpr (!CAUSAL)
                    *reinterpret_cast<uint4 *>(sGl + TD::at(i, c8)) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            }
            if (t < kCc) sC[t] = c0 + t < a.N ? pc : 0.f;
            __syncthreads();
            {   // the next head's rows, or the first head's at the next chunk
                const bool last = rep + 1 == a.nrep;
                const size_t hn = bh0 + (last ? 0 : rep + 1);
                const int cn = last ? c0 + kCc : c0;
                rQ.load(qbase + hn * a.N * D, cn, a.N);
                rG.load(gbase + hn * a.N * D, cn, a.N);
                load_dc(hn, cn);
            }
            // R[fb] += Phi(Q)^T gn, r += Phi(Q)^T c (natural k order: half h
            // holds rows 16s + 8h .. +7)
#pragma unroll
            for (int s = 0; s < kCc / 16; ++s) {
                const int k0 = 16 * s + 8 * h;
                const bf16x8 gb = tr8(tr_addr<TD>(sG, k0, 32 * vb), tr_addr<TD>(sG, k0 + 4, 32 * vb));
                const float4 c_lo = *reinterpret_cast<const float4 *>(sC + k0);
                const float4 c_hi = *reinterpret_cast<const float4 *>(sC + k0 + 4);
                const float cr[8] = {c_lo.x, c_lo.y, c_lo.z, c_lo.w, c_hi.x, c_hi.y, c_hi.z, c_hi.w};
                bf16x8 cb, cl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    cb[e] = (__bf16)cr[e];
                    if constexpr (!CAUSAL) cl[e] = (__bf16)(cr[e] - (float)cb[e]);
                }
                bf16x8 gl;
                if constexpr (!CAUSAL) gl = tr8(tr_addr<TD>(sGl, k0, 32 * vb), tr_addr<TD>(sGl, k0 + 4, 32 * vb));
#pragma unroll
                for (int i = 0; i < FBW; ++i) {
                    const int fb = FBW * fh + i;
                    const bf16x8 qa = tr8(tr_addr<TF>(sQ, k0, 32 * fb), tr_addr<TF>(sQ, k0 + 4, 32 * fb));
                    R[i] = mfma(qa, gb, R[i]);
                    if constexpr (!CAUSAL) R[i] = mfma(qa, gl, R[i]);
                    if (i == vb) {   // feature block w = FBW * fh + vb
                        Zr = mfma(qa, cb, Zr);
                        if constexpr (!CAUSAL) Zr = mfma(qa, cl, Zr);
                    }
                }
            }
        }
    }
    float *Ro = a.ws_Rp + ((size_t)bg * a.nseg + seg) * ((size_t)F * D + F);
#pragma unroll
    for (int i = 0; i < FBW; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            Ro[(size_t)(32 * (FBW * fh + i) + acc_row(r, h)) * D + 32 * vb + l32] = R[i][r];
    if (l32 == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Ro[(size_t)F * D + 32 * w + acc_row(r, h)] = Zr[r];
    }
}

// ---------------------------------------------------------------------------
// k_bwd_kv_cos_mfma: backward over the 32-row chunks of one (batch, KV head,
// segment) from the exclusive suffix (R, r).  Wave w (of F/32) holds R^T for
// feature block w and forms dPhi(k) of that block; waves w < D/32 also form
// dv for value block w.  Per head, wave 0 forms the masked A tile and wave 1
// the P tile for the whole workgroup, as bf16 operands passed through LDS
// (each lane's registers to its own slot).  The sin-half waves pass their
// weighted dPhi(k) tiles to the cos-half waves, which apply phi' and stage
// dk.
// ---------------------------------------------------------------------------
template <int D, int PHI, bool CAUSAL>
__global__ __launch_bounds__(D * 4) __attribute__((amdgpu_waves_per_eu(2)))
void k_bwd_kv_cos_mfma(Args a) {
    constexpr int F = 2 * D, NW = D / 32, FW = F / 32, NT = 64 * FW;
    using TF = PadI<F>;
    using TD = PadI<D>;
    __shared__ __attribute__((aligned(16))) u16 sK[kCc * TF::ld];
    __shared__ __attribute__((aligned(16))) u16 sKr[kCc * TD::ld];   // phi(k) rows (phi'), then dk rows
    __shared__ __attribute__((aligned(16))) u16 sV[kCc * TD::ld];
    __shared__ __attribute__((aligned(16))) u16 sQ[kCc * TF::ld];
    __shared__ __attribute__((aligned(16))) float sX[NW][64 * 16];   // sin halves of dPhi(k)
    __shared__ __attribute__((aligned(16))) u16 sG[kCc * TD::ld];    // gn, then dv rows
    __shared__ __attribute__((aligned(16))) u16 sR[F * TD::ld];
    __shared__ __attribute__((aligned(16))) u16 sGr[kCc * TD::ld];   // raw g rows (for P)
    __shared__ __attribute__((aligned(16))) float sCc[kCc], sIq[kCc];   // c_i, 1 / den_i
    __shared__ float sr[F];
    __shared__ bf16x8 sAop[2][64], sPop[2][64];   // A, P operands of one head, per lane

    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int t = threadIdx.x, l = t & 63, w = t >> 6, h = l >> 5, l32 = l & 31;
    const size_t SD = (size_t)F * D + F;
    const u16 *kh = static_cast<const u16 *>(a.k) + (size_t)bg * a.N * D;
    const u16 *vh = static_cast<const u16 *>(a.v) + (size_t)bg * a.N * D;
    u16 *dkh = static_cast<u16 *>(a.dk) + (size_t)bg * a.N * D;
    u16 *dvh = static_cast<u16 *>(a.dv) + (size_t)bg * a.N * D;
    const size_t bh0 = (size_t)b * a.H + (size_t)g * a.nrep;
    const u16 *qbase = static_cast<const u16 *>(a.q);
    const u16 *gbase = static_cast<const u16 *>(a.g);

    // the segment's exclusive suffix of (R, r) (causal) or the sequence total
    const float *Rp = a.ws_Rs + ((size_t)bg * (a.nseg + 1) + (CAUSAL ? seg : a.nseg)) * SD;
    f32x16 Rt[NW];
#pragma unroll
    for (int db = 0; db < NW; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) Rt[db][r] = Rp[(size_t)(32 * w + l32) * D + 32 * db + acc_row(r, h)];
    for (int e = t; e < F; e += NT) sr[e] = Rp[(size_t)F * D + e];

    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    const int nch = (row1 - row0 + kCc - 1) / kCc;
    constexpr int NV = RawTile<D, NT, kCc>::NV, V8 = D / 8;
    RawTile<D, NT, kCc> rK, rV, rQ, rG;
    // prefetched: den of this thread's G rows, c and den of query t % 32
    float pden[NV], pc, pdq;
    auto load_dc = [&](size_t hh, int cc) {
#pragma unroll
        for (int k = 0; k < NV; ++k) pden[k] = a.ws_den[hh * a.N + min(cc + (t + k * NT) / V8, a.N - 1)];
        pc = a.ws_c[hh * a.N + min(cc + (t & (kCc - 1)), a.N - 1)];
        pdq = a.ws_den[hh * a.N + min(cc + (t & (kCc - 1)), a.N - 1)];
    };
    {
        const int c0 = row0 + (nch - 1) * kCc;
        rK.template load<true>(kh, c0, a.N, a.cw, a.sw);
        rV.load(vh, c0, a.N);
        if constexpr (CAUSAL) {   // the in-chunk terms need the queries' rows
            rQ.template load<true>(qbase + bh0 * a.N * D, c0, a.N, a.cw, a.sw);
            rG.load(gbase + bh0 * a.N * D, c0, a.N);
            load_dc(bh0, c0);
        }
    }
    for (int ci = nch - 1; ci >= 0; --ci) {
        const int c0 = row0 + ci * kCc;
        const int cn = ci > 0 ? c0 - kCc : c0;   // next chunk (none: reload this one)
        __syncthreads();   // the previous chunk's rows are stored
        rK.template store_feat<PHI, true, TF, false, TD>(sK, c0, a.N, nullptr, nullptr, sKr);
        rV.template store<TD>(sV);
        rK.template load<true>(kh, cn, a.N, a.cw, a.sw);
        rV.load(vh, cn, a.N);
        // R (bf16, [feature][value]) for the state terms (bidirectional: the
        // total, staged once)
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
        }
        // one head's query rows into LDS: Phi(Q), gn = g / den (rows past N:
        // zeros), raw g, c, 1 / den
        auto stage_head = [&]() {
            rQ.template store_feat<PHI, true, TF, false>(sQ, c0, a.N, nullptr, nullptr);
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int idx = t + k * NT, i = idx / V8, c8 = (idx % V8) * 8;
                const float inv = c0 + i < a.N ? rcp(pden[k]) : 0.f;
                const uint4 u = rG.v[k];
                uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    wds[e] = pk2(__uint_as_float(wds[e] << 16) * inv, __uint_as_float(wds[e] & 0xffff0000u) * inv);
                *reinterpret_cast<uint4 *>(sG + TD::at(i, c8)) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
            }
            if (t < kCc) {
                sCc[t] = c0 + t < a.N ? pc : 0.f;
                sIq[t] = c0 + t < a.N ? rcp(pdq) : 0.f;
            }
            rG.template store<TD>(sGr);
        };
        // the first head is staged here, in straight-line code, with the chunk
        // (in the head loop, the wait for its rows would also wait for the K, V
        // loads just issued); the state terms read none of its tiles
        if constexpr (CAUSAL) stage_head();
        __syncthreads();

        // state terms: dPhi(k)^T = R V^T - r (block w); dv^T = R^T Phi(K)^T (value block w)
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
#pragma unroll
        for (int r = 0; r < 16; ++r) dK[r] -= sr[32 * w + acc_row(r, h)];
        if (w < NW) {
            dV = mfma_chain<F / 16, 2>(
                [&](int s) { return tr8(tr_addr<TD>(sR, 16 * s + 8 * h, 32 * w), tr_addr<TD>(sR, 16 * s + 8 * h + 4, 32 * w)); },
                [&](int s) { return ld8<TF>(sK, l32, 16 * s + 8 * h); }, dV);
        }

        // causal: the chunk's own queries (in-chunk terms) and the R update
        for (int rep = 0; rep < (CAUSAL ? a.nrep : 0); ++rep) {
            if (rep > 0) {
                __syncthreads();   // the previous head's LDS reads are done
                stage_head();
                __syncthreads();
            }
            {   // Q, G, den, c of the next head, or of the first head at the next chunk
                const bool last = rep + 1 == a.nrep;
                const size_t hn = bh0 + (last ? 0 : rep + 1);
                const int cq = last ? cn : c0;
                rQ.load(qbase + hn * a.N * D, cq, a.N);
                if (last) rQ.load_w(a.cw, a.sw, cq, a.N);   // new positions
                rG.load(gbase + hn * a.N * D, cq, a.N);
                load_dc(hn, cq);
            }
            // A = Phi(Q) Phi(K)^T (over F) on wave 0 and P = (G V^T) / den - c on
            // wave 1 (queries x keys, i >= j), as bf16 operands for every wave;
            // P from the raw g rows scaled in fp32 (it can be a small
            // difference, which bf16-rounded gn would not resolve)
            if (w == 0) {
                f32x16 A = mfma_chain<F / 16, 4>([&](int s) { return ld8<TF>(sQ, l32, 16 * s + 8 * h); },
                                                 [&](int s) { return ld8<TF>(sK, l32, 16 * s + 8 * h); }, zero16());
#pragma unroll
                for (int r = 0; r < 16; ++r) A[r] = acc_row(r, h) >= l32 ? A[r] : 0.f;
                sAop[0][l] = acc_op(A, 0);
                sAop[1][l] = acc_op(A, 1);
            } else if (w == 1) {
                f32x16 P = mfma_chain<D / 16, 4>([&](int s) { return ld8<TD>(sGr, l32, 16 * s + 8 * h); },
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
            // R^T += gn^T Phi(Q) for this chunk's rows; r += Phi(Q)^T c from the
            // same Phi(Q) operand (lane (n, h) holds feature 32w + n of rows
            // 16s + 8h .. +7; the two halves cover the chunk).  Neither needs A or P.
            float racc = 0.f;
#pragma unroll
            for (int s = 0; s < kCc / 16; ++s) {
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
                for (int e = 0; e < 8; ++e) racc += cv[e] * (float)qb[e];
            }
            racc = sum_halves(racc);
            if (h == 0) sr[32 * w + l32] += racc;
            __syncthreads();   // the A and P operands are in LDS
            // in-chunk terms: dPhi(k)^T += Phi(Q)^T P (block w), dv^T += gn^T A (value block w)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int k0 = 16 * s + 4 * h;
                dK = mfma(tr8(tr_addr<TF>(sQ, k0, 32 * w), tr_addr<TF>(sQ, k0 + 8, 32 * w)), sPop[s][l], dK);
                if (w < NW)
                    dV = mfma(tr8(tr_addr<TD>(sG, k0, 32 * w), tr_addr<TD>(sG, k0 + 8, 32 * w)), sAop[s][l], dV);
            }
        }
        // chain rule through cos/sin: the sin-half waves hand sin_j dPhi(k) to
        // the cos-half wave of the same dims
        const int tj = min(c0 + l32, a.N - 1);
        const float mk = w < NW ? a.cw[tj] : a.sw[tj];   // this lane's key weight for block w
#pragma unroll
        for (int r = 0; r < 16; ++r) dK[r] *= mk;
        if (w >= NW) put_acc(sX[w - NW], dK);
        __syncthreads();   // sX complete; every read of sG of the last head is done
        if (w < NW) {
            const f32x16 Ks = get_acc(sX[w]);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d0 = 32 * w + 8 * q4 + 4 * h;
                float kr[4];
                ld4f(sKr + TD::at(l32, d0), kr);
#pragma unroll
                for (int e = 0; e < 4; ++e) dK[4 * q4 + e] = phi_d_feat<PHI>(kr[e]) * (dK[4 * q4 + e] + Ks[4 * q4 + e]);
            }
            // this lane overwrites exactly the phi(k) entries it just read
            stage_out<TD>(sKr, dK, 1.f, 32 * w);
            stage_out<TD>(sG, dV, 1.f, 32 * w);
        }
        __syncthreads();
        store_rows<D, NT, TD>(dkh, sKr, c0, a.N);
        store_rows<D, NT, TD>(dvh, sG, c0, a.N);
    }
}

template <int D, int PHI, bool CAUSAL>
hipError_t run(const Args &a, hipStream_t s) {
    constexpr int F = 2 * D;
    const unsigned n_units = (unsigned)(a.B * a.Hkv);
    const size_t SD = (size_t)F * D + F;
    hipError_t e = a.state_ready ? hipSuccess : mfma_state_run(a, PHI, CAUSAL ? 1 : 0, s);
    if (e != hipSuccess) return e;
    {
        TimedLaunch tl(CAUSAL ? "k_bwd_q_cos_mfma" : "k_bwd_q_cos_bidir_mfma", s);
        hipLaunchKernelGGL((k_bwd_q_cos_mfma<D, PHI, CAUSAL>), dim3(n_units * a.nseg), dim3(4 * D), 0, s, a);
    }
    {
        TimedLaunch tl(CAUSAL ? "k_bwd_r_cos_mfma" : "k_bwd_r_cos_bidir_mfma", s);
        hipLaunchKernelGGL((k_bwd_r_cos_mfma<D, PHI, CAUSAL>), dim3(n_units * a.nseg), dim3(4 * D), 0, s, a);
    }
    {
        TimedLaunch tl("k_scan_R", s);
        // per-segment records are already summed over the group's heads
        e = scan_suffix(a.ws_Rp, a.ws_Rs, a.nseg, SD, a.Hkv, a.Hkv, 1, n_units, CAUSAL, s);
        if (e != hipSuccess) return e;
    }
    {
        TimedLaunch tl(CAUSAL ? "k_bwd_kv_cos_mfma" : "k_bwd_kv_cos_bidir_mfma", s);
        hipLaunchKernelGGL((k_bwd_kv_cos_mfma<D, PHI, CAUSAL>), dim3(n_units * a.nseg), dim3(4 * D), 0, s, a);
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

hipError_t mfma_bwd_cos_run(const Args &a, int phi, int causal, hipStream_t s) {
    if (causal) return a.D == 64 ? by_phi<64, true>(a, phi, s) : by_phi<128, true>(a, phi, s);
    return a.D == 64 ? by_phi<64, false>(a, phi, s) : by_phi<128, false>(a, phi, s);
}

}  // namespace la
