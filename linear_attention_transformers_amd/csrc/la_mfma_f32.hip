// la_mfma_f32.hip -- float32 bidirectional path on the gfx950 matrix cores
// (v_mfma_f32_32x32x2_f32: float32 operands, float32 accumulate), for float32
// storage with F = D in {64, 128}.
//
// Method (SVD_linear_Attention, "Module neuralops.core.triton_kernels.
// linear_attn", module docstring: the bidirectional parallel reduction;
// function bwd: the gradient of fwd).  With the full sums
//   S = sum_j Phi(k_j) v_j^T,  z = sum_j Phi(k_j),
//   den_i = Phi(q_i).z + eps,  out_i = Phi(q_i)^T S / den_i,
// and, for the backward with g_i = dL/dout_i,
//   U_i = S g_i,  c_i = (Phi(q_i).U_i) / den_i^2  (= (g_i.out_i) / den_i),
//   dPhi(q_i) = U_i / den_i - c_i z,
//   R = sum_i Phi(q_i) (g_i / den_i)^T,  r = sum_i c_i Phi(q_i),
//   dPhi(k_j) = R v_j - r,  dv_j = R^T Phi(k_j),
// then dq, dk through phi' (taken from the float32 feature: exact).  Query head
// h reads KV head h / n_rep (gqa page, bwd); (R, r) of a KV head is the sum
// over its n_rep query heads, which the suffix scan forms from per-head,
// per-segment partials.
//
// Work split: the state pass runs per (batch, KV head, segment); the row
// passes per (batch, query head, segment) (forward, dq) or (batch, KV head,
// segment) (dk/dv).  Every product is a 32x32 output tile that a wave owns,
// accumulated over K in steps of 2: operand A[m][k] is lane m + 32k, B[k][n] is
// lane n + 32k, and accumulator register r of lane l is row
// 8(r/4) + 4(l/32) + r%4, column l%32.  Operands come from LDS tiles of
// float32 rows; a tile read by column (32 rows, one column per half-wave) has
// rows 2 floats longer than its data, one read by row 32 floats longer, which
// puts the 64 lanes of every read on 64 distinct banks.
#include "la_common.h"
#include "la_kernels.h"
#include "la_timing.h"

namespace la {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma2(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}

// accumulator row of register r for lane half h
__device__ __forceinline__ int arow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

constexpr int kNT = 256;   // four waves

// Rows per iteration of the row passes: four 32x32 output tiles per
// iteration over the (row block, column block) pairs of a D-wide output.
template <int D>
constexpr int rows_blk() { return 128 * 32 / D; }

// phi'(x) from the float32 feature p = phi(x): relu p > 0 <=> x > 0; elu+1
// p = x + 1 > 1 for x > 0 and p = e^x <= 1 otherwise, so min(p, 1) is phi'(x)
// exactly; identity 1.
template <int PHI>
__device__ __forceinline__ float dphi_feat(float p) {
    if constexpr (PHI == kElu1) return fminf(p, 1.f);
    else if constexpr (PHI == kRelu) return p > 0.f ? 1.f : 0.f;
    else return 1.f;
}

// Rows [r0, r0 + RB) of a [N][D] float32 tensor in registers, float4 per
// vector (rows >= N read as zeros); thread t's vector k is row
// (t + k NT) / (D/4), columns 4 ((t + k NT) % (D/4)).
template <int D, int RB>
struct Rows {
    static constexpr int V4 = D / 4, NV = RB * V4 / kNT;
    static_assert(NV * kNT == RB * V4, "rows split evenly over the threads");
    float4 v[NV];
    __device__ __forceinline__ void load(const float *src, int r0, int N) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = threadIdx.x + k * kNT, r = idx / V4, c4 = (idx % V4) * 4;
            v[k] = *reinterpret_cast<const float4 *>(src + (size_t)min(r0 + r, N - 1) * D + c4);
            if (r0 + r >= N) v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    // raw values into dst[r][ld]
    __device__ __forceinline__ void store(float *dst, int ld) const {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = threadIdx.x + k * kNT, r = idx / V4, c4 = (idx % V4) * 4;
            *reinterpret_cast<float4 *>(dst + r * ld + c4) = v[k];
        }
    }
    // phi of the values into dst[r][ld] (rows >= N give phi(0) * 0 = 0:
    // masked by the row factor); with DEN, also den[r] = phi(row).z + eps, a
    // fixed-order sum over the V4/... threads of a row
    template <int PHI, bool DEN>
    __device__ __forceinline__ void store_feat(float *dst, int ld, int r0, int N, const float *sz,
                                               float eps, float *den) const {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = threadIdx.x + k * kNT, r = idx / V4, c4 = (idx % V4) * 4;
            const float m = r0 + r < N ? 1.f : 0.f;
            float4 f;
            f.x = phi_f<PHI>(v[k].x) * m;
            f.y = phi_f<PHI>(v[k].y) * m;
            f.z = phi_f<PHI>(v[k].z) * m;
            f.w = phi_f<PHI>(v[k].w) * m;
            *reinterpret_cast<float4 *>(dst + r * ld + c4) = f;
            if constexpr (DEN) {
                float d = f.x * sz[c4] + f.y * sz[c4 + 1] + f.z * sz[c4 + 2] + f.w * sz[c4 + 3];
                // the V4 threads of a row are consecutive and aligned: sum
                // them in a fixed order by a butterfly
#pragma unroll
                for (int o = 1; o < V4; o <<= 1) d += __shfl_xor(d, o);
                if (idx % V4 == 0) den[r] = d + eps;
            }
        }
    }
};

// ---------------------------------------------------------------------------
// k_state_f32: per (batch, KV head, segment) the segment sums dS = Phi(K)^T V
// and dz = Phi(K)^T 1, written to the segment's record.  Chunks of 32 rows;
// wave w owns feature block fb and value blocks vbs of S (and the z tile of
// its feature block when it owns value block 0).
// ---------------------------------------------------------------------------
template <int D, int PHI>
__global__ __launch_bounds__(kNT) void k_state_f32(Args a) {
    constexpr int C = 32, NB = D / 32, VBW = NB * NB / 4;   // value blocks per wave
    constexpr int LD = D + 32;                               // read by row
    __shared__ __attribute__((aligned(16))) float sK[C * LD];
    __shared__ __attribute__((aligned(16))) float sV[C * LD];
    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int fbw = NB == 2 ? w >> 1 : w;                    // feature block
    const int vb0 = NB == 2 ? (w & 1) : 0;                   // first value block
    const float *kh = static_cast<const float *>(a.k) + (size_t)bg * a.N * D;
    const float *vh = static_cast<const float *>(a.v) + (size_t)bg * a.N * D;
    f32x16 S[VBW], Z = zero16();
#pragma unroll
    for (int i = 0; i < VBW; ++i) S[i] = zero16();
    const bool zown = vb0 == 0;
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    Rows<D, C> rK, rV;
    rK.load(kh, row0, row1);
    rV.load(vh, row0, row1);
    for (int c0 = row0; c0 < row1; c0 += C) {
        __syncthreads();
        rK.template store_feat<PHI, false>(sK, LD, c0, row1, nullptr, 0.f, nullptr);
        rV.store(sV, LD);
        __syncthreads();
        rK.load(kh, c0 + C, row1);   // next chunk (past the segment: zeros, unused)
        rV.load(vh, c0 + C, row1);
#pragma unroll 4
        for (int j = 0; j < C / 2; ++j) {
            const int t = 2 * j + h;
            const float ka = sK[t * LD + 32 * fbw + l32];
#pragma unroll
            for (int i = 0; i < VBW; ++i) S[i] = mfma2(ka, sV[t * LD + 32 * (vb0 + i) + l32], S[i]);
            if (zown) Z = mfma2(ka, 1.f, Z);
        }
    }
    float *out = a.ws_S + ((size_t)bg * (a.nseg + 1) + seg) * ((size_t)D * D + D);
#pragma unroll
    for (int i = 0; i < VBW; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            out[(size_t)(32 * fbw + arow(r, h)) * D + 32 * (vb0 + i) + l32] = S[i][r];
    if (zown && l32 == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) out[(size_t)D * D + 32 * fbw + arow(r, h)] = Z[r];
    }
}

// ---------------------------------------------------------------------------
// k_fwd_bidir_f32: per (batch, query head, segment): out = Phi(Q) S / den
// against the total (S, z).  Wave w owns row block rb and value block vb of
// each iteration's RB x D output; its slice of S is held as B operands.
// ---------------------------------------------------------------------------
template <int D, int PHI>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 1)))
void k_fwd_bidir_f32(Args a) {
    constexpr int RB = rows_blk<D>(), NB = D / 32, LDQ = D + 2;   // Phi(Q) read by column
    __shared__ __attribute__((aligned(16))) float sQ[RB * LDQ];
    __shared__ float sz[D];
    __shared__ float sden[RB];
    const int seg = blockIdx.x % a.nseg, bh = blockIdx.x / a.nseg;
    const int b = bh / a.H, hq = bh % a.H, bg = b * a.Hkv + hq / a.nrep;
    const int l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rb = w / NB, vb = w % NB;
    const float *qh = static_cast<const float *>(a.q) + (size_t)bh * a.N * D;
    float *oh = static_cast<float *>(a.out) + (size_t)bh * a.N * D;
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + a.nseg) * ((size_t)D * D + D);
    float Sop[D / 2];   // B[k][n] = S[2j + k][32 vb + n] for k-step j
#pragma unroll
    for (int j = 0; j < D / 2; ++j) Sop[j] = Sp[(size_t)(2 * j + h) * D + 32 * vb + l32];
    for (int e = threadIdx.x; e < D; e += kNT) sz[e] = Sp[(size_t)D * D + e];
    __syncthreads();
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    Rows<D, RB> rQ;
    rQ.load(qh, row0, a.N);
    for (int c0 = row0; c0 < row1; c0 += RB) {
        __syncthreads();
        rQ.template store_feat<PHI, true>(sQ, LDQ, c0, a.N, sz, a.eps, sden);
        __syncthreads();
        rQ.load(qh, c0 + RB, a.N);
        f32x16 acc = zero16();
#pragma unroll
        for (int j = 0; j < D / 2; ++j) acc = mfma2(sQ[(32 * rb + l32) * LDQ + 2 * j + h], Sop[j], acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 32 * rb + arow(r, h);
            if (c0 + i < row1) oh[(size_t)(c0 + i) * D + 32 * vb + l32] = acc[r] / sden[i];
        }
    }
}

// ---------------------------------------------------------------------------
// k_bwd_q_bidir_f32: per (batch, query head, segment): dq against the total
// (S, z), and the segment's partial (R, r).  Per iteration (RB rows):
//   U = G S^T (wave: row block ru, feature block fu), c from the row dots
//   Phi(q).U combined over the feature blocks through LDS, dq from U;
//   R += Phi(Q)^T (G / den) (wave: feature block fr, value blocks),
//   r += Phi(Q)^T c (the wave of value block 0).
// ---------------------------------------------------------------------------
// Waves per SIMD the dq kernel is built for: at D = 64 its registers fit
// two (the compiler, left free, takes a few more than 256 and gets one).
template <int D>
constexpr int q_f32_waves() { return D == 64 ? 2 : 1; }

template <int D, int PHI>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(q_f32_waves<D>())))
void k_bwd_q_bidir_f32(Args a) {
    constexpr int RB = rows_blk<D>(), NB = D / 32, VBW = NB * NB / 4;
    constexpr int LDC = D + 2;    // read by column (U's A operand) and by row (R's operands)
    __shared__ __attribute__((aligned(16))) float sQ[RB * LDC];
    __shared__ __attribute__((aligned(16))) float sG[RB * LDC];
    __shared__ float sz[D];
    __shared__ float sden[RB];
    __shared__ float sc[RB];
    __shared__ float spart[NB][RB];   // Phi(q).U over one feature block
    const int seg = blockIdx.x % a.nseg, bh = blockIdx.x / a.nseg;
    const int b = bh / a.H, hq = bh % a.H, bg = b * a.Hkv + hq / a.nrep;
    const int l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ru = w / NB, fu = w % NB;                      // U tile of this wave
    const int fr = NB == 2 ? w >> 1 : w, vr0 = NB == 2 ? (w & 1) : 0;   // R tiles
    const bool rown = vr0 == 0;                              // owns the r tile
    const float *qh = static_cast<const float *>(a.q) + (size_t)bh * a.N * D;
    const float *gh = static_cast<const float *>(a.g) + (size_t)bh * a.N * D;
    float *dqh = static_cast<float *>(a.dq) + (size_t)bh * a.N * D;
    const size_t SD = (size_t)D * D + D;
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + a.nseg) * SD;
    float STop[D / 2];   // B[k][n] = S^T[2j + k][32 fu + n] = S[32 fu + n][2j + k]
#pragma unroll
    for (int j = 0; j < D / 2; ++j) STop[j] = Sp[(size_t)(32 * fu + l32) * D + 2 * j + h];
    for (int e = threadIdx.x; e < D; e += kNT) sz[e] = Sp[(size_t)D * D + e];
    f32x16 R[VBW], rr = zero16();
#pragma unroll
    for (int i = 0; i < VBW; ++i) R[i] = zero16();
    __syncthreads();
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    Rows<D, RB> rQ, rG;
    rQ.load(qh, row0, a.N);
    rG.load(gh, row0, a.N);
    for (int c0 = row0; c0 < row1; c0 += RB) {
        __syncthreads();
        rQ.template store_feat<PHI, true>(sQ, LDC, c0, a.N, sz, a.eps, sden);
        rG.store(sG, LDC);
        __syncthreads();
        rQ.load(qh, c0 + RB, a.N);
        rG.load(gh, c0 + RB, a.N);
        // U tile: rows 32 ru .., features 32 fu ..
        f32x16 U = zero16();
#pragma unroll
        for (int j = 0; j < D / 2; ++j) U = mfma2(sG[(32 * ru + l32) * LDC + 2 * j + h], STop[j], U);
        // partial row dots Phi(q).U over this feature block: lane l32 holds
        // column 32 fu + l32 of rows arow(r, h); sum over the 32 lanes of a half
        float pd[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = U[r] * sQ[(32 * ru + arow(r, h)) * LDC + 32 * fu + l32];
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) x += __shfl_xor(x, o);
            pd[r] = x;
        }
        if (l32 == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) spart[fu][32 * ru + arow(r, h)] = pd[r];
        }
        __syncthreads();
        for (int i = threadIdx.x; i < RB; i += kNT) {
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < NB; ++k) s += spart[k][i];   // fixed order
            const float dn = sden[i];
            sc[i] = c0 + i < row1 ? s / (dn * dn) : 0.f;
        }
        __syncthreads();
        // dq = phi'(q) (U / den - c z) for this wave's tile
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 32 * ru + arow(r, h), f = 32 * fu + l32;
            if (c0 + i < row1) {
                const float dphi = U[r] / sden[i] - sc[i] * sz[f];
                dqh[(size_t)(c0 + i) * D + f] = dphi_feat<PHI>(sQ[i * LDC + f]) * dphi;
            }
        }
        // R += Phi(Q)^T (G / den), r += Phi(Q)^T c over the RB rows
#pragma unroll 4
        for (int j = 0; j < RB / 2; ++j) {
            const int t = 2 * j + h;
            const float qa = sQ[t * LDC + 32 * fr + l32];
            const float inv = 1.f / sden[t];
#pragma unroll
            for (int i = 0; i < VBW; ++i) R[i] = mfma2(qa, sG[t * LDC + 32 * (vr0 + i) + l32] * inv, R[i]);
            if (rown) rr = mfma2(qa, sc[t], rr);
        }
    }
    float *Ro = a.ws_Rp + ((size_t)bh * a.nseg + seg) * SD;
#pragma unroll
    for (int i = 0; i < VBW; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) Ro[(size_t)(32 * fr + arow(r, h)) * D + 32 * (vr0 + i) + l32] = R[i][r];
    if (rown && l32 == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Ro[(size_t)D * D + 32 * fr + arow(r, h)] = rr[r];
    }
}

// ---------------------------------------------------------------------------
// k_bwd_kv_bidir_f32: per (batch, KV head, segment): against the total (R, r)
//   W = V R^T -> dk = phi'(k) (W - r),   dv = Phi(K) R.
// Wave w owns row block rb, feature block fb of W and value block vb of dv;
// its slices of R are held as B operands.
// ---------------------------------------------------------------------------
template <int D, int PHI>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 1)))
void k_bwd_kv_bidir_f32(Args a) {
    constexpr int RB = rows_blk<D>(), NB = D / 32, LDC = D + 2;   // both read by column
    __shared__ __attribute__((aligned(16))) float sK[RB * LDC];
    __shared__ __attribute__((aligned(16))) float sV[RB * LDC];
    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rb = w / NB, cb = w % NB;   // row block; feature block of W = value block of dv
    const float *kh = static_cast<const float *>(a.k) + (size_t)bg * a.N * D;
    const float *vh = static_cast<const float *>(a.v) + (size_t)bg * a.N * D;
    float *dkh = static_cast<float *>(a.dk) + (size_t)bg * a.N * D;
    float *dvh = static_cast<float *>(a.dv) + (size_t)bg * a.N * D;
    const size_t SD = (size_t)D * D + D;
    const float *Rp = a.ws_Rs + ((size_t)bg * (a.nseg + 1) + a.nseg) * SD;
    float RTop[D / 2], Rop[D / 2];
#pragma unroll
    for (int j = 0; j < D / 2; ++j) {
        RTop[j] = Rp[(size_t)(32 * cb + l32) * D + 2 * j + h];   // R^T[2j + k][32 cb + n]
        Rop[j] = Rp[(size_t)(2 * j + h) * D + 32 * cb + l32];    // R[2j + k][32 cb + n]
    }
    const float rf = Rp[(size_t)D * D + 32 * cb + l32];          // r of this lane's column
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    Rows<D, RB> rK, rV;
    rK.load(kh, row0, a.N);
    rV.load(vh, row0, a.N);
    for (int c0 = row0; c0 < row1; c0 += RB) {
        __syncthreads();
        rK.template store_feat<PHI, false>(sK, LDC, c0, a.N, nullptr, 0.f, nullptr);
        rV.store(sV, LDC);
        __syncthreads();
        rK.load(kh, c0 + RB, a.N);
        rV.load(vh, c0 + RB, a.N);
        f32x16 W = zero16(), dV = zero16();
#pragma unroll
        for (int j = 0; j < D / 2; ++j) {
            W = mfma2(sV[(32 * rb + l32) * LDC + 2 * j + h], RTop[j], W);
            dV = mfma2(sK[(32 * rb + l32) * LDC + 2 * j + h], Rop[j], dV);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 32 * rb + arow(r, h), c = 32 * cb + l32;
            if (c0 + i < row1) {
                dkh[(size_t)(c0 + i) * D + c] = dphi_feat<PHI>(sK[i * LDC + c]) * (W[r] - rf);
                dvh[(size_t)(c0 + i) * D + c] = dV[r];
            }
        }
    }
}

template <int D, int PHI>
hipError_t run_fwd(const Args &a, hipStream_t s) {
    const unsigned n_units = (unsigned)(a.B * a.Hkv);
    {
        TimedLaunch tl("k_state_f32", s);
        hipLaunchKernelGGL((k_state_f32<D, PHI>), dim3(n_units * a.nseg), dim3(kNT), 0, s, a);
    }
    hipError_t e;
    {
        TimedLaunch tl("k_scan_S", s);
        e = scan_state(a.ws_S, a.nseg, (size_t)D * D + D, n_units, false, s);
    }
    if (e != hipSuccess) return e;
    TimedLaunch tl("k_fwd_bidir_f32", s);
    hipLaunchKernelGGL((k_fwd_bidir_f32<D, PHI>), dim3((unsigned)(a.B * a.H * a.nseg)), dim3(kNT),
                       0, s, a);
    return hipGetLastError();
}

template <int D, int PHI>
hipError_t run_bwd(const Args &a, hipStream_t s) {
    const unsigned n_units = (unsigned)(a.B * a.Hkv);
    const size_t SD = (size_t)D * D + D;
    hipError_t e;
    if (!a.state_ready) {   // else the forward's records are in ws_S already
        {
            TimedLaunch tl("k_state_f32", s);
            hipLaunchKernelGGL((k_state_f32<D, PHI>), dim3(n_units * a.nseg), dim3(kNT), 0, s, a);
        }
        TimedLaunch tl("k_scan_S", s);
        e = scan_state(a.ws_S, a.nseg, SD, n_units, false, s);
        if (e != hipSuccess) return e;
    }
    {
        TimedLaunch tl("k_bwd_q_bidir_f32", s);
        hipLaunchKernelGGL((k_bwd_q_bidir_f32<D, PHI>), dim3((unsigned)(a.B * a.H * a.nseg)),
                           dim3(kNT), 0, s, a);
    }
    {
        TimedLaunch tl("k_scan_R", s);
        e = scan_suffix(a.ws_Rp, a.ws_Rs, a.nseg, SD, a.H, a.Hkv, a.nrep, n_units, false, s);
    }
    if (e != hipSuccess) return e;
    TimedLaunch tl("k_bwd_kv_bidir_f32", s);
    hipLaunchKernelGGL((k_bwd_kv_bidir_f32<D, PHI>), dim3(n_units * a.nseg), dim3(kNT), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t by_phi(const Args &a, int bwd, int phi, hipStream_t s) {
    switch (phi) {
        case kElu1: return bwd ? run_bwd<D, kElu1>(a, s) : run_fwd<D, kElu1>(a, s);
        case kRelu: return bwd ? run_bwd<D, kRelu>(a, s) : run_fwd<D, kRelu>(a, s);
        default: return bwd ? run_bwd<D, kIdentity>(a, s) : run_fwd<D, kIdentity>(a, s);
    }
}

}  // namespace

bool mfma_f32_serves(int bf16, int causal, int D, int has_cos) {
    return !bf16 && !causal && !has_cos && (D == 64 || D == 128);
}

hipError_t mfma_f32_run(const Args &a, int bwd, int phi, hipStream_t s) {
    return a.D == 64 ? by_phi<64>(a, bwd, phi, s) : by_phi<128>(a, bwd, phi, s);
}

}  // namespace la
