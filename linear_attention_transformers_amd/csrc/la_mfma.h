// la_mfma.h -- gfx950 matrix-core building blocks for the bf16 kernels.
//
// v_mfma_f32_32x32x16_bf16 (D = A x B + C, A 32x16, B 16x32, fp32 C/D):
//   A[m][k] is element k%8 of lane m + 32*(k/8); B[k][n] is element k%8 of
//   lane n + 32*(k/8); D[m][n] is register (m/8)*4 + m%4 of lane
//   n + 32*((m/4)%2).  (Checked on the device with an in-bounds probe.)
// Consequences used throughout:
//   * a row-major LDS tile X[rows][k] gives A (or B) operands with one 16-byte
//     read per lane: row = lane%32, k = 8*(lane/32) .. +7;
//   * an accumulator D (M x N) is an operand for a product that contracts
//     over M (as B, with N the output column; or as A, with N the output
//     row), in a permuted k order: register 8s+e of lane half h holds
//     M-row 16s + 8*(e/4) + 4h + e%4, so the other operand must use the same
//     order (two 8-byte reads);
//   * ds_read_b64_tr_b16 (per 16-lane group, lane i receives element i%4 of
//     the 8-byte rows addressed by lanes 4e + i/4, e = 0..3) turns a row-major
//     tile X[k][n] into operands that contract over its row index k: lane j
//     of the group addresses X[k0 + j/4][n0 + 4*(j%4)] and lane i receives
//     X[k0 + e][n0 + i], e = 0..3.
#pragma once

#include <hip/hip_runtime.h>

#include "la_common.h"

namespace la {
namespace mf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}

// 16-byte operand: 8 consecutive elements of an LDS row.
__device__ __forceinline__ bf16x8 ld8(const u16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Operand in the permuted k order of an accumulator: elements p[0..3], p[8..11].
__device__ __forceinline__ bf16x8 ld4x2(const u16 *p) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(p);
    const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(p + 8);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposed 4-row read (see header comment); p = this lane's address.
__device__ __forceinline__ i16x4 tr4(const u16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

// Two transposed 4-row reads glued into one 8-element operand.
__device__ __forceinline__ bf16x8 tr8(const u16 *p_lo, const u16 *p_hi) {
    const i16x8 v = __builtin_shufflevector(tr4(p_lo), tr4(p_hi), 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 ones8() {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)1.0f;
    return o;
}

// Registers 8s .. 8s+7 of an accumulator as a bf16 operand (round to nearest even).
__device__ __forceinline__ bf16x8 acc_op(const f32x16 &acc, int s) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)acc[8 * s + e];
    return o;
}

constexpr int kC = 64;   // chunk length (rows)

// phi for values that are rounded to bf16 right after: the hardware exp
// (__expf, a few ulp) is far below bf16 resolution.
template <int PHI>
__device__ __forceinline__ float phi_fast(float x) {
    if constexpr (PHI == kElu1) return x > 0.f ? x + 1.f : __expf(x);
    else return phi_f<PHI>(x);
}

__device__ __forceinline__ float bf2f(u16 x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ u16 f2bf(float x) {
    const __bf16 b = (__bf16)x;
    return __builtin_bit_cast(u16, b);
}

// Stage rows [c0, c0 + kC) of one head's [N][D] bf16 tensor into an LDS tile
// [kC][LD] (rows >= N are zeros).  FEAT: apply phi, and with COS write
// [cos_t phi, sin_t phi] (width 2D); otherwise copy.
template <int D, int LD, int NT, bool FEAT, int PHI, bool COS>
__device__ __forceinline__ void stage(u16 *dst, const u16 *src, int c0, int N, const float *cw,
                                      const float *sw) {
    constexpr int V8 = D / 8;   // 16-byte vectors per row
    for (int v = threadIdx.x; v < kC * V8; v += NT) {
        const int r = v / V8, c8 = (v % V8) * 8, t = c0 + r;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (t < N) raw = *reinterpret_cast<const uint4 *>(src + (size_t)t * D + c8);
        if constexpr (!FEAT) {
            *reinterpret_cast<uint4 *>(dst + r * LD + c8) = raw;
        } else {
            const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = t < N ? phi_fast<PHI>(__uint_as_float(w4[e] << 16)) : 0.f;
                f[2 * e + 1] = t < N ? phi_fast<PHI>(__uint_as_float(w4[e] & 0xffff0000u)) : 0.f;
            }
            const float m0 = COS ? (t < N ? cw[t] : 0.f) : 1.f;
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = (uint32_t)f2bf(m0 * f[2 * e]) | ((uint32_t)f2bf(m0 * f[2 * e + 1]) << 16);
            *reinterpret_cast<uint4 *>(dst + r * LD + c8) = make_uint4(o[0], o[1], o[2], o[3]);
            if constexpr (COS) {
                const float m1 = t < N ? sw[t] : 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = (uint32_t)f2bf(m1 * f[2 * e]) | ((uint32_t)f2bf(m1 * f[2 * e + 1]) << 16);
                *reinterpret_cast<uint4 *>(dst + r * LD + D + c8) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
}

// Rows [c0, c0 + C) of one head's [N][D] bf16 tensor held in registers as
// 16-byte vectors (rows >= N read as zeros), so the global loads of the next
// chunk can be in flight while the current one is computed.  Vector k of
// thread t is element-row (t + k*NT) / (D/8), columns 8*((t + k*NT) % (D/8)).
template <int D, int NT, int C = kC>
struct RawTile {
    static constexpr int V8 = D / 8;
    static constexpr int NV = C * V8 / NT;
    static_assert(NV * NT == C * V8, "tile must split evenly over the threads");
    uint4 v[NV];

    __device__ __forceinline__ void load(const u16 *src, int c0, int N) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = threadIdx.x + k * NT, r = idx / V8, c8 = (idx % V8) * 8;
            v[k] = make_uint4(0, 0, 0, 0);
            if (c0 + r < N) v[k] = *reinterpret_cast<const uint4 *>(src + (size_t)(c0 + r) * D + c8);
        }
    }

    __device__ __forceinline__ void store(u16 *dst, int LD) const {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = threadIdx.x + k * NT, r = idx / V8, c8 = (idx % V8) * 8;
            *reinterpret_cast<uint4 *>(dst + r * LD + c8) = v[k];
        }
    }

    // Features: phi, then with COS [cos_t phi, sin_t phi] (row width 2D),
    // rounded to bf16.  With sz != nullptr, also sQZ[r] = Phi(x_r) . z over
    // the rounded features (fixed-order shuffle reduction across the V8
    // threads of a row).
    template <int PHI, bool COS>
    __device__ __forceinline__ void store_feat(u16 *dst, int LD, int c0, int N, const float *cw,
                                               const float *sw, const float *sz,
                                               float *sQZ) const {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = threadIdx.x + k * NT, r = idx / V8, c8 = (idx % V8) * 8, t = c0 + r;
            const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = t < N ? phi_fast<PHI>(__uint_as_float(w4[e] << 16)) : 0.f;
                f[2 * e + 1] = t < N ? phi_fast<PHI>(__uint_as_float(w4[e] & 0xffff0000u)) : 0.f;
            }
            const float m0 = COS ? (t < N ? cw[t] : 0.f) : 1.f;
            float qz = 0.f;
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const u16 lo = f2bf(m0 * f[2 * e]), hi = f2bf(m0 * f[2 * e + 1]);
                o[e] = (uint32_t)lo | ((uint32_t)hi << 16);
                if (sz) qz += bf2f(lo) * sz[c8 + 2 * e] + bf2f(hi) * sz[c8 + 2 * e + 1];
            }
            *reinterpret_cast<uint4 *>(dst + r * LD + c8) = make_uint4(o[0], o[1], o[2], o[3]);
            if constexpr (COS) {
                const float m1 = t < N ? sw[t] : 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const u16 lo = f2bf(m1 * f[2 * e]), hi = f2bf(m1 * f[2 * e + 1]);
                    o[e] = (uint32_t)lo | ((uint32_t)hi << 16);
                    if (sz) qz += bf2f(lo) * sz[D + c8 + 2 * e] + bf2f(hi) * sz[D + c8 + 2 * e + 1];
                }
                *reinterpret_cast<uint4 *>(dst + r * LD + D + c8) = make_uint4(o[0], o[1], o[2], o[3]);
            }
            if (sz) {
#pragma unroll
                for (int o2 = 1; o2 < V8; o2 <<= 1) qz += __shfl_xor(qz, o2);
                if (idx % V8 == 0) sQZ[r] = qz;
            }
        }
    }
};

// Lane address for a transposed 4-row read of tile X (row stride LD): rows
// k0 .. k0+3, this lane's operand index (lane % 32) mapped to columns
// col0 .. col0+31.
__device__ __forceinline__ const u16 *tr_addr(const u16 *X, int LD, int k0, int col0) {
    const int l = threadIdx.x & 63, gi = l >> 4, i16 = l & 15;
    return X + (k0 + (i16 >> 2)) * LD + col0 + 16 * (gi & 1) + 4 * (i16 & 3);
}

// Output rows go through LDS so global stores are whole rows, 16 bytes per
// lane, instead of 8-byte pieces spread over 32 rows per instruction.
// stage_out: this lane's accumulator values for row `lane % 32` and columns
// col0 + 8q + 4h + 0..3 (q = 0..3), scaled by `scale`, into sO[32][LDO].
__device__ __forceinline__ void stage_out(u16 *sO, int LDO, const f32x16 &acc, float scale,
                                          int col0) {
    const int l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
    u16 *row = sO + l32 * LDO + col0 + 4 * h;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t lo = (uint32_t)f2bf(acc[4 * q4] * scale) | ((uint32_t)f2bf(acc[4 * q4 + 1] * scale) << 16);
        const uint32_t hi =
            (uint32_t)f2bf(acc[4 * q4 + 2] * scale) | ((uint32_t)f2bf(acc[4 * q4 + 3] * scale) << 16);
        *reinterpret_cast<uint2 *>(row + 8 * q4) = make_uint2(lo, hi);
    }
}

// store_rows: rows 0..31 of sO (row r -> global row c0 + r of a [N][D]
// tensor, rows >= N skipped), NT threads (numbered tid, default the thread
// index) storing 16-byte pieces.  Call after a barrier that follows the
// stage_out of every wave.
template <int D, int NT>
__device__ __forceinline__ void store_rows(u16 *dst, const u16 *sO, int LDO, int c0, int N,
                                           int tid = -1) {
    constexpr int V8 = D / 8;
    for (int v = tid < 0 ? (int)threadIdx.x : tid; v < 32 * V8; v += NT) {
        const int r = v / V8, c8 = (v % V8) * 8;
        if (c0 + r < N)
            *reinterpret_cast<uint4 *>(dst + (size_t)(c0 + r) * D + c8) =
                *reinterpret_cast<const uint4 *>(sO + r * LDO + c8);
    }
}

}  // namespace mf
}  // namespace la
