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

// Registers 8s .. 8s+7 of an accumulator as a bf16 operand (round to nearest even).
__device__ __forceinline__ bf16x8 acc_op(const f32x16 &acc, int s) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)acc[8 * s + e];
    return o;
}

}  // namespace mf
}  // namespace la
