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

#include <type_traits>

#include "la_common.h"

namespace la {
namespace mf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kC = 64;   // chunk length (rows)

// LDS tile layouts.  A tile with RL bf16 elements per row keeps element
// (r, c) at index L::at(r, c), L::ld elements per row.  The LDS has 64 banks
// of 4 bytes; 16-byte accesses are served 16 lanes at a time and 8-byte ones
// 32 lanes at a time.  Every address below is a lane term plus a compile-time
// constant, so a tile costs one or two base registers however many columns
// are read.
//
// Pad<RL>: rows padded by 8 elements (16 bytes, one bank quad): reads of one
// 16-byte column over 16 consecutive rows are conflict-free, transposed reads
// of 4 consecutive rows collide up to 4-way.
template <int RL>
struct Pad {
    static constexpr int ld = RL + 8;
    static __device__ __forceinline__ int at(int r, int c) { return r * ld + c; }
};

// PadI<RL>: Pad with the rows of every aligned 16-row block permuted:
// logical row 16b + x is stored at physical row 16b + rev(x), rev reversing
// the four bits of x.  Four consecutive logical rows from a multiple of 4 (one
// transposed read, in the natural order or in an accumulator's k order) then
// sit 4 or 8 physical rows apart, on four disjoint bank groups, so every
// transposed read is conflict-free; 16 consecutive aligned rows are one
// permuted block (conflict-free 16-row reads); two adjacent rows of a 64-wide
// tile are 8 physical rows apart (conflict-free row writes); and the physical
// row is a constant plus a lane term, so addresses stay additive.  Tiles with
// this layout have a multiple of 16 rows.
template <int RL>
struct PadI {
    static constexpr int ld = RL + 8;
    static __device__ __forceinline__ int at(int r, int c) {
        const int rev = ((r & 1) << 3) | ((r & 2) << 1) | ((r & 4) >> 1) | ((r & 8) >> 3);
        return ((r & ~15) | rev) * ld + c;
    }
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}

// Operand in the permuted k order of an accumulator: elements (r, c .. c+3)
// and (r, c+8 .. c+11) of a tile with layout L (c a multiple of 4).
template <class L>
__device__ __forceinline__ bf16x8 ld4x2(const u16 *X, int r, int c) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(X + L::at(r, c));
    const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(X + L::at(r, c + 8));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 16-byte operand: elements (r, c .. c+7) of a tile with layout L (c a multiple of 8).
template <class L>
__device__ __forceinline__ bf16x8 ld8(const u16 *X, int r, int c) {
    return *reinterpret_cast<const bf16x8 *>(X + L::at(r, c));
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

// acc + sum over s < S of mfma(lda(s), ldb(s)), in the order s = 0 .. S-1,
// with the LDS reads of step s + AHEAD issued right after the product of step
// s.  Left to itself the scheduler sinks each read next to its product (it
// saves registers), and the chain then waits for a whole LDS round trip every
// product or two; the scheduling fences keep the reads ahead.
template <int S, int AHEAD, class FA, class FB>
__device__ __forceinline__ f32x16 mfma_chain(FA lda, FB ldb, f32x16 acc) {
    constexpr int P = AHEAD < S ? AHEAD : S;
    bf16x8 ra[P], rb[P];
#pragma unroll
    for (int s = 0; s < P; ++s) {
        ra[s] = lda(s);
        rb[s] = ldb(s);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < S; ++s) {
        acc = mfma(ra[s % P], rb[s % P], acc);
        if (s + P < S) {
            ra[s % P] = lda(s + P);
            rb[s % P] = ldb(s + P);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
}

__device__ __forceinline__ bf16x8 ones8() {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)1.0f;
    return o;
}

// Two floats rounded to bf16 (nearest even) and packed low, high into one
// word: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pk2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// Eight floats as a bf16 operand, converted in pairs (four v_cvt_pk_bf16_f32;
// element-wise casts make the compiler convert one element per instruction
// and merge the halves with permutes).
__device__ __forceinline__ bf16x8 pack8(float x0, float x1, float x2, float x3, float x4,
                                        float x5, float x6, float x7) {
    const uint4 u = make_uint4(pk2(x0, x1), pk2(x2, x3), pk2(x4, x5), pk2(x6, x7));
    return __builtin_bit_cast(bf16x8, u);
}

// Registers 8s .. 8s+7 of an accumulator as a bf16 operand (round to nearest
// even).  acc_op leaves the conversion to the compiler (which may convert one
// element per instruction but keeps fewer registers live); acc_pk converts in
// pairs (four instructions), for kernels that have the registers.
__device__ __forceinline__ bf16x8 acc_op(const f32x16 &acc, int s) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)acc[8 * s + e];
    return o;
}

__device__ __forceinline__ bf16x8 acc_pk(const f32x16 &acc, int s) {
    const int b = 8 * s;
    return pack8(acc[b], acc[b + 1], acc[b + 2], acc[b + 3], acc[b + 4], acc[b + 5], acc[b + 6],
                 acc[b + 7]);
}

// The rounding remainders of acc_op: x - bf16(x) for registers 8s .. 8s+7,
// rounded to bf16.  acc_op + acc_lo carry an fp32 accumulator to about 2^-16
// relative, for products whose results are small differences.
__device__ __forceinline__ bf16x8 acc_lo(const f32x16 &acc, int s) {
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = acc[8 * s + e];
        r[e] = x - (float)(__bf16)x;
    }
    return pack8(r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7]);
}

// phi for values that are rounded to bf16 right after: the hardware exp
// (v_exp_f32 of x log2(e), a few ulp) is far below bf16 resolution.  elu+1 is
// taken as max(x + 1, 2^(-|x| log2 e)): for x > 0 the exponential is
// e^-x < 1 < x + 1; for x <= 0 it is e^x >= 1 + x, so the maximum is e^x
// except where the two agree to a few float32 ulp (|x| below about 2^-10),
// far below bf16 resolution.  Four instructions instead of the six of the
// branch form (the sign goes in as a source modifier; no compare or select).
template <int PHI>
__device__ __forceinline__ float phi_fast(float x) {
    if constexpr (PHI == kElu1)
        return __builtin_fmaxf(x + 1.f, __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * 1.44269504088896341f));
    else return phi_f<PHI>(x);
}

// 1 / x by the hardware reciprocal (1 ulp); the quotients it feeds are
// rounded to bf16 or scale bf16 operands.
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Cross-lane sums in registers.  A shuffle through the LDS crossbar
// (ds_bpermute) costs a round trip and a wait per step; these use the
// permute paths of the vector ALU instead.
//
// x + (x of lane ^ 32): the wave's halves swapped by v_permlane32_swap.
// Both lanes of a pair add the same two values, so they get the same bits.
__device__ __forceinline__ float sum_halves(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(p[0]) + __int_as_float(p[1]);
}

// Sum over each group of G consecutive lanes (G = 8 or 16, groups aligned),
// with DPP: pairs, quads, then the mirrored halves of each 8- and 16-lane
// row.  Every lane of a group ends with the same bits (each step adds the
// same two values in both lanes it pairs).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G == 8 || G == 16, "DPP rows hold 16 lanes");
    x = dpp_add<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
    x = dpp_add<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
    x = dpp_add<0x141>(x);   // row_half_mirror: lane i <-> 7 - i within 8 lanes
    if constexpr (G == 16) x = dpp_add<0x140>(x);   // row_mirror: i <-> 15 - i
    return x;
}

__device__ __forceinline__ float bf2f(u16 x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ u16 f2bf(float x) {
    const __bf16 b = (__bf16)x;
    return __builtin_bit_cast(u16, b);
}

// phi'(x) from the bf16 feature p = phi(x) of a bf16 input x.  relu: p > 0
// exactly when x > 0; elu+1: p = x + 1 >= 1 for x > 0 and p = exp(x) <= 1
// otherwise, so phi' = min(p, 1) (exp(x) to bf16 precision); identity: 1.
template <int PHI>
__device__ __forceinline__ float phi_d_feat(float p) {
    if constexpr (PHI == kElu1) return __builtin_amdgcn_fmed3f(p, 0.f, 1.f);   // p >= 0: min(p, 1)
    else if constexpr (PHI == kRelu) return p > 0.f ? 1.f : 0.f;
    else return 1.f;
}

// Rows [c0, c0 + C) of one head's [N][D] bf16 tensor held in registers as
// 16-byte vectors (rows >= N read as zeros), so the global loads of the next
// chunk can be in flight while the current one is computed.  Vector k of
// thread t is element-row (t + k*NT) / (D/8), columns 8*((t + k*NT) % (D/8)).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global load / store; STREAM marks data read or written once
// (non-temporal: the caches keep it at low priority, so it does not push out
// data that will be read again).
template <bool STREAM>
__device__ __forceinline__ uint4 gld16(const u16 *p) {
    if constexpr (STREAM)
        return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
    else return *reinterpret_cast<const uint4 *>(p);
}
template <bool STREAM>
__device__ __forceinline__ void gst16(u16 *p, uint4 x) {
    if constexpr (STREAM)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x), reinterpret_cast<u32x4 *>(p));
    else *reinterpret_cast<uint4 *>(p) = x;
}

template <int D, int NT, int C = kC, bool FAST = false, bool STREAM = false>
struct RawTile {
    static constexpr int V8 = D / 8;
    static constexpr int NV = C * V8 / NT;
    static_assert(NV * NT == C * V8, "tile must split evenly over the threads");
    uint4 v[NV];
    // cos/sin weights of the rows of the vectors (cos/sin staging only), read
    // with the rows so that the staging does not wait for them
    float wc[NV], ws[NV];

    // FAST (for kernels with registers to spare), a whole tile in range: one
    // 16-byte load per vector at a uniform base plus this thread's constant
    // 32-bit offset (scalar base, no 64-bit address arithmetic per load).
    // Otherwise: loads from clamped (in-range) rows, rows >= N then zeroed
    // (N >= 1).
    __device__ __forceinline__ void load(const u16 *src, int c0, int N) {
        if (FAST && c0 + C <= N) {
            // vector k of thread t sits k * (NT / V8) rows below vector 0: the
            // row step goes into the uniform base, the thread term is one
            // 32-bit offset for every k
            const unsigned toff = (threadIdx.x / V8) * D + (threadIdx.x % V8) * 8;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const u16 *base = src + ((size_t)c0 + (size_t)k * (NT / V8)) * D;
                v[k] = gld16<STREAM>(base + toff);
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = threadIdx.x + k * NT, r = idx / V8, c8 = (idx % V8) * 8;
            v[k] = *reinterpret_cast<const uint4 *>(src + (size_t)min(c0 + r, N - 1) * D + c8);
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int r = (threadIdx.x + k * NT) / V8;
            if (c0 + r >= N) v[k] = make_uint4(0, 0, 0, 0);
        }
    }

    // the rows as load(), and with W their cos/sin weights (clamped to an
    // in-range row like the rows themselves)
    template <bool W>
    __device__ __forceinline__ void load(const u16 *src, int c0, int N, const float *cw, const float *sw) {
        load(src, c0, N);
        if constexpr (W) load_w(cw, sw, c0, N);
    }
    // the weights alone (a tile reloaded with other heads' rows at the same
    // positions keeps them)
    __device__ __forceinline__ void load_w(const float *cw, const float *sw, int c0, int N) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int t = min(c0 + (int)(threadIdx.x + k * NT) / V8, N - 1);
            wc[k] = cw[t];
            ws[k] = sw[t];
        }
    }

    template <class L>
    __device__ __forceinline__ void store(u16 *dst) const {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = threadIdx.x + k * NT, r = idx / V8, c8 = (idx % V8) * 8;
            *reinterpret_cast<uint4 *>(dst + L::at(r, c8)) = v[k];
        }
    }

    // Features: phi, then with COS [cos_t phi, sin_t phi] (row width 2D, the
    // weights those load<true> read), rounded to bf16.  With QZ, also sQZ[r] = Phi(x_r) . z (features before
    // rounding, fp32; fixed-order register reduction across the V8 threads of
    // a row).  With a layout LP, also phi itself (unweighted, bf16, row width
    // D) into dphi, for phi' in a backward.  Branch-free per element: rows
    // >= N hold zeros (load) and phi of them is finite; only a ragged tile
    // (uniform test) multiplies them by a 0/1 row factor.
    template <int PHI, bool COS, class L, bool QZ, class LP = void>
    __device__ __forceinline__ void store_feat(u16 *dst, int c0, int N, const float *sz, float *sQZ,
                                               u16 *dphi = nullptr) const {
        const bool ragged = c0 + C > N;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = threadIdx.x + k * NT, r = idx / V8, c8 = (idx % V8) * 8, t = c0 + r;
            const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = phi_fast<PHI>(__uint_as_float(w4[e] << 16));
                f[2 * e + 1] = phi_fast<PHI>(__uint_as_float(w4[e] & 0xffff0000u));
            }
            if (ragged) {
                const float vf = t < N ? 1.f : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] *= vf;
            }
            const float m0 = COS ? wc[k] : 1.f;
            uint32_t o[4];
            if constexpr (!std::is_void_v<LP>) {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = pk2(f[2 * e], f[2 * e + 1]);
                *reinterpret_cast<uint4 *>(dphi + LP::at(r, c8)) = make_uint4(o[0], o[1], o[2], o[3]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = COS ? pk2(m0 * f[2 * e], m0 * f[2 * e + 1]) : pk2(f[2 * e], f[2 * e + 1]);
            *reinterpret_cast<uint4 *>(dst + L::at(r, c8)) = make_uint4(o[0], o[1], o[2], o[3]);
            float qz = 0.f;
            if constexpr (QZ) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d += f[e] * sz[c8 + e];
                qz = m0 * d;
            }
            if constexpr (COS) {
                const float m1 = ws[k];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = pk2(m1 * f[2 * e], m1 * f[2 * e + 1]);
                *reinterpret_cast<uint4 *>(dst + L::at(r, D + c8)) = make_uint4(o[0], o[1], o[2], o[3]);
                if constexpr (QZ) {
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) d += f[e] * sz[D + c8 + e];
                    qz += m1 * d;
                }
            }
            if constexpr (QZ) {
                qz = group_sum<V8>(qz);
                if (idx % V8 == 0) sQZ[r] = qz;
            }
        }
    }
};

// Lane address for a transposed 4-row read of tile X: rows k0 .. k0+3, this
// lane's operand index (lane % 32) mapped to columns col0 .. col0+31
// (col0 a multiple of 32).
template <class L>
__device__ __forceinline__ const u16 *tr_addr(const u16 *X, int k0, int col0) {
    const int l = threadIdx.x & 63, gi = l >> 4, i16 = l & 15;
    return X + L::at(k0 + (i16 >> 2), col0 + 16 * (gi & 1) + 4 * (i16 & 3));
}

// Output rows go through LDS so global stores are whole rows, 16 bytes per
// lane, instead of 8-byte pieces spread over 32 rows per instruction.
// stage_out: this lane's accumulator values for row `lane % 32` and columns
// col0 + 8q + 4h + 0..3 (q = 0..3), scaled by `scale`, into the 32-row tile sO.
template <class L>
__device__ __forceinline__ void stage_out(u16 *sO, const f32x16 &acc, float scale, int col0) {
    const int l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t lo = pk2(acc[4 * q4] * scale, acc[4 * q4 + 1] * scale);
        const uint32_t hi = pk2(acc[4 * q4 + 2] * scale, acc[4 * q4 + 3] * scale);
        *reinterpret_cast<uint2 *>(sO + L::at(l32, col0 + 8 * q4 + 4 * h)) = make_uint2(lo, hi);
    }
}

// store_rows: rows 0..31 of the tile sO (row r -> global row c0 + r of a
// [N][D] tensor, rows >= N skipped; layout L), NT threads storing 16-byte pieces.  Call
// after a barrier that follows the stage_out of every wave.
// FAST (kernels with registers to spare): the pieces of a thread sit at a
// uniform base plus one 32-bit offset (as in RawTile::load); otherwise a lean
// loop.
template <int D, int NT, class L, bool FAST = false, bool STREAM = false>
__device__ __forceinline__ void store_rows(u16 *dst, const u16 *sO, int c0, int N) {
    constexpr int V8 = D / 8, NV = 32 * V8 / NT;
    static_assert(NV * NT == 32 * V8, "rows split evenly over the threads");
    if constexpr (FAST) {
        const unsigned t = threadIdx.x, toff = (t / V8) * D + (t % V8) * 8;
        const bool whole = c0 + 32 <= N;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int r = (int)(t / V8) + k * (NT / V8);
            const uint4 x = *reinterpret_cast<const uint4 *>(sO + L::at(r, (t % V8) * 8));
            u16 *base = dst + ((size_t)c0 + (size_t)k * (NT / V8)) * D;   // uniform
            if (whole || c0 + r < N) gst16<STREAM>(base + toff, x);
        }
    } else {
        for (int v = threadIdx.x; v < 32 * V8; v += NT) {
            const int r = v / V8, c8 = (v % V8) * 8;
            if (c0 + r < N)
                *reinterpret_cast<uint4 *>(dst + (size_t)(c0 + r) * D + c8) =
                    *reinterpret_cast<const uint4 *>(sO + L::at(r, c8));
        }
    }
}

// Accumulator helpers shared by the backward kernels.

// 4 consecutive bf16 of an LDS row as floats.
__device__ __forceinline__ void ld4f(const u16 *p, float *o) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    o[0] = __uint_as_float(u.x << 16);
    o[1] = __uint_as_float(u.x & 0xffff0000u);
    o[2] = __uint_as_float(u.y << 16);
    o[3] = __uint_as_float(u.y & 0xffff0000u);
}

__device__ __forceinline__ void st4bf(u16 *p, const float *x) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pk2(x[0], x[1]), pk2(x[2], x[3]));
}

// An accumulator tile through LDS in its register layout: register 4q + e of
// lane l at float (64q + l) * 4 + e, so each 16-byte access of a wave is
// contiguous.
__device__ __forceinline__ void put_acc(float *dst, const f32x16 &x) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4 *>(dst + (64 * q + l) * 4) = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
}

__device__ __forceinline__ f32x16 get_acc(const float *src) {
    const int l = threadIdx.x & 63;
    f32x16 x;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4 *>(src + (64 * q + l) * 4);
        x[4 * q] = v.x;
        x[4 * q + 1] = v.y;
        x[4 * q + 2] = v.z;
        x[4 * q + 3] = v.w;
    }
    return x;
}

// Accumulator row index of register r for lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// The causal mask of a 32x32 accumulator tile whose row index is the key j
// (accumulator row) and whose column is the query i (lane % 32), applied to
// its bf16 operands: word p of acc_op(T, s) holds registers 8s + 2p and
// 8s + 2p + 1, i.e. rows j0 = acc_row(8s + 2p, h) and j0 + 1, and is and-ed
// with a per-lane constant that keeps a half where j <= i.  The same bits as
// zeroing the masked floats before rounding (a zero rounds to +0), in one
// instruction per pair instead of a conversion, a select and a permute per
// element.
struct CausalMaskT {
    uint32_t w[8];
    __device__ __forceinline__ CausalMaskT(int l32, int h) {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int j0 = acc_row(2 * p, h);
            w[p] = j0 + 1 <= l32 ? 0xffffffffu : (j0 <= l32 ? 0x0000ffffu : 0u);
        }
    }
    // acc_op(T, s) with the mask applied
    __device__ __forceinline__ bf16x8 op(const f32x16 &T, int s) const {
        const int b = 8 * s;
        const uint4 u = make_uint4(pk2(T[b], T[b + 1]) & w[4 * s], pk2(T[b + 2], T[b + 3]) & w[4 * s + 1],
                                   pk2(T[b + 4], T[b + 5]) & w[4 * s + 2],
                                   pk2(T[b + 6], T[b + 7]) & w[4 * s + 3]);
        return __builtin_bit_cast(bf16x8, u);
    }
};

}  // namespace mf
}  // namespace la
