// la_gqa.hip -- grouped-query head expansion and its adjoint, for callers that
// need the expanded heads materialised (SVD_linear_Attention, "Module
// neuralops.core.triton_kernels.gqa"):
//   fwd: out[b, h] = in[b, h / n_rep]            (h = g n_rep + r, n_rep = H / H_kv)
//   bwd: out[b, g] = sum_{r < n_rep} in[b, g n_rep + r]
// The page views the head axis as (H_kv, n_rep) with n_rep fastest, so each
// KV head is repeated n_rep times in place (repeat-interleave, not tiling),
// and the backward sums over that n_rep axis.
//
// Both are HBM streams with no reuse.  Each (batch, head) slab of N*D
// elements is contiguous, and expanded head b*H + g*n_rep + r is slab
// (b*H_kv + g)*n_rep + r, so a block streams 16-byte units of one KV slab:
// the expansion reads a unit once and writes it to the n_rep heads, the sum
// reads the n_rep units and writes one.  The sum accumulates in float64 in
// head order and rounds once to the storage type (bf16: float64 -> float32
// rounding to odd, then float32 -> bf16 to nearest even, which equals a single
// rounding of the float64 value).  A float64 sum of n_rep bf16 or float32
// values is exact while their binary exponents span fewer than
// 29 - log2(n_rep) bits, so the stored result is the exact sum rounded once.
// Slabs whose size or base is not a multiple of 16 bytes take element-wise
// instances of the same kernels.
#include "la_common.h"
#include "la_kernels.h"
#include "la_timing.h"

namespace la {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 4;   // units per thread and source slab (64 bytes in flight)
constexpr long long kUnitsPerBlock = (long long)kThreads * kPerThread;

// grid: x = unit block within the slab, y = b * H_kv + g, z = tensor (0: k, 1: v).
// The four units of a thread live in named registers: a private array indexed
// inside the runtime head loop would be placed in LDS by the compiler.
// Outputs are stored non-temporally: ordinary stores leave the expansion's
// n_rep-fold output dirty in the caches, and the next kernel pays for its
// write-back (expand + reduce: 0.47 ms per step this way, 0.51 ms otherwise).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <bool STREAM, class U>
__device__ __forceinline__ void put(U *__restrict__ dst, long long i, long long slab, const U &x) {
    if (i < slab) {
        if constexpr (!STREAM) {
            dst[i] = x;
        } else if constexpr (sizeof(U) == 16) {
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x), reinterpret_cast<u32x4 *>(dst + i));
        } else {
            __builtin_nontemporal_store(x, dst + i);
        }
    }
}
template <class U>
__global__ __launch_bounds__(kThreads) void k_gqa_expand(const U *__restrict__ k, const U *__restrict__ v,
                                                         U *__restrict__ ko, U *__restrict__ vo,
                                                         long long slab, int nrep) {
    static_assert(kPerThread == 4, "four named units per thread");
    const U *src = (blockIdx.z ? v : k) + (long long)blockIdx.y * slab;
    U *dst = (blockIdx.z ? vo : ko) + (long long)blockIdx.y * nrep * slab;
    const long long i0 = (long long)blockIdx.x * kUnitsPerBlock + threadIdx.x;
    const long long i1 = i0 + kThreads, i2 = i0 + 2 * kThreads, i3 = i0 + 3 * kThreads;
    U x0{}, x1{}, x2{}, x3{};
    if (i0 < slab) x0 = src[i0];
    if (i1 < slab) x1 = src[i1];
    if (i2 < slab) x2 = src[i2];
    if (i3 < slab) x3 = src[i3];
    for (int r = 0; r < nrep; ++r) {
        U *d = dst + (long long)r * slab;
        put<true>(d, i0, slab, x0);
        put<true>(d, i1, slab, x1);
        put<true>(d, i2, slab, x2);
        put<true>(d, i3, slab, x3);
    }
}

// Storage units widened to float64 values and back.
template <bool BF16, class U> struct Lanes;
template <> struct Lanes<true, uint4> {
    static constexpr int n = 8;
    __device__ static void widen(const uint4 &u, double *x) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = (double)__uint_as_float(w[e] << 16);
            x[2 * e + 1] = (double)__uint_as_float(w[e] & 0xffff0000u);
        }
    }
    __device__ static uint4 narrow(const double *x);
};
template <> struct Lanes<true, uint16_t> {
    static constexpr int n = 1;
    __device__ static void widen(const uint16_t &u, double *x) { x[0] = (double)__uint_as_float((uint32_t)u << 16); }
    __device__ static uint16_t narrow(const double *x);
};
template <> struct Lanes<false, uint4> {
    static constexpr int n = 4;
    __device__ static void widen(const uint4 &u, double *x) {
        x[0] = (double)__uint_as_float(u.x);
        x[1] = (double)__uint_as_float(u.y);
        x[2] = (double)__uint_as_float(u.z);
        x[3] = (double)__uint_as_float(u.w);
    }
    __device__ static uint4 narrow(const double *x) {
        return make_uint4(__float_as_uint((float)x[0]), __float_as_uint((float)x[1]),
                          __float_as_uint((float)x[2]), __float_as_uint((float)x[3]));
    }
};
template <> struct Lanes<false, uint32_t> {
    static constexpr int n = 1;
    __device__ static void widen(const uint32_t &u, double *x) { x[0] = (double)__uint_as_float(u); }
    __device__ static uint32_t narrow(const double *x) { return __float_as_uint((float)x[0]); }
};

// float64 -> bf16 bits, one rounding to nearest even: round to odd into
// float32 (truncate, then force the last bit if anything was cut off), then
// round to nearest even into bf16.  float32 keeps 16 more significand bits
// than bf16, so the odd sticky bit decides every tie the way the float64
// value would.
__device__ __forceinline__ uint32_t bf16_bits(double x) {
    float f = __double2float_rz(x);
    if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ uint4 Lanes<true, uint4>::narrow(const double *x) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = bf16_bits(x[2 * e]) | (bf16_bits(x[2 * e + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ uint16_t Lanes<true, uint16_t>::narrow(const double *x) { return (uint16_t)bf16_bits(x[0]); }

// grid: x = unit block within the slab, y = b * H_kv + g, z = tensor.  The
// n_rep source units of a thread's outputs are loaded in batches of kRB (all
// loads of a batch in flight together), then added in head order.  Four
// outputs per thread: 0.240 ms per reduce at B=1, H=32, H_kv=8, N=65536,
// D=128, against 0.269 with one, 0.251 with two and 0.347 with eight (whose
// 256 registers per lane leave one wave per SIMD).
constexpr int kRB = 4;
constexpr int kPerThreadR = 4;
constexpr long long kUnitsPerBlockR = (long long)kThreads * kPerThreadR;
template <bool BF16, class U>
__global__ __launch_bounds__(kThreads) void k_gqa_reduce(const U *__restrict__ gk, const U *__restrict__ gv,
                                                         U *__restrict__ ko, U *__restrict__ vo,
                                                         long long slab, int nrep) {
    using Ln = Lanes<BF16, U>;
    const U *src = (blockIdx.z ? gv : gk) + (long long)blockIdx.y * nrep * slab;
    U *dst = (blockIdx.z ? vo : ko) + (long long)blockIdx.y * slab;
    const long long i0 = (long long)blockIdx.x * kUnitsPerBlockR + threadIdx.x;
    double acc[kPerThreadR][Ln::n];
    for (int r0 = 0; r0 < nrep; r0 += kRB) {
        U x[kRB][kPerThreadR];
#pragma unroll
        for (int rr = 0; rr < kRB; ++rr)
#pragma unroll
            for (int j = 0; j < kPerThreadR; ++j) {
                const long long i = i0 + (long long)j * kThreads;
                if (r0 + rr < nrep && i < slab) x[rr][j] = src[(long long)(r0 + rr) * slab + i];
            }
#pragma unroll
        for (int rr = 0; rr < kRB; ++rr)
#pragma unroll
            for (int j = 0; j < kPerThreadR; ++j) {
                if (r0 + rr >= nrep) continue;
                double t[Ln::n];
                Ln::widen(x[rr][j], t);
#pragma unroll
                for (int e = 0; e < Ln::n; ++e) acc[j][e] = r0 + rr == 0 ? t[e] : acc[j][e] + t[e];
            }
    }
#pragma unroll
    for (int j = 0; j < kPerThreadR; ++j) {
        const long long i = i0 + (long long)j * kThreads;
        put<true>(dst, i, slab, Ln::narrow(acc[j]));
    }
}

bool vec_ok(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % 16) == 0; }

template <class U>
hipError_t launch_expand(const void *k, const void *v, void *ko, void *vo, int B, int Hkv, int nrep,
                         long long slab_bytes, hipStream_t s) {
    const long long slab = slab_bytes / (long long)sizeof(U);
    const dim3 grid((unsigned)((slab + kUnitsPerBlock - 1) / kUnitsPerBlock), (unsigned)(B * Hkv),
                    v ? 2u : 1u);
    TimedLaunch tl("k_gqa_expand", s);
    hipLaunchKernelGGL(k_gqa_expand<U>, grid, dim3(kThreads), 0, s, static_cast<const U *>(k),
                       static_cast<const U *>(v), static_cast<U *>(ko), static_cast<U *>(vo), slab, nrep);
    return hipGetLastError();
}

template <bool BF16, class U>
hipError_t launch_reduce(const void *gk, const void *gv, void *ko, void *vo, int B, int Hkv, int nrep,
                         long long slab_bytes, hipStream_t s) {
    const long long slab = slab_bytes / (long long)sizeof(U);
    const dim3 grid((unsigned)((slab + kUnitsPerBlockR - 1) / kUnitsPerBlockR), (unsigned)(B * Hkv),
                    gv ? 2u : 1u);
    TimedLaunch tl("k_gqa_reduce", s);
    hipLaunchKernelGGL((k_gqa_reduce<BF16, U>), grid, dim3(kThreads), 0, s, static_cast<const U *>(gk),
                       static_cast<const U *>(gv), static_cast<U *>(ko), static_cast<U *>(vo), slab, nrep);
    return hipGetLastError();
}

}  // namespace

hipError_t gqa_expand_run(const void *k, const void *v, void *ko, void *vo, int B, int Hkv, int H,
                          long long slab_elems, int bf16, hipStream_t s) {
    const int nrep = H / Hkv;
    const long long bytes = slab_elems * (bf16 ? 2 : 4);
    if (bytes % 16 == 0 && vec_ok(k) && vec_ok(v) && vec_ok(ko) && vec_ok(vo))
        return launch_expand<uint4>(k, v, ko, vo, B, Hkv, nrep, bytes, s);
    return bf16 ? launch_expand<uint16_t>(k, v, ko, vo, B, Hkv, nrep, bytes, s)
                : launch_expand<uint32_t>(k, v, ko, vo, B, Hkv, nrep, bytes, s);
}

hipError_t gqa_reduce_run(const void *gk, const void *gv, void *ko, void *vo, int B, int Hkv, int H,
                          long long slab_elems, int bf16, hipStream_t s) {
    const int nrep = H / Hkv;
    const long long bytes = slab_elems * (bf16 ? 2 : 4);
    const bool vec = bytes % 16 == 0 && vec_ok(gk) && vec_ok(gv) && vec_ok(ko) && vec_ok(vo);
    if (bf16)
        return vec ? launch_reduce<true, uint4>(gk, gv, ko, vo, B, Hkv, nrep, bytes, s)
                   : launch_reduce<true, uint16_t>(gk, gv, ko, vo, B, Hkv, nrep, bytes, s);
    return vec ? launch_reduce<false, uint4>(gk, gv, ko, vo, B, Hkv, nrep, bytes, s)
               : launch_reduce<false, uint32_t>(gk, gv, ko, vo, B, Hkv, nrep, bytes, s);
}

}  // namespace la
