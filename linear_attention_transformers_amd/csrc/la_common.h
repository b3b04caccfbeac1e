// la_common.h -- shared definitions of the linear-attention HIP library:
// storage-type loads/stores, the feature maps, the launch plan and the
// workspace layout.  Included by every kernel translation unit and by the
// C-ABI front end.
//
// Feature maps (SVD_linear_Attention, "Module
// neuralops.core.triton_kernels.linear_attn", module docstring): elu+1
// (alpha = 1), relu, identity.  The cos/sin modulation of the same docstring
// multiplies phi(x_t) by cos_w[t] and by sin_w[t], giving a feature vector of
// width F = 2D whose halves are the two branches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace la {

enum Phi : int { kElu1 = 0, kRelu = 1, kIdentity = 2 };

// bfloat16 storage as raw 16-bit words.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);

template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

// float32 -> bfloat16, round to nearest even; NaN stays a quiet NaN.
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    uint32_t u = __float_as_uint(x);
    bf16_t r;
    if ((u & 0x7fffffffu) > 0x7f800000u) {
        r.bits = static_cast<uint16_t>((u >> 16) | 0x40u);
        return r;
    }
    u += 0x7fffu + ((u >> 16) & 1u);
    r.bits = static_cast<uint16_t>(u >> 16);
    return r;
}

template <int PHI>
__device__ __forceinline__ float phi_f(float x) {
    if constexpr (PHI == kElu1) return x > 0.f ? x + 1.f : expf(x);
    else if constexpr (PHI == kRelu) return x > 0.f ? x : 0.f;
    else return x;
}

// Derivative; relu'(0) = 0 and both sides of elu+1 give 1 at 0.
template <int PHI>
__device__ __forceinline__ float phi_d(float x) {
    if constexpr (PHI == kElu1) return x > 0.f ? 1.f : expf(x);
    else if constexpr (PHI == kRelu) return x > 0.f ? 1.f : 0.f;
    else return 1.f;
}

// Everything a kernel needs, passed by value.
struct Args {
    const void *q, *k, *v, *g;     // inputs (g = grad_out, backward only)
    void *out, *dq, *dk, *dv;      // outputs
    const float *cw, *sw;          // [N] position weights or nullptr
    float *ws_S;    // [B*Hkv][nseg+1][SD]: per-segment (S, z), then prefix/total
    float *ws_Rp;   // [B*H][nseg][SD]:     per-head, per-segment (R, r) partials
    float *ws_Rs;   // [B*Hkv][nseg+1][SD]: suffix (causal) / total (bidir) of (R, r)
    float *ws_den;  // [B*H][N] denominators (causal backward)
    float *ws_c;    // [B*H][N] c_i = (g_i . out_i) / den_i (causal backward)
    int B, H, Hkv, N, D, F, nrep;
    int L;          // segment length in rows (multiple of every chunk length)
    int nseg;
    float eps;
    int state_ready;  // backward: ws_S already holds the forward's prefix / total records
};

// ---------------------------------------------------------------------------
// Launch plan and workspace layout (host and device agree on these).
// ---------------------------------------------------------------------------
struct Plan {
    int F;          // feature width (D or 2D)
    int L;          // segment length
    int nseg;       // number of segments
    size_t SD;      // floats per state record: F*D + F
    size_t off_S, off_Rp, off_Rs, off_den, off_c, bytes;
};

constexpr int kSegAlign = 64;   // every chunk length divides this

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workgroups of kernel f (nt threads each) the current device holds at once,
// or 0 if the runtime cannot say.
template <class K>
int device_slots(K f, int nt) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, f, nt, 0) != hipSuccess || cus <= 0 || per <= 0)
        return 0;
    return cus * per;
}

// Segments per workgroup for a kernel whose workgroups walk consecutive
// segments: a round of workgroups (as many as the device holds at once)
// costs about the same whether they are short or long, so the qm that
// minimises rounds x segments per workgroup, the larger on ties.  slots1 and
// slotsm: workgroups per round of the build run for qm = 1 and for qm > 1.
inline int segments_by_rounds(int nseg, long long n_units, long long slots1, long long slotsm) {
    if (slots1 <= 0 || slotsm <= 0) return 1;
    int best = 1;
    long long best_t = -1;
    for (int m = 1; m <= nseg; ++m) {
        const long long wgs = n_units * ((nseg + m - 1) / m), slots = m == 1 ? slots1 : slotsm;
        const long long t = (wgs + slots - 1) / slots * m;
        if (best_t < 0 || t <= best_t) best = m, best_t = t;
    }
    return best;
}

// Segment count: about `target` workgroups over the `units` independent
// sequences (each workgroup runs one segment of one unit), but never segments
// shorter than min_L rows (by default 4 * kSegAlign: shorter, the state
// record would outweigh the rows).
inline Plan make_plan(int op_bwd, int B, int H, int Hkv, int N, int D, int causal,
                      int has_cos, int seg_len, long long units, long long target,
                      int min_L = 4 * kSegAlign) {
    Plan p{};
    p.F = has_cos ? 2 * D : D;
    p.SD = (size_t)p.F * D + p.F;
    int L;
    if (seg_len > 0) {
        L = (int)align_up((size_t)seg_len, kSegAlign);
    } else {
        long long nseg = (target + units - 1) / units;
        L = (int)align_up((size_t)((N + nseg - 1) / nseg), kSegAlign);
        if (L < min_L) L = min_L;
    }
    if (L > (int)align_up((size_t)N, kSegAlign)) L = (int)align_up((size_t)N, kSegAlign);
    p.L = L;
    p.nseg = (N + L - 1) / L;
    const size_t a = 256;
    size_t off = 0;
    p.off_S = off;
    off = align_up(off + sizeof(float) * (size_t)B * Hkv * (p.nseg + 1) * p.SD, a);
    p.off_Rp = p.off_Rs = p.off_den = p.off_c = off;
    if (op_bwd) {
        p.off_Rp = off;
        off = align_up(off + sizeof(float) * (size_t)B * H * p.nseg * p.SD, a);
        p.off_Rs = off;
        off = align_up(off + sizeof(float) * (size_t)B * Hkv * (p.nseg + 1) * p.SD, a);
        if (causal || has_cos) {   // the cos/sin R pass reads den and c in both modes
            p.off_den = off;
            off = align_up(off + sizeof(float) * (size_t)B * H * N, a);
            p.off_c = off;
            off = align_up(off + sizeof(float) * (size_t)B * H * N, a);
        }
    }
    p.bytes = off;
    return p;
}

}  // namespace la
