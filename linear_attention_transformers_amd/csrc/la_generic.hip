// la_generic.hip -- float32 vector-ALU kernels for every case the library
// serves (both storage types, D in {32, 64, 128}, causal or bidirectional,
// with or without cos/sin weights, any GQA ratio).  They are the float32
// path, and the path for the cases the bf16 matrix-core kernels do not take.
//
// Method (SVD_linear_Attention, "Module neuralops.core.triton_kernels.
// linear_attn", module docstring: chunked causal streaming with O(N) memory,
// bidirectional parallel reduction; function bwd: the gradient of fwd):
//   S_i = sum_{j in J(i)} Phi(k_j) v_j^T, z_i = sum_{j in J(i)} Phi(k_j),
//   out_i = Phi(q_i)^T S_i / (Phi(q_i) . z_i + eps).
// The sequence of every (batch, head) is cut into segments of L rows that run
// in parallel; a segment's starting state is the exclusive prefix (causal) or
// the total (bidirectional) of per-segment state sums (k_state + k_scan).
// Inside a segment rows are processed in chunks of C: causal rows combine the
// masked intra-chunk sum with the carried state.
//
// Backward (exact derivative of the forward), with gn_i = g_i / den_i and
// c_i = (g_i . out_i) / den_i:
//   dPhi(q_i) = S_i gn_i - c_i z_i,  dPhi(k_j) = R_j v_j - r_j,
//   dv_j = R_j^T Phi(k_j),  R_j = sum_{i : j in J(i)} Phi(q_i) gn_i^T,
//   r_j = sum_{i : j in J(i)} c_i Phi(q_i).
// In chunk form (causal) with A_ij = Phi(q_i).Phi(k_j), T_ij = g_i.v_j,
// U_i = S g_i (exclusive S), P_ij = T_ij / den_i - c_i, j <= i in the chunk:
//   den_i = sum_j A_ij + Phi(q_i).z + eps,
//   c_i   = (sum_j A_ij T_ij + Phi(q_i).U_i) / den_i^2,
//   dPhi(q_i) = sum_j P_ij Phi(k_j) + U_i / den_i - c_i z,
//   dPhi(k_j) = sum_i P_ij Phi(q_i) + R v_j - r,   dv_j = sum_i A_ij gn_i + R^T Phi(k_j)
// with (R, r) the exclusive suffix summed over the n_rep query heads of the
// KV head (gqa page, bwd: KV gradients are the sum over the n_rep heads).
#include "la_common.h"
#include "la_kernels.h"
#include "la_timing.h"

namespace la {
namespace {

constexpr int kNT = 256;

// Chunk lengths chosen so each kernel's LDS tiles stay within 64 KiB.
template <int F, int D> constexpr int chunk_fwd() { return F == 256 ? 16 : 32; }
template <int F, int D> constexpr int chunk_state() { return 32; }
template <int F, int D> constexpr int chunk_bwd_q() {
    return F == 256 ? 8 : (F == 128 ? 16 : 32);
}
template <int F, int D> constexpr int chunk_bwd_kv() {
    return F == 256 ? 8 : ((F == 128 || D == 64) ? 16 : 32);
}
template <int F> constexpr int nt_bwd() { return F == 256 ? 512 : 256; }

template <typename T>
__device__ __forceinline__ float ld(const T *p, size_t i) { return to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ void st(T *p, size_t i, float x) { p[i] = from_f32<T>(x); }

// Features Phi of rows [r0, r0 + C) of one head (rows >= N give zeros) into
// dst[C][F]; optionally the raw values into raw[C][D].
template <typename T, int D, int F, int PHI, int C, int NT>
__device__ void load_feat(float *dst, float *raw, const T *src, int r0, int N,
                          const float *cw, const float *sw) {
    for (int e = threadIdx.x; e < C * D; e += NT) {
        const int r = e / D, d = e % D, t = r0 + r;
        float x = 0.f;
        if (t < N) x = ld(src, (size_t)t * D + d);
        const float f = t < N ? phi_f<PHI>(x) : 0.f;
        if (raw) raw[r * D + d] = x;
        if constexpr (F == 2 * D) {
            const float c = t < N ? cw[t] : 0.f;
            const float s = t < N ? sw[t] : 0.f;
            dst[r * F + d] = c * f;
            dst[r * F + D + d] = s * f;
        } else {
            dst[r * F + d] = f;
        }
    }
}

// Plain rows [r0, r0 + C) as float (zeros past N) into dst[C][D].
template <typename T, int D, int C, int NT>
__device__ void load_rows(float *dst, const T *src, int r0, int N) {
    for (int e = threadIdx.x; e < C * D; e += NT) {
        const int r = e / D, t = r0 + r;
        dst[e] = t < N ? ld(src, (size_t)t * D + (e % D)) : 0.f;
    }
}

template <int P>
__device__ __forceinline__ float reduce_lanes(float x) {
#pragma unroll
    for (int o = 1; o < P; o <<= 1) x += __shfl_xor(x, o);
    return x;
}

// ---------------------------------------------------------------------------
// k_state: per (batch, KV head, segment) the sums dS = sum_j Phi(k_j) v_j^T
// and dz = sum_j Phi(k_j) over the segment's rows.
// Thread t owns column d = t / P and state rows f = r * P + p, p = t % P.
// ---------------------------------------------------------------------------
template <typename T, int D, int F, int PHI>
__global__ __launch_bounds__(kNT) void k_state(Args a) {
    constexpr int C = chunk_state<F, D>();
    constexpr int P = kNT / D, FS = F / P;
    __shared__ float Kf[C * F];
    __shared__ float Vs[C * D];
    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int t = threadIdx.x, d = t / P, p = t % P;
    const T *kh = static_cast<const T *>(a.k) + (size_t)bg * a.N * D;
    const T *vh = static_cast<const T *>(a.v) + (size_t)bg * a.N * D;
    float S[FS];
#pragma unroll
    for (int r = 0; r < FS; ++r) S[r] = 0.f;
    float z = 0.f;
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    for (int c0 = row0; c0 < row1; c0 += C) {
        load_feat<T, D, F, PHI, C, kNT>(Kf, nullptr, kh, c0, a.N, a.cw, a.sw);
        load_rows<T, D, C, kNT>(Vs, vh, c0, a.N);
        __syncthreads();
        #pragma unroll 2
        for (int j = 0; j < C; ++j) {
            const float vj = Vs[j * D + d];
#pragma unroll
            for (int r = 0; r < FS; ++r) S[r] += Kf[j * F + r * P + p] * vj;
        }
        if (t < F)
            for (int j = 0; j < C; ++j) z += Kf[j * F + t];
        __syncthreads();
    }
    float *out = a.ws_S + ((size_t)bg * (a.nseg + 1) + seg) * ((size_t)F * D + F);
#pragma unroll
    for (int r = 0; r < FS; ++r) out[(size_t)(r * P + p) * D + d] = S[r];
    if (t < F) out[(size_t)F * D + t] = z;
}

// ---------------------------------------------------------------------------
// k_scan_S: per (batch, KV head) and state element, over the per-segment
// sums in slots 0 .. nseg-1.  Causal: replace them by their exclusive prefix
// over segments (slot s = rows before segment s; the last segment's record is
// neither read nor needed).  Bidirectional: store their total in slot nseg
// and leave the per-segment slots as they are (only the total is read).
// Fixed order: deterministic.  The records of kScanB segments are loaded
// before any of their slots is written, so a thread waits for memory once
// per kScanB segments, not once per segment.
// ---------------------------------------------------------------------------
constexpr int kScanB = 8;

__global__ __launch_bounds__(kNT) void k_scan_S(float *ws, int nseg, size_t SD, size_t n_units, int causal) {
    const size_t e = (size_t)blockIdx.x * kNT + threadIdx.x;
    const size_t unit = blockIdx.y;
    if (e >= SD || unit >= n_units) return;
    float *base = ws + unit * (nseg + 1) * SD + e;
    const int nin = causal ? nseg - 1 : nseg;   // records that are summed
    float run = 0.f;
    for (int s0 = 0; s0 < nseg; s0 += kScanB) {
        float x[kScanB];
#pragma unroll
        for (int i = 0; i < kScanB; ++i) x[i] = s0 + i < nin ? base[(size_t)(s0 + i) * SD] : 0.f;
#pragma unroll
        for (int i = 0; i < kScanB; ++i) {
            if (s0 + i < nseg) {
                if (causal) base[(size_t)(s0 + i) * SD] = run;
                run += x[i];
            }
        }
    }
    if (!causal) base[(size_t)nseg * SD] = run;
}

// ---------------------------------------------------------------------------
// k_scan_R: per (batch, KV head), sum the per-head partials (R, r) of the
// n_rep query heads (order 0..n_rep-1).  Causal: the exclusive suffix over
// segments (slot s = rows after segment s).  Bidirectional: the total, in
// slot nseg only.  kScanB segments' records are loaded together, from
// clamped (existing) slots with no branch around the loads: under a branch
// each load was followed by its own wait.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kNT) void k_scan_R(const float *Rp, float *Rs, int nseg, size_t SD,
                                                int H, int Hkv, int nrep, size_t n_units, int causal) {
    const size_t e = (size_t)blockIdx.x * kNT + threadIdx.x;
    const size_t unit = blockIdx.y;  // b * Hkv + g
    if (e >= SD || unit >= n_units) return;
    const size_t b = unit / Hkv, g = unit % Hkv;
    float *out = Rs + unit * (nseg + 1) * SD + e;
    const float *in = Rp + (b * H + g * nrep) * nseg * SD + e;   // head r, segment s at (r nseg + s) SD
    float run = 0.f;
    // kScanB segments' partials summed over the heads (order 0 .. nrep-1)
    // before their slots are written (the output does not alias the input)
    for (int s0 = nseg - 1; s0 >= 0; s0 -= kScanB) {
        float x[kScanB];
#pragma unroll
        for (int i = 0; i < kScanB; ++i) x[i] = 0.f;
        for (int r = 0; r < nrep; ++r) {
            float y[kScanB];
#pragma unroll
            for (int i = 0; i < kScanB; ++i) y[i] = in[((size_t)r * nseg + max(s0 - i, 0)) * SD];
#pragma unroll
            for (int i = 0; i < kScanB; ++i) x[i] += s0 - i >= 0 ? y[i] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < kScanB; ++i) {
            if (s0 - i >= 0) {
                if (causal) out[(size_t)(s0 - i) * SD] = run;
                run += x[i];
            }
        }
    }
    if (!causal) out[(size_t)nseg * SD] = run;
}

// ---------------------------------------------------------------------------
// k_fwd_causal: per (batch, query head, segment).  State S in registers
// (column distribution as k_state), z in LDS.
// ---------------------------------------------------------------------------
template <typename T, int D, int F, int PHI>
__global__ __launch_bounds__(kNT) void k_fwd_causal(Args a) {
    constexpr int C = chunk_fwd<F, D>();
    constexpr int P = kNT / D, FS = F / P;
    __shared__ float Qf[C * F];
    __shared__ float Kf[C * F];
    __shared__ float Vs[C * D];
    __shared__ float As[C * C];
    __shared__ float zs[F];
    __shared__ float dn[C];
    const int seg = blockIdx.x % a.nseg, bh = blockIdx.x / a.nseg;
    const int b = bh / a.H, h = bh % a.H, g = h / a.nrep, bg = b * a.Hkv + g;
    const int t = threadIdx.x, d = t / P, p = t % P;
    const size_t SD = (size_t)F * D + F;
    const T *qh = static_cast<const T *>(a.q) + (size_t)bh * a.N * D;
    const T *kh = static_cast<const T *>(a.k) + (size_t)bg * a.N * D;
    const T *vh = static_cast<const T *>(a.v) + (size_t)bg * a.N * D;
    T *oh = static_cast<T *>(a.out) + (size_t)bh * a.N * D;
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + seg) * SD;
    float S[FS];
#pragma unroll
    for (int r = 0; r < FS; ++r) S[r] = Sp[(size_t)(r * P + p) * D + d];
    for (int f = t; f < F; f += kNT) zs[f] = Sp[(size_t)F * D + f];
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    for (int c0 = row0; c0 < row1; c0 += C) {
        load_feat<T, D, F, PHI, C, kNT>(Qf, nullptr, qh, c0, a.N, a.cw, a.sw);
        load_feat<T, D, F, PHI, C, kNT>(Kf, nullptr, kh, c0, a.N, a.cw, a.sw);
        load_rows<T, D, C, kNT>(Vs, vh, c0, a.N);
        __syncthreads();
        for (int e = t; e < C * C; e += kNT) {
            const int i = e / C, j = e % C;
            float acc = 0.f;
            if (j <= i)
                for (int f = 0; f < F; ++f) acc += Qf[i * F + f] * Kf[j * F + f];
            As[e] = acc;
        }
        __syncthreads();
        for (int i = t; i < C; i += kNT) {
            float qz = 0.f;
            for (int f = 0; f < F; ++f) qz += Qf[i * F + f] * zs[f];
            float sa = 0.f;
            for (int j = 0; j <= i; ++j) sa += As[i * C + j];
            dn[i] = sa + qz + a.eps;
        }
        __syncthreads();
        #pragma unroll 2
        for (int i = 0; i < C; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < FS; ++r) acc += Qf[i * F + r * P + p] * S[r];
            for (int j = p; j <= i; j += P) acc += As[i * C + j] * Vs[j * D + d];
            acc = reduce_lanes<P>(acc);
            if (p == (i % P) && c0 + i < a.N) st(oh, (size_t)(c0 + i) * D + d, acc / dn[i]);
        }
        #pragma unroll 2
        for (int j = 0; j < C; ++j) {
            const float vj = Vs[j * D + d];
#pragma unroll
            for (int r = 0; r < FS; ++r) S[r] += Kf[j * F + r * P + p] * vj;
        }
        __syncthreads();
        for (int f = t; f < F; f += kNT) {
            float acc = 0.f;
            for (int j = 0; j < C; ++j) acc += Kf[j * F + f];
            zs[f] += acc;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// k_fwd_bidir: per (batch, query head, segment): rows against the total state.
// ---------------------------------------------------------------------------
template <typename T, int D, int F, int PHI>
__global__ __launch_bounds__(kNT) void k_fwd_bidir(Args a) {
    constexpr int C = chunk_fwd<F, D>();
    constexpr int P = kNT / D, FS = F / P;
    __shared__ float Qf[C * F];
    __shared__ float zs[F];
    __shared__ float dn[C];
    const int seg = blockIdx.x % a.nseg, bh = blockIdx.x / a.nseg;
    const int b = bh / a.H, h = bh % a.H, g = h / a.nrep, bg = b * a.Hkv + g;
    const int t = threadIdx.x, d = t / P, p = t % P;
    const size_t SD = (size_t)F * D + F;
    const T *qh = static_cast<const T *>(a.q) + (size_t)bh * a.N * D;
    T *oh = static_cast<T *>(a.out) + (size_t)bh * a.N * D;
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + a.nseg) * SD;
    float S[FS];
#pragma unroll
    for (int r = 0; r < FS; ++r) S[r] = Sp[(size_t)(r * P + p) * D + d];
    for (int f = t; f < F; f += kNT) zs[f] = Sp[(size_t)F * D + f];
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    for (int c0 = row0; c0 < row1; c0 += C) {
        load_feat<T, D, F, PHI, C, kNT>(Qf, nullptr, qh, c0, a.N, a.cw, a.sw);
        __syncthreads();
        for (int i = t; i < C; i += kNT) {
            float qz = 0.f;
            for (int f = 0; f < F; ++f) qz += Qf[i * F + f] * zs[f];
            dn[i] = qz + a.eps;
        }
        __syncthreads();
        #pragma unroll 2
        for (int i = 0; i < C; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < FS; ++r) acc += Qf[i * F + r * P + p] * S[r];
            acc = reduce_lanes<P>(acc);
            if (p == (i % P) && c0 + i < a.N) st(oh, (size_t)(c0 + i) * D + d, acc / dn[i]);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// k_bwd_q_causal: per (batch, query head, segment), forward over chunks with
// the exclusive prefix state.  Writes dq, den, c and the segment's partial
// (R, r).  Thread t owns state row f = t / P2 and columns d = r * P2 + p2.
// ---------------------------------------------------------------------------
template <typename T, int D, int F, int PHI>
__global__ __launch_bounds__(nt_bwd<F>()) void k_bwd_q_causal(Args a) {
    constexpr int NT = nt_bwd<F>();
    constexpr int C = chunk_bwd_q<F, D>();
    constexpr int P2 = NT / F, DS = D / P2;
    __shared__ float Qf[C * F];
    __shared__ float Kf[C * F];
    __shared__ float Vs[C * D];
    __shared__ float Gs[C * D];
    __shared__ float Qr[C * D];
    __shared__ float As[C * C];
    __shared__ float Ts[C * C];
    __shared__ float Us[C * F];
    __shared__ float zs[F];
    __shared__ float dn[C];
    __shared__ float cc[C];
    const int seg = blockIdx.x % a.nseg, bh = blockIdx.x / a.nseg;
    const int b = bh / a.H, h = bh % a.H, g = h / a.nrep, bg = b * a.Hkv + g;
    const int t = threadIdx.x, f = t / P2, p2 = t % P2;
    const size_t SD = (size_t)F * D + F;
    const T *qh = static_cast<const T *>(a.q) + (size_t)bh * a.N * D;
    const T *gh = static_cast<const T *>(a.g) + (size_t)bh * a.N * D;
    const T *kh = static_cast<const T *>(a.k) + (size_t)bg * a.N * D;
    const T *vh = static_cast<const T *>(a.v) + (size_t)bg * a.N * D;
    T *dqh = static_cast<T *>(a.dq) + (size_t)bh * a.N * D;
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + seg) * SD;
    float S[DS], R[DS];
#pragma unroll
    for (int r = 0; r < DS; ++r) {
        S[r] = Sp[(size_t)f * D + r * P2 + p2];
        R[r] = 0.f;
    }
    float rr = 0.f;
    for (int e = t; e < F; e += NT) zs[e] = Sp[(size_t)F * D + e];
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    for (int c0 = row0; c0 < row1; c0 += C) {
        load_feat<T, D, F, PHI, C, NT>(Qf, Qr, qh, c0, a.N, a.cw, a.sw);
        load_feat<T, D, F, PHI, C, NT>(Kf, nullptr, kh, c0, a.N, a.cw, a.sw);
        load_rows<T, D, C, NT>(Vs, vh, c0, a.N);
        load_rows<T, D, C, NT>(Gs, gh, c0, a.N);
        __syncthreads();
        for (int e = t; e < C * C; e += NT) {
            const int i = e / C, j = e % C;
            float av = 0.f, tv = 0.f;
            if (j <= i) {
                for (int x = 0; x < F; ++x) av += Qf[i * F + x] * Kf[j * F + x];
                for (int x = 0; x < D; ++x) tv += Gs[i * D + x] * Vs[j * D + x];
            }
            As[e] = av;
            Ts[e] = tv;
        }
        for (int i = 0; i < C; ++i) {  // U_i = S g_i
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < DS; ++r) acc += S[r] * Gs[i * D + r * P2 + p2];
            acc = reduce_lanes<P2>(acc);
            if (p2 == 0) Us[i * F + f] = acc;
        }
        __syncthreads();
        for (int i = t; i < C; i += NT) {
            float qz = 0.f, qu = 0.f, sa = 0.f, at = 0.f;
            for (int x = 0; x < F; ++x) {
                qz += Qf[i * F + x] * zs[x];
                qu += Qf[i * F + x] * Us[i * F + x];
            }
            for (int j = 0; j <= i; ++j) {
                sa += As[i * C + j];
                at += As[i * C + j] * Ts[i * C + j];
            }
            const bool ok = c0 + i < a.N;   // rows past N: neutral values
            const float den = ok ? sa + qz + a.eps : 1.f;
            const float c = ok ? (at + qu) / (den * den) : 0.f;
            dn[i] = den;
            cc[i] = c;
            if (ok) {
                a.ws_den[(size_t)bh * a.N + c0 + i] = den;
                a.ws_c[(size_t)bh * a.N + c0 + i] = c;
            }
        }
        __syncthreads();
        for (int e = t; e < C * C; e += NT) {
            const int i = e / C, j = e % C;
            Ts[e] = j <= i ? Ts[e] / dn[i] - cc[i] : 0.f;
        }
        __syncthreads();
        for (int i = p2; i < C; i += P2) {  // dPhi(q_i)[f]
            float acc = Us[i * F + f] / dn[i] - cc[i] * zs[f];
            for (int j = 0; j <= i; ++j) acc += Ts[i * C + j] * Kf[j * F + f];
            Us[i * F + f] = acc;
        }
        __syncthreads();
        for (int e = t; e < C * D; e += NT) {
            const int i = e / D, x = e % D;
            if (c0 + i >= a.N) continue;
            float gphi;
            if constexpr (F == 2 * D)
                gphi = a.cw[c0 + i] * Us[i * F + x] + a.sw[c0 + i] * Us[i * F + D + x];
            else
                gphi = Us[i * F + x];
            st(dqh, (size_t)(c0 + i) * D + x, phi_d<PHI>(Qr[i * D + x]) * gphi);
        }
        #pragma unroll 2
        for (int i = 0; i < C; ++i) {
            const float qf = Qf[i * F + f], inv = 1.f / dn[i];
#pragma unroll
            for (int r = 0; r < DS; ++r) R[r] += qf * (Gs[i * D + r * P2 + p2] * inv);
            rr += cc[i] * qf;
        }
        #pragma unroll 2
        for (int j = 0; j < C; ++j) {
            const float kf = Kf[j * F + f];
#pragma unroll
            for (int r = 0; r < DS; ++r) S[r] += kf * Vs[j * D + r * P2 + p2];
        }
        __syncthreads();
        for (int e = t; e < F; e += NT) {
            float acc = 0.f;
            for (int j = 0; j < C; ++j) acc += Kf[j * F + e];
            zs[e] += acc;
        }
        __syncthreads();
    }
    float *Ro = a.ws_Rp + ((size_t)bh * a.nseg + seg) * SD;
#pragma unroll
    for (int r = 0; r < DS; ++r) Ro[(size_t)f * D + r * P2 + p2] = R[r];
    if (p2 == 0) Ro[(size_t)F * D + f] = rr;
}

// ---------------------------------------------------------------------------
// k_bwd_kv_causal: per (batch, KV head, segment), backward over chunks with
// the exclusive suffix (R, r) of the KV head.  R is held twice: by rows
// (thread (f, p2), for R v) and by columns (thread (d, p), for R^T Phi(k)).
// ---------------------------------------------------------------------------
template <typename T, int D, int F, int PHI>
__global__ __launch_bounds__(nt_bwd<F>()) void k_bwd_kv_causal(Args a) {
    constexpr int NT = nt_bwd<F>();
    constexpr int C = chunk_bwd_kv<F, D>();
    constexpr int P2 = NT / F, DS = D / P2;
    constexpr int P = NT / D, FS = F / P;
    __shared__ float Kf[C * F];
    __shared__ float Vs[C * D];
    __shared__ float Kr[C * D];
    __shared__ float dKs[C * F];
    __shared__ float dVs[C * D];
    __shared__ float Qf[C * F];
    __shared__ float Gs[C * D];
    __shared__ float As[C * C];
    __shared__ float Pm[C * C];
    __shared__ float dn[C];
    __shared__ float cc[C];
    __shared__ float rs[F];
    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int t = threadIdx.x, f = t / P2, p2 = t % P2, d = t / P, p = t % P;
    const size_t SD = (size_t)F * D + F;
    const T *kh = static_cast<const T *>(a.k) + (size_t)bg * a.N * D;
    const T *vh = static_cast<const T *>(a.v) + (size_t)bg * a.N * D;
    T *dkh = static_cast<T *>(a.dk) + (size_t)bg * a.N * D;
    T *dvh = static_cast<T *>(a.dv) + (size_t)bg * a.N * D;
    const float *Rp = a.ws_Rs + ((size_t)bg * (a.nseg + 1) + seg) * SD;
    float Rr[DS], Rc[FS];
#pragma unroll
    for (int r = 0; r < DS; ++r) Rr[r] = Rp[(size_t)f * D + r * P2 + p2];
#pragma unroll
    for (int r = 0; r < FS; ++r) Rc[r] = Rp[(size_t)(r * P + p) * D + d];
    for (int e = t; e < F; e += NT) rs[e] = Rp[(size_t)F * D + e];
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    const int nch = (row1 - row0 + C - 1) / C;
    for (int ci = nch - 1; ci >= 0; --ci) {
        const int c0 = row0 + ci * C;
        load_feat<T, D, F, PHI, C, NT>(Kf, Kr, kh, c0, a.N, a.cw, a.sw);
        load_rows<T, D, C, NT>(Vs, vh, c0, a.N);
        __syncthreads();
        #pragma unroll 2
        for (int j = 0; j < C; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < DS; ++r) acc += Rr[r] * Vs[j * D + r * P2 + p2];
            acc = reduce_lanes<P2>(acc);
            if (p2 == 0) dKs[j * F + f] = acc - rs[f];
            float acv = 0.f;
#pragma unroll
            for (int r = 0; r < FS; ++r) acv += Rc[r] * Kf[j * F + r * P + p];
            acv = reduce_lanes<P>(acv);
            if (p == 0) dVs[j * D + d] = acv;
        }
        for (int rep = 0; rep < a.nrep; ++rep) {
            const size_t bh = (size_t)b * a.H + g * a.nrep + rep;
            const T *qh = static_cast<const T *>(a.q) + bh * a.N * D;
            const T *gh = static_cast<const T *>(a.g) + bh * a.N * D;
            __syncthreads();
            load_feat<T, D, F, PHI, C, NT>(Qf, nullptr, qh, c0, a.N, a.cw, a.sw);
            load_rows<T, D, C, NT>(Gs, gh, c0, a.N);
            for (int i = t; i < C; i += NT) {
                const bool ok = c0 + i < a.N;
                dn[i] = ok ? a.ws_den[bh * a.N + c0 + i] : 1.f;
                cc[i] = ok ? a.ws_c[bh * a.N + c0 + i] : 0.f;
            }
            __syncthreads();
            for (int e = t; e < C * C; e += NT) {
                const int i = e / C, j = e % C;
                float av = 0.f, pv = 0.f;
                if (i >= j && c0 + i < a.N) {
                    for (int x = 0; x < F; ++x) av += Qf[i * F + x] * Kf[j * F + x];
                    float tv = 0.f;
                    for (int x = 0; x < D; ++x) tv += Gs[i * D + x] * Vs[j * D + x];
                    pv = tv / dn[i] - cc[i];
                }
                As[e] = av;
                Pm[e] = pv;
            }
            __syncthreads();
            for (int j = p2; j < C; j += P2) {
                float acc = 0.f;
                for (int i = j; i < C; ++i) acc += Pm[i * C + j] * Qf[i * F + f];
                dKs[j * F + f] += acc;
            }
            for (int j = p; j < C; j += P) {
                float acc = 0.f;
                for (int i = j; i < C; ++i) acc += As[i * C + j] * (Gs[i * D + d] / dn[i]);
                dVs[j * D + d] += acc;
            }
            #pragma unroll 2
            for (int i = 0; i < C; ++i) {
                const float inv = 1.f / dn[i];
                const float qf = Qf[i * F + f];
#pragma unroll
                for (int r = 0; r < DS; ++r) Rr[r] += qf * (Gs[i * D + r * P2 + p2] * inv);
                const float gd = Gs[i * D + d] * inv;
#pragma unroll
                for (int r = 0; r < FS; ++r) Rc[r] += Qf[i * F + r * P + p] * gd;
            }
            for (int e = t; e < F; e += NT) {
                float acc = 0.f;
                for (int i = 0; i < C; ++i) acc += cc[i] * Qf[i * F + e];
                rs[e] += acc;
            }
        }
        __syncthreads();
        for (int e = t; e < C * D; e += NT) {
            const int j = e / D, x = e % D;
            if (c0 + j >= a.N) continue;
            float gphi;
            if constexpr (F == 2 * D)
                gphi = a.cw[c0 + j] * dKs[j * F + x] + a.sw[c0 + j] * dKs[j * F + D + x];
            else
                gphi = dKs[j * F + x];
            st(dkh, (size_t)(c0 + j) * D + x, phi_d<PHI>(Kr[j * D + x]) * gphi);
            st(dvh, (size_t)(c0 + j) * D + x, dVs[e]);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Bidirectional backward.  k_bwd_q_bidir: per (batch, query head, segment):
// dq against the total (S, z), and the segment's partial (R, r).
// ---------------------------------------------------------------------------
template <typename T, int D, int F, int PHI>
__global__ __launch_bounds__(nt_bwd<F>()) void k_bwd_q_bidir(Args a) {
    constexpr int NT = nt_bwd<F>();
    constexpr int C = chunk_bwd_q<F, D>();
    constexpr int P2 = NT / F, DS = D / P2;
    __shared__ float Qf[C * F];
    __shared__ float Gs[C * D];
    __shared__ float Qr[C * D];
    __shared__ float Us[C * F];
    __shared__ float zs[F];
    __shared__ float dn[C];
    __shared__ float cc[C];
    const int seg = blockIdx.x % a.nseg, bh = blockIdx.x / a.nseg;
    const int b = bh / a.H, h = bh % a.H, g = h / a.nrep, bg = b * a.Hkv + g;
    const int t = threadIdx.x, f = t / P2, p2 = t % P2;
    const size_t SD = (size_t)F * D + F;
    const T *qh = static_cast<const T *>(a.q) + (size_t)bh * a.N * D;
    const T *gh = static_cast<const T *>(a.g) + (size_t)bh * a.N * D;
    T *dqh = static_cast<T *>(a.dq) + (size_t)bh * a.N * D;
    const float *Sp = a.ws_S + ((size_t)bg * (a.nseg + 1) + a.nseg) * SD;
    float S[DS], R[DS];
#pragma unroll
    for (int r = 0; r < DS; ++r) {
        S[r] = Sp[(size_t)f * D + r * P2 + p2];
        R[r] = 0.f;
    }
    float rr = 0.f;
    for (int e = t; e < F; e += NT) zs[e] = Sp[(size_t)F * D + e];
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    for (int c0 = row0; c0 < row1; c0 += C) {
        load_feat<T, D, F, PHI, C, NT>(Qf, Qr, qh, c0, a.N, a.cw, a.sw);
        load_rows<T, D, C, NT>(Gs, gh, c0, a.N);
        __syncthreads();
        #pragma unroll 2
        for (int i = 0; i < C; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < DS; ++r) acc += S[r] * Gs[i * D + r * P2 + p2];
            acc = reduce_lanes<P2>(acc);
            if (p2 == 0) Us[i * F + f] = acc;
        }
        __syncthreads();
        for (int i = t; i < C; i += NT) {
            float qz = 0.f, qu = 0.f;
            for (int x = 0; x < F; ++x) {
                qz += Qf[i * F + x] * zs[x];
                qu += Qf[i * F + x] * Us[i * F + x];
            }
            const bool ok = c0 + i < a.N;   // rows past N: neutral values
            const float den = ok ? qz + a.eps : 1.f;
            dn[i] = den;
            cc[i] = ok ? qu / (den * den) : 0.f;
        }
        __syncthreads();
        for (int i = p2; i < C; i += P2) Us[i * F + f] = Us[i * F + f] / dn[i] - cc[i] * zs[f];
        __syncthreads();
        for (int e = t; e < C * D; e += NT) {
            const int i = e / D, x = e % D;
            if (c0 + i >= a.N) continue;
            float gphi;
            if constexpr (F == 2 * D)
                gphi = a.cw[c0 + i] * Us[i * F + x] + a.sw[c0 + i] * Us[i * F + D + x];
            else
                gphi = Us[i * F + x];
            st(dqh, (size_t)(c0 + i) * D + x, phi_d<PHI>(Qr[i * D + x]) * gphi);
        }
        #pragma unroll 2
        for (int i = 0; i < C; ++i) {
            const float qf = Qf[i * F + f], inv = 1.f / dn[i];
#pragma unroll
            for (int r = 0; r < DS; ++r) R[r] += qf * (Gs[i * D + r * P2 + p2] * inv);
            rr += cc[i] * qf;
        }
        __syncthreads();
    }
    float *Ro = a.ws_Rp + ((size_t)bh * a.nseg + seg) * SD;
#pragma unroll
    for (int r = 0; r < DS; ++r) Ro[(size_t)f * D + r * P2 + p2] = R[r];
    if (p2 == 0) Ro[(size_t)F * D + f] = rr;
}

// k_bwd_kv_bidir: per (batch, KV head, segment): dk, dv against the total (R, r).
template <typename T, int D, int F, int PHI>
__global__ __launch_bounds__(nt_bwd<F>()) void k_bwd_kv_bidir(Args a) {
    constexpr int NT = nt_bwd<F>();
    constexpr int C = chunk_bwd_kv<F, D>();
    constexpr int P2 = NT / F, DS = D / P2;
    constexpr int P = NT / D, FS = F / P;
    __shared__ float Kf[C * F];
    __shared__ float Vs[C * D];
    __shared__ float Kr[C * D];
    __shared__ float dKs[C * F];
    __shared__ float rs[F];
    const int seg = blockIdx.x % a.nseg, bg = blockIdx.x / a.nseg;
    const int t = threadIdx.x, f = t / P2, p2 = t % P2, d = t / P, p = t % P;
    const size_t SD = (size_t)F * D + F;
    const T *kh = static_cast<const T *>(a.k) + (size_t)bg * a.N * D;
    const T *vh = static_cast<const T *>(a.v) + (size_t)bg * a.N * D;
    T *dkh = static_cast<T *>(a.dk) + (size_t)bg * a.N * D;
    T *dvh = static_cast<T *>(a.dv) + (size_t)bg * a.N * D;
    const float *Rp = a.ws_Rs + ((size_t)bg * (a.nseg + 1) + a.nseg) * SD;
    float Rr[DS], Rc[FS];
#pragma unroll
    for (int r = 0; r < DS; ++r) Rr[r] = Rp[(size_t)f * D + r * P2 + p2];
#pragma unroll
    for (int r = 0; r < FS; ++r) Rc[r] = Rp[(size_t)(r * P + p) * D + d];
    for (int e = t; e < F; e += NT) rs[e] = Rp[(size_t)F * D + e];
    const int row0 = seg * a.L, row1 = min(row0 + a.L, a.N);
    for (int c0 = row0; c0 < row1; c0 += C) {
        load_feat<T, D, F, PHI, C, NT>(Kf, Kr, kh, c0, a.N, a.cw, a.sw);
        load_rows<T, D, C, NT>(Vs, vh, c0, a.N);
        __syncthreads();
        #pragma unroll 2
        for (int j = 0; j < C; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < DS; ++r) acc += Rr[r] * Vs[j * D + r * P2 + p2];
            acc = reduce_lanes<P2>(acc);
            if (p2 == 0) dKs[j * F + f] = acc - rs[f];
            float acv = 0.f;
#pragma unroll
            for (int r = 0; r < FS; ++r) acv += Rc[r] * Kf[j * F + r * P + p];
            acv = reduce_lanes<P>(acv);
            if (p == (j % P) && c0 + j < a.N) st(dvh, (size_t)(c0 + j) * D + d, acv);
        }
        __syncthreads();
        for (int e = t; e < C * D; e += NT) {
            const int j = e / D, x = e % D;
            if (c0 + j >= a.N) continue;
            float gphi;
            if constexpr (F == 2 * D)
                gphi = a.cw[c0 + j] * dKs[j * F + x] + a.sw[c0 + j] * dKs[j * F + D + x];
            else
                gphi = dKs[j * F + x];
            st(dkh, (size_t)(c0 + j) * D + x, phi_d<PHI>(Kr[j * D + x]) * gphi);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T, int D, int F, int PHI>
hipError_t run_fwd(const Args &a, int causal, hipStream_t s) {
    const unsigned n_units = (unsigned)(a.B * a.Hkv);
    const unsigned n_q = (unsigned)(a.B * a.H * a.nseg);
    const size_t SD = (size_t)F * D + F;
    const dim3 scan_grid((unsigned)((SD + kNT - 1) / kNT), n_units);
    {
        TimedLaunch tl("k_state", s);
        hipLaunchKernelGGL((k_state<T, D, F, PHI>), dim3(n_units * a.nseg), dim3(kNT), 0, s, a);
    }
    {
        TimedLaunch tl("k_scan_S", s);
        hipLaunchKernelGGL(k_scan_S, scan_grid, dim3(kNT), 0, s, a.ws_S, a.nseg, SD,
                           (size_t)n_units, causal);
    }
    if (causal) {
        TimedLaunch tl("k_fwd_causal", s);
        hipLaunchKernelGGL((k_fwd_causal<T, D, F, PHI>), dim3(n_q), dim3(kNT), 0, s, a);
    } else {
        TimedLaunch tl("k_fwd_bidir", s);
        hipLaunchKernelGGL((k_fwd_bidir<T, D, F, PHI>), dim3(n_q), dim3(kNT), 0, s, a);
    }
    return hipGetLastError();
}

template <typename T, int D, int F, int PHI>
hipError_t run_bwd(const Args &a, int causal, hipStream_t s) {
    constexpr int NT = nt_bwd<F>();
    const unsigned n_units = (unsigned)(a.B * a.Hkv);
    const unsigned n_q = (unsigned)(a.B * a.H * a.nseg);
    const unsigned n_kv = n_units * a.nseg;
    const size_t SD = (size_t)F * D + F;
    const dim3 scan_grid((unsigned)((SD + kNT - 1) / kNT), n_units);
    if (!a.state_ready) {   // else the forward's records are in ws_S already
        {
            TimedLaunch tl("k_state", s);
            hipLaunchKernelGGL((k_state<T, D, F, PHI>), dim3(n_units * a.nseg), dim3(kNT), 0, s, a);
        }
        TimedLaunch tl("k_scan_S", s);
        hipLaunchKernelGGL(k_scan_S, scan_grid, dim3(kNT), 0, s, a.ws_S, a.nseg, SD,
                           (size_t)n_units, causal);
    }
    if (causal) {
        TimedLaunch tl("k_bwd_q_causal", s);
        hipLaunchKernelGGL((k_bwd_q_causal<T, D, F, PHI>), dim3(n_q), dim3(NT), 0, s, a);
    } else {
        TimedLaunch tl("k_bwd_q_bidir", s);
        hipLaunchKernelGGL((k_bwd_q_bidir<T, D, F, PHI>), dim3(n_q), dim3(NT), 0, s, a);
    }
    {
        TimedLaunch tl("k_scan_R", s);
        hipLaunchKernelGGL(k_scan_R, scan_grid, dim3(kNT), 0, s, (const float *)a.ws_Rp, a.ws_Rs,
                           a.nseg, SD, a.H, a.Hkv, a.nrep, (size_t)n_units, causal);
    }
    if (causal) {
        TimedLaunch tl("k_bwd_kv_causal", s);
        hipLaunchKernelGGL((k_bwd_kv_causal<T, D, F, PHI>), dim3(n_kv), dim3(NT), 0, s, a);
    } else {
        TimedLaunch tl("k_bwd_kv_bidir", s);
        hipLaunchKernelGGL((k_bwd_kv_bidir<T, D, F, PHI>), dim3(n_kv), dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

template <typename T, int D, int F>
hipError_t by_phi(const Args &a, int bwd, int causal, int phi, hipStream_t s) {
    switch (phi) {
        case kElu1:
            return bwd ? run_bwd<T, D, F, kElu1>(a, causal, s) : run_fwd<T, D, F, kElu1>(a, causal, s);
        case kRelu:
            return bwd ? run_bwd<T, D, F, kRelu>(a, causal, s) : run_fwd<T, D, F, kRelu>(a, causal, s);
        default:
            return bwd ? run_bwd<T, D, F, kIdentity>(a, causal, s)
                       : run_fwd<T, D, F, kIdentity>(a, causal, s);
    }
}

template <typename T>
hipError_t by_shape(const Args &a, int bwd, int causal, int phi, hipStream_t s) {
    const bool cos = a.F == 2 * a.D;
    switch (a.D) {
        case 32:
            return cos ? by_phi<T, 32, 64>(a, bwd, causal, phi, s) : by_phi<T, 32, 32>(a, bwd, causal, phi, s);
        case 64:
            return cos ? by_phi<T, 64, 128>(a, bwd, causal, phi, s) : by_phi<T, 64, 64>(a, bwd, causal, phi, s);
        default:
            return cos ? by_phi<T, 128, 256>(a, bwd, causal, phi, s) : by_phi<T, 128, 128>(a, bwd, causal, phi, s);
    }
}

}  // namespace

hipError_t scan_state(float *ws, int nseg, size_t SD, unsigned n_units, bool causal, hipStream_t s) {
    hipLaunchKernelGGL(k_scan_S, dim3((unsigned)((SD + kNT - 1) / kNT), n_units), dim3(kNT), 0, s,
                       ws, nseg, SD, (size_t)n_units, causal ? 1 : 0);
    return hipGetLastError();
}

hipError_t scan_suffix(const float *Rp, float *Rs, int nseg, size_t SD, int H, int Hkv, int nrep,
                       unsigned n_units, bool causal, hipStream_t s) {
    hipLaunchKernelGGL(k_scan_R, dim3((unsigned)((SD + kNT - 1) / kNT), n_units), dim3(kNT), 0, s,
                       Rp, Rs, nseg, SD, H, Hkv, nrep, (size_t)n_units, causal ? 1 : 0);
    return hipGetLastError();
}

hipError_t generic_run(const Args &a, int bf16, int bwd, int causal, int phi, hipStream_t s) {
    return bf16 ? by_shape<bf16_t>(a, bwd, causal, phi, s) : by_shape<float>(a, bwd, causal, phi, s);
}

}  // namespace la
