// la_api.hip -- the C ABI declared in include/linattn.h: argument validation
// (all of it before any device work), workspace sizing and layout, and
// dispatch to the kernel families.
//
// Validation mirrors what the SVD_linear_Attention pages require of a call:
// "Module neuralops.core.triton_kernels.gqa", function is_supported, rejects
// non-positive head counts and num_heads not divisible by num_kv_heads; the
// linear_attn page's fwd takes cos_weight and sin_weight as a pair.  Where the
// pages fall back to a different implementation for unsupported inputs, this
// library returns LA_ERR_UNSUPPORTED instead.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "linattn.h"
#include "la_gqa.h"
#include "la_lowrank.h"
#include "la_common.h"
#include "la_kernels.h"
#include "la_timing.h"

namespace la {

// Per-thread launch timing (see la_timing.h).
struct TimingRec {
    const char *name;
    hipEvent_t start, stop;
};
thread_local bool g_timing = false;
thread_local std::vector<TimingRec> g_recs;

bool timing_on() { return g_timing; }

void timing_begin(const char *name, hipStream_t s) {
    TimingRec r{name, nullptr, nullptr};
    // timing-only events: no system-scope fence (cache writeback) at each record
    if (hipEventCreateWithFlags(&r.start, hipEventDisableSystemFence) != hipSuccess) return;
    if (hipEventCreateWithFlags(&r.stop, hipEventDisableSystemFence) != hipSuccess) {
        (void)hipEventDestroy(r.start);
        return;
    }
    if (hipEventRecord(r.start, s) != hipSuccess) {
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
        return;
    }
    g_recs.push_back(r);
}

void timing_end(hipStream_t s) {
    if (!g_recs.empty()) (void)hipEventRecord(g_recs.back().stop, s);
}

}  // namespace la

namespace {

thread_local char g_err[512] = "";

la_status fail(la_status st, const char *msg) {
    snprintf(g_err, sizeof g_err, "%s", msg);
    return st;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

la_status check_shape(int B, int H, int H_kv, int N, int D, int dtype, int phi) {
    if (B <= 0 || H <= 0 || H_kv <= 0 || N <= 0 || D <= 0)
        return fail(LA_ERR_INVALID, "B, H, H_kv, N and D must be positive");
    if (H % H_kv != 0) return fail(LA_ERR_INVALID, "H must be a multiple of H_kv");
    if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_ERR_INVALID, "unknown dtype");
    if (phi != LA_PHI_ELU1 && phi != LA_PHI_RELU && phi != LA_PHI_IDENTITY)
        return fail(LA_ERR_INVALID, "unknown feature map");
    // element counts must stay addressable with 64-bit offsets and the
    // kernels' 32-bit row indices
    if ((long long)N * D >= (1LL << 31))
        return fail(LA_ERR_INVALID, "N * D must be below 2^31");
    if (D != 32 && D != 64 && D != 128)
        return fail(LA_ERR_UNSUPPORTED, "head dimension D must be 32, 64 or 128");
    return LA_OK;
}

la_status check_common(int B, int H, int H_kv, int N, int D, int dtype, int phi, float eps,
                       const float *cw, const float *sw, void *ws, size_t ws_bytes,
                       size_t need) {
    la_status st = check_shape(B, H, H_kv, N, D, dtype, phi);
    if (st != LA_OK) return st;
    if (!isfinite(eps) || eps < 0.f) return fail(LA_ERR_INVALID, "eps must be finite and >= 0");
    if ((cw == nullptr) != (sw == nullptr))
        return fail(LA_ERR_INVALID, "cos_w and sin_w must both be given or both be NULL");
    if (cw && (!aligned(cw, 4) || !aligned(sw, 4)))
        return fail(LA_ERR_INVALID, "cos_w / sin_w must be 4-byte aligned");
    if (ws_bytes < need) return fail(LA_ERR_INVALID, "workspace too small");
    if (need > 0 && ws == nullptr) return fail(LA_ERR_INVALID, "workspace pointer is NULL");
    if (ws && !aligned(ws, 256)) return fail(LA_ERR_INVALID, "workspace must be 256-byte aligned");
    return LA_OK;
}

// The kernels that serve a call decide how the sequence is split: the
// matrix-core forward runs one workgroup per (batch, KV head, segment), the
// float32 kernels one per (batch, query head, segment).
bool uses_mfma(int op_bwd, int dtype, int causal, int D, int has_cos) {
    if (op_bwd) return la::mfma_bwd_serves(dtype == LA_BF16, causal != 0, D, has_cos != 0);
    return la::mfma_fwd_serves(dtype == LA_BF16, D);
}

la::Plan plan_for(int op_bwd, int B, int H, int H_kv, int N, int D, int dtype, int causal,
                  int has_cos, int seg_len) {
    // matrix-core kernels: about two workgroups per compute unit (256 on the
    // device) at D = 128.  The causal cos/sin ones there (F = 256) fit one
    // per compute unit; they are as fast with one round of longer segments,
    // and the state records then cost half as much.  At D = 64 the forward
    // and dk/dv workgroups have two waves: aim for six per compute unit (the
    // 256-row minimum segment usually binds first)
    if (uses_mfma(op_bwd, dtype, causal, D, has_cos)) {
        const long long target = D == 64 ? 1536 : has_cos && causal ? 256 : 512;
        return la::make_plan(op_bwd, B, H, H_kv, N, D, causal, has_cos, seg_len,
                             (long long)B * H_kv, target);
    }
    // float32 kernels: one thread walks every row of its segment, so a
    // short sequence over few heads is cut down to 64-row segments (the
    // matrix-core kernels keep 256: their workgroups amortise per-segment
    // set-up over more rows)
    return la::make_plan(op_bwd, B, H, H_kv, N, D, causal, has_cos, seg_len, (long long)B * H,
                         1024, la::kSegAlign);
}

la::Args make_args(const la::Plan &p, int B, int H, int H_kv, int N, int D, float eps,
                   const float *cw, const float *sw, void *ws) {
    la::Args a{};
    char *w = static_cast<char *>(ws);
    a.cw = cw;
    a.sw = sw;
    a.ws_S = reinterpret_cast<float *>(w + p.off_S);
    a.ws_Rp = reinterpret_cast<float *>(w + p.off_Rp);
    a.ws_Rs = reinterpret_cast<float *>(w + p.off_Rs);
    a.ws_den = reinterpret_cast<float *>(w + p.off_den);
    a.ws_c = reinterpret_cast<float *>(w + p.off_c);
    a.B = B;
    a.H = H;
    a.Hkv = H_kv;
    a.N = N;
    a.D = D;
    a.F = p.F;
    a.nrep = H / H_kv;
    a.L = p.L;
    a.nseg = p.nseg;
    a.eps = eps;
    return a;
}

la_status launch_status(hipError_t e) {
    if (e != hipSuccess) {
        snprintf(g_err, sizeof g_err, "HIP: %s", hipGetErrorString(e));
        return LA_ERR_HIP;
    }
    return LA_OK;
}

}  // namespace

namespace la {
// Sets la_last_error for the other translation units of the C ABI.
la_status api_fail(la_status st, const char *msg) { return fail(st, msg); }
}  // namespace la

extern "C" {

size_t la_workspace_bytes_ex(int op, int B, int H, int H_kv, int N, int D, int dtype,
                             int causal, int has_cos, int seg_len) {
    if (op != LA_OP_FWD && op != LA_OP_BWD) return 0;
    if (check_shape(B, H, H_kv, N, D, dtype, LA_PHI_ELU1) != LA_OK) return 0;
    if (seg_len < 0) return 0;
    return plan_for(op == LA_OP_BWD, B, H, H_kv, N, D, dtype, causal, has_cos != 0, seg_len).bytes;
}

size_t la_workspace_bytes(int op, int B, int H, int H_kv, int N, int D, int dtype, int causal,
                          int has_cos) {
    return la_workspace_bytes_ex(op, B, H, H_kv, N, D, dtype, causal, has_cos, 0);
}

la_status la_fwd_ex(const void *q, const void *k, const void *v, void *out, int B, int H,
                    int H_kv, int N, int D, int dtype, int causal, int phi, float eps,
                    const float *cos_w, const float *sin_w, void *ws, size_t ws_bytes,
                    void *stream, int seg_len) {
    g_err[0] = 0;
    if (!q || !k || !v || !out) return fail(LA_ERR_INVALID, "q, k, v and out must be non-NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(LA_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
    if (seg_len < 0) return fail(LA_ERR_INVALID, "seg_len must be >= 0");
    la_status st = check_shape(B, H, H_kv, N, D, dtype, phi);
    if (st != LA_OK) return st;
    const la::Plan p = plan_for(0, B, H, H_kv, N, D, dtype, causal, cos_w != nullptr, seg_len);
    st = check_common(B, H, H_kv, N, D, dtype, phi, eps, cos_w, sin_w, ws, ws_bytes, p.bytes);
    if (st != LA_OK) return st;
    la::Args a = make_args(p, B, H, H_kv, N, D, eps, cos_w, sin_w, ws);
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (uses_mfma(0, dtype, causal, D, cos_w != nullptr))
        return launch_status(la::mfma_fwd_run(a, phi, causal, s));
    if (la::mfma_f32_serves(dtype == LA_BF16, causal, D, cos_w != nullptr))
        return launch_status(la::mfma_f32_run(a, 0, phi, s));
    return launch_status(la::generic_run(a, dtype == LA_BF16, 0, causal != 0, phi, s));
}

la_status la_fwd(const void *q, const void *k, const void *v, void *out, int B, int H, int H_kv,
                 int N, int D, int dtype, int causal, int phi, float eps, const float *cos_w,
                 const float *sin_w, void *ws, size_t ws_bytes, void *stream) {
    return la_fwd_ex(q, k, v, out, B, H, H_kv, N, D, dtype, causal, phi, eps, cos_w, sin_w, ws,
                     ws_bytes, stream, 0);
}

namespace {

// The backward; state_ready: ws holds the forward's state records (la_bwd_saved).
la_status bwd_impl(const void *q, const void *k, const void *v, const void *grad_out, void *dq,
                   void *dk, void *dv, int B, int H, int H_kv, int N, int D, int dtype,
                   int causal, int phi, float eps, const float *cos_w, const float *sin_w,
                   void *ws, size_t ws_bytes, void *stream, int seg_len, int state_ready) {
    g_err[0] = 0;
    if (!q || !k || !v || !grad_out || !dq || !dk || !dv)
        return fail(LA_ERR_INVALID, "q, k, v, grad_out, dq, dk and dv must be non-NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(grad_out, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return fail(LA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
    if (seg_len < 0) return fail(LA_ERR_INVALID, "seg_len must be >= 0");
    la_status st = check_shape(B, H, H_kv, N, D, dtype, phi);
    if (st != LA_OK) return st;
    const la::Plan p = plan_for(1, B, H, H_kv, N, D, dtype, causal, cos_w != nullptr, seg_len);
    st = check_common(B, H, H_kv, N, D, dtype, phi, eps, cos_w, sin_w, ws, ws_bytes, p.bytes);
    if (st != LA_OK) return st;
    la::Args a = make_args(p, B, H, H_kv, N, D, eps, cos_w, sin_w, ws);
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = grad_out;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    // The saved records are laid out by the forward's plan, which is the
    // backward's only when both run the same kernel family.  Every case
    // served today pairs them; a pairing that did not would compute the
    // state again rather than read records of another segmentation.
    const int has_cos = cos_w != nullptr;
    a.state_ready = state_ready && uses_mfma(0, dtype, causal, D, has_cos) ==
                                       uses_mfma(1, dtype, causal, D, has_cos);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (uses_mfma(1, dtype, causal, D, cos_w != nullptr))
        return launch_status(la::mfma_bwd_run(a, phi, causal, s));
    if (la::mfma_f32_serves(dtype == LA_BF16, causal, D, cos_w != nullptr))
        return launch_status(la::mfma_f32_run(a, 1, phi, s));
    return launch_status(la::generic_run(a, dtype == LA_BF16, 1, causal != 0, phi, s));
}

}  // namespace

la_status la_bwd_ex(const void *q, const void *k, const void *v, const void *grad_out, void *dq,
                    void *dk, void *dv, int B, int H, int H_kv, int N, int D, int dtype,
                    int causal, int phi, float eps, const float *cos_w, const float *sin_w,
                    void *ws, size_t ws_bytes, void *stream, int seg_len) {
    return bwd_impl(q, k, v, grad_out, dq, dk, dv, B, H, H_kv, N, D, dtype, causal, phi, eps,
                    cos_w, sin_w, ws, ws_bytes, stream, seg_len, 0);
}

la_status la_bwd(const void *q, const void *k, const void *v, const void *grad_out, void *dq,
                 void *dk, void *dv, int B, int H, int H_kv, int N, int D, int dtype, int causal,
                 int phi, float eps, const float *cos_w, const float *sin_w, void *ws,
                 size_t ws_bytes, void *stream) {
    return bwd_impl(q, k, v, grad_out, dq, dk, dv, B, H, H_kv, N, D, dtype, causal, phi, eps,
                    cos_w, sin_w, ws, ws_bytes, stream, 0, 0);
}

la_status la_bwd_saved_ex(const void *q, const void *k, const void *v, const void *grad_out,
                          void *dq, void *dk, void *dv, int B, int H, int H_kv, int N, int D,
                          int dtype, int causal, int phi, float eps, const float *cos_w,
                          const float *sin_w, void *ws, size_t ws_bytes, void *stream,
                          int seg_len) {
    return bwd_impl(q, k, v, grad_out, dq, dk, dv, B, H, H_kv, N, D, dtype, causal, phi, eps,
                    cos_w, sin_w, ws, ws_bytes, stream, seg_len, 1);
}

la_status la_bwd_saved(const void *q, const void *k, const void *v, const void *grad_out,
                       void *dq, void *dk, void *dv, int B, int H, int H_kv, int N, int D,
                       int dtype, int causal, int phi, float eps, const float *cos_w,
                       const float *sin_w, void *ws, size_t ws_bytes, void *stream) {
    return bwd_impl(q, k, v, grad_out, dq, dk, dv, B, H, H_kv, N, D, dtype, causal, phi, eps,
                    cos_w, sin_w, ws, ws_bytes, stream, 0, 1);
}

const char *la_status_string(int status) {
    switch (status) {
        case LA_OK: return "LA_OK: success";
        case LA_ERR_INVALID: return "LA_ERR_INVALID: invalid argument";
        case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: unsupported configuration";
        case LA_ERR_HIP: return "LA_ERR_HIP: HIP runtime error";
        default: return "unknown status";
    }
}

const char *la_last_error(void) { return g_err; }

la_status la_timing_enable(int enable) {
    la::g_timing = enable != 0;
    return LA_OK;
}

int la_timing_collect(la_kernel_time *out, int max_entries) {
    int n = 0;
    for (const la::TimingRec &r : la::g_recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.stop) != hipSuccess ||
            hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
            ms = -1.f;   // not measurable: reported as a negative total
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
        int slot = -1;
        for (int i = 0; i < n; ++i)
            if (strncmp(out[i].name, r.name, sizeof out[i].name) == 0) slot = i;
        if (slot < 0 && n < max_entries && out) {
            slot = n++;
            snprintf(out[slot].name, sizeof out[slot].name, "%s", r.name);
            out[slot].launches = 0;
            out[slot].total_ms = 0.0;
        }
        if (slot >= 0) {
            out[slot].launches += 1;
            out[slot].total_ms += ms;
        }
    }
    la::g_recs.clear();
    return n;
}

// Grouped-query head expansion and its adjoint (include/la_gqa.h).
static la_status gqa_check(const void *a, const void *b, const void *ao, const void *bo, int B,
                           int H_kv, int H, int N, int D, int dtype) {
    if (B <= 0 || H_kv <= 0 || H <= 0 || N <= 0 || D <= 0)
        return fail(LA_ERR_INVALID, "B, H_kv, H, N and D must be positive");
    if (H % H_kv != 0) return fail(LA_ERR_INVALID, "H must be a multiple of H_kv");
    if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_ERR_INVALID, "unknown dtype");
    if (!a || !ao) return fail(LA_ERR_INVALID, "the k pair of pointers must be non-NULL");
    if ((b == nullptr) != (bo == nullptr))
        return fail(LA_ERR_INVALID, "the v pair of pointers must both be given or both be NULL");
    const uintptr_t es = dtype == LA_BF16 ? 2 : 4;
    if (!aligned(a, es) || !aligned(ao, es) || (b && (!aligned(b, es) || !aligned(bo, es))))
        return fail(LA_ERR_INVALID, "pointers must be aligned to the element size");
    if ((long long)B * H_kv > 65535) return fail(LA_ERR_UNSUPPORTED, "B * H_kv must be at most 65535");
    return LA_OK;
}

la_status la_gqa_expand(const void *k, const void *v, void *k_out, void *v_out, int B, int H_kv,
                        int H, int N, int D, int dtype, void *stream) {
    const la_status st = gqa_check(k, v, k_out, v_out, B, H_kv, H, N, D, dtype);
    if (st != LA_OK) return st;
    const hipError_t e = la::gqa_expand_run(k, v, k_out, v_out, B, H_kv, H, (long long)N * D,
                                            dtype == LA_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LA_OK : fail(LA_ERR_HIP, hipGetErrorString(e));
}

la_status la_gqa_reduce(const void *grad_k, const void *grad_v, void *gk_out, void *gv_out, int B,
                        int H_kv, int H, int N, int D, int dtype, void *stream) {
    const la_status st = gqa_check(grad_k, grad_v, gk_out, gv_out, B, H_kv, H, N, D, dtype);
    if (st != LA_OK) return st;
    const hipError_t e = la::gqa_reduce_run(grad_k, grad_v, gk_out, gv_out, B, H_kv, H,
                                            (long long)N * D, dtype == LA_BF16,
                                            static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LA_OK : fail(LA_ERR_HIP, hipGetErrorString(e));
}

typedef unsigned short u16;   // bf16 storage

// Low-rank projection (include/la_lowrank.h).
struct LowRankPlan {
    size_t off_t, off_gt, off_part, off_bpart, bytes;
};

static LowRankPlan lowrank_plan(int op, int M, int n_in, int rank, int n_out) {
    const size_t a = 256;
    LowRankPlan p{};
    size_t off = 0;
    p.off_t = off;
    off = la::align_up(off + (size_t)M * rank * 2, a);
    if (op == LA_OP_BWD) {
        p.off_gt = off;
        off = la::align_up(off + (size_t)M * rank * 2, a);
        const size_t sU = (size_t)la::lowrank_splits(M, n_out, rank) * n_out * rank;
        const size_t sV = (size_t)la::lowrank_splits(M, rank, n_in) * rank * n_in;
        p.off_part = off;
        off = la::align_up(off + 4 * (sU > sV ? sU : sV), a);
        p.off_bpart = off;
        off = la::align_up(off + 4 * (size_t)la::lowrank_bias_blocks(M) * n_out, a);
    }
    p.bytes = off;
    return p;
}

static la_status lowrank_check(int M, int n_in, int rank, int n_out, int dtype) {
    if (M < 1) return fail(LA_ERR_INVALID, "M must be positive");
    for (int d : {n_in, rank, n_out})
        if (d < 8 || d % 8) return fail(LA_ERR_INVALID, "n_in, rank and n_out must be positive multiples of 8");
    if (dtype == LA_F32) return fail(LA_ERR_UNSUPPORTED, "the low-rank projection serves bf16 storage only");
    if (dtype != LA_BF16) return fail(LA_ERR_INVALID, "unknown dtype");
    return LA_OK;
}

static la_status lowrank_ws(const void *ws, size_t ws_bytes, size_t need) {
    if (ws == nullptr) return fail(LA_ERR_INVALID, "workspace pointer is NULL");
    if (!aligned(ws, 256)) return fail(LA_ERR_INVALID, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(LA_ERR_INVALID, "workspace too small");
    return LA_OK;
}

size_t la_lowrank_workspace_bytes(int op, int M, int n_in, int rank, int n_out, int dtype) {
    if ((op != LA_OP_FWD && op != LA_OP_BWD) || M < 1 || n_in < 8 || rank < 8 || n_out < 8 ||
        (n_in | rank | n_out) % 8 || dtype != LA_BF16)
        return 0;
    return lowrank_plan(op, M, n_in, rank, n_out).bytes;
}

la_status la_lowrank_fwd(const void *x, const void *U, const void *V, const void *bias, void *y, int M,
                         int n_in, int rank, int n_out, int dtype, void *ws, size_t ws_bytes,
                         void *stream) {
    la_status st = lowrank_check(M, n_in, rank, n_out, dtype);
    if (st != LA_OK) return st;
    if (!x || !U || !V || !y) return fail(LA_ERR_INVALID, "x, U, V and y must be non-NULL");
    for (const void *p : {x, U, V, bias, (const void *)y})
        if (p && !aligned(p, 16)) return fail(LA_ERR_INVALID, "tensors must be 16-byte aligned");
    const LowRankPlan p = lowrank_plan(LA_OP_FWD, M, n_in, rank, n_out);
    if ((st = lowrank_ws(ws, ws_bytes, p.bytes)) != LA_OK) return st;
    la::LowRankArgs a{};
    char *w = static_cast<char *>(ws);
    a.x = static_cast<const u16 *>(x); a.U = static_cast<const u16 *>(U); a.V = static_cast<const u16 *>(V);
    a.bias = static_cast<const u16 *>(bias); a.y = static_cast<u16 *>(y);
    a.t = reinterpret_cast<u16 *>(w + p.off_t);
    a.M = M; a.n_in = n_in; a.rank = rank; a.n_out = n_out;
    const hipError_t e = la::lowrank_fwd_run(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LA_OK : fail(LA_ERR_HIP, hipGetErrorString(e));
}

la_status la_lowrank_bwd(const void *x, const void *U, const void *V, const void *grad_out,
                         void *grad_x, void *grad_U, void *grad_V, void *grad_bias, int M, int n_in,
                         int rank, int n_out, int dtype, void *ws, size_t ws_bytes, void *stream) {
    la_status st = lowrank_check(M, n_in, rank, n_out, dtype);
    if (st != LA_OK) return st;
    if (!x || !U || !V || !grad_out || !grad_x || !grad_U || !grad_V)
        return fail(LA_ERR_INVALID, "x, U, V, grad_out, grad_x, grad_U and grad_V must be non-NULL");
    for (const void *p : {x, U, V, grad_out, (const void *)grad_x, (const void *)grad_U,
                          (const void *)grad_V, (const void *)grad_bias})
        if (p && !aligned(p, 16)) return fail(LA_ERR_INVALID, "tensors must be 16-byte aligned");
    const LowRankPlan p = lowrank_plan(LA_OP_BWD, M, n_in, rank, n_out);
    if ((st = lowrank_ws(ws, ws_bytes, p.bytes)) != LA_OK) return st;
    la::LowRankArgs a{};
    char *w = static_cast<char *>(ws);
    a.x = static_cast<const u16 *>(x); a.U = static_cast<const u16 *>(U); a.V = static_cast<const u16 *>(V);
    a.g = static_cast<const u16 *>(grad_out);
    a.gx = static_cast<u16 *>(grad_x); a.gU = static_cast<u16 *>(grad_U); a.gV = static_cast<u16 *>(grad_V);
    a.gbias = static_cast<u16 *>(grad_bias);
    a.t = reinterpret_cast<u16 *>(w + p.off_t);
    a.gt = reinterpret_cast<u16 *>(w + p.off_gt);
    a.part = reinterpret_cast<float *>(w + p.off_part);
    a.bpart = reinterpret_cast<float *>(w + p.off_bpart);
    a.M = M; a.n_in = n_in; a.rank = rank; a.n_out = n_out;
    const hipError_t e = la::lowrank_bwd_run(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LA_OK : fail(LA_ERR_HIP, hipGetErrorString(e));
}

}  // extern "C"
