/*
 * linattn.h -- C ABI of the MI355X (gfx950) fused feature-map linear
 * attention library, liblinattn.so.
 *
 * Operation (SVD_linear_Attention API, page "Module
 * neuralops.core.triton_kernels.linear_attn": module docstring -- feature maps
 * elu+1 / relu / identity, chunked causal streaming, bidirectional reduction,
 * cos/sin modulation; functions fwd and bwd -- arguments is_causal, phi,
 * eps = 1e-6, cos_weight, sin_weight; bwd returns the gradients of fwd with
 * respect to q, k and v):
 *
 *   Phi(x_t) = phi(x_t), or [cos_w[t] phi(x_t), sin_w[t] phi(x_t)] when the
 *              cos/sin weights are given (feature width F = D or 2D)
 *   S_i = sum_{j in J(i)} Phi(k_j) v_j^T,   z_i = sum_{j in J(i)} Phi(k_j)
 *   out_i = Phi(q_i)^T S_i / (Phi(q_i) . z_i + eps)
 *   J(i) = {0..i} when causal (diagonal included), {0..N-1} otherwise.
 *
 * Grouped-query heads (page "Module neuralops.core.triton_kernels.gqa",
 * function bwd: the head axis viewed as (H_kv, n_rep)): with
 * n_rep = H / H_kv, query head h reads KV head h / n_rep, by index mapping
 * (no expanded copy), and dk, dv of a KV head are summed over its n_rep
 * query heads.
 *
 * Layout: every tensor is row-major and contiguous.
 *   q, out, grad_out, dq : [B, H,    N, D]
 *   k, v, dk, dv         : [B, H_kv, N, D]
 *   cos_w, sin_w         : [N] float32 (both or neither), shared by all heads
 * q, k, v, grad_out and all outputs share one element type (la_dtype).
 * Arithmetic is float32 throughout (bf16 inputs are widened exactly; bf16
 * outputs are rounded to nearest-even once at the end).
 *
 * Ownership and execution: all pointers are device memory owned by the
 * caller.  The library allocates nothing and keeps no state between calls
 * (la_fwd_noalloc's static scratch array aside), and only enqueues work on
 * `stream` (a hipStream_t; NULL = the null stream): a call returns before
 * the work is done.  Inputs are read only; outputs are
 * fully overwritten and must not alias inputs or each other.  Results are
 * bitwise reproducible run to run (no floating-point atomics).
 *
 * Workspace: `ws` is caller-allocated device memory of at least
 * la_workspace_bytes(...) bytes for the same arguments, 256-byte aligned; its
 * contents on entry do not matter.  Two calls that are in flight at the same
 * time need separate workspaces.
 *
 * Errors: every argument check runs before any device work is enqueued; on
 * error nothing is launched.  Faults during execution surface at the
 * caller's next synchronisation.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID = 1,     /* bad pointer, size, alignment, workspace or eps */
    LA_ERR_UNSUPPORTED = 2, /* valid request this build does not serve (D) */
    LA_ERR_HIP = 3          /* a HIP runtime call or kernel launch failed */
} la_status;

/* Feature maps named in the linear_attn module docstring.  elu+1 uses
 * alpha = 1: x + 1 for x > 0, exp(x) otherwise.  relu'(0) = 0. */
typedef enum {
    LA_PHI_ELU1 = 0,
    LA_PHI_RELU = 1,
    LA_PHI_IDENTITY = 2
} la_phi;

typedef enum {
    LA_F32 = 0,  /* IEEE float32 storage */
    LA_BF16 = 1  /* bfloat16 storage */
} la_dtype;

typedef enum {
    LA_OP_FWD = 0,
    LA_OP_BWD = 1
} la_op;

/* Head dimensions served: D in {32, 64, 128}.  Any N >= 1, B >= 1,
 * H_kv >= 1 with H % H_kv == 0. */

/*
 * la_workspace_bytes -- bytes of workspace la_fwd (op = LA_OP_FWD) or la_bwd
 * (op = LA_OP_BWD) needs for these arguments.  Returns 0 for arguments that
 * la_fwd / la_bwd would reject.
 */
size_t la_workspace_bytes(int op, int B, int H, int H_kv, int N, int D,
                          int dtype, int causal, int has_cos);

/*
 * la_fwd -- forward pass (linear_attn page, function fwd).
 *   q [B,H,N,D], k, v [B,H_kv,N,D] -> out [B,H,N,D]
 *   causal : nonzero = causal (prefix sums), zero = bidirectional (full sums)
 *   phi    : la_phi;  eps : added to every denominator, finite and >= 0
 *   cos_w, sin_w : NULL, or float32 [N] position weights (both or neither)
 * Pointers must be 16-byte aligned (cos_w, sin_w: 4-byte).
 * Returns LA_OK, LA_ERR_INVALID, LA_ERR_UNSUPPORTED or LA_ERR_HIP.
 */
la_status la_fwd(const void *q, const void *k, const void *v, void *out,
                 int B, int H, int H_kv, int N, int D, int dtype, int causal,
                 int phi, float eps, const float *cos_w, const float *sin_w,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * la_bwd -- gradients of la_fwd's output with respect to q, k and v for the
 * upstream gradient grad_out (linear_attn page, function bwd; gqa page,
 * function bwd for the KV-head sum).  No gradient is produced for cos_w,
 * sin_w or eps.
 *   grad_out [B,H,N,D] -> dq [B,H,N,D], dk, dv [B,H_kv,N,D]
 * dk and dv are already summed over the n_rep query heads of each KV head
 * (fixed order, deterministic).  Other arguments as la_fwd.
 */
la_status la_bwd(const void *q, const void *k, const void *v,
                 const void *grad_out, void *dq, void *dk, void *dv, int B,
                 int H, int H_kv, int N, int D, int dtype, int causal, int phi,
                 float eps, const float *cos_w, const float *sin_w, void *ws,
                 size_t ws_bytes, void *stream);

/*
 * la_fwd_ex / la_bwd_ex -- la_fwd / la_bwd with the sequence split forced to
 * segments of `seg_len` rows (0 = automatic).  seg_len is rounded up to a
 * multiple of 64 rows.  The result equals la_fwd / la_bwd up to float32
 * summation order; it exists so tests can exercise the cross-segment state
 * scan at small N.  la_workspace_bytes_ex sizes it.  The chunk length is not
 * an argument: each kernel's chunk (32 rows in the chunk loops, the 32x32
 * matrix tile the causal mask is built on) is a compile-time constant, and
 * the segment is the one split that varies at run time.
 */
size_t la_workspace_bytes_ex(int op, int B, int H, int H_kv, int N, int D,
                             int dtype, int causal, int has_cos, int seg_len);

la_status la_fwd_ex(const void *q, const void *k, const void *v, void *out,
                    int B, int H, int H_kv, int N, int D, int dtype,
                    int causal, int phi, float eps, const float *cos_w,
                    const float *sin_w, void *ws, size_t ws_bytes,
                    void *stream, int seg_len);

la_status la_bwd_ex(const void *q, const void *k, const void *v,
                    const void *grad_out, void *dq, void *dk, void *dv, int B,
                    int H, int H_kv, int N, int D, int dtype, int causal,
                    int phi, float eps, const float *cos_w, const float *sin_w,
                    void *ws, size_t ws_bytes, void *stream, int seg_len);

/*
 * la_bwd_saved / la_bwd_saved_ex -- la_bwd / la_bwd_ex for a backward that
 * follows la_fwd / la_fwd_ex with the same arguments (inputs, shape, dtype,
 * causal, phi, eps, cos_w, sin_w, seg_len) and the same workspace: the
 * per-segment state records (S, z) that the forward left in ws are used
 * instead of being computed again (the forward's work saved for the
 * backward, as autograd saves activations).  ws must hold at least
 * la_workspace_bytes(LA_OP_BWD, ...) bytes, be given to that la_fwd call,
 * and be left unchanged in between (any other la_fwd / la_bwd on it
 * overwrites the records).  These preconditions are the caller's: the
 * library cannot check them, and when they do not hold the gradients are
 * wrong.  Results are bitwise equal to la_bwd's.  Errors as la_bwd.
 */
la_status la_bwd_saved(const void *q, const void *k, const void *v,
                       const void *grad_out, void *dq, void *dk, void *dv,
                       int B, int H, int H_kv, int N, int D, int dtype,
                       int causal, int phi, float eps, const float *cos_w,
                       const float *sin_w, void *ws, size_t ws_bytes,
                       void *stream);

la_status la_bwd_saved_ex(const void *q, const void *k, const void *v,
                          const void *grad_out, void *dq, void *dk, void *dv,
                          int B, int H, int H_kv, int N, int D, int dtype,
                          int causal, int phi, float eps, const float *cos_w,
                          const float *sin_w, void *ws, size_t ws_bytes,
                          void *stream, int seg_len);

/*
 * la_fwd_noalloc -- la_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The workspace is not an argument: it is a static device
 * array of LA_NOALLOC_SCRATCH_BYTES that the library holds on every device
 * it runs on until the process ends (its address is looked up on the first
 * call on a device).  The caller passes inputs and outputs as for la_fwd;
 * results are bitwise those of la_fwd.  The call allocates nothing (with
 * kernel timing off): no hipMalloc, no hipFree, no allocating library call.
 *   stream : must belong to the current device (NULL = its null stream).
 * Errors: as la_fwd, plus LA_ERR_INVALID when the sizes need more workspace
 * than LA_NOALLOC_SCRATCH_BYTES (la_workspace_bytes(LA_OP_FWD, ...) tells)
 * or the stream belongs to another device.  Every call on one device shares
 * that device's array, which keeps the last call's contents (la_fwd writes
 * every record it reads, so nothing needs clearing): calls that overlap in
 * time on one device (other streams, other threads) race and must not be
 * made.
 */
#define LA_NOALLOC_SCRATCH_BYTES (40u << 20)

la_status la_fwd_noalloc(const void *q, const void *k, const void *v, void *out, int B, int H,
                         int H_kv, int N, int D, int dtype, int causal, int phi, float eps,
                         const float *cos_w, const float *sin_w, void *stream);

/*
 * Kernel timing, for measurement tools.  la_timing_enable(1) makes every
 * kernel launch of later la_fwd / la_bwd calls on the calling thread record
 * a pair of HIP events on that call's stream (creating them allocates host
 * and driver objects, so leave it off in production).  la_timing_collect
 * waits for the recorded events, destroys them and writes up to max_entries
 * records, one per kernel name in first-launch order, with the number of
 * launches and their summed event-to-event time; it returns the number of
 * records written.
 */
typedef struct {
    char name[48];
    int launches;
    double total_ms;
} la_kernel_time;

la_status la_timing_enable(int enable);
int la_timing_collect(la_kernel_time *out, int max_entries);

/* Static, NUL-terminated description of a status code. */
const char *la_status_string(int status);

/* Text of the last error raised on the calling thread ("" if none). */
const char *la_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
