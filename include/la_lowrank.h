/*
 * la_lowrank.h -- C ABI of the low-rank projection in liblinattn.so
 * (MI355X, gfx950).
 *
 * Operation (SVD_linear_Attention API, page "Module
 * neuralops.core.triton_kernels.low_rank": fwd computes
 * y = (x V^T) U^T + bias; bwd returns the gradients of that expression with
 * respect to x, U, V and bias).  With t = x V^T and g = grad_out:
 *
 *   la_lowrank_fwd:  y = t U^T + bias
 *   la_lowrank_bwd:  grad_x = (g U) V,  grad_U = g^T t,
 *                    grad_V = (g U)^T x,  grad_bias = sum over rows of g
 *
 * Layout: row-major, contiguous; x's leading axes flattened into M rows.
 *   x, grad_x: [M, n_in]     y, grad_out: [M, n_out]
 *   U, grad_U: [n_out, rank] V, grad_V: [rank, n_in]   bias, grad_bias: [n_out]
 * Storage: bf16 only (dtype LA_BF16 of linattn.h; LA_F32 is answered with
 * LA_ERR_UNSUPPORTED).  Products accumulate in float32 on the matrix cores;
 * t and g U are rounded to bf16 between products, as a bf16 evaluation of the
 * page's expression rounds them; each output is rounded once to bf16.
 * grad_U and grad_V sum over the M rows in fixed-size row ranges whose
 * float32 partials are added in range order, and grad_bias likewise: every
 * result is bitwise reproducible run to run.
 *
 * Ownership and execution: all pointers are caller-owned device memory; the
 * library allocates nothing and only enqueues on `stream` (a hipStream_t,
 * NULL = the null stream).  Inputs are read only; outputs are fully written
 * and must not overlap inputs, each other or the workspace.  bias (forward)
 * and grad_bias (backward) may be NULL: no bias term, no bias gradient.
 * `ws` is caller-allocated device memory, 256-byte aligned, of at least
 * la_lowrank_workspace_bytes(op, ...) bytes for the same sizes (op = LA_OP_FWD
 * or LA_OP_BWD); its contents on entry do not matter; calls in flight at the
 * same time need separate workspaces.  The backward recomputes t, as the
 * page's bwd does.
 *
 * Errors (la_status; la_last_error() gives the reason), all checked before
 * any launch: LA_ERR_INVALID for M < 1, n_in / rank / n_out not positive
 * multiples of 8, a NULL required pointer, a tensor not 16-byte aligned, a
 * NULL or misaligned or too small workspace, or an unknown dtype;
 * LA_ERR_UNSUPPORTED for LA_F32 storage; LA_ERR_HIP when a launch fails.
 */
#ifndef LA_LOWRANK_H
#define LA_LOWRANK_H

#include <stddef.h>

#include "linattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes for one call (0 for invalid sizes). */
size_t la_lowrank_workspace_bytes(int op, int M, int n_in, int rank, int n_out, int dtype);

la_status la_lowrank_fwd(const void *x, const void *U, const void *V, const void *bias, void *y, int M,
                         int n_in, int rank, int n_out, int dtype, void *ws, size_t ws_bytes,
                         void *stream);

la_status la_lowrank_bwd(const void *x, const void *U, const void *V, const void *grad_out,
                         void *grad_x, void *grad_U, void *grad_V, void *grad_bias, int M, int n_in,
                         int rank, int n_out, int dtype, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_LOWRANK_H */
