/*
 * la_gqa.h -- C ABI of the materialised grouped-query head expansion and its
 * adjoint in liblinattn.so (MI355X, gfx950).
 *
 * Operation (SVD_linear_Attention API, page "Module
 * neuralops.core.triton_kernels.gqa": functions fwd and bwd).  With
 * n_rep = H / H_kv and the head axis of the expanded tensors viewed as
 * (H_kv, n_rep), n_rep fastest:
 *
 *   la_gqa_expand:  k_out[b, g*n_rep + r] = k[b, g]          (same for v)
 *   la_gqa_reduce:  gk_out[b, g] = sum_{r < n_rep} grad_k[b, g*n_rep + r]
 *
 * for every b < B, g < H_kv, r < n_rep and every (n, d).  The expansion is a
 * byte copy; the reduction is the exact sum rounded once to the storage type
 * (round to nearest even), which holds whenever the n_rep summands' binary
 * exponents span fewer than 29 - log2(n_rep) bits (their float64 sum is then
 * exact).  The attention entry points of linattn.h never need these: they
 * map heads by index.  They serve callers that want the expanded heads.
 *
 * Layout: row-major, contiguous.  k, v, gk_out, gv_out: [B, H_kv, N, D];
 * k_out, v_out, grad_k, grad_v: [B, H, N, D].  dtype is LA_F32 or LA_BF16
 * (la_dtype of linattn.h), the same for every tensor of a call.  Pointers
 * must be aligned to the element size; 16-byte aligned pointers with
 * N*D*element_size a multiple of 16 take the vector path.
 *
 * Ownership and execution: all pointers are caller-owned device memory; the
 * library allocates nothing and only enqueues on `stream` (a hipStream_t,
 * NULL = the null stream).  Inputs are read only; outputs are fully written
 * and must not overlap any input or each other.  The v pair is optional:
 * pass v and v_out (or grad_v and gv_out) both NULL to process k alone.
 *
 * Errors (la_status of linattn.h; la_last_error() gives the reason): every
 * check runs before any launch.  LA_ERR_INVALID for a non-positive size,
 * H not a multiple of H_kv, an unknown dtype, a NULL k pointer, exactly one
 * of the v pair NULL, or a misaligned pointer; LA_ERR_UNSUPPORTED when
 * B * H_kv exceeds 65535 (one grid row per KV slab); LA_ERR_HIP when the
 * launch fails.
 */
#ifndef LA_GQA_H
#define LA_GQA_H

#include "linattn.h"

#ifdef __cplusplus
extern "C" {
#endif

la_status la_gqa_expand(const void *k, const void *v, void *k_out, void *v_out, int B, int H_kv,
                        int H, int N, int D, int dtype, void *stream);

la_status la_gqa_reduce(const void *grad_k, const void *grad_v, void *gk_out, void *gv_out, int B,
                        int H_kv, int H, int N, int D, int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_GQA_H */
