// la_kernels.h -- entry points of the kernel translation units, called by the
// C-ABI front end after it has validated the arguments and laid out the
// workspace.
#pragma once

#include "la_common.h"

namespace la {

// Float32 vector-ALU path: every dtype / D / mode / feature map.
hipError_t generic_run(const Args &a, int bf16, int bwd, int causal, int phi, hipStream_t s);

// Per-segment state records ([n_units][nseg + 1][SD] floats, segment s in
// slot s).  causal: replaced in place by their exclusive prefix over segments
// (the last segment's record is not read).  Bidirectional: their total into
// slot nseg (the per-segment slots are left as they are).
hipError_t scan_state(float *ws, int nseg, size_t SD, unsigned n_units, bool causal, hipStream_t s);

// Per-segment (R, r) records ([H units][nseg][SD], n_rep consecutive units
// summed per output unit) into [n_units][nseg + 1][SD]: causal, the exclusive
// suffix over segments in slots 0 .. nseg-1; bidirectional, the total in slot
// nseg.
hipError_t scan_suffix(const float *Rp, float *Rs, int nseg, size_t SD, int H, int Hkv, int nrep,
                       unsigned n_units, bool causal, hipStream_t s);

// bf16 matrix-core kernels, causal and bidirectional (one workgroup per
// batch, KV head, segment).
bool mfma_fwd_serves(int bf16, int D);
hipError_t mfma_fwd_run(const Args &a, int phi, int causal, hipStream_t s);
// per-segment state sums + exclusive prefix and total (the first two steps of both passes)
hipError_t mfma_state_run(const Args &a, int phi, int causal, hipStream_t s);
// backward: causal and bidirectional with F = D; causal with the cos/sin
// features (F = 2D, la_mfma_bwd_cos.hip)
bool mfma_bwd_serves(int bf16, int causal, int D, int has_cos);
hipError_t mfma_bwd_run(const Args &a, int phi, int causal, hipStream_t s);
hipError_t mfma_bwd_cos_run(const Args &a, int phi, int causal, hipStream_t s);
// Segments per bidirectional dk/dv workgroup: such a workgroup first stages
// the whole total (R, r), so the fewest workgroups per (batch, KV head) unit
// that still give every compute unit one, the segments spread evenly.
int bidir_segments_per_wg(int nseg, unsigned n_units);

// float32 bidirectional kernels on the matrix cores (F = D in {64, 128}):
// the float32 path's plan, workspace layout and scans.
bool mfma_f32_serves(int bf16, int causal, int D, int has_cos);
hipError_t mfma_f32_run(const Args &a, int bwd, int phi, hipStream_t s);

// Low-rank projection (la_lowrank.hip): bf16 tensors, fp32 scratch in the workspace.
struct LowRankArgs {
    const unsigned short *x, *U, *V, *bias, *g;   // bf16 inputs (bias, g optional per pass)
    unsigned short *y, *gx, *gU, *gV, *gbias;     // bf16 outputs (gbias optional)
    unsigned short *t, *gt;                        // bf16 [M][rank] intermediates
    float *part, *bpart;                // split partials, bias partials
    int M, n_in, rank, n_out;
};
int lowrank_splits(int M, int rows, int cols);   // K splits of a token-axis product
int lowrank_bias_blocks(int M);                  // row blocks of the bias sum
hipError_t lowrank_fwd_run(const LowRankArgs &a, hipStream_t s);
hipError_t lowrank_bwd_run(const LowRankArgs &a, hipStream_t s);

// Materialised GQA head expansion / n_rep sum (la_gqa.hip); v / vo NULL = k only.
hipError_t gqa_expand_run(const void *k, const void *v, void *ko, void *vo, int B, int Hkv, int H,
                          long long slab_elems, int bf16, hipStream_t s);
hipError_t gqa_reduce_run(const void *gk, const void *gv, void *ko, void *vo, int B, int Hkv, int H,
                          long long slab_elems, int bf16, hipStream_t s);

}  // namespace la
