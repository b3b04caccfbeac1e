/*
 * linattn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU statement of fused feature-map linear attention,
 * forward and backward.  It exists to check the GPU library: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg load it.  It
 * shares no code, header, table or helper with the GPU path, and the GPU
 * path never calls it.
 *
 * What it follows (SVD_linear_Attention API pages):
 *  - "Module neuralops.core.triton_kernels.linear_attn", module docstring:
 *    feature maps phi in {elu+1, relu, identity}; chunked causal streaming;
 *    bidirectional reduction; cosformer-style cos/sin modulation.
 *  - same page, function fwd: arguments is_causal, phi, eps (default 1e-6),
 *    cos_weight, sin_weight.
 *  - same page, function bwd: the gradient is autograd of fwd with respect to
 *    q, k and v only (three gradients; none for cos/sin/eps).
 *  - "Module neuralops.core.triton_kernels.gqa", function bwd: the head axis
 *    of the expanded tensors is viewed as (H_kv, n_rep) with n_rep fastest,
 *    so query head h reads KV head h / n_rep, and KV gradients are the sum
 *    over the n_rep query heads of a group.
 *
 * The pages print no formula.  The plain reading of the docstring, used
 * here, is kernelised attention with a non-negative feature map:
 *
 *   Phi(x_t) = phi(x_t)                            (F = D)
 *   Phi(x_t) = [cos_t * phi(x_t), sin_t * phi(x_t)] (F = 2D, cos/sin given)
 *   S_i = sum_{j in J(i)} Phi(k_j) v_j^T   (F x D)
 *   z_i = sum_{j in J(i)} Phi(k_j)         (F)
 *   out_i = Phi(q_i)^T S_i / (Phi(q_i) . z_i + eps)
 *
 * with J(i) = {0..i} when causal (diagonal included) and {0..N-1} otherwise.
 * eps is added once, after the cos and sin branches are summed.  There is no
 * 1/sqrt(D) scale.  Layout: q, grad_out, out, dq are [B,H,N,D]; k, v, dk, dv
 * are [B,H_kv,N,D]; cos/sin are [N]; all row-major and contiguous.
 *
 * Backward (the exact derivative of the forward; derivation in the comments
 * of oracle_bwd):  with g_i = dL/dout_i,
 *   gn_i = g_i / den_i,   c_i = (g_i . out_i) / den_i
 *   dPhi(q_i) = S_i gn_i - c_i z_i
 *   dPhi(k_j) = R_j v_j - r_j,   dv_j = R_j^T Phi(k_j)
 *   R_j = sum_{i : j in J(i)} Phi(q_i) gn_i^T,   r_j = sum_{i : j in J(i)} c_i Phi(q_i)
 * then the chain rule through cos/sin and phi'.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC -o liboracle.so linattn_oracle.c -lm
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

enum { PHI_ELU1 = 0, PHI_RELU = 1, PHI_IDENTITY = 2 };

/* phi and its derivative (linear_attn page, module docstring: the three named
 * feature maps).  elu uses alpha = 1, so elu(x)+1 = x+1 for x > 0 and e^x
 * otherwise; both one-sided slopes are 1 at 0.  relu'(0) = 0, the autograd
 * convention the bwd function inherits. */
static double phi_val(int phi, double x)
{
    if (phi == PHI_ELU1) return x > 0.0 ? x + 1.0 : exp(x);
    if (phi == PHI_RELU) return x > 0.0 ? x : 0.0;
    return x;
}

static double phi_der(int phi, double x)
{
    if (phi == PHI_ELU1) return x > 0.0 ? 1.0 : exp(x);
    if (phi == PHI_RELU) return x > 0.0 ? 1.0 : 0.0;
    return 1.0;
}

/* Feature vector of one token at position t (length F). */
static void features(int phi, const double *x, int D, const double *cw,
                     const double *sw, int t, double *out)
{
    for (int d = 0; d < D; ++d) {
        double f = phi_val(phi, x[d]);
        if (cw) {
            out[d] = cw[t] * f;
            out[D + d] = sw[t] * f;
        } else {
            out[d] = f;
        }
    }
}

/* dL/dx of one token from dL/dPhi (chain rule through cos/sin and phi). */
static void chain(int phi, const double *x, int D, const double *cw,
                  const double *sw, int t, const double *dPhi, double *dx,
                  int accumulate)
{
    for (int d = 0; d < D; ++d) {
        double gphi = cw ? cw[t] * dPhi[d] + sw[t] * dPhi[D + d] : dPhi[d];
        double val = phi_der(phi, x[d]) * gphi;
        dx[d] = accumulate ? dx[d] + val : val;
    }
}

static int check_args(int B, int H, int Hkv, int N, int D, int phi,
                      const double *cw, const double *sw)
{
    if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || D <= 0) return 1;
    if (H % Hkv != 0) return 1;
    if ((cw == NULL) != (sw == NULL)) return 1;
    if (phi < PHI_ELU1 || phi > PHI_IDENTITY) return 1;
    return 0;
}

/* S += a b^T (F x D), z += a */
static void rank1(double *S, double *z, const double *a, const double *b,
                  int F, int D)
{
    for (int f = 0; f < F; ++f) {
        double af = a[f];
        double *row = S + (size_t)f * D;
        for (int d = 0; d < D; ++d) row[d] += af * b[d];
        if (z) z[f] += af;
    }
}

/* ------------------------------------------------------------------------
 * Forward, token by token (the definition).  den_out (optional, [B,H,N])
 * receives Phi(q_i).z_i + eps.
 * ---------------------------------------------------------------------- */
int oracle_fwd(const double *q, const double *k, const double *v, double *out,
               double *den_out, int B, int H, int Hkv, int N, int D,
               int causal, int phi, double eps, const double *cw,
               const double *sw)
{
    if (check_args(B, H, Hkv, N, D, phi, cw, sw)) return 1;
    const int F = cw ? 2 * D : D;
    const int nrep = H / Hkv;
    int fail = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H, g = h / nrep;
        const double *qh = q + (size_t)(b * H + h) * N * D;
        const double *kh = k + (size_t)(b * Hkv + g) * N * D;
        const double *vh = v + (size_t)(b * Hkv + g) * N * D;
        double *oh = out + (size_t)(b * H + h) * N * D;
        double *S = calloc((size_t)F * D, sizeof(double));
        double *z = calloc((size_t)F, sizeof(double));
        double *qf = malloc(sizeof(double) * F);
        double *kf = malloc(sizeof(double) * F);
        if (!S || !z || !qf || !kf) {
            fail = 1;
        } else {
            if (!causal) {
                for (int j = 0; j < N; ++j) {
                    features(phi, kh + (size_t)j * D, D, cw, sw, j, kf);
                    rank1(S, z, kf, vh + (size_t)j * D, F, D);
                }
            }
            for (int i = 0; i < N; ++i) {
                if (causal) {
                    features(phi, kh + (size_t)i * D, D, cw, sw, i, kf);
                    rank1(S, z, kf, vh + (size_t)i * D, F, D);
                }
                features(phi, qh + (size_t)i * D, D, cw, sw, i, qf);
                double den = eps;
                for (int f = 0; f < F; ++f) den += qf[f] * z[f];
                double *o = oh + (size_t)i * D;
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                for (int f = 0; f < F; ++f) {
                    const double *row = S + (size_t)f * D;
                    for (int d = 0; d < D; ++d) o[d] += qf[f] * row[d];
                }
                for (int d = 0; d < D; ++d) o[d] /= den;
                if (den_out) den_out[(size_t)(b * H + h) * N + i] = den;
            }
        }
        free(S); free(z); free(qf); free(kf);
    }
    return fail ? 2 : 0;
}

/* ------------------------------------------------------------------------
 * Backward, token by token: the exact gradient of oracle_fwd.
 *
 * Derivation.  out_i = num_i / den_i with num_i = sum_j w_ij v_j,
 * den_i = sum_j w_ij + eps, w_ij = Phi(q_i).Phi(k_j) for j in J(i).
 *   dL/dnum_i = g_i / den_i = gn_i,   dL/dden_i = -(g_i.out_i)/den_i = -c_i
 *   dL/dw_ij  = gn_i.v_j - c_i
 *   dL/dPhi(q_i) = sum_{j in J(i)} Phi(k_j)(gn_i.v_j - c_i) = S_i gn_i - c_i z_i
 *   dL/dPhi(k_j) = sum_{i: j in J(i)} Phi(q_i)(gn_i.v_j - c_i) = R_j v_j - r_j
 *   dL/dv_j      = sum_{i: j in J(i)} w_ij gn_i = R_j^T Phi(k_j)
 * KV gradients of a group are accumulated over its query heads in the order
 * r = 0 .. n_rep-1 (gqa page, bwd: sum over the n_rep axis).
 * ---------------------------------------------------------------------- */
int oracle_bwd(const double *q, const double *k, const double *v,
               const double *gout, double *dq, double *dk, double *dv, int B,
               int H, int Hkv, int N, int D, int causal, int phi, double eps,
               const double *cw, const double *sw)
{
    if (check_args(B, H, Hkv, N, D, phi, cw, sw)) return 1;
    const int F = cw ? 2 * D : D;
    const int nrep = H / Hkv;
    int fail = 0;
    /* each query head's share of dk and dv, summed per group afterwards */
    double *dk_h = malloc(sizeof(double) * (size_t)B * H * N * D);
    double *dv_h = malloc(sizeof(double) * (size_t)B * H * N * D);
    if (!dk_h || !dv_h) {
        free(dk_h); free(dv_h);
        return 2;
    }

#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H, g = h / nrep;
        const double *qh = q + (size_t)bh * N * D;
        const double *gh = gout + (size_t)bh * N * D;
        const double *kh = k + (size_t)(b * Hkv + g) * N * D;
        const double *vh = v + (size_t)(b * Hkv + g) * N * D;
        double *dqh = dq + (size_t)bh * N * D;
        double *dkh = dk_h + (size_t)bh * N * D;
        double *dvh = dv_h + (size_t)bh * N * D;
        double *S = malloc(sizeof(double) * (size_t)F * D);
        double *z = malloc(sizeof(double) * F);
        double *qf = malloc(sizeof(double) * (size_t)N * F);
        double *gn = malloc(sizeof(double) * (size_t)N * D);
        double *c = malloc(sizeof(double) * N);
        double *kf = malloc(sizeof(double) * F);
        double *tmp = malloc(sizeof(double) * F);
        double *o = malloc(sizeof(double) * D);
        if (!S || !z || !qf || !gn || !c || !kf || !tmp || !o) {
            fail = 1;
            goto done;
        }

        /* forward sweep: den, out, gn, c and dq */
        memset(S, 0, sizeof(double) * (size_t)F * D);
        memset(z, 0, sizeof(double) * F);
        if (!causal) {
            for (int j = 0; j < N; ++j) {
                features(phi, kh + (size_t)j * D, D, cw, sw, j, kf);
                rank1(S, z, kf, vh + (size_t)j * D, F, D);
            }
        }
        for (int i = 0; i < N; ++i) {
            if (causal) {
                features(phi, kh + (size_t)i * D, D, cw, sw, i, kf);
                rank1(S, z, kf, vh + (size_t)i * D, F, D);
            }
            double *qfi = qf + (size_t)i * F;
            features(phi, qh + (size_t)i * D, D, cw, sw, i, qfi);
            double den = eps;
            for (int f = 0; f < F; ++f) den += qfi[f] * z[f];
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            for (int f = 0; f < F; ++f) {
                const double *row = S + (size_t)f * D;
                for (int d = 0; d < D; ++d) o[d] += qfi[f] * row[d];
            }
            const double *gi = gh + (size_t)i * D;
            double *gni = gn + (size_t)i * D;
            double go = 0.0;
            for (int d = 0; d < D; ++d) {
                o[d] /= den;
                go += gi[d] * o[d];
                gni[d] = gi[d] / den;
            }
            c[i] = go / den;
            for (int f = 0; f < F; ++f) {
                const double *row = S + (size_t)f * D;
                double acc = 0.0;
                for (int d = 0; d < D; ++d) acc += row[d] * gni[d];
                tmp[f] = acc - c[i] * z[f];
            }
            chain(phi, qh + (size_t)i * D, D, cw, sw, i, tmp, dqh + (size_t)i * D, 0);
        }

        /* reverse sweep: R, r and this head's share of dk, dv */
        double *R = S, *rv = z;
        memset(R, 0, sizeof(double) * (size_t)F * D);
        memset(rv, 0, sizeof(double) * F);
        if (!causal) {
            for (int i = 0; i < N; ++i) {
                rank1(R, NULL, qf + (size_t)i * F, gn + (size_t)i * D, F, D);
                for (int f = 0; f < F; ++f) rv[f] += c[i] * qf[(size_t)i * F + f];
            }
        }
        for (int j = N - 1; j >= 0; --j) {
            if (causal) {
                rank1(R, NULL, qf + (size_t)j * F, gn + (size_t)j * D, F, D);
                for (int f = 0; f < F; ++f) rv[f] += c[j] * qf[(size_t)j * F + f];
            }
            features(phi, kh + (size_t)j * D, D, cw, sw, j, kf);
            const double *vj = vh + (size_t)j * D;
            for (int f = 0; f < F; ++f) {
                const double *row = R + (size_t)f * D;
                double acc = 0.0;
                for (int d = 0; d < D; ++d) acc += row[d] * vj[d];
                tmp[f] = acc - rv[f];
            }
            double *dvj = dvh + (size_t)j * D;
            for (int d = 0; d < D; ++d) dvj[d] = 0.0;
            for (int f = 0; f < F; ++f) {
                const double *row = R + (size_t)f * D;
                for (int d = 0; d < D; ++d) dvj[d] += row[d] * kf[f];
            }
            chain(phi, kh + (size_t)j * D, D, cw, sw, j, tmp, dkh + (size_t)j * D, 0);
        }
    done:
        free(S); free(z); free(qf); free(gn); free(c); free(kf); free(tmp);
        free(o);
    }

    /* dk, dv of a KV head: its query heads' shares summed in order r = 0.. */
#pragma omp parallel for schedule(static)
    for (int bg = 0; bg < B * Hkv; ++bg) {
        const int b = bg / Hkv, g = bg % Hkv;
        double *dkg = dk + (size_t)bg * N * D;
        double *dvg = dv + (size_t)bg * N * D;
        for (size_t e = 0; e < (size_t)N * D; ++e) {
            double sk = 0.0, sv = 0.0;
            for (int r = 0; r < nrep; ++r) {
                const size_t bh = (size_t)b * H + (size_t)g * nrep + r;
                sk += dk_h[bh * N * D + e];
                sv += dv_h[bh * N * D + e];
            }
            dkg[e] = sk;
            dvg[e] = sv;
        }
    }
    free(dk_h);
    free(dv_h);
    return fail ? 2 : 0;
}

/* ------------------------------------------------------------------------
 * Chunk form of the forward (linear_attn page, module docstring: "chunked
 * causal streaming"; "bidirectional parallel reduction").
 *
 * Causal: rows are cut into chunks of C.  Each row takes the masked
 * intra-chunk sum over keys j <= i of its own chunk plus the state (S, z)
 * carried from all earlier chunks (exclusive); the state then absorbs the
 * chunk.  Bidirectional: (S, z) is the sum of per-chunk partial sums, then a
 * row pass.  In exact arithmetic both equal oracle_fwd.
 * ---------------------------------------------------------------------- */
int oracle_fwd_chunked(const double *q, const double *k, const double *v,
                       double *out, int B, int H, int Hkv, int N, int D,
                       int causal, int phi, double eps, const double *cw,
                       const double *sw, int C)
{
    if (check_args(B, H, Hkv, N, D, phi, cw, sw) || C <= 0) return 1;
    const int F = cw ? 2 * D : D;
    const int nrep = H / Hkv;
    int fail = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H, g = h / nrep;
        const double *qh = q + (size_t)(b * H + h) * N * D;
        const double *kh = k + (size_t)(b * Hkv + g) * N * D;
        const double *vh = v + (size_t)(b * Hkv + g) * N * D;
        double *oh = out + (size_t)(b * H + h) * N * D;
        double *S = calloc((size_t)F * D, sizeof(double));
        double *z = calloc((size_t)F, sizeof(double));
        double *dS = calloc((size_t)F * D, sizeof(double));
        double *dz = calloc((size_t)F, sizeof(double));
        double *qf = malloc(sizeof(double) * (size_t)C * F);
        double *kf = malloc(sizeof(double) * (size_t)C * F);
        if (!S || !z || !dS || !dz || !qf || !kf) {
            fail = 1;
            goto done;
        }
        if (!causal) {
            for (int c0 = 0; c0 < N; c0 += C) {
                const int c1 = c0 + C < N ? c0 + C : N;
                memset(dS, 0, sizeof(double) * (size_t)F * D);
                memset(dz, 0, sizeof(double) * F);
                for (int j = c0; j < c1; ++j) {
                    features(phi, kh + (size_t)j * D, D, cw, sw, j, kf);
                    rank1(dS, dz, kf, vh + (size_t)j * D, F, D);
                }
                for (size_t e = 0; e < (size_t)F * D; ++e) S[e] += dS[e];
                for (int f = 0; f < F; ++f) z[f] += dz[f];
            }
        }
        for (int c0 = 0; c0 < N; c0 += C) {
            const int c1 = c0 + C < N ? c0 + C : N;
            for (int t = c0; t < c1; ++t) {
                features(phi, qh + (size_t)t * D, D, cw, sw, t, qf + (size_t)(t - c0) * F);
                features(phi, kh + (size_t)t * D, D, cw, sw, t, kf + (size_t)(t - c0) * F);
            }
            for (int i = c0; i < c1; ++i) {
                const double *qfi = qf + (size_t)(i - c0) * F;
                double *o = oh + (size_t)i * D;
                double den = eps;
                for (int f = 0; f < F; ++f) den += qfi[f] * z[f];
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                for (int f = 0; f < F; ++f) {
                    const double *row = S + (size_t)f * D;
                    for (int d = 0; d < D; ++d) o[d] += qfi[f] * row[d];
                }
                if (causal) {
                    for (int j = c0; j <= i; ++j) {
                        const double *kfj = kf + (size_t)(j - c0) * F;
                        double a = 0.0;
                        for (int f = 0; f < F; ++f) a += qfi[f] * kfj[f];
                        const double *vj = vh + (size_t)j * D;
                        for (int d = 0; d < D; ++d) o[d] += a * vj[d];
                        den += a;
                    }
                }
                for (int d = 0; d < D; ++d) o[d] /= den;
            }
            if (causal) {
                for (int j = c0; j < c1; ++j)
                    rank1(S, z, kf + (size_t)(j - c0) * F, vh + (size_t)j * D, F, D);
            }
        }
    done:
        free(S); free(z); free(dS); free(dz); free(qf); free(kf);
    }
    return fail ? 2 : 0;
}

/* ------------------------------------------------------------------------
 * Chunk form of the backward.  Same result as oracle_bwd in exact
 * arithmetic; it states the chunk algebra a chunked GPU kernel follows.
 *
 * Causal, per query head, forward over chunks with exclusive (S, z):
 *   A_ij = Phi(q_i).Phi(k_j), T_ij = g_i.v_j         (j <= i, same chunk)
 *   den_i = sum_j A_ij + Phi(q_i).z + eps
 *   U_i   = S g_i                                   (F)
 *   c_i   = (sum_j A_ij T_ij + Phi(q_i).U_i) / den_i^2
 *   P_ij  = T_ij / den_i - c_i                      (j <= i)
 *   dPhi(q_i) = sum_j P_ij Phi(k_j) + U_i / den_i - c_i z
 * then, backward over chunks with the exclusive suffix (R, r) summed over
 * the group's query heads:
 *   dPhi(k_j) = sum_{heads} sum_{i >= j} P_ij Phi(q_i) + R v_j - r
 *   dv_j      = sum_{heads} sum_{i >= j} A_ij gn_i + R^T Phi(k_j)
 *   R += sum_{heads} sum_i Phi(q_i) gn_i^T,  r += sum_{heads} sum_i c_i Phi(q_i)
 * Bidirectional: (S, z) and (R, r) are sums of per-chunk partial sums and
 * every row takes the full-sum terms only.
 * ---------------------------------------------------------------------- */
int oracle_bwd_chunked(const double *q, const double *k, const double *v,
                       const double *gout, double *dq, double *dk, double *dv,
                       int B, int H, int Hkv, int N, int D, int causal,
                       int phi, double eps, const double *cw, const double *sw,
                       int C)
{
    if (check_args(B, H, Hkv, N, D, phi, cw, sw) || C <= 0) return 1;
    const int F = cw ? 2 * D : D;
    const int nrep = H / Hkv;
    int fail = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int bg = 0; bg < B * Hkv; ++bg) {
        const int b = bg / Hkv, g = bg % Hkv;
        const double *kh = k + (size_t)bg * N * D;
        const double *vh = v + (size_t)bg * N * D;
        double *dkh = dk + (size_t)bg * N * D;
        double *dvh = dv + (size_t)bg * N * D;
        /* per group: features of all heads' q, gn, c, den; features of k */
        double *qf = malloc(sizeof(double) * (size_t)nrep * N * F);
        double *gn = malloc(sizeof(double) * (size_t)nrep * N * D);
        double *cc = malloc(sizeof(double) * (size_t)nrep * N);
        double *kf = malloc(sizeof(double) * (size_t)N * F);
        double *S = malloc(sizeof(double) * (size_t)F * D);
        double *z = malloc(sizeof(double) * F);
        double *U = malloc(sizeof(double) * F);
        double *tmp = malloc(sizeof(double) * F);
        double *dKf = malloc(sizeof(double) * (size_t)N * F);
        double *dS = malloc(sizeof(double) * (size_t)F * D);
        double *dz = malloc(sizeof(double) * F);
        if (!qf || !gn || !cc || !kf || !S || !z || !U || !tmp || !dKf || !dS || !dz) {
            fail = 1;
            goto done;
        }
        for (int j = 0; j < N; ++j)
            features(phi, kh + (size_t)j * D, D, cw, sw, j, kf + (size_t)j * F);

        /* forward pass over chunks, per head: den, c, gn, dq */
        for (int r = 0; r < nrep; ++r) {
            const int h = g * nrep + r;
            const double *qh = q + (size_t)(b * H + h) * N * D;
            const double *gh = gout + (size_t)(b * H + h) * N * D;
            double *dqh = dq + (size_t)(b * H + h) * N * D;
            double *qfh = qf + (size_t)r * N * F;
            double *gnh = gn + (size_t)r * N * D;
            double *ch = cc + (size_t)r * N;
            for (int i = 0; i < N; ++i)
                features(phi, qh + (size_t)i * D, D, cw, sw, i, qfh + (size_t)i * F);
            memset(S, 0, sizeof(double) * (size_t)F * D);
            memset(z, 0, sizeof(double) * F);
            if (!causal) {
                for (int c0 = 0; c0 < N; c0 += C) {
                    const int c1 = c0 + C < N ? c0 + C : N;
                    memset(dS, 0, sizeof(double) * (size_t)F * D);
                    memset(dz, 0, sizeof(double) * F);
                    for (int j = c0; j < c1; ++j)
                        rank1(dS, dz, kf + (size_t)j * F, vh + (size_t)j * D, F, D);
                    for (size_t e = 0; e < (size_t)F * D; ++e) S[e] += dS[e];
                    for (int f = 0; f < F; ++f) z[f] += dz[f];
                }
            }
            for (int c0 = 0; c0 < N; c0 += C) {
                const int c1 = c0 + C < N ? c0 + C : N;
                for (int i = c0; i < c1; ++i) {
                    const double *qfi = qfh + (size_t)i * F;
                    const double *gi = gh + (size_t)i * D;
                    const int jend = causal ? i : c0 - 1; /* intra keys c0..jend */
                    double den = eps, gnum = 0.0;
                    for (int f = 0; f < F; ++f) den += qfi[f] * z[f];
                    for (int j = c0; j <= jend; ++j) {
                        const double *kfj = kf + (size_t)j * F;
                        const double *vj = vh + (size_t)j * D;
                        double a = 0.0, t = 0.0;
                        for (int f = 0; f < F; ++f) a += qfi[f] * kfj[f];
                        for (int d = 0; d < D; ++d) t += gi[d] * vj[d];
                        den += a;
                        gnum += a * t;
                    }
                    for (int f = 0; f < F; ++f) {
                        const double *row = S + (size_t)f * D;
                        double acc = 0.0;
                        for (int d = 0; d < D; ++d) acc += row[d] * gi[d];
                        U[f] = acc;
                        gnum += qfi[f] * acc;
                    }
                    const double ci = gnum / (den * den);
                    ch[i] = ci;
                    for (int d = 0; d < D; ++d) gnh[(size_t)i * D + d] = gi[d] / den;
                    for (int f = 0; f < F; ++f) tmp[f] = U[f] / den - ci * z[f];
                    for (int j = c0; j <= jend; ++j) {
                        const double *kfj = kf + (size_t)j * F;
                        const double *vj = vh + (size_t)j * D;
                        double t = 0.0;
                        for (int d = 0; d < D; ++d) t += gi[d] * vj[d];
                        const double p = t / den - ci;
                        for (int f = 0; f < F; ++f) tmp[f] += p * kfj[f];
                    }
                    chain(phi, qh + (size_t)i * D, D, cw, sw, i, tmp, dqh + (size_t)i * D, 0);
                }
                if (causal) {
                    for (int j = c0; j < c1; ++j)
                        rank1(S, z, kf + (size_t)j * F, vh + (size_t)j * D, F, D);
                }
            }
        }

        /* backward pass over chunks: dk, dv with the suffix state (R, r) */
        double *R = S, *rv = z;
        memset(R, 0, sizeof(double) * (size_t)F * D);
        memset(rv, 0, sizeof(double) * F);
        if (!causal) {
            for (int c0 = 0; c0 < N; c0 += C) {
                const int c1 = c0 + C < N ? c0 + C : N;
                memset(dS, 0, sizeof(double) * (size_t)F * D);
                memset(dz, 0, sizeof(double) * F);
                for (int r = 0; r < nrep; ++r)
                    for (int i = c0; i < c1; ++i) {
                        const double *qfi = qf + ((size_t)r * N + i) * F;
                        rank1(dS, NULL, qfi, gn + ((size_t)r * N + i) * D, F, D);
                        for (int f = 0; f < F; ++f) dz[f] += cc[(size_t)r * N + i] * qfi[f];
                    }
                for (size_t e = 0; e < (size_t)F * D; ++e) R[e] += dS[e];
                for (int f = 0; f < F; ++f) rv[f] += dz[f];
            }
        }
        const int nchunks = (N + C - 1) / C;
        for (int cix = nchunks - 1; cix >= 0; --cix) {
            const int c0 = cix * C;
            const int c1 = c0 + C < N ? c0 + C : N;
            for (int j = c0; j < c1; ++j) {
                const double *kfj = kf + (size_t)j * F;
                const double *vj = vh + (size_t)j * D;
                double *dKfj = dKf + (size_t)j * F;
                double *dvj = dvh + (size_t)j * D;
                for (int f = 0; f < F; ++f) {
                    const double *row = R + (size_t)f * D;
                    double acc = 0.0;
                    for (int d = 0; d < D; ++d) acc += row[d] * vj[d];
                    dKfj[f] = acc - rv[f];
                }
                for (int d = 0; d < D; ++d) dvj[d] = 0.0;
                for (int f = 0; f < F; ++f) {
                    const double *row = R + (size_t)f * D;
                    for (int d = 0; d < D; ++d) dvj[d] += row[d] * kfj[f];
                }
                if (causal) {
                    for (int r = 0; r < nrep; ++r) {
                        for (int i = j; i < c1; ++i) {
                            const double *qfi = qf + ((size_t)r * N + i) * F;
                            const double *gni = gn + ((size_t)r * N + i) * D;
                            /* P_ij = T_ij / den_i - c_i = gn_i.v_j - c_i */
                            double a = 0.0, t = 0.0;
                            for (int f = 0; f < F; ++f) a += qfi[f] * kfj[f];
                            for (int d = 0; d < D; ++d) t += gni[d] * vj[d];
                            const double p = t - cc[(size_t)r * N + i];
                            for (int f = 0; f < F; ++f) dKfj[f] += p * qfi[f];
                            for (int d = 0; d < D; ++d) dvj[d] += a * gni[d];
                        }
                    }
                }
                chain(phi, kh + (size_t)j * D, D, cw, sw, j, dKfj, dkh + (size_t)j * D, 0);
            }
            if (causal) {
                for (int r = 0; r < nrep; ++r)
                    for (int i = c0; i < c1; ++i) {
                        const double *qfi = qf + ((size_t)r * N + i) * F;
                        rank1(R, NULL, qfi, gn + ((size_t)r * N + i) * D, F, D);
                        for (int f = 0; f < F; ++f) rv[f] += cc[(size_t)r * N + i] * qfi[f];
                    }
            }
        }
    done:
        free(qf); free(gn); free(cc); free(kf); free(S); free(z); free(U);
        free(tmp); free(dKf); free(dS); free(dz);
    }
    return fail ? 2 : 0;
}
