/*
 * oracle.c -- plain, sequential, fp64 CPU reference for the minGRU scan engine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file; only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or constant with the GPU
 * path.
 *
 * What it computes (the pages never write the recurrences out; they name the
 * operations and cite their sources):
 *   - minGRU home page (mingru-scans), introduction: minGRU (Feng et al.,
 *     arXiv:2410.01201) is a GRU reduced to the linear recurrence
 *     h_t = a_t * h_{t-1} + b_t, solved by an associative scan; the log-space
 *     baseline uses Heinsen's parallel scan (arXiv:2311.06281).  Heinsen's
 *     log-space evaluation is a re-association of this same recurrence, so the
 *     oracle evaluates the recurrence itself, one step at a time, in fp64.
 *   - The block forms (RotationMinGRU / GivensMinGRU, same page; the scan ops
 *     matrix_affine_scan and matrix_scan in the "Run the benchmarks" how-to,
 *     Step 2 table) replace the scalar a_t by a block-diagonal k x k matrix:
 *     h_t = A_t h_{t-1} + b_t, and the b = 0 product P_t = A_t P_{t-1}, P_0 = I.
 *   - The linear-space elementwise scan (linear_scan in the same page's
 *     speed-up table and in the how-to's Step 2 table; the signed gates of
 *     SignedMinGRU, same page) is the same recurrence with a_t, b_t, h_0 given
 *     directly and a_t of either sign.
 *   - The minGRU cell ahead of the log-space scan (same page, introduction:
 *     minGRU of Feng et al.): from pre-activations k_t, x_t and x_0,
 *     a_t = sigmoid(-k_t), z_t = 1 - a_t, b_t = z_t g(x_t), h_0 = g(x_0), with
 *     g(x) = x + 0.5 for x >= 0 and sigmoid(x) for x < 0 (the pages do not
 *     write g out; this is the reading taken), then the same recurrence.
 *   - The Givens angle-fused block scan (GivensMinGRU, same page; the fused
 *     backward whose memory the how-to's Step 3 measures): A_t per block is
 *     sigmoid(s_t) R(theta_t), R a brick-wall mesh of k layers of disjoint 2 x 2
 *     rotations (Clements et al. / EUNN, cited on the home page): layer l acts
 *     on pairs (i, i+1), i = l mod 2, l mod 2 + 2, ... < k - 1, R = L_{k-1}..L_0,
 *     angles taken in (layer, pair) order, each rotation mapping (x_i, x_j) to
 *     (cos x_i - sin x_j, sin x_i + cos x_j).  The pages name the mesh but do
 *     not fix these conventions; this is the reading taken.
 *   - The delta-rule recurrence of DeltaMinGRU (same page: DeltaMinGRU
 *     reimplements DeltaNet, Yang et al. 2024, arXiv:2406.06484, and uses its
 *     chunked WY representation as the parallel forward).  The pages do not
 *     write the recurrence out; the reading taken is DeltaNet's delta rule
 *     with a matrix state S (dv x dk):
 *         S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T,   o_t = S_t q_t,
 *     i.e. S_t = S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.  The
 *     chunked WY form is a re-association of this loop (exact in real
 *     arithmetic), so the oracle runs the loop itself.
 *   - Gradients are the chain rule applied to these loops for the loss
 *     L = sum_t <dh_t, h_t> (resp. sum_t <dP_t, P_t>).
 *
 * Layouts (row-major, last index fastest):
 *   log scan:   la, lb, h, dh, dla, dlb : (B, T, d);  lh0, dlh0 : (B, d)
 *   linear scan: a, b, h, dh, da, db : (B, T, d);  h0, dh0 : (B, d)
 *   minGRU cell: k, x, h, dh, dk, dx : (B, T, d);  x0, dx0 : (B, d)
 *   Givens scan: theta, dtheta : (B, T, nb, k(k-1)/2);  s, ds : (B, T, nb);
 *                b, h, dh, db : (B, T, d);  h0, dh0 : (B, d)
 *   block ops:  A, dA, P, dP : (B, T, nb, k, k) with nb = d / k and
 *               (A h)_r = sum_c A[r][c] h[c];  b, h, dh, db : (B, T, d);
 *               h0, dh0 : (B, d);  block j owns channels [j*k, (j+1)*k).
 *   delta rule: q, k : (B, T, dk);  v, o : (B, T, dv);  beta : (B, T);
 *               S0, ST : (B, dv, dk), (S k)_r = sum_c S[r][c] k[c].
 * Inputs are the same fp32 arrays the GPU sees, widened exactly to double.
 * Loops over t are sequential; there is no blocking, fusion or reordering.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- log scan */

/* Forward: h_0 = exp(lh0); h_t = exp(la_t) h_{t-1} + exp(lb_t); writes h_1..T. */
void oracle_log_fwd(const double *la, const double *lb, const double *lh0,
                    double *h, int64_t B, int64_t T, int64_t d)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < d; ++c) {
            double hp = exp(lh0[b * d + c]);
            for (int64_t t = 0; t < T; ++t) {
                int64_t i = (b * T + t) * d + c;
                hp = exp(la[i]) * hp + exp(lb[i]);
                h[i] = hp;
            }
        }
}

/* Backward of oracle_log_fwd under upstream dh = dL/dh_t:
 *   g_T = dh_T,  g_t = dh_t + a_{t+1} g_{t+1}          (g_t = dL/dh_t total)
 *   dla_t = g_t a_t h_{t-1},  dlb_t = g_t b_t,  dlh0 = g_1 a_1 h_0
 * (d h_t / d log a_t = a_t h_{t-1}, d h_t / d log b_t = b_t,
 *  d h_1 / d log h_0 = a_1 h_0). */
void oracle_log_bwd(const double *la, const double *lb, const double *lh0,
                    const double *dh, double *dla, double *dlb, double *dlh0,
                    int64_t B, int64_t T, int64_t d)
{
    double *hs = (double *)malloc(sizeof(double) * (size_t)(T + 1));
    if (!hs) return;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < d; ++c) {
            /* hs[t] = h_t for t = 0..T (hs[0] = h_0) */
            hs[0] = exp(lh0[b * d + c]);
            for (int64_t t = 0; t < T; ++t) {
                int64_t i = (b * T + t) * d + c;
                hs[t + 1] = exp(la[i]) * hs[t] + exp(lb[i]);
            }
            double g = 0.0; /* g_{t+1}, zero past the end */
            double a_next = 0.0;
            for (int64_t t = T - 1; t >= 0; --t) {
                int64_t i = (b * T + t) * d + c;
                g = dh[i] + a_next * g;
                double a = exp(la[i]);
                dla[i] = g * a * hs[t];
                dlb[i] = g * exp(lb[i]);
                a_next = a;
            }
            /* here g = g_1 and a_next = a_1 */
            dlh0[b * d + c] = (T > 0) ? g * a_next * hs[0] : 0.0;
        }
    free(hs);
}

/* ------------------------------------------------------------- linear scan */

/* Forward: h_0 = h0; h_t = a_t h_{t-1} + b_t (a_t of either sign); writes h_1..T. */
void oracle_linear_fwd(const double *a, const double *bv, const double *h0,
                       double *h, int64_t B, int64_t T, int64_t d)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < d; ++c) {
            double hp = h0[b * d + c];
            for (int64_t t = 0; t < T; ++t) {
                int64_t i = (b * T + t) * d + c;
                hp = a[i] * hp + bv[i];
                h[i] = hp;
            }
        }
}

/* Backward of oracle_linear_fwd under upstream dh = dL/dh_t:
 *   g_T = dh_T,  g_t = dh_t + a_{t+1} g_{t+1}
 *   da_t = g_t h_{t-1},  db_t = g_t,  dh0 = a_1 g_1. */
void oracle_linear_bwd(const double *a, const double *bv, const double *h0,
                       const double *dh, double *da, double *db, double *dh0,
                       int64_t B, int64_t T, int64_t d)
{
    double *hs = (double *)malloc(sizeof(double) * (size_t)(T + 1));
    if (!hs) return;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < d; ++c) {
            hs[0] = h0[b * d + c];
            for (int64_t t = 0; t < T; ++t) {
                int64_t i = (b * T + t) * d + c;
                hs[t + 1] = a[i] * hs[t] + bv[i];
            }
            double g = 0.0, a_next = 0.0;
            for (int64_t t = T - 1; t >= 0; --t) {
                int64_t i = (b * T + t) * d + c;
                g = dh[i] + a_next * g;
                da[i] = g * hs[t];
                db[i] = g;
                a_next = a[i];
            }
            dh0[b * d + c] = (T > 0) ? a_next * g : 0.0;
        }
    free(hs);
}

/* ------------------------------------------------------ minGRU cell + scan */

static double sigm(double u) { return 1.0 / (1.0 + exp(-u)); }

/* g(x) = x + 0.5 (x >= 0), sigmoid(x) (x < 0), and its derivative */
static double gpos(double x) { return x >= 0.0 ? x + 0.5 : sigm(x); }
static double gpos_d(double x) { return x >= 0.0 ? 1.0 : sigm(x) * (1.0 - sigm(x)); }

/* Forward: a_t = sigmoid(-k_t), b_t = (1 - a_t) g(x_t), h_0 = g(x_0);
 * h_t = a_t h_{t-1} + b_t; writes h_1..T. */
void oracle_mingru_fwd(const double *k, const double *x, const double *x0,
                       double *h, int64_t B, int64_t T, int64_t d)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < d; ++c) {
            double hp = gpos(x0[b * d + c]);
            for (int64_t t = 0; t < T; ++t) {
                int64_t i = (b * T + t) * d + c;
                double a = sigm(-k[i]);
                hp = a * hp + (1.0 - a) * gpos(x[i]);
                h[i] = hp;
            }
        }
}

/* Backward of oracle_mingru_fwd under upstream dh = dL/dh_t, with
 * g_T = dh_T, g_t = dh_t + a_{t+1} g_{t+1} as for the scan, and
 *   dh_t/dk_t = a_t (1 - a_t) (g(x_t) - h_{t-1})   (da/dk = -a(1-a), dz/dk = a(1-a)),
 *   dh_t/dx_t = (1 - a_t) g'(x_t),   dh_1/dx_0 = a_1 g'(x_0). */
void oracle_mingru_bwd(const double *k, const double *x, const double *x0,
                       const double *dh, double *dk, double *dx, double *dx0,
                       int64_t B, int64_t T, int64_t d)
{
    double *hs = (double *)malloc(sizeof(double) * (size_t)(T + 1));
    if (!hs) return;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < d; ++c) {
            hs[0] = gpos(x0[b * d + c]);
            for (int64_t t = 0; t < T; ++t) {
                int64_t i = (b * T + t) * d + c;
                double a = sigm(-k[i]);
                hs[t + 1] = a * hs[t] + (1.0 - a) * gpos(x[i]);
            }
            double g = 0.0, a_next = 0.0;
            for (int64_t t = T - 1; t >= 0; --t) {
                int64_t i = (b * T + t) * d + c;
                g = dh[i] + a_next * g;
                double a = sigm(-k[i]);
                dk[i] = g * a * (1.0 - a) * (gpos(x[i]) - hs[t]);
                dx[i] = g * (1.0 - a) * gpos_d(x[i]);
                a_next = a;
            }
            dx0[b * d + c] = (T > 0) ? g * a_next * gpos_d(x0[b * d + c]) : 0.0;
        }
    free(hs);
}

/* ------------------------------------------------------- block-affine scan */

static const double *blk(const double *M, int64_t b, int64_t t, int64_t j,
                         int64_t T, int64_t nb, int64_t k)
{
    return M + (((b * T + t) * nb + j) * k * k);
}

/* Forward: h_0 = h0 (zero if h0 == NULL); h_t = A_t h_{t-1} + b_t, per block. */
void oracle_block_affine_fwd(const double *A, const double *bv, const double *h0,
                             double *h, int64_t B, int64_t T, int64_t d, int64_t k)
{
    int64_t nb = d / k;
    double *cur = (double *)malloc(sizeof(double) * (size_t)k);
    double *nxt = (double *)malloc(sizeof(double) * (size_t)k);
    if (!cur || !nxt) { free(cur); free(nxt); return; }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < nb; ++j) {
            for (int64_t r = 0; r < k; ++r)
                cur[r] = h0 ? h0[b * d + j * k + r] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double *At = blk(A, b, t, j, T, nb, k);
                for (int64_t r = 0; r < k; ++r) {
                    double s = bv[(b * T + t) * d + j * k + r];
                    for (int64_t c = 0; c < k; ++c) s += At[r * k + c] * cur[c];
                    nxt[r] = s;
                }
                for (int64_t r = 0; r < k; ++r) {
                    cur[r] = nxt[r];
                    h[(b * T + t) * d + j * k + r] = nxt[r];
                }
            }
        }
    free(cur);
    free(nxt);
}

/* Backward of oracle_block_affine_fwd under upstream dh:
 *   g_T = dh_T,  g_t = dh_t + A_{t+1}^T g_{t+1}
 *   dA_t = g_t h_{t-1}^T,  db_t = g_t,  dh0 = A_1^T g_1.
 * h is recomputed here from (A, b, h0). */
void oracle_block_affine_bwd(const double *A, const double *bv, const double *h0,
                             const double *dh, double *dA, double *db, double *dh0,
                             int64_t B, int64_t T, int64_t d, int64_t k)
{
    int64_t nb = d / k;
    double *hs = (double *)malloc(sizeof(double) * (size_t)((T + 1) * k));
    double *g = (double *)malloc(sizeof(double) * (size_t)k);
    double *w = (double *)malloc(sizeof(double) * (size_t)k); /* A_{t+1}^T g_{t+1} */
    if (!hs || !g || !w) { free(hs); free(g); free(w); return; }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < nb; ++j) {
            for (int64_t r = 0; r < k; ++r)
                hs[r] = h0 ? h0[b * d + j * k + r] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double *At = blk(A, b, t, j, T, nb, k);
                for (int64_t r = 0; r < k; ++r) {
                    double s = bv[(b * T + t) * d + j * k + r];
                    for (int64_t c = 0; c < k; ++c) s += At[r * k + c] * hs[t * k + c];
                    hs[(t + 1) * k + r] = s;
                }
            }
            for (int64_t r = 0; r < k; ++r) w[r] = 0.0;
            for (int64_t t = T - 1; t >= 0; --t) {
                for (int64_t r = 0; r < k; ++r)
                    g[r] = dh[(b * T + t) * d + j * k + r] + w[r];
                const double *At = blk(A, b, t, j, T, nb, k);
                double *dAt = dA + (((b * T + t) * nb + j) * k * k);
                for (int64_t r = 0; r < k; ++r) {
                    db[(b * T + t) * d + j * k + r] = g[r];
                    for (int64_t c = 0; c < k; ++c)
                        dAt[r * k + c] = g[r] * hs[t * k + c];
                }
                /* w = A_t^T g_t, used as A_{t}^T g_{t} at step t-1 */
                for (int64_t c = 0; c < k; ++c) {
                    double s = 0.0;
                    for (int64_t r = 0; r < k; ++r) s += At[r * k + c] * g[r];
                    w[c] = s;
                }
            }
            /* after the loop w = A_1^T g_1 (all zeros if T == 0) */
            for (int64_t r = 0; r < k; ++r) dh0[b * d + j * k + r] = w[r];
        }
    free(hs);
    free(g);
    free(w);
}

/* ----------------------------------------- block cumulative product (b = 0) */

/* Forward: P_0 = I; P_t = A_t P_{t-1}; writes P_1..T. */
void oracle_block_matrix_fwd(const double *A, double *P,
                             int64_t B, int64_t T, int64_t d, int64_t k)
{
    int64_t nb = d / k;
    double *cur = (double *)malloc(sizeof(double) * (size_t)(k * k));
    if (!cur) return;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < nb; ++j) {
            for (int64_t r = 0; r < k; ++r)
                for (int64_t c = 0; c < k; ++c) cur[r * k + c] = (r == c) ? 1.0 : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double *At = blk(A, b, t, j, T, nb, k);
                double *Pt = P + (((b * T + t) * nb + j) * k * k);
                for (int64_t r = 0; r < k; ++r)
                    for (int64_t c = 0; c < k; ++c) {
                        double s = 0.0;
                        for (int64_t m = 0; m < k; ++m) s += At[r * k + m] * cur[m * k + c];
                        Pt[r * k + c] = s;
                    }
                memcpy(cur, Pt, sizeof(double) * (size_t)(k * k));
            }
        }
    free(cur);
}

/* Backward of oracle_block_matrix_fwd under upstream dP:
 *   G_T = dP_T,  G_t = dP_t + A_{t+1}^T G_{t+1},  dA_t = G_t P_{t-1}^T.
 * P is recomputed here from A; P_0 = I is a constant (no gradient). */
void oracle_block_matrix_bwd(const double *A, const double *dP, double *dA,
                             int64_t B, int64_t T, int64_t d, int64_t k)
{
    int64_t nb = d / k;
    int64_t kk = k * k;
    double *Ps = (double *)malloc(sizeof(double) * (size_t)((T + 1) * kk));
    double *G = (double *)malloc(sizeof(double) * (size_t)kk);
    double *W = (double *)malloc(sizeof(double) * (size_t)kk); /* A_{t+1}^T G_{t+1} */
    if (!Ps || !G || !W) { free(Ps); free(G); free(W); return; }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < nb; ++j) {
            for (int64_t r = 0; r < k; ++r)
                for (int64_t c = 0; c < k; ++c) Ps[r * k + c] = (r == c) ? 1.0 : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double *At = blk(A, b, t, j, T, nb, k);
                for (int64_t r = 0; r < k; ++r)
                    for (int64_t c = 0; c < k; ++c) {
                        double s = 0.0;
                        for (int64_t m = 0; m < k; ++m) s += At[r * k + m] * Ps[t * kk + m * k + c];
                        Ps[(t + 1) * kk + r * k + c] = s;
                    }
            }
            for (int64_t i = 0; i < kk; ++i) W[i] = 0.0;
            for (int64_t t = T - 1; t >= 0; --t) {
                const double *dPt = blk(dP, b, t, j, T, nb, k);
                for (int64_t i = 0; i < kk; ++i) G[i] = dPt[i] + W[i];
                const double *At = blk(A, b, t, j, T, nb, k);
                double *dAt = dA + (((b * T + t) * nb + j) * kk);
                /* dA_t[r][c] = sum_m G_t[r][m] P_{t-1}[c][m] */
                for (int64_t r = 0; r < k; ++r)
                    for (int64_t c = 0; c < k; ++c) {
                        double s = 0.0;
                        for (int64_t m = 0; m < k; ++m) s += G[r * k + m] * Ps[t * kk + c * k + m];
                        dAt[r * k + c] = s;
                    }
                /* W = A_t^T G_t */
                for (int64_t r = 0; r < k; ++r)
                    for (int64_t c = 0; c < k; ++c) {
                        double s = 0.0;
                        for (int64_t m = 0; m < k; ++m) s += At[m * k + r] * G[m * k + c];
                        W[r * k + c] = s;
                    }
            }
        }
    free(Ps);
    free(G);
    free(W);
}

/* ------------------------------------------------ Givens angle-fused scan */

/* Applies the mesh's layers to the k x k matrix M from the left, in order
 * L_0 .. L_{k-1}.  If rho >= 0, the layer holding angle rho is replaced by its
 * derivative with respect to that angle: the rotation's block becomes
 * d/dtheta [[c, -s], [s, c]] = [[-s, -c], [c, -s]] and every other row of the
 * layer's matrix is zero. */
static void mesh_apply(const double *theta, int64_t k, int64_t rho, double *M)
{
    int64_t idx = 0; /* angle index of the layer's first pair */
    for (int64_t l = 0; l < k; ++l) {
        int64_t n_pairs = 0;
        for (int64_t i = l % 2; i + 1 < k; i += 2) ++n_pairs;
        if (rho >= idx && rho < idx + n_pairs) {
            int64_t i = l % 2 + 2 * (rho - idx), j = i + 1;
            double c = cos(theta[rho]), s = sin(theta[rho]);
            for (int64_t col = 0; col < k; ++col) {
                double xi = M[i * k + col], xj = M[j * k + col];
                for (int64_t r = 0; r < k; ++r) M[r * k + col] = 0.0;
                M[i * k + col] = -s * xi - c * xj;
                M[j * k + col] = c * xi - s * xj;
            }
        } else {
            int64_t a = idx;
            for (int64_t i = l % 2; i + 1 < k; i += 2, ++a) {
                int64_t j = i + 1;
                double c = cos(theta[a]), s = sin(theta[a]);
                for (int64_t col = 0; col < k; ++col) {
                    double xi = M[i * k + col], xj = M[j * k + col];
                    M[i * k + col] = c * xi - s * xj;
                    M[j * k + col] = s * xi + c * xj;
                }
            }
        }
        idx += n_pairs;
    }
}

/* R(theta) (rho < 0) or dR/dtheta_rho into R (k x k) */
static void mesh_matrix(const double *theta, int64_t k, int64_t rho, double *R)
{
    for (int64_t r = 0; r < k; ++r)
        for (int64_t c = 0; c < k; ++c) R[r * k + c] = (r == c) ? 1.0 : 0.0;
    mesh_apply(theta, k, rho, R);
}

static double sigmoid_d(double u) { return 1.0 / (1.0 + exp(-u)); }

/* Forward: A_t = sigmoid(s_t) R(theta_t) per block; h_0 = h0 (zero if NULL);
 * h_t = A_t h_{t-1} + b_t; writes h_1..T. */
void oracle_givens_fwd(const double *theta, const double *sg, const double *bv, const double *h0,
                       double *h, int64_t B, int64_t T, int64_t d, int64_t k)
{
    int64_t nb = d / k, na = k * (k - 1) / 2;
    double *R = (double *)malloc(sizeof(double) * (size_t)(k * k));
    double *cur = (double *)malloc(sizeof(double) * (size_t)k);
    double *nxt = (double *)malloc(sizeof(double) * (size_t)k);
    if (!R || !cur || !nxt) { free(R); free(cur); free(nxt); return; }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < nb; ++j) {
            for (int64_t r = 0; r < k; ++r) cur[r] = h0 ? h0[b * d + j * k + r] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                int64_t blkid = (b * T + t) * nb + j;
                mesh_matrix(theta + blkid * na, k, -1, R);
                double sig = sigmoid_d(sg[blkid]);
                for (int64_t r = 0; r < k; ++r) {
                    double acc = bv[(b * T + t) * d + j * k + r];
                    for (int64_t c = 0; c < k; ++c) acc += sig * R[r * k + c] * cur[c];
                    nxt[r] = acc;
                }
                for (int64_t r = 0; r < k; ++r) {
                    cur[r] = nxt[r];
                    h[(b * T + t) * d + j * k + r] = cur[r];
                }
            }
        }
    free(R);
    free(cur);
    free(nxt);
}

/* Backward of oracle_givens_fwd for L = sum_t <dh_t, h_t>: the block-affine
 * reverse scan g_t = dh_t + A_{t+1}^T g_{t+1} gives dA_t = g_t h_{t-1}^T,
 * db_t = g_t, dh0 = A_1^T g_1; then, through A = sigmoid(s) R(theta),
 *   ds_t = sigmoid'(s_t) <dA_t, R>,   dtheta_rho = sigmoid(s_t) <dA_t, dR/dtheta_rho>,
 * with dR/dtheta_rho formed explicitly for every angle. */
void oracle_givens_bwd(const double *theta, const double *sg, const double *bv, const double *h0,
                       const double *dh, double *dtheta, double *dsg, double *db, double *dh0,
                       int64_t B, int64_t T, int64_t d, int64_t k)
{
    int64_t nb = d / k, na = k * (k - 1) / 2;
    double *hs = (double *)malloc(sizeof(double) * (size_t)((T + 1) * k));
    double *R = (double *)malloc(sizeof(double) * (size_t)(k * k));
    double *dR = (double *)malloc(sizeof(double) * (size_t)(k * k));
    double *g = (double *)malloc(sizeof(double) * (size_t)k);
    double *w = (double *)malloc(sizeof(double) * (size_t)k);
    if (!hs || !R || !dR || !g || !w) { free(hs); free(R); free(dR); free(g); free(w); return; }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < nb; ++j) {
            for (int64_t r = 0; r < k; ++r) hs[r] = h0 ? h0[b * d + j * k + r] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                int64_t blkid = (b * T + t) * nb + j;
                mesh_matrix(theta + blkid * na, k, -1, R);
                double sig = sigmoid_d(sg[blkid]);
                for (int64_t r = 0; r < k; ++r) {
                    double acc = bv[(b * T + t) * d + j * k + r];
                    for (int64_t c = 0; c < k; ++c) acc += sig * R[r * k + c] * hs[t * k + c];
                    hs[(t + 1) * k + r] = acc;
                }
            }
            for (int64_t r = 0; r < k; ++r) w[r] = 0.0;
            for (int64_t t = T - 1; t >= 0; --t) {
                int64_t blkid = (b * T + t) * nb + j;
                for (int64_t r = 0; r < k; ++r) g[r] = dh[(b * T + t) * d + j * k + r] + w[r];
                mesh_matrix(theta + blkid * na, k, -1, R);
                double sig = sigmoid_d(sg[blkid]);
                /* <dA, R> with dA = g h_{t-1}^T */
                double acc = 0.0;
                for (int64_t r = 0; r < k; ++r)
                    for (int64_t c = 0; c < k; ++c) acc += g[r] * hs[t * k + c] * R[r * k + c];
                dsg[blkid] = sig * (1.0 - sig) * acc;
                for (int64_t rho = 0; rho < na; ++rho) {
                    mesh_matrix(theta + blkid * na, k, rho, dR);
                    double a2 = 0.0;
                    for (int64_t r = 0; r < k; ++r)
                        for (int64_t c = 0; c < k; ++c) a2 += g[r] * hs[t * k + c] * dR[r * k + c];
                    dtheta[blkid * na + rho] = sig * a2;
                }
                for (int64_t r = 0; r < k; ++r) db[(b * T + t) * d + j * k + r] = g[r];
                for (int64_t c = 0; c < k; ++c) {
                    double acc2 = 0.0;
                    for (int64_t r = 0; r < k; ++r) acc2 += sig * R[r * k + c] * g[r];
                    w[c] = acc2;
                }
            }
            for (int64_t r = 0; r < k; ++r) dh0[b * d + j * k + r] = w[r];
        }
    free(hs);
    free(R);
    free(dR);
    free(g);
    free(w);
}

/* ----------------------------------------------------------- delta rule */

/* Forward: S_0 = S0 (zero if S0 == NULL); for t = 1..T
 *     p = S_{t-1} k_t,   S_t = S_{t-1} + beta_t (v_t - p) k_t^T,   o_t = S_t q_t;
 * writes o_1..T and, if ST != NULL, the final state S_T. */
void oracle_delta_fwd(const double *q, const double *k, const double *v, const double *beta,
                      const double *S0, double *o, double *ST,
                      int64_t B, int64_t T, int64_t dk, int64_t dv)
{
    double *S = (double *)malloc(sizeof(double) * (size_t)(dv * dk));
    double *p = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < dv * dk; ++i) S[i] = S0 ? S0[b * dv * dk + i] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const double *kt = k + (b * T + t) * dk;
            const double *qt = q + (b * T + t) * dk;
            const double *vt = v + (b * T + t) * dv;
            double bt = beta[b * T + t];
            for (int64_t r = 0; r < dv; ++r) {
                double acc = 0.0;
                for (int64_t c = 0; c < dk; ++c) acc += S[r * dk + c] * kt[c];
                p[r] = acc;
            }
            for (int64_t r = 0; r < dv; ++r) {
                double e = bt * (vt[r] - p[r]);
                for (int64_t c = 0; c < dk; ++c) S[r * dk + c] += e * kt[c];
            }
            for (int64_t r = 0; r < dv; ++r) {
                double acc = 0.0;
                for (int64_t c = 0; c < dk; ++c) acc += S[r * dk + c] * qt[c];
                o[(b * T + t) * dv + r] = acc;
            }
        }
        if (ST)
            for (int64_t i = 0; i < dv * dk; ++i) ST[b * dv * dk + i] = S[i];
    }
    free(S);
    free(p);
}
