/*
 * mgs.h -- C ABI of libmgs, the minGRU scan engine for AMD Instinct MI355X (gfx950).
 *
 * The library solves the linear recurrence h_t = A_t h_{t-1} + b_t by
 * associative scan, forward and backward, in three forms:
 *
 *   1. log-space elementwise scan (A_t = a_t > 0 diagonal), inputs given as
 *      log a_t, log b_t, log h_0 and evaluated in log space in the style of
 *      Heinsen's scan -- the op behind MinGRU / SignedMinGRU
 *      (minGRU home page, introduction; "Triton on GPU" tutorial, section
 *      "What you gain (and where you don't)", op parallel_scan_log);
 *   2. block-affine scan, A_t block-diagonal with k x k blocks -- the op behind
 *      RotationMinGRU / GivensMinGRU ("Run the benchmarks" how-to, Step 2,
 *      op matrix_affine_scan);
 *   3. block cumulative product P_t = A_t P_{t-1}, P_0 = I, the b = 0 case
 *      (same table, op matrix_scan);
 *   1b. the same scan with the minGRU cell fused ahead of it (inputs are the
 *      pre-activations; gradients are returned for them);
 *   2b. the same with A_t = sigmoid(s_t) R(theta_t) formed from Givens angles
 *      and a gate inside the kernels (GivensMinGRU, home page);
 *   4. linear-space elementwise scan, a_t of either sign -- the op the pages
 *      list as linear_scan (home page speed-up table; "Run the benchmarks"
 *      how-to, Step 2), for gates with negative eigenvalues.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every pointer is a DEVICE pointer (HIP global memory) except
 *   `bytes` / `flags` out-parameters, which are host pointers.  The caller owns
 *   every buffer; the library allocates nothing and keeps no per-call state.
 *   Tensors are fp32, dense, row-major with the last index fastest, 16-byte
 *   aligned:
 *     (B,T,d)        sequence tensors; the scan runs over T
 *     (B,d)          initial states and their gradients
 *     (B,T,d/k,k,k)  block transitions; block j acts on channels [j*k,(j+1)*k)
 *                    and (A h)_r = sum_c A[r][c] h[c]
 * Outputs are fully overwritten (never accumulated) and must not overlap any
 * input or each other.
 *
 * Streams.  `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *   stream-ordered and return once the kernels are queued; errors raised while
 *   the kernels run surface at the caller's next synchronisation, as in HIP.
 *
 * Workspace.  Each op has a `*_workspace_size` query.  The workspace is
 *   device memory of at least that many bytes that MUST BE ZERO-FILLED BEFORE
 *   ITS FIRST USE; the library leaves it ready for the next call.  A forward
 *   call stores there what its backward reads (tile carries), so pass the same
 *   workspace to the backward of the same inputs.  Calls that share a
 *   workspace must not run concurrently.
 *
 * Errors.  Arguments are validated before any HIP call:
 *   MGS_ERR_INVALID_VALUE  NULL required pointer, negative size, k <= 0,
 *                          d % k != 0, misaligned pointer, or output aliasing
 *                          an input;
 *   MGS_ERR_UNSUPPORTED    outside the envelope (block ops: k not in
 *                          {1, 2, 4, 8, 16}; Givens scan: k != 8; delta rule:
 *                          d != 64; or a tensor with 2^31 or more elements --
 *                          sizes are bounded one by one and their products are
 *                          overflow-checked, so no combination of sizes wraps
 *                          around); never a silent fallback to another path;
 *   MGS_ERR_WORKSPACE      workspace NULL or smaller than the query says;
 *   MGS_ERR_HIP            a HIP launch error; mgs_last_hip_error() gives the
 *                          hipError_t (per calling thread).
 * Empty tensors.  A size of 0 is valid: the call computes nothing and
 *   returns MGS_OK, except that a backward with T == 0 (and B*d > 0) writes
 *   zeros to the gradient of the initial state (the loss does not depend on
 *   it).  Pointers to empty tensors may be NULL.
 * Non-finite inputs propagate; log_b = -inf (b = 0) and log_h0 = -inf
 * (h_0 = 0) are supported exactly by the log-space scan.
 */
#ifndef MGS_H
#define MGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MGS_OK = 0,
    MGS_ERR_INVALID_VALUE = 1,
    MGS_ERR_UNSUPPORTED = 2,
    MGS_ERR_WORKSPACE = 3,
    MGS_ERR_HIP = 4
} mgs_status;

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int mgs_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char *mgs_status_string(int status);

/* hipError_t of the last MGS_ERR_HIP returned on the calling thread (0 if none). */
int mgs_last_hip_error(void);

/* Reads (synchronously, on `stream`) the workspace's device-side error flags
 * into *flags: 0 = clean; bit 0 = a cross-workgroup wait in a kernel gave up
 * after its spin limit (results of that call are invalid).  Clears the flags.
 * Reads a few bytes of `workspace`; it must be a workspace used by this
 * library. */
mgs_status mgs_workspace_check(void *workspace, void *stream, int *flags);

/* For tests of the failure path, not for production use: sets two fields of
 * the workspace's header (synchronously, on `stream`).  spin_limit is the
 * number of polls after which a cross-workgroup wait gives up (0 restores the
 * built-in 2^20).  fail_waits != 0 makes every such wait expect a launch tag
 * that no launch publishes, so each wait runs to the limit, the kernels still
 * exit, and mgs_workspace_check then reports bit 0; results of calls made
 * meanwhile are invalid.  mgs_workspace_set_waits(ws, 0, 0, s) restores
 * normal operation (a zero-filled workspace starts there).  No effect on the
 * allocation-free entry point, which has no workspace argument. */
mgs_status mgs_workspace_set_waits(void *workspace, unsigned spin_limit, int fail_waits, void *stream);

/* ------------------------------------------------------ log-space scan --- */
/*
 * Forward (minGRU home page, introduction: the log-space MinGRU with Heinsen's
 * scan; op parallel_scan_log):
 *     h_0 = exp(log_h0),   h_t = exp(log_a_t) h_{t-1} + exp(log_b_t),  t = 1..T
 * computed in log space, log h_t = logaddexp(log_a_t + log h_{t-1}, log_b_t),
 * and written as h (linear, h_1..h_T; h_0 is not written).
 *   log_a, log_b : (B,T,d) in     log_h0 : (B,d) in     h : (B,T,d) out
 */
mgs_status mgs_scan_log_workspace_size(int64_t B, int64_t T, int64_t d, size_t *bytes);

mgs_status mgs_scan_log_fwd(const float *log_a, const float *log_b, const float *log_h0,
                            float *h, int64_t B, int64_t T, int64_t d,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward of mgs_scan_log_fwd for L = sum_t <dh_t, h_t>.  It recomputes the
 * forward states (the home page notes the log-space op's backward recomputes
 * its forward) and runs the reverse scan g_T = dh_T, g_t = dh_t + a_{t+1} g_{t+1}:
 *     dlog_a_t = g_t a_t h_{t-1},   dlog_b_t = g_t b_t,   dlog_h0 = g_1 a_1 h_0.
 *   dh : (B,T,d) in;   dlog_a, dlog_b : (B,T,d) out;   dlog_h0 : (B,d) out.
 * fwd_state_valid != 0 promises that mgs_scan_log_fwd ran on these same inputs
 * with this workspace since it was last used by another call; with 0 the
 * backward first recomputes the forward's tile carries itself (one more
 * kernel launch).
 */
mgs_status mgs_scan_log_bwd(const float *log_a, const float *log_b, const float *log_h0,
                            const float *dh, float *dlog_a, float *dlog_b, float *dlog_h0,
                            int64_t B, int64_t T, int64_t d,
                            void *workspace, size_t workspace_bytes, int fwd_state_valid,
                            void *stream);

/* ------------------------------------ minGRU cell + log-space scan --- */
/*
 * The minGRU cell fused ahead of the log-space scan (minGRU home page,
 * introduction: minGRU of Feng et al.; the pages do not write the cell out,
 * so this is the reading taken).  From pre-activations k, x (B,T,d), x0 (B,d):
 *     a_t = sigmoid(-k_t),  b_t = (1 - a_t) g(x_t),  h_0 = g(x0),
 *     g(u) = u + 0.5 (u >= 0), sigmoid(u) (u < 0),
 * then h_t = a_t h_{t-1} + b_t evaluated in log space exactly as
 * mgs_scan_log_fwd does; log a, log b and log h0 are formed in registers and
 * never stored.  Same workspace rules as the log-space scan.
 *   k, x : (B,T,d) in     x0 : (B,d) in     h : (B,T,d) out
 */
mgs_status mgs_scan_mingru_workspace_size(int64_t B, int64_t T, int64_t d, size_t *bytes);

mgs_status mgs_scan_mingru_fwd(const float *k, const float *x, const float *x0, float *h,
                               int64_t B, int64_t T, int64_t d,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward of mgs_scan_mingru_fwd for L = sum_t <dh_t, h_t>: with the reverse
 * scan g_T = dh_T, g_t = dh_t + a_{t+1} g_{t+1} and z_t = 1 - a_t,
 *     dk_t = g_t a_t z_t (g(x_t) - h_{t-1}),   dx_t = g_t z_t g'(x_t),
 *     dx0 = g_1 a_1 g'(x0).
 *   dh : (B,T,d) in;   dk, dx : (B,T,d) out;   dx0 : (B,d) out.
 * fwd_state_valid as for mgs_scan_log_bwd.
 */
mgs_status mgs_scan_mingru_bwd(const float *k, const float *x, const float *x0, const float *dh,
                               float *dk, float *dx, float *dx0,
                               int64_t B, int64_t T, int64_t d,
                               void *workspace, size_t workspace_bytes, int fwd_state_valid,
                               void *stream);

/* --------------------------------------------------- linear-space scan --- */
/*
 * Forward (linear_scan: home page speed-up table and "Run the benchmarks"
 * how-to, Step 2; the signed gates of SignedMinGRU, home page):
 *     h_0 = h0,   h_t = a_t h_{t-1} + b_t,  t = 1..T,   a_t of either sign,
 * evaluated in linear space (a log form cannot hold a negative a_t) and
 * written as h (h_1..h_T).
 *   a, b : (B,T,d) in     h0 : (B,d) in     h : (B,T,d) out
 * Same workspace rules as the log-space scan (its own size query).
 */
mgs_status mgs_scan_linear_workspace_size(int64_t B, int64_t T, int64_t d, size_t *bytes);

mgs_status mgs_scan_linear_fwd(const float *a, const float *b, const float *h0, float *h,
                               int64_t B, int64_t T, int64_t d,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward of mgs_scan_linear_fwd for L = sum_t <dh_t, h_t>: the reverse scan
 * g_T = dh_T, g_t = dh_t + a_{t+1} g_{t+1}, with
 *     da_t = g_t h_{t-1},   db_t = g_t,   dh0 = a_1 g_1.
 * h_{t-1} is recomputed from a, b, h0 and the tile-start states the forward
 * left in the workspace.
 *   dh : (B,T,d) in;   da, db : (B,T,d) out;   dh0 : (B,d) out.
 * fwd_state_valid as for mgs_scan_log_bwd.
 */
mgs_status mgs_scan_linear_bwd(const float *a, const float *b, const float *h0, const float *dh,
                               float *da, float *db, float *dh0,
                               int64_t B, int64_t T, int64_t d,
                               void *workspace, size_t workspace_bytes, int fwd_state_valid,
                               void *stream);

/* --------------------------------------------------- block-affine scan --- */
/*
 * Forward ("Run the benchmarks" how-to, Step 2, matrix_affine_scan; the
 * GivensMinGRU / RotationMinGRU recurrences on the home page):
 *     h_0 = h0 (zeros if h0 == NULL),   h_t = A_t h_{t-1} + b_t
 * with A_t block-diagonal (d/k blocks of k x k).
 *   A : (B,T,d/k,k,k) in;  b : (B,T,d) in;  h0 : (B,d) in or NULL;  h : (B,T,d) out.
 * Envelope: k in {1, 2, 4, 8, 16} (k = 1 is the elementwise linear-space scan
 * with A of shape (B,T,d,1,1)).
 */
mgs_status mgs_block_affine_scan_workspace_size(int64_t B, int64_t T, int64_t d, int64_t k,
                                                size_t *bytes);

mgs_status mgs_block_affine_scan_fwd(const float *A, const float *b, const float *h0, float *h,
                                     int64_t B, int64_t T, int64_t d, int64_t k,
                                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * mgs_block_affine_scan_fwd for callers that cannot allocate device memory --
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation: the same computation and kernels, with no workspace argument.
 * Its workspace is a 16 MiB array in the library's device code, one copy per
 * GPU, zero-filled when that code is loaded and held until the process ends;
 * the call itself allocates nothing (no hipMalloc, no allocating library call).
 *   A, b, h0, h, B, T, d, k, stream : as for mgs_block_affine_scan_fwd.
 * Limits: B*d <= 262144 and the shape's look-back words must fit the rest of
 * the array (at k = 8 and B*d/8 = 128 chains, T up to 24448); larger shapes
 * return MGS_ERR_UNSUPPORTED before any HIP call.  Every call on one GPU shares
 * that GPU's array and keeps it ready for the next call, so nothing needs
 * clearing between calls; calls that overlap in time on one GPU (on different
 * streams, or from different threads) race on it and must not be issued.  The
 * array's error word (a look-back wait that hit its spin limit) is not
 * readable through this interface.
 */
mgs_status mgs_block_affine_scan_fwd_noalloc(const float *A, const float *b, const float *h0, float *h,
                                             int64_t B, int64_t T, int64_t d, int64_t k, void *stream);

/*
 * Backward of mgs_block_affine_scan_fwd for L = sum_t <dh_t, h_t>: the reverse
 * scan g_T = dh_T, g_t = dh_t + A_{t+1}^T g_{t+1}, with
 *     dA_t = g_t h_{t-1}^T (formed in registers, written once),  db_t = g_t,
 *     dh0 = A_1^T g_1.
 *   h : (B,T,d) in, the forward's output (it supplies h_{t-1}); b is not read
 *   and may be NULL; h0 as in the forward;  dh : (B,T,d) in;
 *   dA : (B,T,d/k,k,k) out;  db : (B,T,d) out;  dh0 : (B,d) out (written even
 *   when h0 == NULL).
 */
mgs_status mgs_block_affine_scan_bwd(const float *A, const float *b, const float *h0,
                                     const float *h, const float *dh,
                                     float *dA, float *db, float *dh0,
                                     int64_t B, int64_t T, int64_t d, int64_t k,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------ Givens angle-fused scan --- */
/*
 * The block-affine scan with each transition formed from angles and a gate
 * (GivensMinGRU on the minGRU home page; its fused backward is the memory
 * saving measured in the "Run the benchmarks" how-to, Step 3):
 *     A_t = sigmoid(s_t) R(theta_t),   h_t = A_t h_{t-1} + b_t   per block,
 * R a brick-wall mesh of k layers of 2 x 2 rotations: layer l rotates the
 * pairs (i, i+1), i = l mod 2, l mod 2 + 2, ... < k - 1; R = L_{k-1} .. L_0;
 * angles in (layer, pair) order; each rotation maps (x_i, x_j) to
 * (cos x_i - sin x_j, sin x_i + cos x_j) (the pages name the mesh, not these
 * conventions; this is the reading taken).  A and dA are formed only in
 * registers, never in memory.
 *   theta : (B,T,d/k,k(k-1)/2) in;  s : (B,T,d/k) in;  b : (B,T,d) in;
 *   h0 : (B,d) in or NULL;  h : (B,T,d) out.   Envelope: k == 8.
 * Same workspace rules as the block-affine scan (its own size query).
 */
mgs_status mgs_givens_scan_workspace_size(int64_t B, int64_t T, int64_t d, int64_t k, size_t *bytes);

mgs_status mgs_givens_scan_fwd(const float *theta, const float *s, const float *b, const float *h0,
                               float *h, int64_t B, int64_t T, int64_t d, int64_t k,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward of mgs_givens_scan_fwd for L = sum_t <dh_t, h_t>: the block-affine
 * reverse scan g_t = dh_t + A_{t+1}^T g_{t+1} with dA_t = g_t h_{t-1}^T
 * contracted in registers:
 *     dtheta_t = sigmoid(s_t) <dA_t, dR/dtheta>,   ds_t = sigmoid'(s_t) <dA_t, R>,
 *     db_t = g_t,   dh0 = A_1^T g_1.
 *   h : (B,T,d) in, the forward's output;  h0 as in the forward;  dh : (B,T,d) in;
 *   dtheta : shape of theta, out;  ds : shape of s, out;  db : (B,T,d) out;
 *   dh0 : (B,d) out (written even when h0 == NULL).
 */
mgs_status mgs_givens_scan_bwd(const float *theta, const float *s, const float *h0, const float *h,
                               const float *dh, float *dtheta, float *ds, float *db, float *dh0,
                               int64_t B, int64_t T, int64_t d, int64_t k,
                               void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------ block cumulative product --- */
/*
 * Forward ("Run the benchmarks" how-to, Step 2, matrix_scan): the b = 0 case,
 *     P_0 = I,   P_t = A_t P_{t-1}   per k x k block.
 *   A : (B,T,d/k,k,k) in;   P : (B,T,d/k,k,k) out.   Envelope: k in {1, 2, 4, 8, 16}.
 */
mgs_status mgs_block_matrix_scan_workspace_size(int64_t B, int64_t T, int64_t d, int64_t k,
                                                size_t *bytes);

mgs_status mgs_block_matrix_scan_fwd(const float *A, float *P,
                                     int64_t B, int64_t T, int64_t d, int64_t k,
                                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward of mgs_block_matrix_scan_fwd for L = sum_t <dP_t, P_t>:
 *     G_T = dP_T,  G_t = dP_t + A_{t+1}^T G_{t+1},  dA_t = G_t P_{t-1}^T.
 * P_{t-1} is recomputed from A and the state entering each chunk, which the
 * forward stores in the workspace (one k x k block per chain per chunk of
 * steps); P itself is not read.
 *   dP : in;  dA : out (shape of A).
 * fwd_state_valid != 0 promises that mgs_block_matrix_scan_fwd ran on this A
 * with this workspace since it was last used by another call; with 0 the
 * backward first recomputes those states itself (one more kernel launch).
 */
mgs_status mgs_block_matrix_scan_bwd(const float *A, const float *dP, float *dA,
                                     int64_t B, int64_t T, int64_t d, int64_t k,
                                     void *workspace, size_t workspace_bytes, int fwd_state_valid,
                                     void *stream);

/* ------------------------------------------------------------ delta rule --- */
/*
 * Forward of the delta rule of DeltaMinGRU (minGRU home page: DeltaMinGRU
 * reimplements DeltaNet and runs DeltaNet's chunked WY representation as its
 * parallel forward; the pages do not write the recurrence out, this is
 * DeltaNet's):
 *     S_0 = S0 (zeros if S0 == NULL),
 *     S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T,     o_t = S_t q_t,
 * one state S (d x d, (S k)_r = sum_c S[r][c] k[c]) per sequence, evaluated in
 * chunks of 64 steps in the WY form.  q and k are used as given (DeltaNet
 * scales them to unit norm beforehand; the op does not).
 *   q, k, v : (B,T,d) in;  beta : (B,T) in;  S0 : (B,d,d) in or NULL;
 *   o : (B,T,d) out;  ST : (B,d,d) out (the final state S_T) or NULL.
 * Envelope: d == 64.  The workspace holds per (sequence, chunk) the chunk's
 * state-free WY factors; it carries nothing between calls (zero-filling is
 * not needed, though harmless).
 */
mgs_status mgs_delta_workspace_size(int64_t B, int64_t T, int64_t d, size_t *bytes);

mgs_status mgs_delta_fwd(const float *q, const float *k, const float *v, const float *beta,
                         const float *S0, float *o, float *ST,
                         int64_t B, int64_t T, int64_t d,
                         void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MGS_H */
