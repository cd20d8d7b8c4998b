// block_core.hpp -- device code of the block scans (block-affine scan, block
// cumulative product, Givens angle-fused scan), forward and fused backward,
// for gfx950, written once for every block size k in {1, 2, 4, 8, 16}.
//
// The ops ("Run the benchmarks" how-to, Step 2: matrix_affine_scan and
// matrix_scan; the RotationMinGRU / GivensMinGRU recurrences on the minGRU
// home page):
//     h_t = A_t h_{t-1} + b_t          P_t = A_t P_{t-1},  P_0 = I
// per chain (b, block j), with A_t a k x k block.  Backward for
// L = sum <dh_t, h_t> (resp. <dP_t, P_t>): g_t = dh_t + A_{t+1}^T g_{t+1},
// dA_t = g_t h_{t-1}^T (resp. G_t P_{t-1}^T), db_t = g_t, dh0 = A_1^T g_1.
// dA_t is formed in registers from g_t and h_{t-1} and written once; no
// per-step product or intermediate tensor is ever stored.
//
// Register layout ("row lanes"): a chain's k x k matrices live in k
// consecutive lanes, lane v holding row v, and a half-wave holds 32 / k
// chains.  A product needs, in every lane, the rows held by the chain's other
// lanes; they arrive through DPP broadcasts within the chain's lanes:
//   k = 8:  column slots of a row are rotated by the lane's quad (slot s holds
//           column s ^ (v & 4)), so every operand comes through one of two
//           wave-uniform patterns -- a quad broadcast for rows in the lane's own
//           quad, a half-row mirror plus a quad broadcast for the other quad --
//           and the rotation costs nothing because loads and stores address the
//           two 16-byte halves of a row in swapped order.  An 8 x 8 by 8 x 8
//           product is 64 FMAs with DPP operands plus 8 mirror moves per lane.
//   k = 16: a chain is one DPP row; row_newbcast:m broadcasts row m.
//   k = 4:  quad broadcast;  k = 2: quad_perm [m, m, m+2, m+2];  k = 1: none.
//
// Decomposition: a wave holds 2 sub-chunks of 32 lanes (lane = 32*sub +
// k*chain + row); a workgroup of W waves holds NCH = 2W consecutive chunks of C
// steps each, i.e. one tile of TT = NCH*C steps of 32 / k chains.  Each chunk
// first builds its aggregate (transfer matrix and offset) from a zero state,
// the aggregates meet in LDS, and tiles along T exchange theirs by single-pass
// decoupled look-back (tagged words, launch epochs; see device.hpp).  Each
// chunk then re-runs its recurrence from its true carry-in, keeping the loaded
// A_t in registers, and writes its outputs.
//
// Included by block_scan.hip (k = 8, the Givens scan, host entry points) and
// by block_scan_k.hip (one other k per object file).
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "device.hpp"
#include "launch.hpp"

namespace mgs {

// Kernel arguments of every block op (one struct, fields used per op).
struct BlkArgs {
    const float *A;      // (B,T,nb,k,k)
    const float *x;      // affine: b (fwd) or h (bwd)
    const float *y;      // affine bwd: dh; cumprod bwd: dP
    const float *h0;     // affine: (B,d), or a zero region of the workspace
    float *out;          // affine fwd: h; affine bwd: dA; cumprod fwd: P (NULL: chunk states only); cumprod bwd: dA
    float *out2;         // affine bwd: db
    float *out3;         // affine bwd: dh0
    int64_t nchain;
    int T, d, nb, nCG, nT, nTiles;
    WsHeader *hd;
    uint64_t *agg, *incl;
    float *pstate;       // cumulative product: the state entering every 2^pcs-th step, [t >> pcs][chain group][slot][k]
    int pcs;             // cumulative product: log2 of the steps between saved states (the backward's chunk length)
    const float *theta;  // Givens angle-fused: angles (B,T,nb,28)
    const float *sg;     // Givens angle-fused: gate pre-activations (B,T,nb)
    float *dtheta;       // Givens angle-fused backward: d angles
    float *dsg;          // Givens angle-fused backward: d gate
    int lb_local;        // every tile's look-back partners run on its XCD (tagged_store)
};

// Tile shape per op and block size: waves per workgroup and the cap on steps
// per lane group (a lane keeps up to 3C rows of k floats in registers).  For
// k = 8, eight waves and C <= 8 measured fastest for both ops at both shapes.
#ifndef MGS_AFF_W
#define MGS_AFF_W 8
#endif
#ifndef MGS_AFF_MAXC
#define MGS_AFF_MAXC 8
#endif
#ifndef MGS_MAT_W
#define MGS_MAT_W 8
#endif
#ifndef MGS_MAT_MAXC
#define MGS_MAT_MAXC 8
#endif
struct BlkShape {
    int W, max_c;
};
// k = 16 block-affine: eight-step chunks (up to 234 VGPRs) make the long-T
// workload one generation of 256 tiles (two of 512 with four-step chunks:
// 94.9 -> 83.8 us for the pair)
#ifndef MGS_AFF16_MAXC
#define MGS_AFF16_MAXC 8
#endif
constexpr BlkShape affine_shape(int k)
{
    return k == 8 ? BlkShape{MGS_AFF_W, MGS_AFF_MAXC} : k == 16 ? BlkShape{8, MGS_AFF16_MAXC} : BlkShape{8, 8};
}
// The cumulative product's forward and backward may tile T differently: the
// forward saves the state entering every step the backward starts a chunk at.
// k = 16: the backward's reverse aggregate is two 16 x 16 rows per lane, so it
// runs four waves (LDS buffers at 68 KB, two workgroups per compute unit) of
// four-step chunks, reading its dP rows a second time in the fix-up to stay
// within 256 registers; the forward keeps one row per step and runs eight
// waves of eight-step chunks, whose 128-step tiles fit the long-T workload
// into one workgroup per compute unit.
#ifndef MGS_MAT16_FWD_W
#define MGS_MAT16_FWD_W 8
#endif
#ifndef MGS_MAT16_FWD_MAXC
#define MGS_MAT16_FWD_MAXC 8
#endif
#ifndef MGS_MAT16_BWD_W
#define MGS_MAT16_BWD_W 4
#endif
#ifndef MGS_MAT16_BWD_MAXC
#define MGS_MAT16_BWD_MAXC 4
#endif
constexpr BlkShape matrix_shape(int k, bool forward)
{
    return k == 8    ? BlkShape{MGS_MAT_W, MGS_MAT_MAXC}
           : k == 16 ? (forward ? BlkShape{MGS_MAT16_FWD_W, MGS_MAT16_FWD_MAXC}
                                : BlkShape{MGS_MAT16_BWD_W, MGS_MAT16_BWD_MAXC})
                     : BlkShape{8, 8};
}

enum class BlkOp : int { AffineFwd, AffineBwd, MatrixFwd, MatrixBwd };

// Launches one block op for block size K; each K's kernels are instantiated
// in one object file (k = 8 in block_scan.hip, the others in block_scan_k.hip).
template <int K>
void launch_blk(BlkOp op, const BlockGeom &g, const BlkArgs &a, hipStream_t s);
template <> void launch_blk<1>(BlkOp, const BlockGeom &, const BlkArgs &, hipStream_t);
template <> void launch_blk<2>(BlkOp, const BlockGeom &, const BlkArgs &, hipStream_t);
template <> void launch_blk<4>(BlkOp, const BlockGeom &, const BlkArgs &, hipStream_t);
template <> void launch_blk<8>(BlkOp, const BlockGeom &, const BlkArgs &, hipStream_t);
template <> void launch_blk<16>(BlkOp, const BlockGeom &, const BlkArgs &, hipStream_t);

namespace {

// ------------------------------------------------------ 8-lane row algebra (k = 8)

template <int P>
__device__ __forceinline__ float qb(float x)   // value of quad position P
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), P | (P << 2) | (P << 4) | (P << 6),
                                                   0xF, 0xF, true));
}

__device__ __forceinline__ float hm(float x)   // value of lane 7 - v within the 8-lane group
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
}

// 8 x 8 row algebra with DPP operands folded into the multiply-adds.  The
// compiler does not fold DPP moves into FMAs, so the products are written as
// inline-asm blocks of v_fmac_f32_dpp / v_mul_f32_dpp.  Each block keeps 2 or
// 4 independent accumulators and cycles through them, so consecutive
// instructions never depend on each other.  Every block opens with 5 wait
// states (a VALU write of a DPP source, or of EXEC, may come right before it)
// and closes with 2 (a DPP read of its result may come right after), because
// the compiler's hazard tracking does not look inside inline asm.

// y_v = sum_m R[v][m] x_m + add, R = own row (rotated slots), x one value per lane
__device__ __forceinline__ float mv8(const float *R, float x, float add)
{
    const float mx = hm(x);
    float a0 = add, a1;
    asm("s_nop 4\n\t"
        "v_fmac_f32_dpp %0, %2, %4 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %2, %5 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %6 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %7 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %3, %11 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %10 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %3, %9 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %8 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1"
        : "+&v"(a0), "=&v"(a1)
        : "v"(x), "v"(mx), "v"(R[0]), "v"(R[1]), "v"(R[2]), "v"(R[3]), "v"(R[4]), "v"(R[5]), "v"(R[6]), "v"(R[7]));
    return a0 + a1;
}

// Four output slots S..S+3 of Y = R X (X rows spread over the group, M = hm(X)).
template <int S>
__device__ __forceinline__ void mm8_quarter(const float *R, const float *X, const float *M, float *Y)
{
    asm("s_nop 4\n\t"
        "v_mul_f32_dpp %0, %4, %12 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %5, %12 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %6, %12 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %7, %12 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %13 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %13 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %13 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %13 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %14 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %14 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %14 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %14 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %15 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %15 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %15 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %15 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %19 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %9, %19 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %19 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %11, %19 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %18 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %9, %18 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %18 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %11, %18 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %17 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %9, %17 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %17 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %11, %17 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %16 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %9, %16 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %16 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %11, %16 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1"
        : "=&v"(Y[S]), "=&v"(Y[S + 1]), "=&v"(Y[S + 2]), "=&v"(Y[S + 3])
        : "v"(X[S]), "v"(X[S + 1]), "v"(X[S + 2]), "v"(X[S + 3]),
          "v"(M[S ^ 4]), "v"(M[(S + 1) ^ 4]), "v"(M[(S + 2) ^ 4]), "v"(M[(S + 3) ^ 4]),
          "v"(R[0]), "v"(R[1]), "v"(R[2]), "v"(R[3]), "v"(R[4]), "v"(R[5]), "v"(R[6]), "v"(R[7]));
}

// Y = R X : own row of R, rows of X spread over the group.  Y must not alias X.
__device__ __forceinline__ void mm8(const float *R, const float *X, float *Y)
{
    float M[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) M[s] = hm(X[s]);
    mm8_quarter<0>(R, X, M, Y);
    mm8_quarter<4>(R, X, M, Y);
}

// Output slots P, P+1, 7-P, 6-P of Y = G X^T.
template <int P>
__device__ __forceinline__ void mmT8_quarter(const float *G, const float *X, const float *M, float *Y)
{
    asm("s_nop 4\n\t"
        "v_mul_f32_dpp %0, %4, %20 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %4, %20 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %12, %24 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %12, %24 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %5, %21 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %21 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %13, %25 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %13, %25 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %6, %22 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %6, %22 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %14, %26 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %14, %26 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %7, %23 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %7, %23 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %15, %27 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %15, %27 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %24 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %8, %24 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %16, %20 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %16, %20 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %9, %25 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %9, %25 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %17, %21 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %17, %21 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %10, %26 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %10, %26 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %22 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %18, %22 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %11, %27 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %11, %27 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %19, %23 quad_perm:[%28,%28,%28,%28] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %23 quad_perm:[%29,%29,%29,%29] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1"
        : "=&v"(Y[P]), "=&v"(Y[P + 1]), "=&v"(Y[7 - P]), "=&v"(Y[6 - P])
        : "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]),
          "v"(M[0]), "v"(M[1]), "v"(M[2]), "v"(M[3]), "v"(M[4]), "v"(M[5]), "v"(M[6]), "v"(M[7]),
          "v"(G[0]), "v"(G[1]), "v"(G[2]), "v"(G[3]), "v"(G[4]), "v"(G[5]), "v"(G[6]), "v"(G[7]),
          "n"(P), "n"(P + 1));
}

// Y = G X^T : own row of G, rows of X spread over the group.
__device__ __forceinline__ void mmT8(const float *G, const float *X, float *Y)
{
    float M[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) M[s] = hm(X[s]);
    mmT8_quarter<0>(G, X, M, Y);
    mmT8_quarter<2>(G, X, M, Y);
}

// Row v of x x'^T scaled: Y[slot] = g * x'_{column(slot)}  (x' one value per lane)
__device__ __forceinline__ void outer8(float g, float x, float *Y)
{
    const float mx = hm(x);
    Y[0] = g * qb<0>(x);
    Y[1] = g * qb<1>(x);
    Y[2] = g * qb<2>(x);
    Y[3] = g * qb<3>(x);
    Y[4] = g * qb<3>(mx);
    Y[5] = g * qb<2>(mx);
    Y[6] = g * qb<1>(mx);
    Y[7] = g * qb<0>(mx);
}

__device__ __forceinline__ void eye_row8(int v, float *Y)
{
#pragma unroll
    for (int s = 0; s < 8; ++s) Y[s] = (s == (v & 3)) ? 1.0f : 0.0f;
}

// row v of a row-major 8x8 block at p (16-byte aligned), into rotated slots
__device__ __forceinline__ void load_row8(const float *p, int v, float *R)
{
    const int lo = v & 4;
    const float4 x0 = *reinterpret_cast<const float4 *>(p + v * 8 + lo);
    const float4 x1 = *reinterpret_cast<const float4 *>(p + v * 8 + (lo ^ 4));
    R[0] = x0.x; R[1] = x0.y; R[2] = x0.z; R[3] = x0.w;
    R[4] = x1.x; R[5] = x1.y; R[6] = x1.z; R[7] = x1.w;
}

// row v of the TRANSPOSE of the 8x8 block at p (column v), rotated slots
__device__ __forceinline__ void load_col8(const float *p, int v, float *R)
{
    const int lo = v & 4;
#pragma unroll
    for (int s = 0; s < 8; ++s) R[s] = p[((s ^ lo) * 8) + v];
}

__device__ __forceinline__ float xq(float x)   // value of lane v ^ 4 within the 8-lane group
{
    const float m = hm(x);   // lane 7 - v, then reversed within the quad
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x1B, 0xF, 0xF, true));
}

// row v of a row-major 8x8 block at p (16-byte aligned) from rotated slots.
// Lanes v and v ^ 4 first swap slots 4-7, so that the first 16-byte store of
// the chain's eight lanes covers rows 0-3 (128 contiguous bytes) and the second
// rows 4-7: no 32-byte sector is split between two stores, which matters for
// the nontemporal stores (a split sector would reach HBM twice).  Lane v < 4
// writes row v, columns 0-3, then row v + 4, columns 0-3 (the partner's slots
// 4-7); lane v >= 4 writes row v - 4, columns 4-7 (the partner's slots 4-7),
// then row v, columns 4-7.  Call with all eight lanes of the chain active.
__device__ __forceinline__ void store_row8(float *p, int v, const float *R)
{
    float X[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) X[j] = xq(R[4 + j]);
    const bool low = v < 4;
    float *p1 = p + (v & 3) * 8 + (v & 4);
    store_out4(p1, low ? R[0] : X[0], low ? R[1] : X[1], low ? R[2] : X[2], low ? R[3] : X[3]);
    store_out4(p1 + 32, low ? X[0] : R[0], low ? X[1] : R[1], low ? X[2] : R[2], low ? X[3] : R[3]);
}

// ----------------------------------------------------- 16-lane row algebra (k = 16)
// A chain is one DPP row of 16 lanes; row_newbcast:m hands every lane of the
// row the value of its lane m.  Products are inline-asm blocks of
// v_fmac_f32_dpp / v_mul_f32_dpp for the reason given for k = 8 (same wait
// states around each block).

// Y = R X : own row of R, rows of X spread over the chain (16 x 16).  One
// block of 256 multiply-adds with row_newbcast operands; consecutive
// instructions write different accumulators.  Y must not alias X.
__device__ __forceinline__ void mm16(const float *R, const float *X, float *Y)
{
    asm("s_nop 4\n\t"
        "v_mul_f32_dpp %0, %16, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %17, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %18, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %19, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %4, %20, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %5, %21, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %6, %22, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %7, %23, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %8, %24, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %9, %25, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %10, %26, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %11, %27, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %12, %28, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %13, %29, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %14, %30, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %15, %31, %32 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %33 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %34 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %35 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %36 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %37 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %38 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %39 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %40 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %41 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %42 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %43 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %44 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %45 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %46 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %16, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %20, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %21, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %22, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %23, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %24, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %25, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %26, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %27, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %28, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %29, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %30, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %31, %47 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1"
        : "=&v"(Y[0]), "=&v"(Y[1]), "=&v"(Y[2]), "=&v"(Y[3]), "=&v"(Y[4]), "=&v"(Y[5]), "=&v"(Y[6]), "=&v"(Y[7]), "=&v"(Y[8]), "=&v"(Y[9]), "=&v"(Y[10]), "=&v"(Y[11]), "=&v"(Y[12]), "=&v"(Y[13]), "=&v"(Y[14]), "=&v"(Y[15])
        : "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]),
          "v"(R[0]), "v"(R[1]), "v"(R[2]), "v"(R[3]), "v"(R[4]), "v"(R[5]), "v"(R[6]), "v"(R[7]), "v"(R[8]), "v"(R[9]), "v"(R[10]), "v"(R[11]), "v"(R[12]), "v"(R[13]), "v"(R[14]), "v"(R[15]));
}

// y_v = sum_m R[m] x_m + add (16 x 16), four accumulators
__device__ __forceinline__ float mv16(const float *R, float x, float add)
{
    float a0 = add, a1, a2, a3;
    asm("s_nop 4\n\t"
        "v_fmac_f32_dpp %0, %4, %5 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %4, %6 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %4, %7 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %4, %8 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %9 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %4, %10 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %4, %11 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %4, %12 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %13 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %4, %14 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %4, %15 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %4, %16 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %17 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %4, %18 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %4, %19 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %4, %20 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1"
        : "+&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
        : "v"(x), "v"(R[0]), "v"(R[1]), "v"(R[2]), "v"(R[3]), "v"(R[4]), "v"(R[5]), "v"(R[6]), "v"(R[7]), "v"(R[8]), "v"(R[9]), "v"(R[10]), "v"(R[11]), "v"(R[12]), "v"(R[13]), "v"(R[14]), "v"(R[15]));
    return (a0 + a1) + (a2 + a3);
}

// row v of g x^T (16 x 16): Y[c] = g * x_c
__device__ __forceinline__ void outer16(float g, float x, float *Y)
{
    asm("s_nop 4\n\t"
        "v_mul_f32_dpp %0, %16, %17 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %16, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %16, %17 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %4, %16, %17 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %5, %16, %17 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %6, %16, %17 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %7, %16, %17 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %8, %16, %17 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %9, %16, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %10, %16, %17 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %11, %16, %17 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %12, %16, %17 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %13, %16, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %14, %16, %17 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %15, %16, %17 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1"
        : "=&v"(Y[0]), "=&v"(Y[1]), "=&v"(Y[2]), "=&v"(Y[3]), "=&v"(Y[4]), "=&v"(Y[5]), "=&v"(Y[6]), "=&v"(Y[7]), "=&v"(Y[8]), "=&v"(Y[9]), "=&v"(Y[10]), "=&v"(Y[11]), "=&v"(Y[12]), "=&v"(Y[13]), "=&v"(Y[14]), "=&v"(Y[15])
        : "v"(x), "v"(g));
}

// --------------------------------------------- row algebra for every k
// Rows<K> gathers what the kernels need of a chain's K x K matrices held one
// row per lane (the primary template serves k = 1, 2, 4 with DPP moves the
// compiler places; k = 8 and k = 16 are specialised with inline-asm blocks): products with another matrix or vector spread over the
// chain's lanes, the outer product, the identity row, and loads / stores of a
// row of a row-major block in the lane's slot order.  col(v, s) is the column
// that slot s of lane v holds (an involution in s).

// f(0), f(1), ..., f(N - 1) with compile-time arguments (DPP controls must be
// constants, so the loops over source rows are unrolled at the source level).
template <typename F, int... I>
__device__ __forceinline__ void static_for_(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_(f, std::make_integer_sequence<int, N>{});
}

// Value of x in the lane holding row M of this lane's chain (K in {1, 2, 4}:
// the chain sits inside one quad, so a quad permutation reaches every row).
template <int K, int M>
__device__ __forceinline__ float row_bcast(float x)
{
    static_assert(M >= 0 && M < K, "row index");
    static_assert(K == 1 || K == 2 || K == 4, "block size");
    if constexpr (K == 1) {
        return x;
    } else {
        constexpr int ctrl = K == 2 ? (M | (M << 2) | ((M + 2) << 4) | ((M + 2) << 6))   // quad_perm [M,M,M+2,M+2]
                                    : M * 0x55;                                          // quad_perm [M,M,M,M]
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, true));
    }
}

// K contiguous floats at p (16-byte aligned when K >= 4) <-> registers
template <int K>
__device__ __forceinline__ void load_vec(const float *p, float *x)
{
    if constexpr (K == 1) {
        x[0] = p[0];
    } else if constexpr (K == 2) {
        const float2 u = *reinterpret_cast<const float2 *>(p);
        x[0] = u.x; x[1] = u.y;
    } else {
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
            const float4 u = *reinterpret_cast<const float4 *>(p + 4 * q);
            x[4 * q] = u.x; x[4 * q + 1] = u.y; x[4 * q + 2] = u.z; x[4 * q + 3] = u.w;
        }
    }
}

// K consecutive floats at p (aligned to their size, at most 16 bytes).  The
// lanes of a half-wave store consecutive K-float vectors, so for K <= 4 one
// store instruction covers whole 32-byte sectors and takes the nontemporal
// hint; for K = 8 and 16 each lane's vector spans several 16-byte stores whose
// sectors are completed by the lane's next store, so those stay ordinary
// stores that L2 merges.
template <int K>
__device__ __forceinline__ void store_vec(float *p, const float *x)
{
    if constexpr (K == 1) {
        store_out(p, x[0]);
    } else if constexpr (K == 2) {
        store_out2(p, x[0], x[1]);
    } else if constexpr (K == 4) {
        store_out4(p, x[0], x[1], x[2], x[3]);
    } else {
#pragma unroll
        for (int q = 0; q < K / 4; ++q)
            *reinterpret_cast<float4 *>(p + 4 * q) = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
    }
}

template <int K>
struct Rows {
    static constexpr int k = K;
    // y_v = sum_m R[m] x_m + add  (x one value per lane)
    static __device__ __forceinline__ float mv(const float *R, float x, float add)
    {
        float a0 = add, a1 = 0.0f;
        static_for<K>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            if constexpr (m % 2 == 0) a0 = __builtin_fmaf(R[m], row_bcast<K, m>(x), a0);
            else a1 = __builtin_fmaf(R[m], row_bcast<K, m>(x), a1);
        });
        return K == 1 ? a0 : a0 + a1;
    }
    // Y = R X : own row of R, rows of X spread over the chain.  Y must not alias X.
    static __device__ __forceinline__ void mm(const float *R, const float *X, float *Y)
    {
#pragma unroll
        for (int c = 0; c < K; ++c) Y[c] = 0.0f;
        static_for<K>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
#pragma unroll
            for (int c = 0; c < K; ++c) Y[c] = __builtin_fmaf(R[m], row_bcast<K, m>(X[c]), Y[c]);
        });
    }
    // row v of g x^T: Y[c] = g * x_c  (x one value per lane)
    static __device__ __forceinline__ void outer(float g, float x, float *Y)
    {
        static_for<K>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            Y[c] = g * row_bcast<K, c>(x);
        });
    }
    static __device__ __forceinline__ void eye(int v, float *Y)
    {
#pragma unroll
        for (int s = 0; s < K; ++s) Y[s] = (s == v) ? 1.0f : 0.0f;
    }
    static __device__ __forceinline__ int col(int, int s) { return s; }
    // row v of the row-major K x K block at p
    static __device__ __forceinline__ void load_row(const float *p, int v, float *R) { load_vec<K>(p + v * K, R); }
    // row v of the transpose of the block at p (column v)
    static __device__ __forceinline__ void load_col(const float *p, int v, float *R)
    {
#pragma unroll
        for (int s = 0; s < K; ++s) R[s] = p[s * K + v];
    }
    static __device__ __forceinline__ void store_row(float *p, int v, const float *R) { store_vec<K>(p + v * K, R); }
};

template <>
struct Rows<16> {
    static constexpr int k = 16;
    static __device__ __forceinline__ float mv(const float *R, float x, float add) { return mv16(R, x, add); }
    static __device__ __forceinline__ void mm(const float *R, const float *X, float *Y) { mm16(R, X, Y); }
    static __device__ __forceinline__ void outer(float g, float x, float *Y) { outer16(g, x, Y); }
    static __device__ __forceinline__ void eye(int v, float *Y)
    {
#pragma unroll
        for (int s = 0; s < 16; ++s) Y[s] = (s == v) ? 1.0f : 0.0f;
    }
    static __device__ __forceinline__ int col(int, int s) { return s; }
    static __device__ __forceinline__ void load_row(const float *p, int v, float *R) { load_vec<16>(p + v * 16, R); }
    static __device__ __forceinline__ void load_col(const float *p, int v, float *R)
    {
#pragma unroll
        for (int s = 0; s < 16; ++s) R[s] = p[s * 16 + v];
    }
    static __device__ __forceinline__ void store_row(float *p, int v, const float *R) { store_vec<16>(p + v * 16, R); }
};

template <>
struct Rows<8> {
    static constexpr int k = 8;
    static __device__ __forceinline__ float mv(const float *R, float x, float add) { return mv8(R, x, add); }
    static __device__ __forceinline__ void mm(const float *R, const float *X, float *Y) { mm8(R, X, Y); }
    static __device__ __forceinline__ void outer(float g, float x, float *Y) { outer8(g, x, Y); }
    static __device__ __forceinline__ void eye(int v, float *Y) { eye_row8(v, Y); }
    static __device__ __forceinline__ int col(int v, int s) { return s ^ (v & 4); }
    static __device__ __forceinline__ void load_row(const float *p, int v, float *R) { load_row8(p, v, R); }
    static __device__ __forceinline__ void load_col(const float *p, int v, float *R) { load_col8(p, v, R); }
    static __device__ __forceinline__ void store_row(float *p, int v, const float *R) { store_row8(p, v, R); }
};

struct Tile {
    int lane, wv, v, cgl, sub, slot, q, j, cg, t0;
    bool cv;
    int64_t bb, jb;
    int64_t blk0;    // block index (bb, t=0, jb) in (B,T,nb)
    int64_t ablk0;   // element offset of A block (bb, t=0, jb)
    int64_t astep;   // elements between consecutive t of the same block
    int64_t vec0;    // element offset of (bb, t=0, jb*k + v) in (B,T,d)
    int64_t vstep;   // = d
};

// lane = 32 * sub + K * (chain in the half-wave) + row
template <int K, int C, int W>
__device__ __forceinline__ Tile make_tile(const BlkArgs &a, int tile, bool reverse)
{
    Tile t;
    t.lane = threadIdx.x & 63;
    t.wv = threadIdx.x >> 6;
    t.v = t.lane & (K - 1);
    t.slot = t.lane & 31;
    t.cgl = t.slot / K;
    t.sub = t.lane >> 5;
    t.q = t.wv * 2 + t.sub;
    const int jr = tile / a.nCG;
    t.cg = tile - jr * a.nCG;
    t.j = reverse ? a.nT - 1 - jr : jr;
    const int64_t chain = static_cast<int64_t>(t.cg) * (32 / K) + t.cgl;
    t.cv = chain < a.nchain;
    const int64_t cc = t.cv ? chain : 0;
    t.bb = cc / a.nb;
    t.jb = cc - t.bb * a.nb;
    t.astep = static_cast<int64_t>(a.nb) * K * K;
    t.blk0 = t.bb * a.T * a.nb + t.jb;
    t.ablk0 = t.blk0 * K * K;
    t.vstep = a.d;
    t.vec0 = t.bb * a.T * a.d + t.jb * K + t.v;
    t.t0 = t.j * (2 * W * C) + t.q * C;
    return t;
}

__device__ __forceinline__ int clampT(int t, int T) { return t < T ? t : T - 1; }

// h0 entry of this lane.  When the caller passes no h0, a.h0 points at a
// zero region of the workspace, so the load is unconditional and never sits
// behind a branch that would force a wait on the loads issued before it.
// Lanes of chains past the end read chain 0's entry; their results are never
// stored and their k-lane groups exchange data only among themselves.
template <int K>
__device__ __forceinline__ float load_h0(const BlkArgs &a, const Tile &tl)
{
    return a.h0[tl.bb * a.d + tl.jb * K + tl.v];
}

// ============================================ chunk aggregates
// Each half-wave holds the aggregate of one chunk q = 2 * wave + sub: the
// chunk's transfer matrix row and, for the block-affine scan (one value per
// lane) and the cumulative-product backward (a matrix row), its offset.  Two
// aggregates compose as
//     (M, v) o (M', v') = (M M', M v' + v)
// in either direction: (later o earlier) forward, (earlier o later) for the
// reverse aggregates of the backward.

enum AggKind : int { kMat = 0, kMatVec = 1, kMatMat = 2 };

template <int KIND, int K>
struct AggShape {
    static constexpr int words = KIND == kMat ? K : (KIND == kMatVec ? K + 1 : 2 * K);
    static constexpr int stride = words | 1;   // odd LDS stride: lanes hit distinct banks
};

template <int KIND, int K>
__device__ __forceinline__ void compose_into(float *X, const float *R)
{
    using Rw = Rows<K>;
    if constexpr (KIND == kMatVec) X[K] = Rw::mv(X, R[K], X[K]);
    if constexpr (KIND == kMatMat) {
        float nw[K];
        Rw::mm(X, R + K, nw);
#pragma unroll
        for (int s = 0; s < K; ++s) X[K + s] += nw[s];
    }
    float np[K];
    Rw::mm(X, R, np);
#pragma unroll
    for (int s = 0; s < K; ++s) X[s] = np[s];
}

template <int KIND, int K, int NCH>
__device__ __forceinline__ void ks_store(float (*buf)[32][(AggShape<KIND, K>::stride)], int q, int slot, const float *X)
{
#pragma unroll
    for (int e = 0; e < AggShape<KIND, K>::words; ++e) buf[q][slot][e] = X[e];
}

// ===================================================== Givens mesh in lanes
// The angle-fused kernels form A_t = sigmoid(s_t) R(theta_t) in registers.  R is
// the brick-wall mesh of 8 layers of 2 x 2 rotations (GivensMinGRU on the
// minGRU home page; the Clements / EUNN mesh it cites): layer l rotates the
// pairs (i, i+1), i = l mod 2, l mod 2 + 2, ..., R = L_7 .. L_0, angles in
// (layer, pair) order, each rotation mapping (x_i, x_j) to
// (c x_i - s x_j, s x_i + c x_j).  The forward builds each lane's row of R in
// the lane: lane p of a chain's 8 lanes loads angles 4p..4p+3 (lane 7 none),
// and the chain shares their cosines and sines through LDS, so every angle is
// loaded once and turned into sin / cos once.  The backward applies the mesh
// layer by layer across the chain's lanes (further below).

constexpr int kAngles = 28;
// row stride (floats) of the per-lane cos / sin exchange buffer: 8 values, padded
// to 12 so that 16 consecutive lanes' 16-byte stores fall on distinct banks
constexpr int kCSLd = 12;

__host__ __device__ constexpr int mesh_first(int l) { return (l / 2) * 7 + (l & 1) * 4; }

// sin x and cos x for |x| up to a few thousand: Cody and Waite's reduction
// x = q pi/2 + r with pi/2 split into a float head and tail (fused multiply-
// adds keep q * head exact enough), |r| <= pi/4, then the Taylor series of sin
// to r^9 and of cos to r^10 (truncation below 2e-9) and the quadrant's
// swap / sign.  A few ulp, against the dozens of instructions (and a
// large-argument path) of a general-range sincos.
__device__ __forceinline__ void sincos_cw(float x, float &sn, float &cs)
{
    constexpr float kTwoOverPi = 0.636619772367581f;
    constexpr float kPiHalfHi = 1.57079637050628662f;      // float(pi / 2)
    constexpr float kPiHalfLo = -4.37113900018624e-08f;     // pi / 2 - kPiHalfHi
    const float q = __builtin_rintf(x * kTwoOverPi);
    float r = __builtin_fmaf(q, -kPiHalfHi, x);
    r = __builtin_fmaf(q, -kPiHalfLo, r);
    const float r2 = r * r;
    float ps = __builtin_fmaf(r2, 1.0f / 362880.0f, -1.0f / 5040.0f);
    ps = __builtin_fmaf(r2, ps, 1.0f / 120.0f);
    ps = __builtin_fmaf(r2, ps, -1.0f / 6.0f);
    const float sr = __builtin_fmaf(r * r2, ps, r);
    float pc = __builtin_fmaf(r2, -1.0f / 3628800.0f, 1.0f / 40320.0f);
    pc = __builtin_fmaf(r2, pc, -1.0f / 720.0f);
    pc = __builtin_fmaf(r2, pc, 1.0f / 24.0f);
    pc = __builtin_fmaf(r2, pc, -0.5f);
    const float cr = __builtin_fmaf(r2, pc, 1.0f);
    const int n = static_cast<int>(q);
    const bool swap = (n & 1) != 0;
    const float s0 = swap ? cr : sr, c0 = swap ? sr : cr;
    sn = (n & 2) ? -s0 : s0;
    cs = ((n + 1) & 2) ? -c0 : c0;
}

// cosines and sines of a chain's 28 angles in every lane of the chain
__device__ __forceinline__ void mesh_share(float4 th, float (*cs)[kCSLd], int lane, float (&cc)[kAngles],
                                           float (&ss)[kAngles])
{
    // within a few ulp (the hardware's native sin / cos lose ~1e-6 absolute,
    // which the 28 rotations and the scan then carry)
    float4 c4, s4;
    sincos_cw(th.x, s4.x, c4.x);
    sincos_cw(th.y, s4.y, c4.y);
    sincos_cw(th.z, s4.z, c4.z);
    sincos_cw(th.w, s4.w, c4.w);
    *reinterpret_cast<float4 *>(&cs[lane][0]) = c4;
    *reinterpret_cast<float4 *>(&cs[lane][4]) = s4;
    const int base = lane & ~7;
#pragma unroll
    for (int p = 0; p < 7; ++p) {
        const float4 c = *reinterpret_cast<const float4 *>(&cs[base + p][0]);
        const float4 s = *reinterpret_cast<const float4 *>(&cs[base + p][4]);
        cc[4 * p] = c.x; cc[4 * p + 1] = c.y; cc[4 * p + 2] = c.z; cc[4 * p + 3] = c.w;
        ss[4 * p] = s.x; ss[4 * p + 1] = s.y; ss[4 * p + 2] = s.z; ss[4 * p + 3] = s.w;
    }
}

// row v of R in natural column order: e_v^T L_7 .. L_0
__device__ __forceinline__ void mesh_row(const float (&cc)[kAngles], const float (&ss)[kAngles], int v, float (&r)[8])
{
#pragma unroll
    for (int c = 0; c < 8; ++c) r[c] = (c == v) ? 1.0f : 0.0f;
#pragma unroll
    for (int l = 7; l >= 0; --l)
#pragma unroll
        for (int i = l & 1, a = mesh_first(l); i + 1 < 8; i += 2, ++a) {
            const float ri = r[i], rj = r[i + 1];
            r[i] = cc[a] * ri + ss[a] * rj;
            r[i + 1] = cc[a] * rj - ss[a] * ri;
        }
}

// natural order -> this lane's rotated slots (slot s holds entry s ^ (v & 4)).
// Written as a bitwise blend of two fixed-index registers: a select between
// x[s] and x[s ^ 4] would be folded into a lane-dependent index, which sends
// the array to scratch memory.
__device__ __forceinline__ float blend(float a, float b, int mask)
{
    return __int_as_float((__float_as_int(b) & mask) | (__float_as_int(a) & ~mask));
}

__device__ __forceinline__ void to_slots(const float (&x)[8], int v, float scale, float *y)
{
    const int m = -((v >> 2) & 1);
#pragma unroll
    for (int s = 0; s < 8; ++s) y[s] = scale * blend(x[s], x[s ^ 4], m);
}

__device__ __forceinline__ float sigmoidf_(float u) { return 1.0f / (1.0f + __expf(-u)); }

// Pins eight values in registers at this point of the program: work that
// produces them cannot sink below it, so one step's 56 cosines and sines are
// dead before the next step's are loaded (with a scheduling barrier after it).
__device__ __forceinline__ void settle8(float *x)
{
    asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                 "+v"(x[7]));
    __builtin_amdgcn_sched_barrier(0);
}

// angle slice and gate of this lane's chain at step t (indices clamped in range)
__device__ __forceinline__ float4 load_angles(const BlkArgs &a, const Tile &tl, int t)
{
    const int64_t blk = tl.blk0 + static_cast<int64_t>(t) * a.nb;
    return *reinterpret_cast<const float4 *>(a.theta + blk * kAngles + 4 * min(tl.v, 6));
}

// ------------------------------------------- Givens mesh, layer by layer across the lanes
// Element v of a chain's vectors, and row v of its 8 x 8 matrices (rotated
// slots), sit in lane v of the chain's 8 lanes, and the mesh is applied one
// layer at a time, each lane mixing its value with its pair partner's:
//     x' = c x + s' x_partner,  s' = -s in the pair's first lane, +s in its second.
// Partners: even layers v ^ 1 (quad permutation [1,0,3,2]); odd layers 1-2
// and 5-6 (quad permutation [0,2,1,3], which leaves lanes 0, 3, 4, 7 in place)
// and 3-4 (half-row mirror); lanes 0 and 7 sit odd layers out (c = 1, s = 0).
// Every partner is in the chain's own 8 lanes.  A lane needs only the angles
// of its own pairs, 8 per step: the two lanes of a pair each evaluate the
// sine and cosine of two of the pair's four angles (one split for the even
// layers, one for the odd) and swap them, so each of a chain's 28 angles is
// evaluated once per pass and nothing goes through LDS.

__device__ __forceinline__ float qpe(float x)   // lane v ^ 1
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}

__device__ __forceinline__ float qpo(float x)   // lanes 1 <-> 2 and 5 <-> 6; 0, 3, 4, 7 in place
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xD8, 0xF, 0xF, true));
}

__device__ __forceinline__ float qx2(float x)   // lane v ^ 2
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

// Per-lane constants of the layered mesh.
struct MeshLane {
    int ie, io;      // first angle this lane evaluates for its even / odd pair (the second is 7 further)
    bool re, ro;     // second lane of its even / odd pair
    bool mir;        // lanes 3 and 4: odd-layer partner through the half-row mirror
    bool oddp;       // lanes 1 .. 6: in an odd-layer pair
};

__device__ __forceinline__ MeshLane mesh_lane(int v)
{
    MeshLane m;
    m.re = (v & 1) != 0;
    m.oddp = v >= 1 && v <= 6;
    const int qo = m.oddp ? (v - 1) >> 1 : 0;
    m.ro = m.oddp && ((v - 1) & 1) != 0;
    m.mir = v == 3 || v == 4;
    // even pair v/2: layers 0, 2 (first lane) or 4, 6 (second); odd pair
    // (v-1)/2: layers 1, 3 (first lane) or 5, 7 (second)
    m.ie = 14 * (m.re ? 1 : 0) + (v >> 1);
    m.io = 4 + 14 * (m.ro ? 1 : 0) + qo;
    return m;
}

__device__ __forceinline__ float mesh_partner(float x, int l, bool mir)
{
    if (l & 1) {
        const float q = qpo(x), h = hm(x);
        return mir ? h : q;
    }
    return qpe(x);
}

// The four angles this lane evaluates at step t (lanes 0 and 7: zero for the
// odd pair they do not have).
// This lane's four angles of one step at p (the step's 28 angles).  Lanes
// without an odd-layer pair load their even pair's angles twice; mesh_eval
// replaces those by 0 where the values are used, so no select waits on the
// loads while later ones are still to be issued.
__device__ __forceinline__ float4 mesh_angles_at(const float *p, const MeshLane &ml)
{
    const int io = ml.oddp ? ml.io : ml.ie;
    return make_float4(p[ml.ie], p[ml.ie + 7], p[io], p[io + 7]);
}

// cosines and sines (signed for this lane's place in the pair) of its four angles
__device__ __forceinline__ void mesh_eval(float4 th, const MeshLane &ml, float (&e)[8])
{
    if (!ml.oddp) th.z = th.w = 0.0f;
    float s;
    sincos_cw(th.x, s, e[0]); e[1] = ml.re ? s : -s;
    sincos_cw(th.y, s, e[2]); e[3] = ml.re ? s : -s;
    sincos_cw(th.z, s, e[4]); e[5] = ml.ro ? s : -s;
    sincos_cw(th.w, s, e[6]); e[7] = ml.ro ? s : -s;
}

// Layer coefficients of one step: c[l] and s[l] = s' of layer l in this lane.
// The partner's values arrive with the opposite sign (it holds the other end
// of the pair).
__device__ __forceinline__ void mesh_coef(const float (&e)[8], const MeshLane &ml, float (&c)[8], float (&s)[8])
{
    const float pc0 = qpe(e[0]), ps0 = -qpe(e[1]), pc1 = qpe(e[2]), ps1 = -qpe(e[3]);
    c[0] = ml.re ? pc0 : e[0]; s[0] = ml.re ? ps0 : e[1];
    c[2] = ml.re ? pc1 : e[2]; s[2] = ml.re ? ps1 : e[3];
    c[4] = ml.re ? e[0] : pc0; s[4] = ml.re ? e[1] : ps0;
    c[6] = ml.re ? e[2] : pc1; s[6] = ml.re ? e[3] : ps1;
    const float qc0 = mesh_partner(e[4], 1, ml.mir), qs0 = -mesh_partner(e[5], 1, ml.mir);
    const float qc1 = mesh_partner(e[6], 1, ml.mir), qs1 = -mesh_partner(e[7], 1, ml.mir);
    c[1] = ml.ro ? qc0 : e[4]; s[1] = ml.ro ? qs0 : e[5];
    c[3] = ml.ro ? qc1 : e[6]; s[3] = ml.ro ? qs1 : e[7];
    c[5] = ml.ro ? e[4] : qc0; s[5] = ml.ro ? e[5] : qs0;
    c[7] = ml.ro ? e[6] : qc1; s[7] = ml.ro ? e[7] : qs1;
}

// One layer on a vector (one value per lane).
__device__ __forceinline__ float mesh_vec(float x, float c, float s, int l, bool mir)
{
    return __builtin_fmaf(s, mesh_partner(x, l, mir), c * x);
}

// X <- L_even L_odd X: an odd layer, then an even one (the transposed mesh's
// order; the caller passes negated sines), on eight matrix row entries
// (rotated slots) and a vector entry X[8], which share the coefficients.  Odd
// layer: c1; q1 = s' for the quad-permutation partner (0 in lanes 3, 4), m1
// for the mirror partner (nonzero in lanes 3 and 4 only, whose slot rotations
// are opposite, so row slot k takes the partner's slot k ^ 4).  Even layer:
// c0, s0 (partner v ^ 1, same slot order).  Every DPP source inside the block
// was written at least nine instructions before it is read.
__device__ __forceinline__ void mesh_rows2r(float (&X)[9], float c1, float q1, float m1, float c0, float s0)
{
    float Y[9];
    asm("s_nop 4\n\t"
        "v_mul_f32 %9, %18, %0\n\t"
        "v_mul_f32 %10, %18, %1\n\t"
        "v_mul_f32 %11, %18, %2\n\t"
        "v_mul_f32 %12, %18, %3\n\t"
        "v_mul_f32 %13, %18, %4\n\t"
        "v_mul_f32 %14, %18, %5\n\t"
        "v_mul_f32 %15, %18, %6\n\t"
        "v_mul_f32 %16, %18, %7\n\t"
        "v_mul_f32 %17, %18, %8\n\t"
        "v_fmac_f32_dpp %9, %0, %19 quad_perm:[0,2,1,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %1, %19 quad_perm:[0,2,1,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %2, %19 quad_perm:[0,2,1,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %3, %19 quad_perm:[0,2,1,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %4, %19 quad_perm:[0,2,1,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %5, %19 quad_perm:[0,2,1,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %6, %19 quad_perm:[0,2,1,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %16, %7, %19 quad_perm:[0,2,1,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %17, %8, %19 quad_perm:[0,2,1,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %4, %20 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %5, %20 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %6, %20 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %7, %20 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %0, %20 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %1, %20 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %2, %20 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %16, %3, %20 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %17, %8, %20 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32 %0, %21, %9\n\t"
        "v_mul_f32 %1, %21, %10\n\t"
        "v_mul_f32 %2, %21, %11\n\t"
        "v_mul_f32 %3, %21, %12\n\t"
        "v_mul_f32 %4, %21, %13\n\t"
        "v_mul_f32 %5, %21, %14\n\t"
        "v_mul_f32 %6, %21, %15\n\t"
        "v_mul_f32 %7, %21, %16\n\t"
        "v_mul_f32 %8, %21, %17\n\t"
        "v_fmac_f32_dpp %0, %9, %22 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %10, %22 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %11, %22 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %12, %22 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %13, %22 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %14, %22 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %15, %22 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %16, %22 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %17, %22 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1"
        : "+v"(X[0]), "+v"(X[1]), "+v"(X[2]), "+v"(X[3]), "+v"(X[4]), "+v"(X[5]), "+v"(X[6]), "+v"(X[7]),
          "+v"(X[8]), "=&v"(Y[0]), "=&v"(Y[1]), "=&v"(Y[2]), "=&v"(Y[3]), "=&v"(Y[4]), "=&v"(Y[5]), "=&v"(Y[6]),
          "=&v"(Y[7]), "=&v"(Y[8])
        : "v"(c1), "v"(q1), "v"(m1), "v"(c0), "v"(s0));
}

// sum over the chain's 8 lanes, in every lane
__device__ __forceinline__ float chain_sum8(float x)
{
    x += qpe(x);
    x += qx2(x);
    return x + hm(x);
}

// ====================================================== carry phases
// Shared by every multi-chunk kernel of the block ops.
//
// A tile's NCH chunk aggregates -- per lane, the chunk's transfer matrix row
// and (block-affine, cumulative-product backward) its offset -- meet in a
// tree: node (l, i) composes chunks [i 2^l, (i+1) 2^l), level 0 being the
// chunks themselves.  The forward composes a later segment after an earlier
// one, (M2, v2) o (M1, v1) = (M2 M1, M2 v1 + v2); the backward's reverse
// aggregates compose the other way round.  The root is the tile aggregate,
// published for the look-back as soon as it exists; once the state entering
// the tile is known, each chunk reaches its own entering state by applying at
// most log2(NCH) tree nodes to it, so no prefix of every chunk is ever formed.

// Node (l, i) of the tree of a tile's NCH chunks (NCH / 2^l nodes at level l,
// the root at level log2 NCH).  Once the tree is built, the chunks' entering
// states need only the nodes of a prefix decomposition (forward: even i) or a
// suffix one (reverse: odd i), and the look-back the root.  Those sit after
// the others, so the NCH - 1 nodes dead by then form one block at the start
// of the node array, where the look-back may stage the words it polls.
template <int NCH, int DIR>
__device__ __forceinline__ constexpr int tree_node(int l, int i)
{
    const bool live = (NCH >> l) == 1 || (i & 1) == (DIR > 0 ? 0 : 1);
    return (live ? NCH - 1 : 0) + NCH - (NCH >> l) + (i >> 1);
}

// floats of the block of dead nodes at the start of a node array
template <int KIND, int K, int NCH>
constexpr int dead_nodes_floats()
{
    return (NCH - 1) * 32 * AggShape<KIND, K>::stride;
}

template <int NCH>
__host__ __device__ constexpr int tree_levels()
{
    int l = 0;
    while ((1 << l) < NCH) ++l;
    return l;
}

// The state a lane carries across chunks and tiles (CW words: the block-affine
// scan's vector entry, or a row of the cumulative product's matrix state) and
// how an aggregate (AW words at g) acts on it.
template <int KIND, int K>
struct Carry {
    static constexpr int CW = KIND == kMatVec ? 1 : K;
    static constexpr int AW = AggShape<KIND, K>::words;
    static __device__ __forceinline__ void apply(const float *g, float *c)
    {
        using Rw = Rows<K>;
        if constexpr (KIND == kMatVec) {
            c[0] = Rw::mv(g, c[0], g[K]);
        } else {
            float np[K];
            Rw::mm(g, c, np);
#pragma unroll
            for (int s = 0; s < K; ++s) c[s] = KIND == kMatMat ? np[s] + g[K + s] : np[s];
        }
    }
};

// Workgroup barrier that waits only for this wave's LDS operations: tagged
// stores of the look-back stay in flight across it (a __syncthreads() would
// wait for their acknowledgement from memory).  Only LDS carries data between
// the waves here.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Builds the tree of the tile's chunk aggregates in `nodes` (X holds chunk
// tl.q's aggregate on entry) and leaves the root in X of wave 0 (both
// halves) and in node (L, 0), written by wave 0's lower half and read only by
// it.  DIR = +1: forward composition; DIR = -1: reverse.  Ends with every
// other node visible to the whole workgroup.
template <int KIND, int K, int NCH, int DIR>
__device__ __forceinline__ void tree_build(float (*nodes)[32][(AggShape<KIND, K>::stride)], const Tile &tl,
                                           float (&X)[AggShape<KIND, K>::words])
{
    constexpr int AW = AggShape<KIND, K>::words;
    constexpr int L = tree_levels<NCH>();
#pragma unroll
    for (int e = 0; e < AW; ++e) nodes[tree_node<NCH, DIR>(0, tl.q)][tl.slot][e] = X[e];
    // level 1 inside each wave: its halves hold chunks 2w and 2w + 1 (lanes l
    // and l ^ 32 serve the same row of the same chain).  One permlane32 swap
    // of a value with itself leaves the lower half's value in every lane of
    // the first result and the upper half's in every lane of the second (a
    // VALU exchange, no LDS round trip); both halves then compose the same pair.
    {
        float Y[AW], R[AW];
#pragma unroll
        for (int e = 0; e < AW; ++e) {
            const unsigned u = __float_as_uint(X[e]);
            const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
            const float lo = __uint_as_float(sw[0]), hi = __uint_as_float(sw[1]);
            Y[e] = DIR > 0 ? hi : lo;   // the factor applied last: the later chunk
            R[e] = DIR > 0 ? lo : hi;
        }
        compose_into<KIND, K>(Y, R);
#pragma unroll
        for (int e = 0; e < AW; ++e) X[e] = Y[e];
        if (L > 1 && tl.sub == 0)
#pragma unroll
            for (int e = 0; e < AW; ++e) nodes[tree_node<NCH, DIR>(1, tl.wv)][tl.slot][e] = X[e];
    }
    lds_barrier();
#pragma unroll
    for (int l = 2; l <= L; ++l) {
        if (tl.wv < (NCH >> l)) {
            const float *lo = nodes[tree_node<NCH, DIR>(l - 1, 2 * tl.wv)][tl.slot];
            const float *hi = nodes[tree_node<NCH, DIR>(l - 1, 2 * tl.wv + 1)][tl.slot];
            float R[AW];
#pragma unroll
            for (int e = 0; e < AW; ++e) {
                X[e] = DIR > 0 ? hi[e] : lo[e];
                R[e] = DIR > 0 ? lo[e] : hi[e];
            }
            compose_into<KIND, K>(X, R);
            if (l < L && tl.sub == 0)
#pragma unroll
                for (int e = 0; e < AW; ++e) nodes[tree_node<NCH, DIR>(l, tl.wv)][tl.slot][e] = X[e];
        }
        if (l < L) lds_barrier();
    }
    // the root, for wave 0 alone (publishing the tile's inclusive state later),
    // so that no wave keeps it in registers across the look-back
    if (tl.wv == 0 && tl.sub == 0)
#pragma unroll
        for (int e = 0; e < AW; ++e) nodes[tree_node<NCH, DIR>(L, 0)][tl.slot][e] = X[e];
}

// State entering chunk tl.q from the state c entering the tile: the nodes
// covering chunks [0, q) in order (forward), or [q + 1, NCH) from the end
// (reverse).
template <int KIND, int K, int NCH, int DIR>
__device__ __forceinline__ void tree_apply(float (*nodes)[32][(AggShape<KIND, K>::stride)], const Tile &tl,
                                           float *c)
{
    constexpr int L = tree_levels<NCH>();
    const int r = DIR > 0 ? tl.q : NCH - 1 - tl.q;   // chunks to cover
    int at = DIR > 0 ? 0 : NCH;                        // forward: next start; reverse: current end
#pragma unroll
    for (int l = L - 1; l >= 0; --l) {
        if ((r >> l) & 1) {
            const int i = DIR > 0 ? (at >> l) : ((at >> l) - 1);
            Carry<KIND, K>::apply(nodes[tree_node<NCH, DIR>(l, i)][tl.slot], c);
            at += DIR * (1 << l);
        }
    }
}

// Look-back words in the workspace are word-major per tile ([tile][word][slot]),
// so a word of all 32 slots is 256 contiguous bytes for a tile's loads and stores.
template <int NW>
__device__ __forceinline__ void publish_wm(uint64_t *dst, int tile, int slot, uint32_t tag, const float *x, bool local)
{
    uint64_t *p = dst + static_cast<size_t>(tile) * NW * 32 + slot;
#pragma unroll
    for (int e = 0; e < NW; ++e) tagged_store(p + e * 32, tag, x[e], local);
}

// The look-back walk over matrix carries for k = 8 on v_mfma_f32_4x4x1f32.
// The instruction's 16 blocks are 4 x 4 outer products: block b adds the A
// operand of lane 4b + i times the B operand of lane 4b + j to register i of
// lane 4b + j, and a block never leaves a chain's 8 lanes.  While the staged
// aggregates are applied (c <- G c, plus W for the reverse scan's carries), the
// carry is held by columns, lane v of a chain holding column v: the B operand
// is the lane's own column, the A operand row 4q + i of G read straight from
// the staged words, and register i of instruction q gathers entry 4q + i of
// the new column.  One transpose through LDS each way (sT: this chain's rows,
// written and read by wave 0 alone) frames the walk.
template <int KIND, int SW>
__device__ __forceinline__ void walk_mfma8(float (*sLB)[32][SW], float (*sT)[8], int slot, int v, int stop, float *c)
{
    constexpr int CW = 8;
    const int cb = slot & ~7, i = v & 3;
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // rows (slot s of row v holds column s ^ (v & 4)) -> columns
#pragma unroll
    for (int s = 0; s < 8; ++s) sT[cb + (s ^ (v & 4))][v] = c[s];
    wave_sync();
    float cc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) cc[m] = sT[cb + v][m];
    for (int u = stop - 1; u >= 0; --u) {
        const float *g = &sLB[u][cb][CW];   // row r of G at g + r SW, its column m at word m ^ (r & 4)
        f32x4 d[2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) d[q][e] = KIND == kMatMat ? g[(4 * q + e) * SW + 8 + (v ^ (4 * q))] : 0.0f;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                d[q] = __builtin_amdgcn_mfma_f32_4x4x1f32(g[(4 * q + i) * SW + (m ^ (4 * q))], cc[m], d[q], 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) cc[4 * q + e] = d[q][e];
    }
    // columns -> rows
    wave_sync();
#pragma unroll
    for (int m = 0; m < 8; ++m) sT[cb + m][v] = cc[m];
    wave_sync();
#pragma unroll
    for (int s = 0; s < 8; ++s) c[s] = sT[cb + v][s ^ (v & 4)];
    wave_sync();
}

// Look-back of a tile whose tree is built (X: the tile aggregate, read by
// wave 0's lower half alone, from LDS).
// Polling units -- half-waves of waves 1 .. W-1 when a tile's CW + AW words
// are few, else whole waves whose halves split the words -- each poll one
// predecessor (the nearest units in the scan direction: earlier tiles for
// DIR = +1, later ones for DIR = -1) for its inclusive state and its
// aggregate in one batch of loads, and stage what they find in LDS.  In the
// first round a half-wave unit polls again, back to back, until its
// predecessor shows its aggregate or its inclusive state: every tile
// publishes its aggregate right after its own tree, waiting on no other tile,
// so this wait ends, and the round then needs one barrier instead of a
// barrier round trip per poll.
// Wave 0 then reads every unit's status at once and walks from the nearest
// predecessor: it stops at the first published inclusive state (or past the
// end of the sequence, whose state base0 is known) and applies the
// aggregates of the tiles passed on the way.  A window without an inclusive
// state that does not reach the end of the sequence means another round
// (one poll per unit).  `overlap` runs once on every wave while the first
// poll's loads are in flight (wave 0: before its first wait for the units).  Leaves the state
// entering the tile in c (every lane, its slot) and publishes the tile's
// inclusive state when publish_incl.
template <int KIND, int K, int W, int DIR, typename F>
__device__ __forceinline__ void block_lookback(const BlkArgs &a, const Tile &tl, int ftile, const uint32_t *launch,
                                               const float *X, const float *base0, bool publish_incl,
                                               float *c, float *dead, F &&overlap)
{
    using Cr = Carry<KIND, K>;
    constexpr int CW = Cr::CW, AW = Cr::AW, NWD = CW + AW;
    constexpr bool HALF = NWD <= 12;
    constexpr int NU = HALF ? 2 * (W - 1) : W - 1;
    constexpr int PER = HALF ? NWD : (NWD + 1) / 2;   // words one lane loads
    constexpr int SW = NWD | 1;
    static_assert(NU > 0 && NU < 64, "the look-back needs more than one wave");
    static_assert(HALF || (NWD % 2 == 0 && PER >= CW), "whole-wave units split the words evenly");
    // staging: the tree's dead nodes when they hold it (first written only
    // after a barrier that follows the tree's last reads), else an array of
    // its own
    constexpr bool ALIAS = dead_nodes_floats<KIND, K, 2 * W>() >= NU * 32 * SW;
    float (*sLB)[32][SW];
    if constexpr (ALIAS) {
        sLB = reinterpret_cast<float (*)[32][SW]>(dead);
    } else {
        __shared__ float sOwn[NU][32][SW];
        sLB = sOwn;
    }
    __shared__ int sStat[NU];
    __shared__ float sCar[32][CW];
    __shared__ int sDone;
#pragma unroll
    for (int e = 0; e < CW; ++e) c[e] = base0[e];
    // launch[0]: the tag this launch publishes; [1]: the tag its waits expect; [2]: their poll limit
    const uint32_t tag = launch[0], want = launch[1], limit = launch[2];
    for (uint32_t spin = 0;; ++spin) {
        if (tl.wv > 0) {
            const int u = HALF ? 2 * (tl.wv - 1) + tl.sub : tl.wv - 1;
            const int p = tl.j - DIR * (1 + u);
            const bool in = p >= 0 && p < a.nT;
            const size_t ti = static_cast<size_t>(in ? p : tl.j) * a.nCG + tl.cg;
            // this lane's words e0 .. e0 + PER - 1 of the predecessor's CW
            // inclusive then AW aggregate words (HALF: all of them): two base
            // pointers and constant offsets, so the polling loop holds no
            // per-word addresses
            const bool lower = HALF || tl.sub == 0;
            const int e0 = lower ? 0 : PER;
            const uint64_t *wI = a.incl + ti * CW * 32 + tl.slot;
            const uint64_t *wA = a.agg + ti * AW * 32 + tl.slot;
            const uint64_t *p0 = lower ? wI : wA + (PER - CW) * 32;   // the lane's words i < CW
            const uint64_t *p1 = lower ? wA : wA + PER * 32;          // and i >= CW
            uint64_t wd[PER];
            bool rI, rA;
            for (uint32_t n = 0;; ++n) {
#pragma unroll
                for (int i = 0; i < PER; ++i) wd[i] = tagged_load(i < CW ? p0 + i * 32 : p1 + (i - CW) * 32);
                if (spin == 0 && n == 0) overlap();
                bool okI = true, okA = true;
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    if (lower && i < CW) okI = okI && tag_is(wd[i], want);
                    else if (e0 + i < NWD) okA = okA && tag_is(wd[i], want);
                }
                const uint64_t bI = __ballot(okI), bA = __ballot(okA);
                rI = HALF ? static_cast<uint32_t>(bI >> (32 * tl.sub)) == 0xFFFFFFFFu : bI == ~0ull;
                rA = HALF ? static_cast<uint32_t>(bA >> (32 * tl.sub)) == 0xFFFFFFFFu : bA == ~0ull;
                // first round: again while a unit of this wave sees neither
                // (half-wave units: whole-wave ones, with twice the words per
                // poll, measured slower when they spun -- k = 16 block-affine
                // pair 79.2 -> 83.0 us)
                const bool again = HALF && spin == 0 && in && !rI && !rA && n < limit;
                if (__ballot(again) == 0) break;
            }
            if (ALIAS && spin == 0) lds_barrier();   // the tree's last level has read the dead nodes
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (e0 + i < NWD) sLB[u][tl.slot][e0 + i] = tag_value(wd[i]);
            if (HALF ? tl.slot == 0 : tl.lane == 0) sStat[u] = in ? ((rA ? 1 : 0) | (rI ? 2 : 0)) : 4;
        } else if (spin == 0) {
            overlap();   // wave 0's own work while the units poll
            if (ALIAS) lds_barrier();
        }
        lds_barrier();
        if (tl.wv == 0) {
            // every unit's status at once (4 = past the end of the sequence,
            // 2 = inclusive, 1 = aggregate); stop at the nearest unit showing
            // an inclusive state or the end, every nearer one an aggregate
            const int st = tl.lane < NU ? sStat[tl.lane] : 0;
            const uint64_t mStop = __ballot((st & 6) != 0), mAgg = __ballot((st & 1) != 0);
            const uint64_t mEnd = __ballot((st & 4) != 0);
            const int stop = mStop ? static_cast<int>(__builtin_ctzll(mStop)) : -1;
            const bool ok = stop >= 0 && ((~mAgg) & ((1ull << stop) - 1)) == 0;
            if (ok) {
                if (!((mEnd >> stop) & 1))
#pragma unroll
                    for (int e = 0; e < CW; ++e) c[e] = sLB[stop][tl.slot][e];
                // the aggregates from the farthest to the nearest; a
                // matrix-vector aggregate is read from LDS one step ahead of
                // its use (the larger ones would not fit the registers)
                if constexpr (KIND == kMatVec) {
                    float g[AW];
                    if (stop > 0)
#pragma unroll
                        for (int e = 0; e < AW; ++e) g[e] = sLB[stop - 1][tl.slot][CW + e];
                    for (int u = stop - 1; u >= 0; --u) {
                        float gn[AW];
                        if (u > 0)
#pragma unroll
                            for (int e = 0; e < AW; ++e) gn[e] = sLB[u - 1][tl.slot][CW + e];
                        Cr::apply(g, c);
#pragma unroll
                        for (int e = 0; e < AW; ++e) g[e] = gn[e];
                    }
                } else if constexpr (K == 8) {
                    if (stop > 0) walk_mfma8<KIND, SW>(sLB, sCar, tl.slot, tl.v, stop, c);
                } else {
                    for (int u = stop - 1; u >= 0; --u) Cr::apply(&sLB[u][tl.slot][CW], c);
                }
                if (tl.sub == 0)
#pragma unroll
                    for (int e = 0; e < CW; ++e) sCar[tl.slot][e] = c[e];
            }
            if (tl.lane == 0) sDone = ok ? 1 : 0;
        }
        lds_barrier();
        if (sDone) break;
        if (spin >= limit) {
            if (threadIdx.x == 0) raise_error(&a.hd->err, kErrSpin);
            if (tl.wv == 0 && tl.sub == 0)
#pragma unroll
                for (int e = 0; e < CW; ++e) sCar[tl.slot][e] = base0[e];
            lds_barrier();
            break;
        }
        backoff();
    }
    if (tl.wv == 0) {
        if (publish_incl && tl.sub == 0) {
            float xo[CW];
#pragma unroll
            for (int e = 0; e < CW; ++e) xo[e] = c[e];
            Cr::apply(X, xo);
            publish_wm<CW>(a.incl, ftile, tl.slot, tag, xo, a.lb_local);
        }
    } else {
#pragma unroll
        for (int e = 0; e < CW; ++e) c[e] = sCar[tl.slot][e];
    }
}

// A tile with no predecessor in the scan direction publishes its inclusive
// state, the tile aggregate applied to the known state base0 entering it.
template <int KIND, int K>
__device__ __forceinline__ void publish_first(const BlkArgs &a, const Tile &tl, int ftile, uint32_t tag,
                                              const float *X, const float *base0)
{
    using Cr = Carry<KIND, K>;
    if (tl.wv == 0 && tl.sub == 0) {
        float xo[Cr::CW];
#pragma unroll
        for (int e = 0; e < Cr::CW; ++e) xo[e] = base0[e];
        Cr::apply(X, xo);
        publish_wm<Cr::CW>(a.incl, ftile, tl.slot, tag, xo, a.lb_local);
    }
}

// Forward: X = (row of Phi, entry of u) is the chunk's aggregate.  Builds the
// tile's tree, runs the look-back (multi-tile launches) and returns the state
// entering this lane's chunk.
template <int K, int C, int W, bool MULTI>
__device__ __forceinline__ float affine_fwd_carry(const BlkArgs &a, const Tile &tl, int ftile, const Launch &ep,
                                                  float (&X)[K + 1], float xh0,
                                                  float (&sKS)[2][2 * W][32][(AggShape<kMatVec, K>::stride)],
                                                  float (&sCarry)[32], uint32_t (&sTicket)[3])
{
    constexpr int NCH = 2 * W;
    using S = AggShape<kMatVec, K>;
    using Rw = Rows<K>;
    if constexpr (MULTI) {
        float (*nodes)[32][S::stride] = reinterpret_cast<float (*)[32][S::stride]>(&sKS[0][0][0][0]);
        if (threadIdx.x == 0) epoch_end(a.hd, ep, a.nTiles, sTicket);
        tree_build<kMatVec, K, NCH, +1>(nodes, tl, X);   // its first barrier also shares the tag
        const uint32_t tag = sTicket[0];
        if (tl.wv == 0 && tl.sub == 0 && tl.j < a.nT - 1) publish_wm<S::words>(a.agg, ftile, tl.slot, tag, X, a.lb_local);
        const float *root = nodes[tree_node<NCH, +1>(tree_levels<NCH>(), 0)][tl.slot];
        float c = xh0;
        if (tl.j > 0)
            block_lookback<kMatVec, K, W, +1>(a, tl, ftile, sTicket, root, &xh0, tl.j < a.nT - 1, &c, &nodes[0][0][0],
                                              [] {});
        else if (a.nT > 1)
            publish_first<kMatVec, K>(a, tl, ftile, tag, root, &xh0);
        tree_apply<kMatVec, K, NCH, +1>(nodes, tl, &c);
        return c;
    } else {
        ks_store<kMatVec, K, NCH>(sKS[0], tl.q, tl.slot, X);
        __syncthreads();
        float x = xh0;
        for (int q = 0; q < tl.q; ++q) x = Rw::mv(sKS[0][q][tl.slot], x, sKS[0][q][tl.slot][K]);
        return x;
    }
}

// Backward: X = (row of Psi, entry of Wl) is the chunk's reverse aggregate.
// Returns w entering this lane's chunk from its end.
template <int K, int C, int W, bool MULTI>
__device__ __forceinline__ float affine_bwd_carry(const BlkArgs &a, const Tile &tl, int ftile, const Launch &ep,
                                                  float (&X)[K + 1],
                                                  float (&sKS)[2][2 * W][32][(AggShape<kMatVec, K>::stride)],
                                                  float (&sCarry)[32], uint32_t (&sTicket)[3])
{
    constexpr int NCH = 2 * W;
    using S = AggShape<kMatVec, K>;
    using Rw = Rows<K>;
    if constexpr (MULTI) {
        float (*nodes)[32][S::stride] = reinterpret_cast<float (*)[32][S::stride]>(&sKS[0][0][0][0]);
        if (threadIdx.x == 0) epoch_end(a.hd, ep, a.nTiles, sTicket);
        tree_build<kMatVec, K, NCH, -1>(nodes, tl, X);
        const uint32_t tag = sTicket[0];
        if (tl.wv == 0 && tl.sub == 0 && tl.j > 0) publish_wm<S::words>(a.agg, ftile, tl.slot, tag, X, a.lb_local);
        const float *root = nodes[tree_node<NCH, -1>(tree_levels<NCH>(), 0)][tl.slot];
        const float zero = 0.0f;
        float w = 0.0f;
        if (tl.j < a.nT - 1)
            block_lookback<kMatVec, K, W, -1>(a, tl, ftile, sTicket, root, &zero, tl.j > 0, &w, &nodes[0][0][0],
                                              [] {});
        else if (a.nT > 1)
            publish_first<kMatVec, K>(a, tl, ftile, tag, root, &zero);
        tree_apply<kMatVec, K, NCH, -1>(nodes, tl, &w);
        return w;
    } else {
        ks_store<kMatVec, K, NCH>(sKS[0], tl.q, tl.slot, X);
        __syncthreads();
        float w = 0.0f;
        for (int q = NCH - 1; q > tl.q; --q) w = Rw::mv(sKS[0][q][tl.slot], w, sKS[0][q][tl.slot][K]);
        return w;
    }
}

// ======================================================= block-affine fwd
// GIV = false: A_t is loaded; GIV = true: A_t = sigmoid(s_t) R(theta_t) is
// formed from the angles and the gate (the Givens angle-fused scan).

template <int K, bool GIV, int C, int W, bool MULTI>
__device__ __forceinline__ void affine_fwd_body(const BlkArgs &a)
{
    static_assert(!GIV || K == 8, "the Givens angle-fused scan is built for k = 8");
    constexpr int NCH = 2 * W;
    using Rw = Rows<K>;
    __shared__ float sKS[2][NCH][32][(AggShape<kMatVec, K>::stride)];
    __shared__ float sCarry[32];
    __shared__ uint32_t sTicket[3];
    __shared__ float sCS[GIV ? W : 1][64][kCSLd];

    const int tile = blockIdx.x;
    const Tile tl = make_tile<K, C, W>(a, tile, false);
    const int ftile = tl.j * a.nCG + tl.cg;

    // unconditional (clamped) loads keep every load in flight at once
    float Ar[C][K], bv[C];
    if constexpr (!GIV) {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int t = clampT(tl.t0 + i, a.T);
            Rw::load_row(a.A + tl.ablk0 + t * tl.astep, tl.v, Ar[i]);
            bv[i] = load_once(&a.x[tl.vec0 + t * tl.vstep]);
        }
    } else {
        float4 th[C];
        float sv[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int t = clampT(tl.t0 + i, a.T);
            th[i] = load_angles(a, tl, t);
            sv[i] = a.sg[tl.blk0 + static_cast<int64_t>(t) * a.nb];
            bv[i] = load_once(&a.x[tl.vec0 + t * tl.vstep]);
        }
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float cc[kAngles], ss[kAngles], r[8];
            mesh_share(th[i], sCS[tl.wv % (GIV ? W : 1)], tl.lane, cc, ss);
            mesh_row(cc, ss, tl.v, r);
            to_slots(r, tl.v, sigmoidf_(sv[i]), Ar[i]);
            settle8(Ar[i]);
        }
    }
    const float xh0 = load_h0<K>(a, tl);
    // the launch ticket after the inputs: its atomic returns behind them
    // rather than ahead of them in wave 0's in-order load queue
    Launch ep{0, 0};
    if constexpr (MULTI) ep = epoch_begin(a.hd);
#pragma unroll
    for (int i = 0; i < C; ++i)
        if (!(tl.cv && tl.t0 + i < a.T)) {
            Rw::eye(tl.v, Ar[i]);
            bv[i] = 0.0f;
        }

    // chunk aggregate from a zero state: X = (A_e..A_s, local h_e)
    float X[K + 1];
#pragma unroll
    for (int s = 0; s < K; ++s) X[s] = Ar[0][s];
    X[K] = bv[0];
#pragma unroll
    for (int i = 1; i < C; ++i) {
        float np[K];
        Rw::mm(Ar[i], X, np);
        X[K] = Rw::mv(Ar[i], X[K], bv[i]);
#pragma unroll
        for (int s = 0; s < K; ++s) X[s] = np[s];
    }
    float x = affine_fwd_carry<K, C, W, MULTI>(a, tl, ftile, ep, X, xh0, sKS, sCarry, sTicket);

    // re-run the recurrence from the true state entering the chunk
#pragma unroll
    for (int i = 0; i < C; ++i) {
        x = Rw::mv(Ar[i], x, bv[i]);
        const int t = tl.t0 + i;
        if (tl.cv && t < a.T) store_out(&a.out[tl.vec0 + t * tl.vstep], x);
    }
}

template <int K, int C, int W, bool MULTI>
__global__ void __launch_bounds__(64 * W) baffine_fwd_kernel(BlkArgs a)
{
    affine_fwd_body<K, false, C, W, MULTI>(a);
}

template <int C, int W, bool MULTI>
__global__ void __launch_bounds__(64 * W) bgivens_fwd_kernel(BlkArgs a)
{
    affine_fwd_body<8, true, C, W, MULTI>(a);
}

// ======================================================= block-affine bwd
// Reverse scan on w_t = A_t^T g_t with g_t = dh_t + w_{t+1}; per chunk [s, e]
// w_s = Psi w_{e+1} + Wl with Psi = A_s^T .. A_e^T.

template <int K, int C, int W, bool MULTI>
__global__ void __launch_bounds__(64 * W) baffine_bwd_kernel(BlkArgs a)
{
    constexpr int NCH = 2 * W;
    using Rw = Rows<K>;
    __shared__ float sKS[2][NCH][32][(AggShape<kMatVec, K>::stride)];
    __shared__ float sCarry[32];
    __shared__ uint32_t sTicket[3];

    const int tile = blockIdx.x;
    const Tile tl = make_tile<K, C, W>(a, tile, true);
    const int ftile = tl.j * a.nCG + tl.cg;

    // Multi-tile launches load in the order the chunk aggregate consumes the
    // inputs (the last step first; h_{t-1}, needed only in the fix-up, after
    // all of them): a wave's loads complete in issue order, so the aggregate
    // starts on the last step while the earlier steps' loads are in flight
    // (long-T backward 21.5 -> 20.9 us, k = 16 49.9 -> 48.4 us).  A single
    // tile waits for all its loads at its first barrier anyway, and keeps the
    // plain order (10.2 us against 10.4 us reversed at the lab shape).
    float ATr[C][K], gv[C], hp[C];   // rows of A_t^T, upstream dh_t, h_{t-1}
    if constexpr (MULTI) {
#pragma unroll
        for (int i = C - 1; i >= 0; --i) {
            const int t = clampT(tl.t0 + i, a.T);
            Rw::load_col(a.A + tl.ablk0 + t * tl.astep, tl.v, ATr[i]);
            gv[i] = load_once(&a.y[tl.vec0 + t * tl.vstep]);
        }
#pragma unroll
        for (int i = C - 1; i >= 0; --i) {
            const int t = clampT(tl.t0 + i, a.T);
            hp[i] = load_once(&a.x[tl.vec0 + (t > 0 ? t - 1 : 0) * tl.vstep]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int t = clampT(tl.t0 + i, a.T);
            Rw::load_col(a.A + tl.ablk0 + t * tl.astep, tl.v, ATr[i]);
            gv[i] = load_once(&a.y[tl.vec0 + t * tl.vstep]);
            hp[i] = load_once(&a.x[tl.vec0 + (t > 0 ? t - 1 : 0) * tl.vstep]);
        }
    }
    const float xh0 = load_h0<K>(a, tl);
    // the launch ticket after the inputs (see the forward)
    Launch ep{0, 0};
    if constexpr (MULTI) ep = epoch_begin(a.hd);

    // A step past T (or of a chain past the last) is the identity.  A single
    // tile makes its inputs so up front; a multi-tile launch leaves the loaded
    // registers alone and selects the step's results instead, so that nothing
    // touches a step's registers before the aggregate reaches the step (the
    // compiler would otherwise wait on all the loads at the first select).
    if constexpr (!MULTI) {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int t = tl.t0 + i;
            if (t == 0) hp[i] = xh0;
            if (!(tl.cv && t < a.T)) {
                Rw::eye(tl.v, ATr[i]);
                gv[i] = 0.0f;
                hp[i] = 0.0f;
            }
        }
    }
    auto live = [&](int i) { return !MULTI || (tl.cv && tl.t0 + i < a.T); };

    // chunk aggregate from a zero carry, walking t downwards: X = (Psi, Wl)
    float X[K + 1];
    {
        float E[K];
        Rw::eye(tl.v, E);
        const bool v = live(C - 1);
#pragma unroll
        for (int s = 0; s < K; ++s) X[s] = v ? ATr[C - 1][s] : E[s];
        X[K] = v ? Rw::mv(ATr[C - 1], gv[C - 1], 0.0f) : 0.0f;
    }
#pragma unroll
    for (int i = C - 2; i >= 0; --i) {
        float np[K];
        Rw::mm(ATr[i], X, np);
        const float nw = Rw::mv(ATr[i], gv[i] + X[K], 0.0f);
        const bool v = live(i);
#pragma unroll
        for (int s = 0; s < K; ++s) X[s] = v ? np[s] : X[s];
        X[K] = v ? nw : X[K];
    }
    float w = affine_bwd_carry<K, C, W, MULTI>(a, tl, ftile, ep, X, sKS, sCarry, sTicket);

    // re-run the reverse recurrence from the true carry; emit dA, db, dh0
#pragma unroll
    for (int i = C - 1; i >= 0; --i) {
        const int t = tl.t0 + i;
        const bool v = live(i);
        const float g = (v ? gv[i] : 0.0f) + w;
        const float hprev = !MULTI ? hp[i] : (!v ? 0.0f : (t == 0 ? xh0 : hp[i]));
        float dAr[K];
        Rw::outer(g, hprev, dAr);
        const float wn = Rw::mv(ATr[i], g, 0.0f);
        w = v ? wn : g;
        if (tl.cv && t < a.T) {
            store_out(&a.out2[tl.vec0 + t * tl.vstep], g);
            Rw::store_row(a.out + tl.ablk0 + t * tl.astep, tl.v, dAr);
        }
    }
    if (tl.cv && tl.t0 == 0) store_out(&a.out3[tl.bb * a.d + tl.jb * K + tl.v], w);   // A_1^T g_1
}

// =============================================== Givens angle-fused bwd
// Same reverse scan with A_t = sigmoid(s_t) R(theta_t), the mesh applied
// layer by layer across the chain's lanes (A^T = sigmoid L_0^T .. L_7^T).
// dA_t = g_t h_{t-1}^T is never formed: with y_l the state entering layer l
// (y_0 = h_{t-1}) and z_l the gradient on layer l's output (z_7 = sigmoid g_t,
// z_{l-1} = L_l^T z_l), the angle of the pair (i, j) in layer l has gradient
//     z_j y_{l+1,i} - z_i y_{l+1,j},
// which the pair's two lanes form from each other's values, and
//     ds_t = sigmoid'(s_t) <g_t, R h_{t-1}> = sigmoid'(s_t) <g_t, y_8>.
// z_{-1} = A_t^T g_t is the carry to the step before.  Each lane writes the
// gradients of the four angles it evaluated.

template <int C, int W, bool MULTI>
__global__ void __launch_bounds__(64 * W) bgivens_bwd_kernel(BlkArgs a)
{
    __shared__ float sKS[2][2 * W][32][(AggShape<kMatVec, 8>::stride)];
    __shared__ float sCarry[32];
    __shared__ uint32_t sTicket[3];

    const int tile = blockIdx.x;
    const Tile tl = make_tile<8, C, W>(a, tile, true);
    const int ftile = tl.j * a.nCG + tl.cg;
    const MeshLane ml = mesh_lane(tl.v);

    // Multi-tile launches load in the order the first pass consumes the
    // inputs (the last step first; h_{t-1} after every step's angles, gate and
    // dh_t), and each step is evaluated (sin / cos, gate) inside the pass, so
    // the pass starts on the last step while the others' loads are in flight
    // (long-T backward 30.3 -> 28.8 us).  Their addresses are a base plus a
    // multiple of a launch-wide stride (a step past T reads the tile's first
    // step inside the sequence; the identity step replaces it where it is
    // used): no per-lane 64-bit products between the loads, whose temporaries
    // the compiler would place in registers of loads still in flight.  A
    // single tile keeps the plain order and evaluates up front (14.3 us
    // against 15.6 us the other way at the lab shape).
    float4 th[C];
    float sig[C], sgd[C], gv[C], hp[C];   // gate sigmoid(s), its derivative, dh_t, h_{t-1}
    float ev[C][8];   // this lane's four cosines and signed sines per step
    // with e = exp(-|s|): sigmoid(|s|) = 1 / (1 + e) and sigmoid'(s) =
    // e / (1 + e)^2, exact in relative terms (1 - sigmoid(s) would cancel once
    // sigmoid(s) nears 1); an invalid step is the identity (zero angles, gate 1)
    auto evaluate = [&](int i) {
        const bool valid = tl.cv && tl.t0 + i < a.T;
        if (!valid) {
            th[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            gv[i] = 0.0f;
        }
        const float e = __expf(-fabsf(sig[i])), r = 1.0f / (1.0f + e);
        sgd[i] = valid ? e * r * r : 0.0f;
        sig[i] = valid ? (sig[i] >= 0.0f ? r : e * r) : 1.0f;
        mesh_eval(th[i], ml, ev[i]);
    };
    if constexpr (MULTI) {
        const int64_t nbs = a.nb, vs = tl.vstep;
        const int tin = max(min(tl.t0, a.T - 1), 0);
        const int64_t sb = tl.blk0 + static_cast<int64_t>(tl.t0) * nbs, sbi = tl.blk0 + static_cast<int64_t>(tin) * nbs;
        const int64_t vb = tl.vec0 + static_cast<int64_t>(tl.t0) * vs, vbi = tl.vec0 + static_cast<int64_t>(tin) * vs;
#pragma unroll
        for (int i = C - 1; i >= 0; --i) {
            const bool in = tl.t0 + i < a.T;
            const int64_t si = in ? sb + i * nbs : sbi;
            th[i] = mesh_angles_at(a.theta + si * kAngles, ml);
            sig[i] = a.sg[si];
            gv[i] = load_once(&a.y[in ? vb + i * vs : vbi]);
        }
#pragma unroll
        for (int i = C - 1; i >= 0; --i) {
            const bool in = tl.t0 + i < a.T && tl.t0 + i > 0;
            hp[i] = load_once(&a.x[in ? vb + (i - 1) * vs : vbi]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int t = clampT(tl.t0 + i, a.T);
            const float *p = a.theta + (tl.blk0 + static_cast<int64_t>(t) * a.nb) * kAngles;
            th[i] = make_float4(p[ml.ie], p[ml.ie + 7], ml.oddp ? p[ml.io] : 0.0f, ml.oddp ? p[ml.io + 7] : 0.0f);
            sig[i] = a.sg[tl.blk0 + static_cast<int64_t>(t) * a.nb];
            gv[i] = load_once(&a.y[tl.vec0 + t * tl.vstep]);
            hp[i] = load_once(&a.x[tl.vec0 + (t > 0 ? t - 1 : 0) * tl.vstep]);
        }
    }
    const float xh0 = load_h0<8>(a, tl);
    Launch ep{0, 0};   // the launch ticket after the inputs (see the block-affine forward)
    if constexpr (MULTI) ep = epoch_begin(a.hd);
    if constexpr (!MULTI) {   // a single tile evaluates every step up front
#pragma unroll
        for (int i = 0; i < C; ++i) evaluate(i);
    }

    // chunk aggregate from a zero carry, walking t downwards: X = (Psi, Wl),
    // Psi <- A_t^T Psi, Wl <- A_t^T (dh_t + Wl)
    float X[9];
    eye_row8(tl.v, X);
    X[8] = 0.0f;
#pragma unroll
    for (int i = C - 1; i >= 0; --i) {
        if constexpr (MULTI) evaluate(i);   // a multi-tile launch evaluates each step as it reaches it
        float c[8], s[8];
        mesh_coef(ev[i], ml, c, s);
        c[0] *= sig[i];
        s[0] *= sig[i];
        X[8] += gv[i];
#pragma unroll
        for (int l = 7; l >= 0; l -= 2) {   // transposed layers: sines negated
            const float q = ml.mir ? 0.0f : -s[l], m = ml.mir ? -s[l] : 0.0f;
            mesh_rows2r(X, c[l], q, m, c[l - 1], -s[l - 1]);
        }
    }
    float w = affine_bwd_carry<8, C, W, MULTI>(a, tl, ftile, ep, X, sKS, sCarry, sTicket);

#pragma unroll
    for (int i = C - 1; i >= 0; --i) {
        const float g = gv[i] + w;
        float c[8], s[8], y[8], d[8];
        mesh_coef(ev[i], ml, c, s);
        const int t = tl.t0 + i;
        float x = tl.cv && t < a.T ? (t == 0 ? xh0 : hp[i]) : 0.0f;
#pragma unroll
        for (int l = 0; l < 8; ++l) y[l] = x = mesh_vec(x, c[l], s[l], l, ml.mir);
        const float ds = chain_sum8(g * y[7]) * sgd[i];
        float z = sig[i] * g;
#pragma unroll
        for (int l = 7; l >= 0; --l) {
            const float zp = mesh_partner(z, l, ml.mir), yp = mesh_partner(y[l], l, ml.mir);
            d[l] = zp * y[l] - z * yp;   // the first lane's angle gradient; the second lane's negated
            z = __builtin_fmaf(-s[l], zp, c[l] * z);
        }
        w = z;
        if (tl.cv && t < a.T) {
            float *dth = a.dtheta + (tl.blk0 + static_cast<int64_t>(t) * a.nb) * kAngles;
            store_out(&a.out2[tl.vec0 + t * tl.vstep], g);
            dth[ml.ie] = ml.re ? -d[4] : d[0];
            dth[ml.ie + 7] = ml.re ? -d[6] : d[2];
            if (ml.oddp) {
                dth[ml.io] = ml.ro ? -d[5] : d[1];
                dth[ml.io + 7] = ml.ro ? -d[7] : d[3];
            } else if (tl.v == 7) {
                a.dsg[tl.blk0 + static_cast<int64_t>(t) * a.nb] = ds;
            }
        }
    }
    if (tl.cv && tl.t0 == 0) store_out(&a.out3[tl.bb * a.d + tl.jb * 8 + tl.v], w);   // A_1^T g_1
}

// ================================================ block cumulative product

template <int K, int C, int W, bool MULTI>
__global__ void __launch_bounds__(64 * W) bmatrix_fwd_kernel(BlkArgs a)
{
    constexpr int NCH = 2 * W;
    using S = AggShape<kMat, K>;
    using Rw = Rows<K>;
    __shared__ float sKS[2][NCH][32][S::stride];
    __shared__ uint32_t sTicket[3];

    const int tile = blockIdx.x;
    const Tile tl = make_tile<K, C, W>(a, tile, false);
    const int ftile = tl.j * a.nCG + tl.cg;

    float Ar[C][K];
#pragma unroll
    for (int i = 0; i < C; ++i)
        Rw::load_row(a.A + tl.ablk0 + clampT(tl.t0 + i, a.T) * tl.astep, tl.v, Ar[i]);
    Launch ep{0, 0};   // the launch ticket after the inputs (see the block-affine forward)
    if constexpr (MULTI) ep = epoch_begin(a.hd);
#pragma unroll
    for (int i = 0; i < C; ++i)
        if (!(tl.cv && tl.t0 + i < a.T)) Rw::eye(tl.v, Ar[i]);

    float X[K];
#pragma unroll
    for (int s = 0; s < K; ++s) X[s] = Ar[0][s];
#pragma unroll
    for (int i = 1; i < C; ++i) {
        float np[K];
        Rw::mm(Ar[i], X, np);
#pragma unroll
        for (int s = 0; s < K; ++s) X[s] = np[s];
    }
    float (*nodes)[32][S::stride] = reinterpret_cast<float (*)[32][S::stride]>(&sKS[0][0][0][0]);
    if (MULTI && threadIdx.x == 0) epoch_end(a.hd, ep, a.nTiles, sTicket);
    tree_build<kMat, K, NCH, +1>(nodes, tl, X);   // its first barrier also shares the tag
    // state entering the tile (P_0 = I before the first), then entering the chunk
    float P[K], eye[K];
    Rw::eye(tl.v, eye);
#pragma unroll
    for (int s = 0; s < K; ++s) P[s] = eye[s];
    if constexpr (MULTI) {
        const uint32_t tag = sTicket[0];
        if (tl.wv == 0 && tl.sub == 0 && tl.j < a.nT - 1) publish_wm<K>(a.agg, ftile, tl.slot, tag, X, a.lb_local);
        const float *root = nodes[tree_node<NCH, +1>(tree_levels<NCH>(), 0)][tl.slot];
        if (tl.j > 0)
            block_lookback<kMat, K, W, +1>(a, tl, ftile, sTicket, root, eye, tl.j < a.nT - 1, P, &nodes[0][0][0],
                                           [] {});
        else
            publish_first<kMat, K>(a, tl, ftile, tag, root, eye);
    }
    tree_apply<kMat, K, NCH, +1>(nodes, tl, P);
    // the states entering the steps t = 0 mod 2^pcs of this chunk, for the
    // backward's recompute (slot order kept).  When both directions share one
    // shape, that is the chunk's first step alone.
    constexpr bool kSame = matrix_shape(K, true).W == matrix_shape(K, false).W &&
                           matrix_shape(K, true).max_c == matrix_shape(K, false).max_c;
    auto save = [&](int t) {
        if ((t & ((1 << a.pcs) - 1)) == 0)
            store_vec<K>(a.pstate + ((static_cast<size_t>(t >> a.pcs) * a.nCG + tl.cg) * 32 + tl.slot) * K, P);
    };
    save(tl.t0);
    if (a.out == nullptr && (kSame || (1 << a.pcs) >= C)) return;   // states only (requested by a backward)
#pragma unroll
    for (int i = 0; i < C; ++i) {
        float np[K];
        Rw::mm(Ar[i], P, np);
#pragma unroll
        for (int s = 0; s < K; ++s) P[s] = np[s];
        const int t = tl.t0 + i;
        if (a.out && tl.cv && t < a.T) Rw::store_row(a.out + tl.ablk0 + t * tl.astep, tl.v, P);
        if (!kSame && i + 1 < C) save(t + 1);
    }
}

// Backward: W_t = A_t^T G_t with G_t = dP_t + W_{t+1}; per chunk [s, e]
// W_s = Psi W_{e+1} + Wl.  dA_t = G_t P_{t-1}^T, with P_{t-1} recomputed from
// the state entering the chunk (stored by the forward) and the A_t in hand,
// while the look-back's loads are in flight.
template <int K, int C, int W, bool MULTI>
__global__ void __launch_bounds__(64 * W) bmatrix_bwd_kernel(BlkArgs a)
{
    constexpr int NCH = 2 * W;
    using S = AggShape<kMatMat, K>;
    using Rw = Rows<K>;
    __shared__ float sKS[2][NCH][32][S::stride];
    __shared__ uint32_t sTicket[3];

    const int tile = blockIdx.x;
    const Tile tl = make_tile<K, C, W>(a, tile, true);
    const int ftile = tl.j * a.nCG + tl.cg;

    float ATr[C][K], Gr[C][K];   // rows of A_t^T, dP_t
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int t = clampT(tl.t0 + i, a.T);
        Rw::load_col(a.A + tl.ablk0 + t * tl.astep, tl.v, ATr[i]);
        Rw::load_row(a.y + tl.ablk0 + t * tl.astep, tl.v, Gr[i]);
    }
    // row v of P_{s-1}^T (column v of the state entering the chunk), saved by
    // the forward in its slot order: row m of P sits in lane m's slots, column
    // c of it at slot col(m, c)
    float PT[C][K];
    {
        const float *ps = a.pstate + ((static_cast<size_t>(tl.t0 >> a.pcs) * a.nCG + tl.cg) * 32 + (tl.slot & ~(K - 1))) * K;
#pragma unroll
        for (int s = 0; s < K; ++s) {
            const int m = Rw::col(tl.v, s);
            PT[0][s] = ps[m * K + Rw::col(m, tl.v)];
        }
    }
    Launch ep{0, 0};   // the launch ticket after the inputs (see the block-affine forward)
    if constexpr (MULTI) ep = epoch_begin(a.hd);
#pragma unroll
    for (int i = 0; i < C; ++i) {
        if (!(tl.cv && tl.t0 + i < a.T)) {
            Rw::eye(tl.v, ATr[i]);
#pragma unroll
            for (int s = 0; s < K; ++s) Gr[i][s] = 0.0f;
        }
    }

    // chunk aggregate from a zero carry: X = (Psi, Wl)
    float X[S::words];
#pragma unroll
    for (int s = 0; s < K; ++s) X[s] = ATr[C - 1][s];
    Rw::mm(ATr[C - 1], Gr[C - 1], X + K);
#pragma unroll
    for (int i = C - 2; i >= 0; --i) {
        float np[K], gw[K], nw[K];
        Rw::mm(ATr[i], X, np);
#pragma unroll
        for (int s = 0; s < K; ++s) gw[s] = Gr[i][s] + X[K + s];
        Rw::mm(ATr[i], gw, nw);
#pragma unroll
        for (int s = 0; s < K; ++s) { X[s] = np[s]; X[K + s] = nw[s]; }
    }
    float (*nodes)[32][S::stride] = reinterpret_cast<float (*)[32][S::stride]>(&sKS[0][0][0][0]);
    if (MULTI && threadIdx.x == 0) epoch_end(a.hd, ep, a.nTiles, sTicket);
    tree_build<kMatMat, K, NCH, -1>(nodes, tl, X);
    // P_{t-1}^T = P_{t-2}^T A_{t-1}^T for the chunk's later steps
    auto recompute = [&] {
#pragma unroll
        for (int i = 1; i < C; ++i) Rw::mm(PT[i - 1], ATr[i - 1], PT[i]);
    };
    float Wc[K], zero[K];
#pragma unroll
    for (int s = 0; s < K; ++s) zero[s] = Wc[s] = 0.0f;
    if (MULTI && tl.j < a.nT - 1) {
        const uint32_t tag = sTicket[0];
        if (tl.wv == 0 && tl.sub == 0 && tl.j > 0) publish_wm<S::words>(a.agg, ftile, tl.slot, tag, X, a.lb_local);
        block_lookback<kMatMat, K, W, -1>(a, tl, ftile, sTicket, nodes[tree_node<NCH, -1>(tree_levels<NCH>(), 0)][tl.slot],
                                          zero, tl.j > 0, Wc, &nodes[0][0][0], recompute);
    } else {
        if (MULTI) {   // the last tile along T (nT > 1): nothing after it
            const uint32_t tag = sTicket[0];
            if (tl.wv == 0 && tl.sub == 0) publish_wm<S::words>(a.agg, ftile, tl.slot, tag, X, a.lb_local);
            publish_first<kMatMat, K>(a, tl, ftile, tag, X, zero);
        }
        recompute();
    }
    // With 8 x 8 rows and eight steps per lane, or 16 x 16 rows and four, the
    // dP rows are read again here (from L2 or the Infinity Cache) rather than
    // held across the tree and the look-back: k = 16 fits 256 registers (308
    // otherwise), k = 8 no longer spills (7 registers otherwise; backward 37.4
    // -> 35.6 us at the long-T shape).  The reads overlap tree_apply.
    constexpr bool kReload = (K == 16 && C >= 4) || (K == 8 && C >= 8);
    float Gd[kReload ? C : 1][K];
    if constexpr (kReload) {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            Rw::load_row(a.y + tl.ablk0 + clampT(tl.t0 + i, a.T) * tl.astep, tl.v, Gd[i]);
            if (!(tl.cv && tl.t0 + i < a.T))
#pragma unroll
                for (int s = 0; s < K; ++s) Gd[i][s] = 0.0f;
        }
    }
    tree_apply<kMatMat, K, NCH, -1>(nodes, tl, Wc);   // carry entering the chunk from its end

#pragma unroll
    for (int i = C - 1; i >= 0; --i) {
        const int t = tl.t0 + i;
        const bool valid = tl.cv && t < a.T;
        float G[K], dAr[K], nw[K];
#pragma unroll
        for (int s = 0; s < K; ++s) G[s] = (kReload ? Gd[i][s] : Gr[i][s]) + Wc[s];
        Rw::mm(G, PT[i], dAr);           // dA_t = G_t P_{t-1}^T
        Rw::mm(ATr[i], G, nw);
#pragma unroll
        for (int s = 0; s < K; ++s) Wc[s] = nw[s];
        if (valid) Rw::store_row(a.out + tl.ablk0 + t * tl.astep, tl.v, dAr);
    }
}

// ------------------------------------------------------------ launchers

// NAME<K, W, MAXC>(g, a, s) launches KERNEL<K, C, W, MULTI> for the
// geometry's chunk length C (<= MAXC), multi-tile or single-tile.
#define MGS_DEFINE_BLOCK_LAUNCHER(NAME, KERNEL)                                                   \
    template <int K, int W, int C>                                                                \
    void NAME##_c(const BlockGeom &g, const BlkArgs &a, hipStream_t s)                            \
    {                                                                                             \
        if (g.nT > 1)                                                                             \
            hipLaunchKernelGGL((KERNEL<K, C, W, true>), dim3(g.nTiles), dim3(64 * W), 0, s, a);   \
        else                                                                                      \
            hipLaunchKernelGGL((KERNEL<K, C, W, false>), dim3(g.nTiles), dim3(64 * W), 0, s, a);  \
    }                                                                                             \
    template <int K, int W, int MAXC>                                                             \
    void NAME(const BlockGeom &g, const BlkArgs &a, hipStream_t s)                                \
    {                                                                                             \
        switch (g.C) {                                                                            \
        case 1: NAME##_c<K, W, 1>(g, a, s); break;                                                \
        case 2: if constexpr (MAXC >= 2) NAME##_c<K, W, 2>(g, a, s); break;                       \
        case 4: if constexpr (MAXC >= 4) NAME##_c<K, W, 4>(g, a, s); break;                       \
        case 8: if constexpr (MAXC >= 8) NAME##_c<K, W, 8>(g, a, s); break;                       \
        default: if constexpr (MAXC >= 16) NAME##_c<K, W, 16>(g, a, s); break;                    \
        }                                                                                         \
    }

MGS_DEFINE_BLOCK_LAUNCHER(launch_baffine_fwd, baffine_fwd_kernel)
MGS_DEFINE_BLOCK_LAUNCHER(launch_baffine_bwd, baffine_bwd_kernel)
MGS_DEFINE_BLOCK_LAUNCHER(launch_bmatrix_fwd, bmatrix_fwd_kernel)
MGS_DEFINE_BLOCK_LAUNCHER(launch_bmatrix_bwd, bmatrix_bwd_kernel)

template <int K>
void launch_blk_impl(BlkOp op, const BlockGeom &g, const BlkArgs &a, hipStream_t s)
{
    constexpr BlkShape af = affine_shape(K);
    constexpr BlkShape mf = matrix_shape(K, true), mb = matrix_shape(K, false);
    switch (op) {
    case BlkOp::AffineFwd: launch_baffine_fwd<K, af.W, af.max_c>(g, a, s); break;
    case BlkOp::AffineBwd: launch_baffine_bwd<K, af.W, af.max_c>(g, a, s); break;
    case BlkOp::MatrixFwd: launch_bmatrix_fwd<K, mf.W, mf.max_c>(g, a, s); break;
    case BlkOp::MatrixBwd: launch_bmatrix_bwd<K, mb.W, mb.max_c>(g, a, s); break;
    }
}

}  // namespace
}  // namespace mgs
