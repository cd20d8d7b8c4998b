// delta_scan.hip -- forward of the delta rule (DeltaMinGRU on the minGRU home
// page: DeltaNet's recurrence, run in its chunked WY form), d = 64, for gfx950.
//
//     S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T,     o_t = S_t q_t,
// with a state S (dv x dk = 64 x 64) per sequence.  Within a chunk of C = 64
// steps entered with state S, write u_i = beta_i (v_i - S_{i-1} k_i) (the
// value actually added along k_i).  Then S_t = S + sum_{i<=t} u_i k_i^T and
//     u_i = beta_i (v_i - S k_i - sum_{j<i} (k_i . k_j) u_j),
// a unit lower-triangular system in the chunk's rows:
//     (I + strict_lower(diag(beta) K K^T)) U' = diag(beta) (V - K S^T).
// Its solution splits into a state-free part and a correction:
//     U' = U - W S^T,   with   (I + L) [U W] = diag(beta) [V K]
// (the WY representation), so
//     O = Q S^T + causal(Q K^T) U',     S <- S + U'^T K.
//
// Across chunks the state follows an affine map per chunk:
//     S <- S + U'^T K = S (I - W^T K) + U^T K = S A + Bc.
//
// Three kernels (one when every sequence is a single chunk entered from S = 0):
//   * delta_prep_kernel, one workgroup per (sequence, chunk), all chunks at
//     once: A = strict_lower(diag(beta) K K^T) and M = causal(Q K^T) on MFMA
//     (fp32 16x16x4), the four 16 x 16 diagonal blocks of I + A inverted by
//     substitution, the block solve for [W U] kept in MFMA accumulator
//     registers, then Qt = Q - M W, P = M U, A^T and Bc^T.
//   * delta_state_kernel, one workgroup per (sequence, 16 rows of S; the four
//     of a sequence on one XCD), chunks in order: S <- S A + Bc, one
//     16 x 64 x 64 MFMA product per chunk and one barrier; stores the state
//     entering each chunk.  Rows of S never mix, so the 4 slices run in
//     parallel.
//   * delta_out_kernel, one workgroup per (sequence, chunk), all at once:
//     O = Qt S^T + P from the state entering the chunk.

// MFMA operand layout (v_mfma_f32_16x16x4f32, measured): lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; accumulator register r of lane l is
// D[4 (l / 16) + r][l % 16].  The reduction index is permuted so that lane l
// of MFMA (kb, j) holds reduction index 16 kb + 4 (l / 16) + j: one 16-byte
// load then feeds four MFMAs.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "launch.hpp"

namespace mgs {
namespace {

// chunks of operands the state pass keeps in flight ahead of the one it computes
#ifndef MGS_DELTA_PD
#define MGS_DELTA_PD 3
#endif

// waves per workgroup of the multi-chunk prep kernel
#ifndef MGS_DELTA_PREP_W
#define MGS_DELTA_PREP_W 8
#endif
constexpr int kPrepW = MGS_DELTA_PREP_W;

constexpr int kDD = 64;   // dk = dv
constexpr int kCh = 64;   // steps per chunk
constexpr int kLd = 68;   // LDS row stride (floats) of 64-wide tiles (16-byte aligned rows)
// 64 x 64 tiles per (sequence, chunk) in the workspace: Qt, P^T, A^T, Bc^T and
// the state entering the chunk
constexpr int kWsTiles = 5;

typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4v mfma4(float4 a, float4 b, f4v c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
    return c;
}

struct DeltaArgs {
    const float *q, *k, *v, *beta, *S0;
    float *o, *ST;
    float *wum;   // per (sequence, chunk): Qt, P^T, A^T, Bc^T, entering state, each 64 x 64
    int T, nC;
    int B;
};

__device__ __forceinline__ float4 f4zero() { return make_float4(0.0f, 0.0f, 0.0f, 0.0f); }

// Workgroup barrier that waits only for this wave's LDS operations.  Global
// loads issued before it stay in flight (__syncthreads() also waits for them,
// which would stall the prefetch of the next chunk's operands at every
// barrier).  Only LDS carries data between the waves here.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ------------------------------------------------------------- prep kernel
// Per chunk, with R = diag(beta) [K V] (64 x 128) and L = I + A,
// A = strict_lower(diag(beta) K K^T), in 16-row blocks i, j:
//     [W U]_i = X_ii (R_i - sum_{j<i} A_ij [W U]_j),   X_ii = L_ii^{-1},
// then the state-free parts of the outputs, M = causal(Q K^T):
//     Qt = Q - M W,   P = M U,
// so that the state kernel's output is O = Qt S^T + P.  Each wave owns 16-wide
// column tiles of [W U] (two with 4 waves, one with 8) through all four row
// blocks, so the block solve and the products with M keep every block in
// registers: an MFMA result (accumulator layout, rows 4 (l/16) + r) is
// directly the B operand of the next MFMA under the permuted reduction index.

// The ten 16 x 16 tiles on or below the diagonal, tile = 4 i + j, one per
// nibble (slot s in bits 4s .. 4s+3): slots 0-9 are tiles of G, 10-19 the same
// tiles of M, dealt to the waves (five apiece with 4 waves, two or three with
// 8) and decoded with scalar shifts of a wave-uniform slot.
constexpr uint64_t kPrepTiles = 0xFEDCA98540ull;

// DIRECT: a sequence of one chunk entered with S = 0 (no S0): the state pass
// reduces to O = M U and S_T = U^T K, written here; only U is solved, one
// 16-column tile per wave, and nothing goes through the workspace.
// PW: waves per workgroup, 4 or 8 (DIRECT: 4).  With 8, each wave owns one
// 16-column tile of [W U] and two waves share each SIMD, so one wave's MFMA
// chains and LDS reads overlap the other's.
template <bool DIRECT, int PW>
__global__ void __launch_bounds__(64 * PW) delta_prep_kernel(DeltaArgs a)
{
    static_assert(PW == 4 || (PW == 8 && !DIRECT), "prep workgroups of 4 waves, or 8 without DIRECT");
    __shared__ float sK[kCh][kLd], sV[kCh][kLd], sQ[kCh][kLd], sA[kCh][kLd], sM[kCh][kLd];
    __shared__ float sX[4][16][20];   // the inverses of the diagonal blocks of L
    __shared__ __align__(16) float sB[kCh];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int bc = blockIdx.x;   // sequence * nC + chunk
    const int b = bc / a.nC, ch = bc - b * a.nC;
    const int t0 = ch * kCh;
    const int nrow = min(kCh, a.T - t0);
    const int64_t row0 = static_cast<int64_t>(b) * a.T + t0;

    // the chunk's rows of k, v, q (zero past the end of the sequence).  Loads
    // are unconditional from a clamped row, so all twelve are in flight at
    // once; rows past the end are zeroed after the load.
    constexpr int NIT = 16 / PW;   // rows of 16 float4 per thread and array
    {
        float4 kk[NIT], vv[NIT], qq[NIT];
        const int c4 = (tid & 15) * 4;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int r = (tid >> 4) + 4 * PW * it;
            const int64_t off = (row0 + min(r, nrow - 1)) * kDD + c4;
            kk[it] = *reinterpret_cast<const float4 *>(a.k + off);
            vv[it] = *reinterpret_cast<const float4 *>(a.v + off);
            qq[it] = *reinterpret_cast<const float4 *>(a.q + off);
        }
        const float bt = a.beta[row0 + min(tid & 63, nrow - 1)];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int r = (tid >> 4) + 4 * PW * it;
            const bool in = r < nrow;
            *reinterpret_cast<float4 *>(&sK[r][c4]) = in ? kk[it] : f4zero();
            *reinterpret_cast<float4 *>(&sV[r][c4]) = in ? vv[it] : f4zero();
            *reinterpret_cast<float4 *>(&sQ[r][c4]) = in ? qq[it] : f4zero();
        }
        if (tid < kCh) sB[tid] = tid < nrow ? bt : 0.0f;
    }
    __syncthreads();

    // A = strict_lower(diag(beta) K K^T) and M = causal(Q K^T), lower tiles
    // only, NT tiles per wave: each step of the reduction issues one MFMA of
    // every tile in turn, so consecutive MFMAs do not depend on each other.
    // With 8 waves the 20 tiles fill 24 slots; slots 20-23 repeat tiles 0-3,
    // whose two writers store the same values.
    constexpr int NT = (20 + PW - 1) / PW;
    {
        f4v acc[NT];
        const int wvu = __builtin_amdgcn_readfirstlane(wv);
        int rowL[NT], rowK[NT];
        bool isM[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int slot = (wvu + PW * n) % 20;
            const int tile = static_cast<int>((kPrepTiles >> (4 * (slot % 10))) & 15);
            rowL[n] = 16 * (tile >> 2) + li;
            rowK[n] = 16 * (tile & 3) + li;
            isM[n] = slot >= 10;   // wave-uniform
            acc[n] = f4v{0.0f, 0.0f, 0.0f, 0.0f};
        }
        // beta of the tiles' rows, read up front
        float4 bq[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) bq[n] = *reinterpret_cast<const float4 *>(&sB[rowL[n] - li + 4 * lq]);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            float4 x[NT], y[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const float(*L)[kLd] = isM[n] ? sQ : sK;
                x[n] = *reinterpret_cast<const float4 *>(&L[rowL[n]][16 * kb + 4 * lq]);
                y[n] = *reinterpret_cast<const float4 *>(&sK[rowK[n]][16 * kb + 4 * lq]);
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[n].x, y[n].x, acc[n], 0, 0, 0);
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[n].y, y[n].y, acc[n], 0, 0, 0);
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[n].z, y[n].z, acc[n], 0, 0, 0);
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[n].w, y[n].w, acc[n], 0, 0, 0);
        }
        // lower parts of the tiles (rows scaled by beta for A), stored without
        // branches: the destination and the row scale are chosen per tile (the
        // row scales are pinned in registers first, so that their reads are not
        // sunk into the stores as conditional reads with a wait apiece)
#pragma unroll
        for (int n = 0; n < NT; ++n) asm volatile("" : "+v"(bq[n].x), "+v"(bq[n].y), "+v"(bq[n].z), "+v"(bq[n].w));
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int i0 = rowL[n] - li + 4 * lq, j = rowK[n];
            const float sc[4] = {isM[n] ? 1.0f : bq[n].x, isM[n] ? 1.0f : bq[n].y, isM[n] ? 1.0f : bq[n].z,
                                 isM[n] ? 1.0f : bq[n].w};
            float(*dst)[kLd] = isM[n] ? sM : sA;
            const int diag = isM[n] ? 1 : 0;   // M keeps its diagonal, A does not
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[i0 + r][j] = (j < i0 + r + diag) ? sc[r] * acc[n][r] : 0.0f;
        }
    }
    __syncthreads();

    // X_ww = (I + A_ww)^{-1}: lane c < 16 solves column c, row by row, from
    // the block's rows read up front (16-byte reads, the same address in every
    // lane)
    if (lane < 16 && wv < 4) {
        const int o = 16 * wv;
        float4 rw[16][4];
#pragma unroll
        for (int i = 1; i < 16; ++i)
#pragma unroll
            for (int q = 0; 4 * q < i; ++q) rw[i][q] = *reinterpret_cast<const float4 *>(&sA[o + i][o + 4 * q]);
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s0 = (i == li) ? 1.0f : 0.0f, s1 = 0.0f;
#pragma unroll
            for (int j = 0; j < i; ++j) {
                const float4 r4 = rw[i][j >> 2];
                const float aij = (j & 3) == 0 ? r4.x : (j & 3) == 1 ? r4.y : (j & 3) == 2 ? r4.z : r4.w;
                if (j & 1) s1 = __builtin_fmaf(-aij, x[j], s1);
                else s0 = __builtin_fmaf(-aij, x[j], s0);
            }
            x[i] = s0 + s1;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sX[wv][i][li] = x[i];
    }
    __syncthreads();

    // block solve of this wave's column tiles of [W U] (two with 4 waves; one
    // with 8; DIRECT: one tile of U)
    constexpr int NH = (DIRECT || PW == 8) ? 1 : 2;
    const bool isU = DIRECT || wv >= PW / 2;       // wave-uniform: columns of V give U
    const int cbase = DIRECT ? 16 * wv : (PW == 8 ? 16 * (wv & 3) : 32 * (wv & 1));   // first column within K or V
    float(*R)[kLd] = isU ? sV : sK;
    f4v Y[4][NH];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            f4v t;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i + 4 * lq + r;
                t[r] = sB[row] * R[row][cbase + 16 * h + li];
            }
#pragma unroll
            for (int j = 0; j < i; ++j) {
                const float4 av = *reinterpret_cast<const float4 *>(&sA[16 * i + li][16 * j + 4 * lq]);
                const float4 na = make_float4(-av.x, -av.y, -av.z, -av.w);
                t = __builtin_amdgcn_mfma_f32_16x16x4f32(na.x, Y[j][h][0], t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_16x16x4f32(na.y, Y[j][h][1], t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_16x16x4f32(na.z, Y[j][h][2], t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_16x16x4f32(na.w, Y[j][h][3], t, 0, 0, 0);
            }
            const float4 xv = *reinterpret_cast<const float4 *>(&sX[i][li][4 * lq]);
            f4v y = {0.0f, 0.0f, 0.0f, 0.0f};
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(xv.x, t[0], y, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(xv.y, t[1], y, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(xv.z, t[2], y, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(xv.w, t[3], y, 0, 0, 0);
            Y[i][h] = y;
        }
    }

    if constexpr (DIRECT) {
        // O = M U (rows past the end not stored), S_T = U^T K if requested;
        // the row blocks' (column blocks') products advance together, one MFMA
        // of each in turn
        const int64_t orow0 = static_cast<int64_t>(b) * a.T;
        f4v z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = f4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
            float4 m[4];
#pragma unroll
            for (int i = k2; i < 4; ++i) m[i] = *reinterpret_cast<const float4 *>(&sM[16 * i + li][16 * k2 + 4 * lq]);
#pragma unroll
            for (int i = k2; i < 4; ++i) z[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(m[i].x, Y[k2][0][0], z[i], 0, 0, 0);
#pragma unroll
            for (int i = k2; i < 4; ++i) z[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(m[i].y, Y[k2][0][1], z[i], 0, 0, 0);
#pragma unroll
            for (int i = k2; i < 4; ++i) z[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(m[i].z, Y[k2][0][2], z[i], 0, 0, 0);
#pragma unroll
            for (int i = k2; i < 4; ++i) z[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(m[i].w, Y[k2][0][3], z[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * i + 4 * lq + r;
                if (t < nrow) store_out(&a.o[(orow0 + t) * kDD + cbase + li], z[i][r]);
            }
        }
        if (a.ST) {
            // A: U^T (lane: U[16 kb + 4 lq + j][cbase + li] = Y[kb] register j), B: K[t][16 cb + li]
            f4v st[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) st[cb] = f4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int t = 16 * kb + 4 * lq;
                float kk[4][4];
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) kk[cb][j] = sK[t + j][16 * cb + li];
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb)
                        st[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(Y[kb][0][j], kk[cb][j], st[cb], 0, 0, 0);
            }
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    store_out(&a.ST[(static_cast<int64_t>(b) * kDD + cbase + 4 * lq + r) * kDD + 16 * cb + li], st[cb][r]);
        }
        return;
    }

    // outputs, per chunk (row-major 64 x 64 each): Qt = Q - M W and P^T = (M U)^T
    // for the output kernel; the chunk's affine map of the state,
    //     S -> S A + Bc,   A = I - W^T K,   Bc = U^T K,
    // as A^T = I - K^T W and Bc^T = K^T U for the state pass
    float *wum = a.wum + static_cast<int64_t>(bc) * kWsTiles * kCh * kDD;
    float *gQ = wum, *gPT = wum + kCh * kDD, *gAT = wum + 2 * kCh * kDD, *gBT = wum + 3 * kCh * kDD;
    // the eight (row block, column tile) products advance together, one MFMA
    // of each in turn
    {
        f4v z[4][NH];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) z[i][h][r] = isU ? 0.0f : sQ[16 * i + 4 * lq + r][cbase + 16 * h + li];
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
            float4 m[4];
#pragma unroll
            for (int i = k2; i < 4; ++i) {
                const float4 mv = *reinterpret_cast<const float4 *>(&sM[16 * i + li][16 * k2 + 4 * lq]);
                m[i] = isU ? mv : make_float4(-mv.x, -mv.y, -mv.z, -mv.w);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = k2; i < 4; ++i)
#pragma unroll
                    for (int h = 0; h < NH; ++h) {
                        const float mj = j == 0 ? m[i].x : j == 1 ? m[i].y : j == 2 ? m[i].z : m[i].w;
                        z[i][h] = __builtin_amdgcn_mfma_f32_16x16x4f32(mj, Y[k2][h][j], z[i][h], 0, 0, 0);
                    }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const int col = cbase + 16 * h + li;
                const int row = 16 * i + 4 * lq;
                if (isU) {
                    *reinterpret_cast<float4 *>(gPT + col * kCh + row) =
                        make_float4(z[i][h][0], z[i][h][1], z[i][h][2], z[i][h][3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) gQ[(row + r) * kDD + col] = z[i][h][r];
                }
            }
    }
    // A^T = I - K^T W (W waves) or Bc^T = K^T U (U waves): tile rows 16 cb of
    // the key index, columns this wave's W or U columns; A operand K^T[16 cb +
    // li][t] = K[t][16 cb + li], B operand the solved block registers
    {
        f4v z[4][NH];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    z[cb][h][r] = (!isU && 16 * cb + 4 * lq + r == cbase + 16 * h + li) ? 1.0f : 0.0f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int t = 16 * kb + 4 * lq;
            float kt[4][4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x = sK[t + j][16 * cb + li];
                    kt[cb][j] = isU ? x : -x;
                }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                    for (int h = 0; h < NH; ++h)
                        z[cb][h] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt[cb][j], Y[kb][h][j], z[cb][h], 0, 0, 0);
        }
        float *g = isU ? gBT : gAT;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) g[(16 * cb + 4 * lq + r) * kDD + cbase + 16 * h + li] = z[cb][h][r];
    }
}

// ------------------------------------------------------------ state kernel
// The chunks' affine maps in order: S <- S A + Bc.  Each workgroup owns 16
// rows of S (rows of S never mix), wave w the columns 16w .. 16w+15 of them,
// kept in accumulator registers; before each chunk the state entering it is
// stored for the output kernel.  One barrier per chunk: the slice of S is
// exchanged through two LDS buffers in turn.  The next chunk's operands are
// loaded while this chunk computes.

struct StateOps {
    float4 at[4];   // A^T[16 wv + li][16 kb + 4 lq .. +3] = A[16 kb + 4 lq + j][16 wv + li]
    float4 bt;      // Bc^T[16 wv + li][16 sl + 4 lq .. +3] = Bc[16 sl + 4 lq + r][16 wv + li]
};

__device__ __forceinline__ void load_state_ops(const DeltaArgs &a, int b, int sl, int wv, int li, int lq, int ch,
                                               StateOps &op)
{
    // a workgroup-uniform chunk base plus an unsigned 32-bit lane offset: no
    // per-lane 64-bit address is formed per chunk (such temporaries can land in
    // registers of loads still in flight, which the compiler then waits for)
    const float *wum = a.wum + (static_cast<int64_t>(b) * a.nC + ch) * kWsTiles * kCh * kDD;
    const float *gAT = wum + 2 * kCh * kDD, *gBT = wum + 3 * kCh * kDD;
    const uint32_t ra = 16 * wv + li;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        op.at[kb] = *reinterpret_cast<const float4 *>(gAT + (ra * kDD + 16u * kb + 4u * lq));
    op.bt = *reinterpret_cast<const float4 *>(gBT + (ra * kDD + 16u * sl + 4u * lq));
}

// NC > 0: a sequence of exactly NC chunks, unrolled, with the operands of the
// PD chunks after the one computing in flight (a rotated loop makes the
// compiler wait, at its top, for loads issued one chunk earlier); NC = 0: any
// count, in a loop with one chunk of operands ahead.
template <int NC>
__global__ void __launch_bounds__(256) delta_state_kernel(DeltaArgs a)
{
    __shared__ float sS[2][16][kLd];   // rows 16 sl .. 16 sl + 15 of the state, two buffers in turn
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    // XCD-aware numbering: workgroups are dealt to the 8 XCDs round-robin
    // (XCD = blockIdx mod 8), so the four slices of sequence b get blockIdx
    // 32 (b / 8) + 8 sl + b % 8 and share one XCD's L2 for the rows of A^T they
    // all read.  The grid is padded to a multiple of 32.
    const int xcd = blockIdx.x & 7, rest = blockIdx.x >> 3;
    const int sl = rest & 3, b = (rest >> 2) * 8 + xcd;
    if (b >= a.B) return;   // padding workgroup (whole workgroup, before any barrier)

    // this wave's tile of the state: S[16 sl + 4 lq + r][16 wv + li]
    const int64_t sbase = (static_cast<int64_t>(b) * kDD + 16 * sl + 4 * lq) * kDD + 16 * wv + li;
    f4v S;
#pragma unroll
    for (int r = 0; r < 4; ++r) S[r] = a.S0 ? a.S0[sbase + r * kDD] : 0.0f;

    // one chunk: store the entering state, then S <- S A + Bc
    auto chunk = [&](int ch, const StateOps &cur) {
        float *sj = a.wum + ((static_cast<int64_t>(b) * a.nC + ch) * kWsTiles + 4) * kCh * kDD;
        float(*buf)[kLd] = sS[ch & 1];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            buf[4 * lq + r][16 * wv + li] = S[r];
            sj[(16 * sl + 4 * lq + r) * kDD + 16 * wv + li] = S[r];
        }
        lds_barrier();
        f4v n1 = {cur.bt.x, cur.bt.y, cur.bt.z, cur.bt.w}, n2 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const float4 s4 = *reinterpret_cast<const float4 *>(&buf[li][16 * kb + 4 * lq]);
            if (kb < 2) n1 = mfma4(s4, cur.at[kb], n1);
            else n2 = mfma4(s4, cur.at[kb], n2);
        }
        S = n1 + n2;
    };

    // two operand sets in turn: the next chunk's loads are issued before this
    // chunk computes and are never copied (a copy would wait for them); the
    // loads are unconditional (past the last chunk they reload it), since a
    // conditional load makes the compiler wait for it at the first use of
    // the other set
    const int last = a.nC - 1;
    if constexpr (NC > 0) {
        constexpr int PD = MGS_DELTA_PD < NC ? MGS_DELTA_PD : NC;
        StateOps ops[NC];
#pragma unroll
        for (int c = 0; c < PD; ++c) load_state_ops(a, b, sl, wv, li, lq, c, ops[c]);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (c + PD < NC) load_state_ops(a, b, sl, wv, li, lq, c + PD, ops[c + PD]);
            chunk(c, ops[c]);
        }
    } else if (a.nC == 1) {
        StateOps A;
        load_state_ops(a, b, sl, wv, li, lq, 0, A);
        chunk(0, A);
    } else if (a.nC > 1) {
        StateOps A, B;
        load_state_ops(a, b, sl, wv, li, lq, 0, A);
        for (int ch = 0; ch < a.nC; ch += 2) {
            load_state_ops(a, b, sl, wv, li, lq, min(ch + 1, last), B);
            chunk(ch, A);
            if (ch + 1 > last) break;
            load_state_ops(a, b, sl, wv, li, lq, min(ch + 2, last), A);
            chunk(ch + 1, B);
        }
    }
    if (a.ST) {
#pragma unroll
        for (int r = 0; r < 4; ++r) store_out(&a.ST[sbase + r * kDD], S[r]);
    }
}

// ----------------------------------------------------------- output kernel
// O = Qt S^T + P per chunk, all chunks at once, from the state entering each
// chunk: one workgroup per (sequence, chunk), wave w the chunk rows 16w ..
// 16w+15 (A operand: rows of Qt; B operand: S[16 cb + li][c], rows of S).
__global__ void __launch_bounds__(256) delta_out_kernel(DeltaArgs a)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int bc = blockIdx.x;   // sequence * nC + chunk
    const int b = bc / a.nC, ch = bc - b * a.nC;
    const int t0 = ch * kCh;
    const int nrow = min(kCh, a.T - t0);
    const int64_t row0 = static_cast<int64_t>(b) * a.T + t0;
    const float *wum = a.wum + static_cast<int64_t>(bc) * kWsTiles * kCh * kDD;
    const float *gQ = wum, *gPT = wum + kCh * kDD, *gS = wum + 4 * kCh * kDD;
    float4 q4[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) q4[kb] = *reinterpret_cast<const float4 *>(gQ + (16 * wv + li) * kDD + 16 * kb + 4 * lq);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const float4 p = *reinterpret_cast<const float4 *>(gPT + (16 * cb + li) * kCh + 16 * wv + 4 * lq);
        f4v o1 = {p.x, p.y, p.z, p.w}, o2 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const float4 s4 = *reinterpret_cast<const float4 *>(gS + (16 * cb + li) * kDD + 16 * kb + 4 * lq);
            if (kb < 2) o1 = mfma4(q4[kb], s4, o1);
            else o2 = mfma4(q4[kb], s4, o2);
        }
        const f4v o = o1 + o2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * wv + 4 * lq + r;
            if (t < nrow) store_out(&a.o[(row0 + t) * kDD + 16 * cb + li], o[r]);
        }
    }
}

}  // namespace

DeltaGeom delta_geometry(int64_t B, int64_t T, int64_t d)
{
    DeltaGeom g{};
    g.B = B;
    g.T = static_cast<int>(T);
    g.d = static_cast<int>(d);
    g.nC = static_cast<int>((T + kCh - 1) / kCh);
    g.off_wum = 256;   // after a header kept for the common workspace check
    g.bytes = g.off_wum + static_cast<size_t>(B) * g.nC * kWsTiles * kCh * kDD * sizeof(float);
    return g;
}

hipError_t launch_delta_fwd(const DeltaGeom &g, const float *q, const float *k, const float *v,
                            const float *beta, const float *S0, float *o, float *ST, void *ws, hipStream_t s)
{
    DeltaArgs a{};
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.S0 = S0; a.o = o; a.ST = ST;
    a.wum = reinterpret_cast<float *>(static_cast<char *>(ws) + g.off_wum);
    a.T = g.T;
    a.nC = g.nC;
    if (g.nC == 1 && S0 == nullptr) {   // one chunk from a zero state: no state pass
        hipLaunchKernelGGL((delta_prep_kernel<true, 4>), dim3(static_cast<unsigned>(g.B)), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    if (g.nC > 0) {
        hipLaunchKernelGGL((delta_prep_kernel<false, kPrepW>), dim3(static_cast<unsigned>(g.B * g.nC)), dim3(64 * kPrepW), 0,
                           s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    a.B = static_cast<int>(g.B);
    const unsigned groups = static_cast<unsigned>((g.B + 7) / 8) * 32;   // 4 slices x padded sequences
    switch (g.nC) {
#define MGS_STATE_NC(n) case n: hipLaunchKernelGGL(delta_state_kernel<n>, dim3(groups), dim3(256), 0, s, a); break;
    MGS_STATE_NC(1) MGS_STATE_NC(2) MGS_STATE_NC(3) MGS_STATE_NC(4) MGS_STATE_NC(5) MGS_STATE_NC(6)
    MGS_STATE_NC(7) MGS_STATE_NC(8) MGS_STATE_NC(9) MGS_STATE_NC(10) MGS_STATE_NC(11) MGS_STATE_NC(12)
    MGS_STATE_NC(13) MGS_STATE_NC(14) MGS_STATE_NC(15) MGS_STATE_NC(16)
#undef MGS_STATE_NC
    default: hipLaunchKernelGGL(delta_state_kernel<0>, dim3(groups), dim3(256), 0, s, a); break;
    }
    if (g.nC > 0) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(delta_out_kernel, dim3(static_cast<unsigned>(g.B * g.nC)), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace mgs
