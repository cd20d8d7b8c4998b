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
// Two kernels:
//   * delta_prep_kernel, one workgroup per (sequence, chunk), all chunks at
//     once: G = K K^T and M = causal(Q K^T) on MFMA (fp32 16x16x4), then the
//     forward substitution for the 128 columns of [W U] (one lane per column,
//     column-oriented so each step is a row of independent multiply-adds).
//     Writes W, U, M (3 x 64 x 64 floats per chunk) to the workspace.
//   * delta_state_kernel, one workgroup per (sequence, 16 rows of S), chunks in
//     order: U' = U - W S^T and O = Q S^T + M U' and S += U'^T K, all on MFMA;
//     the wave w of 4 owns chunk rows 16w..16w+15 for U' and O, and columns
//     16w..16w+15 of its 16 x 64 slice of S, kept in accumulator registers
//     across chunks.  Slices of S are independent (the recurrence mixes the
//     columns of S, never its rows), so the 4 slices run in parallel.
//
// MFMA operand layout (v_mfma_f32_16x16x4f32, measured): lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; accumulator register r of lane l is
// D[4 (l / 16) + r][l % 16].  The reduction index is permuted so that lane l
// of MFMA (kb, j) holds reduction index 16 kb + 4 (l / 16) + j: one 16-byte
// load then feeds four MFMAs.
#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace mgs {
namespace {

constexpr int kDD = 64;   // dk = dv
constexpr int kCh = 64;   // steps per chunk
constexpr int kLd = 68;   // LDS row stride (floats) of 64-wide tiles (16-byte aligned rows)

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
    float *wum;   // per (sequence, chunk): W, U, M, each 64 x 64 row-major
    int T, nC;
};

__device__ __forceinline__ float4 f4zero() { return make_float4(0.0f, 0.0f, 0.0f, 0.0f); }

// ------------------------------------------------------------- prep kernel

__global__ void __launch_bounds__(256) delta_prep_kernel(DeltaArgs a)
{
    __shared__ float sK[kCh][kLd], sV[kCh][kLd], sQ[kCh][kLd], sG[kCh][kLd];
    __shared__ float sB[kCh];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int bc = blockIdx.x;   // sequence * nC + chunk
    const int b = bc / a.nC, ch = bc - b * a.nC;
    const int t0 = ch * kCh;
    const int nrow = min(kCh, a.T - t0);
    const int64_t row0 = static_cast<int64_t>(b) * a.T + t0;

    // the chunk's rows of k, v, q (zero past the end of the sequence)
    for (int e = tid; e < kCh * 16; e += 256) {
        const int r = e >> 4, c4 = (e & 15) * 4;
        float4 kk = f4zero(), vv = f4zero(), qq = f4zero();
        if (r < nrow) {
            const int64_t off = (row0 + r) * kDD + c4;
            kk = *reinterpret_cast<const float4 *>(a.k + off);
            vv = *reinterpret_cast<const float4 *>(a.v + off);
            qq = *reinterpret_cast<const float4 *>(a.q + off);
        }
        *reinterpret_cast<float4 *>(&sK[r][c4]) = kk;
        *reinterpret_cast<float4 *>(&sV[r][c4]) = vv;
        *reinterpret_cast<float4 *>(&sQ[r][c4]) = qq;
    }
    if (tid < kCh) sB[tid] = tid < nrow ? a.beta[row0 + tid] : 0.0f;
    __syncthreads();

    float *wum = a.wum + static_cast<int64_t>(bc) * 3 * kCh * kDD;
    float *gW = wum, *gU = wum + kCh * kDD, *gM = wum + 2 * kCh * kDD;

    // G = K K^T (all 16 tiles: row i of G is then row i of the symmetric G,
    // read contiguously by the substitution) and M = causal(Q K^T) (tiles on
    // or below the diagonal).  Wave wv owns row block wv.
    {
        float4 ak[4], aq[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            ak[kb] = *reinterpret_cast<const float4 *>(&sK[16 * wv + li][16 * kb + 4 * lq]);
            aq[kb] = *reinterpret_cast<const float4 *>(&sQ[16 * wv + li][16 * kb + 4 * lq]);
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            f4v g = {0.0f, 0.0f, 0.0f, 0.0f}, m = {0.0f, 0.0f, 0.0f, 0.0f};
            const bool causal = cb <= wv;   // wave-uniform
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const float4 bk = *reinterpret_cast<const float4 *>(&sK[16 * cb + li][16 * kb + 4 * lq]);
                g = mfma4(ak[kb], bk, g);
                if (causal) m = mfma4(aq[kb], bk, m);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * wv + 4 * lq + r, j = 16 * cb + li;
                sG[i][j] = g[r];
                gM[i * kDD + j] = (causal && j <= i) ? m[r] : 0.0f;
            }
        }
    }
    __syncthreads();

    // forward substitution, lane per column: columns 0..63 of K give W,
    // columns 0..63 of V give U.  At step i the lane's running right-hand side
    // y_i is final: x_i = beta_i y_i, then y_r -= G[r][i] x_i for r > i.
    if (tid < 128) {
        const int c = tid & 63;
        float(*X)[kLd] = tid < 64 ? sK : sV;
        float *dst = tid < 64 ? gW : gU;
        float y[kCh];
#pragma unroll
        for (int i = 0; i < kCh; ++i) y[i] = X[i][c];
#pragma unroll
        for (int i = 0; i < kCh; ++i) {
            const float x = sB[i] * y[i];
            dst[i * kDD + c] = x;
#pragma unroll
            for (int r4 = (i + 1) & ~3; r4 < kCh; r4 += 4) {
                const float4 g = *reinterpret_cast<const float4 *>(&sG[i][r4]);
                if (r4 + 0 > i) y[r4 + 0] = __builtin_fmaf(-g.x, x, y[r4 + 0]);
                if (r4 + 1 > i) y[r4 + 1] = __builtin_fmaf(-g.y, x, y[r4 + 1]);
                if (r4 + 2 > i) y[r4 + 2] = __builtin_fmaf(-g.z, x, y[r4 + 2]);
                if (r4 + 3 > i) y[r4 + 3] = __builtin_fmaf(-g.w, x, y[r4 + 3]);
            }
        }
    }
}

// ------------------------------------------------------------ state kernel

__global__ void __launch_bounds__(256) delta_state_kernel(DeltaArgs a)
{
    __shared__ float sS[16][kLd];    // rows 16 sl .. 16 sl + 15 of the state entering the chunk
    __shared__ float sUp[kCh][17];   // U' of the chunk, this slice's 16 columns
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int b = blockIdx.x >> 2, sl = blockIdx.x & 3;

    // this wave's tile of the state: S[16 sl + 4 lq + r][16 wv + li]
    const int64_t sbase = (static_cast<int64_t>(b) * kDD + 16 * sl + 4 * lq) * kDD + 16 * wv + li;
    f4v S;
#pragma unroll
    for (int r = 0; r < 4; ++r) S[r] = a.S0 ? a.S0[sbase + r * kDD] : 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) sS[4 * lq + r][16 * wv + li] = S[r];

    for (int ch = 0; ch < a.nC; ++ch) {
        const int t0 = ch * kCh;
        const int nrow = min(kCh, a.T - t0);
        const int64_t row0 = static_cast<int64_t>(b) * a.T + t0;
        const float *wum = a.wum + (static_cast<int64_t>(b) * a.nC + ch) * 3 * kCh * kDD;
        const float *gW = wum, *gU = wum + kCh * kDD, *gM = wum + 2 * kCh * kDD;

        // operands: chunk rows 16 wv + li (A layout), reduction slices 16 kb + 4 lq
        const int ra = 16 * wv + li;
        float4 w4[4], q4[4], m4[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int c = 16 * kb + 4 * lq;
            w4[kb] = *reinterpret_cast<const float4 *>(gW + ra * kDD + c);
            m4[kb] = *reinterpret_cast<const float4 *>(gM + ra * kDD + c);
            q4[kb] = ra < nrow ? *reinterpret_cast<const float4 *>(a.q + (row0 + ra) * kDD + c) : f4zero();
        }
        f4v up;
#pragma unroll
        for (int r = 0; r < 4; ++r) up[r] = gU[(16 * wv + 4 * lq + r) * kDD + 16 * sl + li];
        float4 kc[4];   // K[16 kb + 4 lq + j][16 wv + li]
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int t = 16 * kb + 4 * lq;
            const float *kp = a.k + (row0 + t) * kDD + 16 * wv + li;
            kc[kb].x = t + 0 < nrow ? kp[0] : 0.0f;
            kc[kb].y = t + 1 < nrow ? kp[kDD] : 0.0f;
            kc[kb].z = t + 2 < nrow ? kp[2 * kDD] : 0.0f;
            kc[kb].w = t + 3 < nrow ? kp[3 * kDD] : 0.0f;
        }
        __syncthreads();   // sS holds the entering state; sUp is free

        // U' = U - W S^T and O = Q S^T (B operand: S[16 sl + li][c])
        f4v o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const float4 s4 = *reinterpret_cast<const float4 *>(&sS[li][16 * kb + 4 * lq]);
            const float4 nw = make_float4(-w4[kb].x, -w4[kb].y, -w4[kb].z, -w4[kb].w);
            up = mfma4(nw, s4, up);
            o = mfma4(q4[kb], s4, o);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sUp[16 * wv + 4 * lq + r][li] = up[r];
        __syncthreads();

        // U'[16 kb + 4 lq + j][16 sl + li]: B operand of M U', A operand of U'^T K
        float4 uu[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int t = 16 * kb + 4 * lq;
            uu[kb] = make_float4(sUp[t][li], sUp[t + 1][li], sUp[t + 2][li], sUp[t + 3][li]);
        }
        // O += causal(Q K^T) U'  (rows of this wave see chunk rows <= 16 wv + 15)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            if (kb <= wv) o = mfma4(m4[kb], uu[kb], o);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * wv + 4 * lq + r;
            if (t < nrow) a.o[(row0 + t) * kDD + 16 * sl + li] = o[r];
        }
        // S += U'^T K on this wave's columns
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) S = mfma4(uu[kb], kc[kb], S);
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[4 * lq + r][16 * wv + li] = S[r];
    }
    if (a.ST) {
#pragma unroll
        for (int r = 0; r < 4; ++r) a.ST[sbase + r * kDD] = S[r];
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
    g.bytes = g.off_wum + static_cast<size_t>(B) * g.nC * 3 * kCh * kDD * sizeof(float);
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
    if (g.nC > 0) {
        hipLaunchKernelGGL(delta_prep_kernel, dim3(static_cast<unsigned>(g.B * g.nC)), dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(delta_state_kernel, dim3(static_cast<unsigned>(g.B * 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace mgs
