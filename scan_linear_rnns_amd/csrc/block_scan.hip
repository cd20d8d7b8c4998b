// block_scan.hip -- host side of the block scans: geometry and workspace
// layout, entry points for every block size, the k = 8 kernels and the
// Givens angle-fused kernels (k = 8).  The device code is in block_core.hpp;
// the kernels of the other block sizes are instantiated in block_scan_k.hip,
// one object file per k.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "block_core.hpp"

namespace mgs {
namespace {

__global__ void fill_zero_kernel(float *p, int64_t n)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// zeros_bytes: size of the zero region that stands in for an absent h0 (at
// least B*d floats; a caller that shares one workspace between shapes passes a
// fixed capacity, so the region never moves onto words another shape wrote).
// pstate_chunks: saved states along T the state region holds (0: none);
// lb_tiles: tiles the look-back regions hold (at least this shape's).
BlockGeom make_geom(int64_t B, int64_t T, int64_t d, int64_t k, int agg_words, int incl_words,
                    BlkShape shape, int64_t pstate_chunks, int64_t lb_tiles, size_t zeros_bytes = 0)
{
    BlockGeom g{};
    g.T = static_cast<int>(T);
    g.d = static_cast<int>(d);
    g.k = static_cast<int>(k);
    g.nb = static_cast<int>(d / k);
    g.nchain = B * g.nb;
    g.G = static_cast<int>(32 / k);   // chains per half-wave
    g.W = shape.W;
    const int nch = 2 * shape.W;
    int C = 1;
    while (C < shape.max_c && static_cast<int64_t>(nch) * C < T) C *= 2;
    g.C = C;
    g.TT = nch * C;
    g.nT = static_cast<int>((T + g.TT - 1) / g.TT);
    g.nCG = static_cast<int>((g.nchain + g.G - 1) / g.G);
    g.nTiles = g.nT * g.nCG;
    g.agg_words = agg_words;
    g.incl_words = incl_words;
    size_t off = sizeof(WsHeader);
    g.off_zeros = off;   // B*d floats, never written: the h0 of calls that pass none
    const size_t zb = static_cast<size_t>(B) * d * 4;
    off = align256(off + (zeros_bytes > zb ? zeros_bytes : zb));
    g.off_pstate = off;  // cumulative product: one k x k state per chain per chunk
    if (pstate_chunks > 0) off = align256(off + static_cast<size_t>(pstate_chunks) * g.nCG * 32 * k * 4);
    if (g.nT > 1 || lb_tiles > 0) {
        const size_t slots = static_cast<size_t>(lb_tiles > g.nTiles ? lb_tiles : g.nTiles) * 32;
        g.off_agg = off;  off = align256(off + slots * agg_words * 8);
        g.off_incl = off; off = align256(off + slots * incl_words * 8);
    }
    g.bytes = off;
    return g;
}

BlkArgs base_args(const BlockGeom &g, void *ws)
{
    char *w = static_cast<char *>(ws);
    WsHeader *hd = reinterpret_cast<WsHeader *>(w);
    BlkArgs a{};
    a.nchain = g.nchain;
    a.T = g.T; a.d = g.d; a.nb = g.nb; a.nCG = g.nCG; a.nT = g.nT; a.nTiles = g.nTiles;
    a.hd = hd;
    a.lb_local = lookback_on_one_xcd(g.nCG);
    if (g.nT > 1) {
        a.agg = reinterpret_cast<uint64_t *>(w + g.off_agg);
        a.incl = reinterpret_cast<uint64_t *>(w + g.off_incl);
    }
    a.pstate = reinterpret_cast<float *>(w + g.off_pstate);
    a.pcs = g.pcs;
    return a;
}

const float *zeros_or(const BlockGeom &g, void *ws, const float *h0)
{
    return h0 ? h0 : reinterpret_cast<const float *>(static_cast<char *>(ws) + g.off_zeros);
}

// Givens kernels: template <int C, int W, bool MULTI>, k = 8.
#define MGS_DEFINE_GIVENS_LAUNCHER(NAME, KERNEL)                                                  \
    template <int W, int C>                                                                       \
    void NAME##_c(const BlockGeom &g, const BlkArgs &a, hipStream_t s)                            \
    {                                                                                             \
        if (g.nT > 1)                                                                             \
            hipLaunchKernelGGL((KERNEL<C, W, true>), dim3(g.nTiles), dim3(64 * W), 0, s, a);      \
        else                                                                                      \
            hipLaunchKernelGGL((KERNEL<C, W, false>), dim3(g.nTiles), dim3(64 * W), 0, s, a);     \
    }                                                                                             \
    template <int W, int MAXC>                                                                    \
    void NAME(const BlockGeom &g, const BlkArgs &a, hipStream_t s)                                \
    {                                                                                             \
        switch (g.C) {                                                                            \
        case 1: NAME##_c<W, 1>(g, a, s); break;                                                   \
        case 2: NAME##_c<W, 2>(g, a, s); break;                                                   \
        case 4: if constexpr (MAXC >= 4) NAME##_c<W, 4>(g, a, s); break;                          \
        case 8: if constexpr (MAXC >= 8) NAME##_c<W, 8>(g, a, s); break;                          \
        default: if constexpr (MAXC >= 16) NAME##_c<W, 16>(g, a, s); break;                       \
        }                                                                                         \
    }

MGS_DEFINE_GIVENS_LAUNCHER(launch_bgivens_fwd, bgivens_fwd_kernel)
MGS_DEFINE_GIVENS_LAUNCHER(launch_bgivens_bwd, bgivens_bwd_kernel)

// one block op for the geometry's block size
void launch_blk_any(BlkOp op, const BlockGeom &g, const BlkArgs &a, hipStream_t s)
{
    switch (g.k) {
    case 1: launch_blk<1>(op, g, a, s); break;
    case 2: launch_blk<2>(op, g, a, s); break;
    case 4: launch_blk<4>(op, g, a, s); break;
    case 8: launch_blk<8>(op, g, a, s); break;
    default: launch_blk<16>(op, g, a, s); break;
    }
}

}  // namespace

template <>
void launch_blk<8>(BlkOp op, const BlockGeom &g, const BlkArgs &a, hipStream_t s)
{
    launch_blk_impl<8>(op, g, a, s);
}

bool block_k_supported(int64_t k)
{
    return k == 1 || k == 2 || k == 4 || k == 8 || k == 16;
}

BlockGeom block_affine_geometry(int64_t B, int64_t T, int64_t d, int64_t k)
{
    return make_geom(B, T, d, k, static_cast<int>(k) + 1, 1, affine_shape(static_cast<int>(k)), 0, 0);
}

BlockGeom block_affine_geometry_fixed_zeros(int64_t B, int64_t T, int64_t d, int64_t k, size_t zeros_bytes)
{
    return make_geom(B, T, d, k, static_cast<int>(k) + 1, 1, affine_shape(static_cast<int>(k)), 0, 0,
                     zeros_bytes);
}

// One workspace layout serves both directions of the cumulative product: the
// saved states (one per backward chunk: the forward writes the state entering
// every step the backward starts a chunk at) and the look-back regions are
// sized for the larger of the two tilings, so the forward's and the
// backward's geometry place every region at the same offset.
BlockGeom block_matrix_geometry(int64_t B, int64_t T, int64_t d, int64_t k, bool forward)
{
    const int ki = static_cast<int>(k);
    const BlockGeom gf = make_geom(B, T, d, k, 2 * ki, ki, matrix_shape(ki, true), 0, 0);
    const BlockGeom gb = make_geom(B, T, d, k, 2 * ki, ki, matrix_shape(ki, false), 0, 0);
    const int64_t steps = std::max(static_cast<int64_t>(gf.nT) * gf.TT, static_cast<int64_t>(gb.nT) * gb.TT);
    const int64_t tiles = (gf.nT > 1 || gb.nT > 1) ? std::max(gf.nTiles, gb.nTiles) : 0;
    BlockGeom g = make_geom(B, T, d, k, 2 * ki, ki, matrix_shape(ki, forward), (steps + gb.C - 1) / gb.C, tiles);
    g.pcs = 0;
    while ((1 << g.pcs) < gb.C) ++g.pcs;   // C is a power of two
    return g;
}

hipError_t launch_block_affine_fwd(const BlockGeom &g, const float *A, const float *b,
                                   const float *h0, float *h, void *ws, hipStream_t s)
{
    BlkArgs a = base_args(g, ws);
    a.A = A; a.x = b; a.out = h;
    a.h0 = zeros_or(g, ws, h0);
    launch_blk_any(BlkOp::AffineFwd, g, a, s);
    return hipGetLastError();
}

hipError_t launch_block_affine_bwd(const BlockGeom &g, const float *A, const float *h0,
                                   const float *h, const float *dh, float *dA, float *db,
                                   float *dh0, void *ws, hipStream_t s)
{
    BlkArgs a = base_args(g, ws);
    a.A = A; a.x = h; a.y = dh; a.out = dA; a.out2 = db; a.out3 = dh0;
    a.h0 = zeros_or(g, ws, h0);
    launch_blk_any(BlkOp::AffineBwd, g, a, s);
    return hipGetLastError();
}

hipError_t launch_givens_fwd(const BlockGeom &g, const float *theta, const float *sg, const float *b,
                             const float *h0, float *h, void *ws, hipStream_t s)
{
    constexpr BlkShape af = affine_shape(8);
    BlkArgs a = base_args(g, ws);
    a.theta = theta; a.sg = sg; a.x = b; a.out = h;
    a.h0 = zeros_or(g, ws, h0);
    launch_bgivens_fwd<af.W, af.max_c>(g, a, s);
    return hipGetLastError();
}

hipError_t launch_givens_bwd(const BlockGeom &g, const float *theta, const float *sg, const float *h0,
                             const float *h, const float *dh, float *dtheta, float *dsg, float *db,
                             float *dh0, void *ws, hipStream_t s)
{
    constexpr BlkShape af = affine_shape(8);
    BlkArgs a = base_args(g, ws);
    a.theta = theta; a.sg = sg; a.x = h; a.y = dh;
    a.dtheta = dtheta; a.dsg = dsg; a.out2 = db; a.out3 = dh0;
    a.h0 = zeros_or(g, ws, h0);
    launch_bgivens_bwd<af.W, af.max_c>(g, a, s);
    return hipGetLastError();
}

hipError_t launch_block_matrix_fwd(const BlockGeom &g, const float *A, float *P, void *ws,
                                   hipStream_t s)
{
    BlkArgs a = base_args(g, ws);
    a.A = A; a.out = P;
    launch_blk_any(BlkOp::MatrixFwd, g, a, s);
    return hipGetLastError();
}

hipError_t launch_block_matrix_bwd(const BlockGeom &gf, const BlockGeom &g, const float *A, const float *dP,
                                   float *dA, void *ws, bool fwd_state_valid, hipStream_t s)
{
    if (!fwd_state_valid) {
        BlkArgs f = base_args(gf, ws);
        f.A = A; f.out = nullptr;    // chunk states only
        launch_blk_any(BlkOp::MatrixFwd, gf, f, s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    BlkArgs a = base_args(g, ws);
    a.A = A; a.y = dP; a.out = dA;
    launch_blk_any(BlkOp::MatrixBwd, g, a, s);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const int threads = 256;
    const int64_t blocks = (n + threads - 1) / threads;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace mgs
