// launch.hpp -- host-side interface between the C ABI (mgs_api.cpp) and the
// kernel translation units.  Geometry (tiling of T and of the chains) and the
// workspace layout are decided here once per shape, so the forward and the
// backward of one op always agree on both.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace mgs {

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// XCDs (compute dies, each with an L2 of its own) of the current device, to
// which the dispatcher deals a launch's workgroups round robin by blockIdx
// (8 on an MI355X in its single-partition mode, fewer per partition
// otherwise); 0 if the runtime cannot say.  Queried once per device.
inline int xcd_count()
{
    constexpr int kDevs = 64;
    static std::atomic<int> cache[kDevs];   // count + 1; 0 = not queried yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n < 0) n = 0;
        v = n + 1;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v - 1;
}

// Whether every reader of a tile's look-back words runs on the writer's XCD:
// the tiles of one chain group lie nCG apart in blockIdx.
inline bool lookback_on_one_xcd(int nCG)
{
    const int n = xcd_count();
    return n > 0 && nCG % n == 0;
}

// ----------------------------- elementwise scans (log, minGRU cell + log, linear)
// One geometry and workspace layout serves every arithmetic.
struct LogGeom {
    int64_t S;      // chains = B*d
    int T, d;
    int CHW;        // chains per wave row
    int W;          // waves per workgroup
    int C;          // steps per lane
    int TT;         // steps per tile
    int nT;         // tiles along T
    int nCG;        // chain groups
    int nTiles;     // nT * nCG
    // workspace layout (byte offsets)
    size_t off_fagg_a, off_fagg_h, off_fincl, off_carry, off_bagg_p, off_bagg_w, off_bincl, bytes;
};

LogGeom log_geometry(int64_t B, int64_t T, int64_t d);

hipError_t launch_log_fwd(const LogGeom &g, const float *la, const float *lb, const float *lh0,
                          float *h, void *ws, hipStream_t s);
hipError_t launch_log_bwd(const LogGeom &g, const float *la, const float *lb, const float *lh0,
                          const float *dh, float *dla, float *dlb, float *dlh0, void *ws,
                          hipStream_t s);
hipError_t launch_mingru_fwd(const LogGeom &g, const float *k, const float *x, const float *x0,
                             float *h, void *ws, hipStream_t s);
hipError_t launch_mingru_bwd(const LogGeom &g, const float *k, const float *x, const float *x0,
                             const float *dh, float *dk, float *dx, float *dx0, void *ws,
                             hipStream_t s);
hipError_t launch_linear_fwd(const LogGeom &g, const float *a, const float *b, const float *h0,
                             float *h, void *ws, hipStream_t s);
hipError_t launch_linear_bwd(const LogGeom &g, const float *a, const float *b, const float *h0,
                             const float *dh, float *da, float *db, float *dh0, void *ws,
                             hipStream_t s);

// ------------------------------------------------------------- block scans
struct BlockGeom {
    int64_t nchain; // B * d/k
    int T, d, k, nb;
    int G;          // chains per half-wave (32 / k)
    int C;          // steps per lane group
    int W;          // waves (chunks) per workgroup
    int TT;         // steps per tile
    int nT;         // tiles along T
    int nCG;        // chain groups (of G chains)
    int nTiles;
    size_t off_zeros;                 // B*d zero floats standing in for an absent h0
    size_t off_pstate;                // cumulative product: chunk-entering states
    size_t off_agg, off_incl, bytes;  // look-back payload (tagged words)
    int agg_words;  // tagged words per chain per tile in the aggregate
    int incl_words; // tagged words per chain per tile in the inclusive prefix
    int pcs;        // cumulative product: log2 of the steps between the saved states
};

// block sizes the block ops are built for: k in {1, 2, 4, 8, 16}
bool block_k_supported(int64_t k);

BlockGeom block_affine_geometry(int64_t B, int64_t T, int64_t d, int64_t k);
// the cumulative product's geometry for one direction; both directions share
// one workspace layout (and size)
BlockGeom block_matrix_geometry(int64_t B, int64_t T, int64_t d, int64_t k, bool forward);
// the block-affine layout with a zero region of at least zeros_bytes at a fixed
// offset (for a workspace shared by calls of different shapes)
BlockGeom block_affine_geometry_fixed_zeros(int64_t B, int64_t T, int64_t d, int64_t k, size_t zeros_bytes);

hipError_t launch_block_affine_fwd(const BlockGeom &g, const float *A, const float *b,
                                   const float *h0, float *h, void *ws, hipStream_t s);
hipError_t launch_block_affine_bwd(const BlockGeom &g, const float *A, const float *h0,
                                   const float *h, const float *dh, float *dA, float *db,
                                   float *dh0, void *ws, hipStream_t s);
hipError_t launch_givens_fwd(const BlockGeom &g, const float *theta, const float *sg, const float *b,
                             const float *h0, float *h, void *ws, hipStream_t s);
hipError_t launch_givens_bwd(const BlockGeom &g, const float *theta, const float *sg, const float *h0,
                             const float *h, const float *dh, float *dtheta, float *dsg, float *db,
                             float *dh0, void *ws, hipStream_t s);
hipError_t launch_block_matrix_fwd(const BlockGeom &g, const float *A, float *P, void *ws,
                                   hipStream_t s);
// gf: the forward's geometry, for the chunk states when they are not valid
hipError_t launch_block_matrix_bwd(const BlockGeom &gf, const BlockGeom &g, const float *A, const float *dP,
                                   float *dA, void *ws, bool fwd_state_valid, hipStream_t s);

// ------------------------------------------------------------- delta rule
struct DeltaGeom {
    int64_t B;
    int T, d;
    int nC;            // chunks of 64 steps
    size_t off_wum;    // W, U, causal(Q K^T) per (sequence, chunk)
    size_t bytes;
};

DeltaGeom delta_geometry(int64_t B, int64_t T, int64_t d);
hipError_t launch_delta_fwd(const DeltaGeom &g, const float *q, const float *k, const float *v,
                            const float *beta, const float *S0, float *o, float *ST, void *ws, hipStream_t s);

// zero-fill of n floats (used for gradients of an empty sequence)
hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s);

}  // namespace mgs
