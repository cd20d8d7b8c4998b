// mgs_api.cpp -- the C ABI declared in include/mgs.h: argument validation,
// workspace sizing and kernel dispatch.  Validation happens before any HIP
// call, so the error paths can be exercised on a host without a GPU.
#include "mgs.h"

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "device.hpp"
#include "launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;

mgs_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return MGS_OK;
    g_last_hip_error = static_cast<int>(e);
    return MGS_ERR_HIP;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    const void *p;
    size_t bytes;
};

bool overlaps(Range a, Range b)
{
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// every output must be disjoint from every input and from the other outputs
bool any_alias(const Range *in, int nin, const Range *out, int nout)
{
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlaps(out[i], in[j])) return true;
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(out[i], out[j])) return true;
    }
    return false;
}

bool all_aligned(const Range *r, int n)
{
    for (int i = 0; i < n; ++i)
        if (r[i].p && !aligned16(r[i].p)) return false;
    return true;
}

// Product of non-negative tensor dimensions, or -1 when a dimension or the
// product exceeds kMaxElems.  Each factor is bounded before it is multiplied
// and the multiplications are overflow-checked, so caller-supplied sizes can
// never wrap around to a small (or zero) element count.
int64_t bounded_product(std::initializer_list<int64_t> dims)
{
    int64_t n = 1;
    for (int64_t x : dims)
        if (x > kMaxElems) return -1;
    for (int64_t x : dims)
        if (__builtin_mul_overflow(n, x, &n) || n > kMaxElems) return -1;
    return n;
}

// Element counts of the (B,T,d) and (B,d) tensors of an elementwise op.
struct ElemSizes {
    int64_t n, s;
};

mgs_status check_sizes(int64_t B, int64_t T, int64_t d, ElemSizes *out)
{
    if (B < 0 || T < 0 || d < 0) return MGS_ERR_INVALID_VALUE;
    const int64_t n = bounded_product({B, T, d}), s = bounded_product({B, d});
    if (n < 0 || s < 0) return MGS_ERR_UNSUPPORTED;
    *out = ElemSizes{n, s};
    return MGS_OK;
}

mgs_status check_workspace(const void *ws, size_t have, size_t need)
{
    if (!ws) return MGS_ERR_WORKSPACE;
    if (have < need) return MGS_ERR_WORKSPACE;
    if (!aligned16(ws)) return MGS_ERR_INVALID_VALUE;
    return MGS_OK;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

// ------------------------------------------------ scratch of the no-allocation entry point
// mgs_block_affine_scan_fwd_noalloc keeps its workspace in this file-scope
// device array: one copy per GPU, at that GPU's own address, zero-filled when
// the library's device code is loaded and held until the process ends.  Its
// layout: the 256-byte header, a fixed zero region of kNoAllocZerosBytes (the
// h0 of calls that pass none; never written, whatever the shape), then the
// look-back words of the call's shape.  The kernels leave the header ready for
// the next call (the launch counter returns to zero, epochs only grow), so
// nothing is cleared per call; words left by an earlier call carry an older
// launch tag and are never taken for the current call's.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
constexpr size_t kNoAllocZerosBytes = size_t(1) << 20;   // B*d <= 262144
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, set up on first use

// Device address of the current device's `scratch`.  In host code the array's
// name is only a host-side stand-in, so kernels receive this address instead.
mgs_status noalloc_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return MGS_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return MGS_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MGS_OK;
}

}  // namespace

extern "C" {

int mgs_version(void) { return 100; }

const char *mgs_status_string(int status)
{
    switch (status) {
    case MGS_OK: return "MGS_OK: success";
    case MGS_ERR_INVALID_VALUE: return "MGS_ERR_INVALID_VALUE: null pointer, bad size, misalignment or aliasing";
    case MGS_ERR_UNSUPPORTED: return "MGS_ERR_UNSUPPORTED: outside the supported envelope";
    case MGS_ERR_WORKSPACE: return "MGS_ERR_WORKSPACE: workspace missing or too small";
    case MGS_ERR_HIP: return "MGS_ERR_HIP: HIP runtime error (see mgs_last_hip_error)";
    default: return "unknown mgs_status";
    }
}

int mgs_last_hip_error(void) { return g_last_hip_error; }

mgs_status mgs_workspace_check(void *workspace, void *stream, int *flags)
{
    if (!workspace || !flags) return MGS_ERR_INVALID_VALUE;
    hipStream_t s = as_stream(stream);
    mgs::WsHeader *hd = static_cast<mgs::WsHeader *>(workspace);
    uint32_t v = 0;
    hipError_t e = hipMemcpyAsync(&v, &hd->err, sizeof(v), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e);
    *flags = static_cast<int>(v);
    if (v) {
        const uint32_t zero = 0;
        e = hipMemcpyAsync(&hd->err, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_status(e);
    }
    return MGS_OK;
}

mgs_status mgs_workspace_set_waits(void *workspace, unsigned spin_limit, int fail_waits, void *stream)
{
    if (!workspace) return MGS_ERR_INVALID_VALUE;
    hipStream_t s = as_stream(stream);
    mgs::WsHeader *hd = static_cast<mgs::WsHeader *>(workspace);
    const uint32_t v[2] = {static_cast<uint32_t>(spin_limit), fail_waits ? 1u : 0u};
    static_assert(offsetof(mgs::WsHeader, fail_waits) == offsetof(mgs::WsHeader, spin_limit) + 4, "header layout");
    hipError_t e = hipMemcpyAsync(&hd->spin_limit, v, sizeof(v), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e == hipSuccess ? MGS_OK : hip_status(e);
}

// --------------------------- elementwise scans (log, minGRU cell + log, linear)

using ElemFwd = hipError_t (*)(const mgs::LogGeom &, const float *, const float *, const float *,
                               float *, void *, hipStream_t);
using ElemBwd = hipError_t (*)(const mgs::LogGeom &, const float *, const float *, const float *,
                               const float *, float *, float *, float *, void *, hipStream_t);

static mgs_status elem_workspace_size(int64_t B, int64_t T, int64_t d, size_t *bytes)
{
    if (!bytes) return MGS_ERR_INVALID_VALUE;
    ElemSizes z;
    if (mgs_status st = check_sizes(B, T, d, &z)) return st;
    if (z.n == 0) { *bytes = sizeof(mgs::WsHeader); return MGS_OK; }
    *bytes = mgs::log_geometry(B, T, d).bytes;
    return MGS_OK;
}

static mgs_status elem_fwd(ElemFwd launch, const float *x1, const float *x2, const float *x0, float *h,
                           int64_t B, int64_t T, int64_t d, void *workspace, size_t workspace_bytes,
                           void *stream)
{
    ElemSizes z;
    if (mgs_status st = check_sizes(B, T, d, &z)) return st;
    const size_t n = static_cast<size_t>(z.n) * 4, s0 = static_cast<size_t>(z.s) * 4;
    if (n > 0 && (!x1 || !x2 || !h)) return MGS_ERR_INVALID_VALUE;
    if (s0 > 0 && !x0) return MGS_ERR_INVALID_VALUE;
    const Range in[] = {{x1, n}, {x2, n}, {x0, s0}};
    const Range out[] = {{h, n}};
    if (!all_aligned(in, 3) || !all_aligned(out, 1)) return MGS_ERR_INVALID_VALUE;
    if (any_alias(in, 3, out, 1)) return MGS_ERR_INVALID_VALUE;
    if (n == 0) return MGS_OK;
    const mgs::LogGeom g = mgs::log_geometry(B, T, d);
    if (mgs_status st = check_workspace(workspace, workspace_bytes, g.bytes)) return st;
    return hip_status(launch(g, x1, x2, x0, h, workspace, as_stream(stream)));
}

static mgs_status elem_bwd(ElemFwd launch_f, ElemBwd launch_b, const float *x1, const float *x2,
                           const float *x0, const float *dh, float *d1, float *d2, float *d0,
                           int64_t B, int64_t T, int64_t d, void *workspace, size_t workspace_bytes,
                           int fwd_state_valid, void *stream)
{
    ElemSizes z;
    if (mgs_status st = check_sizes(B, T, d, &z)) return st;
    const size_t n = static_cast<size_t>(z.n) * 4, s0 = static_cast<size_t>(z.s) * 4;
    if (n > 0 && (!x1 || !x2 || !dh || !d1 || !d2)) return MGS_ERR_INVALID_VALUE;
    if (s0 > 0 && (!x0 || !d0)) return MGS_ERR_INVALID_VALUE;
    const Range in[] = {{x1, n}, {x2, n}, {x0, s0}, {dh, n}};
    const Range out[] = {{d1, n}, {d2, n}, {d0, s0}};
    if (!all_aligned(in, 4) || !all_aligned(out, 3)) return MGS_ERR_INVALID_VALUE;
    if (any_alias(in, 4, out, 3)) return MGS_ERR_INVALID_VALUE;
    if (s0 == 0) return MGS_OK;
    hipStream_t s = as_stream(stream);
    if (T == 0)  // L does not depend on h0 when there are no steps
        return hip_status(mgs::launch_fill_zero(d0, z.s, s));
    const mgs::LogGeom g = mgs::log_geometry(B, T, d);
    if (mgs_status st = check_workspace(workspace, workspace_bytes, g.bytes)) return st;
    if (g.nT > 1 && !fwd_state_valid) {
        hipError_t e = launch_f(g, x1, x2, x0, nullptr, workspace, s);
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(launch_b(g, x1, x2, x0, dh, d1, d2, d0, workspace, s));
}

mgs_status mgs_scan_log_workspace_size(int64_t B, int64_t T, int64_t d, size_t *bytes)
{
    return elem_workspace_size(B, T, d, bytes);
}

mgs_status mgs_scan_log_fwd(const float *log_a, const float *log_b, const float *log_h0, float *h,
                            int64_t B, int64_t T, int64_t d, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    return elem_fwd(mgs::launch_log_fwd, log_a, log_b, log_h0, h, B, T, d, workspace, workspace_bytes,
                    stream);
}

mgs_status mgs_scan_log_bwd(const float *log_a, const float *log_b, const float *log_h0,
                            const float *dh, float *dlog_a, float *dlog_b, float *dlog_h0,
                            int64_t B, int64_t T, int64_t d, void *workspace,
                            size_t workspace_bytes, int fwd_state_valid, void *stream)
{
    return elem_bwd(mgs::launch_log_fwd, mgs::launch_log_bwd, log_a, log_b, log_h0, dh, dlog_a, dlog_b,
                    dlog_h0, B, T, d, workspace, workspace_bytes, fwd_state_valid, stream);
}

mgs_status mgs_scan_mingru_workspace_size(int64_t B, int64_t T, int64_t d, size_t *bytes)
{
    return elem_workspace_size(B, T, d, bytes);
}

mgs_status mgs_scan_mingru_fwd(const float *k, const float *x, const float *x0, float *h,
                               int64_t B, int64_t T, int64_t d, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    return elem_fwd(mgs::launch_mingru_fwd, k, x, x0, h, B, T, d, workspace, workspace_bytes, stream);
}

mgs_status mgs_scan_mingru_bwd(const float *k, const float *x, const float *x0, const float *dh,
                               float *dk, float *dx, float *dx0, int64_t B, int64_t T, int64_t d,
                               void *workspace, size_t workspace_bytes, int fwd_state_valid,
                               void *stream)
{
    return elem_bwd(mgs::launch_mingru_fwd, mgs::launch_mingru_bwd, k, x, x0, dh, dk, dx, dx0, B, T, d,
                    workspace, workspace_bytes, fwd_state_valid, stream);
}

mgs_status mgs_scan_linear_workspace_size(int64_t B, int64_t T, int64_t d, size_t *bytes)
{
    return elem_workspace_size(B, T, d, bytes);
}

mgs_status mgs_scan_linear_fwd(const float *a, const float *b, const float *h0, float *h,
                               int64_t B, int64_t T, int64_t d, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    return elem_fwd(mgs::launch_linear_fwd, a, b, h0, h, B, T, d, workspace, workspace_bytes, stream);
}

mgs_status mgs_scan_linear_bwd(const float *a, const float *b, const float *h0, const float *dh,
                               float *da, float *db, float *dh0, int64_t B, int64_t T, int64_t d,
                               void *workspace, size_t workspace_bytes, int fwd_state_valid,
                               void *stream)
{
    return elem_bwd(mgs::launch_linear_fwd, mgs::launch_linear_bwd, a, b, h0, dh, da, db, dh0, B, T, d,
                    workspace, workspace_bytes, fwd_state_valid, stream);
}

// ---------------------------------------------------------- block scans

// Element counts of a block op's tensors: n of (B,T,d), s of (B,d), na of
// (B,T,d/k,k,k); for the Givens scan nth of the angles (B,T,d/k,k(k-1)/2) and
// ns of the gates (B,T,d/k).  na bounds the others, so none can overflow.
struct BlockSizes {
    int64_t n, s, na, nth, ns;
};

static mgs_status check_block_sizes(int64_t B, int64_t T, int64_t d, int64_t k, BlockSizes *out)
{
    if (B < 0 || T < 0 || d < 0 || k <= 0) return MGS_ERR_INVALID_VALUE;
    if (d % k != 0) return MGS_ERR_INVALID_VALUE;
    if (!mgs::block_k_supported(k)) return MGS_ERR_UNSUPPORTED;
    const int64_t na = bounded_product({B, T, d, k});
    if (na < 0) return MGS_ERR_UNSUPPORTED;
    const int64_t n = B * T * d, nbt = B * T * (d / k);
    *out = BlockSizes{n, B * d, na, nbt * (k * (k - 1) / 2), nbt};
    return MGS_OK;
}

// The Givens angle-fused scan is built for 8 x 8 blocks (28 angles) only.
static mgs_status check_givens_sizes(int64_t B, int64_t T, int64_t d, int64_t k, BlockSizes *out)
{
    if (mgs_status st = check_block_sizes(B, T, d, k, out)) return st;
    return k == 8 ? MGS_OK : MGS_ERR_UNSUPPORTED;
}

mgs_status mgs_block_affine_scan_workspace_size(int64_t B, int64_t T, int64_t d, int64_t k,
                                                size_t *bytes)
{
    if (!bytes) return MGS_ERR_INVALID_VALUE;
    BlockSizes z;
    if (mgs_status st = check_block_sizes(B, T, d, k, &z)) return st;
    if (z.n == 0) { *bytes = sizeof(mgs::WsHeader); return MGS_OK; }
    *bytes = mgs::block_affine_geometry(B, T, d, k).bytes;
    return MGS_OK;
}

mgs_status mgs_block_affine_scan_fwd(const float *A, const float *b, const float *h0, float *h,
                                     int64_t B, int64_t T, int64_t d, int64_t k, void *workspace,
                                     size_t workspace_bytes, void *stream)
{
    BlockSizes z;
    if (mgs_status st = check_block_sizes(B, T, d, k, &z)) return st;
    const size_t n = static_cast<size_t>(z.n) * 4, s0 = static_cast<size_t>(z.s) * 4;
    const size_t na = static_cast<size_t>(z.na) * 4;
    if (n > 0 && (!A || !b || !h)) return MGS_ERR_INVALID_VALUE;
    const Range in[] = {{A, na}, {b, n}, {h0, s0}};
    const Range out[] = {{h, n}};
    if (!all_aligned(in, 3) || !all_aligned(out, 1)) return MGS_ERR_INVALID_VALUE;
    if (any_alias(in, 3, out, 1)) return MGS_ERR_INVALID_VALUE;
    if (n == 0) return MGS_OK;
    const mgs::BlockGeom g = mgs::block_affine_geometry(B, T, d, k);
    if (mgs_status st = check_workspace(workspace, workspace_bytes, g.bytes)) return st;
    return hip_status(mgs::launch_block_affine_fwd(g, A, b, h0, h, workspace,
                                                   as_stream(stream)));
}

mgs_status mgs_block_affine_scan_fwd_noalloc(const float *A, const float *b, const float *h0, float *h,
                                             int64_t B, int64_t T, int64_t d, int64_t k, void *stream)
{
    BlockSizes z;
    if (mgs_status st = check_block_sizes(B, T, d, k, &z)) return st;
    const size_t n = static_cast<size_t>(z.n) * 4, s0 = static_cast<size_t>(z.s) * 4;
    const size_t na = static_cast<size_t>(z.na) * 4;
    if (n > 0 && (!A || !b || !h)) return MGS_ERR_INVALID_VALUE;
    const Range in[] = {{A, na}, {b, n}, {h0, s0}};
    const Range out[] = {{h, n}};
    if (!all_aligned(in, 3) || !all_aligned(out, 1)) return MGS_ERR_INVALID_VALUE;
    if (any_alias(in, 3, out, 1)) return MGS_ERR_INVALID_VALUE;
    if (n == 0) return MGS_OK;
    if (s0 > kNoAllocZerosBytes) return MGS_ERR_UNSUPPORTED;
    const mgs::BlockGeom g = mgs::block_affine_geometry_fixed_zeros(B, T, d, k, kNoAllocZerosBytes);
    if (g.bytes > kNoAllocScratchBytes) return MGS_ERR_UNSUPPORTED;
    void *ws = nullptr;
    if (mgs_status st = noalloc_scratch(&ws)) return st;
    return hip_status(mgs::launch_block_affine_fwd(g, A, b, h0, h, ws, as_stream(stream)));
}

mgs_status mgs_block_affine_scan_bwd(const float *A, const float *b, const float *h0,
                                     const float *h, const float *dh, float *dA, float *db,
                                     float *dh0, int64_t B, int64_t T, int64_t d, int64_t k,
                                     void *workspace, size_t workspace_bytes, void *stream)
{
    BlockSizes z;
    if (mgs_status st = check_block_sizes(B, T, d, k, &z)) return st;
    const size_t n = static_cast<size_t>(z.n) * 4, s0 = static_cast<size_t>(z.s) * 4;
    const size_t na = static_cast<size_t>(z.na) * 4;
    if (n > 0 && (!A || !h || !dh || !dA || !db)) return MGS_ERR_INVALID_VALUE;
    if (s0 > 0 && !dh0) return MGS_ERR_INVALID_VALUE;
    const Range in[] = {{A, na}, {b, n}, {h0, s0}, {h, n}, {dh, n}};
    const Range out[] = {{dA, na}, {db, n}, {dh0, s0}};
    if (!all_aligned(in, 5) || !all_aligned(out, 3)) return MGS_ERR_INVALID_VALUE;
    if (any_alias(in, 5, out, 3)) return MGS_ERR_INVALID_VALUE;
    if (s0 == 0) return MGS_OK;
    hipStream_t s = as_stream(stream);
    if (T == 0) return hip_status(mgs::launch_fill_zero(dh0, z.s, s));
    const mgs::BlockGeom g = mgs::block_affine_geometry(B, T, d, k);
    if (mgs_status st = check_workspace(workspace, workspace_bytes, g.bytes)) return st;
    return hip_status(mgs::launch_block_affine_bwd(g, A, h0, h, dh, dA, db, dh0, workspace, s));
}

mgs_status mgs_givens_scan_workspace_size(int64_t B, int64_t T, int64_t d, int64_t k, size_t *bytes)
{
    if (!bytes) return MGS_ERR_INVALID_VALUE;
    BlockSizes z;
    if (mgs_status st = check_givens_sizes(B, T, d, k, &z)) return st;
    return mgs_block_affine_scan_workspace_size(B, T, d, k, bytes);
}

mgs_status mgs_givens_scan_fwd(const float *theta, const float *s, const float *b, const float *h0,
                               float *h, int64_t B, int64_t T, int64_t d, int64_t k, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    BlockSizes z;
    if (mgs_status st = check_givens_sizes(B, T, d, k, &z)) return st;
    const size_t n = static_cast<size_t>(z.n) * 4, s0 = static_cast<size_t>(z.s) * 4;
    const size_t nth = static_cast<size_t>(z.nth) * 4, ns = static_cast<size_t>(z.ns) * 4;
    if (n > 0 && (!theta || !s || !b || !h)) return MGS_ERR_INVALID_VALUE;
    const Range in[] = {{theta, nth}, {s, ns}, {b, n}, {h0, s0}};
    const Range out[] = {{h, n}};
    if (!all_aligned(in, 4) || !all_aligned(out, 1)) return MGS_ERR_INVALID_VALUE;
    if (any_alias(in, 4, out, 1)) return MGS_ERR_INVALID_VALUE;
    if (n == 0) return MGS_OK;
    const mgs::BlockGeom g = mgs::block_affine_geometry(B, T, d, k);
    if (mgs_status st = check_workspace(workspace, workspace_bytes, g.bytes)) return st;
    return hip_status(mgs::launch_givens_fwd(g, theta, s, b, h0, h, workspace, as_stream(stream)));
}

mgs_status mgs_givens_scan_bwd(const float *theta, const float *s, const float *h0, const float *h,
                               const float *dh, float *dtheta, float *ds, float *db, float *dh0,
                               int64_t B, int64_t T, int64_t d, int64_t k, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    BlockSizes z;
    if (mgs_status st = check_givens_sizes(B, T, d, k, &z)) return st;
    const size_t n = static_cast<size_t>(z.n) * 4, s0 = static_cast<size_t>(z.s) * 4;
    const size_t nth = static_cast<size_t>(z.nth) * 4, ns = static_cast<size_t>(z.ns) * 4;
    if (n > 0 && (!theta || !s || !h || !dh || !dtheta || !ds || !db)) return MGS_ERR_INVALID_VALUE;
    if (s0 > 0 && !dh0) return MGS_ERR_INVALID_VALUE;
    const Range in[] = {{theta, nth}, {s, ns}, {h0, s0}, {h, n}, {dh, n}};
    const Range out[] = {{dtheta, nth}, {ds, ns}, {db, n}, {dh0, s0}};
    if (!all_aligned(in, 5) || !all_aligned(out, 4)) return MGS_ERR_INVALID_VALUE;
    if (any_alias(in, 5, out, 4)) return MGS_ERR_INVALID_VALUE;
    if (s0 == 0) return MGS_OK;
    hipStream_t st = as_stream(stream);
    if (T == 0) return hip_status(mgs::launch_fill_zero(dh0, z.s, st));
    const mgs::BlockGeom g = mgs::block_affine_geometry(B, T, d, k);
    if (mgs_status e = check_workspace(workspace, workspace_bytes, g.bytes)) return e;
    return hip_status(mgs::launch_givens_bwd(g, theta, s, h0, h, dh, dtheta, ds, db, dh0, workspace, st));
}

mgs_status mgs_block_matrix_scan_workspace_size(int64_t B, int64_t T, int64_t d, int64_t k,
                                                size_t *bytes)
{
    if (!bytes) return MGS_ERR_INVALID_VALUE;
    BlockSizes z;
    if (mgs_status st = check_block_sizes(B, T, d, k, &z)) return st;
    if (z.n == 0) { *bytes = sizeof(mgs::WsHeader); return MGS_OK; }
    *bytes = mgs::block_matrix_geometry(B, T, d, k, true).bytes;
    return MGS_OK;
}

mgs_status mgs_block_matrix_scan_fwd(const float *A, float *P, int64_t B, int64_t T, int64_t d,
                                     int64_t k, void *workspace, size_t workspace_bytes,
                                     void *stream)
{
    BlockSizes z;
    if (mgs_status st = check_block_sizes(B, T, d, k, &z)) return st;
    const size_t na = static_cast<size_t>(z.na) * 4;
    if (na > 0 && (!A || !P)) return MGS_ERR_INVALID_VALUE;
    const Range in[] = {{A, na}};
    const Range out[] = {{P, na}};
    if (!all_aligned(in, 1) || !all_aligned(out, 1)) return MGS_ERR_INVALID_VALUE;
    if (any_alias(in, 1, out, 1)) return MGS_ERR_INVALID_VALUE;
    if (na == 0) return MGS_OK;
    const mgs::BlockGeom g = mgs::block_matrix_geometry(B, T, d, k, true);
    if (mgs_status st = check_workspace(workspace, workspace_bytes, g.bytes)) return st;
    return hip_status(mgs::launch_block_matrix_fwd(g, A, P, workspace, as_stream(stream)));
}

mgs_status mgs_block_matrix_scan_bwd(const float *A, const float *dP, float *dA, int64_t B, int64_t T,
                                     int64_t d, int64_t k, void *workspace, size_t workspace_bytes,
                                     int fwd_state_valid, void *stream)
{
    BlockSizes z;
    if (mgs_status st = check_block_sizes(B, T, d, k, &z)) return st;
    const size_t na = static_cast<size_t>(z.na) * 4;
    if (na > 0 && (!A || !dP || !dA)) return MGS_ERR_INVALID_VALUE;
    const Range in[] = {{A, na}, {dP, na}};
    const Range out[] = {{dA, na}};
    if (!all_aligned(in, 2) || !all_aligned(out, 1)) return MGS_ERR_INVALID_VALUE;
    if (any_alias(in, 2, out, 1)) return MGS_ERR_INVALID_VALUE;
    if (na == 0) return MGS_OK;
    const mgs::BlockGeom gf = mgs::block_matrix_geometry(B, T, d, k, true);
    const mgs::BlockGeom g = mgs::block_matrix_geometry(B, T, d, k, false);
    if (mgs_status st = check_workspace(workspace, workspace_bytes, g.bytes)) return st;
    return hip_status(mgs::launch_block_matrix_bwd(gf, g, A, dP, dA, workspace, fwd_state_valid != 0,
                                                   as_stream(stream)));
}

// ------------------------------------------------------------ delta rule

// Element counts of the delta rule's tensors: n of (B,T,d), nb of (B,T),
// ns of (B,d,d).
struct DeltaSizes {
    int64_t n, nb, ns;
};

static mgs_status check_delta_sizes(int64_t B, int64_t T, int64_t d, DeltaSizes *out)
{
    if (B < 0 || T < 0 || d <= 0) return MGS_ERR_INVALID_VALUE;
    if (d != 64) return MGS_ERR_UNSUPPORTED;
    const int64_t n = bounded_product({B, T, d}), ns = bounded_product({B, d, d});
    if (n < 0 || ns < 0) return MGS_ERR_UNSUPPORTED;
    *out = DeltaSizes{n, B * T, ns};
    return MGS_OK;
}

mgs_status mgs_delta_workspace_size(int64_t B, int64_t T, int64_t d, size_t *bytes)
{
    if (!bytes) return MGS_ERR_INVALID_VALUE;
    DeltaSizes z;
    if (mgs_status st = check_delta_sizes(B, T, d, &z)) return st;
    *bytes = mgs::delta_geometry(B, T, d).bytes;
    return MGS_OK;
}

mgs_status mgs_delta_fwd(const float *q, const float *k, const float *v, const float *beta,
                         const float *S0, float *o, float *ST, int64_t B, int64_t T, int64_t d,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    DeltaSizes z;
    if (mgs_status st = check_delta_sizes(B, T, d, &z)) return st;
    const size_t n = static_cast<size_t>(z.n) * 4, nb = static_cast<size_t>(z.nb) * 4;
    const size_t ns = static_cast<size_t>(z.ns) * 4;
    if (n > 0 && (!q || !k || !v || !beta || !o)) return MGS_ERR_INVALID_VALUE;
    const Range in[] = {{q, n}, {k, n}, {v, n}, {beta, nb}, {S0, ns}};
    const Range out[] = {{o, n}, {ST, ns}};
    if (!all_aligned(in, 5) || !all_aligned(out, 2)) return MGS_ERR_INVALID_VALUE;
    if (any_alias(in, 5, out, 2)) return MGS_ERR_INVALID_VALUE;
    if (B == 0 || (T == 0 && !ST)) return MGS_OK;
    const mgs::DeltaGeom g = mgs::delta_geometry(B, T, d);
    if (mgs_status st = check_workspace(workspace, workspace_bytes, g.bytes)) return st;
    return hip_status(mgs::launch_delta_fwd(g, q, k, v, beta, S0, o, ST, workspace, as_stream(stream)));
}

}  // extern "C"
