// elem_scan.hip -- the elementwise scans h_t = a_t h_{t-1} + b_t, forward and
// fused backward, for gfx950, in two arithmetics:
//   * log space (minGRU home page, introduction; "Triton on GPU", section "What
//     you gain (and where you don't)", parallel_scan_log): inputs log a, log b,
//     log h0 with a > 0, evaluated in log space after Heinsen (arXiv:2311.06281);
//   * log space with the minGRU cell fused ahead of it: inputs are the
//     pre-activations k, x, x0 and the kernels form log a, log b, log h0;
//   * linear space (linear_scan in the home page's speed-up table and in the
//     "Run the benchmarks" how-to, Step 2): inputs a, b, h0 with a of either
//     sign (SignedMinGRU's negative-eigenvalue gates, home page).
//
// Work decomposition (same for both arithmetics, forward and backward):
//   chain   = (b, c), flattened as b*d + c; CHW consecutive chains per wave row
//             so each per-step load/store of a wave covers CHW*4 contiguous bytes
//             per row;
//   chunk   = C consecutive steps of one chain, scanned sequentially in the
//             registers of one lane;
//   tile    = one workgroup: W waves x (64/CHW) chunks = NCH chunks = TT steps
//             of CHW chains.  Chunk aggregates meet in LDS;
//   T-tiles = when T > TT, the tiles of one chain group pass their carries by
//             single-pass decoupled look-back (tagged words, tickets; see
//             device.hpp).
//
// Forward state per chunk is a pair (A, H): the chunk's transfer factor and its
// own output from a zero start.  Pairs compose associatively,
//   (A1, H1) then (A2, H2) = (A1 A2, A2 H1 + H2),
// and a carry c entering a segment leaves it as A c + H.  In log space the pair
// is held as (sum of log2 a, log2 H) and the same rules read
//   (LA1 + LA2, lae2(LA2 + LH1, LH2)),  lae2(x, y) = log2(2^x + 2^y);
// everything is re-based at the chunk start, so no running sum of log a ever
// grows with T (a single global cumulative sum of log a would lose fp32 digits
// at long T).  Base 2 maps exp2/log2 to the hardware's native transcendentals.
//
// The backward recomputes h (linear space, from each tile's carried-in state
// that the forward left in the workspace) and runs the reverse scan of
// w_t = a_t g_t with g_t = dh_t + w_{t+1}; per chunk [s, e] the reverse map
// is w_s = W + P w_{e+1} with P = prod a_t, composed the same way.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "launch.hpp"

namespace mgs {
namespace {

// tiles a look-back batch polls at once (measured at the long-T shape, 8
// tiles along T: 4 beats 8 by ~0.2 us per kernel, 16 is ~0.6 us slower; with
// the workgroup-scope publish, 3 beats 4 by ~0.1 us per kernel)
#ifndef MGS_ELEM_LB
#define MGS_ELEM_LB 3
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInf = __builtin_inff();

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// log2(2^x + 2^y).  Exact for -inf operands (returns the other one, or -inf
// for both); NaN propagates.
__device__ __forceinline__ float lae2(float x, float y)
{
    const bool xg = x > y;
    const float m = xg ? x : y;
    const float n = xg ? y : x;
    const float r = m + lg2(1.0f + ex2(n - m));
    return (m == -kInf || m == kInf) ? m : r;
}

// ------------------------------------------------- the two arithmetics

// Log space, base 2: x = log2 a, y = log2 b; pair (A, H) = (sum x, log2 H).
struct LogAlg {
    __device__ static float idA() { return 0.0f; }
    __device__ static float idH() { return -kInf; }
    __device__ static void input(float la, float lb, bool valid, float &x, float &y)
    {
        x = valid ? la * kLog2e : 0.0f;        // masked step: a = 1, b = 0
        y = valid ? lb * kLog2e : -kInf;
    }
    __device__ static void step(float &A, float &H, float x, float y)
    {
        H = lae2(x + H, y);
        A += x;
    }
    // (A1, H1) then (A2, H2)
    __device__ static void combine(float A1, float H1, float A2, float H2, float &A, float &H)
    {
        H = lae2(A2 + H1, H2);
        A = A1 + A2;
    }
    __device__ static float apply(float A, float H, float c) { return lae2(A + c, H); }
    __device__ static float out(float A, float H, float c) { return ex2(A + c) + ex2(H); }
    __device__ static float carry0(float lh0, bool valid) { return valid ? lh0 * kLog2e : -kInf; }
    __device__ static float to_linear(float c) { return ex2(c); }
    // backward: linear-space a and b of a step from its inputs
    __device__ static void lin_ab(float la, float lb, float &a, float &b)
    {
        a = ex2(la * kLog2e);
        b = ex2(lb * kLog2e);
    }
    __device__ static float lin_h0(float lh0) { return ex2(lh0 * kLog2e); }
    // gradients: d/dlog a = g a h_{t-1}, d/dlog b = g b, d/dlog h0 = (a_1 g_1) h0
    __device__ static void grads(float, float, float a, float b, float g, float hprev, float &d1, float &d2)
    {
        d1 = a * g * hprev;
        d2 = g * b;
    }
    __device__ static float grad_h0(float w, float h0, float) { return w * h0; }
};

// Linear space: x = a (any sign), y = b; pair (A, H) as is.
struct LinAlg {
    __device__ static float idA() { return 1.0f; }
    __device__ static float idH() { return 0.0f; }
    __device__ static void input(float a, float b, bool valid, float &x, float &y)
    {
        x = valid ? a : 1.0f;
        y = valid ? b : 0.0f;
    }
    __device__ static void step(float &A, float &H, float x, float y)
    {
        H = x * H + y;
        A *= x;
    }
    __device__ static void combine(float A1, float H1, float A2, float H2, float &A, float &H)
    {
        H = A2 * H1 + H2;
        A = A1 * A2;
    }
    __device__ static float apply(float A, float H, float c) { return A * c + H; }
    __device__ static float out(float A, float H, float c) { return A * c + H; }
    __device__ static float carry0(float h0, bool valid) { return valid ? h0 : 0.0f; }
    __device__ static float to_linear(float c) { return c; }
    __device__ static void lin_ab(float a_in, float b_in, float &a, float &b)
    {
        a = a_in;
        b = b_in;
    }
    __device__ static float lin_h0(float h0) { return h0; }
    // gradients: d/da = g h_{t-1}, d/db = g, d/dh0 = a_1 g_1
    __device__ static void grads(float, float, float, float, float g, float hprev, float &d1, float &d2)
    {
        d1 = g * hprev;
        d2 = g;
    }
    __device__ static float grad_h0(float w, float, float) { return w; }
};

// The minGRU cell ahead of the log-space scan (minGRU home page, introduction:
// Feng et al.'s minGRU): inputs are the pre-activations k, x, x0 and
//     a = sigmoid(-k),  z = 1 - a = sigmoid(k),  b = z g(x),  h_0 = g(x0),
// g(x) = x + 0.5 (x >= 0), sigmoid(x) (x < 0).  The forward forms log2 a,
// log2 b, log2 h_0 in registers and scans them as LogAlg does; the backward
// returns dk, dx, dx0, so no log a / log b tensor or its gradient ever exists.
struct GateAlg : LogAlg {
    __device__ static float rcp(float u) { return __builtin_amdgcn_rcpf(u); }

    // log2 a = log2 sigmoid(-k), log2 b = log2 sigmoid(k) + log2 g(x): one exp2
    // and one log2 for the gate (log2 sigmoid(k) - log2 sigmoid(-k) = k log2 e),
    // one of each for g
    __device__ static void input(float k, float x, bool valid, float &la, float &lb)
    {
        const float kl = k * kLog2e;
        const float tail = lg2(1.0f + ex2(-__builtin_fabsf(kl)));   // log2(1 + e^-|k|)
        const float l2a = __builtin_fminf(-kl, 0.0f) - tail;
        const float xl = x * kLog2e;
        const bool pos = x >= 0.0f;
        const float L = lg2(pos ? x + 0.5f : 1.0f + ex2(xl));          // x < 0: log2(1 + e^x)
        const float l2g = pos ? L : xl - L;                              // log2 sigmoid(x) = x log2 e - L
        la = valid ? l2a : 0.0f;
        lb = valid ? l2a + kl + l2g : -kInf;
    }
    __device__ static float log2_g(float x)
    {
        const float xl = x * kLog2e;
        const bool pos = x >= 0.0f;
        const float L = lg2(pos ? x + 0.5f : 1.0f + ex2(xl));
        return pos ? L : xl - L;
    }
    __device__ static float carry0(float x0, bool valid) { return valid ? log2_g(x0) : -kInf; }

    // sigmoid(-k), sigmoid(k) without cancellation
    __device__ static void gate(float k, float &a, float &z)
    {
        const float e = ex2(-__builtin_fabsf(k) * kLog2e);   // e^-|k|
        const float r = rcp(1.0f + e);
        a = k >= 0.0f ? e * r : r;
        z = k >= 0.0f ? r : e * r;
    }
    // g(x) and g'(x)
    __device__ static void gpos(float x, float &gv, float &gd)
    {
        const float e = ex2(x * kLog2e);                      // x < 0: e^x < 1
        const float r = rcp(1.0f + e);
        const bool pos = x >= 0.0f;
        gv = pos ? x + 0.5f : e * r;                          // sigmoid(x)
        gd = pos ? 1.0f : e * r * r;                          // sigmoid(x) sigmoid(-x)
    }
    __device__ static void lin_ab(float k, float x, float &a, float &b)
    {
        float z, gv, gd;
        gate(k, a, z);
        gpos(x, gv, gd);
        b = z * gv;
    }
    __device__ static float lin_h0(float x0)
    {
        float gv, gd;
        gpos(x0, gv, gd);
        return gv;
    }
    // dk = g a z (g(x) - h_{t-1}),  dx = g z g'(x),  dx0 = (a_1 g_1) g'(x0)
    __device__ static void grads(float k, float x, float a, float, float gr, float hprev, float &d1, float &d2)
    {
        float a2, z, gv, gd;
        gate(k, a2, z);
        gpos(x, gv, gd);
        d1 = gr * a * z * (gv - hprev);
        d2 = gr * z * gd;
    }
    __device__ static float grad_h0(float w, float, float x0)
    {
        float gv, gd;
        gpos(x0, gv, gd);
        return w * gd;
    }
};

// Argument names follow the log-space op; the linear op passes a, b, h0 in the
// same slots and receives da, db, dh0.
struct LogFwdArgs {
    const float *la, *lb, *lh0;
    float *h;                       // nullptr: carries only (used by the backward)
    int64_t S;
    int T, d, nCG, nT, nTiles;
    WsHeader *hd;
    uint64_t *agg_a, *agg_h, *incl; // tagged look-back words, [tile][CHW]
    float *carry;                   // state at each tile start (log2 h or h), [tile][CHW]
    int lb_local;                   // every tile's look-back partners run on its XCD (tagged_store)
};

struct LogBwdArgs {
    const float *la, *lb, *lh0, *dh;
    float *dla, *dlb, *dlh0;
    int64_t S;
    int T, d, nCG, nT, nTiles;
    WsHeader *hd;
    uint64_t *agg_p, *agg_w, *incl;
    const float *carry;
    int lb_local;
};

template <class Alg, int CHW, int C, int W, bool MULTI>
__global__ void __launch_bounds__(64 * W) elem_fwd_kernel(LogFwdArgs a)
{
    constexpr int SUB = 64 / CHW;
    constexpr int NCH = W * SUB;
    constexpr int TT = NCH * C;
    __shared__ float sLA[NCH][CHW];
    __shared__ float sLH[NCH][CHW];
    __shared__ float sPA[MULTI ? NCH : 1][CHW];   // multi-tile: the tile's chunks [0, q) composed
    __shared__ float sPH[MULTI ? NCH : 1][CHW];
    __shared__ float sCarry[CHW];
    __shared__ uint32_t sTicket[3];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int ch = lane % CHW;
    const int q = wv * SUB + lane / CHW;

    const int tile = blockIdx.x;
    const int j = tile / a.nCG;              // T-tile (tiles are numbered T-major)
    const int cg = tile - j * a.nCG;

    const int64_t chain = static_cast<int64_t>(cg) * CHW + ch;
    const bool cv = chain < a.S;
    const int64_t cc = cv ? chain : 0;
    const int64_t bb = cc / a.d;
    const int64_t base = bb * a.T * a.d + (cc - bb * a.d);
    const int t0 = j * TT + q * C;

    // Loads are unconditional (indices clamped into the tensor) so that all of
    // them are in flight at once; masked steps become the identity afterwards.
    float x[C], y[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int t = t0 + i;
        const int64_t off = base + static_cast<int64_t>(t < a.T ? t : a.T - 1) * a.d;
        x[i] = a.la[off];
        y[i] = a.lb[off];
    }
    const float lh0v = a.lh0[cc];
    // the launch ticket after the inputs: its atomic returns behind them
    // rather than ahead of them in wave 0's in-order load queue
    Launch ep{0, 0};
    if constexpr (MULTI) ep = epoch_begin(a.hd);
#pragma unroll
    for (int i = 0; i < C; ++i) Alg::input(x[i], y[i], cv && t0 + i < a.T, x[i], y[i]);

    // chunk-local pair scan from the identity
    float pA[C], pH[C];
    float LA = Alg::idA(), LH = Alg::idH();
#pragma unroll
    for (int i = 0; i < C; ++i) {
        Alg::step(LA, LH, x[i], y[i]);
        pA[i] = LA;
        pH[i] = LH;
    }
    sLA[q][ch] = LA;
    sLH[q][ch] = LH;
    if (MULTI && threadIdx.x == 0) epoch_end(a.hd, ep, a.nTiles, sTicket);
    __syncthreads();
    const uint32_t tag = sTicket[0];

    float carry;
    if constexpr (MULTI) {
        if (threadIdx.x < CHW) {
            float TA = Alg::idA(), TH = Alg::idH();   // tile aggregate, and each chunk's prefix
#pragma unroll
            for (int p = 0; p < NCH; ++p) {
                sPA[p][ch] = TA;
                sPH[p][ch] = TH;
                Alg::combine(TA, TH, sLA[p][ch], sLH[p][ch], TA, TH);
            }
            const size_t slot = static_cast<size_t>(tile) * CHW + ch;
            if (j < a.nT - 1) {
                tagged_store(&a.agg_a[slot], tag, TA, a.lb_local);
                tagged_store(&a.agg_h[slot], tag, TH, a.lb_local);
            }
            const float lh0 = Alg::carry0(lh0v, cv);
            float cin = lh0;
            if (j > 0) {
                // Decoupled look-back over the earlier tiles, nearest first, LB
                // tiles per batch of loads: stop at the first tile whose
                // inclusive state is published, composing the aggregates of the
                // tiles passed on the way (acc covers tiles p+1 .. j-1).  Every
                // tile publishes its aggregate, so a walk that reaches the start
                // of the sequence ends there with the known h0: no tile ever
                // waits for another tile's look-back to finish.
                constexpr int LB = MGS_ELEM_LB;
                float accA = Alg::idA(), accH = Alg::idH(), basev = lh0;
                int p0 = j - 1;
                const uint32_t want = sTicket[1], limit = sTicket[2];
                for (uint32_t spin = 0;;) {
                    uint64_t wi[LB], wa[LB], wh[LB];
#pragma unroll
                    for (int u = 0; u < LB; ++u) {
                        const int p = p0 - u;
                        const size_t ps = (static_cast<size_t>(p < 0 ? 0 : p) * a.nCG + cg) * CHW + ch;
                        wi[u] = tagged_load(&a.incl[ps]);
                        wa[u] = tagged_load(&a.agg_a[ps]);
                        wh[u] = tagged_load(&a.agg_h[ps]);
                    }
                    bool done = false, stop = false;
                    int adv = 0;
#pragma unroll
                    for (int u = 0; u < LB; ++u) {
                        const int p = p0 - u;
                        if (stop) continue;
                        if (p < 0) {
                            done = stop = true;          // reached the start: base is h0
                        } else if (tag_is(wi[u], want)) {
                            basev = tag_value(wi[u]);
                            done = stop = true;
                        } else if (tag_is(wa[u], want) && tag_is(wh[u], want)) {
                            // tile p's aggregate, then the tiles after it
                            Alg::combine(tag_value(wa[u]), tag_value(wh[u]), accA, accH, accA, accH);
                            adv = u + 1;
                        } else {
                            stop = true;
                        }
                    }
                    if (done) break;
                    p0 -= adv;
                    if (adv == 0) {
                        if (++spin >= limit) {
                            raise_error(&a.hd->err, kErrSpin);
                            break;
                        }
                        backoff();
                    }
                }
                cin = Alg::apply(accA, accH, basev);
            }
            if (j < a.nT - 1)
                tagged_store(&a.incl[slot], tag, Alg::apply(TA, TH, cin), a.lb_local);
            a.carry[slot] = cin;
            sCarry[ch] = cin;
        }
        __syncthreads();
        carry = sCarry[ch];
    } else {
        carry = Alg::carry0(lh0v, cv);
    }

    if (a.h == nullptr) return;

    // carry into this lane's chunk (multi-tile: one composed prefix; else the
    // chunks before it one by one), then the fix-up (log space: written as
    // h_t = 2^(LA_t + carry) + 2^(LH_t))
    float cq = carry;
    if constexpr (MULTI)
        cq = Alg::apply(sPA[q][ch], sPH[q][ch], carry);
    else
        for (int p = 0; p < q; ++p) cq = Alg::apply(sLA[p][ch], sLH[p][ch], cq);
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int t = t0 + i;
        if (cv && t < a.T) store_out(&a.h[base + static_cast<int64_t>(t) * a.d], Alg::out(pA[i], pH[i], cq));
    }
}

template <class Alg, int CHW, int C, int W, bool MULTI>
__global__ void __launch_bounds__(64 * W) elem_bwd_kernel(LogBwdArgs a)
{
    constexpr int SUB = 64 / CHW;
    constexpr int NCH = W * SUB;
    constexpr int TT = NCH * C;
    __shared__ float sA[NCH][CHW];   // forward: prod a over the chunk
    __shared__ float sH[NCH][CHW];   // forward: chunk output from a zero start
    __shared__ float sP[NCH][CHW];   // reverse: prod a over the chunk
    __shared__ float sW[NCH][CHW];   // reverse: w at the chunk start from a zero carry
    __shared__ float sCarry[CHW];
    __shared__ uint32_t sTicket[3];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int ch = lane % CHW;
    const int q = wv * SUB + lane / CHW;

    const int tile = blockIdx.x;
    // the launch ticket at kernel start here: the backward's chunk scans are
    // too short to hide the atomic's round trip behind them (log-space long-T
    // backward 8.3 -> 8.6 us, minGRU cell 9.1 -> 10.4 us with it after the loads)
    Launch ep{0, 0};
    if constexpr (MULTI) ep = epoch_begin(a.hd);
    const int jr = tile / a.nCG;             // tiles are numbered from the last T-tile back
    const int cg = tile - jr * a.nCG;
    const int j = a.nT - 1 - jr;
    const int ftile = j * a.nCG + cg;        // the forward's index of this tile

    const int64_t chain = static_cast<int64_t>(cg) * CHW + ch;
    const bool cv = chain < a.S;
    const int64_t cc = cv ? chain : 0;
    const int64_t bb = cc / a.d;
    const int64_t base = bb * a.T * a.d + (cc - bb * a.d);
    const int t0 = j * TT + q * C;

    float r1[C], r2[C], av[C], bv[C], gv[C];   // raw inputs, linear a and b, upstream dh
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int t = t0 + i;
        const int64_t off = base + static_cast<int64_t>(t < a.T ? t : a.T - 1) * a.d;
        r1[i] = load_once(&a.la[off]);
        r2[i] = load_once(&a.lb[off]);
        gv[i] = load_once(&a.dh[off]);
    }
    const float lh0v = a.lh0[cc];
    float cin_f = 0.0f;   // the forward writes a carry for every tile, the first included
    if constexpr (MULTI) cin_f = a.carry[static_cast<size_t>(ftile) * CHW + ch];
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const bool v = cv && t0 + i < a.T;
        Alg::lin_ab(r1[i], r2[i], av[i], bv[i]);
        av[i] = v ? av[i] : 1.0f;
        bv[i] = v ? bv[i] : 0.0f;
        gv[i] = v ? gv[i] : 0.0f;
    }

    // forward recompute, chunk-local from a zero start
    float pA[C], pH[C];
    float A = 1.0f, H = 0.0f;
#pragma unroll
    for (int i = 0; i < C; ++i) {
        H = av[i] * H + bv[i];
        A *= av[i];
        pA[i] = A;
        pH[i] = H;
    }
    // reverse scan, chunk-local from a zero carry
    float wl = 0.0f;
#pragma unroll
    for (int i = C - 1; i >= 0; --i) wl = av[i] * (gv[i] + wl);
    sA[q][ch] = A;
    sH[q][ch] = H;
    sP[q][ch] = A;
    sW[q][ch] = wl;
    if (MULTI && threadIdx.x == 0) epoch_end(a.hd, ep, a.nTiles, sTicket);

    // state entering the tile: h0 for the first tile, else the forward's carry
    const float hin = (j == 0) ? (cv ? Alg::lin_h0(lh0v) : 0.0f) : Alg::to_linear(cin_f);
    __syncthreads();
    const uint32_t tag = sTicket[0];

    float wcarry;
    if constexpr (MULTI) {
        if (threadIdx.x < CHW) {
            float TP = 1.0f, TW = 0.0f;   // tile aggregate, w_s = TW + TP * w_{e+1}
#pragma unroll
            for (int p = NCH - 1; p >= 0; --p) {
                TW = sW[p][ch] + sP[p][ch] * TW;
                TP = sP[p][ch] * TP;
            }
            const size_t slot = static_cast<size_t>(ftile) * CHW + ch;
            if (j > 0) {
                tagged_store(&a.agg_p[slot], tag, TP, a.lb_local);
                tagged_store(&a.agg_w[slot], tag, TW, a.lb_local);
            }
            float cin = 0.0f;
            if (j < a.nT - 1) {
                // look-back over the later tiles, nearest first (acc composes
                // tiles j+1 .. p-1), LB tiles per batch of loads; a walk that
                // passes the last tile ends there (w = 0 beyond the end)
                constexpr int LB = MGS_ELEM_LB;
                float accP = 1.0f, accW = 0.0f, basev = 0.0f;
                int p0 = j + 1;
                const uint32_t want = sTicket[1], limit = sTicket[2];
                for (uint32_t spin = 0;;) {
                    uint64_t wi[LB], wp[LB], ww[LB];
#pragma unroll
                    for (int u = 0; u < LB; ++u) {
                        const int p = p0 + u;
                        const size_t ps = (static_cast<size_t>(p < a.nT ? p : a.nT - 1) * a.nCG + cg) * CHW + ch;
                        wi[u] = tagged_load(&a.incl[ps]);
                        wp[u] = tagged_load(&a.agg_p[ps]);
                        ww[u] = tagged_load(&a.agg_w[ps]);
                    }
                    bool done = false, stop = false;
                    int adv = 0;
#pragma unroll
                    for (int u = 0; u < LB; ++u) {
                        const int p = p0 + u;
                        if (stop) continue;
                        if (p >= a.nT) {
                            done = stop = true;          // past the last tile: base is 0
                        } else if (tag_is(wi[u], want)) {
                            basev = tag_value(wi[u]);
                            done = stop = true;
                        } else if (tag_is(wp[u], want) && tag_is(ww[u], want)) {
                            accW = accW + accP * tag_value(ww[u]);
                            accP = accP * tag_value(wp[u]);
                            adv = u + 1;
                        } else {
                            stop = true;
                        }
                    }
                    if (done) break;
                    p0 += adv;
                    if (adv == 0) {
                        if (++spin >= limit) {
                            raise_error(&a.hd->err, kErrSpin);
                            break;
                        }
                        backoff();
                    }
                }
                cin = accW + accP * basev;
            }
            if (j > 0) tagged_store(&a.incl[slot], tag, TW + TP * cin, a.lb_local);
            sCarry[ch] = cin;
        }
        __syncthreads();
        wcarry = sCarry[ch];
    } else {
        wcarry = 0.0f;
    }

    // state entering this chunk (forward) and w entering it from the right.
    // These stay per-lane folds of linear maps: storing composed prefixes in
    // wave 0's fold, ahead of its look-back, cost the backward more (log
    // space, long T: +0.15-0.3 us) than the folds take.
    float hc = hin;
    for (int p = 0; p < q; ++p) hc = sA[p][ch] * hc + sH[p][ch];
    float wc = wcarry;
    for (int p = NCH - 1; p > q; --p) wc = sW[p][ch] + sP[p][ch] * wc;

#pragma unroll
    for (int i = C - 1; i >= 0; --i) {
        const float hprev = (i == 0) ? hc : pA[i - 1] * hc + pH[i - 1];
        const float g = gv[i] + wc;
        const float ag = av[i] * g;
        wc = ag;
        const int t = t0 + i;
        if (cv && t < a.T) {
            const int64_t off = base + static_cast<int64_t>(t) * a.d;
            float d1, d2;
            Alg::grads(r1[i], r2[i], av[i], bv[i], g, hprev, d1, d2);
            store_out(&a.dla[off], d1);
            store_out(&a.dlb[off], d2);
        }
    }
    if (cv && j == 0 && q == 0) store_out(&a.dlh0[chain], Alg::grad_h0(wc, hin, lh0v));   // from a_1 g_1
}

// ------------------------------------------------------------ host side

// Tile geometry.  Sequences that fit one tile (T <= 128) use 32 chains per
// wave row and 4 waves, which gives the most workgroups at the lab shape;
// longer sequences use 64 chains per row, 8 waves and up to 16 steps per lane
// (fewer, larger tiles along T, hence shorter look-back walks).  Chosen from
// measured sweeps over chains per row {32, 64}, waves {2, 4, 8, 16} and steps
// per lane {8, 16}; the macros below let a build try other shapes.
#ifndef MGS_LOG_SHORT_T
#define MGS_LOG_SHORT_T 128
#endif
#ifndef MGS_SHORT_CHW
#define MGS_SHORT_CHW 32
#endif
#ifndef MGS_SHORT_W
#define MGS_SHORT_W 4
#endif
#ifndef MGS_LONG_CHW
#define MGS_LONG_CHW 64
#endif
#ifndef MGS_LONG_W
#define MGS_LONG_W 8
#endif
#ifndef MGS_LONG_MAXC
#define MGS_LONG_MAXC 16
#endif
constexpr int kShortT = MGS_LOG_SHORT_T;
constexpr int kShortChw = MGS_SHORT_CHW, kShortW = MGS_SHORT_W;
constexpr int kLongChw = MGS_LONG_CHW, kLongW = MGS_LONG_W;
constexpr int kMaxC = 16;
constexpr int kLongMaxC = MGS_LONG_MAXC;

template <class Alg, int CHW, int W, int C>
hipError_t launch_fwd_c(const LogGeom &g, const LogFwdArgs &args, hipStream_t s)
{
    const dim3 grid(g.nTiles), block(64 * W);
    if (g.nT > 1)
        hipLaunchKernelGGL((elem_fwd_kernel<Alg, CHW, C, W, true>), grid, block, 0, s, args);
    else
        hipLaunchKernelGGL((elem_fwd_kernel<Alg, CHW, C, W, false>), grid, block, 0, s, args);
    return hipGetLastError();
}

template <class Alg, int CHW, int W, int C>
hipError_t launch_bwd_c(const LogGeom &g, const LogBwdArgs &args, hipStream_t s)
{
    const dim3 grid(g.nTiles), block(64 * W);
    if (g.nT > 1)
        hipLaunchKernelGGL((elem_bwd_kernel<Alg, CHW, C, W, true>), grid, block, 0, s, args);
    else
        hipLaunchKernelGGL((elem_bwd_kernel<Alg, CHW, C, W, false>), grid, block, 0, s, args);
    return hipGetLastError();
}

#define MGS_ELEM_DISPATCH(FN, ALG, g, a, s)                                                       \
    do {                                                                                          \
        if ((g).CHW == kShortChw && (g).W == kShortW) {                                           \
            switch ((g).C) {                                                                      \
            case 1: return FN<ALG, kShortChw, kShortW, 1>(g, a, s);                               \
            case 2: return FN<ALG, kShortChw, kShortW, 2>(g, a, s);                               \
            case 4: return FN<ALG, kShortChw, kShortW, 4>(g, a, s);                               \
            case 8: return FN<ALG, kShortChw, kShortW, 8>(g, a, s);                               \
            default: return FN<ALG, kShortChw, kShortW, 16>(g, a, s);                             \
            }                                                                                     \
        }                                                                                         \
        switch ((g).C) {                                                                          \
        case 1: return FN<ALG, kLongChw, kLongW, 1>(g, a, s);                                     \
        case 2: return FN<ALG, kLongChw, kLongW, 2>(g, a, s);                                     \
        case 4: return FN<ALG, kLongChw, kLongW, 4>(g, a, s);                                     \
        case 8: return FN<ALG, kLongChw, kLongW, 8>(g, a, s);                                     \
        default: return FN<ALG, kLongChw, kLongW, 16>(g, a, s);                                   \
        }                                                                                         \
    } while (0)

LogFwdArgs fwd_args(const LogGeom &g, const float *x1, const float *x2, const float *x0, float *h,
                    void *ws)
{
    char *w = static_cast<char *>(ws);
    LogFwdArgs a{};
    a.la = x1; a.lb = x2; a.lh0 = x0; a.h = h;
    a.S = g.S; a.T = g.T; a.d = g.d; a.nCG = g.nCG; a.nT = g.nT; a.nTiles = g.nTiles;
    a.hd = reinterpret_cast<WsHeader *>(w);
    a.lb_local = lookback_on_one_xcd(g.nCG);
    if (g.nT > 1) {
        a.agg_a = reinterpret_cast<uint64_t *>(w + g.off_fagg_a);
        a.agg_h = reinterpret_cast<uint64_t *>(w + g.off_fagg_h);
        a.incl = reinterpret_cast<uint64_t *>(w + g.off_fincl);
        a.carry = reinterpret_cast<float *>(w + g.off_carry);
    }
    return a;
}

LogBwdArgs bwd_args(const LogGeom &g, const float *x1, const float *x2, const float *x0,
                    const float *dh, float *d1, float *d2, float *d0, void *ws)
{
    char *w = static_cast<char *>(ws);
    LogBwdArgs a{};
    a.la = x1; a.lb = x2; a.lh0 = x0; a.dh = dh;
    a.dla = d1; a.dlb = d2; a.dlh0 = d0;
    a.S = g.S; a.T = g.T; a.d = g.d; a.nCG = g.nCG; a.nT = g.nT; a.nTiles = g.nTiles;
    a.hd = reinterpret_cast<WsHeader *>(w);
    a.lb_local = lookback_on_one_xcd(g.nCG);
    if (g.nT > 1) {
        a.agg_p = reinterpret_cast<uint64_t *>(w + g.off_bagg_p);
        a.agg_w = reinterpret_cast<uint64_t *>(w + g.off_bagg_w);
        a.incl = reinterpret_cast<uint64_t *>(w + g.off_bincl);
        a.carry = reinterpret_cast<const float *>(w + g.off_carry);
    }
    return a;
}

}  // namespace

LogGeom log_geometry(int64_t B, int64_t T, int64_t d)
{
    LogGeom g{};
    g.S = B * d;
    g.T = static_cast<int>(T);
    g.d = static_cast<int>(d);
    const bool short_t = T <= kShortT;
    g.CHW = short_t ? kShortChw : kLongChw;
    g.W = short_t ? kShortW : kLongW;
    const int nch = g.W * (64 / g.CHW);
    const int maxc = short_t ? kMaxC : kLongMaxC;
    int C = 1;
    while (C < maxc && static_cast<int64_t>(nch) * C < T) C *= 2;
    g.C = C;
    g.TT = nch * C;
    g.nT = static_cast<int>((T + g.TT - 1) / g.TT);
    g.nCG = static_cast<int>((g.S + g.CHW - 1) / g.CHW);
    g.nTiles = g.nT * g.nCG;
    const size_t slots = static_cast<size_t>(g.nTiles) * g.CHW;
    size_t off = sizeof(WsHeader);
    if (g.nT > 1) {
        g.off_fagg_a = off; off = align256(off + slots * 8);
        g.off_fagg_h = off; off = align256(off + slots * 8);
        g.off_fincl = off;  off = align256(off + slots * 8);
        g.off_carry = off;  off = align256(off + slots * 4);
        g.off_bagg_p = off; off = align256(off + slots * 8);
        g.off_bagg_w = off; off = align256(off + slots * 8);
        g.off_bincl = off;  off = align256(off + slots * 8);
    }
    g.bytes = off;
    return g;
}

hipError_t launch_log_fwd(const LogGeom &g, const float *la, const float *lb, const float *lh0,
                          float *h, void *ws, hipStream_t s)
{
    const LogFwdArgs a = fwd_args(g, la, lb, lh0, h, ws);
    MGS_ELEM_DISPATCH(launch_fwd_c, LogAlg, g, a, s);
}

hipError_t launch_log_bwd(const LogGeom &g, const float *la, const float *lb, const float *lh0,
                          const float *dh, float *dla, float *dlb, float *dlh0, void *ws,
                          hipStream_t s)
{
    const LogBwdArgs a = bwd_args(g, la, lb, lh0, dh, dla, dlb, dlh0, ws);
    MGS_ELEM_DISPATCH(launch_bwd_c, LogAlg, g, a, s);
}

hipError_t launch_mingru_fwd(const LogGeom &g, const float *k, const float *x, const float *x0,
                             float *h, void *ws, hipStream_t s)
{
    const LogFwdArgs a = fwd_args(g, k, x, x0, h, ws);
    MGS_ELEM_DISPATCH(launch_fwd_c, GateAlg, g, a, s);
}

hipError_t launch_mingru_bwd(const LogGeom &g, const float *k, const float *x, const float *x0,
                             const float *dh, float *dk, float *dx, float *dx0, void *ws,
                             hipStream_t s)
{
    const LogBwdArgs a = bwd_args(g, k, x, x0, dh, dk, dx, dx0, ws);
    MGS_ELEM_DISPATCH(launch_bwd_c, GateAlg, g, a, s);
}

hipError_t launch_linear_fwd(const LogGeom &g, const float *a_, const float *b, const float *h0,
                             float *h, void *ws, hipStream_t s)
{
    const LogFwdArgs a = fwd_args(g, a_, b, h0, h, ws);
    MGS_ELEM_DISPATCH(launch_fwd_c, LinAlg, g, a, s);
}

hipError_t launch_linear_bwd(const LogGeom &g, const float *a_, const float *b, const float *h0,
                             const float *dh, float *da, float *db, float *dh0, void *ws,
                             hipStream_t s)
{
    const LogBwdArgs a = bwd_args(g, a_, b, h0, dh, da, db, dh0, ws);
    MGS_ELEM_DISPATCH(launch_bwd_c, LinAlg, g, a, s);
}

}  // namespace mgs
