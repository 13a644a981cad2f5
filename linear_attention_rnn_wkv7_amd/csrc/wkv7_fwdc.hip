// WKV7 forward for N = 64: a serial scan on four waves beside eight waves
// that prepare its inputs and compute its outputs on the matrix cores.
//
// The recurrence is rx_wkv7_forward_seq on the Foundry "rwkvx/rx_pretrain.c"
// page: sa = S a;  S <- S diag(w) + v k^T + sa b^T;  y = S r.  Per block of
// 32 steps, with g_t the product of w over the block up to t (per column),
// the rescaled state St = S diag(1/g_t) obeys
//   St_t = St_{t-1} + v_t kt_t^T + sa_t bt_t^T,   kt = k / g_t, bt = b / g_t,
//   sa_t = St_{t-1} ab_t,                         ab = a g_{t-1}.
// Writing St_t = Sh_t + sum_{u<=t} v_u kt_u^T, the serial part only carries
//   sa_t = Sh_{t-1} ab_t + c_t,   Sh_t = Sh_{t-1} + sa_t bt_t^T,
//   c_t  = sum_{u<t} v_u (kt_u . ab_t),
// two FMAs per state element and step, and the block ends with
//   S = (Sh_31 + sum_u v_u kt_u^T) diag(g_31).
// The outputs have the closed form
//   y_t = S0 rb_t + sum_{u<=t} v_u (kt_u . rb_t) + sa_u (bt_u . rb_t),  rb = r g_t,
// with S0 the state before the block.  c, sum_u v_u kt_u^T and y are dense
// products, done with v_mfma_f32_16x16x4f32.
//
// One workgroup of twelve waves per (b, h).  Waves 0-3 run the steps of
// block q (wave w: rows 16 w .. 16 w + 15 of S, 2 rows x 8 columns per
// lane).  Waves 4-11 ("helpers", eight of them, two per SIMD beside one scan
// wave) meanwhile copy block q + 1 into LDS, rescale it and compute its Gram
// tiles, c and sum of v kt^T; they also finish y of block q - 1 (which needs
// its sa) and start y of block q (which needs S0), and write the sa tape and
// the checkpoints.  The helpers synchronise among themselves through an LDS
// arrival counter, and with the scan waves twice per block (X: the block's
// steps are done; Y: the state after the block is in LDS).  Blocks whose
// decays leave [1/16, 1] or whose cumulative decay drops below 2^-60, and a
// final partial block, run the plain step on the scan waves instead (y on
// the VALU, no rescaling).  With fused inputs the w, a, b slots hold the
// decay pre-activation omega, the normalised key kk and the gate ag of the
// page's tm_pre_forward; the kernel forms w = exp(-c sigmoid(omega)),
// a = -kk and b = kk ag where it first reads them (the decay's cumulative
// product, the rescaling pass, the plain steps).  Checkpoints must fall on
// block starts (chunk a multiple of 32).

#include <atomic>
#include <type_traits>

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kTB = 32;                    // steps per block
constexpr float kWMinF = 0.0625f;          // smallest decay of a rescaled block
constexpr float kGMinF = 8.67361738e-19f;  // 2^-60: smallest cumulative decay
constexpr unsigned kSpinMax = 1u << 20;    // bound on one helper wait (polls)
constexpr int kNH = 8;                     // helper waves
constexpr int kThreads = 64 * (4 + kNH);

__device__ __forceinline__ f4 mfma(float a, float b, f4 c)
{
    // D[m][n] += A[m][k] B[k][n] over a 16x16x4 block: lane l supplies
    // A[l % 16][l / 16] and B[l / 16][l % 16] and holds D[4 (l / 16) + i][l % 16].
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Row-major [rows][64] fp32 LDS arrays with the 16-byte groups of each row
// XOR-swizzled by the row, so that rows and 16-row column slices both read
// without bank conflicts.
__device__ __forceinline__ int sw(int t, int j)
{
    return (t << 6) + ((((j >> 2) ^ (t & 15))) << 2) + (j & 3);
}

__device__ __forceinline__ float4 lds4(const float *s, int o)
{
    return *reinterpret_cast<const float4 *>(s + o);
}

__device__ __forceinline__ void put4(float *s, int o, float4 v)
{
    *reinterpret_cast<float4 *>(s + o) = v;
}

// x of the lane in row group g ^ 1 (lane bit 4) and g ^ 2 (lane bit 5)
__device__ __forceinline__ float xor16(float x, int g)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __builtin_bit_cast(float, (g & 1) ? p[0] : p[1]);
}
__device__ __forceinline__ float xor32(float x, int g)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (g & 2) ? p[0] : p[1]);
}

// input slots of a block; a rescaled block holds rb, kt, v, ab, bt there and
// c in the slot of w
enum { vR = 0, vW = 1, vK = 2, vV = 3, vA = 4, vB = 5 };

template <typename TIn>
struct FwdcArgs {
    const TIn *in[6];        // r, w, k, v, a, b
    const float *s0;
    float *y, *sT, *ckpt, *sa;
    int64_t T, H;
    int chunk, nck;
    // sequence split (segments of nckseg checkpoint intervals): mode 0 runs
    // whole (b, h) sequences; mode 1 runs, per (b, h), the segments
    // s = 0 .. nseg - 2 from zero (s0 for s = 0) to their end state Q_s
    // (into the checkpoint at the next segment's start), then s = 1 .. nseg - 2
    // with v = 0 from the identity, giving the segment's transition product
    // P_s (into pbuf), and writes nothing else; mode 2 runs every segment
    // from its carry-in state (the checkpoint at its start) with all outputs.
    // Without a checkpoint record the carries live in y instead, in rows of
    // (b, h) that segment s overwrites itself: steps 0 .. 63 of segment s
    // hold its carry-in state (Q_{s-1}, then S_in(s)), steps 64 .. 127 its
    // P_s; every segment but the last spans at least 128 steps and the last
    // at least 64.  A unit reads its carry-in state before any y store.
    int mode, nseg, nckseg;
    float *pbuf;   // [B*H][nseg][64][64]; null when the carries live in y
    // A helper wait that gives up (see hsync) makes the workgroup overwrite
    // every output it wrote with NaN and set bit 0 of *fault.  inject != 0
    // (a test hook) reports a given-up wait in every workgroup while all
    // waits still complete normally.
    unsigned *fault;
    int inject;
};

// kLite: units that write no y (the split's first pass), which need
// neither the y Gram tiles nor, with v = 0, c and sum v kt^T
template <typename TIn, bool kFused, bool kLite>
__global__ void __launch_bounds__(kThreads) wkv7_fwdc_kernel(FwdcArgs<TIn> p)
{
    constexpr int N = 64, R = 2, CC = 8, LPR = 8;
    __shared__ __align__(16) float slot[2][6][kTB * N];  // block inputs, by q & 1
    __shared__ __align__(16) float gram[12][256];        // Gram tiles, lane-linear
    __shared__ __align__(16) float vkt[N * N];           // sum_u v_u kt_u^T, transposed
    __shared__ __align__(16) float sap[2][kTB * N];      // sa of the block, by q & 1
    __shared__ __align__(16) float sS0[N * N];           // state before the block
    __shared__ __align__(16) float g31[2][N];            // g_31 of the block
    __shared__ int smode[2];                             // 1: block rescaled
    __shared__ int hbad[2];                              // a decay out of range
    __shared__ unsigned hcnt;                            // helper arrivals
    __shared__ int hfault;                               // a helper wait gave up

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t H = p.H;
    // this workgroup's (b, h) and steps [tb0, tb0 + T) of its sequence, its
    // initial state (s0u; or the identity), where its final state goes, and
    // whether it writes y, the sa tape and the checkpoints
    int64_t bh = blockIdx.x, tb0 = 0, T = p.T;
    const float *s0u = p.s0 ? p.s0 + bh * N * N : nullptr;
    float *sTu = p.sT ? p.sT + bh * N * N : nullptr;
    int64_t s0ld = N, sTld = N;   // row strides of the two states
    bool s0_eye = false, zero_v = false, outs = true;
    if (p.mode != 0) {
        const int64_t Tseg = (int64_t)p.nckseg * p.chunk;
        const bool in_y = p.ckpt == nullptr;   // the carries live in y
        // row `row` of segment s's part of the sequence of (b, h) in y
        auto yrow = [&](int s, int row) {
            return p.y + ((bh / H) * p.T * H + bh % H) * N + ((int64_t)s * Tseg + row) * H * N;
        };
        int seg;
        if (p.mode == 1) {
            const int per = 2 * p.nseg - 3, k = (int)((int64_t)blockIdx.x % per);
            bh = (int64_t)blockIdx.x / per;
            outs = false;
            if (k < p.nseg - 1) {   // Q_s
                seg = k;
                s0u = seg == 0 && p.s0 ? p.s0 + bh * N * N : nullptr;
                sTu = in_y ? yrow(seg + 1, 0) : p.ckpt + (bh * p.nck + (int64_t)(seg + 1) * p.nckseg) * N * N;
            } else {                // P_s
                seg = k - (p.nseg - 1) + 1;
                s0u = nullptr;
                s0_eye = zero_v = true;
                sTu = in_y ? yrow(seg, N) : p.pbuf + (bh * p.nseg + seg) * N * N;
            }
            if (in_y) sTld = H * N;
        } else {
            bh = (int64_t)blockIdx.x / p.nseg;
            seg = (int)((int64_t)blockIdx.x % p.nseg);
            if (seg == 0) {
                s0u = p.s0 ? p.s0 + bh * N * N : nullptr;
            } else if (in_y) {
                s0u = yrow(seg, 0);
                s0ld = H * N;
            } else {
                s0u = p.ckpt + (bh * p.nck + (int64_t)seg * p.nckseg) * N * N;
            }
            sTu = seg == p.nseg - 1 && p.sT ? p.sT + bh * N * N : nullptr;
        }
        tb0 = seg * Tseg;
        T = p.T - tb0 < Tseg ? p.T - tb0 : Tseg;
    }
    float *const yp = outs ? p.y : nullptr;
    const int64_t bidx = bh / H, head = bh % H;
    const int64_t stride = H * N;
    const int64_t vbase = (bidx * p.T * H + head) * N + tb0 * stride;
    const int64_t nblk = (T + kTB - 1) / kTB;
    auto steps_of = [&](int64_t blk) -> int {
        const int64_t rem = T - blk * kTB;
        return (int)(rem < kTB ? rem : kTB);
    };

    // Every wave ends here once.  If a helper wait gave up, the LDS data of
    // some block may have been read before it was complete: overwrite every
    // output of this unit with NaN (y rows, sa tape rows, checkpoint slots,
    // the final state or carry) and report it, so that no finite wrong
    // value is left behind.
    auto finish = [&]() {
        __syncthreads();
        if (!hfault) return;
        const float nan = __builtin_nanf("");
        const int64_t n = T * N;
        if (outs && p.y)
            for (int64_t i = tid; i < n; i += kThreads) p.y[vbase + (i >> 6) * stride + (i & 63)] = nan;
        if (outs && p.sa)
            for (int64_t i = tid; i < n; i += kThreads) p.sa[vbase + (i >> 6) * stride + (i & 63)] = nan;
        if (outs && p.ckpt)
            for (int64_t c = (tb0 + p.chunk - 1) / p.chunk; c * p.chunk < tb0 + T; ++c)
                for (int i = tid; i < N * N; i += kThreads) p.ckpt[(bh * p.nck + c) * N * N + i] = nan;
        if (sTu)
            for (int i = tid; i < N * N; i += kThreads) sTu[(i >> 6) * sTld + (i & 63)] = nan;
        if (tid == 0) __hip_atomic_fetch_or(p.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    if (tid == 0) {
        smode[0] = smode[1] = 0;
        hbad[0] = hbad[1] = 0;
        hcnt = 0;
        hfault = p.inject != 0;
    }
    if (zero_v)   // v is never staged: both slots read zeros
        for (int i = tid; i < 2 * kTB * N; i += kThreads) slot[i / (kTB * N)][vV][i % (kTB * N)] = 0.f;
    __syncthreads();

    if (wave < 4) {
        // ================= scan waves =================
        const int cg = lane % LPR, rg = lane / LPR;
        const int row0 = wave * 16 + rg * R, col0 = cg * CC;

        float S[R][CC];
        if (s0_eye) {
#pragma unroll
            for (int e = 0; e < R; ++e)
#pragma unroll
                for (int c = 0; c < CC; ++c) S[e][c] = row0 + e == col0 + c ? 1.f : 0.f;
        } else if (s0u) {
            const float *src = s0u + row0 * s0ld + col0;
#pragma unroll
            for (int e = 0; e < R; ++e)
#pragma unroll
                for (int c = 0; c < CC; c += 4) {
                    const float4 q = *reinterpret_cast<const float4 *>(src + e * s0ld + c);
                    S[e][c] = q.x; S[e][c + 1] = q.y; S[e][c + 2] = q.z; S[e][c + 3] = q.w;
                }
        } else {
#pragma unroll
            for (int e = 0; e < R; ++e)
#pragma unroll
                for (int c = 0; c < CC; ++c) S[e][c] = 0.f;
        }
        auto row8 = [&](const float *s, int t, float (&o)[CC]) {
            const float4 x0 = lds4(s, sw(t, col0)), x1 = lds4(s, sw(t, col0 + 4));
            o[0] = x0.x; o[1] = x0.y; o[2] = x0.z; o[3] = x0.w;
            o[4] = x1.x; o[5] = x1.y; o[6] = x1.z; o[7] = x1.w;
        };
        auto put_state = [&]() {
#pragma unroll
            for (int e = 0; e < R; ++e) {
                put4(sS0, sw(row0 + e, col0), make_float4(S[e][0], S[e][1], S[e][2], S[e][3]));
                put4(sS0, sw(row0 + e, col0 + 4), make_float4(S[e][4], S[e][5], S[e][6], S[e][7]));
            }
        };
        // one value per row, from the lanes cg < R
        auto park = [&](float *base_row_t, const float (&x)[R]) {
            float val = x[0];
#pragma unroll
            for (int e = 1; e < R; ++e)
                if (cg == e) val = x[e];
            if (cg < R) *base_row_t = val;
        };

        put_state();
        __syncthreads();   // block 0 ready, S0 in LDS

        for (int64_t q = 0; q < nblk; ++q) {
            const int bb = (int)(q & 1);
            const int nst = steps_of(q);
            const int64_t t0 = q * kTB;
            float *SA = sap[bb];
            if (__builtin_amdgcn_readfirstlane(smode[bb])) {
                // ---- rescaled steps: sa = Sh ab + c, Sh += sa bt^T
                const float *La = slot[bb][vA], *Lb = slot[bb][vB], *Lc = slot[bb][vW];
                struct Ops {
                    float ab[CC], bt[CC];
                    float2 c;
                };
                auto load_ops = [&](int s, Ops &o) {
                    row8(La, s, o.ab);
                    row8(Lb, s, o.bt);
                    o.c = *reinterpret_cast<const float2 *>(Lc + sw(s, row0));
                };
                // operands one step ahead
                Ops ops[2];
                load_ops(0, ops[0]);
#pragma unroll
                for (int s = 0; s < kTB; ++s) {
                    if (s + 1 < kTB) load_ops(s + 1, ops[(s + 1) & 1]);
                    const Ops &o = ops[s & 1];
                    float sa[R];
#pragma unroll
                    for (int e = 0; e < R; ++e) {
                        float a0 = 0.f, a1 = 0.f;
#pragma unroll
                        for (int c = 0; c < CC; c += 2) {
                            a0 = fmaf(S[e][c], o.ab[c], a0);
                            a1 = fmaf(S[e][c + 1], o.ab[c + 1], a1);
                        }
                        sa[e] = group_allreduce<LPR>(a0 + a1) + (e == 0 ? o.c.x : o.c.y);
                    }
#pragma unroll
                    for (int e = 0; e < R; ++e)
#pragma unroll
                        for (int c = 0; c < CC; ++c) S[e][c] = fmaf(sa[e], o.bt[c], S[e][c]);
                    park(&SA[sw(s, row0 + cg)], sa);
                }
                __syncthreads();   // X: steps done; sum v kt^T is in LDS
                float gr[CC];
                {
                    const float4 x0 = lds4(g31[bb], col0), x1 = lds4(g31[bb], col0 + 4);
                    gr[0] = x0.x; gr[1] = x0.y; gr[2] = x0.z; gr[3] = x0.w;
                    gr[4] = x1.x; gr[5] = x1.y; gr[6] = x1.z; gr[7] = x1.w;
                }
#pragma unroll
                for (int c = 0; c < CC; ++c) {
                    // stored transposed: row col0 + c, columns row0, row0 + 1
                    const float2 vk = *reinterpret_cast<const float2 *>(vkt + sw(col0 + c, row0));
                    S[0][c] = (S[0][c] + vk.x) * gr[c];
                    S[1][c] = (S[1][c] + vk.y) * gr[c];
                }
            } else {
                // ---- plain steps (y on the VALU) from the block's raw inputs
                const float *L = &slot[bb][0][0];
                for (int s = 0; s < nst; ++s) {
                    float av[CC], wv[CC], kv[CC], bv[CC], rv[CC];
                    row8(L + vA * kTB * N, s, av);
                    row8(L + vW * kTB * N, s, wv);
                    row8(L + vK * kTB * N, s, kv);
                    row8(L + vB * kTB * N, s, bv);
                    row8(L + vR * kTB * N, s, rv);
                    if constexpr (kFused) {   // av: kk, bv: gate, wv: omega
#pragma unroll
                        for (int c = 0; c < CC; ++c) {
                            bv[c] = av[c] * bv[c];
                            av[c] = -av[c];
                            wv[c] = decay_from_pre(wv[c]);
                        }
                    }
                    float sa[R], yv[R];
#pragma unroll
                    for (int e = 0; e < R; ++e) {
                        float a0 = 0.f, a1 = 0.f;
#pragma unroll
                        for (int c = 0; c < CC; c += 2) {
                            a0 = fmaf(S[e][c], av[c], a0);
                            a1 = fmaf(S[e][c + 1], av[c + 1], a1);
                        }
                        const float ve = L[vV * kTB * N + sw(s, row0 + e)];
                        float u[CC];
#pragma unroll
                        for (int c = 0; c < CC; ++c) u[c] = fmaf(S[e][c], wv[c], ve * kv[c]);
                        sa[e] = group_allreduce<LPR>(a0 + a1);
                        float y0 = 0.f, y1 = 0.f;
#pragma unroll
                        for (int c = 0; c < CC; c += 2) {
                            S[e][c] = fmaf(sa[e], bv[c], u[c]);
                            S[e][c + 1] = fmaf(sa[e], bv[c + 1], u[c + 1]);
                            y0 = fmaf(S[e][c], rv[c], y0);
                            y1 = fmaf(S[e][c + 1], rv[c + 1], y1);
                        }
                        yv[e] = group_allreduce<LPR>(y0 + y1);
                    }
                    park(&SA[sw(s, row0 + cg)], sa);
                    if (yp && cg < R) yp[vbase + (t0 + s) * stride + row0 + cg] = cg == 0 ? yv[0] : yv[1];
                }
                __syncthreads();   // X
            }
            put_state();           // the state before block q + 1
            __syncthreads();       // Y
        }
        if (sTu) {
            float *dst = sTu + row0 * sTld + col0;
#pragma unroll
            for (int e = 0; e < R; ++e)
#pragma unroll
                for (int c = 0; c < CC; c += 4)
                    *reinterpret_cast<float4 *>(dst + e * sTld + c) =
                        make_float4(S[e][c], S[e][c + 1], S[e][c + 2], S[e][c + 3]);
        }
        finish();
        return;
    }

    // ================= helper waves =================
    // The helper code is instantiated per helper wave (its index h a
    // compile-time constant), and every LDS address is one of a few per-lane
    // offsets plus a constant, so that the helpers spend their issue slots
    // on loads, stores and MFMAs rather than on address arithmetic.
    const int l16 = lane & 15, g = lane >> 4, qa = l16 >> 2, c3 = l16 & 3;
    const bool want_y = yp != nullptr;
    const TIn *in_ptr[6];
#pragma unroll
    for (int v = 0; v < 6; ++v) in_ptr[v] = p.in[v] + vbase;
    float *const y_out = yp ? yp + vbase : nullptr;
    float *const sa_out = outs && p.sa ? p.sa + vbase : nullptr;
    float *const ck_out = outs ? p.ckpt : nullptr;
    const int chunk = p.chunk, nck = p.nck;
    float *const gbuf = &gram[0][0];   // g of the block being rescaled

    // Wait until all helper waves have arrived here.  Every helper wave
    // runs the same sequence of waits; the poll count is bounded so that a
    // broken sequence cannot hang the kernel, and a wait that gives up is
    // recorded (finish() then poisons this unit's outputs and reports it).
    unsigned htarget = 0;
    auto hsync = [&]() {
        htarget += kNH;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) __hip_atomic_fetch_add(&hcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        bool arrived = false;
        for (unsigned it = 0; it < kSpinMax; ++it) {
            if (__hip_atomic_load(&hcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= htarget) {
                arrived = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (!arrived && lane == 0) hfault = 1;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };

    auto helper = [&](auto hw) {
        constexpr int h = decltype(hw)::value;
        // The y and c tile of this wave: steps 16 tb .. 16 tb + 15 of the
        // block (lane: step 16 tb + 4 g + r), rows 16 ib .. 16 ib + 15 (lane:
        // row 16 ib + l16).  Its part of sum v kt^T: rows 16 ib .., column
        // tiles 2 tb and 2 tb + 1.  The second time block has twice the
        // tiles of the first (u <= t); helpers h and h + 4 share a SIMD and
        // take one of each.
        constexpr int tb = (h ^ (h >> 2)) & 1, ib = h >> 1;

        // ---- lane offsets (floats) into the swizzled [rows][64] arrays:
        //   rows 16 X + l16, columns 16 q4 + 4 g .. + 3    L1[q4] + 1024 X
        //   rows 16 U + 4 g + r, column 16 ib + l16         L2[r] + 1024 U
        //   rows 4 k + g, column 16 I + l16    L3 + 256 k + 16 (I ^ (k & 3))
        int L1[4], L2[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) L1[q4] = 64 * l16 + 16 * (q4 ^ qa) + 4 * (g ^ c3);
#pragma unroll
        for (int r = 0; r < 4; ++r) L2[r] = 256 * g + 64 * r + 16 * (ib ^ g) + 4 * (qa ^ r) + c3;
        const int L3 = 64 * g + 4 * (qa ^ g) + c3;
        // sum v kt^T, stored transposed: row j = 16 jt + l16, columns
        // 16 ib + 4 g .. + 3
        const int Lt = 64 * l16 + 4 * ((4 * ib + g) ^ l16);
        // rescaling by rows: step tr, columns 4 cq .. + 3
        const int tr = 4 * h + (lane >> 4), cq = lane & 15;
        const int Lr = 64 * tr + 4 * (cq ^ (tr & 15));
        const int Lp = tr > 0 ? 64 * (tr - 1) + 4 * (cq ^ ((tr - 1) & 15)) : 0;
        // tape: row 4 h + g, columns 4 l16 .. + 3 (from the row 16 (h / 4))
        const int Lq = 64 * g + 4 * (l16 ^ (4 * (h & 3) + g));
        // global offsets (elements)
        const int Ly = 4 * g * (int)stride + l16;   // y: step 4 g, row l16
        const int Ls = g * (int)stride + 4 * l16;   // tape: step g, column 4 l16
        int Ld[4];                                  // staging: step g, swizzled column
#pragma unroll
        for (int u = 0; u < 4; ++u) Ld[u] = g * (int)stride + 4 * (l16 ^ (4 * u + g));

        // ---- staging of block blk into slot[b]: units of 1 KB (4 steps of
        // one input), 6 per helper wave; fp32 by direct HBM -> LDS copies
        // (lane l of a unit lands at float 4 l: step 4 u + l / 16, swizzled
        // column group l % 16), bf16 through registers (widened)
        constexpr int kU = 48 / kNH;
        constexpr bool kDma = std::is_same<TIn, float>::value;
        using Raw = typename InQuad<TIn>::raw;
        Raw pre[kU];
        auto stage_unit = [&](int64_t t0, int b, int k) {
            const int unit = kU * h + k, v = unit >> 3, u = unit & 7;
            if (zero_v && v == vV) return;
            const TIn *base = in_ptr[v] + (t0 + 4 * u) * stride;
            if constexpr (kDma) {
                const unsigned lds = (unsigned)(uintptr_t)(
                    const __attribute__((address_space(3))) float *)&slot[b][v][u * 256];
                dma16_split(base, 4u * (unsigned)Ld[u & 3], lds);
            } else {
                pre[k] = InQuad<TIn>::load(base + Ld[u & 3]);
            }
        };
        auto stage_issue = [&](int64_t blk, int b) {
            const int nst = steps_of(blk);
            const int64_t t0 = blk * kTB;
            if (nst == kTB) {   // a full block: no per-lane condition
#pragma unroll
                for (int k = 0; k < kU; ++k) stage_unit(t0, b, k);
            } else {
#pragma unroll
                for (int k = 0; k < kU; ++k)
                    if (4 * ((kU * h + k) & 7) + g < nst) stage_unit(t0, b, k);
            }
        };
        auto stage_land = [&](int64_t blk, int b) {
            if constexpr (kDma) {
                wait_dma();
            } else {
                const int nst = steps_of(blk);
#pragma unroll
                for (int k = 0; k < kU; ++k) {
                    const int unit = kU * h + k, v = unit >> 3, u = unit & 7;
                    if ((nst == kTB || 4 * u + g < nst) && !(zero_v && v == vV))
                        put4(&slot[b][v][u * 256], 4 * lane, InQuad<TIn>::f32(pre[k]));
                }
            }
        };

        // ---- rescaling of the staged block in slot[b], in place.  First g,
        // per column, by helpers 0-3: lane (l16, g) owns column 16 h + l16
        // and steps 4 u + g, u = 0 .. 7 (prefix products over each group of
        // four steps by lane exchanges); g goes to the Gram area, free until
        // the Gram tiles.  Then, if every column is in range, r, a, k, b are
        // rescaled by rows (four rows per helper).  Returns whether the block
        // is rescaled (the same in every helper).
        auto prep = [&](int b, int nstn) -> bool {
            float *const sb = &slot[b][0][0];
            if constexpr (h < 4) {
                bool ok = nstn == kTB;
                if (ok) {
                    float wv[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        wv[u] = sb[vW * 2048 + L3 + 256 * u + 16 * (h ^ (u & 3))];
                        if constexpr (kFused) wv[u] = decay_from_pre(wv[u]);
                    }
                    float G = 1.f;   // product over the steps before 4 u
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float x = wv[u], x1 = xor16(x, g);
                        const float pre2 = (g & 1) ? x1 * x : x;   // within the pair
                        const float pair = (g & 1) ? pre2 : x * x1;
                        const float other = xor32(pair, g);        // the other pair
                        const float gt = G * ((g & 2) ? other * pre2 : pre2);
                        G *= pair * other;
                        gbuf[L3 + 256 * u + 16 * (h ^ (u & 3))] = gt;
                        ok = ok && x >= kWMinF && x <= 1.f && gt >= kGMinF;
                    }
                }
                if (!ok) hbad[b] = 1;   // every writer stores 1
            }
            hsync();
            const bool fast = nstn == kTB && __builtin_amdgcn_readfirstlane(hbad[b]) == 0;
            if (fast) {
                float4 gt = lds4(gbuf, Lr), gp = lds4(gbuf, Lp);
                if (h == 0 && tr == 0) gp = make_float4(1.f, 1.f, 1.f, 1.f);
                const float4 x0 = lds4(sb + vR * 2048, Lr), x1 = lds4(sb + vA * 2048, Lr);
                const float4 x2 = lds4(sb + vK * 2048, Lr), x3 = lds4(sb + vB * 2048, Lr);
                const float4 iv = make_float4(__builtin_amdgcn_rcpf(gt.x), __builtin_amdgcn_rcpf(gt.y),
                                              __builtin_amdgcn_rcpf(gt.z), __builtin_amdgcn_rcpf(gt.w));
                put4(sb + vR * 2048, Lr, make_float4(x0.x * gt.x, x0.y * gt.y, x0.z * gt.z, x0.w * gt.w));
                put4(sb + vK * 2048, Lr, make_float4(x2.x * iv.x, x2.y * iv.y, x2.z * iv.z, x2.w * iv.w));
                if constexpr (kFused) {   // x1: kk, x3: gate; a = -kk, b = kk gate
                    put4(sb + vA * 2048, Lr, make_float4(-x1.x * gp.x, -x1.y * gp.y, -x1.z * gp.z, -x1.w * gp.w));
                    put4(sb + vB * 2048, Lr, make_float4(x1.x * x3.x * iv.x, x1.y * x3.y * iv.y,
                                                         x1.z * x3.z * iv.z, x1.w * x3.w * iv.w));
                } else {
                    put4(sb + vA * 2048, Lr, make_float4(x1.x * gp.x, x1.y * gp.y, x1.z * gp.z, x1.w * gp.w));
                    put4(sb + vB * 2048, Lr, make_float4(x3.x * iv.x, x3.y * iv.y, x3.z * iv.z, x3.w * iv.w));
                }
                if (h == kNH - 1 && tr == kTB - 1) put4(g31[b], 4 * cq, gt);
            }
            return fast;
        };

        // ---- Gram tile n: kind n / 3 (0: kt . ab with u < t, 1: kt . rb,
        // 2: bt . rb, both u <= t), position n % 3 = (u-block, t-block)
        // (0,0), (0,1), (1,1); D[u][t] in the accumulator layout, stored
        // lane-linear.  Helper h computes tile h, and helpers 4 .. 7 (one
        // per SIMD) each a quarter of tile 8's sum over the 64 columns, into
        // slots 8 .. 11, added where tile 8 is read.
        auto gram_tile = [&](const float *sb, auto nc) {
            constexpr int n = decltype(nc)::value, kind = n / 3, pos = n % 3;
            constexpr int ub = pos == 2 ? 1 : 0, tn = pos == 0 ? 0 : 1;
            constexpr int xo = (kind == 2 ? vB : vK) * 2048 + 1024 * ub;
            constexpr int zo = (kind == 0 ? vA : vR) * 2048 + 1024 * tn;
            float4 xq[4], zq[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                xq[q4] = lds4(sb + xo, L1[q4]);
                zq[q4] = lds4(sb + zo, L1[q4]);
            }
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                acc = mfma(xq[q4].x, zq[q4].x, acc);
                acc = mfma(xq[q4].y, zq[q4].y, acc);
                acc = mfma(xq[q4].z, zq[q4].z, acc);
                acc = mfma(xq[q4].w, zq[q4].w, acc);
            }
            if constexpr (pos != 1) {   // a diagonal tile
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = 4 * g + r - l16;   // u - t within the tile
                    if (kind == 0 ? d >= 0 : d > 0) acc[r] = 0.f;
                }
            }
            *reinterpret_cast<f4 *>(&gram[n][4 * lane]) = acc;
        };
        // quarter h - 4 of tile 8 (bt . rb, u <= t, position (1,1)): columns
        // 16 (h - 4) .. + 15
        auto gram_quarter = [&](const float *sb) {
            constexpr int q4 = h - 4;
            const float4 xq = lds4(sb + vB * 2048 + 1024, L1[q4]);
            const float4 zq = lds4(sb + vR * 2048 + 1024, L1[q4]);
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma(xq.x, zq.x, acc);
            acc = mfma(xq.y, zq.y, acc);
            acc = mfma(xq.z, zq.z, acc);
            acc = mfma(xq.w, zq.w, acc);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r - l16 > 0) acc[r] = 0.f;
            *reinterpret_cast<f4 *>(&gram[8 + q4][4 * lane]) = acc;
        };
        auto grams = [&](const float *sb) {
            gram_tile(sb, std::integral_constant<int, h>{});
            if constexpr (h >= 4) gram_quarter(sb);
        };
        auto gram_get = [&](int kind, int ub) -> f4 {
            const int pos = tb == 0 ? 0 : 1 + ub;
            if (3 * kind + pos != 8) return *reinterpret_cast<const f4 *>(&gram[3 * kind + pos][4 * lane]);
            f4 sum = *reinterpret_cast<const f4 *>(&gram[8][4 * lane]);
#pragma unroll
            for (int k = 9; k < 12; ++k) sum += *reinterpret_cast<const f4 *>(&gram[k][4 * lane]);
            return sum;
        };

        f4 Y, Yv, VK[2], PbA[2], PbB[2], PbC[2];
        bool fastA = false, fastB = false;   // blocks q - 1 and q
        Y = Yv = VK[0] = VK[1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 2; ++m) PbA[m] = PbB[m] = PbC[m] = f4{0.f, 0.f, 0.f, 0.f};

        // y of a block from its S0: Y = Yv + S0 rb_t
        auto y_from_s0 = [&](int b) {
            const float *xs = &slot[b][vR][1024 * tb];
            float4 xr[4], sr[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                xr[q4] = lds4(xs, L1[q4]);
                sr[q4] = lds4(sS0 + 1024 * ib, L1[q4]);
            }
            Y = Yv;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                Y = mfma(xr[q4].x, sr[q4].x, Y);
                Y = mfma(xr[q4].y, sr[q4].y, Y);
                Y = mfma(xr[q4].z, sr[q4].z, Y);
                Y = mfma(xr[q4].w, sr[q4].w, Y);
            }
        };
        // the sa terms of the block whose sa is in sap[b]:
        // Y += sum_u (bt_u . rb_t) sa_u
        auto y_from_sa = [&](int b) {
            float sv[2][4];
#pragma unroll
            for (int ub = 0; ub <= tb; ++ub)
#pragma unroll
                for (int r = 0; r < 4; ++r) sv[ub][r] = sap[b][1024 * ub + L2[r]];
#pragma unroll
            for (int ub = 0; ub <= tb; ++ub)
#pragma unroll
                for (int r = 0; r < 4; ++r) Y = mfma(PbA[ub][r], sv[ub][r], Y);
        };
        auto y_store = [&](int64_t t0) {
            float *dst = y_out + (t0 + 16 * tb) * stride + 16 * ib;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[Ly + r * stride] = Y[r];
        };
        auto tape_out = [&](int64_t blk, int b) {
            if (!sa_out) return;
            const int nst = steps_of(blk);
            float *dst = sa_out + (blk * kTB + 4 * h) * stride;
            if (nst == kTB || 4 * h + g < nst)
                *reinterpret_cast<float4 *>(dst + Ls) = lds4(sap[b] + 256 * (h & 3) + 1024 * (h >> 2), Lq);
        };
        auto ckpt_out = [&](int64_t blk) {
            const int64_t t = blk * kTB;
            if (!ck_out || (tb0 + t) % chunk != 0) return;
            float *dst = ck_out + (bh * nck + (tb0 + t) / chunk) * N * N;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int row = 8 * h + 4 * k + g;
                *reinterpret_cast<float4 *>(dst + 64 * row + 4 * l16) = lds4(sS0, sw(row, 4 * l16));
            }
        };

        // Phase q (q = -1 before the first block): the scan waves run block
        // q while the helpers finish block q - 1, start y of block q and
        // prepare block q + 1 in slot[(q + 1) & 1].
        for (int64_t q = -1; q < nblk; ++q) {
            const int bb = (int)(q & 1), bn = bb ^ 1;
            const bool next = q + 1 < nblk;
            if (q >= 0 && fastB) {
                // sum_u v_u kt_u^T of block q, for the end of its steps
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    put4(vkt + 1024 * (2 * tb + m), Lt, make_float4(VK[m][0], VK[m][1], VK[m][2], VK[m][3]));
            }
            if (next) {
                stage_issue(q + 1, bn);
                if (h == 0 && lane == 0) hbad[bn] = 0;
            }
            if (q >= 1) {
                if (fastA && want_y) {
                    y_from_sa(bn);
                    y_store((q - 1) * kTB);
                }
                tape_out(q - 1, bn);
            }
            if (q >= 0) {
                ckpt_out(q);
                if (fastB && want_y) y_from_s0(bb);
            }
            bool fastC = false;
            if (next) {
                stage_land(q + 1, bn);
                hsync();   // block q + 1 staged
                fastC = prep(bn, steps_of(q + 1));
                if (h == 0 && lane == 0) smode[bn] = fastC ? 1 : 0;
                if (fastC) {
                    const float *sb = &slot[bn][0][0];
                    hsync();   // block q + 1 rescaled
                    f4 cacc = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (kLite) {
                        // no y: only the kt . ab tiles (helpers 0-2) feed c; with
                        // v = 0, c and sum v kt^T vanish and no tile is needed
                        if constexpr (h < 3)
                            if (!zero_v) gram_tile(sb, std::integral_constant<int, h>{});
                        hsync();   // Gram tiles in LDS
                        VK[0] = VK[1] = f4{0.f, 0.f, 0.f, 0.f};
                        if (!zero_v) {
                            f4 Mk[2];
                            float vb[2][4], va[8], kb[8][2];
#pragma unroll
                            for (int ub = 0; ub <= tb; ++ub) {
                                Mk[ub] = gram_get(0, ub);
#pragma unroll
                                for (int r = 0; r < 4; ++r) vb[ub][r] = sb[vV * 2048 + 1024 * ub + L2[r]];
                            }
#pragma unroll
                            for (int kk = 0; kk < 8; ++kk) {
                                va[kk] = sb[vV * 2048 + L3 + 256 * kk + 16 * (ib ^ (kk & 3))];
#pragma unroll
                                for (int m = 0; m < 2; ++m)
                                    kb[kk][m] = sb[vK * 2048 + L3 + 256 * kk + 16 * ((2 * tb + m) ^ (kk & 3))];
                            }
#pragma unroll
                            for (int ub = 0; ub <= tb; ++ub)
#pragma unroll
                                for (int r = 0; r < 4; ++r) cacc = mfma(Mk[ub][r], vb[ub][r], cacc);
#pragma unroll
                            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                                for (int m = 0; m < 2; ++m) VK[m] = mfma(va[kk], kb[kk][m], VK[m]);
                        }
                    } else {
                        grams(sb);
                        hsync();   // Gram tiles in LDS
                        f4 Mk[2], Pk[2];
#pragma unroll
                        for (int ub = 0; ub <= tb; ++ub) {
                            Mk[ub] = gram_get(0, ub);
                            Pk[ub] = gram_get(1, ub);
                            PbC[ub] = gram_get(2, ub);
                        }
                        // c (into the slot of w) and the v terms of y
                        float vb[2][4];
#pragma unroll
                        for (int ub = 0; ub <= tb; ++ub)
#pragma unroll
                            for (int r = 0; r < 4; ++r) vb[ub][r] = sb[vV * 2048 + 1024 * ub + L2[r]];
                        // rows 16 ib .. 16 ib + 15 of sum_u v_u kt_u^T, column
                        // tiles 2 tb, 2 tb + 1: operands
                        float va[8], kb[8][2];
#pragma unroll
                        for (int kk = 0; kk < 8; ++kk) {
                            va[kk] = sb[vV * 2048 + L3 + 256 * kk + 16 * (ib ^ (kk & 3))];
#pragma unroll
                            for (int m = 0; m < 2; ++m)
                                kb[kk][m] = sb[vK * 2048 + L3 + 256 * kk + 16 * ((2 * tb + m) ^ (kk & 3))];
                        }
                        f4 yacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ub = 0; ub <= tb; ++ub)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                cacc = mfma(Mk[ub][r], vb[ub][r], cacc);
                                yacc = mfma(Pk[ub][r], vb[ub][r], yacc);
                            }
                        VK[0] = VK[1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                            for (int m = 0; m < 2; ++m) VK[m] = mfma(va[kk], kb[kk][m], VK[m]);
                        Yv = yacc;
                    }
                    float *cs = &slot[bn][vW][1024 * tb];
#pragma unroll
                    for (int r = 0; r < 4; ++r) cs[L2[r]] = cacc[r];
                }
            }
            if (q >= 0) {
                __syncthreads();   // X: block q's steps done
                __syncthreads();   // Y: the state after block q in LDS
            } else {
                __syncthreads();   // block 0 ready, S0 in LDS
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                PbA[m] = PbB[m];
                PbB[m] = PbC[m];
            }
            fastA = fastB;
            fastB = fastC;
        }
        // the last block's sa terms of y and its tape
        if (nblk > 0) {
            const int bl = (int)((nblk - 1) & 1);
            if (fastA && want_y) {
                y_from_sa(bl);
                y_store((nblk - 1) * kTB);
            }
            tape_out(nblk - 1, bl);
        }
    };
    switch (wave) {
    case 4: helper(std::integral_constant<int, 0>{}); break;
    case 5: helper(std::integral_constant<int, 1>{}); break;
    case 6: helper(std::integral_constant<int, 2>{}); break;
    case 7: helper(std::integral_constant<int, 3>{}); break;
    case 8: helper(std::integral_constant<int, 4>{}); break;
    case 9: helper(std::integral_constant<int, 5>{}); break;
    case 10: helper(std::integral_constant<int, 6>{}); break;
    default: helper(std::integral_constant<int, 7>{}); break;
    }
    finish();
}

template <typename TIn, bool kFused>
hipError_t launch_fwdc_t(const FwdLaunch &a, int mode, hipStream_t stream)
{
    FwdcArgs<TIn> p;
    for (int i = 0; i < 6; ++i) p.in[i] = static_cast<const TIn *>(a.in[i]);
    p.s0 = a.s0;
    p.y = a.y;
    p.sT = a.sT;
    p.ckpt = a.ckpt;
    p.sa = a.satape;
    p.T = a.T;
    p.H = a.H;
    p.chunk = a.chunk;
    p.nck = (int)((a.T + a.chunk - 1) / a.chunk);
    p.mode = mode;
    p.nseg = a.nseg;
    p.nckseg = a.nckseg;
    p.pbuf = a.pbuf;
    p.fault = fault_word();
    p.inject = test_fault_inject();
    if (!p.fault) return hipErrorInvalidDevicePointer;
    const int64_t units = mode == 0 ? a.B * a.H
                        : mode == 1 ? a.B * a.H * (2 * a.nseg - 3) : a.B * a.H * a.nseg;
    if (mode == 1)
        hipLaunchKernelGGL((wkv7_fwdc_kernel<TIn, kFused, true>), dim3((unsigned)units), dim3(kThreads), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((wkv7_fwdc_kernel<TIn, kFused, false>), dim3((unsigned)units), dim3(kThreads), 0,
                           stream, p);
    return hipGetLastError();
}

// Bit 0: a forward helper wait gave up somewhere on this device since the
// word was last cleared (wkv7_fault_status).  One word per device.
__device__ unsigned g_fault_word;

}  // namespace

unsigned *fault_word()
{
    static std::atomic<unsigned *> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    unsigned *ptr = cache[dev].load(std::memory_order_acquire);
    if (!ptr) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(g_fault_word)) != hipSuccess) return nullptr;
        ptr = static_cast<unsigned *>(addr);
        cache[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

bool forward_chunked_supported(const FwdLaunch &a)
{
    return a.N == 64 && a.chunk > 0 && a.chunk % kTB == 0;
}

hipError_t launch_forward_chunked(const FwdLaunch &a, int mode, hipStream_t stream)
{
    if (a.fused)
        return a.dtype == 0 ? launch_fwdc_t<float, true>(a, mode, stream)
                            : launch_fwdc_t<uint16_t, true>(a, mode, stream);
    return a.dtype == 0 ? launch_fwdc_t<float, false>(a, mode, stream)
                        : launch_fwdc_t<uint16_t, false>(a, mode, stream);
}

}  // namespace wkv7
