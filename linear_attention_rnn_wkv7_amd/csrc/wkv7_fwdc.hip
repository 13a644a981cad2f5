// WKV7 forward for N = 64: a serial scan on four waves beside four waves that
// prepare its inputs and compute its outputs on the matrix cores.
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
// One workgroup of eight waves per (b, h).  Waves 0-3 run the steps of block
// q (wave w: rows 16 w .. 16 w + 15 of S, 2 rows x 8 columns per lane) and
// then its y for their rows on the matrix cores.  Waves 4-7 ("helpers")
// meanwhile copy block q + 1 into LDS, rescale it and compute its Gram
// tiles, c and sum of v kt^T; they also write the sa tape of block q - 1 and
// the checkpoints.  The helpers synchronise among themselves through an LDS
// arrival counter, and with the scan waves twice per block (X: the block's
// steps are done; Y: the state after the block is in LDS, and the scan waves
// hold the next block's Gram tiles for y).  Blocks whose decays leave
// [1/16, 1] or whose cumulative decay drops below 2^-60, and a final partial
// block, run the plain step on the scan waves instead (y on the VALU, no
// rescaling).  Checkpoints must fall on block starts (chunk a multiple of 32).

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
};

template <typename TIn>
__global__ void __launch_bounds__(512) wkv7_fwdc_kernel(FwdcArgs<TIn> p)
{
    constexpr int N = 64, R = 2, CC = 8, LPR = 8;
    __shared__ __align__(16) float slot[2][6][kTB * N];  // block inputs, by q & 1
    __shared__ __align__(16) float gram[9][256];         // Gram tiles, lane-linear
    __shared__ __align__(16) float vkt[N * N];           // sum_u v_u kt_u^T, transposed
    __shared__ __align__(16) float sap[2][kTB * N];      // sa of the block, by q & 1
    __shared__ __align__(16) float sS0[N * N];           // state before the block
    __shared__ __align__(16) float g31[2][N];            // g_31 of the block
    __shared__ int smode[2];                             // 1: block rescaled
    __shared__ int hbad[2];                              // a decay out of range
    __shared__ unsigned hcnt;                            // helper arrivals

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = blockIdx.x, T = p.T, H = p.H;
    const int64_t bidx = bh / H, head = bh % H;
    const int64_t stride = H * N;
    const int64_t vbase = (bidx * T * H + head) * N;
    const int64_t nblk = (T + kTB - 1) / kTB;
    auto steps_of = [&](int64_t blk) -> int {
        const int64_t rem = T - blk * kTB;
        return (int)(rem < kTB ? rem : kTB);
    };

    if (tid == 0) {
        smode[0] = smode[1] = 0;
        hbad[0] = hbad[1] = 0;
        hcnt = 0;
    }
    __syncthreads();

    if (wave < 4) {
        // ================= scan waves =================
        const int cg = lane % LPR, rg = lane / LPR;
        const int row0 = wave * 16 + rg * R, col0 = cg * CC;

        float S[R][CC];
        if (p.s0) {
            const float *src = p.s0 + bh * N * N + (int64_t)row0 * N + col0;
#pragma unroll
            for (int e = 0; e < R; ++e)
#pragma unroll
                for (int c = 0; c < CC; c += 4) {
                    const float4 q = *reinterpret_cast<const float4 *>(src + e * N + c);
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

        // The read-out y of a rescaled block, on the matrix cores: tile tb
        // holds steps 16 tb .. 16 tb + 15 (accumulator row 4 gq + i) of rows
        // 16 wave .. 16 wave + 15 of S (accumulator column l16).
        const bool want_y = p.y != nullptr;
        const int l16 = lane & 15, gq = lane >> 4, qa = l16 >> 2, c3 = l16 & 3;
        // rows 16 X + l16, columns 16 q4 + 4 gq .. + 3:  L1[q4] + 1024 X
        int L1[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) L1[q4] = 64 * l16 + 16 * (q4 ^ qa) + 4 * (gq ^ c3);
        // rows 16 U + 4 gq + r, column 16 wave + l16:  Lv[r] + 1024 U
        int Lv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) Lv[r] = 256 * gq + 64 * r + 16 * (wave ^ gq) + 4 * (qa ^ r) + c3;
        // Gram tiles kt.rb and bt.rb of the next block, (u-block, t-block)
        // = (0,0), (0,1), (1,1); read while the helpers leave them in place
        f4 Pk[3], Pb[3];
        auto read_grams = [&]() {
#pragma unroll
            for (int pos = 0; pos < 3; ++pos) {
                Pk[pos] = *reinterpret_cast<const f4 *>(&gram[3 + pos][4 * lane]);
                Pb[pos] = *reinterpret_cast<const f4 *>(&gram[6 + pos][4 * lane]);
            }
        };
        // y_t = S0 rb_t + sum_{u<=t} v_u (kt_u . rb_t) + sa_u (bt_u . rb_t)
        auto y_block = [&](int bb, int64_t t0) {
            const float *rbv = slot[bb][vR], *vv = slot[bb][vV], *sav = sap[bb];
            float4 sr[4], xr[2][4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                sr[q4] = lds4(sS0 + 1024 * wave, L1[q4]);
                xr[0][q4] = lds4(rbv, L1[q4]);
                xr[1][q4] = lds4(rbv + 1024, L1[q4]);
            }
            float vb[2][4], sb[2][4];
#pragma unroll
            for (int ub = 0; ub < 2; ++ub)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    vb[ub][r] = vv[1024 * ub + Lv[r]];
                    sb[ub][r] = sav[1024 * ub + Lv[r]];
                }
            f4 Y[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) Y[tb] = mfma(xr[tb][q4].x, sr[q4].x, Y[tb]);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) Y[tb] = mfma(xr[tb][q4].y, sr[q4].y, Y[tb]);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) Y[tb] = mfma(xr[tb][q4].z, sr[q4].z, Y[tb]);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) Y[tb] = mfma(xr[tb][q4].w, sr[q4].w, Y[tb]);
            }
#pragma unroll
            for (int ub = 0; ub < 2; ++ub)
#pragma unroll
                for (int tb = ub; tb < 2; ++tb) {
                    const int pos = tb == 0 ? 0 : 1 + ub;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        Y[tb] = mfma(Pk[pos][r], vb[ub][r], Y[tb]);
                        Y[tb] = mfma(Pb[pos][r], sb[ub][r], Y[tb]);
                    }
                }
            float *dst = p.y + vbase + t0 * stride + 16 * wave + l16;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(16 * tb + 4 * gq + i) * stride] = Y[tb][i];
        };

        put_state();
        __syncthreads();   // block 0 ready, S0 in LDS
        read_grams();
        __syncthreads();   // the helpers may now replace the Gram tiles

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
                // operands two steps ahead
                Ops ops[3];
                load_ops(0, ops[0]);
                load_ops(1, ops[1]);
#pragma unroll
                for (int s = 0; s < kTB; ++s) {
                    if (s + 2 < kTB) load_ops(s + 2, ops[(s + 2) % 3]);
                    const Ops &o = ops[s % 3];
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
                if (want_y) y_block(bb, t0);
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
                    if (p.y && cg < R) p.y[vbase + (t0 + s) * stride + row0 + cg] = cg == 0 ? yv[0] : yv[1];
                }
                __syncthreads();   // X
            }
            put_state();           // the state before block q + 1
            read_grams();          // (block q + 1's, computed during block q)
            __syncthreads();       // Y
        }
        if (p.sT) {
            float *dst = p.sT + bh * N * N + (int64_t)row0 * N + col0;
#pragma unroll
            for (int e = 0; e < R; ++e)
#pragma unroll
                for (int c = 0; c < CC; c += 4)
                    *reinterpret_cast<float4 *>(dst + e * N + c) =
                        make_float4(S[e][c], S[e][c + 1], S[e][c + 2], S[e][c + 3]);
        }
        return;
    }

    // ================= helper waves =================
    // The helper code is instantiated per helper wave (its index h a
    // compile-time constant), and every LDS address is one of a few per-lane
    // offsets plus a constant, so that the helpers spend their issue slots
    // on loads, stores and MFMAs rather than on address arithmetic.
    const int l16 = lane & 15, g = lane >> 4, qa = l16 >> 2, c3 = l16 & 3;
    const TIn *in_ptr[6];
#pragma unroll
    for (int v = 0; v < 6; ++v) in_ptr[v] = p.in[v] + vbase;
    float *const sa_out = p.sa ? p.sa + vbase : nullptr;
    float *const ck_out = p.ckpt;
    const int chunk = p.chunk, nck = p.nck;
    float *const gbuf = &gram[0][0];   // g of the block being rescaled

    // Wait until all four helper waves have arrived here.  Every helper wave
    // runs the same sequence of waits; the poll count is bounded so that a
    // broken sequence ends the kernel with wrong results instead of a hang.
    unsigned htarget = 0;
    auto hsync = [&]() {
        htarget += 4;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) __hip_atomic_fetch_add(&hcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        for (unsigned it = 0; it < kSpinMax; ++it) {
            if (__hip_atomic_load(&hcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= htarget) break;
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };

    auto helper = [&](auto hw) {
        constexpr int h = decltype(hw)::value;
        // y tiles of this wave: steps 16 tb .. 16 tb + 15, rows 16 (2 ih + m)
        // .. + 15 for m = 0, 1 (lane: step 16 tb + 4 g + r, row .. + l16)
        constexpr int tb = h & 1, ih = h >> 1;

        // ---- lane offsets (floats) into the swizzled [rows][64] arrays:
        //   rows 16 X + l16, columns 16 q4 + 4 g .. + 3    L1[q4] + 1024 X
        //   rows 16 U + 4 g + r, column 16 (2 ih + m) + l16    L2[m][r] + 1024 U
        //   rows 4 k + g, column 16 I + l16    L3 + 256 k + 16 (I ^ (k & 3))
        int L1[4], L2[2][4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) L1[q4] = 64 * l16 + 16 * (q4 ^ qa) + 4 * (g ^ c3);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                L2[m][r] = 256 * g + 64 * r + 16 * ((2 * ih + m) ^ g) + 4 * (qa ^ r) + c3;
        const int L3 = 64 * g + 4 * (qa ^ g) + c3;
        // sum v kt^T, stored transposed: row j = 16 jt + l16, columns
        // 16 h + 4 g .. + 3
        const int Lt = 64 * l16 + 4 * ((4 * h + g) ^ l16);
        // rescaling by rows: step tr, columns 8 cq + 4 m .. + 3
        const int tr = 8 * h + (lane >> 3), cq = lane & 7;
        int Lr[2], Lp[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            Lr[m] = 64 * tr + 4 * ((2 * cq + m) ^ (tr & 15));
            Lp[m] = tr > 0 ? 64 * (tr - 1) + 4 * ((2 * cq + m) ^ ((tr - 1) & 15)) : 0;
        }
        // tape and checkpoints: rows 4 h + 16 k + g, columns 4 l16 .. + 3
        const int Lq = 64 * g + 4 * (l16 ^ (4 * h + g));
        // global offsets (elements)
        const int Ls = g * (int)stride + 4 * l16;   // tape: step g, column 4 l16
        int Ld[4];                                  // staging: step g, swizzled column
#pragma unroll
        for (int u = 0; u < 4; ++u) Ld[u] = g * (int)stride + 4 * (l16 ^ (4 * u + g));

        // ---- staging of block blk into slot[b]: units of 1 KB (4 steps of
        // one input), 12 per helper wave; fp32 by direct HBM -> LDS copies
        // (lane l of a unit lands at float 4 l: step 4 u + l / 16, swizzled
        // column group l % 16), bf16 through registers (widened)
        constexpr bool kDma = std::is_same<TIn, float>::value;
        using Raw = typename InQuad<TIn>::raw;
        Raw pre[12];
        auto stage_unit = [&](int64_t t0, int b, int k) {
            const int unit = 12 * h + k, v = unit >> 3, u = unit & 7;
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
                for (int k = 0; k < 12; ++k) stage_unit(t0, b, k);
            } else {
#pragma unroll
                for (int k = 0; k < 12; ++k)
                    if (4 * ((12 * h + k) & 7) + g < nst) stage_unit(t0, b, k);
            }
        };
        auto stage_land = [&](int64_t blk, int b) {
            if constexpr (kDma) {
                wait_dma();
            } else {
                const int nst = steps_of(blk);
#pragma unroll
                for (int k = 0; k < 12; ++k) {
                    const int unit = 12 * h + k, v = unit >> 3, u = unit & 7;
                    if (nst == kTB || 4 * u + g < nst)
                        put4(&slot[b][v][u * 256], 4 * lane, InQuad<TIn>::f32(pre[k]));
                }
            }
        };

        // ---- rescaling of the staged block in slot[b], in place.  First g,
        // per column: lane (l16, g) owns column 16 h + l16 and steps 4 u + g,
        // u = 0 .. 7 (prefix products over each group of four steps by lane
        // exchanges); g goes to the Gram area, free until the Gram tiles.
        // Then, if every column is in range, r, a, k, b are rescaled by rows.
        // Returns whether the block is rescaled (the same in every helper).
        auto prep = [&](int b, int nstn) -> bool {
            float *const sb = &slot[b][0][0];
            bool ok = nstn == kTB;
            if (ok) {
                float wv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) wv[u] = sb[vW * 2048 + L3 + 256 * u + 16 * (h ^ (u & 3))];
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
            hsync();
            const bool fast = __builtin_amdgcn_readfirstlane(hbad[b]) == 0;
            if (fast) {
                float4 gt[2], gp[2], x[4][2];
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    gt[m] = lds4(gbuf, Lr[m]);
                    gp[m] = lds4(gbuf, Lp[m]);
                    if (h == 0 && tr == 0) gp[m] = make_float4(1.f, 1.f, 1.f, 1.f);
                    x[0][m] = lds4(sb + vR * 2048, Lr[m]);
                    x[1][m] = lds4(sb + vA * 2048, Lr[m]);
                    x[2][m] = lds4(sb + vK * 2048, Lr[m]);
                    x[3][m] = lds4(sb + vB * 2048, Lr[m]);
                }
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const float4 iv = make_float4(__builtin_amdgcn_rcpf(gt[m].x), __builtin_amdgcn_rcpf(gt[m].y),
                                                  __builtin_amdgcn_rcpf(gt[m].z), __builtin_amdgcn_rcpf(gt[m].w));
                    put4(sb + vR * 2048, Lr[m], make_float4(x[0][m].x * gt[m].x, x[0][m].y * gt[m].y,
                                                            x[0][m].z * gt[m].z, x[0][m].w * gt[m].w));
                    put4(sb + vA * 2048, Lr[m], make_float4(x[1][m].x * gp[m].x, x[1][m].y * gp[m].y,
                                                            x[1][m].z * gp[m].z, x[1][m].w * gp[m].w));
                    put4(sb + vK * 2048, Lr[m], make_float4(x[2][m].x * iv.x, x[2][m].y * iv.y,
                                                            x[2][m].z * iv.z, x[2][m].w * iv.w));
                    put4(sb + vB * 2048, Lr[m], make_float4(x[3][m].x * iv.x, x[3][m].y * iv.y,
                                                            x[3][m].z * iv.z, x[3][m].w * iv.w));
                    if (h == 3 && tr == kTB - 1) put4(g31[b], 8 * cq + 4 * m, gt[m]);
                }
            }
            return fast;
        };

        // ---- Gram tile n: kind n / 3 (0: kt . ab with u < t, 1: kt . rb,
        // 2: bt . rb, both u <= t), position n % 3 = (u-block, t-block)
        // (0,0), (0,1), (1,1); D[u][t] in the accumulator layout, stored
        // lane-linear.  Wave h computes tiles h and h + 4 (and 8 for h = 0).
        auto gram_load = [&](const float *sb, auto nc, float4 (&xq)[4], float4 (&zq)[4]) {
            constexpr int n = decltype(nc)::value, kind = n / 3, pos = n % 3;
            constexpr int ub = pos == 2 ? 1 : 0, tn = pos == 0 ? 0 : 1;
            constexpr int xo = (kind == 2 ? vB : vK) * 2048 + 1024 * ub;
            constexpr int zo = (kind == 0 ? vA : vR) * 2048 + 1024 * tn;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                xq[q4] = lds4(sb + xo, L1[q4]);
                zq[q4] = lds4(sb + zo, L1[q4]);
            }
        };
        auto gram_store = [&](auto nc, f4 acc) {
            constexpr int n = decltype(nc)::value, kind = n / 3, pos = n % 3;
            if constexpr (pos != 1) {   // a diagonal tile
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = 4 * g + r - l16;   // u - t within the tile
                    if (kind == 0 ? d >= 0 : d > 0) acc[r] = 0.f;
                }
            }
            *reinterpret_cast<f4 *>(&gram[n][4 * lane]) = acc;
        };
        auto grams = [&](const float *sb) {
            using N0 = std::integral_constant<int, h>;
            using N1 = std::integral_constant<int, h + 4>;
            float4 xa[4], za[4], xb[4], zb[4];
            gram_load(sb, N0{}, xa, za);
            gram_load(sb, N1{}, xb, zb);
            f4 a = {0.f, 0.f, 0.f, 0.f}, c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                a = mfma(xa[q4].x, za[q4].x, a);
                c = mfma(xb[q4].x, zb[q4].x, c);
                a = mfma(xa[q4].y, za[q4].y, a);
                c = mfma(xb[q4].y, zb[q4].y, c);
                a = mfma(xa[q4].z, za[q4].z, a);
                c = mfma(xb[q4].z, zb[q4].z, c);
                a = mfma(xa[q4].w, za[q4].w, a);
                c = mfma(xb[q4].w, zb[q4].w, c);
            }
            gram_store(N0{}, a);
            gram_store(N1{}, c);
            if constexpr (h == 0) {
                using N2 = std::integral_constant<int, 8>;
                gram_load(sb, N2{}, xa, za);
                f4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    e = mfma(xa[q4].x, za[q4].x, e);
                    e = mfma(xa[q4].y, za[q4].y, e);
                    e = mfma(xa[q4].z, za[q4].z, e);
                    e = mfma(xa[q4].w, za[q4].w, e);
                }
                gram_store(N2{}, e);
            }
        };
        auto gram_get = [&](int kind, int ub) -> f4 {
            const int pos = tb == 0 ? 0 : 1 + ub;
            return *reinterpret_cast<const f4 *>(&gram[3 * kind + pos][4 * lane]);
        };

        f4 VK[4];
        bool fastB = false;   // block q
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) VK[jt] = f4{0.f, 0.f, 0.f, 0.f};

        auto tape_out = [&](int64_t blk, int b) {
            if (!sa_out) return;
            const int nst = steps_of(blk);
            float *dst = sa_out + (blk * kTB + 4 * h) * stride;
            if (nst == kTB) {
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    *reinterpret_cast<float4 *>(dst + 16 * k * stride + Ls) = lds4(sap[b] + 256 * h + 1024 * k, Lq);
            } else {
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    if (4 * h + 16 * k + g < nst)
                        *reinterpret_cast<float4 *>(dst + 16 * k * stride + Ls) = lds4(sap[b] + 256 * h + 1024 * k, Lq);
            }
        };
        auto ckpt_out = [&](int64_t blk) {
            const int64_t t = blk * kTB;
            if (!ck_out || t % chunk != 0) return;
            float *dst = ck_out + (bh * nck + t / chunk) * N * N + 256 * h;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                *reinterpret_cast<float4 *>(dst + 1024 * k + 64 * g + 4 * l16) = lds4(sS0 + 256 * h + 1024 * k, Lq);
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
                for (int jt = 0; jt < 4; ++jt)
                    put4(vkt + 1024 * jt, Lt, make_float4(VK[jt][0], VK[jt][1], VK[jt][2], VK[jt][3]));
            }
            if (next) {
                stage_issue(q + 1, bn);
                if (h == 0 && lane == 0) hbad[bn] = 0;
            }
            if (q >= 1) tape_out(q - 1, bn);
            if (q >= 0) ckpt_out(q);
            bool fastC = false;
            if (next) {
                stage_land(q + 1, bn);
                hsync();   // block q + 1 staged
                fastC = prep(bn, steps_of(q + 1));
                if (h == 0 && lane == 0) smode[bn] = fastC ? 1 : 0;
                if (fastC) {
                    const float *sb = &slot[bn][0][0];
                    hsync();   // block q + 1 rescaled
                    grams(sb);
                    hsync();   // Gram tiles in LDS
                    f4 Mk[2];
#pragma unroll
                    for (int ub = 0; ub <= tb; ++ub) Mk[ub] = gram_get(0, ub);
                    // c, into the slot of w
                    float vb[2][2][4];
#pragma unroll
                    for (int ub = 0; ub <= tb; ++ub)
#pragma unroll
                        for (int m = 0; m < 2; ++m)
#pragma unroll
                            for (int r = 0; r < 4; ++r) vb[ub][m][r] = sb[vV * 2048 + 1024 * ub + L2[m][r]];
                    // rows 16 h .. 16 h + 15 of sum_u v_u kt_u^T: operands
                    float va[8], kb[8][4];
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk) {
                        va[kk] = sb[vV * 2048 + L3 + 256 * kk + 16 * (h ^ (kk & 3))];
#pragma unroll
                        for (int jt = 0; jt < 4; ++jt) kb[kk][jt] = sb[vK * 2048 + L3 + 256 * kk + 16 * (jt ^ (kk & 3))];
                    }
                    f4 cacc[2];
#pragma unroll
                    for (int m = 0; m < 2; ++m) cacc[m] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ub = 0; ub <= tb; ++ub)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
#pragma unroll
                            for (int m = 0; m < 2; ++m) cacc[m] = mfma(Mk[ub][r], vb[ub][m][r], cacc[m]);
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt) VK[jt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                        for (int jt = 0; jt < 4; ++jt) VK[jt] = mfma(va[kk], kb[kk][jt], VK[jt]);
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        float *cs = &slot[bn][vW][1024 * tb];
#pragma unroll
                        for (int r = 0; r < 4; ++r) cs[L2[m][r]] = cacc[m][r];
                    }
                }
            }
            if (q >= 0) {
                __syncthreads();   // X: block q's steps done
                __syncthreads();   // Y: the state after block q in LDS
            } else {
                __syncthreads();   // block 0 ready, S0 in LDS
                __syncthreads();   // the scan waves hold block 0's Gram tiles
            }
            fastB = fastC;
        }
        // the last block's tape
        if (nblk > 0) tape_out(nblk - 1, (int)((nblk - 1) & 1));
    };
    switch (wave) {
    case 4: helper(std::integral_constant<int, 0>{}); break;
    case 5: helper(std::integral_constant<int, 1>{}); break;
    case 6: helper(std::integral_constant<int, 2>{}); break;
    default: helper(std::integral_constant<int, 3>{}); break;
    }
}

template <typename TIn>
hipError_t launch_fwdc_t(const FwdLaunch &a, hipStream_t stream)
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
    hipLaunchKernelGGL((wkv7_fwdc_kernel<TIn>), dim3((unsigned)(a.B * a.H)), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool forward_chunked_supported(const FwdLaunch &a)
{
    return a.N == 64 && a.chunk > 0 && a.chunk % kTB == 0;
}

hipError_t launch_forward_chunked(const FwdLaunch &a, hipStream_t stream)
{
    return a.dtype == 0 ? launch_fwdc_t<float>(a, stream) : launch_fwdc_t<uint16_t>(a, stream);
}

}  // namespace wkv7
