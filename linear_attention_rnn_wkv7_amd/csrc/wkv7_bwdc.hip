// Chunk-form WKV7 reverse scan for N = 64 with checkpoints every 64 steps.
//
// The recurrence and its reverse scan are those of the Foundry page
// "rwkvx/rx_pretrain.c" (rx_wkv7_forward_seq, rx_wkv7_backward).  This kernel
// reaches the same gradients by a different, equivalent route that moves most
// of the arithmetic onto the fp32 matrix cores.  Per 64-step chunk of one
// (b, h), with S0 the checkpointed state before the chunk, all products
// relative to the chunk start:
//
//   g_t = w_0 * ... * w_t          (per column j; g_{-1} = 1)
//   rb_t = r_t g_t,  ab_t = a_t g_{t-1},  kt_t = k_t / g_t,  bt_t = b_t / g_t
//
// Forward states:  S_t = (S0 + sum_{u<=t} v_u kt_u^T + sa_u bt_u^T) diag(g_t),
// with sa_u the forward's own S_{u-1} a_u (the tape in the checkpoint record).
// Reverse: with H = dL/dS at the chunk end (from the later chunks) and
// Hb = H diag(g_63), the gradient of the state after step t is
//   G_t = (Hb + sum_{u>=t} dy_u rb_u^T + sum_{u>t} dsa_u ab_u^T) diag(1/g_t),
// and dsa_t = G_t b_t.  dsa is the only quantity with a serial dependency:
// phase 1 runs it step by step (VALU, the state G scaled by g so that the
// decay costs nothing per element).  Phase 2 then forms every gradient with
// dense contractions (MFMA), e.g.
//   dk_t = (1/g_t) (Hb^T v_t + sum_{u>=t} rb_u (dy_u.v_t) + sum_{u>t} ab_u (dsa_u.v_t))
//   dr_t = g_t (S0^T dy_t + sum_{u<=t} kt_u (v_u.dy_t) + bt_u (sa_u.dy_t))
// and dw from the per-column identity
//   w_t dw_t = c + sum_{u<t} (k dk + b db - r dr - a da)_u - a_t da_t,
//   c = sum_i (dL/dS0)[i][j] S0[i][j],
// which follows from S_t = S_{t-1} diag(w_t) + v_t k_t^T + sa_t b_t^T and the
// chain rule (the gradient-state inner product per column is conserved up to
// the terms each step adds).
//
// The rescaled form needs the cumulative decay to stay well inside fp32
// range and w not too small (dw divides by w).  A chunk whose decays fall
// outside [kWMin, 1] or whose cumulative decay drops below kGMin marks its
// (b, h) in `flags`; the host then runs the step-by-step reverse scan for the
// marked heads, which overwrites every output of those heads.

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kWMin = 0.0625f;            // smallest decay taken by this form
constexpr float kGMin = 8.67361738e-19f;    // 2^-60: smallest cumulative decay

__device__ __forceinline__ f4 mfma(float a, float b, f4 c)
{
    // D[m][n] += A[m][k] B[k][n] over a 16x16x4 block: lane l supplies
    // A[l % 16][l / 16] and B[l / 16][l % 16] and holds D[4 (l / 16) + i][l % 16].
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// [64][64] fp32 LDS arrays, 16-byte groups of a row XOR-swizzled by the row:
// rows and 16-row column slices both read without bank conflicts.
__device__ __forceinline__ int sw(int t, int j)
{
    return (t << 6) + ((((j >> 2) ^ (t & 15))) << 2) + (j & 3);
}

// 16x16 tile of a Gram matrix: rows a, b: quarter-rotated so that the four
// rows an MFMA result writes at once fall in different banks.
__device__ __forceinline__ int pt(int a, int b)
{
    return ((a >> 2) << 6) + ((((a & 3) + (a >> 2)) & 3) << 4) + b;
}

// Lower-triangular 16x16 block (ab >= bb) of a 64x64 matrix -> slot 0..9.
__host__ __device__ constexpr int tix(int ab, int bb) { return ab * (ab + 1) / 2 + bb; }
__host__ __device__ constexpr int tab(int n) { return n >= 6 ? 3 : n >= 3 ? 2 : n >= 1 ? 1 : 0; }
__host__ __device__ constexpr int tbb(int n) { return n - tab(n) * (tab(n) + 1) / 2; }

template <typename TIn>
__device__ __forceinline__ float4 ld4(const TIn *p)
{
    return InQuad<TIn>::f32(InQuad<TIn>::load(p));
}

__device__ __forceinline__ float ld1(const float *p) { return *p; }
__device__ __forceinline__ float ld1(const uint16_t *p) { return bf16_lo(*p); }

__device__ __forceinline__ float4 lds4(const float *s, int o)
{
    return *reinterpret_cast<const float4 *>(s + o);
}

__device__ __forceinline__ void put4(float *s, int o, float4 v)
{
    *reinterpret_cast<float4 *>(s + o) = v;
}

// 16 consecutive columns 16q'.. of row t of a swizzled array.
__device__ __forceinline__ void row16(const float *s, int t, int c0, float (&o)[16])
{
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float4 x = lds4(s, sw(t, c0 + 4 * m));
        o[4 * m] = x.x;
        o[4 * m + 1] = x.y;
        o[4 * m + 2] = x.z;
        o[4 * m + 3] = x.w;
    }
}

template <typename TIn>
struct BwdcArgs {
    const TIn *r, *w, *k, *v, *a, *b, *dy;
    const float *sa, *ckpt, *dsT;
    float *dr, *dw, *dk, *dv, *da, *db, *ds0;
    int *flags;
    int64_t T, H;
    int nck;
};

template <typename TIn>
__global__ void __launch_bounds__(256) wkv7_bwdc_kernel(BwdcArgs<TIn> p)
{
    // chunk vectors, [step][feature] swizzled: cumulative decay, rb, ab, kt,
    // bt, dsa, dy, and v (later sa)
    __shared__ __align__(16) float sG[4096], sR[4096], sA[4096], sK[4096], sB[4096];
    __shared__ __align__(16) float sD[4096], sDY[4096], sVS[4096];
    // Hb (a state, [row][col] swizzled) until phase 2 starts, then two Gram
    // matrices (10 lower 16x16 tiles each)
    __shared__ __align__(16) float sP[20 * 256];
    __shared__ __align__(16) float sScan[4][256];
    __shared__ __align__(16) float sCp[4][64];
    __shared__ __align__(16) float sC[64];
    __shared__ float sBeta[68];
    __shared__ int sBad;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.x, T = p.T, H = p.H;
    const int64_t bb_ = bh / H, hh = bh % H;
    const int64_t stride = H * 64;
    const int64_t vbase = (bb_ * T * H + hh) * 64;
    const int nck = p.nck;
    // phase 1: row prow of G, columns 16 pcg .. 16 pcg + 15
    const int prow = wave * 16 + (lane >> 2), pcg = lane & 3;
    // phase 2: feature jw of every output tile
    const int jw = wave * 16 + l16;

    float Gc[16];
    if (p.dsT) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float4 x = *reinterpret_cast<const float4 *>(p.dsT + bh * 4096 + prow * 64 + pcg * 16 + 4 * m);
            Gc[4 * m] = x.x;
            Gc[4 * m + 1] = x.y;
            Gc[4 * m + 2] = x.z;
            Gc[4 * m + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) Gc[q] = 0.f;
    }
    bool bad = false;
    if (tid == 0) sBad = 0;

    for (int c = nck - 1; c >= 0; --c) {
        const int64_t t0 = (int64_t)c * 64;
        const int Lc = (int)(T - t0 < 64 ? T - t0 : 64);

        // ---- stage r, w, k, a, b, v and dy for the chunk (zero past the end,
        // decay 1)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int u = tid + 256 * m, t = u >> 4, j4 = (u & 15) << 2;
            float4 R = make_float4(0.f, 0.f, 0.f, 0.f), W = make_float4(1.f, 1.f, 1.f, 1.f);
            float4 K = R, A = R, Bv = R, V = R, DY = R;
            if (t < Lc) {
                const int64_t off = vbase + (t0 + t) * stride + j4;
                R = ld4(p.r + off);
                W = ld4(p.w + off);
                K = ld4(p.k + off);
                A = ld4(p.a + off);
                Bv = ld4(p.b + off);
                V = ld4(p.v + off);
                DY = ld4(p.dy + off);
            }
            const int o = sw(t, j4);
            put4(sR, o, R);
            put4(sG, o, W);
            put4(sK, o, K);
            put4(sA, o, A);
            put4(sB, o, Bv);
            put4(sVS, o, V);
            put4(sDY, o, DY);
        }
        __syncthreads();

        // ---- cumulative decay, in place of w: 4 segments of 16 steps per column
        {
            const int j = tid & 63, seg = tid >> 6;
            float pr = 1.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) pr *= sG[sw(seg * 16 + u, j)];
            sCp[seg][j] = pr;
        }
        __syncthreads();
        {
            const int j = tid & 63, seg = tid >> 6;
            float pre = 1.f;
            for (int s2 = 0; s2 < seg; ++s2) pre *= sCp[s2][j];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int o = sw(seg * 16 + u, j);
                const float wv = sG[o];
                pre *= wv;
                bad |= !(wv >= kWMin && wv <= 1.f && pre >= kGMin);
                sG[o] = pre;
            }
        }
        __syncthreads();

        // ---- rb = r g, ab = a g_prev, kt = k / g, bt = b / g
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int u = tid + 256 * m, t = u >> 4, j4 = (u & 15) << 2;
            const int o = sw(t, j4);
            const float4 gm = lds4(sG, o);
            const float4 gp = t > 0 ? lds4(sG, sw(t - 1, j4)) : make_float4(1.f, 1.f, 1.f, 1.f);
            const float4 inv = make_float4(1.f / gm.x, 1.f / gm.y, 1.f / gm.z, 1.f / gm.w);
            float4 x = lds4(sR, o);
            put4(sR, o, make_float4(x.x * gm.x, x.y * gm.y, x.z * gm.z, x.w * gm.w));
            x = lds4(sA, o);
            put4(sA, o, make_float4(x.x * gp.x, x.y * gp.y, x.z * gp.z, x.w * gp.w));
            x = lds4(sK, o);
            put4(sK, o, make_float4(x.x * inv.x, x.y * inv.y, x.z * inv.z, x.w * inv.w));
            x = lds4(sB, o);
            put4(sB, o, make_float4(x.x * inv.x, x.y * inv.y, x.z * inv.z, x.w * inv.w));
        }
        __syncthreads();

        // ---- beta_t = ab_t . bt_{t-1} (couples consecutive dsa), and Hb
        {
            const int t = tid >> 2, q = tid & 3;
            float acc = 0.f;
            if (t >= 1) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float4 x = lds4(sA, sw(t, 16 * q + 4 * m));
                    const float4 y = lds4(sB, sw(t - 1, 16 * q + 4 * m));
                    acc = fmaf(x.x, y.x, acc);
                    acc = fmaf(x.y, y.y, acc);
                    acc = fmaf(x.z, y.z, acc);
                    acc = fmaf(x.w, y.w, acc);
                }
            }
            acc = group_allreduce<4>(acc);
            if (q == 0) sBeta[t] = acc;
            if (tid == 0) sBeta[64] = 0.f;
        }
        {
            float g63[16];
            row16(sG, 63, 16 * pcg, g63);
#pragma unroll
            for (int q = 0; q < 16; ++q) Gc[q] *= g63[q];
#pragma unroll
            for (int m = 0; m < 4; ++m)
                put4(sP, sw(prow, 16 * pcg + 4 * m),
                     make_float4(Gc[4 * m], Gc[4 * m + 1], Gc[4 * m + 2], Gc[4 * m + 3]));
        }
        __syncthreads();

        // Hb column jw (rows 16 g ..) and row jw (columns 16 g ..): the B
        // operands of its phase-2 products
        float hB[16], hR[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) hB[s] = sP[sw(16 * g + s, jw)];
        row16(sP, jw, 16 * g, hR);

        // ---- phase 1: dsa_t = G_t b_t, last step first
        {
            float U[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) U[q] = Gc[q];
            float dsa1 = 0.f;   // dsa of the step after t, not yet folded into U
            for (int t = Lc - 1; t >= 0; --t) {
                const float dyv = sDY[sw(t, prow)];
                float rv[16], bv[16];
                row16(sR, t, 16 * pcg, rv);
                row16(sB, t, 16 * pcg, bv);
                float X[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) X[q] = fmaf(dyv, rv[q], U[q]);
                float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
                for (int q = 0; q < 16; q += 4) {
                    s0 = fmaf(X[q], bv[q], s0);
                    s1 = fmaf(X[q + 1], bv[q + 1], s1);
                    s2 = fmaf(X[q + 2], bv[q + 2], s2);
                    s3 = fmaf(X[q + 3], bv[q + 3], s3);
                }
                const float qs = group_allreduce<4>((s0 + s1) + (s2 + s3));
                const float dsa = fmaf(dsa1, sBeta[t + 1], qs);
                if (t + 1 < Lc) {
                    float av[16];
                    row16(sA, t + 1, 16 * pcg, av);
#pragma unroll
                    for (int q = 0; q < 16; ++q) U[q] = fmaf(dsa1, av[q], X[q]);
                } else {
#pragma unroll
                    for (int q = 0; q < 16; ++q) U[q] = X[q];
                }
                dsa1 = dsa;
                if (pcg == 0) sD[sw(t, prow)] = dsa;
            }
            float av[16];
            row16(sA, 0, 16 * pcg, av);
#pragma unroll
            for (int q = 0; q < 16; ++q) Gc[q] = fmaf(dsa1, av[q], U[q]);   // dL/dS0
        }
        for (int u = tid; u < (64 - Lc) * 64; u += 256) sD[sw(Lc + (u >> 6), u & 63)] = 0.f;

        // ---- c = column sums of dL/dS0 (.) S0; ds0 after the first chunk
        const float *S0 = p.ckpt + (bh * nck + c) * 4096;
        {
            float x[16];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 s = *reinterpret_cast<const float4 *>(S0 + prow * 64 + pcg * 16 + 4 * m);
                x[4 * m] = s.x * Gc[4 * m];
                x[4 * m + 1] = s.y * Gc[4 * m + 1];
                x[4 * m + 2] = s.z * Gc[4 * m + 2];
                x[4 * m + 3] = s.w * Gc[4 * m + 3];
            }
            float y[8], z[4];
#pragma unroll
            for (int q = 0; q < 8; ++q) y[q] = swap_add32(x[q], x[q + 8]);
#pragma unroll
            for (int q = 0; q < 4; ++q) z[q] = swap_add16(y[q], y[q + 4]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                z[q] += dpp<kDppRor4>(z[q]);
                z[q] += dpp<kDppRor8>(z[q]);
            }
            if (((lane >> 2) & 3) == 0) {
                const int col = 16 * pcg + 8 * ((lane >> 5) & 1) + 4 * ((lane >> 4) & 1);
                *reinterpret_cast<float4 *>(&sCp[wave][col]) = make_float4(z[0], z[1], z[2], z[3]);
            }
            if (c == 0 && p.ds0) {
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    *reinterpret_cast<float4 *>(p.ds0 + bh * 4096 + prow * 64 + pcg * 16 + 4 * m) =
                        make_float4(Gc[4 * m], Gc[4 * m + 1], Gc[4 * m + 2], Gc[4 * m + 3]);
            }
        }
        // S0 column jw (rows 16 g ..)
        float s0B[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) s0B[s] = S0[(16 * g + s) * 64 + jw];
        __syncthreads();
        if (tid < 64) sC[tid] = (sCp[0][tid] + sCp[1][tid]) + (sCp[2][tid] + sCp[3][tid]);

        // sa for the second pass, loaded while the first one runs
        float4 saR[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int u = tid + 256 * m, t = u >> 4, j4 = (u & 15) << 2;
            saR[m] = t < Lc ? *reinterpret_cast<const float4 *>(p.sa + vbase + (t0 + t) * stride + j4)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }

        // Gram tiles: slot n < 10 holds rows of sX1 times rows of sY, slot
        // 10 + n rows of sX2 times rows of sY, for the lower block pair n
        // (rows a of the first factor, b of the second); the diagonal block
        // keeps a >= b for sX1 and a > b for sX2.  Wave w takes n = w + 4k.
        auto gram = [&](const float *sX1, const float *sX2, const float *sY) {
#pragma unroll 1
            for (int n = wave; n < 20; n += 4) {
                const int pr = n < 10 ? n : n - 10;
                const int ab = tab(pr), bq = tbb(pr);
                const float *sX = n < 10 ? sX1 : sX2;
                float xv[16], yv[16];
                row16(sX, 16 * ab + l16, 16 * g, xv);
                row16(sY, 16 * bq + l16, 16 * g, yv);
                f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 16; ++s) acc = mfma(xv[s], yv[s], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int al = 4 * g + i;
                    float val = acc[i];
                    if (ab == bq && (n < 10 ? al < l16 : al <= l16)) val = 0.f;
                    sP[n * 256 + pt(al, l16)] = val;
                }
            }
        };

        f4 XR[4], XA[4], XK[4], XB[4], XV[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            XR[tb] = f4{0.f, 0.f, 0.f, 0.f};
            XA[tb] = XR[tb];
            XK[tb] = XR[tb];
            XB[tb] = XR[tb];
            XV[tb] = XR[tb];
        }
        // dk / db bracket: Hb term with the value rows in sVS, then the Gram
        // terms over u >= t with rb and ab.
        auto back_terms = [&](f4 (&X)[4]) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                float va[16];
                row16(sVS, 16 * tb + l16, 16 * g, va);
#pragma unroll
                for (int s = 0; s < 16; ++s) X[tb] = mfma(va[s], hB[s], X[tb]);
#pragma unroll 1
                for (int ub = tb; ub < 4; ++ub) {
                    const int slot = tix(ub, tb);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int u = 16 * ub + 4 * g + s;
                        const float a1 = sP[slot * 256 + pt(4 * g + s, l16)];
                        const float a2 = sP[(10 + slot) * 256 + pt(4 * g + s, l16)];
                        X[tb] = mfma(a1, sR[sw(u, jw)], X[tb]);
                        X[tb] = mfma(a2, sA[sw(u, jw)], X[tb]);
                    }
                }
            }
        };
        // dr / da brackets: Gram terms over u <= t with the key-side vector
        // sF (kt with the v Grams, bt with the sa Grams).
        auto fwd_terms = [&](const float *sF) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
#pragma unroll 1
                for (int ub = 0; ub <= tb; ++ub) {
                    const int slot = tix(tb, ub);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int u = 16 * ub + 4 * g + s;
                        const float a1 = sP[slot * 256 + pt(l16, 4 * g + s)];
                        const float a2 = sP[(10 + slot) * 256 + pt(l16, 4 * g + s)];
                        const float bf = sF[sw(u, jw)];
                        XR[tb] = mfma(a1, bf, XR[tb]);
                        XA[tb] = mfma(a2, bf, XA[tb]);
                    }
                }
            }
        };

        // ---- pass 1: Grams dy v^T, dsa v^T; dk bracket; S0 and kt terms of dr, da
        gram(sDY, sD, sVS);
        __syncthreads();
        back_terms(XK);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            float ya[16], da_[16];
            row16(sDY, 16 * tb + l16, 16 * g, ya);
            row16(sD, 16 * tb + l16, 16 * g, da_);
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                XR[tb] = mfma(ya[s], s0B[s], XR[tb]);
                XA[tb] = mfma(da_[s], s0B[s], XA[tb]);
            }
        }
        fwd_terms(sK);
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int u = tid + 256 * m, t = u >> 4, j4 = (u & 15) << 2;
            put4(sVS, sw(t, j4), saR[m]);
        }
        __syncthreads();

        // ---- pass 2: Grams dy sa^T, dsa sa^T; db bracket; bt terms of dr, da
        gram(sDY, sD, sVS);
        __syncthreads();
        back_terms(XB);
        fwd_terms(sB);
        __syncthreads();

        // ---- pass 3: Grams rb kt^T, ab kt^T; dv
        gram(sR, sA, sK);
        __syncthreads();
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            float ka[16];
            row16(sK, 16 * tb + l16, 16 * g, ka);
#pragma unroll
            for (int s = 0; s < 16; ++s) XV[tb] = mfma(ka[s], hR[s], XV[tb]);
#pragma unroll 1
            for (int ub = tb; ub < 4; ++ub) {
                const int slot = tix(ub, tb);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int u = 16 * ub + 4 * g + s;
                    const float a1 = sP[slot * 256 + pt(4 * g + s, l16)];
                    const float a2 = sP[(10 + slot) * 256 + pt(4 * g + s, l16)];
                    XV[tb] = mfma(a1, sDY[sw(u, jw)], XV[tb]);
                    XV[tb] = mfma(a2, sD[sw(u, jw)], XV[tb]);
                }
            }
        }

        // ---- outputs and dw (prefix over steps of k dk + b db - r dr - a da)
        {
            float f[4][4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int o = sw(16 * tb + 4 * g + i, jw);
                    f[tb][i] = sK[o] * XK[tb][i] + sB[o] * XB[tb][i] - sR[o] * XR[tb][i] -
                               sA[o] * XA[tb][i];
                }
                sScan[wave][(4 * tb + g) * 16 + l16] = ((f[tb][0] + f[tb][1]) + f[tb][2]) + f[tb][3];
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            float blk[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) blk[q] = sScan[wave][q * 16 + l16];
            const float cj = sC[jw];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                float ex = 0.f;
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (q < 4 * tb + g) ex += blk[q];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * tb + 4 * g + i;
                    const int o = sw(t, jw);
                    const float gt = sG[o];
                    const float gp = t > 0 ? sG[sw(t - 1, jw)] : 1.f;
                    const float inv = 1.f / gt;
                    const float adA = sA[o] * XA[tb][i];
                    const float wdw = (cj + ex) - adA;
                    if (t < Lc) {
                        const int64_t off = vbase + (t0 + t) * stride + jw;
                        p.dk[off] = XK[tb][i] * inv;
                        p.db[off] = XB[tb][i] * inv;
                        p.dr[off] = XR[tb][i] * gt;
                        p.da[off] = XA[tb][i] * gp;
                        p.dw[off] = wdw * gp * inv;
                        p.dv[off] = XV[tb][i];
                    }
                    ex += f[tb][i];
                }
            }
        }
        __syncthreads();
    }

    if (bad) sBad = 1;
    __syncthreads();
    if (tid == 0) p.flags[bh] = sBad;
}

template <typename TIn>
hipError_t launch_bwdc_t(const BwdLaunch &a, int *flags, hipStream_t stream)
{
    BwdcArgs<TIn> p;
    p.r = static_cast<const TIn *>(a.in[0]);
    p.w = static_cast<const TIn *>(a.in[1]);
    p.k = static_cast<const TIn *>(a.in[2]);
    p.v = static_cast<const TIn *>(a.in[3]);
    p.a = static_cast<const TIn *>(a.in[4]);
    p.b = static_cast<const TIn *>(a.in[5]);
    p.dy = static_cast<const TIn *>(a.in[6]);
    p.sa = a.satape;
    p.ckpt = a.ckpt;
    p.dsT = a.dsT;
    p.dr = a.grad[0];
    p.dw = a.grad[1];
    p.dk = a.grad[2];
    p.dv = a.grad[3];
    p.da = a.grad[4];
    p.db = a.grad[5];
    p.ds0 = a.ds0;
    p.flags = flags;
    p.T = a.T;
    p.H = a.H;
    p.nck = (int)((a.T + 63) / 64);
    hipLaunchKernelGGL((wkv7_bwdc_kernel<TIn>), dim3((unsigned)(a.B * a.H)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool chunked_backward_supported(const BwdLaunch &a)
{
    return a.N == 64 && a.chunk == 64 && a.T > 0;
}

hipError_t launch_backward_chunked(const BwdLaunch &a, int *flags, hipStream_t stream)
{
    return a.dtype == 0 ? launch_bwdc_t<float>(a, flags, stream)
                        : launch_bwdc_t<uint16_t>(a, flags, stream);
}

}  // namespace wkv7
