// RWKV-8 rho / rho_norm recurrence with normalised pre-update readout
// (burn_dragon_kernel page src/sequence/rwkv8/backward.rs), forward and
// backward for latent and embedding size 64, on fp32 matrix cores.
//
// Per (b, h), with R the rho state [l][e], n the rho_norm [l], d the head's
// decay [l], EPS = 1e-6:
//   c_t = q_t / (sum q_t + EPS) / (n_t + EPS),  y_t = R_t^T c_t,
//   R_{t+1} = diag(d) R_t + q_t v_t^T,  n_{t+1} = d n_t + q_t.
// Over a tile of S = 16 steps starting from R0, with p_u = d^u (per row l),
// chat_t = c_t p_t and qhat_u = q_u / p_{u+1}, the states are
// R_t = diag(p_t) (R0 + sum_{u<t} qhat_u v_u^T), so that
//   Y = Chat R0 + M V,  M[t][u] = chat_t . qhat_u (u < t),
//   R_S = diag(p_S) (R0 + Qhat^T V):
// dense 16 x 64 x 64 products plus one 16 x 16 Gram per tile.  n and c are
// a per-latent scalar recurrence, formed per 64-step chunk on the VALU.
//
// The backward takes the same tiles in reverse.  With G = dL/dR at the
// tile's end, Ghat = diag(p_S) G and W[t][u] = dy_t . v_u (u < t):
//   dV    = M^T dY + Qhat Ghat
//   dQhat = W^T Chat + V Ghat^T,   dChat = dY R0^T + W Qhat
//   dL/dR0 = Chat^T dY + Ghat      (the G of the tile before)
//   d dL/dd = sum_t t chat_t o dChat_t - sum_u (u+1) qhat_u o dQhat_u
//             + S sum_e Ghat o (R0 + Qhat^T V)         (through p; per latent)
// then dc = dChat p, dq = dQhat / p + the readout weights' and rho_norm's
// chain (a per-latent reverse scan), as the page's backward_chunk_impl.
//
// The rescaling needs p_S and 1 / p_S inside fp32's normal range: every
// decay of a head must lie in [2^-7, 1].  A head outside it writes NaN to
// all its outputs and sets a bit of the device's fault word.

#include <stdint.h>

#include "rwkv8.h"
#include "wkv7_internal.h"

namespace {

constexpr int kN = 64;                     // latent = embedding size
constexpr int kCk = 64;                    // steps per checkpoint (chunk)
constexpr int kS = 16;                     // steps per tile
constexpr int kThreads = 256;
constexpr float kEps = 1e-6f;
constexpr float kDecayMin = 0.0078125f;    // 2^-7
constexpr int kRec = kN * kN + kN;         // floats per checkpoint block
constexpr int kMs = 17;                    // row stride of the 16 x 16 Grams

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(float a, float b, f4 c)
{
    // D[m][n] += A[m][k] B[k][n] over a 16x16x4 block: lane l supplies
    // A[l % 16][l / 16] and B[l / 16][l % 16] and holds D[4 (l / 16) + i][l % 16].
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// [64][64] fp32 LDS arrays with the 16-byte groups of row r XOR-swizzled by
// f(r) = 4 ((r ^ (r >> 2)) & 3) + (r & 3): reads of 16 rows x one group, of
// 4 rows spaced by 1 or by 4 x 16 columns, meet distinct banks.
__device__ __forceinline__ int xs(int r, int col)
{
    const int f = ((((r ^ (r >> 2)) & 3) << 2) | (r & 3));
    return (r << 6) + ((((col >> 2) ^ f) & 15) << 2) + (col & 3);
}

// 16 x 16 fp32 LDS matrices, the 16-byte groups of row t XOR-swizzled by
// (t >> 2) & 3: reads of elements 4 g .. 4 g + 3 of rows 0..15 meet distinct
// banks.
__device__ __forceinline__ int gm(int t, int u)
{
    return (t << 4) + ((((u >> 2) ^ (t >> 2)) & 3) << 2) + (u & 3);
}

__device__ __forceinline__ float4 lds4(const float *s, int o)
{
    return *reinterpret_cast<const float4 *>(s + o);
}

__device__ __forceinline__ void st4(float *s, int o, float4 v)
{
    *reinterpret_cast<float4 *>(s + o) = v;
}

__device__ __forceinline__ float el(const float4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float powi(float x, int k)
{
    float r = 1.f;
    for (int i = 0; i < k; ++i) r *= x;
    return r;
}

// Stage rows [0, 64) of a [T][64] slice starting at step tc into LDS,
// zeros past nst valid rows.
__device__ __forceinline__ void stage(float *dst, const float *src, int64_t tc, int nst, int tid)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = tid + kThreads * k, row = idx >> 4, col = (idx & 15) << 2;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < nst) x = *reinterpret_cast<const float4 *>(src + (tc + row) * kN + col);
        st4(dst, xs(row, col), x);
    }
}

// Per chunk: sigma_t = sum_l q_t[l] + EPS; then wave w takes tile w and
// lane l latent l: n_t from the chunk's start (the tiles before w combined
// through their increments), c_t = q_t / (sigma_t (n_t + EPS)),
// chat_t = c_t d^u and qhat_t = q_t d^-(u+1) (u = t - 16 w), qhat written
// over q.  nst: valid steps.  nts (optional) receives n at every tile
// start, nend the n after the last valid step.  Contains one barrier; the
// caller synchronises before and after.
__device__ __forceinline__ void prep_chunk(float *Qs, float *Cs, float *sig, float *dlt,
                                           const float *nch, float *nts, float *nend, float dl,
                                           float inv_dl, float p16l, int nst, int tid)
{
    const int lane = tid & 63, w = tid >> 6;
    {
        const int t = tid >> 2, part = tid & 3;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 x = lds4(Qs, xs(t, 16 * part + 4 * j));
            s += (x.x + x.y) + (x.z + x.w);
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        if (part == 0) sig[t] = s + kEps;
    }
    {
        float acc = 0.f;
        for (int u = 0; u < kS; ++u) {
            const int t = kS * w + u;
            if (t < nst) acc = fmaf(dl, acc, Qs[xs(t, lane)]);
        }
        dlt[w * kN + lane] = acc;
    }
    __syncthreads();
    float n = nch[lane];
    for (int k = 0; k < w; ++k) n = fmaf(p16l, n, dlt[k * kN + lane]);
    if (nts) nts[w * kN + lane] = n;
    float pw = 1.f, ip = 1.f;
    for (int u = 0; u < kS; ++u) {
        const int t = kS * w + u;
        const int o = xs(t, lane);
        const float q = Qs[o];
        const float cv = q * __builtin_amdgcn_rcpf(sig[t] * (n + kEps));
        ip *= inv_dl;
        Cs[o] = cv * pw;
        Qs[o] = q * ip;
        if (t < nst) n = fmaf(dl, n, q);
        pw *= dl;
    }
    if (w == ((nst - 1) >> 4)) nend[lane] = n;
}

// out[t][u] (row stride kMs) = X_t . Y_u over the 64 columns for u < t, 0
// otherwise, for the 16 rows t0 .. t0 + 15 of two [64][64] LDS arrays.
__device__ __forceinline__ void gram_tile(const float *X, const float *Y, float *out, int t0, int lane)
{
    const int g = lane >> 4, c = lane & 15;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const float4 a = lds4(X, xs(t0 + c, 16 * s + 4 * g));
        const float4 b = lds4(Y, xs(t0 + c, 16 * s + 4 * g));
        acc = mfma(a.x, b.x, acc);
        acc = mfma(a.y, b.y, acc);
        acc = mfma(a.z, b.z, acc);
        acc = mfma(a.w, b.w, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(4 * g + i) * kMs + c] = c < 4 * g + i ? acc[i] : 0.f;
}

__device__ __forceinline__ bool decay_ok(float d)
{
    return d >= kDecayMin && d <= 1.f;   // false for NaN
}

__device__ void poison(float *p, int64_t n, int tid, int nthreads = kThreads)
{
    if (!p) return;
    const float nan = __builtin_nanf("");
    for (int64_t i = tid; i < n; i += nthreads) p[i] = nan;
}

struct FwdArgs {
    const float *q, *v, *decay, *rho0, *norm0;
    float *y, *rhoT, *normT, *ckpt;
    int64_t T, H, Hv;
    int nck;
    unsigned *fault;
};

constexpr int kFwdThreads = 512;   // 4 consumer + 4 producer waves

// One workgroup of eight waves per (b, h).  Waves 0-3 ("consumers") hold R
// as accumulator tiles (wave w: columns 16 w .. 16 w + 15; element i of tile
// lb: row 16 lb + 4 (lane / 16) + i, column 16 w + lane % 16), so the tiles
// of a chunk need no exchange between waves, and run the four tiles of
// chunk cc.  Waves 4-7 ("producers") meanwhile prepare chunk cc + 1,
// producer pw its tile pw (sigma, the rho_norm chain, chat, qhat and the
// tile's Gram), from the chunk's raw queries, which they staged during the
// chunk before (so that every producer sees all of them and runs the
// rho_norm chain itself, without waiting for the others), and stage chunk
// cc + 2.  All of a chunk's operands are in LDS, double-buffered by chunk
// parity; one barrier per chunk.  The products over the steps of a tile take
// step t0 + 4 g + kk in the K slot of row group g at step kk, so that qhat
// and v, kept transposed ([latent or embedding][step]), and the tile's Gram
// are read 16 bytes at a time.
__global__ void __launch_bounds__(kFwdThreads) rwkv8_fwd_kernel(FwdArgs p)
{
    __shared__ __align__(16) float Qr[2][kN * kN];   // raw q [t][l]
    __shared__ __align__(16) float Qt[2][kN * kN];   // qhat [l][t]
    __shared__ __align__(16) float Cs[2][kN * kN];   // chat [t][l]
    __shared__ __align__(16) float Vt[2][kN * kN];   // v [e][t]
    __shared__ __align__(16) float Qp[4][kS * kN];   // qhat of producer pw's tile [u][l]
    __shared__ __align__(16) float Ms[2][4][kS * kS];   // the tiles' Grams, gm layout
    __shared__ float sig[4][kS];                     // sigma of producer pw's tile
    __shared__ int bad;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
    const int64_t bh = blockIdx.x, H = p.H, T = p.T;
    const int64_t b = bh / H, h = bh % H;
    const int nck = p.nck;
    const float *qg = p.q + bh * T * kN;
    const float *vg = p.v + (b * p.Hv + (p.Hv == 1 ? 0 : h)) * T * kN;
    float *yg = p.y ? p.y + bh * T * kN : nullptr;
    const float *dec = p.decay + h * kN;
    auto steps = [&](int cc) {
        const int64_t rem = T - (int64_t)cc * kCk;
        return (int)(rem < kCk ? rem : kCk);
    };

    if (tid == 0) bad = 0;
    __syncthreads();
    if (w == 0 && !decay_ok(dec[lane])) bad = 1;
    __syncthreads();
    if (bad) {
        poison(yg, T * kN, tid, kFwdThreads);
        poison(p.rhoT ? p.rhoT + bh * kN * kN : nullptr, kN * kN, tid, kFwdThreads);
        poison(p.normT ? p.normT + bh * kN : nullptr, kN, tid, kFwdThreads);
        poison(p.ckpt ? p.ckpt + bh * nck * kRec : nullptr, (int64_t)nck * kRec, tid, kFwdThreads);
        if (tid == 0) __hip_atomic_fetch_or(p.fault, (unsigned)WKV7_FAULT_RWKV8_DECAY, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    if (w < 4) {
        // ================= consumers =================
        // the decays of this lane's state rows and their 16th powers
        float dr[4][4], p16r[4][4];
        f4 Racc[4];
#pragma unroll
        for (int lb = 0; lb < 4; ++lb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int l = 16 * lb + 4 * g + i;
                const float x = dec[l];
                float x16 = x * x;
                x16 *= x16;
                x16 *= x16;
                x16 *= x16;
                dr[lb][i] = x;
                p16r[lb][i] = x16;
                Racc[lb][i] = p.rho0 ? p.rho0[bh * kN * kN + l * kN + 16 * w + c] : 0.f;
            }
        __syncthreads();   // chunk 0 staged (and chunk 1's queries)
        __syncthreads();   // chunk 0 prepared
        for (int cc = 0; cc < nck; ++cc) {
            const int bb = cc & 1;
            const int64_t tc = (int64_t)cc * kCk;
            const int nst = steps(cc);
            const float *C = Cs[bb], *Q = Qt[bb], *V = Vt[bb];
            if (p.ckpt) {   // the state before this chunk (rho part)
                float *ck = p.ckpt + (bh * nck + cc) * kRec;
#pragma unroll
                for (int lb = 0; lb < 4; ++lb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ck[(16 * lb + 4 * g + i) * kN + 16 * w + c] = Racc[lb][i];
            }
            for (int k = 0; k < 4; ++k) {
                const int t0 = kS * k;
                if (t0 >= nst) break;
                const int ns = nst - t0 < kS ? nst - t0 : kS;
                // v of steps t0 + 4 g .. + 3, column 16 w + c
                const float4 v4 = lds4(V, xs(16 * w + c, t0 + 4 * g));
                if (yg) {
                    // Y = Chat R0 + M V for columns 16 w ..: rows t0 + 4 g + i
                    const float4 m4 = lds4(Ms[bb][k], gm(c, 4 * g));
                    f4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int lb = 0; lb < 4; ++lb) {
                        const float4 a = lds4(C, xs(t0 + c, 16 * lb + 4 * g));
                        Y = mfma(a.x, Racc[lb][0], Y);
                        Y = mfma(a.y, Racc[lb][1], Y);
                        Y = mfma(a.z, Racc[lb][2], Y);
                        Y = mfma(a.w, Racc[lb][3], Y);
                    }
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) Y = mfma(el(m4, kk), el(v4, kk), Y);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = t0 + 4 * g + i;
                        if (t < nst) yg[(tc + t) * kN + 16 * w + c] = Y[i];
                    }
                }
                // R <- diag(p_ns) (R + Qhat^T V)
#pragma unroll
                for (int lb = 0; lb < 4; ++lb) {
                    const float4 q4 = lds4(Q, xs(16 * lb + c, t0 + 4 * g));
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) Racc[lb] = mfma(el(q4, kk), el(v4, kk), Racc[lb]);
                }
                if (ns == kS) {
#pragma unroll
                    for (int lb = 0; lb < 4; ++lb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) Racc[lb][i] *= p16r[lb][i];
                } else {
#pragma unroll
                    for (int lb = 0; lb < 4; ++lb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) Racc[lb][i] *= powi(dr[lb][i], ns);
                }
            }
            __syncthreads();   // chunk cc consumed, chunk cc + 1 prepared
        }
        if (p.rhoT) {
#pragma unroll
            for (int lb = 0; lb < 4; ++lb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p.rhoT[bh * kN * kN + (16 * lb + 4 * g + i) * kN + 16 * w + c] = Racc[lb][i];
        }
        return;
    }

    // ================= producers =================
    const int pw = w - 4, t0 = kS * pw;
    const float dl = dec[lane];   // lane = latent
    const float inv_dl = 1.f / dl;
    float n_carry = p.norm0 ? p.norm0[bh * kN + lane] : 0.f;   // n at the start of the next chunk to prepare
    // rows 16 pw + 4 k + lane / 16, columns 4 (lane % 16) .. + 3 of a chunk
    const int srow = t0 + (lane >> 4), scol = 4 * (lane & 15);
    float4 qx[4], vx[4], vnext[4];
    auto issue = [&](int cc, float4 (&qo)[4], float4 (&vo)[4]) {
        const int64_t tc = (int64_t)cc * kCk;
        const int nst = steps(cc);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = srow + 4 * k;
            qo[k] = vo[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row < nst) {
                qo[k] = *reinterpret_cast<const float4 *>(qg + (tc + row) * kN + scol);
                vo[k] = *reinterpret_cast<const float4 *>(vg + (tc + row) * kN + scol);
            }
        }
    };
    auto put = [&](float *dst, const float4 (&x)[4]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) st4(dst, xs(srow + 4 * k, scol), x[k]);
    };
    auto put_t = [&](float *dst, const float4 (&x)[4]) {   // transposed: [column][step]
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[xs(scol + i, srow + 4 * k)] = el(x[k], i);
    };
    // chunk X from its raw queries in Qr[X & 1]: this producer's tile
    auto prep = [&](int X) {
        const int xb = X & 1;
        const int nst = steps(X);
        const float *Q = Qr[xb];
        {   // sigma of the tile's steps: lane (step t0 + lane / 4, quarter lane % 4)
            const int t = t0 + (lane >> 2), part = lane & 3;
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 x = lds4(Q, xs(t, 16 * part + 4 * j));
                s += (x.x + x.y) + (x.z + x.w);
            }
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            if (part == 0) sig[pw][lane >> 2] = s + kEps;
        }
        if (pw == 0 && p.ckpt) p.ckpt[(bh * nck + X) * kRec + kN * kN + lane] = n_carry;
        // the rho_norm chain over the chunk (the queries of each other tile
        // read together, then its steps); c, chat, qhat on this tile
        auto chain16 = [&](int tt, float &n) {
            float qv[kS];
#pragma unroll
            for (int u = 0; u < kS; ++u) qv[u] = Q[xs(kS * tt + u, lane)];
#pragma unroll
            for (int u = 0; u < kS; ++u)
                if (kS * tt + u < nst) n = fmaf(dl, n, qv[u]);
        };
        float n = n_carry;
        for (int tt = 0; tt < pw; ++tt) chain16(tt, n);
        float pu = 1.f, ip = 1.f, qh[kS];
#pragma unroll
        for (int u = 0; u < kS; ++u) {
            const int t = t0 + u, o = xs(t, lane);
            const float q = Q[o];
            const float cv = q * __builtin_amdgcn_rcpf(sig[pw][u] * (n + kEps));
            ip *= inv_dl;
            Cs[xb][o] = cv * pu;
            qh[u] = q * ip;
            Qp[pw][xs(u, lane)] = qh[u];
            if (t < nst) n = fmaf(dl, n, q);
            pu *= dl;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            st4(Qt[xb], xs(lane, t0 + 4 * j), make_float4(qh[4 * j], qh[4 * j + 1], qh[4 * j + 2], qh[4 * j + 3]));
        for (int tt = pw + 1; tt < kCk / kS; ++tt) chain16(tt, n);
        n_carry = n;
        if (yg) {   // M[t][u] = chat_t . qhat_u (u < t) over the tile: lane (g, c) holds M[4 g + i][c]
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const float4 a = lds4(Cs[xb], xs(t0 + c, 16 * s4 + 4 * g));
                const float4 b = lds4(Qp[pw], xs(c, 16 * s4 + 4 * g));
                acc = mfma(a.x, b.x, acc);
                acc = mfma(a.y, b.y, acc);
                acc = mfma(a.z, b.z, acc);
                acc = mfma(a.w, b.w, acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) Ms[xb][pw][gm(4 * g + i, c)] = c < 4 * g + i ? acc[i] : 0.f;
        }
    };

    // chunk 0 and the queries of chunk 1; v of chunk 1 waits in registers
    issue(0, qx, vx);
    put(Qr[0], qx);
    put_t(Vt[0], vx);
    if (nck > 1) {
        issue(1, qx, vnext);
        put(Qr[1], qx);
    }
    __syncthreads();   // chunk 0 staged (and chunk 1's queries)
    prep(0);
    __syncthreads();   // chunk 0 prepared
    for (int cc = 0; cc < nck; ++cc) {
        // during chunk cc: chunk cc + 1's values into their buffer (free since
        // chunk cc - 1), chunk cc + 1 prepared, chunk cc + 2 staged
        const bool has2 = cc + 2 < nck;
        if (has2) issue(cc + 2, qx, vx);
        if (cc + 1 < nck) {
            put_t(Vt[(cc + 1) & 1], vnext);
            prep(cc + 1);
        }
        if (has2) {
            put(Qr[cc & 1], qx);
#pragma unroll
            for (int k = 0; k < 4; ++k) vnext[k] = vx[k];
        }
        __syncthreads();   // chunk cc consumed, chunk cc + 1 prepared
    }
    if (p.normT && pw == 0) p.normT[bh * kN + lane] = n_carry;
}

struct BwdArgs {
    const float *q, *v, *decay, *dy, *drhoT, *dnormT, *ckpt;
    float *dq, *dv, *ddpart, *drho0, *dnorm0;   // dv: per head, [B][H][T][64]
    int64_t T, H, Hv;
    int nck;
    unsigned *fault;
};

// One workgroup per (b, h); wave w holds rows 16 w .. 16 w + 15 of the
// states R0 of a chunk's four tiles and of G = dL/dR, transposed, as
// accumulator tiles (element i of tile j: row 16 w + lane % 16, column
// 16 j + 4 (lane / 16) + i), which are also the B operands of the products
// over the embedding index.  Per tile one exchange (Ghat through LDS, for
// dV); the readout weights' and rho_norm's chain runs per chunk, wave w on
// tile w, lane l on latent l.
__global__ void __launch_bounds__(kThreads) rwkv8_bwd_kernel(BwdArgs p)
{
    __shared__ __align__(16) float Qs[kN * kN];     // q, then qhat
    __shared__ __align__(16) float Vs[kN * kN];
    __shared__ __align__(16) float Ys[kN * kN];     // dy
    __shared__ __align__(16) float Cs[kN * kN];     // chat
    __shared__ __align__(16) float Gs[2][kN * kN];  // Ghat [l][e], by tile parity
    __shared__ __align__(16) float DCs[kN * kN];    // dL/dc per (t, l)
    __shared__ __align__(16) float DQs[kN * kN];    // dL/dq through qhat per (t, l)
    __shared__ float Ms[4][kS * kMs], Ws[4][kS * kMs];
    __shared__ float sig[kN], dlt[4 * kN], nch[kN], nend[kN], nts[4 * kN], lam[4 * kN];
    __shared__ float gnin[kN], gnext[kN], ssum[4][kS], ddl[kN];
    __shared__ int bad;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
    const int64_t bh = blockIdx.x, H = p.H, T = p.T;
    const int64_t b = bh / H, h = bh % H;
    const float *qg = p.q + bh * T * kN;
    const float *vg = p.v + (b * p.Hv + (p.Hv == 1 ? 0 : h)) * T * kN;
    const float *yg = p.dy + bh * T * kN;
    float *dqg = p.dq + bh * T * kN;
    float *dvg = p.dv + bh * T * kN;
    const float *dec = p.decay + h * kN;

    const float dl = dec[lane];   // finisher and prep: lane = latent
    if (tid == 0) bad = 0;
    __syncthreads();
    if (w == 0 && !decay_ok(dl)) bad = 1;
    __syncthreads();
    if (bad) {
        poison(dqg, T * kN, tid);
        poison(dvg, T * kN, tid);
        poison(p.ddpart + bh * kN, kN, tid);
        poison(p.drho0 ? p.drho0 + bh * kN * kN : nullptr, kN * kN, tid);
        poison(p.dnorm0 ? p.dnorm0 + bh * kN : nullptr, kN, tid);
        if (tid == 0) __hip_atomic_fetch_or(p.fault, (unsigned)WKV7_FAULT_RWKV8_DECAY, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const float inv_dl = 1.f / dl;
    float p16l = dl * dl;
    p16l *= p16l;
    p16l *= p16l;
    p16l *= p16l;
    // the decay of this lane's column l = 16 w + c of the transposed tiles,
    // its 16th power, d^(4g + i) and d^-(4g + i + 1)
    const float dc_ = dec[16 * w + c];
    const float inv_dc = 1.f / dc_;
    float p16c = dc_ * dc_;
    p16c *= p16c;
    p16c *= p16c;
    p16c *= p16c;
    float pw[4], ipw[4];
    {
        float x = powi(dc_, 4 * g), y = powi(inv_dc, 4 * g + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pw[i] = x;
            ipw[i] = y;
            x *= dc_;
            y *= inv_dc;
        }
    }

    f4 Gt[4], Rt[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (p.drhoT) {
            const float4 x = *reinterpret_cast<const float4 *>(p.drhoT + bh * kN * kN + (16 * w + c) * kN + 16 * j + 4 * g);
            Gt[j] = f4{x.x, x.y, x.z, x.w};
        } else {
            Gt[j] = f4{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (w == 0) gnin[lane] = p.dnormT ? p.dnormT[bh * kN + lane] : 0.f;
    float ddm = 0.f;   // d * dL/dd through p, column 16 w + c, this lane's rows
    float ddn = 0.f;   // dL/dd through rho_norm, latent `lane`, this wave's tiles

    for (int cc = p.nck - 1; cc >= 0; --cc) {
        const int64_t tc = (int64_t)cc * kCk;
        const int nst = (int)(T - tc < kCk ? T - tc : kCk);
        __syncthreads();   // the later chunk is done with every LDS array
        stage(Qs, qg, tc, nst, tid);
        stage(Vs, vg, tc, nst, tid);
        stage(Ys, yg, tc, nst, tid);
        const float *ck = p.ckpt + (bh * p.nck + cc) * kRec;
        if (w == 0) nch[lane] = ck[kN * kN + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 x = *reinterpret_cast<const float4 *>(ck + (16 * w + c) * kN + 16 * j + 4 * g);
            Rt[0][j] = f4{x.x, x.y, x.z, x.w};
        }
        __syncthreads();
        prep_chunk(Qs, Cs, sig, dlt, nch, nts, nend, dl, inv_dl, p16l, nst, tid);
        __syncthreads();
        gram_tile(Cs, Qs, Ms[w], kS * w, lane);
        gram_tile(Ys, Vs, Ws[w], kS * w, lane);
        // the states at the starts of tiles 1 .. 3 (own rows)
#pragma unroll
        for (int k = 0; k < 3; ++k) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f4 acc = Rt[k][j];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc = mfma(Vs[xs(kS * k + 4 * kk + g, 16 * j + c)], Qs[xs(kS * k + 4 * kk + g, 16 * w + c)], acc);
                Rt[k + 1][j] = acc * p16c;
            }
        }
        __syncthreads();   // Grams in LDS
        // (a rolled loop: unrolled, the compiler keeps too much live)
#pragma unroll 1
        for (int k = 3; k >= 0; --k) {
            const int t0 = kS * k;
            if (t0 >= nst) continue;
            const int ns = nst - t0 < kS ? nst - t0 : kS;
            const float pn = ns == kS ? p16c : powi(dc_, ns);
            f4 Rk[4];   // the state before tile k (k is uniform: a scalar branch)
            switch (k) {
            case 0: Rk[0] = Rt[0][0]; Rk[1] = Rt[0][1]; Rk[2] = Rt[0][2]; Rk[3] = Rt[0][3]; break;
            case 1: Rk[0] = Rt[1][0]; Rk[1] = Rt[1][1]; Rk[2] = Rt[1][2]; Rk[3] = Rt[1][3]; break;
            case 2: Rk[0] = Rt[2][0]; Rk[1] = Rt[2][1]; Rk[2] = Rt[2][2]; Rk[3] = Rt[2][3]; break;
            default: Rk[0] = Rt[3][0]; Rk[1] = Rt[3][1]; Rk[2] = Rt[3][2]; Rk[3] = Rt[3][3]; break;
            }
            float *Gk = Gs[k & 1];
            f4 Gh[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                Gh[j] = Gt[j] * pn;
                st4(Gk, xs(16 * w + c, 16 * j + 4 * g), make_float4(Gh[j][0], Gh[j][1], Gh[j][2], Gh[j][3]));
            }
            __syncthreads();   // Ghat of this tile in LDS
            {   // dV, columns 16 w ..: rows t0 + 4 g + i
                f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc = mfma(Ms[k][(4 * kk + g) * kMs + c], Ys[xs(t0 + 4 * kk + g, 16 * w + c)], acc);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float4 a = lds4(Qs, xs(t0 + c, 16 * s + 4 * g));
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc = mfma(el(a, i), Gk[xs(16 * s + 4 * g + i, 16 * w + c)], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = t0 + 4 * g + i;
                    if (t < nst) dvg[(tc + t) * kN + 16 * w + c] = acc[i];
                }
            }
            __builtin_amdgcn_sched_barrier(0);   // keep each product's operand loads with it
            {   // dQhat for latents 16 w ..: rows t0 + 4 g + i
                f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 a = lds4(Vs, xs(t0 + c, 16 * j + 4 * g));
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc = mfma(el(a, i), Gh[j][i], acc);
                }
                float qh[4], endt = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qh[i] = Qs[xs(t0 + 4 * g + i, 16 * w + c)];
                    endt = fmaf(qh[i], acc[i], endt);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) endt = fmaf(Gh[j][i], Rk[j][i], endt);
                ddm = fmaf((float)ns, endt, ddm);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc = mfma(Ws[k][(4 * kk + g) * kMs + c], Cs[xs(t0 + 4 * kk + g, 16 * w + c)], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ddm = fmaf(-(float)(4 * g + i + 1) * qh[i], acc[i], ddm);
                    DQs[xs(t0 + 4 * g + i, 16 * w + c)] = acc[i] * ipw[i];
                }
            }
            __builtin_amdgcn_sched_barrier(0);   // keep each product's operand loads with it
            {   // dChat for latents 16 w ..: rows t0 + 4 g + i
                f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 a = lds4(Ys, xs(t0 + c, 16 * j + 4 * g));
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc = mfma(el(a, i), Rk[j][i], acc);
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc = mfma(Ws[k][c * kMs + 4 * kk + g], Qs[xs(t0 + 4 * kk + g, 16 * w + c)], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ch = Cs[xs(t0 + 4 * g + i, 16 * w + c)];
                    ddm = fmaf((float)(4 * g + i) * ch, acc[i], ddm);
                    DCs[xs(t0 + 4 * g + i, 16 * w + c)] = acc[i] * pw[i];
                }
            }
            __builtin_amdgcn_sched_barrier(0);   // keep each product's operand loads with it
            // G <- Chat^T dY + Ghat (own rows, transposed)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f4 acc = Gh[j];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc = mfma(Ys[xs(t0 + 4 * kk + g, 16 * j + c)], Cs[xs(t0 + 4 * kk + g, 16 * w + c)], acc);
                Gt[j] = acc;
            }
        }
        __syncthreads();   // DCs, DQs of the chunk complete

        // readout weights and rho_norm: wave w on tile w, lane l on latent l.
        // First pass (forward in t): n_t, gw_t = dL/dc_t / (n_t + EPS) and
        // x_t = -gw_t c_t (dL/dn_t through c) parked in the arrays the tiles
        // no longer need (Cs, Vs, Ys); the products gw_t q_t / sigma_t summed
        // over latents; the tile's rho_norm gradient from zero.
        const int t0 = kS * w;
        const int ns = t0 < nst ? (nst - t0 < kS ? nst - t0 : kS) : 0;
        {
            float pr[kS];
            float n = nts[w * kN + lane], pwr = 1.f, lm = 0.f, pl = 1.f;
            // the tile's operands, read ahead of the chain through n
            float qv[kS], dcv[kS], rsv[kS];
#pragma unroll
            for (int u = 0; u < kS; ++u) {
                const int t = t0 + u, o = xs(t, lane);
                qv[u] = Qs[o];
                dcv[u] = DCs[o];
                rsv[u] = __builtin_amdgcn_rcpf(sig[t]);
            }
#pragma unroll
            for (int u = 0; u < kS; ++u) {
                pr[u] = 0.f;
                if (u < ns) {
                    const int t = t0 + u, o = xs(t, lane);
                    pwr *= dl;
                    const float q = qv[u] * pwr;
                    const float rne = __builtin_amdgcn_rcpf(n + kEps);
                    const float gw = dcv[u] * rne;
                    const float qs = q * rsv[u];
                    const float x = -gw * (qs * rne);
                    Cs[o] = n;
                    Vs[o] = gw;
                    Ys[o] = x;
                    pr[u] = gw * qs;
                    lm = fmaf(pl, x, lm);   // sum_u d^u x_u
                    pl *= dl;
                    n = fmaf(dl, n, q);
                }
            }
            // ssum[w][u] = sum over the 64 latents of pr[u]: halve the
            // vector across lane bits 3 .. 0, then add across bits 4 and 5
            float v8[8], v4[4], v2[2];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool up = lane & 8;
                const float send = up ? pr[i] : pr[i + 8], keep = up ? pr[i + 8] : pr[i];
                v8[i] = keep + __shfl_xor(send, 8);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool up = lane & 4;
                const float send = up ? v8[i] : v8[i + 4], keep = up ? v8[i + 4] : v8[i];
                v4[i] = keep + __shfl_xor(send, 4);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bool up = lane & 2;
                const float send = up ? v4[i] : v4[i + 2], keep = up ? v4[i + 2] : v4[i];
                v2[i] = keep + __shfl_xor(send, 2);
            }
            float v1;
            {
                const bool up = lane & 1;
                const float send = up ? v2[0] : v2[1], keep = up ? v2[1] : v2[0];
                v1 = keep + __shfl_xor(send, 1);
            }
            v1 += __shfl_xor(v1, 16);
            v1 += __shfl_xor(v1, 32);
            if (lane < kS) ssum[w][lane] = v1;
            lam[w * kN + lane] = lm;
        }
        __syncthreads();
        if (ns > 0) {
            // dL/dn at the end of tile w, from the chunk's end through the
            // later tiles; then the tile backwards
            float Gn = gnin[lane];
            for (int k = 3; k > w; --k) {
                const int tk = kS * k;
                if (tk >= nst) continue;
                const int nk = nst - tk < kS ? nst - tk : kS;
                Gn = fmaf(nk == kS ? p16l : powi(dl, nk), Gn, lam[k * kN + lane]);
            }
            for (int u = ns - 1; u >= 0; --u) {
                const int t = t0 + u, o = xs(t, lane);
                const float dqv = DQs[o] + (Vs[o] - ssum[w][u]) * __builtin_amdgcn_rcpf(sig[t]) + Gn;
                dqg[(tc + t) * kN + lane] = dqv;
                ddn = fmaf(Gn, Cs[o], ddn);
                Gn = fmaf(dl, Gn, Ys[o]);
            }
            if (w == 0) gnext[lane] = Gn;
        }
        __syncthreads();
        if (w == 0) gnin[lane] = gnext[lane];
    }

    // outputs: dL/dR0, dL/dn0 and this (b, h)'s share of the decay gradient
    if (p.drho0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float4 *>(p.drho0 + bh * kN * kN + (16 * w + c) * kN + 16 * j + 4 * g) =
                make_float4(Gt[j][0], Gt[j][1], Gt[j][2], Gt[j][3]);
    }
    ddm += __shfl_xor(ddm, 16);
    ddm += __shfl_xor(ddm, 32);
    lam[w * kN + lane] = ddn;
    if (g == 0) ddl[16 * w + c] = ddm * inv_dc;
    __syncthreads();
    if (w == 0) {
        const float s = ddl[lane] + ((lam[lane] + lam[kN + lane]) + (lam[2 * kN + lane] + lam[3 * kN + lane]));
        p.ddpart[bh * kN + lane] = s;
        if (p.dnorm0) p.dnorm0[bh * kN + lane] = gnin[lane];
    }
}

// dv[b][t][e] = sum over h of part[b][h][t][e], in order of h
__global__ void sum_heads_kernel(const float *part, float *dv, int64_t B, int64_t H, int64_t T)
{
    const int64_t n = B * T * kN;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = i / (T * kN), r = i % (T * kN);
        float s = 0.f;
        for (int64_t h = 0; h < H; ++h) s += part[(b * H + h) * T * kN + r];
        dv[i] = s;
    }
}

// dd[h][l] = sum over b of part[b][h][l], in order of b
__global__ void sum_batch_kernel(const float *part, float *dd, int64_t B, int64_t H)
{
    const int64_t n = H * kN;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float s = 0.f;
        for (int64_t b = 0; b < B; ++b) s += part[b * n + i];
        dd[i] = s;
    }
}

// ------------------------------------------------------------------ host

constexpr size_t kAlign = 256;

size_t round_up(size_t x)
{
    return (x + kAlign - 1) / kAlign * kAlign;
}

struct Dims {
    int64_t B, T, H, Hv, nck;
    size_t q_elems, v_elems, ck_bytes;
};

bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    return !__builtin_mul_overflow(a, b, out);
}

int check(const rwkv8_shape *s, Dims *d)
{
    if (!s) return WKV7_ERR_INVALID;
    if (s->B < 0 || s->T < 0 || s->H < 0 || s->L <= 0 || s->E <= 0) return WKV7_ERR_INVALID;
    if (s->Hv != 1 && s->Hv != s->H) return WKV7_ERR_INVALID;
    if (s->L != kN || s->E != kN) return WKV7_ERR_UNSUPPORTED;
    int64_t bh, bht, qe, ve, nck_bh, rec;
    if (!mul_ok(s->B, s->H, &bh) || bh > INT32_MAX) return WKV7_ERR_INVALID;
    if (!mul_ok(bh, s->T, &bht) || !mul_ok(bht, kN, &qe) || !mul_ok(qe, 4, &rec)) return WKV7_ERR_INVALID;
    if (!mul_ok(s->B * s->Hv, s->T * kN, &ve)) return WKV7_ERR_INVALID;
    const int64_t nck = (s->T + kCk - 1) / kCk;
    if (!mul_ok(bh, nck, &nck_bh) || !mul_ok(nck_bh, (int64_t)kRec * 4, &rec)) return WKV7_ERR_INVALID;
    d->B = s->B;
    d->T = s->T;
    d->H = s->H;
    d->Hv = s->Hv;
    d->nck = nck;
    d->q_elems = (size_t)qe;
    d->v_elems = (size_t)ve;
    d->ck_bytes = (size_t)rec;
    return WKV7_OK;
}

bool aligned(const void *p)
{
    return ((uintptr_t)p & 15u) == 0;
}

int status(hipError_t e)
{
    return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

size_t ws_bytes(const Dims &d, bool ckpt_provided)
{
    size_t n = round_up((size_t)(d.B * d.H) * kN * sizeof(float));
    if (d.Hv == 1) n += round_up(d.q_elems * sizeof(float));
    if (!ckpt_provided) n += round_up(d.ck_bytes);
    return n;
}

hipError_t launch_fwd(const Dims &d, const float *q, const float *v, const float *decay,
                      const float *rho0, const float *norm0, float *y, float *rhoT, float *normT,
                      float *ckpt, hipStream_t stream)
{
    FwdArgs a;
    a.q = q;
    a.v = v;
    a.decay = decay;
    a.rho0 = rho0;
    a.norm0 = norm0;
    a.y = y;
    a.rhoT = rhoT;
    a.normT = normT;
    a.ckpt = ckpt;
    a.T = d.T;
    a.H = d.H;
    a.Hv = d.Hv;
    a.nck = (int)d.nck;
    a.fault = wkv7::fault_word();
    if (!a.fault) return hipErrorInvalidDevicePointer;
    hipLaunchKernelGGL(rwkv8_fwd_kernel, dim3((unsigned)(d.B * d.H)), dim3(kFwdThreads), 0, stream, a);
    return hipGetLastError();
}

unsigned grid_for(int64_t n)
{
    const int64_t blocks = (n + 255) / 256;
    return (unsigned)(blocks < 4096 ? (blocks > 0 ? blocks : 1) : 4096);
}

}  // namespace

extern "C" {

size_t rwkv8_checkpoint_bytes(const rwkv8_shape *shape)
{
    Dims d;
    if (check(shape, &d) != WKV7_OK) return 0;
    return d.ck_bytes;
}

size_t rwkv8_backward_workspace_bytes(const rwkv8_shape *shape, int ckpt_provided)
{
    Dims d;
    if (check(shape, &d) != WKV7_OK || d.B * d.H == 0 || d.T == 0) return 0;
    return ws_bytes(d, ckpt_provided != 0);
}

int rwkv8_forward(const rwkv8_shape *shape, const float *q, const float *v, const float *decay,
                  const float *rho0, const float *norm0, float *y, float *rhoT, float *normT,
                  float *ckpt, hipStream_t stream)
{
    Dims d;
    const int rc = check(shape, &d);
    if (rc != WKV7_OK) return rc;
    if (d.B * d.H == 0) return WKV7_OK;
    for (const void *p : {(const void *)rho0, (const void *)norm0, (const void *)y, (const void *)rhoT,
                          (const void *)normT, (const void *)ckpt})
        if (!aligned(p)) return WKV7_ERR_INVALID;
    if (d.T == 0) {
        if (rhoT) {
            const int r = status(wkv7::launch_fill(rhoT, rho0, (size_t)(d.B * d.H) * kN * kN, stream));
            if (r != WKV7_OK) return r;
        }
        if (normT) return status(wkv7::launch_fill(normT, norm0, (size_t)(d.B * d.H) * kN, stream));
        return WKV7_OK;
    }
    for (const void *p : {(const void *)q, (const void *)v, (const void *)decay})
        if (!p || !aligned(p)) return WKV7_ERR_INVALID;
    return status(launch_fwd(d, q, v, decay, rho0, norm0, y, rhoT, normT, ckpt, stream));
}

int rwkv8_backward(const rwkv8_shape *shape, const float *q, const float *v, const float *decay,
                   const float *rho0, const float *norm0, const float *dy, const float *drhoT,
                   const float *dnormT, const float *ckpt, float *dq, float *dv, float *ddecay,
                   float *drho0, float *dnorm0, void *workspace, size_t workspace_bytes,
                   hipStream_t stream)
{
    Dims d;
    int rc = check(shape, &d);
    if (rc != WKV7_OK) return rc;
    if (d.B * d.H == 0) {
        if (d.H > 0 && ddecay && aligned(ddecay))
            return status(wkv7::launch_fill(ddecay, nullptr, (size_t)d.H * kN, stream));
        return d.H > 0 && (!ddecay || !aligned(ddecay)) ? WKV7_ERR_INVALID : WKV7_OK;
    }
    for (const void *p : {(const void *)rho0, (const void *)norm0, (const void *)drhoT,
                          (const void *)dnormT, (const void *)ckpt, (const void *)drho0,
                          (const void *)dnorm0})
        if (!aligned(p)) return WKV7_ERR_INVALID;
    if (!ddecay || !aligned(ddecay)) return WKV7_ERR_INVALID;
    if (d.T == 0) {
        if (drho0) {
            rc = status(wkv7::launch_fill(drho0, drhoT, (size_t)(d.B * d.H) * kN * kN, stream));
            if (rc != WKV7_OK) return rc;
        }
        if (dnorm0) {
            rc = status(wkv7::launch_fill(dnorm0, dnormT, (size_t)(d.B * d.H) * kN, stream));
            if (rc != WKV7_OK) return rc;
        }
        return status(wkv7::launch_fill(ddecay, nullptr, (size_t)d.H * kN, stream));
    }
    for (const void *p : {(const void *)q, (const void *)v, (const void *)decay, (const void *)dy,
                          (const void *)dq, (const void *)dv})
        if (!p || !aligned(p)) return WKV7_ERR_INVALID;
    const size_t need = ws_bytes(d, ckpt != nullptr);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign) != 0)
        return WKV7_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    float *ddpart = reinterpret_cast<float *>(ws);
    size_t off = round_up((size_t)(d.B * d.H) * kN * sizeof(float));
    float *dvpart = dv;
    if (d.Hv == 1) {
        dvpart = reinterpret_cast<float *>(ws + off);
        off += round_up(d.q_elems * sizeof(float));
    }
    const float *ck = ckpt;
    if (!ckpt) {
        float *own = reinterpret_cast<float *>(ws + off);
        rc = status(launch_fwd(d, q, v, decay, rho0, norm0, nullptr, nullptr, nullptr, own, stream));
        if (rc != WKV7_OK) return rc;
        ck = own;
    }
    BwdArgs a;
    a.q = q;
    a.v = v;
    a.decay = decay;
    a.dy = dy;
    a.drhoT = drhoT;
    a.dnormT = dnormT;
    a.ckpt = ck;
    a.dq = dq;
    a.dv = dvpart;
    a.ddpart = ddpart;
    a.drho0 = drho0;
    a.dnorm0 = dnorm0;
    a.T = d.T;
    a.H = d.H;
    a.Hv = d.Hv;
    a.nck = (int)d.nck;
    a.fault = wkv7::fault_word();
    if (!a.fault) return WKV7_ERR_HIP;
    hipLaunchKernelGGL(rwkv8_bwd_kernel, dim3((unsigned)(d.B * d.H)), dim3(kThreads), 0, stream, a);
    rc = status(hipGetLastError());
    if (rc != WKV7_OK) return rc;
    if (d.Hv == 1) {
        hipLaunchKernelGGL(sum_heads_kernel, dim3(grid_for(d.B * d.T * kN)), dim3(256), 0, stream,
                           dvpart, dv, d.B, d.H, d.T);
        rc = status(hipGetLastError());
        if (rc != WKV7_OK) return rc;
    }
    hipLaunchKernelGGL(sum_batch_kernel, dim3(grid_for(d.H * kN)), dim3(256), 0, stream, ddpart, ddecay,
                       d.B, d.H);
    return status(hipGetLastError());
}

}  // extern "C"
