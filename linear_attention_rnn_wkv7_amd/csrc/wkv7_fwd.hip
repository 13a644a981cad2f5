// WKV7 forward scan on gfx950.
//
// Computes, per (batch b, head h), the recurrence of rx_wkv7_forward_seq on
// the Foundry "rwkvx/rx_pretrain.c" page:
//   sa = S a;  S <- S diag(w) + v k^T + sa b^T;  y = S r
// Rows of S never interact (row i only reads the shared per-step vectors and
// its own v[i], sa[i]), so the state is tiled over lanes by rows and columns:
// each lane keeps an R x CC block of S in registers for the whole sequence,
// the LPR = N/CC lanes of one row group reduce their partial row dots with
// DPP, and the per-step vectors go HBM -> registers -> LDS in blocks of TB
// steps (prefetched one block ahead) and are read back as broadcasts.
// One workgroup holds one (b, h): N = 64 -> 4 waves of 16 rows.

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

template <int N> struct FwdTile;
template <> struct FwdTile<64> { static constexpr int R = 2, CC = 8; };
template <> struct FwdTile<16> { static constexpr int R = 1, CC = 4; };

template <int N>
struct FwdGeom {
    static constexpr int R = FwdTile<N>::R;
    static constexpr int CC = FwdTile<N>::CC;
    static constexpr int LPR = N / CC;              // lanes sharing a row
    static constexpr int RW = (kWave / LPR) * R;    // rows per wave
    static constexpr int NW = N / RW;               // waves per workgroup
    static constexpr int NT = NW * kWave;
    static constexpr int TB = 8;                    // steps per staged block
    static constexpr int NV = 6;                    // r, w, k, v, a, b
    static_assert(N % RW == 0 && CC % 4 == 0, "tile");
};

enum { kR = 0, kW = 1, kK = 2, kV = 3, kA = 4, kB = 5 };

template <typename TIn>
struct FwdArgs {
    VecPtrs<TIn, 6> in;
    const float *s0;
    float *y, *sT, *ckpt;
    int64_t T, H;
    int chunk, nck;
};

template <int N, typename TIn>
__global__ void __launch_bounds__(FwdGeom<N>::NT)
wkv7_fwd_kernel(FwdArgs<TIn> p)
{
    using Gm = FwdGeom<N>;
    constexpr int R = Gm::R, CC = Gm::CC, LPR = Gm::LPR, RW = Gm::RW, NT = Gm::NT;
    constexpr int TB = Gm::TB, NV = Gm::NV;
    __shared__ __align__(16) float lds[2][NV][TB][N];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = lane % LPR, rg = lane / LPR;
    const int row0 = wave * RW + rg * R, col0 = cg * CC;
    const int64_t bh = blockIdx.x, T = p.T, H = p.H;
    const int64_t b = bh / H, h = bh % H;
    const int64_t stride = H * N;                 // between time steps
    const int64_t vbase = (b * T * H + h) * N;    // step 0 of (b, h)

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

    Stager<TIn, NV, TB, N, NT> stage;
    const int64_t nblk = (T + TB - 1) / TB;
    if (nblk > 0) {
        const int n0 = (int)(T < TB ? T : TB);
        stage.issue(p.in, vbase, stride, n0, tid);
        stage.commit(&lds[0][0][0][0], n0, tid);
    }
    __syncthreads();

    for (int64_t blk = 0; blk < nblk; ++blk) {
        const int64_t t0 = blk * TB;
        const int nst = (int)((T - t0) < TB ? (T - t0) : TB);
        const bool more = blk + 1 < nblk;
        const int nnext = more ? (int)((T - t0 - TB) < TB ? (T - t0 - TB) : TB) : 0;
        if (more) stage.issue(p.in, vbase + (t0 + TB) * stride, stride, nnext, tid);

        // Checkpoint: the state before step t0 when t0 starts a chunk (the
        // chunk is a multiple of TB, so this is the only step it can be).
        if (p.ckpt && t0 % p.chunk == 0) {
            float *dst = p.ckpt + (bh * p.nck + t0 / p.chunk) * N * N + (int64_t)row0 * N + col0;
#pragma unroll
            for (int e = 0; e < R; ++e)
#pragma unroll
                for (int c = 0; c < CC; c += 4)
                    *reinterpret_cast<float4 *>(dst + e * N + c) =
                        make_float4(S[e][c], S[e][c + 1], S[e][c + 2], S[e][c + 3]);
        }

        const float *L = &lds[blk & 1][0][0][0];
#pragma unroll
        for (int s = 0; s < TB; ++s) {
            if (s >= nst) continue;
            const float *Ls = L + s * N;
            float va[CC], vw[CC], vk[CC], vb[CC], vr[CC], vv[R];
#pragma unroll
            for (int c = 0; c < CC; c += 4) {
                const float4 qa = *reinterpret_cast<const float4 *>(Ls + kA * TB * N + col0 + c);
                const float4 qw = *reinterpret_cast<const float4 *>(Ls + kW * TB * N + col0 + c);
                const float4 qk = *reinterpret_cast<const float4 *>(Ls + kK * TB * N + col0 + c);
                const float4 qb = *reinterpret_cast<const float4 *>(Ls + kB * TB * N + col0 + c);
                const float4 qr = *reinterpret_cast<const float4 *>(Ls + kR * TB * N + col0 + c);
                va[c] = qa.x; va[c + 1] = qa.y; va[c + 2] = qa.z; va[c + 3] = qa.w;
                vw[c] = qw.x; vw[c + 1] = qw.y; vw[c + 2] = qw.z; vw[c + 3] = qw.w;
                vk[c] = qk.x; vk[c + 1] = qk.y; vk[c + 2] = qk.z; vk[c + 3] = qk.w;
                vb[c] = qb.x; vb[c + 1] = qb.y; vb[c + 2] = qb.z; vb[c + 3] = qb.w;
                vr[c] = qr.x; vr[c + 1] = qr.y; vr[c + 2] = qr.z; vr[c + 3] = qr.w;
            }
#pragma unroll
            for (int e = 0; e < R; ++e) vv[e] = Ls[kV * TB * N + row0 + e];

            // sa = S a over the pre-update state (row dot, then group sum)
            float sa[R];
#pragma unroll
            for (int e = 0; e < R; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < CC; ++c) acc = fmaf(S[e][c], va[c], acc);
                sa[e] = group_allreduce<LPR>(acc);
            }
            // S <- S diag(w) + v k^T + sa b^T ; y = S r (post-update)
            float yv[R];
#pragma unroll
            for (int e = 0; e < R; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < CC; ++c) {
                    S[e][c] = fmaf(S[e][c], vw[c], fmaf(vv[e], vk[c], sa[e] * vb[c]));
                    acc = fmaf(S[e][c], vr[c], acc);
                }
                yv[e] = group_allreduce<LPR>(acc);
            }
            if (p.y && cg == 0) {
                float *dst = p.y + vbase + (t0 + s) * stride + row0;
                if constexpr (R == 2)
                    *reinterpret_cast<float2 *>(dst) = make_float2(yv[0], yv[1]);
                else
#pragma unroll
                    for (int e = 0; e < R; ++e) dst[e] = yv[e];
            }
        }

        if (more) stage.commit(&lds[(blk + 1) & 1][0][0][0], nnext, tid);
        __syncthreads();
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
}

template <int N, typename TIn>
hipError_t launch_fwd_t(const FwdLaunch &a, hipStream_t stream)
{
    FwdArgs<TIn> p;
    for (int i = 0; i < 6; ++i) p.in.p[i] = static_cast<const TIn *>(a.in[i]);
    p.s0 = a.s0;
    p.y = a.y;
    p.sT = a.sT;
    p.ckpt = a.ckpt;
    p.T = a.T;
    p.H = a.H;
    p.chunk = a.chunk;
    p.nck = (int)((a.T + a.chunk - 1) / a.chunk);
    const dim3 grid((unsigned)(a.B * a.H)), block(FwdGeom<N>::NT);
    hipLaunchKernelGGL((wkv7_fwd_kernel<N, TIn>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const FwdLaunch &a, hipStream_t stream)
{
    if (a.N == 64)
        return a.dtype == 0 ? launch_fwd_t<64, float>(a, stream)
                            : launch_fwd_t<64, uint16_t>(a, stream);
    return a.dtype == 0 ? launch_fwd_t<16, float>(a, stream)
                        : launch_fwd_t<16, uint16_t>(a, stream);
}

}  // namespace wkv7
