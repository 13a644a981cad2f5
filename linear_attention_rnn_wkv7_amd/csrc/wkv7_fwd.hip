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
    static constexpr int TB = 32;                   // steps per staged block
    static constexpr int NV = 6;                    // r, w, k, v, a, b
    static_assert(N % RW == 0 && CC % 4 == 0, "tile");
};

enum { kR = 0, kW = 1, kK = 2, kV = 3, kA = 4, kB = 5 };

template <typename TIn>
struct FwdArgs {
    VecPtrs<TIn, 6> in;
    const float *s0;
    float *y, *sT, *ckpt;
    float *sa;               // per-step sa = S_{t-1} a_t, [B][T][H][N]; may be null
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
    // y and sa of a block, [buffer][0 = y, 1 = sa][step][row], written one
    // value per lane per step and copied out row-contiguous per block
    __shared__ __align__(16) float outb[2][2][TB][N];
    __shared__ float sink[NT];   // target of the lanes that hold no value

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

    // Per-step operands read back from LDS: this lane's CC columns of a, w,
    // k, b, r and its R entries of v.
    struct StepVals {
        float a[CC], w[CC], k[CC], b[CC], r[CC], v[R];
    };
    auto load_step = [&](const float *Ls, StepVals &sv) {
#pragma unroll
        for (int c = 0; c < CC; c += 4) {
            const float4 qa = *reinterpret_cast<const float4 *>(Ls + kA * TB * N + col0 + c);
            const float4 qw = *reinterpret_cast<const float4 *>(Ls + kW * TB * N + col0 + c);
            const float4 qk = *reinterpret_cast<const float4 *>(Ls + kK * TB * N + col0 + c);
            const float4 qb = *reinterpret_cast<const float4 *>(Ls + kB * TB * N + col0 + c);
            const float4 qr = *reinterpret_cast<const float4 *>(Ls + kR * TB * N + col0 + c);
            sv.a[c] = qa.x; sv.a[c + 1] = qa.y; sv.a[c + 2] = qa.z; sv.a[c + 3] = qa.w;
            sv.w[c] = qw.x; sv.w[c + 1] = qw.y; sv.w[c + 2] = qw.z; sv.w[c + 3] = qw.w;
            sv.k[c] = qk.x; sv.k[c + 1] = qk.y; sv.k[c + 2] = qk.z; sv.k[c + 3] = qk.w;
            sv.b[c] = qb.x; sv.b[c + 1] = qb.y; sv.b[c + 2] = qb.z; sv.b[c + 3] = qb.w;
            sv.r[c] = qr.x; sv.r[c + 1] = qr.y; sv.r[c + 2] = qr.z; sv.r[c + 3] = qr.w;
        }
#pragma unroll
        for (int e = 0; e < R; ++e) sv.v[e] = Ls[kV * TB * N + row0 + e];
    };
    // Where this lane parks one value of a per-row output: lanes cg < R hold
    // row row0 + cg; the others write to a private sink slot (no branch).
    auto park = [&](float *row_base, const float (&x)[R]) {
        float val = x[0];
#pragma unroll
        for (int e = 1; e < R; ++e)
            if (cg == e) val = x[e];
        float *dst = cg < R ? row_base + row0 + cg : &sink[tid];
        *dst = val;
    };
    // One step on S; parks this lane's rows of y and sa in LDS.
    auto do_step = [&](const StepVals &sv, float *ypark, float *sapark) {
        float sa[R], u[R][CC], yv[R];
#pragma unroll
        for (int e = 0; e < R; ++e) {
            // sa = S a over the pre-update state: two partial chains, then
            // the sum over the row group.
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int c = 0; c < CC; c += 2) {
                a0 = fmaf(S[e][c], sv.a[c], a0);
                a1 = fmaf(S[e][c + 1], sv.a[c + 1], a1);
            }
            // the part of the update that does not need sa
#pragma unroll
            for (int c = 0; c < CC; ++c) u[e][c] = fmaf(S[e][c], sv.w[c], sv.v[e] * sv.k[c]);
            sa[e] = group_allreduce<LPR>(a0 + a1);
        }
        // S <- S diag(w) + v k^T + sa b^T ; y = S r over the updated state
#pragma unroll
        for (int e = 0; e < R; ++e) {
            float y0 = 0.f, y1 = 0.f;
#pragma unroll
            for (int c = 0; c < CC; c += 2) {
                S[e][c] = fmaf(sa[e], sv.b[c], u[e][c]);
                S[e][c + 1] = fmaf(sa[e], sv.b[c + 1], u[e][c + 1]);
                y0 = fmaf(S[e][c], sv.r[c], y0);
                y1 = fmaf(S[e][c + 1], sv.r[c + 1], y1);
            }
            yv[e] = group_allreduce<LPR>(y0 + y1);
        }
        park(ypark, yv);
        park(sapark, sa);
    };

    // Input staging runs one block ahead: while block b computes from
    // lds[b & 1], block b+1 is copied into lds[(b+1) & 1] (directly from HBM
    // for fp32 inputs, through registers for bf16).
    using StagerT = InputStager<TIn, NV, TB, N, NT>;
    StagerT stage;
    const int64_t nblk = (T + TB - 1) / TB;
    auto steps_of = [&](int64_t blk) -> int {
        const int64_t rem = T - blk * TB;
        return (int)(rem < TB ? rem : TB);
    };
    if (nblk > 0) {
        stage.issue(p.in, vbase, stride, steps_of(0), wave, lane, &lds[0][0][0][0]);
        stage.commit(&lds[0][0][0][0], steps_of(0), wave, lane);
        if constexpr (StagerT::kDma) wait_dma();
    }
    __syncthreads();

    // Checkpoints: the state before every step that is a multiple of the
    // chunk (a multiple of 8, so within a block only offsets 0, 8, 16, ...).
    static_assert(TB % 8 == 0, "checkpoint offsets are multiples of 8");
    int64_t next_ck = 0, ck_slot = 0;
    auto maybe_checkpoint = [&](int64_t t) {
        if (t == next_ck) {
            if (p.ckpt) {
                float *dst = p.ckpt + (bh * p.nck + ck_slot) * N * N + (int64_t)row0 * N + col0;
#pragma unroll
                for (int e = 0; e < R; ++e)
#pragma unroll
                    for (int c = 0; c < CC; c += 4)
                        *reinterpret_cast<float4 *>(dst + e * N + c) =
                            make_float4(S[e][c], S[e][c + 1], S[e][c + 2], S[e][c + 3]);
            }
            ++ck_slot;
            next_ck += p.chunk;
        }
    };

    // Copy the parked y and sa of block blk (in outb[blk & 1]) to HBM: each
    // step is N contiguous floats per output.
    auto copy_out = [&](int64_t blk) {
        const int64_t t0 = blk * TB;
        const int nst = steps_of(blk);
        constexpr int kQ = 2 * TB * N / 4;            // float4 units
#pragma unroll
        for (int k = 0; k < (kQ + NT - 1) / NT; ++k) {
            const int u = tid + k * NT;
            const int which = u / (TB * N / 4);       // 0 = y, 1 = sa
            const int st = (u / (N / 4)) % TB, n4 = u % (N / 4);
            float *base = which == 0 ? p.y : p.sa;
            if (u < kQ && st < nst && base)
                *reinterpret_cast<float4 *>(base + vbase + (t0 + st) * stride + 4 * n4) =
                    *reinterpret_cast<const float4 *>(&outb[blk & 1][which][st][4 * n4]);
        }
    };

    for (int64_t blk = 0; blk < nblk; ++blk) {
        const int64_t t0 = blk * TB;
        const int nst = steps_of(blk);
        if (blk + 1 < nblk)
            stage.issue(p.in, vbase + (t0 + TB) * stride, stride, steps_of(blk + 1), wave, lane,
                        &lds[(blk + 1) & 1][0][0][0]);
        if (blk > 0) copy_out(blk - 1);

        const float *L = &lds[blk & 1][0][0][0];
        float *Y = &outb[blk & 1][0][0][0];
        float *SA = &outb[blk & 1][1][0][0];
        if (nst == TB) {
            // steady state: straight-line code except the rare mid-block
            // checkpoint test; the next step's operands are read from LDS
            // while the current step computes
            StepVals sv[2];
            load_step(L, sv[0]);
#pragma unroll
            for (int s = 0; s < TB; ++s) {
                if (s % 8 == 0) maybe_checkpoint(t0 + s);
                if (s + 1 < TB) load_step(L + (s + 1) * N, sv[(s + 1) & 1]);
                do_step(sv[s & 1], Y + s * N, SA + s * N);
            }
        } else {
#pragma unroll
            for (int s = 0; s < TB; ++s) {
                if (s < nst) {
                    if (s % 8 == 0) maybe_checkpoint(t0 + s);
                    StepVals sv;
                    load_step(L + s * N, sv);
                    do_step(sv, Y + s * N, SA + s * N);
                }
            }
        }
        if (blk + 1 < nblk) stage.commit(&lds[(blk + 1) & 1][0][0][0], steps_of(blk + 1), wave, lane);
        if constexpr (StagerT::kDma) wait_dma();
        __syncthreads();
    }
    if (nblk > 0) copy_out(nblk - 1);

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
    p.sa = a.satape;
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
    if (a.T == 1) return launch_decode(a, stream);
    if (a.fused && !forward_chunked_supported(a)) return hipErrorInvalidValue;   // checked by the caller
    if (a.N == 64) {
        if (a.nseg > 1) {   // a split sequence (the caller checked that the chunk form applies)
            hipError_t e = launch_forward_chunked(a, 1, stream);
            if (e == hipSuccess) e = launch_compose_forward(a, stream);
            if (e == hipSuccess) e = launch_forward_chunked(a, 2, stream);
            return e;
        }
        if (forward_chunked_supported(a)) return launch_forward_chunked(a, 0, stream);
        return a.dtype == 0 ? launch_fwd_t<64, float>(a, stream)
                            : launch_fwd_t<64, uint16_t>(a, stream);
    }
    return a.dtype == 0 ? launch_fwd_t<16, float>(a, stream)
                        : launch_fwd_t<16, uint16_t>(a, stream);
}

}  // namespace wkv7
