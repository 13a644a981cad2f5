// WKV7 single-step forward (T = 1): the decode step of batched inference.
//
// One step of the recurrence rx_wkv7_forward_seq on the Foundry page
// "rwkvx/rx_pretrain.c" for every (b, h), from its carry-in state:
//   sa = S a;   S' = S diag(w) + v k^T + sa b^T;   y = S' r.
// The step reads and writes the whole N x N state for 7 N-vectors of
// input and output, so it is bound by HBM bandwidth: the kernel streams
// the state through registers once, with fully coalesced 16-byte accesses,
// and keeps everything else in registers.
//
// With fused inputs the w, a, b slots hold the decay pre-activation omega,
// the normalised key kk and the gate ag of the page's tm_pre_forward, and
// the kernel forms w = exp(-c sigmoid(omega)), a = -kk, b = kk ag itself.
//
// One workgroup per (b, h), NT threads.  Thread t owns four consecutive
// columns 4 (t mod TPR) .. of RPT rows, row m RPP + t / TPR for m < RPT, so
// that pass m of the workgroup reads NT float4 = RPP whole rows, contiguous
// in memory.  Row dots (sa, y) are summed over the TPR lanes of a row with
// DPP (fixed order: results are reproducible bit for bit).

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

template <int N>
struct DecGeom {
    static constexpr int NT = N == 64 ? 256 : 64;   // threads per (b, h)
    static constexpr int TPR = N / 4;               // threads per state row
    static constexpr int RPP = NT / TPR;            // rows per pass
    static constexpr int RPT = N / RPP;             // rows per thread
    static_assert(RPT * RPP == N && TPR <= 16, "geometry");
};

template <typename TIn>
struct DecArgs {
    const TIn *r, *w, *k, *v, *a, *b;   // [B][1][H][N]
    const float *s0;                    // [B][H][N][N] or null (zeros)
    float *y, *sT;                      // each may be null
    float *ckpt, *sa;                   // checkpoint slot 0 and the sa tape, or null
};

__device__ __forceinline__ float dot4(float4 x, float4 u)
{
    return fmaf(x.w, u.w, fmaf(x.z, u.z, fmaf(x.y, u.y, x.x * u.x)));
}

template <int N, typename TIn, bool kFused>
__global__ void __launch_bounds__(DecGeom<N>::NT) wkv7_decode_kernel(DecArgs<TIn> p)
{
    using G = DecGeom<N>;
    const int t = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int col = 4 * (t % G::TPR), row0 = t / G::TPR;
    const int64_t vb = bh * N;                  // this (b, h)'s step in [B][1][H][N]
    const int64_t sb = bh * N * N + 4 * t;      // pass m adds m * RPP * N

    float4 s[G::RPT];
    if (p.s0) {
#pragma unroll
        for (int m = 0; m < G::RPT; ++m)
            s[m] = *reinterpret_cast<const float4 *>(p.s0 + sb + m * G::RPP * N);
    } else {
#pragma unroll
        for (int m = 0; m < G::RPT; ++m) s[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float4 a4 = InQuad<TIn>::f32(InQuad<TIn>::load(p.a + vb + col));
    float4 w4 = InQuad<TIn>::f32(InQuad<TIn>::load(p.w + vb + col));
    const float4 k4 = InQuad<TIn>::f32(InQuad<TIn>::load(p.k + vb + col));
    float4 b4 = InQuad<TIn>::f32(InQuad<TIn>::load(p.b + vb + col));
    if constexpr (kFused) {   // a4 holds kk, b4 the gate, w4 omega
        b4 = make_float4(a4.x * b4.x, a4.y * b4.y, a4.z * b4.z, a4.w * b4.w);
        a4 = make_float4(-a4.x, -a4.y, -a4.z, -a4.w);
        w4 = make_float4(decay_from_pre(w4.x), decay_from_pre(w4.y), decay_from_pre(w4.z),
                         decay_from_pre(w4.w));
    }
    const float4 r4 = InQuad<TIn>::f32(InQuad<TIn>::load(p.r + vb + col));
    float vi[G::RPT];
#pragma unroll
    for (int m = 0; m < G::RPT; ++m) {
        const int i = m * G::RPP + row0;
        if constexpr (sizeof(TIn) == 4)
            vi[m] = p.v[vb + i];
        else
            vi[m] = bf16_lo(p.v[vb + i]);
    }

    const bool lead = t % G::TPR == 0;   // writes the row's scalars
#pragma unroll
    for (int m = 0; m < G::RPT; ++m) {
        const int i = m * G::RPP + row0;
        const float4 x = s[m];
        const float sa = group_allreduce<G::TPR>(dot4(x, a4));
        if (p.ckpt) {
            *reinterpret_cast<float4 *>(p.ckpt + sb + m * G::RPP * N) = x;
            if (lead) p.sa[vb + i] = sa;
        }
        float4 u;
        u.x = fmaf(sa, b4.x, fmaf(x.x, w4.x, vi[m] * k4.x));
        u.y = fmaf(sa, b4.y, fmaf(x.y, w4.y, vi[m] * k4.y));
        u.z = fmaf(sa, b4.z, fmaf(x.z, w4.z, vi[m] * k4.z));
        u.w = fmaf(sa, b4.w, fmaf(x.w, w4.w, vi[m] * k4.w));
        if (p.sT) *reinterpret_cast<float4 *>(p.sT + sb + m * G::RPP * N) = u;
        if (p.y) {
            const float yv = group_allreduce<G::TPR>(dot4(u, r4));
            if (lead) p.y[vb + i] = yv;
        }
    }
}

template <int N, typename TIn, bool kFused>
hipError_t launch_dec_t(const FwdLaunch &a, hipStream_t stream)
{
    DecArgs<TIn> p;
    p.r = static_cast<const TIn *>(a.in[0]);
    p.w = static_cast<const TIn *>(a.in[1]);
    p.k = static_cast<const TIn *>(a.in[2]);
    p.v = static_cast<const TIn *>(a.in[3]);
    p.a = static_cast<const TIn *>(a.in[4]);
    p.b = static_cast<const TIn *>(a.in[5]);
    p.s0 = a.s0;
    p.y = a.y;
    p.sT = a.sT;
    p.ckpt = a.ckpt;
    p.sa = a.satape;
    hipLaunchKernelGGL((wkv7_decode_kernel<N, TIn, kFused>), dim3((unsigned)(a.B * a.H)),
                       dim3(DecGeom<N>::NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const FwdLaunch &a, hipStream_t stream)
{
    if (a.fused)   // N = 64 only (checked by the caller)
        return a.dtype == 0 ? launch_dec_t<64, float, true>(a, stream)
                            : launch_dec_t<64, uint16_t, true>(a, stream);
    if (a.N == 64)
        return a.dtype == 0 ? launch_dec_t<64, float, false>(a, stream)
                            : launch_dec_t<64, uint16_t, false>(a, stream);
    return a.dtype == 0 ? launch_dec_t<16, float, false>(a, stream)
                        : launch_dec_t<16, uint16_t, false>(a, stream);
}

}  // namespace wkv7
