// The time-mix epilogue after the WKV7 scan, forward and backward, N = 64.
//
// On the Foundry page "rwkvx/rx_pretrain.c" the scan's output y goes, per
// (b, t, h) over the head's N entries, through gn_forward (group norm with
// epsilon 64e-5 and per-channel ln_x_w, ln_x_b), plus the bonus s v with
// s = sum_j r_j k_j r_k[j], and then the gate g (tg = yb * g, the input of
// the output projection, which stays outside):
//   z = ((y - mean) rstd ln_w + ln_b + s v) g.
// The backward is the page's per-token post-processing backward: gate,
// bonus, group norm, giving dy for the reverse scan, dg, the bonus terms of
// dr, dk, dv, and the per-channel gradients of ln_w, ln_b and r_k summed
// over (b, t).  One pass over the tensors each way instead of the page's
// separate loops.
//
// A row (b, t, h) is 64 contiguous floats: 16 lanes hold 4 each, and its
// sums (mean, variance, bonus, the norm's backward terms) are DPP sums over
// those 16 lanes, in a fixed order.  The backward's workgroups each keep one
// head, or four adjacent heads when H is a multiple of 4 (so that four lane
// groups read 1 KB of contiguous rows), and a range of (b, t); each lane
// group keeps one head and adds the parameter gradients of its rows in
// registers; LDS and a second kernel add the partials in a fixed order:
// results are reproducible bit for bit.

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

constexpr int N = 64;
constexpr float kGnEps = 64e-5f;

__device__ __forceinline__ float sum4(float4 a) { return (a.x + a.y) + (a.z + a.w); }
__device__ __forceinline__ float4 mul4(float4 a, float4 b) { return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w); }
__device__ __forceinline__ float4 axpy4(float s, float4 x, float4 y)
{
    return make_float4(fmaf(s, x.x, y.x), fmaf(s, x.y, y.y), fmaf(s, x.z, y.z), fmaf(s, x.w, y.w));
}
__device__ __forceinline__ float4 ld4f(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void st4f(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }

template <typename TIn>
__device__ __forceinline__ float4 ldin(const TIn *p) { return InQuad<TIn>::f32(InQuad<TIn>::load(p)); }

// The normalised row and 1 / sqrt(var + eps) (two passes over registers).
__device__ __forceinline__ float4 gn_norm(float4 y, float &rstd)
{
    const float mean = group_allreduce<16>(sum4(y)) * (1.f / N);
    const float4 d = make_float4(y.x - mean, y.y - mean, y.z - mean, y.w - mean);
    const float var = group_allreduce<16>(sum4(mul4(d, d))) * (1.f / N);
    rstd = 1.f / sqrtf(var + kGnEps);
    return make_float4(d.x * rstd, d.y * rstd, d.z * rstd, d.w * rstd);
}

template <typename TIn>
struct EpiArgs {
    const float *y, *dz;
    const TIn *r, *k, *v, *g;
    const float *ln_w, *ln_b, *r_k;    // [H][64]
    float *z;                          // forward output
    float *dy, *dg, *dr, *dk, *dv;     // backward outputs
    float *part;                       // [H][nchunk][3][64] backward partials
    int64_t rows, bt, H;               // rows = bt * H
    int nchunk, chunk_rows;            // (b, t) rows per backward workgroup
};

// 16 rows per workgroup of 256 threads.
template <typename TIn>
__global__ void __launch_bounds__(256) epi_fwd_kernel(EpiArgs<TIn> p)
{
    const int t = threadIdx.x, l = t & 15;
    const int64_t row = (int64_t)blockIdx.x * 16 + (t >> 4);
    if (row >= p.rows) return;   // the whole 16-lane row group leaves together
    const int h = (int)(row % p.H);
    const int64_t o = row * N + 4 * l;
    const int po = h * N + 4 * l;
    float rstd;
    const float4 yn = gn_norm(ld4f(p.y + o), rstd);
    const float4 r = ldin(p.r + o), k = ldin(p.k + o), v = ldin(p.v + o), g = ldin(p.g + o);
    const float4 lw = ld4f(p.ln_w + po), lb = ld4f(p.ln_b + po), rk = ld4f(p.r_k + po);
    const float s = group_allreduce<16>(sum4(mul4(mul4(r, k), rk)));
    const float4 yb = axpy4(s, v, make_float4(fmaf(yn.x, lw.x, lb.x), fmaf(yn.y, lw.y, lb.y),
                                              fmaf(yn.z, lw.z, lb.z), fmaf(yn.w, lw.w, lb.w)));
    st4f(p.z + o, mul4(yb, g));
}

// Workgroup (hg, c): heads HPW hg .. + HPW - 1, rows (bt, h) for bt in chunk
// c; lane group grp takes head HPW hg + grp % HPW and every (16 / HPW)-th bt.
template <typename TIn, int HPW>
__global__ void __launch_bounds__(256) epi_bwd_kernel(EpiArgs<TIn> p)
{
    constexpr int kStep = 16 / HPW;   // lane groups per head
    __shared__ float red[16][3][N];
    const int t = threadIdx.x, l = t & 15, grp = t >> 4;
    const int hg = (int)(blockIdx.x / p.nchunk), c = (int)(blockIdx.x % p.nchunk);
    const int h = HPW * hg + grp % HPW;
    const int po = h * N + 4 * l;
    const float4 lw = ld4f(p.ln_w + po), lb = ld4f(p.ln_b + po), rk = ld4f(p.r_k + po);
    float4 alw = make_float4(0.f, 0.f, 0.f, 0.f), alb = alw, ark = alw;   // parameter partials
    const int64_t bt0 = (int64_t)c * p.chunk_rows;
    int64_t bt1 = bt0 + p.chunk_rows;
    if (bt1 > p.bt) bt1 = p.bt;
    for (int64_t bt = bt0 + grp / HPW; bt < bt1; bt += kStep) {
        const int64_t o = (bt * p.H + h) * N + 4 * l;
        float rstd;
        const float4 yn = gn_norm(ld4f(p.y + o), rstd);
        const float4 r = ldin(p.r + o), k = ldin(p.k + o), v = ldin(p.v + o), g = ldin(p.g + o);
        const float4 dz = ld4f(p.dz + o);
        const float s = group_allreduce<16>(sum4(mul4(mul4(r, k), rk)));
        const float4 yb = axpy4(s, v, make_float4(fmaf(yn.x, lw.x, lb.x), fmaf(yn.y, lw.y, lb.y),
                                                  fmaf(yn.z, lw.z, lb.z), fmaf(yn.w, lw.w, lb.w)));
        // gate
        const float4 dyb = mul4(dz, g);
        st4f(p.dg + o, mul4(dz, yb));
        // bonus
        const float ds = group_allreduce<16>(sum4(mul4(dyb, v)));
        st4f(p.dv + o, make_float4(dyb.x * s, dyb.y * s, dyb.z * s, dyb.w * s));
        const float4 kr = mul4(k, rk), rr = mul4(r, rk);
        st4f(p.dr + o, make_float4(ds * kr.x, ds * kr.y, ds * kr.z, ds * kr.w));
        st4f(p.dk + o, make_float4(ds * rr.x, ds * rr.y, ds * rr.z, ds * rr.w));
        ark = axpy4(ds, mul4(r, k), ark);
        // group norm
        alw = axpy4(1.f, mul4(dyb, yn), alw);
        alb = axpy4(1.f, dyb, alb);
        const float4 dn = mul4(dyb, lw);
        const float mdn = group_allreduce<16>(sum4(dn)) * (1.f / N);
        const float mdnn = group_allreduce<16>(sum4(mul4(dn, yn))) * (1.f / N);
        st4f(p.dy + o, make_float4(rstd * (dn.x - mdn - yn.x * mdnn), rstd * (dn.y - mdn - yn.y * mdnn),
                                   rstd * (dn.z - mdn - yn.z * mdnn), rstd * (dn.w - mdn - yn.w * mdnn)));
    }
    // each head's row groups' partials, added in a fixed order
    st4f(&red[grp][0][4 * l], alw);
    st4f(&red[grp][1][4 * l], alb);
    st4f(&red[grp][2][4 * l], ark);
    __syncthreads();
    for (int i = t; i < HPW * 3 * N; i += 256) {
        const int sub = i / (3 * N), kind = (i / N) % 3, j = i % N;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < kStep; ++q) acc += red[q * HPW + sub][kind][j];
        p.part[(((int64_t)(HPW * hg + sub) * p.nchunk + c) * 3 + kind) * N + j] = acc;
    }
}

// dln_w, dln_b, dr_k [H][64]: workgroup (h, kind) adds head h's partials
// of one kind, the 16 waves each the chunks c = wave mod 16 (in chunk
// order), then the 16 wave sums in wave order.
__global__ void __launch_bounds__(1024) epi_reduce_kernel(const float *part, float *dlw, float *dlb,
                                                           float *drk, int nchunk)
{
    __shared__ float red[16][N];
    const int t = threadIdx.x, j = t & 63, wv = t >> 6;
    const int64_t h = blockIdx.x;
    const int kind = (int)blockIdx.y;
    float acc = 0.f;
#pragma unroll 8
    for (int c = wv; c < nchunk; c += 16) acc += part[((h * nchunk + c) * 3 + kind) * N + j];
    red[wv][j] = acc;
    __syncthreads();
    if (t < N) {
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) sum += red[q][t];
        (kind == 0 ? dlw : kind == 1 ? dlb : drk)[h * N + t] = sum;
    }
}

// Heads per backward workgroup: 4 when H is a multiple of 4, else 1.
int epi_hpw(int64_t H) { return H % 4 == 0 ? 4 : 1; }

template <typename TIn>
EpiArgs<TIn> epi_args(const EpiLaunch &a)
{
    EpiArgs<TIn> p;
    p.y = a.y;
    p.dz = a.dz;
    p.r = static_cast<const TIn *>(a.r);
    p.k = static_cast<const TIn *>(a.k);
    p.v = static_cast<const TIn *>(a.v);
    p.g = static_cast<const TIn *>(a.g);
    p.ln_w = a.ln_w;
    p.ln_b = a.ln_b;
    p.r_k = a.r_k;
    p.z = a.z;
    p.dy = a.dy;
    p.dg = a.dg;
    p.dr = a.dr;
    p.dk = a.dk;
    p.dv = a.dv;
    p.part = a.part;
    p.bt = a.BT;
    p.H = a.H;
    p.rows = a.BT * a.H;
    p.nchunk = a.nchunk;
    p.chunk_rows = (int)((a.BT + a.nchunk - 1) / a.nchunk);
    return p;
}

template <typename TIn>
hipError_t launch_epi_fwd_t(const EpiLaunch &a, hipStream_t stream)
{
    const EpiArgs<TIn> p = epi_args<TIn>(a);
    hipLaunchKernelGGL(epi_fwd_kernel<TIn>, dim3((unsigned)((p.rows + 15) / 16)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_epi_bwd_t(const EpiLaunch &a, hipStream_t stream)
{
    const EpiArgs<TIn> p = epi_args<TIn>(a);
    const int hpw = epi_hpw(a.H);
    const dim3 grid((unsigned)(a.H / hpw * a.nchunk));
    if (hpw == 4)
        hipLaunchKernelGGL((epi_bwd_kernel<TIn, 4>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((epi_bwd_kernel<TIn, 1>), grid, dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(epi_reduce_kernel, dim3((unsigned)a.H, 3), dim3(1024), 0, stream, a.part, a.dln_w,
                       a.dln_b, a.dr_k, a.nchunk);
    return hipGetLastError();
}

}  // namespace

int epilogue_chunks(int64_t BT, int64_t H)
{
    // about 2048 workgroups in all (of 4 heads when H is a multiple of 4,
    // else 1), each with at least one row per lane group
    const int64_t hpw = epi_hpw(H);
    int64_t c = (2048 * hpw + H - 1) / H;
    const int64_t most = (BT + 16 / hpw - 1) / (16 / hpw);
    if (c > most) c = most;
    return (int)(c < 1 ? 1 : c);
}

hipError_t launch_epilogue_forward(const EpiLaunch &a, hipStream_t stream)
{
    return a.dtype == 0 ? launch_epi_fwd_t<float>(a, stream) : launch_epi_fwd_t<uint16_t>(a, stream);
}

hipError_t launch_epilogue_backward(const EpiLaunch &a, hipStream_t stream)
{
    return a.dtype == 0 ? launch_epi_bwd_t<float>(a, stream) : launch_epi_bwd_t<uint16_t>(a, stream);
}

}  // namespace wkv7
