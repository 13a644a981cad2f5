// Carries between the segments of a split sequence (N = 64).
//
// A segment of the recurrence S_t = S_{t-1} M_t + v_t k_t^T, with
// M_t = diag(w_t) + a_t b_t^T, maps its carry-in state affinely:
// S_end = S_in P + Q, where P is the product of the segment's M_t (the same
// recurrence with v = 0 started from the identity) and Q the segment's end
// state started from zero.  The reverse scan carries the state gradient the
// other way: dL/dS_in = (dL/dS_end) P^T + Z, with Z the segment's own
// contribution (its reverse scan with a zero incoming gradient).  These
// kernels chain those maps across the segments of each (b, h), one
// workgroup per (b, h), serially over the segments; the segments' scans run
// in parallel in the chunk-form kernels.

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

constexpr int N = 64;

// out = X B + C over 64 x 64 fp32 matrices, 256 threads: thread t owns row
// t / 4, columns 16 (t % 4) .. + 15.  X and B are in LDS (B row-major);
// C and out have row stride ld, and C is read before out is written (they
// may be the same memory).
__device__ __forceinline__ void mma64(const float *X, const float *Bm, const float *C, float *out,
                                      int64_t ld, float *Xnext)
{
    const int t = threadIdx.x, i = t >> 2, j0 = 16 * (t & 3);
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = C[i * ld + j0 + j];
    for (int k = 0; k < N; ++k) {
        const float x = X[i * N + k];
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = fmaf(x, Bm[k * N + j0 + j], acc[j]);
    }
    __syncthreads();   // every thread is done reading X and B
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        out[i * ld + j0 + j] = acc[j];
        Xnext[i * N + j0 + j] = acc[j];
    }
}

// Forward: S_in(s + 1) = S_in(s) P_s + Q_s for s = 1 .. nseg - 2, where
// S_in(1) = Q_0 is already in segment 1's carry slot and Q_s is in segment
// s + 1's (overwritten with S_in(s + 1)).  The carry slot of segment s is
// the checkpoint at its start, P_s in pbuf (row stride 64); without a
// checkpoint record (ckpt null) they are the rows of steps 0 .. 63 and
// 64 .. 127 of segment s in y (row stride H * 64).
__global__ void __launch_bounds__(256) compose_fwd_kernel(float *ckpt, const float *pbuf, float *y,
                                                          int64_t T, int64_t H, int nck, int nseg,
                                                          int nckseg, int chunk)
{
    __shared__ float X[N * N], Pm[N * N];
    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x;
    const bool in_y = ckpt == nullptr;
    const int64_t ld = in_y ? H * N : N;
    auto slot = [&](int s) {
        return in_y ? y + ((bh / H) * T * H + bh % H) * N + (int64_t)s * nckseg * chunk * ld
                    : ckpt + (bh * nck + (int64_t)s * nckseg) * N * N;
    };
    for (int e = t; e < N * N; e += 256) X[e] = slot(1)[(e / N) * ld + e % N];
    for (int s = 1; s <= nseg - 2; ++s) {
        const float *P = in_y ? slot(s) + N * ld : pbuf + (bh * nseg + s) * N * N;
        for (int e = t; e < N * N; e += 256) Pm[e] = P[(e / N) * ld + e % N];
        __syncthreads();
        mma64(X, Pm, slot(s + 1), slot(s + 1), ld, X);
        __syncthreads();
    }
}

// Backward: G_{nseg-1} = Z_{nseg-1} (in place), and for s = nseg - 2 .. 1,
// G_s = G_{s+1} P_s^T + Z_s, in place in gbuf (Z_s there on entry).
__global__ void __launch_bounds__(256) compose_bwd_kernel(float *gbuf, const float *pbuf, int nseg)
{
    __shared__ float X[N * N], Pt[N * N];
    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x;
    float *G = gbuf + bh * nseg * N * N;
    for (int e = t; e < N * N; e += 256) X[e] = G[(int64_t)(nseg - 1) * N * N + e];
    for (int s = nseg - 2; s >= 1; --s) {
        const float *P = pbuf + (bh * nseg + s) * N * N;
        for (int e = t; e < N * N; e += 256) Pt[(e % N) * N + e / N] = P[e];   // P^T
        __syncthreads();
        mma64(X, Pt, G + (int64_t)s * N * N, G + (int64_t)s * N * N, N, X);
        __syncthreads();
    }
}

// flags[bh] = 1 when any segment of (b, h) was flagged by the chunk form
__global__ void flag_reduce_kernel(const int *unit_flags, int *flags, int64_t nbh, int nseg)
{
    const int64_t bh = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= nbh) return;
    int f = 0;
    for (int s = 0; s < nseg; ++s) f |= unit_flags[bh * nseg + s];
    flags[bh] = f;
}

}  // namespace

hipError_t launch_compose_forward(const FwdLaunch &a, hipStream_t stream)
{
    if (a.nseg < 3) return hipSuccess;   // S_in(1) = Q_0 is all there is
    const int nck = (int)((a.T + a.chunk - 1) / a.chunk);
    hipLaunchKernelGGL(compose_fwd_kernel, dim3((unsigned)(a.B * a.H)), dim3(256), 0, stream, a.ckpt,
                       a.pbuf, a.y, a.T, a.H, nck, a.nseg, a.nckseg, a.chunk);
    return hipGetLastError();
}

hipError_t launch_compose_backward(const BwdLaunch &a, hipStream_t stream)
{
    if (a.nseg < 3) return hipSuccess;   // G_1 = Z_1 is all there is
    hipLaunchKernelGGL(compose_bwd_kernel, dim3((unsigned)(a.B * a.H)), dim3(256), 0, stream, a.gbuf,
                       a.pbuf, a.nseg);
    return hipGetLastError();
}

hipError_t launch_flag_reduce(const int *unit_flags, int *flags, int64_t nbh, int nseg, hipStream_t stream)
{
    const unsigned blocks = (unsigned)((nbh + 255) / 256);
    hipLaunchKernelGGL(flag_reduce_kernel, dim3(blocks), dim3(256), 0, stream, unit_flags, flags, nbh, nseg);
    return hipGetLastError();
}

}  // namespace wkv7
