// Host-side launch interface between the C ABI (wkv7_abi.cpp) and the
// kernels.  Shapes and pointers reaching these functions are validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "wkv7.h"

namespace wkv7 {

// Sub-chunk length of the backward's in-register recompute.
constexpr int kSubChunk = 8;

struct FwdLaunch {
    const void *in[6];       // r, w, k, v, a, b
    const float *s0;         // may be null (zeros)
    float *y, *sT, *ckpt;    // each may be null (skipped)
    float *satape;           // per-step sa, [B][T][H][N]; may be null
    int64_t B, T, H, N;
    int dtype;               // 0 f32, 1 bf16
    int chunk;               // checkpoint interval
    int fused;               // w, a, b slots hold omega, kk, gate (N = 64)
    int nseg = 1, nckseg = 0;  // sequence split: segments of nckseg chunks
    float *pbuf = nullptr;   // split: transition products, [B*H][nseg][64][64]
};

struct BwdLaunch {
    const void *in[7];       // r, w, k, v, a, b, dy
    const float *ckpt;       // required
    const float *satape;     // required: the forward's per-step sa
    const float *dsT;        // may be null (zeros)
    float *grad[6];          // dr, dw, dk, dv, da, db
    float *ds0;              // may be null
    float *sub;              // sub-checkpoint scratch (see sub_bytes)
    int *flags;              // B*H ints: heads the chunk form could not take
    int64_t B, T, H, N;
    int dtype;
    int chunk;
    int algo;                // wkv7_algo
    int fused;               // as FwdLaunch; the chunk form only
    int nseg = 1, nckseg = 0;  // sequence split (as the forward's)
    const float *pbuf = nullptr;  // split: the forward's transition products
    float *gbuf = nullptr;   // split: state gradients at segment starts
    int *unit_flags = nullptr;  // split: chunk-form flags per (b, h, segment)
};

// The chunk forms address one (b) slice of a [B][T][H][64] tensor with
// 32-bit byte offsets: T * H * 64 * 4 must stay below 2^31.
inline bool chunk_offsets_fit(int64_t T, int64_t H)
{
    return T > 0 && H > 0 && T <= (int64_t(1) << 31) / (H * 64 * 4) - 1;
}

// Bytes of sub-checkpoint scratch the backward needs for a shape.
size_t sub_bytes(int64_t B, int64_t H, int64_t N, int chunk);

hipError_t launch_forward(const FwdLaunch &a, hipStream_t stream);
// The single-step forward (T = 1) of wkv7_decode.hip.
hipError_t launch_decode(const FwdLaunch &a, hipStream_t stream);
// The forward for N = 64 on a scan plus matrix-core helper waves
// (wkv7_fwdc.hip); it needs checkpoints on 32-step block starts.
bool forward_chunked_supported(const FwdLaunch &a);
// mode 0: whole sequences; 1, 2: the two passes of a split sequence
hipError_t launch_forward_chunked(const FwdLaunch &a, int mode, hipStream_t stream);
// Reverse scan: the chunk form where it applies (and algo allows), then the
// step-by-step scan for every head the chunk form flagged (or all heads).
hipError_t launch_backward(const BwdLaunch &a, hipStream_t stream);
// The chunk form (wkv7_bwdc.hip): N = 64, C = 64.  Writes flags[bh] = 1 for
// heads whose decays it cannot take (their outputs are then undefined).
bool chunked_backward_supported(const BwdLaunch &a);
hipError_t launch_backward_chunked(const BwdLaunch &a, int *flags, int mode, hipStream_t stream);
// Split sequences (wkv7_split.hip): carry-in states and state gradients
// across segments, and the per-(b, h) fallback flags from the per-segment ones.
hipError_t launch_compose_forward(const FwdLaunch &a, hipStream_t stream);
hipError_t launch_compose_backward(const BwdLaunch &a, hipStream_t stream);
hipError_t launch_flag_reduce(const int *unit_flags, int *flags, int64_t nbh, int nseg,
                              hipStream_t stream);
// The time-mix epilogue (wkv7_epilogue.hip): group norm, bonus and gate
// after the scan, N = 64; rows are the B*T*H (b, t, h) of [B][T][H][64].
struct EpiLaunch {
    const float *y = nullptr, *dz = nullptr;
    const void *r = nullptr, *k = nullptr, *v = nullptr, *g = nullptr;   // dtype
    const float *ln_w = nullptr, *ln_b = nullptr, *r_k = nullptr;        // [H][64]
    float *z = nullptr;
    float *dy = nullptr, *dg = nullptr, *dr = nullptr, *dk = nullptr, *dv = nullptr;
    float *dln_w = nullptr, *dln_b = nullptr, *dr_k = nullptr;
    float *part = nullptr;   // backward: [H][nchunk][3][64] partial sums
    int64_t BT = 0, H = 0;
    int dtype = 0, nchunk = 1;
};
// Backward workgroups per head (each a range of (b, t)).
int epilogue_chunks(int64_t BT, int64_t H);
hipError_t launch_epilogue_forward(const EpiLaunch &a, hipStream_t stream);
hipError_t launch_epilogue_backward(const EpiLaunch &a, hipStream_t stream);
// dst[i] = src ? src[i] : 0 for i < n.
hipError_t launch_fill(float *dst, const float *src, size_t n, hipStream_t stream);

// Devices per process the library keeps per-device addresses for.
constexpr int kMaxDevices = 64;
// The current device's fault word (wkv7_fwdc.hip): bit 0 is set when a
// forward helper wait gave up; null when the device's address cannot be had.
unsigned *fault_word();
// Test hooks (wkv7_abi.cpp, wkv7_test_hook): report a given-up helper wait
// in every forward workgroup; turn the status of the next launches into a
// launch failure.
int test_fault_inject();

// The body of wkv7_backward.  With `scratch` non-null the workspace
// arguments are ignored: after validation, scratch(need, &ptr) supplies
// `need` bytes of device workspace (or returns an error status).
int backward_entry(const wkv7_shape *shape, const void *r, const void *w, const void *k,
                   const void *v, const void *a, const void *b, const float *s0,
                   const void *dy, const float *dsT, const float *ckpt,
                   float *dr, float *dw, float *dk, float *dv, float *da, float *db,
                   float *ds0, void *workspace, size_t workspace_bytes,
                   int (*scratch)(size_t need, void **ptr), hipStream_t stream);

}  // namespace wkv7
