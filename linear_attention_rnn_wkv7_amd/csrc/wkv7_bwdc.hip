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
//   dsa_t = Hb bt_t + sum_{u>=t} dy_u (rb_u.bt_t) + sum_{u>t} dsa_u (ab_u.bt_t),
// a unit-triangular system over the chunk's steps, solved in 16-step blocks
// (the inverse of each diagonal block formed step by step on the VALU, the
// rest on MFMA).  Every gradient is then a dense contraction (MFMA), e.g.
//   dk_t = (1/g_t) (Hb^T v_t + sum_{u>=t} rb_u (dy_u.v_t) + sum_{u>t} ab_u (dsa_u.v_t))
//   dr_t = g_t (S0^T dy_t + sum_{u<=t} kt_u (v_u.dy_t) + bt_u (sa_u.dy_t))
// and dw from the per-column identity
//   w_t dw_t = c + sum_{u<t} (k dk + b db - r dr - a da)_u - a_t da_t,
//   c = sum_i (dL/dS0)[i][j] S0[i][j],
// which follows from S_t = S_{t-1} diag(w_t) + v_t k_t^T + sa_t b_t^T and the
// chain rule (the gradient-state inner product per column is conserved up to
// the terms each step adds).
//
// With fused inputs the w, a, b slots hold the decay pre-activation omega,
// the normalised key kk and the gate ag of the page's tm_pre_forward: the
// kernel forms w = exp(-c sigmoid(omega)) where it takes the decay's
// cumulative product, a = -kk and b = kk ag in the rescaling pass, and
// returns d omega = w dw (-c) s (1 - s) (s = sigmoid(omega) = -ln(w) / c),
// d kk = -da + ag db and d ag = kk db in the places of dw, da, db (the
// page's time-mix backward).  Those decays always lie in [exp(-c), 1].
//
// The rescaled form needs the cumulative decay to stay well inside fp32
// range and w not too small (dw divides by w).  A chunk whose decays fall
// outside [kWMin, 1] or whose cumulative decay drops below kGMin marks its
// (b, h) in `flags`; the host then runs the step-by-step reverse scan for the
// marked heads, which overwrites every output of those heads.

#include <type_traits>

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

// [64][64] fp32 LDS arrays, the 16-byte groups of row t XOR-swizzled by
// xs(t & 15).  With x = 4 x_hi + x_lo, xs(x) = 4 (x_lo ^ x_hi) + x_hi: both
// access shapes of the kernel meet 64 distinct banks of the 64-bank LDS (as
// measured with the LDS bank-conflict counter): 16-byte reads of 16 rows
// t..t+15, each lane its own row (16 lanes per row group), and 4-byte reads
// of the 16 columns of a 16-column block in rows t + 4 g + s.
__device__ __forceinline__ int xs(int x)
{
    return (((x & 3) ^ (x >> 2)) << 2) + (x >> 2);
}

__device__ __forceinline__ int sw(int t, int j)
{
    return (t << 6) + ((((j >> 2) ^ xs(t & 15))) << 2) + (j & 3);
}

// Element (a, b) of a 16x16 tile of a Gram matrix.  Rows a = 4 g + s (g the
// lane's row group, s fixed) and columns b = 4 g + s both fall in 64
// distinct banks of the 64-bank LDS: the row's low bits select a 64-float
// quarter, its high bits a 16-float row within it, and they scramble the
// column (b ^ 5 (a & 3)).  Within a row, each aligned group of four
// columns stays together (permuted by a & 3).
__device__ __forceinline__ int pt(int a, int b)
{
    return ((a & 3) << 6) + ((a >> 2) << 4) + (b ^ (5 * (a & 3)));
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

// Per-lane LDS offsets of the phase-2 access patterns, chosen so that the
// block index only adds a constant (an instruction offset):
//   col[s]  : element (16 ub + 4 g + s, jw) of a [64][64] array, minus 1024 ub
//   rowb[m] : float4 (16 tb + l16, 16 g + 4 m .. +3), minus 1024 tb
//   pa[s]   : Gram tile element (4 g + s, l16)
//   pb[s]   : Gram tile element (l16, 4 g + s)
struct LaneAddr {
    int col[4], rowb[4], pa[4], pb[4];
};

__device__ __forceinline__ LaneAddr lane_addr(int l16, int g, int jw)
{
    LaneAddr a;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        a.col[s] = sw(4 * g + s, jw);
        a.rowb[s] = sw(l16, 16 * g + 4 * s);
        a.pa[s] = pt(4 * g + s, l16);
        a.pb[s] = pt(l16, 4 * g + s);
    }
    return a;
}

// 16 floats of row 16 tb + l16 (columns 16 g ..) of a swizzled array
__device__ __forceinline__ void rowl(const float *s, const LaneAddr &A, int tb, float (&o)[16])
{
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float4 x = lds4(s, A.rowb[m] + 1024 * tb);
        o[4 * m] = x.x;
        o[4 * m + 1] = x.y;
        o[4 * m + 2] = x.z;
        o[4 * m + 3] = x.w;
    }
}

// Keeps the scheduler from hoisting loads across this point (bounds the
// registers held by operands in flight).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Runs mma(k, buf) for k = 0 .. N-1 with the operands of group k loaded by
// load(k, buf) D groups ahead into one of D + 1 register buffers, so that
// each group's LDS reads are in flight while the previous groups' MFMAs run.
template <int N, int W, int D = 1, typename L, typename M>
__device__ __forceinline__ void pipelined(L load, M mma)
{
    float buf[D + 1][W];
#pragma unroll
    for (int k = 0; k < D && k < N; ++k) load(k, buf[k]);
#pragma unroll
    for (int k = 0; k < N; ++k) {
        sched_fence();
        if (k + D < N) load(k + D, buf[(k + D) % (D + 1)]);
        mma(k, buf[k % (D + 1)]);
    }
    sched_fence();
}

// X[tb] += rows 16 tb + l16 of the swizzled array sX (columns 16 g + s) times
// bv[s], for tb = 0..3 (K = 64 over s and the row groups).
__device__ __forceinline__ void rows_times(f4 (&X)[4], const float *sX, const LaneAddr &A,
                                           const float (&bv)[16])
{
    pipelined<4, 16>([&](int tb, float (&b)[16]) { rowl(sX, A, tb, b); },
                     [&](int tb, const float (&b)[16]) {
#pragma unroll
                         for (int s = 0; s < 16; ++s) X[tb] = mfma(b[s], bv[s], X[tb]);
                     });
}

template <typename TIn>
struct BwdcArgs {
    const TIn *r, *w, *k, *v, *a, *b, *dy;
    const float *sa, *ckpt, *dsT;
    float *dr, *dw, *dk, *dv, *da, *db, *ds0;
    int *flags;
    int64_t T, H;
    int nck;
    // sequence split: mode 0 runs whole (b, h) sequences (one workgroup per
    // (b, h)); mode 1 (first pass) the segments s = 1 .. nseg - 1 of nckseg
    // chunks each, with zero incoming gradient except the last, forming only
    // the state gradients (the dsa solve and the carry, no outputs) and
    // dL/d(the segment's initial state) to gbuf; mode 2 (second pass) every
    // segment with its incoming gradient (gbuf[s + 1], dsT for the last).
    int mode, nseg, nckseg;
    float *gbuf;   // [B*H][nseg][64][64]
};

// x from the lane of row-group G0 (lane >> 4 == G0) with the same lane & 15,
// in every lane.  v_permlane16_swap(x, x) leaves the even row of each row
// pair in its first result and the odd row in its second; v_permlane32_swap
// does the same for the two halves of the wave.
template <int G0>
__device__ __forceinline__ float bcast_group(float x)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned y = (G0 & 1) ? p[1] : p[0];
    const auto q = __builtin_amdgcn_permlane32_swap(y, y, false, false);
    return __builtin_bit_cast(float, (G0 & 2) ? q[1] : q[0]);
}

// kLite: the split's first pass (mode 1), state gradients only
template <typename TIn, bool kFused, bool kLite>
__global__ void __launch_bounds__(512) wkv7_bwdc_kernel(BwdcArgs<TIn> p)
{
    // chunk vectors, [step][feature] swizzled: cumulative decay, rb, ab, kt,
    // bt, dsa (Hb until dsa is known), dy, and v (later sa)
    __shared__ __align__(16) float sG[4096], sR[4096], sA[4096], sK[4096], sB[4096];
    __shared__ __align__(16) float sD[4096], sDY[4096], sVS[4096];
    // two Gram matrices (10 lower 16x16 tiles each)
    __shared__ __align__(16) float sP[20 * 256];
    __shared__ __align__(16) float sScan[4][256];
    __shared__ __align__(16) float sCj[2][64];
    // inverses of the four diagonal 16x16 blocks of the dsa system
    __shared__ __align__(16) float sTT[4 * 256];
    __shared__ int sBad;

    // 8 waves, two per SIMD: wave w works on feature columns 16 fb .. 16 fb + 15
    // (fb = w % 4) of every output, for the time blocks {0, 3} (w < 4) or
    // {1, 2} (w >= 4) of each chunk; the two waves on a SIMD share its matrix
    // core, and each hides the other's waits.
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fb = wave & 3, half = wave >> 2;
    const int64_t T = p.T, H = p.H;
    const int nck = p.nck;
    // this workgroup's (b, h), chunk range [cb, ce), incoming state gradient
    // and where dL/d(initial state) goes
    int64_t bh = blockIdx.x;
    int seg = 0, cb = 0, ce = nck;
    const float *dsTu = p.dsT ? p.dsT + bh * 4096 : nullptr;
    float *ds0u = p.ds0 ? p.ds0 + bh * 4096 : nullptr;
    int64_t fidx = bh;
    if (p.mode != 0) {
        const int per = p.mode == 1 ? p.nseg - 1 : p.nseg;
        bh = (int64_t)blockIdx.x / per;
        seg = (int)((int64_t)blockIdx.x % per) + (p.mode == 1 ? 1 : 0);
        cb = seg * p.nckseg;
        ce = cb + p.nckseg < nck ? cb + p.nckseg : nck;
        fidx = bh * p.nseg + seg;
        const float *dsT_real = p.dsT ? p.dsT + bh * 4096 : nullptr;
        if (p.mode == 1) {
            dsTu = seg == p.nseg - 1 ? dsT_real : nullptr;
            ds0u = p.gbuf + fidx * 4096;
        } else {
            dsTu = seg == p.nseg - 1 ? dsT_real : p.gbuf + (fidx + 1) * 4096;
            ds0u = seg == 0 && p.ds0 ? p.ds0 + bh * 4096 : nullptr;
        }
    }
    constexpr bool full = !kLite;   // the outputs, not only the state gradients
    const int64_t bidx = bh / H, head = bh % H;
    const int64_t stride = H * 64;
    const int64_t vbase = (bidx * T * H + head) * 64;
    // bytes of this (b, h)'s steps in a [B][T][H][64] tensor, from step 0:
    // buffer accesses past them (the tail of a partial last chunk) read
    // zeros and drop stores
    const uint32_t vext = (uint32_t)(((T - 1) * stride + 64) * 4);
    const uint32_t ustride = (uint32_t)stride;
    // every phase-2 tile of this lane is in feature column jw; state
    // gradients are held as rows 16 g + 4 ib + i of column jw, ib = 2 half + lb
    int l16 = lane & 15, g = lane >> 4, jw = fb * 16 + (lane & 15), ltid = tid;
    // Makes the lane indices opaque again, so that the many LDS addresses
    // derived from them are recomputed where they are used instead of being
    // hoisted out of the chunk loop into (too many) registers.
    LaneAddr A;
    auto refresh = [&]() {
        asm volatile("" : "+v"(l16), "+v"(g), "+v"(jw), "+v"(ltid));
        A = lane_addr(l16, g, jw);
    };

    // dL/dS at the end of the chunk being processed: this wave's 32 rows of
    // column jw
    f4 Hc[2];
#pragma unroll
    for (int lb = 0; lb < 2; ++lb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            Hc[lb][i] = dsTu ? dsTu[(16 * g + 4 * (2 * half + lb) + i) * 64 + jw] : 0.f;
    if (tid == 0) sBad = 0;

    // The inputs of a chunk (r, w, k, a, b, v, dy) and its checkpoint's
    // column jw (rows 16 g + s) are loaded one chunk ahead, during the
    // previous chunk.  Every chunk but the last is full.  fp32 r, w, a, b, v
    // go straight to their LDS arrays once those are free; k and dy, and all
    // bf16 inputs (widened on the way into LDS), go through registers: 2
    // float4 units per thread and input.
    using Raw = typename InQuad<TIn>::raw;
    constexpr bool kDma = std::is_same<TIn, float>::value;
    Raw pre[7][2];
    float s0B[16];
    const TIn *src_[7] = {p.r, p.w, p.k, p.a, p.b, p.v, p.dy};
    float *dst_[7] = {sR, sG, sK, sA, sB, sVS, sDY};
    auto chunk_len = [&](int cc) {
        const int64_t rem = T - (int64_t)cc * 64;
        return (int)(rem < 64 ? rem : 64);
    };
    auto issue_s0 = [&](int cc) {
        const float *S0n = p.ckpt + (bh * nck + cc) * 4096;
#pragma unroll
        for (int s = 0; s < 16; ++s) s0B[s] = S0n[(16 * g + s) * 64 + jw];
    };
    auto issue_regs = [&](int cc, int q) {
        const int64_t tt0 = (int64_t)cc * 64;
        const int Lcc = chunk_len(cc);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int u = ltid + 512 * m, t = u >> 4, j4 = (u & 15) << 2;
            pre[q][m] = InQuad<TIn>::bload(raw_buffer(src_[q] + vbase, vext * sizeof(TIn) / 4),
                                           (uint32_t)(((uint32_t)tt0 + t) * ustride + j4) * sizeof(TIn));
        }
    };
    auto commit_regs = [&](int Lcc, int q) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int u = ltid + 512 * m, t = u >> 4, j4 = (u & 15) << 2;
            const float d = q == 1 ? (kFused ? -INFINITY : 1.f) : 0.f;
            put4(dst_[q], sw(t, j4), t < Lcc ? InQuad<TIn>::f32(pre[q][m]) : make_float4(d, d, d, d));
        }
    };
    // one full chunk of input q straight into its LDS array: 1 KB (4 rows)
    // per wave instruction, lane l landing at float 4 l of the block, i.e.
    // row 4 blk + l / 16, swizzled column group l % 16
    auto issue_dma = [&](int cc, int q) {
        const int64_t tt0 = (int64_t)cc * 64;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int blk = wave + 8 * k2;
            const int t = 4 * blk + ((ltid & 63) >> 4);
            const int j4 = ((ltid & 15) ^ xs(t & 15)) << 2;
            dma16(reinterpret_cast<const float *>(src_[q]) + vbase + (tt0 + t) * stride + j4,
                  dst_[q] + blk * 256);
        }
    };
    // fp32: the cumulative decay of the next chunk is formed in registers
    // during the current one (w read straight from global memory) and put
    // into sG once the current chunk is done with it, so that the next
    // chunk's prologue is a single pass.  Wave w takes columns 8 w ..
    // 8 w + 7; lane (seg, cw) the steps 8 seg .. 8 seg + 7 of column 8 w + cw.
    float gn[8];   // w of the next chunk, then its cumulative decay
    bool gok = true;
    auto load_w = [&](int cc) {
        const int cw = ltid & 7, seg = (ltid >> 3) & 7, j = (ltid >> 6) * 8 + cw;
        const BufRsrc rw = raw_buffer(p.w + vbase, vext * sizeof(TIn) / 4);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            gn[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                rw, (int)((((uint32_t)cc * 64 + 8 * seg + u) * ustride + j) * 4), 0, 0));
    };
    auto scan_w = [&](int Lcc) {
        const int seg = (ltid >> 3) & 7, ln = ltid & 63;
        float pr = 1.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if constexpr (kFused) gn[u] = decay_from_pre(gn[u]);
            if (8 * seg + u >= Lcc) gn[u] = 1.f;   // past the end of the sequence
            pr *= gn[u];
        }
        float inc = pr;   // product over segments 0 .. seg
#pragma unroll
        for (int d = 1; d < 8; d *= 2) {
            const float o = __builtin_bit_cast(
                float, __builtin_amdgcn_ds_bpermute(4 * ((ln - 8 * d) & 63), __builtin_bit_cast(int, inc)));
            inc = seg >= d ? inc * o : inc;
        }
        const float before = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(4 * ((ln - 8) & 63), __builtin_bit_cast(int, inc)));
        float pre_ = seg >= 1 ? before : 1.f;
        bool ok = true;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float wv = gn[u];
            pre_ *= wv;
            ok = ok && wv >= kWMin && wv <= 1.f && pre_ >= kGMin;
            gn[u] = pre_;
        }
        gok = ok;
    };
    auto store_g = [&]() {
        const int cw = ltid & 7, seg = (ltid >> 3) & 7, j = (ltid >> 6) * 8 + cw;
#pragma unroll
        for (int u = 0; u < 8; ++u) sG[sw(seg * 8 + u, j)] = gn[u];
        if (!gok) sBad = 1;   // every writer stores 1
    };
    {
        const int cl = ce - 1, Ll = chunk_len(cl);
#pragma unroll
        for (int q = 0; q < 7; ++q)
            if (!kDma || q != 1) issue_regs(cl, q);
        issue_s0(cl);
        if constexpr (kDma) {
            // r, a, b, v raw into LDS; k and dy stay in registers for the
            // chunk's prologue; the decay goes to sG
            load_w(cl);
#pragma unroll
            for (int q = 0; q < 7; ++q)
                if (q != 1 && q != 2 && q != 6) commit_regs(Ll, q);
            scan_w(Ll);
            store_g();
            __syncthreads();   // (later chunks: the barrier ending the previous one)
        } else {
#pragma unroll
            for (int q = 0; q < 7; ++q) commit_regs(Ll, q);
        }
    }

    for (int c = ce - 1; c >= cb; --c) {
        const int64_t t0 = (int64_t)c * 64;
        const int Lc = chunk_len(c);

        if constexpr (kDma) {
            // ---- prologue in one pass: g is in sG and r, a, b, v in their
            // arrays (published by the previous barrier); k and dy come from
            // registers, k scaled on the way in.  rb = r g, ab = a g_prev,
            // kt = k / g, bt = b / g; Hb = H g_63
            // Every read is issued before the first write, and the step
            // before t = 0 (decay 1) is a select, not a branch.
            refresh();
            float4 gm[2], gp[2], xr[2], xa[2], xb[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int u = ltid + 512 * m, t = u >> 4, j4 = (u & 15) << 2;
                const int o = sw(t, j4);
                gm[m] = lds4(sG, o);
                gp[m] = lds4(sG, sw(t > 0 ? t - 1 : 0, j4));
                xr[m] = lds4(sR, o);
                xa[m] = lds4(sA, o);
                xb[m] = lds4(sB, o);
            }
            commit_regs(Lc, 6);
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int u = ltid + 512 * m, t = u >> 4, j4 = (u & 15) << 2;
                const int o = sw(t, j4);
                const float4 gq = gm[m];
                const float4 gv = t > 0 ? gp[m] : make_float4(1.f, 1.f, 1.f, 1.f);
                const float4 inv = make_float4(__builtin_amdgcn_rcpf(gq.x), __builtin_amdgcn_rcpf(gq.y),
                                               __builtin_amdgcn_rcpf(gq.z), __builtin_amdgcn_rcpf(gq.w));
                const float4 kx = t < Lc ? InQuad<TIn>::f32(pre[2][m]) : make_float4(0.f, 0.f, 0.f, 0.f);
                put4(sK, o, make_float4(kx.x * inv.x, kx.y * inv.y, kx.z * inv.z, kx.w * inv.w));
                put4(sR, o, make_float4(xr[m].x * gq.x, xr[m].y * gq.y, xr[m].z * gq.z, xr[m].w * gq.w));
                if constexpr (kFused) {   // xa: kk, xb: gate; a = -kk, b = kk gate
                    const float4 ka = xa[m], gb = xb[m];
                    put4(sA, o, make_float4(-ka.x * gv.x, -ka.y * gv.y, -ka.z * gv.z, -ka.w * gv.w));
                    put4(sB, o, make_float4(ka.x * gb.x * inv.x, ka.y * gb.y * inv.y, ka.z * gb.z * inv.z,
                                            ka.w * gb.w * inv.w));
                } else {
                    put4(sA, o, make_float4(xa[m].x * gv.x, xa[m].y * gv.y, xa[m].z * gv.z, xa[m].w * gv.w));
                    put4(sB, o, make_float4(xb[m].x * inv.x, xb[m].y * inv.y, xb[m].z * inv.z, xb[m].w * inv.w));
                }
            }
        } else {
        // ---- inputs of the chunk into LDS (the last chunk is there already)
        if (c != ce - 1) {
#pragma unroll
            for (int q = 0; q < 7; ++q) commit_regs(64, q);
        }
        __syncthreads();
        refresh();

        // ---- cumulative decay, in place of w.  Wave w takes columns
        // 8 w .. 8 w + 7; lane (seg, c) the steps 8 seg .. 8 seg + 7 of column
        // 8 w + c: the product over its segment, then the product over the
        // earlier segments by a scan across the lanes (no barrier needed)
        {
            const int c = ltid & 7, seg = (ltid >> 3) & 7, j = (ltid >> 6) * 8 + c;
            const int ln = ltid & 63;
            float wseg[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                wseg[u] = sG[sw(seg * 8 + u, j)];
                if constexpr (kFused) wseg[u] = decay_from_pre(wseg[u]);
            }
            float pr = 1.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) pr *= wseg[u];
            float inc = pr;   // product over segments 0 .. seg
#pragma unroll
            for (int d = 1; d < 8; d *= 2) {
                const float o = __builtin_bit_cast(
                    float, __builtin_amdgcn_ds_bpermute(4 * ((ln - 8 * d) & 63), __builtin_bit_cast(int, inc)));
                inc = seg >= d ? inc * o : inc;
            }
            const float before = __builtin_bit_cast(
                float, __builtin_amdgcn_ds_bpermute(4 * ((ln - 8) & 63), __builtin_bit_cast(int, inc)));
            float pre_ = seg >= 1 ? before : 1.f;
            bool ok = true;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int o = sw(seg * 8 + u, j);
                const float wv = wseg[u];
                pre_ *= wv;
                ok = ok && wv >= kWMin && wv <= 1.f && pre_ >= kGMin;
                sG[o] = pre_;
            }
            if (!ok) sBad = 1;   // every writer stores 1
        }
        __syncthreads();
        refresh();

        // ---- rb = r g, ab = a g_prev, kt = k / g, bt = b / g
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int u = ltid + 512 * m, t = u >> 4, j4 = (u & 15) << 2;
            const int o = sw(t, j4);
            const float4 gm = lds4(sG, o);
            const float4 gp = t > 0 ? lds4(sG, sw(t - 1, j4)) : make_float4(1.f, 1.f, 1.f, 1.f);
            const float4 inv = make_float4(1.f / gm.x, 1.f / gm.y, 1.f / gm.z, 1.f / gm.w);
            float4 x = lds4(sR, o);
            put4(sR, o, make_float4(x.x * gm.x, x.y * gm.y, x.z * gm.z, x.w * gm.w));
            x = lds4(sK, o);
            put4(sK, o, make_float4(x.x * inv.x, x.y * inv.y, x.z * inv.z, x.w * inv.w));
            float4 xa = lds4(sA, o), xb = lds4(sB, o);
            if constexpr (kFused) {   // xa: kk, xb: gate; a = -kk, b = kk gate
                xb = make_float4(xa.x * xb.x, xa.y * xb.y, xa.z * xb.z, xa.w * xb.w);
                xa = make_float4(-xa.x, -xa.y, -xa.z, -xa.w);
            }
            put4(sA, o, make_float4(xa.x * gp.x, xa.y * gp.y, xa.z * gp.z, xa.w * gp.w));
            put4(sB, o, make_float4(xb.x * inv.x, xb.y * inv.y, xb.z * inv.z, xb.w * inv.w));
        }
        }   // bf16 prologue
        {
            const float g63 = sG[sw(63, jw)];
#pragma unroll
            for (int lb = 0; lb < 2; ++lb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sD[sw(16 * g + 4 * (2 * half + lb) + i, jw)] = Hc[lb][i] * g63;
        }
        __syncthreads();
        refresh();
        // the next chunk's decay factors, read now, formed during this chunk
        if (kDma && c > cb) load_w(c - 1);
        // Hb column jw (rows 16 g + s) and row jw (columns 16 g + s): the B
        // operands of its phase-2 products
        float hB[16], hR[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) hB[s] = sD[sw(16 * g + s, jw)];
        row16(sD, jw, 16 * g, hR);

        // Gram tiles: slot n < 10 holds rows of sX1 times rows of sY, slot
        // 10 + n rows of sX2 times rows of sY, for the lower block pair n
        // (rows a of the first factor, b of the second); the diagonal block
        // keeps a >= b for sX1 and a > b for sX2.  Wave w takes n = w, w + 8,
        // w + 16 (< 20), loading tile k + 1 while the MFMAs of tile k run;
        // side(k) is independent work placed beside tile k's MFMAs.
        auto gram_store = [&](int n, f4 acc) {
            const int pr = n < 10 ? n : n - 10;
            // on a diagonal tile, rows al < l16 (first Gram) or al <= l16
            // (second) are zero: rows al < lim, selected without branches
            const int lim = tab(pr) != tbb(pr) ? 0 : n < 10 ? l16 : l16 + 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) sP[n * 256 + A.pa[i]] = 4 * g + i < lim ? 0.f : acc[i];
        };
        auto gram = [&](const float *sX1, const float *sX2, const float *sY, auto side) {
            float xa[16], ya[16], xb[16], yb[16];
            auto load = [&](int n, float (&xv)[16], float (&yv)[16]) {
                const int pr = n < 10 ? n : n - 10;
                rowl(n < 10 ? sX1 : sX2, A, tab(pr), xv);
                rowl(sY, A, tbb(pr), yv);
            };
            auto run = [&](int n, const float (&xv)[16], const float (&yv)[16]) {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 16; ++s) acc = mfma(xv[s], yv[s], acc);
                gram_store(n, acc);
            };
            load(wave, xa, ya);
            load(wave + 8, xb, yb);
            side(0);
            run(wave, xa, ya);
            sched_fence();
            if (wave + 16 < 20) load(wave + 16, xa, ya);
            side(1);
            run(wave + 8, xb, yb);
            sched_fence();
            side(2);
            if (wave + 16 < 20) run(wave + 16, xa, ya);
            sched_fence();
        };
        auto none = [](int) {};
        // Gram tile slot elements (4 g + s, l16) and (l16, 4 g + s), and
        // element (16 ub + 4 g + s, jw) of an array
        auto tA = [&](int slot, int s) { return sP[slot * 256 + A.pa[s]]; };
        auto tAt = [&](int slot, int s) { return sP[slot * 256 + A.pb[s]]; };
        auto colE = [&](const float *arr, int ub, int s) { return arr[A.col[s] + 1024 * ub]; };

        auto body = [&](auto hc) {
            constexpr int HF = decltype(hc)::value;
            constexpr int TB[2] = {HF ? 1 : 0, HF ? 2 : 3};   // this wave's time blocks
            // X[lt] += rows of sX in time block TB[lt] times bv (K = 64)
            auto rows2 = [&](f4 (&X)[2], const float *sX, const float (&bv)[16]) {
                pipelined<2, 16>([&](int lt, float (&b)[16]) { rowl(sX, A, TB[lt], b); },
                                 [&](int lt, const float (&b)[16]) {
#pragma unroll
                                     for (int s = 0; s < 16; ++s) X[lt] = mfma(b[s], bv[s], X[lt]);
                                 });
            };
            f4 XR[2], XA[2], XK[2], XB[2], XV[2];
#pragma unroll
            for (int lt = 0; lt < 2; ++lt) {
                XR[lt] = f4{0.f, 0.f, 0.f, 0.f};
                XA[lt] = XR[lt];
                XK[lt] = XR[lt];
                XB[lt] = XR[lt];
                XV[lt] = XR[lt];
            }
            // the state gradient entering the chunk, this wave's rows: Hb,
            // then + sum_u dy_u rb_u^T (now) and dsa_u ab_u^T (once dsa is
            // known).  MFMA row m = l16 stands for row 16 (m / 4) + 4 ib + m % 4.
            f4 Hn[2];
#pragma unroll
            for (int lb = 0; lb < 2; ++lb)
#pragma unroll
                for (int i = 0; i < 4; ++i) Hn[lb][i] = hB[4 * (2 * HF + lb) + i];
            auto hprev_part = [&](const float *sX, const float *sF) {
                pipelined<16, 6>(
                    [&](int k, float (&b)[6]) {
                        const int ub = k >> 2, s = k & 3;
                        b[0] = colE(sF, ub, s);
#pragma unroll
                        for (int lb = 0; lb < 2; ++lb)
                            b[1 + lb] = sX[1024 * ub + sw(4 * g + s, 16 * (l16 >> 2) + 4 * (2 * HF + lb) + (l16 & 3))];
                    },
                    [&](int k, const float (&b)[6]) {
#pragma unroll
                        for (int lb = 0; lb < 2; ++lb) Hn[lb] = mfma(b[1 + lb], b[0], Hn[lb]);
                    });
            };
            // the products that do not need dsa
            auto pd_xk = [&]() { rows2(XK, sVS, hB); };    // Hb^T v_t
            auto pd_xr = [&]() { rows2(XR, sDY, s0B); };   // S0^T dy_t
            auto pd_xv = [&]() { rows2(XV, sK, hR); };     // Hb kt_t
            auto pd_h = [&]() { hprev_part(sDY, sR); };

            // ---- dsa for the chunk: dsa_t = rhs_t + sum_{u>t} dsa_u (ab_u . bt_t),
            // rhs_t = Hb bt_t + sum_{u>=t} dy_u (rb_u . bt_t).  Rows i = jw,
            // steps t = 16 tb + 4 g + i of f4 Rt[tb].  Blocked back
            // substitution: the inverse of each 16x16 diagonal block,
            // T_b = (I - N_b)^-1 with N_b[t][u] = ab_u . bt_t (u > t, both in
            // block b), depends only on ab and bt, so the second-half wave fb
            // forms T_fb (the step-by-step substitution with the 16 unit
            // vectors as right-hand sides, one per lane column, each finished
            // value broadcast across the row groups) while the first-half
            // waves form rhs; the first half then applies T_3, updates the
            // earlier blocks, applies T_2, ... on MFMA, while the second half
            // runs its dsa-free products on the same matrix cores.
            gram(sR, sA, sB, none);
            __syncthreads();
            refresh();
            f4 Rt[4];
            if constexpr (HF == 0) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) Rt[tb] = f4{0.f, 0.f, 0.f, 0.f};
                rows_times(Rt, sB, A, hR);
                pipelined<16, 5>(
                    [&](int k, float (&b)[5]) {
                        const int ub = k >> 2, s = k & 3;
                        b[0] = colE(sDY, ub, s);
#pragma unroll
                        for (int tb = 0; tb <= ub; ++tb) b[1 + tb] = tA(tix(ub, tb), s);
                    },
                    [&](int k, const float (&b)[5]) {
                        const int ub = k >> 2;
#pragma unroll
                        for (int tb = 0; tb <= ub; ++tb) Rt[tb] = mfma(b[1 + tb], b[0], Rt[tb]);
                    });
                // the second-half waves' block inverses take longer than
                // the right-hand side: two dsa-free products fit beside them
                if constexpr (full) {
                    pd_xk();
                    pd_xv();
                }
            } else {
                const int slot = 10 + tix(fb, fb);
                f4 X;
#pragma unroll
                for (int i = 0; i < 4; ++i) X[i] = (4 * g + i == l16) ? 1.f : 0.f;
                // the coefficient rows are read four steps ahead of the chain
                float4 m[4];
                // row tl, columns 4 g .. 4 g + 3 (stored as one aligned group,
                // column 4 g + j in component j ^ (tl & 3))
                auto mrow = [&](int tl) {
                    const float4 q = lds4(sP, slot * 256 + (pt(tl, 4 * g) & ~3));
                    const float c[4] = {q.x, q.y, q.z, q.w};
                    const int x = tl & 3;
                    return make_float4(c[x], c[1 ^ x], c[2 ^ x], c[3 ^ x]);
                };
#pragma unroll
                for (int tl = 15; tl >= 12; --tl) m[tl & 3] = mrow(tl);
#pragma unroll
                for (int tl = 15; tl >= 1; --tl) {
                    const float d = tl >= 12 ? bcast_group<3>(X[tl & 3])
                                  : tl >= 8 ? bcast_group<2>(X[tl & 3])
                                  : tl >= 4 ? bcast_group<1>(X[tl & 3])
                                            : bcast_group<0>(X[tl & 3]);
                    const float4 mm = m[tl & 3];
                    if (tl >= 5) m[tl & 3] = mrow(tl - 4);
                    X[0] = fmaf(mm.x, d, X[0]);
                    X[1] = fmaf(mm.y, d, X[1]);
                    X[2] = fmaf(mm.z, d, X[2]);
                    X[3] = fmaf(mm.w, d, X[3]);
                }
                // T_fb[t][c] at tile position (t, c)
#pragma unroll
                for (int i = 0; i < 4; ++i) sTT[fb * 256 + A.pa[i]] = X[i];
                if constexpr (full) {
                    pd_xk();
                    pd_xv();
                }
            }
            __syncthreads();
            refresh();
            if constexpr (HF == 0) {
                auto apply_block = [&](auto tbc) {
                    constexpr int tb = decltype(tbc)::value;
                    f4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 4; ++s) x = mfma(sTT[tb * 256 + A.pb[s]], Rt[tb][s], x);
                    Rt[tb] = x;
#pragma unroll
                    for (int tp = 0; tp < tb; ++tp)
#pragma unroll
                        for (int s = 0; s < 4; ++s) Rt[tp] = mfma(tA(10 + tix(tb, tp), s), Rt[tb][s], Rt[tp]);
                };
                // the dsa-free products fill the gaps of the dependent chain
                apply_block(std::integral_constant<int, 3>{});
                if constexpr (full) pd_xr();
                apply_block(std::integral_constant<int, 2>{});
                apply_block(std::integral_constant<int, 1>{});
                pd_h();
                apply_block(std::integral_constant<int, 0>{});
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * tb + 4 * g + i;
                        sD[A.col[i] + 1024 * tb] = t < Lc ? Rt[tb][i] : 0.f;
                    }
            } else {
                if constexpr (full) pd_xr();
                pd_h();
            }
            __syncthreads();
            refresh();
            hprev_part(sD, sA);
            if constexpr (full) rows2(XA, sD, s0B);    // S0^T dsa_t
            // c_j = sum_i (dL/dS0)[i][j] S0[i][j]: this wave's rows; ds0 after
            // the first chunk
            {
                float cp = 0.f;
#pragma unroll
                for (int lb = 0; lb < 2; ++lb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) cp = fmaf(Hn[lb][i], s0B[4 * (2 * HF + lb) + i], cp);
                cp = swap_add16(cp, cp);
                cp = swap_add32(cp, cp);
                if (g == 0 && full) sCj[HF][jw] = cp;
                if (c == cb && ds0u) {
#pragma unroll
                    for (int lb = 0; lb < 2; ++lb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            ds0u[(16 * g + 4 * (2 * HF + lb) + i) * 64 + jw] = Hn[lb][i];
                }
#pragma unroll
                for (int lb = 0; lb < 2; ++lb) Hc[lb] = Hn[lb];
            }
            if (c > cb) issue_s0(c - 1);   // this chunk's S0 column is no longer needed
            // sa for the second pass, loaded while the first one runs
            float4 saR[2];
            if constexpr (full) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int u = ltid + 512 * m, t = u >> 4, j4 = (u & 15) << 2;
                    saR[m] = bload4(raw_buffer(p.sa + vbase, vext), (((uint32_t)t0 + t) * ustride + j4) * 4);
                }
            }

            // One pass over the Grams of the value-side vectors in sVS (v,
            // then sa): X (dk, then db bracket) gets sum_{u>=t} rb_u (dy_u.x_t)
            // + sum_{u>t} ab_u (dsa_u.x_t); the dr, da brackets get
            // sum_{u<=t} f_u (x_u.dy_t) and sum_{u<t} f_u (x_u.dsa_t) with the
            // key-side vector sF (kt, then bt).  Groups (ub, s); per group the
            // operands br, ba, bf, then the A operands in MFMA order.
            auto value_terms = [&](f4 (&X)[2], const float *sF) {
                pipelined<16, 11>(
                    [&](int k, float (&b)[11]) {
                        const int ub = k >> 2, s = k & 3;
                        b[0] = colE(sR, ub, s);
                        b[1] = colE(sA, ub, s);
                        b[2] = colE(sF, ub, s);
                        int n = 3;
#pragma unroll
                        for (int lt = 0; lt < 2; ++lt)
                            if (TB[lt] <= ub) {
                                b[n++] = tA(tix(ub, TB[lt]), s);
                                b[n++] = tA(10 + tix(ub, TB[lt]), s);
                            }
#pragma unroll
                        for (int lt = 0; lt < 2; ++lt)
                            if (TB[lt] >= ub) {
                                b[n++] = tAt(tix(TB[lt], ub), s);
                                b[n++] = tAt(10 + tix(TB[lt], ub), s);
                            }
                    },
                    [&](int k, const float (&b)[11]) {
                        const int ub = k >> 2;
                        int n = 3;
#pragma unroll
                        for (int lt = 0; lt < 2; ++lt)
                            if (TB[lt] <= ub) {
                                X[lt] = mfma(b[n], b[0], X[lt]);
                                X[lt] = mfma(b[n + 1], b[1], X[lt]);
                                n += 2;
                            }
#pragma unroll
                        for (int lt = 0; lt < 2; ++lt)
                            if (TB[lt] >= ub) {
                                XR[lt] = mfma(b[n], b[2], XR[lt]);
                                XA[lt] = mfma(b[n + 1], b[2], XA[lt]);
                                n += 2;
                            }
                    });
            };

            // ---- pass 1: Grams dy v^T, dsa v^T; dk bracket; kt terms of dr, da.
            // v is not read after the Grams: sa replaces it during the pass.
            if constexpr (full) gram(sDY, sD, sVS, none);
            __syncthreads();
            refresh();
            if constexpr (full) {
                value_terms(XK, sK);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int u = ltid + 512 * m, t = u >> 4, j4 = (u & 15) << 2;
                    put4(sVS, sw(t, j4), saR[m]);
                }
            }
            __syncthreads();
            refresh();

            // ---- pass 2: Grams dy sa^T, dsa sa^T (dk written beside them);
            // db bracket; bt terms of dr, da; then the per-block sums of
            // k dk + b db - r dr - a da for the dw prefix
            // this (b, h)'s outputs; element (t0 + t, jw) at byte offset ooff(t)
            const BufRsrc odk = raw_buffer(p.dk + vbase, vext), odb = raw_buffer(p.db + vbase, vext);
            const BufRsrc odr = raw_buffer(p.dr + vbase, vext), oda = raw_buffer(p.da + vbase, vext);
            const BufRsrc odw = raw_buffer(p.dw + vbase, vext), odv = raw_buffer(p.dv + vbase, vext);
            auto ooff = [&](int t) { return (((uint32_t)t0 + t) * ustride + jw) * 4; };
            if constexpr (full) gram(sDY, sD, sVS, [&](int k) {
                if (k > 1) return;
                const int tb = TB[k];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * tb + 4 * g + i;
                    const float gt = sG[A.col[i] + 1024 * tb];
                    bstore(odk, ooff(t), XK[k][i] * __builtin_amdgcn_rcpf(gt));
                }
            });
            __syncthreads();
            refresh();
            // fused inputs: the gate and the decay pre-activation at this
            // lane's output steps, for the outputs after the next barrier
            float gate[2][4], omg[2][4];
            if constexpr (kFused && full) {
                const BufRsrc rg = raw_buffer(p.b + vbase, vext * sizeof(TIn) / 4);
                const BufRsrc rw = raw_buffer(p.w + vbase, vext * sizeof(TIn) / 4);
#pragma unroll
                for (int lt = 0; lt < 2; ++lt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t e = ((uint32_t)t0 + 16 * TB[lt] + 4 * g + i) * ustride + jw;
                        gate[lt][i] = bload1<TIn>(rg, e);
                        omg[lt][i] = bload1<TIn>(rw, e);
                    }
            }
            float f[2][4];
            if constexpr (full) {
                rows2(XB, sVS, hB);    // Hb^T sa_t
                value_terms(XB, sB);
#pragma unroll
                for (int lt = 0; lt < 2; ++lt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int o = A.col[i] + 1024 * TB[lt];
                        f[lt][i] = sK[o] * XK[lt][i] + sB[o] * XB[lt][i] - sR[o] * XR[lt][i] -
                                   sA[o] * XA[lt][i];
                    }
                    sScan[fb][(4 * TB[lt] + g) * 16 + l16] = ((f[lt][0] + f[lt][1]) + f[lt][2]) + f[lt][3];
                }
            }
            __syncthreads();
            refresh();
            // next chunk: v (sa is done with) and, through registers, k and dy
            if (c > cb) {
#pragma unroll
                for (int q = 0; q < 7; ++q) {
                    if (kDma && q == 5) issue_dma(c - 1, q);
                    else if (!kDma || q == 2 || q == 6) issue_regs(c - 1, q);
                }
            }

            // ---- outputs db, dr, da, dw (dw: prefix over steps of
            // k dk + b db - r dr - a da), beside the pass-3 Grams rb kt^T, ab kt^T
            float pre16[17];
            auto outputs = [&](int k) {
                if (k == 0) {
                    // exclusive prefix of the 16 block sums of column jw (fixed order)
                    pre16[0] = 0.f;
#pragma unroll
                    for (int q = 0; q < 16; ++q) pre16[q + 1] = pre16[q] + sScan[fb][q * 16 + l16];
                    return;
                }
                if (k > 2) return;
                const int lt = k - 1, tb = TB[lt];
                const float cj = sCj[0][jw] + sCj[1][jw];
                const int q0 = 4 * tb + g;
                float ex = g == 0 ? pre16[4 * tb] : g == 1 ? pre16[4 * tb + 1]
                         : g == 2 ? pre16[4 * tb + 2] : pre16[4 * tb + 3];
                (void)q0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * tb + 4 * g + i;
                    const int o = A.col[i] + 1024 * tb;
                    const float gt = sG[o];
                    const float gp = i > 0 ? sG[A.col[i - 1] + 1024 * tb] : t > 0 ? sG[sw(t - 1, jw)] : 1.f;
                    const float inv = __builtin_amdgcn_rcpf(gt);
                    const float adA = sA[o] * XA[lt][i];
                    const float wdw = (cj + ex) - adA;
                    const uint32_t off = ooff(t);
                    bstore(odr, off, XR[lt][i] * gt);
                    if constexpr (kFused) {
                        // a = -kk: kk from ab = a g_{t-1}.  d omega = (w dw) ln w
                        // (1 - s) with ln w = -c s, s = sigmoid(omega), formed from
                        // omega itself: ln(g_t / g_{t-1}) would lose its digits
                        // as w nears 1
                        const float rgp = __builtin_amdgcn_rcpf(gp);
                        const float da_ = XA[lt][i] * gp, db_ = XB[lt][i] * inv;
                        const float kk = -sA[o] * rgp;
                        const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * omg[lt][i]));
                        bstore(odb, off, kk * db_);
                        bstore(oda, off, fmaf(gate[lt][i], db_, -da_));
                        bstore(odw, off, wdw * (-kDecayCoeff * sg) * (1.f - sg));
                    } else {
                        bstore(odb, off, XB[lt][i] * inv);
                        bstore(oda, off, XA[lt][i] * gp);
                        bstore(odw, off, wdw * gp * inv);
                    }
                    ex += f[lt][i];
                }
            };
            if constexpr (full) gram(sR, sA, sK, outputs);
            __syncthreads();
            refresh();
            // next chunk: r, w, a, b straight into their (now free) arrays
            if (kDma && c > cb) {
                issue_dma(c - 1, 0);
                issue_dma(c - 1, 3);
                issue_dma(c - 1, 4);
                // sG is done with: the next chunk's cumulative decay
                scan_w(64);
                store_g();
            }
            sched_fence();

            // ---- dv = Hb kt_t + sum_{u>=t} dy_u (rb_u . kt_t) + sum_{u>t} dsa_u (ab_u . kt_t)
            if constexpr (full) pipelined<16, 6>(
                [&](int k, float (&b)[6]) {
                    const int ub = k >> 2, s = k & 3;
                    b[0] = colE(sDY, ub, s);
                    b[1] = colE(sD, ub, s);
                    int n = 2;
#pragma unroll
                    for (int lt = 0; lt < 2; ++lt)
                        if (TB[lt] <= ub) {
                            b[n++] = tA(tix(ub, TB[lt]), s);
                            b[n++] = tA(10 + tix(ub, TB[lt]), s);
                        }
                },
                [&](int k, const float (&b)[6]) {
                    const int ub = k >> 2;
                    int n = 2;
#pragma unroll
                    for (int lt = 0; lt < 2; ++lt)
                        if (TB[lt] <= ub) {
                            XV[lt] = mfma(b[n], b[0], XV[lt]);
                            XV[lt] = mfma(b[n + 1], b[1], XV[lt]);
                            n += 2;
                        }
                });
            // the next chunk's copies land before the barrier that publishes
            // them; the wait (for every earlier memory operation of the wave)
            // comes before dv's stores, so that it does not wait for them
            if (kDma && c > cb) wait_dma();
            if constexpr (full) {
#pragma unroll
                for (int lt = 0; lt < 2; ++lt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * TB[lt] + 4 * g + i;
                        bstore(odv, ooff(t), XV[lt][i]);
                    }
            }
            __syncthreads();
            refresh();
        };
        if (half == 0) body(std::integral_constant<int, 0>{});
        else body(std::integral_constant<int, 1>{});
    }

    __syncthreads();
    if (tid == 0) p.flags[fidx] = sBad;
}

template <typename TIn, bool kFused>
hipError_t launch_bwdc_t(const BwdLaunch &a, int *flags, int mode, hipStream_t stream)
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
    p.mode = mode;
    p.nseg = a.nseg;
    p.nckseg = a.nckseg;
    p.gbuf = a.gbuf;
    const int64_t units = mode == 0 ? a.B * a.H : mode == 1 ? a.B * a.H * (a.nseg - 1) : a.B * a.H * a.nseg;
    if (mode == 1)
        hipLaunchKernelGGL((wkv7_bwdc_kernel<TIn, kFused, true>), dim3((unsigned)units), dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((wkv7_bwdc_kernel<TIn, kFused, false>), dim3((unsigned)units), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool chunked_backward_supported(const BwdLaunch &a)
{
    return a.N == 64 && a.chunk == 64 && chunk_offsets_fit(a.T, a.H);
}

hipError_t launch_backward_chunked(const BwdLaunch &a, int *flags, int mode, hipStream_t stream)
{
    if (a.fused)
        return a.dtype == 0 ? launch_bwdc_t<float, true>(a, flags, mode, stream)
                            : launch_bwdc_t<uint16_t, true>(a, flags, mode, stream);
    return a.dtype == 0 ? launch_bwdc_t<float, false>(a, flags, mode, stream)
                        : launch_bwdc_t<uint16_t, false>(a, flags, mode, stream);
}

}  // namespace wkv7
