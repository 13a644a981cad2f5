// WKV7 reverse (backward-through-time) scan on gfx950.
//
// Per (batch b, head h), with G = dL/dS seeded by dsT, walking t from T-1
// down to 0 (the three steps of rx_wkv7_backward on the Foundry
// "rwkvx/rx_pretrain.c" page; P = state before step t, St = state after):
//   dr = St^T dy;  G += dy r^T
//   dk = G^T v;  db = G^T sa;  dw[j] = sum_i G[i][j] P[i][j]
//   dv = G k;  dsa = G b
//   da = P^T dsa;  G <- G diag(w) + dsa a^T
// and ds0 = G at the end.
//
// States are not cached for all T (the page keeps T*N*N floats).  The
// forward leaves a checkpoint every C steps; each chunk of C steps is
// replayed forward from its checkpoint once to write sub-checkpoints every
// KS steps into workspace (pass A), then sub-chunks are taken in reverse:
// KS + 1 states are regenerated into registers and the KS reverse steps run
// on them (pass B).  G stays in registers for the whole sequence.
//
// Tiling: each lane holds an R x CC block of P/St/G.  Rows of G evolve
// independently (dsa and dv are row dots: DPP sums over the LPR lanes of a
// row group); the five column sums dr, dk, db, dw, da are reduced first in
// lane over R rows, then across the row groups of a wave with gfx950
// permlane swaps (exchange-and-add, leaving each lane one column), then
// across waves through LDS in a fixed order: no atomics, deterministic.

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

template <int N> struct BwdTile;
template <> struct BwdTile<64> { static constexpr int R = 4, CC = 4; };
template <> struct BwdTile<16> { static constexpr int R = 1, CC = 4; };

template <int N>
struct BwdGeom {
    static constexpr int R = BwdTile<N>::R;
    static constexpr int CC = BwdTile<N>::CC;
    static constexpr int LPR = N / CC;              // lanes sharing a row
    static constexpr int RG = kWave / LPR;          // row groups per wave
    static constexpr int RW = RG * R;               // rows per wave
    static constexpr int NW = N / RW;               // waves per workgroup
    static constexpr int NT = NW * kWave;
    static constexpr int KS = kSubChunk;
    static constexpr int NV = 7;                    // r, w, k, v, a, b, dy
    static constexpr int NQ = 5;                    // dr, dk, db, dw, da
    static_assert(CC == 4 && LPR >= 4 && LPR <= 16, "column reduction assumes 4 columns per lane");
};

enum { kR = 0, kW = 1, kK = 2, kV = 3, kA = 4, kB = 5, kDY = 6 };
enum { qDR = 0, qDK = 1, qDB = 2, qDW = 3, qDA = 4 };

template <typename TIn>
struct BwdArgs {
    VecPtrs<TIn, 7> in;
    const float *ckpt, *dsT;
    float *dr, *dw, *dk, *dv, *da, *db, *ds0;
    float *sub;
    int64_t T, H;
    int chunk, nck, nsubw;   // nsubw: sub-checkpoint slots per (b, h)
};

// One unit of work: sub-chunk s of chunk c, in pass A (forward replay) or
// pass B (regenerate + reverse).
struct Item {
    int c, s;
    bool B;
};

template <int N, typename TIn>
__global__ void __launch_bounds__(BwdGeom<N>::NT)
wkv7_bwd_kernel(BwdArgs<TIn> p)
{
    using Gm = BwdGeom<N>;
    constexpr int R = Gm::R, CC = Gm::CC, LPR = Gm::LPR, RW = Gm::RW, NW = Gm::NW;
    constexpr int NT = Gm::NT, KS = Gm::KS, NV = Gm::NV, NQ = Gm::NQ;
    __shared__ __align__(16) float stg[2][NV][KS][N];
    __shared__ __align__(16) float part[KS][NQ][NW][N];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = lane % LPR, rg = lane / LPR;
    const int row0 = wave * RW + rg * R, col0 = cg * CC;
    const int64_t bh = blockIdx.x, T = p.T, H = p.H;
    const int64_t b = bh / H, h = bh % H;
    const int64_t stride = H * N;
    const int64_t vbase = (b * T * H + h) * N;
    const int C = p.chunk;
    const int64_t NN = (int64_t)N * N;
    const int64_t toff = (int64_t)row0 * N + col0;   // this lane's block in a state

    // Column this lane holds after the cross-row-group reduction, and whether
    // it is the one lane of its duplicates that writes it.
    const int ccol = col0 + ((lane >> 4) & 3);
    const bool cwriter = (LPR == 16) || (LPR == 8 && ((lane >> 3) & 1) == 0) ||
                         (LPR == 4 && ((lane >> 2) & 3) == 0);

    auto nsub_of = [&](int c) -> int {
        const int64_t len = T - (int64_t)c * C < C ? T - (int64_t)c * C : C;
        return (int)((len + KS - 1) / KS);
    };
    auto first_of = [&](int c) -> Item { return Item{c, 0, nsub_of(c) < 2}; };
    auto next_of = [&](Item it) -> Item {
        const int ns = nsub_of(it.c);
        if (!it.B) return it.s + 1 <= ns - 2 ? Item{it.c, it.s + 1, false} : Item{it.c, ns - 1, true};
        if (it.s > 0) return Item{it.c, it.s - 1, true};
        return it.c > 0 ? first_of(it.c - 1) : Item{-1, 0, true};
    };
    auto t_begin = [&](Item it) -> int64_t { return (int64_t)it.c * C + (int64_t)it.s * KS; };
    auto n_steps = [&](Item it) -> int {
        const int64_t rem = T - t_begin(it);
        return (int)(rem < KS ? rem : KS);
    };
    // Whether the item starts from a stored state (else it continues from
    // the state the previous item left in registers), and where that is.
    auto loads_state = [&](Item it) -> bool {
        const int ns = nsub_of(it.c);
        return it.B ? (it.s < ns - 1 || ns == 1) : it.s == 0;
    };
    auto state_src = [&](Item it) -> const float * {
        return it.s == 0 ? p.ckpt + (bh * p.nck + it.c) * NN
                         : p.sub + (bh * p.nsubw + (it.s - 1)) * NN;
    };

    auto load_block = [&](const float *src, float (&X)[R][CC]) {
#pragma unroll
        for (int e = 0; e < R; ++e)
#pragma unroll
            for (int c = 0; c < CC; c += 4) {
                const float4 q = *reinterpret_cast<const float4 *>(src + toff + e * N + c);
                X[e][c] = q.x; X[e][c + 1] = q.y; X[e][c + 2] = q.z; X[e][c + 3] = q.w;
            }
    };
    auto store_block = [&](float *dst, const float (&X)[R][CC]) {
#pragma unroll
        for (int e = 0; e < R; ++e)
#pragma unroll
            for (int c = 0; c < CC; c += 4)
                *reinterpret_cast<float4 *>(dst + toff + e * N + c) =
                    make_float4(X[e][c], X[e][c + 1], X[e][c + 2], X[e][c + 3]);
    };
    auto col_vals = [&](const float *Ls, int q, float (&x)[CC]) {
        const float4 v4 = *reinterpret_cast<const float4 *>(Ls + q * KS * N + col0);
        x[0] = v4.x; x[1] = v4.y; x[2] = v4.z; x[3] = v4.w;
    };
    auto row_vals = [&](const float *Ls, int q, float (&x)[R]) {
#pragma unroll
        for (int e = 0; e < R; ++e) x[e] = Ls[q * KS * N + row0 + e];
    };
    // One forward step on X in place; returns sa (pre-update S a) per row.
    auto fwd_step = [&](const float *Ls, float (&X)[R][CC], float (&sa)[R]) {
        float va[CC], vw[CC], vk[CC], vb[CC], vv[R];
        col_vals(Ls, kA, va);
        col_vals(Ls, kW, vw);
        col_vals(Ls, kK, vk);
        col_vals(Ls, kB, vb);
        row_vals(Ls, kV, vv);
#pragma unroll
        for (int e = 0; e < R; ++e) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < CC; ++c) acc = fmaf(X[e][c], va[c], acc);
            sa[e] = group_allreduce<LPR>(acc);
        }
#pragma unroll
        for (int e = 0; e < R; ++e)
#pragma unroll
            for (int c = 0; c < CC; ++c)
                X[e][c] = fmaf(X[e][c], vw[c], fmaf(vv[e], vk[c], sa[e] * vb[c]));
    };

    // ---- seed G with dsT
    float G[R][CC];
    if (p.dsT) {
        load_block(p.dsT + bh * NN, G);
    } else {
#pragma unroll
        for (int e = 0; e < R; ++e)
#pragma unroll
            for (int c = 0; c < CC; ++c) G[e][c] = 0.f;
    }

    Stager<TIn, NV, KS, N, NT> stage;
    float S[R][CC], Snext[R][CC];
    Item it = first_of(p.nck - 1);
    stage.issue(p.in, vbase + t_begin(it) * stride, stride, n_steps(it), tid);
    load_block(state_src(it), S);
    stage.commit(&stg[0][0][0][0], n_steps(it), tid);
    __syncthreads();
    int buf = 0;

    while (it.c >= 0) {
        const Item nx = next_of(it);
        const bool have_next = nx.c >= 0;
        const bool nx_load = have_next && loads_state(nx);
        if (have_next) stage.issue(p.in, vbase + t_begin(nx) * stride, stride, n_steps(nx), tid);
        if (nx_load) load_block(state_src(nx), Snext);
        const float *L = &stg[buf][0][0][0];
        const int nst = n_steps(it);
        const int64_t tb = t_begin(it);

        if (!it.B) {
            // ---- pass A: replay KS steps, then leave a sub-checkpoint when a
            // later pass-B item will start from it.
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                float sa[R];
                fwd_step(L + j * N, S, sa);
            }
            if (it.s + 1 <= nsub_of(it.c) - 2)
                store_block(p.sub + (bh * p.nsubw + it.s) * NN, S);
        } else {
            // ---- pass B: regenerate the sub-chunk's states into registers
            float P[KS + 1][R][CC];
            float sav[KS][R];
#pragma unroll
            for (int e = 0; e < R; ++e)
#pragma unroll
                for (int c = 0; c < CC; ++c) P[0][e][c] = S[e][c];
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                if (j < nst) {
#pragma unroll
                    for (int e = 0; e < R; ++e)
#pragma unroll
                        for (int c = 0; c < CC; ++c) P[j + 1][e][c] = P[j][e][c];
                    fwd_step(L + j * N, P[j + 1], sav[j]);
                }
            }
            // ---- reverse steps
#pragma unroll
            for (int j = KS - 1; j >= 0; --j) {
                if (j >= nst) continue;
                const float *Ls = L + j * N;
                float vr[CC], vw[CC], vk[CC], va[CC], vb[CC], vv[R], vdy[R];
                col_vals(Ls, kR, vr);
                col_vals(Ls, kW, vw);
                col_vals(Ls, kK, vk);
                col_vals(Ls, kA, va);
                col_vals(Ls, kB, vb);
                row_vals(Ls, kV, vv);
                row_vals(Ls, kDY, vdy);

                // read-out: G += dy r^T; dr partial from the post-step state
                float cq[NQ][CC];
#pragma unroll
                for (int c = 0; c < CC; ++c) {
                    float pdr = 0.f;
#pragma unroll
                    for (int e = 0; e < R; ++e) {
                        pdr = fmaf(P[j + 1][e][c], vdy[e], pdr);
                        G[e][c] = fmaf(vdy[e], vr[c], G[e][c]);
                    }
                    cq[qDR][c] = pdr;
                }
                // update gradients
                float dvp[R], dsap[R];
#pragma unroll
                for (int e = 0; e < R; ++e) {
                    float x = 0.f, y = 0.f;
#pragma unroll
                    for (int c = 0; c < CC; ++c) {
                        x = fmaf(G[e][c], vk[c], x);
                        y = fmaf(G[e][c], vb[c], y);
                    }
                    dvp[e] = x;
                    dsap[e] = y;
                }
#pragma unroll
                for (int c = 0; c < CC; ++c) {
                    float xk = 0.f, xb = 0.f, xw = 0.f;
#pragma unroll
                    for (int e = 0; e < R; ++e) {
                        xk = fmaf(G[e][c], vv[e], xk);
                        xb = fmaf(G[e][c], sav[j][e], xb);
                        xw = fmaf(G[e][c], P[j][e][c], xw);
                    }
                    cq[qDK][c] = xk;
                    cq[qDB][c] = xb;
                    cq[qDW][c] = xw;
                }
                float dsa[R], dvv[R];
#pragma unroll
                for (int e = 0; e < R; ++e) {
                    dsa[e] = group_allreduce<LPR>(dsap[e]);
                    dvv[e] = group_allreduce<LPR>(dvp[e]);
                }
                // in-context term and carry to t-1
#pragma unroll
                for (int c = 0; c < CC; ++c) {
                    float x = 0.f;
#pragma unroll
                    for (int e = 0; e < R; ++e) {
                        x = fmaf(dsa[e], P[j][e][c], x);
                        G[e][c] = fmaf(G[e][c], vw[c], dsa[e] * va[c]);
                    }
                    cq[qDA][c] = x;
                }
                // column sums across the row groups of the wave
                float cs[NQ];
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const float u0 = swap_add32(cq[q][0], cq[q][2]);
                    const float u1 = swap_add32(cq[q][1], cq[q][3]);
                    float x = swap_add16(u0, u1);
                    if constexpr (LPR <= 8) x += dpp<kDppRor8>(x);
                    if constexpr (LPR <= 4) x += dpp<kDppRor4>(x);
                    cs[q] = x;
                }
                if (cwriter) {
#pragma unroll
                    for (int q = 0; q < NQ; ++q) part[j][q][wave][ccol] = cs[q];
                }
                if (cg == 0) {
                    float *dst = p.dv + vbase + (tb + j) * stride + row0;
                    if constexpr (R == 4)
                        *reinterpret_cast<float4 *>(dst) = make_float4(dvv[0], dvv[1], dvv[2], dvv[3]);
                    else
#pragma unroll
                        for (int e = 0; e < R; ++e) dst[e] = dvv[e];
                }
            }
            __syncthreads();
            // ---- column outputs of the sub-chunk: fixed-order sum over waves
            for (int idx = tid; idx < nst * NQ * N; idx += NT) {
                const int col = idx % N;
                const int q = (idx / N) % NQ;
                const int j = idx / (N * NQ);
                float x = part[j][q][0][col];
#pragma unroll
                for (int w = 1; w < NW; ++w) x += part[j][q][w][col];
                float *dst = p.dr;
                if (q == qDK) dst = p.dk;
                if (q == qDB) dst = p.db;
                if (q == qDW) dst = p.dw;
                if (q == qDA) dst = p.da;
                dst[vbase + (tb + j) * stride + col] = x;
            }
        }

        if (have_next) {
            stage.commit(&stg[buf ^ 1][0][0][0], n_steps(nx), tid);
            if (nx_load) {
#pragma unroll
                for (int e = 0; e < R; ++e)
#pragma unroll
                    for (int c = 0; c < CC; ++c) S[e][c] = Snext[e][c];
            }
        }
        __syncthreads();
        buf ^= 1;
        it = nx;
    }

    if (p.ds0) store_block(p.ds0 + bh * NN, G);
}

template <int N, typename TIn>
hipError_t launch_bwd_t(const BwdLaunch &a, hipStream_t stream)
{
    BwdArgs<TIn> p;
    for (int i = 0; i < 7; ++i) p.in.p[i] = static_cast<const TIn *>(a.in[i]);
    p.ckpt = a.ckpt;
    p.dsT = a.dsT;
    p.dr = a.grad[0];
    p.dw = a.grad[1];
    p.dk = a.grad[2];
    p.dv = a.grad[3];
    p.da = a.grad[4];
    p.db = a.grad[5];
    p.ds0 = a.ds0;
    p.sub = a.sub;
    p.T = a.T;
    p.H = a.H;
    p.chunk = a.chunk;
    p.nck = (int)((a.T + a.chunk - 1) / a.chunk);
    p.nsubw = a.chunk / kSubChunk - 1;
    const dim3 grid((unsigned)(a.B * a.H)), block(BwdGeom<N>::NT);
    hipLaunchKernelGGL((wkv7_bwd_kernel<N, TIn>), grid, block, 0, stream, p);
    return hipGetLastError();
}

__global__ void fill_kernel(float *dst, const float *src, size_t n)
{
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}

}  // namespace

size_t sub_bytes(int64_t B, int64_t H, int64_t N, int chunk)
{
    const int64_t slots = chunk / kSubChunk - 1;
    return (size_t)(B * H * (slots > 0 ? slots : 0) * N * N) * sizeof(float);
}

hipError_t launch_backward(const BwdLaunch &a, hipStream_t stream)
{
    if (a.N == 64)
        return a.dtype == 0 ? launch_bwd_t<64, float>(a, stream)
                            : launch_bwd_t<64, uint16_t>(a, stream);
    return a.dtype == 0 ? launch_bwd_t<16, float>(a, stream)
                        : launch_bwd_t<16, uint16_t>(a, stream);
}

hipError_t launch_fill(float *dst, const float *src, size_t n, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, src, n);
    return hipGetLastError();
}

}  // namespace wkv7
