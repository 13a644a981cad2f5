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
    VecPtrs<float, 1> satape;   // the forward's per-step sa, [B][T][H][N]
    const float *ckpt, *dsT;
    float *dr, *dw, *dk, *dv, *da, *db, *ds0;
    float *sub;
    const int *only;         // if set, only heads with only[bh] != 0 run
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
    constexpr int kSA = NV;            // extra LDS slot: sa per step (from the tape)
    // stg[buf][vector][step][n]: the 7 staged inputs plus sa
    __shared__ __align__(16) float stg[2][NV + 1][KS][N];
    // per-wave column sums and dv of a pass-B item, double-buffered: item i
    // writes buffer pb, the next item sums and stores it behind the barrier
    // that ends item i
    __shared__ __align__(16) float part[2][KS][NQ][NW][N];
    __shared__ __align__(16) float dvb[2][KS][N];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = lane % LPR, rg = lane / LPR;
    const int row0 = wave * RW + rg * R, col0 = cg * CC;
    const int64_t bh = blockIdx.x, T = p.T, H = p.H;
    if (p.only && p.only[bh] == 0) return;   // uniform over the workgroup
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
        if constexpr (R == 4) {
            const float4 v4 = *reinterpret_cast<const float4 *>(Ls + q * KS * N + row0);
            x[0] = v4.x; x[1] = v4.y; x[2] = v4.z; x[3] = v4.w;
        } else {
#pragma unroll
            for (int e = 0; e < R; ++e) x[e] = Ls[q * KS * N + row0 + e];
        }
    };
    auto row_store = [&](float *dst, const float (&x)[R]) {
        // every lane of the row group writes the same values (no branch)
        if constexpr (R == 4)
            *reinterpret_cast<float4 *>(dst + row0) = make_float4(x[0], x[1], x[2], x[3]);
        else
#pragma unroll
            for (int e = 0; e < R; ++e) dst[row0 + e] = x[e];
    };

    // ---- forward replay of one step, with sa taken from the forward's tape:
    // X <- X diag(w) + v k^T + sa b^T in place
    struct FwdVals {
        float w[CC], k[CC], b[CC], v[R], sa[R];
    };
    auto load_fwd = [&](const float *Ls, FwdVals &x) {
        col_vals(Ls, kW, x.w);
        col_vals(Ls, kK, x.k);
        col_vals(Ls, kB, x.b);
        row_vals(Ls, kV, x.v);
        row_vals(Ls, kSA, x.sa);
    };
    auto fwd_step = [&](const FwdVals &x, float (&X)[R][CC]) {
#pragma unroll
        for (int e = 0; e < R; ++e)
#pragma unroll
            for (int c = 0; c < CC; ++c)
                X[e][c] = fmaf(x.sa[e], x.b[c], fmaf(X[e][c], x.w[c], x.v[e] * x.k[c]));
    };

    // ---- one reverse step
    struct RevVals {
        float r[CC], w[CC], k[CC], a[CC], b[CC], v[R], dy[R], sa[R];
    };
    auto load_rev = [&](const float *Ls, RevVals &x) {
        col_vals(Ls, kR, x.r);
        col_vals(Ls, kW, x.w);
        col_vals(Ls, kK, x.k);
        col_vals(Ls, kA, x.a);
        col_vals(Ls, kB, x.b);
        row_vals(Ls, kV, x.v);
        row_vals(Ls, kDY, x.dy);
        row_vals(Ls, kSA, x.sa);
    };
    float G[R][CC];
    // Pj: state before step j; Pn: state after it.  Leaves the column
    // partials in part[j] and dv in dvb[j]; carries G to step j-1.
    auto rev_step = [&](int j, int pb, const RevVals &x, const float (&Pj)[R][CC],
                        const float (&Pn)[R][CC]) {
        float cq[NQ][CC];
        // read-out: G += dy r^T; dr from the post-step state
#pragma unroll
        for (int c = 0; c < CC; ++c) {
            float pdr = 0.f;
#pragma unroll
            for (int e = 0; e < R; ++e) {
                pdr = fmaf(Pn[e][c], x.dy[e], pdr);
                G[e][c] = fmaf(x.dy[e], x.r[c], G[e][c]);
            }
            cq[qDR][c] = pdr;
        }
        // row dots dsa = G b (needed for the carry) and dv = G k
        float dsa[R], dvv[R];
#pragma unroll
        for (int e = 0; e < R; ++e) {
            float s0 = 0.f, s1 = 0.f, v0 = 0.f, v1 = 0.f;
#pragma unroll
            for (int c = 0; c < CC; c += 2) {
                s0 = fmaf(G[e][c], x.b[c], s0);
                s1 = fmaf(G[e][c + 1], x.b[c + 1], s1);
                v0 = fmaf(G[e][c], x.k[c], v0);
                v1 = fmaf(G[e][c + 1], x.k[c + 1], v1);
            }
            dsa[e] = s0 + s1;
            dvv[e] = v0 + v1;
        }
#pragma unroll
        for (int e = 0; e < R; ++e) dsa[e] = group_allreduce<LPR>(dsa[e]);
        // column partials that do not need dsa, and the carry's G*w part
        float gw[R][CC];
#pragma unroll
        for (int c = 0; c < CC; ++c) {
            float xk = 0.f, xb = 0.f, xw = 0.f;
#pragma unroll
            for (int e = 0; e < R; ++e) {
                xk = fmaf(G[e][c], x.v[e], xk);
                xb = fmaf(G[e][c], x.sa[e], xb);
                xw = fmaf(G[e][c], Pj[e][c], xw);
                gw[e][c] = G[e][c] * x.w[c];
            }
            cq[qDK][c] = xk;
            cq[qDB][c] = xb;
            cq[qDW][c] = xw;
        }
#pragma unroll
        for (int e = 0; e < R; ++e) dvv[e] = group_allreduce<LPR>(dvv[e]);
        // in-context term and carry to t-1: G <- G diag(w) + dsa a^T
#pragma unroll
        for (int c = 0; c < CC; ++c) {
            float xa = 0.f;
#pragma unroll
            for (int e = 0; e < R; ++e) {
                xa = fmaf(dsa[e], Pj[e][c], xa);
                G[e][c] = fmaf(dsa[e], x.a[c], gw[e][c]);
            }
            cq[qDA][c] = xa;
        }
        // column sums across the row groups of the wave
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const float u0 = swap_add32(cq[q][0], cq[q][2]);
            const float u1 = swap_add32(cq[q][1], cq[q][3]);
            float xs = swap_add16(u0, u1);
            if constexpr (LPR <= 8) xs += dpp<kDppRor8>(xs);
            if constexpr (LPR <= 4) xs += dpp<kDppRor4>(xs);
            if (cwriter) part[pb][j][q][wave][ccol] = xs;
        }
        row_store(&dvb[pb][j][0], dvv);
    };

    // ---- outputs of a pass-B item: the column sums (fixed-order sum over
    // waves) and dv, from LDS buffer fb, for steps [ftb, ftb + fnst)
    auto finalize = [&](int fb, int64_t ftb, int fnst) {
        // Unit f covers 4 columns of one (quantity, step) pair; for N = 64
        // a wave's 64 units span 4 pairs of one quantity.
        constexpr int kU = (NQ + 1) * KS * (N / 4);
#pragma unroll
        for (int k = 0; k < (kU + NT - 1) / NT; ++k) {
            const int f = tid + k * NT;
            const int pair = f / (N / 4), c4 = f % (N / 4);
            int q = pair / KS;
            const int j = pair % KS;
            if constexpr (N / 4 * KS % kWave == 0) q = __builtin_amdgcn_readfirstlane(q);
            if (f < kU && j < fnst) {
                float4 xo;
                if (q == NQ) {
                    xo = *reinterpret_cast<const float4 *>(&dvb[fb][j][4 * c4]);
                } else {
                    xo = *reinterpret_cast<const float4 *>(&part[fb][j][q][0][4 * c4]);
#pragma unroll
                    for (int w = 1; w < NW; ++w) {
                        const float4 t = *reinterpret_cast<const float4 *>(&part[fb][j][q][w][4 * c4]);
                        xo.x += t.x; xo.y += t.y; xo.z += t.z; xo.w += t.w;
                    }
                }
                float *dst = q == qDR ? p.dr : q == qDK ? p.dk : q == qDB ? p.db
                           : q == qDW ? p.dw : q == qDA ? p.da : p.dv;
                *reinterpret_cast<float4 *>(dst + vbase + (ftb + j) * stride + 4 * c4) = xo;
            }
        }
    };
    bool fin_pending = false;
    int fin_buf = 0, fin_nst = 0, pb = 0;
    int64_t fin_tb = 0;

    // ---- seed G with dsT
    if (p.dsT) {
        load_block(p.dsT + bh * NN, G);
    } else {
#pragma unroll
        for (int e = 0; e < R; ++e)
#pragma unroll
            for (int c = 0; c < CC; ++c) G[e][c] = 0.f;
    }

    // inputs each item needs: pass A replays with w, k, v, b (+ sa); pass B
    // also needs r, a, dy
    constexpr unsigned kMaskA = (1u << kW) | (1u << kK) | (1u << kV) | (1u << kB);
    constexpr unsigned kMaskB = (1u << NV) - 1u;
    using StagerT = InputStager<TIn, NV, KS, N, NT>;
    StagerT stage;                          // inputs: DMA for fp32, registers for bf16
    DmaStager<1, KS, N, NT> sastage;        // the fp32 sa tape
    float S[R][CC], Snext[R][CC];
    Item it = first_of(p.nck - 1);
    {
        const unsigned m = it.B ? kMaskB : kMaskA;
        stage.issue(p.in, vbase + t_begin(it) * stride, stride, n_steps(it), wave, lane,
                    &stg[0][0][0][0], m);
        sastage.issue(p.satape, vbase + t_begin(it) * stride, stride, n_steps(it), wave, lane,
                      &stg[0][kSA][0][0]);
        load_block(state_src(it), S);
        stage.commit(&stg[0][0][0][0], n_steps(it), wave, lane, m);
        wait_dma();
    }
    __syncthreads();
    int buf = 0;

    while (it.c >= 0) {
        const Item nx = next_of(it);
        const bool have_next = nx.c >= 0;
        const bool nx_load = have_next && loads_state(nx);
        const unsigned nx_mask = nx.B ? kMaskB : kMaskA;
        if (have_next) {
            stage.issue(p.in, vbase + t_begin(nx) * stride, stride, n_steps(nx), wave, lane,
                        &stg[buf ^ 1][0][0][0], nx_mask);
            sastage.issue(p.satape, vbase + t_begin(nx) * stride, stride, n_steps(nx), wave, lane,
                          &stg[buf ^ 1][kSA][0][0]);
        }
        if (nx_load) load_block(state_src(nx), Snext);
        if (fin_pending) {
            finalize(fin_buf, fin_tb, fin_nst);
            fin_pending = false;
        }
        const float *L = &stg[buf][0][0][0];
        const int nst = n_steps(it);
        const int64_t tb = t_begin(it);

        if (!it.B) {
            // ---- pass A (always a full sub-chunk): replay KS steps, then
            // leave a sub-checkpoint when a later pass-B item starts there.
            FwdVals fv[2];
            load_fwd(L, fv[0]);
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                if (j + 1 < KS) load_fwd(L + (j + 1) * N, fv[(j + 1) & 1]);
                fwd_step(fv[j & 1], S);
            }
            if (it.s + 1 <= nsub_of(it.c) - 2)
                store_block(p.sub + (bh * p.nsubw + it.s) * NN, S);
        } else {
            // ---- pass B: regenerate the sub-chunk's KS + 1 states into
            // registers (sa of each step goes to its LDS slot) ...
            float P[KS + 1][R][CC];
#pragma unroll
            for (int e = 0; e < R; ++e)
#pragma unroll
                for (int c = 0; c < CC; ++c) P[0][e][c] = S[e][c];
            if (nst == KS) {
                FwdVals fv[2];
                load_fwd(L, fv[0]);
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                    if (j + 1 < KS) load_fwd(L + (j + 1) * N, fv[(j + 1) & 1]);
#pragma unroll
                    for (int e = 0; e < R; ++e)
#pragma unroll
                        for (int c = 0; c < CC; ++c) P[j + 1][e][c] = P[j][e][c];
                    fwd_step(fv[j & 1], P[j + 1]);
                }
                // ... then run the KS reverse steps on them
                RevVals rv[2];
                load_rev(L + (KS - 1) * N, rv[(KS - 1) & 1]);
#pragma unroll
                for (int j = KS - 1; j >= 0; --j) {
                    if (j > 0) load_rev(L + (j - 1) * N, rv[(j - 1) & 1]);
                    rev_step(j, pb, rv[j & 1], P[j], P[j + 1]);
                }
            } else {
                // tail of the sequence: fewer than KS steps
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                    if (j < nst) {
                        FwdVals fv;
                        load_fwd(L + j * N, fv);
#pragma unroll
                        for (int e = 0; e < R; ++e)
#pragma unroll
                            for (int c = 0; c < CC; ++c) P[j + 1][e][c] = P[j][e][c];
                        fwd_step(fv, P[j + 1]);
                    }
                }
#pragma unroll
                for (int j = KS - 1; j >= 0; --j) {
                    if (j < nst) {
                        RevVals rv;
                        load_rev(L + j * N, rv);
                        rev_step(j, pb, rv, P[j], P[j + 1]);
                    }
                }
            }
            fin_pending = true;
            fin_buf = pb;
            fin_tb = tb;
            fin_nst = nst;
            pb ^= 1;
        }

        if (have_next) {
            stage.commit(&stg[buf ^ 1][0][0][0], n_steps(nx), wave, lane, nx_mask);
            if (nx_load) {
#pragma unroll
                for (int e = 0; e < R; ++e)
#pragma unroll
                    for (int c = 0; c < CC; ++c) S[e][c] = Snext[e][c];
            }
        }
        wait_dma();
        __syncthreads();
        buf ^= 1;
        it = nx;
    }

    if (fin_pending) finalize(fin_buf, fin_tb, fin_nst);
    if (p.ds0) store_block(p.ds0 + bh * NN, G);
}

template <int N, typename TIn>
hipError_t launch_bwd_t(const BwdLaunch &a, const int *only, hipStream_t stream)
{
    BwdArgs<TIn> p;
    for (int i = 0; i < 7; ++i) p.in.p[i] = static_cast<const TIn *>(a.in[i]);
    p.ckpt = a.ckpt;
    p.satape.p[0] = a.satape;
    p.dsT = a.dsT;
    p.dr = a.grad[0];
    p.dw = a.grad[1];
    p.dk = a.grad[2];
    p.dv = a.grad[3];
    p.da = a.grad[4];
    p.db = a.grad[5];
    p.ds0 = a.ds0;
    p.sub = a.sub;
    p.only = only;
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
    const int *only = nullptr;
    const bool chunked = a.algo != 1 && chunked_backward_supported(a);
    if (a.fused && !chunked) return hipErrorInvalidValue;   // checked by the caller
    if (chunked && a.nseg > 1) {
        // a split sequence: the state gradients of the later segments from
        // their own terms alone, the carries, then every segment with its
        // incoming gradient; a head with any flagged segment is redone whole
        // below
        hipError_t e = launch_backward_chunked(a, a.unit_flags, 1, stream);
        if (e == hipSuccess) e = launch_compose_backward(a, stream);
        if (e == hipSuccess) e = launch_backward_chunked(a, a.unit_flags, 2, stream);
        if (e != hipSuccess || a.fused) return e;
        e = launch_flag_reduce(a.unit_flags, a.flags, a.B * a.H, a.nseg, stream);
        if (e != hipSuccess) return e;
        only = a.flags;
    } else if (chunked) {
        const hipError_t e = launch_backward_chunked(a, a.flags, 0, stream);
        // the decays formed from fused inputs lie in [exp(-exp(-0.5)), 1]:
        // the chunk form takes every head
        if (e != hipSuccess || a.fused) return e;
        only = a.flags;
    }
    if (a.N == 64)
        return a.dtype == 0 ? launch_bwd_t<64, float>(a, only, stream)
                            : launch_bwd_t<64, uint16_t>(a, only, stream);
    return a.dtype == 0 ? launch_bwd_t<16, float>(a, only, stream)
                        : launch_bwd_t<16, uint16_t>(a, only, stream);
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
