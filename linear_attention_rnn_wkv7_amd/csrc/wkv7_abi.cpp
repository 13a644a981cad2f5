// libwkv7 C ABI: argument validation, workspace layout and dispatch.
// Every check runs before anything is enqueued on the stream.

#include "wkv7.h"

#include <stdint.h>

#include <atomic>

#include "wkv7_internal.h"

namespace {

// Test hooks (wkv7_test_hook); zero in production.
std::atomic<int> g_fault_inject{0};
std::atomic<int64_t> g_fail_launches{0};

constexpr size_t kAlign = 256;   // workspace sub-buffer alignment

struct Dims {
    int64_t B, T, H, N, C, nck;
    int dtype, algo, fused;
    int nseg, nckseg;                // sequence split (nseg = 1: none)
    size_t vec_elems, state_elems;   // per tensor
};

// Few, long sequences run in segments so that more workgroups than (b, h)
// pairs fill the device: up to 8 segments of at least 2 chunks, while there
// are at most 64 (b, h).  Needs the chunk forms (N = 64, C = 64).  Depends on
// the shape only, so the forward's checkpoint record and the backward agree.
void plan_split(Dims *d)
{
    d->nseg = 1;
    d->nckseg = (int)d->nck;
    const int64_t units = d->B * d->H;
    if (d->N != 64 || d->C != 64 || d->T <= 1 || units == 0 || units > 64 ||
        !wkv7::chunk_offsets_fit(d->T, d->H))
        return;
    int64_t nseg = 256 / units;
    if (nseg > 8) nseg = 8;
    if (nseg > d->nck / 2) nseg = d->nck / 2;
    if (nseg < 2) return;
    const int64_t per = (d->nck + nseg - 1) / nseg;
    nseg = (d->nck + per - 1) / per;   // no empty segment
    if (nseg < 2) return;
    d->nseg = (int)nseg;
    d->nckseg = (int)per;
}

bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    return !__builtin_mul_overflow(a, b, out);
}

int check_shape(const wkv7_shape *s, Dims *d)
{
    if (!s) return WKV7_ERR_INVALID;
    if (s->B < 0 || s->T < 0 || s->H < 0 || s->N <= 0) return WKV7_ERR_INVALID;
    if (s->dtype != WKV7_F32 && s->dtype != WKV7_BF16) return WKV7_ERR_INVALID;
    if (s->algo < WKV7_ALGO_AUTO || s->algo > WKV7_ALGO_CHUNKED || (s->flags & ~WKV7_FUSED_INPUTS) != 0)
        return WKV7_ERR_INVALID;
    const int64_t C = s->chunk == 0 ? 64 : s->chunk;
    if (C < 8 || C > 4096 || C % 8 != 0) return WKV7_ERR_INVALID;
    if (s->N != 16 && s->N != 64) return WKV7_ERR_UNSUPPORTED;
    int64_t bh, bth, vec, st, nck_elems, bytes;
    if (!mul_ok(s->B, s->H, &bh) || bh > INT32_MAX) return WKV7_ERR_INVALID;
    if (!mul_ok(bh, s->T, &bth) || !mul_ok(bth, s->N, &vec)) return WKV7_ERR_INVALID;
    if (!mul_ok(vec, 4, &bytes)) return WKV7_ERR_INVALID;
    if (!mul_ok(bh, s->N * s->N, &st)) return WKV7_ERR_INVALID;
    const int64_t nck = (s->T + C - 1) / C;
    if (nck > INT32_MAX) return WKV7_ERR_INVALID;
    if (!mul_ok(st, nck, &nck_elems) || !mul_ok(nck_elems, 4, &bytes)) return WKV7_ERR_INVALID;
    d->B = s->B;
    d->T = s->T;
    d->H = s->H;
    d->N = s->N;
    d->C = C;
    d->nck = nck;
    d->dtype = s->dtype;
    d->algo = s->algo;
    d->fused = (s->flags & WKV7_FUSED_INPUTS) != 0;
    d->vec_elems = (size_t)vec;
    d->state_elems = (size_t)st;
    plan_split(d);
    return WKV7_OK;
}

// Fused inputs run in the chunk forms (and the single-step kernel): N = 64,
// C = 64, 32-bit offsets within a batch row; not with the step scan.
bool fused_supported(const Dims &d)
{
    return d.N == 64 && d.C == 64 && d.algo != WKV7_ALGO_SCAN &&
           (d.T <= 1 || wkv7::chunk_offsets_fit(d.T, d.H));
}

bool aligned(const void *p)
{
    return ((uintptr_t)p & 15u) == 0;
}

size_t round_up(size_t x)
{
    return (x + kAlign - 1) / kAlign * kAlign;
}

// The checkpoint record: the states every C steps, then (at a 256-byte
// aligned offset) the per-step sa values in the vector layout.
size_t ckpt_state_bytes(const Dims &d)
{
    return d.state_elems * (size_t)d.nck * sizeof(float);
}

// A split sequence's record also holds the segments' transition products,
// after the tape: [B*H][nseg][N][N] fp32.
size_t ckpt_split_bytes(const Dims &d)
{
    return d.nseg > 1 ? (size_t)(d.B * d.H) * d.nseg * d.N * d.N * sizeof(float) : 0;
}

size_t ckpt_bytes(const Dims &d)
{
    const size_t tape = d.vec_elems * sizeof(float);
    if (d.nseg > 1) return round_up(ckpt_state_bytes(d)) + round_up(tape) + ckpt_split_bytes(d);
    return round_up(ckpt_state_bytes(d)) + tape;
}

float *pbuf_of(const float *ck, const Dims &d)
{
    return reinterpret_cast<float *>(const_cast<char *>(reinterpret_cast<const char *>(ck)) +
                                     round_up(ckpt_state_bytes(d)) +
                                     round_up(d.vec_elems * sizeof(float)));
}

const float *tape_of(const float *ck, const Dims &d)
{
    return reinterpret_cast<const float *>(reinterpret_cast<const char *>(ck) +
                                           round_up(ckpt_state_bytes(d)));
}

// Sub-checkpoint scratch first, then the per-head flags of the chunk form,
// then (when needed) the checkpoints.
size_t sub_region(const Dims &d)
{
    return round_up(wkv7::sub_bytes(d.B, d.H, d.N, (int)d.C));
}

size_t flag_region(const Dims &d)
{
    return round_up((size_t)(d.B * d.H) * sizeof(int));
}

// split sequences: per-segment flags, then the state gradients at segment
// starts ([B*H][nseg][N][N] fp32)
size_t split_region(const Dims &d)
{
    if (d.nseg < 2) return 0;
    return round_up((size_t)(d.B * d.H) * d.nseg * sizeof(int)) +
           round_up((size_t)(d.B * d.H) * d.nseg * d.N * d.N * sizeof(float));
}

size_t workspace_bytes(const Dims &d, bool ckpt_provided)
{
    size_t n = sub_region(d) + flag_region(d) + split_region(d);
    if (!ckpt_provided) n += round_up(ckpt_bytes(d));
    return n;
}

int hip_status(hipError_t e)
{
    if (e != hipSuccess) return WKV7_ERR_HIP;
    int64_t n = g_fail_launches.load();
    while (n > 0 && !g_fail_launches.compare_exchange_weak(n, n - 1)) {
    }
    return n > 0 ? WKV7_ERR_HIP : WKV7_OK;
}

}  // namespace

namespace wkv7 {

int test_fault_inject()
{
    return g_fault_inject.load();
}

int backward_entry(const wkv7_shape *shape, const void *r, const void *w, const void *k,
                   const void *v, const void *a, const void *b, const float *s0,
                   const void *dy, const float *dsT, const float *ckpt,
                   float *dr, float *dw, float *dk, float *dv, float *da, float *db,
                   float *ds0, void *workspace, size_t workspace_bytes_given,
                   int (*scratch)(size_t need, void **ptr), hipStream_t stream)
{
    Dims d;
    int rc = check_shape(shape, &d);
    if (rc != WKV7_OK) return rc;
    if (d.B * d.H == 0) return WKV7_OK;
    const void *in[7] = {r, w, k, v, a, b, dy};
    float *grad[6] = {dr, dw, dk, dv, da, db};
    for (const void *p : in) {
        if (d.T > 0 && !p) return WKV7_ERR_INVALID;
        if (!aligned(p)) return WKV7_ERR_INVALID;
    }
    for (float *p : grad) {
        if (d.T > 0 && !p) return WKV7_ERR_INVALID;
        if (!aligned(p)) return WKV7_ERR_INVALID;
    }
    for (const void *p : {(const void *)s0, (const void *)dsT, (const void *)ckpt,
                          (const void *)ds0})
        if (!aligned(p)) return WKV7_ERR_INVALID;

    if (d.algo == WKV7_ALGO_CHUNKED &&
        !(d.N == 64 && d.C == 64 && (d.T == 0 || wkv7::chunk_offsets_fit(d.T, d.H))))
        return WKV7_ERR_UNSUPPORTED;
    if (d.fused && !fused_supported(d)) return WKV7_ERR_UNSUPPORTED;
    if (d.T == 0) {
        if (!ds0) return WKV7_OK;
        return hip_status(wkv7::launch_fill(ds0, dsT, d.state_elems, stream));
    }
    const size_t need = workspace_bytes(d, ckpt != nullptr);
    if (scratch) {   // no caller workspace: the library's own scratch
        rc = scratch(need, &workspace);
        if (rc != WKV7_OK) return rc;
        workspace_bytes_given = need;
    }
    if (need > 0 && (!workspace || workspace_bytes_given < need)) return WKV7_ERR_WORKSPACE;
    if (((uintptr_t)workspace % kAlign) != 0) return WKV7_ERR_WORKSPACE;

    char *ws = static_cast<char *>(workspace);
    float *sub = reinterpret_cast<float *>(ws);
    const float *ck = ckpt;
    if (!ckpt) {
        float *own = reinterpret_cast<float *>(ws + sub_region(d) + flag_region(d) + split_region(d));
        wkv7::FwdLaunch F;
        for (int i = 0; i < 6; ++i) F.in[i] = in[i];
        F.s0 = s0;
        F.y = nullptr;
        F.sT = nullptr;
        F.ckpt = own;
        F.satape = const_cast<float *>(tape_of(own, d));
        F.B = d.B;
        F.T = d.T;
        F.H = d.H;
        F.N = d.N;
        F.dtype = d.dtype;
        F.chunk = (int)d.C;
        F.fused = d.fused;
        if (d.nseg > 1) {
            F.nseg = d.nseg;
            F.nckseg = d.nckseg;
            F.pbuf = pbuf_of(own, d);
        }
        rc = hip_status(wkv7::launch_forward(F, stream));
        if (rc != WKV7_OK) return rc;
        ck = own;
    }
    wkv7::BwdLaunch L;
    for (int i = 0; i < 7; ++i) L.in[i] = in[i];
    L.ckpt = ck;
    L.satape = tape_of(ck, d);
    L.dsT = dsT;
    for (int i = 0; i < 6; ++i) L.grad[i] = grad[i];
    L.ds0 = ds0;
    L.sub = sub;
    L.flags = reinterpret_cast<int *>(ws + sub_region(d));
    L.B = d.B;
    L.T = d.T;
    L.H = d.H;
    L.N = d.N;
    L.dtype = d.dtype;
    L.chunk = (int)d.C;
    L.algo = d.algo;
    L.fused = d.fused;
    if (d.nseg > 1) {
        char *sp = ws + sub_region(d) + flag_region(d);
        L.nseg = d.nseg;
        L.nckseg = d.nckseg;
        L.pbuf = pbuf_of(ck, d);
        L.unit_flags = reinterpret_cast<int *>(sp);
        L.gbuf = reinterpret_cast<float *>(sp + round_up((size_t)(d.B * d.H) * d.nseg * sizeof(int)));
    }
    return hip_status(wkv7::launch_backward(L, stream));
}

}  // namespace wkv7

extern "C" {

size_t wkv7_checkpoint_bytes(const wkv7_shape *shape)
{
    Dims d;
    if (check_shape(shape, &d) != WKV7_OK) return 0;
    return ckpt_bytes(d);
}

size_t wkv7_backward_workspace_bytes(const wkv7_shape *shape, int ckpt_provided)
{
    Dims d;
    if (check_shape(shape, &d) != WKV7_OK || d.B * d.H == 0 || d.T == 0) return 0;
    return workspace_bytes(d, ckpt_provided != 0);
}

int wkv7_forward(const wkv7_shape *shape, const void *r, const void *w, const void *k,
                 const void *v, const void *a, const void *b, const float *s0,
                 float *y, float *sT, float *ckpt, hipStream_t stream)
{
    Dims d;
    int rc = check_shape(shape, &d);
    if (rc != WKV7_OK) return rc;
    if (d.B * d.H == 0) return WKV7_OK;
    const void *in[6] = {r, w, k, v, a, b};
    for (const void *p : in) {
        if (d.T > 0 && !p) return WKV7_ERR_INVALID;
        if (!aligned(p)) return WKV7_ERR_INVALID;
    }
    for (const void *p : {(const void *)s0, (const void *)y, (const void *)sT, (const void *)ckpt})
        if (!aligned(p)) return WKV7_ERR_INVALID;
    if (d.fused && !fused_supported(d)) return WKV7_ERR_UNSUPPORTED;

    if (d.T == 0) {
        if (!sT) return WKV7_OK;
        return hip_status(wkv7::launch_fill(sT, s0, d.state_elems, stream));
    }
    wkv7::FwdLaunch L;
    for (int i = 0; i < 6; ++i) L.in[i] = in[i];
    L.s0 = s0;
    L.y = y;
    L.sT = sT;
    L.ckpt = ckpt;
    L.satape = ckpt ? const_cast<float *>(tape_of(ckpt, d)) : nullptr;
    L.B = d.B;
    L.T = d.T;
    L.H = d.H;
    L.N = d.N;
    L.dtype = d.dtype;
    L.chunk = (int)d.C;
    L.fused = d.fused;
    if (ckpt && d.nseg > 1) {   // the record holds the split's scratch
        L.nseg = d.nseg;
        L.nckseg = d.nckseg;
        L.pbuf = pbuf_of(ckpt, d);
    } else if (!ckpt && y && d.nseg > 1) {
        // no record: the carries go into the segments' own rows of y (a
        // state takes N steps of a (b, h), a carry and a transition product
        // 2N, which segments of at least 2 chunks hold; the last segment
        // needs N steps, else the forward runs whole)
        if ((int64_t)d.nckseg * d.C >= 2 * d.N && d.T - (int64_t)(d.nseg - 1) * d.nckseg * d.C >= d.N) {
            L.nseg = d.nseg;
            L.nckseg = d.nckseg;
        }
    }
    return hip_status(wkv7::launch_forward(L, stream));
}

int wkv7_backward(const wkv7_shape *shape, const void *r, const void *w, const void *k,
                  const void *v, const void *a, const void *b, const float *s0,
                  const void *dy, const float *dsT, const float *ckpt,
                  float *dr, float *dw, float *dk, float *dv, float *da, float *db,
                  float *ds0, void *workspace, size_t workspace_bytes_given,
                  hipStream_t stream)
{
    return wkv7::backward_entry(shape, r, w, k, v, a, b, s0, dy, dsT, ckpt, dr, dw, dk, dv, da, db,
                                ds0, workspace, workspace_bytes_given, nullptr, stream);
}

size_t wkv7_epilogue_workspace_bytes(const wkv7_shape *shape)
{
    Dims d;
    if (check_shape(shape, &d) != WKV7_OK || d.N != 64 || d.B * d.T * d.H == 0) return 0;
    return round_up((size_t)d.H * wkv7::epilogue_chunks(d.B * d.T, d.H) * 3 * 64 * sizeof(float));
}

int wkv7_epilogue_forward(const wkv7_shape *shape, const float *y, const void *r, const void *k,
                          const void *v, const void *g, const float *ln_w, const float *ln_b,
                          const float *r_k, float *z, hipStream_t stream)
{
    Dims d;
    int rc = check_shape(shape, &d);
    if (rc != WKV7_OK) return rc;
    if (d.N != 64) return WKV7_ERR_UNSUPPORTED;
    if (d.B * d.T * d.H == 0) return WKV7_OK;
    for (const void *p : {(const void *)y, r, k, v, g, (const void *)ln_w, (const void *)ln_b,
                          (const void *)r_k, (const void *)z})
        if (!p || !aligned(p)) return WKV7_ERR_INVALID;
    wkv7::EpiLaunch L;
    L.y = y;
    L.r = r;
    L.k = k;
    L.v = v;
    L.g = g;
    L.ln_w = ln_w;
    L.ln_b = ln_b;
    L.r_k = r_k;
    L.z = z;
    L.BT = d.B * d.T;
    L.H = d.H;
    L.dtype = d.dtype;
    return hip_status(wkv7::launch_epilogue_forward(L, stream));
}

int wkv7_epilogue_backward(const wkv7_shape *shape, const float *dz, const float *y, const void *r,
                           const void *k, const void *v, const void *g, const float *ln_w,
                           const float *ln_b, const float *r_k, float *dy, float *dg, float *dr,
                           float *dk, float *dv, float *dln_w, float *dln_b, float *dr_k,
                           void *workspace, size_t workspace_bytes_given, hipStream_t stream)
{
    Dims d;
    int rc = check_shape(shape, &d);
    if (rc != WKV7_OK) return rc;
    if (d.N != 64) return WKV7_ERR_UNSUPPORTED;
    if (d.H == 0) return WKV7_OK;
    for (const void *p : {(const void *)ln_w, (const void *)ln_b, (const void *)r_k, (const void *)dln_w,
                          (const void *)dln_b, (const void *)dr_k})
        if (!p || !aligned(p)) return WKV7_ERR_INVALID;
    if (d.B * d.T == 0) {   // no rows: the parameter gradients are zero
        for (float *p : {dln_w, dln_b, dr_k}) {
            rc = hip_status(wkv7::launch_fill(p, nullptr, (size_t)d.H * 64, stream));
            if (rc != WKV7_OK) return rc;
        }
        return WKV7_OK;
    }
    for (const void *p : {(const void *)dz, (const void *)y, r, k, v, g, (const void *)dy,
                          (const void *)dg, (const void *)dr, (const void *)dk, (const void *)dv})
        if (!p || !aligned(p)) return WKV7_ERR_INVALID;
    const int nchunk = wkv7::epilogue_chunks(d.B * d.T, d.H);
    const size_t need = round_up((size_t)d.H * nchunk * 3 * 64 * sizeof(float));
    if (!workspace || workspace_bytes_given < need || ((uintptr_t)workspace % kAlign) != 0)
        return WKV7_ERR_WORKSPACE;
    wkv7::EpiLaunch L;
    L.y = y;
    L.dz = dz;
    L.r = r;
    L.k = k;
    L.v = v;
    L.g = g;
    L.ln_w = ln_w;
    L.ln_b = ln_b;
    L.r_k = r_k;
    L.dy = dy;
    L.dg = dg;
    L.dr = dr;
    L.dk = dk;
    L.dv = dv;
    L.dln_w = dln_w;
    L.dln_b = dln_b;
    L.dr_k = dr_k;
    L.part = static_cast<float *>(workspace);
    L.BT = d.B * d.T;
    L.H = d.H;
    L.dtype = d.dtype;
    L.nchunk = nchunk;
    return hip_status(wkv7::launch_epilogue_backward(L, stream));
}

int wkv7_fault_status(unsigned *faults, int clear, hipStream_t stream)
{
    if (!faults) return WKV7_ERR_INVALID;
    unsigned *word = wkv7::fault_word();
    if (!word) return WKV7_ERR_HIP;
    static const unsigned zero = 0;
    unsigned host = 0;
    if (hipMemcpyAsync(&host, word, sizeof host, hipMemcpyDeviceToHost, stream) != hipSuccess)
        return WKV7_ERR_HIP;
    if (clear && hipMemcpyAsync(word, &zero, sizeof zero, hipMemcpyHostToDevice, stream) != hipSuccess)
        return WKV7_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return WKV7_ERR_HIP;
    *faults = host;
    return WKV7_OK;
}

int wkv7_test_hook(int hook, int64_t value)
{
    switch (hook) {
    case WKV7_HOOK_FAULT_INJECT:
        if (value != 0 && value != 1) return WKV7_ERR_INVALID;
        g_fault_inject.store((int)value);
        return WKV7_OK;
    case WKV7_HOOK_FAIL_LAUNCHES:
        if (value < 0) return WKV7_ERR_INVALID;
        g_fail_launches.store(value);
        return WKV7_OK;
    default:
        return WKV7_ERR_INVALID;
    }
}

const char *wkv7_status_string(int status)
{
    switch (status) {
    case WKV7_OK: return "ok";
    case WKV7_ERR_INVALID: return "invalid argument";
    case WKV7_ERR_UNSUPPORTED:
        return "unsupported: head size not 16 or 64, or a requested form (chunked, fused inputs) "
               "that does not apply to this shape";
    case WKV7_ERR_WORKSPACE: return "workspace missing or too small";
    case WKV7_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

int wkv7_abi_version(void)
{
    return 105;
}

}  // extern "C"
