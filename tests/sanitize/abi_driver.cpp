// Host-only driver for the C ABI's validation and buffer layout, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize_cpu.py).
// The kernel launchers are replaced by stubs that record what they were
// given; the driver checks every status and that every buffer the ABI hands
// a kernel lies inside the sizes the ABI itself reports.  No GPU is used.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "wkv7.h"
#include "wkv7_internal.h"

namespace {
int g_fails = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            std::fprintf(stderr, "CHECK failed line %d: %s\n", __LINE__, #c); \
            ++g_fails;                                                        \
        }                                                                     \
    } while (0)

std::vector<wkv7::FwdLaunch> g_fwd;
std::vector<wkv7::BwdLaunch> g_bwd;
unsigned g_word;

// a span [p, p + n) lies in [base, base + size)
bool inside(const void *p, size_t n, const void *base, size_t size)
{
    const char *a = static_cast<const char *>(p), *b = static_cast<const char *>(base);
    return a >= b && a + n <= b + size;
}
}  // namespace

// ---- stubs of the device side (the sizes follow the kernels' own rules)
namespace wkv7 {
hipError_t launch_fill(float *, const float *, size_t, hipStream_t) { return hipSuccess; }
hipError_t launch_forward(const FwdLaunch &a, hipStream_t) { g_fwd.push_back(a); return hipSuccess; }
hipError_t launch_backward(const BwdLaunch &a, hipStream_t) { g_bwd.push_back(a); return hipSuccess; }
hipError_t launch_epilogue_forward(const EpiLaunch &, hipStream_t) { return hipSuccess; }
hipError_t launch_epilogue_backward(const EpiLaunch &, hipStream_t) { return hipSuccess; }
int epilogue_chunks(int64_t BT, int64_t H) { (void)H; return (int)(BT < 64 ? 1 : 64); }
size_t sub_bytes(int64_t B, int64_t H, int64_t N, int chunk)
{
    const int64_t slots = chunk / kSubChunk - 1;
    return (size_t)(B * H * (slots > 0 ? slots : 0) * N * N) * sizeof(float);
}
unsigned *fault_word() { return &g_word; }
}  // namespace wkv7
extern "C" hipError_t hipMemcpyAsync(void *, const void *, size_t, hipMemcpyKind, hipStream_t)
{
    return hipSuccess;
}
extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

static void *fake(size_t off = 0) { return reinterpret_cast<void *>(uintptr_t(0x100000) + off); }

static void check_shape(int64_t B, int64_t T, int64_t H, int64_t N, int chunk, int dtype)
{
    wkv7_shape s{B, T, H, N, dtype, chunk, 0, 0};
    const size_t ck = wkv7_checkpoint_bytes(&s);
    CHECK(ck > 0);
    const void *in = fake();
    float *y = (float *)fake(1 << 20), *ckp = (float *)fake(64 << 20);
    g_fwd.clear();
    CHECK(wkv7_forward(&s, in, in, in, in, in, in, nullptr, y, nullptr, ckp, nullptr) == WKV7_OK);
    CHECK(g_fwd.size() == 1);
    if (!g_fwd.empty()) {
        const auto &L = g_fwd[0];
        const size_t tape = (size_t)(B * T * H * N) * 4;
        CHECK(inside(L.satape, tape, ckp, ck));
        if (L.nseg > 1) CHECK(inside(L.pbuf, (size_t)(B * H * L.nseg * N * N) * 4, ckp, ck));
    }
    for (int prov = 0; prov < 2; ++prov) {
        const size_t ws = wkv7_backward_workspace_bytes(&s, prov);
        CHECK(ws > 0);
        char *w = (char *)fake(1 << 30);
        float *g = (float *)fake(2 << 20);
        g_fwd.clear();
        g_bwd.clear();
        CHECK(wkv7_backward(&s, in, in, in, in, in, in, nullptr, in, nullptr, prov ? ckp : nullptr, g, g, g,
                            g, g, g, nullptr, w, ws, nullptr) == WKV7_OK);
        CHECK(wkv7_backward(&s, in, in, in, in, in, in, nullptr, in, nullptr, prov ? ckp : nullptr, g, g, g,
                            g, g, g, nullptr, w, ws - 1, nullptr) == WKV7_ERR_WORKSPACE);
        CHECK(g_bwd.size() == 1);
        if (g_bwd.empty()) continue;
        const auto &L = g_bwd[0];
        CHECK(inside(L.sub, wkv7::sub_bytes(B, H, N, chunk ? chunk : 64), w, ws));
        CHECK(inside(L.flags, (size_t)(B * H) * 4, w, ws));
        if (L.nseg > 1) {
            CHECK(inside(L.unit_flags, (size_t)(B * H * L.nseg) * 4, w, ws));
            CHECK(inside(L.gbuf, (size_t)(B * H * L.nseg * N * N) * 4, w, ws));
        }
        if (!prov) {
            CHECK(g_fwd.size() == 1);
            if (!g_fwd.empty()) {
                CHECK(inside(g_fwd[0].ckpt, ck, w, ws));
                CHECK(L.ckpt == g_fwd[0].ckpt);
            }
        }
    }
}

int main()
{
    // validation
    CHECK(wkv7_forward(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                       nullptr, nullptr) == WKV7_ERR_INVALID);
    wkv7_shape bad{2, 10, 3, 32, 0, 64, 0, 0};
    CHECK(wkv7_checkpoint_bytes(&bad) == 0);
    const void *in = fake();
    CHECK(wkv7_forward(&bad, in, in, in, in, in, in, nullptr, nullptr, nullptr, nullptr, nullptr) ==
          WKV7_ERR_UNSUPPORTED);
    wkv7_shape huge{int64_t(1) << 40, int64_t(1) << 30, 1, 64, 0, 64, 0, 0};
    CHECK(wkv7_forward(&huge, in, in, in, in, in, in, nullptr, nullptr, nullptr, nullptr, nullptr) ==
          WKV7_ERR_INVALID);
    wkv7_shape mis{2, 10, 3, 64, 0, 64, 0, 0};
    CHECK(wkv7_forward(&mis, fake(4), in, in, in, in, in, nullptr, nullptr, nullptr, nullptr, nullptr) ==
          WKV7_ERR_INVALID);
    // a sweep of shapes, chunk intervals and dtypes
    const int64_t Bs[] = {1, 2, 3, 8}, Ts[] = {1, 2, 63, 64, 65, 130, 512, 4097}, Hs[] = {1, 2, 5, 32};
    const int Cs[] = {8, 24, 64, 128}, Ns[] = {16, 64};
    for (int64_t B : Bs)
        for (int64_t T : Ts)
            for (int64_t H : Hs)
                for (int N : Ns)
                    for (int C : Cs)
                        for (int dt = 0; dt < 2; ++dt) check_shape(B, T, H, N, C, dt);
    // test hooks
    CHECK(wkv7_test_hook(WKV7_HOOK_FAIL_LAUNCHES, 1) == WKV7_OK);
    wkv7_shape s{1, 5, 2, 64, 0, 64, 0, 0};
    CHECK(wkv7_forward(&s, in, in, in, in, in, in, nullptr, (float *)fake(), nullptr, nullptr, nullptr) ==
          WKV7_ERR_HIP);
    CHECK(wkv7_forward(&s, in, in, in, in, in, in, nullptr, (float *)fake(), nullptr, nullptr, nullptr) ==
          WKV7_OK);
    unsigned f = 7;
    CHECK(wkv7_fault_status(&f, 1, nullptr) == WKV7_OK);
    CHECK(wkv7_fault_status(nullptr, 1, nullptr) == WKV7_ERR_INVALID);
    // epilogue
    const size_t ew = wkv7_epilogue_workspace_bytes(&s);
    CHECK(ew > 0);
    float *p = (float *)fake();
    CHECK(wkv7_epilogue_backward(&s, p, p, in, in, in, in, p, p, p, p, p, p, p, p, p, p, p, fake(1 << 20), ew,
                                 nullptr) == WKV7_OK);
    CHECK(wkv7_epilogue_backward(&s, p, p, in, in, in, in, p, p, p, p, p, p, p, p, p, p, p, fake(1 << 20),
                                 ew - 1, nullptr) == WKV7_ERR_WORKSPACE);
    for (int st : {0, -1, -2, -3, -4, 9}) CHECK(wkv7_status_string(st) != nullptr);
    std::printf("abi driver: %d failures\n", g_fails);
    return g_fails == 0 ? 0 : 1;
}
