// Host sanitizer driver for the C ABI layer: every entry point of gtr_gla.h
// that validates before launching, with valid and invalid arguments, extreme
// sizes (the overflow checks run under UBSan), aliasing, workspace checks and
// the caller-workspace path (stand-in launches). Exits nonzero on any status
// other than the expected one.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "gtr_gla.h"

static int fails = 0;
static void expect(int got, int want, const char* what)
{
    if (got != want) {
        std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
        ++fails;
    }
}

int main()
{
    // fake, well separated device addresses (never dereferenced)
    auto P = [](int i) { return reinterpret_cast<void*>((uintptr_t)(1ull << 40) + (uintptr_t)i * (1ull << 32)); };
    void *q = P(0), *k = P(1), *v = P(2), *g = P(3), *o = P(4);
    float* fs = static_cast<float*>(P(5));
    void* ws = P(6);
    hipStream_t st = nullptr;
    const int dims[][6] = {{1, 2, 4, 4, 64, 64}, {2, 3, 30, 34, 32, 64}, {1, 1, 1, 1, 64, 64},
                           {3, 1, 7, 5, 128, 96}, {1, 12, 128, 128, 64, 64}};
    for (auto& d : dims) {
        for (int f32 = 0; f32 < 2; ++f32) {
            const size_t n = gtr_gla_workspace_bytes(d[0], d[1], d[2], d[3], d[4], d[5], 64, f32);
            if (n == 0) ++fails;
            int kern = 0, span = 0, grid = 0;
            expect(gtr_gla_plan(d[0], d[1], d[2], d[3], d[4], d[5], 64, f32, &kern, &span, &grid),
                   GTR_GLA_OK, "plan");
            expect(gtr_gla_plan_lowrank(d[0], d[1], d[2], d[3], d[4], d[5], 64, f32, nullptr,
                                        nullptr, nullptr), GTR_GLA_OK, "plan_lowrank");
            // caller workspace: too small, then enough (stand-in launches)
            if (!f32)
                expect(gtr_gla_fwd_ws(q, k, v, g, d[0], d[1], d[2], d[3], d[4], d[5], 1, 64, o, fs,
                                      ws, n - 1, st), GTR_GLA_ERR_WORKSPACE, "ws too small");
            const int r = f32 ? gtr_gla_fwd_f32_ws(static_cast<float*>(q), static_cast<float*>(k),
                                                    static_cast<float*>(v), static_cast<float*>(g),
                                                    d[0], d[1], d[2], d[3], d[4], d[5], 1, 64,
                                                    static_cast<float*>(o), fs, ws, n, st)
                              : gtr_gla_fwd_ws(q, k, v, g, d[0], d[1], d[2], d[3], d[4], d[5], 1,
                                               64, o, fs, ws, n, st);
            expect(r, GTR_GLA_OK, "ws call");
            expect(gtr_gla_fwd_ex(q, k, v, g, fs, o, nullptr, 1e-5f, d[0], d[1], d[2], d[3], d[4],
                                  d[5], 2, 64, f32, o, fs, ws, n, st),
                   GTR_GLA_ERR_NULL, "gate without weight");
        }
    }
    // library workspace: no device in this build
    expect(gtr_gla_fwd(q, k, v, g, 1, 2, 4, 4, 64, 64, 0, 64, o, fs, st), GTR_GLA_ERR_HIP, "no device");
    // invalid arguments
    expect(gtr_gla_fwd(nullptr, k, v, g, 1, 2, 4, 4, 64, 64, 0, 64, o, fs, st), GTR_GLA_ERR_NULL, "null q");
    expect(gtr_gla_fwd(q, k, v, g, 0, 2, 4, 4, 64, 64, 0, 64, o, fs, st), GTR_GLA_ERR_SHAPE, "B=0");
    expect(gtr_gla_fwd(q, k, v, g, INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, 0, 64, o,
                       fs, st), GTR_GLA_ERR_SHAPE, "INT_MAX sizes");
    expect(gtr_gla_fwd(q, k, v, g, 1, 1, 1 << 16, 1 << 16, 64, 64, 0, 64, o, fs, st),
           GTR_GLA_ERR_SHAPE, "L >= 2^31");
    expect(gtr_gla_fwd(q, k, v, g, 2, 1, 32768, 32768, 64, 64, 0, 64, o, fs, st),
           GTR_GLA_ERR_SHAPE, "B * L >= 2^31");
    expect(gtr_gla_fwd(q, k, v, g, 1, 4, 16384, 32768, 64, 64, 0, 64, o, fs, st),
           GTR_GLA_ERR_SHAPE, "B * L * H >= 2^31");
    expect(gtr_gla_fwd(q, k, v, g, 1, 2, 4, 4, 64, 64, 4, 64, o, fs, st), GTR_GLA_ERR_DIR, "dir");
    expect(gtr_gla_fwd(q, k, v, g, 1, 2, 4, 4, 64, 64, -1, 64, o, fs, st), GTR_GLA_ERR_DIR, "dir<0");
    expect(gtr_gla_fwd(q, k, v, g, 1, 2, 4, 4, 64, 64, 0, 48, o, fs, st), GTR_GLA_ERR_CHUNK, "chunk");
    expect(gtr_gla_fwd(q, k, v, g, 1, 2, 4, 4, 129, 64, 0, 64, o, fs, st), GTR_GLA_ERR_UNSUPPORTED, "d_k");
    expect(gtr_gla_fwd(q, k, v, g, 1, 2, 4, 4, 64, 513, 0, 64, o, fs, st), GTR_GLA_ERR_UNSUPPORTED, "d_v");
    expect(gtr_gla_fwd(q, k, v, g, 1, 2, 4, 4, 64, 64, 0, 64, static_cast<char*>(v) + 64, fs, st),
           GTR_GLA_ERR_ALIAS, "out in v");
    expect(gtr_gla_fwd(q, k, v, g, 1, 2, 4, 4, 64, 64, 0, 64, o, static_cast<float*>(q), st),
           GTR_GLA_ERR_ALIAS, "final_state on q");
    const float* nw = static_cast<const float*>(P(7));
    expect(gtr_gla_fwd_ex(q, k, v, g, nullptr, P(8), nw, NAN, 1, 2, 4, 4, 64, 64, 0, 64, 0, o, fs,
                          ws, 1 << 30, st), GTR_GLA_ERR_VALUE, "eps NaN");
    expect(gtr_gla_fwd_ex(q, k, v, g, nullptr, P(8), nw, -1.f, 1, 2, 4, 4, 64, 64, 0, 64, 0, o, fs,
                          ws, 1 << 30, st), GTR_GLA_ERR_VALUE, "eps < 0");
    expect(gtr_gla_fwd_ex(q, k, v, g, static_cast<float*>(o), nullptr, nullptr, 0.f, 1, 2, 4, 4,
                          64, 64, 0, 64, 0, o, fs, ws, 1 << 30, st), GTR_GLA_ERR_ALIAS, "init on out");
    const float* w1 = static_cast<const float*>(P(9));
    const float* w2 = static_cast<const float*>(P(10));
    const float* bias = static_cast<const float*>(P(11));
    expect(gtr_gla_fwd_lowrank(q, k, v, P(12), w1, w2, bias, 0.f, 64, nullptr, nullptr, nullptr,
                               0.f, 1, 2, 4, 4, 64, 64, 0, 64, 0, o, fs, ws, 1 << 30, st),
           GTR_GLA_ERR_VALUE, "inv_tau 0");
    expect(gtr_gla_fwd_lowrank(q, k, v, P(12), w1, w2, bias, 0.0625f, 0, nullptr, nullptr, nullptr,
                               0.f, 1, 2, 4, 4, 64, 64, 0, 64, 0, o, fs, ws, 1 << 30, st),
           GTR_GLA_ERR_SHAPE, "C = 0");
    expect(gtr_gla_fwd_lowrank(q, k, v, P(12), w1, w2, bias, 0.0625f, 128, nullptr, nullptr,
                               nullptr, 0.f, 1, 2, 4, 4, 64, 64, 0, 64, 0, o, fs, ws, 1 << 30, st),
           GTR_GLA_OK, "lowrank ws call");
    expect(gtr_gla_workspace_init(nullptr, 1024, st), GTR_GLA_ERR_NULL, "init null");
    expect(gtr_gla_workspace_init(ws, 100, st), GTR_GLA_ERR_WORKSPACE, "init small");
    expect(gtr_gla_workspace_status(ws, 100, st), GTR_GLA_ERR_WORKSPACE, "status small");
    expect(gtr_gla_set_exchange_wait(0, 0), GTR_GLA_ERR_VALUE, "wait 0");
    expect(gtr_gla_set_exchange_wait(1000, 0), GTR_GLA_OK, "wait");
    expect(gtr_gla_set_policy(7), GTR_GLA_ERR_POLICY, "policy");
    for (int s = -1; s < 20; ++s)
        if (!gtr_gla_status_str(s)) ++fails;
    std::printf("abi sanitizer driver: %d failures\n", fails);
    return fails ? 1 : 0;
}
