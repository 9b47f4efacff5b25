// sswiglu_api.cpp -- the C ABI of the Spatial SwiGLU channel mixer (declared
// in include/gtr_sswiglu.h): argument validation, the library-owned workspace
// and dispatch to the two kernels. Nothing here throws across the ABI.
#include "gtr_sswiglu.h"
#include "gtr_gla.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <utility>

#include "gla_launch.h"

namespace {

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return a && b && x < y + nb && y < x + na;
}

int validate(int B, int gh, int gw, int C, int Hd)
{
    if (B < 1 || gh < 1 || gw < 1 || C < 1 || Hd < 1) return GTR_GLA_ERR_SHAPE;
    if (C % 64 != 0 || Hd % 128 != 0 || C > 8192 || Hd > 32768) return GTR_GLA_ERR_UNSUPPORTED;
    const long long L = (long long)gh * gw;
    const long long lim = 1LL << 31;
    if (L * C * 2 >= lim || (long long)B * L * Hd * 2 >= lim || (long long)B * L >= lim)
        return GTR_GLA_ERR_UNSUPPORTED;
    return GTR_GLA_OK;
}

struct Ws {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_mu;
std::map<std::pair<int, uintptr_t>, Ws> g_ws;

int own_workspace(size_t need, hipStream_t st, void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GTR_GLA_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    Ws& w = g_ws[std::make_pair(dev, (uintptr_t)st)];
    if (w.bytes < need) {
        if (w.ptr) {
            // the previous workspace may still be in use by work on this stream
            if (hipStreamSynchronize(st) != hipSuccess) return GTR_GLA_ERR_HIP;
            (void)hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
        }
        if (hipMalloc(&w.ptr, need) != hipSuccess) {
            w.ptr = nullptr;
            return GTR_GLA_ERR_HIP;
        }
        w.bytes = need;
    }
    *out = w.ptr;
    return GTR_GLA_OK;
}

}  // namespace

extern "C" {

size_t gtr_sswiglu_workspace_bytes(int B, int grid_h, int grid_w, int C, int Hd)
{
    if (validate(B, grid_h, grid_w, C, Hd) != GTR_GLA_OK) return 0;
    return (size_t)B * grid_h * grid_w * Hd * 2;
}

int gtr_sswiglu_fwd(const void* x, const void* w_g, const void* w_v, const float* conv_w,
                    const float* conv_b, const void* w_o, int B, int grid_h, int grid_w, int C,
                    int Hd, void* y, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    int r = validate(B, grid_h, grid_w, C, Hd);
    if (r != GTR_GLA_OK) return r;
    if (!x || !w_g || !w_v || !conv_w || !w_o || !y) return GTR_GLA_ERR_NULL;
    const size_t L = (size_t)grid_h * grid_w;
    const size_t nx = (size_t)B * L * C * 2;
    const size_t nw = (size_t)Hd * C * 2;
    const size_t need = (size_t)B * L * Hd * 2;
    const void* ins[6] = {x, w_g, w_v, conv_w, conv_b, w_o};
    const size_t ns[6] = {nx, nw, nw, (size_t)Hd * 36, (size_t)Hd * 4, nw};
    for (int i = 0; i < 6; ++i)
        if (overlaps(y, nx, ins[i], ns[i])) return GTR_GLA_ERR_ALIAS;
    if (workspace) {
        if (workspace_bytes < need) return GTR_GLA_ERR_WORKSPACE;
        if (overlaps(workspace, need, y, nx)) return GTR_GLA_ERR_ALIAS;
        for (int i = 0; i < 6; ++i)
            if (overlaps(workspace, need, ins[i], ns[i])) return GTR_GLA_ERR_ALIAS;
    } else {
        r = own_workspace(need, stream, &workspace);
        if (r != GTR_GLA_OK) return r;
    }
    const hipError_t e = gtrgla::launch_sswiglu(x, w_g, w_v, conv_w, conv_b, w_o, B, grid_h,
                                                grid_w, C, Hd, y, workspace, stream);
    return e == hipSuccess ? GTR_GLA_OK : GTR_GLA_ERR_HIP;
}

}  // extern "C"
