// gtr_gla_noalloc.hip -- gtr_gla_fwd_noalloc: the fp16 forward for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation). Its workspace is one
// file-scope device array per GPU instead of a library- or caller-allocated
// buffer; everything else is gtr_gla_fwd_ws.
#include "gtr_gla.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "gla_launch.h"

namespace {

// The scratch of every gtr_gla_fwd_noalloc call on a GPU: the fused kernels'
// exchange words (and the generic kernels' chunk summaries), behind the
// 256-byte workspace header. Each GPU holds its own copy until the process
// ends; calls on one GPU share it.
constexpr size_t kScratchBytes = GTR_GLA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device

// Device address of the current device's copy of `scratch`, looked up once per
// device with that device current. (In host code the array's name is only a
// stand-in: kernels and copies take this address.)
int scratch_ptr(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GTR_GLA_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GTR_GLA_ERR_HIP;
        g_scratch[dev] = p;
        // gtr_gla_workspace_status(NULL, ...) checks it with the library's own workspaces
        gtrgla::register_scratch(dev, p, kScratchBytes);
    }
    *out = g_scratch[dev];
    return GTR_GLA_OK;
}

}  // namespace

extern "C" {

int gtr_gla_fwd_noalloc(const void* q, const void* k, const void* v, const void* log_gamma,
                        int B, int H, int grid_h, int grid_w, int d_k, int d_v, int dir, int chunk,
                        void* out, float* final_state, hipStream_t stream)
{
    const int bad = gtrgla::validate_fwd_fp16(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v,
                                              dir, chunk, out, final_state);
    if (bad != GTR_GLA_OK) return bad;
    if (gtr_gla_workspace_bytes(B, H, grid_h, grid_w, d_k, d_v, chunk, 0) > kScratchBytes)
        return GTR_GLA_ERR_SCRATCH;
    void* ws = nullptr;
    const int r = scratch_ptr(&ws);
    if (r != GTR_GLA_OK) return r;
    // The workspace layer zeroes the region (by a kernel, no hipMemsetAsync) on
    // first use and whenever the exchange layout changes; nothing allocates.
    return gtr_gla_fwd_ws(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, dir, chunk, out,
                          final_state, ws, kScratchBytes, stream);
}

}  // extern "C"
