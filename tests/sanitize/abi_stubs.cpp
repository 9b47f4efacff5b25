// Host sanitizer build of the C ABI layer (csrc/gtr_gla_api.cpp): stand-ins for
// the kernel-launch layer (gla_launch.h) and for the HIP runtime calls the ABI
// layer makes, so that its validation, planning glue and workspace bookkeeping
// run under ASan/UBSan on a host with no GPU. Launches "succeed" without doing
// anything; runtime calls that would need a device report no device.
#include <hip/hip_runtime_api.h>

#include <cstring>

#include "gla_launch.h"
#include "gla_ws.h"

namespace gtrgla {

size_t generic_workspace_bytes(const Shape& s)
{
    const size_t nb = (size_t)s.B * s.H * s.n_chunks;
    return kWsHeaderBytes + nb * ((size_t)s.d_k * s.d_v + s.d_k) * sizeof(float);
}
hipError_t launch_generic(const void*, const void*, const void*, const void*, bool, const Shape&,
                          const Extras&, void*, float*, void*, hipStream_t)
{
    return hipSuccess;
}
bool fused_supported(const Shape& s)
{
    return (s.d_k == 64 || s.d_k == 32) && s.d_v == 64 && s.chunk == 64;
}
FusedPlan fused_plan(const Shape& s, int span_override, int, int var)
{
    FusedPlan p;
    p.span = span_override > 0 ? span_override : 1;
    p.keep = true;
    p.rk = false;
    p.n_spans = (s.n_chunks + p.span - 1) / p.span;
    p.seq_batch = s.B * s.H;
    p.grid = p.seq_batch * p.n_spans;
    p.slice_log2 = 12;
    p.var = var;
    return p;
}
size_t fused_workspace_bytes(const Shape&, const FusedPlan& p)
{
    return 256 + (size_t)p.grid * (4 + 16 * 1024 + 8 * 1024);
}
hipError_t launch_fused(const void*, const void*, const void*, const void*, const Shape&,
                        const Extras&, const FusedPlan&, void*, float*, void*, hipStream_t)
{
    return hipSuccess;
}
// span kernels: shapes they take plan like the other fused kernels here
bool span_supported(const Shape& s) { return s.d_k == 32 && s.d_v == 64 && s.chunk == 64; }
FusedPlan span_plan(const Shape& s, int span_override, long long, int var)
{
    FusedPlan p = fused_plan(s, span_override, 0, var);
    p.family = 2;
    p.dk = s.d_k;
    return p;
}
size_t span_workspace_bytes(const Shape& s, const FusedPlan& p) { return fused_workspace_bytes(s, p); }
hipError_t launch_span(const void*, const void*, const void*, const void*, const Shape&,
                       const Extras&, const FusedPlan&, void*, float*, void*, hipStream_t,
                       unsigned int, int, unsigned long long)
{
    return hipSuccess;
}
hipError_t fill_zero(void*, size_t, hipStream_t) { return hipSuccess; }
hipError_t init_workspace(void*, size_t bytes, hipStream_t)
{
    return bytes < (size_t)kWsHeaderBytes ? hipErrorInvalidValue : hipSuccess;
}
static unsigned int g_wait = 20000;
void set_exchange_wait(unsigned int wait_us, int) { g_wait = wait_us; }
unsigned int exchange_wait_us() { return g_wait; }
unsigned int fused_layout_word(const FusedPlan& p) { return (unsigned)p.n_spans; }
hipError_t launch_lowrank_project(const void*, bool, const float*, size_t, int, float*, hipStream_t)
{
    return hipSuccess;
}
hipError_t launch_lowrank_log_gamma(const float*, const float*, const float*, float, size_t, int,
                                    bool, void*, hipStream_t)
{
    return hipSuccess;
}

}  // namespace gtrgla

extern "C" {
hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipMalloc(void**, size_t) { return hipErrorNoDevice; }
hipError_t hipFree(void*) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void*, size_t n, hipMemcpyKind, hipStream_t)
{
    std::memset(dst, 0, n);   // a clean error word
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
const char* hipGetErrorName(hipError_t) { return "hipErrorStub"; }
}
