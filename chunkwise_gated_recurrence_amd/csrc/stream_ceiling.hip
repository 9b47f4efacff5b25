// stream_ceiling.hip -- the practical bandwidth ceiling of a call: a plain
// streaming kernel that reads four fp16 tensors and writes one, the same bytes
// the operator must move for q, k, v, log_gamma and out (o = q + k + v + g, an
// arithmetic that costs nothing next to the traffic). Built as its own library
// (libgtrgla_ceiling.so); only the benchmark uses it, to report the operator's
// time against what a kernel that only streams the same bytes achieves.
// Each thread handles UNROLL consecutive grid-stride steps at once, so that
// 4 * UNROLL 16-byte loads are in flight per thread.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

template <int UNROLL>
__global__ void __launch_bounds__(256)
stream4to1(const h8* __restrict__ a, const h8* __restrict__ b, const h8* __restrict__ c,
           const h8* __restrict__ d, h8* __restrict__ o, size_t n8)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (UNROLL - 1) * stride < n8; i += UNROLL * stride) {
        h8 x[UNROLL], y[UNROLL], z[UNROLL], w[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            x[u] = a[i + u * stride];
            y[u] = b[i + u * stride];
            z[u] = c[i + u * stride];
            w[u] = d[i + u * stride];
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            h8 r;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                r[e] = (_Float16)((float)x[u][e] + (float)y[u][e] + (float)z[u][e] + (float)w[u][e]);
            __builtin_nontemporal_store(r, o + i + u * stride);
        }
    }
    for (; i < n8; i += stride) {
        const h8 x = a[i], y = b[i], z = c[i], w = d[i];
        h8 r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (_Float16)((float)x[e] + (float)y[e] + (float)z[e] + (float)w[e]);
        __builtin_nontemporal_store(r, o + i);
    }
}

}  // namespace

extern "C" {

// o[i] = a[i] + b[i] + c[i] + d[i] over n_halves fp16 elements (a multiple of 8;
// every pointer 16-byte aligned); unroll 1, 2 or 4. Returns 0, 1 on bad
// arguments, 2 on a launch error.
int gtr_stream_ceiling(const void* a, const void* b, const void* c, const void* d, void* o,
                       size_t n_halves, int blocks, int unroll, hipStream_t st)
{
    if (!a || !b || !c || !d || !o || n_halves % 8 != 0 || blocks < 1) return 1;
    if (unroll != 1 && unroll != 2 && unroll != 4) return 1;
    const uintptr_t all = (uintptr_t)a | (uintptr_t)b | (uintptr_t)c | (uintptr_t)d | (uintptr_t)o;
    if (all & 15) return 1;
    const size_t n8 = n_halves / 8;
    const h8 *pa = (const h8*)a, *pb = (const h8*)b, *pc = (const h8*)c, *pd = (const h8*)d;
    if (unroll == 1)
        hipLaunchKernelGGL(stream4to1<1>, dim3(blocks), dim3(256), 0, st, pa, pb, pc, pd, (h8*)o, n8);
    else if (unroll == 2)
        hipLaunchKernelGGL(stream4to1<2>, dim3(blocks), dim3(256), 0, st, pa, pb, pc, pd, (h8*)o, n8);
    else
        hipLaunchKernelGGL(stream4to1<4>, dim3(blocks), dim3(256), 0, st, pa, pb, pc, pd, (h8*)o, n8);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
