// gla_gate.hip -- the data-dependent gate of GTR's token mixer (summary page
// "GTR:门控Token循环实现高效稠密预测", section 核心方法): gamma_t =
// sigma(x_t W1 W2 + b)^{1/tau} with a rank-16 factorisation W1 W2, so
// log_gamma = (1/tau) logsigmoid(x W1 W2 + b).
//
// The rank-16 projection z = x W1 runs here once per token (it is shared by
// every head); the fused kernels compute log_gamma from z, W2 and b on chip
// (no log_gamma tensor in memory). The generic kernels, which read log_gamma,
// get it from the second kernel below.
#include "gla_common.h"
#include "gla_launch.h"

namespace gtrgla {

constexpr int kRank = 16;

// One thread per (token, rank index r): z[token][r] = sum_c x[token][c] W1[c][r],
// fp32 accumulation; stored with the row permuted, r = 4s + k at 4k + s, the
// order in which the fused kernels' MFMAs take it (a lane holds four
// consecutive floats).
template <typename T>
__global__ void __launch_bounds__(256)
lowrank_project_kernel(const T* __restrict__ x, const float* __restrict__ w1, size_t rows, int C,
                       float* __restrict__ z)
{
    const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int r = threadIdx.x & 15;
    if (row >= rows) return;
    const T* xr = x + row * C;
    float acc = 0.f;
    for (int c = 0; c < C; ++c) acc += to_f32(xr[c]) * w1[(size_t)c * kRank + r];
    z[row * kRank + 4 * (r & 3) + (r >> 2)] = acc;
}

// The same for C a multiple of 4 16-byte vectors (and x 16-byte aligned): 64 tokens per workgroup,
// one per lane; wave w takes the w-th quarter of the C features, reading its
// token's row 16 bytes at a time, and W1's rows come through the scalar unit
// (the wave-uniform feature index makes them scalar loads, one 64-byte row per
// 16 FMAs). The four quarters' partial sums meet in LDS.
template <typename T>
__global__ void __launch_bounds__(256)
lowrank_project_tiled_kernel(const T* __restrict__ x, const float* __restrict__ w1, size_t rows,
                             int C, float* __restrict__ z)
{
    constexpr int kVec = 16 / sizeof(T);   // features per 16-byte load
    __shared__ float part[4][64][kRank + 1];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t r0 = (size_t)blockIdx.x * 64;
    const size_t row = r0 + lane < rows ? r0 + lane : rows - 1;
    const int cq = C >> 2;
    const int c0 = w * cq;
    const T* xr = x + row * C + c0;
    float acc[kRank];
#pragma unroll
    for (int r = 0; r < kRank; ++r) acc[r] = 0.f;
    for (int c = 0; c < cq; c += kVec) {
        const uint4 raw = *reinterpret_cast<const uint4*>(xr + c);
        const T* xv = reinterpret_cast<const T*>(&raw);
        const float* wr = w1 + (size_t)(c0 + c) * kRank;
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const float xe = to_f32(xv[e]);
#pragma unroll
            for (int r = 0; r < kRank; ++r) acc[r] += xe * wr[e * kRank + r];
        }
    }
#pragma unroll
    for (int r = 0; r < kRank; ++r) part[w][lane][r] = acc[r];
    __syncthreads();
    // thread: token tid / 4, stored positions 4k .. 4k + 3 (k = tid % 4),
    // i.e. rank indices r = 4s + k, s = 0 .. 3
    const int t = threadIdx.x >> 2, k = threadIdx.x & 3;
    if (r0 + t >= rows) return;
    float o[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        o[s] = part[0][t][4 * s + k] + part[1][t][4 * s + k] + part[2][t][4 * s + k] +
               part[3][t][4 * s + k];
    *reinterpret_cast<float4*>(z + (r0 + t) * kRank + 4 * k) = make_float4(o[0], o[1], o[2], o[3]);
}

// One thread per (token, key dim kk of all heads): log_gamma = inv_tau *
// logsigmoid(sum_r z[r] W2[r][kk] + bias[kk]), in the input precision.
template <typename T>
__global__ void __launch_bounds__(256)
lowrank_log_gamma_kernel(const float* __restrict__ z, const float* __restrict__ w2,
                         const float* __restrict__ bias, float inv_tau, size_t rows, int K,
                         T* __restrict__ lg)
{
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * (size_t)K) return;
    const size_t row = idx / K;
    const int kk = (int)(idx - row * K);
    const float* zr = z + row * kRank;
    float y = bias[kk];
    for (int r = 0; r < kRank; ++r) y += zr[4 * (r & 3) + (r >> 2)] * w2[(size_t)r * K + kk];
    const float ls = fminf(y, 0.f) - log1pf(expf(-fabsf(y)));
    lg[idx] = from_f32<T>(inv_tau * ls);
}

hipError_t launch_lowrank_project(const void* x, bool is_fp32, const float* w1, size_t rows, int C,
                                  float* z, hipStream_t st)
{
    if (rows == 0) return hipSuccess;
    const int vec = is_fp32 ? 4 : 8;
    if (C % (4 * vec) == 0 && ((uintptr_t)x & 15) == 0) {
        const unsigned tiles = (unsigned)((rows + 63) / 64);
        if (is_fp32)
            hipLaunchKernelGGL(lowrank_project_tiled_kernel<float>, dim3(tiles), dim3(256), 0, st,
                               (const float*)x, w1, rows, C, z);
        else
            hipLaunchKernelGGL(lowrank_project_tiled_kernel<__half>, dim3(tiles), dim3(256), 0,
                               st, (const __half*)x, w1, rows, C, z);
        return hipGetLastError();
    }
    const unsigned blocks = (unsigned)((rows + 15) / 16);
    if (is_fp32)
        hipLaunchKernelGGL(lowrank_project_kernel<float>, dim3(blocks), dim3(256), 0, st,
                           (const float*)x, w1, rows, C, z);
    else
        hipLaunchKernelGGL(lowrank_project_kernel<__half>, dim3(blocks), dim3(256), 0, st,
                           (const __half*)x, w1, rows, C, z);
    return hipGetLastError();
}

hipError_t launch_lowrank_log_gamma(const float* z, const float* w2, const float* bias,
                                    float inv_tau, size_t rows, int K, bool is_fp32, void* lg,
                                    hipStream_t st)
{
    const size_t n = rows * (size_t)K;
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (is_fp32)
        hipLaunchKernelGGL(lowrank_log_gamma_kernel<float>, dim3(blocks), dim3(256), 0, st, z, w2,
                           bias, inv_tau, rows, K, (float*)lg);
    else
        hipLaunchKernelGGL(lowrank_log_gamma_kernel<__half>, dim3(blocks), dim3(256), 0, st, z, w2,
                           bias, inv_tau, rows, K, (__half*)lg);
    return hipGetLastError();
}

}  // namespace gtrgla
