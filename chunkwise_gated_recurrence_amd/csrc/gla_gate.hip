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
// fp32 accumulation.
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
    z[row * kRank + r] = acc;
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
    // thread: token tid / 4, ranks 4k .. 4k + 3 (k = tid % 4)
    const int t = threadIdx.x >> 2, k = threadIdx.x & 3;
    if (r0 + t >= rows) return;
    float o[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        o[s] = part[0][t][4 * k + s] + part[1][t][4 * k + s] + part[2][t][4 * k + s] +
               part[3][t][4 * k + s];
    *reinterpret_cast<float4*>(z + (r0 + t) * kRank + 4 * k) = make_float4(o[0], o[1], o[2], o[3]);
}

typedef _Float16 gh8 __attribute__((ext_vector_type(8)));
typedef float gf4 __attribute__((ext_vector_type(4)));

// fp16 x with C a multiple of 128 (and x 16-byte aligned): the product on
// fp16 MFMA (16x16x32, fp32 accumulation), z^T = W1^T x^T for 16 T tokens per
// workgroup (T 16-token tiles per wave, sharing the W1 operand), wave w over
// the w-th quarter of the features. x is exact in fp16; W1 enters as hi + lo,
// two fp16 parts (hi = fp16(W1), lo = fp16(W1 - hi)), one MFMA each, which
// keeps it to about 2^-22 of its value above fp16's normal range and to 2^-24
// absolute below it. The A operand's row m is rank m, so each lane ends with
// ranks 4g .. 4g + 3 of its token; the four quarters meet in LDS.
template <int T>
__global__ void __launch_bounds__(256)
lowrank_project_mfma_kernel(const __half* __restrict__ x, const float* __restrict__ w1,
                            size_t rows, int C, float* __restrict__ z)
{
    __shared__ gf4 part[4][T][64];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, kb = lane >> 4;
    const size_t r0 = (size_t)blockIdx.x * 16 * T;
    const int cq = C >> 2;
    const int c0 = w * cq + 8 * kb;
    const float* wr = w1 + (size_t)c0 * kRank + n;
    const _Float16* xr[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const size_t row = r0 + 16 * t + n < rows ? r0 + 16 * t + n : rows - 1;
        xr[t] = reinterpret_cast<const _Float16*>(x) + row * C + c0;
    }
    gf4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = gf4{0.f, 0.f, 0.f, 0.f};
    if constexpr (T == 1) {
        // groups of four 32-feature steps: every load of a group is issued
        // before its MFMAs (C <= 512: the whole product in one group). The loads
        // are unconditional (a step past the end re-reads the last one, in
        // bounds) so that they form one block; only the MFMAs are skipped.
        for (int c0 = 0; c0 < cq; c0 += 128) {
            gh8 b[4][T];
            float wv[4][8];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int c = min(c0 + 32 * st, cq - 32);
#pragma unroll
                for (int t = 0; t < T; ++t) b[st][t] = *reinterpret_cast<const gh8*>(xr[t] + c);
#pragma unroll
                for (int e = 0; e < 8; ++e) wv[st][e] = wr[(size_t)(c + e) * kRank];
            }
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                if (c0 + 32 * st < cq) {   // uniform
                    gh8 hi, lo;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        hi[e] = (_Float16)wv[st][e];
                        lo[e] = (_Float16)(wv[st][e] - (float)hi[e]);
                    }
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, b[st][t], acc[t], 0, 0, 0);
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, b[st][t], acc[t], 0, 0, 0);
                    }
                }
            }
        }
    } else {
        // long inputs (bandwidth-bound): one step at a time measured faster
        // than the grouped loads above
        for (int c = 0; c < cq; c += 32) {
            gh8 b[T];
#pragma unroll
            for (int t = 0; t < T; ++t) b[t] = *reinterpret_cast<const gh8*>(xr[t] + c);
            gh8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = wr[(size_t)(c + e) * kRank];
                hi[e] = (_Float16)v;
                lo[e] = (_Float16)(v - (float)hi[e]);
            }
#pragma unroll
            for (int t = 0; t < T; ++t) {
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, b[t], acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, b[t], acc[t], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) part[w][t][lane] = acc[t];
    __syncthreads();
    // thread o < 64 T: tile o / 64, lane o % 64 of the waves' results
    const int o = threadIdx.x;
    if (o >= 64 * T) return;
    const int t = o >> 6, l = o & 63;
    const size_t row = r0 + 16 * t + (l & 15);
    if (row >= rows) return;
    const gf4 s = part[0][t][l] + part[1][t][l] + part[2][t][l] + part[3][t][l];
    *reinterpret_cast<gf4*>(z + row * kRank + 4 * (l >> 4)) = s;
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
    for (int r = 0; r < kRank; ++r) y += zr[r] * w2[(size_t)r * K + kk];
    const float ls = fminf(y, 0.f) - log1pf(expf(-fabsf(y)));
    lg[idx] = from_f32<T>(inv_tau * ls);
}

hipError_t launch_lowrank_project(const void* x, bool is_fp32, const float* w1, size_t rows, int C,
                                  float* z, hipStream_t st)
{
    if (rows == 0) return hipSuccess;
    const bool aligned = ((uintptr_t)x & 15) == 0;
    if (!is_fp32 && C % 128 == 0 && aligned) {
        // one 16-token tile per workgroup while that leaves fewer workgroups
        // than two per CU (short sequences: latency), else two sharing W1
        if (rows <= 16 * 512)
            hipLaunchKernelGGL(lowrank_project_mfma_kernel<1>, dim3((unsigned)((rows + 15) / 16)),
                               dim3(256), 0, st, (const __half*)x, w1, rows, C, z);
        else
            hipLaunchKernelGGL(lowrank_project_mfma_kernel<2>, dim3((unsigned)((rows + 31) / 32)),
                               dim3(256), 0, st, (const __half*)x, w1, rows, C, z);
        return hipGetLastError();
    }
    const int vec = is_fp32 ? 4 : 8;
    if (C % (4 * vec) == 0 && aligned) {
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
