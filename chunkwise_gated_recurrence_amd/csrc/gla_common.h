// gla_common.h -- device-side helpers shared by the HIP kernels of libgtrgla.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace gtrgla {

// Spatial token visited at scan step t (token p = row * grid_w + col).
// The pages name the four walks (GTR summary page, section 核心方法: left->right,
// right->left, top->bottom, bottom->top); read as raster order, the reversed
// raster, column-major order and reversed column-major order.
__device__ __forceinline__ int scan_to_spatial(int t, int L, int grid_h, int grid_w, int dir)
{
    if (dir == 1) t = L - 1 - t;
    else if (dir == 3) t = L - 1 - t;
    if (dir >= 2) {
        int col = t / grid_h;
        int row = t - col * grid_h;
        return row * grid_w + col;
    }
    return t;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__half x) { return __half2float(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __half from_f32<__half>(float x) { return __float2half_rn(x); }

// Shape of one call, as the kernels see it.
struct Shape {
    int B, H, grid_h, grid_w, L, d_k, d_v, dir, chunk, n_chunks;
    float scale;   // d_k^{-1/2}
};

// Optional parts of a call: a nonzero initial state, and the RMSNorm + SiLU
// output gate applied to the outputs.
struct Extras {
    const float* init = nullptr;     // [B, H, d_k, d_v] or null (zero)
    const void* gate = nullptr;      // [B, L, H, d_v] in the input precision, or null
    const float* norm_w = nullptr;   // [d_v], with gate
    float eps = 0.f;
    // low-rank gate: log_gamma computed from z = x W1 (fp32 [B, L, 16]),
    // W2 [16, H d_k], bias [H d_k] and 1/tau instead of read
    const float* z = nullptr;
    const float* w2 = nullptr;
    const float* gbias = nullptr;
    float inv_tau = 0.f;
};

}  // namespace gtrgla
