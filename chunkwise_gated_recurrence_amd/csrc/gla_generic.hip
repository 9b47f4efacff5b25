// gla_generic.hip -- the generic three-phase path: any supported shape, fp16 or
// fp32 inputs, fp32 arithmetic throughout.
//
// It is the fallback the pages' specialised operator relies on for settings
// outside its specialisation (GTR summary page, section 局限与改进), and the
// path for fp32 inputs. The three phases are those of the chunkwise evaluation
// (summary page, section 前置知识 › Chunkwise(分块)并行):
//   1. per chunk, in parallel: U_c = state reached from a zero state over the
//      chunk's tokens, d_c = prod of the chunk's gates (per key dim);
//   2. per (batch, head) and state element: the boundary scan
//      S_[c+1] = Diag(d_c) S_[c] + U_c, which also yields final_state;
//   3. per chunk, in parallel: the outputs, from S_[c] stepping token by token.
// Inside a chunk both phase 1 and phase 3 step the recurrence token by token in
// fp32 (one thread per value column j holds S[:, j] in registers), so no
// exponent of a gate sum can overflow, whatever the gates.
#include "gla_common.h"
#include "gla_launch.h"
#include "gla_ws.h"

namespace gtrgla {

constexpr int kTokGroup = 16;   // tokens staged in LDS per round

// Stage up to kTokGroup tokens of the chunk in LDS: spatial position, key row,
// gate, log gate and (optionally) query row. Padding dims get k = q = 0, gate 1.
template <typename T, int DKMAX, bool WITH_Q>
__device__ __forceinline__ void stage_tokens(const T* __restrict__ q, const T* __restrict__ k,
                                             const T* __restrict__ lg, const Shape& s, int b,
                                             int h, int t_first, int ng, int* spos,
                                             float (*sq)[DKMAX], float (*sk)[DKMAX],
                                             float (*sg)[DKMAX], float (*slg)[DKMAX])
{
    for (int u = threadIdx.x; u < ng; u += blockDim.x)
        spos[u] = scan_to_spatial(t_first + u, s.L, s.grid_h, s.grid_w, s.dir);
    __syncthreads();
    for (int e = threadIdx.x; e < kTokGroup * DKMAX; e += blockDim.x) {
        const int u = e / DKMAX, i = e - (e / DKMAX) * DKMAX;
        float kk = 0.f, qq = 0.f, gl = 0.f;
        if (u < ng && i < s.d_k) {
            const size_t off = ((size_t)b * s.L + spos[u]) * s.H * (size_t)s.d_k
                               + (size_t)h * s.d_k + i;
            kk = to_f32(k[off]);
            gl = to_f32(lg[off]);
            if (WITH_Q) qq = to_f32(q[off]);
        }
        sk[u][i] = kk;
        slg[u][i] = gl;
        sg[u][i] = expf(gl);
        if (WITH_Q) sq[u][i] = qq;
    }
    __syncthreads();
}

template <typename T, int DKMAX>
__global__ void __launch_bounds__(512)
generic_summary_kernel(const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ lg,
                       Shape s, float* __restrict__ wsU, float* __restrict__ wsD)
{
    const int bh = blockIdx.x / s.n_chunks;
    const int c = blockIdx.x - bh * s.n_chunks;
    const int b = bh / s.H, h = bh - (bh / s.H) * s.H;
    const int j = threadIdx.x;
    const int t0 = c * s.chunk;
    const int n = min(s.chunk, s.L - t0);

    __shared__ int spos[kTokGroup];
    __shared__ float sk[kTokGroup][DKMAX], sg[kTokGroup][DKMAX], slg[kTokGroup][DKMAX];

    float U[DKMAX];
#pragma unroll
    for (int i = 0; i < DKMAX; ++i) U[i] = 0.f;
    float lgsum = 0.f;   // thread j < d_k: sum of log gates of key dim j

    for (int g0 = 0; g0 < n; g0 += kTokGroup) {
        const int ng = min(kTokGroup, n - g0);
        __syncthreads();
        stage_tokens<T, DKMAX, false>(nullptr, k, lg, s, b, h, t0 + g0, ng, spos, nullptr, sk, sg,
                                      slg);
        if (j < s.d_k)
            for (int u = 0; u < ng; ++u) lgsum += slg[u][j];
        if (j < s.d_v) {
            for (int u = 0; u < ng; ++u) {
                const size_t offv = ((size_t)b * s.L + spos[u]) * s.H * (size_t)s.d_v
                                    + (size_t)h * s.d_v + j;
                const float vj = to_f32(v[offv]);
#pragma unroll
                for (int i = 0; i < DKMAX; ++i) U[i] = sg[u][i] * U[i] + sk[u][i] * vj;
            }
        }
    }
    const size_t cb = (size_t)bh * s.n_chunks + c;
    if (j < s.d_v) {
        float* dst = wsU + cb * s.d_k * (size_t)s.d_v + j;
#pragma unroll
        for (int i = 0; i < DKMAX; ++i)
            if (i < s.d_k) dst[(size_t)i * s.d_v] = U[i];
    }
    if (j < s.d_k) wsD[cb * s.d_k + j] = expf(lgsum);
}

// One thread per (b, h, i, j): S_[0] = the initial state (zero when init is
// null), S_[c+1] = d_c[i] S_[c] + U_c. U_c is replaced in place by S_[c], the
// state entering chunk c. init may be final_state itself: each element is
// read before it is written, by the same thread.
__global__ void __launch_bounds__(256)
generic_scan_kernel(Shape s, float* __restrict__ wsU, const float* __restrict__ wsD,
                    const float* init, float* final_state, size_t total)
{
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total) return;
    const size_t dkdv = (size_t)s.d_k * s.d_v;
    const size_t bh = e / dkdv;
    const size_t ij = e - bh * dkdv;
    const int i = (int)(ij / s.d_v);
    float S = init ? init[e] : 0.f;
    for (int c = 0; c < s.n_chunks; ++c) {
        const size_t cb = bh * s.n_chunks + c;
        float* u = wsU + cb * dkdv + ij;
        const float Uc = *u;
        *u = S;
        S = wsD[cb * s.d_k + i] * S + Uc;
    }
    if (final_state) final_state[e] = S;
}

template <typename T, int DKMAX>
__global__ void __launch_bounds__(512)
generic_output_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                      const T* __restrict__ lg, Shape s, const float* __restrict__ wsS,
                      T* __restrict__ out)
{
    const int bh = blockIdx.x / s.n_chunks;
    const int c = blockIdx.x - bh * s.n_chunks;
    const int b = bh / s.H, h = bh - (bh / s.H) * s.H;
    const int j = threadIdx.x;
    const int t0 = c * s.chunk;
    const int n = min(s.chunk, s.L - t0);

    __shared__ int spos[kTokGroup];
    __shared__ float sq[kTokGroup][DKMAX], sk[kTokGroup][DKMAX], sg[kTokGroup][DKMAX],
        slg[kTokGroup][DKMAX];

    float S[DKMAX];
    const size_t cb = (size_t)bh * s.n_chunks + c;
#pragma unroll
    for (int i = 0; i < DKMAX; ++i)
        S[i] = (j < s.d_v && i < s.d_k) ? wsS[(cb * s.d_k + i) * s.d_v + j] : 0.f;

    for (int g0 = 0; g0 < n; g0 += kTokGroup) {
        const int ng = min(kTokGroup, n - g0);
        __syncthreads();
        stage_tokens<T, DKMAX, true>(q, k, lg, s, b, h, t0 + g0, ng, spos, sq, sk, sg, slg);
        if (j < s.d_v) {
            for (int u = 0; u < ng; ++u) {
                const size_t offv = ((size_t)b * s.L + spos[u]) * s.H * (size_t)s.d_v
                                    + (size_t)h * s.d_v + j;
                const float vj = to_f32(v[offv]);
                float o = 0.f;
#pragma unroll
                for (int i = 0; i < DKMAX; ++i) {
                    S[i] = sg[u][i] * S[i] + sk[u][i] * vj;
                    o += sq[u][i] * S[i];
                }
                out[offv] = from_f32<T>(o * s.scale);
            }
        }
    }
}

// Output epilogue in place on out: one wave per (b, p, h) row of d_v outputs,
// y = o / sqrt(mean(o^2) + eps) * w * SiLU(z).
template <typename T>
__global__ void __launch_bounds__(256)
generic_gate_kernel(T* __restrict__ out, const T* __restrict__ gate, const float* __restrict__ w,
                    float eps, int d_v, size_t rows)
{
    const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    T* o = out + row * d_v;
    const T* z = gate + row * d_v;
    float ss = 0.f;
    for (int j = lane; j < d_v; j += 64) {
        const float x = to_f32(o[j]);
        ss += x * x;
    }
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float f = rsqrtf(ss / (float)d_v + eps);
    for (int j = lane; j < d_v; j += 64) {
        const float zz = to_f32(z[j]);
        o[j] = from_f32<T>(to_f32(o[j]) * f * w[j] * (zz / (1.f + expf(-zz))));
    }
}

size_t generic_workspace_bytes(const Shape& s)
{
    const size_t nb = (size_t)s.B * s.H * s.n_chunks;
    return kWsHeaderBytes + nb * ((size_t)s.d_k * s.d_v + s.d_k) * sizeof(float);
}

// The generic kernels overwrite what a fused launch left past the header:
// mark the header so that no fused launch trusts those words.
__global__ void mark_dirty_kernel(unsigned int* hdr) { hdr[kWsMagicWord] = kWsDirty; }

template <typename T, int DKMAX>
static hipError_t launch_generic_t(const T* q, const T* k, const T* v, const T* lg, const Shape& s,
                                   const Extras& x, T* out, float* final_state, void* ws,
                                   hipStream_t st)
{
    const size_t nb = (size_t)s.B * s.H * s.n_chunks;
    hipLaunchKernelGGL(mark_dirty_kernel, dim3(1), dim3(1), 0, st, static_cast<unsigned int*>(ws));
    float* wsU = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + kWsHeaderBytes);
    float* wsD = wsU + nb * s.d_k * (size_t)s.d_v;
    const int threads = ((s.d_v > 64 ? s.d_v : 64) + 63) / 64 * 64;
    const unsigned grid = (unsigned)nb;
    hipLaunchKernelGGL((generic_summary_kernel<T, DKMAX>), dim3(grid), dim3(threads), 0, st, k, v,
                       lg, s, wsU, wsD);
    const size_t total = (size_t)s.B * s.H * s.d_k * s.d_v;
    hipLaunchKernelGGL(generic_scan_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       st, s, wsU, wsD, x.init, final_state, total);
    hipLaunchKernelGGL((generic_output_kernel<T, DKMAX>), dim3(grid), dim3(threads), 0, st, q, k,
                       v, lg, s, wsU, out);
    if (x.gate) {
        const size_t rows = (size_t)s.B * s.L * s.H;
        hipLaunchKernelGGL((generic_gate_kernel<T>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                           st, out, (const T*)x.gate, x.norm_w, x.eps, s.d_v, rows);
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_generic_dk(const T* q, const T* k, const T* v, const T* lg,
                                    const Shape& s, const Extras& x, T* out, float* fs, void* ws,
                                    hipStream_t st)
{
    if (s.d_k <= 32) return launch_generic_t<T, 32>(q, k, v, lg, s, x, out, fs, ws, st);
    if (s.d_k <= 64) return launch_generic_t<T, 64>(q, k, v, lg, s, x, out, fs, ws, st);
    return launch_generic_t<T, 128>(q, k, v, lg, s, x, out, fs, ws, st);
}

hipError_t launch_generic(const void* q, const void* k, const void* v, const void* lg,
                          bool is_fp32, const Shape& s, const Extras& x, void* out,
                          float* final_state, void* ws, hipStream_t st)
{
    if (is_fp32)
        return launch_generic_dk<float>((const float*)q, (const float*)k, (const float*)v,
                                        (const float*)lg, s, x, (float*)out, final_state, ws, st);
    return launch_generic_dk<__half>((const __half*)q, (const __half*)k, (const __half*)v,
                                     (const __half*)lg, s, x, (__half*)out, final_state, ws, st);
}

}  // namespace gtrgla
