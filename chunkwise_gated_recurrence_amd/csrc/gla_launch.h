// gla_launch.h -- host-side launchers of the kernels, called by the C ABI layer.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#include "gla_common.h"

namespace gtrgla {

// Generic three-phase path (gla_generic.hip).
size_t generic_workspace_bytes(const Shape& s);
hipError_t launch_generic(const void* q, const void* k, const void* v, const void* lg,
                          bool is_fp32, const Shape& s, const Extras& x, void* out,
                          float* final_state, void* ws, hipStream_t st);

// Fused fp16 MFMA path (gla_fused.hip).
struct FusedPlan {
    int span;        // chunks per workgroup
    bool keep;       // outputs kept through the boundary scan
    bool rk;         // kept in registers, next chunk staged in LDS (two workgroups per CU)
    int n_spans;     // spans (workgroups) per (batch, head) sequence
    int seq_batch;   // sequences per launch (every workgroup of a launch is resident)
    int grid;        // workgroups per launch
    int slice_log2;  // log2 of the state elements each owning workgroup scans
    int var;         // kernel variant: 0 plain, 1 with initial state / output gate,
                     // 2 also with log_gamma computed from the low-rank gate
};
bool fused_supported(const Shape& s);
// span_override > 0 forces the span; rk_override > 0 then asks for the
// register-kept variant (when that span has one).
FusedPlan fused_plan(const Shape& s, int span_override, int rk_override, int var);
size_t fused_workspace_bytes(const Shape& s, const FusedPlan& p);
hipError_t launch_fused(const void* q, const void* k, const void* v, const void* lg,
                        const Shape& s, const Extras& x, const FusedPlan& p, void* out,
                        float* final_state, void* ws, hipStream_t st);

// Zero fill by a kernel (graph-capturable); p must be 16-byte aligned.
hipError_t fill_zero(void* p, size_t bytes, hipStream_t st);

// Low-rank gate (gla_gate.hip): z = x W1 per token, [rows, 16] fp32 in
// natural rank order; and log_gamma [rows, K] (K = H dk,
// the input precision) = inv_tau * logsigmoid(z W2 + bias) for the generic path.
hipError_t launch_lowrank_project(const void* x, bool is_fp32, const float* w1, size_t rows, int C,
                                  float* z, hipStream_t st);
hipError_t launch_lowrank_log_gamma(const float* z, const float* w2, const float* bias,
                                    float inv_tau, size_t rows, int K, bool is_fp32, void* lg,
                                    hipStream_t st);

// Spatial SwiGLU: the up kernel (X W_g, X W_v over 8x8 tiles with their halo,
// the 3x3 depthwise convolution, the bias and the SiLU gate) into a_ws
// [B, L, Hd] fp16, then the down kernel y = a_ws W_o^T.
hipError_t launch_sswiglu(const void* x, const void* wg, const void* wv, const float* cw,
                          const float* cb, const void* wo, int B, int gh, int gw, int C, int Hd,
                          void* y, void* a_ws, hipStream_t st);

}  // namespace gtrgla
