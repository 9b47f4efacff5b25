// gla_launch.h -- host-side launchers of the kernels, called by the C ABI layer.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#include "gla_common.h"

namespace gtrgla {

// GTR_GLA_LOG=1: diagnostics on stderr (gtr_gla_api.cpp). log_hip reports a
// failed HIP call by name; it prints only when logging is on.
bool log_enabled();
void log_hip(const char* where, hipError_t e);

// Workgroups of a launch the planners take as resident at once, given the
// occupancy bound per CU and the CU count (gla_fused.hip).
long long resident_cap(int per_cu, int cus);

// Generic three-phase path (gla_generic.hip).
size_t generic_workspace_bytes(const Shape& s);
// The generic kernels use the workspace past its header and mark the header
// dirty (a fused launch that finds it so does not trust the exchange words).
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
    int family = 1;  // 1: the kernels of gla_fused.hip; 2: the span kernels (gla_span.hip)
    int dk = 64;     // key dim of the exchanged state (span kernels: 32 or 64)
};
bool fused_supported(const Shape& s);
// span_override > 0 forces the span; rk_override > 0 then asks for the
// register-kept variant (when that span has one).
FusedPlan fused_plan(const Shape& s, int span_override, int rk_override, int var);
size_t fused_workspace_bytes(const Shape& s, const FusedPlan& p);
hipError_t launch_fused(const void* q, const void* k, const void* v, const void* lg,
                        const Shape& s, const Extras& x, const FusedPlan& p, void* out,
                        float* final_state, void* ws, hipStream_t st);

// Span kernels (gla_span.hip): d_v = 64, d_k 32 or 64, C = 64, no low-rank
// gate, at most 448 chunks per sequence. span_plan returns family 0 when no
// span plan fits; cap_override > 0 caps the resident workgroups (test hook).
bool span_supported(const Shape& s);
FusedPlan span_plan(const Shape& s, int span_override, long long cap_override, int var);
size_t span_workspace_bytes(const Shape& s, const FusedPlan& p);
hipError_t launch_span(const void* q, const void* k, const void* v, const void* lg, const Shape& s,
                       const Extras& x, const FusedPlan& p, void* out, float* final_state,
                       void* ws, hipStream_t st, unsigned int layout, int fault,
                       unsigned long long wait_ticks);

// Zero fill by a kernel (graph-capturable); p must be 16-byte aligned.
hipError_t fill_zero(void* p, size_t bytes, hipStream_t st);
// Workspace (re)initialisation by one kernel (graph-capturable): zero the whole
// region and write a clean header (gla_ws.h). bytes >= kWsHeaderBytes.
hipError_t init_workspace(void* p, size_t bytes, hipStream_t st);

// The in-kernel exchange's wait limit (microseconds per poll loop) and the test
// hook that silences span 0 of every sequence; read at each fused launch.
void set_exchange_wait(unsigned int wait_us, int fault);
unsigned int exchange_wait_us();
// The static scratch of gtr_gla_fwd_noalloc on a device, registered at its
// first use so that gtr_gla_workspace_status(NULL, ...) checks it too.
void register_scratch(int dev, void* p, size_t bytes);
// The argument checks of gtr_gla_fwd (sizes, direction, chunk, pointers,
// aliasing): a gtr_gla_status.
int validate_fwd_fp16(const void* q, const void* k, const void* v, const void* lg, int B, int H,
                      int gh, int gw, int dk, int dv, int dir, int chunk, const void* out,
                      const float* fs);
// Exchange layout word of a plan (the header's word 2).
unsigned int fused_layout_word(const FusedPlan& p);

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
