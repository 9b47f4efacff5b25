/*
 * gtr_gla.h -- C ABI of libgtrgla: the inference forward pass of the key-only
 * gated linear attention (GLA) token mixer of "GTR: Gated Token Recurrence for
 * Efficient Dense Prediction", on AMD Instinct MI355X (gfx950).
 *
 * Operation (GTR summary page "GTR:门控Token循环实现高效稠密预测", section
 * 前置知识 › 门控线性注意力(GLA) and section 核心方法): for every batch entry b
 * and head h, along one scan order over the stride-16 patch grid,
 *
 *     S_t = Diag(gamma_t) S_{t-1} + k_t^T v_t,    o_t = d_k^{-1/2} q_t S_t,
 *
 * with S_0 = 0, gamma_t = exp(log_gamma_t) a per-key-dimension gate and no
 * decay on the value side. It is evaluated chunkwise (section 前置知识 ›
 * Chunkwise(分块)并行 of the same page; section 3.3 of the 0539edu.com page):
 * per-chunk summaries U_c and decays d_c, the boundary scan
 * S_[c+1] = Diag(d_c) S_[c] + U_c, and per-chunk outputs.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors (all contiguous, row-major, device memory owned by the caller):
 *   q, k, log_gamma : [B, L, H, d_k]      v, out : [B, L, H, d_v]
 *   final_state     : [B, H, d_k, d_v] fp32, the state after the last scan
 *                     step, without the d_k^{-1/2} scale. May be NULL.
 *   L = grid_h * grid_w; spatial token p = row * grid_w + col.
 *   log_gamma is the natural log of the gate, finite and <= 0.
 * Scan order (dir): the pages name left->right, right->left, top->bottom and
 *   bottom->top (summary page, section 核心方法). Read here as
 *   0 raster order, 1 the whole raster reversed, 2 column-major order,
 *   3 column-major order reversed. o for token p is written at p.
 * chunk: tokens per chunk, one of 16, 32, 64, 128 (64 is the pages' choice,
 *   summary page section 方法步骤详情).
 * Outputs are fully overwritten, never accumulated into. Outputs must not
 *   overlap inputs or each other. Inputs are read only.
 * Errors: every entry point returns a gtr_gla_status. A call that fails
 *   validation launches nothing and writes nothing. GTR_GLA_ERR_HIP reports a
 *   HIP error seen while launching; faults inside a kernel surface at the
 *   caller's next synchronisation, as for any HIP call. Nothing throws.
 * Synchronisation: every call is asynchronous on `stream`. It performs no
 *   host synchronisation and no device-to-host copy.
 */
#ifndef GTR_GLA_H
#define GTR_GLA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GTR_GLA_L2R = 0,   /* left -> right: raster order            */
    GTR_GLA_R2L = 1,   /* right -> left: raster order reversed   */
    GTR_GLA_T2B = 2,   /* top -> bottom: column-major order      */
    GTR_GLA_B2T = 3    /* bottom -> top: column-major reversed   */
} gtr_gla_dir;

typedef enum {
    GTR_GLA_OK = 0,
    GTR_GLA_ERR_NULL = 1,        /* a required pointer is NULL                       */
    GTR_GLA_ERR_SHAPE = 2,       /* a size is < 1, or a tensor would exceed 2^31 rows */
    GTR_GLA_ERR_DIR = 3,         /* dir not in 0..3                                  */
    GTR_GLA_ERR_CHUNK = 4,       /* chunk not in {16, 32, 64, 128}                    */
    GTR_GLA_ERR_UNSUPPORTED = 5, /* no kernel for these head sizes (d_k > 128 or d_v > 512) */
    GTR_GLA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required          */
    GTR_GLA_ERR_HIP = 7,         /* the HIP runtime reported an error               */
    GTR_GLA_ERR_ALIAS = 8,       /* an output overlaps an input or the other output  */
    GTR_GLA_ERR_POLICY = 9,      /* unknown policy value                             */
    GTR_GLA_ERR_VALUE = 10,      /* invalid scalar argument (norm_eps not finite or < 0,
                                    inv_tau not finite or <= 0, exchange wait out of
                                    range)                                          */
    GTR_GLA_ERR_EXCHANGE = 11,   /* (gtr_gla_workspace_status only) a fused call's
                                    boundary exchange gave up waiting: that call wrote
                                    NaN outputs and final state                      */
    GTR_GLA_ERR_WS_STATE = 12,   /* (gtr_gla_workspace_status only) a fused call found
                                    its workspace neither initialised nor last used by
                                    calls of its layout: it wrote NaN outputs          */
    GTR_GLA_ERR_SCRATCH = 13     /* gtr_gla_fwd_noalloc: the call needs more workspace
                                    than its static scratch holds                     */
} gtr_gla_status;

/* Launch policies (the pages' length-aware scheduling: short sequences take
 * one kernel, long ones an occupancy-aware kernel that overlaps the boundary
 * scan with output computation; 0539edu.com page, section 3.3).            */
typedef enum {
    GTR_GLA_POLICY_AUTO = 0,     /* choose by shape (the default)                    */
    GTR_GLA_POLICY_GENERIC = 1,  /* three generic fp32 kernels: summaries, scan,
                                    outputs. Any supported shape, fp16 or fp32.     */
    GTR_GLA_POLICY_FUSED = 2,    /* one fp16 MFMA kernel, one workgroup per span of
                                    chunks, boundary states exchanged between the
                                    resident workgroups of a launch.                */
    GTR_GLA_POLICY_FUSED_ONE = 3 /* the fused kernel with one chunk per span        */
} gtr_gla_policy;

/*
 * gtr_gla_fwd -- fp16 (IEEE binary16) q, k, v, log_gamma and out; fp32
 * accumulation, fp32 state and fp32 final_state.
 * Uses a workspace that the library allocates on the first call for each
 * (device, stream) pair and grows when a larger shape arrives; call it once
 * outside stream capture for a shape before capturing it.
 *
 * Concurrency of the fused kernels. A fused launch hands boundary states
 * between its workgroups inside the kernel, so it needs all of them resident
 * on the GPU at once; the launch policy sizes its grid to the whole chip. Run
 * fused calls one at a time per GPU (one stream, or streams ordered by
 * events), and not beside other kernels that occupy compute units for long.
 * If some workgroups cannot become resident, every wait in the exchange gives
 * up after its deadline (gtr_gla_set_exchange_wait, 20 ms by default): the
 * call then writes NaN outputs and final state instead of hanging or returning
 * wrong numbers, and gtr_gla_workspace_status reports it.
 */
int gtr_gla_fwd(const void* q, const void* k, const void* v, const void* log_gamma,
                int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                int dir, int chunk, void* out, float* final_state, hipStream_t stream);

/* gtr_gla_fwd_f32 -- the same with every tensor fp32 (generic kernels only). */
int gtr_gla_fwd_f32(const float* q, const float* k, const float* v, const float* log_gamma,
                    int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                    int dir, int chunk, float* out, float* final_state, hipStream_t stream);

/*
 * Caller-managed workspace (the deployment interface of the pages supports a
 * persistent caller-managed workspace, preallocated outputs and graph capture:
 * 0539edu.com page, appendix E.3.1).
 * gtr_gla_workspace_bytes returns the size needed by the _ws entry points for
 * this shape and precision under the current policy, or 0 for invalid sizes.
 * A workspace must be initialised once by gtr_gla_workspace_init before its
 * first use; the kernels leave it ready for the next call of the same layout,
 * and an eager call of another layout re-initialises it first. A fused kernel
 * that finds it in any other state writes NaN outputs (see
 * gtr_gla_workspace_status). One workspace must not be used by two calls that
 * may run at the same time. GTR_GLA_LOG=1 in the environment prints each
 * call's kernel, plan and launch geometry on stderr.
 * The _ws entry points allocate nothing and may be captured in a HIP graph.
 */
/*
 * gtr_gla_fwd_ex -- gtr_gla_fwd (is_fp32 = 0) or gtr_gla_fwd_f32 (is_fp32 = 1)
 * with the two additions the pages' end-to-end operator has around the
 * recurrence (summary page, section 方法步骤详情 step 5, specialises it to a
 * zero initial state and fuses RMSNorm and the output gate into the output
 * epilogue; 0539edu.com page, appendix E.3.1):
 *   initial_state [B, H, d_k, d_v] fp32: S_0 instead of zero, e.g. the
 *     final_state of the preceding part of a scan. NULL: zero. It may be the
 *     very pointer passed as final_state (then updated in place); any other
 *     overlap with an output is GTR_GLA_ERR_ALIAS.
 *   gate [B, L, H, d_v] (fp16, or fp32 when is_fp32), norm_weight [d_v] fp32,
 *     norm_eps: out = o / sqrt(mean_j o_j^2 + norm_eps) * norm_weight *
 *     SiLU(gate), SiLU(z) = z / (1 + e^-z), the mean taken over the d_v
 *     outputs o of one (batch, token, head). norm_weight is shared by the
 *     heads. gate NULL: out = o, and norm_weight and norm_eps are ignored.
 *     With a gate, norm_weight must not be NULL (GTR_GLA_ERR_NULL) and
 *     norm_eps must be finite and >= 0 (GTR_GLA_ERR_VALUE).
 *   final_state is the state after the last step, before the epilogue (which
 *     touches only out).
 * workspace NULL: the library's own workspace, as gtr_gla_fwd. Otherwise a
 * caller-managed one, as gtr_gla_fwd_ws (size from gtr_gla_workspace_bytes,
 * which does not depend on the additions).
 */
int gtr_gla_fwd_ex(const void* q, const void* k, const void* v, const void* log_gamma,
                   const float* initial_state, const void* gate, const float* norm_weight,
                   float norm_eps, int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                   int dir, int chunk, int is_fp32, void* out, float* final_state,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gtr_gla_fwd_lowrank -- gtr_gla_fwd_ex with the gate computed from the input
 * instead of passed in: the data-dependent low-rank gate of the summary page,
 * section 核心方法, gamma_t = sigmoid(x_t W1 W2 + b)^(1/tau), read as
 *     log_gamma_t = inv_tau * log sigmoid(x_t W1 W2 + gate_bias),
 * per head h the columns h*d_k .. h*d_k + d_k - 1 of the H*d_k products.
 *   x         [B, L, C]   the token features the gate is projected from
 *                         (fp16, or fp32 when is_fp32), token order as q.
 *   w1        [C, 16]     fp32, the rank-16 down projection (C >= 1).
 *   w2        [16, H*d_k] fp32, the up projection.
 *   gate_bias [H*d_k]     fp32.
 *   inv_tau   1/tau, finite and > 0 (the pages use tau = 16); else
 *             GTR_GLA_ERR_VALUE.
 * x W1 is computed once per token in fp32 into the workspace; the fused
 * kernels form log_gamma inside the chunk from it (x W1) W2 on fp32 MFMA and
 * never write it to memory, the generic kernels read it from the workspace.
 * None of the four may overlap an output (GTR_GLA_ERR_ALIAS).
 * workspace NULL: the library's own; otherwise at least
 * gtr_gla_lowrank_workspace_bytes, cleared once by gtr_gla_workspace_init.
 */
int gtr_gla_fwd_lowrank(const void* q, const void* k, const void* v, const void* x,
                        const float* w1, const float* w2, const float* gate_bias, float inv_tau,
                        int C, const float* initial_state, const void* gate,
                        const float* norm_weight, float norm_eps, int B, int H, int grid_h,
                        int grid_w, int d_k, int d_v, int dir, int chunk, int is_fp32, void* out,
                        float* final_state, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);
size_t gtr_gla_lowrank_workspace_bytes(int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                                       int chunk, int is_fp32);

size_t gtr_gla_workspace_bytes(int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                               int chunk, int is_fp32);
int gtr_gla_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);
int gtr_gla_fwd_ws(const void* q, const void* k, const void* v, const void* log_gamma,
                   int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                   int dir, int chunk, void* out, float* final_state,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);
int gtr_gla_fwd_f32_ws(const float* q, const float* k, const float* v, const float* log_gamma,
                       int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                       int dir, int chunk, float* out, float* final_state,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gtr_gla_fwd_noalloc -- gtr_gla_fwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, layouts, semantics and errors as
 * gtr_gla_fwd; it allocates nothing (no hipMalloc, hipFree or allocating
 * library call). Its workspace is a static device array of
 * GTR_GLA_NOALLOC_SCRATCH_BYTES bytes per GPU (held until the process ends),
 * cleared by a kernel on its first use and whenever the exchange layout
 * changes. A call whose workspace would be larger returns
 * GTR_GLA_ERR_SCRATCH and launches nothing (gtr_gla_workspace_bytes of the
 * call, with is_fp32 = 0, gives the size). Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (different streams, or different
 * host threads without ordering) race and must not be issued. The first call
 * on each device looks the array's address up on that device; it may be
 * captured in a HIP graph once a call of the same shape has run eagerly.
 * gtr_gla_workspace_status(NULL, 0, stream) also checks this scratch.
 */
#define GTR_GLA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int gtr_gla_fwd_noalloc(const void* q, const void* k, const void* v, const void* log_gamma,
                        int B, int H, int grid_h, int grid_w, int d_k, int d_v, int dir,
                        int chunk, void* out, float* final_state, hipStream_t stream);

/*
 * gtr_gla_workspace_status -- outside the hot path: waits for `stream`, reads
 * and clears the error word of a workspace (NULL: every workspace the library
 * owns for the current device and this stream, and the device's
 * gtr_gla_fwd_noalloc scratch), and re-initialises a workspace
 * whose word was set, so that the next call starts clean. Returns GTR_GLA_OK,
 * GTR_GLA_ERR_EXCHANGE (some fused call on it since the last check gave up in
 * its exchange; that call's outputs are NaN), GTR_GLA_ERR_WS_STATE (some fused
 * call found the workspace uninitialised, written by something else, or last
 * used by calls of another layout, e.g. a captured graph replayed after an
 * eager call of another shape on the same workspace; its outputs are NaN), or
 * GTR_GLA_ERR_HIP / GTR_GLA_ERR_WORKSPACE (workspace_bytes < 256).
 * A workspace is never trusted blindly: its first 256 bytes are a header
 * (error word, layout) that every fused launch checks before it uses the rest.
 */
int gtr_gla_workspace_status(void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gtr_gla_set_exchange_wait -- process-wide, read at each fused launch: the
 * longest time, in microseconds (1 .. 10^7; default 20000), that one wait of a
 * fused kernel's boundary exchange may take before the call gives up (see
 * gtr_gla_fwd). `fault` is a test hook of the give-up path and must be 0 in
 * use: nonzero makes the first span of every sequence publish nothing, so
 * that every fused call gives up after `wait_us`.
 */
int gtr_gla_set_exchange_wait(unsigned int wait_us, int fault);

/*
 * Policy control, for A/B measurement and tests. The setting is process-wide
 * and read at each call; it is not synchronised with calls running on other
 * host threads. A policy that cannot serve a call (fused with fp32 inputs, or
 * with d_v other than 64 or d_k other than 32 and 64) falls back to the
 * generic kernels, as the
 * pages' specialised operator falls back to a generic implementation
 * (summary page, section 局限与改进).
 */
int gtr_gla_set_policy(int policy);
int gtr_gla_get_policy(void);

/*
 * gtr_gla_plan -- describes the launch a call with these arguments would make
 * under the current policy, without launching anything. Any output pointer
 * may be NULL. kernel_out: 1 generic; 2 fused (one-chunk, parked or streamed
 * spans) and 3 fused with register-kept spans; 4 the span kernels (spans of
 * 1..7 chunks, outputs kept in registers through the exchange), the default
 * for d_k = 32, and for d_k = 64 when each sequence takes at most 16 spans
 * (many short sequences); the environment variable GTR_GLA_KERNEL = 2 takes
 * them for every d_k = 64 call, 1 takes kernels 2 and 3 for both key widths.
 * span_out: chunks per workgroup (fused) or 1. grid_out: workgroups of the
 * main kernel (of one launch, when the sequences need several).
 */
int gtr_gla_plan(int B, int H, int grid_h, int grid_w, int d_k, int d_v, int chunk,
                 int is_fp32, int* kernel_out, int* span_out, int* grid_out);
/* gtr_gla_plan_lowrank -- the same for gtr_gla_fwd_lowrank, whose fused
 * kernels hold the gate's tables in LDS as well (fewer may be resident).   */
int gtr_gla_plan_lowrank(int B, int H, int grid_h, int grid_w, int d_k, int d_v, int chunk,
                         int is_fp32, int* kernel_out, int* span_out, int* grid_out);

/* Static description of a status code. Never NULL. */
const char* gtr_gla_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* GTR_GLA_H */
