/*
 * gtr_sswiglu.h -- C ABI of libgtrgla's Spatial SwiGLU channel mixer, the
 * second operator of every GTR block (GTR summary page
 * "GTR:门控Token循环实现高效稠密预测", section 前置知识 › SwiGLU前馈块 and
 * section 核心方法): the SwiGLU mixer with a 3x3 depthwise convolution in its
 * value branch,
 *
 *     Y = (SiLU(X W_g^T) ⊙ DWConv3x3(X W_v^T)) W_o^T,    SiLU(z) = z sigma(z),
 *
 * over the tokens of the stride-16 patch grid, on AMD Instinct MI355X (gfx950).
 *
 * Tensors (contiguous, row-major, device memory owned by the caller; fp16 =
 * IEEE binary16, the pages' deployment precision):
 *   x      [B, L, C]   fp16, L = grid_h * grid_w, token p = row * grid_w + col
 *   w_g    [Hd, C]     fp16, linear-layer weight [out, in] of the gate branch
 *   w_v    [Hd, C]     fp16, of the value branch
 *   conv_w [Hd, 3, 3]  fp32, depthwise kernel: out[i][j] = conv_b +
 *                      sum_{a,c} conv_w[a][c] u[i + a - 1][j + c - 1], zero
 *                      outside the grid (cross-correlation, as a framework's
 *                      2-D convolution layer computes it)
 *   conv_b [Hd]        fp32 bias of the convolution, or NULL (none)
 *   w_o    [C, Hd]     fp16, output projection weight [out, in]
 *   y      [B, L, C]   fp16 output, fully overwritten
 * Hd is the hidden width (the pages use 4 C, and 6 C for the largest model).
 * Arithmetic: fp16 MFMA with fp32 accumulation; X W_g and X W_v stay fp32 on
 * chip, the convolution and the gate are fp32, the gated hidden tile is
 * rounded to fp16 once (the workspace) before the output product.
 *
 * Sizes: B, grid_h, grid_w >= 1; C a multiple of 64 and Hd of 128 (C <= 8192,
 * Hd <= 32768); each of x, y and the hidden tensor [B, L, Hd] under 2^31
 * bytes per batch entry (hidden: in total). Else GTR_GLA_ERR_UNSUPPORTED
 * (GTR_GLA_ERR_SHAPE for sizes < 1).
 * Errors and statuses are gtr_gla_status (gtr_gla.h); a call that fails
 * validation launches nothing. y must not overlap any input
 * (GTR_GLA_ERR_ALIAS).
 * Workspace: the gated hidden tensor, B * L * Hd * 2 bytes
 * (gtr_sswiglu_workspace_bytes). workspace NULL: the library's own, allocated
 * on the first call per (device, stream) and grown when needed (call once
 * outside stream capture for a shape before capturing it). Otherwise at least
 * that many bytes, owned by the caller, not overlapping x, y or the weights;
 * no clearing needed. The call is asynchronous on `stream`.
 */
#ifndef GTR_SSWIGLU_H
#define GTR_SSWIGLU_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int gtr_sswiglu_fwd(const void* x, const void* w_g, const void* w_v, const float* conv_w,
                    const float* conv_b, const void* w_o, int B, int grid_h, int grid_w, int C,
                    int Hd, void* y, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Bytes of workspace gtr_sswiglu_fwd needs for these sizes, or 0 if invalid. */
size_t gtr_sswiglu_workspace_bytes(int B, int grid_h, int grid_w, int C, int Hd);

#ifdef __cplusplus
}
#endif

#endif /* GTR_SSWIGLU_H */
