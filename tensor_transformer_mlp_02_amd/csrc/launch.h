// Host-side launchers shared between the entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace tpmlp {

// The GEMMs of one shard's forward and backward.
enum GemmKind {
  GK_FC1_GELU,     // Z = X A; epilogue: save Z, H = gelu(Z)
  GK_FC1_SWIGLU,   // [G|U] = X [Ag|Au]; epilogue: save G|U, H = silu(G) U
  GK_FC2,          // Y_partial = H B
  GK_DH_GELU,      // dZ = (dY B^T) * gelu'(Z)
  GK_DH_SWIGLU,    // [dG|dU] from dH = dY B^T and the saved G|U
  GK_WGRAD,        // dW = L^T R  (both operands M/N-contiguous), fp32 out
  GK_WGRAD_SPLIT,  // as GK_WGRAD with the columns split over two outputs
  GK_DX,           // dX_partial = dZ A^T
  GK_DX_KSPLIT,    // dX_partial = [dG|dU] [Ag|Au]^T
  GK_WGRAD_ACC,        // dW += L^T R  (fp32 accumulation buffer)
  GK_WGRAD_SPLIT_ACC,  // as GK_WGRAD_SPLIT, adding into both outputs
  // The activation derivative formed as an operand is loaded (the other
  // placement of the derivative): that operand's p0 is dH [rows, split]
  // (pitch ld), p1 the forward's saved Z (GeLU, pitch split) or G|U
  // (SwiGLU, pitch 2 split), split = F_shard; each 8-element piece of dZ
  // (GeLU) or [dG|dU] (SwiGLU) is computed from them on its way to shared
  // memory.
  GK_WGRAD_DACT_GELU,          // dA = X^T (dH * gelu'(Z)), opB formed
  GK_WGRAD_SPLIT_DACT_SWIGLU,  // dA | dA_up = X^T [dG|dU], opB formed
  GK_DX_DACT_GELU,             // dX_partial = (dH * gelu'(Z)) A^T, opA formed
  GK_DX_KSPLIT_DACT_SWIGLU,    // dX_partial = [dG|dU] [Ag|Au]^T, opA formed
  GK_FC1_SWIGLU_F8,    // FP8: [G|U] = Xq [Agq|Auq]^T scaled; SwiGLU; H, Hq, amax
  GK_FC1_GELU_F8,      // FP8: Z = Xq Aq^T scaled; GeLU; H, Hq, amax
  GK_FC2_F8,           // FP8: Y = Hq Bq^T scaled
  GK_DH_GELU_F8,       // FP8 bwd: dZq = code(gelu'(Z) * dYq Bq^T scaled), amax
  GK_DH_SWIGLU_F8,     // FP8 bwd: [dGq|dUq] from dYq Bq^T and the saved G|U, amax
  GK_WGRAD_F8,         // FP8 bwd: dW = (L^T codes)(R^T codes)^T scaled, fp32 out
  GK_WGRAD_SPLIT_F8,   // as GK_WGRAD_F8, columns split over two outputs
  GK_DX_F8,            // FP8 bwd: dX = dZq Aq^T... scaled, bf16 out
  GK_DX_KSPLIT_F8,     // as GK_DX_F8 with K split over [Aq | Auq]
};

// bf16 storage, MFMA path.
hipError_t gemm_bf16(GemmKind kind, GemmArgs& g, hipStream_t stream);
// fp32 storage, fp32 FMA path.
hipError_t gemm_f32(GemmKind kind, GemmArgs& g, hipStream_t stream);

// max_blocks > 0 caps the grid (the kernel strides over the tensor).
hipError_t partial_sum_launch(int dtype, int T, const void* const* parts, int64_t count,
                              void* out, int max_blocks, hipStream_t stream);

// E4M3 operands, both K-contiguous (GK_*_F8 kinds only)
hipError_t gemm_fp8(GemmKind kind, GemmArgs& g, hipStream_t stream);
hipError_t fp8_quantize_launch(int fmt, bool transpose, int64_t rows, int64_t cols,
                               const void* x, const float* scale, void* q, float* amax,
                               hipStream_t stream);
hipError_t zero_float_launch(float* p, hipStream_t stream);
// amax history [n, len] shift, next scale (and its inverse) per tensor
hipError_t fp8_scale_update_launch(int fmt, int n, int len, int margin, float* history,
                                   float* amax, float* scale, float* scale_inv,
                                   hipStream_t stream);
// bytes [rows, cols] -> [cols, rows]; rows, cols multiples of 16
hipError_t byte_transpose_launch(int64_t rows, int64_t cols, const void* in, void* out,
                                 hipStream_t stream);

hipError_t moe_permute_launch(int dtype, const int32_t* row_token, int64_t N, int64_t H,
                              int64_t R, const void* X, void* Xp, hipStream_t stream);
hipError_t moe_combine_launch(int dtype, const int32_t* tok_ptr, const int32_t* tok_rows,
                              const float* w, int64_t N, int64_t H, int64_t R, const void* Yp,
                              void* Y, hipStream_t stream);
hipError_t moe_combine_bwd_launch(int dtype, const int32_t* row_token, const float* w,
                                  int64_t N, int64_t H, int64_t R, const void* dY,
                                  const void* Yp, void* dYp, float* dw, hipStream_t stream);

}  // namespace tpmlp
