// Per-tensor FP8 quantization (E4M3 forward operands, E5M2 gradients):
// code = round-to-nearest-even(clamp(x * scale, -max, max)) with gfx950's
// packed converts (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32, OCP formats), and
// amax = max |x| folded into a device float with an integer atomic max on
// its bit pattern (non-negative floats order like their bits), which does
// not depend on the order of the updates.  Weights are quantized into their
// transposes, so every FP8 GEMM operand is K-contiguous.  HBM-bound.
#include "common.h"
#include "launch.h"

namespace tpmlp {
namespace f8q {

constexpr int NT = 256;

// row-major: q[i] = code(x[i]); 8 elements per thread per pass
constexpr int MAX_BLOCKS = 1024;  // one amax update per workgroup

template <int FMT>
__global__ __launch_bounds__(NT) void quantize_kernel(const bf16_t* x, int64_t n8,
                                                      const float* scale, uint8_t* q,
                                                      float* amax) {
  __shared__ float red[NT / 64];
  const float s = *scale;
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n8; i += (int64_t)gridDim.x * NT) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + 8 * i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = __uint_as_float(w[k] << 16);
      f[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(f[k]));
    uint2 o;
    o.x = fp8x4<FMT>(f[0], f[1], f[2], f[3], s);
    o.y = fp8x4<FMT>(f[4], f[5], f[6], f[7], s);
    *reinterpret_cast<uint2*>(q + 8 * i) = o;
  }
  if (amax) fold_amax_block<NT>(m, amax, red);
}

// transposed: q[c, r] = code(x[r, c]) through a 64 x 64 tile in shared
// memory; rows and cols are multiples of 16 and 8
template <int FMT>
__global__ __launch_bounds__(NT) void quantize_t_kernel(const bf16_t* x, int64_t rows,
                                                        int64_t cols, const float* scale,
                                                        uint8_t* q, float* amax) {
  __shared__ float tile[64][65];
  __shared__ float red[NT / 64];
  const float s = *scale;
  const int64_t tiles_c = (cols + 63) / 64;
  const int64_t tiles = ((rows + 63) / 64) * tiles_c;
  float m = 0.f;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
  const int64_t r0 = (t / tiles_c) * 64, c0 = (t % tiles_c) * 64;
  // load: 64 rows x 8 chunks of 8 columns; thread -> (row tid / 8 + 32 p, chunk tid % 8)
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int rr = threadIdx.x / 8 + 32 * p, cc = (threadIdx.x % 8) * 8;
    const int64_t r = r0 + rr, c = c0 + cc;
    float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (r < rows && c < cols) {
      const uint4 v = *reinterpret_cast<const uint4*>(x + r * cols + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f[2 * k] = __uint_as_float(w[k] << 16);
        f[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      tile[rr][cc + k] = f[k];
      m = fmaxf(m, fabsf(f[k]));
    }
  }
  __syncthreads();
  // store: 64 output rows (columns c) x 4 pieces of 16 codes (rows r)
  {
    const int oc = threadIdx.x / 4, orr = (threadIdx.x % 4) * 16;
    const int64_t c = c0 + oc, r = r0 + orr;
    if (c < cols && r < rows) {
      uint4 o;
      o.x = fp8x4<FMT>(tile[orr][oc], tile[orr + 1][oc], tile[orr + 2][oc], tile[orr + 3][oc], s);
      o.y = fp8x4<FMT>(tile[orr + 4][oc], tile[orr + 5][oc], tile[orr + 6][oc], tile[orr + 7][oc], s);
      o.z = fp8x4<FMT>(tile[orr + 8][oc], tile[orr + 9][oc], tile[orr + 10][oc], tile[orr + 11][oc], s);
      o.w = fp8x4<FMT>(tile[orr + 12][oc], tile[orr + 13][oc], tile[orr + 14][oc], tile[orr + 15][oc], s);
      *reinterpret_cast<uint4*>(q + c * rows + r) = o;
    }
  }
  // the tile is rewritten by the next iteration
  __syncthreads();
  }
  if (amax) fold_amax_block<NT>(m, amax, red);
}

__global__ void zero_kernel(float* p) { *p = 0.0f; }

// out[c, r] = in[r, c] for bytes, 64 x 64 tiles through shared memory;
// rows and cols are multiples of 16
__global__ __launch_bounds__(NT) void byte_transpose_kernel(const uint8_t* in, int64_t rows,
                                                            int64_t cols, uint8_t* out) {
  __shared__ uint8_t tile[64][64 + 4];
  const int64_t tiles_c = (cols + 63) / 64;
  const int64_t tiles = ((rows + 63) / 64) * tiles_c;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t r0 = (t / tiles_c) * 64, c0 = (t % tiles_c) * 64;
    {
      const int rr = threadIdx.x / 4, cc = (threadIdx.x % 4) * 16;
      const int64_t r = r0 + rr, c = c0 + cc;
      uint4 v = {0u, 0u, 0u, 0u};
      if (r < rows && c < cols) v = *reinterpret_cast<const uint4*>(in + r * cols + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 16; ++k) tile[rr][cc + k] = (uint8_t)(w[k / 4] >> (8 * (k % 4)));
    }
    __syncthreads();
    {
      const int oc = threadIdx.x / 4, orr = (threadIdx.x % 4) * 16;
      const int64_t c = c0 + oc, r = r0 + orr;
      if (c < cols && r < rows) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 16; ++k) w[k / 4] |= (uint32_t)tile[orr + k][oc] << (8 * (k % 4));
        *reinterpret_cast<uint4*>(out + c * rows + r) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    __syncthreads();
  }
}

}  // namespace f8q

hipError_t fp8_quantize_launch(int fmt, bool transpose, int64_t rows, int64_t cols,
                               const void* x, const float* scale, void* q, float* amax,
                               hipStream_t stream) {
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  const bf16_t* xb = reinterpret_cast<const bf16_t*>(x);
  uint8_t* qb = reinterpret_cast<uint8_t*>(q);
  if (!transpose) {
    const int64_t n8 = n / 8;
    int64_t blocks = (n8 + f8q::NT - 1) / f8q::NT;
    if (blocks > f8q::MAX_BLOCKS) blocks = f8q::MAX_BLOCKS;
    if (fmt == 0)
      hipLaunchKernelGGL(f8q::quantize_kernel<0>, dim3((unsigned)blocks), dim3(f8q::NT), 0,
                         stream, xb, n8, scale, qb, amax);
    else
      hipLaunchKernelGGL(f8q::quantize_kernel<1>, dim3((unsigned)blocks), dim3(f8q::NT), 0,
                         stream, xb, n8, scale, qb, amax);
  } else {
    int64_t blocks = ((rows + 63) / 64) * ((cols + 63) / 64);
    if (blocks > f8q::MAX_BLOCKS) blocks = f8q::MAX_BLOCKS;
    if (fmt == 0)
      hipLaunchKernelGGL(f8q::quantize_t_kernel<0>, dim3((unsigned)blocks), dim3(f8q::NT), 0,
                         stream, xb, rows, cols, scale, qb, amax);
    else
      hipLaunchKernelGGL(f8q::quantize_t_kernel<1>, dim3((unsigned)blocks), dim3(f8q::NT), 0,
                         stream, xb, rows, cols, scale, qb, amax);
  }
  return hipGetLastError();
}

hipError_t byte_transpose_launch(int64_t rows, int64_t cols, const void* in, void* out,
                                 hipStream_t stream) {
  int64_t tiles = ((rows + 63) / 64) * ((cols + 63) / 64);
  if (tiles == 0) return hipSuccess;
  if (tiles > 2048) tiles = 2048;
  hipLaunchKernelGGL(f8q::byte_transpose_kernel, dim3((unsigned)tiles), dim3(f8q::NT), 0, stream,
                     reinterpret_cast<const uint8_t*>(in), rows, cols,
                     reinterpret_cast<uint8_t*>(out));
  return hipGetLastError();
}

hipError_t zero_float_launch(float* p, hipStream_t stream) {
  hipLaunchKernelGGL(f8q::zero_kernel, dim3(1), dim3(1), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tpmlp
