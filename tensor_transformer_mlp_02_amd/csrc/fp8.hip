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
constexpr int MAX_BLOCKS = 512;  // one amax update per workgroup

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void unpack8(const u32x4_t v, float f[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = __uint_as_float(w[k] << 16);
    f[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}

// Row-major: q[i] = code(x[i]).  A thread converts QU pieces of 8 elements
// per pass, 256 pieces apart (a workgroup covers QU x 4 KiB of x
// contiguously); all QU loads are issued before the first convert, so 128
// bytes per thread are in flight.  Loads are non-temporal (every input byte
// is read once); the codes are stored through the caches, where the GEMM
// that reads them next finds them.
constexpr int QU = 8;
template <int FMT>
__global__ __launch_bounds__(NT) void quantize_kernel(const bf16_t* x, int64_t n8,
                                                      const float* scale, uint8_t* q,
                                                      float* amax) {
  __shared__ float red[NT / 64];
  const float s = *scale;
  float m = 0.f;
  const int64_t pass = (int64_t)gridDim.x * NT * QU;
  for (int64_t base = (int64_t)blockIdx.x * NT * QU + threadIdx.x; base < n8; base += pass) {
    u32x4_t v[QU];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int64_t i = base + (int64_t)u * NT;
      v[u] = (u32x4_t){0u, 0u, 0u, 0u};
      if (i < n8) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + 8 * i));
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int64_t i = base + (int64_t)u * NT;
      float f[8];
      unpack8(v[u], f);
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(f[k]));
      if (i < n8) {
        const u32x2_t o = {fp8x4<FMT>(f[0], f[1], f[2], f[3], s),
                           fp8x4<FMT>(f[4], f[5], f[6], f[7], s)};
        *reinterpret_cast<u32x2_t*>(q + 8 * i) = o;
      }
    }
  }
  if (amax) fold_amax_block<NT>(m, amax, red);
}

// Transposed forms work on blocks of 64 rows x 256 columns: the block's
// codes are staged row-major in shared memory (rows padded to 268 bytes),
// then thread t takes column group t / 4 (4 columns) and row group t % 4
// (16 rows): 16 four-byte reads, a 4 x 4 byte transpose per 4 rows, and a
// 16-byte store per column, so the 4 threads of a column write its 64
// codes contiguously.  rows is a multiple of 16, cols of 8.
constexpr int TB_R = 64, TB_C = 256, TB_PITCH = 268;

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xffu; }

__device__ __forceinline__ void store_block_t(const uint8_t* tile, uint8_t* out, int64_t rows,
                                              int64_t cols, int64_t r0, int64_t c0) {
  const int qg = threadIdx.x >> 2, g = threadIdx.x & 3;
  uint32_t w[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    w[j] = *reinterpret_cast<const uint32_t*>(tile + (16 * g + j) * TB_PITCH + 4 * qg);
  const int64_t r = r0 + 16 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t c = c0 + 4 * qg + i;
    if (c < cols && r < rows) {
      uint32_t o[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        o[b] = byte_of(w[4 * b], i) | (byte_of(w[4 * b + 1], i) << 8) |
               (byte_of(w[4 * b + 2], i) << 16) | (byte_of(w[4 * b + 3], i) << 24);
      const u32x4_t v = {o[0], o[1], o[2], o[3]};
      *reinterpret_cast<u32x4_t*>(out + c * rows + r) = v;
    }
  }
}

// transposed quantize: q[c, r] = code(x[r, c]); a thread loads 8 pieces of
// 8 elements of the block (128 bytes in flight), converts them to codes in
// registers and stages the codes
template <int FMT>
__global__ __launch_bounds__(NT) void quantize_t_kernel(const bf16_t* x, int64_t rows,
                                                        int64_t cols, const float* scale,
                                                        uint8_t* q, float* amax) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[TB_R * TB_PITCH];
  __shared__ float red[NT / 64];
  const float s = *scale;
  const int64_t blocks_c = (cols + TB_C - 1) / TB_C;
  const int64_t blocks = ((rows + TB_R - 1) / TB_R) * blocks_c;
  float m = 0.f;
  for (int64_t b = blockIdx.x; b < blocks; b += gridDim.x) {
    const int64_t r0 = (b / blocks_c) * TB_R, c0 = (b % blocks_c) * TB_C;
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = threadIdx.x + NT * u, rr = j >> 5, k = j & 31;
      const int64_t r = r0 + rr, c = c0 + 8 * k;
      v[u] = (u32x4_t){0u, 0u, 0u, 0u};
      if (r < rows && c < cols)
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + r * cols + c));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = threadIdx.x + NT * u, rr = j >> 5, k = j & 31;
      float f[8];
      unpack8(v[u], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f[e]));
      uint32_t* d = reinterpret_cast<uint32_t*>(tile + rr * TB_PITCH + 8 * k);
      d[0] = fp8x4<FMT>(f[0], f[1], f[2], f[3], s);
      d[1] = fp8x4<FMT>(f[4], f[5], f[6], f[7], s);
    }
    __syncthreads();
    store_block_t(tile, q, rows, cols, r0, c0);
    // the tile is rewritten by the next block
    __syncthreads();
  }
  if (amax) fold_amax_block<NT>(m, amax, red);
}

__global__ void zero_kernel(float* p) { *p = 0.0f; }

// out[c, r] = in[r, c] for bytes (rows and cols multiples of 16): a thread
// loads 4 pieces of 16 bytes of the block (64 bytes in flight)
__global__ __launch_bounds__(NT) void byte_transpose_kernel(const uint8_t* in, int64_t rows,
                                                            int64_t cols, uint8_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[TB_R * TB_PITCH];
  const int64_t blocks_c = (cols + TB_C - 1) / TB_C;
  const int64_t blocks = ((rows + TB_R - 1) / TB_R) * blocks_c;
  for (int64_t b = blockIdx.x; b < blocks; b += gridDim.x) {
    const int64_t r0 = (b / blocks_c) * TB_R, c0 = (b % blocks_c) * TB_C;
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = threadIdx.x + NT * u, rr = j >> 4, k = j & 15;
      const int64_t r = r0 + rr, c = c0 + 16 * k;
      v[u] = (u32x4_t){0u, 0u, 0u, 0u};
      if (r < rows && c < cols)
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(in + r * cols + c));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = threadIdx.x + NT * u, rr = j >> 4, k = j & 15;
      uint32_t* d = reinterpret_cast<uint32_t*>(tile + rr * TB_PITCH + 16 * k);
      d[0] = v[u].x;
      d[1] = v[u].y;
      d[2] = v[u].z;
      d[3] = v[u].w;
    }
    __syncthreads();
    store_block_t(tile, out, rows, cols, r0, c0);
    __syncthreads();
  }
}

// Delayed scaling: one thread per tensor shifts its amax history row one
// place (the oldest value drops out), puts this step's amax at the front and
// clears it for the next step's atomic max, then derives the next scale from
// the largest finite positive value of the window (kept when there is none).
// Every operation is one correctly rounded fp32 operation.
__global__ __launch_bounds__(NT) void scale_update_kernel(int n, int len, float fmax, float mult,
                                                          float* history, float* amax,
                                                          float* scale, float* scale_inv) {
  const int t = blockIdx.x * NT + threadIdx.x;
  if (t >= n) return;
  float* h = history + (int64_t)t * len;
  const float a = amax[t];
  float m = (__builtin_isfinite(a) && a > 0.0f) ? a : 0.0f;
  for (int j = len - 1; j > 0; --j) {
    const float v = h[j - 1];
    h[j] = v;
    if (__builtin_isfinite(v) && v > m) m = v;
  }
  h[0] = a;
  amax[t] = 0.0f;
  float s = scale[t];
  if (m > 0.0f) {
    s = (fmax / m) * mult;
    scale[t] = s;
  }
  if (scale_inv) scale_inv[t] = 1.0f / s;
}

}  // namespace f8q

hipError_t fp8_scale_update_launch(int fmt, int n, int len, int margin, float* history,
                                   float* amax, float* scale, float* scale_inv,
                                   hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const float fmax = fmt == 0 ? 448.0f : 57344.0f;
  const float mult = ldexpf(1.0f, -margin);
  hipLaunchKernelGGL(f8q::scale_update_kernel, dim3((unsigned)((n + f8q::NT - 1) / f8q::NT)),
                     dim3(f8q::NT), 0, stream, n, len, fmax, mult, history, amax, scale,
                     scale_inv);
  return hipGetLastError();
}

hipError_t fp8_quantize_launch(int fmt, bool transpose, int64_t rows, int64_t cols,
                               const void* x, const float* scale, void* q, float* amax,
                               hipStream_t stream) {
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  const bf16_t* xb = reinterpret_cast<const bf16_t*>(x);
  uint8_t* qb = reinterpret_cast<uint8_t*>(q);
  if (!transpose) {
    const int64_t n8 = n / 8;
    int64_t blocks = (n8 + f8q::NT * f8q::QU - 1) / (f8q::NT * f8q::QU);
    if (blocks > f8q::MAX_BLOCKS) blocks = f8q::MAX_BLOCKS;
    if (fmt == 0)
      hipLaunchKernelGGL(f8q::quantize_kernel<0>, dim3((unsigned)blocks), dim3(f8q::NT), 0,
                         stream, xb, n8, scale, qb, amax);
    else
      hipLaunchKernelGGL(f8q::quantize_kernel<1>, dim3((unsigned)blocks), dim3(f8q::NT), 0,
                         stream, xb, n8, scale, qb, amax);
  } else {
    int64_t blocks = ((rows + f8q::TB_R - 1) / f8q::TB_R) * ((cols + f8q::TB_C - 1) / f8q::TB_C);
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
  int64_t tiles = ((rows + f8q::TB_R - 1) / f8q::TB_R) * ((cols + f8q::TB_C - 1) / f8q::TB_C);
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
