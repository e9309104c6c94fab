// Token dispatch and combine around the grouped local experts: the token
// reordering that brings each token to the experts its router picked, and
// the weighted merge of the experts' outputs back into token order
// (Megatron Core 带读 §09: router -> top-k experts -> tokens sent to their
// experts -> expert compute -> results merged by weight -> combine back in
// the original token order).  All three kernels move rows of H elements and
// are HBM-bound: every row is read and written once, 16 bytes per thread
// access.  The routing tables are device arrays; an index outside its range
// contributes nothing (a permuted row becomes zeros), so no table value can
// send an access out of bounds.
#include "common.h"
#include "launch.h"

namespace tpmlp {
namespace moe {

constexpr int NT = 256;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 8 elements (16 bytes of bf16, 32 of fp32) <-> fp32
template <typename T> struct Row8;
template <> struct Row8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float v[8]) {
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float v[8]) {
    u32x4_t q;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4_t*>(p) = q;
  }
};
template <> struct Row8<float> {
  static __device__ __forceinline__ void load(const float* p, float v[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float v[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// X_perm[r] = X[row_token[r]]  (a straight copy of 16-byte pieces)
template <typename T>
__global__ __launch_bounds__(NT) void permute_kernel(const int32_t* row_token, int64_t N,
                                                     int64_t H, int64_t R, const T* X, T* Xp) {
  const int64_t pieces = H * (int64_t)sizeof(T) / 16;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const int32_t t = row_token[r];
    const bool ok = t >= 0 && t < N;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(X + (ok ? (int64_t)t * H : 0));
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(Xp + r * H);
    for (int64_t c = threadIdx.x; c < pieces; c += NT) {
      const u32x4_t v = ok ? src[c] : u32x4_t{0u, 0u, 0u, 0u};
      dst[c] = v;
    }
  }
}

// Y[t] = sum_{j = tok_ptr[t]}^{tok_ptr[t+1]-1} w[tok_rows[j]] Y_perm[tok_rows[j]]
// in fp32, in list order, rounded once (w = 1 when null)
template <typename T>
__global__ __launch_bounds__(NT) void combine_kernel(const int32_t* tok_ptr,
                                                     const int32_t* tok_rows, const float* w,
                                                     int64_t N, int64_t H, int64_t R,
                                                     const T* Yp, T* Y) {
  const int64_t chunks = H / 8;
  for (int64_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int64_t lo = min(max((int64_t)tok_ptr[t], (int64_t)0), R);
    const int64_t hi = min(max((int64_t)tok_ptr[t + 1], lo), R);
    for (int64_t c = threadIdx.x; c < chunks; c += NT) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int64_t j = lo; j < hi; ++j) {
        const int32_t r = tok_rows[j];
        if (r < 0 || r >= R) continue;
        const float s = w ? w[r] : 1.0f;
        float v[8];
        Row8<T>::load(Yp + (int64_t)r * H + 8 * c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += s * v[e];
      }
      Row8<T>::store(Y + t * H + 8 * c, acc);
    }
  }
}

// dY_perm[r] = w[r] dY[t(r)];  dw[r] = <dY[t(r)], Y_perm[r]> (fp32, fixed
// reduction tree: per-thread partial sums, then the wavefront, then the
// four wavefronts in order)
template <typename T>
__global__ __launch_bounds__(NT) void combine_bwd_kernel(const int32_t* row_token, const float* w,
                                                         int64_t N, int64_t H, int64_t R,
                                                         const T* dY, const T* Yp, T* dYp,
                                                         float* dw) {
  __shared__ float part[NT / 64];
  const int64_t chunks = H / 8;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const int32_t t = row_token[r];
    const bool ok = t >= 0 && t < N;
    const float s = w[r];
    float dot = 0.f;
    for (int64_t c = threadIdx.x; c < chunks; c += NT) {
      // a row whose token is out of range reads nothing and gets zeros (its
      // Y_perm row may never have been written)
      float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, o[8];
      if (ok) {
        Row8<T>::load(dY + (int64_t)t * H + 8 * c, g);
        Row8<T>::load(Yp + r * H + 8 * c, y);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = ok ? s * g[e] : 0.f;
        dot += g[e] * y[e];
      }
      Row8<T>::store(dYp + r * H + 8 * c, o);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = dot;
    __syncthreads();
    if (threadIdx.x == 0) {
      float sum = part[0];
#pragma unroll
      for (int k = 1; k < NT / 64; ++k) sum += part[k];
      dw[r] = sum;
    }
    __syncthreads();
  }
}

static unsigned grid_for(int64_t n) {
  return (unsigned)(n < 1 ? 1 : (n > 8192 ? 8192 : n));
}

}  // namespace moe

hipError_t moe_permute_launch(int dtype, const int32_t* row_token, int64_t N, int64_t H,
                              int64_t R, const void* X, void* Xp, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  if (dtype == TP_BF16)
    hipLaunchKernelGGL(moe::permute_kernel<bf16_t>, dim3(moe::grid_for(R)), dim3(moe::NT), 0,
                       stream, row_token, N, H, R, (const bf16_t*)X, (bf16_t*)Xp);
  else
    hipLaunchKernelGGL(moe::permute_kernel<float>, dim3(moe::grid_for(R)), dim3(moe::NT), 0,
                       stream, row_token, N, H, R, (const float*)X, (float*)Xp);
  return hipGetLastError();
}

hipError_t moe_combine_launch(int dtype, const int32_t* tok_ptr, const int32_t* tok_rows,
                              const float* w, int64_t N, int64_t H, int64_t R, const void* Yp,
                              void* Y, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (dtype == TP_BF16)
    hipLaunchKernelGGL(moe::combine_kernel<bf16_t>, dim3(moe::grid_for(N)), dim3(moe::NT), 0,
                       stream, tok_ptr, tok_rows, w, N, H, R, (const bf16_t*)Yp, (bf16_t*)Y);
  else
    hipLaunchKernelGGL(moe::combine_kernel<float>, dim3(moe::grid_for(N)), dim3(moe::NT), 0,
                       stream, tok_ptr, tok_rows, w, N, H, R, (const float*)Yp, (float*)Y);
  return hipGetLastError();
}

hipError_t moe_combine_bwd_launch(int dtype, const int32_t* row_token, const float* w,
                                  int64_t N, int64_t H, int64_t R, const void* dY,
                                  const void* Yp, void* dYp, float* dw, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  if (dtype == TP_BF16)
    hipLaunchKernelGGL(moe::combine_bwd_kernel<bf16_t>, dim3(moe::grid_for(R)), dim3(moe::NT), 0,
                       stream, row_token, w, N, H, R, (const bf16_t*)dY, (const bf16_t*)Yp,
                       (bf16_t*)dYp, dw);
  else
    hipLaunchKernelGGL(moe::combine_bwd_kernel<float>, dim3(moe::grid_for(R)), dim3(moe::NT), 0,
                       stream, row_token, w, N, H, R, (const float*)dY, (const float*)Yp,
                       (float*)dYp, dw);
  return hipGetLastError();
}

}  // namespace tpmlp
