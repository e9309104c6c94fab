// Partial-output sum over T shard outputs resident in one GPU's memory:
// out = sum_{i<T} P_i, summed in fp32 in the fixed order i = 0..T-1 and
// rounded once.  Bandwidth-bound: every byte is read or written once.
//
// A workgroup owns U x 256 consecutive chunks of 8 elements (16 bytes of
// bf16, 32 bytes of fp32) per pass, a thread U of them, 256 chunks apart
// (U = 4 for bf16, 2 for fp32: 64 bytes of each partial per thread either
// way): a wavefront's loads cover 1 KiB contiguous per instruction and a
// workgroup reads one contiguous 16 KiB range of each partial, which the
// memory system serves faster than ranges spread a grid-width apart (8
// bf16 partials of 64 MiB on MI355X: 5.96 TB/s, against 5.76 for 8 KiB
// ranges and 5.2 spread apart).  The partials are taken in groups of PS_G:
// all PS_G x U loads of a group are issued before the first add, which
// keeps 512 bytes per lane in flight; the adds then run in partial order.  The grid strides over the chunks, so any workgroup count covers
// the whole tensor (the capped variant runs on a few compute units beside
// other kernels).  The T partial pointers travel by value.
#include "common.h"
#include "launch.h"

namespace tpmlp {

struct PartialPtrs {
  const void* p[TP_MAX_SHARDS];
};

constexpr int PS_NT = 256;
constexpr int PS_G = 8;  // partials whose loads are in flight together
// chunks per thread per pass
template <typename T> struct PsU { static constexpr int value = sizeof(T) == 2 ? 4 : 2; };

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// one chunk of 8 elements as loaded (raw bits; converted when added).
// Loads and stores are non-temporal: every byte is touched once.
template <typename T> struct Chunk;
template <> struct Chunk<bf16_t> {
  u32x4_t q;
  __device__ __forceinline__ void load(const bf16_t* p, int64_t c) {
    q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + c * 8));
  }
  __device__ __forceinline__ void get(float v[8]) const {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Chunk<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p, int64_t c) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + c * 8));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + c * 8 + 4));
  }
  __device__ __forceinline__ void get(float v[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

__device__ __forceinline__ void store8(bf16_t* p, int64_t c, const float v[8]) {
  u32x4_t q;
  q.x = pack_bf16x2(v[0], v[1]);
  q.y = pack_bf16x2(v[2], v[3]);
  q.z = pack_bf16x2(v[4], v[5]);
  q.w = pack_bf16x2(v[6], v[7]);
  __builtin_nontemporal_store(q, reinterpret_cast<u32x4_t*>(p + c * 8));
}
__device__ __forceinline__ void store8(float* p, int64_t c, const float v[8]) {
  const f32x4_t a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t*>(p + c * 8));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4_t*>(p + c * 8 + 4));
}
__device__ __forceinline__ float load1(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float load1(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void store1(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ void store1(float* p, int64_t i, float v) { p[i] = v; }

// The sum over the chunks a grid of workgroups covers (U chunks per thread
// per pass; see the file comment).
template <typename T, int PS_U>
__device__ __forceinline__ void partial_sum_body(const PartialPtrs& ptrs, int nparts,
                                                 int64_t nchunks, int64_t count, void* out_) {
  T* out = reinterpret_cast<T*>(out_);
  constexpr int64_t stride = PS_NT;  // between a thread's chunks
  const int64_t pass = (int64_t)gridDim.x * PS_NT * PS_U;
  for (int64_t base = (int64_t)blockIdx.x * PS_NT * PS_U + threadIdx.x; base < nchunks;
       base += pass) {
    float s[PS_U][8];
    bool ok[PS_U];
#pragma unroll
    for (int u = 0; u < PS_U; ++u) ok[u] = base + u * stride < nchunks;
    for (int g0 = 0; g0 < nparts; g0 += PS_G) {
      Chunk<T> raw[PS_G][PS_U];
#pragma unroll
      for (int i = 0; i < PS_G; ++i) {
        if (g0 + i < nparts) {
          const T* p = reinterpret_cast<const T*>(ptrs.p[g0 + i]);
#pragma unroll
          for (int u = 0; u < PS_U; ++u)
            if (ok[u]) raw[i][u].load(p, base + u * stride);
        }
      }
#pragma unroll
      for (int i = 0; i < PS_G; ++i) {
        if (g0 + i < nparts) {
#pragma unroll
          for (int u = 0; u < PS_U; ++u) {
            float v[8];
            raw[i][u].get(v);
            if (g0 + i == 0) {
#pragma unroll
              for (int e = 0; e < 8; ++e) s[u][e] = v[e];
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) s[u][e] += v[e];
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < PS_U; ++u)
      if (ok[u]) store8(out, base + u * stride, s[u]);
  }
  // elements past the last whole chunk
  if (blockIdx.x == 0) {
    int64_t i = nchunks * 8 + threadIdx.x;
    if (i < count) {
      float s = load1(reinterpret_cast<const T*>(ptrs.p[0]), i);
      for (int k = 1; k < nparts; ++k) s += load1(reinterpret_cast<const T*>(ptrs.p[k]), i);
      store1(out, i, s);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(PS_NT) void partial_sum_kernel(PartialPtrs ptrs, int nparts,
                                                            int64_t nchunks, int64_t count,
                                                            void* out) {
  partial_sum_body<T, PsU<T>::value>(ptrs, nparts, nchunks, count, out);
}

// The capped sum runs beside GEMMs on another stream.  A GEMM wavefront
// holds at most 416 of the 512 registers per lane of its SIMD, so a
// wavefront of this kernel (one chunk per thread per pass, at most 88
// registers) fits beside it: the sum shares SIMDs with the GEMM's
// wavefronts instead of holding compute units the GEMM's workgroups wait
// for.  Same order of additions, same results as partial_sum_kernel.
constexpr int PS_NARROW_VGPRS = 88;
template <typename T>
__global__ __launch_bounds__(PS_NT) __attribute__((amdgpu_num_vgpr(PS_NARROW_VGPRS)))
void partial_sum_narrow_kernel(PartialPtrs ptrs, int nparts, int64_t nchunks, int64_t count,
                               void* out) {
  partial_sum_body<T, 1>(ptrs, nparts, nchunks, count, out);
}

hipError_t partial_sum_launch(int dtype, int T, const void* const* parts, int64_t count,
                              void* out, int max_blocks, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  PartialPtrs ptrs;
  for (int i = 0; i < TP_MAX_SHARDS; ++i) ptrs.p[i] = i < T ? parts[i] : nullptr;
  const int64_t nchunks = count / 8;
  const bool narrow = max_blocks > 0;
  const int per_block =
      PS_NT * (narrow ? 1 : (dtype == TP_BF16 ? PsU<bf16_t>::value : PsU<float>::value));
  int64_t blocks = (nchunks + per_block - 1) / per_block;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  if (narrow && blocks > max_blocks) blocks = max_blocks;
  const dim3 grid((unsigned)blocks), block(PS_NT);
  if (dtype == TP_BF16) {
    if (narrow)
      hipLaunchKernelGGL(partial_sum_narrow_kernel<bf16_t>, grid, block, 0, stream, ptrs, T,
                         nchunks, count, out);
    else
      hipLaunchKernelGGL(partial_sum_kernel<bf16_t>, grid, block, 0, stream, ptrs, T, nchunks,
                         count, out);
  } else {
    if (narrow)
      hipLaunchKernelGGL(partial_sum_narrow_kernel<float>, grid, block, 0, stream, ptrs, T,
                         nchunks, count, out);
    else
      hipLaunchKernelGGL(partial_sum_kernel<float>, grid, block, 0, stream, ptrs, T, nchunks,
                         count, out);
  }
  return hipGetLastError();
}

}  // namespace tpmlp
