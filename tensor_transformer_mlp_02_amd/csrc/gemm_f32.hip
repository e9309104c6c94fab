// fp32 GEMM (plain fp32 fused multiply-add, fp32 accumulate) with the same
// fused epilogues as the bf16 path.  Used when the shard's storage type is
// fp32.  Block tile 64 x 64 x 16, 256 threads, 4 x 4 outputs per thread;
// both operand tiles are staged in shared memory k-major ([k][m], [k][n]).
// For the SwiGLU forward the block keeps two accumulator sets (gate and up
// projections of the same 64 columns), so the epilogue sees both.
#include "common.h"
#include "launch.h"

namespace tpmlp {
namespace f32tile {

constexpr int BM = 64, BN = 64, BK = 16, NT = 256;

// One element (row, col) of a dZ operand formed from dH (pitch ld) and the
// saved activations (Z, pitch split; or G|U, pitch 2 split): column col of
// [dG | dU] reads dH and G at col mod split.
template <int PRO>
__device__ __forceinline__ float dact_f32(const float* dh, const float* zs, int64_t ld,
                                          int64_t split, int64_t row, int64_t col) {
  const bool second = PRO == DACT_SWIGLU && col >= split;
  const int64_t f = second ? col - split : col;
  const int64_t zld = PRO == DACT_SWIGLU ? 2 * split : split;
  const float u = (PRO == DACT_SWIGLU && !second) ? zs[row * zld + split + f] : 0.0f;
  return dact_elem<PRO>(dh[row * ld + f], zs[row * zld + f], u, second);
}

// PA / PB (DACT_*): opA (K-contiguous) or opB (M/N-contiguous) is a dZ
// formed from dH and the saved activations (p0, p1, split of its operand
// arguments) as it is loaded.
template <bool A_KMAJOR, bool B_KMAJOR, int BMODE, bool DUAL, int EPI, int PA = DACT_NONE,
          int PB = DACT_NONE>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs g) {
  static_assert(PA == DACT_NONE || A_KMAJOR, "dZ as K-contiguous opA");
  static_assert(PB == DACT_NONE || !B_KMAJOR, "dZ as M/N-contiguous opB");
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  __shared__ float Bu[DUAL ? BK : 1][DUAL ? BN + 4 : 1];

  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const TileCoord tc = locate_tile(g, blockIdx.x, gridDim.x, BM);
  const float* a0 = reinterpret_cast<const float*>(g.a.p0) + tc.e * g.a.bstride;
  const float* b0 = reinterpret_cast<const float*>(g.b.p0) + tc.e * g.b.bstride;
  const float* b1 = reinterpret_cast<const float*>(g.b.p1) + tc.e * g.b.bstride;
  const int n_base = tc.tn * BN;
  const int n_lim = DUAL ? (int)g.b.split : g.N;

  float acc[4][4], accu[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) { acc[i][j] = 0.0f; accu[i][j] = 0.0f; }

  for (int k0 = tc.k_begin; k0 < tc.k_end; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int idx = tid + NT * i;
      int m, k;
      if (A_KMAJOR) { m = idx >> 4; k = idx & 15; } else { k = idx >> 6; m = idx & 63; }
      int gm = tc.m_begin + m, gk = k0 + k;
      float v = 0.0f;
      if (gm < tc.m_end && gk < tc.k_end) {
        if constexpr (PA != DACT_NONE)
          v = dact_f32<PA>(a0, reinterpret_cast<const float*>(g.a.p1), g.a.ld, g.a.split, gm, gk);
        else
          v = A_KMAJOR ? a0[(int64_t)gm * g.a.ld + gk] : a0[(int64_t)gk * g.a.ld + gm];
      }
      As[k][m] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int idx = tid + NT * i;
      int n, k;
      if (B_KMAJOR) { n = idx >> 4; k = idx & 15; } else { k = idx >> 6; n = idx & 63; }
      int gn = n_base + n, gk = k0 + k;
      float v = 0.0f, u = 0.0f;
      if (gn < n_lim && gk < tc.k_end) {
        if (B_KMAJOR) {
          if (BMODE == BMODE_KSPLIT && gk >= g.b.split)
            v = b1[(int64_t)gn * g.b.ld + (gk - g.b.split)];
          else
            v = b0[(int64_t)gn * g.b.ld + gk];
        } else if constexpr (PB != DACT_NONE) {
          v = dact_f32<PB>(b0, b1, g.b.ld, g.b.split, gk, gn);
        } else {
          v = b0[(int64_t)gk * g.b.ld + gn];
          if (DUAL) u = b1[(int64_t)gk * g.b.ld + gn];
        }
      }
      Bs[k][n] = v;
      if (DUAL) Bu[k][n] = u;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4], bu[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j] = Bs[kk][tx * 4 + j];
        if (DUAL) bu[j] = Bu[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (DUAL) accu[i][j] = fmaf(a[i], bu[j], accu[i][j]);
        }
    }
    __syncthreads();
  }

  const int64_t n = n_base + tx * 4;
  if (n >= n_lim) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = tc.m_begin + ty * 4 + i;
    if (m >= tc.m_end) continue;
    if constexpr (DUAL) {
      epilogue_swiglu4<float>(g.epi, m, n, acc[i], accu[i]);
    } else {
      epilogue4<EPI, float, float>(g.epi, tc.e, m, n, acc[i]);
    }
  }
}

}  // namespace f32tile

static void fill_tiles_f32(GemmArgs& g, int n_cols) {
  using namespace f32tile;
  g.tiles_n = (n_cols + BN - 1) / BN;
  g.tile_off[0] = 0;
  for (int e = 0; e < g.E; ++e) {
    int rows = (g.ragged == RAGGED_M) ? g.row_off[e + 1] - g.row_off[e] : g.M;
    g.tile_off[e + 1] = g.tile_off[e] + ((rows + BM - 1) / BM) * g.tiles_n;
  }
}

template <bool AK, bool BK_, int BMODE, bool DUAL, int EPI, int PA = DACT_NONE,
          int PB = DACT_NONE>
static hipError_t launch_f32(GemmArgs& g, hipStream_t stream) {
  if ((PA != DACT_NONE || PB != DACT_NONE) &&
      (g.E != 1 || g.ragged != RAGGED_NONE || g.a.bstride || g.b.bstride))
    return hipErrorInvalidValue;  // the formed operand: dense problems only
  fill_tiles_f32(g, DUAL ? (int)g.b.split : g.N);
  int blocks = g.tile_off[g.E];
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((f32tile::gemm_kernel<AK, BK_, BMODE, DUAL, EPI, PA, PB>),
                     dim3(blocks), dim3(f32tile::NT), 0, stream, g);
  return hipGetLastError();
}

hipError_t gemm_f32(GemmKind kind, GemmArgs& g, hipStream_t stream) {
  switch (kind) {
    case GK_FC1_GELU:
      return launch_f32<true, false, BMODE_PLAIN, false, EPI_GELU_FWD>(g, stream);
    case GK_FC1_SWIGLU:
      return launch_f32<true, false, BMODE_PLAIN, true, EPI_SWIGLU_FWD>(g, stream);
    case GK_FC2:
      return launch_f32<true, false, BMODE_PLAIN, false, EPI_STORE>(g, stream);
    case GK_DH_GELU:
      return launch_f32<true, true, BMODE_PLAIN, false, EPI_GELU_BWD>(g, stream);
    case GK_DH_SWIGLU:
      return launch_f32<true, true, BMODE_PLAIN, false, EPI_SWIGLU_BWD>(g, stream);
    case GK_WGRAD:
      return launch_f32<false, false, BMODE_PLAIN, false, EPI_STORE>(g, stream);
    case GK_WGRAD_SPLIT:
      return launch_f32<false, false, BMODE_PLAIN, false, EPI_STORE_SPLIT>(g, stream);
    case GK_DX:
      return launch_f32<true, true, BMODE_PLAIN, false, EPI_STORE>(g, stream);
    case GK_DX_KSPLIT:
      return launch_f32<true, true, BMODE_KSPLIT, false, EPI_STORE>(g, stream);
    case GK_WGRAD_ACC:
      return launch_f32<false, false, BMODE_PLAIN, false, EPI_ACC>(g, stream);
    case GK_WGRAD_SPLIT_ACC:
      return launch_f32<false, false, BMODE_PLAIN, false, EPI_ACC_SPLIT>(g, stream);
    case GK_WGRAD_DACT_GELU:
      return launch_f32<false, false, BMODE_PLAIN, false, EPI_STORE, DACT_NONE, DACT_GELU>(g, stream);
    case GK_WGRAD_SPLIT_DACT_SWIGLU:
      return launch_f32<false, false, BMODE_PLAIN, false, EPI_STORE_SPLIT, DACT_NONE, DACT_SWIGLU>(
          g, stream);
    case GK_DX_DACT_GELU:
      return launch_f32<true, true, BMODE_PLAIN, false, EPI_STORE, DACT_GELU>(g, stream);
    case GK_DX_KSPLIT_DACT_SWIGLU:
      return launch_f32<true, true, BMODE_KSPLIT, false, EPI_STORE, DACT_SWIGLU>(g, stream);
    default:
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
