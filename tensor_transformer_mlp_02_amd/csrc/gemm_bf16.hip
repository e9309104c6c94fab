// bf16 MFMA GEMM for gfx950 with the shard's fused epilogues.
//
// Block tile 256 x 256 x 64, 256 threads = 4 wavefronts in a 2 x 2 grid,
// each wavefront owning a 128 x 128 sub-tile computed as 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 (fp32 accumulators: 256 per lane).
//
// Shared memory holds both operand tiles "K-contiguous": row r (an m of
// opA or an n of opB) stores its 64 k values as eight 16-byte chunks, chunk
// c at position c ^ swz(r), so that the per-lane 16-byte MFMA operand
// reads of 8 or 16 consecutive rows fall in distinct banks.  Two tile
// buffers alternate: while the MFMAs consume one, the next tile's global
// loads are in flight in registers and are written to the other buffer
// afterwards (one barrier per 64-wide k step).
//
// Operands stored K-contiguous in memory are copied 16 bytes at a time.
// Operands stored M/N-contiguous are loaded as 8 x 8 blocks (8 k rows of 8
// consecutive m/n) and transposed in registers before the shared-memory
// write, so the MFMA read path is the same for every operand layout.
//
// The MFMA is issued with the B fragment as its first operand, which
// yields C^T blocks: each lane then holds 4 consecutive output columns of
// one row, and the epilogue stores 8 (bf16) or 16 (fp32) contiguous bytes.
#include "common.h"
#include "launch.h"

namespace tpmlp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace mfma256 {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NT = 256;
constexpr int TILE_ELEMS = (BM + BN) * BK;  // one buffer: A then B

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ int lds_off(int r, int c) {
  return r * BK + ((c ^ swz(r)) << 3);
}

// 8 x 8 transpose of 16-bit elements: in[i] holds row i (8 elements),
// out[j] receives column j (element i of out[j] = element j of in[i]).
__device__ __forceinline__ void transpose8x8(const uint4 in[8], uint4 out[8]) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(in);  // w[i*4 + q]
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t lo = w[(2 * q) * 4 + (j >> 1)];
      uint32_t hi = w[(2 * q + 1) * 4 + (j >> 1)];
      o[j * 4 + q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                             : ((lo & 0xffffu) | (hi << 16));
    }
  }
}

// Staging registers of one operand tile for one thread: 8 x 16 bytes.
struct Stage {
  uint4 v[8];
};

// ---- opA -----------------------------------------------------------------
template <bool KMAJOR>
__device__ __forceinline__ void load_a(const GemmArgs& g, const bf16_t* a0,
                                       const TileCoord& tc, int k0, int tid,
                                       Stage& s) {
  if constexpr (KMAJOR) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = tid + NT * i;
      int r = c >> 3, kc = c & 7;
      int m = tc.m_begin + r;
      int k = k0 + kc * 8;
      if (m < tc.m_end && k < tc.k_end)
        s.v[i] = *reinterpret_cast<const uint4*>(a0 + (int64_t)m * g.a.ld + k);
      else
        s.v[i] = make_uint4(0, 0, 0, 0);
    }
  } else {
    int kb = tid & 7, rb = tid >> 3;
    int m = tc.m_begin + rb * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int k = k0 + kb * 8 + i;
      if (m < tc.m_end && k < tc.k_end)
        s.v[i] = *reinterpret_cast<const uint4*>(a0 + (int64_t)k * g.a.ld + m);
      else
        s.v[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <bool KMAJOR>
__device__ __forceinline__ void store_a(bf16_t* lds, int tid, const Stage& s) {
  if constexpr (KMAJOR) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = tid + NT * i;
      int r = c >> 3, kc = c & 7;
      *reinterpret_cast<uint4*>(lds + lds_off(r, kc)) = s.v[i];
    }
  } else {
    uint4 t[8];
    transpose8x8(s.v, t);
    int kb = tid & 7, rb = tid >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint4*>(lds + lds_off(rb * 8 + j, kb)) = t[j];
  }
}

// ---- opB -----------------------------------------------------------------
template <bool KMAJOR, int BMODE>
__device__ __forceinline__ void load_b(const GemmArgs& g, const bf16_t* b0,
                                       const bf16_t* b1, const TileCoord& tc,
                                       int k0, int tid, Stage& s) {
  const int n_base = tc.tn * BN;
  if constexpr (KMAJOR) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = tid + NT * i;
      int r = c >> 3, kc = c & 7;
      int n = n_base + r;
      int k = k0 + kc * 8;
      if (n < g.N && k < tc.k_end) {
        const bf16_t* p;
        if constexpr (BMODE == BMODE_KSPLIT)
          p = (k < g.b.split) ? b0 + (int64_t)n * g.b.ld + k
                              : b1 + (int64_t)n * g.b.ld + (k - g.b.split);
        else
          p = b0 + (int64_t)n * g.b.ld + k;
        s.v[i] = *reinterpret_cast<const uint4*>(p);
      } else {
        s.v[i] = make_uint4(0, 0, 0, 0);
      }
    }
  } else {
    int kb = tid & 7, rb = tid >> 3;
    int n = n_base + rb * 8;
    const bf16_t* base;
    int col;
    bool ok;
    if constexpr (BMODE == BMODE_PAIR32) {
      int grp = n >> 6, w = n & 63;
      col = grp * 32 + (w & 31);
      base = (w < 32) ? b0 : b1;
      ok = col < g.b.split;  // split = width of each of the two matrices
    } else {
      col = n;
      base = b0;
      ok = n < g.N;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int k = k0 + kb * 8 + i;
      if (ok && k < tc.k_end)
        s.v[i] = *reinterpret_cast<const uint4*>(base + (int64_t)k * g.b.ld + col);
      else
        s.v[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <bool KMAJOR>
__device__ __forceinline__ void store_b(bf16_t* lds, int tid, const Stage& s) {
  store_a<KMAJOR>(lds, tid, s);  // same tile geometry (256 rows x 64 k)
}

// ---- kernel ----------------------------------------------------------------
template <bool A_KMAJOR, bool B_KMAJOR, int BMODE, int EPI, typename OutT>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * TILE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const TileCoord tc = locate_tile(g, blockIdx.x, BM);
  const bf16_t* a0 = reinterpret_cast<const bf16_t*>(g.a.p0) + tc.e * g.a.bstride;
  const bf16_t* b0 = reinterpret_cast<const bf16_t*>(g.b.p0) + tc.e * g.b.bstride;
  const bf16_t* b1 = reinterpret_cast<const bf16_t*>(g.b.p1) + tc.e * g.b.bstride;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (tc.k_end > tc.k_begin) ? (tc.k_end - tc.k_begin + BK - 1) / BK : 0;

  Stage sa, sb;
  if (nk > 0) {
    load_a<A_KMAJOR>(g, a0, tc, tc.k_begin, tid, sa);
    load_b<B_KMAJOR, BMODE>(g, b0, b1, tc, tc.k_begin, tid, sb);
    store_a<A_KMAJOR>(lds, tid, sa);
    store_b<B_KMAJOR>(lds + BM * BK, tid, sb);
  }
  __syncthreads();

  const int r_lane = lane & 31;
  const int c_lane = lane >> 5;

  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = tc.k_begin + (kt + 1) * BK;
      load_a<A_KMAJOR>(g, a0, tc, k0, tid, sa);
      load_b<B_KMAJOR, BMODE>(g, b0, b1, tc, k0, tid, sb);
    }
    const bf16_t* la = lds + (kt & 1) * TILE_ELEMS;
    const bf16_t* lb = la + BM * BK;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8_t af[4], bfr[4];
      const int c = 2 * s + c_lane;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(
            la + lds_off(wm * 128 + i * 32 + r_lane, c));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(
            lb + lds_off(wn * 128 + j * 32 + r_lane, c));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i],
                                                              acc[i][j], 0, 0, 0);
    }
    if (more) {
      bf16_t* nxt = lds + ((kt + 1) & 1) * TILE_ELEMS;
      store_a<A_KMAJOR>(nxt, tid, sa);
      store_b<B_KMAJOR>(nxt + BM * BK, tid, sb);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds rows m, columns n0 + 8 q + 4 c_lane + (0..3)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = tc.m_begin + wm * 128 + i * 32 + r_lane;
    if (m >= tc.m_end) continue;
    if constexpr (EPI == EPI_SWIGLU_FWD) {
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t f = (int64_t)tc.tn * (BN / 2) + wn * 64 + jp * 32 +
                            q * 8 + c_lane * 4;
          if (f >= g.epi.split) continue;
          float gv[4], uv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            gv[v] = acc[i][2 * jp][q * 4 + v];
            uv[v] = acc[i][2 * jp + 1][q * 4 + v];
          }
          epilogue_swiglu4<bf16_t>(g.epi, m, f, gv, uv);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = (int64_t)tc.tn * BN + wn * 128 + j * 32 + q * 8 + c_lane * 4;
          if (n >= g.N) continue;
          float cv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) cv[v] = acc[i][j][q * 4 + v];
          epilogue4<EPI, bf16_t, OutT>(g.epi, tc.e, m, n, cv);
        }
      }
    }
  }
}

}  // namespace mfma256

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static void fill_tiles(GemmArgs& g, int BM, int BN, int n_cols) {
  g.tiles_n = (n_cols + BN - 1) / BN;
  g.tile_off[0] = 0;
  for (int e = 0; e < g.E; ++e) {
    int rows;
    if (g.ragged == RAGGED_M)
      rows = g.row_off[e + 1] - g.row_off[e];
    else
      rows = g.M;
    int tm = (rows + BM - 1) / BM;
    g.tile_off[e + 1] = g.tile_off[e] + tm * g.tiles_n;
  }
}

template <bool AK, bool BK_, int BMODE, int EPI, typename OutT>
static hipError_t launch_mfma(GemmArgs& g, hipStream_t stream) {
  // PAIR32 covers 2 * split logical columns
  int n_cols = (BMODE == BMODE_PAIR32) ? 2 * (int)g.b.split : g.N;
  if (BMODE == BMODE_PAIR32) {
    // logical columns are laid out in 64-wide (gate 32 | up 32) groups
    n_cols = ((int)((g.b.split + 31) / 32)) * 64;
    g.N = n_cols;
  }
  fill_tiles(g, mfma256::BM, mfma256::BN, n_cols);
  int blocks = g.tile_off[g.E];
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((mfma256::gemm_kernel<AK, BK_, BMODE, EPI, OutT>),
                     dim3(blocks), dim3(mfma256::NT), 0, stream, g);
  return hipGetLastError();
}

hipError_t gemm_bf16(GemmKind kind, GemmArgs& g, hipStream_t stream) {
  switch (kind) {
    case GK_FC1_GELU:
      return launch_mfma<true, false, BMODE_PLAIN, EPI_GELU_FWD, bf16_t>(g, stream);
    case GK_FC1_SWIGLU:
      return launch_mfma<true, false, BMODE_PAIR32, EPI_SWIGLU_FWD, bf16_t>(g, stream);
    case GK_FC2:
      return launch_mfma<true, false, BMODE_PLAIN, EPI_STORE, bf16_t>(g, stream);
    case GK_DH_GELU:
      return launch_mfma<true, true, BMODE_PLAIN, EPI_GELU_BWD, bf16_t>(g, stream);
    case GK_DH_SWIGLU:
      return launch_mfma<true, true, BMODE_PLAIN, EPI_SWIGLU_BWD, bf16_t>(g, stream);
    case GK_WGRAD:
      return launch_mfma<false, false, BMODE_PLAIN, EPI_STORE, float>(g, stream);
    case GK_WGRAD_SPLIT:
      return launch_mfma<false, false, BMODE_PLAIN, EPI_STORE_SPLIT, float>(g, stream);
    case GK_DX:
      return launch_mfma<true, true, BMODE_PLAIN, EPI_STORE, bf16_t>(g, stream);
    case GK_DX_KSPLIT:
      return launch_mfma<true, true, BMODE_KSPLIT, EPI_STORE, bf16_t>(g, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
