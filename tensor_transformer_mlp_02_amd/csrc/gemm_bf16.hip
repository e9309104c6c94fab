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

// Buffer resource over an operand: out-of-range offsets read as zero, so a
// load needs no branch.  Offsets stay below 2^31 (dimensions are capped by
// the entry points); OOB_OFF marks a masked-off load.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t OOB_OFF = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7fffffff,
                                           0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// K-contiguous operand tile straight from memory into shared memory: 256 rows
// x 64 k, 8 x 1 KiB per wavefront.  Within each 1 KiB block lane l fills
// the 16 bytes at l*16, i.e. row 8*blk + l/8 at physical chunk l%8, which
// holds logical chunk (l%8) ^ swz(row).  `rs` is based at (row 0, k 0) of
// the tile's row range; rows >= rows_valid and k >= k_lim read as zeros.
__device__ __forceinline__ void direct_kmajor(rsrc_t rs, int64_t ld, int rows_valid,
                                              int k0, int k_lim, bf16_t* tile,
                                              int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = wave * 8 + i;
    const int r = blk * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    const int k = k0 + c * 8;
    const uint32_t off = (r < rows_valid && k < k_lim)
                             ? (uint32_t)(((int64_t)r * ld + k) * 2) : OOB_OFF;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + blk * 512), 16, off,
                                             0, 0, 0);
  }
}

// M/N-contiguous operand tiles (64 k rows x 256 columns) live in shared
// memory as two halves of 128 columns, [half][k][16 granules of 8], with
// granule q of row k stored at q ^ 4 (k % 4).  A 1 KiB direct load then
// covers 4 rows of one half (so it has one source matrix, which the gate /
// up pair needs), and the transposed fragment reads below touch 16
// distinct 16-byte bank slots per 4 rows.
__device__ __forceinline__ int mn_off(int k, int c) {
  const int h = c >> 7, q = (c >> 3) & 15, e = c & 7;
  return h * (BK * 128) + k * 128 + ((q ^ ((k & 3) << 2)) << 3) + e;
}

// Direct load of an M/N-contiguous tile.  rs[h] is based at (k row 0 of the
// tile, column 0 of the source matrix of half h); half h covers columns
// col0[h] .. col0[h] + 127 of it, valid below col_lim, rows below k_valid.
__device__ __forceinline__ void direct_mn(rsrc_t rs0, rsrc_t rs1, int64_t ld, int col00,
                                          int col01, int col_lim, int k_valid, bf16_t* tile,
                                          int wave, int lane) {
  const int half = wave >> 1;
  const rsrc_t rs = half ? rs1 : rs0;
  const int col0 = half ? col01 : col00;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = (wave & 1) * 8 + i;
    const int k = 4 * b + (lane >> 4);
    const int q = (lane & 15) ^ ((k & 3) << 2);
    const int col = col0 + 8 * q;
    const uint32_t off = (k < k_valid && col < col_lim)
                             ? (uint32_t)(((int64_t)k * ld + col) * 2) : OOB_OFF;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + half * (BK * 128) + b * 512),
                                             16, off, 0, 0, 0);
  }
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// MFMA fragment (32 columns from c0, 16 k from k0) of an M/N-contiguous
// tile: lane l gets column c0 + l % 32, k = k0 + 8 (l / 32) + 0..7, the
// same order as a 16-byte read of a K-contiguous row.
__device__ __forceinline__ bf16x8_t frag_mn(const bf16_t* tile, int c0, int k0, int lane) {
  const int g = lane >> 4, r = lane & 15;
  const int c = c0 + 16 * (g & 1) + 4 * (r & 3);
  const int k = k0 + 8 * (g >> 1) + (r >> 2);
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t*)(tile + mn_off(k, c)));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t*)(tile + mn_off(k + 4, c)));
  const auto v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// Staging registers of one operand tile for one thread: 8 x 16 bytes.
struct Stage {
  uint4 v[8];
};

__device__ __forceinline__ uint4 load16_or_zero(const bf16_t* p, const bf16_t* safe, bool ok) {
  uint4 v = *reinterpret_cast<const uint4*>(ok ? p : safe);
  return ok ? v : make_uint4(0, 0, 0, 0);
}

// M/N-contiguous operand tile (64 k rows x 256 m) through registers: thread
// (kb, rb) loads the 8 x 8 block k = 8 kb .. 8 kb + 7, m = 8 rb .. 8 rb + 7.
// `base` points at (k 0, m 0) of the tile's m range; BMODE_PAIR32 maps the
// logical column to one of two matrices (see GemmArgs).
template <int BMODE>
__device__ __forceinline__ void load_mn(const bf16_t* p0, const bf16_t* p1, int64_t ld,
                                        int m_base, int m_lim, int k0, int k_lim, int tid,
                                        Stage& s) {
  const int kb = tid & 7, rb = tid >> 3;
  const int n = m_base + rb * 8;
  const bf16_t* base;
  int col;
  bool okc;
  if constexpr (BMODE == BMODE_PAIR32) {
    const int grp = n >> 6, w = n & 63;
    col = grp * 32 + (w & 31);
    base = (w < 32) ? p0 : p1;
    okc = col < m_lim;
  } else {
    col = n;
    base = p0;
    okc = n < m_lim;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = k0 + kb * 8 + i;
    const bool ok = okc && k < k_lim;
    s.v[i] = load16_or_zero(base + (int64_t)k * ld + col, p0, ok);
  }
}

__device__ __forceinline__ void store_mn(bf16_t* tile, int tid, const Stage& s) {
  uint4 t[8];
  transpose8x8(s.v, t);
  const int kb = tid & 7, rb = tid >> 3;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<uint4*>(tile + lds_off(rb * 8 + j, kb)) = t[j];
}

// K-contiguous operand through registers (used when one tile would need
// two source matrices: a k split that is not a multiple of 64).
template <int BMODE>
__device__ __forceinline__ void load_k(const bf16_t* p0, const bf16_t* p1, int64_t ld,
                                       int64_t split, int r_base, int r_lim, int k0,
                                       int k_lim, int tid, Stage& s) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + NT * i;
    const int r = c >> 3, kc = c & 7;
    const int n = r_base + r;
    const int k = k0 + kc * 8;
    const bool ok = n < r_lim && k < k_lim;
    const bf16_t* p;
    if constexpr (BMODE == BMODE_KSPLIT)
      p = (k < split) ? p0 + (int64_t)n * ld + k : p1 + (int64_t)n * ld + (k - split);
    else
      p = p0 + (int64_t)n * ld + k;
    s.v[i] = load16_or_zero(p, p0, ok);
  }
}

__device__ __forceinline__ void store_k(bf16_t* tile, int tid, const Stage& s) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + NT * i;
    const int r = c >> 3, kc = c & 7;
    *reinterpret_cast<uint4*>(tile + lds_off(r, kc)) = s.v[i];
  }
}

// ---- kernel ----------------------------------------------------------------
// A_KMAJOR: opA K-contiguous (loaded straight into shared memory) or M-
// contiguous (through registers, transposed).  B likewise; B_DIRECT selects
// the direct path for a K-contiguous opB (a k split must then be a multiple
// of 64 so each k tile comes from one matrix).
template <bool A_KMAJOR, bool B_KMAJOR, int BMODE, int EPI, typename OutT, bool B_DIRECT>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) bf16_t lds[2 * TILE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const TileCoord tc = locate_tile(g, blockIdx.x, BM);
  const bf16_t* a0 = reinterpret_cast<const bf16_t*>(g.a.p0) + tc.e * g.a.bstride;
  const bf16_t* b0 = reinterpret_cast<const bf16_t*>(g.b.p0) + tc.e * g.b.bstride;
  const bf16_t* b1 = reinterpret_cast<const bf16_t*>(g.b.p1) + tc.e * g.b.bstride;
  // scalar copies of the argument block: helpers never see its address
  const int64_t lda = g.a.ld, ldb = g.b.ld, bsplit = g.b.split;
  const int Ncols = g.N, Ktot = g.K;
  const EpiArgs ea = g.epi;
  const int n_base = tc.tn * BN;
  const int m_rows = tc.m_end - tc.m_begin;
  // opB's valid extent along N: PAIR32 masks on the per-matrix column
  const int n_lim = (BMODE == BMODE_PAIR32) ? (int)bsplit : Ncols;

  // buffer resources: K-contiguous operands are based at the tile's first
  // row (fixed for the whole k loop); M/N-contiguous ones are re-based at
  // each k tile's first row (see issue)
  const rsrc_t rs_a = make_rsrc(a0 + (A_KMAJOR ? (int64_t)tc.m_begin * lda : 0));
  const rsrc_t rs_b0 = make_rsrc(b0 + (B_KMAJOR ? (int64_t)n_base * ldb : 0));
  const rsrc_t rs_b1 = make_rsrc((BMODE != BMODE_PLAIN ? b1 : b0) +
                                 (B_KMAJOR ? (int64_t)n_base * ldb : 0));

  f32x16_t acc[4][4];
  static_for<0, 4>([&](auto I) {
    static_for<0, 4>([&](auto J) { acc[I][J] = (f32x16_t)(0.0f); });
  });

  const int nk = (tc.k_end > tc.k_begin) ? (tc.k_end - tc.k_begin + BK - 1) / BK : 0;

  Stage sb;  // only for a K-contiguous opB whose k split is not 64-aligned
  // issue the loads of the k tile starting at k0 into buffer `buf`
  auto issue = [&](int k0, bf16_t* buf) {
    if constexpr (A_KMAJOR) {
      direct_kmajor(rs_a, lda, m_rows, k0, tc.k_end, buf, wave, lane);
    } else {
      const rsrc_t r = make_rsrc(a0 + (int64_t)k0 * lda);
      direct_mn(r, r, lda, tc.m_begin, tc.m_begin + 128, tc.m_end, tc.k_end - k0, buf, wave,
                lane);
    }
    bf16_t* tb = buf + BM * BK;
    if constexpr (B_KMAJOR && B_DIRECT) {
      if constexpr (BMODE == BMODE_KSPLIT) {
        if (k0 < bsplit)
          direct_kmajor(rs_b0, ldb, Ncols - n_base, k0, (int)bsplit, tb, wave, lane);
        else
          direct_kmajor(rs_b1, ldb, Ncols - n_base, k0 - (int)bsplit, Ktot - (int)bsplit, tb,
                        wave, lane);
      } else {
        direct_kmajor(rs_b0, ldb, Ncols - n_base, k0, tc.k_end, tb, wave, lane);
      }
    } else if constexpr (B_KMAJOR) {
      load_k<BMODE>(b0, b1, ldb, bsplit, n_base, Ncols, k0, tc.k_end, tid, sb);
    } else if constexpr (BMODE == BMODE_PAIR32) {
      // half 0: gate columns, half 1: up columns, both f = 128 tn ..
      const rsrc_t r0 = make_rsrc(b0 + (int64_t)k0 * ldb);
      const rsrc_t r1 = make_rsrc(b1 + (int64_t)k0 * ldb);
      direct_mn(r0, r1, ldb, tc.tn * 128, tc.tn * 128, (int)bsplit, tc.k_end - k0, tb, wave,
                lane);
    } else {
      const rsrc_t r = make_rsrc(b0 + (int64_t)k0 * ldb);
      direct_mn(r, r, ldb, n_base, n_base + 128, Ncols, tc.k_end - k0, tb, wave, lane);
    }
  };
  auto commit = [&](bf16_t* buf) {
    if constexpr (B_KMAJOR && !B_DIRECT) store_k(buf + BM * BK, tid, sb);
  };

  const int r_lane = lane & 31;
  const int c_lane = lane >> 5;
  // tile column of opB block j of this wavefront
  auto b_col = [&](int j) {
    if constexpr (BMODE == BMODE_PAIR32) return (j & 1) * 128 + wn * 64 + (j >> 1) * 32;
    else return wn * 128 + j * 32;
  };
  bf16x8_t fa[2][4], fb[2][4];
  auto frags = [&](const bf16_t* buf, int s, int slot) {
    const int c = 2 * s + c_lane;
    const bf16_t* la = buf;
    const bf16_t* lb = buf + BM * BK;
    static_for<0, 4>([&](auto I) {
      if constexpr (A_KMAJOR)
        fa[slot][I] = *reinterpret_cast<const bf16x8_t*>(la + lds_off(wm * 128 + I * 32 + r_lane, c));
      else
        fa[slot][I] = frag_mn(la, wm * 128 + I * 32, 16 * s, lane);
    });
    static_for<0, 4>([&](auto J) {
      if constexpr (B_KMAJOR)
        fb[slot][J] = *reinterpret_cast<const bf16x8_t*>(lb + lds_off(wn * 128 + J * 32 + r_lane, c));
      else
        fb[slot][J] = frag_mn(lb, b_col(J), 16 * s, lane);
    });
  };

  if (nk > 0) {
    issue(tc.k_begin, lds);
    commit(lds);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  if (nk > 0) frags(lds, 0, 0);

  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    bf16_t* cur = lds + (kt & 1) * TILE_ELEMS;
    bf16_t* nxt = lds + ((kt + 1) & 1) * TILE_ELEMS;
    if (more) issue(tc.k_begin + (kt + 1) * BK, nxt);
    static_for<0, BK / 16>([&](auto S) {
      constexpr int s = decltype(S)::value;
      if constexpr (s + 1 < BK / 16) frags(cur, s + 1, (s + 1) & 1);
      static_for<0, 4>([&](auto I) {
        static_for<0, 4>([&](auto J) {
          acc[I][J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s & 1][J], fa[s & 1][I],
                                                              acc[I][J], 0, 0, 0);
        });
      });
    });
    if (more) commit(nxt);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (more) frags(nxt, 0, 0);
  }

  // ---- epilogue: lane holds rows m, columns n0 + 8 q + 4 c_lane + (0..3)
  static_for<0, 4>([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int64_t m = tc.m_begin + wm * 128 + i * 32 + r_lane;
    if (m < tc.m_end) {
      if constexpr (EPI == EPI_SWIGLU_FWD) {
        static_for<0, 2>([&](auto JP) {
          constexpr int jp = decltype(JP)::value;
          static_for<0, 4>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            const int64_t f = (int64_t)tc.tn * (BN / 2) + wn * 64 + jp * 32 + q * 8 + c_lane * 4;
            if (f < ea.split) {
              float gv[4], uv[4];
              static_for<0, 4>([&](auto V) {
                constexpr int v = decltype(V)::value;
                gv[v] = acc[i][2 * jp][q * 4 + v];
                uv[v] = acc[i][2 * jp + 1][q * 4 + v];
              });
              epilogue_swiglu4<bf16_t>(ea, m, f, gv, uv);
            }
            __builtin_amdgcn_sched_barrier(0);
          });
        });
      } else {
        static_for<0, 4>([&](auto J) {
          constexpr int j = decltype(J)::value;
          static_for<0, 4>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            const int64_t n = (int64_t)tc.tn * BN + wn * 128 + j * 32 + q * 8 + c_lane * 4;
            if (n < Ncols) {
              float cv[4];
              static_for<0, 4>([&](auto V) {
                constexpr int v = decltype(V)::value;
                cv[v] = acc[i][j][q * 4 + v];
              });
              epilogue4<EPI, bf16_t, OutT>(ea, tc.e, m, n, cv);
            }
            // keep each group's loads and stores local: hoisting all of
            // them would exceed the register file
            __builtin_amdgcn_sched_barrier(0);
          });
        });
      }
    }
  });
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
  int n_cols = g.N;
  if (BMODE == BMODE_PAIR32) {
    // logical columns are laid out in 64-wide (gate 32 | up 32) groups
    n_cols = ((int)((g.b.split + 31) / 32)) * 64;
    g.N = n_cols;
  }
  fill_tiles(g, mfma256::BM, mfma256::BN, n_cols);
  int blocks = g.tile_off[g.E];
  if (blocks == 0) return hipSuccess;
  // a K-contiguous opB goes straight to shared memory unless a 64-wide k
  // tile could straddle its two source matrices
  const bool b_direct = BK_ && (BMODE != BMODE_KSPLIT || g.b.split % mfma256::BK == 0);
  if (b_direct)
    hipLaunchKernelGGL((mfma256::gemm_kernel<AK, BK_, BMODE, EPI, OutT, BK_>),
                       dim3(blocks), dim3(mfma256::NT), 0, stream, g);
  else
    hipLaunchKernelGGL((mfma256::gemm_kernel<AK, BK_, BMODE, EPI, OutT, false>),
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
