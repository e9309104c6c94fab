// Shared device-side pieces of the shard kernels: storage types, the
// activation functions, the GEMM argument block and the fused epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/tpmlp.h"

namespace tpmlp {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
// Register arrays indexed inside stay register arrays whatever the body's
// size (a large unrolled body can otherwise defeat unrolling and push the
// array to scratch memory).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// bf16 <-> f32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round to nearest, ties to even, NaN stays a NaN: gfx950's packed
// conversion (v_cvt_pk_bf16_f32) does this in one instruction per pair.
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_cvt_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_cvt_t));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return (bf16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// activations (fp32)
//
// GeLU, tanh form: gelu(z) = z/2 (1 + tanh(u)), u = c (z + k z^3),
// c = sqrt(2/pi), k = 0.044715.  Since (1 + tanh(u))/2 = sigmoid(2u),
// gelu(z) = z * s with s = sigmoid(2u), and
// gelu'(z) = s + z * 2 s (1 - s) * c (1 + 3 k z^2).
// SwiGLU pieces: silu(g) = g sigmoid(g), silu'(g) = s (1 + g (1 - s)).
// sigmoid(x) = 1 / (1 + exp(-x)); exp via the hardware exp2 (__expf).
// Large |x| saturate correctly: exp -> inf gives 0, exp -> 0 gives 1.
// ---------------------------------------------------------------------------
#define TP_GELU_C 0.7978845608028654f
#define TP_GELU_K 0.044715f

__device__ __forceinline__ float sigmoid_f(float x) {
  return 1.0f / (1.0f + __expf(-x));
}

__device__ __forceinline__ float gelu_f(float z) {
  float u = TP_GELU_C * (z + TP_GELU_K * z * z * z);
  return z * sigmoid_f(2.0f * u);
}

__device__ __forceinline__ float gelu_grad_f(float z) {
  float z2 = z * z;
  float u = TP_GELU_C * (z + TP_GELU_K * z2 * z);
  float s = sigmoid_f(2.0f * u);
  return s + z * 2.0f * s * (1.0f - s) * TP_GELU_C * (1.0f + 3.0f * TP_GELU_K * z2);
}

__device__ __forceinline__ float silu_f(float g) { return g * sigmoid_f(g); }

__device__ __forceinline__ float silu_grad_f(float g) {
  float s = sigmoid_f(g);
  return s * (1.0f + g * (1.0f - s));
}

// The activation derivative applied to dH while a backward GEMM loads its
// dZ operand (instead of in the epilogue of dY B^T): one element of dZ =
// dh gelu'(z) (GeLU), or of [dG | dU] (SwiGLU: second = false gives dG = dh
// u silu'(g), second = true gives dU = dh silu(g)).  This runs once per
// element for every tile that reads it, on the vector ALUs, so the sigmoid
// takes the hardware reciprocal (v_rcp_f32, 1 ulp) instead of a divide.
enum { DACT_NONE = 0, DACT_GELU = 1, DACT_SWIGLU = 2 };

__device__ __forceinline__ float sigmoid_rcp_f(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

template <int PRO>
__device__ __forceinline__ float dact_elem(float dh, float z0, float z1, bool second) {
  if constexpr (PRO == DACT_GELU) {
    const float z2 = z0 * z0;
    const float s = sigmoid_rcp_f(2.0f * TP_GELU_C * (z0 + TP_GELU_K * z2 * z0));
    return dh * (s + z0 * 2.0f * s * (1.0f - s) * TP_GELU_C * (1.0f + 3.0f * TP_GELU_K * z2));
  } else {
    // dU = dh s g and dG = dh s u (1 + g (1 - s)): one select, no branch
    const float s = sigmoid_rcp_f(z0);
    const float t = second ? z0 : z1 * (1.0f + z0 * (1.0f - s));
    return dh * s * t;
  }
}

// ---------------------------------------------------------------------------
// GEMM arguments
//
// C[M,N] = opA[M,K] * opB[K,N], fp32 accumulate.  An operand is
// "K-major" when its K index is the contiguous one in memory.
//   opA K-major:  element (m,k) at a.p0[m*a.ld + k]
//   opA MN-major: element (m,k) at a.p0[k*a.ld + m]
//   opB K-major:  element (k,n) at b.p0[n*b.ld + k]
//                 (BMODE_KSPLIT: k >= b.split reads b.p1 at k - b.split)
//   opB MN-major: element (k,n) at b.p0[k*b.ld + n]
//                 (BMODE_PAIR32: logical column n = 64 g + 32 h + j maps to
//                  matrix h (p0 gate / p1 up), column f = 32 g + j; this
//                  puts the gate and up values of one f in the same lanes)
//
// Grouped problems: E independent problems share every operand; problem e
// covers the rows [row_off[e], row_off[e+1]) of its ragged dimension
// (M for RAGGED_M, K for RAGGED_K; unused for RAGGED_NONE), and its
// "batched" operands/outputs are offset by e * bstride elements.  Row
// indices of the ragged dimension are global (no per-expert rebasing).
// Problem e owns blocks [tile_off[e], tile_off[e+1]).
// ---------------------------------------------------------------------------
enum { BMODE_PLAIN = 0, BMODE_KSPLIT = 1, BMODE_PAIR32 = 2 };
enum { RAGGED_NONE = 0, RAGGED_M = 1, RAGGED_K = 2 };

enum {
  EPI_STORE = 0,        // out0[m,n] = c
  EPI_GELU_FWD = 1,     // out0[m,n] = z (if out0), out1[m,n] = gelu(z)
  EPI_SWIGLU_FWD = 2,   // out0[m,f] = g, out0[m,split+f] = u (if out0),
                        // out1[m,f] = silu(g) u
  EPI_GELU_BWD = 3,     // out0[m,n] = c * gelu'(aux[m,n])
  EPI_SWIGLU_BWD = 4,   // g = aux[m,n], u = aux[m,split+n]:
                        // out0[m,n] = c u silu'(g), out0[m,split+n] = c silu(g)
  EPI_STORE_SPLIT = 5,  // n < split: out0[m,n]; else out1[m,n-split]
  EPI_ACC = 6,          // out0[m,n] += c  (weight-gradient accumulation)
  EPI_ACC_SPLIT = 7,    // EPI_STORE_SPLIT with += (each element has one writer)
};

struct OpArgs {
  const void* p0;
  const void* p1;
  int64_t ld;
  int64_t bstride;  // per-problem element offset (0: shared by all problems)
  int64_t split;
};

struct EpiArgs {
  void* out0;
  void* out1;
  const void* aux;
  int64_t ld0, ld1, ldaux;
  int64_t bstride;  // per-problem element offset of out0/out1 (weight grads)
  int64_t split;
  // FP8 paths only: quantized H (out2, E4M3 bytes, row pitch ld2), the
  // per-tensor scales (x_inv, a_inv, au_inv, b_inv, h_scale) and max |H|
  void* out2;
  int64_t ld2;
  const float* qs;
  float* amax;
  // FP8 backward: dequantize by qs[qi] * qs[qj]; dZ codes use qs[qk]
  int qi, qj, qk;
};

struct GemmArgs {
  OpArgs a, b;
  EpiArgs epi;
  int M, N, K;
  int ragged;
  int E;
  int tiles_n;
  int row_off[TP_MAX_EXPERTS + 1];
  int tile_off[TP_MAX_EXPERTS + 1];
  // Row offsets in device memory (E+1 int32, e.g. written by the routing
  // step on the same stream), read by every workgroup in place of row_off.
  // They are taken clamped: offset 0 into [0, dev_rows], offset e+1 into
  // [offset e, dev_rows], so no value can send an access past dev_rows
  // rows.  A RAGGED_M launch then has workgroups for every split of
  // dev_rows rows into E problems; those past the tiles the offsets need
  // exit at once (TileCoord::e < 0): only the hand-ordered (256 and 128
  // rows), ring, general and thin kernels run such launches.  A RAGGED_K
  // launch takes only its k ranges from them (any kernel).
  const int* dev_off;
  int dev_rows;
  // With dev_off, RAGGED_M: the launcher queues every tiling the host could
  // have picked from host offsets (256-row tiles; with dev_thin > 0 the
  // same with remainders of at most dev_thin rows in a thin launch; with
  // dev_l128 > 0 128-row tiles, their area weighted by dev_l128 / 1000),
  // and every workgroup takes the host's choice from the offsets (fewest
  // weighted tile-area waves over dev_cus compute units): the workgroups
  // of the launches not chosen exit at once.
  int dev_thin, dev_l128, dev_cus;
};

// Problem lookup shared by the GEMM kernels.
//
// Block placement: consecutive workgroup ids are dispatched round-robin to
// the 8 XCDs (each with its own L2), so block b runs on XCD b % 8.  The
// logical tile order gives each XCD a contiguous range of tiles, and
// within a problem tiles are rastered in groups of RASTER_G tile rows
// (column by column inside a group), so the blocks that run together on
// one XCD share a few operand panels instead of touching all of them.
//
// TP_TILE_ORDER (a build option, default 0) exists to measure what that
// saving is worth: 1 places tiles in dispatch order (consecutive tiles on
// different XCDs), 2 rasters groups of a single tile row.  Every order
// computes each tile the same way, so results are identical.
#ifndef TP_TILE_ORDER
#define TP_TILE_ORDER 0
#endif
constexpr int RASTER_G = TP_TILE_ORDER == 2 ? 1 : 4;

struct TileCoord {
  int e, tm, tn;
  int m_begin, m_end, k_begin, k_end;
};

__device__ __forceinline__ int xcd_logical_block(int b, int nb) {
  if constexpr (TP_TILE_ORDER == 1) return b;
  const int xcd = b & 7, slot = b >> 3;
  const int q = nb >> 3, r = nb & 7;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// ---- device-resident offsets: one problem per lane (E <= 64) -------------
// Every lane of the wavefront must be active; results that index a problem
// come back through readlane, so they are wave-uniform (scalar).

// Lane i gets problem i's clamped rows [lo, hi); lanes past E get empty
// problems at the end.  Clamping each offset into [previous one, rows]
// (the first into [0, rows]) is the same as clamping the running maximum
// of the offsets into [0, rows].
__device__ __forceinline__ void dev_lane_rows(const GemmArgs& g, int& lo, int& hi) {
  const int lane = threadIdx.x & 63;
  const int first = g.dev_off[0];
  int v = lane < g.E ? max(g.dev_off[lane + 1], first) : first;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v = max(v, u);
  }
  hi = min(max(v, 0), g.dev_rows);
  const int prev = __shfl_up(hi, 1, 64);
  lo = lane == 0 ? min(max(first, 0), g.dev_rows) : prev;
}

// (the same in every lane: returned as a scalar, so that what is decided
// from it is a uniform branch)
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return __builtin_amdgcn_readfirstlane(x);
}

__device__ __forceinline__ int wave_incl_sum(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(x, d, 64);
    if (lane >= d) x += u;
  }
  return x;
}

// tile rows of `rows` rows in BM-row tiles, the last few left out when
// remainders of at most `thin` rows go to the thin launch
__device__ __forceinline__ int dev_tile_rows(int rows, int BM, int thin) {
  return thin > 0 ? rows / BM + (rows % BM > thin ? 1 : 0) : (rows + BM - 1) / BM;
}

// The tiling the offsets call for (the same in every workgroup of every
// launch): 0 = 256-row tiles, 1 = 256-row tiles with thin remainders,
// 2 = 128-row tiles.  `rows` is this lane's problem's.
enum { DEV_T256 = 0, DEV_T256_THIN = 1, DEV_T128 = 2 };
__device__ __forceinline__ int dev_tiling(const GemmArgs& g, int rows) {
  const int64_t c = g.dev_cus, tn = g.tiles_n;
  auto waves = [&](int tile_rows) { return (int)((wave_sum(tile_rows) * tn + c - 1) / c); };
  int pick = DEV_T256;
  int w256 = waves(dev_tile_rows(rows, 256, 0));
  if (g.dev_thin > 0) {
    const int wt = waves(dev_tile_rows(rows, 256, g.dev_thin));
    if (wt < w256) {
      pick = DEV_T256_THIN;
      w256 = wt;
    }
  }
  // half-height tiles: half the area per wave, weighted by dev_l128 / 1000
  if (g.dev_l128 > 0 && (int64_t)g.dev_l128 * waves(dev_tile_rows(rows, 128, 0)) <
                            (int64_t)2000 * w256)
    pick = DEV_T128;
  return pick;
}

// This launch's tile `block` from the per-lane tile counts `tiles` (tile
// rows x tiles_n per problem): the first `total` workgroups take the tiles
// in the order a launch of exactly that many would, so the work spreads
// over every XCD however far the grid overshoots it.  Returns false for a
// spare workgroup.
__device__ __forceinline__ bool dev_find_tile(int tiles, int block, int lo_l, int hi_l, int& e,
                                              int& t0, int& t1, int& lo, int& hi, int& tile) {
  const int incl = wave_incl_sum(tiles);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  if (block >= total) return false;
  tile = xcd_logical_block(block, total);
  e = __ffsll((unsigned long long)__ballot(tile < incl)) - 1;
  t1 = __builtin_amdgcn_readlane(incl, e);
  t0 = t1 - __builtin_amdgcn_readlane(tiles, e);
  lo = __builtin_amdgcn_readlane(lo_l, e);
  hi = __builtin_amdgcn_readlane(hi_l, e);
  return true;
}

__device__ __forceinline__ TileCoord locate_tile(const GemmArgs& g, int block, int nblocks,
                                                 int BM) {
  TileCoord t;
  int tile, e = 0, t0, t1, lo, hi;
  if (g.dev_off && g.ragged == RAGGED_M) {
    int lo_l, hi_l;
    dev_lane_rows(g, lo_l, hi_l);
    const int pick = dev_tiling(g, hi_l - lo_l);
    if ((BM == 128) != (pick == DEV_T128)) {
      t.e = -1;  // the other tiling's launch does the work
      return t;
    }
    const int thin = pick == DEV_T256_THIN ? g.dev_thin : 0;
    if (!dev_find_tile(dev_tile_rows(hi_l - lo_l, BM, thin) * g.tiles_n, block, lo_l, hi_l, e,
                       t0, t1, lo, hi, tile)) {
      t.e = -1;  // a spare workgroup of the worst-case grid
      return t;
    }
  } else {
    tile = xcd_logical_block(block, nblocks);
    while (e + 1 < g.E && tile >= g.tile_off[e + 1]) ++e;
    t0 = g.tile_off[e];
    t1 = g.tile_off[e + 1];
    if (g.dev_off) {
      // RAGGED_K: the tiles do not depend on the rows, the k range does
      int lo_l, hi_l;
      dev_lane_rows(g, lo_l, hi_l);
      lo = __builtin_amdgcn_readlane(lo_l, e);
      hi = __builtin_amdgcn_readlane(hi_l, e);
    } else {
      lo = g.row_off[e];
      hi = g.row_off[e + 1];
    }
  }
  const int local = tile - t0;
  // tile rows of this problem as the launcher counted them (a ragged
  // problem's last few rows may be left to the thin-tile launch)
  const int tiles_m = (t1 - t0) / g.tiles_n;
  const int group = local / (RASTER_G * g.tiles_n);
  const int first_m = group * RASTER_G;
  const int gm = min(RASTER_G, tiles_m - first_m);
  const int li = local - group * RASTER_G * g.tiles_n;
  t.e = e;
  t.tm = first_m + li % gm;
  t.tn = li / gm;
  if (g.ragged == RAGGED_M) {
    t.m_begin = lo + t.tm * BM; t.m_end = hi; t.k_begin = 0; t.k_end = g.K;
  } else if (g.ragged == RAGGED_K) {
    t.m_begin = t.tm * BM; t.m_end = g.M; t.k_begin = lo; t.k_end = hi;
  } else {
    t.m_begin = t.tm * BM; t.m_end = g.M; t.k_begin = 0; t.k_end = g.K;
  }
  return t;
}

// ---------------------------------------------------------------------------
// storage access for 4 consecutive elements
// ---------------------------------------------------------------------------
template <typename T> struct Store4;

template <> struct Store4<bf16_t> {
  static __device__ __forceinline__ void store(void* base, int64_t off,
                                               const float v[4]) {
    uint2 p;
    p.x = pack_bf16x2(v[0], v[1]);
    p.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(base) + off) = p;
  }
  static __device__ __forceinline__ void load(const void* base, int64_t off,
                                              float v[4]) {
    uint2 p = *reinterpret_cast<const uint2*>(
        reinterpret_cast<const bf16_t*>(base) + off);
    v[0] = __uint_as_float(p.x << 16);
    v[1] = __uint_as_float(p.x & 0xffff0000u);
    v[2] = __uint_as_float(p.y << 16);
    v[3] = __uint_as_float(p.y & 0xffff0000u);
  }
};

template <> struct Store4<float> {
  static __device__ __forceinline__ void store(void* base, int64_t off,
                                               const float v[4]) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off) =
        make_float4(v[0], v[1], v[2], v[3]);
  }
  static __device__ __forceinline__ void load(const void* base, int64_t off,
                                              float v[4]) {
    float4 p = *reinterpret_cast<const float4*>(
        reinterpret_cast<const float*>(base) + off);
    v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
  }
};

// ---------------------------------------------------------------------------
// fused epilogues: 4 consecutive columns n..n+3 of row m
// (T = activation storage type, OutT = type of out0/out1 for EPI_STORE /
//  EPI_STORE_SPLIT)
// ---------------------------------------------------------------------------
template <int EPI, typename T, typename OutT>
__device__ __forceinline__ void epilogue4(const EpiArgs& ea, int e, int64_t m,
                                          int64_t n, const float c[4]) {
  if constexpr (EPI == EPI_STORE) {
    Store4<OutT>::store(ea.out0, e * ea.bstride + m * ea.ld0 + n, c);
  } else if constexpr (EPI == EPI_STORE_SPLIT) {
    if (n < ea.split)
      Store4<OutT>::store(ea.out0, e * ea.bstride + m * ea.ld0 + n, c);
    else
      Store4<OutT>::store(ea.out1, e * ea.bstride + m * ea.ld1 + (n - ea.split), c);
  } else if constexpr (EPI == EPI_ACC || EPI == EPI_ACC_SPLIT) {
    void* o = ea.out0;
    int64_t off = e * ea.bstride + m * ea.ld0 + n;
    if (EPI == EPI_ACC_SPLIT && n >= ea.split) {
      o = ea.out1;
      off = e * ea.bstride + m * ea.ld1 + (n - ea.split);
    }
    float v[4];
    Store4<OutT>::load(o, off, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += c[i];
    Store4<OutT>::store(o, off, v);
  } else if constexpr (EPI == EPI_GELU_FWD) {
    float h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = gelu_f(c[i]);
    if (ea.out0) Store4<T>::store(ea.out0, m * ea.ld0 + n, c);
    Store4<T>::store(ea.out1, m * ea.ld1 + n, h);
  } else if constexpr (EPI == EPI_GELU_BWD) {
    float z[4], d[4];
    Store4<T>::load(ea.aux, m * ea.ldaux + n, z);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = c[i] * gelu_grad_f(z[i]);
    Store4<T>::store(ea.out0, m * ea.ld0 + n, d);
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    float g[4], u[4], dg[4], du[4];
    Store4<T>::load(ea.aux, m * ea.ldaux + n, g);
    Store4<T>::load(ea.aux, m * ea.ldaux + ea.split + n, u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s = sigmoid_f(g[i]);
      dg[i] = c[i] * u[i] * (s * (1.0f + g[i] * (1.0f - s)));
      du[i] = c[i] * (g[i] * s);
    }
    Store4<T>::store(ea.out0, m * ea.ld0 + n, dg);
    Store4<T>::store(ea.out0, m * ea.ld0 + ea.split + n, du);
  }
}

// SwiGLU forward epilogue: gate and up values of columns f..f+3.
template <typename T>
__device__ __forceinline__ void epilogue_swiglu4(const EpiArgs& ea, int64_t m,
                                                 int64_t f, const float g[4],
                                                 const float u[4]) {
  float h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = silu_f(g[i]) * u[i];
  if (ea.out0) {
    Store4<T>::store(ea.out0, m * ea.ld0 + f, g);
    Store4<T>::store(ea.out0, m * ea.ld0 + ea.split + f, u);
  }
  Store4<T>::store(ea.out1, m * ea.ld1 + f, h);
}


// ---------------------------------------------------------------------------
// the same fused epilogues on 8 consecutive columns n..n+7 (one 16-byte
// piece of a bf16 row): used when a tile's sums are read back row-major
// ---------------------------------------------------------------------------
template <typename T> struct Vec8;

template <> struct Vec8<bf16_t> {
  static __device__ __forceinline__ void store(void* base, int64_t off, const float v[8]) {
    uint4 p;
    p.x = pack_bf16x2(v[0], v[1]);
    p.y = pack_bf16x2(v[2], v[3]);
    p.z = pack_bf16x2(v[4], v[5]);
    p.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(base) + off) = p;
  }
  static __device__ __forceinline__ void load(const void* base, int64_t off, float v[8]) {
    const uint4 p = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(base) + off);
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <> struct Vec8<float> {
  static __device__ __forceinline__ void store(void* base, int64_t off, const float v[8]) {
    float* q = reinterpret_cast<float*>(base) + off;
    *reinterpret_cast<float4*>(q) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(q + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  static __device__ __forceinline__ void load(const void* base, int64_t off, float v[8]) {
    const float* q = reinterpret_cast<const float*>(base) + off;
    const float4 a = *reinterpret_cast<const float4*>(q);
    const float4 b = *reinterpret_cast<const float4*>(q + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

template <int EPI, typename T, typename OutT>
__device__ __forceinline__ void epilogue8(const EpiArgs& ea, int e, int64_t m, int64_t n,
                                          const float c[8]) {
  if constexpr (EPI == EPI_STORE) {
    Vec8<OutT>::store(ea.out0, e * ea.bstride + m * ea.ld0 + n, c);
  } else if constexpr (EPI == EPI_STORE_SPLIT) {
    if (n < ea.split)
      Vec8<OutT>::store(ea.out0, e * ea.bstride + m * ea.ld0 + n, c);
    else
      Vec8<OutT>::store(ea.out1, e * ea.bstride + m * ea.ld1 + (n - ea.split), c);
  } else if constexpr (EPI == EPI_ACC || EPI == EPI_ACC_SPLIT) {
    void* o = ea.out0;
    int64_t off = e * ea.bstride + m * ea.ld0 + n;
    if (EPI == EPI_ACC_SPLIT && n >= ea.split) {
      o = ea.out1;
      off = e * ea.bstride + m * ea.ld1 + (n - ea.split);
    }
    float v[8];
    Vec8<OutT>::load(o, off, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] += c[i];
    Vec8<OutT>::store(o, off, v);
  } else if constexpr (EPI == EPI_GELU_FWD) {
    float h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = gelu_f(c[i]);
    if (ea.out0) Vec8<T>::store(ea.out0, m * ea.ld0 + n, c);
    Vec8<T>::store(ea.out1, m * ea.ld1 + n, h);
  } else if constexpr (EPI == EPI_GELU_BWD) {
    float z[8], d[8];
    Vec8<T>::load(ea.aux, m * ea.ldaux + n, z);
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = c[i] * gelu_grad_f(z[i]);
    Vec8<T>::store(ea.out0, m * ea.ld0 + n, d);
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    float g[8], u[8], dg[8], du[8];
    Vec8<T>::load(ea.aux, m * ea.ldaux + n, g);
    Vec8<T>::load(ea.aux, m * ea.ldaux + ea.split + n, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float s = sigmoid_f(g[i]);
      dg[i] = c[i] * u[i] * (s * (1.0f + g[i] * (1.0f - s)));
      du[i] = c[i] * (g[i] * s);
    }
    Vec8<T>::store(ea.out0, m * ea.ld0 + n, dg);
    Vec8<T>::store(ea.out0, m * ea.ld0 + ea.split + n, du);
  }
}

template <typename T>
__device__ __forceinline__ void epilogue_swiglu8(const EpiArgs& ea, int64_t m, int64_t f,
                                                 const float g[8], const float u[8]) {
  float h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = silu_f(g[i]) * u[i];
  if (ea.out0) {
    Vec8<T>::store(ea.out0, m * ea.ld0 + f, g);
    Vec8<T>::store(ea.out0, m * ea.ld0 + ea.split + f, u);
  }
  Vec8<T>::store(ea.out1, m * ea.ld1 + f, h);
}

// ---------------------------------------------------------------------------
// FP8 codes (OCP E4M3 / E5M2): round-to-nearest-even of clamp(x * s) with
// gfx950's packed converts; four values per 32-bit word, first in the low
// byte
// ---------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d, float s) {
  constexpr float VMAX = FMT == 0 ? 448.0f : 57344.0f;
  a = fminf(fmaxf(a * s, -VMAX), VMAX);
  b = fminf(fmaxf(b * s, -VMAX), VMAX);
  c = fminf(fmaxf(c * s, -VMAX), VMAX);
  d = fminf(fmaxf(d * s, -VMAX), VMAX);
  int w;
  if constexpr (FMT == 0) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// FP8 forward epilogues: as the bf16 ones, and H is also written as the
// E4M3 codes of H * hs (out2, 8 bytes per 8 columns) with max |H| tracked
__device__ __forceinline__ void store_h_e4m3(const EpiArgs& ea, int64_t m, int64_t f,
                                             const float h[8], float hs, float& amax) {
  uint2 q;
  q.x = fp8x4<0>(h[0], h[1], h[2], h[3], hs);
  q.y = fp8x4<0>(h[4], h[5], h[6], h[7], hs);
  *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(ea.out2) + m * ea.ld2 + f) = q;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(h[i]));
}

template <typename T>
__device__ __forceinline__ void epilogue_swiglu8_q(const EpiArgs& ea, int64_t m, int64_t f,
                                                   const float g[8], const float u[8], float hs,
                                                   float& amax) {
  float h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = silu_f(g[i]) * u[i];
  if (ea.out0) {
    Vec8<T>::store(ea.out0, m * ea.ld0 + f, g);
    Vec8<T>::store(ea.out0, m * ea.ld0 + ea.split + f, u);
  }
  Vec8<T>::store(ea.out1, m * ea.ld1 + f, h);
  store_h_e4m3(ea, m, f, h, hs, amax);
}

template <typename T>
__device__ __forceinline__ void epilogue_gelu8_q(const EpiArgs& ea, int64_t m, int64_t n,
                                                 const float z[8], float hs, float& amax) {
  float h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = gelu_f(z[i]);
  if (ea.out0) Vec8<T>::store(ea.out0, m * ea.ld0 + n, z);
  Vec8<T>::store(ea.out1, m * ea.ld1 + n, h);
  store_h_e4m3(ea, m, n, h, hs, amax);
}

// FP8 backward: activation derivative from the saved bf16 Z (as
// EPI_GELU_BWD / EPI_SWIGLU_BWD), written as E5M2 codes of dZ * qscale to
// out2 (pitch ld2; SwiGLU: dG at n, dU at split + n), max |dZ| tracked
template <int EPI>
__device__ __forceinline__ void epilogue_dact8_q(const EpiArgs& ea, int64_t m, int64_t n,
                                                 const float c[8], float qscale, float& amax) {
  uint8_t* o = reinterpret_cast<uint8_t*>(ea.out2);
  if constexpr (EPI == EPI_GELU_BWD) {
    float z[8], d[8];
    Vec8<bf16_t>::load(ea.aux, m * ea.ldaux + n, z);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      d[i] = c[i] * gelu_grad_f(z[i]);
      amax = fmaxf(amax, fabsf(d[i]));
    }
    uint2 q;
    q.x = fp8x4<1>(d[0], d[1], d[2], d[3], qscale);
    q.y = fp8x4<1>(d[4], d[5], d[6], d[7], qscale);
    *reinterpret_cast<uint2*>(o + m * ea.ld2 + n) = q;
  } else {
    float g[8], u[8], dg[8], du[8];
    Vec8<bf16_t>::load(ea.aux, m * ea.ldaux + n, g);
    Vec8<bf16_t>::load(ea.aux, m * ea.ldaux + ea.split + n, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float s = sigmoid_f(g[i]);
      dg[i] = c[i] * u[i] * (s * (1.0f + g[i] * (1.0f - s)));
      du[i] = c[i] * (g[i] * s);
      amax = fmaxf(amax, fmaxf(fabsf(dg[i]), fabsf(du[i])));
    }
    uint2 q;
    q.x = fp8x4<1>(dg[0], dg[1], dg[2], dg[3], qscale);
    q.y = fp8x4<1>(dg[4], dg[5], dg[6], dg[7], qscale);
    *reinterpret_cast<uint2*>(o + m * ea.ld2 + n) = q;
    q.x = fp8x4<1>(du[0], du[1], du[2], du[3], qscale);
    q.y = fp8x4<1>(du[4], du[5], du[6], du[7], qscale);
    *reinterpret_cast<uint2*>(o + m * ea.ld2 + ea.split + n) = q;
  }
}

// max over a workgroup of NT threads, folded into *p by one atomic max on
// the bits (non-negative floats order like their bit patterns); red holds
// NT / 64 floats of shared memory; every thread of the workgroup calls it
template <int NT>
__device__ __forceinline__ void fold_amax_block(float m, float* p, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) t = fmaxf(t, red[w]);
    atomicMax(reinterpret_cast<unsigned int*>(p), __float_as_uint(t));
  }
}

}  // namespace tpmlp
