// bf16 MFMA GEMM for gfx950 with the shard's fused epilogues.
//
// Block tile 256 x 256 x 64 (one block per CU: two 64 KiB shared-memory
// tile buffers), 8 wavefronts in a 2 x 4 grid, each owning 128 x 64
// outputs computed as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16.
//
// Operand tiles go from memory straight into shared memory (buffer loads
// with the LDS destination; out-of-range offsets read as zeros, so tile
// edges need no branches).  A K-contiguous operand is stored row by row
// (64 k = eight 16-byte chunks, chunk c of row r at c ^ swz(r)) and its
// MFMA fragments are 16-byte reads; an M/N-contiguous operand keeps its
// memory orientation ([half][k][granule], XOR-swizzled by k) and its
// fragments come from transposing LDS reads (ds_read_b64_tr_b16).  Either
// way each lane receives 8 consecutive k of one row or column, so the
// MFMA sees the same operand order for every memory layout.
//
// Two tile buffers alternate: while the MFMAs consume one, the next k
// tile's loads are in flight into the other (spread over the k steps),
// and the next k step's fragments are read while the current step's MFMAs
// run.  One barrier per 64-wide k tile.
//
// The MFMA is issued with the B fragment as its first operand, which
// yields C^T blocks: each lane then holds 4 consecutive output columns of
// one row, and the epilogue stores 8 (bf16) or 16 (fp32) contiguous bytes.
#include "common.h"
#include "launch.h"

namespace tpmlp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Issue priority of the GEMM wavefronts (0..3) over other kernels' waves
// sharing their SIMDs (e.g. a partial sum on a second stream): a GEMM runs
// one wavefront per SIMD on a hand-ordered schedule, and a co-resident
// stream of loads would otherwise take its issue slots (measured on the
// shard steps with the sums overlapped: 2.065 -> 2.049 ms SwiGLU, 1.013 ->
// 0.990 ms GeLU; unchanged when nothing else runs).
#ifndef TP_GEMM_WAVE_PRIO
#define TP_GEMM_WAVE_PRIO 3
#endif
__device__ __forceinline__ void gemm_wave_prio() {
  if constexpr (TP_GEMM_WAVE_PRIO > 0) __builtin_amdgcn_s_setprio(TP_GEMM_WAVE_PRIO);
}
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace mfma256 {

constexpr int BM = 256, BN = 256, BK = 64;
// Wavefront layouts of the block tile:
//  NW = 4: 2 x 2 wavefronts of 128 x 128 (4 x 4 MFMA blocks, 256 fp32
//          accumulators each, one wavefront per SIMD): fragment reads need
//          0.5 KiB of shared memory per MFMA.
//  NW = 8: 2 x 4 wavefronts of 128 x 64 (two per SIMD: one issues MFMAs
//          while the other waits), 0.75 KiB per MFMA.
// Shared memory serves ~128 B/clk per CU, and the direct loads write 0.25
// KiB per MFMA more, so NW = 8 runs close to that limit; fragment reads
// that transpose cost more than plain ones.
template <int NW>
struct Cfg {
  static constexpr int NWAVES = NW;
  static constexpr int WAVES_N = NW == 8 ? 4 : 2;
  static constexpr int WTM = 128, WTN = NW == 8 ? 64 : 128;  // wavefront tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int NT = 64 * NW;
  // 1 KiB direct loads per wavefront and operand tile (32 per tile)
  static constexpr int LDW = (BM * BK * 2 / 1024) / NW;
  // 16-byte register-staged chunks per thread and operand tile
  static constexpr int STAGE_N = BM * BK / 8 / NT;
};
constexpr int TILE_ELEMS = (BM + BN) * BK;  // one buffer: A then B

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ int lds_off(int r, int c) {
  return r * BK + ((c ^ swz(r)) << 3);
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
// x 64 k, LDW x 1 KiB per wavefront (instructions I0..I1-1 of them here).  Within each 1 KiB block lane l fills
// the 16 bytes at l*16, i.e. row 8*blk + l/8 at physical chunk l%8, which
// holds logical chunk (l%8) ^ swz(row).  `rs` is based at (row 0, k 0) of
// the tile's row range; rows >= rows_valid and k >= k_lim read as zeros.
template <int NW, int I0, int I1>
__device__ __forceinline__ void direct_kmajor(rsrc_t rs, int64_t ld, int rows_valid,
                                              int k0, int k_lim, bf16_t* tile,
                                              int wave, int lane) {
#pragma unroll
  for (int i = I0; i < I1; ++i) {
    const int blk = wave * Cfg<NW>::LDW + i;
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

// Direct load of an M/N-contiguous tile (instructions I0..I1-1 of LDW per
// wavefront; the first half of the wavefronts fills half 0).  rs is based at (k row
// 0 of the tile, column 0 of this half's source matrix); the half covers
// columns col0 .. col0 + 127, valid below col_lim, rows below k_valid.
template <int NW, int I0, int I1>
__device__ __forceinline__ void direct_mn(rsrc_t rs, int64_t ld, int col0, int col_lim,
                                          int k_valid, bf16_t* tile, int wave, int lane) {
  const int half = wave / (NW / 2);
#pragma unroll
  for (int i = I0; i < I1; ++i) {
    const int b = (wave % (NW / 2)) * Cfg<NW>::LDW + i;
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

// ---- in-order main-loop primitives ----------------------------------------
// The k loop is written with these so that the compiler keeps the order
// chosen here: the LDS reads of the next k step are issued ahead of the
// current step's MFMAs, and a step waits for its own fragments only.  An
// LDS read issued here completes asynchronously: its registers are only
// used after lds_wait() has passed them through fence().
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// fragment of a K-contiguous tile: one 16-byte read
struct FragK {
  bf16x8_t v;
  __device__ __forceinline__ void read(uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  }
  __device__ __forceinline__ void fence() { asm volatile("" : "+v"(v)); }
  __device__ __forceinline__ bf16x8_t op() const { return v; }
};

// fragment of an M/N-contiguous tile: two transposing 8-byte reads
struct FragMN {
  i16x4_t lo, hi;
  __device__ __forceinline__ void read(uint32_t a_lo, uint32_t a_hi) {
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(a_lo));
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(hi) : "v"(a_hi));
  }
  __device__ __forceinline__ void fence() { asm volatile("" : "+v"(lo), "+v"(hi)); }
  __device__ __forceinline__ bf16x8_t op() const {
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void mfma_32x32x16(f32x16_t& acc, const bf16x8_t& a,
                                              const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// addresses of the two transposing reads of an M/N-contiguous fragment
__device__ __forceinline__ void frag_mn_addr(const bf16_t* tile, int c0, int k0, int lane,
                                             uint32_t& a_lo, uint32_t& a_hi) {
  const int g = lane >> 4, r = lane & 15;
  const int c = c0 + 16 * (g & 1) + 4 * (r & 3);
  const int k = k0 + 8 * (g >> 1) + (r >> 2);
  a_lo = lds_u32(tile + mn_off(k, c));
  a_hi = lds_u32(tile + mn_off(k + 4, c));
}

// Staging registers of one operand tile for one thread.
template <int NW>
struct Stage {
  uint4 v[Cfg<NW>::STAGE_N];
};

__device__ __forceinline__ uint4 load16_or_zero(const bf16_t* p, const bf16_t* safe, bool ok) {
  uint4 v = *reinterpret_cast<const uint4*>(ok ? p : safe);
  return ok ? v : make_uint4(0, 0, 0, 0);
}

// K-contiguous operand through registers (used when one tile would need
// two source matrices: a k split that is not a multiple of 64).
template <int NW, int BMODE>
__device__ __forceinline__ void load_k(const bf16_t* p0, const bf16_t* p1, int64_t ld,
                                       int64_t split, int r_base, int r_lim, int k0,
                                       int k_lim, int tid, Stage<NW>& s) {
#pragma unroll
  for (int i = 0; i < Cfg<NW>::STAGE_N; ++i) {
    const int c = tid + Cfg<NW>::NT * i;
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

template <int NW>
__device__ __forceinline__ void store_k(bf16_t* tile, int tid, const Stage<NW>& s) {
#pragma unroll
  for (int i = 0; i < Cfg<NW>::STAGE_N; ++i) {
    const int c = tid + Cfg<NW>::NT * i;
    const int r = c >> 3, kc = c & 7;
    *reinterpret_cast<uint4*>(tile + lds_off(r, kc)) = s.v[i];
  }
}

// ---- dZ operand formed from dH and the saved activations -----------------
// The operand tile is taken in STAGE_N pieces per thread of 8 elements
// each: dH and the saved Z (GeLU) or G and U (SwiGLU) at the same place are
// loaded into registers, and the 8 dZ values are formed from them on their
// way into shared memory (as bf16, where the direct loads would have put
// them).  Operand column f of [dG | dU] reads dH and G at f mod split and,
// for dG, U.  Masked pieces read as zeros, which give dZ = 0.  `split` is a
// multiple of 8, so no piece straddles it.  Two register slots take the
// pieces in turn (piece i in slot i % 2), which keeps 128 accumulators and
// the staging within the register file of two wavefronts per SIMD.
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));
template <int PRO>
struct DactStage {
  u32x4v_t dh[2], z0[2], z1[PRO == DACT_SWIGLU ? 2 : 1];
};

// Piece loads are buffer loads with 32-bit offsets from per-tile bases
// (rd: dH, rz: the saved activations), `row` counted from the base; a
// masked piece takes an out-of-range offset and reads zeros.
template <int PRO>
__device__ __forceinline__ void dact_load(rsrc_t rd, rsrc_t rz, int64_t ld, int64_t split,
                                          int row, int64_t f, bool ok, bool second, int slot,
                                          DactStage<PRO>& s) {
  const int64_t zld = PRO == DACT_SWIGLU ? 2 * split : split;
  const uint32_t od = ok ? (uint32_t)((row * ld + f) * 2) : OOB_OFF;
  const uint32_t oz = ok ? (uint32_t)((row * zld + f) * 2) : OOB_OFF;
  s.dh[slot] = __builtin_amdgcn_raw_buffer_load_b128(rd, od, 0, 0);
  s.z0[slot] = __builtin_amdgcn_raw_buffer_load_b128(rz, oz, 0, 0);
  if constexpr (PRO == DACT_SWIGLU)
    s.z1[slot] = __builtin_amdgcn_raw_buffer_load_b128(rz, second ? OOB_OFF : oz,
                                                       (int)(split * 2), 0);
}

template <int PRO>
__device__ __forceinline__ uint4 dact_form(const DactStage<PRO>& s, int slot, bool second) {
  uint32_t o[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t wd = s.dh[slot][p], wz = s.z0[slot][p];
    const uint32_t wu = PRO == DACT_SWIGLU ? s.z1[slot][p] : 0u;
    const float lo = dact_elem<PRO>(__uint_as_float(wd << 16), __uint_as_float(wz << 16),
                                    __uint_as_float(wu << 16), second);
    const float hi = dact_elem<PRO>(__uint_as_float(wd & 0xffff0000u),
                                    __uint_as_float(wz & 0xffff0000u),
                                    __uint_as_float(wu & 0xffff0000u), second);
    o[p] = pack_bf16x2(lo, hi);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// K-contiguous dZ tile (256 rows x 64 k; bases at the tile's first row):
// piece c = tid + NT i covers row c / 8, k chunk c % 8
template <int NW, int PRO>
__device__ __forceinline__ void dact_load_k(rsrc_t rd, rsrc_t rz, int64_t ld, int64_t split,
                                            int rows_valid, int k0, int k_lim, int tid, int i,
                                            DactStage<PRO>& s) {
  const int c = tid + Cfg<NW>::NT * i;
  const int r = c >> 3, k = k0 + (c & 7) * 8;
  const bool second = PRO == DACT_SWIGLU && k >= split;
  dact_load<PRO>(rd, rz, ld, split, r, second ? k - split : k, r < rows_valid && k < k_lim,
                 second, i & 1, s);
}
template <int NW, int PRO>
__device__ __forceinline__ void dact_store_k(bf16_t* tile, int tid, int k0, int64_t split, int i,
                                             const DactStage<PRO>& s) {
  const int c = tid + Cfg<NW>::NT * i;
  const int r = c >> 3, kc = c & 7;
  const bool second = PRO == DACT_SWIGLU && k0 + kc * 8 >= split;
  *reinterpret_cast<uint4*>(tile + lds_off(r, kc)) = dact_form<PRO>(s, i & 1, second);
}

// M/N-contiguous dZ tile (64 k rows x 256 columns; bases at the tile's
// first k row): piece c covers k row c / 32, columns 8 (c % 32) ..
template <int NW, int PRO>
__device__ __forceinline__ void dact_load_mn(rsrc_t rd, rsrc_t rz, int64_t ld, int64_t split,
                                             int n_base, int n_lim, int k_valid, int tid, int i,
                                             DactStage<PRO>& s) {
  const int c = tid + Cfg<NW>::NT * i;
  const int kr = c >> 5, n = n_base + (c & 31) * 8;
  const bool second = PRO == DACT_SWIGLU && n >= split;
  dact_load<PRO>(rd, rz, ld, split, kr, second ? n - split : n, kr < k_valid && n < n_lim,
                 second, i & 1, s);
}
template <int NW, int PRO>
__device__ __forceinline__ void dact_store_mn(bf16_t* tile, int tid, int n_base, int64_t split,
                                              int i, const DactStage<PRO>& s) {
  const int c = tid + Cfg<NW>::NT * i;
  const int kr = c >> 5, col = (c & 31) * 8;
  const bool second = PRO == DACT_SWIGLU && n_base + col >= split;
  *reinterpret_cast<uint4*>(tile + mn_off(kr, col)) = dact_form<PRO>(s, i & 1, second);
}

// ---- epilogue through shared memory ----------------------------------------
// The tile is written out in passes of 64 rows (four for 256-row tiles, two
// for 128-row ones).  In each pass the wavefronts holding those rows store their fp32 sums row-major in shared
// memory (rows padded by 16 bytes, so a wavefront's 16-byte writes spread
// over all banks), then every thread takes 8 consecutive columns of a row:
// saved activations are loaded and outputs stored as 16-byte pieces of
// contiguous rows.  For the paired SwiGLU forward the gate sums go to
// columns 0..127 and the up sums to 128..255 of the staged rows.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int EQ_ROWS = 64;
constexpr int EQ_PITCH = BN + 4;  // floats
constexpr int EQ_BYTES = EQ_ROWS * EQ_PITCH * 4;

// QM (FP8 only): 1 = forward FC1 (sums scaled by x_inv a_inv, resp.
// x_inv au_inv for the up projection; H also written as E4M3 codes of
// H h_scale, max |H| folded into ea.amax), 2 = forward FC2 (sums scaled by
// (1 / h_scale) b_inv), 3 = backward, sums scaled by qs[qi] qs[qj], 4 =
// backward dH: scaled as 3, then the activation derivative written as
// E5M2 codes of dZ qs[qk] with max |dZ| folded into ea.amax
template <int EPI, int BMODE, typename OutT, int FM, int FN, int WTM, int WTN, int NT, int QM = 0,
          int NPASS = 4>
__device__ __forceinline__ void write_tile_staged(const f32x16_t (&acc)[FM][FN],
                                                  const EpiArgs& ea, const TileCoord& tc,
                                                  int wm, int wn, int lane, int tid, int Ncols,
                                                  float* stage) {
  static_assert(WTM == 128 && FM == 4, "passes of 64 rows take two 32-row fragment rows");
  constexpr bool PAIR = EPI == EPI_SWIGLU_FWD;
  const int r_lane = lane & 31, c_lane = lane >> 5;
  float s0 = 1.0f, s1 = 1.0f, hs = 1.0f, amax = 0.0f;
  if constexpr (QM == 1) {
    s0 = ea.qs[0] * ea.qs[1];
    s1 = ea.qs[0] * ea.qs[2];
    hs = ea.qs[4];
  } else if constexpr (QM == 2) {
    s0 = (1.0f / ea.qs[4]) * ea.qs[3];
  } else if constexpr (QM == 3 || QM == 4) {
    s0 = ea.qs[ea.qi] * ea.qs[ea.qj];
    if constexpr (QM == 4) hs = ea.qs[ea.qk];
  }
  static_for<0, NPASS>([&](auto Qc) {
    constexpr int q = decltype(Qc)::value;
    if (wm == q / 2) {
      static_for<0, 2>([&](auto Ic) {
        constexpr int ii = decltype(Ic)::value, i = 2 * (q % 2) + ii;
        const int row = ii * 32 + r_lane;
        static_for<0, FN>([&](auto Jc) {
          constexpr int j = decltype(Jc)::value;
          const int col0 = PAIR ? (j & 1) * (BN / 2) + wn * (WTN / 2) + (j >> 1) * 32
                                : wn * WTN + j * 32;
          static_for<0, 4>([&](auto Gc) {
            constexpr int gq = decltype(Gc)::value;
            const f32x4_t v = {acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                               acc[i][j][4 * gq + 3]};
            *reinterpret_cast<f32x4_t*>(stage + row * EQ_PITCH + col0 + 8 * gq + 4 * c_lane) = v;
          });
        });
      });
    }
    __syncthreads();
    const int64_t m0 = tc.m_begin + EQ_ROWS * q;
    if constexpr (PAIR) {
      constexpr int CH = EQ_ROWS * (BN / 2) / 8;
      static_for<0, CH / NT>([&](auto Kc) {
        const int k = decltype(Kc)::value * NT + tid;
        const int row = k >> 4, cc = (k & 15) * 8;
        const int64_t m = m0 + row;
        const int64_t f = (int64_t)tc.tn * (BN / 2) + cc;
        if (m < tc.m_end && f < ea.split) {
          float gv[8], uv[8];
          const float* src = stage + row * EQ_PITCH + cc;
          *reinterpret_cast<f32x4_t*>(gv) = *reinterpret_cast<const f32x4_t*>(src);
          *reinterpret_cast<f32x4_t*>(gv + 4) = *reinterpret_cast<const f32x4_t*>(src + 4);
          *reinterpret_cast<f32x4_t*>(uv) = *reinterpret_cast<const f32x4_t*>(src + BN / 2);
          *reinterpret_cast<f32x4_t*>(uv + 4) = *reinterpret_cast<const f32x4_t*>(src + BN / 2 + 4);
          if constexpr (QM == 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) { gv[e] *= s0; uv[e] *= s1; }
            epilogue_swiglu8_q<bf16_t>(ea, m, f, gv, uv, hs, amax);
          } else {
            epilogue_swiglu8<bf16_t>(ea, m, f, gv, uv);
          }
        }
      });
    } else {
      constexpr int CH = EQ_ROWS * BN / 8;
      static_for<0, CH / NT>([&](auto Kc) {
        const int k = decltype(Kc)::value * NT + tid;
        const int row = k >> 5, cc = (k & 31) * 8;
        const int64_t m = m0 + row;
        const int64_t n = (int64_t)tc.tn * BN + cc;
        if (m < tc.m_end && n < Ncols) {
          float cv[8];
          const float* src = stage + row * EQ_PITCH + cc;
          *reinterpret_cast<f32x4_t*>(cv) = *reinterpret_cast<const f32x4_t*>(src);
          *reinterpret_cast<f32x4_t*>(cv + 4) = *reinterpret_cast<const f32x4_t*>(src + 4);
          if constexpr (QM != 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) cv[e] *= s0;
          }
          if constexpr (QM == 1 && EPI == EPI_GELU_FWD)
            epilogue_gelu8_q<bf16_t>(ea, m, n, cv, hs, amax);
          else if constexpr (QM == 4)
            epilogue_dact8_q<EPI>(ea, m, n, cv, hs, amax);
          else
            epilogue8<EPI, bf16_t, OutT>(ea, tc.e, m, n, cv);
        }
      });
    }
    // the next pass rewrites the staging rows
    __syncthreads();
  });
  if constexpr (QM == 1 || QM == 4) {
    // the staging rows are free after the last pass's barrier
    if (ea.amax) fold_amax_block<NT>(amax, ea.amax, stage);
  }
}

// ---- kernel ----------------------------------------------------------------
// A_KMAJOR: opA K-contiguous or M-contiguous, loaded straight into shared
// memory.  B likewise; B_DIRECT selects the direct path for a K-contiguous
// opB (a k split must then be a multiple of 64 so each k tile comes from
// one matrix; otherwise opB goes through registers).
// PA / PB (DACT_*): opA (K-contiguous) or opB (M/N-contiguous) is a dZ
// formed from dH and the saved activations as it is loaded, through
// registers, in 4 pieces per thread and k tile.  While the MFMAs consume
// one tile: pieces 0 and 1 of the next are loaded with the other operand's
// direct loads at k step 0, piece i is formed into shared memory at step
// i + 1 (pieces 2 and 3 at the last step, before the barrier), and piece
// i + 2 is loaded into the register slot piece i has left.  The vector work
// is spread over the k steps, beside the other wavefront's MFMAs on the
// same SIMD.
template <int NW, bool A_KMAJOR, bool B_KMAJOR, int BMODE, int EPI, typename OutT, bool B_DIRECT,
          int PA = DACT_NONE, int PB = DACT_NONE>
__global__ __launch_bounds__(64 * NW, 1) void gemm_kernel(GemmArgs g) {
  static_assert(PA == DACT_NONE || (A_KMAJOR && PB == DACT_NONE), "dZ as K-contiguous opA");
  static_assert(PB == DACT_NONE || (!B_KMAJOR && BMODE == BMODE_PLAIN), "dZ as M/N-contiguous opB");
  gemm_wave_prio();
  using C = Cfg<NW>;
  constexpr int NWAVES = C::NWAVES, WAVES_N = C::WAVES_N, WTM = C::WTM, WTN = C::WTN;
  constexpr int FM = C::FM, FN = C::FN, LDW = C::LDW;
  __shared__ __attribute__((aligned(1024))) bf16_t lds[2 * TILE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wavefront index is uniform: keep it (and what derives from it) scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int half_w = wave / (NWAVES / 2);  // tile half this wavefront loads

  const TileCoord tc = locate_tile(g, blockIdx.x, gridDim.x, BM);
  if (tc.e < 0) return;  // spare tile (device-resident offsets)
  const bf16_t* a0 = reinterpret_cast<const bf16_t*>(g.a.p0) + tc.e * g.a.bstride;
  const bf16_t* b0 = reinterpret_cast<const bf16_t*>(g.b.p0) + tc.e * g.b.bstride;
  const bf16_t* b1 = reinterpret_cast<const bf16_t*>(g.b.p1) + tc.e * g.b.bstride;
  // scalar copies of the argument block: helpers never see its address
  const int64_t lda = g.a.ld, ldb = g.b.ld, bsplit = g.b.split;
  const int Ncols = g.N, Ktot = g.K;
  const EpiArgs ea = g.epi;
  const int n_base = tc.tn * BN;
  const int m_rows = tc.m_end - tc.m_begin;
  // the dZ operand's dH, saved activations and split (dense problems only)
  constexpr int PRO = PA != DACT_NONE ? PA : PB;
  const bf16_t* d_dh = PA != DACT_NONE ? a0 : b0;
  const bf16_t* d_zs = reinterpret_cast<const bf16_t*>(PA != DACT_NONE ? g.a.p1 : g.b.p1);
  const int64_t d_ld = PA != DACT_NONE ? lda : ldb;
  const int64_t d_split = PA != DACT_NONE ? g.a.split : bsplit;
  static_assert(PRO == DACT_NONE || C::STAGE_N == BK / 16, "one dZ piece per k step");
  DactStage<PRO == DACT_NONE ? DACT_GELU : PRO> ds;
  // load / form dZ piece i of the k tile starting at k0
  const int64_t d_zld = PRO == DACT_SWIGLU ? 2 * d_split : d_split;
  auto dload = [&](int i, int k0) {
    if constexpr (PA != DACT_NONE)
      dact_load_k<NW, PA>(make_rsrc(d_dh + (int64_t)tc.m_begin * d_ld),
                          make_rsrc(d_zs + (int64_t)tc.m_begin * d_zld), d_ld, d_split, m_rows,
                          k0, tc.k_end, tid, i, ds);
    if constexpr (PB != DACT_NONE)
      dact_load_mn<NW, PB>(make_rsrc(d_dh + (int64_t)k0 * d_ld),
                           make_rsrc(d_zs + (int64_t)k0 * d_zld), d_ld, d_split, n_base, Ncols,
                           tc.k_end - k0, tid, i, ds);
  };
  auto dform = [&](int i, int k0, bf16_t* buf) {
    if constexpr (PA != DACT_NONE) dact_store_k<NW, PA>(buf, tid, k0, d_split, i, ds);
    if constexpr (PB != DACT_NONE) dact_store_mn<NW, PB>(buf + BM * BK, tid, n_base, d_split, i, ds);
  };

  f32x16_t acc[FM][FN];
  static_for<0, FM>([&](auto I) {
    static_for<0, FN>([&](auto J) { acc[I][J] = (f32x16_t)(0.0f); });
  });

  const int nk = (tc.k_end > tc.k_begin) ? (tc.k_end - tc.k_begin + BK - 1) / BK : 0;

  Stage<NW> sb;  // only for a K-contiguous opB whose k split is not 64-aligned
  // Loads of the k tile starting at k0 into buffer `buf`, instructions
  // I0..I1-1 of each wavefront's 8 per operand.  k0 >= k_end masks every
  // load (the tile past the last one reads as zeros and is never used).
  auto issue = [&](auto I0c, auto I1c, int k0, bf16_t* buf) {
    constexpr int I0 = decltype(I0c)::value, I1 = decltype(I1c)::value;
    if constexpr (PA != DACT_NONE) {
      if constexpr (I0 == 0) {
        dload(0, k0);
        dload(1, k0);
      }
    } else if constexpr (A_KMAJOR) {
      direct_kmajor<NW, I0, I1>(make_rsrc(a0 + (int64_t)tc.m_begin * lda), lda, m_rows, k0,
                            tc.k_end, buf, wave, lane);
    } else {
      direct_mn<NW, I0, I1>(make_rsrc(a0 + (int64_t)k0 * lda), lda,
                        tc.m_begin + half_w * 128, tc.m_end, tc.k_end - k0, buf, wave,
                        lane);
    }
    bf16_t* tb = buf + BM * BK;
    if constexpr (B_KMAJOR && B_DIRECT) {
      if constexpr (BMODE == BMODE_KSPLIT) {
        // a 64-aligned split: the whole k tile comes from one matrix
        const bool first = k0 < bsplit;
        const bf16_t* bp = first ? b0 : b1;
        const int kl = first ? k0 : k0 - (int)bsplit;
        const int lim = first ? (int)bsplit : Ktot - (int)bsplit;
        direct_kmajor<NW, I0, I1>(make_rsrc(bp + (int64_t)n_base * ldb), ldb, Ncols - n_base, kl,
                              k0 < tc.k_end ? lim : 0, tb, wave, lane);
      } else {
        direct_kmajor<NW, I0, I1>(make_rsrc(b0 + (int64_t)n_base * ldb), ldb, Ncols - n_base, k0,
                              tc.k_end, tb, wave, lane);
      }
    } else if constexpr (B_KMAJOR) {
      if constexpr (I0 == 0)
        load_k<NW, BMODE>(b0, b1, ldb, bsplit, n_base, Ncols, k0, tc.k_end, tid, sb);
    } else if constexpr (PB != DACT_NONE) {
      if constexpr (I0 == 0) {
        dload(0, k0);
        dload(1, k0);
      }
    } else if constexpr (BMODE == BMODE_PAIR32) {
      // half 0: gate columns, half 1: up columns, both f = 128 tn ..
      const bf16_t* bp = half_w ? b1 : b0;
      direct_mn<NW, I0, I1>(make_rsrc(bp + (int64_t)k0 * ldb), ldb, tc.tn * 128, (int)bsplit,
                        tc.k_end - k0, tb, wave, lane);
    } else {
      direct_mn<NW, I0, I1>(make_rsrc(b0 + (int64_t)k0 * ldb), ldb, n_base + half_w * 128,
                        Ncols, tc.k_end - k0, tb, wave, lane);
    }
  };
  constexpr int NSTEP = BK / 16;
  // at the last k step (before the loop, `first`: every piece in turn) the
  // register-staged operand goes to shared memory
  auto commit = [&](bf16_t* buf, int k0, bool first) {
    if constexpr (B_KMAJOR && !B_DIRECT) store_k(buf + BM * BK, tid, sb);
    if constexpr (PRO != DACT_NONE) {
      if (first) {
        static_for<0, NSTEP - 2>([&](auto Ic) {
          constexpr int i = decltype(Ic)::value;
          dform(i, k0, buf);
          dload(i + 2, k0);
        });
      }
      dform(NSTEP - 2, k0, buf);
      dform(NSTEP - 1, k0, buf);
    }
  };

  const int r_lane = lane & 31;
  const int c_lane = lane >> 5;
  // tile column of opB block j of this wavefront
  auto b_col = [&](int j) {
    if constexpr (BMODE == BMODE_PAIR32) return (j & 1) * 128 + wn * (WTN / 2) + (j >> 1) * 32;
    else return wn * WTN + j * 32;
  };
  using FA = typename std::conditional<A_KMAJOR, FragK, FragMN>::type;
  using FB = typename std::conditional<B_KMAJOR, FragK, FragMN>::type;
  FA fa[2][FM];
  FB fb[2][FN];
  // issue the LDS reads of k step s of tile `buf` into fragment slot `slot`
  auto read_frags = [&](const bf16_t* buf, int s, int slot) {
    const int c = 2 * s + c_lane;
    const bf16_t* la = buf;
    const bf16_t* lb = buf + BM * BK;
    static_for<0, FM>([&](auto I) {
      if constexpr (A_KMAJOR) {
        fa[slot][I].read(lds_u32(la + lds_off(wm * WTM + I * 32 + r_lane, c)));
      } else {
        uint32_t lo, hi;
        frag_mn_addr(la, wm * WTM + I * 32, 16 * s, lane, lo, hi);
        fa[slot][I].read(lo, hi);
      }
    });
    static_for<0, FN>([&](auto J) {
      if constexpr (B_KMAJOR) {
        fb[slot][J].read(lds_u32(lb + lds_off(wn * WTN + J * 32 + r_lane, c)));
      } else {
        uint32_t lo, hi;
        frag_mn_addr(lb, b_col(J), 16 * s, lane, lo, hi);
        fb[slot][J].read(lo, hi);
      }
    });
  };
  auto fence_frags = [&](int slot) {
    lds_wait();
    static_for<0, FM>([&](auto I) { fa[slot][I].fence(); });
    static_for<0, FN>([&](auto J) { fb[slot][J].fence(); });
  };

  if (nk > 0) {
    issue(std::integral_constant<int, 0>{}, std::integral_constant<int, LDW>{}, tc.k_begin, lds);
    commit(lds, tc.k_begin, true);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  if (nk > 0) read_frags(lds, 0, 0);
  // accumulators were zeroed by VALU writes: cover the write-to-MFMA gap
  asm volatile("s_nop 4");

  for (int kt = 0; kt < nk; ++kt) {
    bf16_t* cur = lds + (kt & 1) * TILE_ELEMS;
    bf16_t* nxt = lds + ((kt + 1) & 1) * TILE_ELEMS;
    // next tile's start; past the end on the last iteration (masked loads)
    const int kn = tc.k_begin + (kt + 1) * BK;
    static_for<0, NSTEP>([&](auto S) {
      constexpr int s = decltype(S)::value;
      constexpr int slot = s & 1;
      fence_frags(slot);
      if constexpr (s == 0) {
        issue(std::integral_constant<int, 0>{}, std::integral_constant<int, LDW>{}, kn, nxt);
      }
      if constexpr (s + 1 < NSTEP) {
        read_frags(cur, s + 1, slot ^ 1);
        // `nxt` is free since the last barrier: form dZ piece s - 1 into it
        // and load piece s + 1 into the registers that piece held
        if constexpr (PRO != DACT_NONE && s >= 1) {
          dform(s - 1, kn, nxt);
          dload(s + 1, kn);
        }
      } else {
        // every wavefront is done reading `cur` and its loads into `nxt`
        // have landed: after the barrier, read the next tile's first step
        // while this step's MFMAs run
        commit(nxt, kn, false);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        read_frags(nxt, 0, slot ^ 1);
      }
      static_for<0, FM>([&](auto I) {
        static_for<0, FN>([&](auto J) {
          mfma_32x32x16(acc[I][J], fb[slot][J].op(), fa[slot][I].op());
        });
      });
    });
  }
  // the last iteration's reads of the (unused) next tile may still be in
  // flight into fragment registers, and the last MFMAs' results are read by
  // the epilogue's VALU code: drain both before the registers are reused
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");

  // every wavefront is past its last shared-memory read before the tile
  // is staged through shared memory
  static_assert(EQ_BYTES <= (int)sizeof(lds), "staging rows exceed shared memory");
  __syncthreads();
  write_tile_staged<EPI, BMODE, OutT, FM, FN, WTM, WTN, 64 * NW>(
      acc, ea, tc, wm, wn, lane, tid, Ncols, reinterpret_cast<float*>(lds));
}

// ---- lean kernel: 4 wavefronts of 128 x 128, hand-ordered k loop ----------
//
// One wavefront per SIMD owns 128 x 128 outputs (4 x 4 MFMA blocks, 256
// accumulators): fragment reads cost 0.5 KiB of shared memory per MFMA, so
// reads plus the direct-load writes stay near 75 % of the LDS bandwidth at
// full MFMA rate.  With a single wavefront per SIMD nothing hides a stall,
// so every instruction of the k loop is placed by hand: each MFMA is
// followed by at most three memory instructions (LDS reads for the k step
// two ahead, and at the third k step the direct loads of the tile after
// next); the barrier sits before the third k step, so reads get two steps
// of latency and loads a whole tile.  All per-lane offsets are loop invariant: k
// advances through the buffer load's scalar offset (K-contiguous operands)
// or the buffer base (M/N-contiguous, whose k tail the buffer range masks),
// and k step / buffer parity are immediate offsets of the LDS reads.
// Shared memory: [A buffer 0 | A buffer 1 | B buffer 0 | B buffer 1].
// Requirements (checked by the launcher): a K-contiguous operand has K a
// multiple of 64, and a k split is a multiple of 64.

constexpr int LEAN_NT = 256;
constexpr int W16_NT = 256;
constexpr int TILE_BYTES = BM * BK * 2;  // one operand tile, 32 KiB

template <int OFF>
__device__ __forceinline__ void ds_read_b128_at(bf16x8_t& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_read_tr_at(i16x4_t& v, uint32_t addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
// MFMA that also orders memory: direct loads issued between two of these
// stay where they were written
__device__ __forceinline__ void mfma_ordered(f32x16_t& acc, const bf16x8_t& a,
                                             const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b) : "memory");
}

__device__ __forceinline__ rsrc_t make_rsrc_n(const void* p, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)nbytes,
                                           0x00020000);
}

// byte count of a buffer resource, capped to the largest the kernels use
// (integer compare: keeps the resource in scalar registers)
__device__ __forceinline__ uint32_t clamp_records(int64_t bytes) {
  return bytes > (int64_t)0x7fffffff ? 0x7fffffffu : (uint32_t)bytes;
}


// Tile rows TMR: 256 (2 x 2 wavefronts of 128 x 128, two shared-memory
// stages) or 128 (1 x 4 wavefronts of 128 x 64, three stages).  A 128-row
// tile halves the work per tile for launches whose 256-row tiles would leave
// compute units idle; each of its k steps has half the MFMAs, so its loads
// are issued three tiles ahead instead of two, and its fragment reads cost
// 0.75 KiB of shared memory per MFMA instead of 0.5.  Each stage holds the
// A tile then the B tile.
template <int TMR>
struct LeanCfg {
  static constexpr int FM = 4, FN = TMR == 256 ? 4 : 2;
  static constexpr int WTM = 128, WTN = TMR == 256 ? 128 : 64;
  static constexpr int NBUF = TMR == 256 ? 2 : 3;
  static constexpr int A_BYTES = TMR * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  // 1 KiB direct loads per wavefront and k tile
  static constexpr int LA = A_BYTES / 4096, LB = B_BYTES / 4096, NL = LA + LB;
  // wavefronts per 128-column half of an M/N-contiguous A tile
  static constexpr int A_WPH = 4 * 128 / TMR;
};

// direct load `idx` of a k tile's sequence: A and B alternate while both
// have loads left (A0 B0 A1 B1 ...), then the rest of B
template <int LA>
constexpr int lean_load_seq(int idx) {
  return idx < 2 * LA ? ((idx & 1) ? LA + (idx >> 1) : (idx >> 1)) : idx;
}

// One output tile of the hand-ordered kernel (its prologue, k loop and
// epilogue) in the workgroup's shared memory `lds`.
template <int TMR, bool A_KMAJOR, bool B_KMAJOR, int BMODE, int EPI, typename OutT>
__device__ __forceinline__ void lean_tile(const GemmArgs& g, const TileCoord& tc, bf16_t* lds) {
  using C = LeanCfg<TMR>;
  constexpr int FM = C::FM, FN = C::FN, WTM = C::WTM, WTN = C::WTN, NBUF = C::NBUF;
  constexpr int LA = C::LA, LB = C::LB, NL = C::NL;
  constexpr uint32_t A_BYTES = C::A_BYTES, STAGE = C::STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = TMR == 256 ? wave >> 1 : 0, wn = TMR == 256 ? wave & 1 : wave;
  const int r_lane = lane & 31, c_lane = lane >> 5;

  const bf16_t* a0 = reinterpret_cast<const bf16_t*>(g.a.p0) + tc.e * g.a.bstride;
  const bf16_t* b0 = reinterpret_cast<const bf16_t*>(g.b.p0) + tc.e * g.b.bstride;
  const bf16_t* b1 = reinterpret_cast<const bf16_t*>(g.b.p1) + tc.e * g.b.bstride;
  const int64_t lda = g.a.ld, ldb = g.b.ld, bsplit = g.b.split;
  const int Ncols = g.N;
  const EpiArgs ea = g.epi;
  const int n_base = tc.tn * BN;
  const int m_rows = tc.m_end - tc.m_begin;
  const int nk = (tc.k_end > tc.k_begin) ? (tc.k_end - tc.k_begin + BK - 1) / BK : 0;

  const uint32_t lds0 = lds_u32(lds);

  // ---- loop-invariant direct-load offsets (bytes) and LDS destinations
  // (relative to the stage)
  // (sized for the largest case: arrays of a template-dependent size
  // captured by a generic lambda stop the host compiler from emitting the
  // kernel's launch stub)
  uint32_t voffA[8], voffB[8];
  uint32_t dstA[8], dstB[8];
  static_assert(LA <= 8 && LB <= 8, "direct loads per wavefront");
  static_for<0, LA>([&](auto Ic) {
    constexpr int i = decltype(Ic)::value;
    if constexpr (A_KMAJOR) {
      const int blk = wave * LA + i;
      const int r = blk * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      voffA[i] = r < m_rows ? (uint32_t)(((int64_t)r * lda + c * 8) * 2) : OOB_OFF;
      dstA[i] = blk * 1024;
    } else {
      const int half = wave / C::A_WPH, b = (wave % C::A_WPH) * LA + i;
      const int k = 4 * b + (lane >> 4);
      const int q = (lane & 15) ^ ((k & 3) << 2);
      const int col = tc.m_begin + half * 128 + 8 * q;
      voffA[i] = col < tc.m_end ? (uint32_t)(((int64_t)k * lda + col) * 2) : OOB_OFF;
      dstA[i] = half * (BK * 128 * 2) + b * 1024;
    }
  });
  static_for<0, LB>([&](auto Ic) {
    constexpr int i = decltype(Ic)::value;
    if constexpr (B_KMAJOR) {
      const int blk = wave * LB + i;
      const int r = blk * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      voffB[i] = r < Ncols - n_base ? (uint32_t)(((int64_t)r * ldb + c * 8) * 2) : OOB_OFF;
      dstB[i] = A_BYTES + blk * 1024;
    } else {
      const int half = wave >> 1, b = (wave & 1) * LB + i;
      const int k = 4 * b + (lane >> 4);
      const int q = (lane & 15) ^ ((k & 3) << 2);
      int col, lim;
      if constexpr (BMODE == BMODE_PAIR32) {
        col = tc.tn * 128 + 8 * q;
        lim = (int)bsplit;
      } else {
        col = n_base + half * 128 + 8 * q;
        lim = Ncols;
      }
      voffB[i] = col < lim ? (uint32_t)(((int64_t)k * ldb + col) * 2) : OOB_OFF;
      dstB[i] = A_BYTES + half * (BK * 128 * 2) + b * 1024;
    }
  });
  // buffer resources of the k tile starting at k0 (a past-the-end tile gets
  // an empty range: its loads read zeros)
  rsrc_t rsA, rsB;
  int soA = 0, soB = 0;
  auto set_tile = [&](int k0, bool valid) {
    if constexpr (A_KMAJOR) {
      rsA = make_rsrc_n(a0 + (int64_t)tc.m_begin * lda, valid ? 0x7fffffffu : 0u);
      soA = k0 * 2;
    } else {
      const int64_t rem = (int64_t)(tc.k_end - k0) * lda * 2;
      rsA = make_rsrc_n(a0 + (int64_t)k0 * lda,
                        valid ? clamp_records(rem) : 0u);
    }
    if constexpr (B_KMAJOR) {
      const bool first = BMODE != BMODE_KSPLIT || k0 < bsplit;
      const bf16_t* bp = first ? b0 : b1;
      rsB = make_rsrc_n(bp + (int64_t)n_base * ldb, valid ? 0x7fffffffu : 0u);
      soB = (first ? k0 : k0 - (int)bsplit) * 2;
    } else {
      const bf16_t* bp = (BMODE == BMODE_PAIR32 && (wave >> 1)) ? b1 : b0;
      const int64_t rem = (int64_t)(tc.k_end - k0) * ldb * 2;
      rsB = make_rsrc_n(bp + (int64_t)k0 * ldb,
                        valid ? clamp_records(rem) : 0u);
    }
  };
  auto load_op = [&](auto Lc, uint32_t stage_off) {
    constexpr int l = decltype(Lc)::value;
    if constexpr (l < LA)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsA, (lds_void_t*)(lds + (stage_off + dstA[l]) / 2), 16, voffA[l], soA, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsB, (lds_void_t*)(lds + (stage_off + dstB[l - LA]) / 2), 16, voffB[l - LA], soB,
          0, 0);
  };

  // ---- loop-invariant LDS read addresses (bytes, stage 0)
  // K-contiguous: one per k step s (the chunk XOR is not affine in s);
  // blocks add 4 KiB each, the stage adds its offset.
  // M/N-contiguous: one per block (the granule XOR is not affine in the
  // block); k steps add 4 KiB, the second transposing read 1 KiB.
  uint32_t rdA[4], rdB[4];
  const int sw = swz(r_lane);
  static_for<0, 4>([&](auto Xc) {
    constexpr int x = decltype(Xc)::value;
    if constexpr (A_KMAJOR)
      rdA[x] = lds0 + (wm * 128 + r_lane) * 128 + (((2 * x + c_lane) ^ sw) << 4);
    else {
      uint32_t lo, hi;
      frag_mn_addr(lds, wm * 128 + x * 32, 0, lane, lo, hi);
      rdA[x] = lo;
    }
    if constexpr (B_KMAJOR)
      rdB[x] = lds0 + A_BYTES + (wn * WTN + r_lane) * 128 + (((2 * x + c_lane) ^ sw) << 4);
    else if constexpr (x < FN) {
      const int c0 = (BMODE == BMODE_PAIR32) ? (x & 1) * 128 + wn * (WTN / 2) + (x >> 1) * 32
                                             : wn * WTN + x * 32;
      uint32_t lo, hi;
      frag_mn_addr(lds + A_BYTES / 2, c0, 0, lane, lo, hi);
      rdB[x] = lo;
    }
  });

  using FA = typename std::conditional<A_KMAJOR, FragK, FragMN>::type;
  using FB = typename std::conditional<B_KMAJOR, FragK, FragMN>::type;
  // one fragment slot per k step: reads run two steps ahead of the MFMAs
  FA fa[4][FM];
  FB fb[4][FN];
  constexpr int RA = A_KMAJOR ? FM : 2 * FM, RB = B_KMAJOR ? FN : 2 * FN;
  constexpr int NREAD = RA + RB;
  // LDS reads complete in order, so waiting until at most this many are
  // outstanding lets the most recent step's reads stay in flight
  constexpr int KEEP = NREAD < 15 ? NREAD : 15;
  // read op r of k step S from the stage at byte offset `boff`, into slot S
  auto read_op = [&](auto Rc, auto Sc, uint32_t boff) {
    constexpr int r = decltype(Rc)::value, S = decltype(Sc)::value;
    if constexpr (r < RA) {
      if constexpr (A_KMAJOR) {
        ds_read_b128_at<r * 4096>(fa[S][r].v, rdA[S] + boff);
      } else {
        constexpr int blk = r >> 1, part = r & 1;
        if constexpr (part == 0)
          ds_read_tr_at<S * 4096>(fa[S][blk].lo, rdA[blk] + boff);
        else
          ds_read_tr_at<S * 4096 + 1024>(fa[S][blk].hi, rdA[blk] + boff);
      }
    } else {
      constexpr int rr = r - RA;
      if constexpr (B_KMAJOR) {
        ds_read_b128_at<rr * 4096>(fb[S][rr].v, rdB[S] + boff);
      } else {
        constexpr int blk = rr >> 1, part = rr & 1;
        if constexpr (part == 0)
          ds_read_tr_at<S * 4096>(fb[S][blk].lo, rdB[blk] + boff);
        else
          ds_read_tr_at<S * 4096 + 1024>(fb[S][blk].hi, rdB[blk] + boff);
      }
    }
  };
  auto fence_slot = [&](auto SLc, auto ALLc) {
    constexpr int SL = decltype(SLc)::value;
    if constexpr (decltype(ALLc)::value)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    else
      asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(KEEP) : "memory");
    static_for<0, FM>([&](auto I) { fa[SL][I].fence(); });
    static_for<0, FN>([&](auto J) { fb[SL][J].fence(); });
  };

  f32x16_t acc[FM][FN];
  static_for<0, FM>([&](auto I) {
    static_for<0, FN>([&](auto J) { acc[I][J] = (f32x16_t)(0.0f); });
  });

  // prologue: tiles 0 .. NBUF-1 in flight, wait for tile 0 only (a plain
  // barrier: __syncthreads would also drain the tiles behind it)
  if (nk > 0) {
    for (int t = 0; t < NBUF; ++t) {
      set_tile(tc.k_begin + t * BK, t == 0 || t < nk);
      const uint32_t stage_off = (uint32_t)t * STAGE;
      static_for<0, NL>([&](auto L) { load_op(L, stage_off); });
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NBUF - 1) * NL) : "memory");
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (nk > 0) {
    static_for<0, NREAD>([&](auto R) { read_op(R, std::integral_constant<int, 0>{}, 0u); });
    static_for<0, NREAD>([&](auto R) { read_op(R, std::integral_constant<int, 1>{}, 0u); });
  }
  asm volatile("s_nop 4");

  constexpr int NM = FM * FN;            // MFMAs per k step
  constexpr int RSPAN = NM < 8 ? NM : 8;  // MFMAs that carry the next reads
  int cs = 0;                             // stage of tile kt
  for (int kt = 0; kt < nk; ++kt) {
    // byte offsets of the stage being consumed and of tile kt + 1's
    const uint32_t cur = (uint32_t)cs * STAGE;
    const int ns = cs + 1 == NBUF ? 0 : cs + 1;
    const uint32_t nxt = (uint32_t)ns * STAGE;
    // tile kt + NBUF goes into this stage once everyone has finished with it
    set_tile(tc.k_begin + (kt + NBUF) * BK, kt + NBUF < nk);
    static_for<0, 4>([&](auto Sc) {
      constexpr int S = decltype(Sc)::value;
      // step 2 drains every read: with the barrier this makes the whole
      // stage free and (after vmcnt) tile kt + 1 readable
      fence_slot(std::integral_constant<int, S>{}, std::integral_constant<bool, S == 2>{});
      if constexpr (S == 2) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NBUF - 2) * NL) : "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      // side operations: reads for the step two ahead (steps 2, 3 read the
      // next tile's steps 0, 1), within the first RSPAN MFMAs; at steps 2
      // and 3 the direct loads of tile kt + NBUF, spread over the MFMAs
      constexpr int NLOAD = (S >= 2) ? NL / 2 : 0;
      constexpr int LOFF = (S == 3) ? NL / 2 : 0;  // first direct load of this step
      static_for<0, NM>([&](auto Mc) {
        constexpr int m = decltype(Mc)::value;
        constexpr int i = m / FN, j = m % FN;
        mfma_ordered(acc[i][j], fb[S][j].op(), fa[S][i].op());
        constexpr int r0 = m < RSPAN ? (m * NREAD) / RSPAN : NREAD;
        constexpr int r1 = m < RSPAN ? ((m + 1) * NREAD) / RSPAN : NREAD;
        constexpr int l0 = NREAD + (m * NLOAD) / NM, l1 = NREAD + ((m + 1) * NLOAD) / NM;
        auto side = [&](auto Oc) {
          constexpr int o = decltype(Oc)::value;
          if constexpr (o < NREAD) {
            constexpr int T = (S + 2) & 3;  // k step being read
            read_op(std::integral_constant<int, o>{}, std::integral_constant<int, T>{},
                    S < 2 ? cur : nxt);
          } else {
            constexpr int idx = o - NREAD + LOFF;
            load_op(std::integral_constant<int, lean_load_seq<LA>(idx)>{}, cur);
          }
        };
        static_for<r0, r1>(side);
        static_for<l0, l1>(side);
      });
    });
    cs = ns;
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");

  // every wavefront's loads have landed and its reads are done before the
  // tile is staged through shared memory
  static_assert(EQ_BYTES <= (int)(NBUF * STAGE), "staging rows exceed shared memory");
  __syncthreads();
  write_tile_staged<EPI, BMODE, OutT, FM, FN, WTM, WTN, LEAN_NT, 0, TMR / 64>(
      acc, ea, tc, wm, wn, lane, tid, Ncols, reinterpret_cast<float*>(lds));
}

// LOOP (row-ragged launches with device-resident offsets only): the grid,
// at most one workgroup per compute unit and a multiple of 8 (so that tile
// index b keeps running on XCD b mod 8), walks the tile indices b =
// blockIdx.x, blockIdx.x + gridDim.x, ...; every workgroup stops at the
// first index past the tiles the offsets call for, so no spare workgroup
// is dispatched however far the worst-case tile count overshoots them.
template <int TMR, bool A_KMAJOR, bool B_KMAJOR, int BMODE, int EPI, typename OutT,
          bool LOOP = false>
__global__ __launch_bounds__(LEAN_NT, 1) void gemm_lean(GemmArgs g) {
  gemm_wave_prio();
  using C = LeanCfg<TMR>;
  __shared__ __attribute__((aligned(1024))) bf16_t lds[C::NBUF * C::STAGE / 2];
  if constexpr (!LOOP) {
    const TileCoord tc = locate_tile(g, blockIdx.x, gridDim.x, TMR);
    if (tc.e < 0) return;  // spare tile (device-resident offsets)
    lean_tile<TMR, A_KMAJOR, B_KMAJOR, BMODE, EPI, OutT>(g, tc, lds);
  } else {
    for (int b = blockIdx.x;; b += gridDim.x) {
      const TileCoord tc = locate_tile(g, b, 0, TMR);
      if (tc.e < 0) return;
      lean_tile<TMR, A_KMAJOR, B_KMAJOR, BMODE, EPI, OutT>(g, tc, lds);
      // every wavefront is done with the epilogue's staging rows before
      // the next tile's loads write shared memory
      __syncthreads();
    }
  }
}

// ---- ring kernel: 4-stage shared-memory ring of 32-wide k tiles ------------
//
// Same wavefront layout and hand-ordered k loop as gemm_lean, but the k
// tiles are 32 wide and four of them live in shared memory at once
// ([A stage 0..3 | B stage 0..3], 16 KiB each).  Every k step issues half
// of the direct loads of the tile three ahead (4 per wavefront, one after
// every fourth MFMA), so load issue is spread evenly over the loop and each load
// has two tiles of latency budget; LDS reads run two k steps (one tile)
// ahead; one barrier per tile, at its first step.
constexpr int RBK = 32;
#ifndef RING_STAGES
#define RING_STAGES 4
#endif
constexpr int RTILE = BM * RBK * 2;  // one operand stage, 16 KiB

__device__ __forceinline__ int swz4(int r) { return (r & 3) ^ ((r >> 2) & 3); }

// M/N-contiguous stage tile: [half][k 0..31][16 granules], granule q of row
// k at q ^ 4 (k % 4)
__device__ __forceinline__ int mn_off32(int k, int c) {
  const int h = c >> 7, q = (c >> 3) & 15, e = c & 7;
  return h * (RBK * 128) + k * 128 + ((q ^ ((k & 3) << 2)) << 3) + e;
}

template <bool A_KMAJOR, bool B_KMAJOR, int BMODE, int EPI, typename OutT>
__global__ __launch_bounds__(LEAN_NT, 1) void gemm_ring(GemmArgs g) {
  gemm_wave_prio();
  constexpr int FM = 4, FN = 4, WTM = 128, WTN = 128;
  constexpr int NS = RING_STAGES;
  __shared__ __attribute__((aligned(1024))) bf16_t lds[2 * NS * BM * RBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r_lane = lane & 31, c_lane = lane >> 5;

  const TileCoord tc = locate_tile(g, blockIdx.x, gridDim.x, BM);
  if (tc.e < 0) return;  // spare tile (device-resident offsets)
  const bf16_t* a0 = reinterpret_cast<const bf16_t*>(g.a.p0) + tc.e * g.a.bstride;
  const bf16_t* b0 = reinterpret_cast<const bf16_t*>(g.b.p0) + tc.e * g.b.bstride;
  const bf16_t* b1 = reinterpret_cast<const bf16_t*>(g.b.p1) + tc.e * g.b.bstride;
  const int64_t lda = g.a.ld, ldb = g.b.ld, bsplit = g.b.split;
  const int Ncols = g.N;
  const EpiArgs ea = g.epi;
  const int n_base = tc.tn * BN;
  const int m_rows = tc.m_end - tc.m_begin;
  const int nk = (tc.k_end > tc.k_begin) ? (tc.k_end - tc.k_begin + RBK - 1) / RBK : 0;

  const uint32_t lds0 = lds_u32(lds);
  const uint32_t ldsA = lds0, ldsB = lds0 + NS * RTILE;

  // ---- loop-invariant direct-load offsets (bytes) and destinations
  uint32_t voffA[4], voffB[4], dstA[4], dstB[4];
  static_for<0, 4>([&](auto Ic) {
    constexpr int i = decltype(Ic)::value;
    if constexpr (A_KMAJOR) {
      const int blk = wave * 4 + i;
      const int r = blk * 16 + (lane >> 2);
      const int c = (lane & 3) ^ swz4(r);
      voffA[i] = r < m_rows ? (uint32_t)(((int64_t)r * lda + c * 8) * 2) : OOB_OFF;
      dstA[i] = blk * 1024;
    } else {
      const int half = wave >> 1, b = (wave & 1) * 4 + i;
      const int k = 4 * b + (lane >> 4);
      const int q = (lane & 15) ^ ((k & 3) << 2);
      const int col = tc.m_begin + half * 128 + 8 * q;
      voffA[i] = col < tc.m_end ? (uint32_t)(((int64_t)k * lda + col) * 2) : OOB_OFF;
      dstA[i] = half * (RTILE / 2) + b * 1024;
    }
    if constexpr (B_KMAJOR) {
      const int blk = wave * 4 + i;
      const int r = blk * 16 + (lane >> 2);
      const int c = (lane & 3) ^ swz4(r);
      voffB[i] = r < Ncols - n_base ? (uint32_t)(((int64_t)r * ldb + c * 8) * 2) : OOB_OFF;
      dstB[i] = blk * 1024;
    } else {
      const int half = wave >> 1, b = (wave & 1) * 4 + i;
      const int k = 4 * b + (lane >> 4);
      const int q = (lane & 15) ^ ((k & 3) << 2);
      int col, lim;
      if constexpr (BMODE == BMODE_PAIR32) {
        col = tc.tn * 128 + 8 * q;
        lim = (int)bsplit;
      } else {
        col = n_base + half * 128 + 8 * q;
        lim = Ncols;
      }
      voffB[i] = col < lim ? (uint32_t)(((int64_t)k * ldb + col) * 2) : OOB_OFF;
      dstB[i] = half * (RTILE / 2) + b * 1024;
    }
  });
  rsrc_t rsA, rsB;
  int soA = 0, soB = 0;
  // buffer resources of the k tile starting at k0 (past the end: empty)
  auto set_tile = [&](int k0, bool valid) {
    if constexpr (A_KMAJOR) {
      rsA = make_rsrc_n(a0 + (int64_t)tc.m_begin * lda, valid ? 0x7fffffffu : 0u);
      soA = k0 * 2;
    } else {
      const int64_t rem = (int64_t)(tc.k_end - k0) * lda * 2;
      rsA = make_rsrc_n(a0 + (int64_t)k0 * lda,
                        valid ? clamp_records(rem) : 0u);
    }
    if constexpr (B_KMAJOR) {
      const bool first = BMODE != BMODE_KSPLIT || k0 < bsplit;
      const bf16_t* bp = first ? b0 : b1;
      rsB = make_rsrc_n(bp + (int64_t)n_base * ldb, valid ? 0x7fffffffu : 0u);
      soB = (first ? k0 : k0 - (int)bsplit) * 2;
    } else {
      const bf16_t* bp = (BMODE == BMODE_PAIR32 && (wave >> 1)) ? b1 : b0;
      const int64_t rem = (int64_t)(tc.k_end - k0) * ldb * 2;
      rsB = make_rsrc_n(bp + (int64_t)k0 * ldb,
                        valid ? clamp_records(rem) : 0u);
    }
  };
  // direct load l of a tile (A0 B0 A1 B1 ...) into the stage at `soff`
  auto load_op = [&](auto Lc, uint32_t soff) {
    constexpr int l = decltype(Lc)::value, i = l >> 1;
    if constexpr ((l & 1) == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsA, (lds_void_t*)(lds + (soff + dstA[i]) / 2), 16, voffA[i], soA, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsB, (lds_void_t*)(lds + (NS * RTILE + soff + dstB[i]) / 2), 16, voffB[i], soB, 0, 0);
  };

  // ---- loop-invariant LDS read addresses (bytes, stage 0)
  uint32_t rdA[4], rdB[4];
  const int sw = swz4(r_lane);
  static_for<0, 4>([&](auto Xc) {
    constexpr int x = decltype(Xc)::value;
    if constexpr (A_KMAJOR) {
      if constexpr (x < 2) rdA[x] = ldsA + (wm * 128 + r_lane) * 64 + (((2 * x + c_lane) ^ sw) << 4);
    } else {
      const int gg = lane >> 4, rr = lane & 15;
      const int c = wm * 128 + x * 32 + 16 * (gg & 1) + 4 * (rr & 3);
      const int k = 8 * (gg >> 1) + (rr >> 2);
      rdA[x] = ldsA + 2 * mn_off32(k, c);
    }
    if constexpr (B_KMAJOR) {
      if constexpr (x < 2) rdB[x] = ldsB + (wn * 128 + r_lane) * 64 + (((2 * x + c_lane) ^ sw) << 4);
    } else {
      const int c0 = (BMODE == BMODE_PAIR32) ? (x & 1) * 128 + wn * 64 + (x >> 1) * 32
                                             : wn * 128 + x * 32;
      const int gg = lane >> 4, rr = lane & 15;
      const int c = c0 + 16 * (gg & 1) + 4 * (rr & 3);
      const int k = 8 * (gg >> 1) + (rr >> 2);
      rdB[x] = ldsB + 2 * mn_off32(k, c);
    }
  });

  using FA = typename std::conditional<A_KMAJOR, FragK, FragMN>::type;
  using FB = typename std::conditional<B_KMAJOR, FragK, FragMN>::type;
  FA fa[4][FM];
  FB fb[4][FN];
  constexpr int RA = A_KMAJOR ? 4 : 8, RB = B_KMAJOR ? 4 : 8;
  constexpr int NREAD = RA + RB;
  constexpr int KEEP = NREAD < 15 ? NREAD : 15;
  // read op r of step SP (0/1) of the stage at `soff`, into slot SL
  auto read_op = [&](auto Rc, auto SPc, uint32_t soff, auto SLc) {
    constexpr int r = decltype(Rc)::value, SP = decltype(SPc)::value;
    constexpr int SL = decltype(SLc)::value;
    if constexpr (r < RA) {
      if constexpr (A_KMAJOR) {
        ds_read_b128_at<r * 2048>(fa[SL][r].v, rdA[SP] + soff);
      } else {
        constexpr int blk = r >> 1, part = r & 1;
        ds_read_tr_at<SP * 4096 + part * 1024>(part ? fa[SL][blk].hi : fa[SL][blk].lo,
                                               rdA[blk] + soff);
      }
    } else {
      constexpr int rr = r - RA;
      if constexpr (B_KMAJOR) {
        ds_read_b128_at<rr * 2048>(fb[SL][rr].v, rdB[SP] + soff);
      } else {
        constexpr int blk = rr >> 1, part = rr & 1;
        ds_read_tr_at<SP * 4096 + part * 1024>(part ? fb[SL][blk].hi : fb[SL][blk].lo,
                                               rdB[blk] + soff);
      }
    }
  };
  auto fence_slot = [&](auto SLc) {
    constexpr int SL = decltype(SLc)::value;
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(KEEP) : "memory");
    static_for<0, FM>([&](auto I) { fa[SL][I].fence(); });
    static_for<0, FN>([&](auto J) { fb[SL][J].fence(); });
  };

  f32x16_t acc[FM][FN];
  static_for<0, FM>([&](auto I) {
    static_for<0, FN>([&](auto J) { acc[I][J] = (f32x16_t)(0.0f); });
  });

  // prologue: tiles 0 .. NS-2 in flight, wait for tile 0, read its two steps
  if (nk > 0) {
    static_for<0, NS - 1>([&](auto Tc) {
      constexpr int T = decltype(Tc)::value;
      set_tile(tc.k_begin + T * RBK, T < nk);
      static_for<0, 8>([&](auto L) { load_op(L, (uint32_t)(T * RTILE)); });
    });
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * 8) : "memory");
  }
  // a plain s_barrier: __syncthreads() would also drain the loads of tiles
  // 1 and 2 (the explicit vmcnt waits order the shared-memory traffic)
  __builtin_amdgcn_s_barrier();
  if (nk > 0) {
    static_for<0, NREAD>([&](auto R) {
      read_op(R, std::integral_constant<int, 0>{}, 0u, std::integral_constant<int, 0>{});
    });
    static_for<0, NREAD>([&](auto R) {
      read_op(R, std::integral_constant<int, 1>{}, 0u, std::integral_constant<int, 1>{});
    });
  }
  asm volatile("s_nop 4");

  // two tiles (four k steps) per trip so the fragment slot is a constant; an
  // odd tile count runs one more tile, loaded as zeros (both operands lie
  // past the end), which leaves the sums unchanged
  const int nk2 = (nk + 1) & ~1;
  int st_next = 1 % NS, st_load = NS - 1;  // stages of tiles t + 1 and t + NS - 1
  for (int t0 = 0; t0 < nk2; t0 += 2) {
    static_for<0, 2>([&](auto TPc) {
      constexpr int TP = decltype(TPc)::value;
      const int t = t0 + TP;
      {
        const uint32_t s_next = (uint32_t)st_next * RTILE;  // stage read ahead
        const uint32_t s_load = (uint32_t)st_load * RTILE;  // stage being refilled
        st_next = st_next == NS - 1 ? 0 : st_next + 1;
        st_load = st_load == NS - 1 ? 0 : st_load + 1;
        set_tile(tc.k_begin + (t + NS - 1) * RBK, t + NS - 1 < nk);
        static_for<0, 2>([&](auto SPc) {
          constexpr int SP = decltype(SPc)::value;
          constexpr int S = TP * 2 + SP;  // fragment slot of this step
          fence_slot(std::integral_constant<int, S>{});
          if constexpr (SP == 0) {
            // tile t + 1 has landed everywhere, and everyone has finished
            // reading tile t - 1, whose stage tile t + NS - 1 now refills
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 3) * 8) : "memory");
            __builtin_amdgcn_s_barrier();
          }
          static_for<0, 16>([&](auto Mc) {
            constexpr int m = decltype(Mc)::value;
            constexpr int i = m >> 2, j = m & 3;
            mfma_ordered(acc[i][j], fb[S][j].op(), fa[S][i].op());
            constexpr int r0 = m < 8 ? (m * NREAD) / 8 : NREAD;
            constexpr int r1 = m < 8 ? ((m + 1) * NREAD) / 8 : NREAD;
            static_for<r0, r1>([&](auto Oc) {
              read_op(Oc, std::integral_constant<int, SP>{}, s_next,
                      std::integral_constant<int, (S + 2) & 3>{});
            });
            if constexpr (m % 4 == 1)
              load_op(std::integral_constant<int, SP * 4 + m / 4>{}, s_load);
          });
        });
      }
    });
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");

  // every wavefront's loads have landed and its reads are done before the
  // tile is staged through shared memory
  static_assert(EQ_BYTES <= (int)sizeof(lds), "staging rows exceed shared memory");
  __syncthreads();
  write_tile_staged<EPI, BMODE, OutT, FM, FN, WTM, WTN, LEAN_NT>(
      acc, ea, tc, wm, wn, lane, tid, Ncols, reinterpret_cast<float*>(lds));
}


// ---- 16x16x32 kernel: tiles of BMT x BNT, each 224 or 256 ---------------------
//
// Tiles 224 wide let a GEMM whose extent is a multiple of 224 but not 256
// (F/T = 3584 = 16 x 224) fill every compute unit in whole waves, where
// 256 x 256 tiles leave a partial last wave.  Four wavefronts, 2 x 2, each
// own a (BMT/2) x (BNT/2) block of 16 x 16 accumulators; a 16-wide fragment
// grid is what lets a wavefront cover 112 columns.  k tiles are 64 wide
// (two 32-wide MFMA steps) in two shared-memory buffers, laid out as in
// gemm_lean except for the swizzles: M/N-contiguous tiles also XOR
// granules with bit 3 of k (the four k groups of a 16 x 32 fragment read
// the same 16 columns, and this keeps two neighbouring groups on different
// banks), and K-contiguous tiles swizzle by row mod 8 only.  For the
// paired SwiGLU forward, gate columns fill buffer half 0 and up columns
// half 1 (one source matrix per direct load); the wavefronts of column 0
// compute gate sums and those of column 1 up sums for the same 112 logical
// columns, re-paired by the staged epilogue.
__device__ __forceinline__ int sw16(int k) { return ((k & 3) << 2) ^ (((k >> 3) & 1) << 1); }
// K-contiguous tiles here swizzle chunks by row mod 8 only.  A 16 x 32
// fragment read takes rows r..r+15 at one chunk; with gemm_lean's swizzle
// (which also flips on bit 3 of the row) those reads cost ~4 bank-conflict
// cycles each (counted with SQ_LDS_BANK_CONFLICT on the dH launch and on a
// probe of the read pattern alone), enough to make shared memory, not the
// MFMAs, the k loop's bound; with row mod 8 they cost none.
__device__ __forceinline__ int swzk16(int r) { return r & 7; }
__device__ __forceinline__ int mn16_off(int k, int c) {
  const int h = c >> 7, q = (c >> 3) & 15, e = c & 7;
  return h * (BK * 128) + k * 128 + ((q ^ sw16(k)) << 3) + e;
}
__device__ __forceinline__ void mfma16_ordered(f32x4_t& acc, const bf16x8_t& a,
                                               const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b) : "memory");
}

// staged epilogue for 16 x 16 accumulators: passes of up to 64 rows (four
// fragment rows of one wavefront row); lane l holds row 16 i + l % 16 and
// columns 16 j + 4 (l / 16) + (0..3) of its wavefront block
template <int EPI, int BMODE, typename OutT, int FM, int FN, int WTM, int WTN, int BNT>
__device__ __forceinline__ void write_tile_staged16(const f32x4_t (&acc)[FM][FN],
                                                    const EpiArgs& ea, const TileCoord& tc,
                                                    int wm, int wn, int lane, int tid,
                                                    int Ncols, float* stage) {
  constexpr bool PAIR = EPI == EPI_SWIGLU_FWD;
  constexpr int HALF = (FM + 1) / 2;  // fragment rows of the first pass of a wavefront row
  const int r16 = lane & 15, c16 = lane >> 4;
  static_for<0, 4>([&](auto Pc) {
    constexpr int p = decltype(Pc)::value;
    constexpr int lo = (p & 1) ? HALF : 0, hi = (p & 1) ? FM : HALF;
    constexpr int R = (hi - lo) * 16;
    if (wm == (p >> 1)) {
      static_for<lo, hi>([&](auto Ic) {
        constexpr int i = decltype(Ic)::value;
        const int row = (i - lo) * 16 + r16;
        static_for<0, FN>([&](auto Jc) {
          constexpr int j = decltype(Jc)::value;
          const int col = (PAIR ? wn * 128 : wn * WTN) + 16 * j + 4 * c16;
          *reinterpret_cast<f32x4_t*>(stage + row * EQ_PITCH + col) = acc[i][j];
        });
      });
    }
    __syncthreads();
    const int64_t m0 = tc.m_begin + (p >> 1) * WTM + lo * 16;
    constexpr int CPR = PAIR ? WTN / 8 : BNT / 8;  // 8-column chunks per row
    constexpr int NCH = R * CPR;
    static_for<0, (NCH + W16_NT - 1) / W16_NT>([&](auto Kc) {
      const int k = decltype(Kc)::value * W16_NT + tid;
      if (NCH % W16_NT == 0 || k < NCH) {
        const int row = k / CPR, cc = (k % CPR) * 8;
        const int64_t m = m0 + row;
        const float* src = stage + row * EQ_PITCH + cc;
        if constexpr (PAIR) {
          const int64_t f = (int64_t)tc.tn * WTN + cc;
          if (m < tc.m_end && f < ea.split) {
            float gv[8], uv[8];
            *reinterpret_cast<f32x4_t*>(gv) = *reinterpret_cast<const f32x4_t*>(src);
            *reinterpret_cast<f32x4_t*>(gv + 4) = *reinterpret_cast<const f32x4_t*>(src + 4);
            *reinterpret_cast<f32x4_t*>(uv) = *reinterpret_cast<const f32x4_t*>(src + 128);
            *reinterpret_cast<f32x4_t*>(uv + 4) = *reinterpret_cast<const f32x4_t*>(src + 132);
            epilogue_swiglu8<bf16_t>(ea, m, f, gv, uv);
          }
        } else {
          const int64_t n = (int64_t)tc.tn * BNT + cc;
          if (m < tc.m_end && n < Ncols) {
            float cv[8];
            *reinterpret_cast<f32x4_t*>(cv) = *reinterpret_cast<const f32x4_t*>(src);
            *reinterpret_cast<f32x4_t*>(cv + 4) = *reinterpret_cast<const f32x4_t*>(src + 4);
            epilogue8<EPI, bf16_t, OutT>(ea, tc.e, m, n, cv);
          }
        }
      }
    });
    __syncthreads();
  });
}

template <bool A_KMAJOR, bool B_KMAJOR, int BMODE, int EPI, typename OutT, int BMT, int BNT>
__global__ __launch_bounds__(W16_NT, 1) void gemm_w16(GemmArgs g) {
  gemm_wave_prio();
  static_assert(BMT == 224 || BMT == 256, "tile rows");
  static_assert(BNT == 224 || BNT == 256, "tile columns");
  constexpr bool PAIR = BMODE == BMODE_PAIR32;
  static_assert(!PAIR || (!B_KMAJOR && BNT == 224), "paired tiles: 112 gate + 112 up columns");
  static_assert(BMODE != BMODE_KSPLIT, "k split not supported here");
  constexpr int WTM = BMT / 2, WTN = BNT / 2;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  __shared__ __attribute__((aligned(1024))) bf16_t lds[4 * BM * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, c16 = lane >> 4;

  const TileCoord tc = locate_tile(g, blockIdx.x, gridDim.x, BMT);
  const bf16_t* a0 = reinterpret_cast<const bf16_t*>(g.a.p0) + tc.e * g.a.bstride;
  const bf16_t* b0 = reinterpret_cast<const bf16_t*>(g.b.p0) + tc.e * g.b.bstride;
  const bf16_t* b1 = reinterpret_cast<const bf16_t*>(g.b.p1) + tc.e * g.b.bstride;
  const int64_t lda = g.a.ld, ldb = g.b.ld, bsplit = g.b.split;
  const int Ncols = g.N;
  const EpiArgs ea = g.epi;
  const int n_base = tc.tn * BNT;
  // rows / columns of this tile that exist
  const int m_rows = min(BMT, tc.m_end - tc.m_begin);
  const int n_cols = min(BNT, Ncols - n_base);
  const int nk = (tc.k_end > tc.k_begin) ? (tc.k_end - tc.k_begin + BK - 1) / BK : 0;

  const uint32_t lds0 = lds_u32(lds);
  const uint32_t ldsA = lds0, ldsB = lds0 + 2 * TILE_BYTES;

  // ---- loop-invariant direct-load offsets (bytes) and LDS destinations
  uint32_t voffA[8], voffB[8];
  uint32_t dstA[8], dstB[8];
  static_for<0, 8>([&](auto Ic) {
    constexpr int i = decltype(Ic)::value;
    if constexpr (A_KMAJOR) {
      const int blk = wave * 8 + i;
      const int r = blk * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swzk16(r);
      voffA[i] = r < m_rows ? (uint32_t)(((int64_t)r * lda + c * 8) * 2) : OOB_OFF;
      dstA[i] = blk * 1024;
    } else {
      const int half = wave >> 1, b = (wave & 1) * 8 + i;
      const int k = 4 * b + (lane >> 4);
      const int q = (lane & 15) ^ sw16(k);
      const int cl = half * 128 + 8 * q;
      voffA[i] = cl < m_rows ? (uint32_t)(((int64_t)k * lda + tc.m_begin + cl) * 2) : OOB_OFF;
      dstA[i] = half * (TILE_BYTES / 2) + b * 1024;
    }
    if constexpr (B_KMAJOR) {
      const int blk = wave * 8 + i;
      const int r = blk * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swzk16(r);
      voffB[i] = r < n_cols ? (uint32_t)(((int64_t)r * ldb + c * 8) * 2) : OOB_OFF;
      dstB[i] = blk * 1024;
    } else {
      const int half = wave >> 1, b = (wave & 1) * 8 + i;
      const int k = 4 * b + (lane >> 4);
      const int q = (lane & 15) ^ sw16(k);
      bool ok;
      int64_t col;
      if constexpr (PAIR) {
        // half 0: gate columns, half 1: up columns, 112 of each
        col = (int64_t)tc.tn * WTN + 8 * q;
        ok = q < WTN / 8 && col < bsplit;
      } else {
        const int cl = half * 128 + 8 * q;
        col = n_base + cl;
        ok = cl < n_cols;
      }
      voffB[i] = ok ? (uint32_t)(((int64_t)k * ldb + col) * 2) : OOB_OFF;
      dstB[i] = half * (TILE_BYTES / 2) + b * 1024;
    }
  });
  rsrc_t rsA, rsB;
  int soA = 0, soB = 0;
  auto set_tile = [&](int k0, bool valid) {
    if constexpr (A_KMAJOR) {
      rsA = make_rsrc_n(a0 + (int64_t)tc.m_begin * lda, valid ? 0x7fffffffu : 0u);
      soA = k0 * 2;
    } else {
      const int64_t rem = (int64_t)(tc.k_end - k0) * lda * 2;
      rsA = make_rsrc_n(a0 + (int64_t)k0 * lda, valid ? clamp_records(rem) : 0u);
    }
    if constexpr (B_KMAJOR) {
      rsB = make_rsrc_n(b0 + (int64_t)n_base * ldb, valid ? 0x7fffffffu : 0u);
      soB = k0 * 2;
    } else {
      const bf16_t* bp = (PAIR && (wave >> 1)) ? b1 : b0;
      const int64_t rem = (int64_t)(tc.k_end - k0) * ldb * 2;
      rsB = make_rsrc_n(bp + (int64_t)k0 * ldb, valid ? clamp_records(rem) : 0u);
    }
  };
  auto load_op = [&](auto Lc, uint32_t buf_off) {
    constexpr int l = decltype(Lc)::value;
    if constexpr (l < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsA, (lds_void_t*)(lds + (ldsA - lds0 + buf_off + dstA[l]) / 2), 16, voffA[l], soA, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsB, (lds_void_t*)(lds + (ldsB - lds0 + buf_off + dstB[l - 8]) / 2), 16, voffB[l - 8],
          soB, 0, 0);
  };

  // ---- loop-invariant LDS read addresses (bytes, buffer 0)
  // K-contiguous: one per 32-wide k step (fragment i adds 2 KiB);
  // M/N-contiguous: one per fragment (k step s adds 8 KiB, the second
  // transposing read 1 KiB)
  uint32_t rdA[FM], rdB[FN];
  const int sw = swzk16(r16);  // fragment rows are 16-aligned: row mod 8 = r16 mod 8
  static_for<0, FM>([&](auto Xc) {
    constexpr int x = decltype(Xc)::value;
    if constexpr (A_KMAJOR) {
      if constexpr (x < 2) rdA[x] = ldsA + (wm * WTM + r16) * 128 + (((4 * x + c16) ^ sw) << 4);
    } else {
      const int c = wm * WTM + 16 * x + 4 * (r16 & 3);
      const int k = 8 * c16 + (r16 >> 2);
      rdA[x] = ldsA + 2 * mn16_off(k, c);
    }
  });
  static_for<0, FN>([&](auto Xc) {
    constexpr int x = decltype(Xc)::value;
    if constexpr (B_KMAJOR) {
      if constexpr (x < 2) rdB[x] = ldsB + (wn * WTN + r16) * 128 + (((4 * x + c16) ^ sw) << 4);
    } else {
      const int c = (PAIR ? wn * 128 : wn * WTN) + 16 * x + 4 * (r16 & 3);
      const int k = 8 * c16 + (r16 >> 2);
      rdB[x] = ldsB + 2 * mn16_off(k, c);
    }
  });

  using FA = typename std::conditional<A_KMAJOR, FragK, FragMN>::type;
  using FB = typename std::conditional<B_KMAJOR, FragK, FragMN>::type;
  FA fa[2][FM];
  FB fb[2][FN];
  constexpr int RA = A_KMAJOR ? FM : 2 * FM, RB = B_KMAJOR ? FN : 2 * FN;
  constexpr int NREAD = RA + RB;
  auto read_op = [&](auto Rc, auto Sc, uint32_t boff) {
    constexpr int r = decltype(Rc)::value, S = decltype(Sc)::value;
    if constexpr (r < RA) {
      if constexpr (A_KMAJOR) {
        ds_read_b128_at<r * 2048>(fa[S][r].v, rdA[S] + boff);
      } else {
        constexpr int blk = r >> 1, part = r & 1;
        if constexpr (part == 0)
          ds_read_tr_at<S * 8192>(fa[S][blk].lo, rdA[blk] + boff);
        else
          ds_read_tr_at<S * 8192 + 1024>(fa[S][blk].hi, rdA[blk] + boff);
      }
    } else {
      constexpr int rr = r - RA;
      if constexpr (B_KMAJOR) {
        ds_read_b128_at<rr * 2048>(fb[S][rr].v, rdB[S] + boff);
      } else {
        constexpr int blk = rr >> 1, part = rr & 1;
        if constexpr (part == 0)
          ds_read_tr_at<S * 8192>(fb[S][blk].lo, rdB[blk] + boff);
        else
          ds_read_tr_at<S * 8192 + 1024>(fb[S][blk].hi, rdB[blk] + boff);
      }
    }
  };
  auto fence_slot = [&](auto SLc) {
    constexpr int SL = decltype(SLc)::value;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    static_for<0, FM>([&](auto I) { fa[SL][I].fence(); });
    static_for<0, FN>([&](auto J) { fb[SL][J].fence(); });
  };

  f32x4_t acc[FM][FN];
  static_for<0, FM>([&](auto I) {
    static_for<0, FN>([&](auto J) { acc[I][J] = (f32x4_t)(0.0f); });
  });

  // prologue: tiles 0 and 1 in flight, wait for tile 0, read its first step
  if (nk > 0) {
    set_tile(tc.k_begin, true);
    static_for<0, 16>([&](auto L) { load_op(L, 0u); });
    set_tile(tc.k_begin + BK, nk > 1);
    static_for<0, 16>([&](auto L) { load_op(L, (uint32_t)TILE_BYTES); });
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  }
  __builtin_amdgcn_s_barrier();
  if (nk > 0) {
    static_for<0, NREAD>([&](auto R) { read_op(R, std::integral_constant<int, 0>{}, 0u); });
  }
  asm volatile("s_nop 4");

  constexpr int NMF = FM * FN;  // MFMAs per step
  for (int kt = 0; kt < nk; ++kt) {
    const uint32_t cur = (uint32_t)(kt & 1) * TILE_BYTES;
    const uint32_t nxt = cur ^ TILE_BYTES;
    set_tile(tc.k_begin + (kt + 2) * BK, kt + 2 < nk);
    static_for<0, 2>([&](auto Sc) {
      constexpr int S = decltype(Sc)::value;
      fence_slot(std::integral_constant<int, S>{});
      if constexpr (S == 1) {
        // tile kt + 1 has landed everywhere and every wavefront has read
        // all of this tile: the buffer takes tile kt + 2
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
      }
      constexpr int NLOAD = S == 1 ? 16 : 0;
      static_for<0, NMF>([&](auto Mc) {
        constexpr int m = decltype(Mc)::value;
        constexpr int i = m / FN, j = m % FN;
        mfma16_ordered(acc[i][j], fb[S][j].op(), fa[S][i].op());
        // reads of the next step within the first half of the MFMAs
        constexpr int H = NMF / 2;
        constexpr int r0 = m < H ? (m * NREAD) / H : NREAD;
        constexpr int r1 = m < H ? ((m + 1) * NREAD) / H : NREAD;
        static_for<r0, r1>([&](auto Oc) {
          read_op(Oc, std::integral_constant<int, S ^ 1>{}, S == 0 ? cur : nxt);
        });
        constexpr int l0 = (m * NLOAD) / NMF, l1 = ((m + 1) * NLOAD) / NMF;
        static_for<l0, l1>([&](auto Oc) {
          constexpr int idx = decltype(Oc)::value;
          load_op(std::integral_constant<int, (idx & 1) * 8 + (idx >> 1)>{}, cur);
        });
      });
    });
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");

  static_assert(EQ_BYTES <= (int)sizeof(lds), "staging rows exceed shared memory");
  __syncthreads();
  write_tile_staged16<EPI, BMODE, OutT, FM, FN, WTM, WTN, BNT>(
      acc, ea, tc, wm, wn, lane, tid, Ncols, reinterpret_cast<float*>(lds));
}


// ---- FP8 kernel: E4M3 x E4M3 -> fp32 sums, 256 x 256 tiles --------------------
//
// Both operands K-contiguous (the weights arrive as quantized transposes).
// A k tile is 128 codes: the same 128-byte rows, swizzle and direct loads
// as gemm_lean's 64-wide bf16 tiles.  Four wavefronts of 128 x 128; each k
// tile is two steps of v_mfma_scale_f32_32x32x64_f8f6f4 with unit block
// scales (E8M0 127): lane l gives row l % 32, codes 32 (l / 32) .. + 31 of
// the step's 64 (checked on the GPU against an exact product), i.e. two
// 16-byte chunks.  Reads run one step ahead; one barrier per tile.  The
// per-tensor scales are applied in the staged epilogue (QM).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct Frag8 {
  i32x4_t lo, hi;
  __device__ __forceinline__ void fence() { asm volatile("" : "+v"(lo), "+v"(hi)); }
  __device__ __forceinline__ i32x8_t op() const {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};
template <int OFF>
__device__ __forceinline__ void ds_read_b128_i(i32x4_t& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
// srcA is the B operand's fragment (format FB: cbsz), srcB the A
// operand's (format FA: blgp); 0 = E4M3, 1 = E5M2
template <int FA, int FB>
__device__ __forceinline__ void mfma_f8_ordered(f32x16_t& acc, const i32x8_t& a,
                                                const i32x8_t& b, int unit_scale) {
  if constexpr (FA == 0 && FB == 0)
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                 : "+a"(acc) : "v"(a), "v"(b), "v"(unit_scale) : "memory");
  else if constexpr (FA == 1 && FB == 0)
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] blgp:1"
                 : "+a"(acc) : "v"(a), "v"(b), "v"(unit_scale) : "memory");
  else if constexpr (FA == 0 && FB == 1)
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:1"
                 : "+a"(acc) : "v"(a), "v"(b), "v"(unit_scale) : "memory");
  else
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:1 blgp:1"
                 : "+a"(acc) : "v"(a), "v"(b), "v"(unit_scale) : "memory");
}

template <int BMODE, int EPI, int QM, int FA = 0, int FB = 0, typename OutT = bf16_t>
__global__ __launch_bounds__(LEAN_NT, 1) void gemm_f8(GemmArgs g) {
  gemm_wave_prio();
  constexpr int FM = 4, FN = 4, WTM = 128, WTN = 128;
  constexpr int BKB = 128;  // k codes (bytes) per tile
  constexpr bool PAIR = BMODE == BMODE_PAIR32;
  __shared__ __attribute__((aligned(1024))) bf16_t lds[4 * BM * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r_lane = lane & 31, c_lane = lane >> 5;

  const TileCoord tc = locate_tile(g, blockIdx.x, gridDim.x, BM);
  const uint8_t* a0 = reinterpret_cast<const uint8_t*>(g.a.p0);
  const uint8_t* b0 = reinterpret_cast<const uint8_t*>(g.b.p0);
  const uint8_t* b1 = reinterpret_cast<const uint8_t*>(g.b.p1);
  const int64_t lda = g.a.ld, ldb = g.b.ld, bsplit = g.b.split;
  const int Ncols = g.N;
  const EpiArgs ea = g.epi;
  const int n_base = tc.tn * BN;
  const int m_rows = tc.m_end - tc.m_begin;
  const int nk = (tc.k_end > tc.k_begin) ? (tc.k_end - tc.k_begin + BKB - 1) / BKB : 0;
  // B rows of this tile: paired tiles take 128 gate rows from b0 and 128 up
  // rows from b1 (the same 128 logical columns)
  const int half = wave >> 1;
  const int64_t b_row0 = PAIR ? (int64_t)tc.tn * 128 : n_base;
  const int b_rows = PAIR ? (int)min<int64_t>(128, bsplit - b_row0) : Ncols - n_base;

  const uint32_t lds0 = lds_u32(lds);
  const uint32_t ldsA = lds0, ldsB = lds0 + 2 * TILE_BYTES;

  uint32_t voffA[8], voffB[8];
  uint32_t dstA[8], dstB[8];
  static_for<0, 8>([&](auto Ic) {
    constexpr int i = decltype(Ic)::value;
    const int blk = wave * 8 + i;
    const int r = blk * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    voffA[i] = r < m_rows ? (uint32_t)((int64_t)r * lda + c * 16) : OOB_OFF;
    dstA[i] = blk * 1024;
    // paired: rows 0..127 of the tile (waves 0, 1) are gate rows, 128..255 up
    const int rb = PAIR ? r - 128 * half : r;
    voffB[i] = rb < b_rows ? (uint32_t)((int64_t)rb * ldb + c * 16) : OOB_OFF;
    dstB[i] = blk * 1024;
  });
  rsrc_t rsA, rsB;
  int soA = 0, soB = 0;
  auto set_tile = [&](int k0, bool valid) {
    rsA = make_rsrc_n(a0 + (int64_t)tc.m_begin * lda, valid ? 0x7fffffffu : 0u);
    soA = k0;
    if constexpr (BMODE == BMODE_KSPLIT) {
      // k tiles never straddle the split (a multiple of 128)
      const bool first = k0 < bsplit;
      rsB = make_rsrc_n((first ? b0 : b1) + b_row0 * ldb, valid ? 0x7fffffffu : 0u);
      soB = first ? k0 : k0 - (int)bsplit;
    } else {
      const uint8_t* bp = (PAIR && half) ? b1 : b0;
      rsB = make_rsrc_n(bp + b_row0 * ldb, valid ? 0x7fffffffu : 0u);
      soB = k0;
    }
  };
  auto load_op = [&](auto Lc, uint32_t buf_off) {
    constexpr int l = decltype(Lc)::value;
    if constexpr (l < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsA, (lds_void_t*)(lds + (ldsA - lds0 + buf_off + dstA[l]) / 2), 16, voffA[l], soA, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsB, (lds_void_t*)(lds + (ldsB - lds0 + buf_off + dstB[l - 8]) / 2), 16, voffB[l - 8],
          soB, 0, 0);
  };

  // read addresses: step s, half h -> chunk 4 s + 2 c_lane + h of the row
  uint32_t rdA[4], rdB[4];
  const int sw = swz(r_lane);
  static_for<0, 4>([&](auto Xc) {
    constexpr int x = decltype(Xc)::value;  // 2 s + h
    const int chunk = 4 * (x >> 1) + 2 * c_lane + (x & 1);
    rdA[x] = ldsA + (wm * 128 + r_lane) * 128 + ((chunk ^ sw) << 4);
    // paired B: fragment j of wavefront column wn covers gate (j even) or up
    // (j odd) rows wn * 64 + (j / 2) * 32 of each half, as in gemm_lean
    rdB[x] = ldsB + ((PAIR ? wn * 64 : wn * 128) + r_lane) * 128 + ((chunk ^ sw) << 4);
  });

  Frag8 fa[2][FM], fb[2][FN];
  constexpr int NREAD = 2 * (FM + FN);
  auto read_op = [&](auto Rc, auto Sc, uint32_t boff) {
    constexpr int r = decltype(Rc)::value, S = decltype(Sc)::value;
    constexpr int frag = (r >> 1) % 4, hpart = r & 1;
    if constexpr (r < 2 * FM) {
      if constexpr (hpart == 0) ds_read_b128_i<frag * 4096>(fa[S][frag].lo, rdA[2 * S] + boff);
      else ds_read_b128_i<frag * 4096>(fa[S][frag].hi, rdA[2 * S + 1] + boff);
    } else {
      // fragment j's rows: paired, gate (j even) or up (j odd) rows
      // wn * 64 + (j / 2) * 32 of each 128-row half; else wn * 128 + 32 j
      constexpr int off = PAIR ? (frag & 1) * 16384 + (frag >> 1) * 4096 : frag * 4096;
      if constexpr (hpart == 0) ds_read_b128_i<off>(fb[S][frag].lo, rdB[2 * S] + boff);
      else ds_read_b128_i<off>(fb[S][frag].hi, rdB[2 * S + 1] + boff);
    }
  };
  auto fence_slot = [&](auto SLc) {
    constexpr int SL = decltype(SLc)::value;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    static_for<0, FM>([&](auto I) { fa[SL][I].fence(); });
    static_for<0, FN>([&](auto J) { fb[SL][J].fence(); });
  };

  f32x16_t acc[FM][FN];
  static_for<0, FM>([&](auto I) {
    static_for<0, FN>([&](auto J) { acc[I][J] = (f32x16_t)(0.0f); });
  });
  int unit_scale = 127;
  asm volatile("" : "+v"(unit_scale));

  if (nk > 0) {
    set_tile(tc.k_begin, true);
    static_for<0, 16>([&](auto L) { load_op(L, 0u); });
    set_tile(tc.k_begin + BKB, nk > 1);
    static_for<0, 16>([&](auto L) { load_op(L, (uint32_t)TILE_BYTES); });
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  }
  __builtin_amdgcn_s_barrier();
  if (nk > 0) {
    static_for<0, NREAD>([&](auto R) { read_op(R, std::integral_constant<int, 0>{}, 0u); });
  }
  asm volatile("s_nop 4");

  for (int kt = 0; kt < nk; ++kt) {
    const uint32_t cur = (uint32_t)(kt & 1) * TILE_BYTES;
    const uint32_t nxt = cur ^ TILE_BYTES;
    set_tile(tc.k_begin + (kt + 2) * BKB, kt + 2 < nk);
    static_for<0, 2>([&](auto Sc) {
      constexpr int S = decltype(Sc)::value;
      fence_slot(std::integral_constant<int, S>{});
      if constexpr (S == 1) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
      }
      constexpr int NLOAD = S == 1 ? 16 : 0;
      static_for<0, 16>([&](auto Mc) {
        constexpr int m = decltype(Mc)::value;
        constexpr int i = m >> 2, j = m & 3;
        mfma_f8_ordered<FA, FB>(acc[i][j], fb[S][j].op(), fa[S][i].op(), unit_scale);
        constexpr int r0 = m < 8 ? (m * NREAD) / 8 : NREAD;
        constexpr int r1 = m < 8 ? ((m + 1) * NREAD) / 8 : NREAD;
        static_for<r0, r1>([&](auto Oc) {
          read_op(Oc, std::integral_constant<int, S ^ 1>{}, S == 0 ? cur : nxt);
        });
        constexpr int l0 = (m * NLOAD) / 16, l1 = ((m + 1) * NLOAD) / 16;
        static_for<l0, l1>([&](auto Oc) {
          constexpr int idx = decltype(Oc)::value;
          load_op(std::integral_constant<int, (idx & 1) * 8 + (idx >> 1)>{}, cur);
        });
      });
    });
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");

  static_assert(EQ_BYTES <= (int)sizeof(lds), "staging rows exceed shared memory");
  __syncthreads();
  write_tile_staged<EPI, BMODE, OutT, FM, FN, WTM, WTN, LEAN_NT, QM>(
      acc, ea, tc, wm, wn, lane, tid, Ncols, reinterpret_cast<float*>(lds));
}

// ---- short-row kernel: 32 or 128 rows of a ragged problem ----------------
//
// Tiles of TM rows x 256 columns (TM = 32 or 128), 4 wavefronts side by side,
// each TM x 64 (TM/32 x 2 blocks of 32 x 32 x 16 MFMAs), a ring of NS
// shared-memory stages of [A TM x 64 | B 256 x 64] filled by direct loads
// that run NS - 1 k tiles ahead.  Each output element gets the same chain of
// 32 x 32 x 16 MFMAs over the same 16-wide k steps as in the 256 x 256
// kernels, so its value is the one those compute.  Two uses in grouped
// launches:
//  - TAIL (TM = 32): problems whose rows end a few rows past a multiple of
//    256 (e.g. 518..530 rows per expert) would spend a whole 256-row tile on
//    each problem's last rows, and those tiles make a second wave.  The
//    launcher gives such a remainder (at most THIN_MAX rows) to these tiles.
//  - all rows (TM = 128): a launch whose 256-row tiles leave many compute
//    units idle in its only wave (e.g. 147 tiles on 256 CUs) runs on twice
//    as many half-height tiles instead.
// Requirements (checked by the launcher): opA K-contiguous, a k split a
// multiple of 64.
constexpr int THIN_M = 32;
constexpr int THIN_MAX = 64;
constexpr int THIN_NT = 256;
constexpr int ROWS_M = 128;

template <int TM>
struct RowsCfg {
  static constexpr int FM = TM / 32;          // fragment rows per wavefront
  static constexpr int NS = TM == 32 ? 4 : 3;  // stages (144 KiB either way)
  static constexpr int A_LOADS = TM / 32;     // 1 KiB A loads per wavefront
  static constexpr int LOADS = A_LOADS + 8;   // direct loads per wavefront, k tile
};

template <int TM, bool TAIL, bool B_KMAJOR, int BMODE, int EPI, typename OutT>
__global__ __launch_bounds__(THIN_NT, 1) void gemm_rows(GemmArgs g) {
  gemm_wave_prio();
  using C = RowsCfg<TM>;
  constexpr int FM = C::FM, NS = C::NS;
  constexpr int A_ELEMS = TM * BK;
  constexpr int BUF_ELEMS = A_ELEMS + BN * BK;
  __shared__ __attribute__((aligned(1024))) bf16_t lds[NS * BUF_ELEMS];
  constexpr bool PAIR = EPI == EPI_SWIGLU_FWD;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r_lane = lane & 31, c_lane = lane >> 5;

  // TAIL: problem e's tiles cover its rows from the last multiple of 256 on;
  // otherwise all of its rows
  int e = 0, lo, hi, local, tiles_m;
  if (g.dev_off) {
    // device-resident offsets (remainder tiles only): there are tiles when
    // the offsets call for thin remainders; spare workgroups exit at once
    if (!TAIL) return;
    int lo_l, hi_l, t0, t1, tile;
    dev_lane_rows(g, lo_l, hi_l);
    if (dev_tiling(g, hi_l - lo_l) != DEV_T256_THIN) return;
    const int rem = (hi_l - lo_l) % BM;
    const int tr = (rem > 0 && rem <= g.dev_thin) ? (rem + TM - 1) / TM : 0;
    if (!dev_find_tile(tr * g.tiles_n, blockIdx.x, lo_l, hi_l, e, t0, t1, lo, hi, tile)) return;
    local = tile - t0;
    tiles_m = (t1 - t0) / g.tiles_n;
  } else {
    const int tile = xcd_logical_block(blockIdx.x, gridDim.x);
    while (e + 1 < g.E && tile >= g.tile_off[e + 1]) ++e;
    local = tile - g.tile_off[e];
    lo = g.row_off[e];
    hi = g.row_off[e + 1];
    tiles_m = (g.tile_off[e + 1] - g.tile_off[e]) / g.tiles_n;
  }
  TileCoord tc;
  tc.e = e;
  tc.tm = local % tiles_m;
  tc.tn = local / tiles_m;
  tc.m_begin = lo + (TAIL ? ((hi - lo) / BM) * BM : 0) + tc.tm * TM;
  tc.m_end = hi;
  tc.k_begin = 0;
  tc.k_end = g.K;

  const bf16_t* a0 = reinterpret_cast<const bf16_t*>(g.a.p0) + tc.e * g.a.bstride;
  const bf16_t* b0 = reinterpret_cast<const bf16_t*>(g.b.p0) + tc.e * g.b.bstride;
  const bf16_t* b1 = reinterpret_cast<const bf16_t*>(g.b.p1) + tc.e * g.b.bstride;
  const int64_t lda = g.a.ld, ldb = g.b.ld, bsplit = g.b.split;
  const int Ncols = g.N, Ktot = g.K;
  const EpiArgs ea = g.epi;
  const int n_base = tc.tn * BN;
  const int m_rows = tc.m_end - tc.m_begin;
  const int nk = (Ktot + BK - 1) / BK;
  const int half_w = wave >> 1;

  // k tile from k0 into buffer `buf` (k0 >= K masks every load)
  auto issue = [&](int k0, bf16_t* buf) {
    // A: TM rows x 64 k, TM / 32 direct loads of 1 KiB (8 rows) per wavefront
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      const int blk = wave * C::A_LOADS + i;
      const int r = blk * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      const int k = k0 + c * 8;
      const uint32_t off = (r < m_rows && k < Ktot)
                               ? (uint32_t)(((int64_t)r * lda + k) * 2) : OOB_OFF;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(a0 + (int64_t)tc.m_begin * lda),
                                               (lds_void_t*)(buf + blk * 512), 16, off, 0, 0,
                                               0);
    }
    bf16_t* tb = buf + A_ELEMS;
    if constexpr (B_KMAJOR) {
      if constexpr (BMODE == BMODE_KSPLIT) {
        const bool first = k0 < bsplit;
        const bf16_t* bp = first ? b0 : b1;
        const int kl = first ? k0 : k0 - (int)bsplit;
        const int lim = first ? (int)bsplit : Ktot - (int)bsplit;
        direct_kmajor<4, 0, 8>(make_rsrc(bp + (int64_t)n_base * ldb), ldb, Ncols - n_base, kl,
                               k0 < Ktot ? lim : 0, tb, wave, lane);
      } else {
        direct_kmajor<4, 0, 8>(make_rsrc(b0 + (int64_t)n_base * ldb), ldb, Ncols - n_base, k0,
                               Ktot, tb, wave, lane);
      }
    } else if constexpr (BMODE == BMODE_PAIR32) {
      // half 0: gate columns, half 1: up columns, both f = 128 tn ..
      const bf16_t* bp = half_w ? b1 : b0;
      direct_mn<4, 0, 8>(make_rsrc(bp + (int64_t)k0 * ldb), ldb, tc.tn * 128, (int)bsplit,
                         Ktot - k0, tb, wave, lane);
    } else {
      direct_mn<4, 0, 8>(make_rsrc(b0 + (int64_t)k0 * ldb), ldb, n_base + half_w * 128, Ncols,
                         Ktot - k0, tb, wave, lane);
    }
  };
  // tile column of this wavefront's opB block j
  auto b_col = [&](int j) { return PAIR ? j * (BN / 2) + wave * 32 : wave * 64 + j * 32; };

  f32x16_t acc[FM][2];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    acc[i][0] = (f32x16_t)(0.0f);
    acc[i][1] = (f32x16_t)(0.0f);
  }

  // prologue: tiles 0 .. NS-2 in flight, wait for tile 0
  if (nk > 0) {
#pragma unroll
    for (int t = 0; t < NS - 1; ++t) issue(t * BK, lds + t * BUF_ELEMS);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * C::LOADS) : "memory");
  }
  // a plain s_barrier: __syncthreads() would also drain the loads of the
  // tiles behind tile 0; the empty asm keeps every shared-memory read below it
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  for (int kt = 0; kt < nk; ++kt) {
    const bf16_t* cur = lds + (kt % NS) * BUF_ELEMS;
    // tile kt + NS - 1 refills the stage of tile kt - 1, which every
    // wavefront finished reading before the last barrier (past the end:
    // masked loads, zeros, never read)
    issue((kt + NS - 1) * BK, lds + ((kt + NS - 1) % NS) * BUF_ELEMS);
    const bf16_t* tb = cur + A_ELEMS;
    // fragments of k step s go to slot s % 2: the next step's reads are in
    // flight while this step's MFMAs run
    bf16x8_t fa[2][FM], fb[2][2];
    auto read_step = [&](int s, int slot) {
      const int c = 2 * s + c_lane;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[slot][i] = *reinterpret_cast<const bf16x8_t*>(cur + lds_off(i * 32 + r_lane, c));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (B_KMAJOR)
          fb[slot][j] = *reinterpret_cast<const bf16x8_t*>(tb + lds_off(b_col(j) + r_lane, c));
        else
          fb[slot][j] = frag_mn(tb, b_col(j), 16 * s, lane);
      }
    };
    read_step(0, 0);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      if (s + 1 < BK / 16) read_step(s + 1, (s + 1) & 1);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s & 1][j], fa[s & 1][i],
                                                              acc[i][j], 0, 0, 0);
    }
    // after the barrier, tile kt + 1 has landed for every wavefront (tiles
    // kt + 2 .. kt + NS - 1 stay in flight) and every read of `cur` has
    // completed (lgkmcnt), so the next trip may refill it
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((NS - 2) * C::LOADS) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  // the masked loads of the stages past the end land before the stage
  // area is reused
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // stage the TM x 256 fp32 sums row-major (paired SwiGLU: gate sums in
  // columns 0..127, up sums in 128..255), then each thread takes 8
  // consecutive columns of a row
  float* stage = reinterpret_cast<float*>(lds);
  static_assert(TM * EQ_PITCH * 4 <= (int)sizeof(lds), "staging rows exceed shared memory");
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col0 = b_col(j);
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4_t v = {acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                           acc[i][j][4 * gq + 3]};
        *reinterpret_cast<f32x4_t*>(stage + (i * 32 + r_lane) * EQ_PITCH + col0 + 8 * gq +
                                    4 * c_lane) = v;
      }
    }
  }
  __syncthreads();
  if constexpr (PAIR) {
    constexpr int CH = TM * (BN / 2) / 8;
#pragma unroll
    for (int kk = 0; kk < CH / THIN_NT; ++kk) {
      const int k = kk * THIN_NT + tid;
      const int row = k >> 4, cc = (k & 15) * 8;
      const int64_t m = tc.m_begin + row;
      const int64_t f = (int64_t)tc.tn * (BN / 2) + cc;
      if (m < tc.m_end && f < ea.split) {
        float gv[8], uv[8];
        const float* src = stage + row * EQ_PITCH + cc;
        *reinterpret_cast<f32x4_t*>(gv) = *reinterpret_cast<const f32x4_t*>(src);
        *reinterpret_cast<f32x4_t*>(gv + 4) = *reinterpret_cast<const f32x4_t*>(src + 4);
        *reinterpret_cast<f32x4_t*>(uv) = *reinterpret_cast<const f32x4_t*>(src + BN / 2);
        *reinterpret_cast<f32x4_t*>(uv + 4) = *reinterpret_cast<const f32x4_t*>(src + BN / 2 + 4);
        epilogue_swiglu8<bf16_t>(ea, m, f, gv, uv);
      }
    }
  } else {
    constexpr int CH = TM * BN / 8;
#pragma unroll
    for (int kk = 0; kk < CH / THIN_NT; ++kk) {
      const int k = kk * THIN_NT + tid;
      const int row = k >> 5, cc = (k & 31) * 8;
      const int64_t m = tc.m_begin + row;
      const int64_t n = (int64_t)n_base + cc;
      if (m < tc.m_end && n < Ncols) {
        float cv[8];
        const float* src = stage + row * EQ_PITCH + cc;
        *reinterpret_cast<f32x4_t*>(cv) = *reinterpret_cast<const f32x4_t*>(src);
        *reinterpret_cast<f32x4_t*>(cv + 4) = *reinterpret_cast<const f32x4_t*>(src + 4);
        epilogue8<EPI, bf16_t, OutT>(ea, tc.e, m, n, cv);
      }
    }
  }
}

}  // namespace mfma256

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// general kernel's wavefront layout; hand-ordered kernel on/off
#ifndef TP_NW_DEFAULT
#define TP_NW_DEFAULT 8
#endif
#ifndef TP_USE_LEAN
#define TP_USE_LEAN 1
#endif
#ifndef TP_USE_RING
#define TP_USE_RING 1
#endif
#ifndef TP_USE_W16
#define TP_USE_W16 1
#endif

#ifndef TP_USE_THIN
#define TP_USE_THIN 1
#endif

// Tile rows of a problem with `rows` rows.  With thin_max > 0 a remainder of
// at most thin_max rows past the last whole BM-row tile is left to the thin
// kernel (which then covers it; see fill_thin).
static int row_tiles(int rows, int BM, int thin_max) {
  if (thin_max > 0) {
    const int rem = rows % BM;
    return rows / BM + (rem > thin_max ? 1 : 0);
  }
  return (rows + BM - 1) / BM;
}

static int problem_rows(const GemmArgs& g, int e) {
  return g.ragged == RAGGED_M ? g.row_off[e + 1] - g.row_off[e] : g.M;
}

static void fill_tiles(GemmArgs& g, int BM, int BN, int n_cols, int thin_max = 0) {
  g.tiles_n = (n_cols + BN - 1) / BN;
  g.tile_off[0] = 0;
  for (int e = 0; e < g.E; ++e)
    g.tile_off[e + 1] = g.tile_off[e] + row_tiles(problem_rows(g, e), BM, thin_max) * g.tiles_n;
}

// Short-row tiles (TM rows): with `tail`, of the remainders the 256-row
// tiles leave out (at most THIN_MAX rows past a multiple of 256); without,
// of every row.
static int short_row_tiles(int rows, int TM, bool tail) {
  using namespace mfma256;
  if (!tail) return (rows + TM - 1) / TM;
  const int rem = rows % BM;
  return (rem > 0 && rem <= THIN_MAX) ? (rem + TM - 1) / TM : 0;
}

static void fill_short(GemmArgs& g, int TM, bool tail, int tiles_n) {
  g.tiles_n = tiles_n;
  g.tile_off[0] = 0;
  for (int e = 0; e < g.E; ++e)
    g.tile_off[e + 1] = g.tile_off[e] + short_row_tiles(problem_rows(g, e), TM, tail) * tiles_n;
}

static int count_tiles(const GemmArgs& g, int BMT, int BNT, int n_cols, int thin_max = 0);
static int device_cus();

// The short-row kernel's requirements: ragged rows (the grouped experts), a
// K-contiguous opA, a k split on a 64 boundary.
template <bool AK, bool BK_, int BMODE>
static bool short_rows_ok(const GemmArgs& g) {
  using namespace mfma256;
  if (!TP_USE_THIN || !AK || (BMODE == BMODE_PAIR32 && BK_) || g.ragged != RAGGED_M) return false;
  return BMODE != BMODE_KSPLIT || g.b.split % BK == 0;
}

// Whether a launch leaves remainders to the thin kernel: ragged rows (the
// grouped experts), a K-contiguous opA, a k split on a 64 boundary, at
// least one problem whose rows end a few rows past a multiple of 256, and
// the 256-row launch one wave of tiles over the compute units shorter for
// it (otherwise the thin tiles would only add time after a launch that
// already fits).
template <bool AK, bool BK_, int BMODE>
static int thin_rows_max(const GemmArgs& g) {
  using namespace mfma256;
  if (!short_rows_ok<AK, BK_, BMODE>(g)) return 0;
  bool any = false;
  for (int e = 0; e < g.E; ++e) {
    const int rem = problem_rows(g, e) % BM;
    any = any || (rem > 0 && rem <= THIN_MAX);
  }
  if (!any) return 0;
  const bool pair = BMODE == BMODE_PAIR32;
  const int n_cols = pair ? (int)g.b.split : g.N, bn = pair ? BN / 2 : BN;
  const int cus = device_cus();
  const int w_plain = (count_tiles(g, BM, bn, n_cols, 0) + cus - 1) / cus;
  const int w_thin = (count_tiles(g, BM, bn, n_cols, THIN_MAX) + cus - 1) / cus;
  return w_thin < w_plain ? THIN_MAX : 0;
}

// Whether the whole launch runs on 128-row tiles instead: when its 256-row
// tiles (with any thin remainder tiles) take whole waves over the compute
// units that half-height tiles take fewer of, by tile area.  The half-height
// kernel reads more shared memory per MFMA, so its area counts 1.5 times.
constexpr double ROWS128_FACTOR = 1.5;
template <bool AK, bool BK_, int BMODE>
static bool rows128_pays(const GemmArgs& g, int thin_max) {
  using namespace mfma256;
  if (!short_rows_ok<AK, BK_, BMODE>(g)) return false;
  const bool pair = BMODE == BMODE_PAIR32;
  const int n_cols = pair ? (int)g.b.split : g.N, bn = pair ? BN / 2 : BN;
  const int tn = (n_cols + bn - 1) / bn;
  const int cus = device_cus();
  int t128 = 0;
  for (int e = 0; e < g.E; ++e) t128 += short_row_tiles(problem_rows(g, e), ROWS_M, false) * tn;
  const double c256 = (double)((count_tiles(g, BM, bn, n_cols, thin_max) + cus - 1) / cus) *
                      BM * BN;
  const double c128 = ROWS128_FACTOR * (double)((t128 + cus - 1) / cus) * ROWS_M * BN;
  return c128 < c256;
}

template <int TM, bool TAIL, bool BK_, int BMODE, int EPI, typename OutT>
static hipError_t launch_short(GemmArgs& g, hipStream_t stream) {
  using namespace mfma256;
  fill_short(g, TM, TAIL,
             BMODE == BMODE_PAIR32 ? (int)((g.b.split + 127) / 128) : (g.N + BN - 1) / BN);
  const int blocks = g.tile_off[g.E];
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_rows<TM, TAIL, BK_, BMODE, EPI, OutT>), dim3(blocks), dim3(THIN_NT),
                     0, stream, g);
  return hipGetLastError();
}

// compute units of the current device (cached per device)
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

// tiles of a BMT x BNT grid (n_cols: columns as tiled)
static int count_tiles(const GemmArgs& g, int BMT, int BNT, int n_cols, int thin_max) {
  const int tn = (n_cols + BNT - 1) / BNT;
  int t = 0;
  for (int e = 0; e < g.E; ++e) t += row_tiles(problem_rows(g, e), BMT, thin_max) * tn;
  return t;
}

// Tile shape for the bf16 GEMM: 256 x 256 unless a 224-wide shape fills
// the compute units in fewer tile-area waves (whole waves x tile area).  The
// 16 x 16 x 32 MFMA of the 224-wide kernel takes about 9 % more cycles per
// FLOP than 32 x 32 x 16 (measured on an MFMA-only loop and on the GEMM
// k loop), so its cost is scaled by that.
// Returns 0 (256 x 256), 1 (256 x 224) or 2 (224 x 256).
#ifndef TP_W16_FACTOR
#define TP_W16_FACTOR 1.09
#endif
constexpr double W16_CYCLE_FACTOR = TP_W16_FACTOR;
#ifndef TP_W16_PAIR_EXTRA
#define TP_W16_PAIR_EXTRA 1.1
#endif
constexpr double W16_PAIR_EXTRA = TP_W16_PAIR_EXTRA;
// thin_max: remainders left to the thin kernel by 256-row tiles (the
// 224-row shape covers every row itself).
struct ShapeCost {
  int shape;
  double cost;
};
static ShapeCost pick_shape_cost(const GemmArgs& g, int bmode, bool w16_ok, int thin_max) {
  const int cus = device_cus();
  auto cost = [&](int BMT, int BNT, int tiles) {
    const double f = (BMT == 256 && BNT == 256) ? 1.0 : W16_CYCLE_FACTOR;
    return f * (double)((tiles + cus - 1) / cus) * BMT * BNT;
  };
  const bool w16 = TP_USE_W16 && w16_ok;
  if (bmode == BMODE_PAIR32) {
    // the paired 224-wide tiles also pay a heavier epilogue: measured on
    // the SwiGLU FC1 (4096 tokens, H = 8192, F/T = 3584), 448 256-wide
    // tiles in two waves take 431 us in the overlapped step (406 in order),
    // 512 224-wide ones 480 (442)
    const int split = (int)g.b.split;
    const double c0 = cost(256, 256, count_tiles(g, 256, 128, split, thin_max));
    if (!w16) return {0, c0};
    const double c1 =
        W16_PAIR_EXTRA * cost(256, 224, count_tiles(g, 256, 112, split, thin_max));
    return c1 < c0 ? ShapeCost{1, c1} : ShapeCost{0, c0};
  }
  const double c0 = cost(256, 256, count_tiles(g, 256, 256, g.N, thin_max));
  if (!w16) return {0, c0};
  const double c1 = cost(256, 224, count_tiles(g, 256, 224, g.N, thin_max));
  const double c2 = thin_max > 0 ? 1e300 : cost(224, 256, count_tiles(g, 224, 256, g.N));
  if (c1 < c0 && c1 <= c2) return {1, c1};
  if (c2 < c0) return {2, c2};
  return {0, c0};
}
static int pick_shape(const GemmArgs& g, int bmode, bool w16_ok, int thin_max) {
  return pick_shape_cost(g, bmode, w16_ok, thin_max).shape;
}

// 128-row tiles of the hand-ordered kernel: taken when they fill the compute
// units in fewer tile-area waves than the 256-row launch would (a launch
// with few tiles per compute unit, e.g. a weight gradient of 128 tiles on
// 256 compute units).  Their fragment reads cost 1.5 times the shared
// memory per MFMA, so their area counts TP_LEAN128_FACTOR times.
#ifndef TP_LEAN128_FACTOR
#define TP_LEAN128_FACTOR 1.2
#endif
template <bool AK, bool BK_, int BMODE>
static bool lean_ok(const GemmArgs& g) {
  const bool k_whole = (!AK && !BK_) || g.K % mfma256::BK == 0;
  const bool split_ok = BMODE != BMODE_KSPLIT || g.b.split % mfma256::BK == 0;
  return TP_USE_LEAN && k_whole && split_ok && !(BMODE == BMODE_PAIR32 && BK_);
}
template <bool AK, bool BK_, int BMODE>
static bool lean128_pays(const GemmArgs& g, int thin_max) {
  if (!lean_ok<AK, BK_, BMODE>(g)) return false;
  const bool pair = BMODE == BMODE_PAIR32;
  const int n_cols = pair ? (int)g.b.split : g.N, bn = pair ? 128 : 256;
  const int cus = device_cus();
  const int t128 = count_tiles(g, 128, bn, n_cols, 0);
  const double c128 = TP_LEAN128_FACTOR * (double)((t128 + cus - 1) / cus) * 128 * 256;
  const bool k_whole = (!AK && !BK_) || g.K % mfma256::BK == 0;
  const bool w16_ok = k_whole && BMODE != BMODE_KSPLIT && !(BMODE == BMODE_PAIR32 && BK_);
  return c128 < pick_shape_cost(g, BMODE, w16_ok, thin_max).cost;
}
template <bool AK, bool BK_, int BMODE, int EPI, typename OutT>
static hipError_t launch_lean128(GemmArgs& g, hipStream_t stream) {
  int n_cols = g.N;
  if (BMODE == BMODE_PAIR32) {
    n_cols = ((int)((g.b.split + 31) / 32)) * 64;
    g.N = n_cols;
  }
  fill_tiles(g, 128, mfma256::BN, n_cols, 0);
  const int blocks = g.tile_off[g.E];
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((mfma256::gemm_lean<128, AK, BK_, BMODE, EPI, OutT>), dim3(blocks),
                     dim3(mfma256::LEAN_NT), 0, stream, g);
  return hipGetLastError();
}

template <bool AK, bool BK_, int BMODE, int EPI, typename OutT, int BMT, int BNT>
static hipError_t launch_w16(GemmArgs& g, hipStream_t stream, int thin_max) {
  if constexpr (BMODE == BMODE_KSPLIT || (BMODE == BMODE_PAIR32 && (BK_ || BNT != 224))) {
    return hipErrorInvalidValue;
  } else {
    if (BMODE == BMODE_PAIR32) {
      // 112 gate + 112 up columns per tile
      const int tiles_n = (int)((g.b.split + 111) / 112);
      g.N = tiles_n * 224;
    }
    fill_tiles(g, BMT, BNT, g.N, BMT == 256 ? thin_max : 0);
    const int blocks = g.tile_off[g.E];
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((mfma256::gemm_w16<AK, BK_, BMODE, EPI, OutT, BMT, BNT>), dim3(blocks),
                       dim3(mfma256::W16_NT), 0, stream, g);
    return hipGetLastError();
  }
}

// The 256-row launch, then (for grouped problems ending a few rows past a
// multiple of 256) the thin launch over those rows.
template <int NW, bool AK, bool BK_, int BMODE, int EPI, typename OutT>
static hipError_t launch_rows(GemmArgs& g, hipStream_t stream, int thin_max);

template <int NW, bool AK, bool BK_, int BMODE, int EPI, typename OutT>
static hipError_t launch_256(GemmArgs& g, int blocks, hipStream_t stream);

// Row-ragged grouped launches whose row offsets stay in device memory: the
// host does not see the rows, so the launch covers 256 x 256 tiles for
// every split of dev_rows rows into E problems, at most (dev_rows + E (BM -
// 1)) / BM tile rows in all, and queues the other tilings the host could
// pick beside it: 128-row tiles, and a thin launch for remainders of at
// most THIN_MAX rows.  Every workgroup takes the host's choice from the
// offsets; those of the launches not chosen exit at once, as do those past
// the tiles the offsets need.  (A k-ragged launch's tiles do not
// depend on the rows: it takes the host's usual choice, and its kernels
// read their k ranges from the device offsets.)
template <int NW, bool AK, bool BK_, int BMODE, int EPI, typename OutT>
static hipError_t launch_devoff(GemmArgs& g, hipStream_t stream) {
  using namespace mfma256;
  if (g.ragged != RAGGED_M || g.dev_rows < 0) return hipErrorInvalidValue;
  const int n_given = g.N;  // (the thin kernel takes the columns as given)
  int n_cols = g.N;
  if (BMODE == BMODE_PAIR32) {
    n_cols = ((int)((g.b.split + 31) / 32)) * 64;
    g.N = n_cols;
  }
  g.tiles_n = (n_cols + BN - 1) / BN;
  const int64_t blocks = ((int64_t)g.dev_rows + (int64_t)g.E * (BM - 1)) / BM * g.tiles_n;
  // the other tilings the host could pick (the kernels choose from the
  // offsets as the host would from host ones): remainders of at most
  // THIN_MAX rows on the thin kernel, at most THIN_MAX / THIN_M tile rows
  // per problem; 128-row tiles on the hand-ordered kernel.
  //
  // A workgroup that only finds it has nothing to do still holds a compute
  // unit for ~2 us.  Worst-case grids of more than three waves (R far above
  // the rows routed) therefore run the hand-ordered launches as loops over
  // their tiles on one workgroup per compute unit (their k loop is ~6 %
  // slower: the loop's state spills scalar registers); smaller ones keep
  // one tile per workgroup, the 128-row tiling only when its grid fits one
  // wave (on the grouped-expert workload a grid of 429 idle workgroups
  // added 7.5 us to FC1, where 128-row tiles do not pay).
  const int64_t b128 = ((int64_t)g.dev_rows + (int64_t)g.E * 127) / 128 * g.tiles_n;
  const bool lean = lean_ok<AK, BK_, BMODE>(g);
  const bool thin = short_rows_ok<AK, BK_, BMODE>(g);
  if (blocks > INT32_MAX || b128 > INT32_MAX) return hipErrorInvalidValue;
  g.dev_cus = device_cus();
  const int64_t loop_grid = std::max(8, g.dev_cus / 8 * 8);
  const bool loop = lean && blocks > 3 * loop_grid;
  const bool l128 = lean && (loop || b128 <= g.dev_cus);
  g.dev_thin = thin ? THIN_MAX : 0;
  g.dev_l128 = l128 ? (int)(TP_LEAN128_FACTOR * 1000 + 0.5) : 0;
  if (blocks == 0) return hipSuccess;
  hipError_t he;
  if (loop) {
    hipLaunchKernelGGL((gemm_lean<256, AK, BK_, BMODE, EPI, OutT, true>), dim3((int)loop_grid),
                       dim3(LEAN_NT), 0, stream, g);
    if ((he = hipGetLastError()) != hipSuccess) return he;
    hipLaunchKernelGGL((gemm_lean<128, AK, BK_, BMODE, EPI, OutT, true>),
                       dim3((int)std::min(b128, loop_grid)), dim3(LEAN_NT), 0, stream, g);
  } else {
    he = launch_256<NW, AK, BK_, BMODE, EPI, OutT>(g, (int)blocks, stream);
    if (he != hipSuccess) return he;
    if (l128)
      hipLaunchKernelGGL((gemm_lean<128, AK, BK_, BMODE, EPI, OutT>), dim3((int)b128),
                         dim3(LEAN_NT), 0, stream, g);
  }
  if ((he = hipGetLastError()) != hipSuccess || !thin) return he;
  if (!thin) return hipSuccess;
  if constexpr (AK && !(BMODE == BMODE_PAIR32 && BK_)) {
    g.N = n_given;
    const int tblocks = g.E * (THIN_MAX / THIN_M) * g.tiles_n;
    hipLaunchKernelGGL((gemm_rows<THIN_M, true, BK_, BMODE, EPI, OutT>), dim3(tblocks),
                       dim3(THIN_NT), 0, stream, g);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int NW, bool AK, bool BK_, int BMODE, int EPI, typename OutT>
static hipError_t launch_mfma(GemmArgs& g, hipStream_t stream) {
  if (g.dev_off && g.ragged == RAGGED_M)
    return launch_devoff<NW, AK, BK_, BMODE, EPI, OutT>(g, stream);
  const int thin_max = thin_rows_max<AK, BK_, BMODE>(g);
  if (lean128_pays<AK, BK_, BMODE>(g, thin_max))
    return launch_lean128<AK, BK_, BMODE, EPI, OutT>(g, stream);
  if constexpr (AK && !(BMODE == BMODE_PAIR32 && BK_)) {
    // (the compiler-scheduled 128-row kernel serves launches the hand-ordered
    // one cannot take: k extents that are not whole 64-wide tiles)
    if (!lean_ok<AK, BK_, BMODE>(g) && rows128_pays<AK, BK_, BMODE>(g, thin_max))
      return launch_short<mfma256::ROWS_M, false, BK_, BMODE, EPI, OutT>(g, stream);
    if (thin_max > 0) {
      GemmArgs gt = g;  // the main launch rewrites its tile table (and N)
      hipError_t he = launch_rows<NW, AK, BK_, BMODE, EPI, OutT>(g, stream, thin_max);
      if (he != hipSuccess) return he;
      return launch_short<mfma256::THIN_M, true, BK_, BMODE, EPI, OutT>(gt, stream);
    }
  }
  return launch_rows<NW, AK, BK_, BMODE, EPI, OutT>(g, stream, 0);
}

template <int NW, bool AK, bool BK_, int BMODE, int EPI, typename OutT>
static hipError_t launch_rows(GemmArgs& g, hipStream_t stream, int thin_max) {
  {
    const bool k_whole = (!AK && !BK_) || g.K % mfma256::BK == 0;
    const bool w16_ok = k_whole && BMODE != BMODE_KSPLIT && !(BMODE == BMODE_PAIR32 && BK_);
    switch (pick_shape(g, BMODE, w16_ok, thin_max)) {
      case 1: return launch_w16<AK, BK_, BMODE, EPI, OutT, 256, 224>(g, stream, thin_max);
      case 2:
        // (never chosen when remainders go to the thin kernel: 224-row
        // tiles would cover those rows too)
        if constexpr (BMODE != BMODE_PAIR32)
          if (thin_max == 0) return launch_w16<AK, BK_, BMODE, EPI, OutT, 224, 256>(g, stream, 0);
        break;
      default: break;
    }
  }
  int n_cols = g.N;
  if (BMODE == BMODE_PAIR32) {
    // logical columns are laid out in 64-wide (gate 32 | up 32) groups
    n_cols = ((int)((g.b.split + 31) / 32)) * 64;
    g.N = n_cols;
  }
  fill_tiles(g, mfma256::BM, mfma256::BN, n_cols, thin_max);
  return launch_256<NW, AK, BK_, BMODE, EPI, OutT>(g, g.tile_off[g.E], stream);
}

// `blocks` 256 x 256 tiles on the hand-ordered kernel, else the ring
// kernel, else the general one (whichever first takes the k extents).
template <int NW, bool AK, bool BK_, int BMODE, int EPI, typename OutT>
static hipError_t launch_256(GemmArgs& g, int blocks, hipStream_t stream) {
  if (blocks == 0) return hipSuccess;
  // the hand-ordered kernel needs whole 64-wide k tiles of K-contiguous
  // operands and a 64-aligned k split
  const bool k_whole = (!AK && !BK_) || g.K % mfma256::BK == 0;
  const bool split_ok = BMODE != BMODE_KSPLIT || g.b.split % mfma256::BK == 0;
  // the ring kernel needs whole 32-wide k tiles and a 32-aligned k split
  const bool ring_ok = ((!AK && !BK_) || g.K % mfma256::RBK == 0) &&
                       (BMODE != BMODE_KSPLIT || g.b.split % mfma256::RBK == 0);
  if (TP_USE_LEAN && k_whole && split_ok) {
    hipLaunchKernelGGL((mfma256::gemm_lean<256, AK, BK_, BMODE, EPI, OutT>), dim3(blocks),
                       dim3(mfma256::LEAN_NT), 0, stream, g);
    return hipGetLastError();
  }
  if (TP_USE_RING && ring_ok) {
    hipLaunchKernelGGL((mfma256::gemm_ring<AK, BK_, BMODE, EPI, OutT>), dim3(blocks),
                       dim3(mfma256::LEAN_NT), 0, stream, g);
    return hipGetLastError();
  }
  // a K-contiguous opB goes straight to shared memory unless a 64-wide k
  // tile could straddle its two source matrices
  const bool b_direct = BK_ && split_ok;
  if (b_direct)
    hipLaunchKernelGGL((mfma256::gemm_kernel<NW, AK, BK_, BMODE, EPI, OutT, BK_>),
                       dim3(blocks), dim3(64 * NW), 0, stream, g);
  else
    hipLaunchKernelGGL((mfma256::gemm_kernel<NW, AK, BK_, BMODE, EPI, OutT, false>),
                       dim3(blocks), dim3(64 * NW), 0, stream, g);
  return hipGetLastError();
}

// GEMMs whose dZ operand is formed from dH and the saved activations as it
// is loaded: the general kernel's 8-wavefront layout, whose register file
// has room for the staged pieces beside 128 accumulators per wavefront.
// Dense problems only.
template <int PA, int PB, bool AK, bool BK_, int BMODE, int EPI, typename OutT>
static hipError_t launch_dact(GemmArgs& g, hipStream_t stream) {
  using namespace mfma256;
  if (g.E != 1 || g.ragged != RAGGED_NONE || g.a.bstride || g.b.bstride) return hipErrorInvalidValue;
  fill_tiles(g, BM, BN, g.N);
  const int blocks = g.tile_off[g.E];
  if (blocks == 0) return hipSuccess;
  if constexpr (BK_) {
    if (BMODE != BMODE_KSPLIT || g.b.split % BK == 0) {
      hipLaunchKernelGGL((gemm_kernel<8, AK, BK_, BMODE, EPI, OutT, true, PA, PB>), dim3(blocks),
                         dim3(64 * 8), 0, stream, g);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<8, AK, BK_, BMODE, EPI, OutT, false, PA, PB>), dim3(blocks),
                     dim3(64 * 8), 0, stream, g);
  return hipGetLastError();
}

template <int BMODE, int EPI, int QM, int FA = 0, int FB = 0, typename OutT = bf16_t>
static hipError_t launch_f8(GemmArgs& g, hipStream_t stream) {
  int n_cols = g.N;
  if (BMODE == BMODE_PAIR32) {
    // 128 gate + 128 up columns per tile
    n_cols = (int)((g.b.split + 127) / 128) * 256;
    g.N = n_cols;
  }
  fill_tiles(g, mfma256::BM, mfma256::BN, n_cols);
  const int blocks = g.tile_off[g.E];
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((mfma256::gemm_f8<BMODE, EPI, QM, FA, FB, OutT>), dim3(blocks),
                     dim3(mfma256::LEAN_NT), 0, stream, g);
  return hipGetLastError();
}

hipError_t gemm_fp8(GemmKind kind, GemmArgs& g, hipStream_t stream) {
  switch (kind) {
    case GK_FC1_SWIGLU_F8:
      return launch_f8<BMODE_PAIR32, EPI_SWIGLU_FWD, 1>(g, stream);
    case GK_FC1_GELU_F8:
      return launch_f8<BMODE_PLAIN, EPI_GELU_FWD, 1>(g, stream);
    case GK_FC2_F8:
      return launch_f8<BMODE_PLAIN, EPI_STORE, 2>(g, stream);
    // backward: A operand E5M2 (gradients) or E4M3 (activations), B likewise
    case GK_DH_GELU_F8:
      return launch_f8<BMODE_PLAIN, EPI_GELU_BWD, 4, 1, 0>(g, stream);
    case GK_DH_SWIGLU_F8:
      return launch_f8<BMODE_PLAIN, EPI_SWIGLU_BWD, 4, 1, 0>(g, stream);
    case GK_WGRAD_F8:
      return launch_f8<BMODE_PLAIN, EPI_STORE, 3, 0, 1, float>(g, stream);
    case GK_WGRAD_SPLIT_F8:
      return launch_f8<BMODE_PLAIN, EPI_STORE_SPLIT, 3, 0, 1, float>(g, stream);
    case GK_DX_F8:
      return launch_f8<BMODE_PLAIN, EPI_STORE, 3, 1, 0>(g, stream);
    case GK_DX_KSPLIT_F8:
      return launch_f8<BMODE_KSPLIT, EPI_STORE, 3, 1, 0>(g, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t gemm_bf16(GemmKind kind, GemmArgs& g, hipStream_t stream) {
  switch (kind) {
    case GK_FC1_GELU:
      return launch_mfma<TP_NW_DEFAULT, true, false, BMODE_PLAIN, EPI_GELU_FWD, bf16_t>(g, stream);
    case GK_FC1_SWIGLU:
      return launch_mfma<TP_NW_DEFAULT, true, false, BMODE_PAIR32, EPI_SWIGLU_FWD, bf16_t>(g, stream);
    case GK_FC2:
      return launch_mfma<TP_NW_DEFAULT, true, false, BMODE_PLAIN, EPI_STORE, bf16_t>(g, stream);
    case GK_DH_GELU:
      return launch_mfma<TP_NW_DEFAULT, true, true, BMODE_PLAIN, EPI_GELU_BWD, bf16_t>(g, stream);
    case GK_DH_SWIGLU:
      return launch_mfma<TP_NW_DEFAULT, true, true, BMODE_PLAIN, EPI_SWIGLU_BWD, bf16_t>(g, stream);
    case GK_WGRAD:
      return launch_mfma<TP_NW_DEFAULT, false, false, BMODE_PLAIN, EPI_STORE, float>(g, stream);
    case GK_WGRAD_SPLIT:
      return launch_mfma<TP_NW_DEFAULT, false, false, BMODE_PLAIN, EPI_STORE_SPLIT, float>(g, stream);
    case GK_DX:
      return launch_mfma<TP_NW_DEFAULT, true, true, BMODE_PLAIN, EPI_STORE, bf16_t>(g, stream);
    case GK_DX_KSPLIT:
      return launch_mfma<TP_NW_DEFAULT, true, true, BMODE_KSPLIT, EPI_STORE, bf16_t>(g, stream);
    case GK_WGRAD_ACC:
      return launch_mfma<TP_NW_DEFAULT, false, false, BMODE_PLAIN, EPI_ACC, float>(g, stream);
    case GK_WGRAD_SPLIT_ACC:
      return launch_mfma<TP_NW_DEFAULT, false, false, BMODE_PLAIN, EPI_ACC_SPLIT, float>(g, stream);
    case GK_WGRAD_DACT_GELU:
      return launch_dact<DACT_NONE, DACT_GELU, false, false, BMODE_PLAIN, EPI_STORE, float>(g, stream);
    case GK_WGRAD_SPLIT_DACT_SWIGLU:
      return launch_dact<DACT_NONE, DACT_SWIGLU, false, false, BMODE_PLAIN, EPI_STORE_SPLIT, float>(
          g, stream);
    case GK_DX_DACT_GELU:
      return launch_dact<DACT_GELU, DACT_NONE, true, true, BMODE_PLAIN, EPI_STORE, bf16_t>(g, stream);
    case GK_DX_KSPLIT_DACT_SWIGLU:
      return launch_dact<DACT_SWIGLU, DACT_NONE, true, true, BMODE_KSPLIT, EPI_STORE, bf16_t>(g,
                                                                                            stream);
    default:
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
