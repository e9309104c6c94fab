// extern "C" entry points of libtpmlp.so: argument checks (host only, no
// GPU call until every check has passed), then kernel launches on the
// caller's stream.  Declarations and the contract live in include/tpmlp.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "launch.h"

using namespace tpmlp;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return TP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Buf {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Buf& a, const Buf& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// every output against every input and every other output
int check_alias(const Buf* ins, int nin, const Buf* outs, int nout) {
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlap(outs[o], ins[i]))
        return fail(TP_ERR_ALIAS, "output %s overlaps input %s", outs[o].name, ins[i].name);
    for (int p = o + 1; p < nout; ++p)
      if (overlap(outs[o], outs[p]))
        return fail(TP_ERR_ALIAS, "outputs %s and %s overlap", outs[o].name, outs[p].name);
  }
  return TP_OK;
}

int check_ptrs(const Buf* bufs, int n, bool required) {
  for (int i = 0; i < n; ++i) {
    if (!bufs[i].p) {
      if (required) return fail(TP_ERR_NULL, "%s is NULL", bufs[i].name);
      continue;
    }
    if (!aligned16(bufs[i].p))
      return fail(TP_ERR_ALIGN, "%s is not 16-byte aligned", bufs[i].name);
  }
  return TP_OK;
}

// per-device gfx950 check, cached: 0 unknown, 1 yes, 2 no
std::atomic<int> g_arch[64];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(TP_ERR_DEVICE, "no current HIP device");
  if (dev < 64) {
    int s = g_arch[dev].load(std::memory_order_relaxed);
    if (s == 1) return TP_OK;
    if (s == 2) return fail(TP_ERR_DEVICE, "device %d is not a gfx950", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(TP_ERR_DEVICE, "hipGetDeviceProperties failed on device %d", dev);
  bool yes = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_arch[dev].store(yes ? 1 : 2, std::memory_order_relaxed);
  if (!yes) return fail(TP_ERR_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return TP_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;
// tokens of the FP8 backward: its weight-gradient GEMMs contract over the
// tokens of K-contiguous code rows, 256 rows x N bytes per 32-bit tile offset
constexpr int64_t kMaxFp8Tokens = (int64_t)1 << 22;
// Largest leading dimension (H, and the Z_save width 2 F_shard): the bf16
// kernels address one 256-row tile through 32-bit buffer offsets, so
// 256 rows x ld x 2 bytes must stay below 2^31.
constexpr int64_t kMaxLd = (int64_t)1 << 21;

struct Shard {
  int64_t N, H, Ft;
  int act, dtype;
  size_t elt;
};

int check_desc(const tp_mlp_desc* d, Shard& s) {
  if (!d) return fail(TP_ERR_NULL, "desc is NULL");
  if (d->dtype != TP_F32 && d->dtype != TP_BF16)
    return fail(TP_ERR_DTYPE, "unknown dtype %d", d->dtype);
  if (d->act != TP_ACT_GELU_TANH && d->act != TP_ACT_SWIGLU)
    return fail(TP_ERR_DTYPE, "unknown activation %d", d->act);
  if (d->S < 0 || d->B < 0) return fail(TP_ERR_SHAPE, "S and B must be >= 0");
  if (d->H <= 0 || d->F_shard <= 0) return fail(TP_ERR_SHAPE, "H and F_shard must be > 0");
  if (d->T < 1 || d->T > TP_MAX_SHARDS)
    return fail(TP_ERR_SHAPE, "T must be in 1..%d", TP_MAX_SHARDS);
  if (d->S > kMaxDim || d->B > kMaxDim || d->S * d->B > kMaxDim || d->H > kMaxLd ||
      d->F_shard > kMaxLd / 2)
    return fail(TP_ERR_SHAPE, "dimension too large");
  const int vec = d->dtype == TP_BF16 ? 8 : 4;
  if (d->H % vec || d->F_shard % vec)
    return fail(TP_ERR_SHAPE, "H and F_shard must be multiples of %d for this dtype", vec);
  s.N = d->S * d->B;
  s.H = d->H;
  s.Ft = d->F_shard;
  s.act = d->act;
  s.dtype = d->dtype;
  s.elt = d->dtype == TP_BF16 ? 2 : 4;
  return TP_OK;
}

GemmArgs dense_args(int M, int N, int K) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.M = M; g.N = N; g.K = K;
  g.ragged = RAGGED_NONE;
  g.E = 1;
  return g;
}

// Launch timing (tp_launch_events): this thread's caller-owned events and
// how many of them have been recorded.  One timed unit is one product of
// the path (a GEMM with its fused epilogue, a partial sum, a quantization,
// ...), which may be more than one kernel.
thread_local std::vector<hipEvent_t> g_events;
thread_local size_t g_events_used = 0;

template <typename F>
hipError_t timed(hipStream_t st, F&& launch) {
  if (g_events_used + 2 > g_events.size()) return launch();
  hipError_t he = hipEventRecord(g_events[g_events_used], st);
  if (he != hipSuccess) return he;
  he = launch();
  if (he != hipSuccess) return he;
  he = hipEventRecord(g_events[g_events_used + 1], st);
  if (he == hipSuccess) g_events_used += 2;
  return he;
}

hipError_t run_gemm(int dtype, GemmKind kind, GemmArgs& g, hipStream_t st) {
  return timed(st, [&] { return dtype == TP_BF16 ? gemm_bf16(kind, g, st) : gemm_f32(kind, g, st); });
}
hipError_t tgemm_bf16(GemmKind kind, GemmArgs& g, hipStream_t st) {
  return timed(st, [&] { return gemm_bf16(kind, g, st); });
}
hipError_t tgemm_fp8(GemmKind kind, GemmArgs& g, hipStream_t st) {
  return timed(st, [&] { return gemm_fp8(kind, g, st); });
}
hipError_t t_partial_sum_launch(int dtype, int T, const void* const* parts, int64_t count,
                                void* out, int max_blocks, hipStream_t st) {
  return timed(st, [&] { return partial_sum_launch(dtype, T, parts, count, out, max_blocks, st); });
}
hipError_t t_fp8_quantize_launch(int fmt, bool tr, int64_t rows, int64_t cols, const void* x,
                                 const float* scale, void* q, float* amax, hipStream_t st) {
  return timed(st, [&] { return fp8_quantize_launch(fmt, tr, rows, cols, x, scale, q, amax, st); });
}
hipError_t t_zero_float_launch(float* p, hipStream_t st) {
  return timed(st, [&] { return zero_float_launch(p, st); });
}
hipError_t t_fp8_scale_update_launch(int fmt, int n, int len, int margin, float* history,
                                     float* amax, float* scale, float* scale_inv,
                                     hipStream_t st) {
  return timed(st, [&] {
    return fp8_scale_update_launch(fmt, n, len, margin, history, amax, scale, scale_inv, st);
  });
}
hipError_t t_byte_transpose_launch(int64_t rows, int64_t cols, const void* in, void* out,
                                   hipStream_t st) {
  return timed(st, [&] { return byte_transpose_launch(rows, cols, in, out, st); });
}
hipError_t t_moe_permute_launch(int dtype, const int32_t* row_token, int64_t N, int64_t H,
                                int64_t R, const void* X, void* Xp, hipStream_t st) {
  return timed(st, [&] { return moe_permute_launch(dtype, row_token, N, H, R, X, Xp, st); });
}
hipError_t t_moe_combine_launch(int dtype, const int32_t* tok_ptr, const int32_t* tok_rows,
                                const float* w, int64_t N, int64_t H, int64_t R, const void* Yp,
                                void* Y, hipStream_t st) {
  return timed(st, [&] {
    return moe_combine_launch(dtype, tok_ptr, tok_rows, w, N, H, R, Yp, Y, st);
  });
}
hipError_t t_moe_combine_bwd_launch(int dtype, const int32_t* row_token, const float* w,
                                    int64_t N, int64_t H, int64_t R, const void* dY,
                                    const void* Yp, void* dYp, float* dw, hipStream_t st) {
  return timed(st, [&] {
    return moe_combine_bwd_launch(dtype, row_token, w, N, H, R, dY, Yp, dYp, dw, st);
  });
}

size_t dz_bytes(const Shard& s) {
  return (size_t)s.N * (size_t)s.Ft * (s.act == TP_ACT_SWIGLU ? 2 : 1) * s.elt;
}

}  // namespace

// buffers that are required only when they hold something
int check_sized(const Buf* bufs, int n) {
  for (int i = 0; i < n; ++i) {
    if (bufs[i].bytes == 0) continue;
    if (!bufs[i].p) return fail(TP_ERR_NULL, "%s is NULL", bufs[i].name);
    if (!aligned16(bufs[i].p)) return fail(TP_ERR_ALIGN, "%s is not 16-byte aligned", bufs[i].name);
  }
  return TP_OK;
}
// index / weight tables (int32 or fp32 elements): 4-byte alignment
int check_tables(const Buf* bufs, int n) {
  for (int i = 0; i < n; ++i) {
    if (bufs[i].bytes == 0) continue;
    if (!bufs[i].p) return fail(TP_ERR_NULL, "%s is NULL", bufs[i].name);
    if (reinterpret_cast<uintptr_t>(bufs[i].p) & 3u)
      return fail(TP_ERR_ALIGN, "%s is not 4-byte aligned", bufs[i].name);
  }
  return TP_OK;
}
int check_rows(int32_t dtype, int64_t N, int64_t H, int64_t R) {
  if (dtype != TP_F32 && dtype != TP_BF16) return fail(TP_ERR_DTYPE, "unknown dtype %d", dtype);
  if (N < 0 || R < 0 || H <= 0) return fail(TP_ERR_SHAPE, "N, R must be >= 0 and H > 0");
  if (N > kMaxDim || R > kMaxDim || H > kMaxLd) return fail(TP_ERR_SHAPE, "dimension too large");
  const int vec = dtype == TP_BF16 ? 8 : 4;
  if (H % vec) return fail(TP_ERR_SHAPE, "H must be a multiple of %d for this dtype", vec);
  return TP_OK;
}

extern "C" {

const char* tp_last_error(void) { return g_last_error.c_str(); }

int tp_launch_events(void* const* events, int32_t count) {
  if (count < 0 || count > TP_MAX_LAUNCH_EVENTS || (count & 1))
    return fail(TP_ERR_SHAPE, "count must be even and in 0..%d", TP_MAX_LAUNCH_EVENTS);
  if (count > 0 && !events) return fail(TP_ERR_NULL, "events is NULL");
  for (int32_t i = 0; i < count; ++i)
    if (!events[i]) return fail(TP_ERR_NULL, "events[%d] is NULL", i);
  g_events.assign(reinterpret_cast<const hipEvent_t*>(events),
                  reinterpret_cast<const hipEvent_t*>(events) + count);
  g_events_used = 0;
  return ok();
}

int32_t tp_launch_events_used(void) { return (int32_t)g_events_used; }

const char* tp_status_string(int status) {
  switch (status) {
    case TP_OK: return "TP_OK";
    case TP_ERR_NULL: return "TP_ERR_NULL";
    case TP_ERR_SHAPE: return "TP_ERR_SHAPE";
    case TP_ERR_DTYPE: return "TP_ERR_DTYPE";
    case TP_ERR_ALIGN: return "TP_ERR_ALIGN";
    case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE";
    case TP_ERR_DEVICE: return "TP_ERR_DEVICE";
    case TP_ERR_HIP: return "TP_ERR_HIP";
    case TP_ERR_ALIAS: return "TP_ERR_ALIAS";
  }
  return "TP_ERR_UNKNOWN";
}

int tp_mlp_shard_fwd(const tp_mlp_desc* desc, const void* X, const void* A, const void* A_up,
                     const void* B, void* Z_save, void* H_act, void* Y_partial, void* stream) {
  Shard s;
  int rc = check_desc(desc, s);
  if (rc) return rc;
  const bool sw = s.act == TP_ACT_SWIGLU;
  const size_t e = s.elt;
  Buf req[] = {{X, (size_t)(s.N * s.H) * e, "X"},
               {A, (size_t)(s.H * s.Ft) * e, "A"},
               {B, (size_t)(s.Ft * s.H) * e, "B"},
               {H_act, (size_t)(s.N * s.Ft) * e, "H_act"},
               {Y_partial, (size_t)(s.N * s.H) * e, "Y_partial"}};
  if ((rc = check_ptrs(req, 5, true))) return rc;
  if (sw && !A_up) return fail(TP_ERR_NULL, "A_up is required for SwiGLU");
  if (!sw && A_up) return fail(TP_ERR_SHAPE, "A_up must be NULL for GeLU");
  Buf opt[] = {{A_up, (size_t)(s.H * s.Ft) * e, "A_up"},
               {Z_save, (size_t)(s.N * s.Ft) * (sw ? 2 : 1) * e, "Z_save"}};
  if ((rc = check_ptrs(opt, 2, false))) return rc;
  Buf ins[] = {req[0], req[1], req[2], opt[0]};
  Buf outs[] = {req[3], req[4], opt[1]};
  if ((rc = check_alias(ins, 4, outs, 3))) return rc;
  if ((rc = check_device())) return rc;
  if (s.N == 0) return ok();

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int N = (int)s.N, H = (int)s.H, Ft = (int)s.Ft;

  GemmArgs g1 = dense_args(N, Ft, H);
  g1.a = {X, nullptr, H, 0, 0};
  g1.b = {A, A_up, Ft, 0, sw ? Ft : 0};
  g1.epi.out0 = Z_save;
  g1.epi.out1 = H_act;
  g1.epi.ld0 = sw ? 2 * (int64_t)Ft : Ft;
  g1.epi.ld1 = Ft;
  g1.epi.split = Ft;
  hipError_t he = run_gemm(s.dtype, sw ? GK_FC1_SWIGLU : GK_FC1_GELU, g1, st);
  if (he != hipSuccess) return hip_fail(he, "FC1 launch");

  GemmArgs g2 = dense_args(N, H, Ft);
  g2.a = {H_act, nullptr, Ft, 0, 0};
  g2.b = {B, nullptr, H, 0, 0};
  g2.epi.out0 = Y_partial;
  g2.epi.ld0 = H;
  he = run_gemm(s.dtype, GK_FC2, g2, st);
  if (he != hipSuccess) return hip_fail(he, "FC2 launch");
  return ok();
}

size_t tp_mlp_shard_bwd_workspace(const tp_mlp_desc* desc) {
  Shard s;
  if (check_desc(desc, s)) return 0;
  return dz_bytes(s);
}

namespace {
// Device-resident scratch for tp_mlp_shard_bwd_noalloc: the activation-side
// gradient dZ of one call.  Each GPU the library runs on holds its own copy
// until the process ends.  Host code never uses this name as an address:
// the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[TP_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};

// this device's address of `scratch` (looked up once per device, with that
// device current); NULL and the error message on failure
void* scratch_address(int* err) {
  int dev = -1;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess || dev < 0 || dev >= 64) {
    *err = fail(TP_ERR_DEVICE, "no current HIP device for the scratch buffer");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    he = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (he != hipSuccess || !p) {
      *err = hip_fail(he != hipSuccess ? he : hipErrorInvalidSymbol,
                      "hipGetSymbolAddress of the scratch buffer");
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// use_scratch: the workspace is the device's scratch array (resolved after
// the device check; its size is checked against the array's)
// dact_in_loads: dH is written plainly and the dA / dX GEMMs form dZ from
// it and Z_save as they load it (the workspace then holds dH)
int shard_bwd(const tp_mlp_desc* desc, const void* X, const void* A, const void* A_up,
              const void* B, const void* Z_save, const void* H_act, const void* dY,
              void* dX_partial, float* dA, float* dA_up, float* dB, void* workspace,
              size_t ws_bytes, void* stream, bool accumulate, bool use_scratch = false,
              bool dact_in_loads = false) {
  Shard s;
  int rc = check_desc(desc, s);
  if (rc) return rc;
  const bool sw = s.act == TP_ACT_SWIGLU;
  const size_t e = s.elt;
  Buf in_req[] = {{X, (size_t)(s.N * s.H) * e, "X"},
                  {A, (size_t)(s.H * s.Ft) * e, "A"},
                  {B, (size_t)(s.Ft * s.H) * e, "B"},
                  {Z_save, (size_t)(s.N * s.Ft) * (sw ? 2 : 1) * e, "Z_save"},
                  {H_act, (size_t)(s.N * s.Ft) * e, "H_act"},
                  {dY, (size_t)(s.N * s.H) * e, "dY"}};
  Buf out_req[] = {{dX_partial, (size_t)(s.N * s.H) * e, "dX_partial"},
                   {dA, (size_t)(s.H * s.Ft) * 4, "dA"},
                   {dB, (size_t)(s.Ft * s.H) * 4, "dB"}};
  if ((rc = check_ptrs(in_req, 6, true))) return rc;
  if ((rc = check_ptrs(out_req, 3, true))) return rc;
  if (sw && (!A_up || !dA_up)) return fail(TP_ERR_NULL, "A_up and dA_up are required for SwiGLU");
  if (!sw && (A_up || dA_up)) return fail(TP_ERR_SHAPE, "A_up and dA_up must be NULL for GeLU");
  Buf in_opt[] = {{A_up, (size_t)(s.H * s.Ft) * e, "A_up"}};
  Buf out_opt[] = {{dA_up, (size_t)(s.H * s.Ft) * 4, "dA_up"}};
  if ((rc = check_ptrs(in_opt, 1, false))) return rc;
  if ((rc = check_ptrs(out_opt, 1, false))) return rc;
  const size_t need = dact_in_loads ? (size_t)(s.N * s.Ft) * e : dz_bytes(s);
  if (use_scratch) {
    if (need > (size_t)TP_NOALLOC_SCRATCH_BYTES)
      return fail(TP_ERR_WORKSPACE,
                  "dZ needs %zu bytes, more than the %zu-byte scratch buffer of the "
                  "allocation-free call (N * F_shard%s * element size)",
                  need, (size_t)TP_NOALLOC_SCRATCH_BYTES, sw ? " * 2" : "");
  } else if (need > 0) {
    if (!workspace) return fail(TP_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned16(workspace)) return fail(TP_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (ws_bytes < need)
      return fail(TP_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  }
  Buf ws = {use_scratch ? nullptr : workspace, need, "workspace"};
  Buf ins[] = {in_req[0], in_req[1], in_req[2], in_req[3], in_req[4], in_req[5], in_opt[0]};
  Buf outs[] = {out_req[0], out_req[1], out_req[2], out_opt[0], ws};
  if ((rc = check_alias(ins, 7, outs, 5))) return rc;
  if ((rc = check_device())) return rc;
  if (use_scratch) {
    int err = TP_OK;
    workspace = scratch_address(&err);
    if (!workspace) return err;
    ws_bytes = TP_NOALLOC_SCRATCH_BYTES;
  }

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int N = (int)s.N, H = (int)s.H, Ft = (int)s.Ft;
  const int64_t zld = sw ? 2 * (int64_t)Ft : Ft;
  hipError_t he;

  // 1. dZ = (dY B^T) * act'(Z): the activation derivative in the epilogue
  //    (or dH = dY B^T alone, when the consumers form dZ)
  if (N > 0 && dact_in_loads) {
    GemmArgs g = dense_args(N, Ft, H);
    g.a = {dY, nullptr, H, 0, 0};
    g.b = {B, nullptr, H, 0, 0};
    g.epi.out0 = workspace;
    g.epi.ld0 = Ft;
    // (the plain both-K-contiguous product kind)
    he = run_gemm(s.dtype, GK_DX, g, st);
    if (he != hipSuccess) return hip_fail(he, "dH launch");
  } else if (N > 0) {
    GemmArgs g = dense_args(N, Ft, H);
    g.a = {dY, nullptr, H, 0, 0};
    g.b = {B, nullptr, H, 0, 0};
    g.epi.aux = Z_save;
    g.epi.ldaux = zld;
    g.epi.out0 = workspace;
    g.epi.ld0 = zld;
    g.epi.split = Ft;
    he = run_gemm(s.dtype, sw ? GK_DH_SWIGLU : GK_DH_GELU, g, st);
    if (he != hipSuccess) return hip_fail(he, "dH launch");
  }
  // 2. dB = H^T dY   (K = N; N = 0 writes zeros)
  {
    GemmArgs g = dense_args(Ft, H, N);
    g.a = {H_act, nullptr, Ft, 0, 0};
    g.b = {dY, nullptr, H, 0, 0};
    g.epi.out0 = dB;
    g.epi.ld0 = H;
    he = run_gemm(s.dtype, accumulate ? GK_WGRAD_ACC : GK_WGRAD, g, st);
    if (he != hipSuccess) return hip_fail(he, "dB launch");
  }
  // 3. dA (| dA_up) = X^T dZ
  {
    GemmArgs g = dense_args(H, sw ? 2 * Ft : Ft, N);
    g.a = {X, nullptr, H, 0, 0};
    g.b = {workspace, nullptr, zld, 0, 0};
    g.epi.out0 = dA;
    g.epi.out1 = dA_up;
    g.epi.ld0 = Ft;
    g.epi.ld1 = Ft;
    g.epi.split = Ft;
    GemmKind k = sw ? (accumulate ? GK_WGRAD_SPLIT_ACC : GK_WGRAD_SPLIT)
                    : (accumulate ? GK_WGRAD_ACC : GK_WGRAD);
    if (dact_in_loads) {
      g.b = {workspace, Z_save, Ft, 0, Ft};
      k = sw ? GK_WGRAD_SPLIT_DACT_SWIGLU : GK_WGRAD_DACT_GELU;
    }
    he = run_gemm(s.dtype, k, g, st);
    if (he != hipSuccess) return hip_fail(he, "dA launch");
  }
  // 4. dX_partial = dZ A^T  (SwiGLU: [dG|dU] [Ag|Au]^T)
  if (N > 0) {
    GemmArgs g = dense_args(N, H, sw ? 2 * Ft : Ft);
    g.a = {workspace, nullptr, zld, 0, 0};
    g.b = {A, A_up, Ft, 0, Ft};
    g.epi.out0 = dX_partial;
    g.epi.ld0 = H;
    GemmKind k = sw ? GK_DX_KSPLIT : GK_DX;
    if (dact_in_loads) {
      g.a = {workspace, Z_save, Ft, 0, Ft};
      k = sw ? GK_DX_KSPLIT_DACT_SWIGLU : GK_DX_DACT_GELU;
    }
    he = run_gemm(s.dtype, k, g, st);
    if (he != hipSuccess) return hip_fail(he, "dX launch");
  }
  return ok();
}
}  // namespace

int tp_mlp_shard_bwd(const tp_mlp_desc* desc, const void* X, const void* A, const void* A_up,
                     const void* B, const void* Z_save, const void* H_act, const void* dY,
                     void* dX_partial, float* dA, float* dA_up, float* dB, void* workspace,
                     size_t ws_bytes, void* stream) {
  return shard_bwd(desc, X, A, A_up, B, Z_save, H_act, dY, dX_partial, dA, dA_up, dB, workspace,
                   ws_bytes, stream, false);
}

int tp_mlp_shard_bwd_noalloc(const tp_mlp_desc* desc, const void* X, const void* A,
                             const void* A_up, const void* B, const void* Z_save,
                             const void* H_act, const void* dY, void* dX_partial, float* dA,
                             float* dA_up, float* dB, void* stream) {
  return shard_bwd(desc, X, A, A_up, B, Z_save, H_act, dY, dX_partial, dA, dA_up, dB, nullptr, 0,
                   stream, false, true);
}

int tp_mlp_shard_bwd_dact_prologue(const tp_mlp_desc* desc, const void* X, const void* A,
                                   const void* A_up, const void* B, const void* Z_save,
                                   const void* H_act, const void* dY, void* dX_partial,
                                   float* dA, float* dA_up, float* dB, void* workspace,
                                   size_t ws_bytes, void* stream) {
  return shard_bwd(desc, X, A, A_up, B, Z_save, H_act, dY, dX_partial, dA, dA_up, dB, workspace,
                   ws_bytes, stream, false, false, true);
}

int tp_mlp_shard_bwd_accum(const tp_mlp_desc* desc, const void* X, const void* A,
                           const void* A_up, const void* B, const void* Z_save,
                           const void* H_act, const void* dY, void* dX_partial, float* dA,
                           float* dA_up, float* dB, void* workspace, size_t ws_bytes,
                           void* stream) {
  return shard_bwd(desc, X, A, A_up, B, Z_save, H_act, dY, dX_partial, dA, dA_up, dB, workspace,
                   ws_bytes, stream, true);
}

namespace {
int partial_sum_common(int32_t dtype, int32_t T, const void* const* partials, int64_t count,
                       void* out, int32_t max_blocks, void* stream) {
  if (dtype != TP_F32 && dtype != TP_BF16) return fail(TP_ERR_DTYPE, "unknown dtype %d", dtype);
  if (T < 1 || T > TP_MAX_SHARDS) return fail(TP_ERR_SHAPE, "T must be in 1..%d", TP_MAX_SHARDS);
  if (count < 0) return fail(TP_ERR_SHAPE, "count must be >= 0");
  if (!partials) return fail(TP_ERR_NULL, "partials is NULL");
  const size_t bytes = (size_t)count * (dtype == TP_BF16 ? 2 : 4);
  Buf ob = {out, bytes, "out"};
  if (int rc = check_ptrs(&ob, 1, true)) return rc;
  for (int i = 0; i < T; ++i) {
    if (!partials[i]) return fail(TP_ERR_NULL, "partials[%d] is NULL", i);
    if (!aligned16(partials[i])) return fail(TP_ERR_ALIGN, "partials[%d] is not 16-byte aligned", i);
    Buf pb = {partials[i], bytes, "partial"};
    if (partials[i] != out && overlap(ob, pb))
      return fail(TP_ERR_ALIAS, "out overlaps partials[%d] without being equal to it", i);
  }
  if (int rc = check_device()) return rc;
  if (count == 0) return ok();
  hipError_t he = t_partial_sum_launch(dtype, T, partials, count, out, max_blocks,
                                     reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "partial-sum launch");
  return ok();
}
}  // namespace

int tp_partial_sum(int32_t dtype, int32_t T, const void* const* partials, int64_t count,
                   void* out, void* stream) {
  return partial_sum_common(dtype, T, partials, count, out, 0, stream);
}

int tp_partial_sum_scatter(int32_t dtype, int32_t T, const void* const* partials, int64_t S,
                           int64_t B, int64_t H, int32_t rank, void* out, void* stream) {
  if (dtype != TP_F32 && dtype != TP_BF16) return fail(TP_ERR_DTYPE, "unknown dtype %d", dtype);
  if (T < 1 || T > TP_MAX_SHARDS) return fail(TP_ERR_SHAPE, "T must be in 1..%d", TP_MAX_SHARDS);
  if (S < 0 || B < 0 || H <= 0 || S > kMaxDim || B > kMaxDim || H > kMaxLd || S * B > kMaxDim)
    return fail(TP_ERR_SHAPE, "S, B must be >= 0 and H > 0 within range");
  if (S % T) return fail(TP_ERR_SHAPE, "S must be a multiple of T");
  const int vec = dtype == TP_BF16 ? 8 : 4;
  if (H % vec) return fail(TP_ERR_SHAPE, "H must be a multiple of %d for this dtype", vec);
  if (rank < 0 || rank >= T) return fail(TP_ERR_SHAPE, "rank must be in 0..T-1");
  if (!partials) return fail(TP_ERR_NULL, "partials is NULL");
  const size_t elt = dtype == TP_BF16 ? 2 : 4;
  const int64_t slice = (S / T) * B * H;
  const size_t full_bytes = (size_t)(S * B * H) * elt;
  Buf ob = {out, (size_t)slice * elt, "out"};
  if (int rc = check_ptrs(&ob, 1, true)) return rc;
  const void* sl[TP_MAX_SHARDS];
  for (int i = 0; i < T; ++i) {
    if (!partials[i]) return fail(TP_ERR_NULL, "partials[%d] is NULL", i);
    if (!aligned16(partials[i])) return fail(TP_ERR_ALIGN, "partials[%d] is not 16-byte aligned", i);
    Buf pb = {partials[i], full_bytes, "partial"};
    if (overlap(ob, pb)) return fail(TP_ERR_ALIAS, "out overlaps partials[%d]", i);
    sl[i] = static_cast<const char*>(partials[i]) + (size_t)rank * (size_t)slice * elt;
  }
  if (int rc = check_device()) return rc;
  if (slice == 0) return ok();
  hipError_t he = t_partial_sum_launch(dtype, T, sl, slice, out, 0,
                                     reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "partial-sum launch");
  return ok();
}

int tp_partial_sum_capped(int32_t dtype, int32_t T, const void* const* partials,
                          int64_t count, void* out, int32_t max_workgroups, void* stream) {
  if (max_workgroups < 1) return fail(TP_ERR_SHAPE, "max_workgroups must be >= 1");
  return partial_sum_common(dtype, T, partials, count, out, max_workgroups, stream);
}

// ---------------------------------------------------------------------------
// grouped local experts
// ---------------------------------------------------------------------------
namespace {

struct Experts {
  int64_t H, F, R;
  int E;
};

int check_expert_desc(const tp_expert_desc* d, Experts& x) {
  if (!d) return fail(TP_ERR_NULL, "desc is NULL");
  if (d->dtype != TP_BF16) return fail(TP_ERR_DTYPE, "grouped experts support bf16 only");
  if (d->E < 1 || d->E > TP_MAX_EXPERTS)
    return fail(TP_ERR_SHAPE, "E must be in 1..%d", TP_MAX_EXPERTS);
  if (d->H <= 0 || d->F <= 0 || d->H % 8 || d->F % 8)
    return fail(TP_ERR_SHAPE, "H and F must be positive multiples of 8");
  if (d->H > kMaxLd || d->F > kMaxLd / 2) return fail(TP_ERR_SHAPE, "dimension too large");
  x.H = d->H;
  x.F = d->F;
  x.E = d->E;
  return TP_OK;
}

int check_experts(const tp_expert_desc* d, const int64_t* offsets, Experts& x) {
  int rc = check_expert_desc(d, x);
  if (rc) return rc;
  if (!offsets) return fail(TP_ERR_NULL, "offsets is NULL");
  if (offsets[0] != 0) return fail(TP_ERR_SHAPE, "offsets[0] must be 0");
  for (int e = 0; e < d->E; ++e)
    if (offsets[e + 1] < offsets[e]) return fail(TP_ERR_SHAPE, "offsets must be non-decreasing");
  if (offsets[d->E] > kMaxDim) return fail(TP_ERR_SHAPE, "too many rows");
  x.R = offsets[d->E];
  return TP_OK;
}

// device-resident offsets: the host checks only the capacity R and the table
int check_experts_dev(const tp_expert_desc* d, int64_t R, const int32_t* offsets, Experts& x) {
  int rc = check_expert_desc(d, x);
  if (rc) return rc;
  if (R < 0 || R > kMaxDim) return fail(TP_ERR_SHAPE, "R must be in 0..%lld", (long long)kMaxDim);
  if (!offsets) return fail(TP_ERR_NULL, "offsets is NULL");
  if (reinterpret_cast<uintptr_t>(offsets) & 3u)
    return fail(TP_ERR_ALIGN, "offsets is not 4-byte aligned");
  x.R = R;
  return TP_OK;
}

// where a grouped call's row offsets are: E+1 host values, or E+1 int32 in
// device memory that the kernels read (clamped into [0, R]) when they run
struct Rows {
  const int64_t* host;
  const int32_t* dev;
};

void set_rows(GemmArgs& g, const Experts& x, const Rows& rows, int ragged) {
  g.E = x.E;
  g.ragged = ragged;
  if (rows.dev) {
    g.dev_off = rows.dev;
    g.dev_rows = (int)x.R;
  } else {
    for (int e = 0; e <= x.E; ++e) g.row_off[e] = (int)rows.host[e];
  }
}

int grouped_fwd(const Experts& x, const Rows& rows, const void* X_perm, const void* Wg,
                const void* Wu, const void* Wd, void* Z_save, void* H_act, void* Y_perm,
                void* stream) {
  int rc;
  const size_t wbytes = (size_t)(x.E * x.H * x.F) * 2;
  Buf req[] = {{X_perm, (size_t)(x.R * x.H) * 2, "X_perm"},
               {Wg, wbytes, "Wg"},
               {Wu, wbytes, "Wu"},
               {Wd, wbytes, "Wd"},
               {H_act, (size_t)(x.R * x.F) * 2, "H_act"},
               {Y_perm, (size_t)(x.R * x.H) * 2, "Y_perm"}};
  if ((rc = check_ptrs(req, 6, true))) return rc;
  Buf zs = {Z_save, (size_t)(x.R * x.F) * 4, "Z_save"};
  if ((rc = check_ptrs(&zs, 1, false))) return rc;
  Buf ins[] = {req[0], req[1], req[2], req[3],
               {rows.dev, rows.dev ? (size_t)(x.E + 1) * 4 : 0, "offsets"}};
  Buf outs[] = {req[4], req[5], zs};
  if ((rc = check_alias(ins, 5, outs, 3))) return rc;
  if ((rc = check_device())) return rc;
  if (x.R == 0) return ok();

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int H = (int)x.H, F = (int)x.F;
  GemmArgs g1 = dense_args(0, 2 * F, H);
  set_rows(g1, x, rows, RAGGED_M);
  g1.a = {X_perm, nullptr, H, 0, 0};
  g1.b = {Wg, Wu, F, (int64_t)H * F, F};
  g1.epi.out0 = Z_save;
  g1.epi.out1 = H_act;
  g1.epi.ld0 = 2 * (int64_t)F;
  g1.epi.ld1 = F;
  g1.epi.split = F;
  hipError_t he = tgemm_bf16(GK_FC1_SWIGLU, g1, st);
  if (he != hipSuccess) return hip_fail(he, "grouped FC1 launch");

  GemmArgs g2 = dense_args(0, H, F);
  set_rows(g2, x, rows, RAGGED_M);
  g2.a = {H_act, nullptr, F, 0, 0};
  g2.b = {Wd, nullptr, H, (int64_t)F * H, 0};
  g2.epi.out0 = Y_perm;
  g2.epi.ld0 = H;
  he = tgemm_bf16(GK_FC2, g2, st);
  if (he != hipSuccess) return hip_fail(he, "grouped FC2 launch");
  return ok();
}

}  // namespace

int tp_grouped_expert_fwd(const tp_expert_desc* desc, const int64_t* offsets, const void* X_perm,
                          const void* Wg, const void* Wu, const void* Wd, void* Z_save,
                          void* H_act, void* Y_perm, void* stream) {
  Experts x;
  int rc = check_experts(desc, offsets, x);
  if (rc) return rc;
  return grouped_fwd(x, Rows{offsets, nullptr}, X_perm, Wg, Wu, Wd, Z_save, H_act, Y_perm, stream);
}

int tp_grouped_expert_fwd_devoff(const tp_expert_desc* desc, int64_t R, const int32_t* offsets,
                                 const void* X_perm, const void* Wg, const void* Wu,
                                 const void* Wd, void* Z_save, void* H_act, void* Y_perm,
                                 void* stream) {
  Experts x;
  int rc = check_experts_dev(desc, R, offsets, x);
  if (rc) return rc;
  return grouped_fwd(x, Rows{nullptr, offsets}, X_perm, Wg, Wu, Wd, Z_save, H_act, Y_perm, stream);
}

size_t tp_grouped_expert_bwd_workspace(const tp_expert_desc* desc, const int64_t* offsets) {
  Experts x;
  if (check_experts(desc, offsets, x)) return 0;
  return (size_t)(x.R * x.F) * 2 * 2;
}

namespace {
int grouped_bwd(const Experts& x, const Rows& rows, const void* X_perm, const void* Wg,
                const void* Wu, const void* Wd, const void* Z_save, const void* H_act,
                const void* dY_perm, void* dX_perm, float* dWg, float* dWu, float* dWd,
                void* workspace, size_t ws_bytes, void* stream, bool accumulate) {
  int rc;
  const size_t wbytes = (size_t)(x.E * x.H * x.F) * 2;
  const size_t gbytes = (size_t)(x.E * x.H * x.F) * 4;
  Buf in_req[] = {{X_perm, (size_t)(x.R * x.H) * 2, "X_perm"},
                  {Wg, wbytes, "Wg"},
                  {Wu, wbytes, "Wu"},
                  {Wd, wbytes, "Wd"},
                  {Z_save, (size_t)(x.R * x.F) * 4, "Z_save"},
                  {H_act, (size_t)(x.R * x.F) * 2, "H_act"},
                  {dY_perm, (size_t)(x.R * x.H) * 2, "dY_perm"}};
  Buf out_req[] = {{dX_perm, (size_t)(x.R * x.H) * 2, "dX_perm"},
                   {dWg, gbytes, "dWg"},
                   {dWu, gbytes, "dWu"},
                   {dWd, gbytes, "dWd"}};
  if ((rc = check_ptrs(in_req, 7, true))) return rc;
  if ((rc = check_ptrs(out_req, 4, true))) return rc;
  const size_t need = (size_t)(x.R * x.F) * 4;
  if (need > 0) {
    if (!workspace) return fail(TP_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned16(workspace)) return fail(TP_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (ws_bytes < need)
      return fail(TP_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  }
  Buf ws = {workspace, need, "workspace"};
  Buf outs[] = {out_req[0], out_req[1], out_req[2], out_req[3], ws};
  Buf ins[] = {in_req[0], in_req[1], in_req[2], in_req[3], in_req[4], in_req[5], in_req[6],
               {rows.dev, rows.dev ? (size_t)(x.E + 1) * 4 : 0, "offsets"}};
  if ((rc = check_alias(ins, 8, outs, 5))) return rc;
  if ((rc = check_device())) return rc;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int H = (int)x.H, F = (int)x.F;
  const int64_t HF = (int64_t)H * F;
  hipError_t he;
  if (x.R > 0) {
    GemmArgs g = dense_args(0, F, H);
    set_rows(g, x, rows, RAGGED_M);
    g.a = {dY_perm, nullptr, H, 0, 0};
    g.b = {Wd, nullptr, H, HF, 0};
    g.epi.aux = Z_save;
    g.epi.ldaux = 2 * (int64_t)F;
    g.epi.out0 = workspace;
    g.epi.ld0 = 2 * (int64_t)F;
    g.epi.split = F;
    he = tgemm_bf16(GK_DH_SWIGLU, g, st);
    if (he != hipSuccess) return hip_fail(he, "grouped dH launch");
  }
  {
    GemmArgs g = dense_args(F, H, 0);
    set_rows(g, x, rows, RAGGED_K);
    g.a = {H_act, nullptr, F, 0, 0};
    g.b = {dY_perm, nullptr, H, 0, 0};
    g.epi.out0 = dWd;
    g.epi.ld0 = H;
    g.epi.bstride = HF;
    he = tgemm_bf16(accumulate ? GK_WGRAD_ACC : GK_WGRAD, g, st);
    if (he != hipSuccess) return hip_fail(he, "grouped dWd launch");
  }
  {
    GemmArgs g = dense_args(H, 2 * F, 0);
    set_rows(g, x, rows, RAGGED_K);
    g.a = {X_perm, nullptr, H, 0, 0};
    g.b = {workspace, nullptr, 2 * (int64_t)F, 0, 0};
    g.epi.out0 = dWg;
    g.epi.out1 = dWu;
    g.epi.ld0 = F;
    g.epi.ld1 = F;
    g.epi.split = F;
    g.epi.bstride = HF;
    he = tgemm_bf16(accumulate ? GK_WGRAD_SPLIT_ACC : GK_WGRAD_SPLIT, g, st);
    if (he != hipSuccess) return hip_fail(he, "grouped dWg/dWu launch");
  }
  if (x.R > 0) {
    GemmArgs g = dense_args(0, H, 2 * F);
    set_rows(g, x, rows, RAGGED_M);
    g.a = {workspace, nullptr, 2 * (int64_t)F, 0, 0};
    g.b = {Wg, Wu, F, HF, F};
    g.epi.out0 = dX_perm;
    g.epi.ld0 = H;
    he = tgemm_bf16(GK_DX_KSPLIT, g, st);
    if (he != hipSuccess) return hip_fail(he, "grouped dX launch");
  }
  return ok();
}
}  // namespace

int tp_grouped_expert_bwd(const tp_expert_desc* desc, const int64_t* offsets, const void* X_perm,
                          const void* Wg, const void* Wu, const void* Wd, const void* Z_save,
                          const void* H_act, const void* dY_perm, void* dX_perm, float* dWg,
                          float* dWu, float* dWd, void* workspace, size_t ws_bytes,
                          void* stream) {
  Experts x;
  int rc = check_experts(desc, offsets, x);
  if (rc) return rc;
  return grouped_bwd(x, Rows{offsets, nullptr}, X_perm, Wg, Wu, Wd, Z_save, H_act, dY_perm,
                     dX_perm, dWg, dWu, dWd, workspace, ws_bytes, stream, false);
}

int tp_grouped_expert_bwd_accum(const tp_expert_desc* desc, const int64_t* offsets,
                                const void* X_perm, const void* Wg, const void* Wu,
                                const void* Wd, const void* Z_save, const void* H_act,
                                const void* dY_perm, void* dX_perm, float* dWg, float* dWu,
                                float* dWd, void* workspace, size_t ws_bytes, void* stream) {
  Experts x;
  int rc = check_experts(desc, offsets, x);
  if (rc) return rc;
  return grouped_bwd(x, Rows{offsets, nullptr}, X_perm, Wg, Wu, Wd, Z_save, H_act, dY_perm,
                     dX_perm, dWg, dWu, dWd, workspace, ws_bytes, stream, true);
}

size_t tp_grouped_expert_devoff_workspace(const tp_expert_desc* desc, int64_t R) {
  Experts x;
  if (check_expert_desc(desc, x) || R < 0 || R > kMaxDim) return 0;
  return (size_t)(R * x.F) * 2 * 2;
}

int tp_grouped_expert_bwd_devoff(const tp_expert_desc* desc, int64_t R, const int32_t* offsets,
                                 const void* X_perm, const void* Wg, const void* Wu,
                                 const void* Wd, const void* Z_save, const void* H_act,
                                 const void* dY_perm, void* dX_perm, float* dWg, float* dWu,
                                 float* dWd, void* workspace, size_t ws_bytes,
                                 int32_t accumulate, void* stream) {
  Experts x;
  int rc = check_experts_dev(desc, R, offsets, x);
  if (rc) return rc;
  if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_SHAPE, "accumulate must be 0 or 1");
  return grouped_bwd(x, Rows{nullptr, offsets}, X_perm, Wg, Wu, Wd, Z_save, H_act, dY_perm,
                     dX_perm, dWg, dWu, dWd, workspace, ws_bytes, stream, accumulate == 1);
}

// ---------------------------------------------------------------------------
// FP8
// ---------------------------------------------------------------------------
int tp_fp8_quantize(int32_t fmt, int32_t transpose, int64_t rows, int64_t cols, const void* x,
                    const float* scale, void* q, float* amax, void* stream) {
  if (fmt != TP_FP8_E4M3 && fmt != TP_FP8_E5M2) return fail(TP_ERR_DTYPE, "unknown fp8 format %d", fmt);
  if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim || rows * cols > ((int64_t)1 << 40))
    return fail(TP_ERR_SHAPE, "rows and cols must be >= 0 and within range");
  if (cols % 8) return fail(TP_ERR_SHAPE, "cols must be a multiple of 8");
  if (transpose && rows % 16) return fail(TP_ERR_SHAPE, "rows must be a multiple of 16 to transpose");
  const size_t n = (size_t)(rows * cols);
  Buf in[] = {{x, n * 2, "x"}};
  Buf out[] = {{q, n, "q"}};
  Buf tab[] = {{scale, 4, "scale"}};
  Buf am = {amax, amax ? (size_t)4 : 0, "amax"};
  if (int rc = check_sized(in, 1)) return rc;
  if (int rc = check_sized(out, 1)) return rc;
  if (int rc = check_tables(tab, 1)) return rc;
  if (int rc = check_tables(&am, 1)) return rc;
  Buf ins[] = {in[0], tab[0]};
  Buf outs[] = {out[0], am};
  if (int rc = check_alias(ins, 2, outs, 2)) return rc;
  if (int rc = check_device()) return rc;
  hipError_t he = t_fp8_quantize_launch(fmt, transpose != 0, rows, cols, x, scale, q, amax,
                                      reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "quantize launch");
  return ok();
}

int tp_mlp_shard_fwd_fp8(const tp_mlp_desc* desc, const void* Xq, const void* Aq_t,
                         const void* Auq_t, const void* Bq_t, const float* scales, void* Z_save,
                         void* H_act, void* H_q, float* h_amax, void* Y_partial, void* stream) {
  Shard s;
  int rc = check_desc(desc, s);
  if (rc) return rc;
  if (s.dtype != TP_BF16) return fail(TP_ERR_DTYPE, "the FP8 forward stores bf16 activations");
  if (s.H % 128 || s.Ft % 128)
    return fail(TP_ERR_SHAPE, "H and F_shard must be multiples of 128 for the FP8 path");
  const bool sw = s.act == TP_ACT_SWIGLU;
  Buf req[] = {{Xq, (size_t)(s.N * s.H), "Xq"},
               {Aq_t, (size_t)(s.H * s.Ft), "Aq_t"},
               {Bq_t, (size_t)(s.Ft * s.H), "Bq_t"},
               {H_act, (size_t)(s.N * s.Ft) * 2, "H_act"},
               {H_q, (size_t)(s.N * s.Ft), "H_q"},
               {Y_partial, (size_t)(s.N * s.H) * 2, "Y_partial"}};
  if ((rc = check_ptrs(req, 6, true))) return rc;
  if (sw && !Auq_t) return fail(TP_ERR_NULL, "Auq_t is required for SwiGLU");
  if (!sw && Auq_t) return fail(TP_ERR_SHAPE, "Auq_t must be NULL for GeLU");
  Buf opt[] = {{Auq_t, (size_t)(s.H * s.Ft), "Auq_t"},
               {Z_save, (size_t)(s.N * s.Ft) * (sw ? 2 : 1) * 2, "Z_save"}};
  if ((rc = check_ptrs(opt, 2, false))) return rc;
  Buf tab[] = {{scales, 5 * 4, "scales"}, {h_amax, 4, "h_amax"}};
  if ((rc = check_tables(tab, 2))) return rc;
  Buf ins[] = {req[0], req[1], req[2], opt[0], tab[0]};
  Buf outs[] = {req[3], req[4], req[5], opt[1], tab[1]};
  if ((rc = check_alias(ins, 5, outs, 5))) return rc;
  if ((rc = check_device())) return rc;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t he = t_zero_float_launch(h_amax, st);
  if (he != hipSuccess) return hip_fail(he, "amax reset launch");
  if (s.N == 0) return ok();
  const int N = (int)s.N, H = (int)s.H, Ft = (int)s.Ft;

  GemmArgs g1 = dense_args(N, Ft, H);
  g1.a = {Xq, nullptr, H, 0, 0};
  g1.b = {Aq_t, Auq_t, H, 0, sw ? Ft : 0};
  g1.epi.out0 = Z_save;
  g1.epi.out1 = H_act;
  g1.epi.ld0 = sw ? 2 * (int64_t)Ft : Ft;
  g1.epi.ld1 = Ft;
  g1.epi.split = Ft;
  g1.epi.out2 = H_q;
  g1.epi.ld2 = Ft;
  g1.epi.qs = scales;
  g1.epi.amax = h_amax;
  he = tgemm_fp8(sw ? GK_FC1_SWIGLU_F8 : GK_FC1_GELU_F8, g1, st);
  if (he != hipSuccess) return hip_fail(he, "FP8 FC1 launch");

  GemmArgs g2 = dense_args(N, H, Ft);
  g2.a = {H_q, nullptr, Ft, 0, 0};
  g2.b = {Bq_t, nullptr, Ft, 0, 0};
  g2.epi.out0 = Y_partial;
  g2.epi.ld0 = H;
  g2.epi.qs = scales;
  he = tgemm_fp8(GK_FC2_F8, g2, st);
  if (he != hipSuccess) return hip_fail(he, "FP8 FC2 launch");
  return ok();
}

int tp_fp8_transpose(int64_t rows, int64_t cols, const void* q, void* q_t, void* stream) {
  if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim || rows * cols > ((int64_t)1 << 40))
    return fail(TP_ERR_SHAPE, "rows and cols must be >= 0 and within range");
  if (rows % 16 || cols % 16) return fail(TP_ERR_SHAPE, "rows and cols must be multiples of 16");
  const size_t n = (size_t)(rows * cols);
  Buf in[] = {{q, n, "q"}};
  Buf out[] = {{q_t, n, "q_t"}};
  if (int rc = check_sized(in, 1)) return rc;
  if (int rc = check_sized(out, 1)) return rc;
  if (int rc = check_alias(in, 1, out, 1)) return rc;
  if (int rc = check_device()) return rc;
  hipError_t he = t_byte_transpose_launch(rows, cols, q, q_t, reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "transpose launch");
  return ok();
}

int tp_fp8_scale_update(int32_t fmt, int32_t n, int32_t len, float* history, float* amax,
                        float* scale, float* scale_inv, int32_t margin, void* stream) {
  if (fmt != TP_FP8_E4M3 && fmt != TP_FP8_E5M2) return fail(TP_ERR_DTYPE, "unknown fmt %d", fmt);
  if (n < 0 || n > (1 << 24)) return fail(TP_ERR_SHAPE, "n must be in 0..2^24");
  if (len < 1 || len > 1024) return fail(TP_ERR_SHAPE, "len must be in 1..1024");
  if (margin < 0 || margin > 16) return fail(TP_ERR_SHAPE, "margin must be in 0..16");
  const size_t nb = (size_t)n * 4;
  Buf bufs[] = {{history, nb * (size_t)len, "history"},
                {amax, nb, "amax"},
                {scale, nb, "scale"},
                {scale_inv, scale_inv ? nb : 0, "scale_inv"}};
  if (int rc = check_tables(bufs, 3)) return rc;
  if (scale_inv && (reinterpret_cast<uintptr_t>(scale_inv) & 3u))
    return fail(TP_ERR_ALIGN, "scale_inv is not 4-byte aligned");
  if (int rc = check_alias(nullptr, 0, bufs, 4)) return rc;
  if (int rc = check_device()) return rc;
  hipError_t he = t_fp8_scale_update_launch(fmt, n, len, margin, history, amax, scale, scale_inv,
                                            reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "scale update launch");
  return ok();
}

int tp_mlp_shard_bwd_fp8(const tp_mlp_desc* desc, const void* dYq, const void* dYq_t,
                         const void* Xq_t, const void* Hq_t, const void* Aq, const void* Auq,
                         const void* Bq, const void* Z_save, const float* scales, void* dX_partial,
                         float* dA, float* dA_up, float* dB, void* dZq, void* dZq_t,
                         float* dz_amax, void* stream) {
  Shard s;
  int rc = check_desc(desc, s);
  if (rc) return rc;
  if (s.dtype != TP_BF16) return fail(TP_ERR_DTYPE, "the FP8 backward reads bf16 Z and writes bf16 dX");
  if (s.H % 128 || s.Ft % 128 || s.N % 128)
    return fail(TP_ERR_SHAPE, "N, H and F_shard must be multiples of 128 for the FP8 backward");
  // the weight-gradient GEMMs read 256 rows of N codes through 32-bit offsets
  if (s.N > kMaxFp8Tokens)
    return fail(TP_ERR_SHAPE, "the FP8 backward takes at most %lld tokens", (long long)kMaxFp8Tokens);
  const bool sw = s.act == TP_ACT_SWIGLU;
  const size_t N = (size_t)s.N, H = (size_t)s.H, Ft = (size_t)s.Ft, zw = sw ? 2 * Ft : Ft;
  Buf in[] = {{dYq, N * H, "dYq"}, {dYq_t, N * H, "dYq_t"}, {Xq_t, N * H, "Xq_t"},
              {Hq_t, N * Ft, "Hq_t"}, {Aq, H * Ft, "Aq"}, {Bq, Ft * H, "Bq"},
              {Z_save, N * zw * 2, "Z_save"}};
  Buf out[] = {{dX_partial, N * H * 2, "dX_partial"}, {dA, H * Ft * 4, "dA"},
               {dB, Ft * H * 4, "dB"}, {dZq, N * zw, "dZq"}, {dZq_t, N * zw, "dZq_t"}};
  if ((rc = check_sized(in, 7))) return rc;
  if ((rc = check_sized(out, 5))) return rc;
  if (sw && (!Auq || !dA_up)) return fail(TP_ERR_NULL, "Auq and dA_up are required for SwiGLU");
  if (!sw && (Auq || dA_up)) return fail(TP_ERR_SHAPE, "Auq and dA_up must be NULL for GeLU");
  Buf iopt[] = {{Auq, sw ? H * Ft : 0, "Auq"}};
  Buf oopt[] = {{dA_up, sw ? H * Ft * 4 : 0, "dA_up"}};
  if ((rc = check_sized(iopt, 1)) || (rc = check_sized(oopt, 1))) return rc;
  Buf tab[] = {{scales, 7 * 4, "scales"}, {dz_amax, 4, "dz_amax"}};
  if ((rc = check_tables(tab, 2))) return rc;
  Buf ins[] = {in[0], in[1], in[2], in[3], in[4], in[5], in[6], iopt[0], tab[0]};
  Buf outs[] = {out[0], out[1], out[2], out[3], out[4], oopt[0], tab[1]};
  if ((rc = check_alias(ins, 9, outs, 7))) return rc;
  if ((rc = check_device())) return rc;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t he = t_zero_float_launch(dz_amax, st);
  if (he != hipSuccess) return hip_fail(he, "amax reset launch");
  const int n = (int)N, h = (int)H, f = (int)Ft, z = (int)zw;
  // 1. dZq = code(act'(Z) * (dYq Bq^T) dy_inv b_inv * dz_scale), amax |dZ|
  {
    GemmArgs g = dense_args(n, f, h);
    g.a = {dYq, nullptr, h, 0, 0};
    g.b = {Bq, nullptr, h, 0, 0};
    g.epi.aux = Z_save;
    g.epi.ldaux = z;
    g.epi.split = f;
    g.epi.out2 = dZq;
    g.epi.ld2 = z;
    g.epi.qs = scales;
    g.epi.qi = 0; g.epi.qj = 1; g.epi.qk = 5;
    g.epi.amax = dz_amax;
    he = tgemm_fp8(sw ? GK_DH_SWIGLU_F8 : GK_DH_GELU_F8, g, st);
    if (he != hipSuccess) return hip_fail(he, "FP8 dH launch");
  }
  he = t_byte_transpose_launch(N, zw, dZq, dZq_t, st);
  if (he != hipSuccess) return hip_fail(he, "dZ transpose launch");
  // 2. dB = (Hq^T codes) (dYq codes) h_inv dy_inv
  {
    GemmArgs g = dense_args(f, h, n);
    g.a = {Hq_t, nullptr, n, 0, 0};
    g.b = {dYq_t, nullptr, n, 0, 0};
    g.epi.out0 = dB;
    g.epi.ld0 = h;
    g.epi.qs = scales;
    g.epi.qi = 2; g.epi.qj = 0;
    he = tgemm_fp8(GK_WGRAD_F8, g, st);
    if (he != hipSuccess) return hip_fail(he, "FP8 dB launch");
  }
  // 3. dA (| dA_up) = (Xq^T codes) (dZq codes) x_inv dz_inv
  {
    GemmArgs g = dense_args(h, z, n);
    g.a = {Xq_t, nullptr, n, 0, 0};
    g.b = {dZq_t, nullptr, n, 0, 0};
    g.epi.out0 = dA;
    g.epi.out1 = dA_up;
    g.epi.ld0 = f;
    g.epi.ld1 = f;
    g.epi.split = f;
    g.epi.qs = scales;
    g.epi.qi = 3; g.epi.qj = 6;
    he = tgemm_fp8(sw ? GK_WGRAD_SPLIT_F8 : GK_WGRAD_F8, g, st);
    if (he != hipSuccess) return hip_fail(he, "FP8 dA launch");
  }
  // 4. dX_partial = (dZq codes) ([Aq | Auq] codes)^T dz_inv a_inv
  {
    GemmArgs g = dense_args(n, h, z);
    g.a = {dZq, nullptr, z, 0, 0};
    g.b = {Aq, Auq, f, 0, sw ? f : 0};
    g.epi.out0 = dX_partial;
    g.epi.ld0 = h;
    g.epi.qs = scales;
    g.epi.qi = 6; g.epi.qj = 4;
    he = tgemm_fp8(sw ? GK_DX_KSPLIT_F8 : GK_DX_F8, g, st);
    if (he != hipSuccess) return hip_fail(he, "FP8 dX launch");
  }
  return ok();
}

// ---------------------------------------------------------------------------
// MoE dispatch and combine
// ---------------------------------------------------------------------------
int tp_moe_permute(int32_t dtype, int64_t N, int64_t H, int64_t R, const int32_t* row_token,
                   const void* X, void* X_perm, void* stream) {
  if (int rc = check_rows(dtype, N, H, R)) return rc;
  const size_t e = dtype == TP_BF16 ? 2 : 4;
  Buf tab[] = {{row_token, (size_t)R * 4, "row_token"}};
  Buf in[] = {{X, R > 0 ? (size_t)(N * H) * e : 0, "X"}};
  Buf out[] = {{X_perm, (size_t)(R * H) * e, "X_perm"}};
  if (int rc = check_tables(tab, 1)) return rc;
  if (int rc = check_sized(in, 1)) return rc;
  if (int rc = check_sized(out, 1)) return rc;
  Buf ins[] = {tab[0], in[0]};
  if (int rc = check_alias(ins, 2, out, 1)) return rc;
  if (int rc = check_device()) return rc;
  hipError_t he = t_moe_permute_launch(dtype, row_token, N, H, R, X, X_perm,
                                     reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "permute launch");
  return ok();
}

int tp_moe_combine(int32_t dtype, int64_t N, int64_t H, int64_t R, const int32_t* tok_ptr,
                   const int32_t* tok_rows, const float* row_weight, const void* Y_perm,
                   void* Y, void* stream) {
  if (int rc = check_rows(dtype, N, H, R)) return rc;
  const size_t e = dtype == TP_BF16 ? 2 : 4;
  Buf tab[] = {{tok_ptr, N > 0 ? (size_t)(N + 1) * 4 : 0, "tok_ptr"},
               {tok_rows, N > 0 ? (size_t)R * 4 : 0, "tok_rows"}};
  Buf wt = {row_weight, row_weight ? (size_t)R * 4 : 0, "row_weight"};
  Buf in[] = {{Y_perm, N > 0 ? (size_t)(R * H) * e : 0, "Y_perm"}};
  Buf out[] = {{Y, (size_t)(N * H) * e, "Y"}};
  if (int rc = check_tables(tab, 2)) return rc;
  if (int rc = check_tables(&wt, 1)) return rc;
  if (int rc = check_sized(in, 1)) return rc;
  if (int rc = check_sized(out, 1)) return rc;
  Buf ins[] = {tab[0], tab[1], wt, in[0]};
  if (int rc = check_alias(ins, 4, out, 1)) return rc;
  if (int rc = check_device()) return rc;
  hipError_t he = t_moe_combine_launch(dtype, tok_ptr, tok_rows, row_weight, N, H, R, Y_perm, Y,
                                     reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "combine launch");
  return ok();
}

int tp_moe_combine_bwd(int32_t dtype, int64_t N, int64_t H, int64_t R, const int32_t* row_token,
                       const float* row_weight, const void* dY, const void* Y_perm,
                       void* dY_perm, float* d_weight, void* stream) {
  if (int rc = check_rows(dtype, N, H, R)) return rc;
  const size_t e = dtype == TP_BF16 ? 2 : 4;
  Buf tab[] = {{row_token, (size_t)R * 4, "row_token"},
               {row_weight, (size_t)R * 4, "row_weight"},
               {d_weight, (size_t)R * 4, "d_weight"}};
  Buf in[] = {{dY, R > 0 ? (size_t)(N * H) * e : 0, "dY"},
              {Y_perm, (size_t)(R * H) * e, "Y_perm"}};
  Buf out[] = {{dY_perm, (size_t)(R * H) * e, "dY_perm"}};
  if (int rc = check_tables(tab, 3)) return rc;
  if (int rc = check_sized(in, 2)) return rc;
  if (int rc = check_sized(out, 1)) return rc;
  Buf ins[] = {tab[0], tab[1], in[0], in[1]};
  Buf outs[] = {out[0], tab[2]};
  if (int rc = check_alias(ins, 4, outs, 2)) return rc;
  if (int rc = check_device()) return rc;
  hipError_t he = t_moe_combine_bwd_launch(dtype, row_token, row_weight, N, H, R, dY, Y_perm,
                                         dY_perm, d_weight, reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "combine backward launch");
  return ok();
}

}  // extern "C"
