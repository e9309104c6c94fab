// Drives the C ABI's argument checks (tensor_transformer_mlp_02_amd/csrc/
// api.hip, compiled for the host only) under AddressSanitizer and
// UndefinedBehaviorSanitizer, on a machine without a GPU.  The kernels'
// launchers are stubs that abort: every call must be decided by the
// argument checks or by the device check (no GPU: TP_ERR_DEVICE), so a
// call that reached a launcher, a status outside 1..8, a missing error
// message, or any memory / undefined-behaviour error fails the run.
//
// Cases: the documented rejections (mirroring the CPU ABI tests), then a
// seeded fuzz of descriptors, sizes, offsets tables and pointers (NULL,
// misaligned, overlapping, far apart) over every entry point.  Prints "OK".
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "launch.h"

namespace tpmlp {
[[noreturn]] static void reached(const char* what) {
  fprintf(stderr, "FAIL: %s reached without a GPU\n", what);
  abort();
}
hipError_t gemm_bf16(GemmKind, GemmArgs&, hipStream_t) { reached("gemm_bf16"); }
hipError_t gemm_f32(GemmKind, GemmArgs&, hipStream_t) { reached("gemm_f32"); }
hipError_t partial_sum_launch(int, int, const void* const*, int64_t, void*, int, hipStream_t) {
  reached("partial_sum_launch");
}
hipError_t gemm_fp8(GemmKind, GemmArgs&, hipStream_t) { reached("gemm_fp8"); }
hipError_t fp8_quantize_launch(int, bool, int64_t, int64_t, const void*, const float*, void*,
                               float*, hipStream_t) {
  reached("fp8_quantize_launch");
}
hipError_t zero_float_launch(float*, hipStream_t) { reached("zero_float_launch"); }
hipError_t fp8_scale_update_launch(int, int, int, int, float*, float*, float*, float*,
                                   hipStream_t) {
  reached("fp8_scale_update_launch");
}
hipError_t byte_transpose_launch(int64_t, int64_t, const void*, void*, hipStream_t) {
  reached("byte_transpose_launch");
}
hipError_t moe_permute_launch(int, const int32_t*, int64_t, int64_t, int64_t, const void*, void*,
                              hipStream_t) {
  reached("moe_permute_launch");
}
hipError_t moe_combine_launch(int, const int32_t*, const int32_t*, const float*, int64_t, int64_t,
                              int64_t, const void*, void*, hipStream_t) {
  reached("moe_combine_launch");
}
hipError_t moe_combine_bwd_launch(int, const int32_t*, const float*, int64_t, int64_t, int64_t,
                                  const void*, const void*, void*, float*, hipStream_t) {
  reached("moe_combine_bwd_launch");
}
}  // namespace tpmlp

static int fails = 0;
static long calls = 0;

// every status must be an error with a message (no GPU: nothing succeeds)
static void check(int rc, const char* what, int want = -1) {
  ++calls;
  const char* msg = tp_last_error();
  if (rc < 1 || rc > 8 || !msg || !msg[0] || (want >= 0 && rc != want)) {
    fprintf(stderr, "FAIL %s: status %d (want %d) message '%s'\n", what, rc, want, msg ? msg : "");
    ++fails;
  }
  if (strcmp(tp_status_string(rc), "TP_ERR_UNKNOWN") == 0) {
    fprintf(stderr, "FAIL %s: unnamed status %d\n", what, rc);
    ++fails;
  }
}

static uint64_t st = 0x9e3779b97f4a7c15ull;
static uint64_t rnd() {
  st ^= st << 13; st ^= st >> 7; st ^= st << 17;
  return st;
}
static int64_t pick(const int64_t* v, int n) { return v[rnd() % n]; }

// fake device addresses 1 TiB apart (never dereferenced), some NULL, some
// misaligned, some equal to another (overlap)
static void* fake(int k) { return (void*)(uintptr_t)((1ull << 44) + ((uint64_t)k << 40)); }
static void* ptr_any(int k) {
  switch (rnd() % 12) {
    case 0: return nullptr;
    case 1: return (char*)fake(k) + 4;
    case 2: return fake((int)(rnd() % 6));
    default: return fake(k);
  }
}

int main() {
  const int64_t dims[] = {-1, 0, 1, 4, 7, 8, 12, 64, 128, 256, 300, 4096, (1 << 21) + 8,
                          (int64_t)1 << 31, INT64_MAX};
  const int32_t smalls[] = {-1, 0, 1, 2, 7, 8, 64, 65};
  const int ND = sizeof(dims) / sizeof(dims[0]);
  const int NS = sizeof(smalls) / sizeof(smalls[0]);

  // --- documented rejections (statuses as the header states) -----------------
  tp_mlp_desc d = {64, 2, 256, 128, 8, TP_ACT_GELU_TANH, TP_BF16};
  check(tp_mlp_shard_fwd(nullptr, fake(1), fake(2), nullptr, fake(3), fake(4), fake(5), fake(6),
                         nullptr), "fwd NULL desc", TP_ERR_NULL);
  {
    tp_mlp_desc e = d; e.dtype = 7;
    check(tp_mlp_shard_fwd(&e, fake(1), fake(2), nullptr, fake(3), fake(4), fake(5), fake(6),
                           nullptr), "fwd dtype", TP_ERR_DTYPE);
    e = d; e.H = 12;
    check(tp_mlp_shard_fwd(&e, fake(1), fake(2), nullptr, fake(3), fake(4), fake(5), fake(6),
                           nullptr), "fwd H % 8", TP_ERR_SHAPE);
    e = d; e.T = 0;
    check(tp_mlp_shard_fwd(&e, fake(1), fake(2), nullptr, fake(3), fake(4), fake(5), fake(6),
                           nullptr), "fwd T", TP_ERR_SHAPE);
  }
  check(tp_mlp_shard_fwd(&d, (char*)fake(1) + 2, fake(2), nullptr, fake(3), fake(4), fake(5),
                         fake(6), nullptr), "fwd misaligned X", TP_ERR_ALIGN);
  check(tp_mlp_shard_fwd(&d, fake(1), fake(2), nullptr, fake(3), fake(4), fake(5), fake(1),
                         nullptr), "fwd Y aliases X", TP_ERR_ALIAS);
  check(tp_mlp_shard_fwd(&d, fake(1), fake(2), fake(7), fake(3), fake(4), fake(5), fake(6),
                         nullptr), "fwd A_up for GeLU", TP_ERR_SHAPE);
  check(tp_mlp_shard_fwd(&d, fake(1), fake(2), nullptr, fake(3), fake(4), fake(5), fake(6),
                         nullptr), "fwd valid", TP_ERR_DEVICE);
  {
    const size_t ws = tp_mlp_shard_bwd_workspace(&d);
    float* f = (float*)fake(9);
    check(tp_mlp_shard_bwd(&d, fake(1), fake(2), nullptr, fake(3), fake(4), fake(5), fake(7),
                           fake(8), f, nullptr, (float*)fake(10), fake(14), ws - 16, nullptr),
          "bwd small workspace", TP_ERR_WORKSPACE);
    check(tp_mlp_shard_bwd(&d, fake(1), fake(2), nullptr, fake(3), fake(4), fake(5), fake(7),
                           fake(8), f, nullptr, (float*)fake(10), fake(14), ws, nullptr),
          "bwd valid", TP_ERR_DEVICE);
    // the derivative formed in the operand loads needs dH only: N * F_shard elements
    const size_t dh = (size_t)(d.S * d.B * d.F_shard) * 2;
    check(tp_mlp_shard_bwd_dact_prologue(&d, fake(1), fake(2), nullptr, fake(3), fake(4), fake(5),
                                         fake(7), fake(8), f, nullptr, (float*)fake(10), fake(14),
                                         dh - 16, nullptr),
          "bwd dact small workspace", TP_ERR_WORKSPACE);
    check(tp_mlp_shard_bwd_dact_prologue(&d, fake(1), fake(2), nullptr, fake(3), fake(4), fake(5),
                                         fake(7), fake(8), f, nullptr, (float*)fake(10), fake(14),
                                         dh, nullptr),
          "bwd dact valid", TP_ERR_DEVICE);
  }
  {
    const void* parts[TP_MAX_SHARDS + 1];
    for (int i = 0; i <= TP_MAX_SHARDS; ++i) parts[i] = fake(1 + i % 7);
    check(tp_partial_sum(TP_BF16, TP_MAX_SHARDS + 1, parts, 1024, fake(20), nullptr),
          "psum T", TP_ERR_SHAPE);
    check(tp_partial_sum(TP_BF16, 2, nullptr, 1024, fake(20), nullptr), "psum NULL", TP_ERR_NULL);
    check(tp_partial_sum(TP_BF16, TP_MAX_SHARDS, parts, 1024, fake(20), nullptr), "psum valid",
          TP_ERR_DEVICE);
  }
  {
    tp_expert_desc ed = {256, 128, 4, TP_BF16};
    const int64_t bad[] = {0, 5, 3, 9, 9};   // decreasing
    check(tp_grouped_expert_fwd(&ed, bad, fake(1), fake(2), fake(3), fake(4), fake(5), fake(6),
                                fake(7), nullptr), "grouped offsets", TP_ERR_SHAPE);
    const int32_t* dev_off = reinterpret_cast<const int32_t*>(fake(8));
    check(tp_grouped_expert_fwd_devoff(&ed, -1, dev_off, fake(1), fake(2), fake(3), fake(4),
                                       fake(5), fake(6), fake(7), nullptr),
          "devoff R", TP_ERR_SHAPE);
    check(tp_grouped_expert_fwd_devoff(&ed, 100, nullptr, fake(1), fake(2), fake(3), fake(4),
                                       fake(5), fake(6), fake(7), nullptr),
          "devoff NULL", TP_ERR_NULL);
    check(tp_grouped_expert_bwd_devoff(&ed, 100, dev_off, fake(1), fake(2), fake(3), fake(4),
                                       fake(5), fake(6), fake(9), fake(10), (float*)fake(11),
                                       (float*)fake(12), (float*)fake(13), fake(14),
                                       tp_grouped_expert_devoff_workspace(&ed, 100), 3, nullptr),
          "devoff accumulate", TP_ERR_SHAPE);
    check(tp_grouped_expert_bwd_devoff(&ed, 100, dev_off, fake(1), fake(2), fake(3), fake(4),
                                       fake(5), fake(6), fake(9), fake(10), (float*)fake(11),
                                       (float*)fake(12), (float*)fake(13), fake(14),
                                       tp_grouped_expert_devoff_workspace(&ed, 100), 1, nullptr),
          "devoff valid", TP_ERR_DEVICE);
  }

  // --- fuzz ---------------------------------------------------------------------
  int64_t offs[TP_MAX_EXPERTS + 2];
  const void* parts[TP_MAX_SHARDS];
  for (int it = 0; it < 20000; ++it) {
    tp_mlp_desc e;
    e.S = pick(dims, ND); e.B = pick(dims, ND); e.H = pick(dims, ND); e.F_shard = pick(dims, ND);
    e.T = smalls[rnd() % NS]; e.act = (int32_t)(rnd() % 3); e.dtype = (int32_t)(rnd() % 3);
    const int variant = (int)(rnd() % 10);
    tp_mlp_desc* pd = rnd() % 50 ? &e : nullptr;
    switch (variant) {
      case 0:
        check(tp_mlp_shard_fwd(pd, ptr_any(1), ptr_any(2), ptr_any(3), ptr_any(4), ptr_any(5),
                               ptr_any(6), ptr_any(7), nullptr), "fuzz fwd");
        break;
      case 1: {
        const size_t ws = tp_mlp_shard_bwd_workspace(pd);
        const size_t wsb = rnd() % 2 ? ws : (size_t)(rnd() % 4096);
        const int which = (int)(rnd() % 3);
        auto fn = which == 0 ? tp_mlp_shard_bwd
                             : which == 1 ? tp_mlp_shard_bwd_accum : tp_mlp_shard_bwd_dact_prologue;
        if (rnd() % 3 == 0)
          check(tp_mlp_shard_bwd_noalloc(pd, ptr_any(1), ptr_any(2), ptr_any(3), ptr_any(4),
                                         ptr_any(5), ptr_any(6), ptr_any(7), ptr_any(8),
                                         (float*)ptr_any(9), (float*)ptr_any(10),
                                         (float*)ptr_any(11), nullptr), "fuzz bwd noalloc");
        else
          check(fn(pd, ptr_any(1), ptr_any(2), ptr_any(3), ptr_any(4), ptr_any(5), ptr_any(6),
                   ptr_any(7), ptr_any(8), (float*)ptr_any(9), (float*)ptr_any(10),
                   (float*)ptr_any(11), ptr_any(12), wsb, nullptr), "fuzz bwd");
        break;
      }
      case 2: {
        const int T = smalls[rnd() % NS];
        for (int i = 0; i < TP_MAX_SHARDS; ++i) parts[i] = ptr_any(1 + i % 9);
        const int64_t count = pick(dims, ND);
        const void* out = rnd() % 4 ? ptr_any(20) : parts[0];
        const int which = (int)(rnd() % 3);
        if (which == 0)
          check(tp_partial_sum(e.dtype, T, rnd() % 20 ? parts : nullptr, count, (void*)out,
                               nullptr), "fuzz psum");
        else if (which == 1)
          check(tp_partial_sum_capped(e.dtype, T, parts, count, (void*)out, smalls[rnd() % NS],
                                      nullptr), "fuzz psum capped");
        else
          check(tp_partial_sum_scatter(e.dtype, T, parts, e.S, e.B, e.H, smalls[rnd() % NS],
                                       (void*)out, nullptr), "fuzz scatter");
        break;
      }
      case 3:
      case 4: {
        tp_expert_desc ed = {pick(dims, ND), pick(dims, ND), smalls[rnd() % NS], e.dtype};
        const int E = ed.E >= 1 && ed.E <= TP_MAX_EXPERTS ? ed.E : 1;
        offs[0] = rnd() % 16 ? 0 : 3;
        for (int i = 1; i <= E; ++i) {
          const int64_t step = rnd() % 8 ? (int64_t)(rnd() % 600) : pick(dims, ND);
          // saturate instead of overflowing (a huge or negative step is a
          // bad table either way)
          offs[i] = (step > 0 && offs[i - 1] > INT64_MAX - step) ? INT64_MAX : offs[i - 1] + step;
        }
        tp_expert_desc* pe = rnd() % 50 ? &ed : nullptr;
        const int64_t* po = rnd() % 50 ? offs : nullptr;
        if (rnd() % 3 == 0) {
          // device-resident offsets: the host must never read the table
          // (a fake address here), only check R, its pointer and alignment
          const int64_t R = rnd() % 8 ? (int64_t)(rnd() % 5000) : pick(dims, ND);
          const int32_t* pdo = reinterpret_cast<const int32_t*>(ptr_any(13));
          if (variant == 3) {
            check(tp_grouped_expert_fwd_devoff(pe, R, pdo, ptr_any(1), ptr_any(2), ptr_any(3),
                                               ptr_any(4), ptr_any(5), ptr_any(6), ptr_any(7),
                                               nullptr),
                  "fuzz grouped fwd devoff");
          } else {
            const size_t ws = tp_grouped_expert_devoff_workspace(pe, R);
            check(tp_grouped_expert_bwd_devoff(pe, R, pdo, ptr_any(1), ptr_any(2), ptr_any(3),
                                               ptr_any(4), ptr_any(5), ptr_any(6), ptr_any(7),
                                               ptr_any(8), (float*)ptr_any(9),
                                               (float*)ptr_any(10), (float*)ptr_any(11),
                                               ptr_any(12), rnd() % 2 ? ws : 64,
                                               (int32_t)(rnd() % 4), nullptr),
                  "fuzz grouped bwd devoff");
          }
        } else if (variant == 3) {
          check(tp_grouped_expert_fwd(pe, po, ptr_any(1), ptr_any(2), ptr_any(3), ptr_any(4),
                                      ptr_any(5), ptr_any(6), ptr_any(7), nullptr),
                "fuzz grouped fwd");
        } else {
          const size_t ws = tp_grouped_expert_bwd_workspace(pe, po);
          auto fn = rnd() % 2 ? tp_grouped_expert_bwd : tp_grouped_expert_bwd_accum;
          check(fn(pe, po, ptr_any(1), ptr_any(2), ptr_any(3), ptr_any(4), ptr_any(5),
                   ptr_any(6), ptr_any(7), ptr_any(8), (float*)ptr_any(9), (float*)ptr_any(10),
                   (float*)ptr_any(11), ptr_any(12), rnd() % 2 ? ws : 64, nullptr),
                "fuzz grouped bwd");
        }
        break;
      }
      case 5: {
        const int64_t N = pick(dims, ND), H = pick(dims, ND), R = pick(dims, ND);
        const int which = (int)(rnd() % 3);
        if (which == 0)
          check(tp_moe_permute(e.dtype, N, H, R, (const int32_t*)ptr_any(1), ptr_any(2),
                               ptr_any(3), nullptr), "fuzz permute");
        else if (which == 1)
          check(tp_moe_combine(e.dtype, N, H, R, (const int32_t*)ptr_any(1),
                               (const int32_t*)ptr_any(2), (const float*)ptr_any(3), ptr_any(4),
                               ptr_any(5), nullptr), "fuzz combine");
        else
          check(tp_moe_combine_bwd(e.dtype, N, H, R, (const int32_t*)ptr_any(1),
                                   (const float*)ptr_any(2), ptr_any(3), ptr_any(4), ptr_any(5),
                                   (float*)ptr_any(6), nullptr), "fuzz combine bwd");
        break;
      }
      case 6:
        check(tp_fp8_quantize(smalls[rnd() % NS], (int32_t)(rnd() % 2), pick(dims, ND),
                              pick(dims, ND), ptr_any(1), (const float*)ptr_any(2), ptr_any(3),
                              (float*)ptr_any(4), nullptr), "fuzz quantize");
        break;
      case 7:
        if (rnd() % 2)
          check(tp_fp8_transpose(pick(dims, ND), pick(dims, ND), ptr_any(1), ptr_any(2), nullptr),
                "fuzz transpose");
        else
          check(tp_fp8_scale_update((int32_t)(rnd() % 3), (int32_t)pick(dims, ND),
                                    (int32_t)(rnd() % 1100), (float*)ptr_any(1),
                                    (float*)ptr_any(2), (float*)ptr_any(3), (float*)ptr_any(4),
                                    (int32_t)(rnd() % 20) - 2, nullptr),
                "fuzz scale update");
        break;
      case 8:
        check(tp_mlp_shard_fwd_fp8(pd, ptr_any(1), ptr_any(2), ptr_any(3), ptr_any(4),
                                   (const float*)ptr_any(5), ptr_any(6), ptr_any(7), ptr_any(8),
                                   (float*)ptr_any(9), ptr_any(10), nullptr), "fuzz fwd fp8");
        break;
      default:
        check(tp_mlp_shard_bwd_fp8(pd, ptr_any(1), ptr_any(2), ptr_any(3), ptr_any(4),
                                   ptr_any(5), ptr_any(6), ptr_any(7), ptr_any(8),
                                   (const float*)ptr_any(9), ptr_any(10), (float*)ptr_any(11),
                                   (float*)ptr_any(12), (float*)ptr_any(13), ptr_any(14),
                                   ptr_any(15), (float*)ptr_any(16), nullptr), "fuzz bwd fp8");
        break;
    }
  }
  if (fails) {
    fprintf(stderr, "%d of %ld calls failed\n", fails, calls);
    return 1;
  }
  printf("OK %ld calls\n", calls);
  return 0;
}
