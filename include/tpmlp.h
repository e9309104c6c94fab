/*
 * tpmlp.h -- C ABI of the tensor-parallel MLP shard library (libtpmlp.so).
 *
 * One tensor-parallel rank's share of the paired column-parallel ->
 * activation -> row-parallel MLP, on one gfx950 (MI355X) GPU:
 *
 *   forward   Z_i = X A_i,  H_i = act(Z_i),  Y_i = H_i B_i
 *   backward  dB_i = H_i^T dY,  dZ_i = (dY B_i^T) * act'(Z_i),
 *             dA_i = X^T dZ_i,  dX_i = dZ_i A_i^T
 *
 * The column split of A and the row split of B, and where the two sums
 * over shards sit (Y after the row-parallel product, dX before the
 * column-parallel one), follow "Megatron-LM 源码精读——大模型并行训练全景",
 * §三 3.1 (ColumnParallelLinear), 3.2 (RowParallelLinear), 3.3 (the MLP's
 * column/row pairing and its diagram) and 3.4 (the forward-identity /
 * backward-all-reduce and forward-all-reduce / backward-identity
 * mappings).  Shapes follow "Megatron Core 带读" §02: hidden [S,B,H],
 * column output [S,B,O/p], row input [S,B,I/p], row partial [S,B,O].
 *
 * Citations below use these keys for the pages they come from:
 *   [P1] "Megatron-LM 源码精读——大模型并行训练全景" (sections §三 3.1-3.5
 *        tensor parallelism, §五 5.2 gradient-accumulation fusion, §七
 *        the model's MLP, §八 8.2 FP8); a bare "§" with no key is [P1]
 *   [P2] "Megatron-LM and 3D Parallelism" (context only)
 *   [P3] "Megatron Core 带读" (§02 tensor shapes, §06 sequence
 *        parallelism, §09 MoE dispatch / combine, §10 FP8)
 *   [P4] "Megatron-LM 源码精读" docs index ("MoE 层与 Expert Parallelism":
 *        grouped-GEMM expert compute)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout:    every matrix is row-major and contiguous.  [S,B,H] hidden
 *            states are the [N,H] matrix with N = S*B and row n = s*B + b.
 *            Weights use the mathematical layout: A_i [H, F_shard],
 *            B_i [F_shard, H] (not PyTorch's transposed [out,in] storage).
 * Types:     TP_BF16 tensors are bfloat16 bit patterns (2 bytes); TP_F32
 *            tensors are IEEE float.  Products accumulate in fp32.  bf16
 *            outputs are rounded to nearest even.  Weight gradients are
 *            always fp32.
 * Ownership: the caller owns every buffer.  The library never allocates,
 *            frees or synchronizes; inputs are never written.  Kernels are
 *            enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *            and the call returns without waiting for them.
 * Pointers:  device pointers, 16-byte aligned.  Outputs must not overlap
 *            inputs or each other (tp_partial_sum's in-place form aside).
 * Errors:    a nonzero tp_status is returned and nothing is enqueued when
 *            an argument check fails; tp_last_error() then holds a message
 *            (per thread).  Argument checks touch no GPU state, so they
 *            run on machines without a GPU.  A launch failure returns
 *            TP_ERR_HIP.  Faults inside kernels surface at the caller's
 *            next synchronization, as HIP errors.  The library never
 *            aborts and never prints.
 * Threads:   all entry points are reentrant; the only global state is a
 *            per-device "is this a gfx950" cache filled on first use.
 */
#ifndef TPMLP_H
#define TPMLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tp_dtype { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* GeLU in its tanh form (Hendrycks & Gimpel); SwiGLU = silu(X Ag) * (X Au)
 * (Shazeer, "GLU Variants Improve Transformer").  The pages name GeLU for
 * the MLP (§三 3.3 diagram) and, for Llama-style models, a SwiGLU MLP with
 * three weight matrices (§七 mlp.py), without printing either formula. */
typedef enum tp_act { TP_ACT_GELU_TANH = 0, TP_ACT_SWIGLU = 1 } tp_act;

typedef enum tp_status {
    TP_OK = 0,
    TP_ERR_NULL = 1,      /* a required pointer is NULL                     */
    TP_ERR_SHAPE = 2,     /* a dimension is out of range or indivisible     */
    TP_ERR_DTYPE = 3,     /* unknown dtype / activation, or unsupported mix */
    TP_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned               */
    TP_ERR_WORKSPACE = 5, /* workspace missing or too small                 */
    TP_ERR_DEVICE = 6,    /* no current HIP device, or it is not gfx950     */
    TP_ERR_HIP = 7,       /* a HIP launch failed                            */
    TP_ERR_ALIAS = 8      /* an output overlaps an input or another output  */
} tp_status;

/* Largest shard count accepted (pointers of tp_partial_sum travel by value
 * in the kernel's argument block). */
#define TP_MAX_SHARDS 64
/* Largest number of local experts of one grouped call. */
#define TP_MAX_EXPERTS 64

/*
 * One shard's problem.  N = S*B tokens (may be 0: empty batch), hidden H,
 * shard width F_shard = F/T (the full width divided by the shard count:
 * §三 3.1, the per-partition output size is output size / world size).
 * T (1..TP_MAX_SHARDS) is recorded for checks only: a shard's arithmetic
 * does not depend on it.  act is a tp_act, dtype a tp_dtype.
 * H and F_shard must be positive multiples of 8 (bf16) or 4 (fp32), with
 * H <= 2^21 and F_shard <= 2^20 (row strides are addressed with 32-bit
 * offsets), and N <= 2^30.
 */
typedef struct tp_mlp_desc {
    int64_t S, B, H, F_shard;
    int32_t T, act, dtype;
} tp_mlp_desc;

/*
 * tp_mlp_shard_fwd -- forward of one shard (§三 3.1-3.3).
 *   X         [N,H]        input hidden states (replicated on every shard)
 *   A         [H,F_shard]  column shard of FC1 (the gate projection for
 *                          SwiGLU)
 *   A_up      [H,F_shard]  SwiGLU up projection; must be NULL for GeLU
 *   B         [F_shard,H]  row shard of FC2
 *   Z_save    GeLU: [N,F_shard] pre-activation Z;  SwiGLU: [N,2*F_shard],
 *             row n = [G(n,:) | U(n,:)].  Saved for the backward; NULL =
 *             forward only (nothing saved).
 *   H_act     [N,F_shard]  post-activation (also saved for the backward)
 *   Y_partial [N,H]        this shard's partial output; the full output
 *                          is the sum over shards (tp_partial_sum)
 * The activation is applied in the FC1 kernel's epilogue: Z is never
 * re-read to compute H.
 */
int tp_mlp_shard_fwd(const tp_mlp_desc *desc, const void *X, const void *A,
                     const void *A_up, const void *B, void *Z_save,
                     void *H_act, void *Y_partial, void *stream);

/* Bytes of device workspace tp_mlp_shard_bwd needs: the activation-side
 * gradient dZ ([N,F_shard], SwiGLU [N,2*F_shard], in the dtype).  Returns
 * 0 and sets tp_last_error() for an invalid descriptor (and for N = 0). */
size_t tp_mlp_shard_bwd_workspace(const tp_mlp_desc *desc);

/*
 * tp_mlp_shard_bwd -- backward of one shard.
 *   X, A, A_up, B   as in the forward
 *   Z_save, H_act   the forward's saved tensors (Z_save required)
 *   dY [N,H]        the FULL output gradient: the backward of the sum over
 *                   shards is the identity, so every shard receives all of
 *                   it (§三 3.4, the reduce mapping's backward)
 *   dX_partial [N,H]  this shard's partial input gradient; the input
 *                   gradient is the sum over shards (§三 3.1: dL/dX =
 *                   sum_i dL/dY_i W_i^T), i.e. tp_partial_sum
 *   dA  [H,F_shard] fp32   gradient of A (the gate projection for SwiGLU)
 *   dA_up [H,F_shard] fp32 SwiGLU only, else NULL
 *   dB  [F_shard,H] fp32
 *   workspace, ws_bytes    at least tp_mlp_shard_bwd_workspace(desc) bytes;
 *                   on return it holds dZ, row-major [N,F_shard] in the
 *                   dtype ([N,2*F_shard] = [dG | dU] for SwiGLU)
 * The activation derivative is applied inside the kernel that forms
 * dY B_i^T (in its epilogue); no separate elementwise pass runs.
 * With N = 0 the weight gradients are written as zeros.
 */
int tp_mlp_shard_bwd(const tp_mlp_desc *desc, const void *X, const void *A,
                     const void *A_up, const void *B, const void *Z_save,
                     const void *H_act, const void *dY, void *dX_partial,
                     float *dA, float *dA_up, float *dB, void *workspace,
                     size_t ws_bytes, void *stream);

/*
 * tp_mlp_shard_bwd_noalloc -- tp_mlp_shard_bwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same kernels and the same results bit for bit.  The
 * activation-side gradient dZ goes to a scratch array inside the library
 * (TP_NOALLOC_SCRATCH_BYTES bytes, held by each GPU the library runs on
 * until the process ends); the call allocates nothing.  It fails with
 * TP_ERR_WORKSPACE when dZ needs more (N * F_shard * element size, SwiGLU
 * twice that: up to 2^25 bf16 elements, e.g. 4096 tokens at F_shard = 4096
 * for SwiGLU or 8192 tokens at F_shard = 4096 for GeLU).  Every call on one
 * GPU uses that GPU's one array: calls that overlap on one GPU (on streams
 * that run concurrently) race and must not be made.
 */
#define TP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int tp_mlp_shard_bwd_noalloc(const tp_mlp_desc *desc, const void *X, const void *A,
                             const void *A_up, const void *B, const void *Z_save,
                             const void *H_act, const void *dY, void *dX_partial, float *dA,
                             float *dA_up, float *dB, void *stream);

/*
 * tp_partial_sum -- out = sum_{i=0}^{T-1} partials[i], elementwise: the
 * arithmetic the all-reduce performs over the T shards' partial outputs
 * (§三 3.2/3.3: forward sum of Y_i; backward sum of dX_i), here over
 * partials already resident in one GPU's memory.
 *   dtype     TP_BF16 or TP_F32 (every buffer has this type)
 *   T         1..TP_MAX_SHARDS
 *   partials  HOST array of T device pointers, `count` elements each
 *   out       `count` elements; may be exactly one of the partials
 *             (in-place), must not otherwise overlap them
 * Each element is summed in fp32 in the fixed order i = 0..T-1 and then
 * rounded once to the output type.  count may be 0 (nothing is launched).
 */
int tp_partial_sum(int32_t dtype, int32_t T, const void *const *partials,
                   int64_t count, void *out, void *stream);

/*
 * tp_partial_sum_scatter -- the reduce-scatter form of tp_partial_sum used
 * with sequence parallelism ([P1] §三 3.5; [P3] §06 Sequence Parallel):
 * each of the T ranks keeps only its slice of the sequence, so this rank's
 * output is rows s = rank*S/T .. (rank+1)*S/T - 1 of the summed [S,B,H]
 * tensor (with n = s*B + b these rows are one contiguous range):
 *   out[j] = sum_{i<T} partials[i][rank*(S/T)*B*H + j],  j < (S/T)*B*H
 *   partials  HOST array of T device pointers to full [S,B,H] partials
 *   S, B, H   the full shape; S must be a multiple of T; H a multiple of 8
 *             (bf16) or 4 (fp32)
 *   rank      0..T-1
 *   out       [S/T,B,H]; must not overlap any partial
 * Each element is summed in fp32 in the order i = 0..T-1 and rounded once:
 * the result equals the same rows of tp_partial_sum's output bit for bit.
 * The backward of the sequence all-gather in front of FC1 is this same
 * reduce-scatter applied to the dX partials.
 */
int tp_partial_sum_scatter(int32_t dtype, int32_t T, const void *const *partials,
                           int64_t S, int64_t B, int64_t H, int32_t rank, void *out,
                           void *stream);

/*
 * tp_partial_sum_capped -- tp_partial_sum on at most `max_workgroups`
 * workgroups of 256 threads (which stride over the whole tensor), for a
 * second stream beside the shard's GEMMs, the way the all-reduce it stands
 * in for overlaps computation (§三 3.4 places the reduce between the
 * shard's forward and the next layer, and its backward twin after dX_i).
 * Its kernel keeps few registers per lane, so its wavefronts can share
 * SIMDs with a running GEMM's instead of holding compute units.
 *   max_workgroups  >= 1; other arguments as in tp_partial_sum
 * The result is bitwise identical to tp_partial_sum's (same order).
 */
int tp_partial_sum_capped(int32_t dtype, int32_t T, const void *const *partials,
                          int64_t count, void *out, int32_t max_workgroups,
                          void *stream);

/*
 * Grouped local experts: E experts, each a full SwiGLU MLP of width F
 * (expert tensor parallelism 1), over rows already sorted by expert
 * ("Megatron Core 带读" §09: the dispatcher brings each token to the rank
 * that holds its expert, the local experts compute, combine returns the
 * results; the docs index of "Megatron-LM 源码精读", "MoE 层与 Expert
 * Parallelism": grouped-GEMM expert compute).  bf16 only.
 * H and F must be positive multiples of 8, H <= 2^21, F <= 2^20;
 * 1 <= E <= TP_MAX_EXPERTS.
 */
typedef struct tp_expert_desc {
    int64_t H, F;
    int32_t E, dtype;
} tp_expert_desc;

/*
 * tp_grouped_expert_fwd
 *   offsets  HOST array of E+1 row offsets: expert e owns rows
 *            [offsets[e], offsets[e+1]); offsets[0] = 0, non-decreasing;
 *            R = offsets[E] (experts may own no rows; R may be 0)
 *   X_perm   [R,H]      routed token rows in (expert, token) order
 *   Wg, Wu   [E,H,F]    gate / up projections of each expert
 *   Wd       [E,F,H]    down projection of each expert
 *   Z_save   [R,2F]     row r = [G(r,:) | U(r,:)]; NULL = forward only
 *   H_act    [R,F]
 *   Y_perm   [R,H]      expert outputs, unweighted (the router's weighted
 *                       combine is outside this call)
 */
int tp_grouped_expert_fwd(const tp_expert_desc *desc, const int64_t *offsets,
                          const void *X_perm, const void *Wg, const void *Wu,
                          const void *Wd, void *Z_save, void *H_act,
                          void *Y_perm, void *stream);

/* Bytes of workspace tp_grouped_expert_bwd needs ([R,2F] bf16). */
size_t tp_grouped_expert_bwd_workspace(const tp_expert_desc *desc,
                                       const int64_t *offsets);

/*
 * tp_grouped_expert_bwd -- backward of tp_grouped_expert_fwd.
 *   dY_perm [R,H]   gradient of Y_perm
 *   dX_perm [R,H]   gradient of X_perm
 *   dWg, dWu [E,H,F] fp32, dWd [E,F,H] fp32 (zeros for an expert with no
 *                   rows)
 */
int tp_grouped_expert_bwd(const tp_expert_desc *desc, const int64_t *offsets,
                          const void *X_perm, const void *Wg, const void *Wu,
                          const void *Wd, const void *Z_save,
                          const void *H_act, const void *dY_perm,
                          void *dX_perm, float *dWg, float *dWu, float *dWd,
                          void *workspace, size_t ws_bytes, void *stream);

/*
 * Gradient-accumulation fusion ([P1] §五 5.2: the weight gradients of the
 * M microbatches of one iteration are added straight into the fp32 grad
 * buffer by the weight-gradient kernel, with no intermediate tensor).
 * tp_mlp_shard_bwd_accum and tp_grouped_expert_bwd_accum take the same
 * arguments as tp_mlp_shard_bwd / tp_grouped_expert_bwd, but the weight
 * gradients are in/out: dA += X^T dZ, dA_up += ..., dB += H^T dY (grouped:
 * dWg, dWu, dWd likewise), each element read, added to in fp32 and written
 * once by the one tile that owns it, so the result is deterministic (no
 * atomics).  dX_partial is written as in the plain call.  The caller zeroes
 * the buffers before the first microbatch.  With N = 0 (or an expert with no
 * rows) the buffers are left unchanged.
 */
int tp_mlp_shard_bwd_accum(const tp_mlp_desc *desc, const void *X, const void *A,
                           const void *A_up, const void *B, const void *Z_save,
                           const void *H_act, const void *dY, void *dX_partial,
                           float *dA, float *dA_up, float *dB, void *workspace,
                           size_t ws_bytes, void *stream);

/*
 * tp_mlp_shard_bwd_dact_prologue -- the same backward ([P1] §三 3.4; the
 * SwiGLU MLP of §七) with the activation derivative at the other place a
 * backward GEMM can hold it: dH = dY B_i^T is written plainly, and the
 * GEMMs that consume dZ (dA = X^T dZ and dX_partial = dZ A_i^T) form each
 * piece of dZ (GeLU: dH * gelu'(Z); SwiGLU: [dH * U * silu'(G) | dH *
 * silu(G)]) from dH and Z_save while they load it, before the MFMAs use
 * it.  Every tile that reads a piece forms it again: each element's
 * derivative is computed H / 256 times in each of the two GEMMs (bf16
 * tiles; H / 64 for fp32) instead of once.  It exists to be measured against
 * tp_mlp_shard_bwd, whose placement (in the epilogue of dY B_i^T) is the
 * default.
 *   Arguments, layouts, ownership and errors as tp_mlp_shard_bwd, except:
 *   workspace, ws_bytes    at least N*F_shard elements of the dtype
 *                   (tp_mlp_shard_bwd_workspace(desc) bytes are enough);
 *                   on return it holds dH = dY B_i^T, row-major [N,F_shard]
 * Results agree with tp_mlp_shard_bwd's up to rounding (dZ is formed from
 * the stored dH here, from dH's fp32 sums there), not bit for bit.
 */
int tp_mlp_shard_bwd_dact_prologue(const tp_mlp_desc *desc, const void *X, const void *A,
                                   const void *A_up, const void *B, const void *Z_save,
                                   const void *H_act, const void *dY, void *dX_partial,
                                   float *dA, float *dA_up, float *dB, void *workspace,
                                   size_t ws_bytes, void *stream);
int tp_grouped_expert_bwd_accum(const tp_expert_desc *desc, const int64_t *offsets,
                                const void *X_perm, const void *Wg, const void *Wu,
                                const void *Wd, const void *Z_save,
                                const void *H_act, const void *dY_perm,
                                void *dX_perm, float *dWg, float *dWu, float *dWd,
                                void *workspace, size_t ws_bytes, void *stream);

/*
 * Grouped experts with the row offsets in device memory (the expert compute
 * that follows dispatch in "Megatron Core 带读" §09, taking the per-expert
 * row offsets where a routing step on the GPU leaves them: no copy to the
 * host and no wait for it, so routing and expert compute can be queued, or
 * captured in a graph, in one go).  The same computation as
 * tp_grouped_expert_fwd / _bwd / _bwd_accum, except:
 *   R        HOST value: the rows the buffers hold (X_perm, Z_save, H_act,
 *            Y_perm, dY_perm, dX_perm are [R, ...]); 0 <= R <= 2^30
 *   offsets  DEVICE array of E+1 int32, 4-byte aligned, read by the kernels
 *            when they run (stream order: an earlier kernel on `stream` may
 *            write them).  Valid offsets are as for the host calls with
 *            offsets[E] <= R.  Any values are safe: the kernels take
 *            o[0] = clamp(offsets[0], 0, R) and o[e+1] = clamp(offsets[e+1],
 *            o[e], R), so expert e owns rows [o[e], o[e+1]) and no access
 *            leaves the buffers; rows outside [o[0], o[E]) of every output
 *            are left unwritten.
 *   workspace  tp_grouped_expert_devoff_workspace(desc, R) bytes ([R,2F] bf16)
 *   accumulate 0: weight gradients written (tp_grouped_expert_bwd);
 *            1: added to (tp_grouped_expert_bwd_accum)
 * The host cannot see the rows, so the row-tiled products cover the worst
 * split of R rows (E - 1 more tile rows than R rows need at most):
 * workgroups without a tile exit at once, and where that worst case
 * exceeds three waves over the compute units the launch instead loops over
 * its tiles on one workgroup per compute unit.  The kernels make the host
 * calls' choice among 256-row tiles, 256-row tiles with 32-row remainder
 * tiles and 128-row tiles from the offsets themselves (not the 224-wide
 * tiles; 128-row tiles only where their grid fits one wave or the launch
 * loops): results equal the host-offset calls' bit for bit where both take
 * the same tiling, and otherwise up to summation order; they are
 * bit-identical run to run.
 * Errors: as the host-offset calls (the offsets' values are not checked).
 */
int tp_grouped_expert_fwd_devoff(const tp_expert_desc *desc, int64_t R,
                                 const int32_t *offsets, const void *X_perm,
                                 const void *Wg, const void *Wu, const void *Wd,
                                 void *Z_save, void *H_act, void *Y_perm, void *stream);
size_t tp_grouped_expert_devoff_workspace(const tp_expert_desc *desc, int64_t R);
int tp_grouped_expert_bwd_devoff(const tp_expert_desc *desc, int64_t R,
                                 const int32_t *offsets, const void *X_perm,
                                 const void *Wg, const void *Wu, const void *Wd,
                                 const void *Z_save, const void *H_act,
                                 const void *dY_perm, void *dX_perm, float *dWg,
                                 float *dWu, float *dWd, void *workspace,
                                 size_t ws_bytes, int32_t accumulate, void *stream);

/*
 * MoE token dispatch and combine around the grouped local experts
 * ([P3] §09: router scores -> top-k experts -> tokens sent to their
 * experts -> expert compute -> results merged by weight -> back in the
 * original token order).  The router is not part of this library: its
 * decisions arrive as device tables for the R expert-sorted rows (rows of
 * expert e are offsets[e] .. offsets[e+1]-1, the grouped calls' layout):
 *   row_token  [R] int32   the token of row r
 *   row_weight [R] fp32    the router weight of (row_token[r], expert of r)
 *   tok_ptr    [N+1] int32, tok_rows [R] int32   the rows of token t are
 *              tok_rows[tok_ptr[t] .. tok_ptr[t+1]-1] (CSR), in the order
 *              their contributions are summed
 * Tables need 4-byte alignment, data buffers 16 bytes.  A table entry out
 * of range contributes nothing (a permuted row becomes zeros; in the
 * combine backward its dY_perm row and d_weight are zeros, and its Y_perm
 * row is not read); no entry can make an access leave its buffer.  dtype is TP_BF16 or TP_F32; H a
 * multiple of 8 (bf16) or 4 (fp32).  All three are HBM-bound row moves.
 *
 * tp_moe_permute: X_perm[r, :] = X[row_token[r], :]   (X [N,H], X_perm [R,H])
 * tp_moe_combine: Y[t, :] = sum over the rows r of token t of
 *                 row_weight[r] * Y_perm[r, :], in fp32, rounded once; a
 *                 token without rows gets zeros.  row_weight = NULL means
 *                 weight 1: that is also the backward of tp_moe_permute
 *                 (dX[t] = sum of dX_perm over the rows of t).
 * tp_moe_combine_bwd: the backward of tp_moe_combine:
 *                 dY_perm[r, :] = row_weight[r] * dY[row_token[r], :]  [R,H]
 *                 d_weight[r]   = sum_h dY[row_token[r], h] * Y_perm[r, h]
 *                 (fp32, a fixed reduction order: deterministic)
 */
int tp_moe_permute(int32_t dtype, int64_t N, int64_t H, int64_t R, const int32_t *row_token,
                   const void *X, void *X_perm, void *stream);
int tp_moe_combine(int32_t dtype, int64_t N, int64_t H, int64_t R, const int32_t *tok_ptr,
                   const int32_t *tok_rows, const float *row_weight, const void *Y_perm,
                   void *Y, void *stream);
int tp_moe_combine_bwd(int32_t dtype, int64_t N, int64_t H, int64_t R,
                       const int32_t *row_token, const float *row_weight, const void *dY,
                       const void *Y_perm, void *dY_perm, float *d_weight, void *stream);

/*
 * FP8 ([P1] §8.2: E4M3 forward, E5M2 backward, per-tensor scaling from
 * amax; [P3] §10: quantize by scale/amax -> FP8 kernel -> dequantize).
 * Codes are the OCP 8-bit formats: E4M3 (largest finite 448) and E5M2
 * (57344).
 *
 * tp_fp8_quantize: q = code(clamp(x * scale, -max, max)), round to nearest
 *   even, the product taken in fp32; amax (if not NULL) is raised to
 *   max |x| (an atomic max: the caller sets it, e.g. to 0, beforehand).
 *   fmt        TP_FP8_E4M3 or TP_FP8_E5M2
 *   transpose  0: q [rows,cols];  1: q [cols,rows] (= the code of x^T),
 *              rows a multiple of 16
 *   x          bf16 [rows,cols], cols a multiple of 8
 *   scale      device float (1 value)
 *
 * tp_mlp_shard_fwd_fp8: one shard's forward on E4M3 operands, fp32
 * accumulate, bf16 activations (desc->dtype must be TP_BF16; H and F_shard
 * multiples of 128):
 *   Xq [N,H]; Aq_t, Auq_t [F_shard,H] and Bq_t [H,F_shard]: the codes of
 *       A^T, A_up^T, B^T (tp_fp8_quantize with transpose = 1), so every
 *       GEMM operand is K-contiguous; Auq_t NULL for GeLU
 *   scales  device float[5]: x_inv, a_inv, au_inv, b_inv (the inverses of
 *       the scales the codes were made with) and h_scale (the scale H is
 *       quantized with, e.g. from the amax history)
 *   FC1 sums are multiplied by fp32(x_inv * a_inv) (up projection:
 *       x_inv * au_inv); the activation gives H, stored as bf16 in H_act
 *       (and Z_save as in tp_mlp_shard_fwd) and as the E4M3 codes of
 *       H * h_scale in H_q [N,F_shard]; *h_amax is set to max |H|
 *   FC2: Y_partial (bf16) = (H_q B^T codes) * fp32(fp32(1 / h_scale) * b_inv)
 */
#define TP_FP8_E4M3 0
#define TP_FP8_E5M2 1
int tp_fp8_quantize(int32_t fmt, int32_t transpose, int64_t rows, int64_t cols, const void *x,
                    const float *scale, void *q, float *amax, void *stream);
int tp_mlp_shard_fwd_fp8(const tp_mlp_desc *desc, const void *Xq, const void *Aq_t,
                         const void *Auq_t, const void *Bq_t, const float *scales,
                         void *Z_save, void *H_act, void *H_q, float *h_amax, void *Y_partial,
                         void *stream);

/*
 * tp_fp8_transpose: q_t [cols,rows] = q [rows,cols] for 1-byte codes (rows
 * and cols multiples of 16): the K-contiguous copies the weight-gradient
 * GEMMs of the FP8 backward need (codes of H and dY).
 *
 * tp_mlp_shard_bwd_fp8: one shard's backward on FP8 codes: gradients E5M2,
 * weights and activations E4M3 ([P1] §8.2), fp32 accumulate.  N, H and
 * F_shard multiples of 128, N at most 2^22; desc->dtype TP_BF16.  Codes
 * (1 byte each):
 *   dYq [N,H], dYq_t [H,N]   dY's E5M2 codes and their transpose
 *   Xq_t [H,N], Hq_t [F_shard,N]   transposed E4M3 codes of X and H (the
 *                            forward's H_q, transposed)
 *   Aq, Auq [H,F_shard], Bq [F_shard,H]   the weights' E4M3 codes in their
 *                            own layout (Auq NULL for GeLU)
 *   Z_save    the forward's bf16 Z (SwiGLU: G|U)
 *   scales    device float[7]: dy_inv, b_inv, h_inv, x_inv, a_inv (one
 *             scale for the fused [A | A_up] weight), dz_scale, dz_inv
 *             (= 1 / dz_scale)
 * Outputs: dX_partial (bf16), dA, dA_up, dB (fp32); workspace dZq [N,zw]
 * and dZq_t [zw,N] (zw = F_shard, SwiGLU 2 F_shard) receive the E5M2 codes
 * of dZ * dz_scale; *dz_amax is set to max |dZ|.
 *   dZ  = act'(Z) * (dYq Bq^T codes) * fp32(dy_inv b_inv)
 *   dB  = (Hq_t dYq_t^T codes) * fp32(h_inv dy_inv)
 *   dA  = (Xq_t dZq_t^T codes) * fp32(x_inv dz_inv)   (| dA_up)
 *   dX  = (dZq [Aq|Auq]^T codes) * fp32(dz_inv a_inv)
 */
int tp_fp8_transpose(int64_t rows, int64_t cols, const void *q, void *q_t, void *stream);

/*
 * tp_fp8_scale_update -- delayed per-tensor scaling ([P1] §8.2: each
 * tensor's scale comes from the history of its amax; [P3] §10: scale from
 * amax, then quantize).  For each of n tensors of one format, in device
 * memory (fp32, 4-byte aligned, none overlapping another):
 *   history [n,len]   row t: tensor t's last len amax values, newest first
 *   amax [n]          this step's amax (as tp_fp8_quantize and the FP8
 *                     shard calls leave it); in/out
 *   scale [n]         the scale of the next quantization; in/out
 *   scale_inv [n]     1 / scale (NULL: not written)
 * The call shifts each row one place (its oldest value drops out), stores
 * amax[t] in front and sets amax[t] = 0 for the next step's atomic max.
 * With m the largest finite positive value of the row (the new amax
 * included), scale[t] = (fmax / m) * 2^-margin, fmax = 448 (E4M3) or 57344
 * (E5M2): a tensor whose |x| <= m then quantizes without saturating.  With
 * no such value (zeros, NaN, inf only) scale[t] is kept.  Each step is one
 * correctly rounded fp32 operation.  scale_inv[t] = 1 / scale[t].
 *   fmt TP_FP8_E4M3 or TP_FP8_E5M2; 0 <= n <= 2^24; 1 <= len <= 1024;
 *   0 <= margin <= 16.  Nothing is allocated; no memset (capturable).
 * Errors: TP_ERR_DTYPE (fmt), TP_ERR_SHAPE (n, len, margin), TP_ERR_NULL
 * (history, amax or scale NULL with n > 0), TP_ERR_ALIGN (not 4-byte
 * aligned), TP_ERR_ALIAS (two of the buffers overlap), TP_ERR_DEVICE,
 * TP_ERR_HIP (launch); nothing is enqueued on an error.
 */
int tp_fp8_scale_update(int32_t fmt, int32_t n, int32_t len, float *history, float *amax,
                        float *scale, float *scale_inv, int32_t margin, void *stream);
int tp_mlp_shard_bwd_fp8(const tp_mlp_desc *desc, const void *dYq, const void *dYq_t,
                         const void *Xq_t, const void *Hq_t, const void *Aq, const void *Auq,
                         const void *Bq, const void *Z_save, const float *scales,
                         void *dX_partial, float *dA, float *dA_up, float *dB, void *dZq,
                         void *dZq_t, float *dz_amax, void *stream);

/* Message of the last failed call on this thread ("" if none; a
 * successful call clears it).  The pointer stays valid until this thread's
 * next call into the library. */
const char *tp_last_error(void);

/* Fixed name of a tp_status value. */
const char *tp_status_string(int status);

/*
 * Launch timing (a measurement aid, not a step of the method): the GPU
 * time of each product the calls enqueue, taken with the caller's HIP
 * events on the stream each product runs on.
 * tp_launch_events hands this thread's subsequent calls `count` hipEvent_t
 * handles (created by the caller with timing enabled; they must stay valid
 * while set).  The j-th timed unit records events[2j] on its stream just
 * before its kernels and events[2j+1] just after, so
 * hipEventElapsedTime(events[2j], events[2j+1]) is that unit's time.  A unit
 * is one product of the path: one GEMM with its fused epilogue (a GEMM
 * over ragged rows may be more than one kernel), one partial sum, one
 * quantization, transpose or MoE row move.  Units past the last pair run
 * untimed.  A new call replaces the set and restarts the count; count 0
 * (events may then be NULL) stops the timing.  count must be even and at
 * most TP_MAX_LAUNCH_EVENTS, every handle non-NULL.  Touches no GPU state.
 * tp_launch_events_used: events recorded on this thread since the last
 * tp_launch_events call (twice the number of timed units).
 */
#define TP_MAX_LAUNCH_EVENTS 4096
int tp_launch_events(void *const *events, int32_t count);
int32_t tp_launch_events_used(void);

#ifdef __cplusplus
}
#endif

#endif /* TPMLP_H */
