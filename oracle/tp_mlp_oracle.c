/*
 * fp64 CPU oracle of one tensor-parallel rank's share of the paired
 * ColumnParallelLinear -> activation -> RowParallelLinear MLP.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library
 * shares no code, header or constant with it.
 *
 * Everything here is the plain definition, in double precision, with
 * straightforward loop nests (OpenMP splits independent output rows only;
 * every output element is one sequential sum in index order):
 *
 *   Column split (Megatron-LM 源码精读——大模型并行训练全景, §三 3.1):
 *     the shard A_i holds a block of output columns; Z_i = X A_i needs no
 *     communication because X is replicated, and the input gradient is
 *     the sum over shards of dZ_i A_i^T.
 *   Row split (same page, §三 3.2): B_i holds a block of input rows; the
 *     shard's output Y_i = H_i B_i is a partial of the full output, which
 *     the forward all-reduce sums over shards.
 *   Pairing (same page, §三 3.3 diagram): X -> column shard -> GeLU ->
 *     row shard -> sum; so the activation acts on a shard-local slice.
 *   SwiGLU (same page, §七, "three matrices"): gate and up projections
 *     share the input; H = silu(X Ag) * (X Au); down projection as above.
 *
 * The activation formulas are not printed on the pages.  GeLU uses the
 * tanh form of Hendrycks & Gimpel (2016); SwiGLU uses silu on the gate
 * branch as in Shazeer (2020), "GLU Variants Improve Transformer".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_ACT_GELU_TANH 0
#define ORC_ACT_SWIGLU 1
#define ORC_ACT_IDENTITY 99 /* test-only: lets a test compare the GEMM loops
                               against a library matmul */

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* activations                                                         */
/* ------------------------------------------------------------------ */

/* sqrt(2/pi) and the cubic coefficient of the tanh approximation. */
static const double GELU_C = 0.7978845608028654;
static const double GELU_K = 0.044715;

double orc_gelu_tanh(double z) {
    double u = GELU_C * (z + GELU_K * z * z * z);
    return 0.5 * z * (1.0 + tanh(u));
}

/* d/dz of orc_gelu_tanh. */
double orc_gelu_tanh_grad(double z) {
    double u = GELU_C * (z + GELU_K * z * z * z);
    double t = tanh(u);
    double du = GELU_C * (1.0 + 3.0 * GELU_K * z * z);
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * du;
}

double orc_sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }

double orc_silu(double g) { return g * orc_sigmoid(g); }

/* d/dg of g*sigmoid(g) = s + g*s*(1-s) */
double orc_silu_grad(double g) {
    double s = orc_sigmoid(g);
    return s * (1.0 + g * (1.0 - s));
}

/* ------------------------------------------------------------------ */
/* matrix products (row-major, fp64)                                   */
/* ------------------------------------------------------------------ */

/* C[M,N] = A[M,K] * B[K,N] */
static void mm_nn(int64_t M, int64_t N, int64_t K, const double *A,
                  const double *B, double *C) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double *c = C + i * N;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = A[i * K + k];
            const double *b = B + k * N;
            for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
        }
    }
}

/* C[M,N] = A[M,K] * Bs^T, with Bs stored [N,K] */
static void mm_nt(int64_t M, int64_t N, int64_t K, const double *A,
                  const double *Bs, double *C) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const double *a = A + i * K;
        for (int64_t j = 0; j < N; ++j) {
            const double *b = Bs + j * K;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += a[k] * b[k];
            C[i * N + j] = s;
        }
    }
}

/* C[M,N] = As^T * B, with As stored [K,M] and B stored [K,N] */
static void mm_tn(int64_t M, int64_t N, int64_t K, const double *As,
                  const double *B, double *C) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double *c = C + i * N;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = As[k * M + i];
            const double *b = B + k * N;
            for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
        }
    }
}

/* exposed for the library-matmul pin */
void orc_matmul_nn(int64_t M, int64_t N, int64_t K, const double *A,
                   const double *B, double *C) { mm_nn(M, N, K, A, B, C); }
void orc_matmul_nt(int64_t M, int64_t N, int64_t K, const double *A,
                   const double *Bs, double *C) { mm_nt(M, N, K, A, Bs, C); }
void orc_matmul_tn(int64_t M, int64_t N, int64_t K, const double *As,
                   const double *B, double *C) { mm_tn(M, N, K, As, B, C); }

/* ------------------------------------------------------------------ */
/* one shard: forward                                                  */
/* ------------------------------------------------------------------ */

/*
 * X [N,H], A [H,Ft], Aup [H,Ft] (SwiGLU only), B [Ft,H].
 * Outputs: Z [N,Ft] (pre-activation; the gate projection G for SwiGLU),
 *          U [N,Ft] (SwiGLU up projection, else unused),
 *          Hact [N,Ft], Y [N,H] (this shard's partial output).
 * Returns 0, or -1 on a bad argument.
 */
int orc_mlp_fwd(int64_t N, int64_t H, int64_t Ft, int act, const double *X,
                const double *A, const double *Aup, const double *B,
                double *Z, double *U, double *Hact, double *Y) {
    if (N < 0 || H <= 0 || Ft <= 0) return -1;
    if (act == ORC_ACT_SWIGLU && (!Aup || !U)) return -1;
    mm_nn(N, Ft, H, X, A, Z);
    if (act == ORC_ACT_SWIGLU) mm_nn(N, Ft, H, X, Aup, U);
    for (int64_t e = 0; e < N * Ft; ++e) {
        double z = Z[e];
        if (act == ORC_ACT_GELU_TANH)
            Hact[e] = orc_gelu_tanh(z);
        else if (act == ORC_ACT_SWIGLU)
            Hact[e] = orc_silu(z) * U[e];
        else if (act == ORC_ACT_IDENTITY)
            Hact[e] = z;
        else
            return -1;
    }
    mm_nn(N, H, Ft, Hact, B, Y);
    return 0;
}

/* ------------------------------------------------------------------ */
/* one shard: backward                                                 */
/* ------------------------------------------------------------------ */

/*
 * Inputs: the forward's inputs, its saved Z (G), U and Hact, and the full
 * output gradient dY [N,H] (the forward all-reduce's backward is the
 * identity, so every shard receives the whole dY: same page, §三 3.4).
 * Outputs: dX [N,H] (this shard's partial input gradient; the sum over
 * shards is the input gradient), dA [H,Ft], dAup [H,Ft] (SwiGLU),
 * dB [Ft,H]; optionally dZ [N,Ft] and dU [N,Ft] (may be NULL).
 */
int orc_mlp_bwd(int64_t N, int64_t H, int64_t Ft, int act, const double *X,
                const double *A, const double *Aup, const double *B,
                const double *Z, const double *U, const double *Hact,
                const double *dY, double *dX, double *dA, double *dAup,
                double *dB, double *dZ_out, double *dU_out) {
    if (N < 0 || H <= 0 || Ft <= 0) return -1;
    int swiglu = (act == ORC_ACT_SWIGLU);
    if (swiglu && (!Aup || !U || !dAup)) return -1;
    if (act != ORC_ACT_GELU_TANH && !swiglu && act != ORC_ACT_IDENTITY)
        return -1;
    size_t nf = (size_t)(N * Ft);
    double *dH = (double *)malloc((nf ? nf : 1) * sizeof(double));
    double *dZ = (double *)malloc((nf ? nf : 1) * sizeof(double));
    double *dU = swiglu ? (double *)malloc((nf ? nf : 1) * sizeof(double)) : NULL;
    if (!dH || !dZ || (swiglu && !dU)) {
        free(dH); free(dZ); free(dU);
        return -2;
    }
    /* row-parallel linear: weight gradient stays local, input grad dH */
    mm_tn(Ft, H, N, Hact, dY, dB);
    mm_nt(N, Ft, H, dY, B, dH);
    /* activation derivative */
    for (size_t e = 0; e < nf; ++e) {
        if (act == ORC_ACT_GELU_TANH) {
            dZ[e] = dH[e] * orc_gelu_tanh_grad(Z[e]);
        } else if (swiglu) {
            double g = Z[e];
            dZ[e] = dH[e] * U[e] * orc_silu_grad(g);
            dU[e] = dH[e] * orc_silu(g);
        } else {
            dZ[e] = dH[e];
        }
    }
    /* column-parallel linear: weight gradient and partial input gradient */
    mm_tn(H, Ft, N, X, dZ, dA);
    mm_nt(N, H, Ft, dZ, A, dX);
    if (swiglu) {
        mm_tn(H, Ft, N, X, dU, dAup);
        double *dX2 = (double *)malloc((size_t)(N * H ? N * H : 1) * sizeof(double));
        if (!dX2) { free(dH); free(dZ); free(dU); return -2; }
        mm_nt(N, H, Ft, dU, Aup, dX2);
        for (int64_t e = 0; e < N * H; ++e) dX[e] += dX2[e];
        free(dX2);
    }
    if (dZ_out) memcpy(dZ_out, dZ, nf * sizeof(double));
    if (dU_out && swiglu) memcpy(dU_out, dU, nf * sizeof(double));
    free(dH); free(dZ); free(dU);
    return 0;
}

/* ------------------------------------------------------------------ */
/* partial-output sum                                                   */
/* ------------------------------------------------------------------ */

/* out[j] = sum_{i=0}^{T-1} parts[i][j]: the arithmetic of the all-reduce
 * that merges row-parallel partial outputs (same page, §三 3.2/3.3). */
int orc_partial_sum(int T, int64_t count, const double *const *parts,
                    double *out) {
    if (T < 1 || count < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < count; ++j) {
        double s = 0.0;
        for (int i = 0; i < T; ++i) s += parts[i][j];
        out[j] = s;
    }
    return 0;
}
