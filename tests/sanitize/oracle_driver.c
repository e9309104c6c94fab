/* Exercises every entry of the fp64 oracle (oracle/tp_mlp_oracle.c) on
 * small and degenerate shapes, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: any out-of-bounds access, use of freed
 * memory, signed overflow or misaligned access in the loop nests or in
 * the table walks aborts the run.  A few results are also checked against
 * direct sums written here, so the run is not vacuous.  Prints "OK". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int orc_mlp_fwd(int64_t N, int64_t H, int64_t Ft, int act, const double *X, const double *A,
                const double *Aup, const double *B, double *Z, double *U, double *Hact,
                double *Y);
int orc_mlp_bwd(int64_t N, int64_t H, int64_t Ft, int act, const double *X, const double *A,
                const double *Aup, const double *B, const double *Z, const double *U,
                const double *Hact, const double *dY, double *dX, double *dA, double *dAup,
                double *dB, double *dZ_out, double *dU_out);
int orc_partial_sum(int T, int64_t count, const double *const *parts, double *out);
void orc_matmul_nn(int64_t M, int64_t N, int64_t K, const double *A, const double *B, double *C);
void orc_matmul_nt(int64_t M, int64_t N, int64_t K, const double *A, const double *B, double *C);
void orc_matmul_tn(int64_t M, int64_t N, int64_t K, const double *A, const double *B, double *C);

static uint64_t st = 88172645463325252ull;
static double rnd(void) { /* xorshift64, uniform in [-1, 1) */
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return (double)(st >> 11) / 4503599627370496.0 - 1.0;
}
/* exactly-sized heap buffers, so any overrun is reported */
static double *buf(int64_t n) {
    double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!p) exit(3);
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}

static int fails = 0;
static void expect(int ok, const char *what) {
    if (!ok) { fprintf(stderr, "FAIL %s\n", what); ++fails; }
}

static void run_case(int64_t N, int64_t H, int64_t Ft, int act) {
    const int sw = act == 1;
    double *X = buf(N * H), *A = buf(H * Ft), *Au = sw ? buf(H * Ft) : NULL, *B = buf(Ft * H);
    double *Z = buf(N * Ft), *U = sw ? buf(N * Ft) : NULL, *Hh = buf(N * Ft), *Y = buf(N * H);
    double *dY = buf(N * H), *dX = buf(N * H), *dA = buf(H * Ft), *dAu = sw ? buf(H * Ft) : NULL;
    double *dB = buf(Ft * H), *dZ = buf(N * Ft), *dU = sw ? buf(N * Ft) : NULL;
    expect(orc_mlp_fwd(N, H, Ft, act, X, A, Au, B, Z, U, Hh, Y) == 0, "fwd rc");
    expect(orc_mlp_bwd(N, H, Ft, act, X, A, Au, B, Z, U, Hh, dY, dX, dA, dAu, dB, dZ, dU) == 0,
           "bwd rc");
    /* spot checks against direct sums: Z[n,f] = sum_h X[n,h] A[h,f] and
     * dB[f,h] = sum_n H[n,f] dY[n,h] (zero for N = 0) */
    if (N > 0) {
        int64_t n = N - 1, f = Ft / 2;
        double z = 0.0;
        for (int64_t h = 0; h < H; ++h) z += X[n * H + h] * A[h * Ft + f];
        expect(fabs(z - Z[n * Ft + f]) <= 1e-12 * (1.0 + fabs(z)), "Z entry");
    }
    {
        int64_t f = Ft - 1, h = H / 3;
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n) s += Hh[n * Ft + f] * dY[n * H + h];
        expect(fabs(s - dB[f * H + h]) <= 1e-12 * (1.0 + fabs(s)), "dB entry");
    }
    free(X); free(A); free(Au); free(B); free(Z); free(U); free(Hh); free(Y);
    free(dY); free(dX); free(dA); free(dAu); free(dB); free(dZ); free(dU);
}

int main(void) {
    const int64_t shapes[][3] = {{0, 8, 8}, {1, 8, 8}, {7, 16, 24}, {33, 8, 40}, {5, 64, 4}};
    for (int s = 0; s < 5; ++s)
        for (int act = 0; act < 2; ++act) run_case(shapes[s][0], shapes[s][1], shapes[s][2], act);
    /* rejected arguments return without touching the buffers */
    expect(orc_mlp_fwd(-1, 8, 8, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == -1,
           "negative N");
    expect(orc_mlp_fwd(4, 8, 8, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == -1,
           "SwiGLU without A_up");
    /* partial sums: T = 1 copies, T = 64 over a ragged count, count = 0 */
    for (int T = 1; T <= 64; T += 63) {
        const int64_t count = 1001;
        double **parts = (double **)malloc((size_t)T * sizeof(double *));
        for (int i = 0; i < T; ++i) parts[i] = buf(count);
        double *out = buf(count);
        expect(orc_partial_sum(T, count, (const double *const *)parts, out) == 0, "psum rc");
        double s = 0.0;
        for (int i = 0; i < T; ++i) s += parts[i][count - 1];
        expect(out[count - 1] == s, "psum last element");
        expect(orc_partial_sum(T, 0, (const double *const *)parts, out) == 0, "psum empty");
        for (int i = 0; i < T; ++i) free(parts[i]);
        free(parts); free(out);
    }
    expect(orc_partial_sum(0, 4, NULL, NULL) == -1, "psum T = 0");
    /* the product loops on non-square shapes */
    {
        double *a = buf(3 * 5), *b = buf(5 * 7), *c = buf(3 * 7), *bt = buf(7 * 5), *at = buf(5 * 3);
        orc_matmul_nn(3, 7, 5, a, b, c);
        orc_matmul_nt(3, 7, 5, a, bt, c);
        orc_matmul_tn(3, 7, 5, at, b, c);
        free(a); free(b); free(c); free(bt); free(at);
    }
    if (fails) return 1;
    printf("OK\n");
    return 0;
}
