/*
 * oracle_checks.c -- the fp64 oracle run on small inputs under AddressSanitizer and
 * UndefinedBehaviorSanitizer: forward, carried state, gradients, causal convolution,
 * and every refusal path.  Test infrastructure only.  Exits 0 when the calls return
 * the expected statuses (values are pinned elsewhere, by the Python pin tests).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_selective_scan_fwd(int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*,
                              const double*, const double*, const double*, const double*, const double*, double*, int);
int oracle_selective_scan_state(int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*,
                                const double*, const double*, const double*, const double*, const double*,
                                const double*, double*, double*, int);
int oracle_selective_scan_bwd(int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*,
                              const double*, const double*, const double*, const double*, const double*, const double*,
                              const double*, const double*, double*, double*, double*, double*, double*, double*,
                              double*, double*, double*, int);
int oracle_causal_conv1d(int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*,
                         const double*, int, double*, double*);

static int failed = 0;
#define EXPECT(cond) do { if (!(cond)) { fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); ++failed; } } while (0)

static double* filled(size_t n, double scale, double shift) {
    double* p = (double*)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = shift + scale * sin(0.37 * (double)i + 0.1);
    return p;
}

int main(void) {
    const int64_t B = 2, L = 37, D = 5, N = 6, K = 4;
    const size_t nel = B * D * L, nbc = B * N * L, nh = B * D * N;
    double *u = filled(nel, 1.0, 0.0), *dl = filled(nel, 1.0, -2.0), *z = filled(nel, 2.0, 0.0);
    double *Bm = filled(nbc, 1.0, 0.0), *Cm = filled(nbc, 1.0, 0.0), *A = filled(D * N, 0.5, -1.0);
    double *Dk = filled(D, 1.0, 0.0), *bias = filled(D, 0.5, -1.0), *h0 = filled(nh, 1.0, 0.0);
    double *y = calloc(nel, sizeof(double)), *hl = calloc(nh, sizeof(double)), *dy = filled(nel, 1.0, 0.0);
    double *dhl = filled(nh, 1.0, 0.0);
    double *du = calloc(nel, 8), *dd = calloc(nel, 8), *dA = calloc(D * N, 8), *dB = calloc(nbc, 8),
           *dC = calloc(nbc, 8), *dD = calloc(D, 8), *dz = calloc(nel, 8), *db = calloc(D, 8), *dh0 = calloc(nh, 8);
    double *w = filled(D * K, 0.5, 0.0), *cb = filled(D, 0.1, 0.0), *cst = filled(B * D * (K - 1), 1.0, 0.0);
    double *cout = calloc(nel, 8), *cso = calloc(B * D * (K - 1), 8);

    EXPECT(oracle_selective_scan_fwd(B, L, D, N, u, dl, A, Bm, Cm, Dk, z, bias, y, 2) == 0);
    EXPECT(oracle_selective_scan_fwd(B, L, D, N, u, dl, A, Bm, Cm, NULL, NULL, NULL, y, 1) == 0);
    EXPECT(oracle_selective_scan_state(B, L, D, N, u, dl, A, Bm, Cm, Dk, z, bias, h0, y, hl, 0) == 0);
    EXPECT(oracle_selective_scan_bwd(B, L, D, N, u, dl, A, Bm, Cm, Dk, z, bias, h0, dy, dhl, du, dd, dA, dB, dC, dD, dz,
                                     db, dh0, 2) == 0);
    EXPECT(oracle_selective_scan_bwd(B, L, D, N, u, dl, A, Bm, Cm, NULL, NULL, NULL, NULL, dy, NULL, du, dd, dA, dB, dC,
                                     NULL, NULL, db, dh0, 1) == 0);
    EXPECT(oracle_causal_conv1d(B, L, D, K, u, w, cb, cst, 1, cout, cso) == 0);
    EXPECT(oracle_causal_conv1d(B, L, D, 1, u, w, NULL, NULL, 0, cout, NULL) == 0);
    /* refusals: empty, NULL, non-finite, A > 0 */
    EXPECT(oracle_selective_scan_fwd(B, 0, D, N, u, dl, A, Bm, Cm, Dk, z, bias, y, 1) < 0);
    EXPECT(oracle_selective_scan_fwd(B, L, D, N, NULL, dl, A, Bm, Cm, Dk, z, bias, y, 1) < 0);
    u[7] = NAN;
    EXPECT(oracle_selective_scan_fwd(B, L, D, N, u, dl, A, Bm, Cm, Dk, z, bias, y, 1) < 0);
    u[7] = 0.5;
    A[3] = 0.25;
    EXPECT(oracle_selective_scan_fwd(B, L, D, N, u, dl, A, Bm, Cm, Dk, z, bias, y, 1) < 0);
    EXPECT(oracle_selective_scan_bwd(B, L, D, N, u, dl, A, Bm, Cm, Dk, z, bias, h0, dy, dhl, du, dd, dA, dB, dC, dD, dz,
                                     db, dh0, 1) < 0);
    printf("oracle checks: %d failed\n", failed);
    return failed ? 1 : 0;
}
