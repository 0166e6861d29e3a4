/*
 * oracle.c -- plain fp64 CPU reference of the Mamba-1 selective-scan forward pass.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load or call this library.  It shares
 * no source, header, table or helper with the HIP implementation.
 *
 * It is written to be read against the pages, not to be fast: one sequential
 * recurrence per (batch, channel) row, every quantity in double precision, no
 * blocking, no reordering.  Rows are independent, so an OpenMP loop hands whole
 * rows to threads; nothing inside a row is parallel.
 *
 * Pages cited (titles as they appear on the pages):
 *   [QA]  yo3nglau.github.io  "Mamba 与状态空间模型：面试问题与推荐回答"
 *   [GH]  gheillcoat.github.io "Mamba (状态空间模型)"
 *   [GS]  gongshangzheng.github.io "Mamba"
 *   [QT]  qubittool.com "Mamba 与状态空间模型：机制、演进与工程选型"
 *   [CB]  cnblogs.com "Mamba3 技术浅析"
 *
 * Parity pins: every function below is pinned by tests that do not reuse this
 * code (tests/test_oracle_pins.py): the worked scalar example printed on [QT],
 * the LTI convolution identity, the semiseparable sum of [CB] §2.2.2, the A = 0
 * prefix sum, the constant-input geometric series and structural invariants.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_NULL (-1)
#define OR_ERR_EMPTY (-2)
#define OR_ERR_NONFINITE (-3)
#define OR_ERR_RETAIN (-4)
#define OR_ERR_ALLOC (-5)

/* softplus(x) = log(1 + e^x), written as max(x,0) + log1p(e^-|x|) so that it
 * neither overflows for large x nor loses the small result for very negative x.
 * The step size is the softplus of a projection: [QA] Q4, [GH] "Mamba 的关键创新：
 * 选择性扫描", [GS] §2.1, [QT] "Mamba 增加了内容相关的选择机制". */
double oracle_softplus(double x)
{
    double m = x > 0.0 ? x : 0.0;
    return m + log1p(exp(-fabs(x)));
}

/* SiLU(x) = x * sigmoid(x): the gate of the block's second branch ([GS] §3.1). */
double oracle_silu(double x)
{
    return x / (1.0 + exp(-x));
}

static int all_finite(const double* p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

/*
 * The scalar retain / write / read recurrence of [QT] "一个可运行的标量模型":
 *   state_0 = 0,  state_i = retain_i * state_{i-1} + write_i * value_i,
 *   out_i   = read_i * state_i          (read after the update).
 * Inputs are checked before any state is formed, as on that page: an empty
 * sequence, any non-finite field, or a retain factor outside [0, 1] is refused.
 */
int oracle_selective_recurrence(int64_t n, const double* value, const double* retain,
                                const double* write, const double* read, double* out)
{
    if (n <= 0) return OR_ERR_EMPTY;
    if (!value || !retain || !write || !read || !out) return OR_ERR_NULL;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(value[i]) || !isfinite(retain[i]) || !isfinite(write[i]) || !isfinite(read[i]))
            return OR_ERR_NONFINITE;
        if (retain[i] < 0.0 || retain[i] > 1.0) return OR_ERR_RETAIN;
    }
    double state = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        state = retain[i] * state + write[i] * value[i];
        out[i] = read[i] * state;
    }
    return OR_OK;
}

/*
 * Selective-scan forward with a carried state, one fp64 recurrence per row (b, d).
 *
 * Layouts (row-major, last index contiguous):
 *   u, delta, z, y : (batch, dim, L)
 *   Bm, Cm         : (batch, N, L)      one B_t, C_t per token, shared by all channels
 *   A              : (dim, N)           fixed diagonal decay per channel
 *   Dskip, dt_bias : (dim,)
 *   h0, h_last     : (batch, dim, N)    state before the first and after the last step
 * Dskip, z and dt_bias may be NULL (no skip, no gate, zero bias); h0 may be NULL (the
 * state starts at zero, as the scalar model on [QT] does) and h_last may be NULL (the
 * final state is not returned).  A state carried from one call into the next is the
 * fixed-size per-token state of recurrent decoding ([QA] Q8 and Q11; [QT] "直接回答").
 *
 * Per row, for t = 0 .. L-1 (all in double):
 *   dt    = softplus(delta[t] + dt_bias[d])                         step size ([QA] Q4/Q5)
 *   h[n]  = exp(dt * A[d,n]) * h[n] + dt * B[t,n] * u[t]            ([QT] selection pseudo-code;
 *           exp(dt*A) is the zero-order-hold decay of a diagonal A  ([QA] Q1, [GH] SSM 基础);
 *           the input term is dt*B*u, the first-order rule [CB] §3.1 ascribes to Mamba-1)
 *   y[t]  = (sum_n C[t,n] * h[n] + Dskip[d] * u[t]) * SiLU(z[t])     (readout after the update,
 *           [QT] scalar model; skip term D*u from the continuous output equation, [QA] Q1;
 *           SiLU gate, [GS] §3.1)
 *
 * Refused before anything is computed: a zero or negative size, a NULL required
 * pointer, any non-finite input, or A[d,n] > 0 (which, with dt > 0, would give a
 * retain factor exp(dt*A) > 1, the case [QT]'s scalar model rejects).
 *
 * nthreads <= 0 lets OpenMP choose.  Returns OR_OK or a negative code.
 */
int oracle_selective_scan_state(int64_t batch, int64_t L, int64_t dim, int64_t N,
                                const double* u, const double* delta, const double* A,
                                const double* Bm, const double* Cm, const double* Dskip,
                                const double* z, const double* dt_bias, const double* h0,
                                double* y, double* h_last, int nthreads)
{
    if (batch <= 0 || L <= 0 || dim <= 0 || N <= 0) return OR_ERR_EMPTY;
    if (!u || !delta || !A || !Bm || !Cm || !y) return OR_ERR_NULL;
    const int64_t nel = batch * dim * L;
    const int64_t nbc = batch * N * L;
    if (!all_finite(u, nel) || !all_finite(delta, nel) || !all_finite(A, dim * N) ||
        !all_finite(Bm, nbc) || !all_finite(Cm, nbc))
        return OR_ERR_NONFINITE;
    if ((Dskip && !all_finite(Dskip, dim)) || (z && !all_finite(z, nel)) ||
        (dt_bias && !all_finite(dt_bias, dim)) || (h0 && !all_finite(h0, batch * dim * N)))
        return OR_ERR_NONFINITE;
    for (int64_t i = 0; i < dim * N; ++i)
        if (A[i] > 0.0) return OR_ERR_RETAIN;

    const int64_t rows = batch * dim;
    int failed = 0;
#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#else
    (void)nthreads;
#endif
    {
        double* h = (double*)malloc((size_t)N * sizeof(double));
        if (!h) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t r = 0; r < rows; ++r) {
            if (!h) continue;
            const int64_t b = r / dim;
            const int64_t d = r % dim;
            const double bias = dt_bias ? dt_bias[d] : 0.0;
            const double skip = Dskip ? Dskip[d] : 0.0;
            for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[r * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const double dt = oracle_softplus(delta[r * L + t] + bias);
                const double ut = u[r * L + t];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double a = exp(dt * A[d * N + n]);
                    const double bt = Bm[(b * N + n) * L + t];
                    const double ct = Cm[(b * N + n) * L + t];
                    h[n] = a * h[n] + dt * bt * ut;
                    acc += ct * h[n];
                }
                double out = acc + skip * ut;
                if (z) out *= oracle_silu(z[r * L + t]);
                y[r * L + t] = out;
            }
            if (h_last)
                for (int64_t n = 0; n < N; ++n) h_last[r * N + n] = h[n];
        }
        free(h);
    }
    return failed ? OR_ERR_ALLOC : OR_OK;
}

/* The scan from a zero state, without returning the final state. */
int oracle_selective_scan_fwd(int64_t batch, int64_t L, int64_t dim, int64_t N,
                              const double* u, const double* delta, const double* A,
                              const double* Bm, const double* Cm, const double* Dskip,
                              const double* z, const double* dt_bias, double* y, int nthreads)
{
    return oracle_selective_scan_state(batch, L, dim, N, u, delta, A, Bm, Cm, Dskip, z, dt_bias,
                                       NULL, y, NULL, nthreads);
}

/* Number of threads an OpenMP parallel region would use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
