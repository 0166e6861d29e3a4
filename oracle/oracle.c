/*
 * oracle.c -- plain fp64 CPU reference of the Mamba-1 selective scan: the forward
 * pass (with a carried state) and its gradients.
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
 * code (tests/test_oracle_pins.py): the worked scalar example printed on [QT]
 * (its retain/write/read steps expressed as a one-channel, one-state scan), the
 * LTI convolution identity, the semiseparable sum of [CB] §2.2.2, the A = 0
 * prefix sum, the constant-input geometric series and structural invariants.  The
 * gradients are pinned by tests/test_oracle_bwd_pins.py: central finite differences
 * of the (pinned) forward, hand-derived closed forms for a single step, the adjoint
 * of the LTI convolution, exact homogeneity identities, and the chain rule across a
 * split of the sequence.
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

/* sigmoid(x) = 1 / (1 + e^-x), evaluated on the side where e^(-|x|) cannot overflow.
 * It is the derivative of softplus. */
double oracle_sigmoid(double x)
{
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    const double e = exp(x);
    return e / (1.0 + e);
}

/*
 * Gradients of the selective scan (the forward of oracle_selective_scan_state) by
 * reverse-mode differentiation of the per-row recurrence.  Training needs them; the
 * pages' kernels obtain the states the backward needs by recomputing them from the
 * inputs instead of reading them from memory ([QA] Q7, [QT] "并行训练不会消除递推关系").
 * This reference simply keeps each row's whole state trajectory in host memory.
 *
 * The scalar loss being differentiated is
 *     sum_{b,d,t} dy[b,d,t] * y[b,d,t]  +  sum_{b,d,n} dh_last[b,d,n] * h_L[b,d,n],
 * so dy is the gradient arriving at y and dh_last (NULL = 0) the one arriving at the
 * final state.  With, per row (b, d) and step t,
 *     r_t = delta_t + dt_bias[d],  dt_t = softplus(r_t),  a_t[n] = exp(dt_t A[d,n]),
 *     h_t[n] = a_t[n] h_{t-1}[n] + dt_t B_t[n] u_t      (h_{-1} = h0, or 0),
 *     s_t = sum_n C_t[n] h_t[n] + D[d] u_t,   y_t = s_t * SiLU(z_t),
 * the chain rule gives, walking t = L-1 .. 0 and carrying e[n] (the gradient reaching
 * h_t[n] from step t+1; e starts at dh_last):
 *     ds_t     = dy_t * SiLU(z_t)                        (dy_t without a gate)
 *     dz_t     = dy_t * s_t * SiLU'(z_t),  SiLU'(x) = sig(x) (1 + x (1 - sig(x)))
 *     g_t[n]   = ds_t C_t[n] + e[n]                      (total gradient at h_t[n])
 *     dC_t[n] += ds_t h_t[n]            summed over the channels d of batch row b
 *     dB_t[n] += g_t[n] dt_t u_t        summed over the channels d of batch row b
 *     dA[d,n] += g_t[n] dt_t a_t[n] h_{t-1}[n]           summed over b and t
 *     ddt_t    = sum_n g_t[n] (A[d,n] a_t[n] h_{t-1}[n] + B_t[n] u_t)
 *     du_t     = D[d] ds_t + dt_t sum_n g_t[n] B_t[n]
 *     dD[d]   += ds_t u_t                                 summed over b and t
 *     ddelta_t = ddt_t * sig(r_t)        (softplus' = sigmoid);  ddt_bias[d] += ddelta_t
 *     e[n]     = a_t[n] g_t[n]
 * and finally dh0 = e.
 *
 * Layouts are those of the forward; du, ddelta, dz: (batch, dim, L); dB, dC:
 * (batch, N, L); dA: (dim, N); dD, ddt_bias: (dim,); dh0: (batch, dim, N).  dD is
 * written only if Dskip and dD are given, dz only if z and dz are, ddt_bias and dh0
 * only if given.  Sums over rows are taken per thread (static row split) and then
 * added in thread order.  Same refusals as the forward, plus a non-finite dy or
 * dh_last.
 */
int oracle_selective_scan_bwd(int64_t batch, int64_t L, int64_t dim, int64_t N,
                              const double* u, const double* delta, const double* A,
                              const double* Bm, const double* Cm, const double* Dskip,
                              const double* z, const double* dt_bias, const double* h0,
                              const double* dy, const double* dh_last,
                              double* du, double* ddelta, double* dA, double* dB, double* dC,
                              double* dD, double* dz, double* ddt_bias, double* dh0, int nthreads)
{
    if (batch <= 0 || L <= 0 || dim <= 0 || N <= 0) return OR_ERR_EMPTY;
    if (!u || !delta || !A || !Bm || !Cm || !dy || !du || !ddelta || !dA || !dB || !dC) return OR_ERR_NULL;
    const int64_t nel = batch * dim * L;
    const int64_t nbc = batch * N * L;
    const int64_t nst = batch * dim * N;
    if (!all_finite(u, nel) || !all_finite(delta, nel) || !all_finite(A, dim * N) ||
        !all_finite(Bm, nbc) || !all_finite(Cm, nbc) || !all_finite(dy, nel))
        return OR_ERR_NONFINITE;
    if ((Dskip && !all_finite(Dskip, dim)) || (z && !all_finite(z, nel)) ||
        (dt_bias && !all_finite(dt_bias, dim)) || (h0 && !all_finite(h0, nst)) ||
        (dh_last && !all_finite(dh_last, nst)))
        return OR_ERR_NONFINITE;
    for (int64_t i = 0; i < dim * N; ++i)
        if (A[i] > 0.0) return OR_ERR_RETAIN;

#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    const int nt = 1;
    (void)nthreads;
#endif
    /* per-thread sums: dB, dC (batch*N*L each), dA (dim*N), dD and ddt_bias (dim each) */
    const int64_t per = 2 * nbc + dim * N + 2 * dim;
    double* acc = (double*)calloc((size_t)nt * (size_t)per, sizeof(double));
    if (!acc) return OR_ERR_ALLOC;
    const int64_t rows = batch * dim;
    int failed = 0;
#ifdef _OPENMP
#pragma omp parallel num_threads(nt)
#endif
    {
#ifdef _OPENMP
        const int tid = omp_get_thread_num();
#else
        const int tid = 0;
#endif
        double* tB = acc + (int64_t)tid * per;
        double* tC = tB + nbc;
        double* tA = tC + nbc;
        double* tD = tA + dim * N;
        double* tbias = tD + dim;
        /* the row's states h_{-1} .. h_{L-1}, then the carried gradient e */
        double* hs = (double*)malloc((size_t)(L + 1) * (size_t)N * sizeof(double));
        double* e = (double*)malloc((size_t)N * sizeof(double));
        if (!hs || !e) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t r = 0; r < rows; ++r) {
            if (!hs || !e) continue;
            const int64_t b = r / dim;
            const int64_t d = r % dim;
            const double bias = dt_bias ? dt_bias[d] : 0.0;
            const double skip = Dskip ? Dskip[d] : 0.0;
            /* forward, keeping every state: hs[(t+1)*N + n] = h_t[n] */
            for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[r * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const double dt = oracle_softplus(delta[r * L + t] + bias);
                const double ut = u[r * L + t];
                for (int64_t n = 0; n < N; ++n) {
                    const double a = exp(dt * A[d * N + n]);
                    hs[(t + 1) * N + n] = a * hs[t * N + n] + dt * Bm[(b * N + n) * L + t] * ut;
                }
            }
            /* reverse */
            for (int64_t n = 0; n < N; ++n) e[n] = dh_last ? dh_last[r * N + n] : 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const double rt = delta[r * L + t] + bias;
                const double dt = oracle_softplus(rt);
                const double ut = u[r * L + t];
                const double* ht = hs + (t + 1) * N;
                const double* hp = hs + t * N;
                double s = skip * ut;
                for (int64_t n = 0; n < N; ++n) s += Cm[(b * N + n) * L + t] * ht[n];
                double ds = dy[r * L + t];
                if (z) {
                    const double zt = z[r * L + t];
                    const double sg = oracle_sigmoid(zt);
                    if (dz) dz[r * L + t] = dy[r * L + t] * s * sg * (1.0 + zt * (1.0 - sg));
                    ds = dy[r * L + t] * oracle_silu(zt);
                }
                double ddt = 0.0, dut = skip * ds;
                for (int64_t n = 0; n < N; ++n) {
                    const double an = A[d * N + n];
                    const double a = exp(dt * an);
                    const double bt = Bm[(b * N + n) * L + t];
                    const double ct = Cm[(b * N + n) * L + t];
                    const double g = ds * ct + e[n];
                    tC[(b * N + n) * L + t] += ds * ht[n];
                    tB[(b * N + n) * L + t] += g * dt * ut;
                    tA[d * N + n] += g * dt * a * hp[n];
                    ddt += g * (an * a * hp[n] + bt * ut);
                    dut += dt * g * bt;
                    e[n] = a * g;
                }
                du[r * L + t] = dut;
                const double dr = ddt * oracle_sigmoid(rt);
                ddelta[r * L + t] = dr;
                tD[d] += ds * ut;
                tbias[d] += dr;
            }
            if (dh0)
                for (int64_t n = 0; n < N; ++n) dh0[r * N + n] = e[n];
        }
        free(hs);
        free(e);
    }
    if (failed) {
        free(acc);
        return OR_ERR_ALLOC;
    }
    /* add the per-thread sums in thread order */
    for (int64_t i = 0; i < nbc; ++i) { dB[i] = 0.0; dC[i] = 0.0; }
    for (int64_t i = 0; i < dim * N; ++i) dA[i] = 0.0;
    if (Dskip && dD) for (int64_t i = 0; i < dim; ++i) dD[i] = 0.0;
    if (ddt_bias) for (int64_t i = 0; i < dim; ++i) ddt_bias[i] = 0.0;
    for (int k = 0; k < nt; ++k) {
        const double* tB = acc + (int64_t)k * per;
        const double* tC = tB + nbc;
        const double* tA = tC + nbc;
        const double* tD = tA + dim * N;
        const double* tbias = tD + dim;
        for (int64_t i = 0; i < nbc; ++i) { dB[i] += tB[i]; dC[i] += tC[i]; }
        for (int64_t i = 0; i < dim * N; ++i) dA[i] += tA[i];
        if (Dskip && dD) for (int64_t i = 0; i < dim; ++i) dD[i] += tD[i];
        if (ddt_bias) for (int64_t i = 0; i < dim; ++i) ddt_bias[i] += tbias[i];
    }
    free(acc);
    return OR_OK;
}

/*
 * Causal depthwise convolution of the scan's input, the "local convolution" that a
 * real Mamba layer places before the scan ([QT], the remark after the runnable
 * scalar model), with an optional SiLU (the activation [GS] §3.1 uses in the block).
 * Per row (b, d) and t = 0 .. L-1, with width K:
 *     pre[t] = bias[d] + sum_{k=0}^{K-1} w[d,k] * xs(t - (K-1) + k)
 *     out[t] = SiLU(pre[t]) if silu else pre[t]
 * where xs(s) = x[b,d,s] for s >= 0 and, for s < 0, the carried history
 * state[b,d,(K-1)+s] (the K-1 inputs before the sequence, oldest first), or 0 without a
 * state.  The conv state is part of what recurrent decoding keeps per layer ([QT],
 * the paragraph on inference memory).  state_out (nullable) receives the K-1 inputs
 * xs(L-K+1) .. xs(L-1), the history the next call continues from.
 * Layouts: x, out (batch, dim, L); w (dim, K); bias (dim,) nullable; state, state_out
 * (batch, dim, K-1).  K must be 1 .. 8.  Non-finite inputs are refused.
 */
int oracle_causal_conv1d(int64_t batch, int64_t L, int64_t dim, int64_t K, const double* x, const double* w,
                         const double* bias, const double* state, int silu, double* out, double* state_out)
{
    if (batch <= 0 || L <= 0 || dim <= 0) return OR_ERR_EMPTY;
    if (K < 1 || K > 8) return OR_ERR_EMPTY;
    if (!x || !w || !out) return OR_ERR_NULL;
    const int64_t H = K - 1;
    if (!all_finite(x, batch * dim * L) || !all_finite(w, dim * K) || (bias && !all_finite(bias, dim)) ||
        (state && H > 0 && !all_finite(state, batch * dim * H)))
        return OR_ERR_NONFINITE;
    for (int64_t r = 0; r < batch * dim; ++r) {
        const int64_t d = r % dim;
        for (int64_t t = 0; t < L; ++t) {
            double acc = bias ? bias[d] : 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t s = t - H + k;
                double xv = 0.0;
                if (s >= 0) xv = x[r * L + s];
                else if (state) xv = state[r * H + (H + s)];
                acc += w[d * K + k] * xv;
            }
            out[r * L + t] = silu ? oracle_silu(acc) : acc;
        }
        if (state_out)
            for (int64_t j = 0; j < H; ++j) {
                const int64_t s = L - H + j;
                double xv = 0.0;
                if (s >= 0) xv = x[r * L + s];
                else if (state) xv = state[r * H + (H + s)];
                state_out[r * H + j] = xv;
            }
    }
    return OR_OK;
}
