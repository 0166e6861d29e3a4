"""Pins for the fp64 oracle: each test ties it to something other than itself.

None of these tests reuses the oracle's own formula: they check it against the
worked example printed on the qubittool.com page "Mamba 与状态空间模型：机制、演进与
工程选型" (section "一个可运行的标量模型"), against closed forms (LTI convolution,
the semiseparable sum of the cnblogs.com page "Mamba3 技术浅析" §2.2.2, the A = 0
prefix sum, the constant-input geometric series), against library routines
(numpy.logaddexp for softplus, scipy.special.expit for the sigmoid) and against
structural invariants.  A dropped term, a flipped sign, a wrong index, a transposed
B/C or a read-before-update would each fail at least one of them.
"""
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "qubittool_scalar_example.txt")


def _golden():
    steps, invalid, expect = [], None, {}
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "step":
                steps.append([float(v) for v in vals])
            elif key == "invalid":
                invalid = [float(v) for v in vals]
            else:
                expect[key] = vals
    return np.array(steps), np.array(invalid), expect


def softplus_ref(x):
    return np.logaddexp(0.0, x)


def silu_ref(x):
    return x * expit(x)


# ---------------------------------------------------------------- worked example

def _as_scan_inputs(value, retain, write, read):
    """The page's retain/write/read steps as a one-channel, one-state scan.

    With A = -1 the retain factor exp(dt*A) equals retain when dt = -ln(retain); the
    raw step input is the inverse softplus of that dt, log(expm1(dt)).  The write term
    dt*B*u equals write*value when u = value and B = write/dt.  C = read reads the
    state after the update; D and the gate are absent."""
    value, retain, write, read = (np.asarray(a, dtype=np.float64) for a in (value, retain, write, read))
    dt = -np.log(retain)
    delta_raw = np.array([math.log(math.expm1(v)) for v in dt])
    L = value.shape[0]
    return dict(u=value.reshape(1, 1, L), delta=delta_raw.reshape(1, 1, L), A=np.array([[-1.0]]),
                B=(write / dt).reshape(1, 1, L), C=read.reshape(1, 1, L))


def test_scalar_example_matches_printed_output():
    """The three steps of the page's runnable scalar model, through the oracle's scan:
    the outputs it prints, to the two decimals printed and to fp64 rounding."""
    steps, _, expect = _golden()
    y, h_last = oracle.selective_scan_state(**_as_scan_inputs(*steps.T))
    out = y.reshape(-1)
    printed = expect["expect_outputs_2dp"]
    assert ["%.2f" % v for v in out] == printed
    np.testing.assert_allclose(out, [float(v) for v in printed], rtol=0, atol=1e-12)
    # the second step writes nothing, so its large value never reaches the state:
    # the state only decays, 2.00 -> 0.95 * 2.00
    assert out[1] == pytest.approx(0.95 * out[0], rel=1e-14)
    np.testing.assert_allclose(h_last.reshape(-1), [out[-1]], rtol=0, atol=1e-12)


def test_scalar_example_rejects_invalid_retention():
    """A retain factor of 1.2 (outside [0, 1]) is refused.  In the scan, retain =
    exp(dt*A) with dt = softplus(.) > 0, so retain > 1 is exactly A > 0: with the raw
    step input 0 (dt = ln 2), A = ln(1.2)/ln 2 gives retain 1.2."""
    _, invalid, expect = _golden()
    assert expect["expect_invalid_retention_rejected"] == ["true"]
    value, retain, write, read = invalid
    assert retain > 1.0
    dt = math.log(2.0)
    A = math.log(retain) / dt
    assert math.exp(dt * A) == pytest.approx(retain, rel=1e-15)
    with pytest.raises(oracle.OracleError) as e:
        oracle.selective_scan_fwd(u=[[[value]]], delta=[[[0.0]]], A=[[A]], B=[[[write / dt]]], C=[[[read]]])
    assert e.value.code == oracle.ERR_RETAIN
    # the same step with the retain factor inside [0, 1] is accepted
    oracle.selective_scan_fwd(u=[[[value]]], delta=[[[0.0]]], A=[[-A]], B=[[[write / dt]]], C=[[[read]]])


def test_scalar_example_other_refusals():
    """The page's model refuses an empty sequence and a non-finite field before it
    forms any state; so does the scan oracle."""
    with pytest.raises(oracle.OracleError) as e:
        oracle.selective_scan_fwd(np.zeros((1, 1, 0)), np.zeros((1, 1, 0)), [[-1.0]], np.zeros((1, 1, 0)),
                                  np.zeros((1, 1, 0)))
    assert e.value.code == oracle.ERR_EMPTY
    steps, _, _ = _golden()
    for field in range(4):
        bad = steps.T.copy()
        bad[field, 1] = np.nan
        args = _as_scan_inputs(*bad)
        with pytest.raises(oracle.OracleError) as e:
            oracle.selective_scan_fwd(**args)
        assert e.value.code == oracle.ERR_NONFINITE, field


# ---------------------------------------------------------------- elementwise functions

def test_softplus_against_logaddexp_and_special_values():
    xs = np.concatenate([np.linspace(-60, 60, 2401), [-745.0, -700.0, 0.0, 1e-12, -1e-12, 700.0, 800.0, 1e4]])
    got = np.array([oracle.softplus(x) for x in xs])
    np.testing.assert_allclose(got, softplus_ref(xs), rtol=2e-15, atol=0)
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-16)
    # the inverse of softplus undoes it: softplus(log(expm1(v))) = v
    for v in (1e-6, 1e-3, 0.1, 1.0, 5.0):
        assert oracle.softplus(math.log(math.expm1(v))) == pytest.approx(v, rel=1e-12)


def test_silu_against_expit():
    xs = np.linspace(-40, 40, 1601)
    got = np.array([oracle.silu(x) for x in xs])
    np.testing.assert_allclose(got, silu_ref(xs), rtol=1e-15, atol=1e-300)
    assert oracle.silu(0.0) == 0.0


# ---------------------------------------------------------------- closed forms

def _rand_problem(rng, batch, dim, N, L, a_scale=1.0):
    u = rng.standard_normal((batch, dim, L))
    delta = rng.standard_normal((batch, dim, L))
    z = rng.standard_normal((batch, dim, L))
    Bm = rng.standard_normal((batch, N, L))
    Cm = rng.standard_normal((batch, N, L))
    A = -a_scale * rng.uniform(0.1, 2.0, size=(dim, N))
    D = rng.standard_normal(dim)
    bias = rng.uniform(-2.0, 1.0, size=dim)
    return u, delta, z, Bm, Cm, A, D, bias


def test_lti_case_equals_convolution():
    """delta, B, C constant in time: the scan is a causal convolution with
    K_k = sum_n C_n exp(dt*A_n)^k dt*B_n (LTI identity)."""
    rng = np.random.default_rng(11)
    batch, dim, N, L = 2, 3, 4, 40
    u = rng.standard_normal((batch, dim, L))
    z = rng.standard_normal((batch, dim, L))
    dr = rng.standard_normal((batch, dim))
    Bn = rng.standard_normal((batch, N))
    Cn = rng.standard_normal((batch, N))
    A = -rng.uniform(0.2, 3.0, size=(dim, N))
    D = rng.standard_normal(dim)
    bias = rng.uniform(-1.0, 1.0, size=dim)
    delta = np.repeat(dr[:, :, None], L, axis=2)
    Bm = np.repeat(Bn[:, :, None], L, axis=2)
    Cm = np.repeat(Cn[:, :, None], L, axis=2)
    y = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, D, z, bias)
    k = np.arange(L)
    for b in range(batch):
        for d in range(dim):
            dt = softplus_ref(dr[b, d] + bias[d])
            a = np.exp(dt * A[d])                                  # (N,)
            K = (Cn[b][None, :] * a[None, :] ** k[:, None] * dt * Bn[b][None, :]).sum(axis=1)
            conv = np.convolve(u[b, d], K)[:L]
            ref = (conv + D[d] * u[b, d]) * silu_ref(z[b, d])
            np.testing.assert_allclose(y[b, d], ref, rtol=1e-11, atol=1e-12)


def test_time_varying_case_equals_semiseparable_sum():
    """y_t = sum_{i<=t} sum_n C_{t,n} prod_{k=i+1..t} exp(dt_k A_n) dt_i B_{i,n} u_i,
    plus D*u_t, times SiLU(z_t) -- the semiseparable (matrix) form of the scan."""
    rng = np.random.default_rng(12)
    batch, dim, N, L = 2, 3, 3, 24
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, batch, dim, N, L)
    y = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, D, z, bias)
    for b in range(batch):
        for d in range(dim):
            dt = softplus_ref(delta[b, d] + bias[d])
            S = np.cumsum(dt)                                     # S_t = sum_{k<=t} dt_k
            ref = np.zeros(L)
            for t in range(L):
                acc = 0.0
                for i in range(t + 1):
                    decay = np.exp(A[d] * (S[t] - S[i]))          # (N,) prod over k = i+1..t
                    acc += np.sum(Cm[b, :, t] * decay * dt[i] * Bm[b, :, i]) * u[b, d, i]
                ref[t] = (acc + D[d] * u[b, d, t]) * silu_ref(z[b, d, t])
            np.testing.assert_allclose(y[b, d], ref, rtol=1e-11, atol=1e-12)


def test_zero_decay_is_prefix_sum():
    """A = 0: nothing decays and h_t = cumsum(dt*B*u)."""
    rng = np.random.default_rng(13)
    batch, dim, N, L = 2, 2, 5, 50
    u, delta, z, Bm, Cm, _, D, bias = _rand_problem(rng, batch, dim, N, L)
    A = np.zeros((dim, N))
    y = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, None, None, bias)
    for b in range(batch):
        for d in range(dim):
            dt = softplus_ref(delta[b, d] + bias[d])
            h = np.cumsum(dt[None, :] * Bm[b] * u[b, d][None, :], axis=1)  # (N, L)
            np.testing.assert_allclose(y[b, d], (Cm[b] * h).sum(axis=0), rtol=1e-12, atol=1e-12)


def test_constant_input_is_geometric_series():
    """Constant dt, B, u: h_t = dt*B*u * (1 - a^{t+1}) / (1 - a) with a = exp(dt*A)."""
    N, L = 6, 80
    A = -np.linspace(0.3, 2.5, N).reshape(1, N)
    dr, uv, bias = 0.7, 1.3, -0.4
    Bn = np.linspace(-1.0, 1.5, N)
    Cn = np.linspace(0.5, -0.8, N)
    u = np.full((1, 1, L), uv)
    delta = np.full((1, 1, L), dr)
    Bm = np.repeat(Bn.reshape(1, N, 1), L, axis=2)
    Cm = np.repeat(Cn.reshape(1, N, 1), L, axis=2)
    y = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, dt_bias=np.array([bias]))
    dt = softplus_ref(dr + bias)
    a = np.exp(dt * A[0])
    t = np.arange(L)
    h = dt * Bn[:, None] * uv * (1.0 - a[:, None] ** (t[None, :] + 1)) / (1.0 - a[:, None])
    np.testing.assert_allclose(y[0, 0], (Cn[:, None] * h).sum(axis=0), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- invariants

def test_zero_write_leaves_value_out_of_state():
    """B_t = 0 at step t0 (and no skip, no gate): u_{t0} never reaches the state, so
    changing it changes no output (the zero-write step of the scalar example)."""
    rng = np.random.default_rng(14)
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, 1, 3, 4, 30)
    t0 = 11
    Bm[:, :, t0] = 0.0
    y1 = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, None, None, bias)
    u2 = u.copy()
    u2[:, :, t0] += 9.0
    y2 = oracle.selective_scan_fwd(u2, delta, A, Bm, Cm, None, None, bias)
    np.testing.assert_array_equal(y1, y2)


def test_small_step_keeps_state_close():
    """With A < 0, |h_t - h_{t-1}| <= dt_t (|A| |h_{t-1}| + |B_t u_t|) exactly
    (1 - e^{-x} <= x); with N = 1, C = 1, no skip and no gate, y_t = h_t."""
    rng = np.random.default_rng(15)
    L = 200
    u = rng.standard_normal((1, 1, L))
    delta = rng.standard_normal((1, 1, L)) - 6.0        # small steps
    Bm = rng.standard_normal((1, 1, L))
    Cm = np.ones((1, 1, L))
    A = np.array([[-1.7]])
    h = oracle.selective_scan_fwd(u, delta, A, Bm, Cm)[0, 0]
    dt = softplus_ref(delta[0, 0])
    hp = np.concatenate([[0.0], h[:-1]])
    bound = dt * (1.7 * np.abs(hp) + np.abs(Bm[0, 0] * u[0, 0]))
    assert np.all(np.abs(h - hp) <= bound * (1 + 1e-12) + 1e-300)
    assert np.max(dt) < 0.05


def test_causality():
    rng = np.random.default_rng(16)
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, 2, 2, 3, 40)
    y1 = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, D, z, bias)
    for arr_name in ("u", "delta", "z", "B", "C"):
        arrs = dict(u=u.copy(), delta=delta.copy(), z=z.copy(), B=Bm.copy(), C=Cm.copy())
        arrs[arr_name][:, :, 25:] += 3.0
        y2 = oracle.selective_scan_fwd(arrs["u"], arrs["delta"], A, arrs["B"], arrs["C"], D, arrs["z"], bias)
        np.testing.assert_array_equal(y1[:, :, :25], y2[:, :, :25])
        assert not np.array_equal(y1[:, :, 25:], y2[:, :, 25:])


def test_linear_in_u():
    rng = np.random.default_rng(17)
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, 1, 3, 4, 30)
    u2 = rng.standard_normal(u.shape)
    y1 = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, D, z, bias)
    y2 = oracle.selective_scan_fwd(u2, delta, A, Bm, Cm, D, z, bias)
    y3 = oracle.selective_scan_fwd(u - 2.5 * u2, delta, A, Bm, Cm, D, z, bias)
    np.testing.assert_allclose(y3, y1 - 2.5 * y2, rtol=1e-11, atol=1e-12)


def test_channels_and_batches_are_independent():
    rng = np.random.default_rng(18)
    batch, dim = 3, 5
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, batch, dim, 4, 20)
    y = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, D, z, bias)
    pc = rng.permutation(dim)
    pb = rng.permutation(batch)
    yp = oracle.selective_scan_fwd(u[pb][:, pc], delta[pb][:, pc], A[pc], Bm[pb], Cm[pb], D[pc], z[pb][:, pc], bias[pc])
    np.testing.assert_array_equal(yp, y[pb][:, pc])


def test_zero_input_matrix_leaves_only_skip():
    """B = 0: the state stays zero and y = D*u*SiLU(z)."""
    rng = np.random.default_rng(19)
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, 2, 3, 4, 25)
    y = oracle.selective_scan_fwd(u, delta, A, np.zeros_like(Bm), Cm, D, z, bias)
    np.testing.assert_allclose(y, D[None, :, None] * u * silu_ref(z), rtol=1e-15, atol=0)


def test_missing_optionals_mean_zero_bias_no_skip_no_gate():
    rng = np.random.default_rng(20)
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, 1, 2, 3, 15)
    dim = u.shape[1]
    y0 = oracle.selective_scan_fwd(u, delta, A, Bm, Cm)
    y1 = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, np.zeros(dim), None, np.zeros(dim))
    np.testing.assert_array_equal(y0, y1)


# ---------------------------------------------------------------- refusals

def test_scan_refuses_bad_inputs():
    rng = np.random.default_rng(21)
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, 1, 2, 3, 10)
    Abad = A.copy()
    Abad[1, 2] = 0.5
    with pytest.raises(oracle.OracleError) as e:
        oracle.selective_scan_fwd(u, delta, Abad, Bm, Cm)
    assert e.value.code == oracle.ERR_RETAIN
    ubad = u.copy()
    ubad[0, 1, 3] = np.inf
    with pytest.raises(oracle.OracleError) as e:
        oracle.selective_scan_fwd(ubad, delta, A, Bm, Cm)
    assert e.value.code == oracle.ERR_NONFINITE
    zbad = z.copy()
    zbad[0, 0, 0] = np.nan
    with pytest.raises(oracle.OracleError) as e:
        oracle.selective_scan_fwd(u, delta, A, Bm, Cm, D, zbad, bias)
    assert e.value.code == oracle.ERR_NONFINITE
    with pytest.raises(oracle.OracleError) as e:
        oracle.selective_scan_fwd(u[:, :, :0], delta[:, :, :0], A, Bm[:, :, :0], Cm[:, :, :0])
    assert e.value.code == oracle.ERR_EMPTY


def test_thread_count_does_not_change_result():
    rng = np.random.default_rng(22)
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, 2, 7, 4, 33)
    y1 = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, D, z, bias, nthreads=1)
    y4 = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, D, z, bias, nthreads=4)
    np.testing.assert_array_equal(y1, y4)


# ---------------------------------------------------------------- carried state, decode step

def test_scalar_example_as_decode_steps():
    """The worked example fed one token at a time, the state carried between calls,
    gives the printed outputs (recurrent decoding keeps a fixed-size state)."""
    steps, _, expect = _golden()
    printed = [float(v) for v in expect["expect_outputs_2dp"]]
    h = None
    outs = []
    for value, retain, write, read in steps:
        dt = -math.log(retain)
        dr = math.log(math.expm1(dt))
        y, h = oracle.selective_scan_step(u=[[value]], delta=[[dr]], A=[[-1.0]], B=[[write / dt]], C=[[read]], h=h)
        outs.append(y[0, 0])
    np.testing.assert_allclose(outs, printed, rtol=0, atol=1e-12)
    np.testing.assert_allclose(h.reshape(-1), [printed[-1]], rtol=0, atol=1e-12)


def test_initial_state_closed_form():
    """With a starting state h0: y_t = [sum_n C_{t,n} (e^{A_n S_t} h0_n + sum_{i<=t}
    e^{A_n (S_t - S_i)} dt_i B_{i,n} u_i) + D u_t] SiLU(z_t), S_t = sum_{k<=t} dt_k, and
    the final state is the bracketed state at t = L-1."""
    rng = np.random.default_rng(23)
    batch, dim, N, L = 2, 3, 4, 20
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, batch, dim, N, L)
    h0 = rng.standard_normal((batch, dim, N)) * 3.0
    y, h_last = oracle.selective_scan_state(u, delta, A, Bm, Cm, D, z, bias, h0=h0)
    for b in range(batch):
        for d in range(dim):
            dt = softplus_ref(delta[b, d] + bias[d])
            S = np.cumsum(dt)
            for t in range(L):
                state = np.exp(A[d] * S[t]) * h0[b, d]
                for i in range(t + 1):
                    state = state + np.exp(A[d] * (S[t] - S[i])) * dt[i] * Bm[b, :, i] * u[b, d, i]
                ref = (np.sum(Cm[b, :, t] * state) + D[d] * u[b, d, t]) * silu_ref(z[b, d, t])
                assert y[b, d, t] == pytest.approx(ref, rel=1e-11, abs=1e-12)
            np.testing.assert_allclose(h_last[b, d], state, rtol=1e-11, atol=1e-12)


def test_zero_initial_state_is_the_plain_scan():
    rng = np.random.default_rng(24)
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, 2, 3, 5, 17)
    y0 = oracle.selective_scan_fwd(u, delta, A, Bm, Cm, D, z, bias)
    y1, _ = oracle.selective_scan_state(u, delta, A, Bm, Cm, D, z, bias, h0=np.zeros((2, 3, 5)))
    np.testing.assert_array_equal(y0, y1)


def test_state_refusals():
    rng = np.random.default_rng(25)
    u, delta, z, Bm, Cm, A, D, bias = _rand_problem(rng, 1, 2, 3, 5)
    h0 = np.zeros((1, 2, 3))
    h0[0, 1, 2] = np.nan
    with pytest.raises(oracle.OracleError) as e:
        oracle.selective_scan_state(u, delta, A, Bm, Cm, D, z, bias, h0=h0)
    assert e.value.code == oracle.ERR_NONFINITE
