"""Seeded random shapes through the forward and the backward, each against the oracle.

The shapes are drawn once from a fixed seed, so the cases are the same on every run.
They cover the planner's branches together:
- state counts across the narrow, role-split and wide paths, padding included;
- diagonal and scalar decay, f32 and bf16 rows;
- ragged lengths and channel counts, and lengths that allow or rule out vector loads;
- forced piece counts, including the pieces whose states the matrix cores form;
- and, drawn separately, shapes that run the chunked form of the scalar-decay scan.
Bars are the contract's: 1e-4 for f32 rows, 2e-2 for bf16 (and, for the backward's
float32 reductions, 1e-4 of each tensor's scale; see bwd_cases.py).
"""
import sys

import numpy as np
import pytest

from bwd_cases import compare, run_gpu_bwd, run_oracle_bwd
from scan_cases import TOL, rel_err, run_gpu, run_oracle
from selective_state_space_79_amd.inputs import make_cotangents, make_inputs

pytestmark = pytest.mark.gpu


def _draw(seed: int, count: int, max_elems: int):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        N = int(rng.choice([1, 3, 4, 8, 12, 16, 24, 32, 40, 64, 100, 128]))
        nheads = int(rng.choice([0, 0, 1, 2, 4]))
        head_dim = int(rng.choice([8, 16, 32, 64]))
        dim = nheads * head_dim if nheads else int(rng.integers(1, 200))
        L = int(rng.choice([1, 7, 16, 63, 64, 100, 257, 512, 640, 1000]))
        batch = int(rng.integers(1, 4))
        io = str(rng.choice(["f32", "bf16"]))
        nch = int(rng.choice([0, 0, 2, 3, 5]))
        if batch * L * dim * N > max_elems:
            continue
        cases.append((batch, L, dim, N, io, nheads, nch))
    return cases


FWD = _draw(5150, 24, 3_000_000)
BWD = _draw(5151, 16, 1_000_000)


def announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("case", FWD, ids=lambda c: "b{}L{}d{}N{}{}h{}ch{}".format(*c))
def test_forward_random_shape(case):
    batch, L, dim, N, io, nheads, nch = case
    seed = 5200 + FWD.index(case)
    announce(f"fwd random {case} seed={seed}")
    x = make_inputs(batch, L, dim, N, seed=seed, io=io, nheads=nheads)
    y = run_gpu(x, nchunks=nch)
    err = rel_err(y, run_oracle(x))
    print(f"err={err:.3e}", flush=True)
    assert np.all(np.isfinite(y))
    assert err <= TOL[io]


@pytest.mark.parametrize("case", BWD, ids=lambda c: "b{}L{}d{}N{}{}h{}ch{}".format(*c))
def test_backward_random_shape(case):
    batch, L, dim, N, io, nheads, nch = case
    seed = 5300 + BWD.index(case)
    announce(f"bwd random {case} seed={seed}")
    x = make_inputs(batch, L, dim, N, seed=seed, io=io, nheads=nheads)
    dy, dhl = make_cotangents(x, seed=seed + 1, with_dh_last=True)
    g = run_gpu_bwd(x, dy, dh_last=dhl, nchunks=nch)
    r = run_oracle_bwd(x, dy, dh_last=dhl)
    errs = compare(g, r)
    print(" ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in g.items():
        assert np.all(np.isfinite(v)), k
    for k, e in errs.items():
        bar = 2e-2 if (io == "bf16" and k in ("du", "ddelta", "dz")) else 1e-4
        assert e <= bar, (k, e)


def _draw_chunked(seed: int, count: int, max_elems: int):
    """Shapes the planner gives the chunked form (plan form 1): scalar decay, bf16 rows,
    64 or 128 states, L a multiple of 8; heads of 8..128 channels, ragged channel
    blocks and last chunks, library-chosen or forced piece counts, with or without the
    skip, gate and bias."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        N = int(rng.choice([64, 128]))
        nheads = int(rng.integers(1, 7))
        head_dim = int(rng.choice([8, 13, 40, 64, 128]))
        dim = nheads * head_dim
        L = 8 * int(rng.integers(1, 400))
        batch = int(rng.integers(1, 4))
        nch = int(rng.choice([0, 0, 2, 3, 7]))
        flags = tuple(bool(v) for v in rng.integers(0, 2, size=3))
        if batch * L * dim * N > max_elems:
            continue
        cases.append((batch, L, dim, N, nheads, nch) + flags)
    return cases


CHUNKED = _draw_chunked(5152, 12, 8_000_000)


@pytest.mark.parametrize("case", CHUNKED, ids=lambda c: "b{}L{}d{}N{}h{}ch{}D{:d}z{:d}bias{:d}".format(*c))
def test_chunked_form_random_shape(case):
    import selective_state_space_79_amd as ssm

    batch, L, dim, N, nheads, nch, wD, wz, wb = case
    seed = 5400 + CHUNKED.index(case)
    plan = ssm.ssm_selective_scan_plan(ssm.make_dims(batch, L, dim, N, nheads=nheads, nchunks=nch)).as_dict()
    announce(f"chunked random {case} seed={seed} plan {plan['nchunks']} pieces")
    assert plan["form"] == 1
    x = make_inputs(batch, L, dim, N, seed=seed, io="bf16", nheads=nheads)
    y = run_gpu(x, with_D=wD, with_z=wz, with_bias=wb, nchunks=nch)
    err = rel_err(y, run_oracle(x, with_D=wD, with_z=wz, with_bias=wb))
    print(f"err={err:.3e}", flush=True)
    assert np.all(np.isfinite(y))
    assert err <= TOL["bf16"]
