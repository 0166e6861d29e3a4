"""Numerical stability over a long horizon and under perturbation, GPU against the fp64
oracle.

The recurrence carries its state over the whole sequence, so rounding could build up
with the number of steps, and an error in how pieces of the sequence hand their state
on would show up only far from where it happens.  The pages' production checklist asks
for exactly these checks before deployment: long-horizon and perturbation tests of the
recurrence's numerics (qubittool.com "Mamba 与状态空间模型：机制、演进与工程选型",
section "生产选型清单", item 5).

- Long horizon: a million steps (the pages mention million-token sequences in the same
  article's FAQ), fp32 and bf16 I/O, with the step-size range of the long-sequence
  workload (slow decay, so the state remembers far back), every output and the final
  state against the oracle at the usual bars.
- Perturbation: one input step changed (u, then the raw step size Δraw); the device's
  response y' - y must equal the oracle's response after the changed step and be
  exactly zero before it, for the library's plan and for a plan with many pieces.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from scan_cases import TOL, rel_err
from selective_state_space_79_amd.inputs import make_inputs, to_device

pytestmark = pytest.mark.gpu


def announce(msg):
    print(msg, file=sys.stderr, flush=True)


def gpu_scan(x, *, nchunks=0):
    import torch
    import selective_state_space_79_amd as ssm

    d = to_device(x)
    y, h = ssm.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["dt_bias"],
                                  return_state=True, nchunks=nchunks)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), h.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_million_step_horizon(io):
    L = 1 << 20
    x = make_inputs(1, L, 64, 16, seed=71, io=io, dt_range=(1e-4, 1e-2))
    announce(f"stability: horizon L={L} dim=64 N=16 io={io}")
    y, h = gpu_scan(x)
    yref, href = oracle.selective_scan_state(x.u, x.delta, x.A_dense(), x.B, x.C, x.D, x.z, x.dt_bias)
    ey, eh = rel_err(y, yref), rel_err(h, href)
    # the error does not grow along the sequence: the last 1/16 of the steps are no
    # worse than the bar, and no worse than 4x the first 1/16's error plus the bar's
    # rounding floor
    head = rel_err(y[..., : L // 16], yref[..., : L // 16])
    tail = rel_err(y[..., -(L // 16):], yref[..., -(L // 16):])
    announce(f"stability: err y {ey:.3e} (first 1/16 {head:.3e}, last 1/16 {tail:.3e}), final state {eh:.3e}")
    assert ey <= TOL[io]
    assert eh <= 1e-4
    assert tail <= 4 * head + (1e-6 if io == "f32" else 8e-3)


@pytest.mark.parametrize("what", ["u", "delta"])
@pytest.mark.parametrize("nchunks", [0, 64])
def test_perturbation_response(what, nchunks):
    L, s0 = 65536, 20001
    x = make_inputs(1, L, 64, 16, seed=72, io="f32", dt_range=(1e-4, 1e-2))
    xp = make_inputs(1, L, 64, 16, seed=72, io="f32", dt_range=(1e-4, 1e-2))
    getattr(xp, what)[:, :, s0] += 1.0
    announce(f"stability: perturb {what} at t={s0}, L={L}, nchunks={nchunks}")
    y, _ = gpu_scan(x, nchunks=nchunks)
    yp, _ = gpu_scan(xp, nchunks=nchunks)
    A = x.A_dense()
    yr = oracle.selective_scan_fwd(x.u, x.delta, A, x.B, x.C, x.D, x.z, x.dt_bias)
    yrp = oracle.selective_scan_fwd(xp.u, xp.delta, A, xp.B, xp.C, xp.D, xp.z, xp.dt_bias)
    d, dr = yp - y, yrp - yr
    # nothing before the changed step moves, bit for bit
    assert np.array_equal(yp[..., :s0], y[..., :s0])
    scale = max(1.0, float(np.max(np.abs(dr))))
    err = float(np.max(np.abs(d - dr))) / scale
    # the response still shows 4096 steps later (several pieces on, for the 64-piece
    # plan), and the device resolves it there too: to 1% of its size, above the fp32
    # rounding of outputs of order 1-10
    far = float(np.max(np.abs(dr[..., s0 + 4096:])))
    err_far = float(np.max(np.abs(d[..., s0 + 4096:] - dr[..., s0 + 4096:])))
    announce(f"stability: response max {np.max(np.abs(dr)):.3e}, 4096+ steps later {far:.3e}, err {err:.3e}, "
             f"there {err_far:.3e}")
    assert err <= 1e-4
    assert far > 1e-4
    assert err_far <= 1e-2 * far + 1e-5
