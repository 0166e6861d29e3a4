"""Seeded synthetic inputs for the selective-scan forward pass.

This module only draws random numbers and lays them out.  It holds none of the
scan's arithmetic, so both the HIP path and the fp64 oracle can be fed from it
without sharing any computation.

Recipe (the same for every workload; see ``make_inputs``):

* generator ``numpy.random.Generator(PCG64(seed))``;
* draw order: u, delta_raw, z (batch, dim, L), then B, C (batch, N, L), all
  standard normal in float32, rounded to bfloat16 (round-to-nearest-even) when the
  I/O type is bf16; then the skip D ~ N(0,1) (float32, dim); then per-channel
  step targets dt_d, log-uniform on ``dt_range``; then, in scalar-decay mode,
  one decay a_h = -U(1, 16) per head;
* A[d, n] = -(n + 1) (float32) in diagonal mode;
* dt_bias[d] = log(expm1(dt_d)) in float32, the bias whose softplus is dt_d, so
  that the step size of channel d has median dt_d and spreads by e^{±2} with the
  unit-normal delta_raw.

Values are returned as float32 numpy arrays holding exactly the values the device
sees (bf16 values are exact in float32 and float64).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# The five workloads the scan is tested and measured on.  Shapes follow a
# Mamba layer's scan: dim = d_inner = 2 * d_model, N = d_state.
WORKLOADS = {
    1: dict(name="tiny-fp32", batch=1, L=64, dim=4, N=4, io="f32", nheads=0, dt_range=(1e-3, 1e-1)),
    2: dict(name="mamba-130m-layer", batch=8, L=2048, dim=1536, N=16, io="bf16", nheads=0, dt_range=(1e-3, 1e-1)),
    3: dict(name="mamba-1.3b-layer", batch=4, L=4096, dim=4096, N=16, io="bf16", nheads=0, dt_range=(1e-3, 1e-1)),
    4: dict(name="long-sequence", batch=1, L=131072, dim=2048, N=16, io="bf16", nheads=0, dt_range=(1e-4, 1e-2)),
    5: dict(name="scalar-decay-large-state", batch=2, L=8192, dim=4096, N=128, io="bf16", nheads=64, dt_range=(1e-3, 1e-1)),
}
WORKLOAD_SEEDS = {1: 1, 2: 2, 3: 3, 4: 4, 5: 5}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32.

    Works in place on a float32 copy; inputs are finite normals, so NaN handling is
    not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    bits += np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    bits &= np.uint32(0xFFFF0000)
    return x


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact (as int16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16).view(np.int16)


@dataclasses.dataclass
class ScanInputs:
    batch: int
    L: int
    dim: int
    N: int
    nheads: int
    io: str            # "f32" or "bf16": type of u, delta, z, B, C and y on the device
    u: np.ndarray      # (batch, dim, L)
    delta: np.ndarray  # (batch, dim, L)  raw step input, before bias and softplus
    z: np.ndarray      # (batch, dim, L)
    B: np.ndarray      # (batch, N, L)
    C: np.ndarray      # (batch, N, L)
    A: np.ndarray      # (dim, N) diagonal mode, or (nheads,) scalar-decay mode
    D: np.ndarray      # (dim,)
    dt_bias: np.ndarray  # (dim,)

    def A_dense(self) -> np.ndarray:
        """A as a (dim, N) array; in scalar-decay mode channel d takes its head's a_h.

        Channel d belongs to head d // (dim // nheads) (heads are contiguous
        channel blocks).
        """
        if self.nheads == 0:
            return self.A
        hd = self.dim // self.nheads
        per_channel = np.repeat(self.A, hd)
        return np.ascontiguousarray(np.broadcast_to(per_channel[:, None], (self.dim, self.N)), dtype=np.float32)

    @property
    def updates(self) -> int:
        return self.batch * self.L * self.dim * self.N


def make_inputs(batch: int, L: int, dim: int, N: int, *, seed: int, io: str = "bf16", nheads: int = 0,
                dt_range=(1e-3, 1e-1), a_range=(1.0, 16.0)) -> ScanInputs:
    """Draw one seeded input set (see the module docstring for the recipe)."""
    if io not in ("f32", "bf16"):
        raise ValueError("io must be 'f32' or 'bf16'")
    if nheads and dim % nheads:
        raise ValueError("dim must be a multiple of nheads")
    rng = np.random.Generator(np.random.PCG64(seed))

    def draw(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        return round_to_bf16(x) if io == "bf16" else x

    u = draw((batch, dim, L))
    delta = draw((batch, dim, L))
    z = draw((batch, dim, L))
    B = draw((batch, N, L))
    C = draw((batch, N, L))
    D = rng.standard_normal(dim, dtype=np.float32)
    lo, hi = dt_range
    dt = np.exp(rng.uniform(math.log(lo), math.log(hi), size=dim))
    dt_bias = np.log(np.expm1(dt)).astype(np.float32)
    if nheads:
        A = (-rng.uniform(a_range[0], a_range[1], size=nheads)).astype(np.float32)
    else:
        A = np.ascontiguousarray(np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (dim, N)))
    return ScanInputs(batch, L, dim, N, nheads, io, u, delta, z, B, C, A, D, dt_bias)


def make_workload(index: int, seed: int | None = None) -> ScanInputs:
    """Inputs of one of the five named workloads (seed defaults to its index)."""
    w = WORKLOADS[index]
    return make_inputs(w["batch"], w["L"], w["dim"], w["N"], seed=WORKLOAD_SEEDS[index] if seed is None else seed,
                       io=w["io"], nheads=w["nheads"], dt_range=w["dt_range"])


def to_device(x: ScanInputs, device="cuda"):
    """Upload to torch tensors: u/delta/z/B/C in the I/O type, A/D/dt_bias in float32."""
    import torch

    def io_tensor(a):
        if x.io == "bf16":
            return torch.from_numpy(bf16_bits(a)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    return dict(u=io_tensor(x.u), delta=io_tensor(x.delta), z=io_tensor(x.z), B=io_tensor(x.B), C=io_tensor(x.C),
                A=f32(x.A), D=f32(x.D), dt_bias=f32(x.dt_bias))


def make_cotangents(x: ScanInputs, *, seed: int, with_dh_last: bool = False):
    """Seeded gradients arriving at the scan's outputs, for the backward pass: dy
    (batch, dim, L) standard normal in the I/O type (bf16-rounded like the inputs) and,
    optionally, dh_last (batch, dim, N) standard normal float32.  Returns (dy, dh_last
    or None) as float32 numpy arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dy = rng.standard_normal((x.batch, x.dim, x.L), dtype=np.float32)
    if x.io == "bf16":
        dy = round_to_bf16(dy)
    dhl = rng.standard_normal((x.batch, x.dim, x.N), dtype=np.float32) if with_dh_last else None
    return dy, dhl


def io_to_device(x: ScanInputs, a: np.ndarray, device="cuda"):
    """Upload one (batch, dim, L) array in the I/O type of x."""
    import torch

    if x.io == "bf16":
        return torch.from_numpy(bf16_bits(a)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def make_conv(x: ScanInputs, width: int, *, seed: int, with_bias: bool = True, with_state: bool = False):
    """Seeded parameters of the fused convolution front end for the inputs x (whose u
    then plays the convolution's input): weight (dim, width) ~ N(0, 1/width) float32,
    bias (dim,) ~ N(0, 0.1^2) float32 or None, and optionally a history conv_state
    (batch, dim, width-1) ~ N(0, 1) in the I/O type.  Returns (weight, bias, state)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = (rng.standard_normal((x.dim, width)) / math.sqrt(width)).astype(np.float32)
    b = (0.1 * rng.standard_normal(x.dim)).astype(np.float32) if with_bias else None
    st = None
    if with_state:
        st = rng.standard_normal((x.batch, x.dim, width - 1), dtype=np.float32)
        if x.io == "bf16":
            st = round_to_bf16(st)
    return w, b, st


# The scalar-decay workload with one step size per head, the form the chunked
# state-space-duality path takes (Mamba-2 layout: 64 heads of 64 channels, N = 128).
SSD_WORKLOADS = {
    5: dict(name="scalar-decay-large-state-head-dt", batch=2, L=8192, nheads=64, headdim=64, N=128,
            dt_range=(1e-3, 1e-1)),
}


@dataclasses.dataclass
class SsdInputs:
    """Inputs of the scalar-decay scan with per-head step sizes (all bf16-exact float32
    except A, D and dt_bias).  Head h owns channels h*headdim .. h*headdim+headdim-1."""
    batch: int
    L: int
    nheads: int
    headdim: int
    N: int
    u: np.ndarray        # (batch, dim, L)
    delta: np.ndarray    # (batch, nheads, L)  raw step input, before bias and softplus
    z: np.ndarray        # (batch, dim, L)
    B: np.ndarray        # (batch, N, L)
    C: np.ndarray        # (batch, N, L)
    A: np.ndarray        # (nheads,)  a_h < 0
    D: np.ndarray        # (dim,)
    dt_bias: np.ndarray  # (nheads,)

    @property
    def dim(self) -> int:
        return self.nheads * self.headdim

    @property
    def updates(self) -> int:
        return self.batch * self.L * self.dim * self.N

    def per_channel(self) -> ScanInputs:
        """The same inputs laid out for the per-channel scan: each head's step input,
        bias and decay repeated over its channels (a copy, no arithmetic)."""
        rep = lambda a, axis: np.ascontiguousarray(np.repeat(a, self.headdim, axis=axis))
        return ScanInputs(self.batch, self.L, self.dim, self.N, self.nheads, "bf16", self.u, rep(self.delta, 1),
                          self.z, self.B, self.C, self.A, self.D, rep(self.dt_bias, 0))


def make_ssd_inputs(batch: int, L: int, nheads: int, headdim: int, N: int, *, seed: int, dt_range=(1e-3, 1e-1),
                    a_range=(1.0, 16.0)) -> SsdInputs:
    """Seeded bf16 inputs with one step size per head.  Same recipe as make_inputs in
    scalar-decay mode except that delta_raw is (batch, nheads, L) and dt_h is drawn per
    head: draw order u, delta_raw, z, B, C (standard normal, rounded to bf16), D (N(0,1)
    float32), dt_h (log-uniform on dt_range), a_h = -U(a_range); dt_bias[h] =
    log(expm1(dt_h))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dim = nheads * headdim

    def draw(shape):
        return round_to_bf16(rng.standard_normal(shape, dtype=np.float32))

    u = draw((batch, dim, L))
    delta = draw((batch, nheads, L))
    z = draw((batch, dim, L))
    B = draw((batch, N, L))
    C = draw((batch, N, L))
    D = rng.standard_normal(dim, dtype=np.float32)
    lo, hi = dt_range
    dt = np.exp(rng.uniform(math.log(lo), math.log(hi), size=nheads))
    dt_bias = np.log(np.expm1(dt)).astype(np.float32)
    A = (-rng.uniform(a_range[0], a_range[1], size=nheads)).astype(np.float32)
    return SsdInputs(batch, L, nheads, headdim, N, u, delta, z, B, C, A, D, dt_bias)


def make_ssd_workload(index: int = 5, seed: int | None = None) -> SsdInputs:
    w = SSD_WORKLOADS[index]
    return make_ssd_inputs(w["batch"], w["L"], w["nheads"], w["headdim"], w["N"],
                           seed=WORKLOAD_SEEDS[index] if seed is None else seed, dt_range=w["dt_range"])


def ssd_to_device(x: SsdInputs, device="cuda"):
    """Upload to torch tensors: u/delta/z/B/C bf16, A/D/dt_bias float32."""
    import torch

    bf = lambda a: torch.from_numpy(bf16_bits(a)).view(torch.bfloat16).to(device)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return dict(u=bf(x.u), delta=bf(x.delta), z=bf(x.z), B=bf(x.B), C=bf(x.C), A=f32(x.A), D=f32(x.D),
                dt_bias=f32(x.dt_bias))
