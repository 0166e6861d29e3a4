"""Python binding of libssm.so, the MI355X selective scan (forward, decode step,
backward, fused convolution front end, and the chunked scalar-decay pass with
per-head step sizes).

Argument marshalling only: every step of the scan runs in the HIP kernels of
``csrc/scan_fwd.hip``, ``csrc/scan_bwd.hip`` and ``csrc/ssd_fwd.hip`` behind the C ABI
of ``include/ssm.h``.  There is no CPU or PyTorch fallback: if the library is missing,
every call raises.

The ``ssm_*`` functions carry the C names (see ``EXPORTED``) and take raw device
tensors; ``selective_scan_fwd``, ``selective_scan_step``, ``selective_scan_bwd``,
``selective_scan_fwd_conv``, ``selective_scan_step_conv`` and ``ssd_fwd`` additionally
allocate outputs and the workspace through PyTorch's caching allocator.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libssm.so")

SSM_OK = 0
SSM_ERR_NULL = -1
SSM_ERR_EMPTY = -2
SSM_ERR_DIMS = -3
SSM_ERR_DTYPE = -4
SSM_ERR_ALIGN = -5
SSM_ERR_WORKSPACE = -6
SSM_ERR_HIP = -7
SSM_ERR_ALIAS = -8
SSM_ERR_DEVICE = -9
SSM_ERR_SCRATCH = -10
SSM_F32 = 0
SSM_BF16 = 1
SSM_MAX_DSTATE = 256
SSM_MAX_CHUNKS = 1024

EXPORTED = ("ssm_selective_scan_fwd", "ssm_selective_scan_fwd_state", "ssm_selective_scan_step",
            "ssm_selective_scan_workspace_bytes", "ssm_selective_scan_plan", "ssm_status_string",
            "ssm_selective_scan_bwd", "ssm_selective_scan_bwd_workspace_bytes", "ssm_selective_scan_bwd_plan",
            "ssm_selective_scan_fwd_conv", "ssm_selective_scan_step_conv", "ssm_ssd_fwd",
            "ssm_ssd_fwd_workspace_bytes", "ssm_ssd_fwd_plan", "ssm_selective_scan_ckpt_bytes",
            "ssm_selective_scan_fwd_ckpt", "ssm_selective_scan_bwd_ckpt", "ssm_selective_scan_fwd_noalloc",
            "ssm_selective_scan_noalloc_scratch_bytes")
SSM_MAX_DSTATE_BWD = 128


class SsmDims(ctypes.Structure):
    """Mirror of ``ssm_dims`` in include/ssm.h."""
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("dim", ctypes.c_int64),
        ("dstate", ctypes.c_int64),
        ("nheads", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("nchunks", ctypes.c_int32),
        ("states_per_lane", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class SsmPlan(ctypes.Structure):
    """Mirror of ``ssm_plan`` in include/ssm.h."""
    _fields_ = [
        ("nchunks", ctypes.c_int32),
        ("states_per_lane", ctypes.c_int32),
        ("waves_per_group", ctypes.c_int32),
        ("time_tile", ctypes.c_int32),
        ("chunk_len", ctypes.c_int64),
        ("workgroups", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
        ("lds_bytes", ctypes.c_size_t),
        ("form", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class SsmGrads(ctypes.Structure):
    """Mirror of ``ssm_grads`` in include/ssm.h (device pointers; 0 = NULL)."""
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddt_bias", "dh0")]


class SsmConv(ctypes.Structure):
    """Mirror of ``ssm_conv`` in include/ssm.h."""
    _fields_ = [("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("width", ctypes.c_int32),
                ("silu", ctypes.c_int32)]


class SsmSsdDims(ctypes.Structure):
    """Mirror of ``ssm_ssd_dims`` in include/ssm.h."""
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64),
        ("dstate", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("nsegments", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("reserved2", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class SsmSsdPlan(ctypes.Structure):
    """Mirror of ``ssm_ssd_plan`` in include/ssm.h."""
    _fields_ = [
        ("nsegments", ctypes.c_int32),
        ("chunks_per_segment", ctypes.c_int32),
        ("chunk_len", ctypes.c_int32),
        ("state_pieces", ctypes.c_int32),
        ("nchunks", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class SsmError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {ssm_status_string(status)} (status {status})")
        self.status = status


_lib = None


def load_library():
    """Load libssm.so from the package directory (raises if it was not built).

    torch is imported first: its HIP runtime must be the one libssm.so binds to.  Loaded
    before torch, libssm.so would bring in the system's libamdhip64.so.7 and torch its
    own copy afterwards, two runtimes in one process, and launches on torch's streams
    would then fail."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m selective_state_space_79_amd.build`")
        import torch  # noqa: F401  (binds libamdhip64 before libssm.so needs it)

        lib = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        lib.ssm_selective_scan_fwd.argtypes = [vp] * 9 + [ctypes.POINTER(SsmDims), vp]
        lib.ssm_selective_scan_fwd.restype = ctypes.c_int
        lib.ssm_selective_scan_fwd_state.argtypes = [vp] * 11 + [ctypes.POINTER(SsmDims), vp]
        lib.ssm_selective_scan_fwd_state.restype = ctypes.c_int
        lib.ssm_selective_scan_step.argtypes = [vp] * 10 + [ctypes.POINTER(SsmDims), vp]
        lib.ssm_selective_scan_step.restype = ctypes.c_int
        lib.ssm_selective_scan_workspace_bytes.argtypes = [ctypes.POINTER(SsmDims)]
        lib.ssm_selective_scan_workspace_bytes.restype = ctypes.c_size_t
        lib.ssm_selective_scan_plan.argtypes = [ctypes.POINTER(SsmDims), ctypes.POINTER(SsmPlan)]
        lib.ssm_selective_scan_plan.restype = ctypes.c_int
        lib.ssm_selective_scan_bwd.argtypes = [vp] * 11 + [ctypes.POINTER(SsmGrads), ctypes.POINTER(SsmDims), vp]
        lib.ssm_selective_scan_bwd.restype = ctypes.c_int
        lib.ssm_selective_scan_bwd_workspace_bytes.argtypes = [ctypes.POINTER(SsmDims)]
        lib.ssm_selective_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.ssm_selective_scan_bwd_plan.argtypes = [ctypes.POINTER(SsmDims), ctypes.POINTER(SsmPlan)]
        lib.ssm_selective_scan_bwd_plan.restype = ctypes.c_int
        lib.ssm_selective_scan_fwd_conv.argtypes = [vp, ctypes.POINTER(SsmConv)] + [vp] * 12 + [ctypes.POINTER(SsmDims), vp]
        lib.ssm_selective_scan_fwd_conv.restype = ctypes.c_int
        lib.ssm_selective_scan_step_conv.argtypes = [vp, ctypes.POINTER(SsmConv)] + [vp] * 11 + [ctypes.POINTER(SsmDims), vp]
        lib.ssm_selective_scan_step_conv.restype = ctypes.c_int
        lib.ssm_ssd_fwd.argtypes = [vp] * 11 + [ctypes.POINTER(SsmSsdDims), vp]
        lib.ssm_ssd_fwd.restype = ctypes.c_int
        lib.ssm_ssd_fwd_workspace_bytes.argtypes = [ctypes.POINTER(SsmSsdDims)]
        lib.ssm_ssd_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.ssm_ssd_fwd_plan.argtypes = [ctypes.POINTER(SsmSsdDims), ctypes.POINTER(SsmSsdPlan)]
        lib.ssm_ssd_fwd_plan.restype = ctypes.c_int
        lib.ssm_selective_scan_ckpt_bytes.argtypes = [ctypes.POINTER(SsmDims)]
        lib.ssm_selective_scan_ckpt_bytes.restype = ctypes.c_size_t
        lib.ssm_selective_scan_fwd_ckpt.argtypes = [vp] * 12 + [ctypes.POINTER(SsmDims), vp]
        lib.ssm_selective_scan_fwd_ckpt.restype = ctypes.c_int
        lib.ssm_selective_scan_bwd_ckpt.argtypes = [vp] * 12 + [ctypes.POINTER(SsmGrads), ctypes.POINTER(SsmDims), vp]
        lib.ssm_selective_scan_bwd_ckpt.restype = ctypes.c_int
        lib.ssm_selective_scan_fwd_noalloc.argtypes = [vp] * 11 + [ctypes.POINTER(SsmDims), vp]
        lib.ssm_selective_scan_fwd_noalloc.restype = ctypes.c_int
        lib.ssm_selective_scan_noalloc_scratch_bytes.argtypes = []
        lib.ssm_selective_scan_noalloc_scratch_bytes.restype = ctypes.c_size_t
        lib.ssm_status_string.argtypes = [ctypes.c_int]
        lib.ssm_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def make_dims(batch, seqlen, dim, dstate, *, nheads=0, io_dtype=SSM_BF16, nchunks=0, states_per_lane=0,
              workspace=0, workspace_bytes=0, reserved=0) -> SsmDims:
    return SsmDims(batch, seqlen, dim, dstate, nheads, io_dtype, nchunks, states_per_lane, reserved,
                   workspace or None, workspace_bytes)


def ssm_status_string(status: int) -> str:
    return load_library().ssm_status_string(int(status)).decode()


def ssm_selective_scan_workspace_bytes(dims: SsmDims) -> int:
    return int(load_library().ssm_selective_scan_workspace_bytes(ctypes.byref(dims)))


def ssm_selective_scan_plan(dims: SsmDims) -> SsmPlan:
    plan = SsmPlan()
    st = load_library().ssm_selective_scan_plan(ctypes.byref(dims), ctypes.byref(plan))
    if st != SSM_OK:
        raise SsmError(st, "ssm_selective_scan_plan")
    return plan


def ssm_selective_scan_bwd_workspace_bytes(dims: SsmDims) -> int:
    return int(load_library().ssm_selective_scan_bwd_workspace_bytes(ctypes.byref(dims)))


def ssm_selective_scan_bwd_plan(dims: SsmDims) -> SsmPlan:
    plan = SsmPlan()
    st = load_library().ssm_selective_scan_bwd_plan(ctypes.byref(dims), ctypes.byref(plan))
    if st != SSM_OK:
        raise SsmError(st, "ssm_selective_scan_bwd_plan")
    return plan


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def ssm_selective_scan_fwd(u, delta, A, B, C, D, z, dt_bias, y, dims: SsmDims, stream=None) -> int:
    """Call the C entry point with raw device pointers; returns the status code.

    u, delta, z, y: (batch, dim, L); B, C: (batch, N, L) -- all in the I/O dtype;
    A: float32 (dim, N) or (nheads,); D, dt_bias: float32 (dim,).  D, z and dt_bias
    may be None.  ``stream`` is a torch.cuda.Stream (default: the current stream of
    u's device).
    """
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(u.device)
    return int(load_library().ssm_selective_scan_fwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(y),
        ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream)))


def ssm_selective_scan_fwd_state(u, delta, A, B, C, D, z, dt_bias, h0, y, h_last, dims: SsmDims,
                                 stream=None) -> int:
    """C entry point with a carried state: h0, h_last float32 (batch, dim, N) or None."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(u.device)
    return int(load_library().ssm_selective_scan_fwd_state(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(y),
        _ptr(h_last), ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream)))


def ssm_selective_scan_fwd_noalloc(u, delta, A, B, C, D, z, dt_bias, h0, y, h_last, dims: SsmDims,
                                   stream=None) -> int:
    """C entry point that allocates nothing: ssm_selective_scan_fwd_state with the
    carries between pieces in the library's own per-device scratch (dims' workspace
    fields are ignored)."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(u.device)
    return int(load_library().ssm_selective_scan_fwd_noalloc(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(y),
        _ptr(h_last), ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream)))


def ssm_selective_scan_noalloc_scratch_bytes() -> int:
    return int(load_library().ssm_selective_scan_noalloc_scratch_bytes())


def ssm_selective_scan_ckpt_bytes(dims: SsmDims) -> int:
    return int(load_library().ssm_selective_scan_ckpt_bytes(ctypes.byref(dims)))


def ssm_selective_scan_fwd_ckpt(u, delta, A, B, C, D, z, dt_bias, h0, y, h_last, ckpt, dims: SsmDims,
                                stream=None) -> int:
    """C entry point of the forward that also keeps the state checkpoints (float32
    buffer of ssm_selective_scan_ckpt_bytes(dims) bytes)."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(u.device)
    return int(load_library().ssm_selective_scan_fwd_ckpt(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(y),
        _ptr(h_last), _ptr(ckpt), ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream)))


def ssm_selective_scan_step(u, delta, A, B, C, D, z, dt_bias, h, y, dims: SsmDims, stream=None) -> int:
    """C entry point of one decoding step; h float32 (batch, dim, N) is updated in place."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(u.device)
    return int(load_library().ssm_selective_scan_step(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h), _ptr(y),
        ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream)))


def dims_for(u, B, A, *, nchunks=0, states_per_lane=0) -> SsmDims:
    """ssm_dims for tensors laid out as include/ssm.h describes."""
    import torch

    if u.dim() != 3 or B.dim() != 3:
        raise ValueError("u must be (batch, dim, L) and B (batch, N, L)")
    if u.dtype == torch.bfloat16:
        io = SSM_BF16
    elif u.dtype == torch.float32:
        io = SSM_F32
    else:
        raise TypeError(f"unsupported I/O dtype {u.dtype}")
    batch, dim, L = u.shape
    nheads = A.shape[0] if A.dim() == 1 else 0
    return make_dims(batch, L, dim, B.shape[1], nheads=nheads, io_dtype=io, nchunks=nchunks,
                     states_per_lane=states_per_lane)


def _check_tensors(u, tensors, f32_names=("A", "D", "dt_bias", "h0", "h")):
    import torch

    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if name in f32_names:
            if t.dtype != torch.float32:
                raise TypeError(f"{name} must be float32")
        elif t.dtype != u.dtype:
            raise TypeError(f"{name} must have u's dtype {u.dtype}")


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, dt_bias=None, *, h0=None, return_state=False, out=None,
                       workspace=None, nchunks=0, states_per_lane=0, ckpt=None, stream=None):
    """Allocate y (and the workspace, if the plan needs one) and run the scan.

    Tensors must be contiguous CUDA tensors with the layouts of include/ssm.h.
    h0: optional float32 (batch, dim, N) starting state.  With return_state=True the
    final state is returned too, as (y, h_last).  ckpt: optional float32 device tensor
    of ssm_selective_scan_ckpt_bytes(dims) bytes that receives the state checkpoints
    for selective_scan_bwd (ssm_selective_scan_fwd_ckpt).  Raises SsmError on a
    refused call.
    """
    import torch

    _check_tensors(u, dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, dt_bias=dt_bias, h0=h0, ckpt=ckpt),
                   f32_names=("A", "D", "dt_bias", "h0", "ckpt"))
    dims = dims_for(u, B, A, nchunks=nchunks, states_per_lane=states_per_lane)
    if out is None:
        out = torch.empty_like(u)
    h_last = None
    if return_state:
        h_last = torch.empty((u.shape[0], u.shape[1], B.shape[1]), dtype=torch.float32, device=u.device)
    need = ssm_selective_scan_workspace_bytes(dims)
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
        dims.workspace = workspace.data_ptr()
        dims.workspace_bytes = workspace.numel() * workspace.element_size()
    if ckpt is not None:
        st = ssm_selective_scan_fwd_ckpt(u, delta, A, B, C, D, z, dt_bias, h0, out, h_last, ckpt, dims, stream)
        if st != SSM_OK:
            raise SsmError(st, "ssm_selective_scan_fwd_ckpt")
    else:
        st = ssm_selective_scan_fwd_state(u, delta, A, B, C, D, z, dt_bias, h0, out, h_last, dims, stream)
        if st != SSM_OK:
            raise SsmError(st, "ssm_selective_scan_fwd_state")
    return (out, h_last) if return_state else out


def new_ckpt(u, B, A):
    """A float32 device tensor for the state checkpoints of a forward on these shapes
    (raises SsmError when the shapes have no checkpoint form)."""
    import torch

    n = ssm_selective_scan_ckpt_bytes(dims_for(u, B, A))
    if n == 0:
        raise SsmError(SSM_ERR_DIMS, "ssm_selective_scan_ckpt_bytes")
    return torch.empty(n // 4, dtype=torch.float32, device=u.device)


def selective_scan_step(u, delta, A, B, C, D, z, dt_bias, h, *, out=None, stream=None):
    """One decoding step.  u, delta, z: (batch, dim); B, C: (batch, N); h: float32
    (batch, dim, N), updated in place.  Returns y (batch, dim)."""
    import torch

    _check_tensors(u, dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, dt_bias=dt_bias, h=h))
    if u.dim() != 2 or B.dim() != 2 or h.dim() != 3:
        raise ValueError("u must be (batch, dim), B (batch, N) and h (batch, dim, N)")
    io = SSM_BF16 if u.dtype == torch.bfloat16 else SSM_F32
    dims = make_dims(u.shape[0], 1, u.shape[1], B.shape[1], nheads=A.shape[0] if A.dim() == 1 else 0, io_dtype=io)
    if out is None:
        out = torch.empty_like(u)
    st = ssm_selective_scan_step(u, delta, A, B, C, D, z, dt_bias, h, out, dims, stream)
    if st != SSM_OK:
        raise SsmError(st, "ssm_selective_scan_step")
    return out


def ssm_selective_scan_bwd(u, delta, A, B, C, D, z, dt_bias, h0, dy, dh_last, grads: SsmGrads, dims: SsmDims,
                           stream=None) -> int:
    """C entry point of the backward pass with raw device pointers; returns the status."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(u.device)
    return int(load_library().ssm_selective_scan_bwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(dy),
        _ptr(dh_last), ctypes.byref(grads), ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream)))


def ssm_selective_scan_bwd_ckpt(u, delta, A, B, C, D, z, dt_bias, h0, dy, dh_last, ckpt, grads: SsmGrads,
                                dims: SsmDims, stream=None) -> int:
    """C entry point of the backward from the forward's state checkpoints."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(u.device)
    return int(load_library().ssm_selective_scan_bwd_ckpt(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(dy),
        _ptr(dh_last), _ptr(ckpt), ctypes.byref(grads), ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream)))


def selective_scan_bwd(u, delta, A, B, C, D=None, z=None, dt_bias=None, *, dy, h0=None, dh_last=None,
                       nchunks=0, states_per_lane=0, workspace=None, ckpt=None, stream=None) -> dict:
    """Gradients of sum(dy * y) + sum(dh_last * h_last) for the forward with the same
    inputs.  Allocates the outputs (and the workspace) with torch; returns a dict with
    du, ddelta (u's dtype), dA, dB, dC, dD, ddt_bias, dh0 (float32) and dz (when z is
    given).  ckpt: the checkpoints a selective_scan_fwd(..., ckpt=...) call kept for
    the same inputs (the backward then skips recomputing them).  Raises SsmError on a
    refused call."""
    import torch

    _check_tensors(u, dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, dt_bias=dt_bias, h0=h0, dy=dy,
                           dh_last=dh_last, ckpt=ckpt), f32_names=("A", "D", "dt_bias", "h0", "dh_last", "ckpt"))
    dims = dims_for(u, B, A, nchunks=nchunks, states_per_lane=states_per_lane)
    batch, dim, L = u.shape
    N = B.shape[1]
    f32 = dict(dtype=torch.float32, device=u.device)
    out = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u), "dA": torch.empty(A.shape, **f32),
           "dB": torch.empty((batch, N, L), **f32), "dC": torch.empty((batch, N, L), **f32),
           "dD": torch.empty(dim, **f32), "ddt_bias": torch.empty(dim, **f32),
           "dh0": torch.empty((batch, dim, N), **f32)}
    if z is not None:
        out["dz"] = torch.empty_like(u)
    need = ssm_selective_scan_bwd_workspace_bytes(dims)
    if need == 0:
        raise SsmError(SSM_ERR_DIMS, "ssm_selective_scan_bwd_workspace_bytes")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
    dims.workspace = workspace.data_ptr()
    dims.workspace_bytes = workspace.numel() * workspace.element_size()
    g = SsmGrads(*[out[k].data_ptr() if k in out else None for k, _ in SsmGrads._fields_])
    if ckpt is not None:
        st = ssm_selective_scan_bwd_ckpt(u, delta, A, B, C, D, z, dt_bias, h0, dy, dh_last, ckpt, g, dims, stream)
        if st != SSM_OK:
            raise SsmError(st, "ssm_selective_scan_bwd_ckpt")
    else:
        st = ssm_selective_scan_bwd(u, delta, A, B, C, D, z, dt_bias, h0, dy, dh_last, g, dims, stream)
        if st != SSM_OK:
            raise SsmError(st, "ssm_selective_scan_bwd")
    return out


def _conv_struct(weight, bias, silu):
    return SsmConv(weight.data_ptr(), bias.data_ptr() if bias is not None else None, weight.shape[1], int(bool(silu)))


def ssm_selective_scan_fwd_conv(x, conv: SsmConv, conv_state, delta, A, B, C, D, z, dt_bias, h0, u_out, y, h_last,
                                dims: SsmDims, stream=None) -> int:
    """C entry point of the scan with the fused convolution front end; returns the status."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    return int(load_library().ssm_selective_scan_fwd_conv(
        _ptr(x), ctypes.byref(conv), _ptr(conv_state), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(dt_bias), _ptr(h0), _ptr(u_out), _ptr(y), _ptr(h_last), ctypes.byref(dims),
        ctypes.c_void_p(stream.cuda_stream)))


def ssm_selective_scan_step_conv(x, conv: SsmConv, conv_state, delta, A, B, C, D, z, dt_bias, h, u_out, y,
                                 dims: SsmDims, stream=None) -> int:
    """C entry point of one fused convolution + scan decoding step; returns the status."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    return int(load_library().ssm_selective_scan_step_conv(
        _ptr(x), ctypes.byref(conv), _ptr(conv_state), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(dt_bias), _ptr(h), _ptr(u_out), _ptr(y), ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream)))


def selective_scan_fwd_conv(x, conv_weight, conv_bias, delta, A, B, C, D=None, z=None, dt_bias=None, *, silu=True,
                            conv_state=None, h0=None, return_state=False, return_u=False, out=None, workspace=None,
                            nchunks=0, states_per_lane=0, stream=None):
    """Scan of u = act(conv(x)) with the convolution fused into the scan's staging.
    conv_weight float32 (dim, width <= 4), conv_bias float32 (dim,) or None.  Returns y,
    or a tuple (y, h_last, u) with the pieces asked for by return_state / return_u."""
    import torch

    _check_tensors(x, dict(x=x, delta=delta, A=A, B=B, C=C, D=D, z=z, dt_bias=dt_bias, h0=h0,
                           conv_weight=conv_weight, conv_bias=conv_bias, conv_state=conv_state),
                   f32_names=("A", "D", "dt_bias", "h0", "conv_weight", "conv_bias"))
    dims = dims_for(x, B, A, nchunks=nchunks, states_per_lane=states_per_lane)
    if out is None:
        out = torch.empty_like(x)
    h_last = torch.empty((x.shape[0], x.shape[1], B.shape[1]), dtype=torch.float32, device=x.device) \
        if return_state else None
    u = torch.empty_like(x) if return_u else None
    need = ssm_selective_scan_workspace_bytes(dims)
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        dims.workspace = workspace.data_ptr()
        dims.workspace_bytes = workspace.numel() * workspace.element_size()
    conv = _conv_struct(conv_weight, conv_bias, silu)
    st = ssm_selective_scan_fwd_conv(x, conv, conv_state, delta, A, B, C, D, z, dt_bias, h0, u, out, h_last, dims,
                                     stream)
    if st != SSM_OK:
        raise SsmError(st, "ssm_selective_scan_fwd_conv")
    if not (return_state or return_u):
        return out
    return tuple(v for v, want in ((out, True), (h_last, return_state), (u, return_u)) if want)


def selective_scan_step_conv(x, conv_weight, conv_bias, conv_state, delta, A, B, C, D, z, dt_bias, h, *, silu=True,
                             return_u=False, out=None, stream=None):
    """One decoding step with the fused convolution: conv_state (batch, dim, width-1)
    and h are updated in place.  Returns y (and u when return_u)."""
    import torch

    _check_tensors(x, dict(x=x, delta=delta, A=A, B=B, C=C, D=D, z=z, dt_bias=dt_bias, h=h,
                           conv_weight=conv_weight, conv_bias=conv_bias, conv_state=conv_state),
                   f32_names=("A", "D", "dt_bias", "h", "conv_weight", "conv_bias"))
    io = SSM_BF16 if x.dtype == torch.bfloat16 else SSM_F32
    dims = make_dims(x.shape[0], 1, x.shape[1], B.shape[1], nheads=A.shape[0] if A.dim() == 1 else 0, io_dtype=io)
    if out is None:
        out = torch.empty_like(x)
    u = torch.empty_like(x) if return_u else None
    conv = _conv_struct(conv_weight, conv_bias, silu)
    st = ssm_selective_scan_step_conv(x, conv, conv_state, delta, A, B, C, D, z, dt_bias, h, u, out, dims, stream)
    if st != SSM_OK:
        raise SsmError(st, "ssm_selective_scan_step_conv")
    return (out, u) if return_u else out


def make_ssd_dims(batch, seqlen, nheads, dstate, *, headdim=64, io_dtype=SSM_BF16, nsegments=0, workspace=0,
                  workspace_bytes=0, reserved=0) -> SsmSsdDims:
    return SsmSsdDims(batch, seqlen, nheads, headdim, dstate, io_dtype, nsegments, reserved, 0, workspace or None,
                      workspace_bytes)


def ssm_ssd_fwd_workspace_bytes(dims: SsmSsdDims) -> int:
    return int(load_library().ssm_ssd_fwd_workspace_bytes(ctypes.byref(dims)))


def ssm_ssd_fwd_plan(dims: SsmSsdDims) -> SsmSsdPlan:
    plan = SsmSsdPlan()
    st = load_library().ssm_ssd_fwd_plan(ctypes.byref(dims), ctypes.byref(plan))
    if st != SSM_OK:
        raise SsmError(st, "ssm_ssd_fwd_plan")
    return plan


def ssm_ssd_fwd(u, delta, A, B, C, D, z, dt_bias, h0, y, h_last, dims: SsmSsdDims, stream=None) -> int:
    """C entry point of the chunked scalar-decay pass with per-head step sizes; returns
    the status.  u, z, y (batch, nheads*headdim, L), delta (batch, nheads, L), B, C
    (batch, N, L) bf16; A, dt_bias float32 (nheads,); D float32 (dim,); h0, h_last
    float32 (batch, dim, N) or None."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(u.device)
    return int(load_library().ssm_ssd_fwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(y),
        _ptr(h_last), ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream)))


def ssd_fwd(u, delta, A, B, C, D=None, z=None, dt_bias=None, *, h0=None, return_state=False, out=None,
            workspace=None, nsegments=0, stream=None):
    """Allocate y (and the workspace) and run ssm_ssd_fwd.  Returns y, or (y, h_last)
    with return_state=True.  Raises SsmError on a refused call."""
    import torch

    _check_tensors(u, dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, dt_bias=dt_bias, h0=h0))
    if u.dim() != 3 or delta.dim() != 3 or B.dim() != 3 or A.dim() != 1:
        raise ValueError("u (batch, dim, L), delta (batch, nheads, L), B (batch, N, L) and A (nheads,) expected")
    if u.dtype != torch.bfloat16:
        raise TypeError("the chunked pass takes bf16 inputs")
    batch, dim, L = u.shape
    nheads = delta.shape[1]
    if dim % nheads:
        raise ValueError("dim must be a multiple of nheads")
    dims = make_ssd_dims(batch, L, nheads, B.shape[1], headdim=dim // nheads, nsegments=nsegments)
    if out is None:
        out = torch.empty_like(u)
    h_last = torch.empty((batch, dim, B.shape[1]), dtype=torch.float32, device=u.device) if return_state else None
    need = ssm_ssd_fwd_workspace_bytes(dims)
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
        dims.workspace = workspace.data_ptr()
        dims.workspace_bytes = workspace.numel() * workspace.element_size()
    st = ssm_ssd_fwd(u, delta, A, B, C, D, z, dt_bias, h0, out, h_last, dims, stream)
    if st != SSM_OK:
        raise SsmError(st, "ssm_ssd_fwd")
    return (out, h_last) if return_state else out
