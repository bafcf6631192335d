"""ctypes binding of libfwmem (include/fwmem.h).

Argument marshalling only: every step of the scan and of the decode runs in the
library's HIP kernels. Tensors are torch device tensors; the library receives
their raw pointers and the current HIP stream. There is no fallback: if the
library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# FWMEM_LIB names another build of the same library (the host-sanitizer build of the ABI
# checks); by default the in-tree libfwmem.so
LIB_PATH = os.environ.get("FWMEM_LIB") or os.path.join(PKG, "libfwmem.so")

OK, EINVAL, EUNSUPPORTED, EALIGN, EOVERLAP, ELAUNCH, EWORKSPACE = 0, -1, -2, -3, -4, -5, -6
EWAIT, ESCRATCH = -7, -8
NOALLOC_SCRATCH_BYTES = 64 << 20  # FWMEM_NOALLOC_SCRATCH_BYTES
RULE_DELTA, RULE_ADDITIVE, RULE_INNER, RULE_DELTA_PV = 0, 1, 2, 3
F32, BF16 = 0, 1
PHI_ELU1 = 1 << 0
LAMBDA_PER_CHANNEL = 1 << 1
OUT_BF16 = 1 << 2
QK_L2NORM = 1 << 3
QK_RMSNORM = 1 << 4
BETA_SIGMOID = 1 << 5
BETA_SIGMOID2 = 1 << 6
LAMBDA_PREACT = 1 << 7
ZNORM = 1 << 8
LAMBDA_SCALED = 1 << 9

EXPORTED = ["fwmem_state_bytes", "fwmem_scan_workspace_bytes", "fwmem_scan_fwd",
            "fwmem_scan_chunk_prep", "fwmem_scan_chunk_propagate", "fwmem_step",
            "fwmem_scan_bwd_workspace_bytes", "fwmem_scan_bwd", "fwmem_strerror", "fwmem_version",
            "fwmem_scan_fwd_noalloc", "fwmem_check_device"]
PHASE_BOTH, PHASE_PREP, PHASE_PROPAGATE = "fwmem_scan_fwd", "fwmem_scan_chunk_prep", "fwmem_scan_chunk_propagate"


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Mode(ctypes.Structure):
    _fields_ = [("rule", ctypes.c_int32), ("flags", ctypes.c_uint32), ("eps", ctypes.c_float),
                ("chunk", ctypes.c_int32)]


class FwmemError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {strerror(status)} ({status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfwmem.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"libfwmem not built: {path} (run python -m linear_attention_scan_amd.build)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.fwmem_state_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(sz)]
    lib.fwmem_state_bytes.restype = ctypes.c_int
    lib.fwmem_scan_workspace_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Mode),
                                               ctypes.POINTER(sz)]
    lib.fwmem_scan_workspace_bytes.restype = ctypes.c_int
    for name in (PHASE_BOTH, PHASE_PREP, PHASE_PROPAGATE):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, ctypes.POINTER(Mode), vp, vp, vp,
                       vp, sz, vp]
        fn.restype = ctypes.c_int
    lib.fwmem_scan_fwd_noalloc.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp,
                                           ctypes.POINTER(Mode), vp, vp, vp, vp]
    lib.fwmem_scan_fwd_noalloc.restype = ctypes.c_int
    lib.fwmem_step.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, ctypes.POINTER(Mode),
                               vp, vp, vp, vp]
    lib.fwmem_step.restype = ctypes.c_int
    lib.fwmem_scan_bwd_workspace_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Mode),
                                                   ctypes.POINTER(sz)]
    lib.fwmem_scan_bwd_workspace_bytes.restype = ctypes.c_int
    lib.fwmem_scan_bwd.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, ctypes.POINTER(Mode),
                                   vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fwmem_scan_bwd.restype = ctypes.c_int
    lib.fwmem_check_device.argtypes = [vp]
    lib.fwmem_check_device.restype = ctypes.c_int
    lib.fwmem_strerror.argtypes = [ctypes.c_int]
    lib.fwmem_strerror.restype = ctypes.c_char_p
    lib.fwmem_version.argtypes = []
    lib.fwmem_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().fwmem_strerror(int(status)).decode()


def version() -> str:
    return load().fwmem_version().decode()


def check_device(stream=None) -> int:
    """fwmem_check_device: synchronise the stream, read and clear the GPU's sticky wait
    status; returns OK or EWAIT (ELAUNCH if it could not be read)."""
    return load().fwmem_check_device(_stream(stream))


def shape(B, H, T, dk, dv, dtype) -> Shape:
    return Shape(int(B), int(H), int(T), int(dk), int(dv), int(dtype))


def mode(rule=RULE_DELTA, flags=0, eps=1e-6, chunk=0) -> Mode:
    return Mode(int(rule), int(flags), float(eps), int(chunk))


def state_bytes(shp: Shape) -> int:
    n = ctypes.c_size_t(0)
    st = load().fwmem_state_bytes(ctypes.byref(shp), ctypes.byref(n))
    if st != OK:
        raise FwmemError(st, "fwmem_state_bytes")
    return n.value


def workspace_bytes(shp: Shape, md: Mode) -> int:
    n = ctypes.c_size_t(0)
    st = load().fwmem_scan_workspace_bytes(ctypes.byref(shp), ctypes.byref(md), ctypes.byref(n))
    if st != OK:
        raise FwmemError(st, "fwmem_scan_workspace_bytes")
    return n.value


def bwd_workspace_bytes(shp: Shape, md: Mode) -> int:
    n = ctypes.c_size_t(0)
    st = load().fwmem_scan_bwd_workspace_bytes(ctypes.byref(shp), ctypes.byref(md), ctypes.byref(n))
    if st != OK:
        raise FwmemError(st, "fwmem_scan_bwd_workspace_bytes")
    return n.value


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def scan_fwd_raw(shp: Shape, q, k, v, beta, lam, md: Mode, S_in, out, S_out, workspace,
                 ws_bytes: int, stream=None, entry: str = PHASE_BOTH) -> int:
    """Call fwmem_scan_fwd (or one of its two phases, by entry-point name) with tensors
    (or raw ints / None) and return the status."""
    fn = getattr(load(), entry)
    return fn(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(lam),
              ctypes.byref(md), _ptr(S_in), _ptr(out), _ptr(S_out), _ptr(workspace),
              int(ws_bytes), _stream(stream))


def scan_fwd_noalloc_raw(shp: Shape, q, k, v, beta, lam, md: Mode, S_in, out, S_out,
                         stream=None) -> int:
    """Call fwmem_scan_fwd_noalloc (the scan with the library's fixed device scratch as its
    workspace) with tensors (or raw ints / None) and return the status."""
    return load().fwmem_scan_fwd_noalloc(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(beta), _ptr(lam), ctypes.byref(md), _ptr(S_in),
                                         _ptr(out), _ptr(S_out), _stream(stream))


def step_raw(shp: Shape, q, k, v, beta, lam, md: Mode, S_in, out, S_out, stream=None) -> int:
    """Call fwmem_step with tensors (or raw ints / None) and return the status."""
    return load().fwmem_step(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(lam),
                             ctypes.byref(md), _ptr(S_in), _ptr(out), _ptr(S_out), _stream(stream))


def scan_bwd_raw(shp: Shape, q, k, v, beta, lam, md: Mode, S_in, grad_out, grad_S_out, grad_q,
                 grad_k, grad_v, grad_beta, grad_lam, grad_S_in, workspace, ws_bytes: int,
                 stream=None) -> int:
    """Call fwmem_scan_bwd with tensors (or raw ints / None) and return the status."""
    return load().fwmem_scan_bwd(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                 _ptr(lam), ctypes.byref(md), _ptr(S_in), _ptr(grad_out),
                                 _ptr(grad_S_out), _ptr(grad_q), _ptr(grad_k), _ptr(grad_v),
                                 _ptr(grad_beta), _ptr(grad_lam), _ptr(grad_S_in),
                                 _ptr(workspace), int(ws_bytes), _stream(stream))


# ----------------------------------------------------------------- torch conveniences

class State:
    """A device state buffer with views S [B,H,dk,dv], x_prev [B,H,dk], has_prev [B,H]."""

    def __init__(self, B, H, dk, dv, device="cuda"):
        import torch
        self.B, self.H, self.dk, self.dv = B, H, dk, dv
        nbytes = state_bytes(shape(B, H, 0, dk, dv, F32))
        self.buf = torch.zeros(nbytes // 4, dtype=torch.float32, device=device)
        nS, nX = B * H * dk * dv, B * H * dk
        self.S = self.buf[:nS].view(B, H, dk, dv)
        self.x_prev = self.buf[nS:nS + nX].view(B, H, dk)
        self.has_prev = self.buf[nS + nX:nS + nX + B * H].view(torch.int32).view(B, H)

    def data_ptr(self) -> int:
        return self.buf.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def scan_fwd(q, k, v, beta=None, lam=None, *, rule=RULE_DELTA, flags=0, eps=1e-6, chunk=0,
             S_in: Optional[State] = None, S_out: Optional[State] = None, out=None,
             workspace=None, stream=None):
    """Whole-sequence scan on device tensors q, k [B,H,T,dk], v [B,H,T,dv].

    Allocates `out` (fp32, or bf16 with OUT_BF16), the workspace and, when S_out is
    None, a fresh output State. Returns (out, S_out)."""
    import torch
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    shp = shape(B, H, T, dk, dv, _dtype_code(q))
    md = mode(rule, flags, eps, chunk)
    if out is None:
        odt = torch.bfloat16 if flags & OUT_BF16 else torch.float32
        out = torch.empty((B, H, T, dv), dtype=odt, device=q.device)
    if S_out is None:
        S_out = State(B, H, dk, dv, device=q.device)
    need = workspace_bytes(shp, md)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = scan_fwd_raw(shp, q, k, v, beta, lam, md, S_in.buf if S_in is not None else None, out,
                      S_out.buf, workspace, workspace.numel(), stream)
    if st != OK:
        raise FwmemError(st, "fwmem_scan_fwd")
    return out, S_out


def step(q, k, v, beta=None, lam=None, *, rule=RULE_DELTA, flags=0, eps=1e-6,
         S_in: Optional[State] = None, S_out: Optional[State] = None, out=None, stream=None):
    """One decode step on device tensors q, k [B,H,dk], v [B,H,dv]; returns (out, S_out)."""
    import torch
    B, H, dk = q.shape
    dv = v.shape[-1]
    shp = shape(B, H, 1, dk, dv, _dtype_code(q))
    md = mode(rule, flags, eps, 0)
    if out is None:
        odt = torch.bfloat16 if flags & OUT_BF16 else torch.float32
        out = torch.empty((B, H, dv), dtype=odt, device=q.device)
    if S_out is None:
        S_out = State(B, H, dk, dv, device=q.device)
    st = step_raw(shp, q, k, v, beta, lam, md, S_in.buf if S_in is not None else None, out,
                  S_out.buf, stream)
    if st != OK:
        raise FwmemError(st, "fwmem_step")
    return out, S_out


def scan_bwd(q, k, v, beta, lam, grad_out, *, rule=RULE_DELTA, flags=0, eps=1e-6,
             S_in: Optional[State] = None, grad_S_out: Optional[State] = None,
             workspace=None, stream=None):
    """Backward pass of scan_fwd for L = <grad_out, out> + <grad_S_out.S, S_T>.

    Allocates the gradients and the workspace. Returns a dict of float32 device tensors:
    "q", "k", "v", "beta" and "lam" (None where the input is None) and "state" (a State
    holding dL/dS_0 and dL/dx_prev)."""
    import torch
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    shp = shape(B, H, T, dk, dv, _dtype_code(q))
    md = mode(rule, flags, eps, 0)
    dev = q.device
    g = {"q": torch.empty((B, H, T, dk), dtype=torch.float32, device=dev),
         "k": torch.empty((B, H, T, dk), dtype=torch.float32, device=dev),
         "v": torch.empty((B, H, T, dv), dtype=torch.float32, device=dev),
         "beta": None if beta is None else torch.empty(tuple(beta.shape), dtype=torch.float32, device=dev),
         "lam": None if lam is None else torch.empty(tuple(lam.shape), dtype=torch.float32, device=dev),
         "state": State(B, H, dk, dv, device=dev)}
    need = bwd_workspace_bytes(shp, md)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = scan_bwd_raw(shp, q, k, v, beta, lam, md, S_in.buf if S_in is not None else None,
                      grad_out, grad_S_out.buf if grad_S_out is not None else None, g["q"],
                      g["k"], g["v"], g["beta"], g["lam"], g["state"].buf, workspace,
                      workspace.numel(), stream)
    if st != OK:
        raise FwmemError(st, "fwmem_scan_bwd")
    return g
