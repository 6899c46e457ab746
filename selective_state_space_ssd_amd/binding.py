"""ctypes binding of ``libssd.so`` (the C ABI in ``include/ssd.h``).

This module only marshals arguments: it checks tensor shapes, dtypes and
devices, allocates the outputs and the workspace with torch, and passes raw
device pointers plus torch's current HIP stream to ``ssd_scan_fwd``.  Every
step of the scan runs in the HIP kernels; there is no other code path, and a
missing library is an error.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssd.so")

SSD_F32 = 0
SSD_BF16 = 1
SSD_NUM_STAGES = 4
STAGES = ("prep", "chunk_state", "state_passing", "chunk_scan")
# Kernel paths of ssd_scan_fwd_path (SSD_PATH_* in include/ssd.h)
KERNEL_PATHS = {"auto": 0, "staged": 1, "fused": 2, "fused_head": 3, "fused_group": 4,
                "chain": 5, "chain_segmented": 7}
SSD_ERR_WAIT = -6
NOALLOC_SCRATCH_BYTES = 64 << 20  # SSD_NOALLOC_SCRATCH_BYTES

_lib = None


class SsdError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"ssd_scan_fwd failed: {message} (status {status})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load ``libssd.so``.  torch is imported first so that the library binds
    to the HIP runtime torch already loaded (both carry the same soname), and
    torch's streams are valid handles for it."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (binds the HIP runtime first)
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with __graft_entry__.build() "
            "(python -m selective_state_space_ssd_amd._build); there is no fallback path")
    lib = ctypes.CDLL(path)
    p, i64, f, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    fwd_args = [p, p, p, p, p, p, p, p, f, f, i, i, p, p, p, i64, i64, i64, i64, i64, i, p,
                ctypes.c_size_t, p]
    lib.ssd_scan_fwd.argtypes = fwd_args
    lib.ssd_scan_fwd.restype = i
    lib.ssd_scan_fwd_timed.argtypes = fwd_args + [p]
    lib.ssd_scan_fwd_timed.restype = i
    lib.ssd_scan_fwd_varlen.argtypes = fwd_args[:15] + [p] + fwd_args[15:]
    lib.ssd_scan_fwd_varlen.restype = i
    lib.ssd_scan_fwd_varlen_workspace_size.argtypes = [i64, i64, i64, i64, i64, i, i, i]
    lib.ssd_scan_fwd_varlen_workspace_size.restype = ctypes.c_size_t
    lib.ssd_scan_fwd_path.argtypes = fwd_args[:15] + [p] + fwd_args[15:21] + [i] + fwd_args[21:]
    lib.ssd_scan_fwd_path.restype = i
    lib.ssd_scan_fwd_path_workspace_size.argtypes = [i64, i64, i64, i64, i64, i, i, i, i, i]
    lib.ssd_scan_fwd_path_workspace_size.restype = ctypes.c_size_t
    lib.ssd_scan_fwd_wait_status.argtypes = [p, ctypes.c_size_t, i64, i64, i64, i64, i64, i, i,
                                             i, i, i, p]
    lib.ssd_scan_fwd_wait_status.restype = i
    lib.ssd_scan_fwd_noalloc.argtypes = fwd_args[:21] + [p]
    lib.ssd_scan_fwd_noalloc.restype = i
    lib.ssd_scan_fwd_taken_path.argtypes = [i64, i64, i64, i64, i64, i, i, i, i, i]
    lib.ssd_scan_fwd_taken_path.restype = i
    lib.ssd_split_conv1d_scan_fwd.argtypes = (
        [p, p, p, p, p, p, i, p, f, f, p, f, i64, i, i, p, p, i64, i64, i64, i64, i, i, p,
         ctypes.c_size_t, p])
    lib.ssd_split_conv1d_scan_fwd.restype = i
    lib.ssd_scan_bwd.argtypes = ([p] * 8 + [f, f, i, i] + [p] * 12 + [i64] * 5 +
                                 [i, p, ctypes.c_size_t, p])
    lib.ssd_scan_bwd.restype = i
    lib.ssd_scan_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i, i, i]
    lib.ssd_scan_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ssd_split_conv1d_scan_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i, i, i,
                                                             i, i]
    lib.ssd_split_conv1d_scan_fwd_workspace_size.restype = ctypes.c_size_t
    lib.ssd_scan_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i, i, i]
    lib.ssd_scan_fwd_workspace_size.restype = ctypes.c_size_t
    lib.ssd_status_string.argtypes = [i]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_abi_version.argtypes = []
    lib.ssd_abi_version.restype = i
    lib.ssd_timing_create.argtypes = [ctypes.POINTER(p)]
    lib.ssd_timing_create.restype = i
    lib.ssd_timing_destroy.argtypes = [p]
    lib.ssd_timing_destroy.restype = i
    lib.ssd_timing_read.argtypes = [p, ctypes.POINTER(ctypes.c_float)]
    lib.ssd_timing_read.restype = i
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ssd_status_string(int(status)).decode()


def abi_version() -> int:
    return int(load_library().ssd_abi_version())


def path_code(name: str) -> int:
    """SSD_PATH_* code of a kernel path name ("auto", "staged", "fused",
    "fused_head", "fused_group" or "chain")."""
    if name not in KERNEL_PATHS:
        raise ValueError(f"unknown kernel path {name!r}; one of {sorted(KERNEL_PATHS)}")
    return KERNEL_PATHS[name]


def workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype,
                   kernel_path: str = "auto") -> int:
    """Workspace bytes of a call on kernel path ``kernel_path``."""
    lib = load_library()
    if kernel_path == "auto":
        return int(lib.ssd_scan_fwd_workspace_size(
            batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype))
    return int(lib.ssd_scan_fwd_path_workspace_size(
        batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, 0,
        path_code(kernel_path)))


def varlen_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size,
                          dtype, kernel_path: str = "auto") -> int:
    """Workspace bytes of a packed-sequence (seq_idx) call."""
    lib = load_library()
    if kernel_path == "auto":
        return int(lib.ssd_scan_fwd_varlen_workspace_size(
            batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype))
    return int(lib.ssd_scan_fwd_path_workspace_size(
        batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, 1,
        path_code(kernel_path)))


def taken_path(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, varlen=False,
               kernel_path: str = "auto") -> str:
    """Name of the kernel path a call with these arguments takes ("staged",
    "staged_scan", "fused_head", "fused_group", "chain", "chain_segmented" or "step"); raises
    SsdError for arguments the call would reject."""
    code = int(load_library().ssd_scan_fwd_taken_path(
        int(batch), int(seqlen), int(nheads), int(headdim), int(dstate), int(ngroups),
        int(chunk_size), int(dtype), 1 if varlen else 0, path_code(kernel_path)))
    if code < 0:
        raise SsdError(code, status_string(code))
    names = {v: k for k, v in KERNEL_PATHS.items()}
    names[6] = "step"
    names[8] = "staged_scan"
    return names[code]


def wait_status(workspace_ptr, workspace_bytes, batch, seqlen, nheads, headdim, dstate, ngroups,
                chunk_size, dtype, varlen=False, kernel_path: str = "auto", stream=None) -> int:
    """ssd_scan_fwd_wait_status: synchronizes ``stream`` (torch's current one by
    default) and returns SSD_OK (0) or SSD_ERR_WAIT when a fused-path
    workgroup of the last call on this workspace gave up waiting."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    return int(load_library().ssd_scan_fwd_wait_status(
        workspace_ptr, int(workspace_bytes), int(batch), int(seqlen), int(nheads), int(headdim),
        int(dstate), int(ngroups), int(chunk_size), int(dtype), 1 if varlen else 0,
        path_code(kernel_path), stream))


def block_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype,
                         conv_width=4, norm_groups=1) -> int:
    """Workspace bytes of a block call (split + conv1d, scan, gated RMSNorm)."""
    return int(load_library().ssd_split_conv1d_scan_fwd_workspace_size(
        batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, conv_width,
        norm_groups))


def bwd_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size,
                       dtype=SSD_F32) -> int:
    """Workspace bytes of a backward call."""
    return int(load_library().ssd_scan_bwd_workspace_size(
        batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype))


def _check(status: int):
    if status != 0:
        raise SsdError(status, status_string(status))


class Timing:
    """Per-stage HIP-event timing of one ``scan_fwd`` call (see ssd_timing_*)."""

    def __init__(self):
        lib = load_library()
        h = ctypes.c_void_p()
        _check(lib.ssd_timing_create(ctypes.byref(h)))
        self.handle = h

    def read(self):
        """Milliseconds per stage, in STAGES order (waits for the events)."""
        buf = (ctypes.c_float * SSD_NUM_STAGES)()
        _check(load_library().ssd_timing_read(self.handle, buf))
        return [float(v) for v in buf]

    def __del__(self):
        if getattr(self, "handle", None) is not None and _lib is not None:
            _lib.ssd_timing_destroy(self.handle)
            self.handle = None


def scan_fwd_raw(x_ptr, dt_ptr, A_ptr, B_ptr, C_ptr, D_ptr, z_ptr, dt_bias_ptr, dt_min, dt_max,
                 chunk_size, ngroups, init_ptr, out_ptr, final_ptr, batch, seqlen, nheads,
                 headdim, dstate, dtype, ws_ptr, ws_bytes, stream, timing: Optional[Timing] = None
                 ) -> int:
    """Direct call of the C entry point with integer pointers; returns the status."""
    lib = load_library()
    args = (x_ptr, dt_ptr, A_ptr, B_ptr, C_ptr, D_ptr, z_ptr, dt_bias_ptr, float(dt_min),
            float(dt_max), int(chunk_size), int(ngroups), init_ptr, out_ptr, final_ptr,
            int(batch), int(seqlen), int(nheads), int(headdim), int(dstate), int(dtype), ws_ptr,
            int(ws_bytes), stream)
    if timing is None:
        return int(lib.ssd_scan_fwd(*args))
    return int(lib.ssd_scan_fwd_timed(*args, timing.handle))


def scan_fwd_path_raw(x_ptr, dt_ptr, A_ptr, B_ptr, C_ptr, D_ptr, z_ptr, dt_bias_ptr, dt_min,
                      dt_max, chunk_size, ngroups, init_ptr, out_ptr, final_ptr, seq_ptr, batch,
                      seqlen, nheads, headdim, dstate, dtype, kernel_path, ws_ptr, ws_bytes,
                      stream) -> int:
    """Direct call of ``ssd_scan_fwd_path`` (``kernel_path`` a name or an
    SSD_PATH_* code; ``seq_ptr`` may be None); returns the status."""
    code = path_code(kernel_path) if isinstance(kernel_path, str) else int(kernel_path)
    return int(load_library().ssd_scan_fwd_path(
        x_ptr, dt_ptr, A_ptr, B_ptr, C_ptr, D_ptr, z_ptr, dt_bias_ptr, float(dt_min),
        float(dt_max), int(chunk_size), int(ngroups), init_ptr, out_ptr, final_ptr, seq_ptr,
        int(batch), int(seqlen), int(nheads), int(headdim), int(dstate), int(dtype), code, ws_ptr,
        int(ws_bytes), stream))


def scan_fwd_noalloc_raw(x_ptr, dt_ptr, A_ptr, B_ptr, C_ptr, D_ptr, z_ptr, dt_bias_ptr, dt_min,
                         dt_max, chunk_size, ngroups, init_ptr, out_ptr, final_ptr, batch, seqlen,
                         nheads, headdim, dstate, dtype, stream) -> int:
    """Direct call of ``ssd_scan_fwd_noalloc`` (no workspace argument: the
    library's own scratch); returns the status."""
    return int(load_library().ssd_scan_fwd_noalloc(
        x_ptr, dt_ptr, A_ptr, B_ptr, C_ptr, D_ptr, z_ptr, dt_bias_ptr, float(dt_min),
        float(dt_max), int(chunk_size), int(ngroups), init_ptr, out_ptr, final_ptr, int(batch),
        int(seqlen), int(nheads), int(headdim), int(dstate), int(dtype), stream))


def scan_fwd_varlen_raw(x_ptr, dt_ptr, A_ptr, B_ptr, C_ptr, D_ptr, z_ptr, dt_bias_ptr, dt_min,
                        dt_max, chunk_size, ngroups, init_ptr, out_ptr, final_ptr, seq_ptr, batch,
                        seqlen, nheads, headdim, dstate, dtype, ws_ptr, ws_bytes, stream) -> int:
    """Direct call of ``ssd_scan_fwd_varlen`` with integer pointers; returns the status."""
    return int(load_library().ssd_scan_fwd_varlen(
        x_ptr, dt_ptr, A_ptr, B_ptr, C_ptr, D_ptr, z_ptr, dt_bias_ptr, float(dt_min),
        float(dt_max), int(chunk_size), int(ngroups), init_ptr, out_ptr, final_ptr, seq_ptr,
        int(batch), int(seqlen), int(nheads), int(headdim), int(dstate), int(dtype), ws_ptr,
        int(ws_bytes), stream))


def _ptr(t):
    return None if t is None else t.data_ptr()


def scan_bwd_raw(x_ptr, dt_ptr, A_ptr, B_ptr, C_ptr, D_ptr, z_ptr, dt_bias_ptr, dt_min, dt_max,
                 chunk_size, ngroups, init_ptr, dout_ptr, dfinal_ptr, dx_ptr, ddt_ptr, dA_ptr,
                 dB_ptr, dC_ptr, dD_ptr, dz_ptr, ddt_bias_ptr, dinit_ptr, batch, seqlen, nheads,
                 headdim, dstate, dtype, ws_ptr, ws_bytes, stream) -> int:
    """Direct call of ``ssd_scan_bwd``; returns the status."""
    return int(load_library().ssd_scan_bwd(
        x_ptr, dt_ptr, A_ptr, B_ptr, C_ptr, D_ptr, z_ptr, dt_bias_ptr, float(dt_min),
        float(dt_max), int(chunk_size), int(ngroups), init_ptr, dout_ptr, dfinal_ptr, dx_ptr,
        ddt_ptr, dA_ptr, dB_ptr, dC_ptr, dD_ptr, dz_ptr, ddt_bias_ptr, dinit_ptr, int(batch),
        int(seqlen), int(nheads), int(headdim), int(dstate), int(dtype), ws_ptr, int(ws_bytes),
        stream))


def scan_bwd(x, dt, A, B, C, dout, D=None, z=None, dt_bias=None, dt_limit=(0.0, math.inf),
             chunk_size: int = 128, initial_states=None, dfinal_states=None,
             return_dinitial_states: bool = True, workspace=None):
    """Gradients of sum(dout * out) + sum(dfinal_states * final_states) of
    ``scan_fwd`` with respect to x, dt (raw), A, B, C, D, z, dt_bias and the
    initial state.  x, dt, B, C, z and dout are all float32 or all bfloat16;
    their gradients dx, ddt, dB, dC, dz come back in that dtype, the others
    (dA, dD, ddt_bias, dinitial_states) in float32.  Returns a dict: dx, ddt,
    dA, dB, dC, and dD / dz / ddt_bias when D / z / dt_bias are given,
    dinitial_states when asked for."""
    import torch

    load_library()
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("the backward takes float32 or bfloat16 inputs")
    io = x.dtype
    code = SSD_BF16 if io == torch.bfloat16 else SSD_F32
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    for name, t, want in (("x", x, io), ("dt", dt, io), ("A", A, torch.float32), ("B", B, io),
                          ("C", C, io), ("dout", dout, io), ("D", D, torch.float32), ("z", z, io),
                          ("dt_bias", dt_bias, torch.float32),
                          ("initial_states", initial_states, torch.float32),
                          ("dfinal_states", dfinal_states, torch.float32)):
        if t is None:
            continue
        if t.device != dev or t.dtype != want or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {want} tensor on x's device")
    if tuple(dout.shape) != (b, L, H, P):
        raise ValueError("dout must have x's shape")
    e = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    eio = lambda *shape: torch.empty(shape, dtype=io, device=dev)
    g = {"dx": eio(b, L, H, P), "ddt": eio(b, L, H), "dA": e(H), "dB": eio(b, L, G, N),
         "dC": eio(b, L, G, N), "dD": e(H) if D is not None else None,
         "dz": eio(b, L, H, P) if z is not None else None,
         "ddt_bias": e(H) if dt_bias is not None else None,
         "dinitial_states": e(b, H, P, N) if return_dinitial_states else None}
    ws_bytes = bwd_workspace_size(b, L, H, P, N, G, chunk_size, code)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(scan_bwd_raw(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
        dt_limit[0], dt_limit[1], chunk_size, G, _ptr(initial_states), _ptr(dout),
        _ptr(dfinal_states), _ptr(g["dx"]), _ptr(g["ddt"]), _ptr(g["dA"]), _ptr(g["dB"]),
        _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddt_bias"]),
        _ptr(g["dinitial_states"]), b, L, H, P, N, code, _ptr(workspace), workspace.numel(),
        stream))
    return {k: v for k, v in g.items() if v is not None}


def split_conv1d_scan_fwd_raw(zx_ptr, cw_ptr, cb_ptr, dt_bias_ptr, A_ptr, D_ptr, chunk_size,
                              init_ptr, dt_min, dt_max, norm_w_ptr, eps, headdim, ngroups,
                              norm_groups, out_ptr, final_ptr, batch, seqlen, nheads, dstate,
                              conv_width, dtype, ws_ptr, ws_bytes, stream) -> int:
    """Direct call of ``ssd_split_conv1d_scan_fwd``; returns the status."""
    return int(load_library().ssd_split_conv1d_scan_fwd(
        zx_ptr, cw_ptr, cb_ptr, dt_bias_ptr, A_ptr, D_ptr, int(chunk_size), init_ptr,
        float(dt_min), float(dt_max), norm_w_ptr, float(eps), int(headdim), int(ngroups),
        int(norm_groups), out_ptr, final_ptr, int(batch), int(seqlen), int(nheads), int(dstate),
        int(conv_width), int(dtype), ws_ptr, int(ws_bytes), stream))


def split_conv1d_scan_fwd(zxbcdt, conv1d_weight, conv1d_bias, dt_bias, A, D, chunk_size: int,
                          headdim: int, ngroups: int, dstate: int, rmsnorm_weight=None,
                          rmsnorm_eps: float = 1e-5, norm_groups: int = 1,
                          dt_limit=(0.0, math.inf), initial_states=None,
                          return_final_states: bool = False, out=None, final_states=None,
                          workspace=None):
    """The Mamba-2 block around the scan (mamba issue #647's fused block up to
    its out_proj): zxbcdt [b, L, 2 dim + 2 G N + H] float32 or bfloat16,
    conv1d_weight [dim + 2 G N, W] and bias, dt_bias, A, D, rmsnorm_weight
    [dim] float32.  Returns out [b, L, dim] (zxbcdt's dtype), or (out,
    final_states)."""
    import torch

    load_library()
    if zxbcdt.dtype == torch.float32:
        dtype = SSD_F32
    elif zxbcdt.dtype == torch.bfloat16:
        dtype = SSD_BF16
    else:
        raise TypeError(f"zxbcdt must be float32 or bfloat16, got {zxbcdt.dtype}")
    if zxbcdt.dim() != 3 or conv1d_weight.dim() != 2:
        raise ValueError("expected zxbcdt [b, L, width] and conv1d_weight [channels, W]")
    b, L, width = zxbcdt.shape
    H = A.shape[0]
    dim = H * headdim
    if width != 2 * dim + 2 * ngroups * dstate + H:
        raise ValueError("zxbcdt width must be 2*dim + 2*ngroups*dstate + nheads")
    if conv1d_weight.shape[0] != dim + 2 * ngroups * dstate:
        raise ValueError("conv1d_weight must have dim + 2*ngroups*dstate rows")
    dev = zxbcdt.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    for name, t in (("zxbcdt", zxbcdt), ("conv1d_weight", conv1d_weight),
                    ("conv1d_bias", conv1d_bias), ("dt_bias", dt_bias), ("A", A), ("D", D),
                    ("rmsnorm_weight", rmsnorm_weight), ("initial_states", initial_states)):
        if t is None:
            continue
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on zxbcdt's device")
        if name != "zxbcdt" and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    W = conv1d_weight.shape[1]
    if out is None:
        out = torch.empty((b, L, dim), dtype=zxbcdt.dtype, device=dev)
    if return_final_states and final_states is None:
        final_states = torch.empty((b, H, headdim, dstate), dtype=torch.float32, device=dev)
    ws_bytes = block_workspace_size(b, L, H, headdim, dstate, ngroups, chunk_size, dtype, W,
                                    norm_groups)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(split_conv1d_scan_fwd_raw(
        _ptr(zxbcdt), _ptr(conv1d_weight), _ptr(conv1d_bias), _ptr(dt_bias), _ptr(A), _ptr(D),
        chunk_size, _ptr(initial_states), dt_limit[0], dt_limit[1], _ptr(rmsnorm_weight),
        rmsnorm_eps, headdim, ngroups, norm_groups, _ptr(out),
        _ptr(final_states) if return_final_states else None, b, L, H, dstate, W, dtype,
        _ptr(workspace), workspace.numel(), stream))
    return (out, final_states) if return_final_states else out


def scan_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_limit=(0.0, math.inf),
             chunk_size: int = 128, initial_states=None, return_final_states: bool = False,
             out=None, final_states=None, workspace=None, timing: Optional[Timing] = None,
             seq_idx=None, kernel_path: str = "auto", check_wait: bool = False):
    """SSD chunked selective-scan forward on the GPU.

    x [b, L, H, P], dt [b, L, H], B/C [b, L, G, N], z like x: float32 or
    bfloat16 (all the same); A, D, dt_bias [H] and initial_states [b, H, P, N]
    float32.  Returns out (x's dtype), or (out, final_states) with
    ``return_final_states``.  ``out``, ``final_states`` and ``workspace``
    (uint8) may be given to avoid allocations; ``final_states`` may be the
    ``initial_states`` tensor itself (in-place continuation).  ``seq_idx``
    [b, L] int32 packs several sequences per row (the state resets where the
    label changes; ``ssd_scan_fwd_varlen``).  ``kernel_path`` names the
    kernel path ("auto" is ssd_scan_fwd's own choice; ``ssd_scan_fwd_path``).
    On the fused bf16 path a result is valid only if no workgroup gave up its
    bounded wait for the state entering its block; ``check_wait`` synchronizes
    the stream after the call and raises SsdError(SSD_ERR_WAIT) if one did
    (``ssd_scan_fwd_wait_status``; other paths have no such wait)."""
    import torch

    load_library()
    if x.dtype == torch.float32:
        dtype = SSD_F32
    elif x.dtype == torch.bfloat16:
        dtype = SSD_BF16
    else:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    if x.dim() != 4 or B.dim() != 4 or C.shape != B.shape or dt.dim() != 3:
        raise ValueError("expected x [b,L,H,P], dt [b,L,H], B and C [b,L,G,N]")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (b, L, H) or tuple(B.shape[:2]) != (b, L):
        raise ValueError("dt / B / C shapes do not match x")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    for name, t, want in (("dt", dt, x.dtype), ("B", B, x.dtype), ("C", C, x.dtype),
                          ("z", z, x.dtype), ("A", A, torch.float32), ("D", D, torch.float32),
                          ("dt_bias", dt_bias, torch.float32),
                          ("initial_states", initial_states, torch.float32)):
        if t is None:
            continue
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, x on {dev}")
        if t.dtype != want:
            raise TypeError(f"{name} must be {want}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if tuple(A.shape) != (H,):
        raise ValueError("A must have shape [nheads]")
    for name, t in (("D", D), ("dt_bias", dt_bias)):
        if t is not None and tuple(t.shape) != (H,):
            raise ValueError(f"{name} must have shape [nheads]")
    if z is not None and z.shape != x.shape:
        raise ValueError("z must have x's shape")
    if initial_states is not None and tuple(initial_states.shape) != (b, H, P, N):
        raise ValueError("initial_states must have shape [b, H, P, N]")
    if seq_idx is not None:
        if seq_idx.dtype != torch.int32 or tuple(seq_idx.shape) != (b, L):
            raise ValueError("seq_idx must be int32 of shape [b, L]")
        if seq_idx.device != dev or not seq_idx.is_contiguous():
            raise ValueError("seq_idx must be a contiguous tensor on x's device")
        if timing is not None:
            raise ValueError("per-stage timing is not offered for seq_idx calls")
    code = path_code(kernel_path)
    if code != 0 and timing is not None:
        raise ValueError("per-stage timing is offered on the automatic path only")

    if out is None:
        out = torch.empty_like(x)
    if return_final_states and final_states is None:
        final_states = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    size_fn = workspace_size if seq_idx is None else varlen_workspace_size
    ws_bytes = size_fn(b, L, H, P, N, G, chunk_size, dtype, kernel_path)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def waited():
        if check_wait:
            _check(wait_status(_ptr(workspace), workspace.numel(), b, L, H, P, N, G, chunk_size,
                               dtype, seq_idx is not None, kernel_path, stream))
        return (out, final_states) if return_final_states else out

    if code != 0:
        _check(scan_fwd_path_raw(
            _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
            dt_limit[0], dt_limit[1], chunk_size, G, _ptr(initial_states), _ptr(out),
            _ptr(final_states) if return_final_states else None, _ptr(seq_idx), b, L, H, P, N,
            dtype, code, _ptr(workspace), workspace.numel(), stream))
        return waited()
    if seq_idx is not None:
        _check(scan_fwd_varlen_raw(
            _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
            dt_limit[0], dt_limit[1], chunk_size, G, _ptr(initial_states), _ptr(out),
            _ptr(final_states) if return_final_states else None, _ptr(seq_idx), b, L, H, P, N,
            dtype, _ptr(workspace), workspace.numel(), stream))
        return waited()
    status = scan_fwd_raw(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
        dt_limit[0], dt_limit[1], chunk_size, G, _ptr(initial_states), _ptr(out),
        _ptr(final_states) if return_final_states else None, b, L, H, P, N, dtype,
        _ptr(workspace), workspace.numel(), stream, timing)
    _check(status)
    return waited()
